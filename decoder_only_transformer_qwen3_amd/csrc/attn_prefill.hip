// Causal grouped-query flash attention for prefill (and any multi-token
// chunk at an offset):  o_h[t] = sum_{j <= p(t)} softmax_j(q_h[t].k_g[j] / sqrt(128)) v_g[j]
// with g = h / 2 ("手写Qwen3-0.6B推理" §Attention; "第 3 章" §3.3).
//
// One workgroup = one KV head g of one sequence and 64 query positions, for
// BOTH query heads 2g and 2g+1, so each K/V tile read from the cache feeds
// 128 query rows.  4 waves: wave w takes head 2g + w/2 and 32 positions.
//
// Per 64-key tile, a wave computes S^T = K Q^T with the 32x32x16 MFMA
// (A = K rows from LDS, B = the wave's Q held in registers).  The
// accumulator gives each lane one query (column l%32) and 32 of the 64 key
// scores, so the online-softmax max and sum are lane-local up to one
// exchange with lane l^32.  O^T = V^T P^T then reuses the score registers
// directly as the B operand (P in bf16), with V^T staged in LDS by
// transposing the tile on its way in.
//
// MFMA lane layouts (32x32x16): A row l%32, B column l%32, k-slot (l/32, j);
// C column l%32, rows 8*(i/4) + 4*(l/32) + (i%4).
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int FA_BQ = 64;             // query positions per workgroup
constexpr int FA_BK = 64;             // keys per tile
constexpr int KS_STRIDE = D + 8;      // K tile row (bf16), 272 B
constexpr int VT_STRIDE = FA_BK + 4;  // V^T tile row (bf16), 136 B

__global__ __launch_bounds__(256) void k_attn_prefill(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                                                      const uint16_t* __restrict__ v_cache, uint16_t* __restrict__ out,
                                                      int T, int start, int max_seq) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[FA_BK * KS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VT_STRIDE];

  const int qt = gridDim.x - 1 - blockIdx.x;  // longest (latest) tiles first
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, lh = l >> 5;
  const int hq = 2 * g + (w >> 1);
  const int t0 = qt * FA_BQ + 32 * (w & 1);  // first query of this wave
  const int tq = t0 + lq;                    // this lane's query
  const int tq_c = tq < T ? tq : T - 1;      // rows past the end are computed but not stored
  const int pq = start + tq_c;               // its absolute position
  const int kv_len = start + T;
  const int wave_pmin = start + (t0 < T ? t0 : T - 1);
  const int wave_pmax = start + ((t0 + 31) < T ? (t0 + 31) : T - 1);
  const int wg_pmax = start + ((qt * FA_BQ + FA_BQ - 1) < T ? (qt * FA_BQ + FA_BQ - 1) : T - 1);
  const int n_kt = wg_pmax / FA_BK + 1;

  // Q operand: lane holds dims 16 s + 8 lh + j of its query, s = 0..7
  u32x4 qreg[8];
  {
    const uint16_t* qrow = q + ((size_t)b * T + tq_c) * QDIM + hq * D + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qreg[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
  }

  const uint16_t* kbase = k_cache + ((size_t)b * HKV + g) * max_seq * D;
  const uint16_t* vbase = v_cache + ((size_t)b * HKV + g) * max_seq * D;
  // K staging: chunk c = tid + 256 i -> key c/16, dims 8*(c%16)
  // V staging: keys 4*(tid%16) + i, dims 8*(tid/16) .. +7
  const int v_kg = tid & 15, v_dg = tid >> 4;
  u32x4 kreg[4], vreg[4];

  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      int key = j * FA_BK + (c >> 4);
      key = key < kv_len ? key : kv_len - 1;
      kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * D + (c & 15) * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int key = j * FA_BK + 4 * v_kg + i;
      key = key < kv_len ? key : kv_len - 1;
      vreg[i] = *reinterpret_cast<const u32x4*>(vbase + (size_t)key * D + 8 * v_dg);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&Ks[(c >> 4) * KS_STRIDE + (c & 15) * 8]) = kreg[i];
    }
    // transpose 4 keys x 8 dims into V^T rows (8 B per dim)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int word = e >> 1;
      const bool hi = e & 1;
      uint32_t h0 = hi ? (vreg[0][word] >> 16) : (vreg[0][word] & 0xffffu);
      uint32_t h1 = hi ? (vreg[1][word] >> 16) : (vreg[1][word] & 0xffffu);
      uint32_t h2 = hi ? (vreg[2][word] >> 16) : (vreg[2][word] & 0xffffu);
      uint32_t h3 = hi ? (vreg[3][word] >> 16) : (vreg[3][word] & 0xffffu);
      u32x2 pk = {h0 | (h1 << 16), h2 | (h3 << 16)};
      *reinterpret_cast<u32x2*>(&Vt[(8 * v_dg + e) * VT_STRIDE + 4 * v_kg]) = pk;
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)

  load_tile(0);
  store_tile();
  __syncthreads();

  for (int j = 0; j < n_kt; ++j) {
    if (j + 1 < n_kt) load_tile(j + 1);
    if (j * FA_BK <= wave_pmax) {
      // ---- S^T = K Q^T for keys j*64 .. j*64+63 (two 32-key blocks)
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[(kb * 32 + lq) * KS_STRIDE + 16 * s + 8 * lh]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[s]), sacc[kb], 0, 0, 0);
        }
      }
      // ---- scale (log2 domain) and causal mask
      const bool need_mask = (j * FA_BK + FA_BK - 1) > wave_pmin;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float sv = sacc[kb][i] * sl2;
          if (need_mask) {
            const int key = j * FA_BK + kb * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
            if (key > pq) sv = -INFINITY;
          }
          sacc[kb][i] = sv;
          mx = fmaxf(mx, sv);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2f(sacc[kb][i] - m_new);
          sacc[kb][i] = p;
          lsum += p;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      // ---- O^T += V^T P^T, 16 keys per MFMA step
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, c = st & 1;
        u32x4 pb;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pb[jj] = pack_bf2(sacc[kb][8 * c + 2 * jj], sacc[kb][8 * c + 2 * jj + 1]);
        const int kofs = kb * 32 + 16 * c + 4 * lh;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint16_t* vrow = &Vt[(db * 32 + lq) * VT_STRIDE + kofs];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb), oacc[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (j + 1 < n_kt) {
      store_tile();
      __syncthreads();
    }
  }

  // ---- normalise and store: lane holds dims db*32 + 8*(i/4) + 4*lh + (i%4)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (tq < T) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = out + ((size_t)b * T + tq) * QDIM + hq * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 o;
        o.x = pack_bf2(oacc[db][4 * gq] * inv, oacc[db][4 * gq + 1] * inv);
        o.y = pack_bf2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * gq + 4 * lh) = o;
      }
  }
}

void launch_attn_prefill(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out, int B,
                         int T, int start, int max_seq, hipStream_t s) {
  const dim3 grid((T + FA_BQ - 1) / FA_BQ, HKV, B);
  hipLaunchKernelGGL(k_attn_prefill, grid, dim3(256), 0, s, q, k_cache, v_cache, out, T, start, max_seq);
}

}  // namespace q3
