// Causal grouped-query flash attention for prefill (and any multi-token
// chunk at an offset):  o_h[t] = sum_{j <= p(t)} softmax_j(q_h[t].k_g[j] / sqrt(128)) v_g[j]
// with g = h / 2 ("手写Qwen3-0.6B推理" §Attention; "第 3 章" §3.3).
//
// One workgroup = one KV head g of one sequence and 128 query positions, for
// BOTH query heads 2g and 2g+1, so each K/V tile staged in LDS feeds 256
// query rows.  8 waves: wave w takes head 2g + w/4 and 32 positions.
//
// Per 64-key tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = K rows from LDS, B = the wave's Q held in registers).  The
// accumulator gives each lane one query (column l%32) and 32 of the 64 key
// scores, so the online-softmax max and sum are lane-local up to one
// exchange with lane l^32.  O^T = V^T P^T then takes the score registers,
// rounded to bf16, directly as the B operand; the A operand (8 consecutive
// positions of one dim) comes straight from the blocked V cache layout,
// which is staged into LDS as a plain copy.
//
// The running max is only raised when a new score exceeds it by more than
// 8 (log2 units), so most tiles skip the O rescale; p = 2^(s - m) then stays
// below 256, well inside float and bfloat16 range, and the final O / l is
// unchanged.
//
// MFMA lane layouts (32x32x16): A row l%32, B column l%32, k-slot (l/32, j);
// C column l%32, rows 8*(i/4) + 4*(l/32) + (i%4).
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int FA_BQ = 128;        // query positions per workgroup (per head)
constexpr int FA_BK = 64;         // keys per tile
constexpr int FA_THREADS = 512;   // 8 waves
constexpr int KS_STRIDE = D + 8;  // K tile row (bf16), 272 B
constexpr int VS_ELEMS = FA_BK * D;  // blocked V tile: 8 blocks x 128 dims x 8 positions
constexpr float RESCALE_SLACK = 8.0f;

__global__ __launch_bounds__(FA_THREADS) void k_attn_prefill(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k_cache,
                                                             const uint16_t* __restrict__ v_cache,
                                                             uint16_t* __restrict__ out, int T, int start,
                                                             int max_seq) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][FA_BK * KS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][VS_ELEMS];

  const int qt = gridDim.x - 1 - blockIdx.x;  // longest (latest) tiles first
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, lh = l >> 5;
  const int hq = 2 * g + (w >> 2);
  const int t0 = qt * FA_BQ + 32 * (w & 3);  // first query of this wave
  const int tq = t0 + lq;                    // this lane's query
  const int tq_c = tq < T ? tq : T - 1;      // rows past the end are computed, not stored
  const int pq = start + tq_c;               // its absolute position
  const int kv_len = start + T;
  const int wave_pmin = start + (t0 < T ? t0 : T - 1);
  const int wave_pmax = start + ((t0 + 31) < T ? (t0 + 31) : T - 1);
  const int wg_last = (qt * FA_BQ + FA_BQ - 1) < T ? (qt * FA_BQ + FA_BQ - 1) : T - 1;
  const int n_kt = (start + wg_last) / FA_BK + 1;

  // Q operand: lane holds dims 16 s + 8 lh + j of its query, s = 0..7
  u32x4 qreg[8];
  {
    const uint16_t* qrow = q + ((size_t)b * T + tq_c) * QDIM + hq * D + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qreg[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
  }

  const uint16_t* kbase = k_cache + ((size_t)b * HKV + g) * max_seq * D;
  const uint16_t* vbase = v_cache + ((size_t)b * HKV + g) * max_seq * D;
  u32x4 kreg[2], vreg[2];

  // K: chunk c = tid + 512 i -> key c/16, dims 8*(c%16).  V: the tile's 8
  // position blocks are 16 KB of contiguous cache; chunk c covers dim c%128
  // of block c/128 (8 positions).  Loads only read in-range blocks (clamped
  // to the last real block); positions at or past kv_len are zeroed when the
  // registers are written to LDS, so prefetching never waits on a mask.
  const int last_blk = ((kv_len - 1) >> 3) << 3;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + FA_THREADS * i;
      int key = j * FA_BK + (c >> 4);
      key = key < kv_len ? key : kv_len - 1;
      kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * D + (c & 15) * 8);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + FA_THREADS * i;
      int p0 = j * FA_BK + (c >> 7) * VBLK;
      p0 = p0 < last_blk ? p0 : last_blk;
      vreg[i] = *reinterpret_cast<const u32x4*>(vbase + (size_t)p0 * D + (size_t)(c & 127) * VBLK);
    }
  };
  auto store_tile = [&](int buf, int j) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + FA_THREADS * i;
      *reinterpret_cast<u32x4*>(&Ks[buf][(c >> 4) * KS_STRIDE + (c & 15) * 8]) = kreg[i];
      const int valid = kv_len - (j * FA_BK + (c >> 7) * VBLK);  // real positions in this chunk
      u32x4 v = vreg[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t keep = (2 * e + 1 < valid) ? 0xffffffffu : ((2 * e < valid) ? 0x0000ffffu : 0u);
        v[e] &= keep;
      }
      *reinterpret_cast<u32x4*>(&Vs[buf][c * VBLK]) = v;
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
  store_tile(0, 0);
  __syncthreads();

  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_kt) load_tile(j + 1);
    if (j * FA_BK <= wave_pmax) {
      const uint16_t* ks = Ks[buf];
      const uint16_t* vs = Vs[buf];
      // ---- S^T = K Q^T for keys j*64 .. j*64+63 (two 32-key blocks)
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&ks[(kb * 32 + lq) * KS_STRIDE + 16 * s + 8 * lh]);
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
      // ---- lazy rescale: raise the running max only when it is exceeded by more than the slack
      const bool raise = mx > m_run + RESCALE_SLACK;
      if (__ballot(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_run = m_new;
      }
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][i] - m_run);
          sacc[kb][i] = p;
          lsum += p;
        }
      l_run += lsum;
      // ---- O^T += V^T P^T, 16 keys per MFMA step
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, c = st & 1;
        u32x4 pb;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pb[jj] = pack_bf2(sacc[kb][8 * c + 2 * jj], sacc[kb][8 * c + 2 * jj + 1]);
        // this lane's keys: block (4 kb + 2 c) positions 4 lh..4 lh+3, block (4 kb + 2 c + 1) same positions
        const int blk = 4 * kb + 2 * c;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = db * 32 + lq;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(&vs[(blk * D + d) * VBLK + 4 * lh]);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(&vs[((blk + 1) * D + d) * VBLK + 4 * lh]);
          const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb), oacc[db], 0, 0, 0);
        }
      }
    }
    if (j + 1 < n_kt) store_tile(buf ^ 1, j + 1);
    __syncthreads();
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
  hipLaunchKernelGGL(k_attn_prefill, grid, dim3(FA_THREADS), 0, s, q, k_cache, v_cache, out, T, start, max_seq);
}

}  // namespace q3
