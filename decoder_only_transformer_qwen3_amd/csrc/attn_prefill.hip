// Causal grouped-query flash attention for prefill (and any multi-token
// chunk at an offset):  o_h[t] = sum_{j <= p(t)} softmax_j(q_h[t].k_g[j] / sqrt(128)) v_g[j]
// with g = h / 2 ("手写Qwen3-0.6B推理" §Attention; "第 3 章" §3.3).
//
// One workgroup = one KV head g of one sequence and 64 query positions
// (sequences may differ in length and start: packed rows), for
// both query heads 2g and 2g+1 that share g, so each K/V tile staged in LDS
// feeds 128 query rows.  4 waves: wave w takes head 2g + w/2 and 32
// positions.  Two workgroups share a CU, so each SIMD runs two waves whose
// MFMA and softmax phases overlap.
//
// K/V tiles of 64 keys are copied into LDS with direct-to-LDS loads
// (global_load_lds_dwordx4) into a 2-stage ring, one tile ahead of the
// compute, with one barrier per tile.
//
// Per tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = K rows from LDS, B = the wave's Q held in registers).  The K rows of
// a 32-key block are fed to the A operand in the order
//   A row 8a + 4h + b  <-  key 16(a/2) + 8h + 4(a%2) + b,
// so that the accumulator gives lane l (h = l/32) the scores of keys
// 16s + 8h + 0..7 for s = 0, 1: exactly the keys whose values one 16 B
// chunk of the blocked V cache holds for one dim.  O^T += V^T P^T then takes
// those registers, rounded to bf16, directly as the B operand, and each A
// operand (8 positions of one dim) is a single 16 B LDS read.
// K rows are XOR-swizzled in LDS (16 B chunk c of row r at c ^ (r % 16)):
// an operand read has 16 lanes on 16 different rows of a 16-row group, all
// reading the same logical chunk, so they hit 16 different bank groups.
//
// Softmax works in the log2 domain with the hardware exp2; the running max
// is raised only when a score exceeds it by more than 8, so most tiles skip
// the O rescale (p = 2^(s - m) stays below 256).  The causal mask is applied
// only on tiles that reach past a wave's first query.  Positions of the last
// tile at or past the sequence's end are zeroed in LDS once, so masked
// (p = 0) keys never meet garbage values in the V operand.
//
// MFMA lane layouts (32x32x16): A row l%32, B column l%32, k-slot (l/32, j);
// C column l%32, rows 8*(i/4) + 4*(l/32) + (i%4).
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int FA_BQ = 64;                  // query positions per workgroup (per head)
constexpr int FA_BK = 64;                  // keys per tile
constexpr int FA_NS = 2;                   // LDS stages
constexpr int FA_TILE = FA_BK * D;         // bf16 elements of one K or V tile (16 KB)
constexpr float FA_RESCALE_SLACK = 8.0f;

// 16 B-chunk swizzle of K row r in LDS
__device__ __forceinline__ int fa_kswz(int r) { return r & 15; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <bool QNORM>
__global__ __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_prefill(
    const uint16_t* __restrict__ q, int ldq, const uint16_t* __restrict__ q_norm, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    uint16_t* __restrict__ out, SeqMap sm, int max_seq) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[FA_NS][2][FA_TILE];

  // XCD-aware order: workgroups go round-robin to the 8 XCDs by linear id,
  // so KV head g = id % 8 stays on one XCD, and that XCD walks its slots
  // sequence by sequence, longest (latest) query tiles first: the query
  // tiles of one (sequence, KV head) run together on one XCD and share its
  // L2 for their K/V tiles.
  static_assert(HKV == 8, "one KV head per XCD");
  const int n_qt = gridDim.x / (HKV * sm.n);
  const int g = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int b = slot / n_qt, qt = n_qt - 1 - (slot - b * n_qt);
  const int T = sm_len(sm, b), row0 = sm_row0(sm, b);
  int start = sm_start(sm, b);
  start = start < 0 ? 0 : start;
  if (qt * FA_BQ >= T || start + T > max_seq) return;  // past this sequence's rows (whole workgroup)
  const int tid = threadIdx.x, l = tid & 63, lq = l & 31, lh = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int hq = 2 * g + (w >> 1);
  const int t0 = qt * FA_BQ + 32 * (w & 1);  // first query row of this wave
  const int kv_len = start + T;
  const int wg_last = (qt * FA_BQ + FA_BQ - 1) < T ? (qt * FA_BQ + FA_BQ - 1) : T - 1;
  const int n_kt = (start + wg_last) / FA_BK + 1;  // key tiles of the workgroup
  __builtin_assume(n_kt >= 1);                     // start >= 0 and wg_last >= 0 past the return above
  const int wave_last = (t0 + 31) < T ? (t0 + 31) : T - 1;
  const int wave_kt = t0 < T ? (start + wave_last) / FA_BK + 1 : 0;  // tiles this wave computes
  const int wave_pmin = start + (t0 < T ? t0 : T - 1);

  const uint16_t* kbase = k_cache + ((size_t)b * HKV + g) * max_seq * D;
  const uint16_t* vbase = v_cache + ((size_t)b * HKV + g) * max_seq * D;
  const int last_key = kv_len - 1, last_blk = (kv_len - 1) & ~7;

  // DMA of key tile j into its stage: 8 instructions per thread (4 for K, 4 for V).
  // Lane offsets are fixed; every tile but the last adds a uniform base
  // (j * 64 rows), and only the last clamps its rows to the cache range.
  const int kr_lane = 4 * w + (l >> 4);  // K row within each 16-row quarter
  const int koff = kr_lane * D + 8 * ((l & 15) ^ fa_kswz(kr_lane));
  auto issue = [&](int j) {
    uint16_t* ks = lds[j % FA_NS][0];
    uint16_t* vs = lds[j % FA_NS][1];
    if (j + 1 < n_kt) {
      const uint16_t* kt = kbase + (size_t)j * FA_BK * D;
      const uint16_t* vt = vbase + (size_t)j * FA_BK * D;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        __builtin_amdgcn_global_load_lds((const void*)(kt + 16 * rq * D + koff),
                                         (lds_ptr_t)(ks + (16 * rq + 4 * w) * D), 16, 0, 0);
      }
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int ch = 4 * rq + w;
        __builtin_amdgcn_global_load_lds((const void*)(vt + 8 * (ch >> 1) * D + (ch & 1) * 512 + 8 * l),
                                         (lds_ptr_t)(vs + ch * 512), 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {  // K rows 16 rq + 4 w .. +3, one row per 16 lanes
      const int r = 16 * rq + kr_lane;
      int key = j * FA_BK + r;
      key = key < last_key ? key : last_key;
      __builtin_amdgcn_global_load_lds((const void*)(kbase + (size_t)key * D + (koff - kr_lane * D)),
                                       (lds_ptr_t)(ks + (16 * rq + 4 * w) * D), 16, 0, 0);
    }
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {  // V: the tile's 8 blocks are 16 KB of contiguous cache
      const int ch = 4 * rq + w;      // 1 KB chunk: block ch/2, half ch%2
      int pb = j * FA_BK + 8 * (ch >> 1);
      pb = pb < last_blk ? pb : last_blk;
      __builtin_amdgcn_global_load_lds((const void*)(vbase + (size_t)pb * D + (ch & 1) * 512 + 8 * l),
                                       (lds_ptr_t)(vs + ch * 512), 16, 0, 0);
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  // K row read by this lane's A operand within a 32-key block
  const int krow = 16 * (lq >> 4) + 8 * ((lq >> 2) & 1) + 4 * ((lq >> 3) & 1) + (lq & 3);

  issue(0);

  // ---- Q operand: qreg[s] = dims 16 s + 8 lh .. +7 of query row t0 + lq
  // (loaded after the first K/V tile's DMA is issued, so the two overlap)
  u32x4 qreg[8];
  {
    int tq = t0 + lq;
    tq = tq < T ? tq : T - 1;
    const uint16_t* qrow = q + ((size_t)row0 + tq) * ldq + hq * D + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qreg[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s);
    if constexpr (QNORM) {
      // raw projection: per-head RMSNorm with the q gain, then NeoX RoPE at
      // position start + tq ("手写Qwen3-0.6B推理" §Attention and §Rope).  The
      // lane holds 64 of the head's dims, lane l ^ 32 the other 64, and the
      // RoPE partner of dim d < 64 (qreg[s], s < 4) is d + 64 (qreg[s + 4]).
      int pc = start + tq;
      pc = pc < MAXPOS ? pc : MAXPOS - 1;
      const float* cr = rope_cos + (size_t)pc * ROPE_HALF + 8 * lh;
      const float* sr = rope_sin + (size_t)pc * ROPE_HALF + 8 * lh;
      const uint16_t* gq = q_norm + 8 * lh;
      u32x4 ga[4], gb[4];
      f32x4 c0[4], c1[4], s0[4], s1[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ga[s] = *reinterpret_cast<const u32x4*>(gq + 16 * s);
        gb[s] = *reinterpret_cast<const u32x4*>(gq + 64 + 16 * s);
        c0[s] = *reinterpret_cast<const f32x4*>(cr + 16 * s);
        c1[s] = *reinterpret_cast<const f32x4*>(cr + 16 * s + 4);
        s0[s] = *reinterpret_cast<const f32x4*>(sr + 16 * s);
        s1[s] = *reinterpret_cast<const f32x4*>(sr + 16 * s + 4);
      }
      __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the first wait
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 v = qreg[s];
        ss += bf_lo(v.x) * bf_lo(v.x) + bf_hi(v.x) * bf_hi(v.x) + bf_lo(v.y) * bf_lo(v.y) + bf_hi(v.y) * bf_hi(v.y) +
              bf_lo(v.z) * bf_lo(v.z) + bf_hi(v.z) * bf_hi(v.z) + bf_lo(v.w) * bf_lo(v.w) + bf_hi(v.w) * bf_hi(v.w);
      }
      ss += __shfl_xor(ss, 32, 64);
      const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + EPS);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 xa = qreg[s], xb = qreg[s + 4];
        const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w}, yw[4] = {xb.x, xb.y, xb.z, xb.w};
        const uint32_t gaw[4] = {ga[s].x, ga[s].y, ga[s].z, ga[s].w}, gbw[4] = {gb[s].x, gb[s].y, gb[s].z, gb[s].w};
        const float cs[8] = {c0[s][0], c0[s][1], c0[s][2], c0[s][3], c1[s][0], c1[s][1], c1[s][2], c1[s][3]};
        const float sn[8] = {s0[s][0], s0[s][1], s0[s][2], s0[s][3], s1[s][0], s1[s][1], s1[s][2], s1[s][3]};
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float o0[2], o1[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float x = h ? bf_hi(xw[e]) : bf_lo(xw[e]), y = h ? bf_hi(yw[e]) : bf_lo(yw[e]);
            const float a = x * rinv * (h ? bf_hi(gaw[e]) : bf_lo(gaw[e]));
            const float bb = y * rinv * (h ? bf_hi(gbw[e]) : bf_lo(gbw[e]));
            o0[h] = a * cs[2 * e + h] - bb * sn[2 * e + h];
            o1[h] = bb * cs[2 * e + h] + a * sn[2 * e + h];
          }
          lo[e] = pack_bf2(o0[0], o0[1]);
          hi[e] = pack_bf2(o1[0], o1[1]);
        }
        qreg[s] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        qreg[s + 4] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      }
    }
  }


  // LDS read offsets (bytes) of this lane, fixed for the whole loop: K operand
  // of dim step s in 32-key block 0 (block 1 is 32 rows further), V operand
  // of step 0 (the other steps are constant offsets)
  uint32_t kofs[8];
  {
    const int sw = fa_kswz(krow);  // equal for rows krow and 32 + krow
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) kofs[s8] = 2u * (uint32_t)(krow * D + 8 * ((2 * s8 + lh) ^ sw));
  }
  const uint32_t vofs = 2u * (uint32_t)(lh * (D * VBLK) + lq * VBLK);
  const char* lds_b = reinterpret_cast<const char*>(&lds[0][0][0]);

  // tile j in stage ST = j % 2 (a compile-time constant, so the stage offset
  // folds into the LDS instructions' immediate offsets)
  auto tile = [&](int j, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's part of tile j landed
    __builtin_amdgcn_s_barrier();        // all of tile j is in LDS; stage (j+1)%2 is free
    if (j + 1 < n_kt) issue(j + 1);
    if (j == n_kt - 1 && n_kt * FA_BK > kv_len) {  // zero the V positions past the end, once
      uint16_t* vz = lds[ST][1];
      const int first = kv_len - j * FA_BK;
      for (int e = tid; e < (FA_BK - first) * D; e += 256) {
        const int p = first + e / D, d = e % D;
        vz[(p >> 3) * (D * VBLK) + d * VBLK + (p & 7)] = 0;
      }
      __syncthreads();
    }
    if (j >= wave_kt) return;            // past this wave's causal range (wave-uniform)

    const char* ks = lds_b + ST * (2 * FA_TILE * 2);
    const char* vs = ks + FA_TILE * 2;
    // ---- S^T = K Q^T: sacc[kb] for keys j*64 + 32 kb + (row order above)
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
    {
      // 16 K operand reads (2 key blocks x 8 dim steps) in a ring four reads
      // ahead of the MFMAs
      auto kread = [&](int x) {
        return *reinterpret_cast<const u32x4*>(ks + kofs[x & 7] + (x >> 3) * (32 * D * 2));
      };
      // step y: key block y % 2, dim step y / 2, so consecutive MFMAs go to
      // different accumulators
      auto kx = [](int y) { return 8 * (y & 1) + (y >> 1); };
      u32x4 ka[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) ka[y] = kread(kx(y));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int y = 0; y < 16; ++y) {
        sacc[y & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[y & 3]), as_bf16x8(qreg[y >> 1]),
                                                              sacc[y & 1], 0, 0, 0);
        if (y + 4 < 16) ka[y & 3] = kread(kx(y + 4));
        __builtin_amdgcn_sched_barrier(0);  // keep each read four steps ahead of its MFMA
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- causal mask, lazy online softmax, P packed to bf16.  Lane keys
    // relative to the tile: 32 kb + 16 (i / 8) + 8 lh + i % 8.
    const bool v_tail = (j + 1) * FA_BK > kv_len;  // the tile runs past the cache range
    const bool need_mask = (j * FA_BK + FA_BK - 1) > wave_pmin || v_tail;
    u32x4 pb[4];  // per key step of 16
    {
      float sv[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[16 * kb + i] = sacc[kb][i];
      if (need_mask) {
        // keys above min(query position, kv_len - 1) are excluded
        int lim = start + t0 + lq;
        lim = lim < kv_len - 1 ? lim : kv_len - 1;
        lim -= j * FA_BK + 8 * lh;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sv[16 * kb + i] = (32 * kb + 16 * (i >> 3) + (i & 7)) > lim ? -INFINITY : sv[16 * kb + i];
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) mx = fmaxf(mx, sv[i]);
      {  // with the partner lane l ^ 32 (same query), through a lane swap instead of the LDS crossbar
        const auto sw32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw32[0]), __uint_as_float(sw32[1])) * sl2;
      }
      const bool raise = mx > m_run + FA_RESCALE_SLACK;
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
      const float mneg = -m_run;
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k)  // key step of 16: sv[8k .. 8k+7]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[8 * k + 2 * e], sl2, mneg));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[8 * k + 2 * e + 1], sl2, mneg));
          ls += p0 + p1;
          pb[k][e] = pack_bf2(p0, p1);
        }
      l_run += ls;
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T P^T, 16 keys per MFMA step; A = 8 positions of one dim
    {
      // 16 V operand reads (4 key steps x 4 dim blocks) in a ring four reads ahead
      auto vread = [&](int x) {
        return *reinterpret_cast<const u32x4*>(vs + vofs + 2 * (2 * (x >> 2) * (D * VBLK) + 32 * (x & 3) * VBLK));
      };
      u32x4 va[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) va[x] = vread(x);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int st = x >> 2, db = x & 3;
        u32x4 a = va[x & 3];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pb[st]), oacc[db], 0, 0, 0);
        if (x + 4 < 16) va[x & 3] = vread(x + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int j = 0; j < n_kt; j += 2) {
    tile(j, std::integral_constant<int, 0>{});
    if (j + 1 < n_kt) tile(j + 1, std::integral_constant<int, 1>{});
  }

  // ---- normalise and store: lane holds dims db*32 + 8*(i/4) + 4*lh + (i%4) of its query
  {
    const int tq = t0 + lq;
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (tq < T) {
      const float inv = 1.0f / l_tot;
      uint16_t* orow = out + ((size_t)row0 + tq) * QDIM + hq * D;
#pragma unroll
      for (int db = 0; db < 4; ++db) store_block_bf16(orow + db * 32, oacc[db] * inv, lh);
    }
  }
}

void launch_attn_prefill(const uint16_t* q, int ldq, const uint16_t* q_norm, const float* rope_cos,
                         const float* rope_sin, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out,
                         const SeqMap& sm, int max_T, int max_seq, hipStream_t s) {
  const dim3 grid(((max_T + FA_BQ - 1) / FA_BQ) * HKV * sm.n);
  if (q_norm)
    hipLaunchKernelGGL(k_attn_prefill<true>, grid, dim3(256), 0, s, q, ldq, q_norm, rope_cos, rope_sin, k_cache,
                       v_cache, out, sm, max_seq);
  else
    hipLaunchKernelGGL(k_attn_prefill<false>, grid, dim3(256), 0, s, q, ldq, q_norm, rope_cos, rope_sin, k_cache,
                       v_cache, out, sm, max_seq);
}

}  // namespace q3
