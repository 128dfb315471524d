// Split-K decode attention: one new query per sequence attends to cache
// rows 0..p (p = its position; "古法手撕简易LLM推理器" §prefill与predict
// decodes one token against the whole cache, and "从零开始写Qwen3（二）"
// §Attn notes such a query must see every cached key).
//
// The kernel starts from the raw merged projection of the new token, so the
// per-head q/k RMSNorm and NeoX RoPE ("手写Qwen3-0.6B推理" §Attention and
// §Rope) and the cache write of the new K/V happen here as well:
//   q' = rope_p(gamma_q * q / sqrt(mean(q^2) + eps)), likewise k'; v as is.
// For that step a 16-lane DPP row holds one 128-dim head row (lane j dims
// 8j..8j+7): the head's sum of squares is a row sum and RoPE's partner
// dims (i, i+64) sit in lanes j and j^8 (a row rotate by 8).
//
// Grid (split, KV head g, sequence b); each workgroup reads its key range of
// K and V once for both query heads 2g, 2g+1.  Its 4 waves take 32-key
// tiles round-robin and each keeps its own online softmax, on
// v_mfma_f32_16x16x32_bf16 (lane l: A row l%16, B column l%16, k-slot
// (l/16, j); C column l%16, rows 4(l/16)+i):
//   scores  S^T[key][head] = K q^T, two MFMA chains of 16 keys whose A rows
//           are ordered so that lane l ends up holding keys 8(l/16)+0..7 of
//           head l%16;
//   values  O^T[dim][head] += V^T P^T, where P^T is exactly those registers
//           (exp2, packed to bf16) and the A operand, 8 consecutive
//           positions of one dim, is one 16 B chunk of the blocked V cache.
// Only columns 0 and 1 (the two query heads) are used.  The running max is
// raised only when a score exceeds it by more than 8 (log2 units), so most
// tiles need no cross-lane exchange.  The next tile's loads are in flight
// while a tile is computed.  The split that owns position p writes the new
// K/V into the cache and takes them from LDS rather than from the cache.
//
// The waves combine in LDS; each split writes unnormalised (o, m, l) in
// the log2 domain; the last split to finish for a (b, g) (atomic ticket)
// merges them with log-sum-exp rescaling and writes the two heads' bf16
// outputs.  The key range of a split follows from the sequence's own device
// length, so the result is exact whatever split count the host picked.
//
// With few sequences the launch can also carry workgroups that read the
// weights of the next projections into the L2s that will serve them (below).
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int DT = 32;  // keys per wave tile
constexpr int PART_STRIDE = D + 2;
constexpr int DEC_SPLIT_CAP = 64;
constexpr float DEC_RESCALE_SLACK = 8.0f;

__device__ __forceinline__ void unpack_row8(const u32x4 w, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf_lo(w[e]);
    f[2 * e + 1] = bf_hi(w[e]);
  }
}

// RMSNorm of the head row spread over a 16-lane row (lane j holds dims
// 8j..8j+7): the reciprocal RMS, then gain (gbits: dims 8j..8j+7) and NeoX
// RoPE with the table entries of lane j's frequencies 8(j%8)..8(j%8)+7.
__device__ __forceinline__ float row_rinv8(const float (&f)[8]);
__device__ __forceinline__ void gain_rope8(float (&f)[8], float rinv, const u32x4 gbits, const f32x4 c0,
                                           const f32x4 c1, const f32x4 s0, const f32x4 s1, int j);
// The same from memory: gain row and table rows of position p.
__device__ __forceinline__ void norm_rope8(float (&f)[8], const uint16_t* __restrict__ gamma,
                                           const float* __restrict__ cos_row, const float* __restrict__ sin_row,
                                           int j) {
  const float rinv = row_rinv8(f);
  const u32x4 gbits = *reinterpret_cast<const u32x4*>(gamma + 8 * j);
  const int i0 = 8 * (j & 7);
  gain_rope8(f, rinv, gbits, *reinterpret_cast<const f32x4*>(cos_row + i0),
             *reinterpret_cast<const f32x4*>(cos_row + i0 + 4), *reinterpret_cast<const f32x4*>(sin_row + i0),
             *reinterpret_cast<const f32x4*>(sin_row + i0 + 4), j);
}
__device__ __forceinline__ float row_rinv8(const float (&f)[8]) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
  ss = row16_sum(ss);
  return 1.0f / sqrtf(ss * (1.0f / D) + EPS);
}
__device__ __forceinline__ void gain_rope8(float (&f)[8], float rinv, const u32x4 gbits, const f32x4 c0,
                                           const f32x4 c1, const f32x4 s0, const f32x4 s1, int j) {
  float g[8];
  unpack_row8(gbits, g);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] *= rinv * g[e];
    // partner dim (i + 64 for lanes 0..7, i - 64 for lanes 8..15): DPP row_ror:8
    o[e] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(f[e]), 0x128, 0xf, 0xf, false));
  }
  const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const float sgn = j < 8 ? -1.0f : 1.0f;  // x_i c - x_{i+64} s  |  x_{i+64} c + x_i s
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = f[e] * cs[e] + sgn * o[e] * sn[e];
}

// K/V loads: nontemporal ones stream from HBM faster when the cache is far
// larger than the last-level cache; ordinary ones hit there when it is not.
template <bool NT>
__device__ __forceinline__ u32x4 ld_kv(const uint16_t* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    return *reinterpret_cast<const u32x4*>(p);
}

// ---- L2 warm-up of the weights that follow
// A decode step with a few sequences runs this kernel on a handful of CUs
// while the rest of the chip idles, and the projections that follow are
// latency bound on their weight reads.  Extra workgroups of this launch read
// the o_proj, gate|up and down weights, and the next layer's q|k|v weight,
// so that each byte lands in the L2 of the XCD
// whose workgroups will read it: workgroups are dispatched round-robin over
// the 8 XCDs by linear id, in this launch as in the later ones, so consumer
// workgroup i runs on XCD i % 8, and the warming workgroups of XCD x read
// exactly the slices of the consumers i = x, x + 8, ...  Consumer slices
// (the one-block skinny GEMM and the GEMV of up to 8 rows):
//   o_proj  [1024][2048]: workgroup i (256) reads rows 4i..4i+3   (16 KB)
//   gate|up [6144][1024]: workgroup i (384) reads gate rows 8i..8i+7 and
//                         the matching up rows                    (2 x 16 KB)
//   down    [1024][3072]: workgroup i (256) reads rows 4i..4i+3   (24 KB)
//   q|k|v   [4096][1024]: workgroup i (256) reads rows 16i..16i+15 (32 KB)
// in units of 4 KB (one 16-byte load per thread of a 256-thread group),
// 3.75 MB per XCD, which stays in its 4 MB L2 until read.  On the batch-1
// decode step the gate|up and down regions gave +2.6 %, the next q|k|v
// +2.1 % more and o_proj +1.2 % more.
constexpr int WARM_UG = ((2 * I) / 16 / 8) * 8;  // gate|up units per XCD
constexpr int WARM_UD = (C / 4 / 8) * 6;         // down units per XCD
constexpr int WARM_UQ = (QKV_N / 16 / 8) * 8;    // next layer's q|k|v units per XCD
constexpr int WARM_UO = (C / 4 / 8) * 4;         // o_proj units per XCD
constexpr int WARM_UNITS = WARM_UO + WARM_UG + WARM_UD + WARM_UQ;  // 960
// Loads per thread, all in flight at once: fewer, fuller workgroups were
// measured faster (24 loads: +1.1 % on the batch-1 decode step, 48: +2.6 %;
// issuing them in two waits, or spreading them over more workgroups, lost).
constexpr int WARM_LOADS = 48;
constexpr int WARM_PER_XCD = (WARM_UNITS + WARM_LOADS - 1) / WARM_LOADS;  // 20 workgroups per XCD
static_assert(WARM_PER_XCD * WARM_LOADS >= WARM_UNITS, "every unit needs a load slot");

// j: index of the warming workgroup (its linear id is congruent to j mod 8).
__device__ __forceinline__ void warm_weights(const uint8_t* __restrict__ wo, const uint8_t* __restrict__ wgu,
                                             const uint8_t* __restrict__ wdown, const uint8_t* __restrict__ wqkv,
                                             int j) {
  const int x = j & 7, r = j >> 3;  // XCD of this workgroup, its rank there
  const size_t t16 = (size_t)threadIdx.x * 16;
  u32x4 v[WARM_LOADS];
#pragma unroll
  for (int q = 0; q < WARM_LOADS; ++q) {
    int u = r * WARM_LOADS + q;  // a contiguous run of units
    u = u < WARM_UNITS ? u : r;  // no unit left: re-read the first one (keeps the loads branch-free)
    const uint8_t* a;
    if (u < WARM_UO) {
      a = wo + (size_t)(x + 8 * (u >> 2)) * 16384 + (u & 3) * 4096;
    } else if ((u -= WARM_UO) < WARM_UG) {  // (u counts from the gate|up region on)
      const int half = (u & 7) >> 2;
      a = wgu + (size_t)half * (I * C * 2) + (size_t)(x + 8 * (u >> 3)) * 16384 + (u & 3) * 4096;
    } else if (u < WARM_UG + WARM_UD) {
      const int g = u - WARM_UG;
      a = wdown + (size_t)(x + 8 * (g / 6)) * 24576 + (g % 6) * 4096;
    } else {
      const int g = u - WARM_UG - WARM_UD;
      a = wqkv + (size_t)(x + 8 * (g >> 3)) * 32768 + (g & 7) * 4096;
    }
    v[q] = *reinterpret_cast<const u32x4*>(a + t16);
  }
#pragma unroll
  for (int q = 0; q < WARM_LOADS; ++q) asm volatile("" ::"v"(v[q]));
}

template <bool NT, int NW, bool ONE>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_attn_decode(const uint16_t* __restrict__ qkv,
                                                        const uint16_t* __restrict__ q_norm,
                                                        const uint16_t* __restrict__ k_norm,
                                                        const float* __restrict__ rope_cos,
                                                        const float* __restrict__ rope_sin,
                                                        uint16_t* __restrict__ k_cache,
                                                        uint16_t* __restrict__ v_cache, float* __restrict__ part,
                                                        int* __restrict__ counters, uint16_t* __restrict__ out,
                                                        int max_seq, const int32_t* __restrict__ pos_dev, int start,
                                                        int n_split, int n_seq, const uint8_t* __restrict__ warm_o,
                                                        const uint8_t* __restrict__ warm_gu,
                                                        const uint8_t* __restrict__ warm_down,
                                                        const uint8_t* __restrict__ warm_qkv) {
  if ((int)blockIdx.z >= n_seq) {  // a warming workgroup (z-slices past the n_seq sequences)
    warm_weights(warm_o, warm_gu, warm_down, warm_qkv, blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * (blockIdx.z - n_seq)));
    return;
  }
  __shared__ __attribute__((aligned(16))) uint16_t qs[NW][2][D];  // per wave: rotated q of heads 2g, 2g+1
  __shared__ __attribute__((aligned(16))) uint16_t knew[NW][D];   // per wave: the new key (rotated)
  __shared__ __attribute__((aligned(16))) uint16_t vnew[NW][D];   // per wave: the new value
  __shared__ float wo[NW][2][D];
  __shared__ float wml[NW][2][2];
  __shared__ float mls[2][DEC_SPLIT_CAP][2];
  __shared__ int last_ticket;

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, col = l & 15, grp = l >> 4;
  const size_t head_base = ((size_t)b * HKV + g) * max_seq * D;
  const uint16_t* kbase = k_cache + head_base;
  const uint16_t* vbase = v_cache + head_base;
  // key of A row `col` in score chain `set`: 8*(col/4) + 4*set + col%4 (see the header)
  const int krel0 = 8 * (col >> 2) + (col & 3);
  // two tiles' registers per wave: while one tile is computed, the next is in flight
  u32x4 kA[8], vA[8], kB[8], vB[8];
#define Q3_DEC_LOAD_TILE_AT(TB, KR, VR, LK, LB)                                            \
  {                                                                                        \
    const int tb_ = (TB);                                                                  \
    _Pragma("unroll") for (int set = 0; set < 2; ++set) {                                  \
      int key = tb_ + krel0 + 4 * set;                                                     \
      key = key < (LK) ? key : (LK);                                                       \
      const uint16_t* kp = kbase + (size_t)key * D + 8 * grp;                              \
      _Pragma("unroll") for (int st = 0; st < 4; ++st) KR[4 * set + st] =                  \
          ld_kv<NT>(kp + 32 * st);                                                         \
    }                                                                                      \
    int pb_ = tb_ + 8 * grp;                                                               \
    pb_ = pb_ < (LB) ? pb_ : (LB);                                                         \
    const uint16_t* vp = vbase + (size_t)pb_ * D + col * VBLK;                             \
    _Pragma("unroll") for (int db = 0; db < 8; ++db) VR[db] =                              \
        ld_kv<NT>(vp + 16 * db * VBLK);                                                    \
  }
  // The new token's row (wave rows hold q(2g), q(2g+1), k(g), v(g); lane j
  // dims 8j..8j+7), its gain and its rotary table entries.  With one split
  // (ONE) the key range starts at 0, so a wave's first tile is known before
  // the sequence's position is and is loaded in parallel with it (clamped
  // to the cache; keys past the position are masked and their values
  // zeroed below).  With caches that stay in the last-level cache (EARLY)
  // the row and the gain are loaded before that tile (waiting for them then
  // does not wait for the tile) and the table entries as soon as the
  // position is known; otherwise they are loaded as the norm needs them,
  // which was measured faster there, as was loading only one tile here.
  constexpr bool EARLY = ONE && !NT;
  u32x4 xin, gin;
  f32x4 c0, c1, s0, s1;
  if constexpr (EARLY) {
    const int off = grp < 2 ? (2 * g + grp) * D : QDIM + (grp - 2) * HKV * D + g * D;
    xin = *reinterpret_cast<const u32x4*>(qkv + (size_t)b * QKV_N + off + 8 * col);
    gin = *reinterpret_cast<const u32x4*>((grp < 2 ? q_norm : k_norm) + 8 * col);
  }
  if constexpr (ONE) Q3_DEC_LOAD_TILE_AT(w * DT, kA, vA, max_seq - 1, (max_seq - 1) & ~7);
  const int p = pos_dev ? pos_dev[b] : start;
  if constexpr (EARLY) {
    const int pc = p < 0 ? 0 : (p >= MAXPOS ? MAXPOS - 1 : p);
    const int i0 = 8 * (col & 7);
    const float* cos_row = rope_cos + (size_t)pc * ROPE_HALF + i0;
    const float* sin_row = rope_sin + (size_t)pc * ROPE_HALF + i0;
    c0 = *reinterpret_cast<const f32x4*>(cos_row);
    c1 = *reinterpret_cast<const f32x4*>(cos_row + 4);
    s0 = *reinterpret_cast<const f32x4*>(sin_row);
    s1 = *reinterpret_cast<const f32x4*>(sin_row + 4);
  }
  int n = p + 1;
  n = n < max_seq ? n : max_seq;
  n = n > 0 ? n : 0;
  const int cs = (((n + n_split - 1) / n_split) + DT - 1) & ~(DT - 1);
  const int k0 = s * cs;
  const int k1 = (k0 + cs) < n ? (k0 + cs) : n;
  const bool own = p >= k0 && p < k1;  // this split holds the new token (then p < n <= max_seq)
  const int n_tile = k1 > k0 ? (k1 - k0 + DT - 1) / DT : 0;
  const int last_key = k1 - 1, last_blk = (k1 - 1) & ~7;

#define Q3_DEC_LOAD_TILE(T, KR, VR) Q3_DEC_LOAD_TILE_AT(k0 + (T) * DT, KR, VR, last_key, last_blk)

  // a wave's tiles are w, w + NW, w + 2 NW, ...; loads past the last tile
  // re-load it (clamped), so every iteration issues the same number of loads
  auto clamp_tile = [&](int tt) { return tt < n_tile ? tt : n_tile - 1; };
  if constexpr (!ONE) {
    if (n_tile > 0) Q3_DEC_LOAD_TILE(clamp_tile(w), kA, vA);
  }

  // ---- the new token: q/k norm and rotation, v as is
  {
    float f[8];
    if constexpr (EARLY) {
      unpack_row8(xin, f);
    } else {
      const uint16_t* row = qkv + (size_t)b * QKV_N +
                            (grp < 2 ? (2 * g + grp) * D : (grp == 2 ? QDIM + g * D : QDIM + HKV * D + g * D));
      unpack_row8(*reinterpret_cast<const u32x4*>(row + 8 * col), f);
    }
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = f[e];
    if constexpr (EARLY) {
      gain_rope8(r, row_rinv8(r), gin, c0, c1, s0, s1, col);
      // computed on every lane (the v rows discard it), which keeps the
      // table loads out of a branch, where they would be issued only after
      // the norm
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(r[e]));
    } else {
      const int pc = p < 0 ? 0 : (p >= MAXPOS ? MAXPOS - 1 : p);
      norm_rope8(r, grp < 2 ? q_norm : k_norm, rope_cos + (size_t)pc * ROPE_HALF,
                 rope_sin + (size_t)pc * ROPE_HALF, col);
    }
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pk[e] = grp < 3 ? pack_bf2(r[2 * e], r[2 * e + 1]) : pack_bf2(f[2 * e], f[2 * e + 1]);
    uint16_t* dst = grp < 2 ? &qs[w][grp][0] : (grp == 2 ? &knew[w][0] : &vnew[w][0]);
    *reinterpret_cast<u32x4*>(dst + 8 * col) = pk;
    if (own && w == 0) {
      if (grp == 2) *reinterpret_cast<u32x4*>(k_cache + head_base + (size_t)p * D + 8 * col) = pk;
      if (grp == 3) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v_cache[head_base + vblk_index(p, 8 * col + 2 * e)] = (uint16_t)(pk[e] & 0xffffu);
          v_cache[head_base + vblk_index(p, 8 * col + 2 * e + 1)] = (uint16_t)(pk[e] >> 16);
        }
      }
    }
  }
  // q as the B operand (column col, heads 0 and 1 only; dims 32*st + 8*grp .. +7)
  // is re-read from LDS for every tile, which keeps registers for the K/V buffers
  const uint16_t* qsrc = &qs[w][col & 1][8 * grp];
  const bool qcol = col < 2;

  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](int t, u32x4(&ka)[8], u32x4(&va)[8]) __attribute__((always_inline)) {
    const int tb = k0 + t * DT;
    if (own && p - tb < DT) {  // the tile holding the new token: take it from LDS (wave-uniform branch)
#pragma unroll
      for (int set = 0; set < 2; ++set)
        if (tb + krel0 + 4 * set == p)
#pragma unroll
          for (int st = 0; st < 4; ++st) ka[4 * set + st] = *reinterpret_cast<const u32x4*>(&knew[w][32 * st + 8 * grp]);
      const int slot = p - tb - 8 * grp;
      if (slot >= 0 && slot < 8) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const uint32_t vbits = vnew[w][16 * db + col];
          const int e = slot >> 1;
          const uint32_t keep = (slot & 1) ? 0x0000ffffu : 0xffff0000u;
          const uint32_t put = (slot & 1) ? (vbits << 16) : vbits;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == e) va[db][q] = (va[db][q] & keep) | put;
        }
      }
    }
    const bool tail = tb + DT > k1;
    if (tail) {  // positions at or past the range end: zero V (the cache may hold anything there)
      const int valid = k1 - tb - 8 * grp;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t keep = (2 * e + 1 < valid) ? 0xffffffffu : ((2 * e < valid) ? 0x0000ffffu : 0u);
#pragma unroll
        for (int db = 0; db < 8; ++db) va[db][e] &= keep;
      }
    }
    // ---- scores of keys tb + 8*grp + j, j = 0..7, head col
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 qop = qcol ? *reinterpret_cast<const u32x4*>(qsrc + 32 * st) : u32x4{0u, 0u, 0u, 0u};
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[st]), as_bf16x8(qop), sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[4 + st]), as_bf16x8(qop), sb, 0, 0, 0);
    }
    float sv[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = sv[j] * sl2;
      if (tail && tb + 8 * grp + j >= k1) x = -INFINITY;
      sv[j] = x;
      mx = fmaxf(mx, x);
    }
    // ---- lazy online softmax: raise the running max only past the slack
    if (__ballot(col < 2 && mx > m_run + DEC_RESCALE_SLACK)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    u32x4 pb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(sv[2 * e] - m_run);
      const float p1 = __builtin_amdgcn_exp2f(sv[2 * e + 1] - m_run);
      l_run += p0 + p1;
      pb[e] = pack_bf2(p0, p1);
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 8; ++db)
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[db]), as_bf16x8(pb), oacc[db], 0, 0, 0);
  };
  // the two buffers alternate; each is refilled with the tile two steps ahead
  // as soon as it has been consumed (no register copies between iterations)
  for (int t = w; t < n_tile; t += 2 * NW) {
    Q3_DEC_LOAD_TILE(clamp_tile(t + NW), kB, vB);
    process(t, kA, vA);
    if (t + NW >= n_tile) break;
    Q3_DEC_LOAD_TILE(clamp_tile(t + 2 * NW), kA, vA);
    process(t + NW, kB, vB);
  }
#undef Q3_DEC_LOAD_TILE
#undef Q3_DEC_LOAD_TILE_AT

  // ---- combine the 4 waves: lane (grp, col < 2) holds dims 16*db + 4*grp + i of head col
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (col < 2) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[w][col][16 * db + 4 * grp + i] = oacc[db][i];
    if (grp == 0) {
      wml[w][col][0] = m_run;
      wml[w][col][1] = l_run;
    }
  }
  __syncthreads();
  // threads 0..255 finish (head hh, dim d); the others mirror them and store nothing
  const int hh = (tid >> 7) & 1, d = tid & 127;
  const bool fin = tid < 2 * D;
  {
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, wml[ww][hh][0]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = wml[ww][hh][0];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
      o += f * wo[ww][hh][d];
      lsum += f * wml[ww][hh][1];
    }
    if (n_split == 1) {  // a single split is already the whole softmax
      if (fin) out[(size_t)b * QDIM + (2 * g + hh) * D + d] = (uint16_t)f2bf(o / lsum);
      return;
    }
    if (fin) {
      float* dst = part + (((size_t)b * HQ + 2 * g + hh) * n_split + s) * PART_STRIDE;
      st_dev(dst + d, o);
      if (d == 0) {
        st_dev(dst + D, mm);
        st_dev(dst + D + 1, lsum);
      }
    }
  }

  // ---- the last split of (b, g) merges: o = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s
  vm_drain();
  __syncthreads();
  if (tid == 0) last_ticket = atomicAdd(counters + b * HKV + g, 1) == n_split - 1;
  __syncthreads();
  if (!last_ticket) return;
  if (tid < 2 * n_split) {
    const int h = tid / n_split, sp = tid - h * n_split;
    const float* src = part + (((size_t)b * HQ + 2 * g + h) * n_split + sp) * PART_STRIDE;
    mls[h][sp][0] = ld_dev(src + D);
    mls[h][sp][1] = ld_dev(src + D + 1);
  }
  __syncthreads();
  if (!fin) return;
  float mm = -INFINITY;
  for (int sp = 0; sp < n_split; ++sp) mm = fmaxf(mm, mls[hh][sp][0]);
  const float* src = part + ((size_t)b * HQ + 2 * g + hh) * n_split * PART_STRIDE + d;
  float num = 0.f, den = 0.f;
#pragma unroll 16
  for (int sp = 0; sp < n_split; ++sp) {
    const float ms = mls[hh][sp][0];
    const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - mm);
    num += f * ld_dev(src + (size_t)sp * PART_STRIDE);
    den += f * mls[hh][sp][1];
  }
  out[(size_t)b * QDIM + (2 * g + hh) * D + d] = (uint16_t)f2bf(num / den);
  if (tid == 0) counters[b * HKV + g] = 0;  // ready for the next call
}

void launch_attn_decode(const uint16_t* qkv, const uint16_t* q_norm, const uint16_t* k_norm, const float* rope_cos,
                        const float* rope_sin, uint16_t* k_cache, uint16_t* v_cache, float* part, int* counters,
                        uint16_t* out, int B, int max_seq, const int32_t* pos_dev, int start, int n_split,
                        bool streaming, hipStream_t s, const void* warm_o, const void* warm_gate_up,
                        const void* warm_down, const void* warm_qkv) {
  // streaming: caches far larger than the last-level cache, nontemporal
  // loads; otherwise ordinary loads (4-wave workgroups either way)
  // warming workgroups: whole z-slices of n_split * 8 after the B sequences
  // (so their linear ids keep j's residue modulo 8), 8 * WARM_PER_XCD or more
  const bool warm = warm_o && warm_gate_up && warm_down && warm_qkv;
  const int per_z = n_split * HKV;
  const int extra_z = warm ? (8 * WARM_PER_XCD + per_z - 1) / per_z : 0;
  const dim3 grid(n_split, HKV, B + extra_z);
#define Q3_DEC_LAUNCH(NT_, NW_, ONE_)                                                                    \
  hipLaunchKernelGGL((k_attn_decode<NT_, NW_, ONE_>), grid, dim3(64 * NW_), 0, s, qkv, q_norm, k_norm, rope_cos, \
                     rope_sin, k_cache, v_cache, part, counters, out, max_seq, pos_dev, start, n_split, B, \
                     static_cast<const uint8_t*>(warm_o), static_cast<const uint8_t*>(warm_gate_up),       \
                     static_cast<const uint8_t*>(warm_down), \
                     static_cast<const uint8_t*>(warm_qkv))
  if (streaming) {
    if (n_split == 1) Q3_DEC_LAUNCH(true, 4, true);
    else Q3_DEC_LAUNCH(true, 4, false);
  } else {
    if (n_split == 1) Q3_DEC_LAUNCH(false, 4, true);
    else Q3_DEC_LAUNCH(false, 4, false);
  }
#undef Q3_DEC_LAUNCH
}

}  // namespace q3
