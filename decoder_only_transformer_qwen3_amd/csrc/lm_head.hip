// Tied lm_head for up to 64 rows (decode, and the last rows of a prefill):
//   logits[m][n] = (1 / rms(r_m)) * sum_k X[m][k] E[n][k],   n < 151936,
// with X = bf16(gamma_final * r) and the per-row sums of squares of r (the
// final RMSNorm folded into the product, "手写Qwen3-0.6B推理" §Qwen3Model
// applies the norm and then the tied embedding), and the greedy token of
// each row ("第 3 章" §4.3; lowest index among equal maxima, NaN first).
//
// The 311 MB embedding is the whole cost, so the kernel is a persistent
// stream over it: one workgroup per CU, eight waves, each wave owning whole
// 16-row blocks (all of K, so no cross-wave reduction) and keeping the next
// block's 32 KB of weight loads in flight while it multiplies the current
// one.  The activation rows are read once per workgroup into LDS, where
// every MFMA takes its B operand (16-byte chunks XOR-swizzled by row, so the
// 16 rows of an operand read hit 16 different bank groups).
//
// Greedy choice: each wave keeps its rows' best (value, index) over its
// blocks, the workgroup combines its waves in LDS and stores one candidate
// per row with device-coherent stores; the last workgroup to finish (an
// atomic ticket) combines the candidates of all workgroups and writes the
// token and the sequence length.  The order is a total order, so the token
// does not depend on how the candidates were grouped.
//
// v_mfma_f32_16x16x32_bf16, C^T = E X^T: A = 16 embedding rows (lane l: row
// l%16, k 32s + 8(l/16) .. +7), B = 16 activation rows with the same k
// slots, C lane l: activation row l%16, embedding rows 4(l/16) + i.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int LH_WAVES = 8;
constexpr int LH_KSTEPS = C / 32;         // 32-wide k-steps per block
constexpr int LH_CHUNK = 8;               // k-steps per load group
constexpr int LH_NCHUNK = LH_KSTEPS / LH_CHUNK;
constexpr int LH_RING = 2;                   // chunks of weight loads in flight per wave (4 measured no faster)
constexpr int LH_BLOCKS = V / 16;         // 9496 blocks of 16 embedding rows

template <int NB>
__global__ __launch_bounds__(64 * LH_WAVES, 1) void k_lm_head(const uint16_t* __restrict__ X, int ldx,
                                                               const float* __restrict__ ssq, int ssq_ld, int ssq_n,
                                                               const uint16_t* __restrict__ E, float* __restrict__ out,
                                                               int ldo, uint64_t* __restrict__ cand, int M,
                                                               int* __restrict__ ticket, HeadPick pick) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[NB * 16 * C];
  __shared__ float rsc[NB * 16];
  __shared__ float bsv[LH_WAVES][NB * 16];
  __shared__ int bsi[LH_WAVES][NB * 16];
  __shared__ int last_ticket;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, r = l & 15, qd = l >> 4;

  // ---- activation rows into LDS (rows past M are zero), chunk c of row
  // rr at c ^ (rr % 16); the reciprocal RMS of each row
  for (int e = t; e < NB * 16 * (C / 8); e += 64 * LH_WAVES) {
    const int rr = e / (C / 8), c = e % (C / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (rr < M) v = *reinterpret_cast<const u32x4*>(X + (size_t)rr * ldx + 8 * c);
    *reinterpret_cast<u32x4*>(xs + rr * C + 8 * (c ^ (rr & 15))) = v;
  }
  {
    // 8 threads per row, each summing ssq_n / 8 partials
    const int rr = t >> 3, part = t & 7;
    float s = 0.f;
    if (ssq && rr < NB * 16 && rr < M) {
      const int per = ssq_n / 8;
      const float* sp = ssq + (size_t)rr * ssq_ld + part * per;
      for (int i = 0; i < per; i += 4) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(sp + i);
        s += (q.x + q.y) + (q.z + q.w);
      }
    }
    s = group_sum_dpp<8>(s);
    if (part == 0 && rr < NB * 16) rsc[rr] = ssq ? 1.0f / sqrtf(s * (1.0f / C) + EPS) : 1.0f;
  }
  __syncthreads();

  // ---- this wave's blocks: the workgroup's contiguous range, round-robin over its waves
  const int b0 = (int)(((long long)blockIdx.x * LH_BLOCKS) / gridDim.x);
  const int b1 = (int)(((long long)(blockIdx.x + 1) * LH_BLOCKS) / gridDim.x);
  const int nblk = b1 - b0 > w ? (b1 - b0 - w + LH_WAVES - 1) / LH_WAVES : 0;
  auto blk_of = [&](int i) { return b0 + w + LH_WAVES * i; };

  // B-operand LDS offsets of k-step s: row 16 nb + r, chunk 4 s + qd (swizzled)
  const uint16_t* xrow = xs + r * C;
  auto xread = [&](int nb, int s) {
    return *reinterpret_cast<const u32x4*>(xrow + nb * 16 * C + 8 * ((4 * s + qd) ^ r));
  };
  // weight loads of chunk c (8 k-steps) of block b: lane reads row r, k 32 s + 8 qd
  auto wload = [&](u32x4(&dst)[LH_CHUNK], int b, int c) {
    const uint16_t* wp = E + ((size_t)b * 16 + r) * C + 8 * qd + 32 * LH_CHUNK * c;
#pragma unroll
    for (int s = 0; s < LH_CHUNK; ++s) dst[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + 32 * s));
  };

  // LH_RING chunks of weight loads in flight (8 KB per wave each): chunk c of
  // a block lives in wb[c % LH_RING]; once it is multiplied, its registers take
  // chunk c + LH_RING (of the same block, or of the next one).
  u32x4 wb[LH_RING][LH_CHUNK];
  if (nblk > 0) {
#pragma unroll
    for (int c = 0; c < LH_RING; ++c) wload(wb[c], blk_of(0), c);
  }
  // this wave's best (value, index) per row over its blocks
  float rv[NB];
  int ri[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    rv[nb] = -INFINITY;
    ri[nb] = 0x7fffffff;
  }

  for (int i = 0; i < nblk; ++i) {
    const int blk = blk_of(i), nxt = blk_of(i + 1);
    const bool more = i + 1 < nblk;
    f32x4 acc[NB], acc2[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = acc2[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < LH_NCHUNK; ++c) {
      u32x4(&wc)[LH_CHUNK] = wb[c % LH_RING];
      // B operands one k-step ahead of their MFMAs
      u32x4 xb[2][NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) xb[0][nb] = xread(nb, LH_CHUNK * c);
#pragma unroll
      for (int st = 0; st < LH_CHUNK; ++st) {
        if (st + 1 < LH_CHUNK) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) xb[(st + 1) & 1][nb] = xread(nb, LH_CHUNK * c + st + 1);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x4& a = (st & 1) ? acc2[nb] : acc[nb];
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wc[st]), as_bf16x8(xb[st & 1][nb]), a, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c + LH_RING < LH_NCHUNK)
        wload(wc, blk, c + LH_RING);
      else if (more)
        wload(wc, nxt, c + LH_RING - LH_NCHUNK);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- epilogue: scale, store the logits, the block's (max, argmax) per row
    const int n = blk * 16 + 4 * qd;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int m = nb * 16 + r;
      f32x4 v = (acc[nb] + acc2[nb]) * rsc[m];
      float bv = v[0];
      int bi = n;
#pragma unroll
      for (int e = 1; e < 4; ++e)
        if (am_better(v[e], n + e, bv, bi)) {
          bv = v[e];
          bi = n + e;
        }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (am_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (am_better(bv, bi, rv[nb], ri[nb])) {
        rv[nb] = bv;
        ri[nb] = bi;
      }
      if (out && m < M) *reinterpret_cast<f32x4*>(out + (size_t)m * ldo + n) = v;
    }
  }

  // ---- the workgroup's candidate per row (lanes of equal r hold equal values)
  if (qd == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bsv[w][nb * 16 + r] = rv[nb];
      bsi[w][nb * 16 + r] = ri[nb];
    }
  }
  __syncthreads();
  if (t < M) {
    float bv = bsv[0][t];
    int bi = bsi[0][t];
#pragma unroll
    for (int ww = 1; ww < LH_WAVES; ++ww)
      if (am_better(bsv[ww][t], bsi[ww][t], bv, bi)) {
        bv = bsv[ww][t];
        bi = bsi[ww][t];
      }
    st_dev_u64(cand + (size_t)blockIdx.x * M + t, ((uint64_t)(uint32_t)bi << 32) | __float_as_uint(bv));
  }
  vm_drain();
  __syncthreads();
  if (t == 0) last_ticket = atomicAdd(ticket, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!last_ticket) return;
  // ---- last workgroup: row m's candidates over all workgroups, one wave per row
  for (int m = w; m < M; m += LH_WAVES) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int g = l; g < (int)gridDim.x; g += 64) {
      const uint64_t c = ld_dev_u64(cand + (size_t)g * M + m);
      const float cv = __uint_as_float((uint32_t)c);
      const int ci = (int)(uint32_t)(c >> 32);
      if (am_better(cv, ci, bv, bi)) {
        bv = cv;
        bi = ci;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (am_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (l == 0)
      am_finish(pick.r0 + m, bi, pick.out_idx, pick.seq_lens, pick.seq_mode, pick.seq_val, pick.in_ids, pick.eos,
                &pick.sm);
  }
  if (t == 0) *ticket = 0;  // ready for the next call
}

void launch_lm_head(const SkinnyArgs& a, const HeadPick& pick, int* ticket, hipStream_t s) {
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 256;
  const dim3 grid(n_cu > 0 ? n_cu : 256), block(64 * LH_WAVES);
  const int ldx = a.ldx ? a.ldx : C;
  uint64_t* cand = static_cast<uint64_t*>(a.amax_part);
  float* out = static_cast<float*>(a.out);
#define Q3_LH_LAUNCH(NB_)                                                                                      \
  hipLaunchKernelGGL(k_lm_head<NB_>, grid, block, 0, s, a.X, ldx, a.ssq, a.ssq_ld, a.ssq_n, a.W, out, a.ldo, cand, \
                     a.M, ticket, pick)
  switch ((a.M + 15) / 16) {
    case 1: Q3_LH_LAUNCH(1); break;
    case 2: Q3_LH_LAUNCH(2); break;
    case 3: Q3_LH_LAUNCH(3); break;
    default: Q3_LH_LAUNCH(4); break;
  }
#undef Q3_LH_LAUNCH
}

}  // namespace q3
