// Skinny GEMM for decode-sized row counts (M <= 128 tokens):
//   out = X[M, K] * W[N, K]^T
// Bandwidth-bound on the weights, so every weight byte is read exactly once
// per call and streamed straight from HBM into MFMA operands (no LDS
// staging).  The transposed product C^T = W X^T is formed with
// v_mfma_f32_16x16x32_bf16: the A operand is 16 weight rows, the B operand
// is 16 tokens, so one MFMA row block covers 16 output features.
//
// Lane layout of the 16x16x32 MFMA (lane l, element j of the 8-wide operand):
//   A: row l%16, k-slot (l/16, j);  B: column l%16, k-slot (l/16, j);
//   C: column l%16, rows 4*(l/16) + i, i = 0..3.
// The mapping of k-slots to actual k is free as long as A and B agree; here
// k-slot (q, j) of k-step s is k = 32*s + 8*q + j, so the 4 lanes of one
// weight row read 64 contiguous bytes per step.
//
// Work split: one workgroup (4 waves) per 16 weight rows and K range
// (grid.y splits K).  The 4 waves take interleaved 32-wide k-steps, are
// reduced through LDS, and the epilogue runs once per output element.
//
// Input RMSNorm folded into the GEMM ("手写Qwen3-0.6B推理" §Qwen3RMSNorm):
// with h = gamma * r / rms(r), h W^T = (1 / rms(r)) * ((gamma * r) W^T), so
// the producer of r stores X = bf16(gamma * r) and, per 4-column group j,
// ssq[m][j] = sum of r^2 over the group; this kernel multiplies each output
// row by 1 / sqrt(sum_j ssq[m][j] / 1024 + eps) in the epilogue.
//
// Split-K with an in-kernel finish (EPI_PARTIAL with a residual): every
// workgroup stores its partial sums, and the last of the grid.y workgroups
// of a 16-column block (an atomic ticket per block) adds all of them to the
// float32 residual, and, when a gain is given, writes the next norm's
// bf16(gamma * r) and the block's sum of squares ("第 3 章" §3.2 fuses the
// residual add with the following norm in the same way).
#include "common.hpp"
#include "launch.hpp"

namespace q3 {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int XL_ELEMS = 32768;  // activation tile capacity in LDS (bf16 elements, 64 KB)

constexpr int WL_MAXK = 1024;    // longest K range whose weight tile goes through LDS

template <int NB, int RB, int EPI, int U, int WV, bool XL, bool WL>
__global__ __launch_bounds__(64 * WV) void k_gemm_skinny(SkinnyArgs a) {
  __shared__ float red[WV][RB][NB * 16][17];
  __shared__ __attribute__((aligned(16))) uint16_t xs[XL ? XL_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t wsl[WL ? RB * 16 * WL_MAXK : 8];
  __shared__ float rsc[NB * 16];
  __shared__ int last_ticket;
  const uint16_t* __restrict__ X = a.X;
  const uint16_t* __restrict__ W = a.W;
  const int M = a.M, N = a.N, K = a.K, kspan = a.kspan;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 15, qd = l >> 4;
  const int split = blockIdx.y;
  const int t = threadIdx.x;
  // norm statistics are loaded first so their latency hides behind the
  // weight stream: SG threads share a row, each reading NSQ / SG partials
  // (a.ssq_n is NSQ only for up to 8 rows, so SQV below covers both layouts)
  constexpr int SG = NB == 1 ? 16 : (NB == 2 ? 8 : (NB <= 4 ? 4 : 2));
  constexpr int SQV = NB == 1 ? NSQ / SG / 4 : NSQ_BLK / SG / 4;
  const int sqv = a.ssq_n / (SG * 4);
  const int sm = t / SG;
  f32x4 sq[SQV];
#pragma unroll
  for (int i = 0; i < SQV; ++i) sq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool scaled = a.ssq != nullptr;
  if (scaled && t < 256 && sm < M) {
    // a fixed number of loads (no per-load branch, so the compiler keeps the
    // weight loads in flight); slots past sqv reload slot 0 and are ignored
    const f32x4* sp = reinterpret_cast<const f32x4*>(a.ssq + (size_t)sm * a.ssq_ld + (t % SG) * (4 * sqv));
#pragma unroll
    for (int i = 0; i < SQV; ++i) sq[i] = sp[i < sqv ? i : 0];
  }
  const size_t k_base = (size_t)split * kspan + qd * 8;
  const uint16_t* wp[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int blk = blockIdx.x * RB + rb;  // 16-row weight block
    int wrow;
    if constexpr (EPI == EPI_SILU) {
      // rows 0..7 of a block are gate rows, 8..15 the matching up rows
      const int half = N >> 1;
      wrow = (r < 8) ? blk * 8 + r : half + blk * 8 + (r - 8);
    } else {
      wrow = blk * 16 + r;
    }
    wp[rb] = W + (size_t)wrow * K + k_base;
  }
  const uint16_t* xp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int m = nb * 16 + r;
    m = m < M ? m : M - 1;
    xp[nb] = X + (size_t)m * a.ldx + k_base;
  }
  // two accumulator sets (even / odd k-steps) halve the dependent MFMA chain
  f32x4 acc[RB][NB], acc2[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = acc2[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = kspan >> 5;  // 32-wide k-steps in this workgroup's range
  // k-step of load u: with an even U a wave takes adjacent pairs of 32-wide
  // steps, so each weight row's 128-byte lines are read whole by one wave
  auto kstep = [&](int s0, int u) {
    return (U % 2 == 0) ? (s0 - w) + 2 * ((u >> 1) * WV + w) + (u & 1) : s0 + WV * u;
  };
  if constexpr (XL || WL) {
    // Operand tiles through LDS: the weight rows (WL) and / or the
    // activation rows (XL) of this K range are copied to LDS once, with
    // direct-to-LDS loads of 1 KB of one row per instruction (16-byte chunk
    // c of row rr at slot c ^ (rr % 16), so that the 16 rows of an operand
    // read hit 16 different bank groups), all in flight together with the
    // first register loads of the other operand; the MFMAs then read their
    // staged operands from LDS.
    // Above 4 token blocks the activation tile goes through LDS in K chunks
    // of XKC columns (the whole K range otherwise).
    constexpr int XKC = (XL && NB > 4) ? XL_ELEMS / 128 : 0;
    const int kc = XKC ? XKC : kspan;
    const int cpr = kc >> 3, lcpr = 31 - __builtin_clz(cpr);  // 16-byte chunks per staged activation row
    const int cpw = kspan >> 3, lcpw = 31 - __builtin_clz(cpw);  // ... per staged weight row
    const size_t kg = (size_t)split * kspan;
    u32x4 wa[U][RB];
    u32x4 bx[U][NB];
    auto load_regs = [&](int s0) {
      if constexpr (!WL) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            wa[u][rb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp[rb] + (size_t)kstep(s0, u) * 32));
      }
      if constexpr (!XL) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            bx[u][nb] = *reinterpret_cast<const u32x4*>(xp[nb] + (size_t)kstep(s0, u) * 32);
      }
    };
    if constexpr (WL) {
      for (int base = w * 64; base < RB * 16 * cpw; base += 64 * WV) {
        const int p = base + l, rr = p >> lcpw, c = (p & (cpw - 1)) ^ (rr & 15);
        const int blk = blockIdx.x * RB + (rr >> 4), rl = rr & 15;
        int wrow;
        if constexpr (EPI == EPI_SILU)
          wrow = (rl < 8) ? blk * 8 + rl : (N >> 1) + blk * 8 + (rl - 8);
        else
          wrow = blk * 16 + rl;
        __builtin_amdgcn_global_load_lds((const void*)(W + (size_t)wrow * K + kg + 8 * c),
                                         (lds_ptr_t)(wsl + base * 8), 16, 0, 0);
      }
    }
    // one pass over the K range, or one per activation chunk: the first
    // k-step's register loads, the chunk's activation rows into LDS, then
    // the chunk's k-steps (kc / 32 of them, a multiple of WV * U)
    for (int k0 = 0; k0 < kspan; k0 += kc) {
      const int c0 = k0 >> 5;  // first k-step of the chunk
      if (k0) __syncthreads();  // every wave is done with the previous chunk
      load_regs(c0 + w);
      if constexpr (XL) {
        for (int base = w * 64; base < NB * 16 * cpr; base += 64 * WV) {
          const int p = base + l, rr = p >> lcpr, c = (p & (cpr - 1)) ^ (rr & 15);
          const int m = rr < M ? rr : M - 1;  // rows past M re-read row M - 1 (never stored)
          __builtin_amdgcn_global_load_lds((const void*)(X + (size_t)m * a.ldx + kg + k0 + 8 * c),
                                           (lds_ptr_t)(xs + base * 8), 16, 0, 0);
        }
      }
      vm_drain();
      __syncthreads();
      for (int s0 = c0 + w; s0 < c0 + (kc >> 5); s0 += WV * U) {
        if (s0 != c0 + w) load_regs(s0);
        if constexpr (WL) {
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              wa[u][rb] = *reinterpret_cast<const u32x4*>(wsl + ((rb * 16 + r) * cpw + ((4 * kstep(s0, u) + qd) ^ r)) * 8);
        }
        if constexpr (XL) {
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              bx[u][nb] = *reinterpret_cast<const u32x4*>(
                  xs + ((nb * 16 + r) * cpr + ((4 * (kstep(s0, u) - c0) + qd) ^ r)) * 8);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              f32x4& c = (u & 1) ? acc2[rb][nb] : acc[rb][nb];
              c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[u][rb]), as_bf16x8(bx[u][nb]), c, 0, 0, 0);
            }
      }
    }
  } else {
    for (int s0 = w; s0 < nsteps; s0 += WV * U) {
      u32x4 wa[U][RB];
      u32x4 bx[U][NB];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          wa[u][rb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp[rb] + (size_t)kstep(s0, u) * 32));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bx[u][nb] = *reinterpret_cast<const u32x4*>(xp[nb] + (size_t)kstep(s0, u) * 32);
      __builtin_amdgcn_sched_barrier(0);  // every load of the step is in flight before the first MFMA waits
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            f32x4& c = (u & 1) ? acc2[rb][nb] : acc[rb][nb];
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wa[u][rb]), as_bf16x8(bx[u][nb]), c, 0, 0, 0);
          }
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rb][nb] += acc2[rb][nb];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][rb][nb * 16 + r][4 * qd + i] = acc[rb][nb][i];
  if (scaled) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < SQV; ++i) ss += i < sqv ? (sq[i].x + sq[i].y) + (sq[i].z + sq[i].w) : 0.f;
    ss = group_sum_dpp<SG>(ss);
    if (t < 256 && (t % SG) == 0 && sm < NB * 16) rsc[sm] = 1.0f / sqrtf(ss * (1.0f / C) + EPS);
  }
  __syncthreads();
  if constexpr (EPI == EPI_SILU) {
    // out[m][blk*8 + j] = silu(gate) * up
    for (int e = t; e < RB * NB * 16 * 8; e += 64 * WV) {
      const int rb = e / (NB * 16 * 8), m = (e >> 3) % (NB * 16), j = e & 7;
      if (m >= M) continue;
      const float rs = scaled ? rsc[m] : 1.0f;
      float gsum = 0.f, usum = 0.f;
#pragma unroll
      for (int ww = 0; ww < WV; ++ww) {
        gsum += red[ww][rb][m][j];
        usum += red[ww][rb][m][8 + j];
      }
      gsum *= rs;
      usum *= rs;
      const float sg = gsum / (1.0f + __expf(-gsum));
      reinterpret_cast<uint16_t*>(a.out)[(size_t)m * a.ldo + (blockIdx.x * RB + rb) * 8 + j] = (uint16_t)f2bf(sg * usum);
    }
  } else {
    for (int e = t; e < RB * NB * 16 * 4; e += 64 * WV) {
      const int rb = e / (NB * 16 * 4), m = (e >> 2) % (NB * 16), ng = e & 3;
      const int blk = blockIdx.x * RB + rb;
      // whole groups of 4 lanes share (rb, m), so the shuffles below stay inside active groups
      if (m < M) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ww = 0; ww < WV; ++ww)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += red[ww][rb][m][4 * ng + i];
        if (scaled) v *= rsc[m];
        const int n = blk * 16 + 4 * ng;
        void* const out = a.out;
        const int ldo = a.ldo;
        if constexpr (EPI == EPI_BF16) {
          u32x2 o;
          o.x = pack_bf2(v[0], v[1]);
          o.y = pack_bf2(v[2], v[3]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + (size_t)m * ldo + n) = o;
        } else if constexpr (EPI == EPI_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)m * ldo + n) = v;
        } else if constexpr (EPI == EPI_ADD_F32) {
          f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)m * ldo + n);
          v = *dst + v;
          *dst = v;
          if (a.gamma) {  // the next norm's operand for this residual row (N == ldo == 1024)
            const u32x2 g = *reinterpret_cast<const u32x2*>(a.gamma + n);
            u32x2 o;
            o.x = pack_bf2(v.x * bf_lo(g.x), v.y * bf_hi(g.x));
            o.y = pack_bf2(v.z * bf_lo(g.y), v.w * bf_hi(g.y));
            *reinterpret_cast<u32x2*>(a.hg + (size_t)m * N + n) = o;
            float ss = (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
            if (a.ssq_n == NSQ) {
              a.ssq_out[(size_t)m * NSQ + 4 * blk + ng] = ss;
            } else {
              ss += __shfl_xor(ss, 1, 64);  // the 4 lanes of row m are whole and active
              ss += __shfl_xor(ss, 2, 64);
              if (ng == 0) a.ssq_out[(size_t)m * NSQ_BLK + blk] = ss;
            }
          }
        } else {  // EPI_PARTIAL (device-coherent stores: the last workgroup of the block reads them)
          float* pp = reinterpret_cast<float*>(out) + ((size_t)split * M + m) * N + n;
#pragma unroll
          for (int i = 0; i < 4; ++i) st_dev(pp + i, v[i]);
        }
      }
    }
  }
  if constexpr (EPI == EPI_PARTIAL) {
    if (a.resid == nullptr) return;
    // ticket: the last workgroup of this column range finishes it
    vm_drain();
    __syncthreads();
    if (t == 0) last_ticket = atomicAdd(a.counters + blockIdx.x, 1) == (int)gridDim.y - 1;
    __syncthreads();
    if (!last_ticket) return;
    for (int e = t; e < RB * NB * 16 * 4; e += 64 * WV) {
      const int rb = e / (NB * 16 * 4), m = (e >> 2) % (NB * 16), ng = e & 3;
      const int blk = blockIdx.x * RB + rb;
      const int n = blk * 16 + 4 * ng;
      float ss = 0.f;
      if (m < M) {
        f32x4* rp = reinterpret_cast<f32x4*>(a.resid + (size_t)m * N + n);
        f32x4 v = *rp;
        const float* pp = reinterpret_cast<const float*>(a.out) + (size_t)m * N + n;
        for (int sp = 0; sp < (int)gridDim.y; ++sp) {
          const float* q = pp + (size_t)sp * M * N;
          v += f32x4{ld_dev(q), ld_dev(q + 1), ld_dev(q + 2), ld_dev(q + 3)};
        }
        *rp = v;
        if (a.gamma) {
          const u32x2 g = *reinterpret_cast<const u32x2*>(a.gamma + n);
          u32x2 o;
          o.x = pack_bf2(v.x * bf_lo(g.x), v.y * bf_hi(g.x));
          o.y = pack_bf2(v.z * bf_lo(g.y), v.w * bf_hi(g.y));
          *reinterpret_cast<u32x2*>(a.hg + (size_t)m * N + n) = o;
          ss = (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
        }
      }
      if (a.gamma) {
        if (a.ssq_n == NSQ) {
          if (m < M) a.ssq_out[(size_t)m * NSQ + 4 * blk + ng] = ss;
        } else {
          ss += __shfl_xor(ss, 1, 64);  // groups of 4 lanes share m and are whole inside the wave
          ss += __shfl_xor(ss, 2, 64);
          if (m < M && ng == 0) a.ssq_out[(size_t)m * NSQ_BLK + blk] = ss;
        }
      }
    }
    if (t == 0) a.counters[blockIdx.x] = 0;  // ready for the next call
  }
}

// ---------------------------------------------------------------------------
// Residual projection for up to 8 rows: r[m][n] += sum_k X[m][k] W[n][k].
// One wave per output column n (4 per workgroup, N / 4 workgroups, so every
// CU streams weights); lane l reads 16 B of the weight row per 512-wide
// chunk, fully coalesced, and forms bf16 dot products with v_dot2c.  No K
// split, so the workgroup finishes its columns itself: the residual update
// and, with a gain, hg = bf16(gamma * r) and the 4-column sum of squares.
template <int MR, int NCH>
__global__ __launch_bounds__(256) void k_gemv_resid(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                    float* __restrict__ resid, int M,
                                                    const uint16_t* __restrict__ gamma, uint16_t* __restrict__ hg,
                                                    float* __restrict__ ssq_out) {
  constexpr int K = NCH * 512;
  __shared__ float rsq[4][MR];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + w;
  const uint16_t* wr = W + (size_t)n * K + 8 * l;
  u32x4 wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) wv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wr + 512 * i));
  // activation rows (rows past M re-read row M - 1 and are not stored), then
  // the residual entries and the gain of column n: all loads are issued
  // before the first is waited on, with no branch in between (a branch join
  // would make the compiler drain the weight loads first)
  u32x4 xv[MR][NCH];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const uint16_t* xr = X + (size_t)(m < M ? m : M - 1) * K + 8 * l;
#pragma unroll
    for (int i = 0; i < NCH; ++i) xv[m][i] = *reinterpret_cast<const u32x4*>(xr + 512 * i);
  }
  float rpre[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) rpre[m] = resid[(size_t)(m < M ? m : M - 1) * C + n];
  const uint16_t* gp = gamma ? gamma : W;  // (any readable address when there is no gain)
  float gpre = bf2f(gp[n]);
  // keep these loads here (the compiler would otherwise sink them into the
  // finishing lane's branch, after the reduction)
#pragma unroll
  for (int m = 0; m < MR; ++m) asm volatile("" : "+v"(rpre[m]));
  asm volatile("" : "+v"(gpre));
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    acc[m] = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[m] = dot2_bf16(wv[i][e], xv[m][i][e], acc[m]);
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = wave_sum_dpp(acc[m]);
  if (l == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m < M) {
        const float r = rpre[m] + acc[m];
        resid[(size_t)m * C + n] = r;
        if (gamma) {
          hg[(size_t)m * C + n] = (uint16_t)f2bf(r * gpre);
          rsq[w][m] = r * r;
        }
      }
    }
  }
  if (gamma) {
    __syncthreads();
    const int t = threadIdx.x;
    if (t < MR && t < M) ssq_out[(size_t)t * NSQ + blockIdx.x] = (rsq[0][t] + rsq[1][t]) + (rsq[2][t] + rsq[3][t]);
  }
}

template <int MR>
static void launch_gemv_mr(const uint16_t* X, const uint16_t* W, int K, float* resid, int M, const uint16_t* gamma,
                           uint16_t* hg, float* ssq_out, hipStream_t s) {
  const dim3 grid(C / 4), block(256);
  switch (K) {
    case 1024: hipLaunchKernelGGL((k_gemv_resid<MR, 2>), grid, block, 0, s, X, W, resid, M, gamma, hg, ssq_out); break;
    case 2048: hipLaunchKernelGGL((k_gemv_resid<MR, 4>), grid, block, 0, s, X, W, resid, M, gamma, hg, ssq_out); break;
    default: hipLaunchKernelGGL((k_gemv_resid<MR, 6>), grid, block, 0, s, X, W, resid, M, gamma, hg, ssq_out); break;
  }
}

void launch_gemv_resid(const uint16_t* X, const uint16_t* W, int K, float* resid, int M, const uint16_t* gamma,
                       uint16_t* hg, float* ssq_out, hipStream_t s) {
  if (M <= 1) launch_gemv_mr<1>(X, W, K, resid, M, gamma, hg, ssq_out, s);
  else if (M <= 2) launch_gemv_mr<2>(X, W, K, resid, M, gamma, hg, ssq_out, s);
  else if (M <= 4) launch_gemv_mr<4>(X, W, K, resid, M, gamma, hg, ssq_out, s);
  else launch_gemv_mr<8>(X, W, K, resid, M, gamma, hg, ssq_out, s);
}

template <int NB, int RB, int EPI, int WV, int U, bool XL, bool WL>
static void launch_k(const SkinnyArgs& a, int gx, int n_split, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_skinny<NB, RB, EPI, U, WV, XL, WL>), dim3(gx, n_split), dim3(64 * WV), 0, s, a);
}

// Unroll U: as many 32-wide k-steps per wave and iteration as divide the
// workgroup's range, with at most LOADS 16-byte registers of loads per lane
// in flight (PER_U per k-step: the weight rows and, straight from memory,
// the activation rows; from LDS the activation operands live briefly).
// Every caller keeps the K range a multiple of 32 * WV (q3_linear:
// K % 512 == 0; the residual projections' splits: 512-wide ranges), so the
// U = 1 kernel always fits.
template <int NB, int RB, int EPI, int WV, bool XL, bool WL>
static void launch_u(const SkinnyArgs& a, int gx, int n_split, hipStream_t s) {
  // 32-wide k-steps per workgroup, or per activation chunk (XL above 4 token blocks)
  const int nsteps = (XL && NB > 4) ? XL_ELEMS / 128 / 32 : a.kspan >> 5;
  constexpr int PER_U = (XL ? (NB + 1) / 2 : NB) + (WL ? (RB + 1) / 2 : RB);
  constexpr int LOADS = (XL || WL) ? 32 : ((RB == 1 && NB <= 2) ? 36 : 24);
  if (12 * PER_U <= LOADS && nsteps % (WV * 12) == 0)
    launch_k<NB, RB, EPI, WV, (12 * PER_U <= LOADS ? 12 : 1), XL, WL>(a, gx, n_split, s);
  else if (8 * PER_U <= LOADS && nsteps % (WV * 8) == 0)
    launch_k<NB, RB, EPI, WV, (8 * PER_U <= LOADS ? 8 : 1), XL, WL>(a, gx, n_split, s);
  else if (4 * PER_U <= LOADS && nsteps % (WV * 4) == 0)
    launch_k<NB, RB, EPI, WV, (4 * PER_U <= LOADS ? 4 : 1), XL, WL>(a, gx, n_split, s);
  else if (nsteps % (WV * 2) == 0)
    launch_k<NB, RB, EPI, WV, 2, XL, WL>(a, gx, n_split, s);
  else
    launch_k<NB, RB, EPI, WV, 1, XL, WL>(a, gx, n_split, s);
}

// XL: the activation tile of a workgroup's K range through LDS (2 to 4
// token blocks whose tile fits XL_ELEMS; 5 to 8 blocks in chunks of 256
// columns); otherwise straight from memory.
template <int NB, int RB, int EPI, int WV>
static void launch_wv(const SkinnyArgs& a, int gx, int n_split, hipStream_t s) {
  if constexpr (NB > 4) {
    launch_u<NB, RB, EPI, WV, true, false>(a, gx, n_split, s);
  } else {
    if constexpr (NB >= 2) {
      if (NB * 16 * a.kspan <= XL_ELEMS) {
        if constexpr (RB <= 2 && WV == 4 && RB * NB <= 4) {  // (both tiles and the reduction fit the LDS)
          if (a.kspan <= WL_MAXK) {
            launch_u<NB, RB, EPI, WV, true, true>(a, gx, n_split, s);
            return;
          }
        }
        launch_u<NB, RB, EPI, WV, true, false>(a, gx, n_split, s);
        return;
      }
    }
    if constexpr (NB == 1 && RB <= 2) {
      if (a.kspan <= WL_MAXK) {
        launch_u<NB, RB, EPI, WV, false, true>(a, gx, n_split, s);
        return;
      }
    }
    launch_u<NB, RB, EPI, WV, false, false>(a, gx, n_split, s);
  }
}

template <int NB, int RB, int EPI>
static void launch_rb(const SkinnyArgs& a, int n_split, hipStream_t s) {
  const int gx = ((EPI == EPI_SILU) ? (a.N / 2) / 8 : a.N / 16) / RB;
  // The residual-add projections run one K range per 16 columns, so they use
  // 8 waves per workgroup to keep enough weight bytes in flight.
  if constexpr (EPI == EPI_ADD_F32 && RB == 1) {
    if (((a.kspan >> 5) % 32) == 0) {
      launch_wv<NB, RB, EPI, 8>(a, gx, n_split, s);
      return;
    }
  }
  // Above 64 rows each k-step loads NB activation chunks per lane: 8 waves
  // spread the k-steps so that fewer rounds of loads run one after another
  // (one row block: with two, 8 waves would spill).
  if constexpr (NB > 4 && RB == 1) {
    if (((a.kspan >> 5) % 16) == 0) {
      launch_wv<NB, RB, EPI, 8>(a, gx, n_split, s);
      return;
    }
  }
  launch_wv<NB, RB, EPI, 4>(a, gx, n_split, s);
}

// 16-row weight blocks per workgroup.  Every workgroup reads the
// activation rows of its K range once, so from 16 rows on (where that read
// costs as much as the weights) more weight rows per workgroup pay off, as
// long as enough workgroups remain to keep every CU streaming: the gate|up
// projection (384 blocks) takes 2, a projection as wide as the vocabulary
// (9496 blocks, through q3_linear) takes 4 (2 above 64 rows).
static int rows_blocks(const SkinnyArgs& a, Epi epi) {
  if (a.M < 16) return 1;
  if (epi == EPI_SILU) return 2;
  if (a.N >= 16384) return 4;
  return 1;
}

template <int NB, int EPI>
static void launch_nb(const SkinnyArgs& a, int n_split, hipStream_t s) {
  switch (rows_blocks(a, static_cast<Epi>(EPI))) {
    case 4: launch_rb<NB, (NB <= 4 ? 4 : 2), EPI>(a, n_split, s); break;  // (4 x 8 blocks would spill)
    case 2: launch_rb<NB, 2, EPI>(a, n_split, s); break;
    default: launch_rb<NB, 1, EPI>(a, n_split, s); break;
  }
}

template <int EPI>
static void launch_epi(const SkinnyArgs& a, int n_split, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: launch_nb<1, EPI>(a, n_split, s); break;
    case 2: launch_nb<2, EPI>(a, n_split, s); break;
    case 3: launch_nb<3, EPI>(a, n_split, s); break;
    case 4: launch_nb<4, EPI>(a, n_split, s); break;
    case 5: launch_nb<5, EPI>(a, n_split, s); break;
    case 6: launch_nb<6, EPI>(a, n_split, s); break;
    case 7: launch_nb<7, EPI>(a, n_split, s); break;
    default: launch_nb<8, EPI>(a, n_split, s); break;
  }
}

void launch_gemm_skinny(SkinnyArgs a, int n_split, Epi epi, hipStream_t s) {
  if (a.ldx == 0) a.ldx = a.K;
  a.kspan = a.K / n_split;
  switch (epi) {
    case EPI_BF16: launch_epi<EPI_BF16>(a, n_split, s); break;
    case EPI_F32: launch_epi<EPI_F32>(a, n_split, s); break;
    case EPI_ADD_F32: launch_epi<EPI_ADD_F32>(a, n_split, s); break;
    case EPI_SILU: launch_epi<EPI_SILU>(a, n_split, s); break;
    case EPI_PARTIAL: launch_epi<EPI_PARTIAL>(a, n_split, s); break;
  }
}

void launch_gemm_skinny(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo, int n_split,
                        Epi epi, hipStream_t s) {
  SkinnyArgs a{};
  a.X = X;
  a.W = W;
  a.out = out;
  a.M = M;
  a.N = N;
  a.K = K;
  a.ldo = ldo;
  launch_gemm_skinny(a, n_split, epi, s);
}

}  // namespace q3
