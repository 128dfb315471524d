// MFMA tiled GEMM for prefill-sized row counts:  out = X[M, K] * W[N, K]^T.
//
// Both operands are K-contiguous ([rows][K] row-major), which is the native
// operand order of the MFMA unit.  The kernel forms C^T = W X^T so that the
// accumulator of v_mfma_f32_32x32x16_bf16 holds, per lane, 4 consecutive
// output features of one token; the epilogue then writes 8 B (bf16) or
// 16 B (f32) vectors.
//
// Lane layout of the 32x32x16 MFMA (lane l, element j of the 8-wide operand):
//   A: row l%32, k-slot (l/32, j);  B: column l%32, k-slot (l/32, j);
//   C: column l%32, rows 8*(i/4) + 4*(l/32) + (i%4), i = 0..15.
// k-slot (h, j) of k-step s is k = 16 s + 8 h + j.
//
// Tile: 128 (features) x 128 (tokens) x 64 (K), 4 waves as 2 x 2, each wave
// 64 x 64 = 2 x 2 MFMA blocks.  Global -> register -> LDS double buffering,
// one barrier per K step.  LDS rows are padded by 16 B.
//
// Workgroup order: consecutive workgroup ids land on different XCDs (round
// robin over 8), so ids are remapped to give each XCD a contiguous range of
// tiles, walked in groups of GM token tiles per feature tile so that the
// X row blocks and the W tile stay in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int TB_N = 128, TB_M = 128, TB_K = 64;
constexpr int T_LDS = TB_K + 8;  // padded row, bf16 elements (144 B)
constexpr int GM = 8;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_tiled(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                    void* __restrict__ out, int M, int N, int K, int ldo,
                                                    int n_tiles, int m_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][TB_N * T_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][TB_M * T_LDS];

  // ---- tile scheduling (XCD-contiguous, grouped)
  const int nwg = gridDim.x, bid = blockIdx.x;
  int logical = bid;
  if ((nwg & 7) == 0) logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int group_size = GM * n_tiles;
  const int group = logical / group_size;
  const int first_m = group * GM;
  const int gm = (m_tiles - first_m) < GM ? (m_tiles - first_m) : GM;
  const int within = logical - group * group_size;
  const int tile_m = first_m + within % gm;
  const int tile_n = within / gm;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, lh = l >> 5;
  const int wn = w >> 1, wm = w & 1;

  // ---- global load assignment: 4 chunks of 16 B per thread per operand
  const uint16_t* wsrc[4];
  const uint16_t* xsrc[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3, kc = (c & 7) * 8;
    int wrow;
    if constexpr (EPI == EPI_SILU) {
      // tile row r: wave half r/64, block (r/32)%2 (0 gate, 1 up), index r%32
      const int half = N >> 1;
      const int idx = tile_n * 64 + (row >> 6) * 32 + (row & 31);
      wrow = ((row >> 5) & 1) ? half + idx : idx;
    } else {
      wrow = tile_n * TB_N + row;
    }
    int xrow = tile_m * TB_M + row;
    xrow = xrow < M ? xrow : M - 1;
    wsrc[i] = W + (size_t)wrow * K + kc;
    xsrc[i] = X + (size_t)xrow * K + kc;
    lds_off[i] = row * T_LDS + kc;
  }

  u32x4 wreg[4], xreg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wreg[i] = *reinterpret_cast<const u32x4*>(wsrc[i]);
    xreg[i] = *reinterpret_cast<const u32x4*>(xsrc[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<u32x4*>(&Ws[0][lds_off[i]]) = wreg[i];
    *reinterpret_cast<u32x4*>(&Xs[0][lds_off[i]]) = xreg[i];
  }
  __syncthreads();

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int nk = K / TB_K;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wreg[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + (kt + 1) * TB_K);
        xreg[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + (kt + 1) * TB_K);
      }
    }
    const uint16_t* wsb = Ws[cur];
    const uint16_t* xsb = Xs[cur];
#pragma unroll
    for (int s = 0; s < TB_K / 16; ++s) {
      u32x4 av[2], bv[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        av[nb] = *reinterpret_cast<const u32x4*>(&wsb[(wn * 64 + nb * 32 + lq) * T_LDS + 16 * s + 8 * lh]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        bv[mb] = *reinterpret_cast<const u32x4*>(&xsb[(wm * 64 + mb * 32 + lq) * T_LDS + 16 * s + 8 * lh]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[nb]), as_bf16x8(bv[mb]), acc[nb][mb], 0, 0, 0);
    }
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(&Ws[cur ^ 1][lds_off[i]]) = wreg[i];
        *reinterpret_cast<u32x4*>(&Xs[cur ^ 1][lds_off[i]]) = xreg[i];
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds features 8*(i/4) + 4*lh + (i%4) of token lq in each block
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = tile_m * TB_M + wm * 64 + mb * 32 + lq;
    if (m >= M) continue;
    if constexpr (EPI == EPI_SILU) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = acc[0][mb][4 * g + i], up = acc[1][mb][4 * g + i];
          v[i] = gt / (1.0f + __expf(-gt)) * up;
        }
        const int n = tile_n * 64 + wn * 32 + 8 * g + 4 * lh;
        u32x2 o;
        o.x = pack_bf2(v[0], v[1]);
        o.y = pack_bf2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + (size_t)m * ldo + n) = o;
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = tile_n * TB_N + wn * 64 + nb * 32 + 8 * g + 4 * lh;
          f32x4 v = {acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3]};
          if constexpr (EPI == EPI_BF16) {
            u32x2 o;
            o.x = pack_bf2(v[0], v[1]);
            o.y = pack_bf2(v[2], v[3]);
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + (size_t)m * ldo + n) = o;
          } else if constexpr (EPI == EPI_F32) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)m * ldo + n) = v;
          } else {  // EPI_ADD_F32
            f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)m * ldo + n);
            *dst = *dst + v;
          }
        }
    }
  }
}

void launch_gemm_tiled(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo, Epi epi,
                       hipStream_t s) {
  const int m_tiles = (M + TB_M - 1) / TB_M;
  const int n_tiles = (epi == EPI_SILU) ? (N / 2) / 64 : N / TB_N;
  const dim3 grid(m_tiles * n_tiles), block(256);
  switch (epi) {
    case EPI_BF16: hipLaunchKernelGGL(k_gemm_tiled<EPI_BF16>, grid, block, 0, s, X, W, out, M, N, K, ldo, n_tiles, m_tiles); break;
    case EPI_F32: hipLaunchKernelGGL(k_gemm_tiled<EPI_F32>, grid, block, 0, s, X, W, out, M, N, K, ldo, n_tiles, m_tiles); break;
    case EPI_ADD_F32: hipLaunchKernelGGL(k_gemm_tiled<EPI_ADD_F32>, grid, block, 0, s, X, W, out, M, N, K, ldo, n_tiles, m_tiles); break;
    case EPI_SILU: hipLaunchKernelGGL(k_gemm_tiled<EPI_SILU>, grid, block, 0, s, X, W, out, M, N, K, ldo, n_tiles, m_tiles); break;
    default: break;
  }
}

}  // namespace q3
