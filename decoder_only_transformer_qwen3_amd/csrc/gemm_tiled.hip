// MFMA tiled GEMM for prefill-sized row counts:  out = X[M, K] * W[N, K]^T.
//
// Both operands are K-contiguous ([rows][K] row-major), which is the native
// operand order of the MFMA unit.  The kernel forms C^T = W X^T so that the
// accumulator of v_mfma_f32_32x32x16_bf16 holds, per lane, 4 consecutive
// output features of one token.  The bf16 epilogues trade groups between
// the two half-waves (lane l and l + 32 hold adjacent groups of the same
// token) and write 16 B per lane; the fp32 residual add reads a batch of
// rows before it writes any of them.
//
// Lane layout of the 32x32x16 MFMA (lane l, element j of the 8-wide operand):
//   A: row l%32, k-slot (l/32, j);  B: column l%32, k-slot (l/32, j);
//   C: column l%32, rows 8*(i/4) + 4*(l/32) + (i%4), i = 0..15.
// k-slot (h, j) of k-step s is k = 16 s + 8 h + j.
//
// Tile: 4 waves as 2 x 2; each wave owns WN x WM MFMA blocks of 32 x 32
// (features x tokens), so the workgroup tile is 64 WN x 64 WM with K steps
// of 64 (launched with WN = WM = 2).  Global -> register -> LDS double
// buffering, one barrier per K step, LDS rows padded by 16 B.
//
// Workgroup order: consecutive workgroup ids land on different XCDs (round
// robin over 8), so ids are remapped to give each XCD a contiguous range of
// tiles, walked in groups of GM token tiles per feature tile so that the
// X row blocks and the W tile stay in that XCD's L2.
#include "common.hpp"
#include "launch.hpp"

namespace q3 {

// row[b * 32 + 8 j + 4 h .. + 3] += group j of block(b) for NB blocks.  All
// loads are issued before the first store: the compiler keeps the program
// order of accesses that may alias, so interleaved load-add-store would wait
// a full memory round trip per 16 bytes.
template <int NB, typename Block>
__device__ __forceinline__ void add_blocks_f32(float* row, Block block, int lh) {
  f32x4 r[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) r[b][g] = *reinterpret_cast<const f32x4*>(row + b * 32 + 8 * g + 4 * lh);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& a = block(b);
      r[b][g] += f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
      *reinterpret_cast<f32x4*>(row + b * 32 + 8 * g + 4 * lh) = r[b][g];
    }
}

constexpr int TB_K = 64;
constexpr int T_LDS = TB_K + 8;  // padded row, bf16 elements (144 B)
constexpr int GM = 8;

template <int EPI, int WN, int WM>
__global__ __launch_bounds__(256, (WN * WM > 4) ? 1 : 2) void k_gemm_tiled(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ out, int M, int N, int K,
    int ldo, int n_tiles, int m_tiles, int n_split, float* __restrict__ part) {
  constexpr int BN = 64 * WN, BM = 64 * WM;
  constexpr int W_CHUNKS = BN * TB_K / 8 / 256;  // 16 B chunks per thread
  constexpr int X_CHUNKS = BM * TB_K / 8 / 256;
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * T_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][BM * T_LDS];

  // ---- tile scheduling (XCD-contiguous, grouped); workgroup bid takes K
  // split bid / tiles of tile bid % tiles
  const int nwg = m_tiles * n_tiles;
  const int split = blockIdx.x / nwg, bid = blockIdx.x - split * nwg;
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
  const int k_begin = split * (K / n_split);

  // ---- global load assignment
  const uint16_t* wsrc[W_CHUNKS];
  const uint16_t* xsrc[X_CHUNKS];
  int wlds[W_CHUNKS], xlds[X_CHUNKS];
#pragma unroll
  for (int i = 0; i < W_CHUNKS; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3, kc = (c & 7) * 8;
    int wrow;
    if constexpr (EPI == EPI_SILU) {
      // tile row r: wave half r/(32 WN), block b = (r/32) % WN; blocks < WN/2 are gate rows,
      // the others the up rows of the same intermediate indices
      const int half = N >> 1;
      const int wh = row / (32 * WN), blk = (row >> 5) % WN;
      const int idx = tile_n * (BN / 2) + wh * (16 * WN) + (blk % (WN / 2)) * 32 + (row & 31);
      wrow = (blk >= WN / 2) ? half + idx : idx;
    } else {
      wrow = tile_n * BN + row;
    }
    wsrc[i] = W + (size_t)wrow * K + k_begin + kc;
    wlds[i] = row * T_LDS + kc;
  }
#pragma unroll
  for (int i = 0; i < X_CHUNKS; ++i) {
    const int c = tid + 256 * i;
    const int row = c >> 3, kc = (c & 7) * 8;
    int xrow = tile_m * BM + row;
    xrow = xrow < M ? xrow : M - 1;
    xsrc[i] = X + (size_t)xrow * K + k_begin + kc;
    xlds[i] = row * T_LDS + kc;
  }

  u32x4 wreg[W_CHUNKS], xreg[X_CHUNKS];
#pragma unroll
  for (int i = 0; i < W_CHUNKS; ++i) wreg[i] = *reinterpret_cast<const u32x4*>(wsrc[i]);
#pragma unroll
  for (int i = 0; i < X_CHUNKS; ++i) xreg[i] = *reinterpret_cast<const u32x4*>(xsrc[i]);
#pragma unroll
  for (int i = 0; i < W_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&Ws[0][wlds[i]]) = wreg[i];
#pragma unroll
  for (int i = 0; i < X_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&Xs[0][xlds[i]]) = xreg[i];
  __syncthreads();

  f32x16 acc[WN][WM];
#pragma unroll
  for (int a = 0; a < WN; ++a)
#pragma unroll
    for (int b = 0; b < WM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  const int nk = K / TB_K / n_split;
  constexpr int NS = TB_K / 16;  // MFMA k-steps per K tile
  // operand registers, double-buffered across k-steps so the LDS reads of
  // step s+1 are in flight while step s's MFMAs issue
  u32x4 av[2][WN], bv[2][WM];
  auto read_ops = [&](const uint16_t* wsb, const uint16_t* xsb, int s, int slot) {
#pragma unroll
    for (int nb = 0; nb < WN; ++nb)
      av[slot][nb] = *reinterpret_cast<const u32x4*>(&wsb[(wn * 32 * WN + nb * 32 + lq) * T_LDS + 16 * s + 8 * lh]);
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
      bv[slot][mb] = *reinterpret_cast<const u32x4*>(&xsb[(wm * 32 * WM + mb * 32 + lq) * T_LDS + 16 * s + 8 * lh]);
  };
  read_ops(Ws[0], Xs[0], 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
#pragma unroll
      for (int i = 0; i < W_CHUNKS; ++i) wreg[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + (kt + 1) * TB_K);
#pragma unroll
      for (int i = 0; i < X_CHUNKS; ++i) xreg[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + (kt + 1) * TB_K);
    }
    const uint16_t* wsb = Ws[cur];
    const uint16_t* xsb = Xs[cur];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int slot = s & 1;
      if (s + 1 < NS) read_ops(wsb, xsb, s + 1, slot ^ 1);
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int mb = 0; mb < WM; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[slot][nb]), as_bf16x8(bv[slot][mb]),
                                                                acc[nb][mb], 0, 0, 0);
      if (s == NS / 2 - 1 && more) {
        // the other buffer was last read before the previous barrier: fill it now,
        // overlapping the LDS writes with the remaining k-steps
#pragma unroll
        for (int i = 0; i < W_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&Ws[cur ^ 1][wlds[i]]) = wreg[i];
#pragma unroll
        for (int i = 0; i < X_CHUNKS; ++i) *reinterpret_cast<u32x4*>(&Xs[cur ^ 1][xlds[i]]) = xreg[i];
      }
    }
    __syncthreads();
    if (more) read_ops(Ws[cur ^ 1], Xs[cur ^ 1], 0, 0);
  }

  if (n_split > 1) {
    // K split: store this split's fp32 sums at [split][m][W row]; a reduce
    // kernel adds the splits in order and applies the epilogue
    float* pp = part + (size_t)split * M * N;
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
      const int m = tile_m * BM + wm * 32 * WM + mb * 32 + lq;
      if (m >= M) continue;
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          int wrow;
          if constexpr (EPI == EPI_SILU) {
            const int idx = tile_n * (BN / 2) + wn * (16 * WN) + (nb % (WN / 2)) * 32 + 8 * g + 4 * lh;
            wrow = (nb >= WN / 2) ? (N >> 1) + idx : idx;
          } else {
            wrow = tile_n * BN + wn * 32 * WN + nb * 32 + 8 * g + 4 * lh;
          }
          *reinterpret_cast<f32x4*>(pp + (size_t)m * N + wrow) =
              f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3]};
        }
    }
    return;
  }

  // ---- epilogue: lane holds features 8*(i/4) + 4*lh + (i%4) of token lq in each block
#pragma unroll
  for (int mb = 0; mb < WM; ++mb) {
    const int m = tile_m * BM + wm * 32 * WM + mb * 32 + lq;
    if (m >= M) continue;
    if constexpr (EPI == EPI_SILU) {
#pragma unroll
      for (int nb = 0; nb < WN / 2; ++nb) {
        f32x16 v;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float gt = acc[nb][mb][i], up = acc[nb + WN / 2][mb][i];
          v[i] = gt / (1.0f + __expf(-gt)) * up;
        }
        store_block_bf16(reinterpret_cast<uint16_t*>(out) + (size_t)m * ldo + tile_n * (BN / 2) + wn * (16 * WN) +
                             nb * 32,
                         v, lh);
      }
    } else if constexpr (EPI == EPI_BF16) {
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
        store_block_bf16(reinterpret_cast<uint16_t*>(out) + (size_t)m * ldo + tile_n * BN + wn * 32 * WN + nb * 32,
                         acc[nb][mb], lh);
    } else if constexpr (EPI == EPI_F32) {
#pragma unroll
      for (int nb = 0; nb < WN; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = tile_n * BN + wn * 32 * WN + nb * 32 + 8 * g + 4 * lh;
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)m * ldo + n) =
              f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3]};
        }
    } else {  // EPI_ADD_F32
      add_blocks_f32<WN>(reinterpret_cast<float*>(out) + (size_t)m * ldo + tile_n * BN + wn * 32 * WN,
                         [&](int b) -> const f32x16& { return acc[b][mb]; }, lh);
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M variant: persistent workgroups fed by direct-to-LDS loads
// (global_load_lds_dwordx4).  One workgroup per CU walks a list of 256 x 256
// tiles; a 2-stage LDS ring of K = 64 slices runs continuously across tile
// boundaries (one slice in flight while the other is consumed, one barrier
// per 4 MFMA k-steps), so the next tile's first loads overlap the current
// tile's epilogue and no registers are spent on staging.  Each DMA
// instruction fills 1 KB of LDS contiguously (lane i -> bytes 16 i), so rows
// are not padded; instead the eight 16-byte chunks of each 128-byte row are
// XOR-swizzled by (row / 2) % 8, which keeps the 32-row MFMA operand reads
// free of bank conflicts (16 lanes on 16 rows hit 16 different bank groups).
//
// 8 waves as 2 (features) x 4 (tokens), each owning 4 x 2 MFMA blocks of
// 32 x 32 (128 features of 64 tokens), i.e. two waves per SIMD.  A wave's
// epilogue covers 512 contiguous bytes of each fp32 output row, which made
// the residual-add projections 5-10 % faster than 64-feature wave tiles
// (same operand reads and MFMAs per k-step).  Tiles are dealt out XCD-contiguously:
// the 32 workgroups on one XCD process consecutive tiles in the grouped
// order, which keeps their X and W panels in that XCD's L2.
constexpr int DK = 64;        // K per stage
constexpr int DSTAGES = 2;
constexpr int DKS = DK / 16;  // MFMA k-steps per stage
constexpr int DROWS = 256;    // rows per operand tile
constexpr int DSTAGE_ELEMS = DROWS * DK;  // bf16 per operand per stage (32 KB)
constexpr int PWG_XCD = 32;   // persistent workgroups per XCD (one per CU)

__device__ __forceinline__ int dswz(int row, int chunk) { return row * DK + ((chunk ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ float silu_mul(float g, float u) {
  // silu(g) * u = g * u / (1 + e^-g), with the hardware exp2 and reciprocal
  return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void k_gemm_persist(const uint16_t* __restrict__ X,
                                                         const uint16_t* __restrict__ W,
                                                         void* __restrict__ out, int M, int N, int K, int ldo,
                                                         int n_tiles, int m_tiles, int per_xcd) {
  constexpr int WGN = 2, WGM = 4, NWAVES = 8;
  constexpr int BN = 256, BM = 256;
  constexpr int WN = BN / 32 / WGN, WM = BM / 32 / WGM;  // 4 x 2 blocks per wave
  constexpr int DMA_PER_WAVE = (DSTAGE_ELEMS * 2 / 1024) / NWAVES;  // 1 KB DMAs per operand per stage per wave
  __shared__ __attribute__((aligned(1024))) uint16_t Ls[DSTAGES][2][DSTAGE_ELEMS];  // [stage][W, X]

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 31, lh = l >> 5;
  const int wn = w / WGM, wm = w % WGM;
  const int total = m_tiles * n_tiles;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int first = xcd * per_xcd + slot;
  const int lim = ((xcd + 1) * per_xcd) < total ? ((xcd + 1) * per_xcd) : total;
  const int my_tiles = first < lim ? (lim - first + PWG_XCD - 1) / PWG_XCD : 0;
  if (my_tiles == 0) return;  // workgroup-uniform
  const int nk = K / DK;
  const int n_stages = my_tiles * nk;

  auto tile_coords = [&](int i, int& tm, int& tn) {
    const int logical = first + PWG_XCD * i;
    const int group_size = GM * n_tiles;
    const int group = logical / group_size;
    const int first_m = group * GM;
    const int gm = (m_tiles - first_m) < GM ? (m_tiles - first_m) : GM;
    const int within = logical - group * group_size;
    tm = first_m + within % gm;
    tn = within / gm;
  };
  // DMA sources of this lane: wave w, instruction i fills LDS rows 8 (4 w + i) .. +7;
  // lane l writes row 8 (.) + l / 8, slot l % 8, which holds logical chunk (l % 8) ^ swizzle.
  auto set_src = [&](int i_tile, const uint16_t* (&ws)[DMA_PER_WAVE], const uint16_t* (&xs)[DMA_PER_WAVE]) {
    int tm, tn;
    tile_coords(i_tile, tm, tn);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int row = 8 * (DMA_PER_WAVE * w + i) + (l >> 3);
      const int chunk = (l & 7) ^ ((row >> 1) & 7);
      int wrow;
      if constexpr (EPI == EPI_SILU) {
        const int half = N >> 1;
        const int wh = row / (32 * WN), blk = (row >> 5) % WN;
        const int idx = tn * (BN / 2) + wh * (16 * WN) + (blk % (WN / 2)) * 32 + (row & 31);
        wrow = (blk >= WN / 2) ? half + idx : idx;
      } else {
        wrow = tn * BN + row;
      }
      int xrow = tm * BM + row;
      xrow = xrow < M ? xrow : M - 1;
      ws[i] = W + (size_t)wrow * K + chunk * 8;
      xs[i] = X + (size_t)xrow * K + chunk * 8;
    }
  };
  // issue state: the next stage to load, its tile and k index
  const uint16_t* iw[DMA_PER_WAVE];
  const uint16_t* ix[DMA_PER_WAVE];
  int is_tile = 0, is_k = 0, is_g = 0;
  set_src(0, iw, ix);
  auto issue_next = [&]() {
    // past the last stage, re-load the last one into the free buffer (keeps wait counts uniform)
    const int kk = is_g < n_stages ? is_k : nk - 1;
    const int st = is_g % DSTAGES;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(iw[i] + kk * DK),
                                       (__attribute__((address_space(3))) void*)&Ls[st][0][(DMA_PER_WAVE * w + i) * 512],
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(ix[i] + kk * DK),
                                       (__attribute__((address_space(3))) void*)&Ls[st][1][(DMA_PER_WAVE * w + i) * 512],
                                       16, 0, 0);
    }
    ++is_g;
    if (is_g < n_stages && ++is_k == nk) {
      is_k = 0;
      ++is_tile;
      set_src(is_tile, iw, ix);
    }
  };

  f32x16 acc[WN][WM];
  auto zero_acc = [&]() {
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
      for (int b = 0; b < WM; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
  };
  u32x4 ra0[WN], rb0[WM], ra1[WN], rb1[WM];
  auto rd = [&](int g, int s, u32x4* ra, u32x4* rb) {
    const uint16_t* wsb = Ls[g % DSTAGES][0];
    const uint16_t* xsb = Ls[g % DSTAGES][1];
#pragma unroll
    for (int nb = 0; nb < WN; ++nb)
      ra[nb] = *reinterpret_cast<const u32x4*>(&wsb[dswz(wn * 32 * WN + nb * 32 + lq, 2 * s + lh)]);
#pragma unroll
    for (int mb = 0; mb < WM; ++mb)
      rb[mb] = *reinterpret_cast<const u32x4*>(&xsb[dswz(wm * 32 * WM + mb * 32 + lq, 2 * s + lh)]);
  };
  auto mm = [&](const u32x4* ra, const u32x4* rb) {
#pragma unroll
    for (int nb = 0; nb < WN; ++nb)
#pragma unroll
      for (int mb = 0; mb < WM; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ra[nb]), as_bf16x8(rb[mb]), acc[nb][mb], 0,
                                                              0, 0);
  };
  auto epilogue = [&](int i_tile) {
    int tm, tn;
    tile_coords(i_tile, tm, tn);
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
      const int m = tm * BM + wm * 32 * WM + mb * 32 + lq;
      if (m >= M) continue;
      if constexpr (EPI == EPI_SILU) {
#pragma unroll
        for (int nb = 0; nb < WN / 2; ++nb) {
          const f32x16& ga = acc[nb][mb];
          const f32x16& ua = acc[nb + WN / 2][mb];
          f32x16 v;
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = silu_mul(ga[i], ua[i]);
          store_block_bf16(reinterpret_cast<uint16_t*>(out) + (size_t)m * ldo + tn * (BN / 2) + wn * (16 * WN) +
                               nb * 32,
                           v, lh);
        }
      } else if constexpr (EPI == EPI_BF16) {
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
          store_block_bf16(reinterpret_cast<uint16_t*>(out) + (size_t)m * ldo + tn * BN + wn * 32 * WN + nb * 32,
                           acc[nb][mb], lh);
      } else if constexpr (EPI == EPI_F32) {
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = tn * BN + wn * 32 * WN + nb * 32 + 8 * g + 4 * lh;
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)m * ldo + n) =
                f32x4{acc[nb][mb][4 * g], acc[nb][mb][4 * g + 1], acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3]};
          }
      } else {  // EPI_ADD_F32: two blocks (32 registers of residual) per batch
        float* row = reinterpret_cast<float*>(out) + (size_t)m * ldo + tn * BN + wn * 32 * WN;
#pragma unroll
        for (int q = 0; q < WN / 2; ++q) {
          add_blocks_f32<2>(row + 64 * q, [&](int b) -> const f32x16& { return acc[2 * q + b][mb]; }, lh);
        }
      }
    }
  };

  // Prologue: stages 0 and 1 into both buffers, then wait for stage 0 (stage
  // 1's 8 DMAs per wave may still be in flight) and a plain barrier: no
  // fence, since each wave has waited for its own DMA writes and a fenced
  // __syncthreads would wait for every stage in flight.
  for (int p = 0; p < DSTAGES; ++p) issue_next();
  static_assert(2 * DMA_PER_WAVE == 8, "wait count below");
  __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
  __builtin_amdgcn_s_barrier();
  zero_acc();
  rd(0, 0, ra0, rb0);
  int kt = 0, tile = 0;
  auto stage_body = [&](int g) {
    // k-steps 0 .. DKS-2 of stage g, each with the next step's operand reads in flight
#pragma unroll
    for (int ks = 1; ks < DKS; ++ks) {
      if (ks & 1) {
        rd(g, ks, ra1, rb1);
        mm(ra0, rb0);
      } else {
        rd(g, ks, ra0, rb0);
        mm(ra1, rb1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, WN + WM, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, WN * WM - 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int g = 0; g + 1 < n_stages; ++g) {
    stage_body(g);
    // stage g+1 landed; every wave's reads of stage g have returned before the
    // barrier, so the DMA below may refill its buffer
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    issue_next();
    rd(g + 1, 0, ra0, rb0);
    mm(ra1, rb1);  // k-step DKS-1 of stage g (DKS even)
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * DMA_PER_WAVE, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, WN + WM, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, WN * WM - 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (++kt == nk) {
      epilogue(tile);
      zero_acc();
      kt = 0;
      ++tile;
    }
  }
  // last stage
  stage_body(n_stages - 1);
  mm(ra1, rb1);
  epilogue(tile);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no DMA may still target LDS at exit
}

template <int EPI>
static void launch_persist(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo,
                           hipStream_t s) {
  const int m_tiles = (M + 255) / 256;
  const int n_tiles = (EPI == EPI_SILU) ? (N / 2) / 128 : N / 256;
  const int total = m_tiles * n_tiles;
  const int per_xcd = (total + 7) / 8;
  const int slots = per_xcd < PWG_XCD ? per_xcd : PWG_XCD;
  hipLaunchKernelGGL((k_gemm_persist<EPI>), dim3(8 * slots), dim3(512), 0, s, X, W, out, M, N, K, ldo, n_tiles,
                     m_tiles, per_xcd);
}

// Sum of the K splits in split order, then the epilogue: one thread per 4
// output columns of one row.
template <int EPI>
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int n_split, int M, int N,
                                                      void* __restrict__ out, int ldo) {
  const int cols = (EPI == EPI_SILU) ? N / 2 : N;
  const int per_row = cols / 4;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= M * per_row) return;
  const int m = e / per_row, n = 4 * (e - m * per_row);
  const size_t stride = (size_t)M * N;
  const float* p = part + (size_t)m * N + n;
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  for (int sp = 1; sp < n_split; ++sp) v += *reinterpret_cast<const f32x4*>(p + sp * stride);
  if constexpr (EPI == EPI_SILU) {
    const float* q = p + N / 2;
    f32x4 u = *reinterpret_cast<const f32x4*>(q);
    for (int sp = 1; sp < n_split; ++sp) u += *reinterpret_cast<const f32x4*>(q + sp * stride);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = v[i] / (1.0f + __expf(-v[i])) * u[i];
  }
  if constexpr (EPI == EPI_BF16 || EPI == EPI_SILU) {
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

template <int EPI, int WN, int WM>
static void launch_t(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo, hipStream_t s,
                     int n_split, float* part, bool reduce) {
  constexpr int BN = 64 * WN, BM = 64 * WM;
  const int m_tiles = (M + BM - 1) / BM;
  const int n_tiles = (EPI == EPI_SILU) ? (N / 2) / (BN / 2) : N / BN;
  hipLaunchKernelGGL((k_gemm_tiled<EPI, WN, WM>), dim3(m_tiles * n_tiles * n_split), dim3(256), 0, s, X, W, out, M,
                     N, K, ldo, n_tiles, m_tiles, n_split, part);
  if (n_split > 1 && reduce) {
    const int per_row = ((EPI == EPI_SILU) ? N / 2 : N) / 4;
    hipLaunchKernelGGL((k_split_reduce<EPI>), dim3((M * per_row + 255) / 256), dim3(256), 0, s, part, n_split, M, N,
                       out, ldo);
  }
}

template <int EPI>
static void launch_e(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo, hipStream_t s,
                     int n_split, float* part, bool reduce) {
  // the 256 x 256 tile needs N % 256 == 0 and enough token tiles to fill the chip
  if (M >= 2048 && (N % 256) == 0)
    launch_persist<EPI>(X, W, out, M, N, K, ldo, s);
  else
    launch_t<EPI, 2, 2>(X, W, out, M, N, K, ldo, s, part ? n_split : 1, part, reduce);
}

void launch_gemm_tiled(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo, Epi epi,
                       hipStream_t s, int n_split, float* part, bool reduce) {
  switch (epi) {
    case EPI_BF16: launch_e<EPI_BF16>(X, W, out, M, N, K, ldo, s, n_split, part, reduce); break;
    case EPI_F32: launch_e<EPI_F32>(X, W, out, M, N, K, ldo, s, n_split, part, reduce); break;
    case EPI_ADD_F32: launch_e<EPI_ADD_F32>(X, W, out, M, N, K, ldo, s, n_split, part, reduce); break;
    case EPI_SILU: launch_e<EPI_SILU>(X, W, out, M, N, K, ldo, s, n_split, part, reduce); break;
    default: break;
  }
}

}  // namespace q3
