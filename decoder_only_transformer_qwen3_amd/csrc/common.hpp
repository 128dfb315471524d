// Shared device helpers for the gfx950 kernels: fixed model dimensions,
// bfloat16 bit conversions, MFMA operand vector types and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

constexpr int C = 1024;        // hidden size
constexpr int HQ = 16;         // query heads
constexpr int HKV = 8;         // key/value heads
constexpr int D = 128;         // head dim
constexpr int I = 3072;        // MLP intermediate size
constexpr int V = 151936;      // vocabulary
constexpr int NL = 28;         // layers
constexpr int MAXPOS = 40960;  // max position
constexpr int QKV_N = (HQ + 2 * HKV) * D;  // 4096
constexpr int QDIM = HQ * D;               // 2048
constexpr int ROPE_HALF = D / 2;           // 64 table columns
constexpr float EPS = 1e-6f;
// The norm folded into a projection gets, per residual row, partial sums of
// squares: NSQ (one per 4 columns) when at most 8 rows are in flight (the
// VALU GEMV writes one per 4-column workgroup), NSQ_BLK (one per 16
// columns) otherwise (fewer for the consumers to read).
constexpr int NSQ = C / 4;
constexpr int NSQ_BLK = C / 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c on packed bf16 pairs (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// float32 -> bfloat16 (round to nearest even, NaN stays NaN); gfx950 does
// this in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2 r;
  r.x = (__bf16)lo;
  r.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of
// the row receives the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));  // row_mirror
  return v;
}

// V cache layout: per (sequence, KV head) the positions are grouped in
// blocks of 8; a block stores its 128 dims x 8 positions dim-major, so
// element (p, d) sits at ((p / 8) * 128 + d) * 8 + p % 8.  Eight consecutive
// positions of one dim are 16 contiguous bytes (an MFMA operand chunk), and
// a block of 8 positions is 2 KB of contiguous memory.
constexpr int VBLK = 8;
__device__ __forceinline__ size_t vblk_index(int p, int d) {
  return ((size_t)(p >> 3) * D + d) * VBLK + (p & 7);
}

// Exchange between workgroups of one kernel without writing back or
// invalidating the L2 caches: relaxed device-scope atomic loads and stores
// carry the device-scope cache policy, so they are coherent across the
// XCDs' separate L2 caches by themselves.  A producer stores its data with
// st_dev, waits until the stores have completed (vm_drain), and only then
// takes a ticket; the workgroup that draws the last ticket reads with
// ld_dev.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Stores from the accumulator layout of v_mfma_f32_32x32x16_bf16 with the
// output row along B: in a 32 x 32 block, lane (r, h) = (l % 32, l / 32)
// holds columns 8 j + 4 h .. + 3 (group j = 0..3, elements 4 j .. 4 j + 3)
// of row r.

// 16-byte store of 8 consecutive bf16 columns from groups j = 2 p (lo) and
// 2 p + 1 (hi): one swap between the half-waves gives lane h = 0 columns
// 16 p .. 16 p + 7 and lane h = 1 columns 16 p + 8 .. 16 p + 15, both of
// row r.  dst is the address of the lane's 8 columns; the lane and its
// partner l ^ 32 must both be active.
__device__ __forceinline__ void store_pair16(uint16_t* dst, u32x2 lo, u32x2 hi) {
  const auto x = __builtin_amdgcn_permlane32_swap(lo.x, hi.x, false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(lo.y, hi.y, false, false);
  u32x4 v;
  v.x = x[0];
  v.y = y[0];
  v.z = x[1];
  v.w = y[1];
  *reinterpret_cast<u32x4*>(dst) = v;
}

// bf16 columns 16 p + 8 h .. + 7 of one block (column 0 of the block at row + 0).
__device__ __forceinline__ void store_block_bf16(uint16_t* row, const f32x16& a, int lh) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    u32x2 o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = 2 * p + h;
      o[h].x = pack_bf2(a[4 * g], a[4 * g + 1]);
      o[h].y = pack_bf2(a[4 * g + 2], a[4 * g + 3]);
    }
    store_pair16(row + 16 * p + 8 * lh, o[0], o[1]);
  }
}

// Rows of a multi-token call and the (sequence, position) each belongs to.
// Uniform: n sequences of T rows, row m = s*T + t at position
// (pos ? pos[s] : start) + t.  Packed (off != null): sequence s owns rows
// off[s] .. off[s+1]-1 at positions (pos ? pos[s] : 0) + t, and there are
// rows = off[n] of them.  The row offsets come from the caller's device
// memory, so every lookup is clamped to [0, rows]: bad offsets give wrong
// sequences, never out-of-range rows.
struct SeqMap {
  const int32_t* off;
  const int32_t* pos;
  int n, T, start, rows;
};
__device__ __forceinline__ int sm_row0(const SeqMap& sm, int s) {
  if (!sm.off) return s * sm.T;
  const int r = sm.off[s];
  return r < 0 ? 0 : (r > sm.rows ? sm.rows : r);
}
__device__ __forceinline__ int sm_len(const SeqMap& sm, int s) {
  if (!sm.off) return sm.T;
  const int r1 = sm.off[s + 1];
  const int e = r1 < 0 ? 0 : (r1 > sm.rows ? sm.rows : r1);
  const int b = sm_row0(sm, s);
  return e > b ? e - b : 0;
}
__device__ __forceinline__ int sm_start(const SeqMap& sm, int s) {
  return sm.pos ? sm.pos[s] : (sm.off ? 0 : sm.start);
}

// Greedy choice ("手写Qwen3-0.6B推理" §推理) over (value, index) candidates.
// Order: NaN above every number (first NaN wins), otherwise larger value,
// ties to the lower index.
__device__ __forceinline__ bool am_better(float a, int ia, float b, int ib) {
  const bool an = a != a, bn = b != b;
  if (an || bn) return an && (!bn || ia < ib);
  return a > b || (a == b && ia < ib);
}

// The chosen token of row r: out_idx[r], and the row's sequence length.
// seq_mode 2 with eos >= 0: a row whose input token in_ids[r] is eos has
// finished; it keeps its length and emits eos again (in_ids may alias
// out_idx: it is read first).
// seq_mode 3 (packed prefill): seq_lens[r] = start + rows of sequence r.
__device__ __forceinline__ void am_finish(int r, int bi, int32_t* out_idx, int32_t* seq_lens, int seq_mode,
                                          int seq_val, const int32_t* in_ids = nullptr, int eos = -1,
                                          const SeqMap* sm = nullptr) {
  const bool fin = seq_mode == 2 && eos >= 0 && in_ids[r] == eos;
  out_idx[r] = fin ? eos : bi;
  if (seq_mode == 1) seq_lens[r] = seq_val;
  if (seq_mode == 2 && !fin) seq_lens[r] += 1;
  if (seq_mode == 3) seq_lens[r] = sm_start(*sm, r) + sm_len(*sm, r);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over the 64 lanes without the LDS crossbar: DPP within rows of 16,
// then the row and half swaps.  Every lane must be active.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = row16_sum(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Sum over aligned groups of G = 2, 4, 8 or 16 lanes (DPP only); every lane
// of a group receives the total.  Every lane must be active.
template <int G>
__device__ __forceinline__ float group_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));  // lane ^ 1
  if constexpr (G >= 4)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));  // lane ^ 2
  if constexpr (G >= 8)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));  // half-row mirror
  if constexpr (G >= 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));  // row mirror
  return v;
}

}  // namespace q3
