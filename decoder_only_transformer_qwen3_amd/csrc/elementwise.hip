// Bandwidth-bound kernels: embedding gather, (residual-add +) RMSNorm,
// per-head q/k RMSNorm + NeoX RoPE + KV-cache write, row argmax.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

// ---------------------------------------------------------------- embedding
// x = E[id] with no scaling ("手写Qwen3-0.6B推理" §Qwen3Model), plus, when a
// gain is given, the operand of the first layer's norm-folded projection:
// hg = bf16(gamma * x) and the sums of squares per 4 columns (ssq[m][256])
// or per 16 columns (ssq[m][64]) (the GEMM applies 1 / rms(x) itself).  One
// wave per token; lane l owns columns 16l .. 16l+15.  Block 0 also clears
// the call's workgroup tickets.
__device__ __forceinline__ void norm_operand_row(const float (&x)[16], int lane, const uint16_t* __restrict__ gamma,
                                                 uint16_t* __restrict__ hg_row, float* __restrict__ ssq_row,
                                                 int nsq) {
  const u32x4* gp = reinterpret_cast<const u32x4*>(gamma + 16 * lane);
  const u32x4 g0 = gp[0], g1 = gp[1];
  const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  u32x4 o[2];
  f32x4 ss = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    o[e >> 2][e & 3] = pack_bf2(x[2 * e] * bf_lo(gw[e]), x[2 * e + 1] * bf_hi(gw[e]));
    ss[e >> 1] += x[2 * e] * x[2 * e] + x[2 * e + 1] * x[2 * e + 1];
  }
  u32x4* dst = reinterpret_cast<u32x4*>(hg_row + 16 * lane);
  dst[0] = o[0];
  dst[1] = o[1];
  if (nsq == NSQ)
    *reinterpret_cast<f32x4*>(ssq_row + 4 * lane) = ss;
  else
    ssq_row[lane] = (ss.x + ss.y) + (ss.z + ss.w);
}

__device__ __forceinline__ void clear_tickets(int* counters, int n) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n; i += blockDim.x) counters[i] = 0;
}

__global__ __launch_bounds__(256) void k_embed(const int32_t* __restrict__ ids, const uint16_t* __restrict__ E,
                                               float* __restrict__ resid, int M, const uint16_t* __restrict__ gamma,
                                               uint16_t* __restrict__ hg, float* __restrict__ ssq, int nsq,
                                               int* __restrict__ counters, int n_counters) {
  clear_tickets(counters, n_counters);
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  int id = ids[m];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);  // out-of-range ids are clamped, never read out of bounds
  const u32x4* src = reinterpret_cast<const u32x4*>(E + (size_t)id * C + 16 * lane);
  const u32x4 w0 = src[0], w1 = src[1];
  const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float x[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[2 * e] = bf_lo(ww[e]);
    x[2 * e + 1] = bf_hi(ww[e]);
  }
  f32x4* dst = reinterpret_cast<f32x4*>(resid + (size_t)m * C + 16 * lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
  if (gamma) norm_operand_row(x, lane, gamma, hg + (size_t)m * C, ssq + (size_t)m * nsq, nsq);
}

void launch_embed(const int32_t* ids, const uint16_t* E, float* resid, int M, const uint16_t* gamma, uint16_t* hg,
                  float* ssq, int nsq, int* counters, int n_counters, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3((M + 3) / 4), dim3(256), 0, s, ids, E, resid, M, gamma, hg, ssq, nsq, counters,
                     n_counters);
}

// Norm-folded operand of n_rows residual rows (row r of the output reads
// resid row r*row_step + row_off): hg[r] = bf16(gamma * x), ssq[r][nsq].
__global__ __launch_bounds__(256) void k_norm_operand(const float* __restrict__ resid, int n_rows, int row_step,
                                                      int row_off, const uint16_t* __restrict__ gamma,
                                                      uint16_t* __restrict__ hg, float* __restrict__ ssq, int nsq,
                                                      int* __restrict__ counters, int n_counters, SeqMap last) {
  clear_tickets(counters, n_counters);
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  // packed rows (last.off set): the last row of sequence r
  size_t row = (size_t)r * row_step + row_off;
  if (last.off) {
    const int e = sm_row0(last, r) + sm_len(last, r);
    row = e > 0 ? (size_t)(e - 1) : 0;
  }
  const f32x4* src = reinterpret_cast<const f32x4*>(resid + row * C + 16 * lane);
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 v = src[i];
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
  norm_operand_row(x, lane, gamma, hg + (size_t)r * C, ssq + (size_t)r * nsq, nsq);
}

void launch_norm_operand(const float* resid, int n_rows, int row_step, int row_off, const uint16_t* gamma,
                         uint16_t* hg, float* ssq, int nsq, int* counters, int n_counters, hipStream_t s,
                         const SeqMap* last) {
  const int blocks = n_rows > 0 ? (n_rows + 3) / 4 : 1;  // one block still clears the tickets
  const SeqMap none{nullptr, nullptr, 0, 1, 0, 0};
  hipLaunchKernelGGL(k_norm_operand, dim3(blocks), dim3(256), 0, s, resid, n_rows, row_step, row_off,
                     gamma, hg, ssq, nsq, counters, n_counters, last ? *last : none);
}

// ---------------------------------------------------------------- RMSNorm
// gamma * r / sqrt(mean(r^2) + eps) in float32 ("手写Qwen3-0.6B推理"
// §Qwen3RMSNorm), preceded by the deferred residual add of split-K partial
// sums ("第 3 章" §3.2 folds the residual add into the norm the same way).
// One wave per row; lane l owns columns 4*(l + 64 j) .. +3, j = 0..3.
__global__ __launch_bounds__(256) void k_rmsnorm(float* __restrict__ resid, const float* __restrict__ part,
                                                 int n_part, int part_rows, const uint16_t* __restrict__ gamma,
                                                 uint16_t* __restrict__ out, int n_rows, int row_step,
                                                 int row_off) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= n_rows) return;
  const size_t row = (size_t)r * row_step + row_off;
  f32x4* x = reinterpret_cast<f32x4*>(resid + row * C);
  f32x4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = x[lane + 64 * j];
  if (n_part > 0) {
    // the split sums in split order, then the residual: the same additions
    // as the split-K reduce kernel's residual epilogue
    f32x4 ps[4];
    const f32x4* p0 = reinterpret_cast<const f32x4*>(part + row * C);
#pragma unroll
    for (int j = 0; j < 4; ++j) ps[j] = p0[lane + 64 * j];
    for (int p = 1; p < n_part; ++p) {
      const f32x4* pp = reinterpret_cast<const f32x4*>(part + ((size_t)p * part_rows + row) * C);
#pragma unroll
      for (int j = 0; j < 4; ++j) ps[j] += pp[lane + 64 * j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = v[j] + ps[j];
      x[lane + 64 * j] = v[j];
    }
  }
  if (out == nullptr) return;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  ss = wave_sum(ss);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / C) + EPS);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c0 = 4 * (lane + 64 * j);
    const u32x2 g = *reinterpret_cast<const u32x2*>(gamma + c0);
    u32x2 o;
    o.x = pack_bf2(v[j].x * rinv * bf_lo(g.x), v[j].y * rinv * bf_hi(g.x));
    o.y = pack_bf2(v[j].z * rinv * bf_lo(g.y), v[j].w * rinv * bf_hi(g.y));
    *reinterpret_cast<u32x2*>(out + (size_t)r * C + c0) = o;
  }
}

void launch_rmsnorm(float* resid, const float* part, int n_part, int part_rows, const uint16_t* gamma,
                    uint16_t* out, int n_rows, int row_step, int row_off, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3((n_rows + 3) / 4), dim3(256), 0, s, resid, part, n_part, part_rows, gamma,
                     out, n_rows, row_step, row_off);
}

// ---------------------------------------------------------------- k norm + RoPE, K/V cache write
// The new tokens' K and V rows of a multi-token call into the cache.  K gets
// the per-head RMSNorm with the head_dim-long k_norm gain
// ("手写Qwen3-0.6B推理" §Attention) and NeoX RoPE at the token's absolute
// position ("手写Qwen3-0.6B推理" §Rope; half-swap pairing per
// "古法手撕简易LLM推理器" §RoPE的细节):
//   y = x / sqrt(mean(x^2) + eps) * gamma
//   (y_i, y_{i+64}) -> (y_i c - y_{i+64} s, y_{i+64} c + y_i s),  c, s = cos, sin(p * 1e6^(-2i/128)),
// and the cache keeps normed, rotated K ("古法手撕简易LLM推理器"
// §核心计算函数与Transformer层) and raw V.  (q gets the same treatment, with
// q_norm, where the prefill attention loads it.)
//
// One workgroup per (32-position chunk, KV head, sequence); chunks start at
// multiples of 8 so they hold whole V blocks.  The 8 KV heads of a chunk run
// as consecutive workgroups on one XCD (workgroup ids are dealt to the 8
// XCDs in turn), so the chunk's rotary-table rows come from HBM once and
// the other heads read them from that XCD's L2.  K: 16 lanes per position,
// lane j holding dims 4j..4j+3 and 64+4j..64+4j+3, so the RoPE pairs stay in
// the lane and the head's sum of squares is a 16-lane DPP row sum.  V: the
// chunk's positions are staged in LDS and written to the blocked V cache
// (8 positions x 128 dims per 2 KB block, dim-major) as position-contiguous
// 8-byte groups.  Positions of the chunk outside the call's range are left
// untouched (they may hold earlier tokens).
constexpr int KVS_POS = 32;  // positions per workgroup

__global__ __launch_bounds__(256) void k_kv_store(const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ k_norm,
                                                  const float* __restrict__ rope_cos,
                                                  const float* __restrict__ rope_sin, uint16_t* __restrict__ k_cache,
                                                  uint16_t* __restrict__ v_cache, SeqMap sm, int max_seq,
                                                  int n_chunks) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[KVS_POS][D];
  // workgroup L: XCD L % 8, slot L / 8; head g = slot % 8 of unit 8 (slot / 8) + L % 8
  const int slot = blockIdx.x >> 3, g = slot & 7;
  const int unit = (slot >> 3) * 8 + (blockIdx.x & 7);
  if (unit >= n_chunks * sm.n) return;  // whole workgroup
  const int b = unit / n_chunks, chunk = unit - b * n_chunks, tid = threadIdx.x;
  const int T = sm_len(sm, b), row0 = sm_row0(sm, b);
  const int p_first = sm_start(sm, b);
  const int c0 = (p_first & ~7) + KVS_POS * chunk;  // first position of the chunk
  const int p_lo = p_first > c0 ? p_first : c0;
  int p_hi = (p_first + T) < (c0 + KVS_POS) ? (p_first + T) : (c0 + KVS_POS);
  p_hi = p_hi < max_seq ? p_hi : max_seq;
  if (p_first < 0 || p_lo >= p_hi) return;  // whole workgroup
  const size_t kv_base = ((size_t)b * HKV + g) * max_seq * D;
  // Every load of the workgroup is issued before the first is used, with no
  // branch between them: positions outside the range read a row of the range
  // instead (their values are dropped), since a conditional load would make
  // the compiler wait for each one before issuing the next.
  auto clamp_p = [&](int p) { return p < p_lo ? p_lo : (p >= p_hi ? p_hi - 1 : p); };
  const uint16_t* rows = qkv + (size_t)(row0 - p_first) * QKV_N;  // row of position p at rows + p * QKV_N
  u32x4 vv[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int e = it * 256 + tid;
    vv[it] = *reinterpret_cast<const u32x4*>(rows + (size_t)clamp_p(c0 + (e >> 4)) * QKV_N + (HQ + HKV + g) * D +
                                             8 * (e & 15));
  }
  constexpr int KIT = KVS_POS / 16;  // K passes of 16 positions
  const int j4 = 4 * (tid & 15);
  u32x2 klo[KIT], khi[KIT];
  f32x4 cs[KIT], sn[KIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int pc = clamp_p(c0 + it * 16 + (tid >> 4));
    const uint16_t* src = rows + (size_t)pc * QKV_N + (HQ + g) * D;
    klo[it] = *reinterpret_cast<const u32x2*>(src + j4);
    khi[it] = *reinterpret_cast<const u32x2*>(src + 64 + j4);
    const int pr = pc >= MAXPOS ? MAXPOS - 1 : pc;
    cs[it] = *reinterpret_cast<const f32x4*>(rope_cos + (size_t)pr * ROPE_HALF + j4);
    sn[it] = *reinterpret_cast<const f32x4*>(rope_sin + (size_t)pr * ROPE_HALF + j4);
  }
  const u32x2 g0 = *reinterpret_cast<const u32x2*>(k_norm + j4);
  const u32x2 g1 = *reinterpret_cast<const u32x2*>(k_norm + 64 + j4);
  // ---- V rows of the chunk into LDS (zeros outside the range, never written back)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int e = it * 256 + tid, r = e >> 4, c8 = 8 * (e & 15);
    const int p = c0 + r;
    const u32x4 v = (p >= p_lo && p < p_hi) ? vv[it] : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&tile[r][c8]) = v;
  }
  // ---- K rows: 16 positions per pass, 16 lanes per position
  const float ga[4] = {bf_lo(g0.x), bf_hi(g0.x), bf_lo(g0.y), bf_hi(g0.y)};
  const float gb[4] = {bf_lo(g1.x), bf_hi(g1.x), bf_lo(g1.y), bf_hi(g1.y)};
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int p = c0 + it * 16 + (tid >> 4);
    const float x[4] = {bf_lo(klo[it].x), bf_hi(klo[it].x), bf_lo(klo[it].y), bf_hi(klo[it].y)};
    const float y[4] = {bf_lo(khi[it].x), bf_hi(khi[it].x), bf_lo(khi[it].y), bf_hi(khi[it].y)};
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += x[i] * x[i] + y[i] * y[i];
    ss = row16_sum(ss);  // the 16 lanes of one position
    if (p >= p_lo && p < p_hi) {
      const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + EPS);
      float o0[4], o1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = x[i] * rinv * ga[i], bb = y[i] * rinv * gb[i];
        o0[i] = a * cs[it][i] - bb * sn[it][i];
        o1[i] = bb * cs[it][i] + a * sn[it][i];
      }
      uint16_t* dst = k_cache + kv_base + (size_t)p * D;
      *reinterpret_cast<u32x2*>(dst + j4) = u32x2{pack_bf2(o0[0], o0[1]), pack_bf2(o0[2], o0[3])};
      *reinterpret_cast<u32x2*>(dst + 64 + j4) = u32x2{pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3])};
    }
  }
  __syncthreads();
  // ---- V blocks: thread (d, half) writes 4 positions of dim d of each block
  const int d = tid >> 1, h4 = 4 * (tid & 1);
#pragma unroll
  for (int blk = 0; blk < KVS_POS / VBLK; ++blk) {
    const int q0 = c0 + blk * VBLK + h4, r0 = blk * VBLK + h4;
    uint16_t* dst = v_cache + kv_base + ((size_t)((c0 >> 3) + blk) * D + d) * VBLK + h4;
    if (q0 >= p_lo && q0 + 4 <= p_hi) {
      const u32x2 w = {(uint32_t)tile[r0][d] | ((uint32_t)tile[r0 + 1][d] << 16),
                       (uint32_t)tile[r0 + 2][d] | ((uint32_t)tile[r0 + 3][d] << 16)};
      *reinterpret_cast<u32x2*>(dst) = w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (q0 + i >= p_lo && q0 + i < p_hi) dst[i] = tile[r0 + i][d];
    }
  }
}

void launch_kv_store(const uint16_t* qkv, const uint16_t* k_norm, const float* rope_cos, const float* rope_sin,
                     uint16_t* k_cache, uint16_t* v_cache, const SeqMap& sm, int max_T, int max_seq, hipStream_t s) {
  // a run of up to max_T positions from an unaligned start spans at most max_T + 7 positions
  // from the 8-aligned position below its start
  const int n_chunks = (max_T + 7 + KVS_POS - 1) / KVS_POS;
  static_assert(HKV == 8, "one head per slot of an 8-slot group");
  const int n_groups = (n_chunks * sm.n + 7) / 8;
  hipLaunchKernelGGL(k_kv_store, dim3(n_groups * 64), dim3(256), 0, s, qkv, k_norm, rope_cos, rope_sin, k_cache,
                     v_cache, sm, max_seq, n_chunks);
}

// ---------------------------------------------------------------- argmax
// Greedy choice over one row per block ("手写Qwen3-0.6B推理" §推理).
__device__ __forceinline__ void am_wave_block_reduce(float& best, int& bi, float* sv, int* si) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (am_better(ov, oi, best, bi)) {
      best = ov;
      bi = oi;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
      if (am_better(sv[w], si[w], best, bi)) {
        best = sv[w];
        bi = si[w];
      }
  }
}

// One block of 1024 threads per row; 16 B loads when the row is 16-byte
// aligned, 8 loads in flight per thread.
__global__ __launch_bounds__(1024) void k_argmax(const float* __restrict__ logits, int vocab, int64_t stride,
                                                 int32_t* __restrict__ out_idx, int32_t* __restrict__ seq_lens,
                                                 int seq_mode, int seq_val) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* row = logits + (size_t)r * stride;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  int i0 = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    const int nvec = vocab >> 2;
    const f32x4* rv = reinterpret_cast<const f32x4*>(row);
    for (int base = 0; base < nvec; base += 1024 * 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * 1024 + tid;
        v[u] = i < nvec ? rv[i] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * 1024 + tid;
        if (i < nvec)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (am_better(v[u][e], 4 * i + e, best, bi)) {
              best = v[u][e];
              bi = 4 * i + e;
            }
      }
    }
    i0 = nvec << 2;
  }
  for (int base = i0; base < vocab; base += 1024 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 1024 + tid;
      v[u] = i < vocab ? row[i] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 1024 + tid;
      if (i < vocab && am_better(v[u], i, best, bi)) {
        best = v[u];
        bi = i;
      }
    }
  }
  am_wave_block_reduce(best, bi, sv, si);
  if (tid == 0) am_finish(r, bi, out_idx, seq_lens, seq_mode, seq_val);
}

void launch_argmax(const float* logits, int rows, int vocab, int64_t row_stride, int32_t* out_idx,
                   int32_t* seq_lens, int seq_mode, int seq_val, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax, dim3(rows), dim3(1024), 0, s, logits, vocab, row_stride, out_idx, seq_lens, seq_mode,
                     seq_val);
}

// ---------------------------------------------------------------------------
// Interleaved rotary pairs -> half-swap pairs: destination dim j of a q or k
// head takes source dim P(j) = 2j (j < 64), 2(j - 64) + 1 (j >= 64), so the
// half-swap pair (j, j + 64) is the interleaved pair (2j, 2j + 1).
// Blocks 0..4095 copy one weight row each (128 threads x 16 B); block 4096
// permutes the two gains.
__device__ __forceinline__ int half_from_interleaved(int j) { return j < D / 2 ? 2 * j : 2 * (j - D / 2) + 1; }

__global__ __launch_bounds__(128) void k_rope_pair_permute(const uint16_t* __restrict__ w_qkv,
                                                           const uint16_t* __restrict__ q_norm,
                                                           const uint16_t* __restrict__ k_norm,
                                                           uint16_t* __restrict__ w_out, uint16_t* __restrict__ qn_out,
                                                           uint16_t* __restrict__ kn_out) {
  const int r = blockIdx.x, t = threadIdx.x;
  if (r < QKV_N) {
    // rows 0..3071 are q and k heads of 128 rows; v rows are copied as they are
    const int src = r < QDIM + HKV * D ? (r / D) * D + half_from_interleaved(r % D) : r;
    reinterpret_cast<u32x4*>(w_out + (size_t)r * C)[t] = reinterpret_cast<const u32x4*>(w_qkv + (size_t)src * C)[t];
  } else {
    qn_out[t] = q_norm[half_from_interleaved(t)];
    kn_out[t] = k_norm[half_from_interleaved(t)];
  }
}

void launch_rope_pair_permute(const uint16_t* w_qkv, const uint16_t* q_norm, const uint16_t* k_norm,
                              uint16_t* w_out, uint16_t* qn_out, uint16_t* kn_out, hipStream_t s) {
  static_assert(C / 8 == 128 && D == 128, "one 128-thread block per 1024-wide row, one thread per gain");
  hipLaunchKernelGGL(k_rope_pair_permute, dim3(QKV_N + 1), dim3(128), 0, s, w_qkv, q_norm, k_norm, w_out, qn_out,
                     kn_out);
}

}  // namespace q3
