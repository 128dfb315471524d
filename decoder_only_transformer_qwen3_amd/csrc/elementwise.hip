// Bandwidth-bound kernels: embedding gather, (residual-add +) RMSNorm,
// per-head q/k RMSNorm + NeoX RoPE + KV-cache write, row argmax.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

// ---------------------------------------------------------------- embedding
// x = E[id] with no scaling ("手写Qwen3-0.6B推理" §Qwen3Model).  One block of
// 128 threads per token; each thread widens 8 bf16 values (one 16 B load).
__global__ __launch_bounds__(128) void k_embed(const int32_t* __restrict__ ids, const uint16_t* __restrict__ E,
                                               float* __restrict__ resid) {
  const int m = blockIdx.x;
  int id = ids[m];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);  // out-of-range ids are clamped, never read out of bounds
  const u32x4 w = *reinterpret_cast<const u32x4*>(E + (size_t)id * C + threadIdx.x * 8);
  f32x4 a = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
  f32x4 b = {bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
  f32x4* dst = reinterpret_cast<f32x4*>(resid + (size_t)m * C) + threadIdx.x * 2;
  dst[0] = a;
  dst[1] = b;
}

void launch_embed(const int32_t* ids, const uint16_t* E, float* resid, int M, hipStream_t s) {
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(128), 0, s, ids, E, resid);
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
    for (int p = 0; p < n_part; ++p) {
      const f32x4* pp = reinterpret_cast<const f32x4*>(part + ((size_t)p * part_rows + row) * C);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += pp[lane + 64 * j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) x[lane + 64 * j] = v[j];
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

// ---------------------------------------------------------------- q/k norm + RoPE + KV write
// One wave per (token, head slot): slots 0..15 are query heads, 16..23 key
// heads, 24..31 value heads.  Lane l holds dimensions l and l + 64, which
// are exactly a RoPE pair in the half-swap (NeoX) form, so the rotation
// needs no cross-lane traffic:
//   y = x / sqrt(mean(x^2) + eps) * gamma             ("手写Qwen3-0.6B推理" §Attention, q_norm/k_norm)
//   (y_l, y_{l+64}) -> (y_l c - y_{l+64} s, y_{l+64} c + y_l s)
//   with c, s = cos, sin(p * 1e6^(-2l/128))           (§Rope; "古法手撕简易LLM推理器" §RoPE的细节)
// K (normed + rotated) and raw V go to cache row p ("古法手撕简易LLM推理器"
// §核心计算函数与Transformer层).
__global__ __launch_bounds__(256) void k_qknorm_rope(const uint16_t* __restrict__ qkv,
                                                     const uint16_t* __restrict__ q_norm,
                                                     const uint16_t* __restrict__ k_norm,
                                                     const float* __restrict__ rope_cos,
                                                     const float* __restrict__ rope_sin, uint16_t* __restrict__ q_out,
                                                     uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                                     int B, int T, int max_seq, const int32_t* __restrict__ pos_dev,
                                                     int start) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave;
  const int m = gw >> 5, slot = gw & 31;
  if (m >= B * T) return;
  const int b = m / T, t = m - b * T;
  const int p = (pos_dev ? pos_dev[b] : start) + t;
  const bool in_cache = p >= 0 && p < max_seq;
  const uint16_t* src = qkv + (size_t)m * QKV_N + slot * D;
  const uint32_t b0 = src[lane], b1 = src[lane + 64];
  if (slot >= HQ + HKV) {  // value head: raw copy into the cache
    if (in_cache) {
      uint16_t* dst = v_cache + (((size_t)b * HKV + (slot - HQ - HKV)) * max_seq + p) * D;
      dst[lane] = (uint16_t)b0;
      dst[lane + 64] = (uint16_t)b1;
    }
    return;
  }
  const float x0 = bf2f(b0), x1 = bf2f(b1);
  const uint16_t* g = slot < HQ ? q_norm : k_norm;
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + EPS);
  const float y0 = x0 * rinv * bf2f(g[lane]);
  const float y1 = x1 * rinv * bf2f(g[lane + 64]);
  const int pc = p < 0 ? 0 : (p >= MAXPOS ? MAXPOS - 1 : p);
  const float c = rope_cos[(size_t)pc * ROPE_HALF + lane];
  const float sn = rope_sin[(size_t)pc * ROPE_HALF + lane];
  const uint16_t o0 = (uint16_t)f2bf(y0 * c - y1 * sn);
  const uint16_t o1 = (uint16_t)f2bf(y1 * c + y0 * sn);
  if (slot < HQ) {
    uint16_t* dst = q_out + (size_t)m * QDIM + slot * D;
    dst[lane] = o0;
    dst[lane + 64] = o1;
  } else if (in_cache) {
    uint16_t* dst = k_cache + (((size_t)b * HKV + (slot - HQ)) * max_seq + p) * D;
    dst[lane] = o0;
    dst[lane + 64] = o1;
  }
}

void launch_qknorm_rope(const uint16_t* qkv, const uint16_t* q_norm, const uint16_t* k_norm,
                        const float* rope_cos, const float* rope_sin, uint16_t* q_out, uint16_t* k_cache,
                        uint16_t* v_cache, int B, int T, int max_seq, const int32_t* pos_dev, int start,
                        hipStream_t s) {
  const int waves = B * T * 32;
  hipLaunchKernelGGL(k_qknorm_rope, dim3((waves + 3) / 4), dim3(256), 0, s, qkv, q_norm, k_norm, rope_cos,
                     rope_sin, q_out, k_cache, v_cache, B, T, max_seq, pos_dev, start);
}

// ---------------------------------------------------------------- argmax
// Greedy choice over one row per block ("手写Qwen3-0.6B推理" §推理).
// Order: NaN above every number (first NaN wins), otherwise larger value,
// ties to the lower index.
__device__ __forceinline__ bool am_better(float a, int ia, float b, int ib) {
  const bool an = a != a, bn = b != b;
  if (an || bn) return an && (!bn || ia < ib);
  return a > b || (a == b && ia < ib);
}

__global__ __launch_bounds__(1024) void k_argmax(const float* __restrict__ logits, int vocab, int64_t stride,
                                                 int32_t* __restrict__ out_idx, int32_t* __restrict__ seq_lens,
                                                 int seq_mode, int seq_val) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int r = blockIdx.x;
  const float* row = logits + (size_t)r * stride;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < vocab; i += 1024) {
    const float v = row[i];
    if (am_better(v, i, best, bi)) {
      best = v;
      bi = i;
    }
  }
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
    float b = sv[0];
    int i = si[0];
    for (int w = 1; w < 16; ++w)
      if (am_better(sv[w], si[w], b, i)) {
        b = sv[w];
        i = si[w];
      }
    out_idx[r] = i;
    if (seq_mode == 1) seq_lens[r] = seq_val;
    if (seq_mode == 2) seq_lens[r] += 1;
  }
}

void launch_argmax(const float* logits, int rows, int vocab, int64_t row_stride, int32_t* out_idx,
                   int32_t* seq_lens, int seq_mode, int seq_val, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax, dim3(rows), dim3(1024), 0, s, logits, vocab, row_stride, out_idx, seq_lens, seq_mode,
                     seq_val);
}

}  // namespace q3
