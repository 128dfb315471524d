// Split-K decode attention: one new query per sequence attends to cache
// rows 0..p (p = its position; "古法手撕简易LLM推理器" §prefill与predict
// decodes one token against the whole cache, and "从零开始写Qwen3（二）"
// §Attn notes such a query must see every cached key).
//
// The kernel starts from the raw merged projection of the new token, so the
// per-head q/k RMSNorm and NeoX RoPE ("手写Qwen3-0.6B推理" §Attention and
// §Rope) and the cache write of the new K/V happen here as well:
//   q' = rope_p(gamma_q * q / sqrt(mean(q^2) + eps)), likewise k'; v as is.
// A 16-lane DPP row holds one 128-dim head row, lane j dims 8j..8j+7, so the
// head's sum of squares is a row sum and RoPE's partner dims (i, i+64) sit
// in lanes j and j^8 (a row rotate by 8).
//
// Grid (split, KV head g, sequence b).  A workgroup reads its key range of
// K and V exactly once and serves both query heads 2g, 2g+1 that share g.
// Keys are processed in sub-chunks of up to 512: pass 1 computes scores
// into LDS (16 lanes per key row, 16 B per lane, row sums over the 16
// lanes with DPP), the sub-chunk's softmax statistics are merged into a
// running (max, sum), and pass 2 accumulates p * V over the blocked V
// cache (8 positions x 128 dims per 2 KB block): lane l owns dims 2l and
// 2l+1 and reads their 8 positions as two 16 B loads.  The workgroup whose
// range holds p takes the new key and value from registers / LDS rather
// than from the cache it is writing.
//
// Each split writes unnormalised (o, m, l) in the log2 domain; the last
// split to finish for a (b, g) (atomic ticket) combines them with the usual
// log-sum-exp rescaling and writes the two heads' bf16 outputs.  The key
// range of a split follows from the sequence's own device length, so the
// result is exact whatever split count the host picked.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int DEC_SUB = 512;  // keys per LDS sub-chunk
constexpr int PART_STRIDE = D + 2;
constexpr int DEC_SPLIT_CAP = 64;

__device__ __forceinline__ void load_row8(const uint16_t* src, float (&f)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf_lo(w[e]);
    f[2 * e + 1] = bf_hi(w[e]);
  }
}

// RMSNorm of the head row spread over a 16-lane row (lane j holds dims
// 8j..8j+7), gain, then NeoX RoPE with the table row of position p.
__device__ __forceinline__ void norm_rope8(float (&f)[8], const uint16_t* __restrict__ gamma,
                                           const float* __restrict__ cos_row, const float* __restrict__ sin_row,
                                           int j) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
  ss = row16_sum(ss);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + EPS);
  float g[8];
  load_row8(gamma + 8 * j, g);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] *= rinv * g[e];
    // partner dim (i + 64 for lanes 0..7, i - 64 for lanes 8..15): DPP row_ror:8
    o[e] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(f[e]), 0x128, 0xf, 0xf, false));
  }
  const int i0 = 8 * (j & 7);
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(cos_row + i0);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(cos_row + i0 + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(sin_row + i0);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(sin_row + i0 + 4);
  const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const float sgn = j < 8 ? -1.0f : 1.0f;  // x_i c - x_{i+64} s  |  x_{i+64} c + x_i s
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = f[e] * cs[e] + sgn * o[e] * sn[e];
}

__global__ __launch_bounds__(256) void k_attn_decode(const uint16_t* __restrict__ qkv,
                                                     const uint16_t* __restrict__ q_norm,
                                                     const uint16_t* __restrict__ k_norm,
                                                     const float* __restrict__ rope_cos,
                                                     const float* __restrict__ rope_sin,
                                                     uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                                     float* __restrict__ part, int* __restrict__ counters,
                                                     uint16_t* __restrict__ out, int max_seq,
                                                     const int32_t* __restrict__ pos_dev, int start, int n_split) {
  __shared__ __attribute__((aligned(16))) float sc[2][DEC_SUB];
  __shared__ float red[4][2][D];
  __shared__ float stat[2][8];
  __shared__ float vnew[D];
  __shared__ float mls[2][DEC_SPLIT_CAP][2];
  __shared__ int last_ticket;

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int p = pos_dev ? pos_dev[b] : start;
  int n = p + 1;
  n = n < max_seq ? n : max_seq;
  n = n > 0 ? n : 0;
  const int cs = (((n + n_split - 1) / n_split) + 15) & ~15;
  const int k0 = s * cs;
  const int k1 = (k0 + cs) < n ? (k0 + cs) : n;
  const bool own = p >= k0 && p < k1;  // this split holds the new token (then p < n <= max_seq)
  const int p_own = own ? p : -1;
  const int kc_end = own ? p : k1;     // keys read from the cache: k0 .. kc_end-1

  // ---- q (and, for the owner, k and v) of the new token
  const int j = l & 15, d0 = 8 * j, krow = l >> 4;
  const int pc = p < 0 ? 0 : (p >= MAXPOS ? MAXPOS - 1 : p);
  const float* cos_row = rope_cos + (size_t)pc * ROPE_HALF;
  const float* sin_row = rope_sin + (size_t)pc * ROPE_HALF;
  const uint16_t* qrow = qkv + (size_t)b * QKV_N;
  float qf0[8], qf1[8];
  load_row8(qrow + (2 * g) * D + d0, qf0);
  load_row8(qrow + (2 * g + 1) * D + d0, qf1);
  norm_rope8(qf0, q_norm, cos_row, sin_row, j);
  norm_rope8(qf1, q_norm, cos_row, sin_row, j);
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
  float s_new0 = 0.f, s_new1 = 0.f;
  if (own) {
    float kf[8], vf[8];
    load_row8(qrow + QDIM + g * D + d0, kf);
    load_row8(qrow + QDIM + HKV * D + g * D + d0, vf);
    norm_rope8(kf, k_norm, cos_row, sin_row, j);
    u32x4 kb;
#pragma unroll
    for (int e = 0; e < 4; ++e) kb[e] = pack_bf2(kf[2 * e], kf[2 * e + 1]);
    // the score uses the key exactly as the cache will hold it
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[2 * e] = bf_lo(kb[e]);
      kf[2 * e + 1] = bf_hi(kb[e]);
    }
    float d0s = 0.f, d1s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      d0s += qf0[e] * kf[e];
      d1s += qf1[e] * kf[e];
    }
    s_new0 = row16_sum(d0s) * sl2;
    s_new1 = row16_sum(d1s) * sl2;
    if (w == 0 && l < 16) {
      const size_t head_base = ((size_t)b * HKV + g) * max_seq * D;
      *reinterpret_cast<u32x4*>(k_cache + head_base + (size_t)p * D + d0) = kb;
      const u32x4 vb = *reinterpret_cast<const u32x4*>(qrow + QDIM + HKV * D + g * D + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v_cache[head_base + vblk_index(p, d0 + 2 * e)] = (uint16_t)(vb[e] & 0xffffu);
        v_cache[head_base + vblk_index(p, d0 + 2 * e + 1)] = (uint16_t)(vb[e] >> 16);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vnew[d0 + e] = vf[e];
    }
  }

  const uint16_t* kbase = k_cache + ((size_t)b * HKV + g) * max_seq * D + d0;
  const uint16_t* vbase = v_cache + ((size_t)b * HKV + g) * max_seq * D + 2 * l * VBLK;

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  // acc[h][e]: head 2g+h, dim 2l+e
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  float vn[2] = {0.f, 0.f};
  bool vn_loaded = false;

  for (int c0 = k0; c0 < k1; c0 += DEC_SUB) {
    const int c1 = (c0 + DEC_SUB) < k1 ? (c0 + DEC_SUB) : k1;
    const int c1c = c1 < kc_end ? c1 : kc_end;  // cache keys of this sub-chunk end here
    // ---- pass 1: scores for keys c0..c1c-1 from the cache, the new key from registers
    for (int base = c0; base < c1c; base += 64) {
      u32x4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int key = base + 16 * u + 4 * w + krow;
        key = key < c1c ? key : c1c - 1;
        kv[u] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * D);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float d0s = 0.f, d1s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = bf_lo(kv[u][e]), x1 = bf_hi(kv[u][e]);
          d0s += x0 * qf0[2 * e] + x1 * qf0[2 * e + 1];
          d1s += x0 * qf1[2 * e] + x1 * qf1[2 * e + 1];
        }
        d0s = row16_sum(d0s);
        d1s = row16_sum(d1s);
        const int key = base + 16 * u + 4 * w + krow;
        if (key < c1c) {
          if (j == 0) sc[0][key - c0] = d0s * sl2;
          if (j == 1) sc[1][key - c0] = d1s * sl2;
        }
      }
    }
    if (p_own >= c0 && p_own < c1 && tid == 0) {
      sc[0][p_own - c0] = s_new0;
      sc[1][p_own - c0] = s_new1;
    }
    __syncthreads();
    if (!vn_loaded) {  // vnew is visible after the first barrier
      vn[0] = vnew[2 * l];
      vn[1] = vnew[2 * l + 1];
      vn_loaded = true;
    }
    // ---- sub-chunk max per head (threads 0..127 head 0, 128..255 head 1)
    const int hh = tid >> 7, ti = tid & 127;
    const int cnt = c1 - c0;
    float mx = -INFINITY;
    for (int i = ti; i < cnt; i += 128) mx = fmaxf(mx, sc[hh][i]);
    mx = wave_max(mx);
    if (l == 0) stat[hh][w & 1] = mx;
    __syncthreads();
    float m_new[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) m_new[h] = fmaxf(m_run[h], fmaxf(stat[h][0], stat[h][1]));
    float ls = 0.f;
    for (int i = ti; i < cnt; i += 128) {
      const float pv = __builtin_amdgcn_exp2f(sc[hh][i] - m_new[hh]);
      sc[hh][i] = pv;
      ls += pv;
    }
    ls = wave_sum(ls);
    if (l == 0) stat[hh][2 + (w & 1)] = ls;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new[h]);
      l_run[h] = l_run[h] * alpha + stat[h][2] + stat[h][3];
      m_run[h] = m_new[h];
      acc[h][0] *= alpha;
      acc[h][1] *= alpha;
    }
    // ---- pass 2: acc += p * V, one 8-position block per wave step
    for (int blk0 = c0 + 8 * w; blk0 < c1; blk0 += 64) {
      u32x4 vv[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pb = blk0 + 32 * u;
        if (pb < c1) {
          const uint16_t* src = vbase + (size_t)pb * D;
          vv[u][0] = *reinterpret_cast<const u32x4*>(src);
          vv[u][1] = *reinterpret_cast<const u32x4*>(src + VBLK);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pb = blk0 + 32 * u;
        if (pb >= c1) continue;
        const int valid = c1 - pb;  // positions beyond the range get p = 0 and a zeroed value
        float pr[2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sc[h][pb - c0]);
          const f32x4 bq = *reinterpret_cast<const f32x4*>(&sc[h][pb - c0 + 4]);
          pr[h][0] = a.x; pr[h][1] = a.y; pr[h][2] = a.z; pr[h][3] = a.w;
          pr[h][4] = bq.x; pr[h][5] = bq.y; pr[h][6] = bq.z; pr[h][7] = bq.w;
        }
        const int knew = p_own - pb;  // slot of the new token in this block, if any
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t word = vv[u][e][k >> 1];
            float x = (k & 1) ? bf_hi(word) : bf_lo(word);
            x = k == knew ? vn[e] : x;
            x = k < valid ? x : 0.f;
            acc[0][e] += (k < valid ? pr[0][k] : 0.f) * x;
            acc[1][e] += (k < valid ? pr[1][k] : 0.f) * x;
          }
      }
    }
    __syncthreads();  // sc is rewritten by the next sub-chunk
  }

  // ---- reduce acc over the 4 waves, store this split's (o, m, l)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    red[w][h][2 * l] = acc[h][0];
    red[w][h][2 * l + 1] = acc[h][1];
  }
  __syncthreads();
  const int hh = tid >> 7, d = tid & 127;
  {
    const float o = red[0][hh][d] + red[1][hh][d] + red[2][hh][d] + red[3][hh][d];
    float* dst = part + (((size_t)b * HQ + 2 * g + hh) * n_split + s) * PART_STRIDE;
    st_dev(dst + d, o);
    if (d == 0) {
      st_dev(dst + D, m_run[hh]);
      st_dev(dst + D + 1, l_run[hh]);
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
                        hipStream_t s) {
  hipLaunchKernelGGL(k_attn_decode, dim3(n_split, HKV, B), dim3(256), 0, s, qkv, q_norm, k_norm, rope_cos, rope_sin,
                     k_cache, v_cache, part, counters, out, max_seq, pos_dev, start, n_split);
}

}  // namespace q3
