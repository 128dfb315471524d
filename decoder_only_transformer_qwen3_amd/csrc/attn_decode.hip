// Split-K decode attention: one new query per sequence attends to cache
// rows 0..p (p = its position; "古法手撕简易LLM推理器" §prefill与predict
// decodes one token against the whole cache, and "从零开始写Qwen3（二）"
// §Attn notes such a query must see every cached key).
//
// Grid (split, KV head g, sequence b).  A workgroup reads its key range of
// K and V exactly once and serves both query heads 2g, 2g+1 that share g.
// Keys are processed in sub-chunks of up to 512: pass 1 computes scores
// into LDS (16 lanes per key row, 16 B per lane, row sums over the 16
// lanes with DPP), the sub-chunk's softmax statistics are merged into a
// running (max, sum), and pass 2 accumulates p * V over the blocked V
// cache (8 positions x 128 dims per 2 KB block): lane l owns dims 2l and
// 2l+1 and reads their 8 positions as two 16 B loads.  Each split writes unnormalised (o, m, l) in the log2 domain; the
// merge kernel combines splits with the usual log-sum-exp rescaling.  The
// key range of a split is derived from the sequence's own device length,
// so the result is exact whatever split count the host picked.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int DEC_SUB = 512;  // keys per LDS sub-chunk
constexpr int PART_STRIDE = D + 2;

__global__ __launch_bounds__(256) void k_attn_decode(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                                                     const uint16_t* __restrict__ v_cache, float* __restrict__ part,
                                                     int max_seq, const int32_t* __restrict__ pos_dev, int start,
                                                     int n_split) {
  __shared__ float sc[2][DEC_SUB];
  __shared__ float red[4][2][D];
  __shared__ float stat[2][8];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int p = pos_dev ? pos_dev[b] : start;
  int n = p + 1;
  n = n < max_seq ? n : max_seq;
  n = n > 0 ? n : 0;
  const int cs = (((n + n_split - 1) / n_split) + 15) & ~15;
  const int k0 = s * cs;
  const int k1 = (k0 + cs) < n ? (k0 + cs) : n;

  // lane layout: key = base + 4*w + (l >> 4) within a 16-key step, dims 8*(l & 15)
  const int d0 = 8 * (l & 15), krow = l >> 4;
  const uint16_t* qh0 = q + (size_t)b * QDIM + (2 * g) * D + d0;
  const u32x4 q0 = *reinterpret_cast<const u32x4*>(qh0);
  const u32x4 q1 = *reinterpret_cast<const u32x4*>(qh0 + D);
  float qf0[8], qf1[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    qf0[2 * e] = bf_lo(q0[e]);
    qf0[2 * e + 1] = bf_hi(q0[e]);
    qf1[2 * e] = bf_lo(q1[e]);
    qf1[2 * e + 1] = bf_hi(q1[e]);
  }
  const uint16_t* kb = k_cache + ((size_t)b * HKV + g) * max_seq * D + d0;
  const uint16_t* vb = v_cache + ((size_t)b * HKV + g) * max_seq * D + 2 * l * VBLK;
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  // acc[h][e]: head 2g+h, dim 2l+e
  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};

  for (int c0 = k0; c0 < k1; c0 += DEC_SUB) {
    const int c1 = (c0 + DEC_SUB) < k1 ? (c0 + DEC_SUB) : k1;
    // ---- pass 1: scores for keys c0..c1-1
    for (int base = c0; base < c1; base += 64) {
      u32x4 kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int key = base + 16 * u + 4 * w + krow;
        key = key < c1 ? key : c1 - 1;
        kv[u] = *reinterpret_cast<const u32x4*>(kb + (size_t)key * D);
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
        if (key < c1) {
          if ((l & 15) == 0) sc[0][key - c0] = d0s * sl2;
          if ((l & 15) == 1) sc[1][key - c0] = d1s * sl2;
        }
      }
    }
    __syncthreads();
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
      const float pv = exp2f(sc[hh][i] - m_new[hh]);
      sc[hh][i] = pv;
      ls += pv;
    }
    ls = wave_sum(ls);
    if (l == 0) stat[hh][2 + (w & 1)] = ls;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float alpha = exp2f(m_run[h] - m_new[h]);
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
          const uint16_t* src = vb + (size_t)pb * D;
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
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t word = vv[u][e][k >> 1];
            float x = (k & 1) ? bf_hi(word) : bf_lo(word);
            x = k < valid ? x : 0.f;
            acc[0][e] += (k < valid ? pr[0][k] : 0.f) * x;
            acc[1][e] += (k < valid ? pr[1][k] : 0.f) * x;
          }
      }
    }
    __syncthreads();  // sc is rewritten by the next sub-chunk
  }

  // ---- reduce acc over the 4 waves
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    red[w][h][2 * l] = acc[h][0];
    red[w][h][2 * l + 1] = acc[h][1];
  }
  __syncthreads();
  {
    const int h = tid >> 7, d = tid & 127;
    const float o = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
    float* dst = part + (((size_t)b * HQ + 2 * g + h) * n_split + s) * PART_STRIDE;
    dst[d] = o;
    if (d == 0) {
      dst[D] = m_run[h];
      dst[D + 1] = l_run[h];
    }
  }
}

// Combine the splits of one (sequence, query head): o = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s.
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                    int n_split) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* base = part + (size_t)bh * n_split * PART_STRIDE;
  float m = -INFINITY;
  for (int s = 0; s < n_split; ++s) m = fmaxf(m, base[s * PART_STRIDE + D]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float ms = base[s * PART_STRIDE + D];
    const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - m);
    num += f * base[s * PART_STRIDE + d];
    den += f * base[s * PART_STRIDE + D + 1];
  }
  const int b = bh / HQ, h = bh - b * HQ;
  out[(size_t)b * QDIM + h * D + d] = (uint16_t)f2bf(num / den);
}

void launch_attn_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, float* part,
                        uint16_t* out, int B, int max_seq, const int32_t* pos_dev, int start, int n_split,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_attn_decode, dim3(n_split, HKV, B), dim3(256), 0, s, q, k_cache, v_cache, part, max_seq,
                     pos_dev, start, n_split);
  hipLaunchKernelGGL(k_attn_merge, dim3(B * HQ), dim3(128), 0, s, part, out, n_split);
}

}  // namespace q3
