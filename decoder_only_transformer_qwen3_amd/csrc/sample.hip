// Temperature / top-k / top-p sampling of logits rows, the path that
// "第 3 章 前向与生成（代码走读）" §4.3 (Sampler.sample) takes when
// temperatures are given (the greedy path is the lm_head's fused argmax).
// Per row r, with T = temperature[r], k = top_k[r], p = top_p[r] and the
// caller's uniform draw u = uniform[r] in [0, 1):
//   T <= 0 (or NaN)  -> greedy: lowest index of the maximum;
//   z = logits / T;
//   candidates: every token with z >= the k-th largest z (k = 4096 when
//     top_k <= 0 or > 4096; at most the vocabulary), ordered by z
//     descending then index ascending, at most 4096 of them;
//   softmax over the candidates, cumulative in that order; keep the
//     shortest prefix whose mass reaches p (p outside (0, 1] means 1);
//   pick the first kept position whose cumulative mass exceeds u times
//     the kept mass.
//
// One 1024-thread workgroup per row:
//   1. k-th largest z by radix select on the order-preserving 32-bit keys of
//      z (four 8-bit digits, most significant first, LDS histograms of
//      integer counts, so the result does not depend on thread timing;
//      lanes of a wave that share a bin add to it with one atomic);
//   2. the candidates gathered into LDS slots (their order is fixed by the
//      sort; ties beyond the 4096 cap are cut in index order);
// every pass over the row keeps 8 coalesced 16-byte loads per thread in flight;
//   3. a bitonic sort of at most 4096 (key, index) pairs in LDS;
//   4. exp, an in-order block scan of the masses, the top-p cut and the
//      draw, all in float32.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace q3 {

constexpr int SK_MAX = 4096;  // candidate cap
constexpr int SK_T = 1024;    // threads per row
constexpr int SK_E = 32;      // row values per thread and batch (8 x 16-byte loads in flight)

// A batch of the row: thread t holds v[j] = x[base + 4 * (u * SK_T + t) + c]
// for j = 4u + c (0 past the row end).  VEC: 16-byte loads (rows 16-byte
// aligned); otherwise the same elements one by one.
template <bool VEC>
__device__ __forceinline__ void load_batch(const float* x, int vocab, int base, float (&v)[SK_E]) {
#pragma unroll
  for (int u = 0; u < SK_E / 4; ++u) {
    const int i = base + 4 * (u * SK_T + (int)threadIdx.x);
    if (VEC && i + 3 < vocab) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(x + i);
      v[4 * u] = q.x;
      v[4 * u + 1] = q.y;
      v[4 * u + 2] = q.z;
      v[4 * u + 3] = q.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * u + c] = i + c < vocab ? x[i + c] : 0.f;
    }
  }
}
__device__ __forceinline__ int batch_index(int base, int j) {
  return base + 4 * ((j >> 2) * SK_T + (int)threadIdx.x) + (j & 3);
}

// order-preserving map of float32 to uint32 (larger float -> larger key); NaN keys above +inf
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// hist[bin] += 1 for every lane with pred.  Keys of one row crowd into a
// few bins of the leading digits, where plain LDS atomics would serialise:
// up to four rounds count the lanes that share a leader's bin with one
// ballot and add them with one atomic; lanes left after that add their own.
__device__ __forceinline__ void hist_add(int* hist, bool pred, uint32_t bin) {
  const int lane = threadIdx.x & 63;
  bool done = !pred;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const uint64_t rem = __ballot(!done);
    if (rem == 0) return;
    const int leader = __ffsll((unsigned long long)rem) - 1;
    const uint32_t lb = __shfl(bin, leader, 64);
    const bool same = !done && bin == lb;
    const uint64_t group = __ballot(same);
    if (lane == leader) atomicAdd(&hist[lb], __popcll(group));
    done = done || same;
  }
  if (!done) atomicAdd(&hist[bin], 1);
}

// exclusive scan of one int per thread over the workgroup; returns the total
__device__ int block_excl_scan(int v, int* lds_warp, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) lds_warp[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < SK_T / 64; ++i) {
    const int c = lds_warp[i];
    if (i < w) base += c;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

template <bool VEC>
__global__ __launch_bounds__(SK_T) void k_sample(const float* __restrict__ logits, int vocab, int64_t stride,
                                                 const float* __restrict__ temperature,
                                                 const int32_t* __restrict__ top_k, const float* __restrict__ top_p,
                                                 const float* __restrict__ uniform, int32_t* __restrict__ out) {
  __shared__ int hist[256];
  __shared__ int scan_w[SK_T / 64];
  __shared__ uint32_t ck[SK_MAX];  // candidate keys
  __shared__ int ci[SK_MAX];       // candidate indices
  __shared__ float cm[SK_MAX];     // cumulative masses
  __shared__ uint32_t sel_prefix;
  __shared__ int sel_rem, n_cand, cut, n_gt_s, n_eq_s;
  __shared__ float red_v[SK_T / 64];
  __shared__ int red_i[SK_T / 64];

  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* x = logits + (size_t)r * stride;
  const float T = temperature[r];

  if (!(T > 0.f)) {  // greedy: lowest index of the maximum (a NaN counts as the largest, the first NaN wins)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int base = 0; base < vocab; base += SK_T * SK_E) {
      float vv[SK_E];
      load_batch<VEC>(x, vocab, base, vv);
#pragma unroll
      for (int j = 0; j < SK_E; ++j) {
        const int i = batch_index(base, j);
        const float v = vv[j];
        const bool vn = v != v, bn = bv != bv;
        if (i < vocab && ((vn && !bn) || (!vn && !bn && (v > bv || (v == bv && i < bi))) || (vn && bn && i < bi))) {
          bv = v;
          bi = i;
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      const bool on = ov != ov, bn = bv != bv;
      if ((on && !bn) || (!on && !bn && (ov > bv || (ov == bv && oi < bi))) || (on && bn && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      red_v[w] = bv;
      red_i[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int i = 1; i < SK_T / 64; ++i) {
        const float ov = red_v[i];
        const int oi = red_i[i];
        const bool on = ov != ov, bn = bv != bv;
        if ((on && !bn) || (!on && !bn && (ov > bv || (ov == bv && oi < bi))) || (on && bn && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      out[r] = bi;
    }
    return;
  }

  int k = top_k[r];
  k = (k <= 0 || k > SK_MAX) ? SK_MAX : k;
  k = k < vocab ? k : vocab;
  float p = top_p[r];
  p = (p > 0.f && p <= 1.f) ? p : 1.f;
  float u = uniform[r];
  u = u > 0.f ? (u < 1.f ? u : 0.99999994f) : 0.f;

  // ---- 1. key of the k-th largest z: radix select, most significant digit first
  if (tid == 0) {
    sel_prefix = 0u;
    sel_rem = k;
  }
  uint32_t mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += SK_T) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sel_prefix;
    for (int base = 0; base < vocab; base += SK_T * SK_E) {  // wave-uniform trip count: hist_add needs whole waves
      float v[SK_E];
      load_batch<VEC>(x, vocab, base, v);
#pragma unroll
      for (int j = 0; j < SK_E; ++j) {
        const uint32_t key = fkey(v[j] / T);
        hist_add(hist, batch_index(base, j) < vocab && (key & mask) == prefix, (key >> shift) & 255u);
      }
    }
    __syncthreads();
    if (tid == 0) {  // the bin, from the top, where the remaining rank falls
      int rem = sel_rem, b = 255;
      for (; b > 0; --b) {
        if (hist[b] >= rem) break;
        rem -= hist[b];
      }
      sel_rem = rem;
      sel_prefix = prefix | ((uint32_t)b << shift);
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t kth = sel_prefix;

  // ---- 2. candidates: keys above kth (fewer than k), then the ties (all of
  // them when they fit under the cap; the sort below fixes the order, so the
  // slots can be taken in any order).  When the ties overflow the cap, the
  // lowest-index ones are kept: an ordered pass over contiguous chunks.
  if (tid == 0) n_gt_s = 0;
  __syncthreads();
  int my_eq = 0;
  for (int base = 0; base < vocab; base += SK_T * SK_E) {
    float v[SK_E];
    load_batch<VEC>(x, vocab, base, v);
#pragma unroll
    for (int j = 0; j < SK_E; ++j) {
      const int i = batch_index(base, j);
      const uint32_t key = fkey(v[j] / T);
      if (i < vocab && key > kth) {
        const int slot = atomicAdd(&n_gt_s, 1);
        ck[slot] = key;
        ci[slot] = i;
      } else if (i < vocab && key == kth) {
        ++my_eq;
      }
    }
  }
  int tot_eq;
  block_excl_scan(my_eq, scan_w, tot_eq);  // (also orders the slot writes above before the reads below)
  const int tot_gt = n_gt_s;
  if (tid == 0) n_eq_s = tot_eq;
  __syncthreads();
  if (tot_gt + tot_eq <= SK_MAX) {
    for (int base = 0; base < vocab; base += SK_T * SK_E) {
      float v[SK_E];
      load_batch<VEC>(x, vocab, base, v);
#pragma unroll
      for (int j = 0; j < SK_E; ++j) {
        const int i = batch_index(base, j);
        if (i < vocab && fkey(v[j] / T) == kth) {
          const int slot = tot_gt + atomicAdd(&n_eq_s, -1) - 1;  // counts down from tot_eq
          ck[slot] = kth;
          ci[slot] = i;
        }
      }
    }
  } else {
    const int chunk = (vocab + SK_T - 1) / SK_T;
    const int c0 = tid * chunk, c1 = (c0 + chunk) < vocab ? (c0 + chunk) : vocab;
    int n_eq = 0;
    for (int i = c0; i < c1; ++i) n_eq += fkey(x[i] / T) == kth;
    int unused;
    int pos = tot_gt + block_excl_scan(n_eq, scan_w, unused);
    for (int i = c0; i < c1 && pos < SK_MAX; ++i)
      if (fkey(x[i] / T) == kth) {
        ck[pos] = kth;
        ci[pos] = i;
        ++pos;
      }
  }
  const int n = (tot_gt + tot_eq) < SK_MAX ? (tot_gt + tot_eq) : SK_MAX;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  for (int j = n + tid; j < np2; j += SK_T) {  // padding sorts last
    ck[j] = 0u;
    ci[j] = 0x7fffffff;
  }
  __syncthreads();

  // ---- 3. bitonic sort: key descending, index ascending
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride2 = size >> 1; stride2 > 0; stride2 >>= 1) {
      for (int j = tid; j < np2; j += SK_T) {
        const int partner = j ^ stride2;
        if (partner > j) {
          const bool desc = (j & size) == 0;  // this run sorts "before-first" when desc
          const uint32_t ka = ck[j], kb = ck[partner];
          const int ia = ci[j], ib = ci[partner];
          const bool a_first = ka > kb || (ka == kb && ia < ib);
          if (a_first != desc) {
            ck[j] = kb;
            ck[partner] = ka;
            ci[j] = ib;
            ci[partner] = ia;
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- 4. masses in sorted order, cumulative (each thread 4 consecutive candidates, then a block scan)
  const float zmax = x[ci[0]] / T;
  float e[SK_MAX / SK_T];
  float run = 0.f;
#pragma unroll
  for (int q = 0; q < SK_MAX / SK_T; ++q) {
    const int j = tid * (SK_MAX / SK_T) + q;
    e[q] = j < n ? __expf(x[ci[j]] / T - zmax) : 0.f;
    run += e[q];
  }
  // float exclusive scan over threads (fixed order)
  float incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) red_v[w] = incl;
  __syncthreads();
  float base = 0.f;
  for (int i = 0; i < w; ++i) base += red_v[i];
  base += incl - run;
#pragma unroll
  for (int q = 0; q < SK_MAX / SK_T; ++q) {
    base += e[q];
    const int j = tid * (SK_MAX / SK_T) + q;
    if (j < n) cm[j] = base;
  }
  if (tid == 0) {
    n_cand = n;
    cut = n - 1;      // stays if no crossing is found (only with NaN masses)
    out[r] = ci[0];   // likewise for the draw below
  }
  __syncthreads();
  const float total = cm[n - 1];
  // top-p: the first position whose cumulative mass reaches p * total
  for (int j = tid; j < n; j += SK_T)
    if (cm[j] >= p * total && (j == 0 || cm[j - 1] < p * total)) cut = j;
  __syncthreads();
  const int c = cut;
  const float target = u * cm[c];
  for (int j = tid; j <= c; j += SK_T)
    if (cm[j] > target && (j == 0 || cm[j - 1] <= target)) out[r] = ci[j];
}

void launch_sample(const float* logits, int rows, int vocab, int64_t stride, const float* temperature,
                   const int32_t* top_k, const float* top_p, const float* uniform, int32_t* out, hipStream_t s) {
  const bool vec = ((uintptr_t)logits & 15u) == 0 && (stride & 3) == 0;
  if (vec)
    hipLaunchKernelGGL(k_sample<true>, dim3(rows), dim3(SK_T), 0, s, logits, vocab, stride, temperature, top_k, top_p,
                       uniform, out);
  else
    hipLaunchKernelGGL(k_sample<false>, dim3(rows), dim3(SK_T), 0, s, logits, vocab, stride, temperature, top_k,
                       top_p, uniform, out);
}

}  // namespace q3
