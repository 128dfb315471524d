// Temperature / top-k / top-p sampling of logits rows over the whole
// vocabulary, the path that "第 3 章 前向与生成（代码走读）" §4.3
// (Sampler.sample) takes when temperatures are given (the greedy path is the
// lm_head's fused argmax).  Per row r, with T = temperature[r],
// k = top_k[r], p = top_p[r] and the caller's uniform draw u = uniform[r]:
//   T <= 0 (or NaN)  -> greedy: lowest index of the maximum;
//   z = logits / T;
//   candidates: every token with z >= the k-th largest z, ties included
//     (k <= 0 or k >= vocab: every token), ordered by z descending then
//     index ascending;
//   softmax over the candidates, cumulative in that order; keep the
//     shortest prefix whose mass reaches p (p outside (0, 1] means 1);
//   pick the first kept position whose cumulative mass exceeds u times
//     the kept mass.
//
// No sort.  Every decision is a selection in the (z descending, index
// ascending) order, found by radix select over order-preserving 32-bit keys
// of z, most significant 8-bit digit first:
//   - the k-th largest key, by element counts;
//   - the top-p cut and the draw, by probability mass: masses are
//     exp(z - z_max) in 40-bit fixed point (uint64), so every sum is exact
//     integer arithmetic, independent of summation order, and a run is
//     reproducible bit for bit;
//   - inside the final key's group of equal values (equal masses) the
//     position is a division, and the index is the j-th one with that key in
//     index order.
// Each row is split into G contiguous chunks, one 256-thread workgroup each.
// A launch makes one pass over the row: every workgroup histograms its chunk
// in LDS and writes the histogram to the workspace; the last workgroup of the
// row (a ticket) adds the G histograms in chunk order and advances the row's
// state.  Thirteen passes follow an initialising launch:
//   0      row maximum (and the greedy answer) + first top-k digit
//   1..3   top-k digits
//   4..7   top-p digits (rows with p < 1)
//   8..11  draw digits
//   12     the j-th index among equal keys (only when j > 0)
// A pass that does not apply to a row returns at once for that row.
// Fast path: when the top-k select leaves at most min(SP_FAST_CAP, 256 G)
// candidates (ties included), one launch gathers them into the row's mass
// histograms (unused until pass 4, which such a row skips) and a second
// sorts them in one workgroup per row and makes the top-p cut and the draw
// with the same fixed-point arithmetic as the passes (same token); passes
// 4-12 then return at once for that row.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "validate.hpp"

namespace q3 {

constexpr int SP_T = 256;      // threads per workgroup (one per histogram bin)
constexpr int SP_BINS = 256;   // 8-bit digits
constexpr int SP_COPIES = 4;   // LDS histogram copies (lane % 4) against same-bin contention
constexpr int SP_PAD = SP_BINS + 1;
constexpr int SP_PASSES = 13;
constexpr int SP_MAX_G = 32;   // chunks per row at most (q3v::sample_chunks)
constexpr float SP_FIX = 1099511627776.0f;  // 2^40: mass fixed point
constexpr int SP_FAST_CAP = 1024;            // most candidates the fast path sorts (one workgroup)

// Per-row state, written by the initialising launch and by each pass's
// finishing workgroup, read by the next launch.
struct alignas(64) SampRow {
  float inv_t;        // 1 / T
  float p, u;
  int mode;           // 0: done (greedy rows after pass 0, or a result is final); 1: sampling
  int topk;           // 1: a top-k threshold is selected (0 < k < vocab)
  int topp;           // 1: a top-p cut is selected (p < 1)
  uint32_t k;         // rank of the top-k threshold
  float zmax;
  uint32_t lo_key;    // candidates: key >= lo_key (top-k threshold, then top-p cut)
  uint32_t prefix;    // digits selected so far by the running select
  uint32_t tu_key;    // key of the drawn group (pass 12)
  int32_t j;          // position of the drawn token among that key's tokens, in index order
  uint64_t need;      // the running select's remaining count / mass to reach
  uint64_t above;     // mass of the keys above the running select's prefix
  uint64_t kept;      // kept mass (after the top-p cut, or all candidates)
  uint32_t n_cand;    // candidates after the top-k select (ties included)
  int fast;           // 1: the fast path finishes this row
  int n_gath;         // candidates the fast path has gathered so far
};

// order-preserving map of float32 to uint32 (larger float -> larger key);
// -0 maps as +0.  NaN: nan_key.
__device__ __forceinline__ uint32_t skey(float f, uint32_t nan_key) {
  if (f != f) return nan_key;
  if (f == 0.f) f = 0.f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float skey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// fixed-point mass of z (0 for NaN or underflow)
__device__ __forceinline__ uint64_t smass(float z, float zmax) {
  const float w = expf(z - zmax);
  return (w == w && w > 0.f) ? (uint64_t)(w * SP_FIX) : 0ull;
}

struct SampWs {
  SampRow* st;
  int* tick;
  uint32_t* cnt;   // [rows][G][256]
  uint64_t* mass;  // [rows][G][256]
  uint32_t* mini;  // [rows][G][256] lowest index per bin (last draw digit)
  uint64_t* best;  // [rows][G] (key << 32 | ~index) maxima
};
// fast path: the row's candidates as (key << 32 | ~index), in its mass histograms
__device__ __forceinline__ uint64_t* fast_list(const SampWs& ws, int r, int G) {
  return ws.mass + (size_t)r * G * SP_BINS;
}
__device__ __forceinline__ int fast_cap(int G) { return G * SP_BINS < SP_FAST_CAP ? G * SP_BINS : SP_FAST_CAP; }

// inclusive scan of one uint64 per thread over the 256 threads
__device__ __forceinline__ uint64_t block_incl_scan_u64(uint64_t v, uint64_t* lds4) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) lds4[w] = v;
  __syncthreads();
  uint64_t base = 0;
  for (int i = 0; i < w; ++i) base += lds4[i];
  __syncthreads();
  return base + v;
}

__global__ __launch_bounds__(SP_T) void k_sample_init(int rows, int vocab, const float* __restrict__ temperature,
                                                      const int32_t* __restrict__ top_k,
                                                      const float* __restrict__ top_p,
                                                      const float* __restrict__ uniform, SampWs ws) {
  const int r = blockIdx.x * SP_T + threadIdx.x;
  if (r >= rows) return;
  SampRow s{};
  const float t = temperature[r];
  s.mode = t > 0.f ? 1 : 0;
  s.inv_t = t > 0.f ? 1.0f / t : 1.0f;
  const int k = top_k[r];
  s.topk = (k > 0 && k < vocab) ? 1 : 0;
  s.k = s.topk ? (uint32_t)k : 0u;
  const float p = top_p[r];
  s.p = (p > 0.f && p <= 1.f) ? p : 1.f;
  s.topp = s.p < 1.f ? 1 : 0;
  const float u = uniform[r];
  s.u = u > 0.f ? (u < 1.f ? u : 0.99999994f) : 0.f;
  s.lo_key = 0u;
  ws.st[r] = s;
  ws.tick[r] = 0;
}

// One pass (see the file comment) over chunk blockIdx.x of row blockIdx.y.
template <bool VEC>
__global__ __launch_bounds__(SP_T) void k_sample_pass(int pass, const float* __restrict__ logits, int vocab,
                                                      int64_t stride, int G, int chunk, SampWs ws,
                                                      int32_t* __restrict__ out) {
  __shared__ uint32_t h_cnt[SP_COPIES][SP_PAD];
  __shared__ uint64_t h_mass[SP_COPIES][SP_PAD];
  __shared__ uint32_t h_min[SP_COPIES][SP_PAD];
  __shared__ uint64_t red[SP_T / 64];
  __shared__ int is_last;
  __shared__ int found;

  const int r = blockIdx.y, g = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  SampRow s = ws.st[r];
  // which select this pass runs (0: max, 1: top-k, 2: top-p, 3: draw, 4: tie index)
  const int kind = pass == 0 ? 0 : pass <= 3 ? 1 : pass <= 7 ? 2 : pass <= 11 ? 3 : 4;
  const bool greedy = pass == 0 && s.mode == 0;
  if (!greedy) {
    if (s.mode != 1) return;
    if (kind == 1 && !s.topk) return;
    if (kind == 2 && !s.topp) return;
    if (kind == 4 && s.j <= 0) return;
  }
  // digit 3 is bits 31..24; pass 0 takes the first top-k digit
  const int digit = kind == 0 ? 3 : kind == 1 ? 3 - pass : kind == 2 ? 7 - pass : kind == 3 ? 11 - pass : 0;
  const int shift = 8 * digit;
  const uint32_t hi_mask = digit == 3 ? 0u : ~((1u << (shift + 8)) - 1u);
  const bool do_cnt = greedy ? false : (kind == 0 ? s.topk != 0 : kind != 4);
  const bool do_mass = kind == 2 || kind == 3;
  const bool do_min = kind == 3 && digit == 0;

  const float* x = logits + (size_t)r * stride;
  const int c0 = g * chunk, c1 = (c0 + chunk) < vocab ? (c0 + chunk) : vocab;
  const float inv_t = greedy ? 1.0f : s.inv_t;
  const uint32_t nan_key = greedy ? 0xffffffffu : 0u;
  const uint32_t lo = kind == 2 ? s.lo_key : kind == 3 ? s.lo_key : 0u;
  const uint32_t prefix = s.prefix;
  const float zmax = s.zmax;
  const int cp = lane & (SP_COPIES - 1);

  for (int i = tid; i < SP_COPIES * SP_PAD; i += SP_T) {
    (&h_cnt[0][0])[i] = 0u;
    (&h_mass[0][0])[i] = 0ull;
    (&h_min[0][0])[i] = 0xffffffffu;
  }
  __syncthreads();

  uint64_t best = 0;       // kind 0: max of (key << 32 | ~index)
  uint32_t n_tie = 0;      // kind 4: elements equal to tu_key
  auto visit = [&](float v, int i) {
    const float z = v * inv_t;
    const uint32_t key = skey(z, nan_key);
    if (kind == 0) {
      const uint64_t c = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)i;
      best = c > best ? c : best;
      if (do_cnt) atomicAdd(&h_cnt[cp][key >> 24], 1u);
      return;
    }
    if (kind == 4) {
      n_tie += key == s.tu_key;
      return;
    }
    if (key < lo || (key & hi_mask) != prefix) return;
    const uint32_t b = (key >> shift) & 255u;
    atomicAdd(&h_cnt[cp][b], 1u);
    if (do_mass) atomicAdd((unsigned long long*)&h_mass[cp][b], (unsigned long long)smass(z, zmax));
    if (do_min) atomicMin(&h_min[cp][b], (uint32_t)i);
  };
  if (VEC) {
    // c0 is a multiple of 4 and the row 16-byte aligned; 4 vectors per thread in flight
    constexpr int U = 4;
    int i = c0 + 4 * tid;
    for (; i + 4 * SP_T * (U - 1) + 3 < c1; i += 4 * SP_T * U) {
      f32x4 q[U];
#pragma unroll
      for (int u = 0; u < U; ++u) q[u] = *reinterpret_cast<const f32x4*>(x + i + 4 * SP_T * u);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) visit(q[u][c], i + 4 * SP_T * u + c);
    }
    for (; i < c1; i += 4 * SP_T) {
      if (i + 3 < c1) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(x + i);
#pragma unroll
        for (int c = 0; c < 4; ++c) visit(q[c], i + c);
      } else {
        for (int c = 0; c < 4 && i + c < c1; ++c) visit(x[i + c], i + c);
      }
    }
  } else {
    for (int i = c0 + tid; i < c1; i += SP_T) visit(x[i], i);
  }

  // ---- this chunk's result to the workspace
  const size_t rg = (size_t)r * G + g;
  if (kind == 0) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t t = __shfl_xor(best, o, 64);
      best = t > best ? t : best;
    }
    if (lane == 0) red[tid >> 6] = best;
  } else if (kind == 4) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n_tie += __shfl_xor(n_tie, o, 64);
    if (lane == 0) red[tid >> 6] = n_tie;
  }
  __syncthreads();
  if (kind == 0 || kind == 4) {
    if (tid == 0) {
      uint64_t v = red[0];
      for (int w = 1; w < SP_T / 64; ++w) v = kind == 0 ? (red[w] > v ? red[w] : v) : v + red[w];
      st_dev_u64(&ws.best[rg], v);
    }
  }
  if (do_cnt) {
    const int b = tid;
    uint32_t c = 0, mi = 0xffffffffu;
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < SP_COPIES; ++k) {
      c += h_cnt[k][b];
      m += h_mass[k][b];
      mi = h_min[k][b] < mi ? h_min[k][b] : mi;
    }
    st_dev_u32(&ws.cnt[rg * SP_BINS + b], c);
    if (do_mass) st_dev_u64(&ws.mass[rg * SP_BINS + b], m);
    if (do_min) st_dev_u32(&ws.mini[rg * SP_BINS + b], mi);
  }
  vm_drain();
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(&ws.tick[r], 1) == G - 1;
  __syncthreads();
  if (!is_last) return;

  // ---- last workgroup of the row: combine the G chunks in chunk order.
  // Every device-coherent load a thread needs is issued before the first is
  // used, so their latencies overlap.
  if (tid == 0) {
    __hip_atomic_store(&ws.tick[r], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    found = 0;
  }
  __shared__ uint64_t per_chunk[SP_MAX_G];
  if (kind == 0 || kind == 4) {
    if (tid < G) per_chunk[tid] = ld_dev_u64(&ws.best[(size_t)r * G + tid]);
    __syncthreads();
  }
  if (kind == 0 && tid == 0) {
    uint64_t v = 0;
    for (int q = 0; q < G; ++q) v = per_chunk[q] > v ? per_chunk[q] : v;
    const int idx = (int)~(uint32_t)v;
    out[r] = idx;  // the greedy answer, or the fallback of a sampling row (never used unless masses vanish)
    if (greedy) {
      ws.st[r].mode = 0;
    } else {
      ws.st[r].zmax = skey_inv((uint32_t)(v >> 32));
    }
  }
  if (kind == 4) {
    // the chunk holding the j-th tied token, then that token by an ordered scan of the chunk
    __shared__ int tg, tj;
    if (tid == 0) {
      int j = s.j, q = 0;
      for (; q < G; ++q) {
        const int n = (int)per_chunk[q];
        if (j < n) break;
        j -= n;
      }
      tg = q < G ? q : G - 1;
      tj = j;
    }
    __syncthreads();
    const int q0 = tg * chunk, q1 = (q0 + chunk) < vocab ? (q0 + chunk) : vocab;
    int before = 0;
    for (int base = q0; base < q1; base += SP_T) {  // uniform trip count
      const int i = base + tid;
      const bool hit = i < q1 && skey(x[i] * s.inv_t, 0u) == s.tu_key;
      const uint64_t bal = __ballot(hit);
      const int wn = __popcll(bal);
      if (lane == 0) red[tid >> 6] = (uint64_t)wn;
      __syncthreads();
      int wbefore = 0, tot = 0;
      for (int w = 0; w < SP_T / 64; ++w) {
        if (w < (tid >> 6)) wbefore += (int)red[w];
        tot += (int)red[w];
      }
      const int rank = before + wbefore + __popcll(bal & ((1ull << lane) - 1ull));
      if (hit && rank == tj) {
        out[r] = i;
        found = 1;
      }
      before += tot;
      __syncthreads();
      if (found || before > tj) break;
    }
    return;
  }
  if (!do_cnt) return;

  // per-bin totals over the chunks (thread b holds bin 255 - b, so an
  // inclusive scan over threads is the suffix sum from the top bin down):
  // count, mass and lowest index of the bin
  const int b = SP_BINS - 1 - tid;
  uint32_t n_b = 0, min_b = 0xffffffffu;
  uint64_t m_b = 0;
  {
    uint32_t c[SP_MAX_G], mi[SP_MAX_G];
    uint64_t m[SP_MAX_G];
#pragma unroll
    for (int q = 0; q < SP_MAX_G; ++q) {
      const size_t e = ((size_t)r * G + (q < G ? q : G - 1)) * SP_BINS + b;
      c[q] = ld_dev_u32(&ws.cnt[e]);
      m[q] = do_mass ? ld_dev_u64(&ws.mass[e]) : 0ull;
      mi[q] = do_min ? ld_dev_u32(&ws.mini[e]) : 0xffffffffu;
    }
#pragma unroll
    for (int q = 0; q < SP_MAX_G; ++q) {
      if (q < G) {
        n_b += c[q];
        m_b += m[q];
        min_b = mi[q] < min_b ? mi[q] : min_b;
      }
    }
  }
  const uint64_t v = do_mass ? m_b : (uint64_t)n_b;
  const uint64_t incl = block_incl_scan_u64(v, red);
  __shared__ uint64_t grand;
  if (tid == SP_T - 1) grand = incl;
  __syncthreads();

  // the threshold this select must reach, fixed on its first digit
  uint64_t need = s.need;
  if (digit == 3) {
    if (kind == 1 || (kind == 0 && s.topk)) {
      need = s.k;
    } else if (kind == 2) {  // top-p: the shortest prefix whose mass reaches p of all candidates
      const double pz = (double)s.p * (double)grand;
      uint64_t pp = (uint64_t)ceil(pz);
      pp = pp < 1 ? 1 : (pp > grand ? grand : pp);
      need = pp;
    } else {  // draw: first cumulative mass above u * kept
      const uint64_t kept = s.topp ? s.kept : grand;
      const uint64_t target = (uint64_t)floor((double)s.u * (double)kept);
      need = target + 1;
      if (tid == 0) ws.st[r].kept = kept;
    }
  }
  const uint64_t excl = incl - v;
  const bool mine = need >= 1 && excl < need && incl >= need;
  if (mine) found = 1;
  __syncthreads();
  if (!found) {
    // masses vanished (a non-finite row): keep the row's maximum (written by pass 0)
    if (tid == 0) ws.st[r].mode = 0;
    return;
  }
  if (mine) {
    const uint32_t key = prefix | ((uint32_t)b << shift);
    const uint64_t rem = need - excl;  // >= 1
    const uint64_t above = (digit == 3 ? 0ull : s.above) + excl;
    SampRow& o = ws.st[r];
    if (digit != 0) {
      o.prefix = key;
      o.need = rem;
      o.above = above;
    } else {
      // the selected key's group: every member has the same z, hence the same mass
      o.prefix = 0u;
      o.need = 0;
      o.above = 0;
      if (kind <= 1) {
        o.lo_key = key;  // candidates: key >= the k-th largest key
        const uint64_t n_cand = above + n_b;
        o.n_cand = (uint32_t)(n_cand < 0xffffffffull ? n_cand : 0xffffffffull);
        o.fast = n_cand <= (uint64_t)fast_cap(G) ? 1 : 0;
      } else if (kind == 2) {
        const uint64_t w = n_b ? m_b / n_b : 0;
        uint64_t keep = w ? (rem + w - 1) / w : n_b;
        keep = keep > n_b ? n_b : (keep < 1 ? 1 : keep);
        o.kept = above + keep * w;
        o.lo_key = key;  // the cut's group: only its first `keep` members are kept
      } else {
        const uint64_t w = n_b ? m_b / n_b : 0;
        uint64_t jj = w ? (rem - 1) / w : 0;
        jj = jj >= n_b ? (n_b ? n_b - 1 : 0) : jj;
        o.tu_key = key;
        o.j = (int32_t)jj;
        if (jj == 0) {
          out[r] = (int)min_b;
          o.mode = 0;
        }
      }
    }
  }
}

// ---- fast path, launch 1: chunk blockIdx.x of row blockIdx.y appends its
// candidates (key >= lo_key) to the row's list.  Each thread takes 16
// values per step (four 16-byte loads in flight when VEC); a wave with hits
// reserves its slots with one atomic add.
template <bool VEC>
__global__ __launch_bounds__(SP_T) void k_sample_gather(const float* __restrict__ logits, int vocab, int64_t stride,
                                                        int G, int chunk, SampWs ws) {
  constexpr int E = 16;
  const int r = blockIdx.y, g = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const SampRow s = ws.st[r];
  if (s.mode != 1 || !s.fast) return;
  const float* x = logits + (size_t)r * stride;
  const int c0 = g * chunk, c1 = (c0 + chunk) < vocab ? (c0 + chunk) : vocab;
  const float inv_t = s.inv_t;
  const uint32_t lo = s.lo_key;
  uint64_t* list = fast_list(ws, r, G);
  const int cap = fast_cap(G);
  // one step: value e of the thread is element idx(e); uniform trip count
  for (int step = c0; step < c1; step += E * SP_T) {
    float v[E];
    int idx[E];
#pragma unroll
    for (int e = 0; e < E; ++e) idx[e] = VEC ? step + 4 * tid + 4 * SP_T * (e >> 2) + (e & 3) : step + tid + SP_T * e;
    if (VEC && step + E * SP_T <= c1) {
#pragma unroll
      for (int u = 0; u < E / 4; ++u) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(x + idx[4 * u]);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[4 * u + c] = q[c];
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = idx[e] < c1 ? x[idx[e]] : 0.f;
    }
    uint32_t key[E];
    uint32_t hm = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      key[e] = skey(v[e] * inv_t, 0u);
      hm |= (uint32_t)(idx[e] < c1 && key[e] >= lo) << e;
    }
    const int cnt = __popc(hm);
    if (__ballot(cnt != 0) == 0ull) continue;
    int incl = cnt;  // inclusive scan of the counts over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    int wbase = 0;
    if (lane == 63) wbase = atomicAdd(&ws.st[r].n_gath, incl);
    wbase = __shfl(wbase, 63, 64);
    int pos = wbase + incl - cnt;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((hm >> e) & 1u) {
        if (pos < cap) list[pos] = ((uint64_t)key[e] << 32) | (uint32_t)~(uint32_t)idx[e];
        ++pos;
      }
  }
}

// ---- fast path, launch 2: one workgroup of SP_FT threads per row sorts its
// candidates by (z descending, index ascending), takes the inclusive mass
// sums, and makes the top-p cut and the draw with the passes' integer
// arithmetic: the cut's group keeps ceil(rem / w) members, the draw lands on
// member (rem - 1) / w of its group, w being the (equal) mass of one member.
constexpr int SP_FT = SP_FAST_CAP;  // one candidate per thread
__global__ __launch_bounds__(SP_FT) void k_sample_finish(int G, SampWs ws, int32_t* __restrict__ out) {
  constexpr int N = SP_FAST_CAP;
  __shared__ uint64_t e[N];
  __shared__ uint64_t cum[N];
  __shared__ uint64_t red[SP_FT / 64];
  __shared__ int pos_c, pos_s, cnt_g;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const SampRow s = ws.st[r];
  if (s.mode != 1 || !s.fast) return;
  // a count that differs from the select's (cannot happen) leaves the row to the passes
  const int n = s.n_gath;
  if (n < 1 || n > fast_cap(G) || (uint32_t)n != s.n_cand) return;
  int P = 1;  // sort the next power of two: entries n .. P-1 are 0 and sort last (no entry is 0)
  while (P < n) P <<= 1;
  e[tid] = tid < n ? fast_list(ws, r, G)[tid] : 0ull;
  __syncthreads();
  // bitonic sort, descending; thread tid owns the pair (tid, tid ^ j) when tid is its lower end
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int ij = tid ^ j;
      if (tid < P && ij > tid) {
        const uint64_t a = e[tid], b = e[ij];
        if (((tid & k) == 0) ? (a < b) : (a > b)) {
          e[tid] = b;
          e[ij] = a;
        }
      }
      __syncthreads();
    }
  // inclusive sums of the fixed-point masses
  uint64_t v = tid < n ? smass(skey_inv((uint32_t)(e[tid] >> 32)), s.zmax) : 0ull;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) red[wv] = v;
  __syncthreads();
  for (int w = 0; w < wv; ++w) v += red[w];
  cum[tid] = v;
  __syncthreads();
  const uint64_t grand = cum[n - 1];
  // the position where the inclusive sum first reaches `need`, its key's
  // group (first position and size), or -1
  auto cross = [&](uint64_t need) {
    __syncthreads();  // the previous call's results have been read
    if (tid == 0) {
      pos_c = -1;
      cnt_g = 0;
    }
    __syncthreads();
    if (tid < n && cum[tid] >= need && (tid == 0 || cum[tid - 1] < need)) pos_c = tid;
    __syncthreads();
    const int c = pos_c;
    if (c >= 0 && tid < n) {
      const uint32_t kc = (uint32_t)(e[c] >> 32);
      if ((uint32_t)(e[tid] >> 32) == kc) {
        atomicAdd(&cnt_g, 1);
        if (tid == 0 || (uint32_t)(e[tid - 1] >> 32) != kc) pos_s = tid;
      }
    }
    __syncthreads();
    return c;
  };
  uint64_t kept = grand;
  if (s.topp) {
    const double pz = (double)s.p * (double)grand;
    uint64_t pp = (uint64_t)ceil(pz);
    pp = pp < 1 ? 1 : (pp > grand ? grand : pp);
    if (cross(pp) < 0) {  // masses vanished: keep the row's maximum (written by pass 0)
      if (tid == 0) ws.st[r].mode = 0;
      return;
    }
    const int sg = pos_s, ng = cnt_g;
    const uint64_t above = sg > 0 ? cum[sg - 1] : 0ull;
    const uint64_t w = cum[sg] - above;  // one member's mass
    const uint64_t rem = pp - above;
    uint64_t keep = w ? (rem + w - 1) / w : (uint64_t)ng;
    keep = keep > (uint64_t)ng ? (uint64_t)ng : (keep < 1 ? 1 : keep);
    kept = above + keep * w;
  }
  const uint64_t need = (uint64_t)floor((double)s.u * (double)kept) + 1;
  if (cross(need) < 0) {
    if (tid == 0) ws.st[r].mode = 0;
    return;
  }
  if (tid == 0) {
    const int sg = pos_s, ng = cnt_g;
    const uint64_t above = sg > 0 ? cum[sg - 1] : 0ull;
    const uint64_t w = cum[sg] - above;
    const uint64_t rem = need - above;
    uint64_t jj = w ? (rem - 1) / w : 0;
    jj = jj >= (uint64_t)ng ? (ng ? (uint64_t)ng - 1 : 0) : jj;
    out[r] = (int32_t)~(uint32_t)e[sg + (int)jj];
    ws.st[r].mode = 0;
  }
}

static_assert(sizeof(SampRow) == q3v::SAMPLE_ROW_BYTES, "row state size must match the workspace layout");

void launch_sample(const float* logits, int rows, int vocab, int64_t stride, const float* temperature,
                   const int32_t* top_k, const float* top_p, const float* uniform, int32_t* out, void* wsp,
                   hipStream_t s) {
  const int G = q3v::sample_chunks(rows, vocab);
  int chunk = (vocab + G - 1) / G;
  chunk = (chunk + 3) & ~3;
  const q3v::SampleWsLayout L = q3v::sample_ws_layout(rows, vocab);
  char* p = static_cast<char*>(wsp);
  SampWs ws;
  ws.st = reinterpret_cast<SampRow*>(p + L.st);
  ws.tick = reinterpret_cast<int*>(p + L.tick);
  ws.cnt = reinterpret_cast<uint32_t*>(p + L.cnt);
  ws.mass = reinterpret_cast<uint64_t*>(p + L.mass);
  ws.mini = reinterpret_cast<uint32_t*>(p + L.mini);
  ws.best = reinterpret_cast<uint64_t*>(p + L.best);
  hipLaunchKernelGGL(k_sample_init, dim3((rows + SP_T - 1) / SP_T), dim3(SP_T), 0, s, rows, vocab, temperature,
                     top_k, top_p, uniform, ws);
  const bool vec = ((uintptr_t)logits & 15u) == 0 && (stride & 3) == 0;
  for (int pass = 0; pass < SP_PASSES; ++pass) {
    if (pass == 4) {  // after the top-k select: the fast path for rows with few candidates
      if (vec)
        hipLaunchKernelGGL(k_sample_gather<true>, dim3(G, rows), dim3(SP_T), 0, s, logits, vocab, stride, G, chunk, ws);
      else
        hipLaunchKernelGGL(k_sample_gather<false>, dim3(G, rows), dim3(SP_T), 0, s, logits, vocab, stride, G, chunk,
                           ws);
      hipLaunchKernelGGL(k_sample_finish, dim3(rows), dim3(SP_FT), 0, s, G, ws, out);
    }
    if (vec)
      hipLaunchKernelGGL(k_sample_pass<true>, dim3(G, rows), dim3(SP_T), 0, s, pass, logits, vocab, stride, G, chunk,
                         ws, out);
    else
      hipLaunchKernelGGL(k_sample_pass<false>, dim3(G, rows), dim3(SP_T), 0, s, pass, logits, vocab, stride, G,
                         chunk, ws, out);
  }
}

}  // namespace q3
