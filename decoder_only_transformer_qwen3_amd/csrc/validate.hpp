// Host-only argument validation and workspace layout for the C ABI.
// Plain C++ (no HIP), so it is also built and tested on its own with
// g++ and the address/undefined-behaviour sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/q3.h"

namespace q3v {

constexpr int PART_MAX_SPLIT = 8;    // skinny-GEMM K splits held in the workspace
constexpr int DEC_SPLIT_MAX = 64;    // decode-attention splits held in the workspace
constexpr int SKINNY_MAX_ROWS = 128;  // row counts up to this use the skinny GEMM
constexpr int LM_HEAD_MAX_ROWS = 64;   // rows per lm_head launch
constexpr int64_t MAX_TOKENS = 1 << 22;

struct WsLayout {
  size_t resid, h, qkv, ao, act, part, tpart, apart, amax, fh, ssq, tick;
  size_t total;
};

// Byte offsets of every workspace region for `batch` x `n_tokens` (256-B aligned).
WsLayout ws_layout(int32_t batch, int32_t n_tokens);
// `rows` token rows over `batch` sequences (packed calls: rows = tokens of
// all sequences); one_token: every sequence adds exactly one token (decode).
WsLayout ws_layout_rows(int32_t batch, int64_t rows, bool one_token);

// Tiled-GEMM K splits for row counts between the skinny and the persistent
// paths: a 128 x 128 output tile per workgroup leaves most of the chip idle
// when there are few tiles (128 rows x 1024 features: 8 tiles), so the K
// range is split until about 256 workgroups run, each with at least two
// 64-wide K steps, at most 16 splits.  The splits' fp32 sums go to the
// workspace and a second kernel adds them in split order.
inline int64_t tiled_tiles(int64_t M, int N, bool silu) {
  return ((M + 127) / 128) * (silu ? (N / 2) / 64 : N / 128);
}
inline int tiled_splits(int64_t M, int N, int K, bool silu) {
  if (M <= SKINNY_MAX_ROWS || (M >= 2048 && N % 256 == 0)) return 1;  // skinny / persistent paths
  const int64_t tiles = tiled_tiles(M, N, silu);
  const int ksteps = K / 64;
  int s = 1;
  while (tiles * s < 256 && 2 * s <= 16 && ksteps % (2 * s) == 0 && ksteps / (2 * s) >= 2) s *= 2;
  return s;
}
// Partial-sum bytes of one layer's four projections at `rows` rows (the largest).
inline int64_t tiled_part_bytes(int64_t rows) {
  int64_t b = 0;
  const int64_t c[4][3] = {{Q3_QKV_ROWS, Q3_HIDDEN, 0},
                           {Q3_HIDDEN, Q3_N_HEADS * Q3_HEAD_DIM, 0},
                           {2 * Q3_INTER, Q3_HIDDEN, 1},
                           {Q3_HIDDEN, Q3_INTER, 0}};
  for (const auto& p : c) {
    const int s = tiled_splits(rows, (int)p[0], (int)p[1], p[2] != 0);
    if (s > 1) {
      const int64_t t = (int64_t)s * rows * p[0] * 4;
      b = t > b ? t : b;
    }
  }
  return b;
}

// Workgroup tickets in the workspace: 64 column blocks + 8 per sequence.
inline int ticket_count(int32_t batch) { return 64 + 8 * batch + 1; }
inline int head_ticket(int32_t batch) { return 64 + 8 * batch; }  // index of the lm_head's ticket

// Decode attention over `batch` sequences of at most `ctx` keys: whether it
// runs in its streaming configuration (caches far larger than the
// last-level cache), and its number of splits.
bool decode_streaming(int32_t batch, int32_t ctx);
int decode_splits(int32_t batch, int32_t ctx);

int check_layer_call(const q3_layer_weights* w, const float* rope_cos, const float* rope_sin, const void* k_layer,
                     const void* v_layer, int32_t batch, int32_t n_tokens, int32_t max_seq, int32_t start_pos,
                     const float* residual, const void* ws, size_t ws_bytes);

int check_prefill_call(const q3_model* m, const q3_kv* kv, int32_t batch, int32_t prompt_len, const int32_t* ids,
                       const float* last_logits, const int32_t* next_ids, const int32_t* seq_lens, const void* ws,
                       size_t ws_bytes);

int check_decode_call(const q3_model* m, const q3_kv* kv, int32_t batch, const int32_t* in_ids,
                      const int32_t* seq_lens, int32_t max_len_hint, const float* logits, const int32_t* out_ids,
                      const void* ws, size_t ws_bytes);

int check_rope_convert_call(const void* w_qkv, const void* q_norm, const void* k_norm, const void* w_qkv_out,
                            const void* q_norm_out, const void* k_norm_out);
// Sampling: each row is split into sample_chunks() contiguous chunks, one
// workgroup each (about 512 workgroups in all, at most 32 per row, chunks of
// at least 1024 tokens); the workspace holds per-row state and per-chunk
// 256-bin histograms.
constexpr size_t SAMPLE_ROW_BYTES = 128;
inline int sample_chunks(int32_t rows, int32_t vocab) {
  int g = (int)((512 + (int64_t)rows - 1) / rows);
  g = g > 32 ? 32 : g;
  const int by_len = vocab / 1024;
  g = g > by_len ? by_len : g;
  return g < 1 ? 1 : g;
}
struct SampleWsLayout {
  size_t st, tick, cnt, mass, mini, best, total;
};
SampleWsLayout sample_ws_layout(int32_t rows, int32_t vocab);
constexpr int32_t SAMPLE_MAX_ROWS = 1 << 16;
int check_sample_call(const float* logits, int32_t rows, int32_t vocab, int64_t row_stride, const float* temperature,
                      const int32_t* top_k, const float* top_p, const float* uniform, const int32_t* out_idx,
                      const void* ws, size_t ws_bytes);
int check_prefill_packed_call(const q3_model* m, const q3_kv* kv, int32_t n_seqs, int32_t n_tokens,
                              const int32_t* ids, const int32_t* cu_seqlens, const int32_t* start_pos,
                              int32_t max_seq_tokens, const float* last_logits, const int32_t* next_ids,
                              const int32_t* seq_lens, const void* ws, size_t ws_bytes);
int check_linear_call(const void* x, const void* w, const void* out, int32_t m, int32_t n, int32_t k, int32_t ldo,
                      int32_t epilogue);

int check_attn_prefill_call(const void* q, const void* k_layer, const void* v_layer, int32_t batch, int32_t n_tokens,
                            int32_t start_pos, int32_t max_seq, const void* out);
int check_attn_prefill_qkv_call(const void* qkv, const void* q_norm, const void* k_norm, const float* rope_cos,
                                const float* rope_sin, const void* k_layer, const void* v_layer, int32_t batch,
                                int32_t n_tokens, int32_t start_pos, int32_t max_seq, int32_t write_kv,
                                const void* out);

int check_attn_decode_call(const void* qkv, const void* q_norm, const void* k_norm, const float* rope_cos,
                           const float* rope_sin, const void* k_layer, const void* v_layer, int32_t batch,
                           int32_t max_seq, const int32_t* positions, int32_t max_len_hint, const void* out,
                           const void* ws, size_t ws_bytes);

int check_argmax_call(const float* logits, int32_t rows, int32_t vocab, int64_t row_stride, const int32_t* out_idx);

}  // namespace q3v
