// Host-only validation of C-ABI arguments (see validate.hpp).  The order of
// checks fixes which code a call with several faults gets:
// NULL, then SHAPE, then POSITION, then ALIGN, then WORKSPACE.
#include "validate.hpp"

namespace q3v {

static inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

WsLayout ws_layout(int32_t batch, int32_t n_tokens) {
  if (batch < 1 || n_tokens < 1) return WsLayout{};
  return ws_layout_rows(batch, (int64_t)batch * n_tokens, n_tokens == 1);
}

WsLayout ws_layout_rows(int32_t batch, int64_t rows, bool one_token) {
  WsLayout L{};
  if (batch < 1 || rows < 1) return L;
  const size_t M = (size_t)rows;
  const int32_t n_tokens = one_token ? 1 : 2;  // only "one token per sequence" matters below
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = up256(off + bytes);
    return at;
  };
  L.resid = take(M * Q3_HIDDEN * 4);
  L.h = take(M * Q3_HIDDEN * 2);
  L.qkv = take(M * Q3_QKV_ROWS * 2);
  L.ao = take(M * Q3_N_HEADS * Q3_HEAD_DIM * 2);
  L.act = take(M * Q3_INTER * 2);
  L.part = take(M <= (size_t)SKINNY_MAX_ROWS ? (size_t)PART_MAX_SPLIT * M * Q3_HIDDEN * 4 : 0);
  L.tpart = take((size_t)tiled_part_bytes((int64_t)M));
  L.apart = take(n_tokens == 1 ? (size_t)batch * Q3_N_HEADS * DEC_SPLIT_MAX * (Q3_HEAD_DIM + 2) * 4 : 0);
  L.amax = take((size_t)batch * (Q3_VOCAB / 16) * 8);
  L.fh = take((size_t)batch * Q3_HIDDEN * 2);
  L.ssq = take(M * (Q3_HIDDEN / 4) * 4);
  L.tick = take((size_t)ticket_count(batch) * 4);
  L.total = off;
  return L;
}

bool decode_streaming(int32_t batch, int32_t ctx) {
  // the layers' caches together (4 KB per position, sequence and layer)
  // outgrow the 256 MB last-level cache
  return (double)batch * ctx * 4096.0 * Q3_N_LAYERS > 128.0 * (1 << 20);
}

int decode_splits(int32_t batch, int32_t ctx) {
  // one wave of launches: streaming, one 8-wave workgroup per CU with at
  // least 512 keys (two 32-key tiles per wave) per split; otherwise two
  // 4-wave workgroups per CU with at least 256 keys per split
  const bool streaming = decode_streaming(batch, ctx);
  const int target_workgroups = streaming ? 256 : 512;
  const int min_keys = streaming ? 512 : 256;
  const int pairs = batch * Q3_N_KV_HEADS;
  int s = (target_workgroups + pairs - 1) / pairs;
  const int cap = (ctx + min_keys - 1) / min_keys;
  if (s > cap) s = cap;
  if (s > DEC_SPLIT_MAX) s = DEC_SPLIT_MAX;
  if (s < 1) s = 1;
  return s;
}

static int layer_ptrs_null(const q3_layer_weights* w) {
  return !w->input_norm || !w->w_qkv || !w->q_norm || !w->k_norm || !w->w_o || !w->post_norm || !w->w_gate_up ||
         !w->w_down;
}
static int layer_ptrs_misaligned(const q3_layer_weights* w) {
  return !al16(w->input_norm) || !al16(w->w_qkv) || !al16(w->q_norm) || !al16(w->k_norm) || !al16(w->w_o) ||
         !al16(w->post_norm) || !al16(w->w_gate_up) || !al16(w->w_down);
}
static int model_null(const q3_model* m) {
  if (!m->embed || !m->final_norm || !m->rope_cos || !m->rope_sin) return 1;
  for (int l = 0; l < Q3_N_LAYERS; ++l)
    if (layer_ptrs_null(&m->layer[l])) return 1;
  return 0;
}
static int model_misaligned(const q3_model* m) {
  if (!al16(m->embed) || !al16(m->final_norm) || !al16(m->rope_cos) || !al16(m->rope_sin)) return 1;
  for (int l = 0; l < Q3_N_LAYERS; ++l)
    if (layer_ptrs_misaligned(&m->layer[l])) return 1;
  return 0;
}

int check_layer_call(const q3_layer_weights* w, const float* rope_cos, const float* rope_sin, const void* k_layer,
                     const void* v_layer, int32_t batch, int32_t n_tokens, int32_t max_seq, int32_t start_pos,
                     const float* residual, const void* ws, size_t ws_bytes) {
  if (!w || !rope_cos || !rope_sin || !k_layer || !v_layer || !residual || !ws) return Q3_ERR_NULL;
  if (layer_ptrs_null(w)) return Q3_ERR_NULL;
  if (batch < 1 || n_tokens < 1 || max_seq < 8 || max_seq > Q3_MAX_POS || (max_seq % 8) != 0) return Q3_ERR_SHAPE;
  if ((int64_t)batch * n_tokens > MAX_TOKENS) return Q3_ERR_SHAPE;
  if (start_pos < 0 || (int64_t)start_pos + n_tokens > max_seq) return Q3_ERR_POSITION;
  if (layer_ptrs_misaligned(w) || !al16(rope_cos) || !al16(rope_sin) || !al16(k_layer) || !al16(v_layer) ||
      !al16(residual) || !al16(ws))
    return Q3_ERR_ALIGN;
  if (ws_bytes < ws_layout(batch, n_tokens).total) return Q3_ERR_WORKSPACE;
  return Q3_OK;
}

int check_prefill_call(const q3_model* m, const q3_kv* kv, int32_t batch, int32_t prompt_len, const int32_t* ids,
                       const float* last_logits, const int32_t* next_ids, const int32_t* seq_lens, const void* ws,
                       size_t ws_bytes) {
  if (!m || !kv || !ids || !next_ids || !seq_lens || !ws) return Q3_ERR_NULL;
  if (model_null(m) || !kv->k || !kv->v) return Q3_ERR_NULL;
  if (kv->batch < 1 || kv->max_seq < 8 || kv->max_seq > Q3_MAX_POS || (kv->max_seq % 8) != 0) return Q3_ERR_SHAPE;
  if (batch < 1 || batch > kv->batch || prompt_len < 1) return Q3_ERR_SHAPE;
  if ((int64_t)batch * prompt_len > MAX_TOKENS) return Q3_ERR_SHAPE;
  if (prompt_len > kv->max_seq) return Q3_ERR_POSITION;
  if (model_misaligned(m) || !al16(kv->k) || !al16(kv->v) || !al4(ids) || !al4(next_ids) || !al4(seq_lens) ||
      (last_logits && !al16(last_logits)) || !al16(ws))
    return Q3_ERR_ALIGN;
  if (ws_bytes < ws_layout(batch, prompt_len).total) return Q3_ERR_WORKSPACE;
  return Q3_OK;
}

int check_decode_call(const q3_model* m, const q3_kv* kv, int32_t batch, const int32_t* in_ids,
                      const int32_t* seq_lens, int32_t max_len_hint, const float* logits, const int32_t* out_ids,
                      const void* ws, size_t ws_bytes) {
  if (!m || !kv || !in_ids || !seq_lens || !out_ids || !ws) return Q3_ERR_NULL;
  if (model_null(m) || !kv->k || !kv->v) return Q3_ERR_NULL;
  if (kv->batch < 1 || kv->max_seq < 8 || kv->max_seq > Q3_MAX_POS || (kv->max_seq % 8) != 0) return Q3_ERR_SHAPE;
  if (batch < 1 || batch > kv->batch) return Q3_ERR_SHAPE;
  if (max_len_hint < 1 || max_len_hint > kv->max_seq) return Q3_ERR_POSITION;
  if (model_misaligned(m) || !al16(kv->k) || !al16(kv->v) || !al4(in_ids) || !al4(seq_lens) || !al4(out_ids) ||
      (logits && !al16(logits)) || !al16(ws))
    return Q3_ERR_ALIGN;
  if (ws_bytes < ws_layout(batch, 1).total) return Q3_ERR_WORKSPACE;
  return Q3_OK;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_rope_convert_call(const void* w_qkv, const void* q_norm, const void* k_norm, const void* w_qkv_out,
                            const void* q_norm_out, const void* k_norm_out) {
  if (!w_qkv || !q_norm || !k_norm || !w_qkv_out || !q_norm_out || !k_norm_out) return Q3_ERR_NULL;
  const size_t wb = (size_t)Q3_QKV_ROWS * Q3_HIDDEN * 2, gb = (size_t)Q3_HEAD_DIM * 2;
  const void* in[3] = {w_qkv, q_norm, k_norm};
  const size_t in_n[3] = {wb, gb, gb};
  const void* out[3] = {w_qkv_out, q_norm_out, k_norm_out};
  const size_t out_n[3] = {wb, gb, gb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(out[i], out_n[i], in[j], in_n[j])) return Q3_ERR_SHAPE;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out[i], out_n[i], out[j], out_n[j])) return Q3_ERR_SHAPE;
  }
  if (!al16(w_qkv) || !al16(q_norm) || !al16(k_norm) || !al16(w_qkv_out) || !al16(q_norm_out) || !al16(k_norm_out))
    return Q3_ERR_ALIGN;
  return Q3_OK;
}

SampleWsLayout sample_ws_layout(int32_t rows, int32_t vocab) {
  SampleWsLayout L{};
  const size_t G = (size_t)sample_chunks(rows, vocab), R = (size_t)rows;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  size_t off = 0;
  L.st = off;
  off += al(SAMPLE_ROW_BYTES * R);
  L.tick = off;
  off += al(4 * R);
  L.cnt = off;
  off += al(4 * R * G * 256);
  L.mass = off;
  off += al(8 * R * G * 256);
  L.mini = off;
  off += al(4 * R * G * 256);
  L.best = off;
  off += al(8 * R * G);
  L.total = off;
  return L;
}

int check_sample_call(const float* logits, int32_t rows, int32_t vocab, int64_t row_stride, const float* temperature,
                      const int32_t* top_k, const float* top_p, const float* uniform, const int32_t* out_idx,
                      const void* ws, size_t ws_bytes) {
  if (!logits || !temperature || !top_k || !top_p || !uniform || !out_idx || !ws) return Q3_ERR_NULL;
  if (rows < 1 || rows > SAMPLE_MAX_ROWS || vocab < 1 || row_stride < vocab) return Q3_ERR_SHAPE;
  if (!al4(logits) || !al4(temperature) || !al4(top_k) || !al4(top_p) || !al4(uniform) || !al4(out_idx) ||
      !al16(ws))
    return Q3_ERR_ALIGN;
  if (ws_bytes < sample_ws_layout(rows, vocab).total) return Q3_ERR_WORKSPACE;
  return Q3_OK;
}

int check_prefill_packed_call(const q3_model* m, const q3_kv* kv, int32_t n_seqs, int32_t n_tokens,
                              const int32_t* ids, const int32_t* cu_seqlens, const int32_t* start_pos,
                              int32_t max_seq_tokens, const float* last_logits, const int32_t* next_ids,
                              const int32_t* seq_lens, const void* ws, size_t ws_bytes) {
  if (!m || !kv || !ids || !cu_seqlens || !next_ids || !seq_lens || !ws) return Q3_ERR_NULL;
  if (model_null(m) || !kv->k || !kv->v) return Q3_ERR_NULL;
  if (kv->batch < 1 || kv->max_seq < 8 || kv->max_seq > Q3_MAX_POS || (kv->max_seq % 8) != 0) return Q3_ERR_SHAPE;
  if (n_seqs < 1 || n_seqs > kv->batch || n_tokens < n_seqs || n_tokens > MAX_TOKENS) return Q3_ERR_SHAPE;
  if (max_seq_tokens < 1 || max_seq_tokens > n_tokens) return Q3_ERR_SHAPE;
  if (max_seq_tokens > kv->max_seq) return Q3_ERR_POSITION;
  if (model_misaligned(m) || !al16(kv->k) || !al16(kv->v) || !al4(ids) || !al4(cu_seqlens) ||
      (start_pos && !al4(start_pos)) || !al4(next_ids) || !al4(seq_lens) || (last_logits && !al16(last_logits)) ||
      !al16(ws))
    return Q3_ERR_ALIGN;
  if (ws_bytes < ws_layout_rows(n_seqs, n_tokens, false).total) return Q3_ERR_WORKSPACE;
  return Q3_OK;
}

int check_linear_call(const void* x, const void* w, const void* out, int32_t m, int32_t n, int32_t k, int32_t ldo,
                      int32_t epilogue) {
  if (!x || !w || !out) return Q3_ERR_NULL;
  if (epilogue < Q3_EPI_STORE_BF16 || epilogue > Q3_EPI_SILU_GATE) return Q3_ERR_SHAPE;
  if (m < 1 || n < 128 || k < 512 || (n % 128) != 0 || (k % 512) != 0) return Q3_ERR_SHAPE;
  if ((int64_t)m > MAX_TOKENS) return Q3_ERR_SHAPE;
  const int32_t out_cols = epilogue == Q3_EPI_SILU_GATE ? n / 2 : n;
  if (ldo < out_cols || (ldo % 4) != 0) return Q3_ERR_SHAPE;
  if (!al16(x) || !al16(w) || !al16(out)) return Q3_ERR_ALIGN;
  return Q3_OK;
}

static bool cache_shape_ok(int32_t max_seq) { return max_seq >= 8 && max_seq <= Q3_MAX_POS && (max_seq % 8) == 0; }

int check_attn_prefill_call(const void* q, const void* k_layer, const void* v_layer, int32_t batch, int32_t n_tokens,
                            int32_t start_pos, int32_t max_seq, const void* out) {
  if (!q || !k_layer || !v_layer || !out) return Q3_ERR_NULL;
  if (batch < 1 || n_tokens < 1 || !cache_shape_ok(max_seq)) return Q3_ERR_SHAPE;
  if ((int64_t)batch * n_tokens > MAX_TOKENS) return Q3_ERR_SHAPE;
  if (start_pos < 0 || (int64_t)start_pos + n_tokens > max_seq) return Q3_ERR_POSITION;
  if (!al16(q) || !al16(k_layer) || !al16(v_layer) || !al16(out)) return Q3_ERR_ALIGN;
  return Q3_OK;
}

int check_attn_prefill_qkv_call(const void* qkv, const void* q_norm, const void* k_norm, const float* rope_cos,
                                const float* rope_sin, const void* k_layer, const void* v_layer, int32_t batch,
                                int32_t n_tokens, int32_t start_pos, int32_t max_seq, int32_t write_kv,
                                const void* out) {
  if (!q_norm || !k_norm || !rope_cos || !rope_sin) return Q3_ERR_NULL;
  const int st = check_attn_prefill_call(qkv, k_layer, v_layer, batch, n_tokens, start_pos, max_seq, out);
  if (st != Q3_OK) return st;
  if (write_kv != 0 && write_kv != 1) return Q3_ERR_SHAPE;
  if (!al16(q_norm) || !al16(k_norm) || !al16(rope_cos) || !al16(rope_sin)) return Q3_ERR_ALIGN;
  return Q3_OK;
}

int check_attn_decode_call(const void* qkv, const void* q_norm, const void* k_norm, const float* rope_cos,
                           const float* rope_sin, const void* k_layer, const void* v_layer, int32_t batch,
                           int32_t max_seq, const int32_t* positions, int32_t max_len_hint, const void* out,
                           const void* ws, size_t ws_bytes) {
  if (!qkv || !q_norm || !k_norm || !rope_cos || !rope_sin || !k_layer || !v_layer || !positions || !out || !ws)
    return Q3_ERR_NULL;
  if (batch < 1 || batch > (int32_t)(MAX_TOKENS / 8) || !cache_shape_ok(max_seq)) return Q3_ERR_SHAPE;
  if (max_len_hint < 1 || max_len_hint > max_seq) return Q3_ERR_POSITION;
  if (!al16(qkv) || !al16(q_norm) || !al16(k_norm) || !al16(rope_cos) || !al16(rope_sin) || !al16(k_layer) ||
      !al16(v_layer) || !al4(positions) || !al16(out) || !al16(ws))
    return Q3_ERR_ALIGN;
  if (ws_bytes < ws_layout(batch, 1).total) return Q3_ERR_WORKSPACE;
  return Q3_OK;
}

int check_argmax_call(const float* logits, int32_t rows, int32_t vocab, int64_t row_stride, const int32_t* out_idx) {
  if (!logits || !out_idx) return Q3_ERR_NULL;
  if (rows < 1 || vocab < 1 || row_stride < vocab) return Q3_ERR_SHAPE;
  if (!al4(logits) || !al4(out_idx)) return Q3_ERR_ALIGN;
  return Q3_OK;
}

}  // namespace q3v
