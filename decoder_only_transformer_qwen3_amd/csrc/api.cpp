// C-ABI entry points: validate on the host, carve the caller's workspace,
// enqueue the kernel chain on the caller's stream.  No allocation, no
// synchronisation, no state kept between calls.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "../../include/q3.h"
#include "common.hpp"
#include "launch.hpp"
#include "validate.hpp"

using namespace q3;

static_assert(Q3_EPI_STORE_BF16 == EPI_BF16 && Q3_EPI_STORE_F32 == EPI_F32 && Q3_EPI_ADD_F32 == EPI_ADD_F32 &&
                  Q3_EPI_SILU_GATE == EPI_SILU,
              "public epilogue ids must match the kernel epilogue ids");

namespace {

// Skinny-GEMM K splits: o_proj K = 2048 -> 4 x 512, down K = 3072 -> 3 x 1024.
constexpr int SPLIT_O = 4;
constexpr int SPLIT_DOWN = 3;
// Row counts up to this run o_proj / down as a VALU GEMV without a K split.
constexpr int GEMV_MAX_ROWS = 8;

struct Ws {
  float* resid;
  uint16_t *h, *qkv, *ao, *act, *fh;
  float *part, *tpart, *apart, *ssq;
  int* tick;  // 64 column-block tickets, batch * 8 attention tickets, the lm_head ticket
  int n_tick;
  void* amax;
};

Ws carve_rows(void* base, int32_t batch, int64_t rows, bool one_token) {
  const q3v::WsLayout L = q3v::ws_layout_rows(batch, rows, one_token);
  char* p = static_cast<char*>(base);
  Ws w;
  w.resid = reinterpret_cast<float*>(p + L.resid);
  w.h = reinterpret_cast<uint16_t*>(p + L.h);
  w.qkv = reinterpret_cast<uint16_t*>(p + L.qkv);
  w.ao = reinterpret_cast<uint16_t*>(p + L.ao);
  w.act = reinterpret_cast<uint16_t*>(p + L.act);
  w.part = reinterpret_cast<float*>(p + L.part);
  w.tpart = reinterpret_cast<float*>(p + L.tpart);
  w.apart = reinterpret_cast<float*>(p + L.apart);
  w.amax = p + L.amax;
  w.fh = reinterpret_cast<uint16_t*>(p + L.fh);
  w.ssq = reinterpret_cast<float*>(p + L.ssq);
  w.tick = reinterpret_cast<int*>(p + L.tick);
  w.n_tick = q3v::ticket_count(batch);
  return w;
}

Ws carve(void* base, int32_t batch, int32_t n_tokens) {
  return carve_rows(base, batch, (int64_t)batch * n_tokens, n_tokens == 1);
}

struct LayerCtx {
  const q3_layer_weights* w;
  const float *cos, *sin;
  uint16_t *kl, *vl;
  int B, T, max_seq, start;
  const int32_t* pos_dev;  // per-sequence start positions on the device (decode), or null
  int M;                   // rows of the call (all sequences)
  SeqMap sm;               // row -> (sequence, position); packed or uniform
  int max_T;               // bound on the rows of one sequence
  int dec_splits;          // decode-attention splits (T == 1 only)
  bool dec_stream;         // decode attention in its streaming configuration (T == 1 only)
  float* resid;
  const uint16_t* gamma_next;  // gain of the norm that follows this layer, or null
  // Tiled path (65-2047 rows): a residual projection split over K may leave
  // its fp32 split sums in ws.tpart for the RMSNorm that reads the residual
  // next, which adds them (one kernel fewer).  defer_down: this layer's down
  // projection may do so (a next layer follows); in_pending: the residual
  // entering this layer still owes the previous layer's down split sums.
  bool defer_down;
  bool in_pending;
  const void* w_qkv_next;      // the q|k|v weight read next (layer l + 1, or layer 0 after the last), or null
  Ws ws;
  hipStream_t s;
};

inline const uint16_t* U(const void* p) { return static_cast<const uint16_t*>(p); }

inline bool skinny_rows(int M) { return M <= q3v::SKINNY_MAX_ROWS; }

// Tiled / persistent GEMM of the layer's rows, with the K split the
// workspace was sized for.
inline void tiled(const LayerCtx& c, const uint16_t* X, const void* W, void* out, int N, int K, int ldo, Epi epi) {
  const int n_split = q3v::tiled_splits(c.M, N, K, epi == EPI_SILU);
  launch_gemm_tiled(X, U(W), out, c.M, N, K, ldo, epi, c.s, n_split, c.ws.tpart);
}

// Residual projection on the tiled path whose split sums (if K is split) are
// left in ws.tpart for the next RMSNorm; returns the number of splits left
// there (0: the residual is already complete).
inline int tiled_resid_deferred(const LayerCtx& c, const uint16_t* X, const void* W, int K) {
  const int n_split = q3v::tiled_splits(c.M, C, K, false);
  launch_gemm_tiled(X, U(W), c.resid, c.M, C, K, C, EPI_ADD_F32, c.s, n_split, c.ws.tpart, n_split == 1);
  return n_split > 1 ? n_split : 0;
}

// Partial sums of squares per residual row (see NSQ in common.hpp).
inline int nsq_for(int M) { return M <= GEMV_MAX_ROWS ? NSQ : NSQ_BLK; }

// Skinny GEMM whose input is the norm-folded operand ws.h / ws.ssq.
inline void skinny_normed(const LayerCtx& c, const void* W, void* out, int N, int ldo, Epi epi) {
  SkinnyArgs a{};
  a.X = c.ws.h;
  a.W = U(W);
  a.out = out;
  a.M = c.M;
  a.N = N;
  a.K = C;
  a.ldo = ldo;
  a.ssq = c.ws.ssq;
  a.ssq_n = nsq_for(a.M);
  a.ssq_ld = a.ssq_n;
  launch_gemm_skinny(a, 1, epi, c.s);
}

// Projection into the residual that also prepares the next norm's operand
// (when gamma is set).  Up to 8 rows a VALU GEMV covers each column over the
// whole K range; above that the MFMA skinny GEMM splits K and the last
// workgroup per column block adds the splits.
inline void skinny_residual(const LayerCtx& c, const uint16_t* X, const void* W, int K, int n_split,
                            const uint16_t* gamma) {
  const int M = c.M;
  if (M <= GEMV_MAX_ROWS) {
    launch_gemv_resid(X, U(W), K, c.resid, M, gamma, c.ws.h, c.ws.ssq, c.s);
    return;
  }
  SkinnyArgs a{};
  a.X = X;
  a.W = U(W);
  a.M = M;
  a.N = C;
  a.K = K;
  a.ldo = C;
  a.gamma = gamma;
  a.hg = c.ws.h;
  a.ssq_out = c.ws.ssq;
  a.ssq_n = nsq_for(M);
  a.out = c.ws.part;
  a.resid = c.resid;
  a.counters = c.ws.tick;
  launch_gemm_skinny(a, n_split, EPI_PARTIAL, c.s);
}

// One decoder layer ("手写Qwen3-0.6B推理" §Qwen3DecoderLayer).
// Up to 128 rows (skinny path) the layer expects ws.h = bf16(gamma_in * r)
// and ws.ssq = the row sums of squares, and leaves the same for gamma_next;
// above that the norms run as separate kernels around the tiled GEMMs.
void run_layer(const LayerCtx& c) {
  const int M = c.M;
  const bool skinny = skinny_rows(M);
  const q3_layer_weights* w = c.w;
  // input RMSNorm + merged q|k|v projection
  if (skinny) {
    skinny_normed(c, w->w_qkv, c.ws.qkv, QKV_N, QKV_N, EPI_BF16);
  } else {
    const int pend = c.in_pending ? q3v::tiled_splits(M, C, I, false) : 1;
    launch_rmsnorm(c.resid, pend > 1 ? c.ws.tpart : nullptr, pend > 1 ? pend : 0, M, U(w->input_norm), c.ws.h, M,
                   1, 0, c.s);
    tiled(c, c.ws.h, w->w_qkv, c.ws.qkv, QKV_N, C, QKV_N, EPI_BF16);
  }
  // q/k RMSNorm + RoPE, K/V into the cache, causal GQA attention
  if (c.T == 1) {
    // decode of up to 8 rows whose attention leaves most CUs idle: the launch
    // also reads the o_proj, gate|up and down weights and the next layer's
    // q|k|v weight into the L2s that the skinny GEMM and the GEMV will read
    // them through (after the last layer, layer 0's q|k|v, which the next
    // decode step reads first; a single-layer call re-reads its own)
    const bool warm = M <= GEMV_MAX_ROWS && c.dec_splits * HKV * c.B <= 64;
    const void* next_qkv = c.w_qkv_next ? c.w_qkv_next : w->w_qkv;
    launch_attn_decode(c.ws.qkv, U(w->q_norm), U(w->k_norm), c.cos, c.sin, c.kl, c.vl, c.ws.apart, c.ws.tick + 64,
                       c.ws.ao, c.B, c.max_seq, c.pos_dev, c.start, c.dec_splits, c.dec_stream, c.s,
                       warm ? w->w_o : nullptr, warm ? w->w_gate_up : nullptr, warm ? w->w_down : nullptr,
                       warm ? next_qkv : nullptr);
  } else {
    // k norm + RoPE and V into the cache; q is normed and rotated as the attention loads it
    launch_kv_store(c.ws.qkv, U(w->k_norm), c.cos, c.sin, c.kl, c.vl, c.sm, c.max_T, c.max_seq, c.s);
    launch_attn_prefill(c.ws.qkv, QKV_N, U(w->q_norm), c.cos, c.sin, c.kl, c.vl, c.ws.ao, c.sm, c.max_T,
                        c.max_seq, c.s);
  }
  // o_proj + residual, post-attention RMSNorm, gate|up with silu(gate) * up, down + residual
  if (skinny) {
    skinny_residual(c, c.ws.ao, w->w_o, QDIM, SPLIT_O, U(w->post_norm));
    skinny_normed(c, w->w_gate_up, c.ws.act, 2 * I, I, EPI_SILU);
    skinny_residual(c, c.ws.act, w->w_down, I, SPLIT_DOWN, c.gamma_next);
  } else {
    const int po = tiled_resid_deferred(c, c.ws.ao, w->w_o, QDIM);
    launch_rmsnorm(c.resid, po ? c.ws.tpart : nullptr, po, M, U(w->post_norm), c.ws.h, M, 1, 0, c.s);
    tiled(c, c.ws.h, w->w_gate_up, c.ws.act, 2 * I, C, I, EPI_SILU);
    if (c.defer_down)
      tiled_resid_deferred(c, c.ws.act, w->w_down, I);
    else
      tiled(c, c.ws.act, w->w_down, c.resid, C, I, C, EPI_ADD_F32);
  }
}

// Final RMSNorm on each sequence's last row, tied lm_head, argmax
// ("手写Qwen3-0.6B推理" §Qwen3Model; "第 3 章" §4.1 and §4.3).  On the
// skinny path the last layer already left bf16(gamma_f * r) and the sums of
// squares for every row; otherwise they are formed here for the B last rows.
void run_head(const q3_model* m, const Ws& ws, int B, int T, float* logits, int32_t* next_ids, int32_t* seq_lens,
              int seq_mode, int seq_val, hipStream_t s, const int32_t* in_ids = nullptr, int eos = -1,
              const SeqMap* packed = nullptr) {
  const uint16_t* X;
  const float* ssq;
  int ldx, ssq_ld, ssq_n;
  if (packed) {  // each sequence's last row, gathered through the row map
    ssq_n = NSQ_BLK;
    launch_norm_operand(ws.resid, B, 1, 0, U(m->final_norm), ws.fh, ws.ssq, ssq_n, nullptr, 0, s, packed);
    X = ws.fh;
    ldx = C;
    ssq = ws.ssq;
    ssq_ld = ssq_n;
  } else if (skinny_rows(B * T)) {
    ssq_n = nsq_for(B * T);
    X = ws.h + (size_t)(T - 1) * C;
    ldx = T * C;
    ssq = ws.ssq + (size_t)(T - 1) * ssq_n;
    ssq_ld = T * ssq_n;
  } else {
    ssq_n = NSQ_BLK;
    launch_norm_operand(ws.resid, B, T, T - 1, U(m->final_norm), ws.fh, ws.ssq, ssq_n, nullptr, 0, s);
    X = ws.fh;
    ldx = C;
    ssq = ws.ssq;
    ssq_ld = ssq_n;
  }
  // logits (when asked for) and the greedy token of each sequence; the
  // candidates of the lm_head's workgroups go to ws.amax, its ticket follows
  // the attention tickets
  constexpr int n_part = V / 16;
  HeadPick pick{};
  pick.out_idx = next_ids;
  pick.seq_lens = seq_lens;
  pick.seq_mode = seq_mode;
  pick.seq_val = seq_val;
  pick.in_ids = in_ids;
  pick.eos = eos;
  pick.sm = packed ? *packed : SeqMap{nullptr, nullptr, 0, 1, 0, 0};
  for (int r0 = 0; r0 < B; r0 += q3v::LM_HEAD_MAX_ROWS) {
    const int rows = (B - r0) < q3v::LM_HEAD_MAX_ROWS ? (B - r0) : q3v::LM_HEAD_MAX_ROWS;
    SkinnyArgs a{};
    a.X = X + (size_t)r0 * ldx;
    a.ldx = ldx;
    a.W = U(m->embed);
    a.out = logits ? logits + (size_t)r0 * V : nullptr;  // null: the caller wants no logits
    a.M = rows;
    a.N = V;
    a.K = C;
    a.ldo = V;
    a.amax_part = static_cast<char*>(ws.amax) + (size_t)r0 * n_part * 8;
    a.ssq = ssq + (size_t)r0 * ssq_ld;
    a.ssq_ld = ssq_ld;
    a.ssq_n = ssq_n;
    pick.r0 = r0;
    launch_lm_head(a, pick, ws.tick + q3v::head_ticket(B), s);
  }
}

inline int launch_status() { return hipGetLastError() == hipSuccess ? Q3_OK : Q3_ERR_HIP; }

inline uint16_t* layer_cache(void* base, int layer, const q3_kv* kv) {
  return static_cast<uint16_t*>(base) + (size_t)layer * kv->batch * HKV * kv->max_seq * D;
}

}  // namespace

// Scratch of q3_decode_step_noalloc: the decode step's workspace for up to
// Q3_NOALLOC_MAX_BYTES, one copy per GPU the library runs on, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (its
// host-side name is not a device address): each device's address is looked
// up once with hipGetSymbolAddress and kept in noalloc_ptr.
static __device__ __align__(256) unsigned char scratch[Q3_NOALLOC_MAX_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[NOALLOC_MAX_DEVICES];

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with that device current).
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return Q3_ERR_HIP;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return Q3_ERR_HIP;
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return Q3_OK;
}

}  // namespace

extern "C" {

const char* q3_status_str(int status) {
  switch (status) {
    case Q3_OK: return "ok";
    case Q3_ERR_NULL: return "a required pointer is NULL";
    case Q3_ERR_SHAPE: return "invalid batch, token count or cache shape";
    case Q3_ERR_POSITION: return "positions exceed the cache capacity or the maximum position";
    case Q3_ERR_ALIGN: return "a pointer is not suitably aligned";
    case Q3_ERR_WORKSPACE: return "workspace smaller than q3_workspace_bytes()";
    case Q3_ERR_HIP: return "a HIP kernel launch failed";
    case Q3_ERR_TOO_LARGE: return "the call needs more than the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

int q3_rope_table_host(float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out) return Q3_ERR_NULL;
  double inv[ROPE_HALF];
  for (int i = 0; i < ROPE_HALF; ++i) inv[i] = pow(1e6, -(2.0 * i) / (double)D);
  for (int p = 0; p < MAXPOS; ++p)
    for (int i = 0; i < ROPE_HALF; ++i) {
      const double a = (double)p * inv[i];
      cos_out[(size_t)p * ROPE_HALF + i] = (float)cos(a);
      sin_out[(size_t)p * ROPE_HALF + i] = (float)sin(a);
    }
  return Q3_OK;
}

size_t q3_workspace_bytes(int32_t batch, int32_t n_tokens) {
  if (batch < 1 || n_tokens < 1) return 0;
  return q3v::ws_layout(batch, n_tokens).total;
}

int q3_layer_forward(const q3_layer_weights* w, const float* rope_cos, const float* rope_sin, void* k_layer,
                     void* v_layer, int32_t batch, int32_t n_tokens, int32_t max_seq, int32_t start_pos,
                     float* residual, void* ws, size_t ws_bytes, void* stream) {
  const int st = q3v::check_layer_call(w, rope_cos, rope_sin, k_layer, v_layer, batch, n_tokens, max_seq, start_pos,
                                       residual, ws, ws_bytes);
  if (st != Q3_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  LayerCtx c;
  c.w = w;
  c.cos = rope_cos;
  c.sin = rope_sin;
  c.kl = static_cast<uint16_t*>(k_layer);
  c.vl = static_cast<uint16_t*>(v_layer);
  c.B = batch;
  c.T = n_tokens;
  c.M = batch * n_tokens;
  c.sm = SeqMap{nullptr, nullptr, batch, n_tokens, start_pos, batch * n_tokens};
  c.max_T = n_tokens;
  c.max_seq = max_seq;
  c.start = start_pos;
  c.pos_dev = nullptr;
  c.dec_splits = q3v::decode_splits(batch, start_pos + 1);
  c.dec_stream = q3v::decode_streaming(batch, start_pos + 1);
  c.resid = residual;
  c.gamma_next = nullptr;
  c.w_qkv_next = nullptr;
  c.defer_down = false;
  c.in_pending = false;
  c.ws = carve(ws, batch, n_tokens);
  c.s = s;
  const int M = batch * n_tokens;
  // the skinny path starts from the norm-folded operand; both paths start with zeroed tickets
  launch_norm_operand(residual, skinny_rows(M) ? M : 0, 1, 0, U(w->input_norm), c.ws.h, c.ws.ssq, nsq_for(M),
                      c.ws.tick, c.ws.n_tick, s);
  run_layer(c);
  return launch_status();
}

int q3_prefill(const q3_model* m, const q3_kv* kv, int32_t batch, int32_t prompt_len, const int32_t* ids,
               float* last_logits, int32_t* next_ids, int32_t* seq_lens, void* ws, size_t ws_bytes, void* stream) {
  const int st =
      q3v::check_prefill_call(m, kv, batch, prompt_len, ids, last_logits, next_ids, seq_lens, ws, ws_bytes);
  if (st != Q3_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws wsp = carve(ws, batch, prompt_len);
  const int M = batch * prompt_len;
  const bool sk = skinny_rows(M);
  launch_embed(ids, U(m->embed), wsp.resid, M, sk ? U(m->layer[0].input_norm) : nullptr, wsp.h, wsp.ssq, nsq_for(M),
               wsp.tick, wsp.n_tick, s);
  LayerCtx c;
  c.cos = m->rope_cos;
  c.sin = m->rope_sin;
  c.B = batch;
  c.T = prompt_len;
  c.M = batch * prompt_len;
  c.sm = SeqMap{nullptr, nullptr, batch, prompt_len, 0, batch * prompt_len};
  c.max_T = prompt_len;
  c.max_seq = kv->max_seq;
  c.start = 0;
  c.pos_dev = nullptr;
  c.dec_splits = q3v::decode_splits(batch, 1);
  c.dec_stream = false;
  c.resid = wsp.resid;
  c.ws = wsp;
  c.s = s;
  for (int l = 0; l < NL; ++l) {
    c.w = &m->layer[l];
    c.kl = layer_cache(kv->k, l, kv);
    c.vl = layer_cache(kv->v, l, kv);
    c.gamma_next = U(l + 1 < NL ? m->layer[l + 1].input_norm : m->final_norm);
    c.in_pending = l > 0;        // (only acted on where the previous layer deferred)
    c.defer_down = l + 1 < NL;
    c.w_qkv_next = m->layer[(l + 1) % NL].w_qkv;  // after the last layer: the next step's first
    run_layer(c);
  }
  run_head(m, wsp, batch, prompt_len, last_logits, next_ids, seq_lens, 1, prompt_len, s);
  return launch_status();
}

size_t q3_workspace_bytes_packed(int32_t n_seqs, int32_t n_tokens) {
  if (n_seqs < 1 || n_tokens < 1) return 0;
  return q3v::ws_layout_rows(n_seqs, n_tokens, false).total;
}

int q3_prefill_packed(const q3_model* m, const q3_kv* kv, int32_t n_seqs, int32_t n_tokens, const int32_t* ids,
                      const int32_t* cu_seqlens, const int32_t* start_pos, int32_t max_seq_tokens,
                      float* last_logits, int32_t* next_ids, int32_t* seq_lens, void* ws, size_t ws_bytes,
                      void* stream) {
  const int st = q3v::check_prefill_packed_call(m, kv, n_seqs, n_tokens, ids, cu_seqlens, start_pos, max_seq_tokens,
                                                last_logits, next_ids, seq_lens, ws, ws_bytes);
  if (st != Q3_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws wsp = carve_rows(ws, n_seqs, n_tokens, false);
  const int M = n_tokens;
  const bool sk = skinny_rows(M);
  launch_embed(ids, U(m->embed), wsp.resid, M, sk ? U(m->layer[0].input_norm) : nullptr, wsp.h, wsp.ssq, nsq_for(M),
               wsp.tick, wsp.n_tick, s);
  LayerCtx c;
  c.cos = m->rope_cos;
  c.sin = m->rope_sin;
  c.B = n_seqs;
  c.T = 0;  // rows per sequence vary: never the one-token path
  c.M = M;
  c.sm = SeqMap{cu_seqlens, start_pos, n_seqs, 0, 0, n_tokens};
  c.max_T = max_seq_tokens;
  c.max_seq = kv->max_seq;
  c.start = 0;
  c.pos_dev = nullptr;
  c.dec_splits = 1;
  c.dec_stream = false;
  c.resid = wsp.resid;
  c.ws = wsp;
  c.s = s;
  for (int l = 0; l < NL; ++l) {
    c.w = &m->layer[l];
    c.kl = layer_cache(kv->k, l, kv);
    c.vl = layer_cache(kv->v, l, kv);
    c.gamma_next = U(l + 1 < NL ? m->layer[l + 1].input_norm : m->final_norm);
    c.in_pending = l > 0;        // (only acted on where the previous layer deferred)
    c.defer_down = l + 1 < NL;
    c.w_qkv_next = m->layer[(l + 1) % NL].w_qkv;  // after the last layer: the next step's first
    run_layer(c);
  }
  run_head(m, wsp, n_seqs, 0, last_logits, next_ids, seq_lens, 3, 0, s, nullptr, -1,
           &c.sm);
  return launch_status();
}

int q3_decode_step_eos(const q3_model* m, const q3_kv* kv, int32_t batch, const int32_t* in_ids, int32_t* seq_lens,
                       int32_t max_len_hint, int32_t eos_id, float* logits, int32_t* out_ids, void* ws,
                       size_t ws_bytes, void* stream) {
  int st = q3v::check_decode_call(m, kv, batch, in_ids, seq_lens, max_len_hint, logits, out_ids, ws, ws_bytes);
  if (st == Q3_OK && (eos_id < -1 || eos_id >= Q3_VOCAB)) st = Q3_ERR_SHAPE;
  if (st != Q3_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws wsp = carve(ws, batch, 1);
  const bool sk = skinny_rows(batch);
  launch_embed(in_ids, U(m->embed), wsp.resid, batch, sk ? U(m->layer[0].input_norm) : nullptr, wsp.h, wsp.ssq,
               nsq_for(batch), wsp.tick, wsp.n_tick, s);
  LayerCtx c;
  c.cos = m->rope_cos;
  c.sin = m->rope_sin;
  c.B = batch;
  c.T = 1;
  c.M = batch;
  c.sm = SeqMap{nullptr, seq_lens, batch, 1, 0, batch};
  c.max_T = 1;
  c.max_seq = kv->max_seq;
  c.start = 0;
  c.pos_dev = seq_lens;
  c.dec_splits = q3v::decode_splits(batch, max_len_hint);
  c.dec_stream = q3v::decode_streaming(batch, max_len_hint);
  c.resid = wsp.resid;
  c.ws = wsp;
  c.s = s;
  for (int l = 0; l < NL; ++l) {
    c.w = &m->layer[l];
    c.kl = layer_cache(kv->k, l, kv);
    c.vl = layer_cache(kv->v, l, kv);
    c.gamma_next = U(l + 1 < NL ? m->layer[l + 1].input_norm : m->final_norm);
    c.in_pending = l > 0;        // (only acted on where the previous layer deferred)
    c.defer_down = l + 1 < NL;
    c.w_qkv_next = m->layer[(l + 1) % NL].w_qkv;  // after the last layer: the next step's first
    run_layer(c);
  }
  run_head(m, wsp, batch, 1, logits, out_ids, seq_lens, 2, 0, s, in_ids, eos_id);
  return launch_status();
}

int q3_decode_step(const q3_model* m, const q3_kv* kv, int32_t batch, const int32_t* in_ids, int32_t* seq_lens,
                   int32_t max_len_hint, float* logits, int32_t* out_ids, void* ws, size_t ws_bytes, void* stream) {
  return q3_decode_step_eos(m, kv, batch, in_ids, seq_lens, max_len_hint, -1, logits, out_ids, ws, ws_bytes,
                            stream);
}

int q3_decode_step_noalloc(const q3_model* m, const q3_kv* kv, int32_t batch, const int32_t* in_ids,
                           int32_t* seq_lens, int32_t max_len_hint, int32_t eos_id, float* logits, int32_t* out_ids,
                           void* stream) {
  if (batch >= 1 && q3_workspace_bytes(batch, 1) > (size_t)Q3_NOALLOC_MAX_BYTES) return Q3_ERR_TOO_LARGE;
  const size_t need = batch >= 1 ? q3_workspace_bytes(batch, 1) : 0;
  // every other argument is validated before the scratch is looked up (the
  // workspace check is the scratch's own, just passed above)
  int st = q3v::check_decode_call(m, kv, batch, in_ids, seq_lens, max_len_hint, logits, out_ids,
                                  reinterpret_cast<const void*>((uintptr_t)256), need);
  if (st == Q3_OK && (eos_id < -1 || eos_id >= Q3_VOCAB)) st = Q3_ERR_SHAPE;
  if (st != Q3_OK) return st;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != Q3_OK) return st;
  // the kernel chain clears the tickets it uses (first kernel of the step), so
  // whatever an earlier call left in the scratch is never read
  return q3_decode_step_eos(m, kv, batch, in_ids, seq_lens, max_len_hint, eos_id, logits, out_ids, ws, need, stream);
}

int q3_linear(const void* x, const void* w, void* out, int32_t m, int32_t n, int32_t k, int32_t ldo, int32_t epilogue,
              void* stream) {
  const int st = q3v::check_linear_call(x, w, out, m, n, k, ldo, epilogue);
  if (st != Q3_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Epi e = static_cast<Epi>(epilogue);  // Q3_EPI_* values equal the internal epilogue ids
  if (m <= q3v::SKINNY_MAX_ROWS)
    launch_gemm_skinny(U(x), U(w), out, m, n, k, ldo, 1, e, s);
  else
    launch_gemm_tiled(U(x), U(w), out, m, n, k, ldo, e, s);
  return launch_status();
}

int q3_attention_prefill(const void* q, const void* k_layer, const void* v_layer, int32_t batch, int32_t n_tokens,
                         int32_t start_pos, int32_t max_seq, void* out, void* stream) {
  const int st = q3v::check_attn_prefill_call(q, k_layer, v_layer, batch, n_tokens, start_pos, max_seq, out);
  if (st != Q3_OK) return st;
  const SeqMap sm{nullptr, nullptr, batch, n_tokens, start_pos, batch * n_tokens};
  launch_attn_prefill(U(q), QDIM, nullptr, nullptr, nullptr, U(k_layer), U(v_layer), static_cast<uint16_t*>(out), sm,
                      n_tokens, max_seq, static_cast<hipStream_t>(stream));
  return launch_status();
}

int q3_attention_prefill_qkv(const void* qkv, const void* q_norm, const void* k_norm, const float* rope_cos,
                             const float* rope_sin, void* k_layer, void* v_layer, int32_t batch, int32_t n_tokens,
                             int32_t start_pos, int32_t max_seq, int32_t write_kv, void* out, void* stream) {
  const int st = q3v::check_attn_prefill_qkv_call(qkv, q_norm, k_norm, rope_cos, rope_sin, k_layer, v_layer, batch,
                                                  n_tokens, start_pos, max_seq, write_kv, out);
  if (st != Q3_OK) return st;
  const SeqMap sm{nullptr, nullptr, batch, n_tokens, start_pos, batch * n_tokens};
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* kl = static_cast<uint16_t*>(k_layer);
  uint16_t* vl = static_cast<uint16_t*>(v_layer);
  if (write_kv) launch_kv_store(U(qkv), U(k_norm), rope_cos, rope_sin, kl, vl, sm, n_tokens, max_seq, s);
  launch_attn_prefill(U(qkv), QKV_N, U(q_norm), rope_cos, rope_sin, kl, vl, static_cast<uint16_t*>(out), sm, n_tokens,
                      max_seq, s);
  return launch_status();
}

int q3_attention_decode_warm(const void* qkv, const void* q_norm, const void* k_norm, const float* rope_cos,
                             const float* rope_sin, void* k_layer, void* v_layer, int32_t batch, int32_t max_seq,
                             const int32_t* positions, int32_t max_len_hint, void* out, void* ws, size_t ws_bytes,
                             const void* w_o, const void* w_gate_up, const void* w_down, const void* w_qkv_next,
                             void* stream) {
  int st = q3v::check_attn_decode_call(qkv, q_norm, k_norm, rope_cos, rope_sin, k_layer, v_layer, batch, max_seq,
                                       positions, max_len_hint, out, ws, ws_bytes);
  if (st != Q3_OK) return st;
  const bool with_weights = w_o || w_gate_up || w_down || w_qkv_next;
  if (with_weights) {
    if (!w_o || !w_gate_up || !w_down || !w_qkv_next) return Q3_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(w_o) | reinterpret_cast<uintptr_t>(w_gate_up) |
         reinterpret_cast<uintptr_t>(w_down) | reinterpret_cast<uintptr_t>(w_qkv_next)) & 15)
      return Q3_ERR_ALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws w = carve(ws, batch, 1);
  const int n_split = q3v::decode_splits(batch, max_len_hint);
  const bool warm = with_weights && batch <= GEMV_MAX_ROWS && n_split * HKV * batch <= 64;
  // the split merge's tickets start at zero (a single split takes none)
  if (n_split > 1) launch_norm_operand(nullptr, 0, 1, 0, nullptr, nullptr, nullptr, NSQ, w.tick, w.n_tick, s);
  launch_attn_decode(U(qkv), U(q_norm), U(k_norm), rope_cos, rope_sin, static_cast<uint16_t*>(k_layer),
                     static_cast<uint16_t*>(v_layer), w.apart, w.tick + 64, static_cast<uint16_t*>(out), batch,
                     max_seq, positions, 0, n_split, q3v::decode_streaming(batch, max_len_hint), s,
                     warm ? w_o : nullptr, warm ? w_gate_up : nullptr, warm ? w_down : nullptr,
                     warm ? w_qkv_next : nullptr);
  return launch_status();
}

int q3_attention_decode(const void* qkv, const void* q_norm, const void* k_norm, const float* rope_cos,
                        const float* rope_sin, void* k_layer, void* v_layer, int32_t batch, int32_t max_seq,
                        const int32_t* positions, int32_t max_len_hint, void* out, void* ws, size_t ws_bytes,
                        void* stream) {
  return q3_attention_decode_warm(qkv, q_norm, k_norm, rope_cos, rope_sin, k_layer, v_layer, batch, max_seq,
                                  positions, max_len_hint, out, ws, ws_bytes, nullptr, nullptr, nullptr, nullptr,
                                  stream);
}

int q3_argmax(const float* logits, int32_t rows, int32_t vocab, int64_t row_stride, int32_t* out_idx, void* stream) {
  const int st = q3v::check_argmax_call(logits, rows, vocab, row_stride, out_idx);
  if (st != Q3_OK) return st;
  launch_argmax(logits, rows, vocab, row_stride, out_idx, nullptr, 0, 0, static_cast<hipStream_t>(stream));
  return launch_status();
}

int q3_rope_interleaved_to_half(const void* w_qkv, const void* q_norm, const void* k_norm, void* w_qkv_out,
                                void* q_norm_out, void* k_norm_out, void* stream) {
  const int st = q3v::check_rope_convert_call(w_qkv, q_norm, k_norm, w_qkv_out, q_norm_out, k_norm_out);
  if (st != Q3_OK) return st;
  launch_rope_pair_permute(U(w_qkv), U(q_norm), U(k_norm), static_cast<uint16_t*>(w_qkv_out),
                           static_cast<uint16_t*>(q_norm_out), static_cast<uint16_t*>(k_norm_out),
                           static_cast<hipStream_t>(stream));
  return launch_status();
}

size_t q3_sample_workspace_bytes(int32_t rows, int32_t vocab) {
  if (rows < 1 || rows > q3v::SAMPLE_MAX_ROWS || vocab < 1) return 0;
  return q3v::sample_ws_layout(rows, vocab).total;
}

int q3_sample(const float* logits, int32_t rows, int32_t vocab, int64_t row_stride, const float* temperature,
              const int32_t* top_k, const float* top_p, const float* uniform, int32_t* out_idx, void* ws,
              size_t ws_bytes, void* stream) {
  const int st = q3v::check_sample_call(logits, rows, vocab, row_stride, temperature, top_k, top_p, uniform, out_idx,
                                        ws, ws_bytes);
  if (st != Q3_OK) return st;
  launch_sample(logits, rows, vocab, row_stride, temperature, top_k, top_p, uniform, out_idx, ws,
                static_cast<hipStream_t>(stream));
  return launch_status();
}

}  // extern "C"
