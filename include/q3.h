/*
 * q3.h -- C ABI of the Qwen3-0.6B-shape decoder forward on MI355X (gfx950).
 *
 * The model computed is the Qwen3 decoder as the source pages define it:
 *   - "手写Qwen3-0.6B推理": sections Qwen3Model, Qwen3DecoderLayer,
 *     Qwen3RMSNorm, Attention, Rope, MLP, 推理 (greedy argmax loop);
 *   - "第 3 章 前向与生成（代码走读）": 3.2 (fused residual + RMSNorm),
 *     3.3 (merged QKV projection, q/k norm, RoPE, causal GQA),
 *     3.4 (merged gate/up + silu(gate)*up), 4.1 (lm_head on the last
 *     position only), 4.3 (greedy argmax);
 *   - "古法手撕简易LLM推理器": sections 工具函数 (RMSNorm, RoPE table,
 *     SiLU), 核心计算函数与Transformer层 (KV cache holds normed+rotated K
 *     and raw V), prefill与predict (prefill, then one token per step with a
 *     growing offset);
 *   - "Pytorch手写大模型推理": section 模型 (configuration values).
 *
 * Shapes are fixed at compile time (Qwen3-0.6B): hidden C = 1024, 16 query
 * heads, 8 KV heads, head_dim D = 128, intermediate I = 3072, vocab
 * V = 151936, 28 layers, RMSNorm eps = 1e-6, RoPE theta = 1e6,
 * max position 40960.  Only batch, token count, positions and cache
 * capacity vary at run time.
 *
 * Conventions
 *   - Every floating-point weight and activation buffer is bfloat16 (raw
 *     16-bit patterns) unless stated; the residual stream is float32.
 *   - Every projection weight is row-major [out, in] and applied as
 *     y = x W^T (no bias).
 *   - All pointers are DEVICE pointers unless stated, 16-byte aligned.
 *   - The caller owns all memory.  The library never allocates, never
 *     frees, keeps no state between calls and never synchronises: each
 *     call validates its arguments on the host, enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the default stream) and returns.
 *   - On a validation error nothing is enqueued and nothing is written.
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Calls that share a workspace or KV cache must be ordered on one
 *     stream; concurrent calls on different streams need their own
 *     workspaces.
 */
#ifndef Q3_H
#define Q3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q3_HIDDEN 1024
#define Q3_N_HEADS 16
#define Q3_N_KV_HEADS 8
#define Q3_HEAD_DIM 128
#define Q3_INTER 3072
#define Q3_VOCAB 151936
#define Q3_N_LAYERS 28
#define Q3_MAX_POS 40960
#define Q3_QKV_ROWS 4096     /* 2048 q rows | 1024 k rows | 1024 v rows */
#define Q3_GATE_UP_ROWS 6144 /* 3072 gate rows | 3072 up rows */

/* Status codes returned by every entry point. */
enum {
  Q3_OK = 0,
  Q3_ERR_NULL = -1,      /* a required pointer is NULL */
  Q3_ERR_SHAPE = -2,     /* batch/token count < 1, or above a stated limit */
  Q3_ERR_POSITION = -3,  /* positions exceed the cache capacity or 40960 */
  Q3_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned */
  Q3_ERR_WORKSPACE = -5, /* workspace smaller than q3_workspace_bytes() */
  Q3_ERR_HIP = -6,       /* a kernel launch failed (hipGetLastError) */
  Q3_ERR_TOO_LARGE = -7  /* q3_decode_step_noalloc: batch beyond its fixed scratch */
};

/* One decoder layer ("手写Qwen3-0.6B推理" §打印模型结构 lists the tensors;
 * the merged row order follows "第 3 章" §3.3 and §3.4). */
typedef struct {
  const void *input_norm; /* [1024]        input_layernorm gain           */
  const void *w_qkv;      /* [4096, 1024]  rows 0..2047 q_proj,
                                            2048..3071 k_proj, 3072..4095 v_proj */
  const void *q_norm;     /* [128]         shared by the 16 query heads   */
  const void *k_norm;     /* [128]         shared by the 8 KV heads       */
  const void *w_o;        /* [1024, 2048]  o_proj                         */
  const void *post_norm;  /* [1024]        post_attention_layernorm gain  */
  const void *w_gate_up;  /* [6144, 1024]  rows 0..3071 gate_proj,
                                            3072..6143 up_proj             */
  const void *w_down;     /* [1024, 3072]  down_proj                      */
} q3_layer_weights;

/* Whole model.  The lm_head is tied to the embedding
 * ("手写Qwen3-0.6B推理" §Qwen3Model; tie_word_embeddings on
 * "Pytorch手写大模型推理" §模型). */
typedef struct {
  const void *embed;      /* [151936, 1024] embedding and lm_head         */
  const void *final_norm; /* [1024]                                       */
  q3_layer_weights layer[Q3_N_LAYERS];
  const float *rope_cos;  /* [40960, 64] float32, from q3_rope_table_host */
  const float *rope_sin;  /* [40960, 64] float32                          */
} q3_model;

/* KV cache: K after q/k-norm and RoPE, raw V ("古法手撕简易LLM推理器"
 * §核心计算函数与Transformer层), bf16, one region of
 * max_seq * 128 elements per (layer, sequence, KV head), regions ordered
 * [28][batch][8]:
 *   K region: position-major, element (p, d) at p * 128 + d;
 *   V region: blocks of 8 positions, dim-major inside a block, element
 *             (p, d) at ((p / 8) * 128 + d) * 8 + p % 8.
 * Both are caller-allocated, 28 * batch * 8 * max_seq * 128 * 2 bytes each. */
typedef struct {
  void *k;
  void *v;
  int32_t batch;
  int32_t max_seq;        /* multiple of 8, 8 .. 40960 */
} q3_kv;

/* Human-readable text for a status code (static storage). */
const char *q3_status_str(int status);

/* HOST function.  Fills the RoPE tables cos_out/sin_out (host memory,
 * float32 [40960, 64] each): entry [p, i] = cos/sin(p * 1e6^(-2i/128)),
 * evaluated in double precision and rounded once to float32
 * ("古法手撕简易LLM推理器" §工具函数 precomputes the same table up to
 * max_position_embeddings; "手写Qwen3-0.6B推理" §Rope gives the inverse
 * frequencies).  Dimension i < 64 pairs with i + 64 (half-swap form), so
 * the 128-wide table of the pages is these 64 columns twice.
 * Returns Q3_ERR_NULL on NULL pointers. */
int q3_rope_table_host(float *cos_out, float *sin_out);

/* Bytes of device workspace needed by a q3_layer_forward,
 * q3_prefill or q3_decode_step call with `batch` sequences of
 * `n_tokens` new tokens each (n_tokens = 1 for q3_decode_step).
 * Returns 0 for non-positive arguments. */
size_t q3_workspace_bytes(int32_t batch, int32_t n_tokens);

/* One decoder layer over batch x n_tokens new tokens at positions
 * start_pos .. start_pos + n_tokens - 1 of every sequence
 * ("手写Qwen3-0.6B推理" §Qwen3DecoderLayer: h = x + Attn(RMSNorm(x)),
 * out = h + MLP(RMSNorm(h)); attention per §Attention with q/k RMSNorm,
 * NeoX RoPE, causal GQA where query head h reads KV head h/2, scale
 * 1/sqrt(128); MLP per §MLP).
 *   w           layer weights (device pointers inside a HOST struct)
 *   rope_cos/sin  [40960, 64] float32 device tables
 *   k_layer, v_layer  this layer's cache regions for `batch` sequences in
 *               the q3_kv layouts (max_seq a multiple of 8); positions
 *               start_pos .. start_pos+n_tokens-1 are written, positions
 *               0 .. start_pos-1 must already hold the earlier tokens.
 *   residual    in/out float32 [batch * n_tokens, 1024], row b*n_tokens+t.
 *   ws          device workspace of at least
 *               q3_workspace_bytes(batch, n_tokens) bytes.
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (batch < 1, n_tokens < 1,
 * max_seq not a multiple of 8 in 8 .. 40960), Q3_ERR_POSITION (start_pos < 0 or
 * start_pos + n_tokens > max_seq), Q3_ERR_ALIGN, Q3_ERR_WORKSPACE,
 * Q3_ERR_HIP. */
int q3_layer_forward(const q3_layer_weights *w, const float *rope_cos, const float *rope_sin,
                     void *k_layer, void *v_layer, int32_t batch, int32_t n_tokens,
                     int32_t max_seq, int32_t start_pos, float *residual, void *ws,
                     size_t ws_bytes, void *stream);

/* Prefill of `batch` prompts of equal length prompt_len from position 0
 * ("古法手撕简易LLM推理器" §prefill与predict: prefill then the next-token
 * choice; "第 3 章" §4.1: logits only at each sequence's last position).
 *   kv          cache (HOST struct of device pointers); rows
 *               0 .. prompt_len-1 of every layer are overwritten.
 *   ids         int32 [batch, prompt_len], values in [0, 151936).
 *   last_logits float32 [batch, 151936] logits of the last position, or
 *               NULL to skip writing them.
 *   next_ids    int32 [batch]: greedy argmax of those logits (lowest
 *               index among equal maxima).
 *   seq_lens    int32 [batch]: set to prompt_len.
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (batch < 1 or > kv->batch,
 * prompt_len < 1, kv->max_seq invalid), Q3_ERR_POSITION (prompt_len > kv->max_seq),
 * Q3_ERR_ALIGN, Q3_ERR_WORKSPACE (q3_workspace_bytes(batch, prompt_len)),
 * Q3_ERR_HIP. */
int q3_prefill(const q3_model *m, const q3_kv *kv, int32_t batch, int32_t prompt_len,
               const int32_t *ids, float *last_logits, int32_t *next_ids, int32_t *seq_lens,
               void *ws, size_t ws_bytes, void *stream);

/* Prefill of packed, ragged sequences: n_seqs prompts of different
 * lengths concatenated into n_tokens rows ("第 3 章" §3.1 feeds the
 * engine's packed [tokens, C] layout with per-sequence positions and takes
 * logits only at each sequence's last position, §4.1).  Sequence s owns
 * rows cu_seqlens[s] .. cu_seqlens[s+1] - 1 and cache row s of kv; its
 * tokens sit at positions p0 .. p0 + len - 1 with p0 = start_pos[s] (0
 * when start_pos is NULL), so a call can also continue sequences whose
 * cache already holds positions 0 .. p0 - 1 (chunked prefill).
 *   ids         int32 [n_tokens];  cu_seqlens int32 [n_seqs + 1];
 *   start_pos   int32 [n_seqs] or NULL  (all device).
 *   max_seq_tokens  host bound on every sequence's length (sizes grids).
 *   last_logits float32 [n_seqs, 151936] or NULL; next_ids int32 [n_seqs]
 *               (greedy argmax); seq_lens int32 [n_seqs] set to p0 + len.
 *   ws          q3_workspace_bytes_packed(n_seqs, n_tokens) bytes.
 * The caller guarantees cu_seqlens[0] = 0, lengths >= 1 and <=
 * max_seq_tokens, cu_seqlens[n_seqs] = n_tokens and p0 + len <= kv->max_seq;
 * otherwise results are unspecified, with no out-of-range access.
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (n_seqs outside 1 .. kv->batch,
 * n_tokens < n_seqs, max_seq_tokens outside 1 .. n_tokens, cache shape),
 * Q3_ERR_POSITION (max_seq_tokens > kv->max_seq), Q3_ERR_ALIGN,
 * Q3_ERR_WORKSPACE, Q3_ERR_HIP. */
size_t q3_workspace_bytes_packed(int32_t n_seqs, int32_t n_tokens);
int q3_prefill_packed(const q3_model *m, const q3_kv *kv, int32_t n_seqs, int32_t n_tokens, const int32_t *ids,
                      const int32_t *cu_seqlens, const int32_t *start_pos, int32_t max_seq_tokens,
                      float *last_logits, int32_t *next_ids, int32_t *seq_lens, void *ws, size_t ws_bytes,
                      void *stream);

/* One greedy decode step for `batch` sequences ("古法手撕简易LLM推理器"
 * §prefill与predict, predict loop): sequence b feeds token in_ids[b] at
 * position seq_lens[b], appends its K/V at that cache row, attends to rows
 * 0 .. seq_lens[b], and on exit out_ids[b] holds the argmax of its logits
 * and seq_lens[b] has grown by one.  Lengths may differ per sequence.
 *   in_ids      int32 [batch] (may alias out_ids).
 *   seq_lens    int32 [batch] device lengths (read and advanced on device,
 *               so consecutive steps need no host round trip).
 *   max_len_hint  host-side upper bound on max(seq_lens) + 1; only sizes
 *               the attention split.  Must be in 1 .. kv->max_seq.  Any
 *               device length below kv->max_seq is handled correctly
 *               whatever the hint; a length >= kv->max_seq is a caller
 *               error: its cache write is skipped and its outputs are
 *               unspecified (no out-of-bounds access).
 *   logits      float32 [batch, 151936], or NULL.
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (batch < 1 or > kv->batch,
 * kv->max_seq invalid), Q3_ERR_POSITION (max_len_hint out of range), Q3_ERR_ALIGN,
 * Q3_ERR_WORKSPACE (q3_workspace_bytes(batch, 1)), Q3_ERR_HIP. */
int q3_decode_step(const q3_model *m, const q3_kv *kv, int32_t batch, const int32_t *in_ids,
                   int32_t *seq_lens, int32_t max_len_hint, float *logits, int32_t *out_ids,
                   void *ws, size_t ws_bytes, void *stream);

/* q3_decode_step with an end-of-sequence token ("第 3 章" §4.3: generation
 * stops once eos_id is produced and keeps it in the output;
 * "手写Qwen3-0.6B推理" §推理 and "古法手撕简易LLM推理器" §prefill与predict
 * stop on EOS 151645).  The input token is the done mask: a sequence whose
 * in_ids[b] == eos_id has finished, so out_ids[b] = eos_id and seq_lens[b]
 * stays as it is (its logits and the cache row at seq_lens[b] are
 * scratch).  Every other sequence steps as in q3_decode_step, so a
 * fixed number of calls can be captured in one graph and replayed with no
 * host check between steps; a sequence that has finished just repeats
 * eos_id.  eos_id = -1 disables the rule (q3_decode_step).
 * Errors: those of q3_decode_step, and Q3_ERR_SHAPE for eos_id outside
 * -1 .. 151935. */
int q3_decode_step_eos(const q3_model *m, const q3_kv *kv, int32_t batch, const int32_t *in_ids,
                       int32_t *seq_lens, int32_t max_len_hint, int32_t eos_id, float *logits,
                       int32_t *out_ids, void *ws, size_t ws_bytes, void *stream);

/* q3_decode_step_eos for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step with the same results, but the workspace is a
 * fixed scratch array inside the library, one per GPU, held until the
 * process ends (Q3_NOALLOC_MAX_BYTES, enough for q3_workspace_bytes(batch,
 * 1) up to batch 32).  The call itself allocates and frees nothing; its
 * first call on a device looks up that device's scratch address (with the
 * device current).  The caller still passes inputs and outputs as for
 * q3_decode_step_eos; `stream` must belong to the current device.  Every
 * call on one GPU shares that GPU's scratch, so calls that overlap on one
 * GPU (different streams, different threads) race: order them.  Nothing in
 * the scratch needs to start at zero (the step clears its own tickets).
 * Errors: those of q3_decode_step_eos, and Q3_ERR_TOO_LARGE when
 * q3_workspace_bytes(batch, 1) exceeds Q3_NOALLOC_MAX_BYTES (batch > 32). */
#define Q3_NOALLOC_MAX_BYTES (21u << 20)
int q3_decode_step_noalloc(const q3_model *m, const q3_kv *kv, int32_t batch, const int32_t *in_ids,
                           int32_t *seq_lens, int32_t max_len_hint, int32_t eos_id, float *logits,
                           int32_t *out_ids, void *stream);

/* Row-wise greedy argmax ("手写Qwen3-0.6B推理" §推理; "第 3 章" §4.3):
 * out_idx[r] = lowest index v with logits[r*row_stride + v] equal to the
 * row maximum (a NaN counts as larger than every number; the first NaN
 * wins).
 *   logits      float32, `rows` rows of `vocab` values, row_stride
 *               elements apart (row_stride >= vocab; 16-byte aligned rows
 *               are faster but not required).
 *   out_idx     int32 [rows].
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (rows < 1, vocab < 1,
 * row_stride < vocab), Q3_ERR_HIP. */
int q3_argmax(const float *logits, int32_t rows, int32_t vocab, int64_t row_stride,
              int32_t *out_idx, void *stream);


/* Temperature / top-k / top-p sampling of logits rows over the whole
 * vocabulary: the path "第 3 章" §4.3's Sampler.sample takes when
 * temperatures are given (the pages name the steps; this is their plain
 * reading).  Row r, with T = temperature[r], k = top_k[r], p = top_p[r],
 * u = uniform[r]:
 *   - T <= 0 (or NaN): greedy, as q3_argmax;
 *   - z = logits / T;
 *   - candidates: every token with z >= the k-th largest z, ties included
 *     (k <= 0 or k >= vocab: every token), ordered by z descending then
 *     index ascending;
 *   - softmax over the candidates; keep the shortest prefix of that order
 *     whose mass reaches p (p outside (0, 1] means 1);
 *   - out_idx[r] = the first kept candidate whose cumulative mass exceeds
 *     u times the kept mass (u is clamped to [0, 1)).
 * There is no cap on the number of candidates.  z is float32 (logits times
 * 1/T); masses are exp(z - max z) in float32, summed exactly as 40-bit fixed
 * point integers, so a call is reproducible bit for bit; the random draw is
 * the caller's.  Rows holding NaN or +inf give some index in [0, vocab).
 *   logits       float32, rows x vocab, row_stride elements apart.
 *   temperature  float32 [rows]; top_k int32 [rows]; top_p float32 [rows];
 *   uniform      float32 [rows]; out_idx int32 [rows]  (all device).
 *   ws           device workspace of q3_sample_workspace_bytes(rows, vocab)
 *                bytes (about 100 KB per row), 16-byte aligned; no initial
 *                content is needed.
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (rows outside 1 .. 65536, vocab < 1,
 * row_stride < vocab), Q3_ERR_ALIGN (4-byte alignment; ws 16-byte),
 * Q3_ERR_WORKSPACE, Q3_ERR_HIP. */
size_t q3_sample_workspace_bytes(int32_t rows, int32_t vocab);
int q3_sample(const float *logits, int32_t rows, int32_t vocab, int64_t row_stride, const float *temperature,
              const int32_t *top_k, const float *top_p, const float *uniform, int32_t *out_idx, void *ws,
              size_t ws_bytes, void *stream);

/* Epilogues of q3_linear. */
enum {
  Q3_EPI_STORE_BF16 = 0, /* out bf16 [m, ldo]:  out[i, j] = (x W^T)[i, j]            */
  Q3_EPI_STORE_F32 = 1,  /* out f32  [m, ldo]                                         */
  Q3_EPI_ADD_F32 = 2,    /* out f32  [m, ldo] += x W^T  (residual add)                */
  Q3_EPI_SILU_GATE = 3   /* W is [gate; up] with n rows; out bf16 [m, ldo] holds
                            silu(x Wg^T) * (x Wu^T), n/2 columns                      */
};

/* Helper: one projection y = x W^T on the same MFMA GEMM kernels the model
 * uses (skinny weight-streaming kernel for m <= 128 rows, LDS-tiled kernel
 * above), e.g. the tied lm_head of "手写Qwen3-0.6B推理" §Qwen3Model or a
 * merged projection of "第 3 章" §3.3/§3.4.
 *   x    bf16 [m, k] row-major;  w  bf16 [n, k] row-major ([out, in]).
 *   out  see the epilogue; ldo is its row stride in elements (>= n, or
 *        >= n/2 for Q3_EPI_SILU_GATE).
 * Requirements: m >= 1, n % 128 == 0, k % 512 == 0.
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (sizes, ldo or epilogue invalid),
 * Q3_ERR_ALIGN (16-byte alignment), Q3_ERR_HIP. */
int q3_linear(const void *x, const void *w, void *out, int32_t m, int32_t n, int32_t k, int32_t ldo,
              int32_t epilogue, void *stream);

/* Helper: causal GQA attention of a chunk of n_tokens queries over one
 * layer's filled KV cache ("手写Qwen3-0.6B推理" §Attention; "第 3 章" §3.3).
 * For sequence b, query head h (KV head h/2) and chunk row t at position
 * p = start_pos + t:
 *   out[b, t, h, :] = sum_{j <= p} softmax_j(q[b, t, h, :] . K[b, h/2, j, :] / sqrt(128)) V[b, h/2, j, :]
 *   q        bf16 [batch, n_tokens, 16, 128], already normed and rotated;
 *   k_layer, v_layer  one layer of a KV cache of capacity max_seq (layouts
 *            as in q3_kv); rows 0 .. start_pos + n_tokens - 1 are read;
 *   out      bf16 [batch, n_tokens, 2048].
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (batch or n_tokens < 1, max_seq not a
 * multiple of 8 in 8..40960), Q3_ERR_POSITION (start_pos < 0 or
 * start_pos + n_tokens > max_seq), Q3_ERR_ALIGN (16 B), Q3_ERR_HIP. */
int q3_attention_prefill(const void *q, const void *k_layer, const void *v_layer, int32_t batch,
                         int32_t n_tokens, int32_t start_pos, int32_t max_seq, void *out, void *stream);

/* Helper: the attention half of a multi-token call as q3_layer_forward and
 * q3_prefill run it ("古法手撕简易LLM推理器" §prefill与predict): for a chunk
 * of n_tokens rows per sequence at positions p = start_pos .. start_pos +
 * n_tokens - 1, from the raw projection rows, the per-head k RMSNorm and
 * RoPE at p write the rotated K and the raw V into cache row p, then each
 * query head gets the q RMSNorm and RoPE at its position as the attention
 * loads it, and attends over rows 0..p as in q3_attention_prefill.
 *   qkv       bf16 [batch, n_tokens, 4096] raw q|k|v rows (as
 *             q3_layer_weights.w_qkv orders them);
 *   q_norm, k_norm  bf16 [128] gains; rope_cos, rope_sin as in q3_model;
 *   k_layer, v_layer  one layer of a KV cache of capacity max_seq;
 *   write_kv  1: write the chunk's K and V rows first; 0: those rows
 *             already hold them (an earlier call with 1) and only the
 *             attention runs;
 *   out       bf16 [batch, n_tokens, 2048].
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (as q3_attention_prefill, or write_kv
 * not 0 or 1), Q3_ERR_POSITION (start_pos < 0 or start_pos + n_tokens >
 * max_seq), Q3_ERR_ALIGN (16 B), Q3_ERR_HIP. */
int q3_attention_prefill_qkv(const void *qkv, const void *q_norm, const void *k_norm, const float *rope_cos,
                             const float *rope_sin, void *k_layer, void *v_layer, int32_t batch, int32_t n_tokens,
                             int32_t start_pos, int32_t max_seq, int32_t write_kv, void *out, void *stream);

/* Helper: the attention half of one decode step for one new token per
 * sequence, as q3_decode_step runs it ("古法手撕简易LLM推理器"
 * §prefill与predict): from the raw projection rows of the new tokens it
 * applies the per-head q/k RMSNorm and RoPE at each token's position p,
 * writes the rotated K and the raw V into cache row p, and attends over
 * rows 0..p.
 *   qkv        bf16 [batch, 4096] raw q|k|v rows (as q3_layer_weights.w_qkv orders them);
 *   q_norm, k_norm  bf16 [128] gains; rope_cos, rope_sin as in q3_model;
 *   k_layer, v_layer  one layer of a KV cache of capacity max_seq;
 *   positions  device int32 [batch]: p of each new token (p < max_seq);
 *   max_len_hint  host bound with max(positions) < max_len_hint <= max_seq
 *              (it sets only the number of key-range splits);
 *   out        bf16 [batch, 2048];
 *   ws         >= q3_workspace_bytes(batch, 1) bytes (split partials, tickets).
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE, Q3_ERR_POSITION (max_len_hint outside
 * 1..max_seq), Q3_ERR_ALIGN, Q3_ERR_WORKSPACE, Q3_ERR_HIP. */
int q3_attention_decode(const void *qkv, const void *q_norm, const void *k_norm, const float *rope_cos,
                        const float *rope_sin, void *k_layer, void *v_layer, int32_t batch, int32_t max_seq,
                        const int32_t *positions, int32_t max_len_hint, void *out, void *ws, size_t ws_bytes,
                        void *stream);

/* Helper: q3_attention_decode as q3_decode_step launches it for up to 8
 * sequences whose attention occupies at most 64 workgroups: the same
 * launch also reads the layer's o_proj weight (bf16 [1024][2048]), its
 * gate|up weight (bf16 [6144][1024]), its down weight (bf16 [1024][3072])
 * and the next layer's q|k|v weight (bf16 [4096][1024]) into the L2 caches
 * of the XCDs whose workgroups read them in the projections that follow.  The results are those of
 * q3_attention_decode; only the time differs.  When the condition does not
 * hold the weights are ignored.  The four pointers are read only
 * (ownership stays with the caller).
 * Errors: as q3_attention_decode, and Q3_ERR_NULL / Q3_ERR_ALIGN (16 B) for
 * the weights. */
int q3_attention_decode_warm(const void *qkv, const void *q_norm, const void *k_norm, const float *rope_cos,
                             const float *rope_sin, void *k_layer, void *v_layer, int32_t batch, int32_t max_seq,
                             const int32_t *positions, int32_t max_len_hint, void *out, void *ws,
                             size_t ws_bytes, const void *w_o, const void *w_gate_up, const void *w_down,
                             const void *w_qkv_next, void *stream);

/* Rotary-pairing conversion for weights trained with interleaved rotary
 * pairs (dims 2i, 2i+1 rotated by p * 1e6^(-2i/128); "从零开始写Qwen3（二）"
 * §rope/原理 describes this pairing next to the half-swap one that Qwen3
 * uses, "古法手撕简易LLM推理器" §RoPE的细节).  Such a layer equals a
 * half-swap layer whose q and k projection rows and q/k norm gains are
 * permuted within each head by P(j) = 2j (j < 64), 2(j - 64) + 1 (j >= 64):
 * attention scores are q.k sums, unchanged by a common permutation of the
 * q and k dims, and the per-head RMSNorm commutes with it.  This call
 * writes that permuted copy; the layer then runs on every other entry
 * point unchanged (its cache holds the keys in the permuted dim order).
 *   w_qkv   bf16 [4096, 1024] merged rows as in q3_layer_weights;
 *           w_qkv_out gets q rows (heads 0..15) and k rows (heads 0..7)
 *           permuted, v rows copied.
 *   q_norm, k_norm  bf16 [128] gains; *_out their permuted copies.
 * Outputs must not overlap the inputs.
 * Errors: Q3_ERR_NULL, Q3_ERR_SHAPE (an output overlaps an input),
 * Q3_ERR_ALIGN (16 B), Q3_ERR_HIP. */
int q3_rope_interleaved_to_half(const void *w_qkv, const void *q_norm, const void *k_norm, void *w_qkv_out,
                                void *q_norm_out, void *k_norm_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q3_H */
