// Host-side launchers of the gfx950 kernels (internal to libq3).
// Every launcher only enqueues on the given stream; shapes are validated
// by the C-ABI entry points before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

enum Epi : int {
  EPI_BF16 = 0,     // out bf16 [M, ldo] (column offset = output row of W)
  EPI_F32 = 1,      // out f32 [M, ldo]
  EPI_ADD_F32 = 2,  // out f32 [M, ldo] += result (residual add)
  EPI_SILU = 3,     // W rows are [gate; up]; out bf16 [M, ldo] = silu(gate) * up
  EPI_PARTIAL = 4,  // out f32 [split][M][N] partial sums over a K range
};

// x[m] = E[ids[m]] widened to f32 (one row of 1024 per token); with a gain
// also hg[m] = bf16(gamma * x[m]) and ssq[m][j] = sum of x^2 over columns
// group j (nsq = NSQ: 4 columns, NSQ_BLK: 16 columns).  The first
// n_counters ints of `counters` are set to zero.
void launch_embed(const int32_t* ids, const uint16_t* E, float* resid, int M, const uint16_t* gamma, uint16_t* hg,
                  float* ssq, int nsq, int* counters, int n_counters, hipStream_t s);

// hg[r] = bf16(gamma * resid[r*row_step + row_off]) and ssq[r][nsq] for r < n_rows;
// clears n_counters tickets.
// With `last` (packed rows), row r is instead the last row of sequence r.
void launch_norm_operand(const float* resid, int n_rows, int row_step, int row_off, const uint16_t* gamma,
                         uint16_t* hg, float* ssq, int nsq, int* counters, int n_counters, hipStream_t s,
                         const SeqMap* last = nullptr);

// For r < n_rows, row = r*row_step + row_off:
//   resid[row] += sum_{j < n_part} part[j][row]      (written back when n_part > 0)
//   out[r] = bf16(resid[row] / sqrt(mean(resid[row]^2) + eps) * gamma)   (when out != null)
// part is [n_part][part_rows][1024].
void launch_rmsnorm(float* resid, const float* part, int n_part, int part_rows, const uint16_t* gamma,
                    uint16_t* out, int n_rows, int row_step, int row_off, hipStream_t s);

// K rows (per-head k RMSNorm + NeoX RoPE) and raw V rows of the merged qkv
// projection [rows][4096] into the cache, each row at its sequence and
// position (SeqMap); max_T bounds the rows of one sequence.
void launch_kv_store(const uint16_t* qkv, const uint16_t* k_norm, const float* rope_cos, const float* rope_sin,
                     uint16_t* k_cache, uint16_t* v_cache, const SeqMap& sm, int max_T, int max_seq, hipStream_t s);

// MFMA tiled GEMM, out = X[M,K] * W[N,K]^T with the chosen epilogue.
// Requires N % 128 == 0 (EPI_SILU: N = 2*ldo-columns, (N/2) % 64 == 0), K % 64 == 0.
// n_split > 1 (128 x 128 tiles only; (K / 64) % n_split == 0) splits K:
// part holds n_split * M * N fp32 partial sums, added in split order by a
// second kernel that applies the epilogue.  reduce = false (EPI_ADD_F32
// into a [M][1024] residual) leaves that sum to the RMSNorm that reads the
// residual next (launch_rmsnorm with part / n_split).
void launch_gemm_tiled(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo,
                       Epi epi, hipStream_t s, int n_split = 1, float* part = nullptr, bool reduce = true);

// MFMA skinny GEMM for M <= 128 rows (weight streaming), split into n_split K ranges.
// Requires N % 16 == 0 and (K / n_split) % 512 == 0; EPI_PARTIAL writes [n_split][M][N].
struct SkinnyArgs {
  const uint16_t* X;  // activations, row m at X + m * ldx (ldx = 0 means K)
  const uint16_t* W;  // weights [N, K]
  void* out;
  int M, N, K, ldo, ldx, kspan;
  void* amax_part;    // launch_lm_head: its workgroups' (max, argmax) candidates
  // Optional input-norm scale: X holds bf16(gamma * r); output row m is
  // multiplied by 1 / sqrt(sum_{j<ssq_n} ssq[m * ssq_ld + j] / 1024 + eps).
  // ssq_n (also the layout of ssq_out below) is NSQ for up to 8 rows, else NSQ_BLK.
  const float* ssq;
  int ssq_ld, ssq_n;
  // EPI_PARTIAL finish (N == 1024, resid != null): the last workgroup of
  // each 16-column block adds all K splits to resid [M][1024]; with a gain
  // it also writes hg = bf16(gamma * r) [M][1024] and ssq_out [M][ssq_n].
  // counters: 64 ints, zero on entry and left zero on exit.
  // EPI_ADD_F32 with a gain (N == ldo == 1024): after out += X W^T, the same
  // hg and ssq_out of the updated rows.
  float* resid;
  const uint16_t* gamma;
  uint16_t* hg;
  float* ssq_out;
  int* counters;
};
void launch_gemm_skinny(SkinnyArgs a, int n_split, Epi epi, hipStream_t s);

// Greedy choice of the rows r0 .. r0 + M - 1 of a head call: out_idx[r],
// and seq_lens[r] by seq_mode (1: = seq_val; 2: += 1, except that with
// eos >= 0 a row whose input token in_ids[r] is eos has finished and emits
// eos again with its length kept; 3: start + rows of sequence r of sm,
// packed prefill).
struct HeadPick {
  int32_t* out_idx;
  int32_t* seq_lens;
  int seq_mode, seq_val;
  const int32_t* in_ids;
  int eos;
  SeqMap sm;  // seq_mode 3 only
  int r0;
};
// Tied lm_head over up to 64 rows: out [M][ldo] (skipped when out is null)
// = (1 / rms) * X E^T for E = W [151936][1024], and the greedy token of
// each row (pick).  Uses X, ldx, W, out, M, ldo, ssq, ssq_ld, ssq_n of the
// arguments; amax_part is scratch of at least (number of CUs) * M float2
// and `ticket` one int that is zero on entry (and left zero).
void launch_lm_head(const SkinnyArgs& a, const HeadPick& pick, int* ticket, hipStream_t s);

// resid[M][1024] += X[M][K] W[1024][K]^T for M <= 8, K in {1024, 2048, 3072};
// with a gain also hg = bf16(gamma * r) and ssq_out [M][256].
void launch_gemv_resid(const uint16_t* X, const uint16_t* W, int K, float* resid, int M, const uint16_t* gamma,
                       uint16_t* hg, float* ssq_out, hipStream_t s);
void launch_gemm_skinny(const uint16_t* X, const uint16_t* W, void* out, int M, int N, int K, int ldo,
                        int n_split, Epi epi, hipStream_t s);

// Copy of the merged q|k|v rows and the q/k gains with the q and k rows of
// every head (and the gains) permuted by P(j) = 2j (j < 64), 2(j-64)+1.
void launch_rope_pair_permute(const uint16_t* w_qkv, const uint16_t* q_norm, const uint16_t* k_norm,
                              uint16_t* w_out, uint16_t* qn_out, uint16_t* kn_out, hipStream_t s);

// Temperature / top-k / top-p sampling of `rows` logits rows over the whole
// vocabulary (radix selects over the row in chunks, one workgroup per chunk);
// per-row parameters and uniform draws; ws laid out by q3v::sample_ws_layout.
void launch_sample(const float* logits, int rows, int vocab, int64_t stride, const float* temperature,
                   const int32_t* top_k, const float* top_p, const float* uniform, int32_t* out, void* ws,
                   hipStream_t s);

// Causal GQA flash attention over the cache for the rows of a multi-token
// call: the rows of sequence s at positions start_s .. start_s + T_s - 1
// (SeqMap); max_T bounds T_s.  Query row m is q + m * ldq (16 heads of 128).
// With q_norm, the query rows are the raw projection: each head gets the
// q RMSNorm and NeoX RoPE at its position as it is loaded.
void launch_attn_prefill(const uint16_t* q, int ldq, const uint16_t* q_norm, const float* rope_cos,
                         const float* rope_sin, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out,
                         const SeqMap& sm, int max_T, int max_seq, hipStream_t s);

// Split-K decode attention for one new token per sequence, from the raw
// merged projection qkv [B][4096]: per-head q/k RMSNorm + RoPE of the new
// token, its K/V written into the cache at its position, attention over
// positions 0..p, and the log-sum-exp merge of the splits done by the last
// workgroup of each (sequence, KV head) (counters: B*8 ints, zero on entry,
// left zero).  out is [B][2048] bf16; part holds [B][16][n_split][130] f32.
// warm_o / warm_gate_up / warm_down / warm_qkv (all or none): the layer's
// o_proj [1024][2048], gate|up [6144][1024] and down [1024][3072] weights and
// the next layer's q|k|v [4096][1024] weight, read ahead into the L2 caches
// that the one-block skinny GEMM and the up-to-8-row GEMV will read them
// through (worth it only when the attention itself occupies few CUs).
void launch_attn_decode(const uint16_t* qkv, const uint16_t* q_norm, const uint16_t* k_norm, const float* rope_cos,
                        const float* rope_sin, uint16_t* k_cache, uint16_t* v_cache, float* part, int* counters,
                        uint16_t* out, int B, int max_seq, const int32_t* pos_dev, int start, int n_split,
                        bool streaming, hipStream_t s, const void* warm_o = nullptr,
                        const void* warm_gate_up = nullptr, const void* warm_down = nullptr,
                        const void* warm_qkv = nullptr);

// Row argmax (lowest index on ties, first NaN wins).  seq_mode: 0 none,
// 1 seq_lens[r] = seq_val, 2 seq_lens[r] += 1 (done after the argmax).
void launch_argmax(const float* logits, int rows, int vocab, int64_t row_stride, int32_t* out_idx,
                   int32_t* seq_lens, int seq_mode, int seq_val, hipStream_t s);

}  // namespace q3
