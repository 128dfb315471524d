// Host-only checks of the C-ABI argument validation, built with g++ and the
// address/undefined-behaviour sanitizers (no GPU, no HIP runtime).
#include <cstdio>
#include <initializer_list>
#include <cstdlib>
#include <cstdint>

#include "../../decoder_only_transformer_qwen3_amd/csrc/validate.hpp"

static int failures = 0;
#define EXPECT_EQ(a, b)                                                              \
  do {                                                                               \
    long long _a = (long long)(a), _b = (long long)(b);                              \
    if (_a != _b) {                                                                  \
      std::printf("FAIL %s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #a, _a, _b); \
      ++failures;                                                                    \
    }                                                                                \
  } while (0)

// fake, never dereferenced device addresses
static void* A(uintptr_t x) { return reinterpret_cast<void*>(x); }

static q3_layer_weights good_layer() {
  q3_layer_weights w;
  w.input_norm = A(0x1000); w.w_qkv = A(0x2000); w.q_norm = A(0x3000); w.k_norm = A(0x4000);
  w.w_o = A(0x5000); w.post_norm = A(0x6000); w.w_gate_up = A(0x7000); w.w_down = A(0x8000);
  return w;
}

static q3_model good_model() {
  q3_model m;
  m.embed = A(0x10000); m.final_norm = A(0x20000);
  for (int l = 0; l < Q3_N_LAYERS; ++l) m.layer[l] = good_layer();
  m.rope_cos = static_cast<const float*>(A(0x30000)); m.rope_sin = static_cast<const float*>(A(0x40000));
  return m;
}

int main() {
  using namespace q3v;
  // ---- workspace layout
  EXPECT_EQ(ws_layout(0, 5).total, 0);
  EXPECT_EQ(ws_layout(1, 0).total, 0);
  const WsLayout L1 = ws_layout(1, 16), L2 = ws_layout(32, 1), L3 = ws_layout(8, 4096);
  EXPECT_EQ(L1.total > 0, 1);
  EXPECT_EQ(L1.apart, L1.amax);                // no decode partials for multi-token calls
  EXPECT_EQ(L2.apart < L2.amax, 1);            // decode partials present for one-token calls
  EXPECT_EQ(L3.part, L3.apart);                // no skinny partials above 64 rows
  EXPECT_EQ(L1.resid % 256, 0); EXPECT_EQ(L1.h % 256, 0); EXPECT_EQ(L1.fh % 256, 0);
  EXPECT_EQ(L3.total >= (size_t)8 * 4096 * (1024 * 4 + 1024 * 2 + 4096 * 2 + 2048 * 2 + 3072 * 2), 1);
  // ---- decode splits
  EXPECT_EQ(decode_streaming(1, 192), 0);     // 22 MB of caches: stays in the last-level cache
  EXPECT_EQ(decode_streaming(32, 2176), 1);
  EXPECT_EQ(decode_splits(32, 2176), 1);      // 256 (sequence, KV head) pairs fill the CUs
  EXPECT_EQ(decode_splits(4, 32832), 8);
  EXPECT_EQ(decode_splits(1, 1), 1);
  EXPECT_EQ(decode_splits(1, 192), 1);
  EXPECT_EQ(decode_streaming(2, 512), 0);
  EXPECT_EQ(decode_splits(2, 512), 2);        // not streaming: at least 256 keys per split
  EXPECT_EQ(decode_splits(1, 40960), 32);
  for (int b = 1; b <= 64; ++b)
    for (int c = 1; c < 40961; c += 997) {
      const int s = decode_splits(b, c);
      EXPECT_EQ(s >= 1 && s <= DEC_SPLIT_MAX, 1);
    }

  // ---- attention helpers
  {
    const void* p = A(0x1000);
    EXPECT_EQ(check_attn_prefill_call(p, p, p, 2, 16, 0, 64, p), Q3_OK);
    EXPECT_EQ(check_attn_prefill_call(nullptr, p, p, 2, 16, 0, 64, p), Q3_ERR_NULL);
    EXPECT_EQ(check_attn_prefill_call(p, p, p, 2, 16, 48, 64, p), Q3_OK);
    EXPECT_EQ(check_attn_prefill_call(p, p, p, 2, 16, 49, 64, p), Q3_ERR_POSITION);
    EXPECT_EQ(check_attn_prefill_call(p, p, p, 2, 16, 0, 68, p), Q3_ERR_SHAPE);
    const float* f = static_cast<const float*>(p);
    const int32_t* pos = static_cast<const int32_t*>(p);
    const size_t need = ws_layout(3, 1).total;
    EXPECT_EQ(check_attn_decode_call(p, p, p, f, f, p, p, 3, 64, pos, 64, p, p, need), Q3_OK);
    EXPECT_EQ(check_attn_decode_call(p, p, p, f, f, p, p, 3, 64, pos, 65, p, p, need), Q3_ERR_POSITION);
    EXPECT_EQ(check_attn_decode_call(p, p, p, f, f, p, p, 3, 64, nullptr, 64, p, p, need), Q3_ERR_NULL);
    EXPECT_EQ(check_attn_decode_call(p, p, p, f, f, p, p, 3, 64, pos, 64, p, p, need - 1), Q3_ERR_WORKSPACE);
  }

  // ---- q3_layer_forward
  q3_layer_weights w = good_layer();
  const float* cs = static_cast<const float*>(A(0x50000));
  void* kl = A(0x60000); void* vl = A(0x70000);
  const float* res = static_cast<const float*>(A(0x80000));
  void* ws = A(0x90000);
  const size_t need = ws_layout(2, 16).total;
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 64, 0, res, ws, need), Q3_OK);
  EXPECT_EQ(check_layer_call(nullptr, cs, cs, kl, vl, 2, 16, 64, 0, res, ws, need), Q3_ERR_NULL);
  q3_layer_weights wn = w; wn.w_down = nullptr;
  EXPECT_EQ(check_layer_call(&wn, cs, cs, kl, vl, 2, 16, 64, 0, res, ws, need), Q3_ERR_NULL);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 0, 16, 64, 0, res, ws, need), Q3_ERR_SHAPE);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 0, 64, 0, res, ws, need), Q3_ERR_SHAPE);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 40961, 0, res, ws, need), Q3_ERR_SHAPE);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 60, 0, res, ws, need), Q3_ERR_SHAPE);  // not a multiple of 8
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 4, 0, res, ws, need), Q3_ERR_SHAPE);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 64, 49, res, ws, need), Q3_ERR_POSITION);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 64, 48, res, ws, need), Q3_OK);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 64, -1, res, ws, need), Q3_ERR_POSITION);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 64, 0x7fffffff, res, ws, need), Q3_ERR_POSITION);
  q3_layer_weights wa = w; wa.q_norm = A(0x3002);
  EXPECT_EQ(check_layer_call(&wa, cs, cs, kl, vl, 2, 16, 64, 0, res, ws, need), Q3_ERR_ALIGN);
  EXPECT_EQ(check_layer_call(&w, cs, cs, A(0x60008), vl, 2, 16, 64, 0, res, ws, need), Q3_ERR_ALIGN);
  EXPECT_EQ(check_layer_call(&w, cs, cs, kl, vl, 2, 16, 64, 0, res, ws, need - 1), Q3_ERR_WORKSPACE);
  // precedence: NULL before SHAPE
  EXPECT_EQ(check_layer_call(&w, nullptr, cs, kl, vl, 0, 16, 64, 0, res, ws, need), Q3_ERR_NULL);

  // ---- q3_prefill
  q3_model m = good_model();
  q3_kv kv; kv.k = A(0xA0000); kv.v = A(0xB0000); kv.batch = 4; kv.max_seq = 256;
  const int32_t* ids = static_cast<const int32_t*>(A(0xC0004));  // 4-byte alignment is enough
  int32_t* nid = static_cast<int32_t*>(A(0xD0000));
  int32_t* sl = static_cast<int32_t*>(A(0xE0000));
  const size_t pneed = ws_layout(4, 128).total;
  EXPECT_EQ(check_prefill_call(&m, &kv, 4, 128, ids, nullptr, nid, sl, ws, pneed), Q3_OK);
  EXPECT_EQ(check_prefill_call(&m, &kv, 5, 128, ids, nullptr, nid, sl, ws, pneed), Q3_ERR_SHAPE);
  EXPECT_EQ(check_prefill_call(&m, &kv, 4, 257, ids, nullptr, nid, sl, ws, ws_layout(4, 257).total), Q3_ERR_POSITION);
  EXPECT_EQ(check_prefill_call(&m, &kv, 4, 128, ids, static_cast<const float*>(A(0xF0004)), nid, sl, ws, pneed), Q3_ERR_ALIGN);
  EXPECT_EQ(check_prefill_call(&m, &kv, 4, 128, static_cast<const int32_t*>(A(0xC0002)), nullptr, nid, sl, ws, pneed), Q3_ERR_ALIGN);
  EXPECT_EQ(check_prefill_call(&m, &kv, 4, 128, ids, nullptr, nid, sl, ws, pneed - 256), Q3_ERR_WORKSPACE);
  q3_model mn = m; mn.layer[27].w_o = nullptr;
  EXPECT_EQ(check_prefill_call(&mn, &kv, 4, 128, ids, nullptr, nid, sl, ws, pneed), Q3_ERR_NULL);
  q3_kv kc = kv; kc.max_seq = 250;
  EXPECT_EQ(check_prefill_call(&m, &kc, 4, 128, ids, nullptr, nid, sl, ws, pneed), Q3_ERR_SHAPE);
  q3_kv kb = kv; kb.max_seq = 40961;
  EXPECT_EQ(check_prefill_call(&m, &kb, 4, 128, ids, nullptr, nid, sl, ws, pneed), Q3_ERR_SHAPE);

  // ---- q3_decode_step
  const size_t dneed = ws_layout(4, 1).total;
  EXPECT_EQ(check_decode_call(&m, &kv, 4, ids, sl, 200, nullptr, nid, ws, dneed), Q3_OK);
  EXPECT_EQ(check_decode_call(&m, &kv, 4, ids, sl, 257, nullptr, nid, ws, dneed), Q3_ERR_POSITION);
  EXPECT_EQ(check_decode_call(&m, &kv, 4, ids, sl, 0, nullptr, nid, ws, dneed), Q3_ERR_POSITION);
  EXPECT_EQ(check_decode_call(&m, &kv, 0, ids, sl, 200, nullptr, nid, ws, dneed), Q3_ERR_SHAPE);
  EXPECT_EQ(check_decode_call(&m, &kv, 4, nullptr, sl, 200, nullptr, nid, ws, dneed), Q3_ERR_NULL);
  EXPECT_EQ(check_decode_call(&m, &kv, 4, ids, sl, 200, nullptr, nid, ws, dneed - 1), Q3_ERR_WORKSPACE);

  // ---- q3_argmax
  const float* lg = static_cast<const float*>(A(0x100000));
  int32_t* out = static_cast<int32_t*>(A(0x110000));
  EXPECT_EQ(check_argmax_call(lg, 3, 151936, 151936, out), Q3_OK);
  EXPECT_EQ(check_argmax_call(lg, 3, 10, 9, out), Q3_ERR_SHAPE);
  EXPECT_EQ(check_argmax_call(lg, 0, 10, 10, out), Q3_ERR_SHAPE);
  EXPECT_EQ(check_argmax_call(nullptr, 3, 10, 10, out), Q3_ERR_NULL);
  EXPECT_EQ(check_argmax_call(static_cast<const float*>(A(0x100002)), 3, 10, 10, out), Q3_ERR_ALIGN);

  if (failures) { std::printf("%d failures\n", failures); return 1; }
  // sampling workspace: regions in order, 256-B aligned, disjoint, sized for every row and chunk
  for (int rows : {1, 3, 32, 1 << 16}) {
    for (int vocab : {1, 50, 1023, 1024, 151936}) {
      const int G = sample_chunks(rows, vocab);
      EXPECT_EQ(G >= 1 && G <= 32 && (G == 1 || vocab / G >= 1024), true);
      const SampleWsLayout L = sample_ws_layout(rows, vocab);
      const size_t R = rows, RG = (size_t)rows * G;
      EXPECT_EQ(L.st, (size_t)0);
      EXPECT_EQ(L.tick >= L.st + SAMPLE_ROW_BYTES * R && L.cnt >= L.tick + 4 * R, true);
      EXPECT_EQ(L.mass >= L.cnt + 4 * RG * 256 && L.mini >= L.mass + 8 * RG * 256, true);
      EXPECT_EQ(L.best >= L.mini + 4 * RG * 256 && L.total >= L.best + 8 * RG, true);
      EXPECT_EQ((L.tick | L.cnt | L.mass | L.mini | L.best | L.total) % 256, (size_t)0);
    }
  }
  {
    const size_t need = sample_ws_layout(4, 100).total;
    const float* f = static_cast<const float*>(A(0x100000));
    const int32_t* k = static_cast<const int32_t*>(A(0x200000));
    int32_t* o = static_cast<int32_t*>(A(0x300000));
    EXPECT_EQ(check_sample_call(f, 4, 100, 100, f, k, f, f, o, A(0x400000), need), Q3_OK);
    EXPECT_EQ(check_sample_call(f, 4, 100, 100, f, k, f, f, o, A(0x400000), need - 1), Q3_ERR_WORKSPACE);
    EXPECT_EQ(check_sample_call(f, 4, 100, 100, f, k, f, f, o, nullptr, need), Q3_ERR_NULL);
    EXPECT_EQ(check_sample_call(f, 4, 100, 100, f, k, f, f, o, A(0x400004), need), Q3_ERR_ALIGN);
    EXPECT_EQ(check_sample_call(f, SAMPLE_MAX_ROWS + 1, 100, 100, f, k, f, f, o, A(0x400000), need), Q3_ERR_SHAPE);
  }
  std::printf("validate_test: all checks passed\n");
  return 0;
}
