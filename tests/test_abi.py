"""CPU-side checks of the C-ABI library: it loads, exports every function
that include/q3.h declares, rejects bad arguments before touching the GPU,
and its host-side RoPE table matches the oracle's angles.  No kernel is
launched here."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q3.h")


@pytest.fixture(scope="module")
def B():
    from decoder_only_transformer_qwen3_amd import build as bld
    if not os.path.exists(bld.LIB):
        bld.build(verbose=False)
    from decoder_only_transformer_qwen3_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q3_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("q3_layer_forward", "q3_prefill", "q3_decode_step", "q3_argmax",
              "q3_workspace_bytes", "q3_rope_table_host", "q3_status_str"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(B.EXPORTS)
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
        exported = set(re.findall(r"\b(q3_\w+)\b", out))
        assert set(declared_functions()) <= exported


def test_status_strings(B):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert B.q3_status_str(code) and B.q3_status_str(code) != "unknown status"
    assert B.q3_status_str(12345) == "unknown status"


def test_workspace_bytes(B):
    assert B.q3_workspace_bytes(0, 1) == 0 and B.q3_workspace_bytes(1, 0) == 0
    a, b = B.q3_workspace_bytes(1, 128), B.q3_workspace_bytes(8, 4096)
    assert 0 < a < b
    assert B.q3_workspace_bytes(32, 1) > B.q3_workspace_bytes(1, 1)


def _layer_struct(B, base=0x10000):
    w = B.q3_layer_weights()
    for i, (n, _) in enumerate(B.q3_layer_weights._fields_):
        setattr(w, n, base + 0x1000 * i)
    return w


def test_layer_forward_rejects_bad_arguments_before_any_launch(B):
    w = _layer_struct(B)
    need = B.q3_workspace_bytes(2, 16)
    args = dict(rope_cos=0x80000, rope_sin=0x90000, k_layer=0xA0000, v_layer=0xB0000, batch=2, n_tokens=16,
                max_seq=64, start_pos=0, residual=0xC0000, ws=0xD0000, ws_bytes=need)

    def call(**over):
        a = dict(args)
        a.update(over)
        return B.q3_layer_forward(over.pop("w", w), a["rope_cos"], a["rope_sin"], a["k_layer"], a["v_layer"],
                                  a["batch"], a["n_tokens"], a["max_seq"], a["start_pos"], a["residual"],
                                  a["ws"], a["ws_bytes"], stream=0, check=False)

    assert call(residual=None) == B.Q3_ERR_NULL
    wn = _layer_struct(B)
    wn.w_down = None
    assert call(w=wn) == B.Q3_ERR_NULL
    assert call(batch=0) == B.Q3_ERR_SHAPE
    assert call(n_tokens=-3) == B.Q3_ERR_SHAPE
    assert call(max_seq=40961) == B.Q3_ERR_SHAPE
    assert call(start_pos=49) == B.Q3_ERR_POSITION
    assert call(residual=0xC0004) == B.Q3_ERR_ALIGN
    assert call(ws_bytes=need - 1) == B.Q3_ERR_WORKSPACE
    with pytest.raises(B.Q3Error):
        B.q3_layer_forward(w, 0, 0x1, 0x1, 0x1, 1, 1, 1, 0, 0x1, 0x1, 1, stream=0)


def test_prefill_decode_argmax_reject_bad_arguments(B):
    m = B.q3_model()
    m.embed, m.final_norm, m.rope_cos, m.rope_sin = 0x100000, 0x110000, 0x120000, 0x130000
    for i in range(B.N_LAYERS):
        m.layer[i] = _layer_struct(B, 0x200000 + 0x10000 * i)
    kv = B.q3_kv()
    kv.k, kv.v, kv.batch, kv.max_seq = 0x400000, 0x500000, 4, 256
    need = B.q3_workspace_bytes(4, 128)
    st = B.q3_prefill(m, kv, 5, 128, 0x600000, None, 0x610000, 0x620000, 0x700000, need, stream=0, check=False)
    assert st == B.Q3_ERR_SHAPE
    st = B.q3_prefill(m, kv, 4, 300, 0x600000, None, 0x610000, 0x620000, 0x700000,
                      B.q3_workspace_bytes(4, 300), stream=0, check=False)
    assert st == B.Q3_ERR_POSITION
    st = B.q3_prefill(m, kv, 4, 128, 0x600000, None, 0x610000, 0x620000, 0x700000, need - 1, stream=0, check=False)
    assert st == B.Q3_ERR_WORKSPACE
    m2 = B.q3_model.from_buffer_copy(m)
    m2.layer[13].w_qkv = None
    st = B.q3_prefill(m2, kv, 4, 128, 0x600000, None, 0x610000, 0x620000, 0x700000, need, stream=0, check=False)
    assert st == B.Q3_ERR_NULL
    dneed = B.q3_workspace_bytes(4, 1)
    st = B.q3_decode_step(m, kv, 4, 0x600000, 0x620000, 257, None, 0x610000, 0x700000, dneed, stream=0, check=False)
    assert st == B.Q3_ERR_POSITION
    st = B.q3_decode_step(m, kv, 4, 0x600000, None, 100, None, 0x610000, 0x700000, dneed, stream=0, check=False)
    assert st == B.Q3_ERR_NULL
    eos = lambda e, hint=100: B.q3_decode_step_eos(m, kv, 4, 0x600000, 0x620000, hint, e, None, 0x610000, 0x700000,
                                                   dneed, stream=0, check=False)
    assert eos(B.VOCAB) == B.Q3_ERR_SHAPE and eos(-2) == B.Q3_ERR_SHAPE
    assert eos(151645, hint=257) == B.Q3_ERR_POSITION    # the decode-step checks come first
    pneed = B.q3_workspace_bytes_packed(3, 200)
    assert pneed > 0 and B.q3_workspace_bytes_packed(0, 5) == 0

    def pk(**kw):
        a = dict(n_seqs=3, n_tokens=200, ids=0x600000, cu=0x630000, start=None, mx=120, logits=None,
                 nxt=0x610000, seq=0x620000, ws=0x700000, nb=pneed)
        a.update(kw)
        return B.q3_prefill_packed(m, kv, a["n_seqs"], a["n_tokens"], a["ids"], a["cu"], a["start"], a["mx"],
                                   a["logits"], a["nxt"], a["seq"], a["ws"], a["nb"], stream=0, check=False)

    assert pk(cu=None) == B.Q3_ERR_NULL
    assert pk(n_seqs=5) == B.Q3_ERR_SHAPE              # more sequences than cache rows
    assert pk(n_tokens=2) == B.Q3_ERR_SHAPE            # fewer tokens than sequences
    assert pk(mx=201) == B.Q3_ERR_SHAPE                # a sequence longer than all the tokens
    assert pk(n_tokens=300, mx=260, nb=B.q3_workspace_bytes_packed(3, 300)) == B.Q3_ERR_POSITION
    assert pk(cu=0x630002) == B.Q3_ERR_ALIGN
    assert pk(start=0x640001) == B.Q3_ERR_ALIGN
    assert pk(nb=pneed - 1) == B.Q3_ERR_WORKSPACE
    assert B.q3_argmax(0x800000, 2, 10, 5, 0x900000, stream=0, check=False) == B.Q3_ERR_SHAPE
    lin = lambda *a: B.q3_linear(*a, stream=0, check=False)
    assert lin(None, 0x1000, 0x2000, 1, 128, 512, 128, 0) == B.Q3_ERR_NULL
    assert lin(0x1000, 0x2000, 0x3000, 1, 100, 512, 128, 0) == B.Q3_ERR_SHAPE
    assert lin(0x1000, 0x2000, 0x3000, 1, 128, 500, 128, 0) == B.Q3_ERR_SHAPE
    assert lin(0x1000, 0x2000, 0x3000, 1, 128, 512, 64, 0) == B.Q3_ERR_SHAPE
    assert lin(0x1000, 0x2000, 0x3000, 0, 128, 512, 128, 0) == B.Q3_ERR_SHAPE
    assert lin(0x1000, 0x2000, 0x3000, 1, 128, 512, 128, 7) == B.Q3_ERR_SHAPE
    assert lin(0x1008, 0x2000, 0x3000, 1, 128, 512, 128, 0) == B.Q3_ERR_ALIGN
    assert B.q3_argmax(None, 2, 10, 10, 0x900000, stream=0, check=False) == B.Q3_ERR_NULL


def test_attention_helpers_reject_bad_arguments(B):
    pf = lambda *a: B.q3_attention_prefill(*a, stream=0, check=False)
    assert pf(None, 0x2000, 0x3000, 2, 16, 0, 64, 0x4000) == B.Q3_ERR_NULL
    assert pf(0x1000, 0x2000, 0x3000, 0, 16, 0, 64, 0x4000) == B.Q3_ERR_SHAPE
    assert pf(0x1000, 0x2000, 0x3000, 2, 16, 0, 60, 0x4000) == B.Q3_ERR_SHAPE
    assert pf(0x1000, 0x2000, 0x3000, 2, 16, 49, 64, 0x4000) == B.Q3_ERR_POSITION
    assert pf(0x1000, 0x2000, 0x3000, 2, 16, -1, 64, 0x4000) == B.Q3_ERR_POSITION
    assert pf(0x1000, 0x2008, 0x3000, 2, 16, 0, 64, 0x4000) == B.Q3_ERR_ALIGN
    pq = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 2, 16, 0, 64, 1, 0x8000]

    def pqkv(i, value):
        a = list(pq)
        a[i] = value
        return B.q3_attention_prefill_qkv(*a, stream=0, check=False)

    assert pqkv(1, None) == B.Q3_ERR_NULL        # q gain
    assert pqkv(4, None) == B.Q3_ERR_NULL        # sin table
    assert pqkv(0, None) == B.Q3_ERR_NULL        # projection rows
    assert pqkv(11, 2) == B.Q3_ERR_SHAPE         # write_kv
    assert pqkv(7, 0) == B.Q3_ERR_SHAPE
    assert pqkv(9, 49) == B.Q3_ERR_POSITION
    assert pqkv(2, 0x3008) == B.Q3_ERR_ALIGN     # k gain
    assert pqkv(3, 0x4004) == B.Q3_ERR_ALIGN     # cos table
    need = B.q3_workspace_bytes(3, 1)
    base = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 3, 64, 0x8000, 64, 0x9000, 0xA000, need]

    def dec(i, value):
        a = list(base)
        a[i] = value
        return B.q3_attention_decode(*a, stream=0, check=False)

    assert dec(9, None) == B.Q3_ERR_NULL
    assert dec(7, 0) == B.Q3_ERR_SHAPE
    assert dec(8, 20) == B.Q3_ERR_SHAPE
    assert dec(10, 65) == B.Q3_ERR_POSITION
    assert dec(10, 0) == B.Q3_ERR_POSITION
    assert dec(9, 0x8002) == B.Q3_ERR_ALIGN
    assert dec(13, need - 1) == B.Q3_ERR_WORKSPACE


def test_rope_conversion_rejects_bad_arguments(B):
    conv = lambda *a: B.q3_rope_interleaved_to_half(*a, stream=0, check=False)
    W = 4096 * 1024 * 2
    ok = [0x10000000, 0x20000000, 0x20001000, 0x30000000, 0x40000000, 0x40001000]
    for i in range(6):
        a = list(ok)
        a[i] = None
        assert conv(*a) == B.Q3_ERR_NULL
    a = list(ok); a[3] = ok[0] + W - 16          # output rows overlap the input's tail
    assert conv(*a) == B.Q3_ERR_SHAPE
    a = list(ok); a[4] = ok[1] + 128             # output gain overlaps the input gain
    assert conv(*a) == B.Q3_ERR_SHAPE
    a = list(ok); a[5] = ok[4]                   # the two output gains overlap
    assert conv(*a) == B.Q3_ERR_SHAPE
    a = list(ok); a[4] = ok[4] + 8
    assert conv(*a) == B.Q3_ERR_ALIGN


def test_sample_rejects_bad_arguments(B):
    smp = lambda *a: B.q3_sample(*a, stream=0, check=False)
    need = B.q3_sample_workspace_bytes(4, 100)
    assert need > 0 and B.q3_sample_workspace_bytes(0, 100) == 0 and B.q3_sample_workspace_bytes(4, 0) == 0
    assert B.q3_sample_workspace_bytes(4, 151936) > B.q3_sample_workspace_bytes(4, 100)
    ok = [0x1000, 4, 100, 100, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x10000, need]
    for i in (0, 4, 5, 6, 7, 8, 9):
        a = list(ok)
        a[i] = None
        assert smp(*a) == B.Q3_ERR_NULL
    for i, bad in ((1, 0), (1, (1 << 16) + 1), (2, 0), (3, 99)):
        a = list(ok)
        a[i] = bad
        assert smp(*a) == B.Q3_ERR_SHAPE
    a = list(ok); a[7] = 0x5002
    assert smp(*a) == B.Q3_ERR_ALIGN
    a = list(ok); a[9] = 0x10004
    assert smp(*a) == B.Q3_ERR_ALIGN
    a = list(ok); a[10] = need - 1
    assert smp(*a) == B.Q3_ERR_WORKSPACE


def test_rope_table_matches_oracle_angles(B):
    import oracle as O
    cos = np.empty((B.MAX_POS, 64), dtype=np.float32)
    sin = np.empty((B.MAX_POS, 64), dtype=np.float32)
    B.q3_rope_table_host(cos, sin)
    pos = np.array([0, 1, 2, 15, 127, 2047, 4095, 32767, 32831, 40959])
    ang = pos[:, None] * O.rope_inv_freq(128, 1e6)[None, :]
    # one rounding of a double-precision value to float32
    np.testing.assert_allclose(cos[pos], np.cos(ang), rtol=0, atol=6e-8)
    np.testing.assert_allclose(sin[pos], np.sin(ang), rtol=0, atol=6e-8)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)


def test_host_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "validate_test"
    src = [os.path.join(ROOT, "tests", "native", "validate_test.cpp"),
           os.path.join(ROOT, "decoder_only_transformer_qwen3_amd", "csrc", "validate.cpp")]
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", ROOT, *src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_attention_decode_warm_rejects_partial_or_misaligned_weights(B):
    """The read-ahead weights come as a set of four 16-byte-aligned pointers,
    checked before any launch."""
    need = B.q3_workspace_bytes(1, 1)
    base = (0x10000, 0x11000, 0x12000, 0x13000, 0x14000, 0x20000, 0x30000, 1, 64, 0x40000, 8, 0x50000, 0x60000,
            need)

    def call(wo, gu, dn, qk):
        return B.q3_attention_decode_warm(*base, wo, gu, dn, qk, stream=0, check=False)

    assert call(0x68000, 0x70000, None, 0x90000) == B.Q3_ERR_NULL
    assert call(None, None, 0x80000, None) == B.Q3_ERR_NULL
    assert call(0x68000, 0x70000, 0x80008, 0x90000) == B.Q3_ERR_ALIGN


def test_noalloc_decode_validates_before_touching_the_device(B):
    """The no-allocation decode step rejects a batch beyond its fixed scratch,
    and invalid arguments, on the host: no HIP call is made for them."""
    m, kv = B.q3_model(), B.q3_kv()
    assert B.q3_decode_step_noalloc(m, kv, 33, 0x1000, 0x2000, 8, -1, None, 0x3000, stream=0,
                                    check=False) == B.Q3_ERR_TOO_LARGE
    assert "scratch" in B.q3_status_str(B.Q3_ERR_TOO_LARGE)
    assert B.q3_decode_step_noalloc(m, kv, 4, 0x1000, 0x2000, 8, -1, None, 0x3000, stream=0,
                                    check=False) == B.Q3_ERR_NULL
