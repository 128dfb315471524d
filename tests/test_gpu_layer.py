"""GPU parity of one decoder layer (q3_layer_forward) and of q3_argmax
against the float64 oracle, through the C ABI.

Shapes cover the one-layer workload (1 x 16 tokens), the skinny/tiled GEMM
boundary (128 / 129 rows), several tiles with a ragged tail, a multi-token
chunk at an offset into a filled cache, decode-shaped calls (one token) at
small, capacity-edge and full sizes (batch 32 over 2048 cached positions,
batch 4 over 32768, 129 rows on the tiled GEMMs), the last position the
rotary table holds (40959), and the 8 x 4096 prefill shape (one sequence
checked against the oracle).
"""
import numpy as np
import pytest

import oracle as O
from decoder_only_transformer_qwen3_amd import inputs as I

from gpu_common import (REL_TOL, bf16_tensor_to_f64, cache_fill_bits, log, rel_err, v_blocked_to_dense,
                        v_dense_to_blocked)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoder_only_transformer_qwen3_amd import binding, device
    return binding, device


@pytest.fixture(scope="module")
def layer0(lib):
    B, dev = lib
    bits = I.layer_weights(seed=0, i=0)
    return bits, O.LayerW(bits), dev.DeviceLayer(bits)


@pytest.fixture(scope="module")
def rope(lib):
    B, dev = lib
    return dev.rope_tables()


def run_layer_case(lib, layer0, rope, batch, T, start, max_seq, check_seqs=None, seed=7):
    B, dev = lib
    bits, ow, dl = layer0
    log(f"[layer] batch={batch} T={T} start={start} max_seq={max_seq}")
    x_bits = I.hidden_states(seed, (batch, T, B.HIDDEN))
    kshape = (batch, B.N_KV_HEADS, max_seq, B.HEAD_DIM)
    kc_bits = np.zeros(kshape, dtype=np.uint16)
    vc_bits = np.zeros(kshape, dtype=np.uint16)
    if start > 0:
        kc_bits[:, :, :start] = cache_fill_bits(seed + 1, (batch, B.N_KV_HEADS, start, B.HEAD_DIM))
        vc_bits[:, :, :start] = cache_fill_bits(seed + 2, (batch, B.N_KV_HEADS, start, B.HEAD_DIM))
    kc = dev.to_device_bf16(kc_bits)
    vc = dev.to_device_bf16(v_dense_to_blocked(vc_bits))
    resid = torch.from_numpy(O.widen_bf16(x_bits).astype(np.float32)).cuda().reshape(batch * T, B.HIDDEN)
    ws, nbytes = dev.workspace(batch, T)
    B.q3_layer_forward(dl.struct(), rope[0], rope[1], kc, vc, batch, T, max_seq, start, resid, ws, nbytes)
    torch.cuda.synchronize()
    got = resid.cpu().numpy().astype(np.float64).reshape(batch, T, B.HIDDEN)
    kg, vg = bf16_tensor_to_f64(kc), v_blocked_to_dense(bf16_tensor_to_f64(vc))
    assert np.all(np.isfinite(got))

    seqs = range(batch) if check_seqs is None else check_seqs
    worst = 0.0
    for b in seqs:
        x = O.widen_bf16(x_bits[b:b + 1])
        ko = O.widen_bf16(kc_bits[b:b + 1]).copy()
        vo = O.widen_bf16(vc_bits[b:b + 1]).copy()
        ref = O.layer_forward(ow, x, ko, vo, start, O.QWEN3)
        e = rel_err(got[b], ref[0])
        ek = rel_err(kg[b, :, start:start + T], ko[0, :, start:start + T])
        ev = rel_err(vg[b, :, start:start + T], vo[0, :, start:start + T])
        # earlier rows and rows past the new ones are untouched
        np.testing.assert_array_equal(kg[b, :, :start], ko[0, :, :start])
        np.testing.assert_array_equal(vg[b, :, :start], vo[0, :, :start])
        np.testing.assert_array_equal(kg[b, :, start + T:], 0.0)
        np.testing.assert_array_equal(vg[b, :, start + T:], 0.0)
        log(f"   seq {b}: residual rel={e:.3e} K rel={ek:.3e} V rel={ev:.3e}")
        assert e <= REL_TOL and ek <= REL_TOL and ev <= REL_TOL
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("batch,T,start,max_seq", [
    (1, 16, 0, 16),       # one-layer workload: 1 x 16 tokens, positions 0..15
    (1, 64, 0, 64),       # 64 rows: four 16-row token blocks in the skinny GEMM
    (1, 65, 0, 80),       # 65 rows: five token blocks, one of them ragged
    (1, 128, 0, 128),     # largest skinny-GEMM row count (eight token blocks)
    (1, 129, 0, 136),     # smallest tiled-GEMM row count
    (2, 100, 0, 128),     # several tiles + ragged tail on every axis
    (2, 77, 50, 160),     # multi-token chunk at an offset into a filled cache
    (3, 1, 700, 1024),    # decode-shaped, host start position
    (4, 2, 30, 64),       # 8 rows: the largest fused post-attention kernel
    (1, 5, 3, 16),        # 5 rows at an offset
    (1, 1, 0, 8),         # single key
    (2, 1, 4095, 4096),   # decode into the last cache row
    (5, 3, 13, 16),       # tiny chunk, several sequences, cache full afterwards
    (2, 11, 53, 72),      # unaligned chunk spanning three 8-position V blocks
    (1, 200, 0, 200),     # 128-position query tiles with a ragged last tile
    (65, 1, 100, 128),    # 65 decode rows: the skinny GEMMs over five token blocks
    (129, 1, 100, 128),   # 129 decode rows: the tiled GEMMs with one token per sequence
    (97, 2, 10, 16),      # 194 rows over 97 sequences: two row tiles, K split
    (1, 1, 40959, 40960), # decode at the last position of the rotary table
    (1, 64, 40896, 40960),  # a prefill chunk ending at the position limit
    (3, 777, 100, 896),   # 2331 rows at an offset: the persistent GEMMs, q/k norm + RoPE in the
                          # q|k|v epilogue, a ragged last row tile of 27 rows
])
def test_layer_forward_parity(lib, layer0, rope, batch, T, start, max_seq):
    run_layer_case(lib, layer0, rope, batch, T, start, max_seq)


def test_layer_forward_decode_batch32_ctx2048(lib, layer0, rope):
    """Decode-bound shape: batch 32, 2048 cached positions, new token at 2048."""
    run_layer_case(lib, layer0, rope, 32, 1, 2048, 2176, check_seqs=[0, 13, 31])


def test_layer_forward_decode_long_context(lib, layer0, rope):
    """Long-context shape: batch 4, 32768 cached positions."""
    run_layer_case(lib, layer0, rope, 4, 1, 32768, 32832, check_seqs=[0, 3])


def test_layer_forward_prefill_8x4096(lib, layer0, rope):
    """Prefill-bound shape: 8 x 4096 tokens from position 0 (sequence 5 checked)."""
    run_layer_case(lib, layer0, rope, 8, 4096, 0, 4096, check_seqs=[5])


def test_layer_forward_repeatable(lib, layer0, rope):
    """Two identical calls give bit-identical results (no atomics, fixed order)."""
    B, dev = lib
    bits, ow, dl = layer0
    outs = []
    for _ in range(2):
        x = torch.from_numpy(O.widen_bf16(I.hidden_states(3, (40, B.HIDDEN))).astype(np.float32)).cuda()
        kc = torch.zeros((4, 8, 64, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        ws, nb = dev.workspace(4, 10)
        B.q3_layer_forward(dl.struct(), rope[0], rope[1], kc, vc, 4, 10, 64, 0, x, ws, nb)
        torch.cuda.synchronize()
        outs.append(x.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])


# ------------------------------------------------------------------ argmax

def test_argmax_exact(lib):
    B, dev = lib
    V = B.VOCAB
    rng = np.random.default_rng(0)
    rows = rng.standard_normal((9, V)).astype(np.float32)
    rows[1, :] = 0.0                        # all equal -> 0
    rows[2, [5, 77, 150000]] = 9.0          # duplicate maxima -> lowest
    rows[3, V - 1] = 50.0                   # max at the end
    rows[4, 0] = 50.0                       # max at the start
    rows[5, [10, 20]] = np.nan              # first NaN wins
    rows[6, :] = -np.inf
    rows[6, 12345] = -1e30
    rows[7, :] = -np.inf                    # all -inf -> 0
    t = torch.from_numpy(rows).cuda()
    out = torch.empty(9, dtype=torch.int32, device="cuda")
    B.q3_argmax(t, 9, V, V, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    expect = np.argmax(rows, axis=1)        # numpy: first occurrence, first NaN
    np.testing.assert_array_equal(got, expect)
    assert got[1] == 0 and got[2] == 5 and got[3] == V - 1 and got[5] == 10 and got[6] == 12345 and got[7] == 0


def test_argmax_strided_and_short_rows(lib):
    B, dev = lib
    rng = np.random.default_rng(1)
    for vocab, stride, nrows in ((1, 1, 3), (7, 9, 4), (1000, 1003, 5), (151936, 152000, 2)):
        buf = rng.standard_normal((nrows, stride)).astype(np.float32)
        t = torch.from_numpy(buf).cuda()
        out = torch.empty(nrows, dtype=torch.int32, device="cuda")
        B.q3_argmax(t, nrows, vocab, stride, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), np.argmax(buf[:, :vocab], axis=1))
