"""GPU parity of the projection kernels (q3_linear) and of HIP-graph replay
of the decode step.

q3_linear runs the skinny weight-streaming GEMM for up to 128 rows and the
LDS-tiled GEMM above; both are checked against the plain float64 product
x W^T on the layer's real projection shapes, with ragged row counts and
every epilogue.
"""
import numpy as np
import pytest

import oracle as O
from decoder_only_transformer_qwen3_amd import inputs as I

from gpu_common import REL_TOL, bf16_tensor_to_f64, log, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoder_only_transformer_qwen3_amd import binding, device
    return binding, device


SHAPES = [  # (name, n, k)
    ("qkv", 4096, 1024),
    ("o_proj", 1024, 2048),
    ("down", 1024, 3072),
    ("gate_up", 6144, 1024),
]


@pytest.mark.parametrize("m", [1, 7, 16, 33, 64, 65, 128, 129, 200, 2048, 2100])
@pytest.mark.parametrize("name,n,k", SHAPES)
def test_linear_all_epilogues(lib, m, name, n, k):
    B, dev = lib
    xb = I.normal_bf16(11, f"x{m}{name}", (m, k))
    wb = I.normal_bf16(12, f"w{name}", (n, k), std=0.02)
    x64, w64 = O.widen_bf16(xb), O.widen_bf16(wb)
    ref = x64 @ w64.T
    x, w = dev.to_device_bf16(xb), dev.to_device_bf16(wb)
    # bf16 store
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    B.q3_linear(x, w, out, m, n, k, n, B.Q3_EPI_STORE_BF16)
    # f32 store with a wider row stride
    out32 = torch.full((m, n + 4), 7.0, dtype=torch.float32, device="cuda")
    B.q3_linear(x, w, out32, m, n, k, n + 4, B.Q3_EPI_STORE_F32)
    # residual add
    base = np.random.default_rng(m).standard_normal((m, n)).astype(np.float32)
    acc = torch.from_numpy(base).cuda()
    B.q3_linear(x, w, acc, m, n, k, n, B.Q3_EPI_ADD_F32)
    torch.cuda.synchronize()
    e1 = rel_err(bf16_tensor_to_f64(out), ref)
    o32 = out32.cpu().numpy()
    e2 = rel_err(o32[:, :n], ref)
    assert np.all(o32[:, n:] == 7.0)  # padding columns untouched
    e3 = rel_err(acc.cpu().numpy().astype(np.float64) - base.astype(np.float64), ref)
    log(f"[linear] {name} m={m}: bf16 {e1:.2e} f32 {e2:.2e} add {e3:.2e}")
    assert e1 <= REL_TOL and e2 <= 1e-3 and e3 <= 1e-3
    if name == "gate_up":
        half = n // 2
        act = torch.empty((m, half), dtype=torch.bfloat16, device="cuda")
        B.q3_linear(x, w, act, m, n, k, half, B.Q3_EPI_SILU_GATE)
        torch.cuda.synchronize()
        ref_act = O.silu(ref[:, :half]) * ref[:, half:]
        e4 = rel_err(bf16_tensor_to_f64(act), ref_act)
        log(f"[linear] gate_up silu m={m}: {e4:.2e}")
        assert e4 <= REL_TOL


@pytest.mark.parametrize("m", [1, 5, 32])
def test_linear_lm_head_shape(lib, m):
    """The tied lm_head: 151936 x 1024 weight stream."""
    B, dev = lib
    k, n = 1024, B.VOCAB
    xb = I.normal_bf16(13, f"h{m}", (m, k))
    wb = I.normal_bf16(14, "embed_like", (n, k), std=0.02)
    out = torch.empty((m, n), dtype=torch.float32, device="cuda")
    B.q3_linear(dev.to_device_bf16(xb), dev.to_device_bf16(wb), out, m, n, k, n, B.Q3_EPI_STORE_F32)
    torch.cuda.synchronize()
    ref = O.widen_bf16(xb) @ O.widen_bf16(wb).T
    e = rel_err(out.cpu().numpy(), ref)
    log(f"[linear] lm_head m={m}: {e:.2e}")
    assert e <= 1e-3


def test_decode_graph_replay_matches_eager(lib):
    """A captured sequence of decode steps, replayed three times with eager
    work and synchronisation in between, reproduces the eager tokens and
    logits exactly on every replay."""
    B, dev = lib
    bits = I.model_weights(0)
    dm = dev.DeviceModel(bits)
    T, steps, batch = 32, 4, 3
    ids = torch.from_numpy(I.token_ids(6, (batch, T))).cuda()
    kv = dev.DeviceKV(batch, (T + steps + 7) // 8 * 8)
    ws, nb = dev.workspace(batch, T)
    wsd, nbd = dev.workspace(batch, 1)
    nxt = torch.zeros(batch, dtype=torch.int32, device="cuda")
    seq = torch.zeros(batch, dtype=torch.int32, device="cuda")
    logits = torch.zeros((batch, B.VOCAB), dtype=torch.float32, device="cuda")
    B.q3_prefill(dm.struct, kv.struct, batch, T, ids, None, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    nxt0, seq0 = nxt.clone(), seq.clone()

    def steps_fn():
        toks = []
        for _ in range(steps):
            B.q3_decode_step(dm.struct, kv.struct, batch, nxt, seq, T + steps, logits, nxt, wsd, nbd)
            toks.append(nxt.clone())
        return toks

    eager_toks = [t.cpu().numpy() for t in steps_fn()]
    eager_logits = logits.cpu().numpy().copy()
    nxt.copy_(nxt0)
    seq.copy_(seq0)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps_fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        graph_toks = steps_fn()
    for rep in range(3):
        nxt.copy_(nxt0)
        seq.copy_(seq0)
        logits.zero_()
        junk = torch.randn(1000, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            np.testing.assert_array_equal(graph_toks[i].cpu().numpy(), eager_toks[i])
        np.testing.assert_array_equal(logits.cpu().numpy(), eager_logits)
        assert seq.cpu().numpy().tolist() == [T + steps] * batch
        del junk
