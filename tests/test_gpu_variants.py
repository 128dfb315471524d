"""GPU parity of the model variants the pages describe next to Qwen3's own
choices, through the C ABI.

Interleaved rotary pairs ("从零开始写Qwen3（二）" §rope/原理): a model
trained with pairs (2i, 2i+1) runs on the half-swap kernels after
q3_rope_interleaved_to_half permutes its q/k rows and q/k gains; the result
must match the oracle computing interleaved rotary directly.
"""
import numpy as np
import pytest

import oracle as O
from decoder_only_transformer_qwen3_amd import inputs as I

from gpu_common import GreedyReport, check_greedy_step, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoder_only_transformer_qwen3_amd import binding, device
    return binding, device


def _half_perm(d=128):
    return np.concatenate([2 * np.arange(d // 2), 2 * np.arange(d // 2) + 1])


def test_rope_pair_permutation_is_exact(lib):
    """The conversion moves bits only: q and k rows permuted within each head,
    v rows and every other element untouched, gains permuted."""
    B, dev = lib
    lw = I.layer_weights(5, 0)
    w = np.concatenate([lw["wq"], lw["wk"], lw["wv"]], axis=0)
    w_d, qn_d, kn_d = dev.to_device_bf16(w), dev.to_device_bf16(lw["q_norm"]), dev.to_device_bf16(lw["k_norm"])
    w_o, qn_o, kn_o = torch.empty_like(w_d), torch.empty_like(qn_d), torch.empty_like(kn_d)
    B.q3_rope_interleaved_to_half(w_d, qn_d, kn_d, w_o, qn_o, kn_o)
    torch.cuda.synchronize()
    P = _half_perm()
    heads = w[:3072].reshape(24, 128, 1024)[:, P].reshape(3072, 1024)
    expect = np.concatenate([heads, w[3072:]], axis=0)
    as_bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(as_bits(w_o), expect)
    np.testing.assert_array_equal(as_bits(qn_o), lw["q_norm"][P])
    np.testing.assert_array_equal(as_bits(kn_o), lw["k_norm"][P])


def test_interleaved_rope_model_prefill_and_greedy_steps(lib):
    """28 layers with interleaved rotary: 1 x 24 prompt, prefill, 8 greedy
    steps on the converted weights, against the oracle with interleaved
    rotary (teacher-forced on the GPU tokens, greedy-token protocol)."""
    B, dev = lib
    log("[variant] generating 28-layer random-init weights (seed 3)")
    bits = I.model_weights(3)
    dm = dev.DeviceModel(bits)
    for i, dl in enumerate(dm.layers):
        w_o, qn_o, kn_o = torch.empty_like(dl.w_qkv), torch.empty_like(dl.q_norm), torch.empty_like(dl.k_norm)
        B.q3_rope_interleaved_to_half(dl.w_qkv, dl.q_norm, dl.k_norm, w_o, qn_o, kn_o)
        dl.w_qkv, dl.q_norm, dl.k_norm = w_o, qn_o, kn_o
        dl.fill(dm.struct.layer[i])
    torch.cuda.synchronize()
    om = O.Model(bits, O.Cfg(rope_style="interleaved"))
    T, steps = 24, 8
    ids = I.token_ids(4, (1, T))
    kv = dev.DeviceKV(1, T + steps)
    logits = torch.empty((1, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    seq = torch.empty(1, dtype=torch.int32, device="cuda")
    ws, nb = dev.workspace(1, T)
    B.q3_prefill(dm.struct, kv.struct, 1, T, torch.from_numpy(ids).cuda(), logits, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    toks, lgs = [int(nxt.item())], [logits.cpu().numpy()[0].copy()]
    wsd, nbd = dev.workspace(1, 1)
    for _ in range(steps):
        B.q3_decode_step(dm.struct, kv.struct, 1, nxt, seq, T + steps, logits, nxt, wsd, nbd)
        torch.cuda.synchronize()
        toks.append(int(nxt.item()))
        lgs.append(logits.cpu().numpy()[0].copy())
    log(f"[variant] gpu tokens: {toks}")
    _, o_logits = O.generate_cached(om, ids, steps + 1, forced=toks)
    rep = GreedyReport()
    for i in range(steps + 1):
        check_greedy_step(rep, toks[i], lgs[i], o_logits[i])
    # the half-swap oracle on the unconverted weights is a different model
    _, h_logits = O.generate_cached(O.Model(bits), ids, 1)
    assert np.max(np.abs(h_logits[0] - o_logits[0])) > 20 * np.max(np.abs(lgs[0] - o_logits[0]))
    log(f"[variant] greedy report: {rep}")
