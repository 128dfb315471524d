"""GPU parity of q3_prefill_packed: ragged prompts packed into one token
array (the engine layout "第 3 章" §3.1 describes, logits only at each
sequence's last position, §4.1), against the oracle run on each sequence
alone.  Covers the tiled-GEMM row counts, the skinny ones, the persistent
GEMMs (over 2048 rows, q/k norm + RoPE in the q|k|v epilogue), query blocks
that straddle sequences, and a chunked continuation (start positions > 0)."""
import numpy as np
import pytest

import oracle as O
from decoder_only_transformer_qwen3_amd import inputs as I

from gpu_common import REL_TOL, bf16_tensor_to_f64, check_greedy_step, GreedyReport, log, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoder_only_transformer_qwen3_amd import binding, device
    log("[packed] generating 28-layer random-init weights (seed 0)")
    bits = I.model_weights(0)
    return binding, device, device.DeviceModel(bits), O.Model(bits)


def _packed_call(B, dev, dm, kv, seqs, starts=None):
    lens = [len(s) for s in seqs]
    n, N = len(seqs), int(sum(lens))
    ids = torch.from_numpy(np.concatenate(seqs).astype(np.int32)).cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    st = None if starts is None else torch.tensor(np.asarray(starts, dtype=np.int32), device="cuda")
    logits = torch.empty((n, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(n, dtype=torch.int32, device="cuda")
    seq = torch.empty(n, dtype=torch.int32, device="cuda")
    nb = B.q3_workspace_bytes_packed(n, N)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    B.q3_prefill_packed(dm.struct, kv.struct, n, N, ids, cu, st, max(lens), logits, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), nxt.cpu().numpy(), seq.cpu().numpy()


@pytest.mark.parametrize("lens", [
    [1, 7, 64, 130, 300],   # 502 rows: tiled GEMMs; query blocks of 64 cross every sequence boundary
    [3, 1, 9],              # 13 rows: skinny GEMMs
    [1100, 3, 950],         # 2053 rows: persistent GEMMs, q/k norm + RoPE through the row map
])
def test_packed_prefill_matches_each_sequence_alone(setup, lens):
    B, dev, dm, om = setup
    seqs = [I.token_ids(100 + i, (1, t))[0] for i, t in enumerate(lens)]
    kv = dev.DeviceKV(len(lens), (max(lens) + 7) // 8 * 8)
    logits, nxt, seq = _packed_call(B, dev, dm, kv, seqs)
    np.testing.assert_array_equal(seq, lens)
    rep = GreedyReport()
    for s, ids in enumerate(seqs):
        o_logits, _, cache, _ = O.prefill(om, ids[None, :])
        check_greedy_step(rep, int(nxt[s]), logits[s], o_logits[0])
        if s == len(seqs) - 1:  # the cache rows this sequence wrote, last layer
            kg = bf16_tensor_to_f64(kv.k[27, s, :, :len(ids)])
            e = rel_err(kg, cache.k[27][0])
            log(f"[packed] sequence {s}: last-layer K rows rel err {e:.2e}")
            assert e <= REL_TOL
    log(f"[packed] lengths {lens}: {rep}")
    assert rep.near_ties == 0, rep


def test_packed_chunked_continuation(setup):
    """Two packed calls: the first prefills 5 and 40 tokens, the second
    continues the same sequences with 20 and 3 more at start positions 5
    and 40; the result must be the prefill of the 25- and 43-token prompts."""
    B, dev, dm, om = setup
    full = [I.token_ids(200, (1, 25))[0], I.token_ids(201, (1, 43))[0]]
    kv = dev.DeviceKV(2, 48)
    _packed_call(B, dev, dm, kv, [full[0][:5], full[1][:40]])
    logits, nxt, seq = _packed_call(B, dev, dm, kv, [full[0][5:], full[1][40:]], starts=[5, 40])
    np.testing.assert_array_equal(seq, [25, 43])
    rep = GreedyReport()
    for s in range(2):
        o_logits, _, _, _ = O.prefill(om, full[s][None, :])
        check_greedy_step(rep, int(nxt[s]), logits[s], o_logits[0])
    log(f"[packed] chunked continuation: {rep}")
    assert rep.near_ties == 0, rep


def test_packed_head_over_more_than_64_sequences(setup):
    """70 short packed prompts: the head runs two lm_head launches (64 + 6
    rows) that share one ticket; sequences on both sides of the split and
    at its edges against the oracle, and every sequence's length."""
    B, dev, dm, om = setup
    lens = [2 + (i * 3) % 5 for i in range(70)]  # 2..6 tokens, 280 rows
    seqs = [I.token_ids(300 + i, (1, t))[0] for i, t in enumerate(lens)]
    kv = dev.DeviceKV(len(lens), 8)
    logits, nxt, seq = _packed_call(B, dev, dm, kv, seqs)
    np.testing.assert_array_equal(seq, lens)
    rep = GreedyReport()
    for s in (0, 1, 62, 63, 64, 65, 69):
        o_logits, _, _, _ = O.prefill(om, seqs[s][None, :])
        check_greedy_step(rep, int(nxt[s]), logits[s], o_logits[0])
    log(f"[packed] 70 sequences: {rep}")
    assert rep.near_ties == 0, rep
