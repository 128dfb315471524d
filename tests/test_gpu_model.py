"""GPU parity of the full 28-layer stack (q3_prefill, q3_decode_step)
against the float64 oracle, through the C ABI.

Greedy tokens follow the protocol in gpu_common.check_greedy_step: the GPU
runs free, the oracle is teacher-forced on the GPU's tokens, every step's
logits must be within the relative tolerance, and a token may differ from
the oracle's argmax only at a near tie inside the measured error.  (The
long-context case compares with stored oracle logits, so there the GPU is
fed the oracle's tokens instead.)
"""
import json
import os

import numpy as np
import pytest

import oracle as O
from decoder_only_transformer_qwen3_amd import inputs as I

from gpu_common import GreedyReport, REL_TOL, check_greedy_step, log, oracle_prefill_logged, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoder_only_transformer_qwen3_amd import binding, device
    return binding, device


@pytest.fixture(scope="module")
def models(lib):
    B, dev = lib
    log("[model] generating 28-layer random-init weights (seed 0)")
    bits = I.model_weights(0)
    dm = dev.DeviceModel(bits)
    om = O.Model(bits)
    return dm, om


def test_prefill_then_64_greedy_steps(lib, models):
    """Full stack, batch 1, 128-token prompt, prefill then 64 greedy decode steps."""
    B, dev = lib
    dm, om = models
    T, steps = 128, 64
    ids = I.token_ids(1, (1, T))
    kv = dev.DeviceKV(1, T + steps)
    ids_d = torch.from_numpy(ids).cuda()
    logits = torch.empty((1, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    seq = torch.empty(1, dtype=torch.int32, device="cuda")
    ws, nb = dev.workspace(1, T)
    log("[model] prefill 1 x 128")
    B.q3_prefill(dm.struct, kv.struct, 1, T, ids_d, logits, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    assert int(seq.item()) == T
    gpu_logits = [logits.cpu().numpy()[0].copy()]
    gpu_tokens = [int(nxt.item())]
    # the returned token is the argmax of the returned logits, exactly
    assert gpu_tokens[0] == int(np.argmax(gpu_logits[0]))
    wsd, nbd = dev.workspace(1, 1)
    for i in range(steps):
        B.q3_decode_step(dm.struct, kv.struct, 1, nxt, seq, T + steps, logits, nxt, wsd, nbd)
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()[0].copy()
        tok = int(nxt.item())
        assert tok == int(np.argmax(lg))
        gpu_logits.append(lg)
        gpu_tokens.append(tok)
    assert int(seq.item()) == T + steps
    log(f"[model] gpu tokens: {gpu_tokens}")

    log("[model] oracle, teacher-forced on the GPU tokens")
    _, o_logits = O.generate_cached(om, ids, steps + 1, forced=gpu_tokens)
    rep = GreedyReport()
    for i in range(steps + 1):
        check_greedy_step(rep, gpu_tokens[i], gpu_logits[i], o_logits[i])
    if rep.strict_prefix is None:
        rep.strict_prefix = steps + 1
    log(f"[model] greedy report: {rep}")
    assert rep.near_ties == 0, rep


def test_decode_sequences_of_different_lengths(lib, models):
    """Batch 4 decode where each sequence sits at its own length."""
    B, dev = lib
    dm, om = models
    T0, lens = 24, [24, 17, 9, 21]
    ids = I.token_ids(2, (4, T0 + 3))
    kv = dev.DeviceKV(4, 40)
    ws, nb = dev.workspace(4, T0)
    nxt = torch.empty(4, dtype=torch.int32, device="cuda")
    seq = torch.empty(4, dtype=torch.int32, device="cuda")
    B.q3_prefill(dm.struct, kv.struct, 4, T0, torch.from_numpy(np.ascontiguousarray(ids[:, :T0])).cuda(), None,
                 nxt, seq, ws, nb)
    # truncate sequences to their own lengths; feed the next prompt token of each
    seq.copy_(torch.tensor(lens, dtype=torch.int32))
    feed = torch.tensor([int(ids[b, lens[b]]) for b in range(4)], dtype=torch.int32, device="cuda")
    logits = torch.empty((4, B.VOCAB), dtype=torch.float32, device="cuda")
    wsd, nbd = dev.workspace(4, 1)
    B.q3_decode_step(dm.struct, kv.struct, 4, feed, seq, 40, logits, nxt, wsd, nbd)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    assert seq.cpu().numpy().tolist() == [n + 1 for n in lens]
    for b in range(4):
        ref, _, _, _ = O.prefill(om, ids[b:b + 1, :lens[b] + 1])
        e = rel_err(got[b], ref[0])
        log(f"   seq {b} (len {lens[b]}): logits rel={e:.3e}")
        assert e <= REL_TOL
        assert int(nxt[b].item()) == int(np.argmax(got[b]))


@pytest.mark.timeout(1200)
def test_prefill_8x4096_vs_oracle(lib, models):
    """The prefill-bound workload (batch 8 x 4096-token prompts of uniform
    random ids, drawn as the benchmark draws them): the last-position logits
    and greedy tokens of sequences 0 and 7 against the float64 oracle run on
    each prompt alone ("古法手撕简易LLM推理器" §prefill与predict: prefill,
    then the next token), and each sequence's logits equal, bit for bit,
    those of the same prompt prefilled alone."""
    B, dev = lib
    dm, om = models
    Bn, T = 8, 4096
    ids = I.token_ids(1000 + Bn, (Bn, T))
    kv = dev.DeviceKV(Bn, T)
    ws, nb = dev.workspace(Bn, T)
    logits = torch.empty((Bn, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(Bn, dtype=torch.int32, device="cuda")
    seq = torch.empty(Bn, dtype=torch.int32, device="cuda")
    log("[model] prefill 8 x 4096")
    B.q3_prefill(dm.struct, kv.struct, Bn, T, torch.from_numpy(ids).cuda(), logits, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    toks = nxt.cpu().numpy()
    assert np.all(np.isfinite(lg))
    np.testing.assert_array_equal(toks, np.argmax(lg, axis=1))
    assert seq.cpu().numpy().tolist() == [T] * Bn
    del kv, ws
    kv1 = dev.DeviceKV(1, T)
    ws1, nb1 = dev.workspace(1, T)
    rep = GreedyReport()
    for b in (0, 7):
        l1 = torch.empty((1, B.VOCAB), dtype=torch.float32, device="cuda")
        B.q3_prefill(dm.struct, kv1.struct, 1, T, torch.from_numpy(np.ascontiguousarray(ids[b:b + 1])).cuda(), l1,
                     nxt[:1], seq[:1], ws1, nb1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(l1.cpu().numpy()[0], lg[b])
        log(f"[model] oracle prefill of sequence {b} (4096 tokens)")
        ref, _, _ = oracle_prefill_logged(om, ids[b:b + 1], tag=f"seq {b}")
        check_greedy_step(rep, int(toks[b]), lg[b], ref[0])
        log(f"   seq {b}: token {toks[b]} (oracle {int(np.argmax(ref[0]))}), logits rel={rel_err(lg[b], ref[0]):.3e}")
    log(f"[model] 8 x 4096: {rep}")
    assert rep.near_ties == 0, rep


@pytest.mark.timeout(1200)
def test_decode_b32_ctx2048_vs_oracle(lib, models):
    """The decode-bound workload's shape: batch 32 prompts of 2048 uniform
    random ids (drawn as the benchmark draws them), prefill, then two greedy
    decode steps at positions 2048 and 2049.  Sequences 0 and 31 against the
    float64 oracle, teacher-forced on the GPU's tokens, at every step."""
    B, dev = lib
    dm, om = models
    Bn, T, steps = 32, 2048, 2
    ids = I.token_ids(1000 + Bn, (Bn, T))
    kv = dev.DeviceKV(Bn, T + 8)
    ws, nb = dev.workspace(Bn, T)
    logits = torch.empty((Bn, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(Bn, dtype=torch.int32, device="cuda")
    seq = torch.empty(Bn, dtype=torch.int32, device="cuda")
    log("[model] prefill 32 x 2048")
    B.q3_prefill(dm.struct, kv.struct, Bn, T, torch.from_numpy(ids).cuda(), logits, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    del ws
    lgs, toks = [logits.cpu().numpy().copy()], [nxt.cpu().numpy().copy()]
    wsd, nbd = dev.workspace(Bn, 1)
    for i in range(steps):
        B.q3_decode_step(dm.struct, kv.struct, Bn, nxt, seq, T + steps, logits, nxt, wsd, nbd)
        torch.cuda.synchronize()
        lgs.append(logits.cpu().numpy().copy())
        toks.append(nxt.cpu().numpy().copy())
    assert seq.cpu().numpy().tolist() == [T + steps] * Bn
    for i in range(steps + 1):
        np.testing.assert_array_equal(toks[i], np.argmax(lgs[i], axis=1))
    rep = GreedyReport()
    for b in (0, Bn - 1):
        forced = [int(toks[i][b]) for i in range(steps + 1)]
        log(f"[model] oracle: sequence {b}, 2048-token prefill + {steps} teacher-forced steps")
        lg0, _, cache = oracle_prefill_logged(om, ids[b:b + 1], max_seq=T + steps, tag=f"seq {b}")
        o_logits = [lg0[0]]
        for i in range(steps):   # "古法手撕简易LLM推理器" §prefill与predict: one token per step
            lg_i, _ = O.decode_step(om, cache, [forced[i]], [T + i])
            o_logits.append(lg_i[0])
        for i in range(steps + 1):
            check_greedy_step(rep, forced[i], lgs[i][b], o_logits[i])
        log(f"   seq {b}: tokens {forced}")
    log(f"[model] batch 32 x 2048: {rep}")
    assert rep.near_ties == 0, rep


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.timeout(600)
def test_long_context_b4_ctx32768_vs_oracle(lib, models):
    """The long-context workload's shape: batch 4 prompts of 32768 uniform
    random ids (drawn as the benchmark draws them), prefill, then two decode
    steps at positions 32768 and 32769.  Sequence 0 against the float64
    oracle's logits, stored by tests/golden/make_long_context.py (a float64
    prefill of this length takes about an hour, too long to run here).  The
    stored run is greedy on the oracle's own tokens, so sequence 0 is fed
    those tokens here (the other sequences run free); every step's logits
    must be within the tolerance and the GPU's token must be the oracle's."""
    B, dev = lib
    dm, _ = models
    z = np.load(os.path.join(GOLDEN, "long_context_b4_ctx32768_seq0.npz"))
    meta = json.loads(str(z["meta"]))
    Bn, T, steps = meta["batch"], meta["prompt_len"], meta["steps"]
    assert meta["weight_seed"] == 0 and meta["sequence"] == 0
    o_logits = z["logits"].astype(np.float64)
    o_tokens = [int(t) for t in z["tokens"]]
    assert o_tokens == [int(O.argmax_lowest(l[None])[0]) for l in o_logits]
    ids = I.token_ids(meta["id_seed"], (Bn, T))
    kv = dev.DeviceKV(Bn, T + 8)
    ws, nb = dev.workspace(Bn, T)
    logits = torch.empty((Bn, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(Bn, dtype=torch.int32, device="cuda")
    seq = torch.empty(Bn, dtype=torch.int32, device="cuda")
    log(f"[model] prefill {Bn} x {T}")
    B.q3_prefill(dm.struct, kv.struct, Bn, T, torch.from_numpy(ids).cuda(), logits, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    del ws
    lgs, toks = [logits[0].cpu().numpy().copy()], [int(nxt[0].item())]
    wsd, nbd = dev.workspace(Bn, 1)
    for i in range(steps):
        nxt[0] = o_tokens[i]
        B.q3_decode_step(dm.struct, kv.struct, Bn, nxt, seq, T + steps, logits, nxt, wsd, nbd)
        torch.cuda.synchronize()
        lgs.append(logits[0].cpu().numpy().copy())
        toks.append(int(nxt[0].item()))
    assert seq.cpu().numpy().tolist() == [T + steps] * Bn
    rep = GreedyReport()
    for i in range(steps + 1):
        check_greedy_step(rep, toks[i], lgs[i], o_logits[i])
        log(f"   step {i}: token {toks[i]} (oracle {o_tokens[i]}), logits rel={rel_err(lgs[i], o_logits[i]):.3e}")
    log(f"[model] batch 4 x 32768, sequence 0: {rep}")
    assert rep.near_ties == 0, rep


def test_fused_argmax_ties_take_the_lowest_index(lib, models):
    """The lm_head's fused argmax breaks exact ties toward the lowest index
    ("手写Qwen3-0.6B推理" §推理: torch.argmax), across 16-column blocks and
    inside one: copies of the winning token's embedding row at other indices
    (none of them fed as input) tie its logit exactly; q3_prefill and
    q3_decode_step must then return the lowest of the tied indices."""
    B, dev = lib
    dm, om = models
    T = 16
    ids = I.token_ids(11, (1, T))
    f = int(I.token_ids(12, (1, 1))[0, 0])
    kv = dev.DeviceKV(1, 24)
    ws, nb = dev.workspace(1, T)
    wsd, nbd = dev.workspace(1, 1)
    logits = torch.empty((1, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    seq = torch.empty(1, dtype=torch.int32, device="cuda")
    feed = torch.tensor([f], dtype=torch.int32, device="cuda")

    def run(m):
        B.q3_prefill(m, kv.struct, 1, T, torch.from_numpy(ids).cuda(), logits, nxt, seq, ws, nb)
        torch.cuda.synchronize()
        lp, tp = logits.cpu().numpy()[0].copy(), int(nxt.item())
        B.q3_decode_step(m, kv.struct, 1, feed, seq, 24, logits, nxt, wsd, nbd)
        torch.cuda.synchronize()
        return lp, tp, logits.cpu().numpy()[0].copy(), int(nxt.item())

    lp, top_p, ld, top_d = run(dm.struct)
    used = set(ids[0].tolist()) | {f, top_p, top_d}

    def free(cands):
        out = []
        for c in cands:
            if 0 <= c < B.VOCAB and c not in used and c not in out:
                out.append(c)
        return out

    # prefill: a lower copy in another 16-column block, higher copies next to and far from the winner
    tie_p = free([top_p - 37, top_p - 53, top_p + 1, top_p + 50])
    # decode: a lower copy inside the winner's 16-column block when there is room, and a higher one
    tie_d = free([top_d - 1, top_d - 2, top_d + 20, top_d + 3])
    used |= set(tie_p) | set(tie_d)
    embed2 = dm.embed.clone()
    for c in tie_p:
        embed2[c] = embed2[top_p]
    for c in tie_d:
        embed2[c] = embed2[top_d]
    m2 = B.q3_model.from_buffer_copy(dm.struct)
    m2.embed = embed2.data_ptr()
    lp2, tp2, ld2, td2 = run(m2)
    # the copies tie exactly on the GPU (same weights, same arithmetic) ...
    assert all(lp2[c] == lp2[top_p] for c in tie_p), [(c, lp2[c], lp2[top_p]) for c in tie_p]
    assert all(ld2[c] == ld2[top_d] for c in tie_d), [(c, ld2[c], ld2[top_d]) for c in tie_d]
    assert lp2[top_p] == lp[top_p] and ld2[top_d] == ld[top_d]
    # ... and the fused argmax returns the lowest tied index
    want_p, want_d = min(tie_p + [top_p]), min(tie_d + [top_d])
    log(f"[model] tie: prefill winner {top_p}, copies {tie_p} -> {tp2} (want {want_p}); "
        f"decode winner {top_d}, copies {tie_d} -> {td2} (want {want_d})")
    assert tp2 == want_p and td2 == want_d
    assert tp2 == int(np.argmax(lp2)) and td2 == int(np.argmax(ld2))


def test_prefill_tiled_path_parity(lib, models):
    """Full stack on the tiled-GEMM + flash-attention path (2 x 300 tokens)."""
    B, dev = lib
    dm, om = models
    ids = I.token_ids(5, (2, 300))
    kv = dev.DeviceKV(2, 304)
    ws, nb = dev.workspace(2, 300)
    logits = torch.empty((2, B.VOCAB), dtype=torch.float32, device="cuda")
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    seq = torch.empty(2, dtype=torch.int32, device="cuda")
    B.q3_prefill(dm.struct, kv.struct, 2, 300, torch.from_numpy(ids).cuda(), logits, nxt, seq, ws, nb)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    ref, _, _, _ = O.prefill(om, ids)
    rep = GreedyReport()
    for b in range(2):
        e = rel_err(got[b], ref[b])
        log(f"   seq {b}: logits rel={e:.3e}")
        check_greedy_step(rep, int(nxt[b].item()), got[b], ref[b])
    log(f"[model] {rep}")
    assert rep.near_ties == 0, rep
