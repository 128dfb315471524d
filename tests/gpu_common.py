"""Helpers shared by the GPU parity tests: seeded inputs on both sides,
error metrics, and the greedy-token protocol."""
import sys

import numpy as np

import oracle as O
from decoder_only_transformer_qwen3_amd import inputs as I

REL_TOL = 2e-2  # max |gpu - oracle| / max |oracle| for hidden states and logits (bf16, fp32 accumulation)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return O.widen_bf16(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))


def v_blocked_to_dense(v: np.ndarray) -> np.ndarray:
    """[..., S, D] array read from the blocked V cache (blocks of 8 positions,
    dim-major inside a block) -> position-major [..., S, D]."""
    *lead, S, Dd = v.shape
    return v.reshape(*lead, S // 8, Dd, 8).swapaxes(-1, -2).reshape(*lead, S, Dd)


def v_dense_to_blocked(v: np.ndarray) -> np.ndarray:
    """Inverse of v_blocked_to_dense (the array keeps its [..., S, D] shape)."""
    *lead, S, Dd = v.shape
    return np.ascontiguousarray(v.reshape(*lead, S // 8, 8, Dd).swapaxes(-1, -2)).reshape(*lead, S, Dd)


def cache_fill_bits(seed: int, shape) -> np.ndarray:
    """Synthetic earlier-position cache content: N(0, 1) bf16 bits."""
    return I.normal_bf16(seed, "cache_fill", shape, std=1.0)


class GreedyReport:
    def __init__(self):
        self.steps = 0
        self.near_ties = 0
        self.ties = []          # (step, gpu token, oracle token, oracle gap, 2 * max logit error)
        self.strict_prefix = None
        self.max_rel = 0.0

    def __repr__(self):
        return (f"steps={self.steps} near_ties={self.near_ties} strict_prefix={self.strict_prefix} "
                f"max_rel={self.max_rel:.3e} ties={self.ties}")


def check_greedy_step(rep: GreedyReport, gpu_token: int, gpu_logits: np.ndarray, oracle_logits: np.ndarray):
    """The GPU token must equal the oracle's argmax, except at a near tie:
    logit_o[top] - logit_o[gpu] <= 2 * max_v |logit_gpu[v] - logit_o[v]|.
    Near ties are recorded with their gap; the tests assert that their
    fixed seeds meet none."""
    err = float(np.max(np.abs(gpu_logits.astype(np.float64) - oracle_logits)))
    rel = err / float(np.max(np.abs(oracle_logits)))
    rep.max_rel = max(rep.max_rel, rel)
    assert rel <= REL_TOL, f"step {rep.steps}: logits rel err {rel:.3e}"
    top = int(O.argmax_lowest(oracle_logits)[0])
    if gpu_token != top:
        gap = float(oracle_logits[top] - oracle_logits[gpu_token])
        assert gap <= 2 * err, f"step {rep.steps}: token {gpu_token} vs oracle {top}, gap {gap:.4g} > 2*err {2*err:.4g}"
        rep.near_ties += 1
        rep.ties.append((rep.steps, gpu_token, top, round(gap, 6), round(2 * err, 6)))
        log(f"   near tie at step {rep.steps}: gpu {gpu_token}, oracle {top}, oracle gap {gap:.3e}, "
            f"2 * max logit error {2 * err:.3e}")
        if rep.strict_prefix is None:
            rep.strict_prefix = rep.steps
    rep.steps += 1


def oracle_prefill_logged(om, ids, max_seq=None, tag="oracle"):
    """O.prefill (embed, the layers in order, final logits), one log line per
    few layers so a long float64 run shows its progress."""
    ids = np.asarray(ids)
    b_sz, t_len = ids.shape
    cache = O.KVCache(om.cfg, len(om.layers), b_sz, max_seq or t_len)
    x = O.embed(om, ids)
    for li, w in enumerate(om.layers):
        x = O.layer_forward(w, x, cache.k[li], cache.v[li], 0, om.cfg)
        if li % 7 == 6:
            log(f"   [{tag}] {t_len}-token prefill: layer {li + 1}/{len(om.layers)}")
    logits = O.final_logits(om, x[:, -1, :])
    return logits, O.argmax_lowest(logits), cache
