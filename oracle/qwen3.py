"""Plain, slow, float64 CPU oracle of the Qwen3 decoder forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this module.

Every function computes the plain definition of one step, in the order and
notation of the pages it cites:

* "手写Qwen3-0.6B推理" (sections Qwen3Model, Qwen3DecoderLayer,
  Qwen3RMSNorm, Attention, Rope, MLP, 推理),
* "第 3 章 前向与生成（代码走读）" (sections 3.1-3.4, 4.1-4.3, 5),
* "从零开始写Qwen3（二）" (sections norm, rope/原理, rope/简单计算),
* "古法手撕简易LLM推理器" (sections 处理参数和超参数, 工具函数,
  核心计算函数与Transformer层, prefill与predict, RoPE的细节),
* "Pytorch手写大模型推理" (section 模型: the configuration values).

Inputs are bfloat16 bit patterns (uint16) that are widened exactly to
float64; nothing is rounded afterwards.  Only library primitives used as
steps: NumPy matrix products, exp, sqrt, sin, cos, max, sum.

Pinned by ``tests/test_oracle_pins.py`` against closed forms, invariants,
brute force and independent library routines.  The full 28-layer forward
on random weights has no printed numeric example on the pages: its values
are "parity unpinned" beyond the per-step pins and the model-level
invariants (causality, KV-cache equivalence, GQA reduction).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "Cfg", "QWEN3", "widen_bf16", "rmsnorm", "silu", "rope_inv_freq", "rope", "rope_interleaved", "apply_rope",
    "attention", "LayerW", "Model", "KVCache", "embed", "layer_forward",
    "final_logits", "prefill", "decode_step", "argmax_lowest", "sample",
    "generate_nocache", "generate_cached",
]


@dataclass(frozen=True)
class Cfg:
    """Hyper-parameters.  Defaults are the Qwen3-0.6B values printed in the
    configuration on "Pytorch手写大模型推理" (section 模型) and read from
    config.json on "古法手撕简易LLM推理器" (section 处理参数和超参数)."""

    hidden: int = 1024
    n_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    inter: int = 3072
    vocab: int = 151936
    n_layers: int = 28
    eps: float = 1e-6
    theta: float = 1e6
    max_pos: int = 40960
    # "neox": pairs (i, i + D/2), Qwen3's form; "interleaved": pairs (2i, 2i+1),
    # the other pairing "从零开始写Qwen3（二）" §rope/原理 describes
    rope_style: str = "neox"


QWEN3 = Cfg()


def widen_bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly (a bf16 value is the top
    half of a float32).  Large arrays go through torch's CPU bf16 -> f64
    conversion (multi-threaded, also exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if b.size >= (1 << 20):
        import torch
        return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return np.left_shift(b, 16, dtype=np.uint32).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- elementwise

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float = QWEN3.eps) -> np.ndarray:
    """RMSNorm over the last axis: gamma * x / sqrt(mean(x^2) + eps).

    "手写Qwen3-0.6B推理" §Qwen3RMSNorm (eps inside the square root);
    "古法手撕简易LLM推理器" §工具函数 (RMSNorm).  Used for the input and
    post-attention norms, the final norm and the per-head q/k norms."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) ("古法手撕简易LLM推理器" §工具函数)."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """theta^(-2i/d) for i = 0 .. d/2-1 ("手写Qwen3-0.6B推理" §Rope;
    "从零开始写Qwen3（二）" §rope/原理 gives the base angle beta^(-2i/d))."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-(2.0 * i) / head_dim)


def rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """NeoX ("rotate_half") rotary embedding.

    x has shape [..., T, H, D]; positions is broadcastable to [..., T].
    Dimension i < D/2 is paired with i + D/2 and the pair is rotated by the
    angle p * theta^(-2i/D):  x' = x*cos + rotate_half(x)*sin with
    rotate_half(x) = [-x2, x1] ("手写Qwen3-0.6B推理" §Rope;
    "古法手撕简易LLM推理器" §工具函数 and §RoPE的细节: Qwen3 uses the
    half-swap pairing, base theta from the config)."""
    d = x.shape[-1]
    half = d // 2
    p = np.asarray(positions, dtype=np.float64)
    ang = p[..., None] * rope_inv_freq(d, theta)          # [..., T, D/2]
    c = np.cos(ang)[..., None, :]                          # [..., T, 1, D/2]
    s = np.sin(ang)[..., None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_interleaved(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """Interleaved ("GPT-J style") rotary embedding: dimension 2i is paired
    with 2i+1 and the pair is rotated by p * theta^(-2i/D)
    ("从零开始写Qwen3（二）" §rope/原理 rotates consecutive dimension pairs by
    the pair's base angle; "古法手撕简易LLM推理器" §RoPE的细节 contrasts it
    with the half-swap form).  Shapes as in ``rope``."""
    d = x.shape[-1]
    p = np.asarray(positions, dtype=np.float64)
    ang = p[..., None] * rope_inv_freq(d, theta)          # [..., T, D/2]
    c = np.cos(ang)[..., None, :]
    s = np.sin(ang)[..., None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x, dtype=np.float64)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xo * c + xe * s
    return y


def apply_rope(x: np.ndarray, positions, cfg: "Cfg") -> np.ndarray:
    """The configuration's rotary form (half-swap for Qwen3)."""
    if cfg.rope_style == "interleaved":
        return rope_interleaved(x, positions, cfg.theta)
    return rope(x, positions, cfg.theta)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos, block: int = 1024) -> np.ndarray:
    """Causal grouped-query scaled-dot-product attention for one sequence.

    q: [Hq, Tq, D]; k, v: [Hkv, S, D] (cache rows 0..S-1); q_pos: [Tq]
    absolute positions.  Query head h reads KV head h // (Hq/Hkv) (the
    expand-then-flatten of "手写Qwen3-0.6B推理" §Attention, the
    repeat_interleave of "第 3 章" §3.3).  A query at position p sees keys
    0..p exactly (bottom-right aligned; "从零开始写Qwen3（二）" §Attn warns a
    one-token decode query must see every cached key).  Scores are scaled by
    1/sqrt(D) and normalised with a max-shifted softmax
    ("古法手撕简易LLM推理器" §工具函数).

    Query rows are processed in blocks only to bound memory, and a block
    reads keys only up to its largest position (every later key is masked
    for all of its rows).  The steps run as float64 torch CPU ops, which use
    every host core."""
    import torch
    hq, tq, d = q.shape
    hkv, s_len, _ = k.shape
    assert hq % hkv == 0, "Hq must be a multiple of Hkv"
    groups = hq // hkv
    q_pos = np.asarray(q_pos, dtype=np.int64).reshape(tq)
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))
    pos_t = torch.from_numpy(q_pos)
    out = torch.empty((hq, tq, d), dtype=torch.float64)
    scale = 1.0 / np.sqrt(d)
    for r0 in range(0, tq, block):
        r1 = min(tq, r0 + block)
        n_keys = min(s_len, int(q_pos[r0:r1].max()) + 1)
        visible = torch.arange(n_keys)[None, :] <= pos_t[r0:r1, None]       # [tb, n_keys]
        for h in range(hq):
            g = h // groups
            sc = (qt[h, r0:r1] @ kt[g, :n_keys].T) * scale                      # [tb, n_keys]
            sc = torch.where(visible, sc, -torch.inf)
            m = torch.max(sc, dim=-1, keepdim=True).values
            e = torch.where(visible, torch.exp(sc - m), 0.0)
            w = e / torch.sum(e, dim=-1, keepdim=True)
            out[h, r0:r1] = w @ vt[g, :n_keys]
    return out.numpy()


# ---------------------------------------------------------------- weights

class LayerW:
    """One decoder layer in float64, unmerged as in the state dict printed on
    "手写Qwen3-0.6B推理" §打印模型结构 (all projections stored [out, in],
    applied as y = x W^T, no bias)."""

    KEYS = ("input_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
            "post_norm", "wg", "wu", "wd")

    def __init__(self, bits: dict):
        for key in self.KEYS:
            setattr(self, key, widen_bf16(bits[key]))


class Model:
    """Widened model: embedding (tied lm_head), final norm, layers."""

    def __init__(self, bits: dict, cfg: Cfg = QWEN3):
        self.cfg = cfg
        self.embed = widen_bf16(bits["embed"])
        self.final_norm = widen_bf16(bits["final_norm"])
        self.layers = [LayerW(lw) for lw in bits["layers"]]


class KVCache:
    """Per-layer K (after q/k-norm and RoPE) and raw V, [B, Hkv, S_max, D]
    ("古法手撕简易LLM推理器" §核心计算函数与Transformer层: the cache keeps the
    projected, normalised, rotated K and the projected V)."""

    def __init__(self, cfg: Cfg, n_layers: int, batch: int, max_seq: int):
        shape = (batch, cfg.n_kv_heads, max_seq, cfg.head_dim)
        self.k = [np.zeros(shape) for _ in range(n_layers)]
        self.v = [np.zeros(shape) for _ in range(n_layers)]
        self.max_seq = max_seq


# ---------------------------------------------------------------- model steps

def embed(model: Model, ids) -> np.ndarray:
    """x = E[ids], no scaling ("手写Qwen3-0.6B推理" §Qwen3Model;
    "第 3 章" §3.1)."""
    return model.embed[np.asarray(ids, dtype=np.int64)]


def layer_forward(w: LayerW, x: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  start_pos, cfg: Cfg = QWEN3) -> np.ndarray:
    """One pre-norm decoder layer on x [B, T, C]; returns the new residual.

    h = x + Attn(RMSNorm_in(x)); out = h + MLP(RMSNorm_post(h))
    ("手写Qwen3-0.6B推理" §Qwen3DecoderLayer; "第 3 章" §3.2).
    Attention: q/k/v projections, per-head RMSNorm of q and k with a
    head_dim-long gain shared by all heads, RoPE on q and k at absolute
    positions start..start+T-1, K/V written into the cache at those rows,
    causal GQA over cache rows 0..p, head-major concat, o_proj
    ("手写Qwen3-0.6B推理" §Attention; "古法手撕简易LLM推理器"
    §核心计算函数与Transformer层).  MLP: down(silu(gate x) * up x)
    ("手写Qwen3-0.6B推理" §MLP).

    start_pos is an int or one int per sequence.  k_cache/v_cache are
    [B, Hkv, S_max, D] and are updated in place."""
    b_sz, t_len, _ = x.shape
    hq, hkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    starts = np.broadcast_to(np.asarray(start_pos, dtype=np.int64), (b_sz,))
    pos = starts[:, None] + np.arange(t_len)[None, :]             # [B, T]

    h = rmsnorm(x, w.input_norm, cfg.eps)
    q = (h @ w.wq.T).reshape(b_sz, t_len, hq, d)
    k = (h @ w.wk.T).reshape(b_sz, t_len, hkv, d)
    v = (h @ w.wv.T).reshape(b_sz, t_len, hkv, d)
    q = rmsnorm(q, w.q_norm, cfg.eps)
    k = rmsnorm(k, w.k_norm, cfg.eps)
    q = apply_rope(q, pos, cfg)
    k = apply_rope(k, pos, cfg)

    o = np.empty((b_sz, t_len, hq * d))
    for b in range(b_sz):
        p0 = int(starts[b])
        k_cache[b, :, p0:p0 + t_len] = k[b].transpose(1, 0, 2)
        v_cache[b, :, p0:p0 + t_len] = v[b].transpose(1, 0, 2)
        n_keys = p0 + t_len
        ob = attention(q[b].transpose(1, 0, 2), k_cache[b, :, :n_keys], v_cache[b, :, :n_keys], pos[b])
        o[b] = ob.transpose(1, 0, 2).reshape(t_len, hq * d)       # head h -> columns h*D..h*D+D-1

    x = x + o @ w.wo.T
    h2 = rmsnorm(x, w.post_norm, cfg.eps)
    return x + (silu(h2 @ w.wg.T) * (h2 @ w.wu.T)) @ w.wd.T


def final_logits(model: Model, x_last: np.ndarray) -> np.ndarray:
    """logits = RMSNorm_f(x) E^T with the lm_head tied to the embedding
    ("手写Qwen3-0.6B推理" §Qwen3Model; only each sequence's last row is
    projected, "第 3 章" §4.1)."""
    return rmsnorm(x_last, model.final_norm, model.cfg.eps) @ model.embed.T


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Greedy choice: index of the maximum, the lowest index among equal
    maxima ("手写Qwen3-0.6B推理" §推理; "第 3 章" §4.3).  np.argmax returns
    the first occurrence (and the first NaN if any)."""
    return np.argmax(np.atleast_2d(logits), axis=-1).astype(np.int64)


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float) -> int:
    """Temperature / top-k / top-p sampling of one logits row, the path
    "第 3 章" §4.3 (Sampler.sample) takes when temperatures are given; the
    pages name its steps but print no body, so this is their plain reading
    over the whole vocabulary:

    1. temperature <= 0 (or NaN) means greedy: argmax_lowest.
    2. z = logits / temperature.
    3. Candidates: every token whose z is at least the k-th largest z, ties
       included (k = top_k; top_k <= 0 or >= the vocabulary size means every
       token), in order of z descending, index ascending.
    4. Softmax over the candidates; keep the shortest prefix of that order
       whose probability mass reaches top_p (top_p outside (0, 1] means 1).
    5. The token at the first position of the kept prefix whose cumulative
       mass exceeds u times the kept mass, u in [0, 1) drawn by the caller.
    """
    x = np.asarray(logits, dtype=np.float64).reshape(-1)
    if not temperature > 0:
        return int(argmax_lowest(x)[0])
    z = x / temperature
    v = z.size
    k = v if (top_k <= 0 or top_k >= v) else top_k
    order = np.lexsort((np.arange(v), -z))           # z descending, index ascending
    tau = z[order[k - 1]]
    cand = order[z[order] >= tau]
    e = np.exp(z[cand] - z[cand[0]])
    cum = np.cumsum(e)
    p = 1.0 if not (0.0 < top_p <= 1.0) else top_p
    cut = int(np.argmax(cum >= p * cum[-1]))          # first prefix reaching the mass
    target = u * cum[cut]
    j = int(np.argmax(cum[:cut + 1] > target))
    return int(cand[j])


def prefill(model: Model, ids, max_seq: int | None = None, n_layers: int | None = None):
    """Prefill a batch of equal-length prompts ids [B, T] from position 0.

    Returns (logits of each sequence's last position [B, V], next ids [B],
    KV cache, final residual [B, T, C])
    ("古法手撕简易LLM推理器" §prefill与predict: prefill then lastOutputToken)."""
    ids = np.asarray(ids)
    b_sz, t_len = ids.shape
    nl = len(model.layers) if n_layers is None else n_layers
    cache = KVCache(model.cfg, nl, b_sz, max_seq or t_len)
    x = embed(model, ids)
    for li in range(nl):
        x = layer_forward(model.layers[li], x, cache.k[li], cache.v[li], 0, model.cfg)
    logits = final_logits(model, x[:, -1, :])
    return logits, argmax_lowest(logits), cache, x


def decode_step(model: Model, cache: KVCache, ids, positions):
    """One greedy step: each sequence b feeds token ids[b] at position
    positions[b] (its current length) and attends to cache rows 0..p
    ("古法手撕简易LLM推理器" §prefill与predict, predict loop).
    Returns (logits [B, V], next ids [B])."""
    ids = np.asarray(ids).reshape(-1)
    x = embed(model, ids[:, None])                                  # [B, 1, C]
    for li, w in enumerate(model.layers):
        x = layer_forward(w, x, cache.k[li], cache.v[li], np.asarray(positions), model.cfg)
    logits = final_logits(model, x[:, 0, :])
    return logits, argmax_lowest(logits)


def generate_nocache(model: Model, prompt, n_new: int, eos_id: int | None = None):
    """Greedy generation that recomputes the whole prefix each step, as the
    loops on "手写Qwen3-0.6B推理" §推理 and "第 3 章" §4.2 do.  0 new tokens
    means no model call; EOS, when met, is kept in the output."""
    tokens = [int(t) for t in np.asarray(prompt).reshape(-1)]
    out = []
    for _ in range(n_new):
        logits, nxt, _, _ = prefill(model, np.asarray([tokens]))
        tok = int(nxt[0])
        out.append(tok)
        tokens.append(tok)
        if eos_id is not None and tok == eos_id:
            break
    return out


def generate_cached(model: Model, prompt, n_new: int, forced=None):
    """Greedy generation with the KV cache: prefill, then one decode step per
    token.  With ``forced`` (a token list), the step inputs are taken from it
    instead of the oracle's own choices (teacher forcing).  Returns
    (tokens chosen by the oracle, per-step logits list)."""
    prompt = np.asarray(prompt).reshape(1, -1)
    t_len = prompt.shape[1]
    logits, nxt, cache, _ = prefill(model, prompt, max_seq=t_len + max(n_new, 1))
    chosen, all_logits = [int(nxt[0])], [logits[0]]
    inp = int(nxt[0]) if forced is None else int(forced[0])
    for i in range(1, n_new):
        lg, nx = decode_step(model, cache, [inp], [t_len + i - 1])
        chosen.append(int(nx[0]))
        all_logits.append(lg[0])
        inp = int(nx[0]) if forced is None else int(forced[i])
    return chosen[:n_new], all_logits[:n_new]
