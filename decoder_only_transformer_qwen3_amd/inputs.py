"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws numbers and encodes them; it holds none of the
model's arithmetic.  Every tensor is drawn from its own NumPy PCG64 stream
keyed by ``(seed, crc32(name))`` so that any single tensor can be
regenerated without drawing the others.

Encoding: floating-point tensors are produced as bfloat16 bit patterns
(``uint16``), rounded from float32 with round-to-nearest-even.  Both sides
consume the same bits: the oracle widens them exactly to float64, the HIP
path uploads them as-is.

Weight names and shapes follow the state-dict listing printed on the page
"手写Qwen3-0.6B推理" (section 打印模型结构); the random-init law (weights
N(0, 0.02), norm gains 1 + N(0, 0.02)) uses the ``initializer_range = 0.02``
value from the configuration printed on "Pytorch手写大模型推理" (section 模型)
as a standard deviation.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Dims:
    """Model dimensions (Qwen3-0.6B values by default)."""

    hidden: int = 1024
    n_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    inter: int = 3072
    vocab: int = 151936
    n_layers: int = 28


QWEN3_0P6B = Dims()
# The worked shape example on "第 3 章 前向与生成（代码走读）" (section 5,
# 用形状与因果性检查理解): B=1, T=3, C=32, Hq=4, Hkv=2, D=8, V=64.
TINY = Dims(hidden=32, n_heads=4, n_kv_heads=2, head_dim=8, inter=48, vocab=64, n_layers=2)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stream(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), zlib.crc32(name.encode())])


def normal_bf16(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    g = stream(seed, name)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return f32_to_bf16_bits(x)


def layer_names(i: int) -> dict:
    p = f"model.layers.{i}."
    return {
        "input_norm": p + "input_layernorm.weight",
        "wq": p + "self_attn.q_proj.weight",
        "wk": p + "self_attn.k_proj.weight",
        "wv": p + "self_attn.v_proj.weight",
        "q_norm": p + "self_attn.q_norm.weight",
        "k_norm": p + "self_attn.k_norm.weight",
        "wo": p + "self_attn.o_proj.weight",
        "post_norm": p + "post_attention_layernorm.weight",
        "wg": p + "mlp.gate_proj.weight",
        "wu": p + "mlp.up_proj.weight",
        "wd": p + "mlp.down_proj.weight",
    }


def layer_shapes(d: Dims) -> dict:
    return {
        "input_norm": (d.hidden,),
        "wq": (d.n_heads * d.head_dim, d.hidden),
        "wk": (d.n_kv_heads * d.head_dim, d.hidden),
        "wv": (d.n_kv_heads * d.head_dim, d.hidden),
        "q_norm": (d.head_dim,),
        "k_norm": (d.head_dim,),
        "wo": (d.hidden, d.n_heads * d.head_dim),
        "post_norm": (d.hidden,),
        "wg": (d.inter, d.hidden),
        "wu": (d.inter, d.hidden),
        "wd": (d.hidden, d.inter),
    }


GAINS = ("input_norm", "q_norm", "k_norm", "post_norm")


def layer_weights(seed: int, i: int, d: Dims = QWEN3_0P6B, std: float = 0.02) -> dict:
    """One decoder layer's weights as bf16 bits, keyed by short names."""
    names, shapes = layer_names(i), layer_shapes(d)
    out = {}
    for k, nm in names.items():
        if k in GAINS:
            out[k] = normal_bf16(seed, nm, shapes[k], std=std, mean=1.0)
        else:
            out[k] = normal_bf16(seed, nm, shapes[k], std=std)
    return out


def model_weights(seed: int = 0, d: Dims = QWEN3_0P6B, n_layers: int | None = None,
                  std: float = 0.02, threads: int = 8) -> dict:
    """Full model: {'embed', 'final_norm', 'layers': [layer dicts]} as bf16 bits.

    The lm_head is tied to ``embed`` (no separate tensor).  Tensors are drawn
    in parallel threads; each has its own stream, so the result does not
    depend on the thread count.
    """
    from concurrent.futures import ThreadPoolExecutor
    n = d.n_layers if n_layers is None else n_layers
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        emb = ex.submit(normal_bf16, seed, "model.embed_tokens.weight", (d.vocab, d.hidden), std)
        layers = list(ex.map(lambda i: layer_weights(seed, i, d, std), range(n)))
        return {
            "embed": emb.result(),
            "final_norm": normal_bf16(seed, "model.norm.weight", (d.hidden,), std=std, mean=1.0),
            "layers": layers,
        }


def token_ids(seed: int, shape, vocab: int = QWEN3_0P6B.vocab) -> np.ndarray:
    """Uniform token ids in [0, vocab) (stand-in for tokenized prompts)."""
    return stream(seed, "token_ids").integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32)


def hidden_states(seed: int, shape) -> np.ndarray:
    """N(0, 1) hidden states as bf16 bits (one-layer workload)."""
    return normal_bf16(seed, "hidden_states", shape, std=1.0)
