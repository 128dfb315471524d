"""Device-memory plumbing: upload bf16 weight bits, allocate the KV cache and
workspace with PyTorch, and fill the C structs the library takes.

Nothing here computes any step of the model; it only moves bytes and
builds pointer tables.  Weight dicts are the ones produced by
``inputs.model_weights`` (bf16 bit patterns keyed by the state-dict short
names); the merged projections follow the library's row order
([q; k; v] and [gate; up]).
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def rope_tables(device="cuda"):
    cos = np.empty((B.MAX_POS, 64), dtype=np.float32)
    sin = np.empty((B.MAX_POS, 64), dtype=np.float32)
    B.q3_rope_table_host(cos, sin)
    return torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device)


class DeviceLayer:
    def __init__(self, lw: dict, device="cuda"):
        self.input_norm = to_device_bf16(lw["input_norm"], device)
        self.w_qkv = to_device_bf16(np.concatenate([lw["wq"], lw["wk"], lw["wv"]], axis=0), device)
        self.q_norm = to_device_bf16(lw["q_norm"], device)
        self.k_norm = to_device_bf16(lw["k_norm"], device)
        self.w_o = to_device_bf16(lw["wo"], device)
        self.post_norm = to_device_bf16(lw["post_norm"], device)
        self.w_gate_up = to_device_bf16(np.concatenate([lw["wg"], lw["wu"]], axis=0), device)
        self.w_down = to_device_bf16(lw["wd"], device)

    def fill(self, s: B.q3_layer_weights) -> B.q3_layer_weights:
        for name, _ in B.q3_layer_weights._fields_:
            setattr(s, name, getattr(self, name).data_ptr())
        return s

    def struct(self) -> B.q3_layer_weights:
        return self.fill(B.q3_layer_weights())


class DeviceModel:
    def __init__(self, bits: dict, device="cuda"):
        assert len(bits["layers"]) == B.N_LAYERS
        self.embed = to_device_bf16(bits["embed"], device)
        self.final_norm = to_device_bf16(bits["final_norm"], device)
        self.layers = [DeviceLayer(lw, device) for lw in bits["layers"]]
        self.rope_cos, self.rope_sin = rope_tables(device)
        m = B.q3_model()
        m.embed = self.embed.data_ptr()
        m.final_norm = self.final_norm.data_ptr()
        for i, dl in enumerate(self.layers):
            dl.fill(m.layer[i])
        m.rope_cos = self.rope_cos.data_ptr()
        m.rope_sin = self.rope_sin.data_ptr()
        self.struct = m


class DeviceKV:
    def __init__(self, batch: int, max_seq: int, n_layers: int = B.N_LAYERS, device="cuda"):
        shape = (n_layers, batch, B.N_KV_HEADS, max_seq, B.HEAD_DIM)
        self.k = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        self.v = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        s = B.q3_kv()
        s.k, s.v, s.batch, s.max_seq = self.k.data_ptr(), self.v.data_ptr(), batch, max_seq
        self.struct = s
        self.batch, self.max_seq = batch, max_seq


def workspace(batch: int, n_tokens: int, device="cuda"):
    nbytes = B.q3_workspace_bytes(batch, n_tokens)
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes
