"""ctypes binding of libq3.so: the C-ABI functions under the same names.

Argument marshalling only.  Device buffers may be passed as torch tensors
(their data_ptr is used) or as integer addresses; the stream defaults to
torch's current stream.  A non-zero status raises Q3Error.  There is no
fallback: if the shared library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq3.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decoder_only_transformer_qwen3_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

HIDDEN, N_HEADS, N_KV_HEADS, HEAD_DIM = 1024, 16, 8, 128
INTER, VOCAB, N_LAYERS, MAX_POS = 3072, 151936, 28, 40960
QKV_ROWS, GATE_UP_ROWS = 4096, 6144

Q3_OK, Q3_ERR_NULL, Q3_ERR_SHAPE, Q3_ERR_POSITION = 0, -1, -2, -3
Q3_ERR_ALIGN, Q3_ERR_WORKSPACE, Q3_ERR_HIP, Q3_ERR_TOO_LARGE = -4, -5, -6, -7
NOALLOC_MAX_BYTES = 21 << 20

_vp = ctypes.c_void_p


class q3_layer_weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("input_norm", "w_qkv", "q_norm", "k_norm", "w_o",
                                   "post_norm", "w_gate_up", "w_down")]


class q3_model(ctypes.Structure):
    _fields_ = [("embed", _vp), ("final_norm", _vp), ("layer", q3_layer_weights * N_LAYERS),
                ("rope_cos", _vp), ("rope_sin", _vp)]


class q3_kv(ctypes.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("batch", ctypes.c_int32), ("max_seq", ctypes.c_int32)]


_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_status_str = _sig("q3_status_str", ctypes.c_char_p, ctypes.c_int)
_rope = _sig("q3_rope_table_host", ctypes.c_int, _vp, _vp)
_wsb = _sig("q3_workspace_bytes", _sz, _i32, _i32)
_layer = _sig("q3_layer_forward", ctypes.c_int, ctypes.POINTER(q3_layer_weights), _vp, _vp, _vp, _vp,
              _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp)
_prefill = _sig("q3_prefill", ctypes.c_int, ctypes.POINTER(q3_model), ctypes.POINTER(q3_kv), _i32, _i32,
                _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_decode = _sig("q3_decode_step", ctypes.c_int, ctypes.POINTER(q3_model), ctypes.POINTER(q3_kv), _i32, _vp,
               _vp, _i32, _vp, _vp, _vp, _sz, _vp)
_argmax = _sig("q3_argmax", ctypes.c_int, _vp, _i32, _i32, _i64, _vp, _vp)
_linear = _sig("q3_linear", ctypes.c_int, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp)
_attn_prefill = _sig("q3_attention_prefill", ctypes.c_int, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp)
_attn_prefill_qkv = _sig("q3_attention_prefill_qkv", ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                         _i32, _i32, _i32, _vp, _vp)
_attn_decode = _sig("q3_attention_decode", ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp,
                    _i32, _vp, _vp, _sz, _vp)
_attn_decode_warm = _sig("q3_attention_decode_warm", ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                         _vp, _i32, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp)
_rope_conv = _sig("q3_rope_interleaved_to_half", ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp)
_decode_eos = _sig("q3_decode_step_eos", ctypes.c_int, ctypes.POINTER(q3_model), ctypes.POINTER(q3_kv), _i32, _vp,
                     _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp)
_sample = _sig("q3_sample", ctypes.c_int, _vp, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_wsb_sample = _sig("q3_sample_workspace_bytes", _sz, _i32, _i32)
_wsb_packed = _sig("q3_workspace_bytes_packed", _sz, _i32, _i32)
_decode_noalloc = _sig("q3_decode_step_noalloc", ctypes.c_int, ctypes.POINTER(q3_model), ctypes.POINTER(q3_kv), _i32,
                       _vp, _vp, _i32, _i32, _vp, _vp, _vp)
_prefill_packed = _sig("q3_prefill_packed", ctypes.c_int, ctypes.POINTER(q3_model), ctypes.POINTER(q3_kv), _i32, _i32,
                       _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp)

Q3_EPI_STORE_BF16, Q3_EPI_STORE_F32, Q3_EPI_ADD_F32, Q3_EPI_SILU_GATE = 0, 1, 2, 3

EXPORTS = ("q3_status_str", "q3_rope_table_host", "q3_workspace_bytes", "q3_layer_forward",
           "q3_prefill", "q3_decode_step", "q3_argmax", "q3_linear", "q3_attention_prefill",
           "q3_attention_decode", "q3_attention_decode_warm", "q3_rope_interleaved_to_half", "q3_decode_step_eos",
           "q3_sample", "q3_sample_workspace_bytes", "q3_workspace_bytes_packed", "q3_prefill_packed",
           "q3_decode_step_noalloc", "q3_attention_prefill_qkv")


class Q3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({q3_status_str(status)})")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, ctypes.Array):
        return ctypes.addressof(x)
    raise TypeError(f"cannot take a pointer of {type(x)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st, where):
    if st != Q3_OK:
        raise Q3Error(st, where)


def q3_status_str(status: int) -> str:
    return _status_str(status).decode()


def q3_rope_table_host(cos_out, sin_out) -> None:
    """Fill host float32 [40960, 64] tables (numpy arrays or host tensors)."""
    def hp(a):
        if hasattr(a, "ctypes"):
            return a.ctypes.data
        return _ptr(a)
    _check(_rope(hp(cos_out), hp(sin_out)), "q3_rope_table_host")


def q3_workspace_bytes(batch: int, n_tokens: int) -> int:
    return int(_wsb(batch, n_tokens))


def q3_layer_forward(w: q3_layer_weights, rope_cos, rope_sin, k_layer, v_layer, batch, n_tokens, max_seq,
                     start_pos, residual, ws, ws_bytes, stream=None, check=True) -> int:
    st = _layer(ctypes.byref(w), _ptr(rope_cos), _ptr(rope_sin), _ptr(k_layer), _ptr(v_layer), batch, n_tokens,
                max_seq, start_pos, _ptr(residual), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "q3_layer_forward")
    return st


def q3_prefill(m: q3_model, kv: q3_kv, batch, prompt_len, ids, last_logits, next_ids, seq_lens, ws, ws_bytes,
               stream=None, check=True) -> int:
    st = _prefill(ctypes.byref(m), ctypes.byref(kv), batch, prompt_len, _ptr(ids), _ptr(last_logits),
                  _ptr(next_ids), _ptr(seq_lens), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "q3_prefill")
    return st


def q3_decode_step(m: q3_model, kv: q3_kv, batch, in_ids, seq_lens, max_len_hint, logits, out_ids, ws, ws_bytes,
                   stream=None, check=True) -> int:
    st = _decode(ctypes.byref(m), ctypes.byref(kv), batch, _ptr(in_ids), _ptr(seq_lens), max_len_hint,
                 _ptr(logits), _ptr(out_ids), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "q3_decode_step")
    return st


def q3_argmax(logits, rows, vocab, row_stride, out_idx, stream=None, check=True) -> int:
    st = _argmax(_ptr(logits), rows, vocab, row_stride, _ptr(out_idx), _stream(stream))
    if check:
        _check(st, "q3_argmax")
    return st


def q3_linear(x, w, out, m, n, k, ldo, epilogue, stream=None, check=True) -> int:
    st = _linear(_ptr(x), _ptr(w), _ptr(out), m, n, k, ldo, epilogue, _stream(stream))
    if check:
        _check(st, "q3_linear")
    return st


def q3_attention_prefill(q, k_layer, v_layer, batch, n_tokens, start_pos, max_seq, out, stream=None,
                         check=True) -> int:
    st = _attn_prefill(_ptr(q), _ptr(k_layer), _ptr(v_layer), batch, n_tokens, start_pos, max_seq, _ptr(out),
                       _stream(stream))
    if check:
        _check(st, "q3_attention_prefill")
    return st


def q3_attention_prefill_qkv(qkv, q_norm, k_norm, rope_cos, rope_sin, k_layer, v_layer, batch, n_tokens, start_pos,
                             max_seq, write_kv, out, stream=None, check=True) -> int:
    st = _attn_prefill_qkv(_ptr(qkv), _ptr(q_norm), _ptr(k_norm), _ptr(rope_cos), _ptr(rope_sin), _ptr(k_layer),
                           _ptr(v_layer), batch, n_tokens, start_pos, max_seq, int(write_kv), _ptr(out),
                           _stream(stream))
    if check:
        _check(st, "q3_attention_prefill_qkv")
    return st


def q3_attention_decode(qkv, q_norm, k_norm, rope_cos, rope_sin, k_layer, v_layer, batch, max_seq, positions,
                        max_len_hint, out, ws, ws_bytes, stream=None, check=True) -> int:
    st = _attn_decode(_ptr(qkv), _ptr(q_norm), _ptr(k_norm), _ptr(rope_cos), _ptr(rope_sin), _ptr(k_layer),
                      _ptr(v_layer), batch, max_seq, _ptr(positions), max_len_hint, _ptr(out), _ptr(ws), ws_bytes,
                      _stream(stream))
    if check:
        _check(st, "q3_attention_decode")
    return st


def q3_attention_decode_warm(qkv, q_norm, k_norm, rope_cos, rope_sin, k_layer, v_layer, batch, max_seq, positions,
                             max_len_hint, out, ws, ws_bytes, w_o, w_gate_up, w_down, w_qkv_next, stream=None,
                             check=True) -> int:
    st = _attn_decode_warm(_ptr(qkv), _ptr(q_norm), _ptr(k_norm), _ptr(rope_cos), _ptr(rope_sin), _ptr(k_layer),
                           _ptr(v_layer), batch, max_seq, _ptr(positions), max_len_hint, _ptr(out), _ptr(ws),
                           ws_bytes, _ptr(w_o), _ptr(w_gate_up), _ptr(w_down), _ptr(w_qkv_next), _stream(stream))
    if check:
        _check(st, "q3_attention_decode_warm")
    return st


def q3_rope_interleaved_to_half(w_qkv, q_norm, k_norm, w_qkv_out, q_norm_out, k_norm_out, stream=None,
                                check=True) -> int:
    st = _rope_conv(_ptr(w_qkv), _ptr(q_norm), _ptr(k_norm), _ptr(w_qkv_out), _ptr(q_norm_out), _ptr(k_norm_out),
                    _stream(stream))
    if check:
        _check(st, "q3_rope_interleaved_to_half")
    return st


def q3_decode_step_eos(m: q3_model, kv: q3_kv, batch, in_ids, seq_lens, max_len_hint, eos_id, logits, out_ids, ws,
                       ws_bytes, stream=None, check=True) -> int:
    st = _decode_eos(ctypes.byref(m), ctypes.byref(kv), batch, _ptr(in_ids), _ptr(seq_lens), max_len_hint, eos_id,
                     _ptr(logits), _ptr(out_ids), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "q3_decode_step_eos")
    return st


def q3_sample_workspace_bytes(rows: int, vocab: int) -> int:
    return int(_wsb_sample(rows, vocab))


def q3_sample(logits, rows, vocab, row_stride, temperature, top_k, top_p, uniform, out_idx, ws, ws_bytes,
              stream=None, check=True) -> int:
    st = _sample(_ptr(logits), rows, vocab, row_stride, _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(uniform),
                 _ptr(out_idx), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "q3_sample")
    return st


def q3_workspace_bytes_packed(n_seqs: int, n_tokens: int) -> int:
    return int(_wsb_packed(n_seqs, n_tokens))


def q3_prefill_packed(m: q3_model, kv: q3_kv, n_seqs, n_tokens, ids, cu_seqlens, start_pos, max_seq_tokens,
                      last_logits, next_ids, seq_lens, ws, ws_bytes, stream=None, check=True) -> int:
    st = _prefill_packed(ctypes.byref(m), ctypes.byref(kv), n_seqs, n_tokens, _ptr(ids), _ptr(cu_seqlens),
                         _ptr(start_pos), max_seq_tokens, _ptr(last_logits), _ptr(next_ids), _ptr(seq_lens),
                         _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check(st, "q3_prefill_packed")
    return st


def q3_decode_step_noalloc(m: q3_model, kv: q3_kv, batch, in_ids, seq_lens, max_len_hint, eos_id, logits, out_ids,
                           stream=None, check=True) -> int:
    st = _decode_noalloc(ctypes.byref(m), ctypes.byref(kv), batch, _ptr(in_ids), _ptr(seq_lens), max_len_hint, eos_id,
                         _ptr(logits), _ptr(out_ids), _stream(stream))
    if check:
        _check(st, "q3_decode_step_noalloc")
    return st
