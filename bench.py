"""Benchmark of the Qwen3-0.6B-shape forward on one MI355X.

Default workload (the headline): the prefill-bound configuration, the full
28-layer stack with random-init bf16 weights prefilling 8 prompts of 4096
uniform random ids, logits at each sequence's last position.  One "step" is
that whole prefill, captured once as a HIP graph and replayed; value =
prompt tokens / second.  The same run then measures the decode-bound
configuration (batch 32, 2048 cached positions, 128 greedy steps; its setup
prefill untimed) and reports it under "decode_b32_ctx2048".

Other workloads (--workload) measure the batch-1 prompt + greedy decode,
long-context decode (batch 4, 32768 cached positions) and packed ragged
prefill shapes.

Besides the headline value, the script times the dominant kernel alone with
HIP events on the stream it runs on (through the library's helper entry
points, same kernel, shape and launch configuration as inside the step) for
the roofline object, each prefill projection alone in its in-step
configuration (gemm_rooflines), reports the whole timed phase against the
roofline (step_roofline), and times the float64 CPU oracle on a bounded
sample of the same workload for the cpu_baseline object.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill & decode tokens/s (Qwen3-0.6B shape, bf16) + % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    # name: (batch, prompt_len, decode_steps, prefill_timed)
    "prefill128_decode64": (1, 128, 64, True),
    "decode_b32_ctx2048": (32, 2048, 128, False),
    "prefill_8x4096": (8, 4096, 0, True),
    "decode_b4_ctx32768": (4, 32768, 64, False),
    # packed ragged prefill: 16 prompts of seeded lengths in [256, 3840] (about 32K tokens)
    "prefill_packed_ragged": (16, 0, 0, True),
}


def ragged_lengths(n=16, lo=256, hi=3840, seed=77):
    return np.random.default_rng(seed).integers(lo, hi + 1, n).tolist()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill_8x4096", choices=sorted(WORKLOADS))
    ap.add_argument("--no-decode-extra", action="store_true",
                    help="with the default workload, skip the batch-32 decode measurement")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sample", default=None, metavar="T,K,P",
                    help="decode by temperature / top-k / top-p sampling (q3_sample on the step's logits)")
    ap.add_argument("--eos-id", type=int, default=None,
                    help="decode with q3_decode_step_eos (on-device done mask) and this end-of-sequence token")
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--kernel-only", nargs="?", const="dominant", default=None, choices=("dominant", "gemm"),
                    help="time only the workload's dominant kernel (or, with 'gemm', its four prefill "
                         "projections): the runs the counter passes profile")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="copy 1 GiB on the device three times (counter calibration) and exit")
    return ap.parse_args()


class Runner:
    """Holds device state for one workload and runs prefill / decode phases."""

    def __init__(self, torch, B, dev, dm, batch, prompt_len, steps, eos_id=None, sample=None):
        self.torch, self.B, self.dev, self.dm = torch, B, dev, dm
        self.eos_id = eos_id
        self.sample = None
        if sample is not None:  # per-row parameters and one seeded uniform draw per step and row
            t, k, p = sample
            g = torch.Generator(device="cuda").manual_seed(1234)
            self.sample = (torch.full((batch,), t, dtype=torch.float32, device="cuda"),
                           torch.full((batch,), k, dtype=torch.int32, device="cuda"),
                           torch.full((batch,), p, dtype=torch.float32, device="cuda"),
                           torch.rand((max(steps, 1), batch), generator=g, device="cuda"),
                           torch.empty((batch, B.VOCAB), dtype=torch.float32, device="cuda"),
                           torch.empty(B.q3_sample_workspace_bytes(batch, B.VOCAB), dtype=torch.uint8,
                                       device="cuda"))
        self.batch, self.T, self.steps = batch, prompt_len, steps
        from decoder_only_transformer_qwen3_amd import inputs as I
        self.lens = None
        if prompt_len == 0:  # packed ragged prompts
            self.lens = ragged_lengths(batch)
            self.ids_np = I.token_ids(1000 + batch, (1, sum(self.lens)))[0]
            self.cu = torch.tensor(np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32), device="cuda")
            prompt_len = max(self.lens)
            self.T = prompt_len
            nb = B.q3_workspace_bytes_packed(batch, int(sum(self.lens)))
            self.ws_p, self.nb_p = torch.empty(nb, dtype=torch.uint8, device="cuda"), nb
        else:
            self.ids_np = I.token_ids(1000 + batch, (batch, prompt_len))
            self.ws_p, self.nb_p = dev.workspace(batch, prompt_len)
        self.ids = torch.from_numpy(self.ids_np).cuda()
        self.max_seq = (prompt_len + max(steps, 1) + 7) // 8 * 8  # capacity: a multiple of 8
        self.kv = dev.DeviceKV(batch, self.max_seq)
        self.ws_d, self.nb_d = dev.workspace(batch, 1)
        self.nxt = torch.zeros(batch, dtype=torch.int32, device="cuda")
        self.seq = torch.zeros(batch, dtype=torch.int32, device="cuda")
        self.nxt0 = torch.zeros_like(self.nxt)
        self.seq0 = torch.zeros_like(self.seq)

    def prefill(self):
        B = self.B
        if self.lens is not None:
            B.q3_prefill_packed(self.dm.struct, self.kv.struct, self.batch, int(sum(self.lens)), self.ids, self.cu,
                                None, max(self.lens), None, self.nxt, self.seq, self.ws_p, self.nb_p)
            return
        B.q3_prefill(self.dm.struct, self.kv.struct, self.batch, self.T, self.ids, None, self.nxt, self.seq,
                     self.ws_p, self.nb_p)

    def save_state(self):
        self.nxt0.copy_(self.nxt)
        self.seq0.copy_(self.seq)

    def restore_state(self):
        self.nxt.copy_(self.nxt0)
        self.seq.copy_(self.seq0)

    def decode_loop(self):
        B = self.B
        for i in range(self.steps):
            if self.sample is not None:
                temps, ks, ps, us, logits, sws = self.sample
                B.q3_decode_step(self.dm.struct, self.kv.struct, self.batch, self.nxt, self.seq,
                                 self.T + self.steps, logits, self.nxt, self.ws_d, self.nb_d)
                B.q3_sample(logits, self.batch, B.VOCAB, B.VOCAB, temps, ks, ps, us[i], self.nxt, sws, sws.numel())
            elif self.eos_id is None:
                B.q3_decode_step(self.dm.struct, self.kv.struct, self.batch, self.nxt, self.seq,
                                 self.T + self.steps, None, self.nxt, self.ws_d, self.nb_d)
            else:
                B.q3_decode_step_eos(self.dm.struct, self.kv.struct, self.batch, self.nxt, self.seq,
                                     self.T + self.steps, self.eos_id, None, self.nxt, self.ws_d, self.nb_d)


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the allocator-free path once on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        fn()
    torch.cuda.synchronize()
    return g


# Matmul parameters of one layer (merged q|k|v, o, merged gate|up, down) and
# of the tied lm_head; the norm gains are negligible next to them.
LAYER_MATMUL_PARAMS = 4096 * 1024 + 1024 * 2048 + 6144 * 1024 + 1024 * 3072
LMHEAD_PARAMS = 151936 * 1024
KV_BYTES_PER_POS = 28 * 8 * 128 * 2 * 2  # K and V rows of one position, all layers and KV heads


def _time_launches(torch, fn, iters, reps=10, use_graph=True):
    """Average duration (s) of one fn() launch: `reps` back-to-back launches
    are captured as one HIP graph, which is replayed between HIP events on
    the current stream (the stream the kernels run on), so host launch
    overhead does not enter short kernels' figures.  Falls back to eager
    launches bracketed by events if capture is not possible."""
    stream = torch.cuda.current_stream()
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    n_rep = max(1, iters // reps)
    try:
        if not use_graph:
            raise RuntimeError("eager launches requested")
        g = capture(torch, lambda: [fn() for _ in range(reps)])
        per_replay = reps
        run = g.replay
    except Exception:
        per_replay, run = 1, fn
        n_rep = iters
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_rep)]
    for i in range(n_rep):
        ev[2 * i].record(stream)
        run()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_rep)])) * 1e-3 / per_replay


def dominant_kernel(torch, B, dev, dm, r, workload, iters, use_graph=True):
    """Roofline of the kernel that takes most of the workload's step time
    (per the rocprofv3 kernel summaries), timed alone with HIP events on the
    stream it runs on, at the workload's shape and launch configuration:

    - batch-1 prefill + decode: the decode attention launch, which at batch
      1 also reads the layer's gate|up and down weights and the next layer's
      q|k|v weight ahead into the L2s of the projections that follow (the
      largest share of the step), at the middle position of the decode;
    - decode-bound and long-context decode: the decode attention kernel at
      the middle position of the timed steps (KV streaming);
    - 8 x 4096 prefill: the causal flash-attention kernel.
    """
    batch, T, steps, _ = WORKLOADS[workload]
    extra = {}
    if workload == "prefill128_decode64":
        # one launch per layer's weights in turn (28 x 31.5 MB read ahead, more
        # than the 256 MB last-level cache), so they stream from HBM as in the step
        p = T + steps // 2
        qkv = torch.randn((batch, B.QKV_ROWS), device="cuda").to(torch.bfloat16)
        pos = torch.full((batch,), p, dtype=torch.int32, device="cuda")
        out = torch.empty((batch, B.N_HEADS * B.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
        kl, vl = r.kv.k[0], r.kv.v[0]
        lw0 = dm.layers[0]
        nl = len(dm.layers)
        cursor = [0]

        def fn():
            i = cursor[0] % nl
            cursor[0] += 1
            lw, nxt = dm.layers[i], dm.layers[(i + 1) % nl]
            B.q3_attention_decode_warm(qkv, lw0.q_norm, lw0.k_norm, dm.rope_cos, dm.rope_sin, kl, vl, batch,
                                       r.max_seq, pos, r.T + r.steps, out, r.ws_d, r.nb_d, lw.w_o, lw.w_gate_up,
                                       lw.w_down, nxt.w_qkv)
        warm_bytes = (B.HIDDEN * B.N_HEADS * B.HEAD_DIM + 2 * B.INTER * B.HIDDEN + B.HIDDEN * B.INTER
                      + B.QKV_ROWS * B.HIDDEN) * 2
        extra["read_ahead_bytes_per_launch"] = warm_bytes
        algo = float(batch * (p + 1) * 8 * 128 * 2 * 2 + batch * (B.QKV_ROWS + 2048) * 2)
        name, bound, per = (f"k_attn_decode + L2 read-ahead (batch {batch}, position {p}, one layer)", "hbm",
                            "the attention's own bytes: K and V of positions 0..p + q|k|v in + out (the "
                            "weights the same launch reads ahead for the projections after it are "
                            "read_ahead_bytes_per_launch, not counted here)")
        iters = max(iters, 280)
        reps = 28
    elif workload == "prefill_packed_ragged":
        # the largest GEMM over all packed rows (persistent MFMA kernel), as in the step
        M, N, K = int(sum(r.lens)), 2 * B.INTER, B.HIDDEN
        x = torch.randn((M, K), device="cuda").to(torch.bfloat16)
        out = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda")
        w = dm.layers[0].w_gate_up
        fn = lambda: B.q3_linear(x, w, out, M, N, K, N // 2, B.Q3_EPI_SILU_GATE)
        algo = float(2 * M * N * K)
        name, bound, per = f"k_gemm_persist<EPI_SILU> (gate|up, M={M} N={N} K={K})", "mfma", "2*M*N*K flops"
        reps = 10
    elif workload in ("decode_b32_ctx2048", "decode_b4_ctx32768"):
        reps = 10
        p = T + steps // 2  # middle of the timed decode steps
        qkv = torch.randn((batch, B.QKV_ROWS), device="cuda").to(torch.bfloat16)
        pos = torch.full((batch,), p, dtype=torch.int32, device="cuda")
        out = torch.empty((batch, B.N_HEADS * B.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
        lw = dm.layers[0]
        kl, vl = r.kv.k[0], r.kv.v[0]
        fn = lambda: B.q3_attention_decode(qkv, lw.q_norm, lw.k_norm, dm.rope_cos, dm.rope_sin, kl, vl, batch,
                                           r.max_seq, pos, r.T + r.steps, out, r.ws_d, r.nb_d)
        algo = float(batch * (p + 1) * 8 * 128 * 2 * 2 + batch * (B.QKV_ROWS + 2048) * 2)
        name, bound, per = f"k_attn_decode (batch {batch}, position {p}, one layer)", "hbm", \
            "K and V bytes of positions 0..p for every (sequence, KV head) + q|k|v in + out"
    else:
        # as the layer runs it: q from the raw projection rows, normed and rotated
        # as the kernel loads it, over layer 0's cache (its K/V rows written once
        # by the same entry point, then only the attention is timed)
        reps = 10
        qkv = torch.randn((batch, T, B.QKV_ROWS), device="cuda").to(torch.bfloat16)
        out = torch.empty((batch, T, B.N_HEADS * B.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
        kl, vl = r.kv.k[0], r.kv.v[0]
        lw = dm.layers[0]
        B.q3_attention_prefill_qkv(qkv, lw.q_norm, lw.k_norm, dm.rope_cos, dm.rope_sin, kl, vl, batch, T, 0,
                                   r.max_seq, 1, out)
        fn = lambda: B.q3_attention_prefill_qkv(qkv, lw.q_norm, lw.k_norm, dm.rope_cos, dm.rope_sin, kl, vl, batch,
                                                T, 0, r.max_seq, 0, out)
        algo = float(batch * (T * (T + 1) // 2) * 4 * B.HEAD_DIM * B.N_HEADS)
        name, bound, per = f"k_attn_prefill ({batch} x {T}, one layer)", "mfma", \
            "causal flops: 4 * 128 * 16 per (query, key <= query) pair"
    t = _time_launches(torch, fn, iters, reps, use_graph)
    if bound == "hbm":
        achieved, peak, unit = algo / t / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = algo / t / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
    traffic = measured_traffic(workload)
    out = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": round(traffic) if traffic else None, "kernel": name,
           "avg_launch_us": round(t * 1e6, 2), "algorithmic_per_launch": algo, "algorithmic_unit": per}
    if "read_ahead_bytes_per_launch" in extra:
        out.update(extra)
        out["achieved_with_read_ahead"] = round((algo + extra["read_ahead_bytes_per_launch"]) / t / 1e9, 1)
    return out


# The four projections of a layer as the prefill runs them (persistent MFMA
# GEMM at >= 2048 rows): name, N (weight rows), K, epilogue.
PREFILL_GEMMS = (("q|k|v", 4096, 1024, "Q3_EPI_STORE_BF16"), ("o_proj + residual", 1024, 2048, "Q3_EPI_ADD_F32"),
                 ("gate|up + silu(gate)*up", 6144, 1024, "Q3_EPI_SILU_GATE"),
                 ("down + residual", 1024, 3072, "Q3_EPI_ADD_F32"))


def gemm_rooflines(torch, B, dm, M, iters, use_graph=True):
    """Each prefill projection alone at M rows, in the launch configuration the
    layer uses (q3_linear runs the same kernel and epilogue as the step), timed
    with HIP events on its stream; fraction of the bf16 MFMA peak."""
    res = []
    lw = dm.layers[0]
    weights = {4096: lw.w_qkv, 6144: lw.w_gate_up}
    gen = torch.Generator(device="cuda").manual_seed(9)
    for name, N, K, epi in PREFILL_GEMMS:
        x = torch.randn((M, K), device="cuda", generator=gen).to(torch.bfloat16)
        w = weights.get(N, lw.w_o if K == 2048 else lw.w_down)
        e = getattr(B, epi)
        cols = N // 2 if e == B.Q3_EPI_SILU_GATE else N
        dt = torch.float32 if e == B.Q3_EPI_ADD_F32 else torch.bfloat16
        out = torch.zeros((M, cols), dtype=dt, device="cuda")
        fn = lambda x=x, w=w, out=out, N=N, K=K, e=e, cols=cols: B.q3_linear(x, w, out, M, N, K, cols, e)
        t = _time_launches(torch, fn, iters, 10, use_graph)
        tf = 2.0 * M * N * K / t / 1e12
        res.append({"gemm": name, "M": M, "N": N, "K": K, "avg_launch_us": round(t * 1e6, 2),
                    "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        del x, out
    return res


# Source files of each workload's dominant kernel.  The HBM traffic measured
# by the counter passes (profiles/traffic.json) belongs to one version of the
# kernel: it is reported only while these files hash to the recorded digest.
KERNEL_SOURCES = {
    "prefill128_decode64": ["attn_decode.hip", "common.hpp"],
    "decode_b32_ctx2048": ["attn_decode.hip", "common.hpp"],
    "decode_b4_ctx32768": ["attn_decode.hip", "common.hpp"],
    "prefill_8x4096": ["attn_prefill.hip", "common.hpp"],
    "prefill_packed_ragged": ["gemm_tiled.hip", "common.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_digest(workload):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[workload]:
        with open(os.path.join(ROOT, "decoder_only_transformer_qwen3_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel (calibrated FETCH_SIZE +
    WRITE_SIZE counters), or None when no counters were taken for the
    current version of its source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_digest(workload):
        return None
    return float(rec["fetch_bytes_per_launch"]) + float(rec["write_bytes_per_launch"])


def step_roofline(workload, pre_ms, dec_ms):
    """Whole-phase figure for context: algorithmic bytes (decode) or flops
    (prefill-bound workload) of the timed phase over its measured time."""
    batch, T, steps, prefill_timed = WORKLOADS[workload]
    if workload in ("prefill_8x4096", "prefill_packed_ragged"):
        lens = [T] * batch if workload == "prefill_8x4096" else ragged_lengths(batch)
        flops = sum(lens) * 2 * LAYER_MATMUL_PARAMS * 28 + sum(t * (t + 1) // 2 for t in lens) * 8192 * 28 \
            + batch * 2 * LMHEAD_PARAMS
        a = flops / (pre_ms * 1e-3) / 1e12
        return {"phase": "prefill", "bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / BF16_PEAK_TFLOPS, 4)}
    weights = 2 * (28 * LAYER_MATMUL_PARAMS + LMHEAD_PARAMS)
    mean_ctx = T + (steps + 1) / 2.0
    per_step = weights + batch * mean_ctx * KV_BYTES_PER_POS
    a = per_step * steps / (dec_ms * 1e-3) / 1e9
    return {"phase": "decode", "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "bytes_per_step": round(per_step)}


def cpu_baseline(workload, bits, om=None):
    """The float64 oracle on a bounded sample of the workload (host cores):
    - batch-1 prompt + decode: the whole workload (one sequence), repeated to
      about 10 s;
    - 8 x 4096 prefill: sequence 0's full 4096-token prefill;
    - packed prefill: the first packed sequence's full prefill;
    - decode workloads: sequence 0, a few greedy decode steps at the
      workload's full context.  The float64 cache of those positions is
      filled with seeded N(0, 1) values instead of an oracle prefill of the
      prompt (hours of float64 work at 32768 positions); the timed steps are
      the oracle's own decode arithmetic over that many cached positions."""
    import oracle as O
    from decoder_only_transformer_qwen3_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        ncores = len(os.sched_getaffinity(0))
        threadpool_limits(limits=ncores)
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    batch, T, steps, _ = WORKLOADS[workload]
    t0 = time.perf_counter()
    if om is None:
        om = O.Model(bits)
    setup = time.perf_counter() - t0
    if workload == "prefill128_decode64":
        ids = I.token_ids(1000 + batch, (batch, T))[:1]
        n_dec = steps  # the whole workload: prefill + every decode step, repeated to about 10 s
        reps, el = 0, 0.0
        while reps < 8 and (reps == 0 or el < 10.0):
            t0 = time.perf_counter()
            _, nxt, cache, _ = O.prefill(om, ids, max_seq=T + n_dec)
            tok = int(nxt[0])
            for i in range(n_dec):
                _, nx = O.decode_step(om, cache, [tok], [T + i])
                tok = int(nx[0])
            el += time.perf_counter() - t0
            reps += 1
        sample = (f"sequence 0: {T}-token prefill + {n_dec} greedy decode steps ({T + n_dec} tokens), "
                  f"the whole workload, run {reps} times")
        toks = (T + n_dec) * reps
    elif workload == "prefill_8x4096":
        ids = I.token_ids(1000 + batch, (batch, T))[:1]
        t0 = time.perf_counter()
        O.prefill(om, ids)
        el = time.perf_counter() - t0
        sample = f"sequence 0: its full {T}-token prefill with last-position logits"
        toks = T
    elif workload == "prefill_packed_ragged":
        n0 = ragged_lengths(batch)[0]
        ids = I.token_ids(1000 + batch, (1, sum(ragged_lengths(batch))))[:, :n0]
        t0 = time.perf_counter()
        O.prefill(om, ids)
        el = time.perf_counter() - t0
        sample = f"packed sequence 0: its full {n0}-token prefill"
        toks = n0
    else:
        n_dec = 4
        rng = np.random.default_rng(77)
        cache = O.KVCache(om.cfg, len(om.layers), 1, T + n_dec)
        for li in range(len(om.layers)):
            cache.k[li][:, :, :T] = rng.standard_normal((1, 8, T, 128))
            cache.v[li][:, :, :T] = rng.standard_normal((1, 8, T, 128))
        tok = int(I.token_ids(1000 + batch, (batch, 1))[0, 0])
        t0 = time.perf_counter()
        for i in range(n_dec):
            _, nx = O.decode_step(om, cache, [tok], [T + i])
            tok = int(nx[0])
        el = time.perf_counter() - t0
        sample = (f"sequence 0: {n_dec} greedy decode steps at positions {T}..{T + n_dec - 1} over a float64 "
                  f"cache of {T} positions (seeded N(0,1) cache content, not an oracle prefill)")
        toks = n_dec
    return {"value": round(toks / el, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "seconds": round(el, 2), "weights_setup_s": round(setup, 2)}


def run_workload(args, workload, torch, B, dev, dm):
    """Time one workload's step; returns its fields of the bench line."""
    batch, T, steps, prefill_timed = WORKLOADS[workload]
    log(f"[bench] workload {workload}: batch {batch}, prompt {T}, decode steps {steps}")
    sample = None
    if args.sample:
        t, k, p = args.sample.split(",")
        sample = (float(t), int(k), float(p))
    r = Runner(torch, B, dev, dm, batch, T, steps, args.eos_id, sample)
    use_graph = not args.no_graph
    # setup prefill (untimed); decode-only workloads restart from this state each step
    r.prefill()
    torch.cuda.synchronize()
    r.save_state()

    if prefill_timed:
        phase_a, phase_b = r.prefill, (r.decode_loop if steps > 0 else None)
    else:
        phase_a, phase_b = None, (lambda: (r.restore_state(), r.decode_loop()))
    g_a = g_b = None
    if use_graph:
        try:
            if phase_a is not None:
                g_a = capture(torch, phase_a)
            if phase_b is not None:
                r.prefill()  # capture's warm-up run of the decode loop starts from a fresh prefill state
                torch.cuda.synchronize()
                g_b = capture(torch, phase_b)
        except Exception as e:  # pragma: no cover
            log(f"[bench] graph capture failed ({e}); running eagerly")
            g_a = g_b = None
            use_graph = False

    stream = torch.cuda.current_stream()

    def one_step(ev=None):
        if ev:
            ev[0].record(stream)
        if phase_a is not None:
            g_a.replay() if g_a is not None else phase_a()
        if ev:
            ev[1].record(stream)
        if phase_b is not None:
            g_b.replay() if g_b is not None else phase_b()
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    step_ms = wall * 1e3 / args.steps
    log(f"[bench] {workload}: {step_ms:.3f} ms per step")

    tokens_prefill = (sum(r.lens) if r.lens is not None else batch * T) if prefill_timed else 0
    tokens_decode = batch * steps
    value = (tokens_prefill + tokens_decode) / (step_ms * 1e-3)
    res = {
        "value": round(value, 2), "ms_per_step": round(step_ms, 4),
        "config": {"workload": workload, "layers": 28, "batch": batch, "prompt_len": T,
                   "decode_steps": steps, "prefill_timed": prefill_timed, "hip_graph": use_graph,
                   "parallelism": "single GPU", **({"eos_id": args.eos_id} if args.eos_id is not None else {}),
                   **({"sampling": args.sample} if args.sample else {}),
                   **({"packed_lengths": r.lens, "packed_tokens": sum(r.lens)} if r.lens is not None else {})},
        "prefill_ms": round(pre_ms, 4), "decode_ms": round(dec_ms, 4),
        "prefill_tok_s": round(tokens_prefill / (pre_ms * 1e-3), 1) if prefill_timed else None,
        "decode_tok_s": round(tokens_decode / (dec_ms * 1e-3), 1) if steps > 0 else None,
    }
    try:
        res["roofline"] = dominant_kernel(torch, B, dev, dm, r, workload, args.kernel_iters, use_graph)
    except Exception as e:  # pragma: no cover
        log(f"[bench] kernel timing failed: {e}")
        res["roofline"] = None
    res["step_roofline"] = step_roofline(workload, pre_ms, dec_ms)
    if workload in ("prefill_8x4096", "prefill_packed_ragged"):
        M = int(sum(r.lens)) if r.lens is not None else batch * T
        del r
        torch.cuda.empty_cache()
        res["gemm_rooflines"] = gemm_rooflines(torch, B, dm, M, max(args.kernel_iters // 4, 20), use_graph)
    else:
        del r
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the hot path runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    from decoder_only_transformer_qwen3_amd import binding as B
    from decoder_only_transformer_qwen3_amd import device as dev
    from decoder_only_transformer_qwen3_amd import inputs as I

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        x = torch.empty(1 << 28, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": 4 << 28, "bytes_written": 4 << 28,
                          "launches": 3}), flush=True)
        return
    bits = I.model_weights(0)
    dm = dev.DeviceModel(bits)
    if args.kernel_only:
        batch, T, steps, _ = WORKLOADS[args.workload]
        sample = None
        r = Runner(torch, B, dev, dm, batch, T, steps, args.eos_id, sample)
        # no prefill ran: give the layer-0 cache the attention kernels read
        # N(0, 1) values, as a prefill would leave there (all-zero keys would
        # time a different, lower-power instruction stream)
        gen = torch.Generator(device="cuda").manual_seed(5)
        for c in (r.kv.k[0], r.kv.v[0]):
            c.copy_(torch.randn(c.shape, device="cuda", generator=gen).to(torch.bfloat16))
        if args.kernel_only == "gemm":
            M = batch * T if T else int(sum(r.lens))
            del r
            rl = gemm_rooflines(torch, B, dm, M, args.kernel_iters, not args.no_graph)
            print(json.dumps({"workload": args.workload, "gemm_rooflines": rl}), flush=True)
            return
        rl = dominant_kernel(torch, B, dev, dm, r, args.workload, args.kernel_iters, not args.no_graph)
        rl["source_sha256"] = kernel_source_digest(args.workload)
        print(json.dumps({"workload": args.workload, "roofline": rl}), flush=True)
        return

    res = run_workload(args, args.workload, torch, B, dev, dm)
    out = {
        "metric": METRIC, "value": res["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,0.02), uniform random token ids)",
    }
    out.update({k: v for k, v in res.items() if k not in ("value", "ms_per_step")})
    extra = None
    if args.workload == "prefill_8x4096" and not args.no_decode_extra and args.sample is None \
            and args.eos_id is None:
        extra = run_workload(args, "decode_b32_ctx2048", torch, B, dev, dm)
        out["decode_b32_ctx2048"] = {k: extra[k] for k in ("value", "ms_per_step", "decode_ms", "decode_tok_s",
                                                          "roofline", "step_roofline", "config")}
    if not args.no_cpu_baseline:
        import oracle as O
        log("[bench] timing the float64 oracle on the host")
        om = O.Model(bits)
        out["cpu_baseline"] = cpu_baseline(args.workload, bits, om)
        if extra is not None:
            out["decode_b32_ctx2048"]["cpu_baseline"] = cpu_baseline("decode_b32_ctx2048", bits, om)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
