"""Writes long_context_b4_ctx32768_seq0.npz: the float64 oracle's expected
logits for sequence 0 of the long-context decode workload (batch 4, 32768
prompt tokens per sequence, uniform random ids drawn as the benchmark draws
them, random-init 28-layer weights of seed 0), run the way the pages run
generation ("古法手撕简易LLM推理器" §prefill与predict): a 32768-token
prefill, then one token per step with the KV cache.

Stored: the prefill logits of the last position and the logits of the next
two greedy decode steps (each step feeds the oracle's own argmax), the three
greedy tokens, and the inputs' description.  Only oracle/ and the seeded
input generators are called; nothing here touches the GPU path.

A float64 prefill of 32768 tokens takes about an hour on 8 host cores and
about 25 GB of host memory:

    python tests/golden/make_long_context.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from decoder_only_transformer_qwen3_amd import inputs as I  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_b4_ctx32768_seq0.npz")
BATCH, T, STEPS, WEIGHT_SEED = 4, 32768, 2, 0
ID_SEED = 1000 + BATCH  # the benchmark's prompt draw for this batch size


def main():
    t0 = time.time()
    log = lambda m: print(f"[{time.time() - t0:7.0f} s] {m}", flush=True)
    bits = I.model_weights(WEIGHT_SEED)
    om = O.Model(bits)
    ids = I.token_ids(ID_SEED, (BATCH, T))[:1]
    log("weights and ids ready")
    cache = O.KVCache(om.cfg, len(om.layers), 1, T + STEPS)
    x = O.embed(om, ids)
    for li, w in enumerate(om.layers):
        x = O.layer_forward(w, x, cache.k[li], cache.v[li], 0, om.cfg)
        log(f"prefill layer {li + 1}/{len(om.layers)}")
    logits = [O.final_logits(om, x[:, -1, :])[0]]
    del x
    tokens = [int(O.argmax_lowest(logits[0][None])[0])]
    for i in range(STEPS):
        lg, nxt = O.decode_step(om, cache, [tokens[-1]], [T + i])
        logits.append(lg[0])
        tokens.append(int(nxt[0]))
        log(f"decode step {i + 1}: token {tokens[-1]}")
    meta = {"batch": BATCH, "prompt_len": T, "sequence": 0, "id_seed": ID_SEED, "weight_seed": WEIGHT_SEED,
            "steps": STEPS, "tokens": tokens,
            "note": "logits[0]: prefill, last position; logits[i]: decode step i at position T + i - 1, "
                    "fed tokens[i - 1]"}
    np.savez_compressed(OUT, logits=np.stack(logits).astype(np.float32), tokens=np.asarray(tokens, dtype=np.int64),
                        top_gap=np.asarray([float(np.sort(l)[-1] - np.sort(l)[-2]) for l in logits]),
                        meta=np.asarray(json.dumps(meta)))
    log(f"wrote {OUT}: tokens {tokens}")


if __name__ == "__main__":
    main()
