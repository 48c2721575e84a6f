"""Runs the fp64 oracle on one slice of heads saved as .npy files (test
infrastructure, started as a child process by oracle_pool.py).

    python tests/oracle_worker.py <dir>

<dir>/meta.json names the entry point ("prefill" or "prefill_gated").  The
inputs are q, k, v [T, h, d], decay [T, h, d_k] (log alpha, or the decay
logits of the gated map), beta [T, h] (beta, or its logits), and optionally
init_state [N, h, d_k, d_v], cu_seqlens [N + 1] and a_log [h] (gated).  A file
named <name>.bf16.npy holds the raw 16-bit words of a bf16 tensor and is
widened exactly to fp32 here.  When o_gpu and fin_gpu are present the worker
compares them with the oracle.  It writes stats.json: the oracle's wall time,
the token-heads it ran, and max |gpu - ref| and max |ref| for o and the final
state; with "keep_o_ref" in meta.json it also writes the oracle's o as
o_ref.npy.

Kind "decode": the worker's slice of (sequence, head) pairs over a run of
decode steps.  state0 [n, H, d_k, d_v] is the state before the first step;
step s has its own files <name>_<s> for q, k, v, decay (log alpha), beta and
o_gpu ([n, H, .]); fin_gpu is the state after the last step.  stats.json
then holds, per step, max |gpu - ref| and max |ref| of o, and the same for
the final state.
"""
import json
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402


def load(d: str, name: str):
    p = os.path.join(d, name + ".npy")
    if os.path.exists(p):
        return np.load(p)
    p = os.path.join(d, name + ".bf16.npy")
    if os.path.exists(p):
        return (np.load(p).astype(np.uint32) << 16).view(np.float32)
    return None


def decode(d: str, meta: dict):
    S = load(d, "state0").astype(np.float64)
    o_err, o_ref_max, o_finite = [], [], True
    t0 = time.perf_counter()
    for s in range(meta["steps"]):
        x = {n: load(d, f"{n}_{s}") for n in ("q", "k", "v", "decay", "beta", "o_gpu")}
        o, S = oracle.kda_decode_step(x["q"], x["k"], x["v"], x["decay"], x["beta"], S)
        o_err.append(float(np.abs(x["o_gpu"].astype(np.float64) - o).max()))
        o_ref_max.append(float(np.abs(o).max()))
        o_finite = o_finite and bool(np.isfinite(x["o_gpu"]).all())
    seconds = time.perf_counter() - t0
    f_gpu = load(d, "fin_gpu")
    return {"seconds": seconds, "pair_steps": int(S.shape[0] * S.shape[1] * meta["steps"]),
            "o_err_max": o_err, "o_ref_max": o_ref_max,
            "f_err_max": float(np.abs(f_gpu.astype(np.float64) - S).max()), "f_ref_max": float(np.abs(S).max()),
            "o_finite": o_finite, "f_finite": bool(np.isfinite(f_gpu).all())}


def main(d: str):
    with open(os.path.join(d, "meta.json")) as f:
        meta = json.load(f)
    if meta["kind"] == "decode":
        with open(os.path.join(d, "stats.json"), "w") as f:
            json.dump(decode(d, meta), f)
        return
    q, k, v, decay, beta = (load(d, n) for n in ("q", "k", "v", "decay", "beta"))
    init, cu, a_log = load(d, "init_state"), load(d, "cu_seqlens"), load(d, "a_log")
    t0 = time.perf_counter()
    if meta["kind"] == "prefill_gated":
        o, fin = oracle.kda_prefill_gated(q, k, v, decay, a_log, beta, init, cu)
    else:
        o, fin = oracle.kda_prefill(q, k, v, decay, beta, init, cu)
    stats = {"seconds": time.perf_counter() - t0, "token_heads": int(q.shape[0] * q.shape[1]),
             "o_ref_max": float(np.abs(o).max()) if o.size else 0.0,
             "f_ref_max": float(np.abs(fin).max()) if fin.size else 0.0}
    o_gpu, f_gpu = load(d, "o_gpu"), load(d, "fin_gpu")
    if o_gpu is not None:
        stats["o_err_max"] = float(np.abs(o_gpu.astype(np.float64) - o).max()) if o.size else 0.0
        stats["o_finite"] = bool(np.isfinite(o_gpu).all())
    if f_gpu is not None:
        stats["f_err_max"] = float(np.abs(f_gpu.astype(np.float64) - fin).max()) if fin.size else 0.0
        stats["f_finite"] = bool(np.isfinite(f_gpu).all())
    if meta.get("keep_o_ref"):
        np.save(os.path.join(d, "o_ref.npy"), o)
    with open(os.path.join(d, "stats.json"), "w") as f:
        json.dump(stats, f)


if __name__ == "__main__":
    main(sys.argv[1])
