#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one chunkwise prefill of the long-context workload (one sequence,
T = 65,536 tokens, H = 96 heads, d_k = d_v = 128, bf16 q/k/v, fp32 log-decay
and beta, fp32 state) followed by one decode step of the batched-decode
workload (512 sequences x 96 heads, fp32 state of 3.2 GB updated in place).
Inputs are synthetic, seeded, and resident in device memory before timing.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-gated]
                    [--no-epilogue] [--no-split] [--no-varlen] [--capacity] [--cpu-baselines]

Prints one JSON line.  `value` is prefill tokens/s; decode state-update
bandwidth is reported under "decode".  Timed after the headline step:
- "gated": the gated entry points;
- "epilogue": the output epilogue (standalone, after the gated prefill, fused
  into the gated decode);
- "prologue": the input prologue (standalone, the whole prefill layer core,
  the one-kernel decode step);
- "split": the time-split prefill against the plain one at one GPU's share of
  the heads (H = 12);
- "varlen": the packed workload of 16 sequences of 1K to 8K tokens.
Kernel durations come from HIP events recorded on the stream the kernels are
launched on.  "wait_giveups" counts bounded in-kernel waits that ran out
(0 when every wait ended normally).  --cpu-baselines adds the fp64 oracle
timed beside every workload on the host cores.  `python bench.py --record-counters DIR` builds the HBM traffic
record from rocprofv3 counter runs instead (no GPU).
"""

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published

T_PREFILL, H, D = 65536, 96, 128
N_DECODE = 512
# Algorithmic bytes (bf16 q/k/v, fp32 log-decay, fp32 beta, bf16 o).
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * D * 2 + D * 4 + 4 + D * 2          # 1540
STATE_BYTES = D * D * 4                                                  # 64 KiB
DECODE_BYTES_PER_PAIR = 2 * STATE_BYTES + 3 * D * 2 + D * 4 + 4 + D * 2  # 132,612
# Gated entry points: bf16 decay logits replace fp32 log-decay, fp32 beta logits replace beta.
GATED_PREFILL_BYTES_PER_TOKEN_HEAD = 3 * D * 2 + D * 2 + 4 + D * 2        # 1284
GATED_DECODE_BYTES_PER_PAIR = 2 * STATE_BYTES + 3 * D * 2 + D * 2 + 4 + D * 2
# Output epilogue: read o and the gate logits, write y (bf16); the gain is d_v fp32 per launch.
EPILOGUE_BYTES_PER_TOKEN_HEAD = 3 * D * 2                                # 768
# Gated decode with the epilogue fused: the gate logits are read, y replaces o.
EPILOGUE_DECODE_BYTES_PER_PAIR = GATED_DECODE_BYTES_PER_PAIR + D * 2
# Input prologue: read x_q, x_k, x_v and write q, k, v (bf16).
PROLOGUE_BYTES_PER_TOKEN_HEAD = 2 * 3 * D * 2                            # 1536
CONV_C = 3 * D                                                           # packed channels per head
# Whole fused decode step: the gated decode with the epilogue, plus the convolution state
# (3 entries per channel read, 3 written).
FUSED_DECODE_BYTES_PER_PAIR = EPILOGUE_DECODE_BYTES_PER_PAIR + 2 * 3 * CONV_C * 2
# Algorithmic flops per token-head, chunk 64, causal triangles only.
PREFILL_FLOPS_PER_TOKEN_HEAD = 6 * D * D + 2 * 64 * (D + D)              # 131,072


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(budget_s: float = 12.0, max_workers: int = 16):
    """Time the fp64 oracle (as it stands) on a bounded sample of the prefill
    workload.  Up to `max_workers` single-threaded processes (one per available
    core) each run 8 heads of the 64K-token sequence, consecutive 1024-token
    segments with the state carried, until the time budget is spent; the heads
    are independent, so the processes share nothing.  `cores` is the number of
    processes."""
    code = r"""
import json, sys, time
sys.path.insert(0, %r)
import numpy as np
import kda_inputs as ki
import oracle
w = int(sys.argv[1])
x = ki.prefill_inputs([65536], H=8, d=%d, dtype="bf16", la_law="uniform53", init="normal", seed=3 + w)
n = ki.to_numpy
q, k, v, la, b, S = (n(x.q), n(x.k), n(x.v), n(x.log_alpha), n(x.beta), n(x.init_state)[0].astype(np.float64))
print("ready", flush=True)
sys.stdin.readline()
done, t0 = 0, time.perf_counter()
while done < q.shape[0]:
    sl = slice(done, done + 1024)
    _, S = oracle.kda_recurrence(q[sl], k[sl], v[sl], la[sl], b[sl], S)
    done += 1024
    if time.perf_counter() - t0 > %f:
        break
dt = time.perf_counter() - t0
print(json.dumps({"token_heads": done * 8, "seconds": dt}), flush=True)
""" % (ROOT, D, budget_s)
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    procs = [subprocess.Popen([sys.executable, "-c", code, str(w)], stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                              stderr=subprocess.PIPE, text=True, env=env) for w in range(workers)]
    try:
        # Every process draws its inputs first; the timed loops then start together.
        for p in procs:
            if p.stdout.readline().strip() != "ready":
                raise RuntimeError(p.stderr.read()[-2000:])
        t0 = time.perf_counter()
        for p in procs:
            p.stdin.write("go\n")
            p.stdin.flush()
        res = [json.loads(p.communicate(timeout=600)[0].strip().splitlines()[-1]) for p in procs]
        wall = time.perf_counter() - t0
    finally:
        for p in procs:
            if p.poll() is None:
                p.kill()
    token_heads = sum(r["token_heads"] for r in res)
    th_per_s = token_heads / wall
    return {"value": th_per_s / H, "unit": "tokens/s (H=96 equivalent)", "cores": workers, "kind": "oracle",
            "sample": f"fp64 oracle, {workers} single-threaded process{'es' if workers > 1 else ''} x 8 heads x "
                      f"{min(r['token_heads'] for r in res) // 8}-{max(r['token_heads'] for r in res) // 8} tokens "
                      f"of the 64K prefill workload ({wall:.1f} s wall, {th_per_s:.0f} token-heads/s) on "
                      f"{_cpu_model()}"}


DECODE_WORKER = r"""
import json, sys, time
sys.path.insert(0, %r)
import numpy as np
import kda_inputs as ki
import oracle
w, n_seq, steps = int(sys.argv[1]), int(sys.argv[2]), int(sys.argv[3])
S = ki.decode_state(n_seq, 96, 128, seed=4 + 1000 * w).numpy().astype(np.float64)
xs = [{k: ki.to_numpy(v) for k, v in ki.decode_inputs(n_seq, 96, 128, seed=4 + 1000 * w, step=t).items()}
      for t in range(steps)]
print("ready", flush=True)
sys.stdin.readline()
t0 = time.perf_counter()
for x in xs:
    _, S = oracle.kda_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S)
print(json.dumps({"seconds": time.perf_counter() - t0, "pair_steps": n_seq * 96 * steps}), flush=True)
"""


def cpu_baselines():
    """The fp64 oracle timed beside every workload on the host cores (inputs of
    the same laws and shapes drawn on the host): the tiny workload in full, the
    4K workload on all 96 heads, the packed varlen workload in full, the long
    workloads on 4 heads (64K and 1M tokens), and the decode workload's 100
    steps on all 512 x 96 pairs.  Prefill heads run in child processes, one
    slice of heads each; the decode pairs in 16 processes of 32 sequences."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import numpy as np
    import kda_inputs as ki
    import oracle
    import oracle_pool
    cores = oracle_pool.host_cores()
    out = {"cpu": oracle_pool.cpu_model(), "cores": cores, "kind": "oracle", "unit": "seconds of wall time"}

    def pool_run(name, x, heads=None, workers=None):
        r = oracle_pool.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens, heads=heads,
                                workers=workers, progress=lambda m: print(m, file=sys.stderr, flush=True))
        out[name] = {"seconds": round(r["seconds"], 3), "token_heads": r["token_heads"], "processes": r["workers"],
                     "token_heads_per_s": round(r["token_heads"] / r["seconds"], 1)}
        print(f"[cpu-baselines] {name}: {out[name]}", file=sys.stderr, flush=True)

    x = ki.workload_inputs("tiny_fp32")
    n = ki.to_numpy
    t0 = time.perf_counter()
    oracle.kda_prefill(n(x.q), n(x.k), n(x.v), n(x.log_alpha), n(x.beta), None)
    dt = time.perf_counter() - t0
    out["tiny_fp32"] = {"seconds": round(dt, 3), "token_heads": 512, "processes": 1,
                        "token_heads_per_s": round(512 / dt, 1)}
    pool_run("bf16_4k_96_heads", ki.workload_inputs("bf16_4k"))
    pool_run("varlen16_96_heads", ki.workload_inputs("varlen16"))
    heads4 = sorted(np.random.default_rng(3).choice(96, 4, replace=False).tolist())
    for T, name in ((65536, "long_64k_4_heads"), (1048576, "long_1m_4_heads")):
        x = ki.prefill_inputs([T], H=4, d=128, dtype="bf16", la_law="uniform53", init="normal", seed=3)
        pool_run(name, x, workers=4)
        del x
    # decode: 100 steps of 512 x 96 pairs, 16 processes of 32 sequences
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    procs = [subprocess.Popen([sys.executable, "-c", DECODE_WORKER % ROOT, str(w), "32", "100"],
                              stdin=subprocess.PIPE, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                              env=env) for w in range(16)]
    try:
        for p in procs:
            if p.stdout.readline().strip() != "ready":
                raise RuntimeError(p.stderr.read()[-2000:])
        t0 = time.perf_counter()
        for p in procs:
            p.stdin.write("go\n")
            p.stdin.flush()
        last = t0
        while any(p.poll() is None for p in procs):
            time.sleep(0.05)
            if time.perf_counter() - last > 20:
                last = time.perf_counter()
                print(f"  oracle decode: {sum(p.poll() is not None for p in procs)}/{len(procs)} processes done "
                      f"after {last - t0:.0f} s", file=sys.stderr, flush=True)
        wall = time.perf_counter() - t0
        res = [json.loads(p.communicate()[0].strip().splitlines()[-1]) for p in procs]
    finally:
        for p in procs:
            if p.poll() is None:
                p.kill()
    ps = sum(r["pair_steps"] for r in res)
    out["decode_100_steps_512x96"] = {"seconds": round(wall, 3), "pair_steps": ps, "processes": len(procs),
                                      "pair_steps_per_s": round(ps / wall, 1)}
    print(f"[cpu-baselines] decode: {out['decode_100_steps_512x96']}", file=sys.stderr, flush=True)
    return out


KERNEL_SOURCES = {
    "prefill": ["gated_delta_rule_09_amd/csrc/kda_prefill.hip", "gated_delta_rule_09_amd/csrc/kda_device.h",
                "gated_delta_rule_09_amd/csrc/kda_internal.h"],
    "decode": ["gated_delta_rule_09_amd/csrc/kda_decode.hip", "gated_delta_rule_09_amd/csrc/kda_device.h",
               "gated_delta_rule_09_amd/csrc/kda_internal.h"],
    "epilogue": ["gated_delta_rule_09_amd/csrc/kda_epilogue.hip", "gated_delta_rule_09_amd/csrc/kda_device.h",
                 "gated_delta_rule_09_amd/csrc/kda_internal.h"],
    "prologue": ["gated_delta_rule_09_amd/csrc/kda_prologue.hip", "gated_delta_rule_09_amd/csrc/kda_device.h",
                 "gated_delta_rule_09_amd/csrc/kda_internal.h"],
    "split": ["gated_delta_rule_09_amd/csrc/kda_split.hip", "gated_delta_rule_09_amd/csrc/kda_device.h",
              "gated_delta_rule_09_amd/csrc/kda_internal.h"],
}


def kernel_digest(kernel: str) -> str:
    """SHA-256 of a kernel's source files with comments and whitespace removed,
    so that an edit of comments alone keeps a counter measurement valid while
    any change of code voids it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(rel.encode() + b"\0" + "".join(src.split()).encode() + b"\0")
    return h.hexdigest()


def measured_util(kernel: str):
    """rocprofv3 MfmaUtil / VALUBusy (percent) recorded for the kernel's current code, or None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("code_digest") != kernel_digest(kernel):
        return None, None
    return rec.get("mfma_util_pct"), rec.get("valu_busy_pct")


def measured_traffic(kernel: str, launch_ms: float):
    """HBM bytes per launch measured by the rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes (calibrated against a plain copy), as GB/s over this run's launch
    time; None when the kernel's code changed since the counters were taken or
    no measurement is stored."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("code_digest") != kernel_digest(kernel):
        return None
    return round((rec["hbm_bytes_read"] + rec["hbm_bytes_written"]) / (launch_ms * 1e-3) / 1e9, 1)


def _timed(args, stream, fn, reps):
    """Average duration of fn() over reps back-to-back calls, HIP events on `stream`."""
    import torch
    for _ in range(max(1, args.warmup)):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_epilogue(args, dev, stream, ki, lib):
    """The output epilogue (Sigmoid(W_g x) * RMSNorm(o), head-wise): the standalone
    kernel on the 64K x 96-head output, the gated prefill followed by it, and the
    gated decode with it fused, timed outside the headline step."""
    import torch
    e = ki.epilogue_inputs((T_PREFILL, H, D), "bf16", seed=64, device=dev)
    y = torch.empty_like(e["o"])
    epi_ms = _timed(args, stream, lambda: lib.kda_output_gate_rmsnorm(e["o"], e["gate"], e["weight"], y=y),
                    max(1, args.steps))
    epi_bytes = T_PREFILL * H * EPILOGUE_BYTES_PER_TOKEN_HEAD + D * 4
    del y
    xg = ki.gated_inputs([T_PREFILL], H=H, d=D, dtype="bf16", seed=3, device=dev)
    yp = torch.empty_like(xg.v)
    fg = torch.empty_like(xg.init_state)
    pre_ms = _timed(args, stream, lambda: lib.kda_chunk_prefill_gated_epilogue(
        xg.q, xg.k, xg.v, xg.g_logits, xg.a_log, xg.beta_logits, e["gate"], e["weight"],
        init_state=xg.init_state, y=yp, final_state=fg), max(1, args.steps))
    del xg, yp, fg, e
    w = ki.DECODE_WORKLOAD
    sg = ki.decode_state(w["N"], w["H"], w["d"], seed=w["seed"], device=dev)
    dg = ki.decode_gated_inputs(w["N"], w["H"], w["d"], dtype=w["dtype"], seed=w["seed"], step=0, device=dev)
    og = ki.out_gate_inputs((w["N"], w["H"], w["d"]), "bf16", seed=w["seed"], device=dev)
    yd = torch.empty_like(dg["v"])
    dec_ms = _timed(args, stream, lambda: lib.kda_decode_step_gated_epilogue(
        dg["q"], dg["k"], dg["v"], dg["g_logits"], dg["a_log"], dg["beta_logits"], og["gate"], sg,
        norm_weight=og["weight"], y=yd), max(1, args.steps))
    dec_bytes = N_DECODE * H * EPILOGUE_DECODE_BYTES_PER_PAIR
    epi_gbps = epi_bytes / (epi_ms * 1e-3) / 1e9
    return {"standalone": {"ms": round(epi_ms, 4), "gbps": round(epi_gbps, 1),
                           "frac": round(epi_gbps / HBM_PEAK_GBPS, 4),
                           "traffic": measured_traffic("epilogue", epi_ms),
                           "bytes_per_token_head": EPILOGUE_BYTES_PER_TOKEN_HEAD,
                           "kernel": "gate_rmsnorm_kernel", "rows": T_PREFILL * H},
            "prefill_gated_epilogue": {"ms": round(pre_ms, 4),
                                       "tokens_per_s": round(T_PREFILL / (pre_ms * 1e-3), 1)},
            "decode_gated_epilogue": {"ms": round(dec_ms, 4),
                                      "gbps": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
                                      "frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "config": "y = Sigmoid(g) * w * o / sqrt(mean(o^2) + 1e-5) per (token, head); o ~ N(0, 1) x "
                      "10^U[-3, 1] per row, g ~ N(0, 4), w ~ U[0.5, 1.5]; 64K x 96 x 128 bf16 and the "
                      "512 x 96 gated decode"}


def time_prologue(args, dev, stream, ki, lib):
    """The input prologue (ShortConv(4), Swish, L2 norm of q and k): the standalone
    kernel on the 64K x 96-head inputs, the whole prefill layer core (prologue,
    gated prefill, epilogue) and the one-kernel fused decode step."""
    import torch
    reps = max(1, args.steps)
    x = ki.prologue_inputs([T_PREFILL], H=H, d=D, dtype="bf16", seed=3, device=dev)
    q, k, v = torch.empty_like(x["x_q"]), torch.empty_like(x["x_k"]), torch.empty_like(x["x_v"])
    cso = torch.empty_like(x["conv_state"])
    pro_ms = _timed(args, stream, lambda: lib.kda_short_conv_prologue(
        x["x_q"], x["x_k"], x["x_v"], x["conv_w"], x["conv_state"], q=q, k=k, v=v, conv_state_out=cso), reps)
    pro_bytes = T_PREFILL * H * PROLOGUE_BYTES_PER_TOKEN_HEAD + 2 * H * 3 * CONV_C * 2 + H * CONV_C * 16
    xg = ki.gated_inputs([T_PREFILL], H=H, d=D, dtype="bf16", seed=3, device=dev)
    og = ki.out_gate_inputs((T_PREFILL, H, D), "bf16", seed=3, device=dev)
    y = torch.empty_like(xg.v)
    fin = torch.empty_like(xg.init_state)

    def layer():
        lib.kda_short_conv_prologue(x["x_q"], x["x_k"], x["x_v"], x["conv_w"], x["conv_state"], q=q, k=k, v=v,
                                    conv_state_out=cso)
        lib.kda_chunk_prefill_gated_epilogue(q, k, v, xg.g_logits, xg.a_log, xg.beta_logits, og["gate"],
                                             og["weight"], init_state=xg.init_state, y=y, final_state=fin)

    layer_ms = _timed(args, stream, layer, reps)
    del x, q, k, v, cso, xg, og, y, fin
    w = ki.DECODE_WORKLOAD
    sg = ki.decode_state(w["N"], w["H"], w["d"], seed=w["seed"], device=dev)
    dp = ki.decode_prologue_inputs(w["N"], w["H"], w["d"], "bf16", seed=w["seed"], device=dev)
    dg = ki.decode_gated_inputs(w["N"], w["H"], w["d"], dtype=w["dtype"], seed=w["seed"], step=0, device=dev)
    dog = ki.out_gate_inputs((w["N"], w["H"], w["d"]), "bf16", seed=w["seed"], device=dev)
    yd = torch.empty_like(dp["x_v"])
    dec_ms = _timed(args, stream, lambda: lib.kda_decode_step_fused(
        dp["x_q"], dp["x_k"], dp["x_v"], dp["conv_w"], dp["conv_state"], dg["g_logits"], dg["a_log"],
        dg["beta_logits"], dog["gate"], sg, norm_weight=dog["weight"], y=yd), reps)
    dec_bytes = N_DECODE * H * FUSED_DECODE_BYTES_PER_PAIR + H * CONV_C * 16
    pro_gbps = pro_bytes / (pro_ms * 1e-3) / 1e9
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    return {"standalone": {"ms": round(pro_ms, 4), "gbps": round(pro_gbps, 1),
                           "frac": round(pro_gbps / HBM_PEAK_GBPS, 4),
                           "traffic": measured_traffic("prologue", pro_ms),
                           "bytes_per_token_head": PROLOGUE_BYTES_PER_TOKEN_HEAD, "kernel": "prologue_kernel"},
            "prefill_layer": {"ms": round(layer_ms, 4), "tokens_per_s": round(T_PREFILL / (layer_ms * 1e-3), 1),
                              "kernels": "prologue, gated prefill, epilogue"},
            "decode_fused": {"ms": round(dec_ms, 4), "gbps": round(dec_gbps, 1),
                             "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                             "bytes_per_pair": FUSED_DECODE_BYTES_PER_PAIR},
            "config": "x_q, x_k, x_v ~ N(0, 1) bf16, taps ~ U[-1/2, 1/2], conv state ~ N(0, 1); 64K x 96 x 128 "
                      "prefill and the 512 x 96 decode"}


def time_capacity(args, dev, stream, ki, prefill):
    """The capacity run: one sequence of T = 1,048,576 tokens, H = 96, d = 128,
    bf16, log-decay U[-5, -3] (about 150 GB of inputs and outputs resident)."""
    import torch
    x = ki.workload_inputs("long_1m", device=dev)
    T = x.q.shape[0]
    o = torch.empty_like(x.v)
    fin = torch.empty_like(x.init_state)
    ms = _timed(args, stream, lambda: prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, None, o=o,
                                              final_state=fin), max(1, min(args.steps, 3)))
    byts = T * H * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * H * STATE_BYTES
    return {"tokens": T, "ms": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "gbps": round(byts / (ms * 1e-3) / 1e9, 1), "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def time_gated(args, dev, stream, ki, prefill_gated, decode_gated):
    """The gated entry points (decay / write-strength logits mapped in-kernel) on the
    same 64K prefill and 512 x 96 decode shapes, timed outside the headline step."""
    import torch
    xg = ki.gated_inputs([T_PREFILL], H=H, d=D, dtype="bf16", seed=3, device=dev)
    og = torch.empty_like(xg.v)
    fg = torch.empty_like(xg.init_state)
    w = ki.DECODE_WORKLOAD
    sg = ki.decode_state(w["N"], w["H"], w["d"], seed=w["seed"], device=dev)
    dg = ki.decode_gated_inputs(w["N"], w["H"], w["d"], dtype=w["dtype"], seed=w["seed"], step=0, device=dev)
    odg = torch.empty_like(dg["v"])

    def run_prefill():
        prefill_gated(xg.q, xg.k, xg.v, xg.g_logits, xg.a_log, xg.beta_logits, xg.init_state, None, o=og,
                      final_state=fg)

    def run_decode():
        decode_gated(dg["q"], dg["k"], dg["v"], dg["g_logits"], dg["a_log"], dg["beta_logits"], sg, o=odg)

    pre_ms = _timed(args, stream, run_prefill, max(1, args.steps))
    dec_ms = _timed(args, stream, run_decode, max(1, args.steps))
    pre_bytes = T_PREFILL * H * GATED_PREFILL_BYTES_PER_TOKEN_HEAD + 2 * H * STATE_BYTES
    dec_bytes = N_DECODE * H * GATED_DECODE_BYTES_PER_PAIR
    return {"prefill_ms": round(pre_ms, 4), "prefill_tokens_per_s": round(T_PREFILL / (pre_ms * 1e-3), 1),
            "prefill_gbps": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1),
            "prefill_bytes_per_token_head": GATED_PREFILL_BYTES_PER_TOKEN_HEAD,
            "decode_ms": round(dec_ms, 4), "decode_gbps": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
            "decode_frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "config": "gated entry points: bf16 decay logits z ~ N(0, 4), A_h ~ U[-1, 1], fp32 beta logits "
                      "~ N(0, 1); same shapes as the headline step"}


def time_varlen(args, dev, stream, ki, prefill):
    """The packed workload: 16 sequences of U{1024..8192} tokens, H = 96, d = 128,
    bf16, each with its own initial and final state (3,072 workgroups, enough to
    occupy every CU, unlike the single 64K sequence)."""
    import torch
    x = ki.workload_inputs("varlen16", device=dev)
    T = x.q.shape[0]
    N = x.cu_seqlens.shape[0] - 1
    o = torch.empty_like(x.v)
    fin = torch.empty_like(x.init_state)
    ms = _timed(args, stream, lambda: prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, x.cu_seqlens,
                                              o=o, final_state=fin), max(1, args.steps))
    byts = T * H * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * N * H * STATE_BYTES
    return {"sequences": N, "tokens": T, "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "gbps": round(byts / (ms * 1e-3) / 1e9, 1), "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


SPLIT_HEADS = 12    # one GPU's share of the 96 heads under an 8-way head split


def time_split_capacity(args, dev, stream, ki, lib):
    """The time split at the capacity length: one sequence of T = 1,048,576 tokens at
    H = 12 (one GPU's share of 96 heads split 8 ways), d = 128, bf16, log-decay U[-5, -3]."""
    import torch
    T, Hs = 1 << 20, SPLIT_HEADS
    x = ki.prefill_inputs([T], H=Hs, d=D, dtype="bf16", la_law="uniform53", init="normal", seed=3, device=dev)
    o = torch.empty_like(x.v)
    fin = torch.empty_like(x.init_state)
    seg = lib.split_segments(T, Hs, D, D, device=dev)
    ws = torch.empty((max(1, lib.split_workspace_bytes(T, Hs, D, D, torch.bfloat16, seg)),), dtype=torch.uint8,
                     device=dev)
    reps = max(1, min(args.steps, 3))
    plain_ms = _timed(args, stream, lambda: lib.kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state,
                                                                  None, o=o, final_state=fin), reps)
    split_ms = _timed(args, stream, lambda: lib.kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta,
                                                                        x.init_state, segments=seg, workspace=ws,
                                                                        o=o, final_state=fin), reps)
    return {"heads": Hs, "tokens": T, "segments": seg, "plain_ms": round(plain_ms, 3),
            "split_ms": round(split_ms, 3), "split_tokens_per_s": round(T / (split_ms * 1e-3), 1),
            "speedup": round(plain_ms / split_ms, 3)}


def time_split(args, dev, stream, ki, lib):
    """The time-split prefill against the plain one on one GPU's share of a 96-head
    layer split 8 ways over heads: T = 65,536, H = 12, d = 128, bf16, log-decay
    U[-5, -3].  The plain kernel fills 24 of the CUs there; the split runs the
    segments at once (the library's own segment count) and joins them."""
    import torch
    T, Hs = T_PREFILL, SPLIT_HEADS
    x = ki.prefill_inputs([T], H=Hs, d=D, dtype="bf16", la_law="uniform53", init="normal", seed=3, device=dev)
    o = torch.empty_like(x.v)
    fin = torch.empty_like(x.init_state)
    seg = lib.split_segments(T, Hs, D, D, device=dev)
    ws = torch.empty((max(1, lib.split_workspace_bytes(T, Hs, D, D, torch.bfloat16, seg)),), dtype=torch.uint8,
                     device=dev)
    reps = max(1, args.steps)
    plain_ms = _timed(args, stream, lambda: lib.kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state,
                                                                  None, o=o, final_state=fin), reps)
    split_ms = _timed(args, stream, lambda: lib.kda_chunk_prefill_split(x.q, x.k, x.v, x.log_alpha, x.beta,
                                                                        x.init_state, segments=seg, workspace=ws,
                                                                        o=o, final_state=fin), reps)
    byts = T * Hs * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * Hs * STATE_BYTES
    return {"heads": Hs, "tokens": T, "segments": seg,
            "plain_ms": round(plain_ms, 4), "plain_tokens_per_s": round(T / (plain_ms * 1e-3), 1),
            "split_ms": round(split_ms, 4), "split_tokens_per_s": round(T / (split_ms * 1e-3), 1),
            "speedup": round(plain_ms / split_ms, 3),
            "split_gbps_algorithmic": round(byts / (split_ms * 1e-3) / 1e9, 1),
            "split_frac": round(byts / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "config": "kda_chunk_prefill_split vs kda_chunk_prefill, T=65536 H=12 d=128 bf16 (one GPU's share "
                      "of 96 heads split 8 ways), log-decay U[-5,-3], fp32 state; algorithmic bytes as the "
                      "plain prefill's"}


# Algorithmic bytes (read, written) per launch of each counted kernel, as bench.py runs it.
_ROWS = T_PREFILL * H
_PAIRS = N_DECODE * H
ALG_BYTES = {
    "prefill": (_ROWS * (3 * D * 2 + D * 4 + 4) + H * STATE_BYTES, _ROWS * D * 2 + H * STATE_BYTES),
    "prefill_gated": (_ROWS * (3 * D * 2 + D * 2 + 4) + H * STATE_BYTES, _ROWS * D * 2 + H * STATE_BYTES),
    "decode": (_PAIRS * (STATE_BYTES + 3 * D * 2 + D * 4 + 4), _PAIRS * (STATE_BYTES + D * 2)),
    "decode_epilogue": (_PAIRS * (STATE_BYTES + 3 * D * 2 + D * 2 + 4 + D * 2), _PAIRS * (STATE_BYTES + D * 2)),
    "decode_fused": (_PAIRS * (STATE_BYTES + 3 * D * 2 + 3 * CONV_C * 2 + D * 2 + 4 + D * 2) + H * CONV_C * 16,
                     _PAIRS * (STATE_BYTES + D * 2 + 3 * CONV_C * 2)),
    "epilogue": (_ROWS * D * 2 * 2 + D * 4, _ROWS * D * 2),
    "epilogue_after_prefill": (_ROWS * D * 2 * 2 + D * 4, _ROWS * D * 2),
    "prologue": (_ROWS * 3 * D * 2 + H * 3 * CONV_C * 2 + H * CONV_C * 16, _ROWS * 3 * D * 2 + H * 3 * CONV_C * 2),
}
# Source group (for the code digest) of each counted kernel.
_LABEL_SOURCE = {"prefill": "prefill", "prefill_gated": "prefill", "decode": "decode",
                 "decode_epilogue": "decode", "decode_fused": "decode", "epilogue": "epilogue",
                 "epilogue_after_prefill": "epilogue", "prologue": "prologue"}


def _read_dispatches(path):
    """[(kernel name, {counter: value summed over instances})] in dispatch order, from a rocprofv3
    results DB or its counter_collection.csv."""
    if path.endswith(".csv"):
        import csv
        acc, grids = {}, {}
        with open(path, newline="") as fh:
            for r in csv.DictReader(fh):
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"])
                acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
                if r.get("Grid_Size"):
                    grids[int(r["Dispatch_Id"])] = float(r["Grid_Size"])
        rows = sorted((d, n, c, v) for (d, n, c), v in acc.items())
        rows += [(d, None, "_grid", g) for d, g in grids.items()]
        rows.sort(key=lambda t: t[0])
    else:
        import sqlite3
        con = sqlite3.connect(path)
        rows = con.execute("SELECT dispatch_id, kernel_name, counter_name, SUM(value) FROM counters_collection "
                           "GROUP BY dispatch_id, counter_name ORDER BY dispatch_id").fetchall()
        con.close()
    out, idx = [], {}
    for disp, name, counter, value in rows:
        if disp not in idx:
            idx[disp] = len(out)
            out.append((name, {}))
        if name is not None and out[idx[disp]][0] is None:
            out[idx[disp]] = (name, out[idx[disp]][1])
        out[idx[disp]][1][counter] = value
    return out


def _label_dispatches(disp):
    """Name each dispatch of a `bench.py --no-gated --no-split --no-varlen` run after the kernel and the step it
    belongs to: a prologue followed by a gated prefill is part of the timed layer (not labelled), and
    an epilogue directly after a gated prefill is the gated prefill's epilogue.  A run with the split
    timing is refused: its 12-head prefills launch the same kernel as the headline prefill."""
    import re
    names = [d[0] for d in disp]
    if any("split_scan_kernel" in n or "split_correct_kernel" in n for n in names):
        raise SystemExit("the counter runs must be made with --no-split")
    labels = []
    for i, n in enumerate(names):
        m = re.search(r"prefill_kernel<[^,]+, 128, 128, (true|false)>", n)
        d = re.search(r"decode_kernel<[^,]+, 128, 128, (true|false), (true|false), (true|false), \d+>", n)
        prev_gp = i > 0 and re.search(r"prefill_kernel<[^>]*true>", names[i - 1]) is not None
        j = i + 1   # the prologue entry point also launches a small kernel for the convolution state
        while j < len(names) and "prologue_empty_kernel" in names[j]:
            j += 1
        next_gp = j < len(names) and re.search(r"prefill_kernel<[^>]*true>", names[j]) is not None
        if m:
            labels.append("prefill_gated" if m.group(1) == "true" else "prefill")
        elif d:
            gated, norm, pro = (g == "true" for g in d.groups())
            labels.append("decode_fused" if pro else "decode_epilogue" if norm else
                          None if gated else "decode")
        elif "gate_rmsnorm_kernel" in n:
            labels.append("epilogue_after_prefill" if prev_gp else "epilogue")
        elif "prologue_kernel" in n:
            labels.append(None if next_gp else "prologue")
        else:
            labels.append(None)
    # Every dispatch of one label must have one launch shape (the varlen timing launches the
    # headline prefill's kernel on another grid).
    grids = {}
    for lab, (_, c) in zip(labels, disp):
        if lab is not None and "_grid" in c:
            grids.setdefault(lab, set()).add(c["_grid"])
    if any(len(g) > 1 for g in grids.values()):
        raise SystemExit("dispatches of one kernel on different grids: make the counter runs with "
                         "--no-gated --no-split --no-varlen")
    return labels


def record_counters(pmc_dir: str, copy_gib: float):
    """Build profiles/hbm_traffic.json from three rocprofv3 runs of
    `bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-gated --no-split --no-varlen --calibrate-copy-gib G`
    stored under
    pmc_dir/fetch (--pmc FETCH_SIZE), pmc_dir/write (--pmc WRITE_SIZE) and pmc_dir/util
    (--pmc MfmaUtil VALUBusy), each a results DB or --output-format csv.  HBM bytes are the counters scaled by what they read for the plain
    copy of G GiB; every record carries the code digest of its kernel's sources."""
    import glob
    dbs = {}
    for part in ("fetch", "write", "util"):
        found = sorted(glob.glob(os.path.join(pmc_dir, part, "**", "*_results.db"), recursive=True) +
                       glob.glob(os.path.join(pmc_dir, part, "**", "*counter_collection.csv"), recursive=True))
        if not found:
            raise SystemExit(f"no rocprofv3 results under {os.path.join(pmc_dir, part)}")
        dbs[part] = _read_dispatches(found[0])
    copy_kib = copy_gib * (1 << 30) / 1024

    # The calibration copy is the one dispatch that writes about G GiB (WRITE_SIZE counts bytes
    # written one to one); the three runs dispatch the same kernels in the same order.
    wr = [c.get("WRITE_SIZE", 0.0) for _, c in dbs["write"]]
    idx = [i for i, v in enumerate(wr) if 0.9 * copy_kib < v < 1.1 * copy_kib]
    if len(idx) != 1 or len(dbs["fetch"]) != len(dbs["write"]) or \
            dbs["fetch"][idx[0]][0] != dbs["write"][idx[0]][0]:
        raise SystemExit("cannot identify the calibration copy in the counter runs")
    write_factor = wr[idx[0]] / copy_kib
    fetch_factor = dbs["fetch"][idx[0]][1]["FETCH_SIZE"] / copy_kib
    per = {}
    for part, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"), ("util", "MfmaUtil"),
                          ("util", "VALUBusy")):
        disp = dbs[part]
        for lab, (_, c) in zip(_label_dispatches(disp), disp):
            if lab is not None and counter in c:
                per.setdefault(lab, {}).setdefault(counter, []).append(c[counter])
    rec = {}
    for lab, vals in per.items():
        src = _LABEL_SOURCE[lab]
        f, w = vals.get("FETCH_SIZE", []), vals.get("WRITE_SIZE", [])
        if not f or not w:
            continue
        rd = sum(f) / len(f) * 1024 / fetch_factor
        wr = sum(w) / len(w) * 1024 / write_factor
        alg_r, alg_w = ALG_BYTES[lab]
        mu, vb = vals.get("MfmaUtil", []), vals.get("VALUBusy", [])
        rec[lab] = {"source": KERNEL_SOURCES[src][0], "code_digest": kernel_digest(src),
                    "hbm_bytes_read": rd, "hbm_bytes_written": wr, "alg_bytes_read": alg_r,
                    "alg_bytes_written": alg_w, "fetch_kib_raw": f, "write_kib_raw": w,
                    "mfma_util_pct": sum(mu) / len(mu) if mu else None,
                    "valu_busy_pct": sum(vb) / len(vb) if vb else None}
    rec["calibration"] = {"fetch_factor": fetch_factor, "write_factor": write_factor,
                          "copy_bytes": int(copy_gib * (1 << 30))}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"calibration: FETCH_SIZE factor {fetch_factor:.4f}, WRITE_SIZE factor {write_factor:.4f} "
          f"(copy of {copy_gib:g} GiB)")
    print(f"{'kernel (per dispatch, mean)':28s} {'GB read':>8s} {'GB wrtn':>8s} {'alg rd':>8s} {'alg wr':>8s}  "
          f"measured / algorithmic   MfmaUtil %  VALUBusy %")
    for lab, r in rec.items():
        if lab == "calibration":
            continue
        mu = "-" if r["mfma_util_pct"] is None else f"{r['mfma_util_pct']:.1f}"
        vb = "-" if r["valu_busy_pct"] is None else f"{r['valu_busy_pct']:.1f}"
        print(f"{lab:28s} {r['hbm_bytes_read'] / 1e9:8.3f} {r['hbm_bytes_written'] / 1e9:8.3f} "
              f"{r['alg_bytes_read'] / 1e9:8.3f} {r['alg_bytes_written'] / 1e9:8.3f}  "
              f"{r['hbm_bytes_read'] / r['alg_bytes_read']:.2f}x / {r['hbm_bytes_written'] / r['alg_bytes_written']:.2f}x"
              f"          {mu:>6s}      {vb:>6s}")
    print(f"wrote {os.path.relpath(path, ROOT)}")


def _smi_power_clocks():
    """One `amd-smi metric -p -c` reading: (socket power in W, [gfx clocks in MHz]), or None."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                           timeout=10)
        j = json.loads(r.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    def find(o):      # the first object holding both the power and the clock readings
        if isinstance(o, dict):
            if "power" in o and "clock" in o:
                return o
            o = list(o.values())
        if isinstance(o, list):
            for v in o:
                r = find(v)
                if r is not None:
                    return r
        return None
    g = find(j)
    try:
        watts = float(g["power"]["socket_power"]["value"])
        clocks = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                  if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
    except (KeyError, TypeError, ValueError):
        return None
    return watts, clocks


def sample_power(dev, x, o, fin, seconds):
    """Socket power and shader clocks while the prefill runs back to back for `seconds`, read with
    amd-smi every 0.3 s on a second thread (the first 0.5 s, while the clocks ramp, is dropped)."""
    import threading
    import torch
    from gated_delta_rule_09_amd import kda_chunk_prefill
    reads, stop = [], threading.Event()

    def sampler(t0):
        while not stop.is_set():
            r = _smi_power_clocks()
            if r is not None and time.perf_counter() - t0 > 0.5:
                reads.append(r)
            stop.wait(0.3)

    idle = _smi_power_clocks()
    t0 = time.perf_counter()
    th = threading.Thread(target=sampler, args=(t0,), daemon=True)
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, None, o=o, final_state=fin)
        torch.cuda.synchronize()
        n += 20
    wall = time.perf_counter() - t0
    stop.set()
    th.join()
    if not reads:
        return {"error": "amd-smi gave no reading"}
    watts = sorted(r[0] for r in reads)
    clocks = sorted(c for r in reads for c in r[1])
    return {"prefills": n, "ms_per_prefill": round(1e3 * wall / n, 4), "readings": len(reads),
            "socket_power_w_median": watts[len(watts) // 2], "socket_power_w_range": [watts[0], watts[-1]],
            "gfx_clock_mhz_median": clocks[len(clocks) // 2], "gfx_clock_mhz_range": [clocks[0], clocks[-1]],
            "idle_socket_power_w": None if idle is None else idle[0]}


def time_stream_reference(dev, stream, gib=3.0, reps=10):
    """Plain streaming rates of this GPU, as context for the HBM fractions: torch's own in-place scale
    (read:write 1:1), add (2:1), fill (write only) and copy over fp32 buffers of `gib` GiB each.
    Median of `reps` launches after one untimed launch."""
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a).fill_(2.0)
    c = torch.empty_like(a)
    nb = 4 * n
    ops = {"inplace_scale_1to1": (lambda: a.mul_(1.0), 2 * nb),
           "copy_1to1": (lambda: c.copy_(a), 2 * nb),
           "add_2to1": (lambda: torch.add(a, b, out=c), 3 * nb),
           "fill_write_only": (lambda: c.fill_(3.0), nb)}
    out = {"buffer_gib": gib}
    for name, (fn, moved) in ops.items():
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        ts.sort()
        out[name + "_gbps"] = round(moved / (ts[len(ts) // 2] * 1e-3) / 1e9, 1)
    del a, b, c
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="also time the fp64 oracle beside every workload (several minutes of host time)")
    ap.add_argument("--no-gated", action="store_true", help="skip the timing of the gated entry points")
    ap.add_argument("--no-epilogue", action="store_true",
                    help="skip the timing of the output epilogue and the input prologue")
    ap.add_argument("--no-varlen", action="store_true", help="skip the timing of the packed varlen workload")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the time-split prefill at one GPU's share of the heads (H = 12)")
    ap.add_argument("--capacity", action="store_true",
                    help="also time the 1,048,576-token prefill (about 150 GB of device memory), and the time "
                         "split at that length with 12 heads")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="also run one plain device-to-device copy of this many GiB (counter calibration)")
    ap.add_argument("--power-seconds", type=float, default=0.0,
                    help="also run the prefill back to back for this many seconds while amd-smi reads the "
                         "socket power and shader clocks")
    ap.add_argument("--stream-reference", action="store_true",
                    help="also time torch's plain streaming ops (in-place scale, copy, add, fill) on 3 GiB buffers")
    ap.add_argument("--record-counters", metavar="PMC_DIR",
                    help="no GPU run: build profiles/hbm_traffic.json from the rocprofv3 passes under PMC_DIR "
                         "(fetch/, write/, util/) of a run made with --calibrate-copy-gib")
    args = ap.parse_args()
    if args.record_counters:
        record_counters(args.record_counters, args.calibrate_copy_gib or 4.0)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the library's path is single-GPU "
                                   "(--gpus must be 1)"}))
        sys.exit(2)

    import torch
    import kda_inputs as ki
    from gated_delta_rule_09_amd import (kda_chunk_prefill, kda_chunk_prefill_gated, kda_decode_step,
                                         kda_decode_step_gated)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = ki.workload_inputs("long_64k", device=dev)
    o = torch.empty_like(x.v)
    fin = torch.empty_like(x.init_state)
    w = ki.DECODE_WORKLOAD
    state = ki.decode_state(w["N"], w["H"], w["d"], seed=w["seed"], device=dev)
    dx = ki.decode_inputs(w["N"], w["H"], w["d"], dtype=w["dtype"], la_law=w["la_law"], seed=w["seed"], step=0,
                          device=dev)
    od = torch.empty_like(dx["v"])
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        kda_chunk_prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.init_state, None, o=o, final_state=fin)
        if ev is not None:
            ev[1].record(stream)
        kda_decode_step(dx["q"], dx["k"], dx["v"], dx["log_alpha"], dx["beta"], state, o=od)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    pre_all = sorted(e[0].elapsed_time(e[1]) for e in evs)
    dec_all = sorted(e[1].elapsed_time(e[2]) for e in evs)
    pre_ms = sum(pre_all) / args.steps
    dec_ms = sum(dec_all) / args.steps
    median = lambda v: (v[(len(v) - 1) // 2] + v[len(v) // 2]) / 2

    if args.calibrate_copy_gib > 0:
        nbytes = int(args.calibrate_copy_gib * (1 << 30))
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    pre_bytes = T_PREFILL * H * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * H * STATE_BYTES
    pre_gbps = pre_bytes / (pre_ms * 1e-3) / 1e9
    pre_tflops = T_PREFILL * H * PREFILL_FLOPS_PER_TOKEN_HEAD / (pre_ms * 1e-3) / 1e12
    dec_bytes = N_DECODE * H * DECODE_BYTES_PER_PAIR
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    tok_s = T_PREFILL / (pre_ms * 1e-3)

    res = {
        "metric": "KDA prefill tokens/s (H=96,d=128,T=64K) + decode state-update HBM GB/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_prefill T=65536 H=96 d=128 bf16 (log-decay U[-5,-3], fp32 state) "
                               "+ kda_decode_step N=512 H=96 d=128 bf16 (fp32 state 3.2 GB in place)",
                   "prefill_tokens": T_PREFILL, "heads": H, "d_k": D, "d_v": D, "chunk": 64,
                   "decode_sequences": N_DECODE},
        "roofline": {"bound": "hbm", "achieved": round(pre_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(pre_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("prefill", pre_ms),
                     "kernel": "prefill_kernel", "avg_launch_ms": round(pre_ms, 4),
                     "median_launch_ms": round(median(pre_all), 4),
                     "algorithmic_bytes_per_launch": pre_bytes,
                     "mfma_frac_algorithmic": round(pre_tflops / BF16_DENSE_PEAK_TFLOPS, 4),
                     "mfma_util_rocprof_pct": measured_util("prefill")[0],
                     "valu_busy_rocprof_pct": measured_util("prefill")[1]},
        "decode": {"gbps": round(dec_gbps, 1), "ms_per_step": round(dec_ms, 4),
                   "median_ms_per_step": round(median(dec_all), 4),
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                                "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                                "traffic": measured_traffic("decode", dec_ms),
                                "kernel": "decode_kernel", "algorithmic_bytes_per_launch": dec_bytes}},
    }
    if args.power_seconds > 0:
        res["power"] = sample_power(dev, x, o, fin, args.power_seconds)
    if not args.no_varlen:
        res["varlen"] = time_varlen(args, dev, stream, ki, kda_chunk_prefill)
    if not args.no_gated:
        res["gated"] = time_gated(args, dev, stream, ki, kda_chunk_prefill_gated, kda_decode_step_gated)
    if not args.no_epilogue:
        del x, o, fin, state, dx, od
        torch.cuda.empty_cache()
        import gated_delta_rule_09_amd as lib
        res["epilogue"] = time_epilogue(args, dev, stream, ki, lib)
        torch.cuda.empty_cache()
        res["prologue"] = time_prologue(args, dev, stream, ki, lib)
    if not args.no_split:
        torch.cuda.empty_cache()
        import gated_delta_rule_09_amd as lib
        res["split"] = time_split(args, dev, stream, ki, lib)
    if args.capacity:
        torch.cuda.empty_cache()
        res["capacity"] = time_capacity(args, dev, stream, ki, kda_chunk_prefill)
        if not args.no_split:
            torch.cuda.empty_cache()
            import gated_delta_rule_09_amd as lib
            res["capacity_split"] = time_split_capacity(args, dev, stream, ki, lib)
    if args.stream_reference:
        torch.cuda.empty_cache()
        res["stream_reference"] = time_stream_reference(dev, stream)
    from gated_delta_rule_09_amd import wait_giveups
    res["wait_giveups"] = wait_giveups()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
    if args.cpu_baselines:
        res["cpu_baselines"] = cpu_baselines()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
