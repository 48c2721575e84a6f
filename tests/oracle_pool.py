"""Fans the fp64 oracle out over child processes, one slice of heads (prefill)
or of sequences (decode) each (test infrastructure: the GPU parity tests use
it to compare every head of the larger prefill workloads and every pair of
the decode workload, and bench.py's oracle timings use it to time the oracle
on the host cores).

Heads are independent, so each child runs the plain token loop of the oracle
on its slice and nothing is shared.  Inputs travel as .npy files in a scratch
directory (memory-backed /dev/shm when it has room): bf16 tensors as their
raw 16-bit words, so the child sees exactly the values the GPU saw.  The
children are fresh interpreters (subprocess), started after the caller's GPU
work; they never touch the GPU.
"""
import json
import os
import shutil
import subprocess
import sys
import tempfile
import time

import numpy as np
import torch

WORKER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_worker.py")


def host_cores(max_workers: int = 16) -> int:
    """Processes to start: one per available core, at most max_workers."""
    return max(1, min(max_workers, len(os.sched_getaffinity(0))))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _scratch(nbytes: int) -> str:
    shm = "/dev/shm"
    if os.path.isdir(shm) and os.access(shm, os.W_OK) and shutil.disk_usage(shm).free > 2 * nbytes + (1 << 30):
        return tempfile.mkdtemp(prefix="kda_oracle_", dir=shm)
    return tempfile.mkdtemp(prefix="kda_oracle_")


def _save(d: str, name: str, t):
    if t is None:
        return
    if isinstance(t, torch.Tensor):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            np.save(os.path.join(d, name + ".bf16.npy"), t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
            return
        t = t.contiguous().cpu().numpy()
    np.save(os.path.join(d, name + ".npy"), np.ascontiguousarray(t))


def _nbytes(*ts):
    return sum(t.numel() * t.element_size() for t in ts if isinstance(t, torch.Tensor))


def prefill(q, k, v, decay, beta, init_state=None, cu_seqlens=None, a_log=None, o_gpu=None, fin_gpu=None,
            heads=None, workers=None, progress=None, return_o_ref=False):
    """Run the oracle prefill (gated when a_log is given) on `heads` (default:
    all), split over `workers` child processes, and compare with o_gpu and
    fin_gpu when given.

    Tensors are [T, H, .] (torch, any device, or NumPy); init_state [N, H, ...].
    Returns a dict: rel_o and rel_f (max |gpu - ref| / max |ref| over the
    heads run, as the suite's metric), finite, seconds (wall time of the
    children, which start together), token_heads, workers; with return_o_ref,
    also o_ref [T, len(heads), d_v] in fp64 (heads in ascending order)."""
    H = q.shape[1]
    hs = list(range(H)) if heads is None else sorted(int(h) for h in heads)
    W = max(1, min(workers or host_cores(), len(hs)))
    groups = [g.tolist() for g in np.array_split(np.array(hs), W) if len(g)]
    gated = a_log is not None
    root = _scratch(_nbytes(q, k, v, decay, beta, o_gpu) * len(hs) // max(H, 1))
    dirs = []
    try:
        for gi, g in enumerate(groups):
            d = os.path.join(root, f"w{gi}")
            os.makedirs(d)
            idx = torch.tensor(g) if isinstance(q, torch.Tensor) else np.array(g)
            pick = lambda t, ax=1: None if t is None else (
                t.index_select(ax, idx.to(t.device)) if isinstance(t, torch.Tensor) else np.take(t, idx, axis=ax))
            for name, t in (("q", q), ("k", k), ("v", v), ("decay", decay), ("beta", beta), ("o_gpu", o_gpu)):
                _save(d, name, pick(t))
            _save(d, "init_state", pick(init_state))
            _save(d, "fin_gpu", pick(fin_gpu))
            _save(d, "a_log", pick(a_log, 0))
            if cu_seqlens is not None:
                cu = cu_seqlens.cpu().numpy() if isinstance(cu_seqlens, torch.Tensor) else np.asarray(cu_seqlens)
                np.save(os.path.join(d, "cu_seqlens.npy"), cu.astype(np.int64))
            with open(os.path.join(d, "meta.json"), "w") as f:
                json.dump({"kind": "prefill_gated" if gated else "prefill", "keep_o_ref": bool(return_o_ref)}, f)
            dirs.append(d)
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
        t0 = time.perf_counter()
        procs = [subprocess.Popen([sys.executable, WORKER, d], env=env) for d in dirs]
        last = t0
        while any(p.poll() is None for p in procs):
            time.sleep(0.05)
            if progress is not None and time.perf_counter() - last > 20:
                last = time.perf_counter()
                progress(f"  oracle: {sum(p.poll() is not None for p in procs)}/{len(procs)} processes done "
                         f"after {last - t0:.0f} s")
        wall = time.perf_counter() - t0
        if any(p.returncode != 0 for p in procs):
            raise RuntimeError(f"oracle workers failed: {[p.returncode for p in procs]}")
        stats = []
        for d in dirs:
            with open(os.path.join(d, "stats.json")) as f:
                stats.append(json.load(f))
        o_ref = np.concatenate([np.load(os.path.join(d, "o_ref.npy")) for d in dirs], axis=1) if return_o_ref else None
    finally:
        shutil.rmtree(root, ignore_errors=True)
    res = {"seconds": wall, "oracle_seconds_max": max(s["seconds"] for s in stats),
           "token_heads": sum(s["token_heads"] for s in stats), "workers": len(dirs), "heads": len(hs)}
    if o_gpu is not None:
        den = max(s["o_ref_max"] for s in stats)
        res["rel_o"] = max(s["o_err_max"] for s in stats) / (den if den > 0 else 1.0)
    if fin_gpu is not None:
        den = max(s["f_ref_max"] for s in stats)
        res["rel_f"] = max(s["f_err_max"] for s in stats) / (den if den > 0 else 1.0)
    res["finite"] = all(s.get("o_finite", True) and s.get("f_finite", True) for s in stats)
    if return_o_ref:
        res["o_ref"] = o_ref
    return res


class DecodeRun:
    """The oracle decode over every (sequence, head) pair of a run of steps,
    split over child processes by sequence.

    Used as a context manager (its scratch directory is removed on exit).
    The caller saves the state before the first step (save_state0), then each
    step's inputs and the GPU's output as it goes (save_step), and finally
    calls compare() with the GPU's state after the last step.  Each child then
    runs the oracle's decode steps on its sequences in fp64 from the saved
    state.  compare() returns rel_o (the largest per-step max |gpu - ref| /
    max |ref| of o), rel_f (the same for the final state), finite, seconds
    and pair_steps."""

    def __init__(self, N: int, H: int, d_k: int, d_v: int, workers=None):
        self.N, self.steps = N, 0
        W = max(1, min(workers or host_cores(), N))
        self.ranges = [(int(a[0]), int(a[-1]) + 1) for a in np.array_split(np.arange(N), W) if len(a)]
        per_step = N * H * (8 * d_k + 4 * d_v + 4)      # q, k, v, o in bf16; log alpha and beta fp32
        self.root = _scratch(100 * per_step + 2 * N * H * d_k * d_v * 4)
        self.dirs = []
        for wi in range(len(self.ranges)):
            d = os.path.join(self.root, f"w{wi}")
            os.makedirs(d)
            self.dirs.append(d)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        shutil.rmtree(self.root, ignore_errors=True)
        return False

    def _split_save(self, name, t):
        t = t.detach()
        for d, (a, b) in zip(self.dirs, self.ranges):
            _save(d, name, t[a:b])

    def save_state0(self, state):
        self._split_save("state0", state.cpu())

    def save_step(self, x: dict, o):
        s = self.steps
        for name, key in (("q", "q"), ("k", "k"), ("v", "v"), ("decay", "log_alpha"), ("beta", "beta")):
            self._split_save(f"{name}_{s}", x[key].cpu())
        self._split_save(f"o_gpu_{s}", o.cpu())
        self.steps += 1

    def compare(self, fin_gpu, progress=None) -> dict:
        self._split_save("fin_gpu", fin_gpu.cpu())
        for d in self.dirs:
            with open(os.path.join(d, "meta.json"), "w") as f:
                json.dump({"kind": "decode", "steps": self.steps}, f)
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
        t0 = time.perf_counter()
        procs = [subprocess.Popen([sys.executable, WORKER, d], env=env) for d in self.dirs]
        try:
            last = t0
            while any(p.poll() is None for p in procs):
                time.sleep(0.05)
                if progress is not None and time.perf_counter() - last > 20:
                    last = time.perf_counter()
                    progress(f"  oracle: {sum(p.poll() is not None for p in procs)}/{len(procs)} processes done "
                             f"after {last - t0:.0f} s")
        finally:
            for p in procs:
                if p.poll() is None:
                    p.kill()
                    p.wait()
        wall = time.perf_counter() - t0
        if any(p.returncode != 0 for p in procs):
            raise RuntimeError(f"oracle workers failed: {[p.returncode for p in procs]}")
        stats = []
        for d in self.dirs:
            with open(os.path.join(d, "stats.json")) as f:
                stats.append(json.load(f))
        rel_o = 0.0
        for s in range(self.steps):
            den = max(st["o_ref_max"][s] for st in stats)
            rel_o = max(rel_o, max(st["o_err_max"][s] for st in stats) / (den if den > 0 else 1.0))
        den = max(st["f_ref_max"] for st in stats)
        return {"rel_o": rel_o, "rel_f": max(st["f_err_max"] for st in stats) / (den if den > 0 else 1.0),
                "finite": all(st["o_finite"] and st["f_finite"] for st in stats), "seconds": wall,
                "pair_steps": sum(st["pair_steps"] for st in stats), "workers": len(self.dirs)}

