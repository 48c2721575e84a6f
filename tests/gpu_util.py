"""Helpers for the GPU parity tests."""
import numpy as np
import torch

import kda_inputs as ki

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / (den if den > 0 else 1.0)


def host(x):
    return ki.to_numpy(x)


def device():
    return torch.device("cuda:0")


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
