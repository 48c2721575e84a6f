"""Runs the fp64 oracle on one head's inputs saved as .npy files (test
infrastructure for the long-context parity test, started as a child process).

    python tests/oracle_worker.py <dir>

reads q, k, v, log_alpha [T, 1, d], beta [T, 1], init_state [1, 1, d_k, d_v]
from <dir>/*.npy and writes o_ref.npy [T, 1, d_v] and final_ref.npy.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402


def main(d: str):
    ld = lambda n: np.load(os.path.join(d, n + ".npy"))
    o, fin = oracle.kda_prefill(ld("q"), ld("k"), ld("v"), ld("log_alpha"), ld("beta"), ld("init_state"))
    np.save(os.path.join(d, "o_ref.npy"), o)
    np.save(os.path.join(d, "final_ref.npy"), fin)


if __name__ == "__main__":
    main(sys.argv[1])
