"""Writes oracle_regression.json: the fp64 oracle's output on one small seeded
packed batch.  Calls only ``oracle`` (and NumPy for the seeded inputs); its
output guards the oracle against accidental change.  Regenerate only with a
commit that names the passage of the pages justifying the change.

    python tests/golden/make_oracle_regression.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def case():
    rng = np.random.default_rng(20260101)
    lengths = [7, 0, 12, 1]
    T, H, d_k, d_v = sum(lengths), 2, 4, 3
    q = rng.standard_normal((T, H, d_k)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, d_k)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, d_v))
    la = -np.minimum(np.log1p(np.exp(rng.standard_normal((T, H, d_k)))), 5.0)
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    init = 0.02 * rng.standard_normal((len(lengths), H, d_k, d_v))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=b, init_state=init, cu_seqlens=cu)


def main():
    c = case()
    o, fin = oracle.kda_prefill(c["q"], c["k"], c["v"], c["log_alpha"], c["beta"],
                                init_state=c["init_state"], cu_seqlens=c["cu_seqlens"])
    out = {"generator": "tests/golden/make_oracle_regression.py (seed 20260101)",
           "o": o.tolist(), "final_state": fin.tolist()}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()
