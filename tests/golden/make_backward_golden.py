"""Writes backward_small.npz: every gradient of oracle/gdla_grad.py's gdla_backward on two small
problems (full causal; a window of 3 with packed documents), as the oracle computed them when each
head's probability matrix was kept for the whole call.  The backward pins compare later versions of
the oracle (which hold one head's probabilities at a time) with these values.  Calls only oracle/
(and the seeded input generators).  Run from the repository root:

    python tests/golden/make_backward_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle.gdla_grad as gg  # noqa: E402
import oracle.gdla_ref as ref  # noqa: E402
from tests.oracle_pins import make_dims, small_problem  # noqa: E402

CASES = ((0, None, 101), (3, [0, 0, 0, 3, 3, 3, 3, 7, 7], 102))


def case_gradients(i):
    win, docs, seed = CASES[i]
    cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=9, seed=seed)
    dims = make_dims(ref, cfg, win)
    dout = np.random.default_rng(seed + 1000).standard_normal((9, cfg["d_model"]))
    return gg.gdla_backward(x, w, dims, dout, doc_start=None if docs is None else np.array(docs))


if __name__ == "__main__":
    out = {}
    for i in range(len(CASES)):
        for k, v in case_gradients(i).items():
            if v is not None:
                out[f"case{i}_{k}"] = np.asarray(v, dtype=np.float64)
    np.savez_compressed(os.path.join(os.path.dirname(os.path.abspath(__file__)), "backward_small.npz"), **out)
    print("wrote", len(out), "arrays")
