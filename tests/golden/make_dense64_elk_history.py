"""Writes dense64_gru_elk_full_history.json: the fp64 oracle's quasi-ELK
history (damping lambda = 0.1) on the full dense-GRU workload (B=16,
T=16384, d=32, n=64, tol 1e-5, seed 5).

Only the oracle is called.  The GPU test compares its sweep count and delta
history with this record instead of re-running the fp64 solve each time.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from nonlinear_rnn_evaluation_newton_amd import synthetic as sy  # noqa: E402

LAMBDA = 0.1
p = sy.make_problem(5, with_g=False)
h, iters, status, deltas = oracle.elk(p, LAMBDA)
h_seq = oracle.rollout(p)
out = {
    "source": "oracle.elk(lam=0.1) on synthetic.make_problem(5) (dense GRU n=64, B=16, T=16384, d=32, tol=1e-5)",
    "lambda": LAMBDA, "iters": int(iters), "status": int(status), "deltas": [float(x) for x in deltas],
    "max_abs_elk_minus_rollout": float(abs(h - h_seq).max()),
}
with open(os.path.join(HERE, "dense64_gru_elk_full_history.json"), "w") as f:
    json.dump(out, f, indent=1)
print({k: (v if not isinstance(v, list) else len(v)) for k, v in out.items()})
