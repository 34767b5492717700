"""Writes p4_tanh_n1.json: a scalar tanh RNN worked by hand, closed forms only.

Cell: h_t = tanh(w_h h_{t-1} + w_x x_t), w_h = 0.5, w_x = 1, no bias, h_{-1} = 0,
x = (1, 0).  The values are the closed-form rollout and the Newton (DEER)
iterates derived on paper from the method the DEER summary describes
(Approach: linearise with the Jacobians, solve the linear recurrence); only
the Python math module is used.
"""
import json
import math
import os

wh = 0.5
h1 = math.tanh(1.0)
h2 = math.tanh(wh * h1)
# sweep 1 at h = (0, 0): f = (tanh 1, tanh 0), J_2 = wh (1 - 0^2), r = f - 0
k1 = [h1, wh * h1]
# sweep 2 at h = k1: f_2 = tanh(wh h1) = h2, J_2 = wh (1 - h2^2), r_2 = h2 - wh h1
J2 = wh * (1.0 - h2 * h2)
r2 = h2 - wh * h1
k2 = [h1, wh * h1 + r2]          # dh_1 = r_1 = 0, dh_2 = J_2 * 0 + r_2
out = {
    "citation": "closed-form hand derivation of one DEER/Newton solve; method per 'Parallelizing "
                "non-linear sequential models over the sequence length' (Approach)",
    "cell": "tanh_rnn", "w_h": wh, "w_x": 1.0, "x": [1.0, 0.0], "h0": 0.0,
    "rollout": [h1, h2],
    "iterate_1": k1, "delta_1": h1,
    "J2_at_iterate_1": J2, "r2_at_iterate_1": r2,
    "iterate_2": k2, "delta_2": abs(r2),
    # the stop rule ends a solve after sweep T (exact by then), whatever max_iters >= T
    "iters_tol_1e-6_max_iters_3": 2,
    "iters_tol_1e-6_max_iters_T": 2,
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "p4_tanh_n1.json"), "w") as f:
    json.dump(out, f, indent=1)
