"""Writes cifg_peephole_hand.json: a one-channel CIFG LSTM with peepholes
worked step by step from the textbook equations, with the Python math module
only.

Definition (the peephole LSTM of Gers and Schmidhuber, with the input gate
coupled to the forget gate, i = 1 - f, the "CIFG" variant; the Para-Seq
README, Main features, names the ParaLSTM cell "CIFG/peephole"):
  f_t = sigm(W_f x_t + b_xf + w_f h_{t-1} + b_hf + p_f c_{t-1})
  g_t = tanh(W_g x_t + b_xg + w_g h_{t-1} + b_hg)
  c_t = f_t c_{t-1} + (1 - f_t) g_t
  o_t = sigm(W_o x_t + b_xo + w_o h_{t-1} + b_ho + p_o c_t)
  h_t = o_t tanh(c_t)
The forget gate's peephole sees the previous cell state, the output gate's
the new one.  The record also holds the states the two easy misreadings
would give (output peephole on c_{t-1}; forget peephole on c_t is circular,
so the other misreading is the uncoupled input gate i = f), so a test can
check that the example tells them apart.
"""
import json
import math
import os


def sigm(a):
    return 1.0 / (1.0 + math.exp(-a))


W = {"f": 0.8, "g": -0.6, "o": 0.5}      # input weights (d = 1)
BX = {"f": 0.1, "g": 0.2, "o": -0.3}     # input biases
WH = {"f": 0.4, "g": -0.7, "o": 0.9}     # diagonal recurrent weights
BH = {"f": -0.05, "g": 0.15, "o": 0.05}  # recurrent biases
PF, PO = 0.6, -0.8                       # peepholes
X = [1.0, -0.5, 2.0]
C0, H0 = 0.3, -0.2


def run(out_peep_old=False, coupled=True):
    c, h = C0, H0
    states = []
    for x in X:
        f = sigm(W["f"] * x + BX["f"] + WH["f"] * h + BH["f"] + PF * c)
        g = math.tanh(W["g"] * x + BX["g"] + WH["g"] * h + BH["g"])
        i = (1.0 - f) if coupled else f
        c_new = f * c + i * g
        o = sigm(W["o"] * x + BX["o"] + WH["o"] * h + BH["o"] + PO * (c if out_peep_old else c_new))
        h = o * math.tanh(c_new)
        c = c_new
        states.append([c, h])
    return states


out = {
    "citation": "peephole LSTM (Gers and Schmidhuber) with coupled input and forget gates; the ParaLSTM "
                "'CIFG/peephole' cell named in the Para-Seq README, Main features",
    "gate_order": "f|g|o", "W_x": [W["f"], W["g"], W["o"]], "b_x": [BX["f"], BX["g"], BX["o"]],
    "W_h": [WH["f"], WH["g"], WH["o"]], "b_h": [BH["f"], BH["g"], BH["o"]], "peep": [PF, PO],
    "x": X, "h0_c_h": [C0, H0],
    "states_c_h": run(),
    "misreading_output_peephole_on_old_c": run(out_peep_old=True),
    "misreading_uncoupled_input_gate": run(coupled=False),
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "cifg_peephole_hand.json"), "w") as f:
    json.dump(out, f, indent=1)
print(out["states_c_h"])
