"""Writes hand_example_n2.json: a two-token attention example worked by hand.

The values are closed forms of the definition of standard attention
(bornlex.github.io "Flash Attention", section "Standard Attention"), evaluated
with the math module only; nothing here calls the oracle or the GPU library.

  q = [1, 0], k = [1, -1], v = [2, 0] (N = 2, d = 1), scale = 1
  row 0: S = [1, -1], P = [1, e^-2] / (1 + e^-2), O = 2 / (1 + e^-2) = 1 + tanh(1),
         lse = ln(e + e^-1)
  row 1: S = [0, 0], P = [1/2, 1/2], O = 1, lse = ln 2
  causal (key j allowed iff j <= i): row 0 sees only key 0, O = 2, lse = 1;
         row 1 is unchanged.
"""
import json
import math
import os

ex = {
    "source": "closed forms of standard attention worked by hand (bornlex.github.io "
              "'Flash Attention', section 'Standard Attention'); see make_hand_example.py",
    "q": [[1.0], [0.0]], "k": [[1.0], [-1.0]], "v": [[2.0], [0.0]], "scale": 1.0,
    "O": [[1.0 + math.tanh(1.0)], [1.0]],
    "lse": [math.log(math.e + math.exp(-1.0)), math.log(2.0)],
    "causal_O": [[2.0], [1.0]],
    "causal_lse": [1.0, math.log(2.0)],
}
if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_example_n2.json")
    with open(path, "w") as f:
        json.dump(ex, f, indent=1)
