"""Writes closed_form.json: hand-derived closed-form attention cases.

Each value below is the result of the derivation written out in README.md (the
pages print no worked example).  The script uses only ``math``; it calls neither
the oracle nor the HIP path.  Run from the repository root:
``python tests/golden/make_closed_form.py``.
"""
import json
import math
import os

ln2, ln3, ln4 = math.log(2.0), math.log(3.0), math.log(4.0)

CASES = [
    {"name": "two_keys_ln3", "scale": 1.0, "causal": False,
     "q": [[[[1.0]]]], "k": [[[[0.0], [ln3]]]], "v": [[[[2.0], [6.0]]]],
     "do": [[[[1.0]]]],
     "o": [[[[5.0]]]], "lse": [[[ln4]]],
     "dq": [[[[0.75 * ln3]]]], "dk": [[[[-0.75], [0.75]]]], "dv": [[[[0.25], [0.75]]]]},
    {"name": "causal_bottom_right_2x3", "scale": 1.0, "causal": True,
     "q": [[[[0.0], [0.0]]]], "k": [[[[1.0], [2.0], [4.0]]]],
     "v": [[[[3.0], [6.0], [9.0]]]], "do": [[[[1.0], [1.0]]]],
     "o": [[[[4.5], [6.0]]]], "lse": [[[ln2, ln3]]],
     "dq": [[[[0.75], [3.0]]]], "dk": [[[[0.0], [0.0], [0.0]]]],
     "dv": [[[[5.0 / 6], [5.0 / 6], [1.0 / 3]]]]},
    {"name": "gqa_two_heads_one_kv", "scale": 1.0, "causal": False,
     "q": [[[[1.0]], [[0.0]]]], "k": [[[[0.0], [ln3]]]], "v": [[[[2.0], [6.0]]]],
     "do": [[[[1.0]], [[2.0]]]],
     "o": [[[[5.0]], [[4.0]]]], "lse": [[[ln4], [ln2]]],
     "dq": [[[[0.75 * ln3]], [[2.0 * ln3]]]], "dk": [[[[-0.75], [0.75]]]],
     "dv": [[[[1.25], [1.75]]]]},
    {"name": "empty_row", "scale": 1.0, "causal": True,
     "q": [[[[5.0], [7.0]]]], "k": [[[[3.0]]]], "v": [[[[2.0]]]],
     "do": [[[[1.0], [1.0]]]],
     "o": [[[[0.0], [2.0]]]], "lse": [[["-inf", 21.0]]],
     "dq": [[[[0.0], [0.0]]]], "dk": [[[[0.0]]]], "dv": [[[[1.0]]]]},
]

if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_form.json")
    with open(path, "w") as f:
        json.dump({"source": "closed forms derived by hand; derivations in README.md",
                   "cases": CASES}, f, indent=1)
    print("wrote", path)
