"""Write tests/golden/closed_form.json from the closed-form derivation in oracle/closed_form.py.

The LinearARD pages print no worked example, so the stored values are the closed-form
relation KL of structured inputs (X_t = a E, X_s = b E, E = leading identity rows then
zero rows), derived from the definitions on the pith.science verdict page
(key_machinery: R_m = softmax(X X^T / sqrt(d) + M), row-wise forward KL, gradient
R_s - R_t) and evaluated in 50-digit decimal arithmetic.

Run:  python tests/golden/make_golden.py
"""

import json
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
from oracle.closed_form import structured_case  # noqa: E402


def f32_scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))


CASES = [
    # name, N, d, a, b, causal, g, dx rows stored (None = all)
    ("small_causal", 5, 8, 3.0, 2.0, True, 1.0, None),
    ("small_noncausal", 7, 16, 2.0, 4.0, False, 1.0, None),
    ("zero_rows_causal", 12, 8, 1.0, 3.0, True, 0.5, None),
    ("gpu_d64_causal", 300, 64, 2.0, 3.0, True, 1.0, [0, 1, 31, 32, 63, 64, 65, 150, 299]),
    ("gpu_d128_noncausal", 200, 128, 4.0, 3.0, False, 1.0, [0, 1, 63, 64, 127, 128, 199]),
    ("gpu_d128_causal", 257, 128, 3.0, 4.0, True, 2.0, [0, 5, 127, 128, 200, 256]),
]


def main():
    out = {"citation": "closed form of the definitions on the pith.science LinearARD verdict "
                       "page (pith_extraction.key_machinery); inputs X_t=a*E, X_s=b*E",
           "cases": []}
    for name, n, d, a, b, causal, g, rows in CASES:
        scale = f32_scale(d)
        r = structured_case(n, d, a, b, scale, causal, g)
        rows_out = list(range(n)) if rows is None else rows
        out["cases"].append({
            "name": name, "N": n, "d": d, "a": a, "b": b, "causal": causal, "g": g,
            "scale": scale, "lse_t": r["lse_t"], "lse_s": r["lse_s"], "row_kl": r["row_kl"],
            "loss": r["loss"], "dx_rows": rows_out, "dx": [r["dx"][i] for i in rows_out],
        })
    path = os.path.join(os.path.dirname(__file__), "closed_form.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
