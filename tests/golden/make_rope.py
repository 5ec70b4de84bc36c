"""Write tests/golden/rope_program.json: the paired sine / cosine program of
the rotary embedding as the oracle fits it.

Calls only the oracle.  "Fast Polynomial Transcendentals for LLMs", Appendix
B.2 (a D5 sine and a D6 cosine on the signed Q15 half-turn coordinate u, the
angle being pi u) with the fitting workflow of section 3.2: least squares on
Chebyshev nodes in FP64 with the endpoint values imposed (Eq. 8), every
coefficient rounded to BF16.  Also records the maximum error of the FP16
replay over every Q15 coordinate against sin(pi u) and cos(pi u).
Run from the repository root:  python tests/golden/make_rope.py
"""
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle as O  # noqa: E402


def main():
    s64, c64 = O.rope_fit()
    rp = O.rope_prog()
    phase = np.arange(65536, dtype=np.uint64) << 16
    sb, cb = O.rope_sincos(rp, phase)
    v = np.arange(65536)
    v = np.where(v >= 32768, v - 65536, v) / 32768.0
    es = float(np.max(np.abs(sb.view(np.float16).astype(np.float64) - np.sin(math.pi * v))))
    ec = float(np.max(np.abs(cb.view(np.float16).astype(np.float64) - np.cos(math.pi * v))))
    out = {"generator": "tests/golden/make_rope.py",
           "sin_fp64": [float(x) for x in s64], "cos_fp64": [float(x) for x in c64],
           "sin_bits": [int(b) for b in rp.sin_c], "cos_bits": [int(b) for b in rp.cos_c],
           "max_err_sin_f16": es, "max_err_cos_f16": ec}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_program.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
