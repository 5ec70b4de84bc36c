"""Write tests/golden/programs.json: the deployed programs as the oracle's
fitter and (Li, Lc) search select them.

Calls only the oracle.  The selection follows "Fast Polynomial
Transcendentals for LLMs", section 3.2 (Eq. 8 fit, BF16 rounding, replay,
8,000-point objective, Lc <= Li + 1) with the printed Table 2 bounds as the
restriction (the upper end of each printed value's rounding interval).
Run from the repository root:  python tests/golden/make_programs.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle as O  # noqa: E402

SIG_LC = 5.28125   # the configured runtime clamp of the D3 sigmoid (Fig. 2's Lc)


def entry(name, p, obj, met, bound):
    return {"name": name, "func": int(p.func), "deriv": int(p.deriv),
            "degree": int(p.degree), "Li": p.Li, "Lc": p.Lc,
            "coeff_bits": [int(b) for b in p.coeff_bits()],
            "search_objective": obj, "table2_metric": met,
            "table2_bound": bound}


def main():
    out = []
    p, obj, met = O.search(O.SIGMOID, 0, 3, Lc_fixed=SIG_LC, bound=5.445e-3)
    out.append(entry("sigmoid_fwd_d3", p, obj, met, 5.445e-3))
    silu = O.make_prog(O.SILU, 0, 3, p.Li, p.Lc)
    out.append(entry("silu_fwd_d3", silu, O.search_objective(silu)[0],
                     O.table2_metric(silu), 21.745e-3))
    p, obj, met = O.search(O.TANH, 0, 4, bound=9.615e-3)
    out.append(entry("tanh_fwd_d4", p, obj, met, 9.615e-3))
    p, obj, met = O.search(O.GELU, 0, 5, bound=1.065e-3)
    out.append(entry("gelu_fwd_d5", p, obj, met, 1.065e-3))
    p, obj, met = O.search(O.SIGMOID, 1, 4, bound=4.465e-3)
    out.append(entry("sigmoid_bwd_d4", p, obj, met, 4.465e-3))
    p, obj, met = O.search(O.TANH, 1, 4)
    out.append(entry("tanh_bwd_d4", p, obj, met, None))
    # centered-odd derivative fits (Eq. 9): SiLU' D3 as in the B1 probe, GELU' at
    # the forward GELU's degree D5 (its degree is not printed; D5 also has the
    # lowest search objective among D3-D6)
    p, obj, met = O.search(O.SILU, 1, 3)
    out.append(entry("silu_bwd_d3", p, obj, met, None))
    p, obj, met = O.search(O.GELU, 1, 5)
    out.append(entry("gelu_bwd_d5", p, obj, met, None))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "programs.json")
    with open(path, "w") as f:
        json.dump({"generator": "tests/golden/make_programs.py", "programs": out}, f,
                  indent=1)
        f.write("\n")
    for e in out:
        print(e["name"], e["Li"], e["Lc"], [hex(b) for b in e["coeff_bits"]],
              f"{e['table2_metric']:.4e}")


if __name__ == "__main__":
    main()
