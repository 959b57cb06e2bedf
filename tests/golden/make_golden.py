"""Writes tests/golden/oracle_regression.json: the fp64 oracle's outputs on a
small seeded case, so that any later change to the oracle's arithmetic shows
up as a failing regression test and has to be made deliberately.

Calls only oracle/ (and numpy for the seeded inputs).  Run from the repo root:
    python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import kla_chunkwise, kla_recurrence  # noqa: E402


def case():
    rng = np.random.default_rng(20261202)
    L, dk, dv = 23, 4, 3
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk)) * np.exp(0.5 * rng.standard_normal(L))[:, None]
    v = rng.standard_normal((L, dv))
    g = -np.log1p(np.exp(rng.standard_normal(L)))
    eta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    return dict(q=q, k=k, v=v, g=g, eta=eta, eps=1e-3, S0=S0)


def main():
    c = case()
    o, S = kla_recurrence(c["q"], c["k"], c["v"], c["g"], c["eta"], c["eps"], c["S0"])
    oc, Sc = kla_chunkwise(c["q"], c["k"], c["v"], c["g"], c["eta"], c["eps"], c["S0"], 8)
    out = {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
    out.update(o=o.tolist(), S=S.tolist(), o_chunk8=oc.tolist(), S_chunk8=Sc.tolist(),
               note="written by tests/golden/make_golden.py from oracle/ only")
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
