"""Regression guard: the oracle still reproduces the stored outputs written by
tests/golden/make_golden.py (which calls only oracle/).  A deliberate change to
the oracle's arithmetic regenerates the file and says why in its commit."""

import json
import os

import numpy as np

from oracle import kla_chunkwise, kla_recurrence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")


def test_oracle_reproduces_stored_outputs():
    with open(GOLDEN) as f:
        d = json.load(f)
    a = {k: np.array(d[k]) for k in ("q", "k", "v", "g", "eta", "S0")}
    o, S = kla_recurrence(a["q"], a["k"], a["v"], a["g"], a["eta"], d["eps"], a["S0"])
    np.testing.assert_allclose(o, np.array(d["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S, np.array(d["S"]), rtol=0, atol=1e-14)
    oc, Sc = kla_chunkwise(a["q"], a["k"], a["v"], a["g"], a["eta"], d["eps"], a["S0"], 8)
    np.testing.assert_allclose(oc, np.array(d["o_chunk8"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sc, np.array(d["S_chunk8"]), rtol=0, atol=1e-13)
