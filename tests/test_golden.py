"""Oracle against hand-worked values (tests/golden/).  CPU only."""

import json
import os

import numpy as np

from oracle import recurrent_fwd

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_worked_example_d2():
    """Three tokens of the gated delta rule worked by hand (the fixture holds
    the derivation): pins the decay, the delta update, the output taken on the
    updated state and the stored state's transpose."""
    with open(os.path.join(GOLDEN, "worked_example_d2.json")) as f:
        case = json.load(f)
    x = case["inputs"]
    o, hT = recurrent_fwd(np.array(x["q"]), np.array(x["k"]), np.array(x["v"]),
                          np.array(x["beta"]), np.log(np.array(x["alpha"])),
                          np.array(x["cu_seqlens"]), qk_l2norm=False)
    tol = case["tolerance"]
    np.testing.assert_allclose(o, np.array(case["expected"]["o"]), rtol=0, atol=tol)
    np.testing.assert_allclose(hT, np.array(case["expected"]["hT"]), rtol=0, atol=tol)
