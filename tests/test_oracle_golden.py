"""The oracle still reproduces its stored outputs on the seeded one-layer workload
(tests/golden/oracle_tiny.json, written by tests/golden/make_golden.py from
oracle/ alone).  Guards against silent drift of the oracle's arithmetic."""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_golden  # noqa: E402


def test_oracle_matches_stored_golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")) as f:
        g = json.load(f)
    case, h, kp, vp = make_golden.tiny_outputs()
    assert case["ctx_lens"].tolist() == g["ctx_lens"]
    k_new, v_new = make_golden.appended(case, kp, vp)
    # stored values are f16; a different BLAS may flip the last bit of a few
    np.testing.assert_allclose(h.astype(np.float64).ravel(), g["hidden_out"], atol=2e-3, rtol=2e-3)
    np.testing.assert_allclose(k_new.astype(np.float64).ravel(), g["k_appended"], atol=2e-3, rtol=2e-3)
    np.testing.assert_allclose(v_new.astype(np.float64).ravel(), g["v_appended"], atol=2e-3, rtol=2e-3)
