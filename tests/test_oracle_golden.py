"""The oracle reproduces its recorded values bit for bit.

``tests/golden/oracle_B1-H1-N256-d64.json`` was written by
``tests/golden/make_golden.py``, which calls only the oracle; a change in the
oracle's arithmetic shows up here and must be justified.
"""
import json
import os

import numpy as np

import oracle
from attention_attn_fwd_08_amd.inputs import WORKLOADS, workload_inputs


def test_oracle_matches_recorded_rows():
    with open(os.path.join(os.path.dirname(__file__), "golden", "oracle_B1-H1-N256-d64.json")) as f:
        rec = json.load(f)
    w = WORKLOADS["B1-H1-N256-d64"]
    q, k, v = workload_inputs(w)
    for key, causal in (("non_causal", False), ("causal", True)):
        r = rec[key]
        o, lse = oracle.attention_rows(q, k, v, causal, w.scale, r["rows"])
        assert np.array_equal(o, np.array([[float.fromhex(x) for x in row] for row in r["o"]]))
        assert np.array_equal(lse, np.array([float.fromhex(x) for x in r["lse"]]))
