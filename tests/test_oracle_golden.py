"""The oracle still produces the digests recorded by tests/golden/make_golden.py."""
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_recorded_digests():
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(HERE, "golden", "oracle_digests.json")) as f:
        want = json.load(f)
    got = mod.compute()
    assert set(got) == set(want)
    for name in want:
        for key in ("a_global_scale_bits", "w_global_scale_bits", "act_quant_sha256",
                    "w_quant_sha256"):
            assert got[name][key] == want[name][key], (name, key)
        assert np.array_equal(np.array(got[name]["gemm_corner_8x8"]),
                              np.array(want[name]["gemm_corner_8x8"])), name
