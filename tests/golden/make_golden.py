"""Write tests/golden/oracle_digests.json from the oracle alone.

Run from the repository root: ``python tests/golden/make_golden.py``. It calls only
``oracle/`` (and the seeded input generators in ``workloads/``); no value here comes
from the HIP library. The digests pin the oracle against accidental drift: a change
to its arithmetic must regenerate this file, and the commit doing so must name the
passage of the pages (or the reading of it) that justifies the change.
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import nvfp4_oracle as O  # noqa: E402
from workloads import make  # noqa: E402

CASES = ["tiny", "attn_out", "qkv", "odd_m17"]
ROWS = 128


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def compute():
    out = {}
    for name in CASES:
        d = make(name).generate()
        x, w = d["x"], d["w"]
        ags = O.global_scale(x)
        wgs = O.global_scale(w)
        xp, xs = O.quantize(x[:ROWS], ags)
        wp, ws = O.quantize(w[:ROWS], wgs)
        ref, _ = O.gemm_ref(xp[:8], xs[:8], ags, wp[:8], ws[:8], wgs, with_abs=False)
        out[name] = {
            "a_global_scale_bits": int(np.float32(ags).view(np.uint32)),
            "w_global_scale_bits": int(np.float32(wgs).view(np.uint32)),
            "act_quant_sha256": digest(xp, xs),
            "w_quant_sha256": digest(wp, ws),
            "gemm_corner_8x8": [float(v) for v in ref.reshape(-1)],
        }
    return out


if __name__ == "__main__":
    path = os.path.join(HERE, "oracle_digests.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", path)
