"""Write tests/golden/oracle_digests.json: SHA-256 digests of the oracle's
outputs on the small configuration cells (seeded synthetic inputs).

The file is a regression snapshot of the oracle, not a pin: it only changes
when the oracle's arithmetic changes on purpose.  This script calls nothing
but oracle/ and the shared input generators.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(HERE, "oracle_digests.json")


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def small_cells():
    cells = list(W.config1_cells())
    cells += [c for c in W.config2_cells() if c.T <= 8]
    cells += [c for c in W.config4_cells() if c.T <= 16]
    cells += [c for c in W.config5_cells() if c.T == 1]
    return cells


def run_cell(orc, c):
    if isinstance(c, W.PrologueCell):
        i = c.inputs()
        qo, ko = orc.qknorm_rope(i["q"], i["k"], i["w_q"], i["w_k"], i["cos_sin"], i["pos"],
                                 c.rot, c.eps, c.weight_offset, c.layout, c.dtype)
        return digest(qo, ko)
    if isinstance(c, W.NormCell):
        i = c.inputs()
        if c.fp8:
            cal = c.calibration_inputs()
            amax = orc.fused_add_rmsnorm_amax(cal["x"], cal["residual"], i["w"], c.eps,
                                              c.weight_offset, c.dtype)
            y, r = orc.fused_add_rmsnorm_fp8(i["x"], i["residual"], i["w"],
                                             W.fp8_inv_scale(amax), c.eps, c.weight_offset,
                                             c.dtype)
            return digest(y, r)
        x, r = orc.fused_add_rmsnorm(i["x"], i["residual"], i["w"], c.eps, c.weight_offset,
                                     c.dtype)
        return digest(x, r)
    i = c.inputs()
    if c.fp8:
        amax = orc.gated_act_amax(c.calibration_inputs()["gate_up"], c.act, c.dtype)
        return digest(orc.gated_act_fp8(i["gate_up"], W.fp8_inv_scale(amax), c.act, c.dtype))
    return digest(orc.gated_act(i["gate_up"], c.act, c.dtype))


def compute():
    orc = oracle.default()
    return {c.name: run_cell(orc, c) for c in small_cells()}


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(compute(), f, indent=1, sort_keys=True)
    print(OUT)
