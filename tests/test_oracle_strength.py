"""Strength control of the oracle's pins.

In the spirit of the strength control in ninfer PR #273 ("Verification":
scaling the rotation by 1.000001 must make the exact comparisons fail), each
case below builds a copy of the oracle with one planted mistake (compiled in
through MBT_ORACLE_MUTATION, on the CPU) and requires that at least one pin
rejects it.  The unmutated build must pass every pin (test_oracle_pins.py).
"""
import os

import pytest

import oracle
from oracle import build as obuild
import pins

MUTATIONS = {
    1: "rotation scaled by 1.000001 (the PR's strength control)",
    2: "eps dropped from the mean square",
    3: "prologue mean taken over rot_dim instead of head_dim",
    4: "sin sign flipped",
    5: "rotate-half partner off by one",
    6: "weight offset (1 + w) ignored",
    7: "GELU cubic coefficient 0.0447 instead of 0.044715",
    8: "e4m3fn rounding truncates",
    9: "bf16 rounding truncates",
    10: "residual sum normalised before rounding",
    11: "key heads normalised with the query weight",
    12: "positions past the cache clamped to its last row",
    13: "a missing weight read as 1 + 1 (no-weight norm doubled)",
    14: "single-rounding prologue rounds the norm result before rotating",
    15: "adaptive norm scales by scale instead of 1 + scale",
    16: "adaptive norm ignores the residual gate",
    17: "norm FP8 epilogue quantizes the dtype-rounded value",
    18: "norm calibration amax of the dtype-rounded value",
    19: "adaptive norm FP8 epilogue quantizes the dtype-rounded value",
    20: "adaptive norm calibration amax of the dtype-rounded value",
    21: "activation FP8 epilogue quantizes the dtype-rounded value",
    22: "activation calibration amax of the dtype-rounded value",
    23: "gate and up halves of gate_up swapped",
    24: "fp16 rounding truncates (normal range)",
    25: "interleaved pairs take cos/sin at the channel index 2i",
    26: "the cache's last row (max_pos - 1) treated as outside",
    27: "SiLU takes the sigmoid of -g",
    28: "mean square divided by D - 1",
    29: "e4m3fn overflow gives NaN instead of saturating",
    30: "calibration amax takes the signed maximum",
    31: "rotate-half o_b subtracts the partner term",
    32: "negative positions wrap around the cache",
    33: "eps added outside the square root",
    34: "residual stream not written back",
    35: "activation rounded to the dtype before the product with u",
    36: "norm rounds x * inv to the dtype before the weight",
}

# fast pins first: most mutations are caught within a second
ORDER = sorted(pins.ALL_PINS, key=lambda f: f in (pins.pin_act_exhaustive_bf16,
                                                  pins.pin_rmsnorm_bruteforce))


@pytest.mark.parametrize("mutation", sorted(MUTATIONS), ids=lambda m: f"m{m}")
def test_planted_mistake_is_caught(tmp_path, mutation):
    lib = obuild.build(out=str(tmp_path / f"liboracle_m{mutation}.so"), mutation=mutation)
    orc = oracle.Oracle(lib)
    caught = []
    for pin in ORDER:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches mutation {mutation}: {MUTATIONS[mutation]}"


def test_rotation_nudge_fails_exact_checks(tmp_path):
    """The 1e-6 nudge is far below one bf16 ulp; only exact comparisons see
    it.  It must fail the bitwise closed forms and the fp32 complex pin."""
    orc = oracle.Oracle(obuild.build(out=str(tmp_path / "m1.so"), mutation=1))
    for pin in (pins.pin_rope_closed_forms, pins.pin_rope_complex):
        with pytest.raises(AssertionError):
            pin(orc)
    assert os.path.exists(oracle.DEFAULT_LIB)
