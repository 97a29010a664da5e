"""Every launch shape of the gated activation against the oracle, on the GPU.

The host picks, from the half width d and the row count T: for 16-bit
inputs at narrow launches, half-chunk lanes (up to 1024 waves for a dtype
output or the calibration pass, 8192 for FP8 output); otherwise one or,
from 400k chunks per launch, two 16-byte chunks per lane -- with two, the
flat-group kernel where a row is a whole number (at least two) of
256-chunk groups; and the scalar kernel for odd widths.  The cells below are
chosen by (d, T) to land on each, in bf16, fp16 and fp32, SiLU and GELU-tanh
in turn, with a dtype output and with FP8 output (after its calibration
pass).  The names follow those thresholds; a name that no longer matches
after a retuning still leaves a valid parity case."""
import pytest

import workloads as W
from test_gpu_parity import check_act_cell, mbt, orc  # noqa: F401

pytestmark = pytest.mark.gpu

_DT = {W.BF16: "bf16", W.F16: "f16", W.F32: "f32"}

# (dtype, d, T, fp8, intended shape)
_SHAPES = [
    (W.BF16, 1024, 100, False, "half"), (W.BF16, 10240, 150, True, "half"),
    (W.BF16, 10240, 30, False, "vec_u1"), (W.BF16, 10240, 250, True, "vec_u1"),
    (W.BF16, 2400, 2000, False, "vec_u2"), (W.BF16, 2400, 2000, True, "vec_u2"),
    (W.BF16, 10240, 400, False, "flat"), (W.BF16, 10240, 400, True, "flat"),
    (W.BF16, 37, 64, False, "scalar"), (W.BF16, 37, 64, True, "scalar"),
    (W.F16, 10240, 150, True, "half"), (W.F16, 10240, 400, False, "flat"),
    (W.F16, 2400, 2000, True, "vec_u2"),
    (W.F32, 4096, 50, False, "vec_u1"), (W.F32, 4096, 50, True, "vec_u1"),
    (W.F32, 1200, 2000, False, "vec_u2"), (W.F32, 1200, 2000, True, "vec_u2"),
    (W.F32, 4096, 500, False, "flat"), (W.F32, 4096, 500, True, "flat"),
    (W.F32, 37, 64, True, "scalar"),
]


def _cells():
    return [W.ActCell(name=f"ashape_{_DT[dt]}_d{d}_T{T}_{'fp8' if f8 else 'dt'}_{shape}",
                      config=84, cell=n, T=T, d=d, act=W.SILU if n % 2 == 0 else W.GELU_TANH,
                      dtype=dt, fp8=f8)
            for n, (dt, d, T, f8, shape) in enumerate(_SHAPES)]


@pytest.mark.parametrize("cell", _cells(), ids=lambda c: c.name)
def test_act_launch_shape(mbt, orc, cell):
    check_act_cell(mbt, orc, cell)
