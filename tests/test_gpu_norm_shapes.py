"""Every launch shape of the residual norm and the adaptive norm against the
oracle, on the GPU.

The host picks, from the row width H and the row count T: rows of at most
64 chunks as G-lane segments (G = 4 ... 64); for 16-bit rows of at most
four 64-chunk groups at narrow launches, half-chunk lanes; otherwise the
wide kernel with WPR waves per row (one per 64-chunk group while the launch
is narrow, capped at 16, else as few as six chunks per lane allow) and NCH
chunks per lane (1 ... 6), several rows per block when WPR is 1, 2 or 4; and
the scalar kernel for odd widths.  The configuration cells reach a few of
these; the cells below are chosen by (H, T) to land on each, in bf16 and
fp32 (fp16 where it has its own half-chunk path), alternating dtype and FP8
output (with its calibration pass), with and without a residual or a
weight.  The names follow the launch thresholds (half-chunk lanes up to
4096 waves; the narrow wide-kernel shape up to 8192 rows x groups, 5000
where a row's groups do not split evenly over four SIMDs); a name that no
longer matches after a retuning still leaves a valid parity case."""
import pytest

import workloads as W
from test_gpu_parity import check_norm_cell, mbt, orc  # noqa: F401
import test_gpu_adarms as ada

pytestmark = pytest.mark.gpu

_DT = {W.BF16: "bf16", W.F16: "f16", W.F32: "f32"}

# (dtype, H, T, intended shape)
_SHAPES = [
    *[(W.BF16, H, 40, f"small_g{g}") for H, g in ((32, 4), (64, 8), (128, 16), (256, 32),
                                                    (512, 64))],
    (W.BF16, 1024, 300, "half_w4"), (W.BF16, 2048, 100, "half_w8"),
    (W.BF16, 2560, 100, "wide_wpr5_nch1"), (W.BF16, 4096, 100, "wide_wpr8_nch1"),
    (W.BF16, 1024, 4096, "wide_wpr1_nch2"), (W.BF16, 1536, 1700, "wide_wpr1_nch3"),
    (W.BF16, 2048, 2048, "wide_wpr1_nch4"), (W.BF16, 4096, 1024, "wide_wpr2_nch4"),
    (W.BF16, 2560, 1000, "wide_wpr1_nch5"), (W.BF16, 3072, 900, "wide_wpr1_nch6"),
    (W.BF16, 8192, 512, "wide_wpr3_nch6"), (W.BF16, 12288, 10, "wide_wpr16_nch2"),
    (W.BF16, 333, 50, "scalar"),
    (W.F16, 1024, 300, "half_w4"), (W.F16, 2048, 2048, "wide_wpr1_nch4"),
    (W.F16, 3072, 900, "wide_wpr1_nch6"),
    *[(W.F32, H, 40, f"small_g{g}") for H, g in ((16, 4), (32, 8), (64, 16), (128, 32),
                                                   (256, 64))],
    (W.F32, 1280, 100, "wide_wpr5_nch1"), (W.F32, 512, 4096, "wide_wpr1_nch2"),
    (W.F32, 768, 1700, "wide_wpr1_nch3"), (W.F32, 1024, 2048, "wide_wpr1_nch4"),
    (W.F32, 2048, 1024, "wide_wpr2_nch4"), (W.F32, 1280, 1000, "wide_wpr1_nch5"),
    (W.F32, 1536, 900, "wide_wpr1_nch6"), (W.F32, 4096, 512, "wide_wpr3_nch6"),
    (W.F32, 6144, 10, "wide_wpr16_nch2"), (W.F32, 37, 50, "scalar"),
]


def _norm_cells():
    out = []
    for n, (dt, H, T, shape) in enumerate(_SHAPES):
        weight = n % 5 != 4
        delta = (n % 2) if weight else 0
        out.append(W.NormCell(
            name=f"nshape_{_DT[dt]}_H{H}_T{T}_{shape}", config=86, cell=n, T=T, H=H,
            dtype=dt, weight_offset=delta, w_mean=0.0 if delta else 1.0, w_std=0.05,
            residual=n % 4 != 3, fp8=n % 2 == 1, weight=weight))
    return out


@pytest.mark.parametrize("cell", _norm_cells(), ids=lambda c: c.name)
def test_norm_launch_shape(mbt, orc, cell):
    check_norm_cell(mbt, orc, cell)


# The adaptive norm takes the small and wide kernels (no half-chunk lanes):
# its in-place, FP8 and calibration forms at each wide shape.
_ADA = [(W.BF16, 2048, 100, "wide_wpr4_nch1"), (W.BF16, 1024, 4096, "wide_wpr1_nch2"),
        (W.BF16, 1536, 1700, "wide_wpr1_nch3"), (W.BF16, 2048, 2048, "wide_wpr1_nch4"),
        (W.BF16, 4096, 1024, "wide_wpr2_nch4"), (W.BF16, 2560, 1000, "wide_wpr1_nch5"),
        (W.BF16, 3072, 900, "wide_wpr1_nch6"), (W.BF16, 8192, 512, "wide_wpr3_nch6"),
        (W.F32, 768, 1700, "wide_wpr1_nch3"), (W.F32, 1536, 900, "wide_wpr1_nch6")]


def _ada_cells():
    return [W.AdaCell(name=f"ashape_{_DT[dt]}_H{H}_T{T}_{shape}", config=85, cell=n, T=T, H=H,
                      dtype=dt, residual=n % 3 != 2, gate=n % 3 == 0)
            for n, (dt, H, T, shape) in enumerate(_ADA)]


@pytest.mark.parametrize("cell", _ada_cells(), ids=lambda c: c.name)
def test_adarms_launch_shape(mbt, orc, cell):
    ada.check(mbt, orc, cell)
