"""Every launch shape of the dense prologue against the oracle, on the GPU.

The host picks the chunks per lane (C = 1, 2, 4) and, for C >= 2, the load
order (0: early cos/sin; 2: cos/sin behind a block barrier after the
reduction; 1: whole-block weight staging) from the launch's wave count, and
splits a launch of one to one and a half resident rounds into two.  The
configuration cells reach most of these shapes in bf16 and fp16 only; the
cells below pick token counts that land in each band for all three dtypes
and both pairings at head_dim 256, (Q, K) = (24, 4), so every compiled
instantiation of the dense kernel meets the oracle.  The bands named in the
cell names follow the launch thresholds (one chunk per lane up to 2560
waves, 6000 for interleaved pairs; order 2 from 2560 waves, order 1 from
5000, one round up to 8192); a shape name that no longer matches them after
a retuning still leaves a valid parity case.  Tokens 1 and 3 sit outside
the cache (positions -1 and max_pos), and every other cell runs in place."""
import pytest

import workloads as W
from test_gpu_parity import check_prologue_cell, mbt, orc  # noqa: F401

pytestmark = pytest.mark.gpu

_DT = {W.BF16: "bf16", W.F16: "f16", W.F32: "f32"}

# (dtype, layout, T, intended shape)
_SHAPES = [
    # rotate-half, rot_dim 64: 16-bit rows are 32 chunks, fp32 rows 64
    *[(dt, W.ROTATE_HALF, T, s) for dt in (W.BF16, W.F16) for T, s in (
        (100, "c1"), (300, "c2_o0"), (600, "c4_o0"), (1000, "c4_o2"), (2000, "c4_o1"),
        (2600, "split_c4_o2"))],
    *[(W.F32, W.ROTATE_HALF, T, s) for T, s in (
        (50, "c1"), (150, "c2_o0"), (300, "c4_o0"), (600, "c4_o2"), (1000, "c4_o1"),
        (1300, "split_c4_o2"))],
    # interleaved, full rotary (rot_dim 256)
    *[(dt, W.INTERLEAVED, T, s) for dt in (W.BF16, W.F16) for T, s in (
        (400, "c1"), (500, "c2_o2"), (1000, "c2_o1"), (1300, "c4_o2"), (2000, "c4_o1"))],
    *[(W.F32, W.INTERLEAVED, T, s) for T, s in (
        (200, "c1"), (300, "c2_o2"), (500, "c2_o1"), (700, "c4_o2"), (1100, "c4_o1"))],
]


def _cells():
    out = []
    for n, (dt, layout, T, shape) in enumerate(_SHAPES):
        rot = 64 if layout == W.ROTATE_HALF else 256
        lay = "half" if layout == W.ROTATE_HALF else "inter"
        out.append(W.PrologueCell(
            name=f"shape_{_DT[dt]}_{lay}_T{T}_{shape}", config=87, cell=n, T=T, Q=24, K=4,
            D=256, rot=rot, theta=1e7, layout=layout, dtype=dt, weight_offset=1, w_mean=0.0,
            w_std=0.05, x_std=2.0, max_pos=T + 8, positions="arange",
            outside=((1, -1), (3, T + 8)), in_place=(n % 2 == 1)))
    return out


@pytest.mark.parametrize("cell", _cells(), ids=lambda c: c.name)
def test_prologue_launch_shape(mbt, orc, cell):
    check_prologue_cell(mbt, orc, cell, in_place=cell.in_place)


# The general kernel (token strides, slot table and value rows, the
# single-rounding flag) has the same launch shapes; its cells in bf16 and
# fp32 go through the strided-view and KV-cache checks of
# test_gpu_prologue_ex (against the oracle, and bit for bit against the
# dense op), the single-rounding flag on every other cell.
import test_gpu_prologue_ex as ex  # noqa: E402

_GEN = [c for c in _cells() if c.dtype in (W.BF16, W.F32)]


@pytest.mark.parametrize("cell", _GEN, ids=lambda c: c.name)
def test_strided_launch_shape(mbt, orc, cell):
    ex.test_strided_views(mbt, orc, cell, round_once=cell.cell % 2 == 0, pad=0)


@pytest.mark.parametrize("cell", _GEN, ids=lambda c: c.name)
def test_cache_launch_shape(mbt, orc, cell):
    ex.test_qkv_cache(mbt, orc, cell, round_once=cell.cell % 2 == 1)
