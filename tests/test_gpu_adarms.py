"""Adaptive RMSNorm on the GPU against the oracle (FlashRT's fused_adarms /
gate_res_adarms kernels, in the reading s = R(r + g x), m = (s inv)(1 +
scale) + shift): dtype output within 1 ulp (fp32: rel 1e-5) except where
n (1 + scale) and the shift cancel (compare.check_modulated), the residual
stream bit for bit, FP8 codes within one step, the calibration amax within
rel 1e-5; over the small-row, wide-row and scalar kernels, with and without a
residual or a gate, and in every dtype."""
import numpy as np
import pytest
import torch

import compare as C
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mbt():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    import memory_bound_transformer_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def dev(bits, dtype, offset=0):
    if bits is None:
        return None
    flat = np.concatenate([np.zeros(offset, bits.dtype), bits.ravel()])
    return W.to_torch(flat, dtype, DEV)[offset:].view(bits.shape)


def host(t, dtype):
    torch.cuda.synchronize()
    return W.from_torch(t, dtype)


def _cell(**kw):
    base = dict(name="ada", config=96, cell=0, T=10, H=2048, dtype=W.BF16)
    base.update(kw)
    return W.AdaCell(**base)


CELLS = [
    _cell(name="pi05_decoder_S10_H2048", cell=1),
    _cell(name="bf16_H1024_T512", H=1024, T=512, cell=2),
    _cell(name="bf16_no_gate", gate=False, cell=3),
    _cell(name="bf16_no_residual", residual=False, gate=False, cell=4),
    _cell(name="f16_H2048", dtype=W.F16, cell=5),
    _cell(name="f32_H1024", dtype=W.F32, H=1024, cell=6),
    _cell(name="bf16_H256_small", H=256, T=33, cell=7),
    _cell(name="bf16_H16384_wide", H=16384, T=3, cell=8),
    _cell(name="bf16_H333_scalar", H=333, T=7, cell=9),
    _cell(name="f32_H8192_wide", dtype=W.F32, H=8192, T=4, cell=10),
]


def check(mbt, orc, cell, offset=0):
    i = cell.inputs()
    dt = cell.dtype
    x, r = dev(i["x"], dt, offset), dev(i["residual"], dt, offset)
    g, sc, sh = dev(i["gate"], dt, offset), dev(i["scale"], dt, offset), dev(i["shift"], dt, offset)
    # dtype output, in place
    mbt.adarms(x, r, g, sc, sh, cell.eps)
    xo, ro = orc.adarms(i["x"], i["residual"], i["gate"], i["scale"], i["shift"], cell.eps, dt)
    # magnitudes for the cancellation bound: a = n (1 + scale) from the
    # oracle's no-weight norm of the rounded sum, and the shift
    s_bits = ro if ro is not None else i["x"]
    n = W.bits_to_f32(orc.fused_add_rmsnorm(s_bits, None, None, cell.eps, 0, dt)[0], dt).astype(np.float64) \
        if dt != W.F32 else orc.fused_add_rmsnorm(s_bits, None, None, cell.eps, 0, dt)[0].astype(np.float64)
    f = (lambda b: W.bits_to_f32(b, dt).astype(np.float64)) if dt != W.F32 else \
        (lambda b: b.astype(np.float64))
    a_mag = np.abs(n * (1.0 + f(i["scale"])))
    st = C.check_modulated(host(x, dt), xo, a_mag, np.abs(f(i["shift"])) + 0 * a_mag, cell.H, dt,
                           label=f"{cell.name} out")
    if r is not None:
        C.check_bitwise(host(r, dt), ro, label=f"{cell.name} residual")
    # calibration and FP8
    cal = cell.calibration_inputs()
    amax_o = orc.adarms_amax(cal["x"], cal["residual"], i["gate"], i["scale"], i["shift"],
                             cell.eps, dt)
    amax_g = float(mbt.adarms_amax(dev(cal["x"], dt), dev(cal["residual"], dt), g, sc, sh,
                                   cell.eps).item())
    assert abs(amax_g - amax_o) <= 1e-5 * amax_o, f"amax {amax_g} vs {amax_o}"
    inv_scale = W.fp8_inv_scale(amax_o)
    x, r = dev(i["x"], dt, offset), dev(i["residual"], dt, offset)
    y = mbt.adarms_fp8(x, r, g, sc, sh, inv_scale, cell.eps)
    yo, ro8 = orc.adarms_fp8(i["x"], i["residual"], i["gate"], i["scale"], i["shift"], inv_scale,
                             cell.eps, dt)
    s8 = C.check_fp8(y.cpu().numpy(), yo, label=f"{cell.name} fp8")
    C.check_bitwise(host(x, dt), i["x"], label=f"{cell.name} x untouched by the FP8 form")
    if r is not None:
        C.check_bitwise(host(r, dt), ro8, label=f"{cell.name} residual (FP8 form)")
    print(f"{cell.name}: out {st} fp8 {s8}", flush=True)


@pytest.mark.parametrize("cell", CELLS, ids=lambda c: c.name)
def test_adarms(mbt, orc, cell):
    check(mbt, orc, cell)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_adarms_unaligned(mbt, orc, dtype):
    check(mbt, orc, _cell(name=f"unaligned_{dtype}", dtype=dtype, H=1024, T=5,
                          cell=20 + dtype), offset=1)


def test_adarms_identity_is_no_weight_norm(mbt):
    """scale = shift = 0, no residual: the no-weight residual norm, bit for
    bit (same kernels, weight path 1 + 0 and a zero shift)."""
    c = _cell(name="ident", residual=False, gate=False, H=2048, T=16, cell=30)
    i = c.inputs()
    zero = W.to_bits(np.full(c.H, 0.0), c.dtype)
    x1, x2 = dev(i["x"], c.dtype), dev(i["x"], c.dtype)
    mbt.adarms(x1, None, None, dev(zero, c.dtype), dev(zero, c.dtype), c.eps)
    mbt.fused_add_rmsnorm(x2, None, None, c.eps, 0)
    a, b = host(x1, c.dtype), host(x2, c.dtype)
    # +0 shift turns a -0 result into +0; compare values, then bits elsewhere
    nz = W.bits_to_f32(b, c.dtype) != 0
    assert np.array_equal(a[nz], b[nz])
    assert np.all(W.bits_to_f32(a, c.dtype)[~nz] == 0)
