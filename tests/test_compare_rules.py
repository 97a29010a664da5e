"""The comparison rules the GPU parity tests use (tests/compare.py), on the
CPU: each accepts what the numerics contract allows and rejects what it does
not.  The "GPU" side is a copy of an oracle result with a deviation planted
on the host, so no kernel runs here."""
import numpy as np
import pytest

import compare as C
import oracle
import workloads as W

BF16, F16, F32 = W.BF16, W.F16, W.F32


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _bump(bits, i, k):
    """bits with element i moved k steps away from zero (same sign)."""
    out = np.array(bits, copy=True)
    flat = out.reshape(-1)
    flat[i] = flat[i] + k
    return out


def _inputs(dtype, layout, T=4, H=3, D=64):
    g = np.random.default_rng([31, dtype, layout])
    q = W.to_bits(g.standard_normal((T, H, D)) * 2.0, dtype)
    k = W.to_bits(g.standard_normal((T, 1, D)) * 2.0, dtype)
    w = W.to_bits(g.standard_normal(D) * 0.05, dtype)
    return q, k, w


def _prologue(orc, dtype, layout=W.ROTATE_HALF, rot=64, pos=(3, 17, 40, 63)):
    q, k, w = _inputs(dtype, layout)
    T, H, D = q.shape
    cs = W.rope_cache(64, rot, 1e4)
    pos = np.array(pos, np.int64)
    qo, _ = orc.qknorm_rope(q, k, w, w, cs, pos, rot, 1e-6, 1, layout, dtype)
    n = orc.rmsnorm_rows(q.reshape(T * H, D), w, 1e-6, 1, dtype).reshape(T, H, D)
    return qo, n, cs, pos, rot


def _steps_within(bits, i, dtype, limit):
    """The largest k (<= 4096) such that moving element i k steps away from
    zero changes its value by at most `limit`."""
    v0 = float(W.bits_to_f32(bits.reshape(-1)[i:i + 1], dtype)[0])
    k = 0
    while k < 4096:
        v = float(W.bits_to_f32(_bump(bits, i, k + 1).reshape(-1)[i:i + 1], dtype)[0])
        if not np.isfinite(v) or abs(v - v0) > limit:
            break
        k += 1
    return k


def test_ulp16_distance_orders_across_zero():
    assert int(C.ulp16_dist(0x0000, 0x8000)) == 0            # +0 and -0
    assert int(C.ulp16_dist(0x3F80, 0x3F81)) == 1            # bf16 1.0 and its successor
    assert int(C.ulp16_dist(0x0001, 0x8001)) == 2            # +-least subnormal
    assert int(C.ulp16_dist(0xBF80, 0xBF82)) == 2


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_values_rule(dtype):
    g = np.random.default_rng(3)
    ora = W.to_bits(g.standard_normal(4000), dtype)
    assert C.check_values(ora.copy(), ora, dtype)["differ"] == 0
    assert C.check_values(_bump(ora, 10, 1), ora, dtype)["differ"] == 1
    with pytest.raises(AssertionError, match="max ulp 2"):
        C.check_values(_bump(ora, 10, 2), ora, dtype)
    # one step everywhere is a systematic rounding error, not noise
    many = ora.copy()
    many[::50] += 1                                           # 80 of 4000 = 2 %
    with pytest.raises(AssertionError, match="systematic"):
        C.check_values(many, ora, dtype)


@pytest.mark.parametrize("dtype", [BF16, F16, F32])
def test_values_rule_nan_and_inf(dtype):
    vals = np.array([1.0, -2.5, np.inf, -np.inf, np.nan, 0.0], np.float32)
    ora = vals if dtype == F32 else W.to_bits(vals, dtype)
    C.check_values(ora.copy(), ora, dtype)
    # a NaN of the other sign or another payload is still a NaN
    other = ora.copy()
    if dtype == F32:
        other[4] = np.array([0xFFC00001], np.uint32).view(np.float32)[0]
    else:
        other[4] = 0xFF81 if dtype == BF16 else 0xFC01
    C.check_values(other, ora, dtype)
    # a NaN where the oracle has a number, and a number where it has a NaN
    for i, v in ((0, np.nan), (4, 1.0)):
        g = vals.copy()
        g[i] = v
        g = g if dtype == F32 else W.to_bits(g, dtype)
        with pytest.raises(AssertionError, match="NaN on one side"):
            C.check_values(g, ora, dtype)
    # an infinity where the oracle has a finite value, or the other infinity
    for i, v in ((1, np.inf), (2, -np.inf)):
        g = vals.copy()
        g[i] = v
        g = g if dtype == F32 else W.to_bits(g, dtype)
        with pytest.raises(AssertionError):
            C.check_values(g, ora, dtype)


def test_values_rule_fp32():
    ora = np.linspace(-3.0, 3.0, 1001, dtype=np.float32)
    near = (ora.astype(np.float64) * (1 + 0.9e-5)).astype(np.float32)
    C.check_values(near, ora, F32)
    far = (ora.astype(np.float64) * (1 + 1.5e-5)).astype(np.float32)
    far[ora == 0] = 0
    with pytest.raises(AssertionError, match="beyond rel 1e-5"):
        C.check_values(far, ora, F32)


@pytest.mark.parametrize("layout", [W.ROTATE_HALF, W.INTERLEAVED])
def test_prologue_rule(orc, layout):
    qo, n, cs, pos, rot = _prologue(orc, BF16, layout)
    assert C.check_prologue(qo.copy(), qo, n, cs, pos, rot, layout, BF16)["differ"] == 0
    T, H, D = qo.shape
    # a channel past rot_dim is not rotated: two steps there always fail
    qo_p, n_p, cs_p, pos_p, rot_p = _prologue(orc, BF16, layout, rot=32)
    with pytest.raises(AssertionError, match="beyond tolerance"):
        C.check_prologue(_bump(qo_p, D - 1, 2), qo_p, n_p, cs_p, pos_p, rot_p, layout, BF16)
    # a rotated output that cancelled: a one-step change in its inputs moves
    # it by (|c| + |s|) ulp(n), many of its own steps.  Take the element
    # where that allowance is widest, in units of the output's own step.
    ch = np.tile(np.arange(D), T * H)
    part = C._partner(D, rot, layout)
    half = rot // 2
    j = np.where(ch < half, ch, ch - half) if layout == W.ROTATE_HALF else ch >> 1
    j = np.clip(j, 0, half - 1)
    p = np.repeat(pos, H * D)
    c, s = cs[p, j].astype(np.float64), cs[p, half + j].astype(np.float64)
    sp_n = C.spacing16(n.reshape(-1), BF16)
    sp_np = C.spacing16(n.reshape(-1, D)[:, part].reshape(-1), BF16)
    sp_o = C.spacing16(qo.reshape(-1), BF16)
    allow = (np.abs(c) + np.abs(s)) * np.maximum(sp_n, sp_np) + sp_o
    i = int(np.argmax(allow / sp_o))
    k_in = _steps_within(qo, i, BF16, 0.9 * allow[i])   # inside the allowance
    assert k_in >= 3, "no cancelled output in this draw; the case would prove nothing"
    r = C.check_prologue(_bump(qo, i, k_in), qo, n, cs, pos, rot, layout, BF16)
    assert r["escapes"] == 1 and r["max_ulp"] == k_in
    k_out = _steps_within(qo, i, BF16, 1.1 * allow[i]) + 1   # past it
    with pytest.raises(AssertionError, match="beyond tolerance"):
        C.check_prologue(_bump(qo, i, k_out), qo, n, cs, pos, rot, layout, BF16)
    # the same element with its token outside the cache is not rotated, so
    # the same change has no allowance
    out_pos = np.where(pos == p[i], 10_000, pos)
    qo2, n2, cs2, pos2, _ = _prologue(orc, BF16, layout, pos=tuple(out_pos))
    with pytest.raises(AssertionError, match="beyond tolerance"):
        C.check_prologue(_bump(qo2, i, 3), qo2, n2, cs2, pos2, rot, layout, BF16)


def test_prologue_rule_fp32(orc):
    qo, n, cs, pos, rot = _prologue(orc, F32)
    C.check_prologue(qo.copy(), qo, n, cs, pos, rot, W.ROTATE_HALF, F32)
    D = qo.shape[-1]
    nf = n.reshape(-1, D).astype(np.float64)
    pair = np.hypot(nf, nf[:, C._partner(D, rot, W.ROTATE_HALF)]).reshape(-1)
    scale = np.maximum(np.abs(qo.reshape(-1).astype(np.float64)), pair)
    for rel, ok in ((0.8e-5, True), (2e-5, False)):
        g = qo.copy()
        g.reshape(-1)[5] = np.float32(float(qo.reshape(-1)[5]) + rel * scale[5])
        if ok:
            C.check_prologue(g, qo, n, cs, pos, rot, W.ROTATE_HALF, F32)
        else:
            with pytest.raises(AssertionError, match="beyond rel 1e-5"):
                C.check_prologue(g, qo, n, cs, pos, rot, W.ROTATE_HALF, F32)


def test_bitwise_rule():
    a = np.array([1.0, -0.0, np.nan, 3.5], np.float32)
    C.check_bitwise(a.copy(), a)
    b = a.copy()
    b[1] = 0.0                                                # the sign of zero counts
    with pytest.raises(AssertionError, match="not bit-identical"):
        C.check_bitwise(b, a)
    u = np.arange(300, dtype=np.uint16)
    v = u.copy()
    v[7] ^= 1
    with pytest.raises(AssertionError):
        C.check_bitwise(v, u)


def test_fp8_rule(orc):
    g = np.random.default_rng(5)
    codes = orc.quantize_fp8(g.standard_normal(5000).astype(np.float32) * 40, 1.0)
    assert C.check_fp8(codes.copy(), codes)["differ"] == 0
    one = codes.copy()
    one[100] = (one[100] & 0x80) | ((one[100] & 0x7F) + 1 if (one[100] & 0x7F) < 0x7E
                                    else (one[100] & 0x7F) - 1)
    assert C.check_fp8(one, codes)["differ"] == 1
    two = codes.copy()
    m = two[200] & 0x7F
    two[200] = (two[200] & 0x80) | (m + 2 if m < 0x7D else m - 2)
    with pytest.raises(AssertionError, match="2 steps apart"):
        C.check_fp8(two, codes)
    # +0 and -0 are one value; a NaN code must match a NaN code
    z = np.array([0x00, 0x80, 0x7F], np.uint8)
    C.check_fp8(np.array([0x80, 0x00, 0xFF], np.uint8), z)
    with pytest.raises(AssertionError, match="NaN"):
        C.check_fp8(np.array([0x00, 0x80, 0x7E], np.uint8), z)
    # many one-step differences: a systematic rounding error
    many = codes.copy()
    sel = (many & 0x7F) < 0x7E
    sel[1::2] = False
    many[sel] += 1
    with pytest.raises(AssertionError, match="FP8 codes differ"):
        C.check_fp8(many, codes)


def test_modulated_rule():
    # a = n (1 + scale) cancelled by the shift: an escape within the bound
    # passes (and is counted), one past it fails
    H = 2048
    a_mag = np.full(1000, 4.0)
    shift = -np.full(1000, 4.0) + 1e-3
    o = W.to_bits(a_mag + shift, BF16)
    assert C.check_modulated(o.copy(), o, a_mag, shift, H, BF16)["escapes"] == 0
    u = 2.0 ** -24
    bound = ((H + 8) / 2.0 + np.log2(H) + 8) * u * 4.0 + 2 * u * 4.0
    step = float(C.spacing16(o[:1], BF16)[0])
    k_in = int(bound // step)                 # inside the cancellation bound
    assert k_in >= 2
    r = C.check_modulated(_bump(o, 3, k_in), o, a_mag, shift, H, BF16)
    assert r["escapes"] == 1
    with pytest.raises(AssertionError, match="cancellation bound"):
        C.check_modulated(_bump(o, 3, int(bound // step) + 3), o, a_mag, shift, H, BF16)
