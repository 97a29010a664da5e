"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with an independent fact:

* library routines: torch / numpy dtype casts, ``torch.nn.functional.rms_norm``,
  ``silu`` and ``gelu(approximate="tanh")``, complex multiplication, eager add;
* closed forms: a power-of-two constant row normalises to exactly +-R(w + delta),
  a zero row to zero; a (cos, sin) = (0, 1) cache swaps each pair with one sign
  flip, (-1, 0) negates it, position 0 is the identity;
* invariants: scale invariance at eps = 0, rotation preserves pair norms and
  composes additively in the angle, the fused ops equal the composition of the
  separately written row primitives;
* brute force against exact (mpmath) arithmetic on tiny heads and over every
  bf16 input of the activations.

The same functions run against deliberately mutated builds of the oracle
(tests/test_oracle_strength.py) to show that each plausible mistake is caught.
"""
import math

import mpmath
import numpy as np
import torch
import torch.nn.functional as F

import workloads as W

F32, F16, BF16 = W.F32, W.F16, W.BF16
U32 = 2.0 ** -24  # unit roundoff of binary32


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _ord16(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp16(a_bits, b_bits):
    """ulp distance of two bf16 / fp16 arrays (sign-magnitude order, +0 == -0)."""
    return np.abs(_ord16(a_bits) - _ord16(b_bits))


def same_bits(a, b, dtype):
    """Bitwise equality, treating +0 / -0 as equal and NaN == NaN."""
    if dtype == F32:
        a = np.asarray(a, np.float32)
        b = np.asarray(b, np.float32)
        return np.all((a == b) | (np.isnan(a) & np.isnan(b)))
    return np.all(ulp16(a, b) == 0)


def f32(bits, dtype):
    return W.bits_to_f32(bits, dtype)


def round_exact(v, dtype):
    """Round an exact real (float64 or mpmath value) to `dtype`, nearest-even,
    from its float64 value.  Returns (rounded float64 value, ambiguous flag):
    ambiguous when v lies within 1e-6 relative of a midpoint, where an fp32
    computation may legitimately land on either side."""
    v = float(v)
    if v == 0.0 or not math.isfinite(v):
        return v, False
    p = {BF16: 8, F16: 11, F32: 24}[dtype]
    m, e = math.frexp(abs(v))                    # |v| = m 2^e, m in [0.5, 1)
    if dtype == F16:
        e = max(e, -13)                          # subnormal grid 2^-24
    elif dtype == BF16:
        e = max(e, -125)
    q = math.ldexp(1.0, e - p)
    lo = math.floor(abs(v) / q) * q
    hi = lo + q
    mid = lo + q / 2
    amb = abs(abs(v) - mid) <= 1e-6 * abs(v)
    if abs(v) < mid:
        r = lo
    elif abs(v) > mid:
        r = hi
    else:
        r = lo if (lo / q) % 2 == 0 else hi
    return math.copysign(r, v), amb


# ---------------------------------------------------------------------------
# converters (IEEE 754 / OCP OFP8 vs torch and numpy casts)
# ---------------------------------------------------------------------------

def _fp32_sweep(n=400_000, seed=7):
    g = np.random.default_rng(seed)
    rand = g.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    hi = np.arange(65536, dtype=np.uint32) << 16
    near_mid = np.concatenate([hi | 0x7FFF, hi | 0x8000, hi | 0x8001, hi, hi | 0xFFFF])
    return np.concatenate([rand, near_mid]).view(np.float32)


def pin_bf16_converter(orc):
    bits = np.arange(65536, dtype=np.uint16)
    dec = orc.decode(bits, BF16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert same_bits(dec, ref, F32), "bf16 decode differs from torch"
    vals = _fp32_sweep()
    enc = orc.encode(vals, BF16)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(vals)
    assert np.array_equal(enc[~nan], ref[~nan]), "bf16 RNE encode differs from torch"
    assert np.all((enc[nan] & 0x7F80) == 0x7F80) and np.all(enc[nan] & 0x7F), "NaN lost"


def pin_f16_converter(orc):
    bits = np.arange(65536, dtype=np.uint16)
    dec = orc.decode(bits, F16)
    ref = bits.view(np.float16).astype(np.float32)
    assert same_bits(dec, ref, F32), "fp16 decode differs from numpy"
    # every fp16 value, its midpoints to the next value and one fp32 ulp around
    finite = bits[(bits & 0x7C00) != 0x7C00]
    v = finite.view(np.float16).astype(np.float64)
    with np.errstate(over="ignore"):
        nxt = np.nextafter(finite.view(np.float16), np.float16(np.inf)).astype(np.float64)
    mid = ((v + nxt) / 2).astype(np.float32)
    extra = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)),
                            np.nextafter(mid, np.float32(-np.inf)),
                            np.float32([65504, 65519.99, 65520, 1e5, 2 ** -25, 2 ** -26,
                                        3 * 2 ** -26, 2 ** -24 * 1.5])])
    vals = np.concatenate([_fp32_sweep(seed=8), extra]).astype(np.float32)
    enc = orc.encode(vals, F16)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    nan = np.isnan(vals)
    assert np.array_equal(enc[~nan], ref[~nan]), "fp16 RNE encode differs from numpy"


def e4m3fn_closed_form(code):
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * m / 8.0 * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def pin_e4m3fn_converter(orc):
    codes = np.arange(256, dtype=np.uint8)
    dec = orc.decode_e4m3fn(codes)
    closed = np.array([e4m3fn_closed_form(int(c)) for c in codes], dtype=np.float32)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert same_bits(dec, closed, F32) and same_bits(dec, lib, F32), "e4m3fn decode"
    # every code value, midpoints between neighbours and one fp32 ulp around them
    fin = np.sort(np.unique(closed[np.isfinite(closed)].astype(np.float64)))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    g = np.random.default_rng(3)
    rnd = (g.standard_normal(200_000) * np.exp2(g.integers(-12, 9, 200_000))).astype(np.float32)
    vals = np.concatenate([fin.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf)), rnd])
    inr = np.abs(vals) <= 464.0
    enc = orc.encode_e4m3fn(vals[inr])
    ref = torch.from_numpy(vals[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of zero; e4m3fn has both zeros, so compare bitwise
    assert np.array_equal(enc, ref), "e4m3fn RNE encode differs from torch"
    sat = orc.encode_e4m3fn(np.float32([448.5, 470, 1e6, np.inf, -500, -np.inf]))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE], "e4m3fn saturation"
    nan = orc.encode_e4m3fn(np.float32([np.nan]))
    assert (nan[0] & 0x7F) == 0x7F, "e4m3fn NaN"


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def pin_rmsnorm_vs_torch(orc):
    """fp32 rows against torch.nn.functional.rms_norm in float64.  Bound from
    the recursive-summation error of sum(x^2) ((D-1) u relative), halved by
    the square root, plus the divide, the sqrt and two products."""
    g = np.random.default_rng(11)
    for D in (7, 64, 128, 256, 2560):
        for eps in (1e-6, 0.5):
            for delta in (0, 1):
                x = g.standard_normal((16, D)).astype(np.float32) * 1.7
                w = (g.standard_normal(D) * 0.05 + (1 - delta)).astype(np.float32)
                y = orc.rmsnorm_rows(x, w, eps, delta, F32).astype(np.float64)
                ref = F.rms_norm(torch.from_numpy(x.astype(np.float64)), (D,),
                                 weight=torch.from_numpy(w.astype(np.float64) + delta),
                                 eps=float(np.float32(eps))).numpy()
                tol = ((D + 8) / 2.0) * U32 * np.abs(ref) + 1e-30
                assert np.all(np.abs(y - ref) <= tol), f"rmsnorm vs torch D={D} eps={eps}"


def pin_rmsnorm_closed_forms(orc):
    g = np.random.default_rng(12)
    for dtype in (BF16, F16, F32):
        for D in (4, 64, 256):
            for delta in (0, 1):
                w = W.to_bits(g.standard_normal(D) * 0.05 + (1 - delta), dtype)
                wd = f32(w, dtype).astype(np.float64) + delta
                # power-of-two constant rows: x * inv is exactly +-1 at eps = 0
                for c in (1.0, -4.0, 0.25, 64.0):
                    x = W.to_bits(np.full((1, D), c), dtype)
                    y = orc.rmsnorm_rows(x, w, 0.0, delta, dtype)
                    ref = W.to_bits(np.sign(c) * wd, dtype)
                    assert same_bits(y[0], ref, dtype), f"constant row c={c}"
                # zero row with eps > 0: exactly zero
                z = W.to_bits(np.zeros((1, D)), dtype)
                y = orc.rmsnorm_rows(z, w, 1e-6, delta, dtype)
                assert np.all(f32(y, dtype) == 0.0), "zero row"
                # scale invariance at eps = 0: x * 2^k gives the same bits
                x = W.to_bits(g.standard_normal((4, D)), dtype)
                y0 = orc.rmsnorm_rows(x, w, 0.0, delta, dtype)
                for k in (-3, 2):
                    xs = W.to_bits(f32(x, dtype).astype(np.float64) * 2.0 ** k, dtype)
                    # only where the scaled row is itself exact (no fp16 subnormals)
                    if not np.array_equal(f32(xs, dtype), f32(x, dtype) * np.float32(2.0 ** k)):
                        continue
                    yk = orc.rmsnorm_rows(xs, w, 0.0, delta, dtype)
                    assert same_bits(y0, yk, dtype), "scale invariance"


_GRID = [0.5, -1.0, 1.5, -3.0, 0.1015625, -2.75, 7.0, 0.0, -0.03125, 12.5]


def pin_rmsnorm_bruteforce(orc):
    """All rows of D = 2 and D = 4 drawn from a small bf16 grid, against the
    exact value (mpmath, 40 digits) rounded once to bf16."""
    mpmath.mp.dps = 40
    eps = float(np.float32(1e-6))
    for D, delta in ((2, 0), (4, 1), (4, 0)):
        rows = np.array(np.meshgrid(*([_GRID] * D), indexing="ij")).reshape(D, -1).T
        w = np.array([0.75, -0.5, 1.25, 0.0625][:D]) - (0.0 if delta == 0 else 1.0)
        xb = W.to_bits(rows, BF16)
        wb = W.to_bits(w, BF16)
        y = f32(orc.rmsnorm_rows(xb, wb, eps, delta, BF16), BF16)
        xv = f32(xb, BF16).astype(np.float64)
        wv = f32(wb, BF16).astype(np.float64) + delta
        amb = bad = 0
        for r in range(rows.shape[0]):
            ms = mpmath.fsum(mpmath.mpf(v) ** 2 for v in xv[r]) / D
            inv = 1 / mpmath.sqrt(ms + mpmath.mpf(eps))
            for i in range(D):
                exact, a = round_exact(mpmath.mpf(xv[r, i]) * inv * mpmath.mpf(wv[i]), BF16)
                if y[r, i] != exact:
                    if a:
                        amb += 1
                    else:
                        bad += 1
        assert bad == 0, f"brute force D={D}: {bad} wrong roundings"
        assert amb <= rows.size // 200, f"brute force D={D}: {amb} midpoint cases"


def pin_rmsnorm_no_weight(orc):
    """No weight (w = None; the norm's scale folded into the next GEMM, as in
    the FlashRT weight-folding paragraph): fp32 rows against torch's
    rms_norm with weight=None in float64 (same bound as with a weight);
    power-of-two constant rows give exactly +-1 in every dtype; every row of
    D = 4 over the bf16 grid against mpmath rounded once; and the fused
    residual, FP8 and amax variants agree with the plain row function."""
    g = np.random.default_rng(13)
    for D in (7, 256, 2560):
        for eps in (1e-6, 0.5):
            x = g.standard_normal((16, D)).astype(np.float32) * 1.7
            y = orc.rmsnorm_rows(x, None, eps, 0, F32).astype(np.float64)
            ref = F.rms_norm(torch.from_numpy(x.astype(np.float64)), (D,), weight=None,
                             eps=float(np.float32(eps))).numpy()
            tol = ((D + 8) / 2.0) * U32 * np.abs(ref) + 1e-30
            assert np.all(np.abs(y - ref) <= tol), f"no-weight rmsnorm vs torch D={D}"
    for dtype in (BF16, F16, F32):
        for c in (1.0, -4.0, 0.25, 64.0):
            x = W.to_bits(np.full((1, 64), c), dtype)
            y = f32(orc.rmsnorm_rows(x, None, 0.0, 0, dtype), dtype)
            assert np.all(y == np.sign(c)), f"no-weight constant row c={c}"
    mpmath.mp.dps = 40
    eps = float(np.float32(1e-6))
    rows = np.array(np.meshgrid(*([_GRID] * 4), indexing="ij")).reshape(4, -1).T
    xb = W.to_bits(rows, BF16)
    y = f32(orc.rmsnorm_rows(xb, None, eps, 0, BF16), BF16)
    xv = f32(xb, BF16).astype(np.float64)
    amb = bad = 0
    for r in range(rows.shape[0]):
        inv = 1 / mpmath.sqrt(mpmath.fsum(mpmath.mpf(v) ** 2 for v in xv[r]) / 4
                              + mpmath.mpf(eps))
        for i in range(4):
            exact, a = round_exact(mpmath.mpf(xv[r, i]) * inv, BF16)
            if y[r, i] != exact:
                amb, bad = (amb + 1, bad) if a else (amb, bad + 1)
    assert bad == 0 and amb <= rows.size // 200, f"no-weight brute force: {bad} / {amb}"
    x = W.to_bits(g.standard_normal((6, 1024)), BF16)
    r = W.to_bits(g.standard_normal((6, 1024)), BF16)
    xo, ro = orc.fused_add_rmsnorm(x, r, None, 1e-6, 0, BF16)
    assert same_bits(xo, orc.rmsnorm_rows(ro, None, 1e-6, 0, BF16), BF16)
    xf, rf = f32(x, BF16), f32(r, BF16)
    xo32, _ = orc.fused_add_rmsnorm(xf, rf, None, 1e-6, 0, F32)
    amax = orc.fused_add_rmsnorm_amax(xf, rf, None, 1e-6, 0, F32)
    assert amax == float(np.max(np.abs(xo32))), "no-weight amax"
    y8, _ = orc.fused_add_rmsnorm_fp8(xf, rf, None, np.float32(448.0 / amax), 1e-6, 0, F32)
    assert np.array_equal(y8, orc.quantize_fp8(xo32, np.float32(448.0 / amax)))


def pin_adarms(orc):
    """Adaptive RMSNorm (FlashRT's fused_adarms / gate_res_adarms kernels, in
    the reading m = (s inv)(1 + scale) + shift, s = R(r + g x)).
    * scale = shift = 0 and no residual: exactly the no-weight RMSNorm;
    * fp32 rows against float64 torch (rms_norm without weight, then the
      modulation), bound (D+8)/2 u on the norm plus 3 u for the modulation;
    * the gated residual equals numpy's fp32 r + g * x (product and sum
      rounded separately) rounded once to the dtype;
    * every row of D = 4 over the bf16 grid against mpmath, rounded once;
    * FP8 == quantize_fp8 of the fp32 output, amax == max |output|;
    * a gate without a residual is refused."""
    g = np.random.default_rng(14)
    H = 64
    for dtype in (BF16, F16, F32):
        x = W.to_bits(g.standard_normal((5, H)) + 0.01, dtype)
        zero = W.to_bits(np.zeros(H), dtype)
        xo, _ = orc.adarms(x, None, None, zero, zero, 1e-6, dtype)
        assert same_bits(xo, orc.rmsnorm_rows(x, None, 1e-6, 0, dtype), dtype), \
            f"identity modulation != no-weight norm ({dtype})"
    for D in (7, 256, 2048):
        x = (g.standard_normal((8, D)) * 1.5).astype(np.float32)
        sc = (g.standard_normal(D) * 0.2).astype(np.float32)
        sh = (g.standard_normal(D) * 0.2).astype(np.float32)
        y, _ = orc.adarms(x, None, None, sc, sh, 1e-6, F32)
        n = F.rms_norm(torch.from_numpy(x.astype(np.float64)), (D,), weight=None,
                       eps=float(np.float32(1e-6))).numpy()
        a = n * (1.0 + sc.astype(np.float64))
        ref = a + sh.astype(np.float64)
        tol = ((D + 8) / 2.0 + 3) * U32 * np.abs(a) + 2 * U32 * np.abs(ref) + 1e-30
        assert np.all(np.abs(y.astype(np.float64) - ref) <= tol), f"adarms vs torch D={D}"
    for dtype in (BF16, F16, F32):
        x = W.to_bits(g.standard_normal((6, 96)), dtype)
        r = W.to_bits(g.standard_normal((6, 96)) * 2, dtype)
        gt = W.to_bits(g.standard_normal(96) * 0.5 + 1, dtype)
        sc = W.to_bits(g.standard_normal(96) * 0.1, dtype)
        sh = W.to_bits(g.standard_normal(96) * 0.1, dtype)
        _, ro = orc.adarms(x, r, gt, sc, sh, 1e-6, dtype)
        want = f32(r, dtype) + f32(gt, dtype) * f32(x, dtype)        # numpy fp32, unfused
        assert same_bits(ro, W.to_bits(want.astype(np.float64), dtype), dtype), \
            f"gated residual ({dtype})"
        _, ro1 = orc.adarms(x, r, None, sc, sh, 1e-6, dtype)
        want1 = f32(r, dtype) + f32(x, dtype)
        assert same_bits(ro1, W.to_bits(want1.astype(np.float64), dtype), dtype), "plain residual"
    mpmath.mp.dps = 40
    eps = float(np.float32(1e-6))
    rows = np.array(np.meshgrid(*([_GRID] * 4), indexing="ij")).reshape(4, -1).T
    xb = W.to_bits(rows, BF16)
    scb = W.to_bits(np.array([0.25, -0.5, 0.0625, 1.5]), BF16)
    shb = W.to_bits(np.array([-0.125, 0.0, 0.75, 0.03125]), BF16)
    y = f32(orc.adarms(xb, None, None, scb, shb, eps, BF16)[0], BF16)
    xv = f32(xb, BF16).astype(np.float64)
    scv, shv = f32(scb, BF16).astype(np.float64), f32(shb, BF16).astype(np.float64)
    amb = bad = 0
    for rr in range(rows.shape[0]):
        inv = 1 / mpmath.sqrt(mpmath.fsum(mpmath.mpf(v) ** 2 for v in xv[rr]) / 4
                              + mpmath.mpf(eps))
        for i in range(4):
            exact = mpmath.mpf(xv[rr, i]) * inv * (1 + mpmath.mpf(scv[i])) + mpmath.mpf(shv[i])
            e, a = round_exact(exact, BF16)
            if y[rr, i] != e:
                amb, bad = (amb + 1, bad) if a else (amb, bad + 1)
    assert bad == 0 and amb <= rows.size // 200, f"adarms brute force: {bad} / {amb}"
    x = g.standard_normal((8, 512)).astype(np.float32)
    r = g.standard_normal((8, 512)).astype(np.float32)
    gt = (g.standard_normal(512) * 0.3 + 1).astype(np.float32)
    sc = (g.standard_normal(512) * 0.1).astype(np.float32)
    sh = (g.standard_normal(512) * 0.1).astype(np.float32)
    xo, ro = orc.adarms(x, r, gt, sc, sh, 1e-6, F32)
    amax = orc.adarms_amax(x, r, gt, sc, sh, 1e-6, F32)
    assert amax == float(np.max(np.abs(xo))), "adarms amax"
    y8, ro8 = orc.adarms_fp8(x, r, gt, sc, sh, np.float32(448.0 / amax), 1e-6, F32)
    assert np.array_equal(ro8, ro) and np.array_equal(y8, orc.quantize_fp8(xo, np.float32(448.0 / amax)))
    try:
        orc.adarms(x, None, gt, sc, sh, 1e-6, F32)
    except Exception:
        pass
    else:
        raise AssertionError("a gate without a residual must be refused")


# ---------------------------------------------------------------------------
# rotary embedding
# ---------------------------------------------------------------------------

def _complex_pairs(x, rot, layout):
    if layout == W.ROTATE_HALF:
        a, b = np.arange(rot // 2), np.arange(rot // 2) + rot // 2
    else:
        a, b = np.arange(0, rot, 2), np.arange(1, rot, 2)
    return a, b


def pin_rope_complex(orc):
    """fp32 rotation against complex multiplication by cos + i sin (numpy
    complex128, with the cache's own fp32 values as the exact angle): bound
    3u |z| per component (two rounded products and one rounded sum)."""
    g = np.random.default_rng(21)
    for layout in (W.ROTATE_HALF, W.INTERLEAVED):
        for D, rot in ((128, 128), (256, 64), (64, 32), (8, 4)):
            cs = W.rope_cache(512, rot, 1e4)
            T, H = 9, 3
            x = g.standard_normal((T, H, D)).astype(np.float32)
            pos = g.integers(0, 512, T).astype(np.int64)
            y = orc.rope(x, cs, pos, rot, layout, F32)
            a, b = _complex_pairs(x, rot, layout)
            c = cs[pos][:, None, : rot // 2].astype(np.float64)
            s = cs[pos][:, None, rot // 2:].astype(np.float64)
            z = x[..., a].astype(np.float64) + 1j * x[..., b].astype(np.float64)
            o = z * (c + 1j * s)
            tol = 3 * U32 * np.abs(z) + 1e-30
            assert np.all(np.abs(y[..., a] - o.real) <= tol), "rope real part"
            assert np.all(np.abs(y[..., b] - o.imag) <= tol), "rope imaginary part"
            assert np.array_equal(y[..., rot:], x[..., rot:]), "channels past rot changed"


def pin_rope_closed_forms(orc):
    g = np.random.default_rng(22)
    for dtype in (BF16, F16, F32):
        for layout in (W.ROTATE_HALF, W.INTERLEAVED):
            D, rot = 32, 16
            x = W.to_bits(g.standard_normal((5, 2, D)), dtype)
            a, b = _complex_pairs(None, rot, layout)
            # quarter turn: (c, s) = (0, 1) maps (a, b) -> (-b, a) exactly
            cs = np.zeros((3, rot), np.float32)
            cs[0, :rot // 2] = 1.0                      # row 0: identity
            cs[1, rot // 2:] = 1.0                      # row 1: quarter turn
            cs[2, :rot // 2] = -1.0                     # row 2: half turn
            xv = f32(x, dtype)
            for p, want_a, want_b in ((0, xv[..., a], xv[..., b]),
                                      (1, -xv[..., b], xv[..., a]),
                                      (2, -xv[..., a], -xv[..., b])):
                y = f32(orc.rope(x, cs, np.full(5, p), rot, layout, dtype), dtype)
                assert np.array_equal(y[..., a], want_a) and np.array_equal(y[..., b], want_b), \
                    f"rope closed form p={p} layout={layout}"
                assert np.array_equal(y[..., rot:], xv[..., rot:]), "tail channels"
            # outside the cache: untouched (p = max_pos, p < 0)
            y = orc.rope(x, cs, np.array([3, -1, 1 << 40, 3, -7]), rot, layout, dtype)
            assert same_bits(y, x, dtype), "out-of-range position must leave the token untouched"


def pin_rope_invariants(orc):
    """Pair norm preserved and angles additive (fp32 I/O, real cache)."""
    g = np.random.default_rng(23)
    D, rot = 64, 64
    cs = W.rope_cache(4096, rot, 1e6)
    x = g.standard_normal((6, 4, D)).astype(np.float32)
    for layout in (W.ROTATE_HALF, W.INTERLEAVED):
        a, b = _complex_pairs(None, rot, layout)
        p1 = g.integers(0, 2048, 6)
        p2 = g.integers(0, 2048, 6)
        y1 = orc.rope(x, cs, p1, rot, layout, F32)
        n0 = x[..., a].astype(np.float64) ** 2 + x[..., b].astype(np.float64) ** 2
        n1 = y1[..., a].astype(np.float64) ** 2 + y1[..., b].astype(np.float64) ** 2
        assert np.all(np.abs(n1 - n0) <= 12 * U32 * n0 + 1e-30), "pair norm"
        y12 = orc.rope(y1, cs, p2, rot, layout, F32)
        y3 = orc.rope(x, cs, p1 + p2, rot, layout, F32)
        scale = np.sqrt(n0)
        # the cache rows themselves carry fp32 rounding: allow a few u |z|
        assert np.all(np.abs(y12[..., a] - y3[..., a]) <= 16 * U32 * scale + 1e-30) and \
            np.all(np.abs(y12[..., b] - y3[..., b]) <= 16 * U32 * scale + 1e-30), "additivity"


# ---------------------------------------------------------------------------
# fused QK-norm + RoPE prologue
# ---------------------------------------------------------------------------

def pin_prologue_composition(orc):
    """The fused prologue equals rmsnorm_rows (w_q on query heads, w_k on key
    heads) -> round -> rope, bit for bit, for every dtype, both layouts,
    partial rotation and positions inside and outside the cache."""
    g = np.random.default_rng(31)
    for dtype in (BF16, F16, F32):
        for layout in (W.ROTATE_HALF, W.INTERLEAVED):
            for (Q, K, D, rot, delta) in ((4, 2, 64, 64, 0), (3, 1, 256, 64, 1),
                                          (2, 2, 128, 32, 1), (1, 0, 16, 0, 0)):
                T = 5
                q = W.to_bits(g.standard_normal((T, Q, D)) * 2, dtype)
                k = W.to_bits(g.standard_normal((T, K, D)) * 2, dtype)
                wq = W.to_bits(g.standard_normal(D) * 0.05 + (1 - delta), dtype)
                wk = W.to_bits(g.standard_normal(D) * 0.05 + (1 - delta), dtype)
                cs = W.rope_cache(64, rot, 1e7)
                pos = np.array([0, 63, 64, -1, 17])[:T]
                qo, ko = orc.qknorm_rope(q, k, wq, wk, cs, pos, rot, 1e-6, delta, layout, dtype)
                qn = orc.rmsnorm_rows(q, wq, 1e-6, delta, dtype)
                kn = orc.rmsnorm_rows(k, wk, 1e-6, delta, dtype)
                qr = orc.rope(qn, cs, pos, rot, layout, dtype)
                kr = orc.rope(kn, cs, pos, rot, layout, dtype) if K else kn
                assert same_bits(qo, qr, dtype), f"prologue q composition {dtype} {layout}"
                assert same_bits(ko, kr, dtype), f"prologue k composition {dtype} {layout}"


def pin_prologue_constant_head(orc):
    """A power-of-two constant head at position 0 comes out as +-R(w + delta)
    exactly, whatever the rotated width (the mean is over head_dim)."""
    for dtype in (BF16, F32):
        for (D, rot) in ((256, 64), (128, 128), (64, 16)):
            for delta in (0, 1):
                w = W.to_bits(np.linspace(-0.1, 0.1, D) + (1 - delta), dtype)
                q = W.to_bits(np.full((1, 2, D), -2.0), dtype)
                k = W.to_bits(np.full((1, 1, D), 0.5), dtype)
                cs = W.rope_cache(8, rot, 1e6)
                qo, ko = orc.qknorm_rope(q, k, w, w, cs, np.array([0]), rot, 0.0, delta,
                                         W.ROTATE_HALF, dtype)
                wd = W.to_bits(f32(w, dtype).astype(np.float64) + delta, dtype)
                assert same_bits(qo[0, 0], W.to_bits(-f32(wd, dtype), dtype), dtype), "q head"
                assert same_bits(ko[0, 0], wd, dtype), "k head"


def pin_prologue_round_once(orc):
    """Single-rounding variant (the ninfer PR's review item 1: rotate the fp32
    norm result, round once).  Closed forms: with an identity, quarter-turn or
    half-turn cache row the rotated channels are exactly R(n), (-R(n_b),
    R(n_a)) and (-R(n_a), -R(n_b)) of the plain RMSNorm; channels past
    rot_dim and tokens outside the cache equal the plain RMSNorm.  Against
    float64: the exact rotation of the exact norm result, rounded once, must
    match wherever it is farther from a rounding midpoint than the oracle's
    own fp32 error bound (sum of squares (D+8)/2 u, products and sum 3 u)."""
    g = np.random.default_rng(33)
    for dtype in (BF16, F16, F32):
        for layout in (W.ROTATE_HALF, W.INTERLEAVED):
            D, rot, Q, K = 32, 16, 2, 1
            q = W.to_bits(g.standard_normal((5, Q, D)) * 2, dtype)
            k = W.to_bits(g.standard_normal((5, K, D)) * 2, dtype)
            w = W.to_bits(g.standard_normal(D) * 0.05, dtype)
            cs = np.zeros((3, rot), np.float32)
            cs[0, :rot // 2] = 1.0                      # identity
            cs[1, rot // 2:] = 1.0                      # quarter turn
            cs[2, :rot // 2] = -1.0                     # half turn
            a, b = _complex_pairs(None, rot, layout)
            qn = f32(orc.rmsnorm_rows(q, w, 1e-6, 1, dtype), dtype)
            for p, fa, fb in ((0, lambda v: v[..., a], lambda v: v[..., b]),
                              (1, lambda v: -v[..., b], lambda v: v[..., a]),
                              (2, lambda v: -v[..., a], lambda v: -v[..., b])):
                qo, _ = orc.qknorm_rope(q, k, w, w, cs, np.full(5, p), rot, 1e-6, 1, layout,
                                        dtype, round_once=True)
                qo = f32(qo, dtype)
                assert np.array_equal(qo[..., a], fa(qn)) and np.array_equal(qo[..., b], fb(qn)), \
                    f"round-once closed form p={p} dtype={dtype} layout={layout}"
                assert np.array_equal(qo[..., rot:], qn[..., rot:]), "round-once tail channels"
            qo, _ = orc.qknorm_rope(q, k, w, w, cs, np.array([3, -1, 7, 1 << 40, 5]), rot, 1e-6,
                                    1, layout, dtype, round_once=True)
            assert np.array_equal(f32(qo, dtype), qn), "round-once outside the cache"
    for dtype in (BF16, F16):
        for layout in (W.ROTATE_HALF, W.INTERLEAVED):
            D, rot, T, Q, K = 128, 64, 4, 3, 1
            q = W.to_bits(g.standard_normal((T, Q, D)) * 2, dtype)
            k = W.to_bits(g.standard_normal((T, K, D)) * 2, dtype)
            wq = W.to_bits(g.standard_normal(D) * 0.05, dtype)
            wk = W.to_bits(g.standard_normal(D) * 0.05, dtype)
            cs = W.rope_cache(4096, rot, 1e6)
            pos = g.integers(0, 4096, T)
            qo, ko = orc.qknorm_rope(q, k, wq, wk, cs, pos, rot, 1e-6, 1, layout, dtype,
                                     round_once=True)
            a, b = _complex_pairs(None, rot, layout)
            c = cs[pos][:, None, : rot // 2].astype(np.float64)
            s_ = cs[pos][:, None, rot // 2:].astype(np.float64)
            decided = amb = 0
            for x, wt, y in ((q, wq, qo), (k, wk, ko)):
                xv = f32(x, dtype).astype(np.float64)
                inv = 1.0 / np.sqrt(np.mean(xv * xv, axis=-1, keepdims=True) + float(np.float32(1e-6)))
                n = xv * inv * (f32(wt, dtype).astype(np.float64) + 1.0)
                oa = n[..., a] * c - n[..., b] * s_
                ob = n[..., b] * c + n[..., a] * s_
                mag = np.abs(n[..., a] * c) + np.abs(n[..., b] * s_)
                bound = ((D + 8) / 2.0 + 3) * U32 * mag
                yv = f32(y, dtype)
                for exact, got, bd in ((oa, yv[..., a], bound), (ob, yv[..., b], bound)):
                    for e, gv, bb in zip(exact.ravel(), got.ravel(), bd.ravel()):
                        lo, _ = round_exact(e - bb, dtype)
                        hi, _ = round_exact(e + bb, dtype)
                        if lo != hi:
                            amb += 1
                            continue
                        decided += 1
                        assert gv == lo, f"round-once rotation: {gv} vs exact {e} ({dtype})"
            assert amb <= 0.08 * (decided + amb), f"round-once: {amb} undecided of {decided + amb}"


# ---------------------------------------------------------------------------
# fused residual-add RMSNorm and its FP8 variant
# ---------------------------------------------------------------------------

def pin_residual_add(orc):
    """Residual stream equals torch's eager add (bf16 / fp16) or numpy's
    (fp32) bit for bit, and the normalised output equals rmsnorm_rows of the
    rounded sum."""
    g = np.random.default_rng(41)
    for dtype in (BF16, F16, F32):
        for H in (37, 1024):
            x = W.to_bits(g.standard_normal((6, H)), dtype)
            r = W.to_bits(g.standard_normal((6, H)) * 3, dtype)
            w = W.to_bits(g.standard_normal(H) * 0.05 + 1, dtype)
            xo, ro = orc.fused_add_rmsnorm(x, r, w, 1e-6, 0, dtype)
            if dtype == F32:
                eager = (x + r).astype(np.float32)
            else:
                tx, tr = W.to_torch(x, dtype), W.to_torch(r, dtype)
                eager = W.from_torch(tx + tr, dtype)
            assert same_bits(ro, eager, dtype), f"residual != eager add ({dtype})"
            assert same_bits(xo, orc.rmsnorm_rows(ro, w, 1e-6, 0, dtype), dtype), \
                "normalised output != rmsnorm(rounded sum)"
            xo2, ro2 = orc.fused_add_rmsnorm(x, None, w, 1e-6, 1, dtype)
            assert ro2 is None and same_bits(xo2, orc.rmsnorm_rows(x, w, 1e-6, 1, dtype), dtype)


def pin_norm_fp8(orc):
    """FP8 variant == quantize_fp8 of the fp32 output of the plain op (fp32
    I/O: that output is the unrounded value), and the calibration amax is the
    largest magnitude of that same output."""
    g = np.random.default_rng(42)
    H = 2048
    x = g.standard_normal((8, H)).astype(np.float32)
    r = g.standard_normal((8, H)).astype(np.float32)
    w = (g.standard_normal(H) * 0.05 + 1).astype(np.float32)
    for delta in (0, 1):
        xo, ro = orc.fused_add_rmsnorm(x, r, w, 1e-6, delta, F32)
        amax = orc.fused_add_rmsnorm_amax(x, r, w, 1e-6, delta, F32)
        assert amax == float(np.max(np.abs(xo))), "norm amax"
        for inv_scale in (448.0 / amax, 200.0 / amax, 1000.0 / amax):
            y, ro8 = orc.fused_add_rmsnorm_fp8(x, r, w, np.float32(inv_scale), 1e-6, delta, F32)
            assert np.array_equal(ro8, ro)
            assert np.array_equal(y, orc.quantize_fp8(xo, np.float32(inv_scale))), "norm fp8"


def pin_quantize_vs_torch(orc):
    g = np.random.default_rng(43)
    x = (g.standard_normal(100_000) * 3).astype(np.float32)
    for inv_scale in (1.0, 37.5, 0.01):
        y = orc.quantize_fp8(x, np.float32(inv_scale))
        v = (x * np.float32(inv_scale)).astype(np.float32)
        inr = np.abs(v) <= 464
        ref = torch.from_numpy(v[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(y[inr], ref), "quantize vs torch"
        assert np.all((y[~inr] & 0x7F) == 0x7E), "quantize saturation"


# ---------------------------------------------------------------------------
# gated activations
# ---------------------------------------------------------------------------

def pin_act_vs_torch(orc):
    """fp32 against torch silu / gelu(tanh) in float64 on g in [-4, 6], where
    torch's float64 tanh form is accurate.  Bound: a few u plus 2|z| times the
    rounding of z, as e^{-2z} magnifies it."""
    g = np.random.default_rng(51)
    d = 4096
    gv = g.uniform(-4, 6, (3, d)).astype(np.float32)
    uv = g.standard_normal((3, d)).astype(np.float32)
    gu = np.concatenate([gv, uv], axis=1)
    gt, ut = torch.from_numpy(gv.astype(np.float64)), torch.from_numpy(uv.astype(np.float64))
    for act, ref in ((W.SILU, F.silu(gt) * ut),
                     (W.GELU_TANH, F.gelu(gt, approximate="tanh") * ut)):
        out = orc.gated_act(gu, act, F32).astype(np.float64)
        ref = ref.numpy()
        z = np.abs(gv.astype(np.float64)) * (1 + 0.045 * gv.astype(np.float64) ** 2)
        tol = (16 + 8 * z) * U32 * np.abs(ref) + 1e-35
        assert np.all(np.abs(out - ref) <= tol), f"act {act} vs torch"


def pin_act_exhaustive_bf16(orc):
    """Every finite bf16 gate value with up = 1, against the exact activation
    (mpmath, 60 digits: 1 + tanh(z) needs ~40 of them before bf16 underflows)
    rounded once to bf16."""
    mpmath.mp.dps = 60
    bits = np.arange(65536, dtype=np.uint16)
    gv = f32(bits, BF16)
    keep = np.isfinite(gv)
    bits, gv = bits[keep], gv[keep].astype(np.float64)
    one = W.to_bits(np.ones(bits.size), BF16)
    gu = np.concatenate([bits, one])[None, :]
    c = mpmath.sqrt(2 / mpmath.pi)
    for act in (W.SILU, W.GELU_TANH):
        out = f32(orc.gated_act(gu, act, BF16)[0], BF16)
        bad = amb = 0
        for i in range(bits.size):
            x = mpmath.mpf(gv[i])
            if act == W.SILU:
                ex = x / (1 + mpmath.exp(-x))
            else:
                ex = x / 2 * (1 + mpmath.tanh(c * (x + mpmath.mpf("0.044715") * x ** 3)))
            r, a = round_exact(ex, BF16)
            if out[i] != r:
                if a:
                    amb += 1
                else:
                    bad += 1
        assert bad == 0, f"act {act}: {bad} bf16 inputs round wrongly"
        assert amb <= 64, f"act {act}: {amb} midpoint cases"


def pin_act_single_rounding_16bit(orc):
    """bf16 and fp16 I/O with u away from 1: out = R(act(g) u), the product
    rounded once.  Reference: act(g) u in float64 (g times the logistic of g,
    or of 2z for GELU-tanh), rounded with round_exact; every output that is
    not within fp32 error of a rounding midpoint must equal it.  Rounding
    act(g) to the dtype before the product (the unfused two-op form) moves
    about a quarter of the outputs by one step, which the exhaustive pin
    (u = 1) and the fp32 pins cannot see."""
    g = np.random.default_rng(57)
    d = 4096
    c = math.sqrt(2.0 / math.pi)
    for dtype in (BF16, F16):
        gb = W.to_bits(g.uniform(-6.0, 6.0, (2, d)), dtype)
        ub = W.to_bits(g.standard_normal((2, d)) * 1.5, dtype)
        gv, uv = f32(gb, dtype).astype(np.float64), f32(ub, dtype).astype(np.float64)
        gu = np.concatenate([gb, ub], axis=1)
        for act in (W.SILU, W.GELU_TANH):
            z = gv if act == W.SILU else 2.0 * c * (gv + 0.044715 * gv ** 3)
            exact = (gv / (1.0 + np.exp(-z))) * uv
            out = f32(orc.gated_act(gu, act, dtype), dtype).astype(np.float64)
            bad = amb = 0
            for o, v in zip(out.ravel(), exact.ravel()):
                r, a = round_exact(v, dtype)
                if o != r:
                    if a:
                        amb += 1
                    else:
                        bad += 1
            assert bad == 0, f"act {act} dtype {dtype}: {bad} outputs not rounded once"
            assert amb <= exact.size // 100, f"act {act} dtype {dtype}: {amb} midpoint cases"


def pin_act_identities(orc):
    """act(g) - act(-g) = g for SiLU and GELU-tanh; act(0) = 0; for large g
    the gate is exactly g, so out = R(g u)."""
    g = np.random.default_rng(52)
    d = 2048
    gv = g.uniform(-5, 5, (1, d)).astype(np.float32)
    one = np.ones((1, d), np.float32)
    for act in (W.SILU, W.GELU_TANH):
        pos = orc.gated_act(np.concatenate([gv, one], 1), act, F32).astype(np.float64)
        neg = orc.gated_act(np.concatenate([-gv, one], 1), act, F32).astype(np.float64)
        assert np.all(np.abs((pos - neg) - gv) <= 8 * U32 * np.abs(gv) + 1e-30), "odd part"
        zero = orc.gated_act(np.zeros((1, 2 * d), np.float32), act, F32)
        assert np.all(zero == 0)
        big = g.uniform(30, 1000, (1, d)).astype(np.float32)
        u = g.standard_normal((1, d)).astype(np.float32)
        for dtype in (BF16, F32):
            gu = W.to_bits(np.concatenate([big, u], 1), dtype)
            out = orc.gated_act(gu, act, dtype)
            ref = W.to_bits(f32(gu[:, :d], dtype).astype(np.float64)
                            * f32(gu[:, d:], dtype).astype(np.float64), dtype)
            assert same_bits(out, ref, dtype), "large-g limit"


def pin_act_fp8(orc):
    g = np.random.default_rng(53)
    gu = (g.standard_normal((4, 2 * 1024)) * 1.5).astype(np.float32)
    for act in (W.SILU, W.GELU_TANH):
        out = orc.gated_act(gu, act, F32)
        amax = orc.gated_act_amax(gu, act, F32)
        assert amax == float(np.max(np.abs(out))), "act amax"
        for inv_scale in (448.0 / amax, 100.0 / amax):
            y = orc.gated_act_fp8(gu, np.float32(inv_scale), act, F32)
            assert np.array_equal(y, orc.quantize_fp8(out, np.float32(inv_scale))), "act fp8"


# ---------------------------------------------------------------------------
# FP8 epilogues at 16-bit I/O: one rounding, from the fp32 value
# ---------------------------------------------------------------------------

def _e4m3_order(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def _torch_e4m3(v64, inv_scale):
    """torch's float8_e4m3fn cast of float64 values times inv_scale, after
    the saturation to +-448 the epilogues apply (torch's cast does not
    saturate); a library reference independent of the oracle's encoder."""
    v = np.clip(v64 * float(inv_scale), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _check_fp8_once(orc, y, amax, v32, v64, inv_scales, codes_for, what):
    """y: codes at the calibrated scale (inv_scales[0]); v32: the oracle's
    fp32 value the epilogue must quantize; v64: a float64 library value of
    the same; codes_for(inv): the epilogue's codes at another scale."""
    assert amax == float(np.max(np.abs(v32))), f"{what}: amax != max |fp32 value|"
    for k, inv in enumerate(inv_scales):
        yk = y if k == 0 else codes_for(inv)
        assert np.array_equal(yk, orc.quantize_fp8(v32, inv)), \
            f"{what}: codes != E4M3FN(fp32 value * inv_scale) at inv_scale {inv}"
        lib = _torch_e4m3(v64, inv)
        step = np.abs(_e4m3_order(yk) - _e4m3_order(lib))
        assert step.max() <= 1, f"{what}: codes more than one step from torch's cast"
        assert np.mean(step > 0) <= 0.01, f"{what}: {np.mean(step > 0):.4f} differ from torch"


def pin_fp8_epilogues_16bit(orc):
    """At bf16 and fp16 I/O the FP8 epilogues quantize the fp32 value of the
    op once (FlashRT optimization details: the static-FP8 kernels go from the
    fp32 result straight to the 8-bit code), not that value first rounded to
    the I/O dtype; the calibration passes take the largest magnitude of the
    same fp32 value.

    16-bit inputs decode exactly, so the value each epilogue must quantize is
    the oracle's fp32 path -- pinned to float64 torch by the pins above --
    run on the decoded inputs (for the residual forms, on the decoded rounded
    sum, which pin_residual_add ties to eager add).  Required: codes ==
    E4M3FN(value * inv_scale) bit for bit at three scales (one saturating),
    amax == max |value| exactly, and, independently of the oracle's encoder,
    codes within one step of torch's float8_e4m3fn cast of a float64 value.
    A dtype-rounded source moves about one code in sixteen (bf16) and fails."""
    g = np.random.default_rng(44)
    eps = 1e-6
    for dtype in (BF16, F16):
        # residual-add RMSNorm, both weight conventions and no weight
        H = 2048
        x = W.to_bits(g.standard_normal((8, H)), dtype)
        r = W.to_bits(g.standard_normal((8, H)), dtype)
        for delta, w in ((0, W.to_bits(g.standard_normal(H) * 0.05 + 1, dtype)),
                         (1, W.to_bits(g.standard_normal(H) * 0.05, dtype)), (0, None)):
            _, s_bits = orc.fused_add_rmsnorm(x, r, w, eps, delta, dtype)
            sv = f32(s_bits, dtype)
            wv = None if w is None else f32(w, dtype)
            v32 = orc.rmsnorm_rows(sv, wv, eps, delta, F32)
            v64 = F.rms_norm(torch.from_numpy(sv.astype(np.float64)), (H,), weight=None,
                             eps=float(np.float32(eps))).numpy()
            if w is not None:
                v64 = v64 * (wv.astype(np.float64) + delta)
            amax = orc.fused_add_rmsnorm_amax(x, r, w, eps, delta, dtype)
            invs = [np.float32(448.0 / amax), np.float32(200.0 / amax),
                    np.float32(1000.0 / amax)]
            y, r8 = orc.fused_add_rmsnorm_fp8(x, r, w, invs[0], eps, delta, dtype)
            assert same_bits(r8, s_bits, dtype), "FP8 norm: residual stream"
            _check_fp8_once(orc, y, amax, v32, v64, invs,
                            lambda inv: orc.fused_add_rmsnorm_fp8(x, r, w, inv, eps, delta,
                                                                  dtype)[0],
                            f"norm fp8 ({dtype}, delta {delta}, weight {w is not None})")
        # gated activations
        d = 1024
        gu = W.to_bits(g.standard_normal((6, 2 * d)) * 1.5, dtype)
        guv = f32(gu, dtype)
        gt = torch.from_numpy(guv[:, :d].astype(np.float64))
        ut = guv[:, d:].astype(np.float64)
        for act, lib in ((W.SILU, F.silu(gt).numpy()),
                         (W.GELU_TANH, F.gelu(gt, approximate="tanh").numpy())):
            v32 = orc.gated_act(guv, act, F32)
            amax = orc.gated_act_amax(gu, act, dtype)
            invs = [np.float32(448.0 / amax), np.float32(100.0 / amax),
                    np.float32(2000.0 / amax)]
            y = orc.gated_act_fp8(gu, invs[0], act, dtype)
            _check_fp8_once(orc, y, amax, v32, lib * ut, invs,
                            lambda inv: orc.gated_act_fp8(gu, inv, act, dtype),
                            f"act fp8 ({dtype}, act {act})")
        # adaptive RMSNorm: gated residual, plain residual, no residual
        H = 512
        x = W.to_bits(g.standard_normal((6, H)), dtype)
        r = W.to_bits(g.standard_normal((6, H)) * 2, dtype)
        gt_ = W.to_bits(g.standard_normal(H) * 0.3 + 1, dtype)
        sc = W.to_bits(g.standard_normal(H) * 0.1, dtype)
        sh = W.to_bits(g.standard_normal(H) * 0.1, dtype)
        scv, shv = f32(sc, dtype), f32(sh, dtype)
        for res, gate in ((r, gt_), (r, None), (None, None)):
            if res is None:
                s_bits = x
            else:
                s_bits = orc.adarms(x, res, gate, sc, sh, eps, dtype)[1]
            sv = f32(s_bits, dtype)
            v32 = orc.adarms(sv, None, None, scv, shv, eps, F32)[0]
            n64 = F.rms_norm(torch.from_numpy(sv.astype(np.float64)), (H,), weight=None,
                             eps=float(np.float32(eps))).numpy()
            v64 = n64 * (1.0 + scv.astype(np.float64)) + shv.astype(np.float64)
            amax = orc.adarms_amax(x, res, gate, sc, sh, eps, dtype)
            invs = [np.float32(448.0 / amax), np.float32(150.0 / amax),
                    np.float32(900.0 / amax)]
            y, r8 = orc.adarms_fp8(x, res, gate, sc, sh, invs[0], eps, dtype)
            if res is not None:
                assert same_bits(r8, s_bits, dtype), "FP8 adaptive norm: residual stream"
            _check_fp8_once(orc, y, amax, v32, v64, invs,
                            lambda inv: orc.adarms_fp8(x, res, gate, sc, sh, inv, eps,
                                                       dtype)[0],
                            f"adarms fp8 ({dtype}, residual {res is not None}, "
                            f"gate {gate is not None})")


ALL_PINS = [
    pin_bf16_converter, pin_f16_converter, pin_e4m3fn_converter,
    pin_rmsnorm_vs_torch, pin_rmsnorm_closed_forms, pin_rmsnorm_bruteforce,
    pin_rmsnorm_no_weight, pin_adarms,
    pin_rope_complex, pin_rope_closed_forms, pin_rope_invariants,
    pin_prologue_composition, pin_prologue_constant_head, pin_prologue_round_once,
    pin_residual_add, pin_norm_fp8, pin_quantize_vs_torch,
    pin_act_vs_torch, pin_act_exhaustive_bf16, pin_act_single_rounding_16bit,
    pin_act_identities, pin_act_fp8,
    pin_fp8_epilogues_16bit,
]
