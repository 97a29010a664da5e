"""Comparison of HIP results with the oracle, by the tolerance rules of the
numerics contract:

* integer / bit results (the residual sum, FP8 conversion of a given fp32
  value, indexing): identical bits;
* normalised and rotated bf16 / fp16 values: at most 1 ulp apart;
* fp32 values: |a - b| <= 1e-5 |b|;
* a rotated element may exceed 1 ulp only through its inputs: a 1-ulp
  difference in a normalised value n_a or n_b moves o = n_a c -+ n_b s by up
  to (|c| + |s|) ulp(n), which can be many ulps of a cancelled o.  Such an
  element passes if |a - b| <= (|c| + |s|) max(ulp(n_a), ulp(n_b)) + ulp(o);
  the count of these escapes is reported and must stay small;
* FP8 codes computed from slightly different fp32 values: at most one code
  step apart in magnitude order.

Every check also bounds the fraction of non-identical elements: with
round-to-nearest-even on both sides a difference needs an fp32 value within
a few fp32 ulps of a rounding midpoint, which is rare; a systematic rounding
error (truncation, a wrong mode) would differ in a large fraction.
"""
import numpy as np

import workloads as W

F32, F16, BF16 = W.F32, W.F16, W.BF16


def ulp16_dist(a, b):
    a = np.asarray(a, np.uint16).astype(np.int64)
    b = np.asarray(b, np.uint16).astype(np.int64)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(oa - ob)


def spacing16(bits, dtype):
    """Distance from |v| to the next representable magnitude (one ulp)."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    if dtype == BF16:
        e = np.maximum((b >> 7) & 0xFF, 1)
        return np.exp2(e - 127 - 7)
    e = np.maximum((b >> 10) & 0x1F, 1)
    return np.exp2(e - 15 - 10)


def _partner(D, rot, layout):
    ch = np.arange(D)
    if layout == W.ROTATE_HALF:
        half = rot // 2
        return np.where(ch < half, ch + half, np.where(ch < rot, ch - half, ch))
    return np.where(ch < rot, ch ^ 1, ch)


def check_prologue(gpu, ora, n_ora, cos_sin, pos, rot, layout, dtype, max_pos=None,
                   label=""):
    """gpu, ora, n_ora: [T, H, D] (raw bits); n_ora is the oracle's rounded
    normalised value (the composition pin makes it the prologue's own)."""
    gpu, ora, n_ora = (np.asarray(x) for x in (gpu, ora, n_ora))
    T, H, D = ora.shape
    if T * H * D == 0:
        return dict(n=0)
    # a NaN matches any NaN and nothing else (a row holding a NaN is NaN
    # throughout, its rotation included)
    as_f = (lambda a: a.astype(np.float64)) if dtype == F32 else _bits_f64(dtype)
    nan_o = np.isnan(as_f(ora))
    odd = int(np.count_nonzero(np.isnan(as_f(gpu)) != nan_o))
    assert odd == 0, f"{label}: {odd} elements are NaN on one side only"
    mp = cos_sin.shape[0] if max_pos is None else max_pos
    pos = np.asarray(pos, np.int64)
    inr = (pos >= 0) & (pos < mp)
    ch = np.arange(D)
    rotated = inr[:, None, None] & (ch < rot)[None, None, :]
    rotated = np.broadcast_to(rotated, ora.shape)
    part = _partner(D, rot, layout)
    half = rot // 2
    j = np.where(layout == W.ROTATE_HALF, np.where(ch < half, ch, ch - half), ch >> 1)
    j = np.clip(j, 0, max(half - 1, 0))
    safe_pos = np.where(inr, pos, 0)
    if rot > 0 and mp > 0:
        c = cos_sin[safe_pos][:, j].astype(np.float64)[:, None, :]
        s = cos_sin[safe_pos][:, half + j].astype(np.float64)[:, None, :]
    else:
        c = np.ones((T, 1, D))
        s = np.zeros((T, 1, D))
    if dtype == F32:
        g = gpu.astype(np.float64)
        o = ora.astype(np.float64)
        n = n_ora.astype(np.float64)
        scale = np.abs(o)
        pair = np.hypot(n, n[..., part])
        scale = np.where(rotated, np.maximum(scale, pair), scale)
        with np.errstate(invalid="ignore"):
            ok = (g == o) | nan_o | (np.isfinite(o) & (np.abs(g - o) <= 1e-5 * scale + 1e-35))
        bad = int(np.count_nonzero(~ok))
        assert bad == 0, f"{label}: {bad} fp32 elements beyond rel 1e-5"
        return dict(n=ora.size, differ=int(np.count_nonzero(g != o)))
    d = np.where(nan_o, 0, ulp16_dist(gpu, ora))
    ok = d <= 1
    esc_mask = (~ok) & rotated
    if np.any(esc_mask):
        g = W.bits_to_f32(gpu, dtype).astype(np.float64)
        o = W.bits_to_f32(ora, dtype).astype(np.float64)
        sp_n = spacing16(n_ora, dtype)
        sp_np = sp_n[..., part]
        bound = (np.abs(c) + np.abs(s)) * np.maximum(sp_n, sp_np) + spacing16(ora, dtype)
        ok = ok | (rotated & (np.abs(g - o) <= bound))
    bad = int(np.count_nonzero(~ok))
    worst = int(d.max())
    assert bad == 0, f"{label}: {bad} elements beyond tolerance (max ulp {worst})"
    differ = int(np.count_nonzero(d))
    assert differ <= max(4, 0.005 * d.size), \
        f"{label}: {differ}/{d.size} elements differ (systematic rounding?)"
    return dict(n=d.size, differ=differ, escapes=int(np.count_nonzero(esc_mask)), max_ulp=worst)


def _bits_f64(dtype):
    """16-bit patterns -> float64 values; a signalling NaN pattern quietly
    becomes a NaN (numpy flags the conversion as invalid)."""
    def f(a):
        with np.errstate(invalid="ignore"):
            return W.bits_to_f32(a, dtype).astype(np.float64)
    return f


def check_values(gpu, ora, dtype, label="", max_differ_frac=0.005):
    """Normalised / activated values: <= 1 ulp (bf16, fp16) or rel 1e-5 (fp32).
    A NaN matches any NaN (sign and payload carry nothing) and nothing else;
    an infinity matches only the same infinity."""
    gpu, ora = np.asarray(gpu).ravel(), np.asarray(ora).ravel()
    if ora.size == 0:
        return dict(n=0)
    as_f = (lambda a: a.astype(np.float64)) if dtype == F32 else _bits_f64(dtype)
    gn, on = np.isnan(as_f(gpu)), np.isnan(as_f(ora))
    odd = int(np.count_nonzero(gn != on))
    assert odd == 0, f"{label}: {odd} elements are NaN on one side only"
    gpu, ora = gpu[~on], ora[~on]
    if ora.size == 0:
        return dict(n=0, nan=int(np.count_nonzero(on)))
    if dtype == F32:
        g, o = gpu.astype(np.float64), ora.astype(np.float64)
        with np.errstate(invalid="ignore"):
            ok = (g == o) | (np.isfinite(o) & (np.abs(g - o) <= 1e-5 * np.abs(o) + 1e-35))
        bad = int(np.count_nonzero(~ok))
        assert bad == 0, f"{label}: {bad} fp32 elements beyond rel 1e-5"
        return dict(n=ora.size, differ=int(np.count_nonzero(g != o)))
    d = ulp16_dist(gpu, ora)
    assert int(d.max()) <= 1, f"{label}: max ulp {int(d.max())}"
    differ = int(np.count_nonzero(d))
    assert differ <= max(4, max_differ_frac * d.size), \
        f"{label}: {differ}/{d.size} elements differ (systematic rounding?)"
    return dict(n=d.size, differ=differ, max_ulp=int(d.max()))


def check_modulated(gpu, ora, a_mag, shift_mag, H, dtype, label="", max_escape_frac=None):
    """Adaptive-norm outputs m = a + shift, a = n (1 + scale).  The rule of
    check_values, except where a and the shift cancel: both sides' n differ
    by at most ((H + 8)/2 + log2 H + 8) u |n| (the oracle's sequential sum of
    squares against the kernels' tree, the square root and the products), so
    an element may also pass within that much of |a| plus 2 u |shift| plus one
    output step.  Such escapes are counted and bounded (fp32 outputs have no
    output rounding to absorb the difference, so more of them lie past rel
    1e-5: 1 % of elements there, 0.1 % for 16-bit outputs)."""
    if max_escape_frac is None:
        max_escape_frac = 0.01 if dtype == F32 else 0.001
    gpu, ora = np.asarray(gpu), np.asarray(ora)
    if ora.size == 0:
        return dict(n=0)
    g = W.bits_to_f32(gpu, dtype).astype(np.float64) if dtype != F32 else gpu.astype(np.float64)
    o = W.bits_to_f32(ora, dtype).astype(np.float64) if dtype != F32 else ora.astype(np.float64)
    u = 2.0 ** -24
    bound = ((H + 8) / 2.0 + np.log2(H) + 8) * u * np.abs(a_mag) + 2 * u * np.abs(shift_mag)
    if dtype == F32:
        near = np.abs(g - o) <= 1e-5 * np.abs(o) + 1e-35
        step = np.spacing(np.abs(o).astype(np.float32)).astype(np.float64)
    else:
        near = ulp16_dist(gpu, ora) <= 1
        step = spacing16(ora, dtype)
    esc = ~near & (np.abs(g - o) <= bound + step)
    bad = int(np.count_nonzero(~near & ~esc))
    assert bad == 0, f"{label}: {bad} elements beyond the cancellation bound"
    escapes = int(np.count_nonzero(esc))
    assert escapes <= max(4, max_escape_frac * o.size), f"{label}: {escapes} escapes"
    differ = int(np.count_nonzero(g != o))
    if dtype != F32:
        assert differ <= max(4, 0.005 * o.size), \
            f"{label}: {differ}/{o.size} elements differ (systematic rounding?)"
    return dict(n=int(o.size), differ=differ, escapes=escapes)


def check_bitwise(gpu, ora, label=""):
    gpu, ora = np.asarray(gpu), np.asarray(ora)
    if gpu.dtype == np.float32:
        same = (gpu == ora) | (np.isnan(gpu) & np.isnan(ora))
        same &= np.signbit(gpu) == np.signbit(ora)
    else:
        same = gpu == ora
    bad = int(np.count_nonzero(~same))
    assert bad == 0, f"{label}: {bad} of {ora.size} elements not bit-identical"


def _code_order(c):
    c = np.asarray(c, np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_fp8(gpu, ora, label="", max_differ_frac=0.002):
    gpu, ora = np.asarray(gpu, np.uint8), np.asarray(ora, np.uint8)
    if ora.size == 0:
        return dict(n=0)
    nan_o = (ora & 0x7F) == 0x7F
    nan_g = (gpu & 0x7F) == 0x7F
    assert np.array_equal(nan_o, nan_g), f"{label}: NaN codes differ"
    d = np.abs(_code_order(gpu) - _code_order(ora))
    d[nan_o] = 0
    # +0 / -0 are one value
    zero = ((gpu & 0x7F) == 0) & ((ora & 0x7F) == 0)
    d[zero] = 0
    assert int(d.max()) <= 1, f"{label}: FP8 codes {int(d.max())} steps apart"
    differ = int(np.count_nonzero(d))
    assert differ <= max(4, max_differ_frac * d.size), \
        f"{label}: {differ}/{d.size} FP8 codes differ"
    return dict(n=d.size, differ=differ)
