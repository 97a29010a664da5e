"""ctypes binding of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the CPU-baseline leg of bench.py may import
this package.  It never touches a GPU and never imports the product package.

Arrays are numpy arrays holding raw element bits: uint16 for bf16 / fp16,
float32 for fp32, uint8 for e4m3fn codes.  Every call copies its inputs into
fresh contiguous arrays and returns new output arrays, so the caller's data
is never modified.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
ROTATE_HALF, INTERLEAVED = 0, 1
SILU, GELU_TANH = 0, 1

_STORAGE = {F32: np.float32, F16: np.uint16, BF16: np.uint16}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float

_SIGS = {
    "mbt_ref_bf16_to_f32": (_f32, [ctypes.c_uint16]),
    "mbt_ref_f32_to_bf16": (ctypes.c_uint16, [_f32]),
    "mbt_ref_f16_to_f32": (_f32, [ctypes.c_uint16]),
    "mbt_ref_f32_to_f16": (ctypes.c_uint16, [_f32]),
    "mbt_ref_e4m3fn_to_f32": (_f32, [ctypes.c_uint8]),
    "mbt_ref_f32_to_e4m3fn": (ctypes.c_uint8, [_f32]),
    "mbt_ref_encode": (None, [_vp, _vp, _i64, _i32]),
    "mbt_ref_decode": (None, [_vp, _vp, _i64, _i32]),
    "mbt_ref_encode_e4m3fn": (None, [_vp, _vp, _i64]),
    "mbt_ref_decode_e4m3fn": (None, [_vp, _vp, _i64]),
    "mbt_ref_rmsnorm_rows": (_i32, [_vp, _vp, _vp, _i64, _i32, _f32, _i32, _i32]),
    "mbt_ref_rope": (_i32, [_vp, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _i32, _i32]),
    "mbt_ref_qknorm_rope": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp,
                                   _i32, _i32, _i64, _i32, _i32, _f32, _i32, _i32, _i32]),
    "mbt_ref_qknorm_rope_round_once": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp,
                                   _i32, _i32, _i64, _i32, _i32, _f32, _i32, _i32, _i32]),
    "mbt_ref_fused_add_rmsnorm": (_i32, [_vp, _vp, _vp, _i64, _i32, _f32, _i32, _i32]),
    "mbt_ref_fused_add_rmsnorm_fp8": (_i32, [_vp, _vp, _vp, _vp, _f32, _i64, _i32,
                                             _f32, _i32, _i32]),
    "mbt_ref_adarms": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _f32, _i32]),
    "mbt_ref_adarms_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _i64, _i32, _f32, _i32]),
    "mbt_ref_adarms_amax": (_f32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _f32, _i32]),
    "mbt_ref_gated_act": (_i32, [_vp, _vp, _i64, _i32, _i32, _i32]),
    "mbt_ref_gated_act_fp8": (_i32, [_vp, _vp, _f32, _i64, _i32, _i32, _i32]),
    "mbt_ref_quantize_fp8": (_i32, [_vp, _vp, _i64, _f32]),
    "mbt_ref_fused_add_rmsnorm_amax": (_f32, [_vp, _vp, _vp, _i64, _i32, _f32, _i32, _i32]),
    "mbt_ref_gated_act_amax": (_f32, [_vp, _i64, _i32, _i32, _i32]),
}


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Fresh C-contiguous copy with the storage type the oracle expects
    (None stays None: a NULL pointer)."""
    if a is None:
        return None
    return np.array(a, dtype=_STORAGE[dtype] if isinstance(dtype, int) else dtype,
                    order="C", copy=True)


class OracleError(RuntimeError):
    pass


class Oracle:
    """One loaded build of the oracle (the default one, or a mutated copy)."""

    def __init__(self, path=DEFAULT_LIB):
        if not os.path.exists(path):
            raise OracleError(f"oracle library not built: {path} (run oracle/build.py)")
        self.path = path
        self._lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(self._lib, name)
            fn.restype = res
            fn.argtypes = args

    def _check(self, rc, name):
        if rc != 0:
            raise OracleError(f"{name}: oracle rejected its arguments")

    # ---- converters ------------------------------------------------------
    def encode(self, values_f32, dtype):
        v = np.ascontiguousarray(values_f32, dtype=np.float32)
        out = np.empty(v.shape, dtype=_STORAGE[dtype])
        self._lib.mbt_ref_encode(_ptr(v), _ptr(out), v.size, dtype)
        return out

    def decode(self, bits, dtype):
        b = _c(bits, dtype)
        out = np.empty(b.shape, dtype=np.float32)
        self._lib.mbt_ref_decode(_ptr(b), _ptr(out), b.size, dtype)
        return out

    def encode_e4m3fn(self, values_f32):
        v = np.ascontiguousarray(values_f32, dtype=np.float32)
        out = np.empty(v.shape, dtype=np.uint8)
        self._lib.mbt_ref_encode_e4m3fn(_ptr(v), _ptr(out), v.size)
        return out

    def decode_e4m3fn(self, codes):
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float32)
        self._lib.mbt_ref_decode_e4m3fn(_ptr(c), _ptr(out), c.size)
        return out

    # ---- row primitives --------------------------------------------------
    def rmsnorm_rows(self, x, w, eps, weight_offset, dtype):
        x = _c(x, dtype)
        D = x.shape[-1]
        y = np.empty_like(x)
        rc = self._lib.mbt_ref_rmsnorm_rows(_ptr(x), _ptr(y), _ptr(_c(w, dtype)),
                                            x.size // D, D, eps, weight_offset, dtype)
        self._check(rc, "rmsnorm_rows")
        return y

    def rope(self, x, cos_sin, pos, rot_dim, layout, dtype):
        """x: [T][heads][D]; returns the rotated copy."""
        x = _c(x, dtype)
        T, heads, D = x.shape
        cs = np.ascontiguousarray(cos_sin, dtype=np.float32)
        p = np.ascontiguousarray(pos, dtype=np.int64)
        rc = self._lib.mbt_ref_rope(_ptr(x), _ptr(cs), cs.shape[0], _ptr(p), T,
                                    heads, D, rot_dim, layout, dtype)
        self._check(rc, "rope")
        return x

    # ---- the path --------------------------------------------------------
    def qknorm_rope(self, q, k, w_q, w_k, cos_sin, pos, rot_dim, eps,
                    weight_offset, layout, dtype, max_pos=None, round_once=False):
        """q: [T][Q][D], k: [T][K][D]; returns (q_out, k_out).  round_once
        selects the single-rounding variant."""
        q = _c(q, dtype)
        k = _c(k, dtype)
        T, Q, D = q.shape
        K = k.shape[1]
        cs = np.ascontiguousarray(cos_sin, dtype=np.float32)
        p = np.ascontiguousarray(pos, dtype=np.int64)
        mp = cs.shape[0] if max_pos is None else max_pos
        qo, ko = np.empty_like(q), np.empty_like(k)
        fn = (self._lib.mbt_ref_qknorm_rope_round_once if round_once
              else self._lib.mbt_ref_qknorm_rope)
        rc = fn(
            _ptr(q), _ptr(k), _ptr(qo), _ptr(ko), _ptr(_c(w_q, dtype)),
            _ptr(_c(w_k, dtype)), _ptr(cs), mp, _ptr(p), Q, K, T, D, rot_dim,
            eps, weight_offset, layout, dtype)
        self._check(rc, "qknorm_rope")
        return qo, ko

    def fused_add_rmsnorm(self, x, residual, w, eps, weight_offset, dtype):
        """Returns (x_out, residual_out); residual may be None."""
        x = _c(x, dtype)
        H = x.shape[-1]
        r = None if residual is None else _c(residual, dtype)
        rc = self._lib.mbt_ref_fused_add_rmsnorm(_ptr(x), _ptr(r), _ptr(_c(w, dtype)),
                                                 x.size // H, H, eps, weight_offset, dtype)
        self._check(rc, "fused_add_rmsnorm")
        return x, r

    def fused_add_rmsnorm_fp8(self, x, residual, w, inv_scale, eps, weight_offset, dtype):
        """Returns (y_codes, residual_out)."""
        x = _c(x, dtype)
        H = x.shape[-1]
        r = None if residual is None else _c(residual, dtype)
        y = np.empty(x.shape, dtype=np.uint8)
        rc = self._lib.mbt_ref_fused_add_rmsnorm_fp8(
            _ptr(x), _ptr(r), _ptr(_c(w, dtype)), _ptr(y), float(inv_scale),
            x.size // H, H, eps, weight_offset, dtype)
        self._check(rc, "fused_add_rmsnorm_fp8")
        return y, r

    def fused_add_rmsnorm_amax(self, x, residual, w, eps, weight_offset, dtype):
        x = _c(x, dtype)
        H = x.shape[-1]
        r = None if residual is None else _c(residual, dtype)
        return float(self._lib.mbt_ref_fused_add_rmsnorm_amax(
            _ptr(x), _ptr(r), _ptr(_c(w, dtype)), x.size // H, H, eps,
            weight_offset, dtype))

    def adarms(self, x, residual, gate, scale, shift, eps, dtype):
        """Adaptive RMSNorm, dtype output.  Returns (x_out, residual_out)."""
        x = _c(x, dtype)
        H = x.shape[-1]
        r = None if residual is None else _c(residual, dtype)
        rc = self._lib.mbt_ref_adarms(_ptr(x), _ptr(r), _ptr(_c(gate, dtype)),
                                      _ptr(_c(scale, dtype)), _ptr(_c(shift, dtype)),
                                      x.size // H, H, eps, dtype)
        self._check(rc, "adarms")
        return x, r

    def adarms_fp8(self, x, residual, gate, scale, shift, inv_scale, eps, dtype):
        """Returns (y_codes, residual_out)."""
        x = _c(x, dtype)
        H = x.shape[-1]
        r = None if residual is None else _c(residual, dtype)
        y = np.empty(x.shape, dtype=np.uint8)
        rc = self._lib.mbt_ref_adarms_fp8(_ptr(x), _ptr(r), _ptr(_c(gate, dtype)),
                                          _ptr(_c(scale, dtype)), _ptr(_c(shift, dtype)), _ptr(y),
                                          float(inv_scale), x.size // H, H, eps, dtype)
        self._check(rc, "adarms_fp8")
        return y, r

    def adarms_amax(self, x, residual, gate, scale, shift, eps, dtype):
        x = _c(x, dtype)
        H = x.shape[-1]
        r = None if residual is None else _c(residual, dtype)
        return float(self._lib.mbt_ref_adarms_amax(
            _ptr(x), _ptr(r), _ptr(_c(gate, dtype)), _ptr(_c(scale, dtype)),
            _ptr(_c(shift, dtype)), x.size // H, H, eps, dtype))

    def gated_act(self, gate_up, act, dtype):
        gu = _c(gate_up, dtype)
        d = gu.shape[-1] // 2
        T = gu.size // (2 * d)
        out = np.empty(gu.shape[:-1] + (d,), dtype=_STORAGE[dtype])
        rc = self._lib.mbt_ref_gated_act(_ptr(gu), _ptr(out), T, d, act, dtype)
        self._check(rc, "gated_act")
        return out

    def gated_act_fp8(self, gate_up, inv_scale, act, dtype):
        gu = _c(gate_up, dtype)
        d = gu.shape[-1] // 2
        T = gu.size // (2 * d)
        out = np.empty(gu.shape[:-1] + (d,), dtype=np.uint8)
        rc = self._lib.mbt_ref_gated_act_fp8(_ptr(gu), _ptr(out), float(inv_scale), T, d, act,
                                              dtype)
        self._check(rc, "gated_act_fp8")
        return out

    def gated_act_amax(self, gate_up, act, dtype):
        gu = _c(gate_up, dtype)
        d = gu.shape[-1] // 2
        return float(self._lib.mbt_ref_gated_act_amax(_ptr(gu), gu.size // (2 * d), d,
                                                      act, dtype))

    def quantize_fp8(self, x, inv_scale):
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty(x.shape, dtype=np.uint8)
        self._check(self._lib.mbt_ref_quantize_fp8(_ptr(x), _ptr(y), x.size, float(inv_scale)),
                    "quantize_fp8")
        return y


_DEFAULT = None


def default():
    """The unmutated oracle, built on first use if it is missing."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(DEFAULT_LIB):
            from . import build as _build
            _build.build()
        _DEFAULT = Oracle(DEFAULT_LIB)
    return _DEFAULT
