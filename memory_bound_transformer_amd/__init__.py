"""Python binding of libmbt: fused memory-bound decoder ops on MI355X.

Argument marshalling only.  Every operation runs in the HIP kernels of
libmbt.so (built in-tree by ``python -m memory_bound_transformer_amd.build``);
PyTorch supplies device memory and the current stream.  There is no CPU or
eager fallback: if the library is missing, importing this package fails.

The entry points mirror include/mbt.h:

    qknorm_rope            fused per-head QK-RMSNorm + RoPE prologue
    qknorm_rope_ex         the same on strided views, optional single rounding
    qkv_norm_rope_cache    the prologue on a fused QKV buffer + KV-cache write
    rope                   standalone rotary embedding, in place
    fused_add_rmsnorm      residual add + RMSNorm, in place
    fused_add_rmsnorm_fp8  the same with static-scale e4m3fn output
    fused_add_rmsnorm_amax calibration pass (amax of the FP8 input)
    adarms                 adaptive RMSNorm (style scale / shift / gate), in place
    adarms_fp8             the same with static-scale e4m3fn output
    adarms_amax            its calibration pass
    gated_act              SiLU / GELU-tanh gated activation
    gated_act_fp8          the same with static-scale e4m3fn output
    gated_act_amax         calibration pass
    quantize_fp8           standalone static e4m3fn quantization
"""
import ctypes
import os

import torch

__all__ = [
    "qknorm_rope", "qknorm_rope_ex", "qkv_norm_rope_cache", "rope", "fused_add_rmsnorm", "fused_add_rmsnorm_fp8", "fused_add_rmsnorm_amax",
    "adarms", "adarms_fp8", "adarms_amax", "gated_act", "gated_act_fp8", "gated_act_amax", "quantize_fp8", "MbtError",
    "ROTATE_HALF", "INTERLEAVED", "SILU", "GELU_TANH", "LIB_PATH", "abi_version",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmbt.so")

ROTATE_HALF, INTERLEAVED = 0, 1
ROUND_ONCE = 1                      # MBT_QK_ROUND_ONCE
SILU, GELU_TANH = 0, 1
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libmbt.so is not built ({LIB_PATH}); run: python -m memory_bound_transformer_amd.build")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_SIGS = {
    "mbt_qknorm_rope": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32, _i32, _i64, _i32,
                        _i32, _f32, _i32, _i32, _i32, _vp],
    "mbt_qknorm_rope_ex": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32, _i32, _i64, _i32,
                           _i32, _f32, _i32, _i32, _i32, _i64, _i64, _i64, _i64, _i32, _vp],
    "mbt_qkv_norm_rope_cache": [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _i32,
                                _i32, _i64, _i32, _i32, _f32, _i32, _i32, _i32, _i32, _vp],
    "mbt_rope": [_vp, _vp, _vp, _i64, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _vp],
    "mbt_fused_add_rmsnorm": [_vp, _vp, _vp, _i64, _i32, _f32, _i32, _i32, _vp],
    "mbt_fused_add_rmsnorm_fp8": [_vp, _vp, _vp, _vp, _f32, _i64, _i32, _f32, _i32, _i32, _vp],
    "mbt_fused_add_rmsnorm_amax": [_vp, _vp, _vp, _vp, _i64, _i32, _f32, _i32, _i32, _vp],
    "mbt_adarms": [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _f32, _i32, _vp],
    "mbt_adarms_fp8": [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _i64, _i32, _f32, _i32, _vp],
    "mbt_adarms_amax": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _f32, _i32, _vp],
    "mbt_gated_act": [_vp, _vp, _i64, _i32, _i32, _i32, _vp],
    "mbt_gated_act_fp8": [_vp, _vp, _f32, _i64, _i32, _i32, _i32, _vp],
    "mbt_gated_act_amax": [_vp, _vp, _i64, _i32, _i32, _i32, _vp],
    "mbt_quantize_fp8": [_vp, _vp, _i64, _f32, _vp],
    "mbt_stream_copy": [_vp, _vp, _i64, _i32, _i32, _vp],
}
for _name, _args in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int
_lib.mbt_status_string.argtypes = [ctypes.c_int]
_lib.mbt_status_string.restype = ctypes.c_char_p
_lib.mbt_last_error.argtypes = []
_lib.mbt_last_error.restype = ctypes.c_char_p
_lib.mbt_abi_version.argtypes = []
_lib.mbt_abi_version.restype = ctypes.c_int32


class MbtError(RuntimeError):
    """A libmbt call returned a non-OK status."""

    def __init__(self, status, detail):
        self.status = status
        name = _lib.mbt_status_string(status).decode()
        super().__init__(f"{name}: {detail}")


def abi_version():
    return int(_lib.mbt_abi_version())


def _check(status):
    if status != 0:
        raise MbtError(status, _lib.mbt_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")


def _on_current_gpu(tensors, current_device=None):
    """Every tensor on the current GPU.  The kernels run on the device of
    the stream they are given (the current device's, by default) and
    address every pointer from there, so a tensor on another GPU would be
    read and written from the wrong device."""
    cur = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libmbt operates on GPU tensors only")
        if cur is None:
            cur = (current_device or torch.cuda.current_device)()
        if t.device.index != cur:
            raise ValueError(f"a tensor is on {t.device} but the current device is cuda:{cur}; "
                             f"call inside torch.cuda.device({t.device.index})")


def _dev(*tensors):
    _on_current_gpu(tensors)
    for t in tensors:
        if t is not None and not t.is_contiguous():
            raise ValueError("libmbt needs contiguous tensors")


def _stream(stream, current_device=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    cur = (current_device or torch.cuda.current_device)()
    if stream.device.index != cur:
        raise ValueError(f"stream is on {stream.device} but the current device is cuda:{cur}")
    return stream.cuda_stream


def _same_dtype(ref, *tensors):
    for t in tensors:
        if t is not None and t.dtype != ref.dtype:
            raise TypeError(f"dtype mismatch: {t.dtype} vs {ref.dtype}")


# The C ABI takes sizes on trust; these checks make every tensor handed over
# at least as large as the sizes passed with it, so a mismatch is an error
# here rather than an out-of-bounds access on the GPU.
def _shape(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _numel(t, n, name):
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")


def _codes(t, shape, name):
    if t is not None:
        _shape(t, shape, name)
        if t.dtype != torch.uint8:
            raise TypeError(f"{name} must be uint8 (e4m3fn codes)")


def _amax_out(t):
    if t is not None and (t.dtype != torch.float32 or t.numel() < 1):
        raise TypeError("amax must be a float32 tensor of at least one element")


def _rows(x, name="x"):
    """(T, H) of a tensor of rows, H its last dimension."""
    if x.dim() < 1 or x.shape[-1] < 1:
        raise ValueError(f"{name} needs a non-empty last dimension")
    return x.numel() // x.shape[-1], x.shape[-1]


def _norm_args(x, residual, w):
    T, H = _rows(x)
    _shape(residual, x.shape, "residual")
    _numel(w, H, "w")
    return T, H


def _ada_args(x, residual, gate, scale, shift):
    T, H = _rows(x)
    _shape(residual, x.shape, "residual")
    for t, n in ((gate, "gate"), (scale, "scale"), (shift, "shift")):
        _numel(t, H, n)
    return T, H


def _act_rows(gate_up):
    """(T, d) of gate_up [..., 2d]."""
    if gate_up.dim() < 1 or gate_up.shape[-1] < 2 or gate_up.shape[-1] % 2:
        raise ValueError("gate_up must end in an even dimension 2d >= 2")
    return gate_up.numel() // gate_up.shape[-1], gate_up.shape[-1] // 2


def _heads3(t, name):
    if t.dim() != 3:
        raise ValueError(f"{name} must be [T, heads, head_dim]")
    return t.shape


def _rope_tables(cos_sin, pos, T, rot_dim, max_pos):
    """pos int64 [T]; cos_sin float32 [rows, rot_dim] (cos | sin).  Returns
    the max_pos to pass: the rows of the cache unless a smaller one is given."""
    if pos.dtype != torch.int64:
        raise TypeError("pos must be int64")
    _numel(pos, T, "pos")
    if cos_sin is None:
        if max_pos:
            raise ValueError("cos_sin is required when max_pos > 0")
        return 0
    if cos_sin.dtype != torch.float32:
        raise TypeError("cos_sin must be float32")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != rot_dim:
        raise ValueError(f"cos_sin must be [max_pos, rot_dim={rot_dim}], got "
                         f"{tuple(cos_sin.shape)}")
    mp = cos_sin.shape[0] if max_pos is None else int(max_pos)
    if not 0 <= mp <= cos_sin.shape[0]:
        raise ValueError(f"max_pos {mp} must lie in [0, {cos_sin.shape[0]}] (rows of cos_sin)")
    return mp


def qknorm_rope(q, k, w_q, w_k, cos_sin, pos, rot_dim, eps=1e-6, weight_offset=0,
                layout=ROTATE_HALF, q_out=None, k_out=None, max_pos=None, stream=None):
    """q [T, Q, D], k [T, K, D] -> (q_out, k_out) of the same shapes.
    Pass q_out=q / k_out=k for the in-place form.  cos_sin is float32
    [max_pos, rot_dim] (cos | sin), pos int64 [T]."""
    _dev(q, k, w_q, w_k, cos_sin, pos, q_out, k_out)
    _same_dtype(q, k, w_q, w_k, q_out, k_out)
    T, Q, D = _heads3(q, "q")
    K = _heads3(k, "k")[1]
    _shape(k, (T, K, D), "k")
    _shape(q_out, q.shape, "q_out")
    _shape(k_out, k.shape, "k_out")
    _numel(w_q if Q else None, D, "w_q")
    _numel(w_k if K else None, D, "w_k")
    mp = _rope_tables(cos_sin, pos, T, rot_dim, max_pos)
    if q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = torch.empty_like(k)
    _check(_lib.mbt_qknorm_rope(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(w_q),
                                _ptr(w_k), _ptr(cos_sin), mp, _ptr(pos), Q, K, T, D, rot_dim,
                                eps, weight_offset, layout, _dtype(q), _stream(stream)))
    return q_out, k_out


def _token_stride(t, name):
    """Token stride (elements) of a [T, heads, D] view whose heads of one
    token are contiguous; the tokens may be any distance apart."""
    if t.dim() != 3:
        raise ValueError(f"{name} must be [T, heads, head_dim]")
    if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{name}: the heads of one token must be contiguous")
    row = t.shape[1] * t.shape[2]
    if t.shape[0] <= 1:
        return row
    # A broadcast (expand()ed) view has token stride 0, and the C ABI reads
    # 0 as "dense": it would then address T rows where the allocation holds
    # one.  Any stride below a token's row would make tokens overlap.
    if row and t.stride(0) < row:
        raise ValueError(f"{name}: token stride {t.stride(0)} is below one token's "
                         f"{row} elements (a broadcast or overlapping view)")
    return t.stride(0)


def qknorm_rope_ex(q_in, k_in, w_q, w_k, cos_sin, pos, rot_dim, eps=1e-6, weight_offset=0,
                   layout=ROTATE_HALF, q_out=None, k_out=None, round_once=False, max_pos=None,
                   stream=None):
    """mbt_qknorm_rope on strided [T, heads, D] views (e.g. q and k slices of
    a fused QKV buffer), with the single-rounding variant on request.  Pass
    q_out=q_in / k_out=k_in for the in-place form."""
    _on_current_gpu((q_in, k_in, w_q, w_k, cos_sin, pos, q_out, k_out))
    for t in (w_q, w_k, cos_sin, pos):
        if t is not None and not t.is_contiguous():
            raise ValueError("weights, cos_sin and pos must be contiguous")
    _same_dtype(q_in, k_in, w_q, w_k, q_out, k_out)
    T, Q, D = _heads3(q_in, "q_in")
    K = _heads3(k_in, "k_in")[1]
    _shape(k_in, (T, K, D), "k_in")
    _shape(q_out, (T, Q, D), "q_out")
    _shape(k_out, (T, K, D), "k_out")
    _numel(w_q if Q else None, D, "w_q")
    _numel(w_k if K else None, D, "w_k")
    mp = _rope_tables(cos_sin, pos, T, rot_dim, max_pos)
    if q_out is None:
        q_out = torch.empty((T, Q, D), dtype=q_in.dtype, device=q_in.device)
    if k_out is None:
        k_out = torch.empty((T, K, D), dtype=k_in.dtype, device=k_in.device)
    st = [_token_stride(t, n) for t, n in ((q_in, "q_in"), (k_in, "k_in"), (q_out, "q_out"),
                                           (k_out, "k_out"))]
    _check(_lib.mbt_qknorm_rope_ex(_ptr(q_in), _ptr(k_in), _ptr(q_out), _ptr(k_out), _ptr(w_q),
                                   _ptr(w_k), _ptr(cos_sin), mp, _ptr(pos), Q, K, T, D, rot_dim,
                                   eps, weight_offset, layout, _dtype(q_in), *st,
                                   ROUND_ONCE if round_once else 0, _stream(stream)))
    return q_out, k_out


def qkv_norm_rope_cache(qkv, w_q, w_k, cos_sin, pos, slot, k_cache, v_cache, Q, rot_dim,
                        eps=1e-6, weight_offset=0, layout=ROTATE_HALF, q_out=None,
                        round_once=False, max_pos=None, stream=None):
    """qkv [T, Q + 2K, D] -> q_out [T, Q, D]; the prologue's key heads and
    the unchanged value heads of token t go to row slot[t] of
    k_cache / v_cache [n_slots, K, D] (slots outside [0, n_slots): no write).
    Tokens sharing a slot race for its row: each element holds one of
    theirs, which one is unspecified."""
    _dev(qkv, w_q, w_k, cos_sin, pos, slot, k_cache, v_cache, q_out)
    _same_dtype(qkv, w_q, w_k, k_cache, v_cache, q_out)
    if slot.dtype != torch.int64:
        raise TypeError("slot must be int64")
    T, QKV, D = _heads3(qkv, "qkv")
    K = (QKV - Q) // 2
    if K < 1 or Q + 2 * K != QKV:
        raise ValueError("qkv must be [T, Q + 2K, head_dim] with K >= 1")
    if k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != (K, D) or \
            v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [n_slots, K, head_dim]")
    _numel(slot, T, "slot")
    _shape(q_out, (T, Q, D), "q_out")
    _numel(w_q if Q else None, D, "w_q")
    _numel(w_k, D, "w_k")
    mp = _rope_tables(cos_sin, pos, T, rot_dim, max_pos)
    if q_out is None:
        q_out = torch.empty((T, Q, D), dtype=qkv.dtype, device=qkv.device)
    _check(_lib.mbt_qkv_norm_rope_cache(_ptr(qkv), _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(slot), k_cache.shape[0], _ptr(w_q), _ptr(w_k),
                                        _ptr(cos_sin), mp, _ptr(pos), Q, K, T, D, rot_dim, eps,
                                        weight_offset, layout, _dtype(qkv),
                                        ROUND_ONCE if round_once else 0, _stream(stream)))
    return q_out


def rope(q, k, cos_sin, pos, rot_dim, layout=ROTATE_HALF, max_pos=None, stream=None):
    """In place: rotate the first rot_dim channels of q [T, Q, D] and
    k [T, K, D] by cos_sin[pos[t]]; tokens outside the cache are untouched."""
    _dev(q, k, cos_sin, pos)
    _same_dtype(q, k)
    T, Q, D = _heads3(q, "q")
    K = _heads3(k, "k")[1]
    _shape(k, (T, K, D), "k")
    mp = _rope_tables(cos_sin, pos, T, rot_dim, max_pos)
    _check(_lib.mbt_rope(_ptr(q), _ptr(k), _ptr(cos_sin), mp, _ptr(pos), Q, K, T, D, rot_dim,
                         layout, _dtype(q), _stream(stream)))
    return q, k


def fused_add_rmsnorm(x, residual, w, eps=1e-6, weight_offset=0, stream=None):
    """In place: residual <- R(x + residual); x <- RMSNorm of it.  x [T, H]."""
    _dev(x, residual, w)
    _same_dtype(x, residual, w)
    T, H = _norm_args(x, residual, w)
    _check(_lib.mbt_fused_add_rmsnorm(_ptr(x), _ptr(residual), _ptr(w), T, H, eps,
                                      weight_offset, _dtype(x), _stream(stream)))
    return x


def fused_add_rmsnorm_fp8(x, residual, w, inv_scale, eps=1e-6, weight_offset=0, y=None,
                          stream=None):
    """residual <- R(x + residual); returns y = e4m3fn codes (uint8 [T, H])."""
    _dev(x, residual, w, y)
    _same_dtype(x, residual, w)
    T, H = _norm_args(x, residual, w)
    _codes(y, x.shape, "y")
    if y is None:
        y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.mbt_fused_add_rmsnorm_fp8(_ptr(x), _ptr(residual), _ptr(w), _ptr(y),
                                          float(inv_scale), T, H, eps,
                                          weight_offset, _dtype(x), _stream(stream)))
    return y


def fused_add_rmsnorm_amax(x, residual, w, eps=1e-6, weight_offset=0, amax=None,
                           stream=None):
    """Calibration pass: returns a float32 [1] device tensor holding
    max(amax_in, max |normalised value|).  A new `amax` starts at 0."""
    _dev(x, residual, w, amax)
    _same_dtype(x, residual, w)
    T, H = _norm_args(x, residual, w)
    _amax_out(amax)
    if amax is None:
        amax = torch.zeros(1, dtype=torch.float32, device=x.device)
    _check(_lib.mbt_fused_add_rmsnorm_amax(_ptr(x), _ptr(residual), _ptr(w), _ptr(amax),
                                           T, H, eps, weight_offset, _dtype(x),
                                           _stream(stream)))
    return amax


def adarms(x, residual, gate, scale, shift, eps=1e-6, stream=None):
    """In place: residual <- R(residual + gate * x) (gate None: 1);
    x <- R(RMSNorm(s) * (1 + scale) + shift).  x [T, H]; scale, shift,
    gate [H]."""
    _dev(x, residual, gate, scale, shift)
    _same_dtype(x, residual, gate, scale, shift)
    T, H = _ada_args(x, residual, gate, scale, shift)
    _check(_lib.mbt_adarms(_ptr(x), _ptr(residual), _ptr(gate), _ptr(scale), _ptr(shift),
                           T, H, eps, _dtype(x), _stream(stream)))
    return x


def adarms_fp8(x, residual, gate, scale, shift, inv_scale, eps=1e-6, y=None, stream=None):
    """residual <- R(residual + gate * x); returns e4m3fn codes (uint8
    [T, H]) of (RMSNorm(s) * (1 + scale) + shift) * inv_scale."""
    _dev(x, residual, gate, scale, shift, y)
    _same_dtype(x, residual, gate, scale, shift)
    T, H = _ada_args(x, residual, gate, scale, shift)
    _codes(y, x.shape, "y")
    if y is None:
        y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.mbt_adarms_fp8(_ptr(x), _ptr(residual), _ptr(gate), _ptr(scale), _ptr(shift),
                               _ptr(y), float(inv_scale), T, H, eps, _dtype(x),
                               _stream(stream)))
    return y


def adarms_amax(x, residual, gate, scale, shift, eps=1e-6, amax=None, stream=None):
    _dev(x, residual, gate, scale, shift, amax)
    _same_dtype(x, residual, gate, scale, shift)
    T, H = _ada_args(x, residual, gate, scale, shift)
    _amax_out(amax)
    if amax is None:
        amax = torch.zeros(1, dtype=torch.float32, device=x.device)
    _check(_lib.mbt_adarms_amax(_ptr(x), _ptr(residual), _ptr(gate), _ptr(scale), _ptr(shift),
                                _ptr(amax), T, H, eps, _dtype(x), _stream(stream)))
    return amax


def gated_act(gate_up, act=SILU, out=None, stream=None):
    """gate_up [T, 2d] = [g | u] -> out [T, d] = R(act(g) * u)."""
    _dev(gate_up, out)
    _same_dtype(gate_up, out)
    T, d = _act_rows(gate_up)
    _shape(out, gate_up.shape[:-1] + (d,), "out")
    if out is None:
        out = torch.empty(gate_up.shape[:-1] + (d,), dtype=gate_up.dtype, device=gate_up.device)
    _check(_lib.mbt_gated_act(_ptr(gate_up), _ptr(out), T, d, act, _dtype(gate_up),
                              _stream(stream)))
    return out


def gated_act_fp8(gate_up, inv_scale, act=SILU, out=None, stream=None):
    """gate_up [T, 2d] -> e4m3fn codes (uint8 [T, d]) of act(g) * u * inv_scale."""
    _dev(gate_up, out)
    T, d = _act_rows(gate_up)
    _codes(out, gate_up.shape[:-1] + (d,), "out")
    if out is None:
        out = torch.empty(gate_up.shape[:-1] + (d,), dtype=torch.uint8, device=gate_up.device)
    _check(_lib.mbt_gated_act_fp8(_ptr(gate_up), _ptr(out), float(inv_scale), T, d, act,
                                  _dtype(gate_up), _stream(stream)))
    return out


def gated_act_amax(gate_up, act=SILU, amax=None, stream=None):
    _dev(gate_up, amax)
    T, d = _act_rows(gate_up)
    _amax_out(amax)
    if amax is None:
        amax = torch.zeros(1, dtype=torch.float32, device=gate_up.device)
    _check(_lib.mbt_gated_act_amax(_ptr(gate_up), _ptr(amax), T, d, act, _dtype(gate_up),
                                   _stream(stream)))
    return amax


def quantize_fp8(x, inv_scale, y=None, stream=None):
    """float32 x -> e4m3fn codes (uint8, same shape) of x * inv_scale."""
    _dev(x, y)
    if x.dtype != torch.float32:
        raise TypeError("quantize_fp8 takes float32 input")
    _codes(y, x.shape, "y")
    if y is None:
        y = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.mbt_quantize_fp8(_ptr(x), _ptr(y), x.numel(), float(inv_scale),
                                 _stream(stream)))
    return y


def stream_copy(src, dst, chunks_per_lane=1, block_sync=False, stream=None):
    """Calibration copy of src's bytes into dst (same byte count, 16-byte
    aligned, disjoint) with the kernels' streaming loads and stores;
    block_sync: every load of a block lands before any of its stores."""
    _dev(src, dst)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError(f"dst holds {dst.numel() * dst.element_size()} bytes, src {n}")
    _check(_lib.mbt_stream_copy(_ptr(src), _ptr(dst), n, int(chunks_per_lane),
                                int(bool(block_sync)), _stream(stream)))
    return dst
