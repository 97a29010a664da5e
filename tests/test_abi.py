"""The C ABI on the CPU: libmbt.so loads, exports exactly the functions
include/mbt.h declares, and rejects every invalid argument with its
documented status before any HIP call (validation comes first, so these
calls never reach the runtime and need no GPU).  No valid compute call is
made here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mbt.h")
LIB = os.path.join(ROOT, "memory_bound_transformer_amd", "libmbt.so")

OK, NULLP, SHAPE, DTYPE, ENUM, SCALAR, ALIAS, HIP, ALIGN = range(9)
BF16, F16, F32 = 2, 1, 0
NAN = float("nan")
INF = float("inf")


def declared():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^MBT_API [^(]*?\b(mbt_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmbt.so not built: run python -m memory_bound_transformer_amd.build")
    lib = ctypes.CDLL(LIB)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sigs = {
        "mbt_qknorm_rope": [vp, vp, vp, vp, vp, vp, vp, i64, vp, i32, i32, i64, i32, i32, f32,
                            i32, i32, i32, vp],
        "mbt_qknorm_rope_ex": [vp, vp, vp, vp, vp, vp, vp, i64, vp, i32, i32, i64, i32, i32,
                               f32, i32, i32, i32, i64, i64, i64, i64, i32, vp],
        "mbt_qkv_norm_rope_cache": [vp, vp, vp, vp, vp, i64, vp, vp, vp, i64, vp, i32, i32, i64,
                                    i32, i32, f32, i32, i32, i32, i32, vp],
        "mbt_rope": [vp, vp, vp, i64, vp, i32, i32, i64, i32, i32, i32, i32, vp],
        "mbt_fused_add_rmsnorm": [vp, vp, vp, i64, i32, f32, i32, i32, vp],
        "mbt_fused_add_rmsnorm_fp8": [vp, vp, vp, vp, f32, i64, i32, f32, i32, i32, vp],
        "mbt_fused_add_rmsnorm_amax": [vp, vp, vp, vp, i64, i32, f32, i32, i32, vp],
        "mbt_adarms": [vp, vp, vp, vp, vp, i64, i32, f32, i32, vp],
        "mbt_adarms_fp8": [vp, vp, vp, vp, vp, vp, f32, i64, i32, f32, i32, vp],
        "mbt_adarms_amax": [vp, vp, vp, vp, vp, vp, i64, i32, f32, i32, vp],
        "mbt_gated_act": [vp, vp, i64, i32, i32, i32, vp],
        "mbt_gated_act_fp8": [vp, vp, f32, i64, i32, i32, i32, vp],
        "mbt_gated_act_amax": [vp, vp, i64, i32, i32, i32, vp],
        "mbt_quantize_fp8": [vp, vp, i64, f32, vp],
        "mbt_stream_copy": [vp, vp, i64, i32, i32, vp],
    }
    for name, args in sigs.items():
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = ctypes.c_int
    lib.mbt_status_string.argtypes = [ctypes.c_int]
    lib.mbt_status_string.restype = ctypes.c_char_p
    lib.mbt_last_error.restype = ctypes.c_char_p
    lib.mbt_abi_version.restype = ctypes.c_int32
    return lib


def test_exports_match_header(lib):
    names = declared()
    assert len(names) == 18
    for n in names:
        assert hasattr(lib, n), f"{n} declared in mbt.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T mbt_" in l})
    assert exported == names, "exported mbt_* symbols differ from the header"


def test_version_and_strings(lib):
    assert lib.mbt_abi_version() == 1
    for s, name in enumerate(["MBT_OK", "MBT_ERR_NULL_POINTER", "MBT_ERR_BAD_SHAPE",
                              "MBT_ERR_BAD_DTYPE", "MBT_ERR_BAD_ENUM", "MBT_ERR_BAD_SCALAR",
                              "MBT_ERR_ALIAS", "MBT_ERR_HIP", "MBT_ERR_ALIGN"]):
        assert lib.mbt_status_string(s).decode() == name


# fake, never dereferenced addresses: every call below fails validation
A = 0x7F0000000000
B = 0x7F0001000000
C = 0x7F0002000000
D_ = 0x7F0003000000
W1 = 0x7F0004000000
W2 = 0x7F0005000000
CS = 0x7F0006000000
POS = 0x7F0007000000


def qk(lib, **kw):
    a = dict(q_in=A, k_in=B, q_out=C, k_out=D_, w_q=W1, w_k=W2, cos_sin=CS, max_pos=4096,
             pos=POS, Q=16, K=2, T=8, head_dim=256, rot_dim=64, eps=1e-6, weight_offset=1,
             layout=0, dtype=BF16)
    a.update(kw)
    return lib.mbt_qknorm_rope(a["q_in"], a["k_in"], a["q_out"], a["k_out"], a["w_q"],
                               a["w_k"], a["cos_sin"], a["max_pos"], a["pos"], a["Q"], a["K"],
                               a["T"], a["head_dim"], a["rot_dim"], a["eps"],
                               a["weight_offset"], a["layout"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(layout=2), ENUM), (dict(weight_offset=2), ENUM),
    (dict(Q=0, K=0), SHAPE), (dict(Q=-1), SHAPE), (dict(T=-1), SHAPE),
    (dict(Q=(1 << 20) + 1), SHAPE), (dict(Q=2**31 - 1, K=2**31 - 1), SHAPE),
    (dict(head_dim=0), SHAPE), (dict(head_dim=513), SHAPE),
    (dict(rot_dim=63), SHAPE), (dict(rot_dim=258), SHAPE), (dict(rot_dim=-2), SHAPE),
    (dict(eps=NAN), SCALAR), (dict(eps=-1e-6), SCALAR), (dict(eps=INF), SCALAR),
    (dict(max_pos=-1), SCALAR),
    (dict(T=1 << 40), SHAPE),
    (dict(pos=None), NULLP), (dict(q_in=None), NULLP), (dict(w_k=None), NULLP),
    (dict(cos_sin=None), NULLP),
    (dict(q_in=A + 1), ALIGN), (dict(pos=POS + 4), ALIGN), (dict(cos_sin=CS + 2), ALIGN),
    (dict(dtype=F32, k_out=D_ + 2), ALIGN),
    (dict(q_out=A + 2), ALIAS),                  # partial overlap of q_out and q_in
    (dict(k_out=A), ALIAS),                      # k_out on top of q_in
    (dict(q_out=W1), ALIAS),                     # output over the weight
    (dict(k_out=C + 512), ALIAS),                # k_out inside q_out
    (dict(q_out=POS - 256), ALIAS),              # output over the positions
])
def test_qknorm_rope_rejects(lib, kw, status):
    assert qk(lib, **kw) == status
    assert lib.mbt_last_error().decode() != ""


def test_qknorm_rope_empty_is_noop(lib):
    # T = 0 succeeds without any pointer
    assert qk(lib, T=0, q_in=None, k_in=None, q_out=None, k_out=None, w_q=None, w_k=None,
              cos_sin=None, pos=None) == OK
    assert lib.mbt_last_error().decode() == ""


def test_norm_rejects(lib):
    f = lib.mbt_fused_add_rmsnorm
    assert f(A, B, W1, 4, 2560, 1e-6, 0, 7, None) == DTYPE
    assert f(A, B, W1, 4, 2560, 1e-6, 3, BF16, None) == ENUM
    assert f(A, B, W1, 4, 0, 1e-6, 0, BF16, None) == SHAPE
    assert f(A, B, W1, 4, (1 << 28) + 1, 1e-6, 0, BF16, None) == SHAPE
    assert f(A, B, W1, -1, 8, 1e-6, 0, BF16, None) == SHAPE
    assert f(A, B, W1, 4, 8, NAN, 0, BF16, None) == SCALAR
    assert f(None, B, W1, 4, 8, 1e-6, 0, BF16, None) == NULLP
    assert f(A, B, None, 4, 8, 1e-6, 1, BF16, None) == NULLP     # no weight needs offset 0
    # no weight with offset 0 passes the pointer check (each call below still
    # fails later, on alignment or aliasing, so nothing is launched)
    assert f(A + 1, B, None, 4, 8, 1e-6, 0, BF16, None) == ALIGN
    assert f(A, A + 16, None, 4, 8, 1e-6, 0, BF16, None) == ALIAS
    assert f(A + 1, B, W1, 4, 8, 1e-6, 0, BF16, None) == ALIGN
    assert f(A, A, W1, 4, 8, 1e-6, 0, BF16, None) == ALIAS       # residual == x
    assert f(A, A + 16, W1, 4, 8, 1e-6, 0, BF16, None) == ALIAS  # residual inside x
    assert f(A, B, A + 8, 4, 8, 1e-6, 0, BF16, None) == ALIAS    # weight inside x
    assert f(None, None, None, 0, 8, 1e-6, 0, BF16, None) == OK  # empty
    g = lib.mbt_fused_add_rmsnorm_fp8
    assert g(A, B, W1, C, 0.0, 4, 8, 1e-6, 0, BF16, None) == SCALAR
    assert g(A, B, W1, C, INF, 4, 8, 1e-6, 0, BF16, None) == SCALAR
    assert g(A, B, W1, None, 1.0, 4, 8, 1e-6, 0, BF16, None) == NULLP
    assert g(A, B, None, C, 1.0, 4, 8, 1e-6, 1, BF16, None) == NULLP
    assert g(A, B, None, B + 3, 1.0, 4, 8, 1e-6, 0, BF16, None) == ALIAS
    assert g(A, B, W1, B + 3, 1.0, 4, 8, 1e-6, 0, BF16, None) == ALIAS  # y inside residual
    h = lib.mbt_fused_add_rmsnorm_amax
    assert h(A, B, W1, None, 4, 8, 1e-6, 0, BF16, None) == NULLP
    assert h(A, B, None, C, 4, 8, 1e-6, 1, BF16, None) == NULLP
    assert h(A, B, None, C + 2, 4, 8, 1e-6, 0, BF16, None) == ALIGN
    assert h(A, B, W1, C + 2, 4, 8, 1e-6, 0, BF16, None) == ALIGN
    assert h(A, B, W1, A + 4, 4, 8, 1e-6, 0, BF16, None) == ALIAS


def test_act_rejects(lib):
    f = lib.mbt_gated_act
    assert f(A, B, 4, 10240, 2, BF16, None) == ENUM
    assert f(A, B, 4, 10240, 0, 9, None) == DTYPE
    assert f(A, B, 4, 0, 0, BF16, None) == SHAPE
    assert f(A, B, 4, 2**31 - 1, 0, BF16, None) == SHAPE
    assert f(A, B, -2, 16, 0, BF16, None) == SHAPE
    assert f(None, B, 4, 16, 0, BF16, None) == NULLP
    assert f(A, None, 4, 16, 0, BF16, None) == NULLP
    assert f(A, B + 1, 4, 16, 0, BF16, None) == ALIGN
    assert f(A, A + 64, 4, 16, 0, BF16, None) == ALIAS
    assert f(None, None, 0, 16, 1, BF16, None) == OK
    g = lib.mbt_gated_act_fp8
    assert g(A, B, -1.0, 4, 16, 0, BF16, None) == SCALAR
    assert g(A, B, NAN, 4, 16, 0, BF16, None) == SCALAR
    assert g(A, A + 100, 1.0, 4, 16, 0, BF16, None) == ALIAS
    h = lib.mbt_gated_act_amax
    assert h(A, None, 4, 16, 0, BF16, None) == NULLP
    assert h(A, A, 4, 16, 0, BF16, None) == ALIAS
    q = lib.mbt_quantize_fp8
    assert q(A, B, -1, 1.0, None) == SHAPE
    assert q(A, B, 16, 0.0, None) == SCALAR
    assert q(A + 2, B, 16, 1.0, None) == ALIGN
    assert q(A, A + 8, 16, 1.0, None) == ALIAS
    assert q(None, None, 0, 1.0, None) == OK


def test_stream_copy_rejects(lib):
    c = lib.mbt_stream_copy
    assert c(A, B, -16, 1, 0, None) == SHAPE
    assert c(A, B, 24, 1, 0, None) == SHAPE         # not a multiple of 16
    assert c(A, B, 2**40 + 16, 1, 0, None) == SHAPE
    assert c(A, B, 4096, 3, 0, None) == ENUM
    assert c(A, B, 4096, 16, 1, None) == ENUM
    assert c(A, B, 4096, 4, 2, None) == ENUM        # block_sync 0 or 1
    assert c(A, B, 4096, 4, -1, None) == ENUM
    assert c(None, B, 4096, 1, 0, None) == NULLP
    assert c(A, None, 4096, 1, 1, None) == NULLP
    assert c(A + 8, B, 4096, 1, 0, None) == ALIGN
    assert c(A, B + 4, 4096, 1, 1, None) == ALIGN
    assert c(A, A, 4096, 1, 0, None) == ALIAS       # no in-place form
    assert c(A, A + 2048, 4096, 2, 1, None) == ALIAS
    assert c(A + 2048, A, 4096, 4, 0, None) == ALIAS
    assert c(None, None, 0, 8, 1, None) == OK


def test_rope_rejects(lib):
    f = lib.mbt_rope
    ok = dict(q=A, k=B, cs=CS, mp=4096, pos=POS, Q=16, K=2, T=8, D=256, rot=64, lay=0, dt=BF16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["cs"], a["mp"], a["pos"], a["Q"], a["K"], a["T"], a["D"],
                 a["rot"], a["lay"], a["dt"], None)
    assert call(dt=5) == DTYPE
    assert call(lay=3) == ENUM
    assert call(Q=0, K=0) == SHAPE
    assert call(Q=2**31 - 1, K=2**31 - 1) == SHAPE
    assert call(rot=65) == SHAPE
    assert call(D=600) == SHAPE
    assert call(mp=-1) == SCALAR
    assert call(pos=None) == NULLP
    assert call(q=None) == NULLP
    assert call(cs=None) == NULLP
    assert call(q=A + 1) == ALIGN
    assert call(k=A + 1024) == ALIAS            # k inside q
    assert call(q=CS + 64) == ALIAS             # q over the cache
    assert call(T=0, q=None, k=None, cs=None, pos=None) == OK


def qk_ex(lib, **kw):
    a = dict(q_in=A, k_in=B, q_out=C, k_out=D_, w_q=W1, w_k=W2, cos_sin=CS, max_pos=4096,
             pos=POS, Q=16, K=2, T=8, head_dim=256, rot_dim=64, eps=1e-6, weight_offset=1,
             layout=0, dtype=BF16, qis=0, kis=0, qos=0, kos=0, flags=1)
    a.update(kw)
    return lib.mbt_qknorm_rope_ex(a["q_in"], a["k_in"], a["q_out"], a["k_out"], a["w_q"],
                                  a["w_k"], a["cos_sin"], a["max_pos"], a["pos"], a["Q"], a["K"],
                                  a["T"], a["head_dim"], a["rot_dim"], a["eps"],
                                  a["weight_offset"], a["layout"], a["dtype"], a["qis"], a["kis"],
                                  a["qos"], a["kos"], a["flags"], None)


# a fused QKV buffer at A: Q = 2, K = 1, D = 8 bf16, token stride 32 elements
FQ = dict(Q=2, K=1, head_dim=8, rot_dim=8, qis=32, kis=32, qos=32, kos=32,
          q_in=A, k_in=A + 32, q_out=A, k_out=A + 32)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=2), ENUM), (dict(flags=-1), ENUM),
    (dict(qis=-256), SHAPE), (dict(kis=511), SHAPE),           # stride below K * D
    (dict(qos=4095), SHAPE), (dict(kos=1 << 41), SHAPE),
    (dict(dtype=4), DTYPE), (dict(rot_dim=3), SHAPE), (dict(eps=NAN), SCALAR),
    (dict(q_in=A + 1), ALIGN),
    # q_out over the key slice of the same buffer
    (dict(FQ, q_out=A + 32), ALIAS),
    # q_out one head into the query slice: overlaps the query input rows
    (dict(FQ, q_out=A + 16), ALIAS),
    # k_out over the query rows of the next token (stride 32 elements = 64 B)
    (dict(FQ, k_out=A + 64), ALIAS),
    # same base, different stride: not the in-place form
    (dict(FQ, qos=16), ALIAS),
    # the two outputs on top of each other
    (dict(FQ, q_out=C, k_out=C), ALIAS),
])
def test_qknorm_rope_ex_rejects(lib, kw, status):
    assert qk_ex(lib, **kw) == status
    assert lib.mbt_last_error().decode() != ""


def test_qknorm_rope_ex_empty_is_noop(lib):
    assert qk_ex(lib, T=0, q_in=None, k_in=None, q_out=None, k_out=None, w_q=None, w_k=None,
                 cos_sin=None, pos=None) == OK


def qkv_cache(lib, **kw):
    a = dict(qkv=A, q_out=B, kc=C, vc=D_, slot=POS + 4096, n_slots=64, w_q=W1, w_k=W2,
             cos_sin=CS, max_pos=4096, pos=POS, Q=16, K=2, T=8, head_dim=256, rot_dim=64,
             eps=1e-6, weight_offset=1, layout=0, dtype=BF16, flags=0)
    a.update(kw)
    return lib.mbt_qkv_norm_rope_cache(a["qkv"], a["q_out"], a["kc"], a["vc"], a["slot"],
                                       a["n_slots"], a["w_q"], a["w_k"], a["cos_sin"],
                                       a["max_pos"], a["pos"], a["Q"], a["K"], a["T"],
                                       a["head_dim"], a["rot_dim"], a["eps"], a["weight_offset"],
                                       a["layout"], a["dtype"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), SHAPE), (dict(Q=-1), SHAPE), (dict(head_dim=600), SHAPE),
    (dict(Q=2**31 - 1, K=2**30), SHAPE),
    (dict(dtype=7), DTYPE), (dict(flags=8), ENUM), (dict(n_slots=-1), SCALAR),
    (dict(slot=None), NULLP), (dict(kc=None), NULLP), (dict(vc=None), NULLP),
    (dict(qkv=None), NULLP), (dict(q_out=None), NULLP),
    (dict(slot=POS + 4100), ALIGN), (dict(vc=D_ + 1), ALIGN),
    (dict(kc=A + 1024), ALIAS),                 # key cache inside qkv
    (dict(vc=C + 256), ALIAS),                  # the two caches overlap
    (dict(q_out=C), ALIAS),                     # q_out on the key cache
    (dict(kc=POS), ALIAS),                      # key cache over the positions
    (dict(slot=D_ + 64), ALIAS),                # slot table inside the value cache
])
def test_qkv_norm_rope_cache_rejects(lib, kw, status):
    assert qkv_cache(lib, **kw) == status
    assert lib.mbt_last_error().decode() != ""


def test_qkv_norm_rope_cache_empty_is_noop(lib):
    assert qkv_cache(lib, T=0, qkv=None, q_out=None, kc=None, vc=None, slot=None, w_q=None,
                     w_k=None, cos_sin=None, pos=None) == OK


def test_adarms_rejects(lib):
    f, g, h = lib.mbt_adarms, lib.mbt_adarms_fp8, lib.mbt_adarms_amax
    SC, SH, GT = W1, W2, CS
    assert f(A, B, GT, SC, SH, 4, 2048, 1e-6, 9, None) == DTYPE
    assert f(A, B, GT, SC, SH, 4, 0, 1e-6, BF16, None) == SHAPE
    assert f(A, B, GT, SC, SH, 4, 2048, NAN, BF16, None) == SCALAR
    assert f(A, None, GT, SC, SH, 4, 2048, 1e-6, BF16, None) == NULLP    # gate needs residual
    assert f(A, B, GT, None, SH, 4, 2048, 1e-6, BF16, None) == NULLP
    assert f(A, B, GT, SC, None, 4, 2048, 1e-6, BF16, None) == NULLP
    assert f(A, B, GT, SC, SH + 1, 4, 2048, 1e-6, BF16, None) == ALIGN
    assert f(A, B, GT + 1, SC, SH, 4, 2048, 1e-6, BF16, None) == ALIGN
    assert f(A, B, GT, SC, A + 64, 4, 2048, 1e-6, BF16, None) == ALIAS   # shift inside x
    assert f(A, B, B + 64, SC, SH, 4, 2048, 1e-6, BF16, None) == ALIAS   # gate inside residual
    assert f(A, B, GT, A + 128, SH, 4, 2048, 1e-6, BF16, None) == ALIAS  # scale inside x
    assert f(None, None, None, None, None, 0, 2048, 1e-6, BF16, None) == OK
    assert g(A, B, GT, SC, SH, C, 0.0, 4, 2048, 1e-6, BF16, None) == SCALAR
    assert g(A, B, GT, SC, SH, None, 1.0, 4, 2048, 1e-6, BF16, None) == NULLP
    assert g(A, B, GT, SC, SH, SH + 8, 1.0, 4, 2048, 1e-6, BF16, None) == ALIAS  # y over shift
    assert g(A, B, GT, SC, SH, B + 4, 1.0, 4, 2048, 1e-6, BF16, None) == ALIAS   # y in residual
    assert h(A, B, GT, SC, SH, None, 4, 2048, 1e-6, BF16, None) == NULLP
    assert h(A, B, GT, SC, SH, C + 2, 4, 2048, 1e-6, BF16, None) == ALIGN
    assert h(A, B, GT, SC, SH, GT + 4, 4, 2048, 1e-6, BF16, None) == ALIAS       # amax on gate


def test_last_error_is_per_thread(lib):
    # Eight threads reject calls with their own T at once (ctypes releases
    # the interpreter lock inside each call, so the calls interleave); each
    # reads back its own detail, and its own successful no-op clears it.
    import threading
    errors = []

    def worker(tid):
        try:
            for it in range(3000):
                T = -(1 + tid * 100_000 + it)
                assert lib.mbt_gated_act(A, B, T, 16, 0, BF16, None) == SHAPE
                got = lib.mbt_last_error().decode()
                assert got == f"T={T} d=16", (tid, it, got)
                if it % 7 == 0:
                    assert lib.mbt_gated_act(None, None, 0, 16, 0, BF16, None) == OK
                    assert lib.mbt_last_error().decode() == "", (tid, it)
        except AssertionError as e:
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
