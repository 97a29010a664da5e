"""The extended prologue entry points on the GPU.

* mbt_qknorm_rope_ex with MBT_QK_ROUND_ONCE (the single-rounding variant of
  the ninfer PR's review item 1) against the oracle's round-once path, over
  the vector and scalar kernels, decode and prefill widths, both pairings
  and all dtypes; and its batch / alignment invariance;
* mbt_qknorm_rope_ex on strided views (thox-edge-ops v2, section 6: strided
  views; q and k as slices of one fused QKV buffer): out of place, in place
  inside the buffer and into padded outputs, against the oracle within the
  contract's tolerance and bit for bit equal to the dense op, with the rest
  of the buffer untouched;
* mbt_qkv_norm_rope_cache (FlashRT's qkv_split_rope_kvcache with the
  per-head norm; thox-edge-ops v2, section 10, item 4): q_out and the key
  rows at their slots against the oracle (and bit for bit against the dense
  prologue), value rows equal to a scatter of the value input by slot,
  invalid slots write nothing; tokens sharing a slot leave each element of
  that row equal to one of theirs.
"""
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
    flat = np.concatenate([np.zeros(offset, bits.dtype), bits.ravel()])
    return W.to_torch(flat, dtype, DEV)[offset:].view(bits.shape)


def host(t, dtype):
    torch.cuda.synchronize()
    return W.from_torch(t.contiguous(), dtype)


def _cell(**kw):
    base = dict(name="ex", config=95, cell=0, T=37, Q=6, K=2, D=256, rot=64, theta=1e7,
                layout=W.ROTATE_HALF, dtype=W.BF16, weight_offset=1, w_mean=0.0, w_std=0.05,
                x_std=2.0, max_pos=64, outside=((3, -1), (5, 64)))
    base.update(kw)
    return W.PrologueCell(**base)


def dense(mbt, cell, i, offset=0):
    """The plain prologue (dense tensors, contract rounding)."""
    dt = cell.dtype
    qo, ko = mbt.qknorm_rope(dev(i["q"], dt, offset), dev(i["k"], dt, offset),
                             dev(i["w_q"], dt, offset), dev(i["w_k"], dt, offset),
                             torch.from_numpy(i["cos_sin"]).to(DEV),
                             torch.from_numpy(i["pos"]).to(DEV), cell.rot, cell.eps,
                             cell.weight_offset, cell.layout)
    return host(qo, dt), host(ko, dt)


def once(mbt, cell, i, offset=0):
    dt = cell.dtype
    qo, ko = mbt.qknorm_rope_ex(dev(i["q"], dt, offset), dev(i["k"], dt, offset),
                                dev(i["w_q"], dt, offset), dev(i["w_k"], dt, offset),
                                torch.from_numpy(i["cos_sin"]).to(DEV),
                                torch.from_numpy(i["pos"]).to(DEV), cell.rot, cell.eps,
                                cell.weight_offset, cell.layout, round_once=True)
    return host(qo, dt), host(ko, dt)


def oracle_check(orc, cell, i, gq, gk, round_once, label, k_rows=None):
    """The prologue's results against the oracle, by the contract's rules:
    gq [T, Q, D] bits (or None), gk [T, K, D] bits (or None), or with
    `k_rows` the key results of those tokens only, in that order."""
    dt = cell.dtype
    qo, ko = orc.qknorm_rope(i["q"], i["k"], i["w_q"], i["w_k"], i["cos_sin"], i["pos"],
                             cell.rot, cell.eps, cell.weight_offset, cell.layout, dt,
                             max_pos=cell.max_pos, round_once=round_once)
    qn = orc.rmsnorm_rows(i["q"], i["w_q"], cell.eps, cell.weight_offset, dt)
    kn = orc.rmsnorm_rows(i["k"], i["w_k"], cell.eps, cell.weight_offset, dt)
    cs, pos = i["cos_sin"], i["pos"]
    stats = []
    if gq is not None and cell.Q:
        stats.append(C.check_prologue(gq, qo, qn, cs, pos, cell.rot, cell.layout, dt,
                                      cell.max_pos, label=f"{label} q vs oracle"))
    if gk is not None and cell.K:
        if k_rows is not None:
            ko, kn, pos = ko[k_rows], kn[k_rows], pos[k_rows]
        stats.append(C.check_prologue(gk, ko, kn, cs, pos, cell.rot, cell.layout, dt,
                                      cell.max_pos, label=f"{label} k vs oracle"))
    return stats


ONCE_CELLS = [
    _cell(name="once_bf16_d256_rot64", cell=1),
    _cell(name="once_f16_d256_rot64", dtype=W.F16, cell=2),
    _cell(name="once_f32_d256_rot64", dtype=W.F32, cell=3),
    _cell(name="once_bf16_d128_full", D=128, rot=128, weight_offset=0, w_mean=1.0, cell=4),
    _cell(name="once_bf16_d256_inter", rot=256, layout=W.INTERLEAVED, cell=5),
    _cell(name="once_bf16_d256_inter_partial", rot=40, layout=W.INTERLEAVED, cell=6),
    _cell(name="once_bf16_d256_rot48_hv3", rot=48, cell=7),
    _cell(name="once_bf16_d96_scalar", D=96, rot=32, cell=8),
    _cell(name="once_f32_d512_full", dtype=W.F32, D=512, rot=512, cell=9),
    _cell(name="once_bf16_prefill_24x4", T=2048, Q=24, K=4, positions="arange", max_pos=4096,
          outside=(), cell=10),
    _cell(name="once_f16_prefill_16x2_inter", T=2048, Q=16, K=2, dtype=W.F16, rot=256,
          layout=W.INTERLEAVED, positions="arange", max_pos=4096, outside=(), cell=11),
    _cell(name="once_bf16_c2_rot96", rot=96, T=1024, Q=16, K=2, max_pos=4096, cell=12),
    _cell(name="once_bf16_c4_inter32", rot=32, layout=W.INTERLEAVED, T=1024, Q=16, K=2,
          max_pos=4096, cell=13),
    _cell(name="once_f32_c4_rot64", dtype=W.F32, T=1024, Q=16, K=2, max_pos=4096, cell=14),
]


@pytest.mark.parametrize("cell", ONCE_CELLS, ids=lambda c: c.name)
def test_round_once_matches_oracle(mbt, orc, cell):
    i = cell.inputs()
    dt = cell.dtype
    gq, gk = once(mbt, cell, i)
    qo, ko = orc.qknorm_rope(i["q"], i["k"], i["w_q"], i["w_k"], i["cos_sin"], i["pos"],
                             cell.rot, cell.eps, cell.weight_offset, cell.layout, dt,
                             max_pos=cell.max_pos, round_once=True)
    qn = orc.rmsnorm_rows(i["q"], i["w_q"], cell.eps, cell.weight_offset, dt)
    kn = orc.rmsnorm_rows(i["k"], i["w_k"], cell.eps, cell.weight_offset, dt)
    sq = C.check_prologue(gq, qo, qn, i["cos_sin"], i["pos"], cell.rot, cell.layout, dt,
                          cell.max_pos, label=f"{cell.name} q")
    sk = C.check_prologue(gk, ko, kn, i["cos_sin"], i["pos"], cell.rot, cell.layout, dt,
                          cell.max_pos, label=f"{cell.name} k")
    print(f"{cell.name}: q {sq} k {sk}", flush=True)
    # the tail channels are the contract's (one rounding either way)
    dq, dk = dense(mbt, cell, i)
    C.check_bitwise(gq[..., cell.rot:], dq[..., cell.rot:], label=f"{cell.name} q tail")
    C.check_bitwise(gk[..., cell.rot:], dk[..., cell.rot:], label=f"{cell.name} k tail")


@pytest.mark.parametrize("cell", [c for c in ONCE_CELLS if c.D % 8 == 0 and c.T < 100],
                         ids=lambda c: c.name)
def test_round_once_alignment_invariant(mbt, cell):
    i = cell.inputs()
    aq, ak = once(mbt, cell, i)
    uq, uk = once(mbt, cell, i, offset=1)
    C.check_bitwise(uq, aq, label=f"{cell.name} unaligned q")
    C.check_bitwise(uk, ak, label=f"{cell.name} unaligned k")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_round_once_batch_invariant(mbt, dtype):
    cell = _cell(name="once_batch", T=2048, Q=24, K=4, dtype=dtype, positions="arange",
                 max_pos=4096, outside=(), cell=30 + dtype)
    i = cell.inputs()
    fq, fk = once(mbt, cell, i)
    for t in (0, 1, 1500, 2047):
        one = {k: (v[t:t + 1] if k in ("q", "k", "pos") else v) for k, v in i.items()}
        c1 = _cell(name="one", T=1, Q=24, K=4, dtype=dtype, max_pos=4096, outside=())
        oq, ok = once(mbt, c1, one)
        C.check_bitwise(oq[0], fq[t], label=f"token {t} q")
        C.check_bitwise(ok[0], fk[t], label=f"token {t} k")


# ---------------------------------------------------------------------------
# strided views of a fused QKV buffer
# ---------------------------------------------------------------------------

def fused_buffer(i, cell, pad, seed):
    """qkv [T, (Q + 2K) * D + pad] holding q, k and a random v per token."""
    dt, T, Q, K, D = cell.dtype, cell.T, cell.Q, cell.K, cell.D
    v = W.normal_bits((95, cell.cell, 7, seed), (T, K, D), 0.0, 1.0, dt)
    tail = W.normal_bits((95, cell.cell, 8, seed), (T, pad), 0.0, 1.0, dt)
    rows = np.concatenate([i["q"].reshape(T, Q * D), i["k"].reshape(T, K * D),
                           v.reshape(T, K * D), tail], axis=1)
    return rows, v


def views(buf, cell):
    Q, K, D = cell.Q, cell.K, cell.D
    q = buf[:, :Q * D].unflatten(1, (Q, D))
    k = buf[:, Q * D:(Q + K) * D].unflatten(1, (K, D))
    return q, k


STRIDE_CELLS = [
    _cell(name="qkv_bf16_16x2", Q=16, K=2, T=128, positions="uniform", max_pos=4096,
          outside=((3, -1),), cell=40),
    _cell(name="qkv_bf16_prefill_24x4", Q=24, K=4, T=2048, positions="arange", max_pos=4096,
          outside=(), cell=41),
    _cell(name="qkv_f32_16x8_d128", dtype=W.F32, Q=16, K=8, D=128, rot=128, T=9, cell=42),
    _cell(name="qkv_f16_inter", dtype=W.F16, rot=256, layout=W.INTERLEAVED, cell=43),
    _cell(name="qkv_bf16_mid_T999", Q=24, K=4, T=999, positions="arange", max_pos=4096,
          outside=(), cell=44),
    # one to one and a half resident rounds (9225 waves): two launches over
    # the token halves, at the views' own strides
    _cell(name="qkv_bf16_split_16x2_T4100", Q=16, K=2, T=4100, positions="arange",
          max_pos=4096, outside=((4099, 4096),), cell=45),
]


@pytest.mark.parametrize("pad", [0, 1], ids=["aligned", "odd_stride"])
@pytest.mark.parametrize("round_once", [False, True], ids=["contract", "once"])
@pytest.mark.parametrize("cell", STRIDE_CELLS, ids=lambda c: c.name)
def test_strided_views(mbt, orc, cell, round_once, pad):
    """pad 0: 16-byte strides (vector kernel); pad 1: odd strides (scalar).
    Every result is checked against the oracle; the dense op's result, also
    checked against it, must then match bit for bit."""
    i = cell.inputs()
    dt = cell.dtype
    ref = once(mbt, cell, i) if round_once else dense(mbt, cell, i)
    oracle_check(orc, cell, i, ref[0], ref[1], round_once, f"{cell.name} dense")
    rows, _ = fused_buffer(i, cell, pad, 1)
    wq, wk = dev(i["w_q"], dt), dev(i["w_k"], dt)
    cs = torch.from_numpy(i["cos_sin"]).to(DEV)
    pos = torch.from_numpy(i["pos"]).to(DEV)
    args = (wq, wk, cs, pos, cell.rot, cell.eps, cell.weight_offset, cell.layout)

    # out of place, dense outputs
    buf = dev(rows, dt)
    q, k = views(buf, cell)
    qo, ko = mbt.qknorm_rope_ex(q, k, *args, round_once=round_once)
    st = oracle_check(orc, cell, i, host(qo, dt), host(ko, dt), round_once,
                      f"{cell.name} strided in")
    print(f"{cell.name} strided: {st}", flush=True)
    C.check_bitwise(host(qo, dt), ref[0], label=f"{cell.name} strided in q")
    C.check_bitwise(host(ko, dt), ref[1], label=f"{cell.name} strided in k")
    C.check_bitwise(host(buf, dt), rows, label=f"{cell.name} input buffer untouched")

    # in place inside the fused buffer: only the q and k slices change
    mbt.qknorm_rope_ex(q, k, *args, q_out=q, k_out=k, round_once=round_once)
    want = rows.copy()
    Q, K, D, T = cell.Q, cell.K, cell.D, cell.T
    want[:, :Q * D] = ref[0].reshape(T, Q * D)
    want[:, Q * D:(Q + K) * D] = ref[1].reshape(T, K * D)
    got = host(buf, dt)
    oracle_check(orc, cell, i, got[:, :Q * D].reshape(T, Q, D),
                 got[:, Q * D:(Q + K) * D].reshape(T, K, D), round_once,
                 f"{cell.name} in place")
    C.check_bitwise(got, want, label=f"{cell.name} in place in qkv")

    # into padded outputs (token stride (heads + 1) * D + pad)
    qpad = torch.full((T, (Q + 1) * D + pad), 7.0, dtype=buf.dtype, device=DEV)
    kpad = torch.full((T, (K + 1) * D + pad), 7.0, dtype=buf.dtype, device=DEV)
    q, k = views(dev(rows, dt), cell)
    mbt.qknorm_rope_ex(q, k, *args, q_out=qpad[:, :Q * D].unflatten(1, (Q, D)),
                       k_out=kpad[:, :K * D].unflatten(1, (K, D)), round_once=round_once)
    gq, gk = host(qpad, dt), host(kpad, dt)
    oracle_check(orc, cell, i, gq[:, :Q * D].reshape(T, Q, D), gk[:, :K * D].reshape(T, K, D),
                 round_once, f"{cell.name} padded out")
    C.check_bitwise(gq[:, :Q * D].reshape(T, Q, D), ref[0], label=f"{cell.name} padded q")
    C.check_bitwise(gk[:, :K * D].reshape(T, K, D), ref[1], label=f"{cell.name} padded k")
    seven = W.to_bits(np.full(1, 7.0), dt)[0]
    assert np.all(gq[:, Q * D:] == seven) and np.all(gk[:, K * D:] == seven), "padding written"


# ---------------------------------------------------------------------------
# fused QKV -> q_out + KV cache
# ---------------------------------------------------------------------------

CACHE_CELLS = [
    _cell(name="cache_bf16_16x2_decode", Q=16, K=2, T=64, positions="uniform", max_pos=4096,
          outside=((3, -1),), cell=50),
    _cell(name="cache_bf16_prefill_24x4", Q=24, K=4, T=2048, positions="arange",
          max_pos=4096, outside=(), cell=51),
    _cell(name="cache_f32_d128", dtype=W.F32, Q=8, K=8, D=128, rot=128, T=17, cell=52),
    _cell(name="cache_bf16_d96_scalar", D=96, rot=32, T=21, cell=53),
    _cell(name="cache_f16_inter_q0", dtype=W.F16, Q=0, K=4, rot=256, layout=W.INTERLEAVED,
          T=33, cell=54),
    # spare waves and partly filled last waves (one chunk per lane; and the
    # chunked kernel's other load orders)
    _cell(name="cache_bf16_ragged_q5k3", Q=5, K=3, T=7, max_pos=4096, cell=55),
    _cell(name="cache_bf16_mid_T999", Q=24, K=4, T=999, positions="arange", max_pos=4096,
          outside=(), cell=56),
    _cell(name="cache_bf16_thr_T1501", Q=24, K=4, T=1501, positions="arange", max_pos=4096,
          outside=(), cell=57),
]


@pytest.mark.parametrize("round_once", [False, True], ids=["contract", "once"])
@pytest.mark.parametrize("cell", CACHE_CELLS, ids=lambda c: c.name)
def test_qkv_cache(mbt, orc, cell, round_once):
    """q_out and each written key row against the oracle (and bit for bit
    against the dense prologue); value rows against a numpy scatter of the
    value input by slot; rows no token maps to keep their sentinel."""
    i = cell.inputs()
    dt, T, Q, K, D = cell.dtype, cell.T, cell.Q, cell.K, cell.D
    ref_q, ref_k = once(mbt, cell, i) if round_once else dense(mbt, cell, i)
    rows, v = fused_buffer(i, cell, 0, 2)
    qkv = dev(rows, dt).view(T, Q + 2 * K, D)
    n_slots = T + 9
    g = np.random.default_rng([95, cell.cell, 3])
    slot = g.permutation(n_slots)[:T].astype(np.int64)
    slot[g.random(T) < 0.1] = -1                        # padding tokens
    slot[g.random(T) < 0.05] = n_slots + 3              # past the cache: no write
    sentinel = W.to_bits(np.full(1, -3.0), dt)[0]
    kc = torch.full((n_slots, K, D), -3.0, dtype=qkv.dtype, device=DEV)
    vc = torch.full((n_slots, K, D), -3.0, dtype=qkv.dtype, device=DEV)
    q_out = mbt.qkv_norm_rope_cache(qkv, dev(i["w_q"], dt), dev(i["w_k"], dt),
                                    torch.from_numpy(i["cos_sin"]).to(DEV),
                                    torch.from_numpy(i["pos"]).to(DEV),
                                    torch.from_numpy(slot).to(DEV), kc, vc, Q, cell.rot,
                                    cell.eps, cell.weight_offset, cell.layout,
                                    round_once=round_once)
    gq = host(q_out, dt)
    gk, gv = host(kc, dt), host(vc, dt)
    valid = (slot >= 0) & (slot < n_slots)
    # q_out, and the key row at each written slot, token by token
    st = oracle_check(orc, cell, i, gq, gk[slot[valid]], round_once, f"{cell.name} cache",
                      k_rows=np.nonzero(valid)[0])
    print(f"{cell.name} cache: {st}", flush=True)
    if Q:
        C.check_bitwise(gq, ref_q, label=f"{cell.name} q_out")
    C.check_bitwise(gk[slot[valid]], ref_k[valid], label=f"{cell.name} key cache rows")
    want_v = np.full_like(gv, sentinel)
    want_v[slot[valid]] = v[valid]                      # numpy scatter of the value input
    C.check_bitwise(gv, want_v, label=f"{cell.name} value cache")
    untouched = np.setdiff1d(np.arange(n_slots), slot[valid])
    assert np.all(gk[untouched] == sentinel) and np.all(gv[untouched] == sentinel), \
        "a cache row without a token was written"
    C.check_bitwise(host(qkv, dt).reshape(T, -1), rows, label=f"{cell.name} qkv untouched")


@pytest.mark.parametrize("cell", [c for c in CACHE_CELLS
                                  if c.name in ("cache_bf16_16x2_decode",
                                                "cache_bf16_prefill_24x4", "cache_f32_d128")],
                         ids=lambda c: c.name)
def test_qkv_cache_shared_slots(mbt, orc, cell):
    """Tokens mapped to one slot race for its row; which token's value lands
    there is unspecified.  Each element of such a row must still be that
    element of one of the contending tokens' rows (the dense prologue's key
    row, itself checked against the oracle here, or the value input), q_out
    is unaffected, and rows no token maps to keep their sentinel."""
    i = cell.inputs()
    dt, T, Q, K, D = cell.dtype, cell.T, cell.Q, cell.K, cell.D
    ref_q, ref_k = dense(mbt, cell, i)
    oracle_check(orc, cell, i, ref_q, ref_k, False, f"{cell.name} dense")
    rows, v = fused_buffer(i, cell, 0, 3)
    qkv = dev(rows, dt).view(T, Q + 2 * K, D)
    n_slots = max(4, T // 3)
    slot = np.random.default_rng([95, cell.cell, 4]).integers(0, n_slots, T).astype(np.int64)
    assert len(np.unique(slot)) < T, "the case needs shared slots"
    sentinel = W.to_bits(np.full(1, -3.0), dt)[0]
    kc = torch.full((n_slots + 2, K, D), -3.0, dtype=qkv.dtype, device=DEV)
    vc = torch.full((n_slots + 2, K, D), -3.0, dtype=qkv.dtype, device=DEV)
    q_out = mbt.qkv_norm_rope_cache(qkv, dev(i["w_q"], dt), dev(i["w_k"], dt),
                                    torch.from_numpy(i["cos_sin"]).to(DEV),
                                    torch.from_numpy(i["pos"]).to(DEV),
                                    torch.from_numpy(slot).to(DEV), kc, vc, Q, cell.rot,
                                    cell.eps, cell.weight_offset, cell.layout)
    C.check_bitwise(host(q_out, dt), ref_q, label=f"{cell.name} q_out")
    gk, gv = host(kc, dt), host(vc, dt)
    shared = 0
    for s in np.unique(slot):
        toks = np.nonzero(slot == s)[0]
        shared += len(toks) > 1
        ok_k = np.zeros((K, D), bool)
        ok_v = np.zeros((K, D), bool)
        for t in toks:
            ok_k |= gk[s] == ref_k[t]
            ok_v |= gv[s] == v[t]
        assert ok_k.all(), f"slot {s}: a key element from none of tokens {toks.tolist()}"
        assert ok_v.all(), f"slot {s}: a value element from none of tokens {toks.tolist()}"
    untouched = np.setdiff1d(np.arange(n_slots + 2), slot)
    assert np.all(gk[untouched] == sentinel) and np.all(gv[untouched] == sentinel)
    print(f"{cell.name}: {shared} shared slots of {len(np.unique(slot))}", flush=True)
