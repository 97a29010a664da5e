"""Parity of the HIP path (through the C ABI) with the CPU oracle on one
MI355X: every configuration cell at its full size, plus edge cases.

Marked `gpu`; run on a machine with an MI355X with
    python -u -m pytest tests -m gpu -x -v --timeout 120 --timeout-method thread
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


def dev(bits, dtype):
    return W.to_torch(bits, dtype, DEV)


def host(t, dtype):
    torch.cuda.synchronize()
    return W.from_torch(t, dtype)


# ---------------------------------------------------------------------------
# the fused QK-norm + RoPE prologue
# ---------------------------------------------------------------------------

def run_prologue(mbt, cell, i, in_place=False, offset=0):
    """Run the prologue on the GPU; `offset` shifts every tensor by that many
    elements inside a larger allocation (unaligned storage)."""
    dt = cell.dtype

    def place(bits):
        t = dev(np.concatenate([np.zeros(offset, bits.dtype), bits.ravel()]), dt)
        return t[offset:].view(bits.shape)

    q, k = place(i["q"]), place(i["k"])
    wq, wk = place(i["w_q"]), place(i["w_k"])
    cs = torch.from_numpy(i["cos_sin"]).to(DEV)
    pos = torch.from_numpy(i["pos"]).to(DEV)
    qo, ko = (q, k) if in_place else (None, None)
    qo, ko = mbt.qknorm_rope(q, k, wq, wk, cs, pos, cell.rot, cell.eps, cell.weight_offset,
                             cell.layout, q_out=qo, k_out=ko, max_pos=cell.max_pos)
    return host(qo, dt), host(ko, dt)


def oracle_prologue(orc, cell, i):
    qo, ko = orc.qknorm_rope(i["q"], i["k"], i["w_q"], i["w_k"], i["cos_sin"], i["pos"],
                             cell.rot, cell.eps, cell.weight_offset, cell.layout, cell.dtype,
                             max_pos=cell.max_pos)
    qn = orc.rmsnorm_rows(i["q"], i["w_q"], cell.eps, cell.weight_offset, cell.dtype)
    kn = orc.rmsnorm_rows(i["k"], i["w_k"], cell.eps, cell.weight_offset, cell.dtype)
    return qo, ko, qn, kn


def check_prologue_cell(mbt, orc, cell, i=None, **kw):
    i = cell.inputs() if i is None else i
    gq, gk = run_prologue(mbt, cell, i, **kw)
    qo, ko, qn, kn = oracle_prologue(orc, cell, i)
    sq = C.check_prologue(gq, qo, qn, i["cos_sin"], i["pos"], cell.rot, cell.layout,
                          cell.dtype, cell.max_pos, label=f"{cell.name} q")
    sk = C.check_prologue(gk, ko, kn, i["cos_sin"], i["pos"], cell.rot, cell.layout,
                          cell.dtype, cell.max_pos, label=f"{cell.name} k")
    print(f"{cell.name}: q {sq} k {sk}", flush=True)
    return gq, gk


PROLOGUE_CELLS = W.config1_cells() + W.config2_cells() + W.config3_cells()


@pytest.mark.parametrize("cell", PROLOGUE_CELLS, ids=lambda c: c.name)
def test_prologue_config(mbt, orc, cell):
    check_prologue_cell(mbt, orc, cell)


def _cell(**kw):
    base = dict(name="edge", config=90, cell=0, T=5, Q=4, K=2, D=128, rot=64, theta=1e4,
                layout=W.ROTATE_HALF, dtype=W.BF16, weight_offset=1, w_mean=0.0, w_std=0.05,
                x_std=2.0, max_pos=512)
    base.update(kw)
    return W.PrologueCell(**base)


EDGE_PROLOGUE = [
    _cell(name="fp32_d256", dtype=W.F32, D=256, rot=64, cell=1),
    _cell(name="fp32_d128_full_inter", dtype=W.F32, D=128, rot=128, layout=W.INTERLEAVED,
          cell=2),
    _cell(name="f16_d64", dtype=W.F16, D=64, rot=32, cell=3),
    _cell(name="bf16_d512", D=512, rot=128, cell=4),
    _cell(name="bf16_d32", D=32, rot=16, cell=5),
    _cell(name="rot0", rot=0, cell=6),
    _cell(name="rot_full_half", rot=128, cell=7),
    _cell(name="inter_partial_12", rot=12, layout=W.INTERLEAVED, cell=8),
    _cell(name="half_rot_not_vec_24", rot=24, cell=9),         # scalar kernel
    _cell(name="odd_d37", D=37, rot=36, cell=10),              # scalar kernel
    _cell(name="d96", D=96, rot=32, cell=11),                  # scalar kernel
    _cell(name="q_only", K=0, cell=12),
    _cell(name="k_only", Q=0, K=3, cell=13),
    _cell(name="one_head", Q=1, K=0, T=3, cell=14),
    _cell(name="T1", T=1, cell=15),
    _cell(name="eps_big_theta", eps=0.25, theta=3.0e5, cell=16),
    _cell(name="direct_weight", weight_offset=0, w_mean=1.0, cell=17),
    _cell(name="positions_out", T=6, outside=((0, -1), (2, 512), (3, 1 << 40), (5, -(1 << 40))),
          cell=18),
    _cell(name="long_T", T=3000, Q=3, K=1, cell=19),
    # prefill-width launch shapes (>= 12288 head-rows): two chunks per lane
    # (rot 96: 12 rotated chunks need 16 lanes), four with interleaved pairs,
    # four in fp32
    _cell(name="c2_bf16_d256_rot96", D=256, rot=96, T=1024, Q=16, K=2, max_pos=4096, cell=30),
    _cell(name="c4_bf16_d256_inter32", D=256, rot=32, layout=W.INTERLEAVED, T=1024, Q=16,
          K=2, max_pos=4096, cell=31),
    _cell(name="c4_f32_d256_rot64", dtype=W.F32, D=256, rot=64, T=1024, Q=16, K=2,
          max_pos=4096, cell=32),
    _cell(name="c2_f16_d128_full", dtype=W.F16, D=128, rot=128, T=1024, Q=16, K=2,
          max_pos=4096, cell=33),
    # the three load orders of the chunked kernels (chosen by wave count:
    # the early cos/sin order up to 2560 waves, the barrier-after-the-sum
    # order up to 5000, the whole-block order up to 8192), each with a ragged
    # last block -- spare waves and a partly filled last wave -- and with
    # interleaved pairs
    _cell(name="c4_mid_ragged_T999", D=256, rot=64, T=999, Q=24, K=4, max_pos=4096,
          positions="arange", cell=34),
    _cell(name="c4_thr_ragged_T1501", D=256, rot=64, T=1501, Q=24, K=4, max_pos=4096,
          positions="arange", cell=39),
    _cell(name="c4_lat_ragged_T501", D=256, rot=64, T=501, Q=24, K=4, max_pos=4096,
          positions="arange", cell=35),
    _cell(name="c4_thr_inter32", D=256, rot=32, layout=W.INTERLEAVED, T=1024, Q=24, K=4,
          max_pos=4096, cell=36),
    _cell(name="c2_thr_rot96", D=256, rot=96, T=1024, Q=24, K=4, max_pos=4096, cell=37),
    _cell(name="c4_thr_f16_rot0", dtype=W.F16, D=256, rot=0, T=1024, Q=24, K=4, cell=38),
    # a dense launch of one to one and a half resident rounds (8192 to
    # 12288 waves) runs as two launches over the token halves: an even split
    # with random positions, an odd one (the halves differ by a token) with
    # in-place storage, and interleaved fp16; just past the bound, one launch
    _cell(name="split_16x2_T4100", D=256, rot=64, T=4100, Q=16, K=2, max_pos=4096,
          outside=((1, -1), (4099, 4096)), cell=40),
    _cell(name="split_odd_24x4_T3001", D=256, rot=64, T=3001, Q=24, K=4, max_pos=4096,
          positions="arange", in_place=True, cell=41),
    _cell(name="split_inter_f16_T2500", dtype=W.F16, D=256, rot=256, layout=W.INTERLEAVED,
          T=2500, Q=24, K=4, max_pos=4096, cell=42),
    _cell(name="unsplit_24x4_T3512", D=256, rot=64, T=3512, Q=24, K=4, max_pos=4096,
          positions="arange", cell=43),
]


@pytest.mark.parametrize("cell", EDGE_PROLOGUE, ids=lambda c: c.name)
def test_prologue_edges(mbt, orc, cell):
    check_prologue_cell(mbt, orc, cell, in_place=cell.in_place)


@pytest.mark.parametrize("T,layout", [(1024, W.ROTATE_HALF), (2048, W.ROTATE_HALF),
                                      (2048, W.INTERLEAVED)])
def test_prologue_width_invariant(mbt, T, layout):
    """A prefill-width launch (chunked rows, whole-block load order) and the
    same tokens in 16-token launches (one chunk per lane, early cos/sin
    order) give identical bits: the reduction tree and the rounding do not
    depend on the launch shape."""
    cell = [c for c in W.config3_cells()
            if c.dtype == W.BF16 and c.Q == 24 and c.T == T and c.layout == layout][0]
    i = cell.inputs()
    dt = cell.dtype
    q, k = dev(i["q"], dt), dev(i["k"], dt)
    wq, wk = dev(i["w_q"], dt), dev(i["w_k"], dt)
    cs = torch.from_numpy(i["cos_sin"]).to(DEV)
    pos = torch.from_numpy(i["pos"]).to(DEV)
    args = (cell.rot, cell.eps, cell.weight_offset, cell.layout)
    qo, ko = mbt.qknorm_rope(q, k, wq, wk, cs, pos, *args)
    qs, ks = torch.empty_like(q), torch.empty_like(k)
    for t0 in range(0, T, 16):
        mbt.qknorm_rope(q[t0:t0 + 16], k[t0:t0 + 16], wq, wk, cs, pos[t0:t0 + 16], *args,
                        q_out=qs[t0:t0 + 16], k_out=ks[t0:t0 + 16])
    torch.cuda.synchronize()
    assert torch.equal(qo.view(torch.int16), qs.view(torch.int16))
    assert torch.equal(ko.view(torch.int16), ks.view(torch.int16))


def test_prologue_split_invariant(mbt):
    """A launch of one to one and a half resident rounds, run as two
    launches over the token halves, gives the bits of the same tokens in
    16-token launches."""
    cell = [c for c in EDGE_PROLOGUE if c.name == "split_16x2_T4100"][0]
    i = cell.inputs()
    dt = cell.dtype
    q, k = dev(i["q"], dt), dev(i["k"], dt)
    wq, wk = dev(i["w_q"], dt), dev(i["w_k"], dt)
    cs = torch.from_numpy(i["cos_sin"]).to(DEV)
    pos = torch.from_numpy(i["pos"]).to(DEV)
    args = (cell.rot, cell.eps, cell.weight_offset, cell.layout)
    qo, ko = mbt.qknorm_rope(q, k, wq, wk, cs, pos, *args)
    qs, ks = torch.empty_like(q), torch.empty_like(k)
    for t0 in range(0, cell.T, 16):
        mbt.qknorm_rope(q[t0:t0 + 16], k[t0:t0 + 16], wq, wk, cs, pos[t0:t0 + 16], *args,
                        q_out=qs[t0:t0 + 16], k_out=ks[t0:t0 + 16])
    torch.cuda.synchronize()
    assert torch.equal(qo.view(torch.int16), qs.view(torch.int16))
    assert torch.equal(ko.view(torch.int16), ks.view(torch.int16))


RAGGED_IN_PLACE = [
    # spare waves in the last block (they read the last wave's rows and store
    # nothing) and partly filled last waves, written in place: one chunk per
    # lane, and the three orders of the chunked kernel
    _cell(name="ip_c1_T1", D=256, rot=64, T=1, Q=16, K=2, max_pos=4096, cell=40),
    _cell(name="ip_c1_T7_q5k3", D=256, rot=64, T=7, Q=5, K=3, max_pos=4096, cell=41),
    _cell(name="ip_c4_lat_T501", D=256, rot=64, T=501, Q=24, K=4, max_pos=4096,
          positions="arange", cell=42),
    _cell(name="ip_c4_mid_T999", D=256, rot=64, T=999, Q=24, K=4, max_pos=4096,
          positions="arange", cell=43),
    _cell(name="ip_c4_thr_T1501", D=256, rot=64, T=1501, Q=24, K=4, max_pos=4096,
          positions="arange", cell=44),
]


@pytest.mark.parametrize("cell", RAGGED_IN_PLACE, ids=lambda c: c.name)
def test_prologue_in_place_ragged(mbt, orc, cell):
    check_prologue_cell(mbt, orc, cell, in_place=True)


@pytest.mark.parametrize("dtype", [W.BF16, W.F16, W.F32])
def test_prologue_in_place_and_unaligned(mbt, orc, dtype):
    cell = _cell(name=f"inplace_{dtype}", dtype=dtype, cell=20 + dtype)
    check_prologue_cell(mbt, orc, cell, in_place=True)
    check_prologue_cell(mbt, orc, cell, offset=1)            # 2- or 4-byte aligned only
    check_prologue_cell(mbt, orc, cell, in_place=True, offset=3)


def test_prologue_empty(mbt):
    q = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(128, dtype=torch.bfloat16, device=DEV)
    cs = torch.zeros((8, 64), dtype=torch.float32, device=DEV)
    pos = torch.zeros(0, dtype=torch.int64, device=DEV)
    qo, ko = mbt.qknorm_rope(q, k, w, w, cs, pos, 64)
    assert qo.shape == q.shape and ko.shape == k.shape


@pytest.mark.parametrize("layout", [W.ROTATE_HALF, W.INTERLEAVED])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_prologue_pairing_exact(mbt, dtype, layout):
    """Synthetic cache rows: identity at position 0, a quarter turn at 1 and
    a half turn at 2, applied to the same heads.  The GPU's own outputs must
    relate exactly: quarter turn (a, b) -> (-b, a) and half turn -> negation
    of the identity output; channels past rot_dim are equal."""
    D, rot = 128, 64
    g = np.random.default_rng(5)
    q = np.stack([W.to_bits(g.standard_normal((4, D)), dtype)] * 3)
    k = np.stack([W.to_bits(g.standard_normal((2, D)), dtype)] * 3)
    w = W.to_bits(g.standard_normal(D) * 0.05 + 1, dtype)
    cs = np.zeros((3, rot), np.float32)
    cs[0, :rot // 2] = 1
    cs[1, rot // 2:] = 1
    cs[2, :rot // 2] = -1
    if layout == W.ROTATE_HALF:
        a, b = np.arange(rot // 2), np.arange(rot // 2, rot)
    else:
        a, b = np.arange(0, rot, 2), np.arange(1, rot, 2)
    qo, ko = mbt.qknorm_rope(dev(q, dtype), dev(k, dtype), dev(w, dtype), dev(w, dtype),
                             torch.from_numpy(cs).to(DEV), torch.arange(3, device=DEV), rot,
                             layout=layout)
    for out in (host(qo, dtype), host(ko, dtype)):
        v = W.bits_to_f32(out, dtype)
        assert np.array_equal(v[1][..., a], -v[0][..., b])
        assert np.array_equal(v[1][..., b], v[0][..., a])
        assert np.array_equal(v[2][..., :rot], -v[0][..., :rot])
        assert np.array_equal(v[1][..., rot:], v[0][..., rot:])
        assert np.array_equal(v[2][..., rot:], v[0][..., rot:])


def test_prologue_deterministic_and_guarded(mbt):
    """Two runs give identical bits, and nothing outside the outputs moves."""
    cell = W.config2_cells()[-1]
    i = cell.inputs()
    dt = cell.dtype
    guard = 4096
    qn = i["q"].size
    big = torch.full((qn + 2 * guard,), 0x5A5A, dtype=torch.int16, device=DEV)
    q_out = big[guard:guard + qn].view(torch.bfloat16).view(i["q"].shape)
    args = (dev(i["q"], dt), dev(i["k"], dt), dev(i["w_q"], dt), dev(i["w_k"], dt),
            torch.from_numpy(i["cos_sin"]).to(DEV), torch.from_numpy(i["pos"]).to(DEV),
            cell.rot, cell.eps, cell.weight_offset, cell.layout)
    mbt.qknorm_rope(*args, q_out=q_out)
    first = host(q_out, dt).copy()
    mbt.qknorm_rope(*args, q_out=q_out)
    assert np.array_equal(first, host(q_out, dt))
    g = big.cpu().numpy()
    assert np.all(g[:guard] == 0x5A5A) and np.all(g[guard + qn:] == 0x5A5A), "guard bytes"


# ---------------------------------------------------------------------------
# fused residual-add RMSNorm (+ FP8, + calibration)
# ---------------------------------------------------------------------------

def check_norm_cell(mbt, orc, cell, offset=0):
    i = cell.inputs()
    dt = cell.dtype

    def place(bits):
        if bits is None:
            return None
        t = dev(np.concatenate([np.zeros(offset, bits.dtype), bits.ravel()]), dt)
        return t[offset:].view(bits.shape)

    x, r, w = place(i["x"]), place(i["residual"]), place(i["w"])
    if cell.fp8:
        cal = cell.calibration_inputs()
        amax_o = orc.fused_add_rmsnorm_amax(cal["x"], cal["residual"], i["w"], cell.eps,
                                            cell.weight_offset, dt)
        amax_g = mbt.fused_add_rmsnorm_amax(dev(cal["x"], dt), None if cal["residual"] is None
                                            else dev(cal["residual"], dt), w, cell.eps,
                                            cell.weight_offset)
        amax_g = float(amax_g.item())
        assert abs(amax_g - amax_o) <= 1e-5 * amax_o, f"amax {amax_g} vs {amax_o}"
        inv_scale = W.fp8_inv_scale(amax_o)
        y = mbt.fused_add_rmsnorm_fp8(x, r, w, inv_scale, cell.eps, cell.weight_offset)
        yo, ro = orc.fused_add_rmsnorm_fp8(i["x"], i["residual"], i["w"], inv_scale, cell.eps,
                                           cell.weight_offset, dt)
        st = C.check_fp8(y.cpu().numpy(), yo, label=cell.name)
        C.check_bitwise(host(x, dt), i["x"], label=f"{cell.name} x untouched")
    else:
        mbt.fused_add_rmsnorm(x, r, w, cell.eps, cell.weight_offset)
        xo, ro = orc.fused_add_rmsnorm(i["x"], i["residual"], i["w"], cell.eps,
                                       cell.weight_offset, dt)
        st = C.check_values(host(x, dt), xo, dt, label=cell.name)
    if r is not None:
        gr = host(r, dt)
        C.check_bitwise(gr, ro, label=f"{cell.name} residual vs oracle")
        eager = dev(i["x"], dt) + dev(i["residual"], dt)          # torch's eager add on GPU
        C.check_bitwise(gr, host(eager, dt), label=f"{cell.name} residual vs eager")
    print(f"{cell.name}: {st}", flush=True)


NORM_CELLS = W.config4_cells() + [c for c in W.config5_cells() if isinstance(c, W.NormCell)]


@pytest.mark.parametrize("cell", NORM_CELLS, ids=lambda c: c.name)
def test_norm_config(mbt, orc, cell):
    check_norm_cell(mbt, orc, cell)


def _ncell(**kw):
    base = dict(name="nedge", config=91, cell=0, T=7, H=1024, dtype=W.BF16, weight_offset=0,
                w_mean=1.0, w_std=0.05)
    base.update(kw)
    return W.NormCell(**base)


EDGE_NORM = [
    _ncell(name="odd_H37", H=37, cell=1),
    _ncell(name="H1", H=1, cell=2),
    _ncell(name="no_residual", residual=False, cell=3),
    _ncell(name="f32_H8192_wide", dtype=W.F32, H=8192, T=3, cell=4),
    _ncell(name="bf16_H16384", H=16384, T=2, cell=5),
    _ncell(name="bf16_H65536", H=65536, T=2, cell=6),
    _ncell(name="bf16_H80000_scalar", H=80000, T=2, cell=7),
    _ncell(name="f16_H2560_T2000", dtype=W.F16, H=2560, T=2000, cell=8),
    _ncell(name="fp8_no_residual", residual=False, fp8=True, cell=9),
    _ncell(name="fp8_odd", H=333, fp8=True, cell=10),
    _ncell(name="fp8_f32", dtype=W.F32, H=2048, fp8=True, cell=11),
    _ncell(name="eps_big", eps=0.5, cell=12),
    # no weight (w = NULL): the scale is folded into the next GEMM
    _ncell(name="noweight_bf16_H1024", weight=False, cell=13),
    _ncell(name="noweight_bf16_H256_small", weight=False, H=256, T=33, cell=14),
    _ncell(name="noweight_f16_H2560", weight=False, dtype=W.F16, H=2560, cell=15),
    _ncell(name="noweight_f32_H8192", weight=False, dtype=W.F32, H=8192, T=3, cell=16),
    _ncell(name="noweight_odd_H37", weight=False, H=37, cell=17),
    _ncell(name="noweight_no_residual", weight=False, residual=False, cell=18),
    _ncell(name="noweight_fp8_H2048_T512", weight=False, fp8=True, H=2048, T=512, cell=19),
    _ncell(name="noweight_fp8_odd", weight=False, fp8=True, H=333, cell=20),
    # the wide kernel's buffer ranges: four rows per block with the last
    # block partly past T, two rows per block likewise, and rows whose last
    # wave (or last chunk of a lane) lies partly past H
    _ncell(name="wide_rpb4_T2049", H=2048, T=2049, cell=21),
    _ncell(name="wide_rpb4_T2049_fp8", H=2048, T=2049, fp8=True, cell=22),
    _ncell(name="wide_rpb2_H4096_T1025", H=4096, T=1025, cell=23),
    _ncell(name="partial_wave_H2504", H=2504, cell=24),
    _ncell(name="partial_chunks_H2504_T2001", H=2504, T=2001, cell=25),
    _ncell(name="partial_fp8_f32_H2500_T3001", dtype=W.F32, H=2500, T=3001, fp8=True, cell=26),
    _ncell(name="wide_no_residual_T2049", residual=False, H=2048, T=2049, cell=27),
    # the small kernel's buffer ranges: rows past T inside a wave, and lanes
    # past the row's last chunk (25 chunks on 32 lanes; 3 on 4)
    _ncell(name="small_H256_T33", H=256, T=33, cell=28),
    _ncell(name="small_H200_T9", H=200, T=9, cell=29),
    _ncell(name="small_fp8_H200_T9", H=200, T=9, fp8=True, cell=30),
    _ncell(name="small_fp8_f32_H12_T7", dtype=W.F32, H=12, T=7, fp8=True, cell=31),
    _ncell(name="small_no_residual_H200_T9", residual=False, H=200, T=9, cell=32),
    _ncell(name="small_f16_H24_T65", dtype=W.F16, H=24, T=65, cell=33),
    # half-chunk lanes: a last wave partly past the row (250 chunks on 256
    # half-chunk pairs), three groups (six waves), and no residual
    _ncell(name="half_H2000_T5", H=2000, T=5, cell=34),
    _ncell(name="half_fp8_H1032_T3", H=1032, T=3, fp8=True, cell=35),
    _ncell(name="half_f16_no_residual_H2048_T64", dtype=W.F16, residual=False, H=2048, T=64,
           cell=36),
    _ncell(name="half_noweight_fp8_H2048_T128", weight=False, fp8=True, H=2048, T=128, cell=37),
    # widths whose 64-chunk groups do not split evenly over four SIMDs take
    # fewer waves per row from 5000 rows x groups: either side of that bound
    # at H = 2560 (5 groups), fp32 at 10 groups and at 6, and 7 groups
    _ncell(name="uneven_H2560_T999", H=2560, T=999, cell=38),
    _ncell(name="uneven_H2560_T1000", H=2560, T=1000, cell=39),
    _ncell(name="uneven_fp8_f32_H2560_T768", dtype=W.F32, H=2560, T=768, fp8=True, cell=40),
    _ncell(name="uneven_H3584_T1023", H=3584, T=1023, cell=41),
    _ncell(name="uneven_fp8_f32_H1536_T1023", dtype=W.F32, H=1536, T=1023, fp8=True, cell=42),
]


@pytest.mark.parametrize("cell", EDGE_NORM, ids=lambda c: c.name)
def test_norm_edges(mbt, orc, cell):
    check_norm_cell(mbt, orc, cell)


@pytest.mark.parametrize("dtype", [W.BF16, W.F16, W.F32])
def test_norm_unaligned(mbt, orc, dtype):
    check_norm_cell(mbt, orc, _ncell(name=f"unaligned_{dtype}", dtype=dtype, cell=30 + dtype),
                    offset=1)


@pytest.mark.parametrize("dtype", [W.BF16, W.F16, W.F32])
def test_norm_no_weight_unaligned(mbt, orc, dtype):
    check_norm_cell(mbt, orc, _ncell(name=f"noweight_unaligned_{dtype}", dtype=dtype,
                                     weight=False, cell=40 + dtype), offset=1)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_norm_no_weight_equals_unit_weight(mbt, dtype):
    """w = NULL gives the bits of a weight of ones (multiplying by exactly 1
    changes nothing), for the vector and the scalar kernel."""
    for H in (1024, 37):
        c = _ncell(name="unit", dtype=dtype, H=H, cell=50 + H)
        i = c.inputs()
        outs = []
        for w in (None, np.full(H, 1.0)):
            x, r = dev(i["x"], dtype), dev(i["residual"], dtype)
            mbt.fused_add_rmsnorm(x, r, None if w is None else dev(W.to_bits(w, dtype), dtype),
                                  c.eps, 0)
            outs.append(host(x, dtype))
        C.check_bitwise(outs[0], outs[1], label=f"no weight vs ones H={H}")


# ---------------------------------------------------------------------------
# gated activations (+ FP8, + calibration) and the quantizer
# ---------------------------------------------------------------------------

def check_act_cell(mbt, orc, cell, offset=0):
    i = cell.inputs()
    dt = cell.dtype
    gu_bits = i["gate_up"]
    t = dev(np.concatenate([np.zeros(offset, gu_bits.dtype), gu_bits.ravel()]), dt)
    gu = t[offset:].view(gu_bits.shape)
    if cell.fp8:
        cal = cell.calibration_inputs()["gate_up"]
        amax_o = orc.gated_act_amax(cal, cell.act, dt)
        amax_g = float(mbt.gated_act_amax(dev(cal, dt), cell.act).item())
        assert abs(amax_g - amax_o) <= 1e-5 * amax_o, f"amax {amax_g} vs {amax_o}"
        inv_scale = W.fp8_inv_scale(amax_o)
        y = mbt.gated_act_fp8(gu, inv_scale, cell.act)
        st = C.check_fp8(y.cpu().numpy(), orc.gated_act_fp8(gu_bits, inv_scale, cell.act, dt),
                         label=cell.name)
    else:
        out = mbt.gated_act(gu, cell.act)
        st = C.check_values(host(out, dt), orc.gated_act(gu_bits, cell.act, dt), dt,
                            label=cell.name)
    print(f"{cell.name}: {st}", flush=True)


ACT_CELLS = [c for c in W.config5_cells() if isinstance(c, W.ActCell)]


@pytest.mark.parametrize("cell", ACT_CELLS, ids=lambda c: c.name)
def test_act_config(mbt, orc, cell):
    check_act_cell(mbt, orc, cell)


def _acell(**kw):
    base = dict(name="aedge", config=92, cell=0, T=5, d=1024, act=W.SILU, dtype=W.BF16)
    base.update(kw)
    return W.ActCell(**base)


EDGE_ACT = [
    _acell(name="odd_d37", d=37, cell=1),
    _acell(name="d1", d=1, act=W.GELU_TANH, cell=2),
    _acell(name="f32_gelu", dtype=W.F32, act=W.GELU_TANH, cell=3),
    _acell(name="f32_silu_fp8", dtype=W.F32, fp8=True, cell=4),
    _acell(name="f16_gelu_fp8", dtype=W.F16, act=W.GELU_TANH, fp8=True, cell=5),
    _acell(name="odd_fp8", d=333, fp8=True, cell=6),
    _acell(name="wide_std", x_std=8.0, act=W.GELU_TANH, cell=7),
    _acell(name="T600", T=600, d=4096, cell=8),
    # half-chunk lanes: a last block partly past d, fp16, and the
    # calibration amax of a narrow launch
    _acell(name="half_partial_d1000", d=1000, T=3, cell=9),
    _acell(name="half_f16_d2056", dtype=W.F16, d=2056, T=7, act=W.GELU_TANH, cell=10),
    # FP8 output takes half-chunk lanes up to 8192 waves (40 per row at
    # d = 10240): either side of that bound, a partial last block, fp16
    _acell(name="half_fp8_d1000", d=1000, T=3, fp8=True, cell=11),
    _acell(name="half_fp8_T204", d=10240, T=204, fp8=True, cell=12),
    _acell(name="full_fp8_T205", d=10240, T=205, act=W.GELU_TANH, fp8=True, cell=13),
    _acell(name="half_f16_fp8_d2056", dtype=W.F16, d=2056, T=7, act=W.GELU_TANH, fp8=True,
           cell=14),
    # rows of whole 256-chunk groups with two chunks per lane take the
    # flat-group kernel: an odd number of groups (the last block's second
    # group past the last row) and blocks straddling two rows, in bf16
    # (FP8 out and its calibration), fp16 and fp32
    _acell(name="flat_odd_groups_fp8", d=10240, T=333, act=W.GELU_TANH, fp8=True, cell=15),
    _acell(name="flat_f16_odd_groups", dtype=W.F16, d=10240, T=333, cell=16),
    _acell(name="flat_f32_gpr3", dtype=W.F32, d=3072, T=521, act=W.GELU_TANH, cell=17),
]


@pytest.mark.parametrize("cell", EDGE_ACT, ids=lambda c: c.name)
def test_act_edges(mbt, orc, cell):
    check_act_cell(mbt, orc, cell)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_act_unaligned(mbt, orc, dtype):
    check_act_cell(mbt, orc, _acell(name=f"unaligned_{dtype}", dtype=dtype, cell=40 + dtype),
                   offset=1)


@pytest.mark.parametrize("rows,pad", [(1, False), (20, False), (50, False), (50, True)],
                         ids=["half_chunk_per_lane", "one_chunk_per_lane", "two_chunks_per_lane",
                              "two_chunks_flat_groups"])
def test_act_exhaustive_bf16_gate(mbt, orc, rows, pad):
    """Every finite bf16 gate value with up = 1: GPU vs oracle, <= 1 ulp.
    One row is a narrow launch (half a chunk per lane); 20 and 50 copies of
    the row make it wide enough for one and two chunks per lane.  Padded
    with zeros to 65536 gate values, a row is 32 whole 256-chunk groups and
    50 rows take the flat-group kernel."""
    bits = np.arange(65536, dtype=np.uint16)
    keep = np.isfinite(W.bits_to_f32(bits, W.BF16))
    bits = bits[keep]
    if pad:
        bits = np.concatenate([bits, np.zeros(65536 - bits.size, np.uint16)])
    gu = np.concatenate([bits, W.to_bits(np.ones(bits.size), W.BF16)])[None, :]
    gu = np.repeat(gu, rows, axis=0)
    for act in (W.SILU, W.GELU_TANH):
        out = host(mbt.gated_act(dev(gu, W.BF16), act), W.BF16)
        C.check_values(out, orc.gated_act(gu, act, W.BF16), W.BF16, label=f"act {act}")


def test_quantize_fp8_exhaustive(mbt, orc):
    """The hardware e4m3fn conversion against the oracle on the same fp32
    inputs: every code value, every midpoint, one fp32 ulp either side,
    saturation, infinities, NaN and a random sweep -- identical codes."""
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.decode_e4m3fn(codes)
    fin = np.unique(vals[np.isfinite(vals)].astype(np.float64))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    g = np.random.default_rng(9)
    rnd = (g.standard_normal(1 << 20) * np.exp2(g.integers(-14, 10, 1 << 20))).astype(np.float32)
    x = np.concatenate([fin.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(-np.inf)),
                        np.float32([448.0, 449.0, 464.0, 480.0, 1e30, np.inf, -np.inf,
                                    -1e30, 0.0, -0.0, 2 ** -10, 2 ** -11, 1e-40, np.nan]),
                        # NaNs of both signs, quiet and signalling payloads
                        np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF,
                                  0xFFFFFFFF], dtype=np.uint32).view(np.float32),
                        rnd]).astype(np.float32)
    for inv_scale in (1.0, 3.0):
        y = mbt.quantize_fp8(torch.from_numpy(x).to(DEV), inv_scale).cpu().numpy()
        yo = orc.quantize_fp8(x, inv_scale)
        nan = np.isnan(x)
        C.check_bitwise(y[~nan], yo[~nan], label=f"quantize inv_scale={inv_scale}")
        # NaN stays NaN.  Both e4m3fn NaN codes (0x7F, 0xFF) denote NaN and a
        # NaN's sign carries no information: the oracle keeps the input's
        # sign, gfx950's conversion gives 0xFF for every NaN, and either is
        # accepted
        assert np.all((y[nan] & 0x7F) == 0x7F) and np.all((yo[nan] & 0x7F) == 0x7F)
    # odd length at a 4-byte offset: the scalar path
    xt = torch.from_numpy(x[:1002].copy()).to(DEV)
    y = mbt.quantize_fp8(xt[1:1002], 1.0).cpu().numpy()
    ok = ~np.isnan(x[1:1002])
    C.check_bitwise(y[ok], orc.quantize_fp8(x[1:1002], 1.0)[ok], label="quantize tail")
