"""Degenerate rows through the HIP path, against the oracle, for every op that
normalises (the QK-norm + RoPE prologue, the residual RMSNorm in place, to FP8
and its calibration amax) in every dtype, at eps = 0 and eps > 0:

* a zero row: exactly zero with eps > 0, and 0 * (1 / sqrt(0)) = NaN on both
  sides with eps = 0;
* power-of-two constant rows: x / rms is exactly +-1, so the output is
  +-R(w + delta) (the oracle's closed-form pin, here on the GPU);
* rows whose sum of squares overflows fp32 (bf16 / fp32 values near 3e38):
  1 / sqrt(inf) = 0, so every output is a signed zero;
* a row holding one infinity (that element NaN, the rest signed zeros) and a
  row holding one NaN (NaN throughout, its rotation included);
* subnormal rows, whose squares underflow to zero (the output is then
  x / sqrt(eps) (w + delta));
* a random row beside them, as a control.

And special gate and up values through the gated activation.

The comparison rules are the parity tests' (compare.py); a NaN matches any
NaN, since neither side's NaN payload or sign carries information.  Each row
kind is repeated so that both the narrow (decode-width) and the wide launch
shapes of each op see it."""
import numpy as np
import pytest
import torch

import compare as C
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = [W.BF16, W.F16, W.F32]
DT_IDS = ["bf16", "f16", "f32"]


@pytest.fixture(scope="module")
def mbt():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    import memory_bound_transformer_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def rows(dtype, D, seed):
    """(names, fp32 values [n, D]) of the degenerate row kinds for dtype."""
    g = np.random.default_rng([seed, dtype, D])
    kinds = {
        "zero": np.zeros(D),
        "pow2": np.full(D, 2.0),
        "neg_pow2": np.full(D, -0.25),
        "one_inf": g.standard_normal(D),
        "one_nan": g.standard_normal(D),
        "random": g.standard_normal(D) * 2.0,
    }
    kinds["one_inf"][D // 3] = np.inf
    kinds["one_nan"][D // 2] = np.nan
    if dtype in (W.BF16, W.F32):
        # |x| ~ 3e38: x^2 overflows, so the sum of squares is +inf
        kinds["huge"] = np.where(np.arange(D) % 2, 3.0e38, -2.5e38)
        # subnormal in bf16 and fp32: every square underflows to zero
        kinds["subnormal"] = g.choice([-1.0, 1.0], D) * g.integers(1, 64, D) * 2.0 ** -133
    else:
        # fp16 subnormals (below 2^-14); their squares are normal fp32
        kinds["subnormal"] = g.choice([-1.0, 1.0], D) * g.integers(1, 64, D) * 2.0 ** -24
    names = list(kinds)
    return names, np.stack([kinds[n] for n in names]).astype(np.float32)


def canon_nan(bits, dtype):
    """16-bit patterns with every NaN replaced by one canonical NaN."""
    bits = np.array(bits, copy=True)
    if dtype != W.F32:
        bits[np.isnan(W.bits_to_f32(bits, dtype))] = 0x7FC0 if dtype == W.BF16 else 0x7E00
    return bits


def check_bitwise_nan(gpu, ora, dtype, label):
    """Bit-identical, except that a NaN matches any NaN."""
    if dtype == W.F32:
        g, o = np.asarray(gpu, np.float32), np.asarray(ora, np.float32)
        nan = np.isnan(g) & np.isnan(o)
        C.check_bitwise(np.where(nan, 0.0, g).astype(np.float32),
                        np.where(nan, 0.0, o).astype(np.float32), label)
    else:
        C.check_bitwise(canon_nan(gpu, dtype), canon_nan(ora, dtype), label)


def expected_specials(names, out_f32, eps, label):
    """The closed-form outcomes the module docstring lists, row by row."""
    for r, name in enumerate(names):
        v = out_f32[r]
        if name == "zero":
            if eps > 0:
                assert np.all(v == 0.0), f"{label}: zero row not zero"
            else:
                assert np.all(np.isnan(v)), f"{label}: zero row at eps 0 not NaN"
        elif name == "huge":
            assert np.all(v == 0.0), f"{label}: overflowing row not zero"
        elif name == "one_nan":
            assert np.all(np.isnan(v)), f"{label}: NaN row not NaN throughout"
        elif name == "one_inf":
            nan = np.isnan(v)
            assert nan.sum() == 1 and np.all(v[~nan] == 0.0), f"{label}: infinity row"


@pytest.mark.parametrize("eps", [0.0, 1e-6], ids=["eps0", "eps1e-6"])
@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("H,reps", [(2048, 1), (2560, 1), (2048, 200), (1001, 3)],
                         ids=["H2048_narrow", "H2560_narrow", "H2048_wide", "H1001_scalar"])
def test_norm_degenerate_rows(mbt, orc, dtype, H, reps, eps):
    names, vals = rows(dtype, H, seed=1)
    n = len(names)
    x_bits = W.to_bits(np.tile(vals, (reps, 1)), dtype)
    g = np.random.default_rng([2, dtype, H])
    w_bits = W.to_bits(g.normal(0.0, 0.1, H), dtype)
    print(f"norm degenerate dtype={dtype} H={H} T={x_bits.shape[0]} eps={eps}", flush=True)
    for wo in (0, 1):
        # in place, no residual: x <- RMSNorm(x)
        x = W.to_torch(x_bits, dtype, DEV)
        mbt.fused_add_rmsnorm(x, None, W.to_torch(w_bits, dtype, DEV), eps, wo)
        xo, _ = orc.fused_add_rmsnorm(x_bits, None, w_bits, eps, wo, dtype)
        got = W.from_torch(x, dtype)
        label = f"norm wo={wo}"
        C.check_values(got, xo, dtype, label=label)
        expected_specials(names, W.bits_to_f32(got[:n], dtype) if dtype != W.F32 else got[:n],
                          eps, label)
        # the residual form: x = 0, residual = the rows, so R(x + r) = r
        z = np.zeros_like(x_bits)
        x = W.to_torch(z, dtype, DEV)
        r = W.to_torch(x_bits, dtype, DEV)
        mbt.fused_add_rmsnorm(x, r, W.to_torch(w_bits, dtype, DEV), eps, wo)
        xo, ro = orc.fused_add_rmsnorm(z, x_bits, w_bits, eps, wo, dtype)
        C.check_values(W.from_torch(x, dtype), xo, dtype, label=f"{label} residual form")
        check_bitwise_nan(W.from_torch(r, dtype), ro, dtype, f"{label} residual sum")
        # FP8 out: the codes, NaN codes matching NaN codes
        x = W.to_torch(z, dtype, DEV)
        r = W.to_torch(x_bits, dtype, DEV)
        y = mbt.fused_add_rmsnorm_fp8(x, r, W.to_torch(w_bits, dtype, DEV), 3.0, eps, wo)
        yo, _ = orc.fused_add_rmsnorm_fp8(z, x_bits, w_bits, 3.0, eps, wo, dtype)
        C.check_fp8(y.cpu().numpy(), yo, label=f"{label} fp8")
        # calibration amax over the kinds without a NaN output (a NaN has no
        # order); at eps = 0 a subnormal row normalises to infinities
        fin = [i for i, nm in enumerate(names)
               if nm not in ("one_inf", "one_nan") and not (nm == "zero" and eps == 0.0)]
        xf = np.tile(W.to_bits(vals[fin], dtype), (reps, 1))
        am = float(mbt.fused_add_rmsnorm_amax(W.to_torch(xf, dtype, DEV), None,
                                              W.to_torch(w_bits, dtype, DEV), eps, wo).item())
        amo = orc.fused_add_rmsnorm_amax(xf, None, w_bits, eps, wo, dtype)
        assert am == amo or abs(am - amo) <= 1e-5 * amo, f"{label} amax {am} vs {amo}"


@pytest.mark.parametrize("eps", [0.0, 1e-6], ids=["eps0", "eps1e-6"])
@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("D,rot,layout,reps",
                         [(128, 128, W.ROTATE_HALF, 1), (256, 64, W.ROTATE_HALF, 60),
                          (128, 128, W.INTERLEAVED, 1), (72, 24, W.ROTATE_HALF, 2)],
                         ids=["D128_full_decode", "D256_rot64_prefill", "D128_interleaved",
                              "D72_scalar"])
def test_prologue_degenerate_rows(mbt, orc, dtype, D, rot, layout, reps, eps):
    names, vals = rows(dtype, D, seed=3)
    n = len(names)
    Q, K = 3, 1
    # token t holds kind t in every head (q and k), repeated reps times
    T = n * reps
    base = np.tile(vals, (reps, 1))
    q_bits = W.to_bits(np.repeat(base[:, None, :], Q, axis=1), dtype)
    k_bits = W.to_bits(base[:, None, :], dtype)
    g = np.random.default_rng([4, dtype, D])
    wq = W.to_bits(g.normal(0.0, 0.1, D), dtype)
    wk = W.to_bits(g.normal(0.0, 0.1, D), dtype)
    max_pos = 64
    cs = W.rope_cache(max_pos, rot, 1e4)
    # every other token outside the cache (norm only)
    pos = np.where(np.arange(T) % 2 == 0, np.arange(T) % max_pos, max_pos + np.arange(T))
    pos = pos.astype(np.int64)
    print(f"prologue degenerate dtype={dtype} D={D} rot={rot} layout={layout} T={T} "
          f"eps={eps}", flush=True)
    for wo in (0, 1):
        qo, ko = mbt.qknorm_rope(W.to_torch(q_bits, dtype, DEV), W.to_torch(k_bits, dtype, DEV),
                                 W.to_torch(wq, dtype, DEV), W.to_torch(wk, dtype, DEV),
                                 torch.from_numpy(cs).to(DEV), torch.from_numpy(pos).to(DEV),
                                 rot, eps, wo, layout)
        oq, ok_ = orc.qknorm_rope(q_bits, k_bits, wq, wk, cs, pos, rot, eps, wo, layout, dtype)
        for name, got_t, ora, x, w in (("q", qo, oq, q_bits, wq), ("k", ko, ok_, k_bits, wk)):
            got = W.from_torch(got_t, dtype)
            H = x.shape[1]
            n_ora = orc.rmsnorm_rows(x.reshape(-1, D), w, eps, wo, dtype).reshape(T, H, D)
            label = f"prologue {name} wo={wo}"
            C.check_prologue(got, ora, n_ora, cs, pos, rot, layout, dtype, label=label)
            gf = got if dtype == W.F32 else W.bits_to_f32(got, dtype)
            expected_specials(names, gf[:n, 0, :], eps, label)


@pytest.mark.parametrize("dtype", DTYPES, ids=DT_IDS)
@pytest.mark.parametrize("d,T", [(1024, 4), (10240, 40), (1000, 3)],
                         ids=["narrow", "wide", "scalar"])
def test_act_degenerate_values(mbt, orc, dtype, d, T):
    """Gate values +-inf, NaN, +-0, the largest finite magnitudes and
    subnormals, against up values 1, +-inf, NaN, 0 and a random one: act(g) u
    on the GPU agrees with the oracle (inf * 0 and NaN propagate as NaN on
    both sides), to a dtype and to FP8."""
    big = 3.0e38 if dtype != W.F16 else 65504.0
    tiny = 2.0 ** -133 if dtype != W.F16 else 2.0 ** -24
    gates = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, big, -big, tiny, -tiny, 1.5, -1.5,
                      -90.0, 30.0], np.float32)
    ups = np.array([1.0, np.inf, -np.inf, np.nan, 0.0, -2.0], np.float32)
    gg, uu = np.meshgrid(gates, ups)
    g_row, u_row = gg.ravel(), uu.ravel()                       # every pair once
    rng = np.random.default_rng([5, dtype, d])
    g = rng.standard_normal((T, d)).astype(np.float32)
    u = rng.standard_normal((T, d)).astype(np.float32)
    for t in range(T):                                          # the pairs in every row
        at = (t * 97) % (d - g_row.size)
        g[t, at:at + g_row.size] = g_row
        u[t, at:at + u_row.size] = u_row
    gu = W.to_bits(np.concatenate([g, u], axis=1), dtype)
    print(f"act degenerate dtype={dtype} d={d} T={T}", flush=True)
    for act in (W.SILU, W.GELU_TANH):
        out = W.from_torch(mbt.gated_act(W.to_torch(gu, dtype, DEV), act), dtype)
        C.check_values(out, orc.gated_act(gu, act, dtype), dtype, label=f"act {act}")
        y = mbt.gated_act_fp8(W.to_torch(gu, dtype, DEV), 0.5, act).cpu().numpy()
        C.check_fp8(y, orc.gated_act_fp8(gu, 0.5, act, dtype), label=f"act {act} fp8")
