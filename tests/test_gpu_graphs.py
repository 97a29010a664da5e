"""The library's launches captured in a HIP graph and replayed: the decode
layer's memory-bound sequence (residual RMSNorm -> FP8, the QK-norm + RoPE
prologue, residual RMSNorm -> FP8, SiLU-gate -> FP8) plus a calibration pass
whose amax is cleared by a fill kernel inside the graph.  Each replay starts
from the same inputs (reset eagerly, with other eager work and a
synchronisation between replays) and must give the eager run's bits; the
eager run is checked against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import compare as C
import workloads as W

pytestmark = pytest.mark.gpu

T, H, Q, K, D, ROT, DFF = 64, 2048, 16, 2, 256, 64, 10240
EPS = 1e-6
SCALE_N, SCALE_A = 448.0 / 12.0, 448.0 / 20.0


@pytest.fixture(scope="module")
def mbt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_transformer_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle.default()


def _host_inputs():
    g = np.random.default_rng([61, 1])
    bf = lambda a: W.to_bits(a, W.BF16)
    return {
        "x": bf(g.standard_normal((T, H))), "res": bf(g.standard_normal((T, H))),
        "wn": bf(g.normal(1.0, 0.05, H)),
        "q": bf(g.standard_normal((T, Q, D)) * 2.0), "k": bf(g.standard_normal((T, K, D)) * 2.0),
        "wq": bf(g.normal(0.0, 0.05, D)), "wk": bf(g.normal(0.0, 0.05, D)),
        "cs": W.rope_cache(4096, ROT, 1e7), "pos": g.integers(0, 4096, T).astype(np.int64),
        "gu": bf(g.standard_normal((T, 2 * DFF)) * 1.5),
    }


def _device(h):
    d = {}
    for k, v in h.items():
        if k in ("cs", "pos"):
            d[k] = torch.from_numpy(v).to("cuda:0")
        else:
            d[k] = W.to_torch(v, W.BF16, "cuda:0")
    return d


def _outputs():
    dev = "cuda:0"
    u8 = torch.uint8
    return {"y1": torch.empty((T, H), dtype=u8, device=dev),
            "qo": torch.empty((T, Q, D), dtype=torch.bfloat16, device=dev),
            "ko": torch.empty((T, K, D), dtype=torch.bfloat16, device=dev),
            "y2": torch.empty((T, H), dtype=u8, device=dev),
            "ya": torch.empty((T, DFF), dtype=u8, device=dev),
            "amax": torch.empty(1, dtype=torch.float32, device=dev)}


def _sequence(mbt, i, o):
    """One decode-layer pass; the residual is updated in place twice."""
    mbt.fused_add_rmsnorm_fp8(i["x"], i["res"], i["wn"], SCALE_N, EPS, 0, y=o["y1"])
    mbt.qknorm_rope(i["q"], i["k"], i["wq"], i["wk"], i["cs"], i["pos"], ROT, EPS, 1,
                    q_out=o["qo"], k_out=o["ko"])
    mbt.fused_add_rmsnorm_fp8(i["x"], i["res"], i["wn"], SCALE_N, EPS, 0, y=o["y2"])
    mbt.gated_act_fp8(i["gu"], SCALE_A, mbt.SILU, out=o["ya"])
    o["amax"].zero_()                               # a fill kernel, not a memset
    mbt.fused_add_rmsnorm_amax(i["x"], i["res"], i["wn"], EPS, 0, amax=o["amax"])


def _snapshot(i, o):
    s = {k: v.clone() for k, v in o.items()}
    s["res"] = i["res"].clone()
    return s


def test_graph_replays_match_eager(mbt, orc):
    h = _host_inputs()
    print(f"graph: decode-layer sequence T={T}", flush=True)
    # eager
    ie, oe = _device(h), _outputs()
    _sequence(mbt, ie, oe)
    torch.cuda.synchronize()
    eager = _snapshot(ie, oe)

    # the eager run against the oracle
    r1 = h["res"].copy()
    y1 = orc.fused_add_rmsnorm_fp8(h["x"], r1, h["wn"], SCALE_N, EPS, 0, W.BF16)
    qo, ko = orc.qknorm_rope(h["q"], h["k"], h["wq"], h["wk"], h["cs"], h["pos"], ROT, EPS, 1,
                             W.ROTATE_HALF, W.BF16)
    y2 = orc.fused_add_rmsnorm_fp8(h["x"], y1[1], h["wn"], SCALE_N, EPS, 0, W.BF16)
    ya = orc.gated_act_fp8(h["gu"], SCALE_A, W.SILU, W.BF16)
    am = orc.fused_add_rmsnorm_amax(h["x"], y2[1], h["wn"], EPS, 0, W.BF16)
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    C.check_fp8(eager["y1"].cpu().numpy(), y1[0], "y1")
    C.check_fp8(eager["y2"].cpu().numpy(), y2[0], "y2")
    C.check_fp8(eager["ya"].cpu().numpy(), ya, "act")
    C.check_bitwise(bits(eager["res"]), y2[1], "residual after two updates")
    n_q = orc.rmsnorm_rows(h["q"].reshape(-1, D), h["wq"], EPS, 1, W.BF16).reshape(T, Q, D)
    C.check_prologue(bits(eager["qo"]), qo, n_q, h["cs"], h["pos"], ROT, W.ROTATE_HALF,
                     W.BF16, label="q")
    n_k = orc.rmsnorm_rows(h["k"].reshape(-1, D), h["wk"], EPS, 1, W.BF16).reshape(T, K, D)
    C.check_prologue(bits(eager["ko"]), ko, n_k, h["cs"], h["pos"], ROT, W.ROTATE_HALF,
                     W.BF16, label="k")
    assert abs(float(eager["amax"][0]) - am) <= 1e-5 * am

    # captured once, replayed three times from reset inputs
    ig, og = _device(h), _outputs()
    res0 = ig["res"].clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        _sequence(mbt, ig, og)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"graph: replay {rep}", flush=True)
        ig["res"].copy_(res0)
        for v in og.values():
            v.fill_(0x5A if v.dtype == torch.uint8 else 7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(ig, og)
        for key, ref in eager.items():
            assert torch.equal(got[key], ref), f"replay {rep}: {key} differs from the eager run"
        # eager work of the program's own between replays
        _sequence(mbt, ie, oe)
        torch.cuda.synchronize()
