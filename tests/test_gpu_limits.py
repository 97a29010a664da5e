"""The prologue at its row-count limits, on the GPU.

The vector kernels find a row's token with a float reciprocal and one
correction, exact for fewer than 2^24 rows per tensor; at 2^24 rows and more
the library takes the scalar kernel instead.  These cells sit on both sides
of that boundary at full size (gigabytes of input, drawn on the device from
a seeded generator) and check sampled tokens -- the first and last ones, the
ones whose rows cross powers of two, and random ones -- against the oracle
computed on those tokens alone."""
import numpy as np
import pytest
import torch

import compare as C
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (name, Q, K, D, rot, layout, T): rows per tensor T * Q and T * K
LIMIT_CELLS = [
    # 24 heads: 1/24 is inexact in fp32; the last query row is 2^24 - 17
    ("q24k4_rows_below_2p24", 24, 4, 256, 64, W.ROTATE_HALF, (1 << 24) // 24),
    # one head per tensor: the last row is 2^24 - 1, the largest the vector kernel takes
    ("q1k1_rows_2p24_minus_1", 1, 1, 64, 64, W.ROTATE_HALF, (1 << 24) - 1),
    # 2^24 rows: the scalar kernel
    ("q1k1_rows_2p24_scalar", 1, 1, 64, 64, W.INTERLEAVED, 1 << 24),
]


@pytest.fixture(scope="module")
def mbt():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    import memory_bound_transformer_amd as m
    return m


def sample_tokens(T, heads, seed):
    g = np.random.default_rng(seed)
    t = {0, 1, T // 2, T - 2, T - 1}
    for k in range(16, 25):                          # rows crossing 2^k
        for r in ((1 << k) - 1, 1 << k):
            if r // heads < T:
                t.add(r // heads)
    t.update(int(x) for x in g.integers(0, T, 40))
    return np.array(sorted(t), dtype=np.int64)


@pytest.mark.parametrize("case", LIMIT_CELLS, ids=lambda c: c[0])
def test_prologue_row_limits(mbt, case):
    name, Q, K, D, rot, layout, T = case
    dt = W.BF16
    print(f"{name}: T={T} rows q={T * Q} k={T * K}", flush=True)
    q = W.device_normal((96, T, Q, 0), (T, Q, D), 2.0, dt, DEV)
    k = W.device_normal((96, T, K, 1), (T, K, D), 2.0, dt, DEV)
    w_q = W.normal_bits((96, Q, 2), (D,), 0.0, 0.05, dt)
    w_k = W.normal_bits((96, K, 3), (D,), 0.0, 0.05, dt)
    pos = torch.randint(-8, 4104, (T,), generator=torch.Generator(device=DEV).manual_seed(97),
                        device=DEV, dtype=torch.int64)
    cs = W.rope_cache(4096, rot, 1e7)
    qo, ko = mbt.qknorm_rope(q, k, W.to_torch(w_q, dt, DEV), W.to_torch(w_k, dt, DEV),
                             torch.from_numpy(cs).to(DEV), pos, rot, 1e-6, 1, layout)
    torch.cuda.synchronize()
    orc = oracle.default()
    for heads, x, xo, w, label in ((Q, q, qo, w_q, "q"), (K, k, ko, w_k, "k")):
        sel = sample_tokens(T, heads, 98)
        idx = torch.from_numpy(sel).to(DEV)
        xs = W.from_torch(x.index_select(0, idx).contiguous(), dt)
        gs = W.from_torch(xo.index_select(0, idx).contiguous(), dt)
        ps = pos.index_select(0, idx).cpu().numpy()
        ref, _ = orc.qknorm_rope(xs, xs[:, :0], w, w, cs, ps, rot, 1e-6, 1, layout, dt)
        n = orc.rmsnorm_rows(xs, w, 1e-6, 1, dt)
        st = C.check_prologue(gs, ref, n, cs, ps, rot, layout, dt, label=f"{name} {label}")
        print(f"{name} {label}: {len(sel)} tokens {st}", flush=True)
    del q, k, qo, ko, pos
    torch.cuda.empty_cache()
