"""Seeded random shapes against the oracle, on the GPU.

The configuration cells and the hand-picked edges fix the shapes the pages
name; this sweep draws the rest of the accepted domain -- head_dim up to 512
(multiples of the vector width and odd ones), partial and full rotary in both
pairings, any head counts including zero of one kind, short and ragged token
counts, caches of a few hundred rows with positions inside and outside them,
both weight conventions, in place and unaligned storage; norm rows of any
width with and without residual or weight, FP8 or dtype output; activation
rows of any width, and prologue and activation launches wide enough for
two and four chunks per lane -- so every launch-shape branch (vector or
scalar kernel, chunks per lane, load order, segment width) meets inputs it
was not tuned on.  Each case
is fixed by its seed: `random_prologue_17` is always the same cell."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import (check_act_cell, check_norm_cell, check_prologue_cell,  # noqa: F401
                             mbt, orc)

pytestmark = pytest.mark.gpu

DTYPES = (W.BF16, W.F16, W.F32)
HEAD_DIMS = (16, 32, 48, 64, 80, 96, 128, 136, 160, 192, 256, 320, 384, 512, 37, 50, 200)


def _even(x):
    return int(x) & ~1


def prologue_case(n):
    g = np.random.default_rng([93, n])
    D = int(g.choice(HEAD_DIMS))
    rot = int(g.choice([0, D, _even(D // 2), _even(g.integers(0, D + 1))]))
    rot = _even(min(rot, D))
    Q, K = int(g.integers(0, 13)), int(g.integers(0, 7))
    if Q + K == 0:
        Q = 1
    T = int(np.exp(g.uniform(0, np.log(300))))
    mp = int(g.integers(1, 600))
    delta = int(g.integers(0, 2))
    cell = W.PrologueCell(
        name=f"random_prologue_{n}", config=93, cell=n, T=T, Q=Q, K=K, D=D, rot=rot,
        theta=float(10 ** g.uniform(4, 7)), layout=int(g.integers(0, 2)),
        dtype=int(g.choice(DTYPES, p=[0.4, 0.4, 0.2])), weight_offset=delta,
        w_mean=0.0 if delta else 1.0, w_std=0.05, x_std=float(g.choice([0.5, 2.0, 8.0])),
        eps=float(g.choice([1e-6, 1e-3])), max_pos=mp, outside=((1, -1), (2, mp)))
    return cell, dict(offset=int(g.integers(0, 2)), in_place=bool(g.integers(0, 2)))


def norm_case(n):
    g = np.random.default_rng([92, n])
    H = int(g.choice([int(g.integers(1, 6000)), 8 * int(g.integers(1, 700))]))
    weight = bool(g.integers(0, 4) > 0)
    delta = int(g.integers(0, 2)) if weight else 0
    cell = W.NormCell(
        name=f"random_norm_{n}", config=92, cell=n, T=int(g.integers(1, 200)), H=H,
        dtype=int(g.choice(DTYPES)), weight_offset=delta, w_mean=0.0 if delta else 1.0,
        w_std=0.05, x_std=float(g.choice([1.0, 4.0])), residual=bool(g.integers(0, 4) > 0),
        fp8=bool(g.integers(0, 2)), weight=weight)
    return cell, int(g.integers(0, 2))


def act_case(n):
    g = np.random.default_rng([91, n])
    d = int(g.choice([int(g.integers(1, 12000)), 8 * int(g.integers(1, 1500))]))
    cell = W.ActCell(name=f"random_act_{n}", config=91, cell=n, T=int(g.integers(1, 100)), d=d,
                     act=int(g.integers(0, 2)), dtype=int(g.choice(DTYPES)),
                     x_std=float(g.choice([1.5, 6.0])), fp8=bool(g.integers(0, 2)))
    return cell, int(g.integers(0, 2))


def prefill_prologue_case(n):
    """Prologue launches of 2k to 30k head-rows of the vector-kernel head
    dims, so that two and four chunks per lane and every load order (by
    wave count) meet head dims, rotary spans and head counts other than the
    configurations'."""
    g = np.random.default_rng([89, n])
    D = int(g.choice([64, 128, 256, 512]))
    rot = int(g.choice([D, D // 2, D // 4]))
    Q, K = int(g.integers(1, 33)), int(g.integers(1, 9))
    T = max(1, int(g.integers(2_000, 30_000)) // (Q + K))
    mp = int(g.integers(T // 2, 2 * T))
    delta = int(g.integers(0, 2))
    cell = W.PrologueCell(
        name=f"random_prefill_prologue_{n}", config=89, cell=n, T=T, Q=Q, K=K, D=D, rot=rot,
        theta=float(10 ** g.uniform(4, 7)), layout=int(g.integers(0, 2)),
        dtype=int(g.choice(DTYPES, p=[0.5, 0.3, 0.2])), weight_offset=delta,
        w_mean=0.0 if delta else 1.0, w_std=0.05, x_std=2.0, eps=1e-6, max_pos=mp,
        outside=((1, -1), (2, mp)))
    return cell, dict(offset=0, in_place=bool(g.integers(0, 2)))


def prefill_act_case(n):
    """Activation rows wide enough for two chunks per lane (at least 400k
    chunks in the launch): half the widths whole 256-chunk groups (the
    flat-group kernel), the others any multiple of the vector width (one
    block per pair of a row's groups, the last one partly past d)."""
    g = np.random.default_rng([90, n])
    dtype = int(g.choice(DTYPES))
    V = 4 if dtype == W.F32 else 8
    if n % 2 == 0:
        d = 256 * V * int(g.integers(2, 7))
    else:
        d = V * int(g.integers(300, 1600))
    chunks = d // V
    T = -(-int(g.integers(400_000, 1_200_000)) // chunks)
    cell = W.ActCell(name=f"random_prefill_act_{n}", config=90, cell=n, T=T, d=d,
                     act=int(g.integers(0, 2)), dtype=dtype,
                     x_std=float(g.choice([1.5, 6.0])), fp8=bool(g.integers(0, 2)))
    return cell, 0                              # aligned: the vector kernels


@pytest.mark.parametrize("n", range(48), ids=lambda n: f"random_prologue_{n}")
def test_random_prologue(mbt, orc, n):
    cell, kw = prologue_case(n)
    print(f"{cell.name}: T={cell.T} Q={cell.Q} K={cell.K} D={cell.D} rot={cell.rot} "
          f"layout={cell.layout} dtype={cell.dtype} max_pos={cell.max_pos} {kw}", flush=True)
    check_prologue_cell(mbt, orc, cell, **kw)


@pytest.mark.parametrize("n", range(32), ids=lambda n: f"random_norm_{n}")
def test_random_norm(mbt, orc, n):
    cell, offset = norm_case(n)
    print(f"{cell.name}: T={cell.T} H={cell.H} dtype={cell.dtype} res={cell.residual} "
          f"w={cell.weight} fp8={cell.fp8} offset={offset}", flush=True)
    check_norm_cell(mbt, orc, cell, offset=offset)


@pytest.mark.parametrize("n", range(24), ids=lambda n: f"random_act_{n}")
def test_random_act(mbt, orc, n):
    cell, offset = act_case(n)
    print(f"{cell.name}: T={cell.T} d={cell.d} act={cell.act} dtype={cell.dtype} "
          f"fp8={cell.fp8} offset={offset}", flush=True)
    check_act_cell(mbt, orc, cell, offset=offset)


@pytest.mark.parametrize("n", range(12), ids=lambda n: f"random_prefill_act_{n}")
def test_random_prefill_act(mbt, orc, n):
    cell, offset = prefill_act_case(n)
    print(f"{cell.name}: T={cell.T} d={cell.d} act={cell.act} dtype={cell.dtype} "
          f"fp8={cell.fp8} offset={offset}", flush=True)
    check_act_cell(mbt, orc, cell, offset=offset)


@pytest.mark.parametrize("n", range(12), ids=lambda n: f"random_prefill_prologue_{n}")
def test_random_prefill_prologue(mbt, orc, n):
    cell, kw = prefill_prologue_case(n)
    print(f"{cell.name}: T={cell.T} Q={cell.Q} K={cell.K} D={cell.D} rot={cell.rot} "
          f"layout={cell.layout} dtype={cell.dtype} max_pos={cell.max_pos} {kw}", flush=True)
    check_prologue_cell(mbt, orc, cell, **kw)
