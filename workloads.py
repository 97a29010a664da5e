"""Seeded synthetic workloads shared by the tests, the smoke check and bench.py.

This module holds input generation only: random draws, casts to the storage
dtype through library routines (torch / numpy), the caller-built rotary
cos/sin cache and the list of configuration cells.  None of the operations'
arithmetic lives here, so the oracle and the HIP path can both consume its
output without sharing any of the method.

No dataset or trained weight is involved: the pages measure on model
*shapes* (Qwen3 / Gemma 3 decode widths in "thox-edge-ops v2", section 7.1;
the 256-wide text heads of ninfer PR #273, model geometry table), so random
tensors at those shapes stand in for activations and norm weights.

Recipe: every tensor is drawn from ``numpy.random.default_rng([config, cell,
tensor])`` in float64, cast to float32, then rounded to the storage dtype
(bf16 through torch's round-to-nearest-even cast, fp16 through numpy's).
Tensor ids: 0 q / x / gate_up, 1 k / residual, 2 w_q / w, 3 w_k, 4 positions.
"""
from dataclasses import dataclass

import numpy as np
import torch

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
TORCH_DTYPES = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}
STORAGE = {F32: np.float32, F16: np.uint16, BF16: np.uint16}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}
ROTATE_HALF, INTERLEAVED = 0, 1
SILU, GELU_TANH = 0, 1

# tensor ids inside one cell's seed
T_Q, T_K, T_WQ, T_WK, T_POS = 0, 1, 2, 3, 4
CALIBRATION_TENSOR = 99


def rng(*key):
    return np.random.default_rng([int(k) for k in key])


def to_bits(values, dtype):
    """float array -> raw storage bits of `dtype` (RNE, by library casts)."""
    f32 = np.ascontiguousarray(values, dtype=np.float32)
    if dtype == F32:
        return f32
    if dtype == F16:
        return f32.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits, dtype):
    """raw storage bits -> float32 values (exact, by library casts)."""
    if dtype == F32:
        return np.asarray(bits, dtype=np.float32)
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float32)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()


def normal_bits(key, shape, mean, std, dtype):
    g = rng(*key)
    return to_bits(g.normal(mean, std, size=shape), dtype)


def device_normal(key, shape, std, dtype, device):
    """Seeded N(0, std) tensor drawn on the device, in the storage dtype, for
    inputs too large to draw on the host (gigabytes at the row-count limits).
    The same key gives the same bits; tests copy sampled rows back to the
    host, so the oracle and the kernels consume identical inputs."""
    seed = int(np.random.SeedSequence([int(k) for k in key]).generate_state(1)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (x * std).to(TORCH_DTYPES[dtype])


def rope_cache(max_pos, rot_dim, theta):
    """Caller-side rotary cache, fp32 [max_pos][rot_dim]: cos in the first
    rot_dim/2 columns, sin in the last rot_dim/2.  Angle of pair i at position
    p is p * theta^(-2i/rot_dim) (RoFormer's frequency schedule, with the
    exponent taken over the rotated width), evaluated in float64 and rounded
    to fp32 once."""
    half = rot_dim // 2
    if half == 0:
        return np.zeros((max_pos, 0), dtype=np.float32)
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rot_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def to_torch(bits, dtype, device="cpu"):
    """Raw storage bits -> a torch tensor of the matching dtype (a copy)."""
    a = np.ascontiguousarray(bits)
    if dtype == F32:
        t = torch.from_numpy(a.astype(np.float32, copy=True))
    else:
        t = torch.from_numpy(a.view(np.int16).copy()).view(TORCH_DTYPES[dtype])
    return t.to(device)


def from_torch(t, dtype):
    """torch tensor -> raw storage bits (numpy, on the host)."""
    t = t.detach().to("cpu").contiguous()
    if dtype == F32:
        return t.numpy().astype(np.float32, copy=True)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# --------------------------------------------------------------------------
# Configuration cells.
# --------------------------------------------------------------------------

@dataclass
class PrologueCell:
    name: str
    config: int
    cell: int
    T: int
    Q: int
    K: int
    D: int
    rot: int
    theta: float
    layout: int
    dtype: int
    weight_offset: int
    w_mean: float
    w_std: float
    x_std: float
    eps: float = 1e-6
    max_pos: int = 4096
    positions: str = "uniform"          # "uniform" in [0, max_pos) or "arange"
    outside: tuple = ()                 # (index, position) overrides
    in_place: bool = False

    def inputs(self):
        k = (self.config, self.cell)
        q = normal_bits(k + (T_Q,), (self.T, self.Q, self.D), 0.0, self.x_std, self.dtype)
        kk = normal_bits(k + (T_K,), (self.T, self.K, self.D), 0.0, self.x_std, self.dtype)
        wq = normal_bits(k + (T_WQ,), (self.D,), self.w_mean, self.w_std, self.dtype)
        wk = normal_bits(k + (T_WK,), (self.D,), self.w_mean, self.w_std, self.dtype)
        if self.positions == "arange":
            pos = np.arange(self.T, dtype=np.int64)
        else:
            pos = rng(*k, T_POS).integers(0, self.max_pos, size=self.T, dtype=np.int64)
        for i, p in self.outside:
            if i < self.T:
                pos[i] = p
        cs = rope_cache(self.max_pos, self.rot, self.theta)
        return dict(q=q, k=kk, w_q=wq, w_k=wk, pos=pos, cos_sin=cs)

    def bytes_algorithmic(self):
        """Bytes the op must move (q, k read + written; cos/sin rows of the
        T tokens; both weight vectors; positions)."""
        s = ELEM_BYTES[self.dtype]
        return (2 * (self.Q + self.K) * self.D * s * self.T + self.T * self.rot * 4
                + 2 * self.D * s + 8 * self.T)

    def bytes_logical(self):
        """q, k read + q_out, k_out written only (the PR's 'logical traffic')."""
        return 2 * (self.Q + self.K) * self.D * ELEM_BYTES[self.dtype] * self.T


@dataclass
class NormCell:
    name: str
    config: int
    cell: int
    T: int
    H: int
    dtype: int
    weight_offset: int
    w_mean: float
    w_std: float
    x_std: float = 1.0
    eps: float = 1e-6
    residual: bool = True
    fp8: bool = False
    weight: bool = True         # False: no weight (w = None, weight_offset 0)

    def inputs(self):
        k = (self.config, self.cell)
        x = normal_bits(k + (T_Q,), (self.T, self.H), 0.0, self.x_std, self.dtype)
        r = normal_bits(k + (T_K,), (self.T, self.H), 0.0, self.x_std, self.dtype) \
            if self.residual else None
        w = normal_bits(k + (T_WQ,), (self.H,), self.w_mean, self.w_std, self.dtype) \
            if self.weight else None
        return dict(x=x, residual=r, w=w)

    def calibration_inputs(self):
        """Inputs of the one calibration pass: same shapes, another seed."""
        k = (self.config, self.cell, CALIBRATION_TENSOR)
        x = normal_bits(k + (T_Q,), (self.T, self.H), 0.0, self.x_std, self.dtype)
        r = normal_bits(k + (T_K,), (self.T, self.H), 0.0, self.x_std, self.dtype) \
            if self.residual else None
        return dict(x=x, residual=r)

    def bytes_algorithmic(self):
        s = ELEM_BYTES[self.dtype]
        rd = 2 if self.residual else 1          # x (+ residual) read
        wb = self.H * s if self.weight else 0   # the weight, once
        if self.fp8:
            wr = (1 if self.residual else 0) * s + 1
            return (rd * s + wr) * self.H * self.T + wb
        wr = rd                                 # x (+ residual) written back
        return (rd + wr) * s * self.H * self.T + wb


@dataclass
class ActCell:
    name: str
    config: int
    cell: int
    T: int
    d: int
    act: int
    dtype: int
    x_std: float = 1.5
    fp8: bool = False

    def inputs(self):
        k = (self.config, self.cell)
        return dict(gate_up=normal_bits(k + (T_Q,), (self.T, 2 * self.d), 0.0, self.x_std,
                                        self.dtype))

    def calibration_inputs(self):
        k = (self.config, self.cell, CALIBRATION_TENSOR)
        return dict(gate_up=normal_bits(k + (T_Q,), (self.T, 2 * self.d), 0.0, self.x_std,
                                        self.dtype))

    def bytes_algorithmic(self):
        s = ELEM_BYTES[self.dtype]
        return (2 * self.d * s + self.d * (1 if self.fp8 else s)) * self.T


@dataclass
class AdaCell:
    """Adaptive RMSNorm inputs: rows x (and a residual stream) ~ N(0, x_std),
    and one synthetic style vector per call -- scale, shift ~ N(0, 0.1) and a
    residual gate ~ N(1, 0.1) -- standing in for the per-prompt modulation
    the pages describe (no model weights exist here)."""
    name: str
    config: int
    cell: int
    T: int
    H: int
    dtype: int
    residual: bool = True
    gate: bool = True
    fp8: bool = False
    x_std: float = 1.0
    eps: float = 1e-6

    def inputs(self):
        k = (self.config, self.cell)
        shp = (self.T, self.H)
        return dict(
            x=normal_bits(k + (T_Q,), shp, 0.0, self.x_std, self.dtype),
            residual=normal_bits(k + (T_K,), shp, 0.0, self.x_std, self.dtype)
            if self.residual else None,
            gate=normal_bits(k + (T_WK,), (self.H,), 1.0, 0.1, self.dtype)
            if self.gate else None,
            scale=normal_bits(k + (T_WQ,), (self.H,), 0.0, 0.1, self.dtype),
            shift=normal_bits(k + (T_POS,), (self.H,), 0.0, 0.1, self.dtype))

    def calibration_inputs(self):
        k = (self.config, self.cell, CALIBRATION_TENSOR)
        shp = (self.T, self.H)
        return dict(x=normal_bits(k + (T_Q,), shp, 0.0, self.x_std, self.dtype),
                    residual=normal_bits(k + (T_K,), shp, 0.0, self.x_std, self.dtype)
                    if self.residual else None)

    def bytes_algorithmic(self):
        s = ELEM_BYTES[self.dtype]
        rd = 2 if self.residual else 1                   # x (+ residual) read
        vec = (3 if self.gate else 2) * self.H * s       # style vectors, once
        wr = (1 if self.residual else 0) * s + (1 if self.fp8 else s)
        return (rd * s + wr) * self.H * self.T + vec


# Configuration 1: Qwen3-style per-head QK-norm + RoPE, head_dim 128, full
# rotary, (Q, K) = (16, 8), four tokens, one of them at position 4096 (just
# outside a 4096-row cache: normalised, not rotated).
def config1_cells():
    base = dict(config=1, Q=16, K=8, D=128, rot=128, theta=1e6, layout=ROTATE_HALF,
                dtype=BF16, weight_offset=0, w_mean=1.0, w_std=0.05, x_std=1.0)
    return [
        PrologueCell(name="qwen3_d128_T4", cell=0, T=4, outside=((1, 4096),), **base),
        PrologueCell(name="qwen3_d128_T4_negpos", cell=1, T=4, outside=((1, -1),), **base),
    ]


# Configuration 2: 256-wide text heads with a 64-channel rotation, (16, 2),
# offset weight (1 + w), theta 1e7, decode widths.
def config2_cells():
    base = dict(config=2, Q=16, K=2, D=256, rot=64, theta=1e7, layout=ROTATE_HALF,
                dtype=BF16, weight_offset=1, w_mean=0.0, w_std=0.05, x_std=2.0)
    return [PrologueCell(name=f"text16x2_T{T}", cell=i, T=T, **base)
            for i, T in enumerate((1, 8, 32, 64, 128))]


# Configuration 3: the same prologue at prefill widths, (24, 4) and (16, 2),
# bf16 and fp16, positions 0..T-1; plus the interleaved layout with full
# rotary on head_dim 256.
def config3_cells():
    cells = []
    i = 0
    for dtype in (BF16, F16):
        for (Q, K) in ((24, 4), (16, 2)):
            for T in (256, 512, 1024, 2048):
                cells.append(PrologueCell(
                    name=f"prefill{Q}x{K}_{DTYPE_NAMES[dtype]}_T{T}", config=3, cell=i,
                    T=T, Q=Q, K=K, D=256, rot=64, theta=1e7, layout=ROTATE_HALF,
                    dtype=dtype, weight_offset=1, w_mean=0.0, w_std=0.05, x_std=2.0,
                    positions="arange"))
                i += 1
    # widths 256 and 2048 first, then 512 and 1024, so each cell keeps the
    # seed it had before the middle widths were added
    for widths in ((256, 2048), (512, 1024)):
        for (Q, K) in ((24, 4), (16, 2)):
            for T in widths:
                cells.append(PrologueCell(
                    name=f"interleaved{Q}x{K}_T{T}", config=3, cell=i, T=T, Q=Q, K=K, D=256,
                    rot=256, theta=1e7, layout=INTERLEAVED, dtype=BF16, weight_offset=1,
                    w_mean=0.0, w_std=0.05, x_std=2.0, positions="arange"))
                i += 1
    return cells


# Configuration 4: fused residual-add RMSNorm, in place.
def config4_cells():
    cells = []
    i = 0
    for dtype in (F32, F16, BF16):
        for H in (2560, 1024):
            for T in (1, 16, 128, 512):
                for delta, wm in ((0, 1.0), (1, 0.0)):
                    cells.append(NormCell(
                        name=f"resnorm_{DTYPE_NAMES[dtype]}_H{H}_T{T}_d{delta}", config=4,
                        cell=i, T=T, H=H, dtype=dtype, weight_offset=delta, w_mean=wm,
                        w_std=0.05))
                    i += 1
    return cells


# Configuration 5: gated activations (bf16 out and static-FP8 out) and the
# residual-add RMSNorm emitting FP8 at D=2048, T=512.
def config5_cells():
    cells = []
    i = 0
    for T in (1, 64, 512):
        for act in (SILU, GELU_TANH):
            for fp8 in (False, True):
                cells.append(ActCell(
                    name=f"gated_{'silu' if act == SILU else 'gelu'}_T{T}"
                         f"{'_fp8' if fp8 else ''}",
                    config=5, cell=i, T=T, d=10240, act=act, dtype=BF16, fp8=fp8))
                i += 1
    for delta, wm in ((0, 1.0), (1, 0.0)):
        cells.append(NormCell(name=f"resnorm_fp8_D2048_T512_d{delta}", config=5, cell=i,
                              T=512, H=2048, dtype=BF16, weight_offset=delta, w_mean=wm,
                              w_std=0.05, fp8=True))
        i += 1
    return cells


def all_cells():
    return (config1_cells() + config2_cells() + config3_cells() + config4_cells()
            + config5_cells())


def fp8_inv_scale(amax):
    """Static scale from one calibration pass: map the calibration amax onto
    the largest finite e4m3fn magnitude (448).  Computed once on the host and
    handed, as the same float, to every consumer."""
    return float(np.float32(448.0 / float(amax)))
