"""Throughput of the fused memory-bound decoder path on one MI355X.

One step = one pass of the whole path over a batch of T synthetic tokens,
the memory-bound half of a decoder layer with FP8 GEMM inputs:

    residual-add RMSNorm -> e4m3fn      (H = 2048, static scale)
    fused QK-RMSNorm + RoPE prologue    ((Q, K) = (16, 2), head_dim 256,
                                         rot_dim 64, 1 + w weight, theta 1e7)
    residual-add RMSNorm -> e4m3fn      (H = 2048)
    gated SiLU -> e4m3fn                (gate_up [T, 2 x 10240])

in bf16 storage with fp32 arithmetic.  T defaults to 128, the widest decode
batch of the 256-wide text-head configuration.  Inputs are resident in HBM
before timing starts.  Each step reads and writes its own slot of a buffer
ring larger than 1 GiB (four times the 256 MB Infinity Cache), so the timed
traffic really comes from HBM; the graph of one pass over the ring is
captured once and replayed.  The FP8 scales come from one calibration pass
on the GPU (amax entry points) over inputs drawn with another seed.

Reported on one JSON line: tokens/s of the step, the roofline of the
dominant kernel (algorithmic bytes / its own average duration, timed with
HIP events over graphs of back-to-back launches), the oracle timed on the
host CPU, plus the prologue's own figures: microseconds per call at T = 1
(warm, graph of 32 calls, the method of the PR the text-head shapes come
from), decode-width sweep and prefill widths T = 256 .. 2048 (cold).

    python bench.py [--steps K] [--warmup W] [--tokens T]
"""
import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QK-norm+RoPE tokens/s & achieved HBM GB/s (% of peak); µs/call at T=1"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
RING_BYTES = int(1.25 * 2 ** 30)
# Ring slots per graph: enough buffer sets to cover RING_BYTES (five times the
# 256 MB Infinity Cache), but at most MAX_SLOTS, so a small call (a decode
# row) does not become a graph of tens of thousands of launches.  At the
# cap a ring still spans MAX_SLOTS distinct buffer sets.
MAX_SLOTS = 4096


def ring_slots(nbytes):
    return max(8, min(MAX_SLOTS, -(-RING_BYTES // max(1, nbytes))))


def phase(name):
    """Progress marker on stderr (the JSON line alone goes to stdout)."""
    print(f"bench: {name}", file=sys.stderr, flush=True)
KERNEL_SOURCES = {
    "qknorm_rope": "qknorm_rope.hip",
    "rmsnorm": "rmsnorm.hip",
    "gated_act": "gated_act.hip",
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--tokens", type=int, default=128)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work for the oracle baseline (0 disables it)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the prologue sweeps")
    ap.add_argument("--only", default=None,
                    help="profiling aid: run one kernel of the step repeatedly "
                         "(norm_fp8 | prologue | act_fp8), or the prefill prologue "
                         "(prologue_prefill), and exit")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="profiling aid: copy this many bytes with torch 20 times and exit")
    return ap.parse_args()


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(p / 100.0 * len(xs)))]


class Step:
    """Device buffers of the decode-layer step, one slot per ring entry."""

    def __init__(self, torch, mbt, W, T):
        self.torch, self.mbt, self.W, self.T = torch, mbt, W, T
        dev = "cuda:0"
        dt = W.BF16
        self.H, self.d = 2048, 10240
        self.pro = W.PrologueCell(name="step_prologue", config=2, cell=4, T=T, Q=16, K=2,
                                  D=256, rot=64, theta=1e7, layout=W.ROTATE_HALF, dtype=dt,
                                  weight_offset=1, w_mean=0.0, w_std=0.05, x_std=2.0)
        self.norm = W.NormCell(name="step_norm_fp8", config=5, cell=20, T=T, H=self.H,
                               dtype=dt, weight_offset=0, w_mean=1.0, w_std=0.05, fp8=True)
        self.act = W.ActCell(name="step_act_fp8", config=5, cell=21, T=T, d=self.d,
                             act=W.SILU, dtype=dt, fp8=True)
        pi, ni, ai = self.pro.inputs(), self.norm.inputs(), self.act.inputs()
        t = lambda bits: W.to_torch(bits, dt, dev)
        # shared: weights, rotary cache, positions
        self.w_q, self.w_k = t(pi["w_q"]), t(pi["w_k"])
        self.cos_sin = torch.from_numpy(pi["cos_sin"]).to(dev)
        self.pos = torch.from_numpy(pi["pos"]).to(dev)
        self.w1, self.w2 = t(ni["w"]), t(ni["w"])
        # calibration pass on the GPU over inputs drawn with another seed
        nc, ac = self.norm.calibration_inputs(), self.act.calibration_inputs()
        amax_n = mbt.fused_add_rmsnorm_amax(t(nc["x"]), t(nc["residual"]), self.w1, 1e-6, 0)
        amax_a = mbt.gated_act_amax(t(ac["gate_up"]), W.SILU)
        self.inv_n = W.fp8_inv_scale(float(amax_n.item()))
        self.inv_a = W.fp8_inv_scale(float(amax_a.item()))
        self.slot_bytes = (self.pro.bytes_algorithmic() + 2 * self.norm.bytes_algorithmic()
                           + self.act.bytes_algorithmic())
        self.R = ring_slots(self.slot_bytes)
        base = dict(x1=t(ni["x"]), r1=t(ni["residual"]), q=t(pi["q"]), k=t(pi["k"]),
                    x2=t(ni["x"]), r2=t(ni["residual"]), gu=t(ai["gate_up"]))
        self.slots = []
        for _ in range(self.R):
            s = {k: v.clone() for k, v in base.items()}
            s["y1"] = torch.empty((T, self.H), dtype=torch.uint8, device=dev)
            s["y2"] = torch.empty((T, self.H), dtype=torch.uint8, device=dev)
            s["qo"] = torch.empty_like(s["q"])
            s["ko"] = torch.empty_like(s["k"])
            s["ao"] = torch.empty((T, self.d), dtype=torch.uint8, device=dev)
            self.slots.append(s)
        torch.cuda.synchronize()

    # the four launches of one step
    def norm1(self, s):
        self.mbt.fused_add_rmsnorm_fp8(s["x1"], s["r1"], self.w1, self.inv_n, 1e-6, 0, y=s["y1"])

    def prologue(self, s):
        p = self.pro
        self.mbt.qknorm_rope(s["q"], s["k"], self.w_q, self.w_k, self.cos_sin, self.pos, p.rot,
                             p.eps, p.weight_offset, p.layout, q_out=s["qo"], k_out=s["ko"])

    def norm2(self, s):
        self.mbt.fused_add_rmsnorm_fp8(s["x2"], s["r2"], self.w2, self.inv_n, 1e-6, 0, y=s["y2"])

    def act_fp8(self, s):
        self.mbt.gated_act_fp8(s["gu"], self.inv_a, self.W.SILU, out=s["ao"])

    def step(self, s):
        self.norm1(s)
        self.prologue(s)
        self.norm2(s)
        self.act_fp8(s)


def capture(torch, fn, n):
    """A graph of fn(0) .. fn(n - 1), captured on a side stream."""
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def timed_replays(torch, graphs):
    """Elapsed ms of replaying `graphs` (a list) back to back, bracketed by
    synchronisations and HIP events on the current stream."""
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for g in graphs:
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def run_steps(torch, st, gfull, grem, n):
    graphs = [gfull] * (n // st.R) + ([grem[n % st.R]] if n % st.R else [])
    return timed_replays(torch, graphs)


def kernel_time_us(torch, fn, R, launches):
    """Average duration of one launch: graphs of R back-to-back launches over
    the ring slots, replayed until `launches` launches are timed."""
    g = capture(torch, fn, R)
    timed_replays(torch, [g])                    # warm the graph itself
    reps = max(1, launches // R)
    ms = timed_replays(torch, [g] * reps)
    return 1000.0 * ms / (reps * R)


def prologue_warm_us(torch, mbt, W, cell, samples=200, inner=32):
    """P2-style: a graph of 32 calls on one buffer set, timed per replay."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    q, k, wq, wk = t(i["q"]), t(i["k"]), t(i["w_q"]), t(i["w_k"])
    cs = torch.from_numpy(i["cos_sin"]).to(dev)
    pos = torch.from_numpy(i["pos"]).to(dev)
    qo, ko = torch.empty_like(q), torch.empty_like(k)

    def call(_):
        mbt.qknorm_rope(q, k, wq, wk, cs, pos, cell.rot, cell.eps, cell.weight_offset,
                        cell.layout, q_out=qo, k_out=ko)

    g = capture(torch, call, inner)
    for _ in range(20):
        g.replay()
    xs = [1000.0 * timed_replays(torch, [g]) / inner for _ in range(samples)]
    # stream mode: direct launches from Python, host dispatch included
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(inner * 8):
        call(0)
    b.record()
    torch.cuda.synchronize()
    stream_us = 1000.0 * a.elapsed_time(b) / (inner * 8)
    return dict(median=median(xs), p25=pct(xs, 25), p75=pct(xs, 75), stream=stream_us)


def prologue_cold_us(torch, mbt, W, cell, launches=2000):
    """Cold: each launch of the graph reads and writes its own ring slot."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    wq, wk = t(i["w_q"]), t(i["w_k"])
    cs = torch.from_numpy(i["cos_sin"]).to(dev)
    pos = torch.from_numpy(i["pos"]).to(dev)
    R = ring_slots(cell.bytes_algorithmic())
    q0, k0 = t(i["q"]), t(i["k"])
    ring = [(q0.clone(), k0.clone(), torch.empty_like(q0), torch.empty_like(k0))
            for _ in range(R)]

    def call(j):
        q, k, qo, ko = ring[j]
        mbt.qknorm_rope(q, k, wq, wk, cs, pos, cell.rot, cell.eps, cell.weight_offset,
                        cell.layout, q_out=qo, k_out=ko)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us


def route_us(torch, mbt, W, cell, cold, passes=7, samples=50, inner=32, launches=6000):
    """The fused prologue against the split route it replaces -- RMSNorm of
    the q head-rows, RMSNorm of the k head-rows (mbt_fused_add_rmsnorm with
    residual NULL), then mbt_rope -- both in place, with a null arm: the
    fused route is timed twice per pass, before and after the split route,
    and a pass whose two fused timings differ by more than 1 % (2 % cold:
    identical cold-ring replays jitter by up to 2 % on MI355X) is dropped.
    Returns medians over the kept passes (None if every pass was dropped).
    Warm: a graph of `inner` calls on one buffer set; cold: graphs over a
    ring of buffer sets larger than the Infinity Cache."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    wq, wk = t(i["w_q"]), t(i["w_k"])
    cs = torch.from_numpy(i["cos_sin"]).to(dev)
    pos = torch.from_numpy(i["pos"]).to(dev)
    R = ring_slots(cell.bytes_algorithmic()) if cold else 1
    q0, k0 = t(i["q"]), t(i["k"])
    ring = [(q0.clone(), k0.clone()) for _ in range(R)]

    def fused(j):
        q, k = ring[j % R]
        mbt.qknorm_rope(q, k, wq, wk, cs, pos, cell.rot, cell.eps, cell.weight_offset,
                        cell.layout, q_out=q, k_out=k)

    def split(j):
        q, k = ring[j % R]
        mbt.fused_add_rmsnorm(q.view(-1, cell.D), None, wq, cell.eps, cell.weight_offset)
        mbt.fused_add_rmsnorm(k.view(-1, cell.D), None, wk, cell.eps, cell.weight_offset)
        mbt.rope(q, k, cs, pos, cell.rot, cell.layout)

    n = R if cold else inner
    g = {"fused": capture(torch, fused, n), "split": capture(torch, split, n)}
    for gg in g.values():
        for _ in range(3):
            gg.replay()
    reps = max(1, launches // n) if cold else 1

    def one(name):
        if cold:
            return 1000.0 * timed_replays(torch, [g[name]] * reps) / (reps * n)
        return median([1000.0 * timed_replays(torch, [g[name]]) / n for _ in range(samples)])

    kept, dropped = [], 0
    for _ in range(passes):
        a = one("fused")
        b = one("split")
        c = one("fused")
        if abs(a - c) > (0.02 if cold else 0.01) * min(a, c):
            dropped += 1
            continue
        kept.append((0.5 * (a + c), b, abs(a - c) / min(a, c)))
    del ring, g
    torch.cuda.empty_cache()
    if not kept:
        return {"T": cell.T, "QK": f"{cell.Q}x{cell.K}", "dropped": dropped}
    fu = median([x[0] for x in kept])
    sp = median([x[1] for x in kept])
    return {"T": cell.T, "QK": f"{cell.Q}x{cell.K}", "fused_us": round(fu, 3),
            "split_us": round(sp, 3), "split_over_fused": round(sp / fu, 3),
            "null_arm_max_diff": round(max(x[2] for x in kept), 4), "dropped": dropped}


def qkv_cache_bytes(cell):
    """Algorithmic bytes of the fused QKV -> q_out + KV-cache op: qkv read,
    q_out and both cache rows written, the cos/sin rows, both weights, the
    positions and the slots."""
    s = 4 if cell.dtype == 0 else 2
    T, Q, K, D = cell.T, cell.Q, cell.K, cell.D
    return 2 * T * (Q + 2 * K) * D * s + 4 * cell.rot * T + 2 * D * s + 16 * T


def extended_cold_us(torch, mbt, W, cell, form, launches=2000):
    """Cold timing of the extended prologue forms over a ring of buffer sets:
    form "once" (mbt_qknorm_rope_ex, single rounding, dense) or "qkv_cache"
    (mbt_qkv_norm_rope_cache, each token to its own cache slot)."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    wq, wk = t(i["w_q"]), t(i["w_k"])
    cs = torch.from_numpy(i["cos_sin"]).to(dev)
    pos = torch.from_numpy(i["pos"]).to(dev)
    T, Q, K, D = cell.T, cell.Q, cell.K, cell.D
    nbytes = cell.bytes_algorithmic() if form == "once" else qkv_cache_bytes(cell)
    R = ring_slots(nbytes)
    q0, k0 = t(i["q"]), t(i["k"])
    if form == "once":
        ring = [(q0.clone(), k0.clone(), torch.empty_like(q0), torch.empty_like(k0))
                for _ in range(R)]

        def call(j):
            q, k, qo, ko = ring[j]
            mbt.qknorm_rope_ex(q, k, wq, wk, cs, pos, cell.rot, cell.eps, cell.weight_offset,
                               cell.layout, q_out=qo, k_out=ko, round_once=True)
    else:
        qkv0 = torch.cat([q0, k0, k0], dim=1).contiguous()      # [T, Q + 2K, D]
        slot = torch.arange(T, dtype=torch.int64, device=dev)
        ring = [(qkv0.clone(), torch.empty_like(q0), torch.empty_like(k0), torch.empty_like(k0))
                for _ in range(R)]

        def call(j):
            qkv, qo, kc, vc = ring[j]
            mbt.qkv_norm_rope_cache(qkv, wq, wk, cs, pos, slot, kc, vc, Q, cell.rot, cell.eps,
                                    cell.weight_offset, cell.layout, q_out=qo)
    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us, nbytes


def norm_fp8_cold_us(torch, mbt, W, cell, inv_scale, launches=2000):
    """Residual RMSNorm -> FP8, cold: each launch uses its own ring slot."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    w = None if i["w"] is None else t(i["w"])
    R = ring_slots(cell.bytes_algorithmic())
    x0, r0 = t(i["x"]), t(i["residual"])
    ring = [(x0.clone(), r0.clone(), torch.empty(x0.shape, dtype=torch.uint8, device=dev))
            for _ in range(R)]

    def call(j):
        x, r, y = ring[j]
        mbt.fused_add_rmsnorm_fp8(x, r, w, inv_scale, cell.eps, cell.weight_offset, y=y)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us


def adarms_fp8_cold_us(torch, mbt, W, cell, launches=2000):
    """Adaptive RMSNorm -> FP8 (gated residual), cold; the scale comes from
    the GPU's own calibration pass over seed data."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: None if b is None else W.to_torch(b, cell.dtype, dev)
    g, sc, sh = t(i["gate"]), t(i["scale"]), t(i["shift"])
    cal = cell.calibration_inputs()
    amax = mbt.adarms_amax(t(cal["x"]), t(cal["residual"]), g, sc, sh, cell.eps)
    inv_scale = W.fp8_inv_scale(float(amax.item()))
    R = ring_slots(cell.bytes_algorithmic())
    x0, r0 = t(i["x"]), t(i["residual"])
    ring = [(x0.clone(), r0.clone(), torch.empty(x0.shape, dtype=torch.uint8, device=dev))
            for _ in range(R)]

    def call(j):
        x, r, y = ring[j]
        mbt.adarms_fp8(x, r, g, sc, sh, inv_scale, cell.eps, y=y)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us


def norm_cold_us(torch, mbt, W, cell, launches=1500):
    """Residual RMSNorm in place (dtype output), cold: each launch uses its
    own ring slot."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    w = t(i["w"])
    R = ring_slots(cell.bytes_algorithmic())
    x0, r0 = t(i["x"]), t(i["residual"])
    ring = [(x0.clone(), r0.clone()) for _ in range(R)]

    def call(j):
        x, r = ring[j]
        mbt.fused_add_rmsnorm(x, r, w, cell.eps, cell.weight_offset)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us


def act_cold_us(torch, mbt, W, cell, inv_scale=1.0, launches=1500):
    """Gated activation, dtype or FP8 output, cold."""
    dev = "cuda:0"
    gu0 = W.to_torch(cell.inputs()["gate_up"], cell.dtype, dev)
    R = ring_slots(cell.bytes_algorithmic())
    odt = torch.uint8 if cell.fp8 else gu0.dtype
    ring = [(gu0.clone(), torch.empty((cell.T, cell.d), dtype=odt, device=dev))
            for _ in range(R)]

    def call(j):
        gu, out = ring[j]
        if cell.fp8:
            mbt.gated_act_fp8(gu, inv_scale, cell.act, out=out)
        else:
            mbt.gated_act(gu, cell.act, out=out)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us


def copy_ceiling_gbps(torch, nbytes, launches=1000):
    """torch's device copy of nbytes/2 -> nbytes/2 (nbytes of traffic), cold."""
    half = max(16, nbytes // 2)
    R = ring_slots(nbytes)
    src = [torch.empty(half, dtype=torch.uint8, device="cuda:0") for _ in range(R)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda:0") for _ in range(R)]
    us = kernel_time_us(torch, lambda j: dst[j].copy_(src[j]), R, launches)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * half / us / 1e3


def prefill_cell(W):
    """The widest prefill cell: (Q, K) = (24, 4), T = 2048, bf16."""
    return max((c for c in W.config3_cells()
                if c.dtype == W.BF16 and c.layout == W.ROTATE_HALF),
               key=lambda c: c.bytes_algorithmic())


def source_digest(kernel):
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "memory_bound_transformer_amd")
    # the compiler flags (build.py) shape the kernel as much as its source;
    # comments and layout do not, so they are left out of the digest
    for path in (os.path.join(pkg, "csrc", KERNEL_SOURCES[kernel]),
                 os.path.join(pkg, "csrc", "mbt_device.hpp"), os.path.join(pkg, "build.py")):
        with open(path) as f:
            h.update(_code_only(f.read(), path.endswith(".py")).encode())
    return h.hexdigest()


def _code_only(text, python):
    """Source text without comments and blank lines, each line stripped."""
    if python:
        text = re.sub(r'(?m)^\s*#.*$', "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.strip() for l in text.splitlines() if l.strip())


def traffic_for(key, kernel):
    """HBM bytes per launch of launch `key` from the committed counter
    summary (profiles/traffic.json), or None once the kernel's source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(W, st, seconds):
    """The oracle, as it stands, on the host: the same step on the same
    inputs, single-threaded, repeated until `seconds` of CPU work."""
    import oracle
    orc = oracle.default()
    pi, ni, ai = st.pro.inputs(), st.norm.inputs(), st.act.inputs()
    p = st.pro
    # the oracle's own calibration pass (nothing here comes from the GPU)
    nc, ac = st.norm.calibration_inputs(), st.act.calibration_inputs()
    inv_n = W.fp8_inv_scale(orc.fused_add_rmsnorm_amax(nc["x"], nc["residual"], ni["w"], 1e-6,
                                                       0, W.BF16))
    inv_a = W.fp8_inv_scale(orc.gated_act_amax(ac["gate_up"], W.SILU, W.BF16))
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.fused_add_rmsnorm_fp8(ni["x"], ni["residual"], ni["w"], inv_n, 1e-6, 0, W.BF16)
        orc.qknorm_rope(pi["q"], pi["k"], pi["w_q"], pi["w_k"], pi["cos_sin"], pi["pos"], p.rot,
                        p.eps, p.weight_offset, p.layout, W.BF16)
        orc.fused_add_rmsnorm_fp8(ni["x"], ni["residual"], ni["w"], inv_n, 1e-6, 0, W.BF16)
        orc.gated_act_fp8(ai["gate_up"], inv_a, W.SILU, W.BF16)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds and n >= 2:
            break
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(n * st.T / el, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full steps of T={st.T} tokens ({el:.1f} s), single thread, "
                      f"host CPU: {model}, {len(os.sched_getaffinity(0))} cores visible"}


def cpu_baseline_threads(W, st, seconds):
    """The same oracle calls, as they stand, from several host threads at
    once, each thread on its own contiguous slice of the step's tokens (the
    token-parallel CPU structure of "thox-edge-ops v2", section 5.3; ctypes
    releases the interpreter lock inside the C oracle)."""
    import concurrent.futures as cf
    import oracle
    orc = oracle.default()
    pi, ni, ai = st.pro.inputs(), st.norm.inputs(), st.act.inputs()
    p = st.pro
    nc, ac = st.norm.calibration_inputs(), st.act.calibration_inputs()
    inv_n = W.fp8_inv_scale(orc.fused_add_rmsnorm_amax(nc["x"], nc["residual"], ni["w"], 1e-6,
                                                       0, W.BF16))
    inv_a = W.fp8_inv_scale(orc.gated_act_amax(ac["gate_up"], W.SILU, W.BF16))
    n_thr = max(1, min(len(os.sched_getaffinity(0)), st.T, 16))
    bounds = [(i * st.T // n_thr, (i + 1) * st.T // n_thr) for i in range(n_thr)]

    def work(b):
        a, e = b
        orc.fused_add_rmsnorm_fp8(ni["x"][a:e], ni["residual"][a:e], ni["w"], inv_n, 1e-6, 0,
                                  W.BF16)
        orc.qknorm_rope(pi["q"][a:e], pi["k"][a:e], pi["w_q"], pi["w_k"], pi["cos_sin"],
                        pi["pos"][a:e], p.rot, p.eps, p.weight_offset, p.layout, W.BF16)
        orc.fused_add_rmsnorm_fp8(ni["x"][a:e], ni["residual"][a:e], ni["w"], inv_n, 1e-6, 0,
                                  W.BF16)
        orc.gated_act_fp8(ai["gate_up"][a:e], inv_a, W.SILU, W.BF16)

    n = 0
    with cf.ThreadPoolExecutor(n_thr) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(work, bounds))
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds and n >= 2:
                break
    lo, hi = st.T // n_thr, -(-st.T // n_thr)
    per = f"{lo}" if lo == hi else f"{lo}-{hi}"
    return {"value": round(n * st.T / el, 1), "unit": "tokens/s", "cores": n_thr,
            "kind": "oracle",
            "sample": f"{n} full steps of T={st.T} tokens ({el:.1f} s wall), {n_thr} threads, "
                      f"each on {per} tokens of every step"}


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every op of this path is independent per "
              "token row, so the multi-GPU layout is token sharding with no exchange; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import memory_bound_transformer_amd as mbt
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe:
        x = torch.empty(args.copy_probe // 2, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(20):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_moved": 2 * (args.copy_probe // 2)}))
        return

    phase("step buffers")
    st = Step(torch, mbt, W, args.tokens)
    kernels = {"norm_fp8": (st.norm1, st.norm.bytes_algorithmic(), "rmsnorm"),
               "prologue": (st.prologue, st.pro.bytes_algorithmic(), "qknorm_rope"),
               "act_fp8": (st.act_fp8, st.act.bytes_algorithmic(), "gated_act")}

    if args.only == "prologue_prefill":
        prologue_cold_us(torch, mbt, W, prefill_cell(W), launches=args.steps)
        print(json.dumps({"only": args.only, "launches": args.steps}))
        return
    if args.only:
        fn = kernels[args.only][0]
        for j in range(max(args.steps, st.R)):
            fn(st.slots[j % st.R])
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "launches": max(args.steps, st.R)}))
        return

    R = st.R
    gfull = capture(torch, lambda j: st.step(st.slots[j]), R)
    grem = {}
    for n in {args.steps % R, args.warmup % R} - {0}:
        grem[n] = capture(torch, lambda j: st.step(st.slots[j]), n)
    run_steps(torch, st, gfull, grem, args.warmup)                    # warmup
    ms = run_steps(torch, st, gfull, grem, args.steps)                # timed
    ms_per_step = ms / args.steps
    tokens_per_s = args.tokens * args.steps / (ms / 1e3)

    # per-kernel average launch durations (same cold ring, graphs of R launches)
    per = {}
    for name, (fn, nbytes, _) in kernels.items():
        us = kernel_time_us(torch, lambda j, fn=fn: fn(st.slots[j]), R, 2000)
        per[name] = dict(us=round(us, 3), bytes=nbytes, GBps=round(nbytes / us / 1e3, 1),
                         frac_peak=round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4))
    # norm_fp8 runs twice per step
    share = {k: v["us"] * (2 if k == "norm_fp8" else 1) for k, v in per.items()}
    dom = max(share, key=share.get)
    dom_fn, dom_bytes, dom_src = kernels[dom]
    achieved = dom_bytes / per[dom]["us"] / 1e3
    phase("roofline")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic_for(f"{dom}_T{args.tokens}", dom_src), "kernel": dom,
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": per[dom]["us"],
                "copy_ceiling_GBps": round(copy_ceiling_gbps(torch, dom_bytes), 1)}

    # the prologue's own figures (the headline metric's parts)
    out_extra = {}
    prologue = {"step_T": args.tokens,
                "tokens_per_s": round(args.tokens / per["prologue"]["us"] * 1e6, 1),
                "GBps": per["prologue"]["GBps"], "frac_peak": per["prologue"]["frac_peak"]}
    if not args.no_sweep:
        t1 = [c for c in W.config2_cells() if c.T == 1][0]
        w1 = prologue_warm_us(torch, mbt, W, t1)
        prologue["us_per_call_T1"] = {k: round(v, 3) for k, v in w1.items()}
        phase("decode sweep")
        sweep = []
        for c in W.config2_cells():
            w = prologue_warm_us(torch, mbt, W, c, samples=50)
            sweep.append({"T": c.T, "warm_us": round(w["median"], 3),
                          "tokens_per_s": round(c.T / w["median"] * 1e6, 1),
                          "logical_GBps_warm": round(c.bytes_logical() / w["median"] / 1e3, 1)})
        prologue["decode_sweep_16x2"] = sweep
        pre = []
        for c in W.config3_cells():
            if c.dtype != W.BF16 or c.layout != W.ROTATE_HALF:
                continue
            us = prologue_cold_us(torch, mbt, W, c)
            gbps = c.bytes_algorithmic() / us / 1e3
            pre.append({"QK": f"{c.Q}x{c.K}", "T": c.T, "cold_us": round(us, 3),
                        "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_HBM_GBPS, 4),
                        "tokens_per_s": round(c.T / us * 1e6, 1)})
        prologue["prefill_cold"] = pre
        phase("prefill, other cells")
        # the rest of configuration 3: fp16, and interleaved pairs with full
        # rotary on head_dim 256
        other = []
        for c in W.config3_cells():
            if c.dtype == W.BF16 and c.layout == W.ROTATE_HALF:
                continue
            if c.T not in (256, 2048):
                continue
            us = prologue_cold_us(torch, mbt, W, c)
            gbps = c.bytes_algorithmic() / us / 1e3
            other.append({"cell": c.name, "QK": f"{c.Q}x{c.K}", "T": c.T,
                          "layout": "interleaved" if c.layout == W.INTERLEAVED else "rotate_half",
                          "rot_dim": c.rot, "dtype": W.DTYPE_NAMES[c.dtype],
                          "cold_us": round(us, 3), "GBps": round(gbps, 1),
                          "frac_peak": round(gbps / PEAK_HBM_GBPS, 4)})
        prologue["prefill_cold_other"] = other
        # the residual norm (configuration 4, bf16 and fp32, both weight
        # conventions folded: delta 0) and the gated activation
        # (configuration 5), as rows/s and GB/s
        phase("norm sweep (configuration 4)")
        nsweep = []
        for c in W.config4_cells():
            if c.weight_offset != 0 or c.dtype == W.F16:
                continue
            us = norm_cold_us(torch, mbt, W, c)
            gbps = c.bytes_algorithmic() / us / 1e3
            nsweep.append({"dtype": W.DTYPE_NAMES[c.dtype], "H": c.H, "T": c.T,
                           "cold_us": round(us, 3), "rows_per_s": round(c.T / us * 1e6, 1),
                           "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_HBM_GBPS, 4)})
        phase("activation sweep (configuration 5)")
        asweep = []
        for c in W.config5_cells():
            if not isinstance(c, W.ActCell):
                continue
            us = act_cold_us(torch, mbt, W, c)
            gbps = c.bytes_algorithmic() / us / 1e3
            asweep.append({"act": "silu" if c.act == W.SILU else "gelu_tanh", "T": c.T,
                           "out": "fp8" if c.fp8 else "bf16", "d": c.d, "cold_us": round(us, 3),
                           "rows_per_s": round(c.T / us * 1e6, 1), "GBps": round(gbps, 1),
                           "frac_peak": round(gbps / PEAK_HBM_GBPS, 4)})
        out_extra = {"norm_sweep_config4": nsweep, "act_sweep_config5": asweep}
        # fused vs split route (norm q rows, norm k rows, rope), in place
        phase("routes")
        routes = {"warm": [route_us(torch, mbt, W, c, cold=False)
                           for c in W.config2_cells() if c.T in (1, 8, 32, 128)],
                  "cold": [route_us(torch, mbt, W, c, cold=True)
                           for c in W.config3_cells()
                           if c.dtype == W.BF16 and c.layout == W.ROTATE_HALF]}
        prologue["routes"] = routes
        # the prefill launch the >= 70 % HBM target is set for
        big = prefill_cell(W)
        us = [x for x in pre if x["QK"] == f"{big.Q}x{big.K}" and x["T"] == big.T][0]["cold_us"]
        gbps = big.bytes_algorithmic() / us / 1e3
        prologue["roofline_prefill"] = {
            "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic_for("prologue_prefill", "qknorm_rope"),
            "kernel": f"prologue {big.Q}x{big.K} T={big.T} bf16", "avg_launch_us": us,
            "algorithmic_bytes_per_launch": big.bytes_algorithmic(),
            "copy_ceiling_GBps": round(copy_ceiling_gbps(torch, big.bytes_algorithmic()), 1)}
        # the extended forms: single rounding, and the fused QKV -> KV-cache op
        ext = []
        for c in (st.pro, big):
            base = [x for x in pre if x["QK"] == f"{c.Q}x{c.K}" and x["T"] == c.T]
            row = {"QK": f"{c.Q}x{c.K}", "T": c.T,
                   "contract_us": base[0]["cold_us"] if base else per["prologue"]["us"]}
            for form in ("once", "qkv_cache"):
                us, nb = extended_cold_us(torch, mbt, W, c, form)
                row[form + "_us"] = round(us, 3)
                row[form + "_GBps"] = round(nb / us / 1e3, 1)
            ext.append(row)
        prologue["extended_forms_cold"] = ext

    # RMSNorm -> FP8 with the weight against the no-weight form (the scale
    # folded into the next GEMM), H = 2048, bf16, cold
    phase("no-weight norm")
    noweight = []
    if not args.no_sweep:
        for T in (args.tokens, 512):
            row = {"T": T, "H": st.H}
            for wt in (True, False):
                c = W.NormCell(name="nw", config=5, cell=60 + T, T=T, H=st.H, dtype=W.BF16,
                               weight_offset=0 if not wt else 1, w_mean=0.0, w_std=0.05,
                               fp8=True, weight=wt)
                us = norm_fp8_cold_us(torch, mbt, W, c, st.inv_n)
                key = "weighted" if wt else "no_weight"
                row[key + "_us"] = round(us, 3)
                row[key + "_GBps"] = round(c.bytes_algorithmic() / us / 1e3, 1)
            noweight.append(row)
    # adaptive RMSNorm -> FP8 with a gated residual (style vector per call):
    # the Pi0.5 decoder's 10-token rows and a 512-token batch, H = 2048
    phase("adaptive norm")
    adarms = []
    if not args.no_sweep:
        for T in (10, 512):
            c = W.AdaCell(name="ada", config=5, cell=70 + T, T=T, H=st.H, dtype=W.BF16, fp8=True)
            us = adarms_fp8_cold_us(torch, mbt, W, c)
            adarms.append({"T": T, "H": st.H, "us": round(us, 3),
                           "GBps": round(c.bytes_algorithmic() / us / 1e3, 1),
                           "frac_peak": round(c.bytes_algorithmic() / us / 1e3 / PEAK_HBM_GBPS, 4)})

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode-layer memory-bound path: residual RMSNorm->fp8, "
                               "QK-RMSNorm+RoPE, residual RMSNorm->fp8, SiLU-gate->fp8",
                   "tokens": args.tokens, "io_dtype": "bf16", "heads_q": 16, "heads_kv": 2,
                   "head_dim": 256, "rot_dim": 64, "hidden": st.H, "intermediate": st.d,
                   "ring_slots": R, "ring_bytes": R * st.slot_bytes, "mode": "cold, hipGraph",
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kernels": per,
        "prologue": prologue,
        "norm_fp8_weight_vs_none": noweight,
        "adarms_fp8_gated": adarms,
        **out_extra,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(W, st, args.cpu_seconds)
        out["cpu_baseline_threads"] = cpu_baseline_threads(W, st, min(args.cpu_seconds, 5.0))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
