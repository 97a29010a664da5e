"""Throughput of the fused QK-RMSNorm + RoPE prologue on one MI355X, with the
sibling memory-bound ops measured beside it.

Headline step: one launch of the prologue over the widest prefill batch of
the 256-wide text-head geometry -- (Q, K) = (24, 4) heads, head_dim 256,
rot_dim 64 (rotate-half), 1 + w weights, theta 1e7, T = 2048 tokens at
positions 0 .. 2047, bf16 storage with fp32 arithmetic.  Inputs are resident
in HBM before timing starts.  Each step reads and writes its own slot of a
buffer ring larger than 1 GiB (five times the 256 MB Infinity Cache), so the
traffic comes from HBM; graphs captured over the ring are replayed.  W
untimed steps, then exactly K timed steps between HIP events, with a device
synchronisation on both sides.  `value` = tokens/s of the K steps; `roofline`
= the algorithmic bytes of one launch over the average launch time of the
same K steps, against 8 TB/s.

Also reported: microseconds per call at T = 1 (warm, a graph of 32 calls,
median of 200 samples: the method of the ninfer PR the text-head shapes come
from); the fraction of peak of every prefill cell (T >= 256), event-timed and
from the committed rocprofv3 kernel trace, each beside the library's
streaming copy of the same bytes (mbt_stream_copy, cold: the attainable
floor for a kernel that moves those bytes); the decode-width sweep; the
decode-layer step (norm -> FP8, prologue, norm -> FP8, SiLU -> FP8 at
T = 128); the residual-norm and activation sweeps; the fused-vs-split route
comparison; the extended prologue forms; the oracle timed on the host CPU.

    python bench.py [--steps K] [--warmup W] [--no-sweep] [--no-cpu] [--sustained]

Profiling aids (each runs committed code only):

    python bench.py --only {prologue_prefill|prefill_cells|norm_fp8|prologue|act_fp8}
    python bench.py --copy-probe BYTES
    python bench.py --trace-stats TRACE.csv OUT.csv       (no GPU)
    python bench.py --write-profiles DIR                  (no GPU)
"""
import argparse
import csv
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QK-norm+RoPE tokens/s & achieved HBM GB/s (% of peak); µs/call at T=1"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
INFINITY_CACHE_BYTES = 256 * 2 ** 20
RING_BYTES = int(1.25 * 2 ** 30)
# A graph is captured over one pass of a ring, so its slot count is the
# graph's node count.  Graphs are kept at or below MAX_SLOTS nodes (see
# ring_slots).
MAX_SLOTS = 4096

KERNEL_SOURCES = {
    "qknorm_rope": "qknorm_rope.hip",
    "rmsnorm": "rmsnorm.hip",
    "gated_act": "gated_act.hip",
}


def ring_slots(nbytes, cache_resident_ok=False):
    """Buffer sets in a ring for a call that moves `nbytes`: enough to cover
    RING_BYTES, so consecutive calls never find their data in the Infinity
    Cache.  A call small enough to need more than MAX_SLOTS sets raises,
    unless the caller accepts a ring of MAX_SLOTS sets and labels its figure
    with ring_mode() (such a ring can stay resident in the cache)."""
    need = max(8, -(-RING_BYTES // max(1, nbytes)))
    if need <= MAX_SLOTS:
        return need
    if not cache_resident_ok:
        raise ValueError(f"a cold ring for {nbytes} B calls needs {need} buffer sets, more "
                         f"than the {MAX_SLOTS} one captured graph may hold")
    return MAX_SLOTS


def ring_mode(nbytes, R):
    """How a ring of R buffer sets of nbytes each meets the Infinity Cache."""
    total = R * nbytes
    if total >= RING_BYTES:
        return "cold"
    return "cache-resident" if total <= INFINITY_CACHE_BYTES else "partly cache-resident"


_T0 = time.monotonic()


def phase(name):
    """Progress marker on stderr (the JSON line alone goes to stdout), with
    the seconds since start."""
    print(f"bench: {name} (+{time.monotonic() - _T0:.1f} s)", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-sweep", action="store_true",
                    help="headline, T = 1 and the prefill fractions only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--sustained", action="store_true",
                    help="also time the headline over twelve back-to-back runs of 2000 steps "
                         "(headline_sustained), after every other GPU figure")
    ap.add_argument("--only", default=None,
                    choices=["prologue_prefill", "prefill_cells", "norm_fp8", "prologue",
                             "act_fp8", "act_prefill", "norm_prefill"],
                    help="profiling aid: launch one thing repeatedly and exit: "
                         "prologue_prefill (the headline launch), prefill_cells (every "
                         "prefill cell in turn), or a kernel of the decode-layer step "
                         "(norm_fp8 | prologue | act_fp8)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="profiling aid: copy this many bytes with torch 20 times and exit")
    ap.add_argument("--trace-stats", nargs=2, metavar=("TRACE_CSV", "OUT_CSV"),
                    help="reduce a rocprofv3 kernel trace to per-launch-size statistics")
    ap.add_argument("--write-profiles", metavar="DIR",
                    help="write the profiles/ summaries from a profiling run's outputs")
    return ap.parse_args()


def median(xs):
    return statistics.median(xs)


def pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(p / 100.0 * len(xs)))]


# ---------------------------------------------------------------------------
# graphs and timing
# ---------------------------------------------------------------------------

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


def kernel_time_us(torch, fn, R, launches):
    """Average duration of one launch: graphs of R back-to-back launches over
    the ring slots, replayed until `launches` launches are timed."""
    g = capture(torch, fn, R)
    timed_replays(torch, [g])                    # warm the graph itself
    reps = max(1, launches // R)
    ms = timed_replays(torch, [g] * reps)
    return 1000.0 * ms / (reps * R)


class Steps:
    """Steps fn(slot) over a ring of R slots, each run continuing where the
    last one stopped, so a slot is reused only after the other R - 1 (a
    warm-up never leaves the first timed slots in the Infinity Cache).
    Graphs (one full pass from a start slot, or a shorter run) are captured
    by prepare(), or on first use, always before the timed region."""

    def __init__(self, torch, fn, R):
        self.torch, self.fn, self.R = torch, fn, R
        self.pos = 0
        self.graphs = {}

    def _graph(self, start, n):
        if (start, n) not in self.graphs:
            self.graphs[(start, n)] = capture(self.torch, lambda j: self.fn(start + j), n)
        return self.graphs[(start, n)]

    def run(self, n):
        start = self.pos % self.R
        graphs = [self._graph(start, self.R)] * (n // self.R)
        if n % self.R:
            graphs.append(self._graph(start, n % self.R))
        self.pos += n
        return timed_replays(self.torch, graphs)

    def prepare(self, runs):
        """Capture every graph of a planned sequence of run lengths, replay
        each once, then replay one whole pass over the ring from the current
        slot, all untimed.  A short timed run right after a capture or an
        allocation was slower per step (a fresh 20-step graph of the
        headline: 10.8 - 11.0 us against 10.2 on its later replays) while a
        run over slots the GPU had just streamed through was not; the whole
        pass comes last, after every allocation, and touches every slot.  It
        ends on the slots just before the current one, so the warm-up and the
        timed steps that follow still start on slots the Infinity Cache no
        longer holds."""
        pos = self.pos
        order = []
        for n in runs:
            start = pos % self.R
            if n // self.R:
                order.append(self._graph(start, self.R))
            if n % self.R:
                order.append(self._graph(start, n % self.R))
            pos += n
        whole = self._graph(self.pos % self.R, self.R)
        for g in order:
            g.replay()
        whole.replay()
        self.torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# the headline step and the decode-layer step
# ---------------------------------------------------------------------------

def prefill_cell(W):
    """The widest prefill cell: (Q, K) = (24, 4), T = 2048, bf16, rotate-half."""
    return max((c for c in W.config3_cells()
                if c.dtype == W.BF16 and c.layout == W.ROTATE_HALF),
               key=lambda c: c.bytes_algorithmic())


class Headline:
    """Device buffers of the headline step: the prologue over the widest
    prefill cell, out of place, one ring slot per step."""

    def __init__(self, torch, mbt, W):
        self.mbt = mbt
        self.cell = c = prefill_cell(W)
        i = c.inputs()
        t = lambda bits: W.to_torch(bits, c.dtype, "cuda:0")
        self.wq, self.wk = t(i["w_q"]), t(i["w_k"])
        self.cs = torch.from_numpy(i["cos_sin"]).to("cuda:0")
        self.pos = torch.from_numpy(i["pos"]).to("cuda:0")
        self.bytes = c.bytes_algorithmic()
        self.R = ring_slots(self.bytes)
        q0, k0 = t(i["q"]), t(i["k"])
        self.ring = [(q0.clone(), k0.clone(), torch.empty_like(q0), torch.empty_like(k0))
                     for _ in range(self.R)]
        torch.cuda.synchronize()

    def step(self, j):
        c = self.cell
        q, k, qo, ko = self.ring[j % self.R]
        self.mbt.qknorm_rope(q, k, self.wq, self.wk, self.cs, self.pos, c.rot, c.eps,
                             c.weight_offset, c.layout, q_out=qo, k_out=ko)


class DecodeStep:
    """Device buffers of the decode-layer step (the memory-bound half of a
    decoder layer with FP8 GEMM inputs) at T tokens: residual RMSNorm -> FP8
    (H = 2048), the prologue at (16, 2), residual RMSNorm -> FP8, SiLU-gate
    -> FP8 (d = 10240); one ring slot per step.  The FP8 scales come from one
    calibration pass on the GPU over inputs drawn with another seed."""

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
        self.w_q, self.w_k = t(pi["w_q"]), t(pi["w_k"])
        self.cos_sin = torch.from_numpy(pi["cos_sin"]).to(dev)
        self.pos = torch.from_numpy(pi["pos"]).to(dev)
        self.w1, self.w2 = t(ni["w"]), t(ni["w"])
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

    def step(self, j):
        s = self.slots[j % self.R]
        self.norm1(s)
        self.prologue(s)
        self.norm2(s)
        self.act_fp8(s)

    def kernels(self):
        return {"norm_fp8": (self.norm1, self.norm.bytes_algorithmic(), "rmsnorm"),
                "prologue": (self.prologue, self.pro.bytes_algorithmic(), "qknorm_rope"),
                "act_fp8": (self.act_fp8, self.act.bytes_algorithmic(), "gated_act")}


def decode_layer_step(torch, mbt, W, T=128, steps=2000):
    """The decode-layer step at T tokens: tokens/s over `steps` cold steps and
    each kernel's own average launch time."""
    st = DecodeStep(torch, mbt, W, T)
    run = Steps(torch, st.step, st.R)
    run.prepare([200, steps])
    run.run(200)
    ms = run.run(steps)
    per = {}
    for name, (fn, nbytes, _) in st.kernels().items():
        us = kernel_time_us(torch, lambda j, fn=fn: fn(st.slots[j]), st.R, 2000)
        per[name] = dict(us=round(us, 3), bytes=nbytes, GBps=round(nbytes / us / 1e3, 1),
                         frac_peak=round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4),
                         traffic=traffic_for(f"{name}_T{T}", st.kernels()[name][2]))
    out = {"workload": "residual RMSNorm->fp8 (H 2048), QK-RMSNorm+RoPE (16,2) D256 rot64, "
                       "residual RMSNorm->fp8, SiLU-gate->fp8 (d 10240), bf16",
           "tokens": T, "steps": steps, "ms_per_step": round(ms / steps, 6),
           "tokens_per_s": round(T * steps / (ms / 1e3), 1), "ring_slots": st.R,
           "ring": ring_mode(st.slot_bytes, st.R), "kernels": per}
    del st
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# per-cell measurements
# ---------------------------------------------------------------------------

def prologue_warm_us(torch, mbt, W, cell, samples=200, inner=32):
    """The ninfer PR's method: a graph of 32 calls on one buffer set, 20
    warm-up replays, then `samples` replays each timed on its own."""
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
    """Residual RMSNorm -> FP8 over a ring of buffer sets.  Returns (us, ring mode)."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    w = None if i["w"] is None else t(i["w"])
    R = ring_slots(cell.bytes_algorithmic(), cache_resident_ok=True)
    x0, r0 = t(i["x"]), t(i["residual"])
    ring = [(x0.clone(), r0.clone(), torch.empty(x0.shape, dtype=torch.uint8, device=dev))
            for _ in range(R)]

    def call(j):
        x, r, y = ring[j]
        mbt.fused_add_rmsnorm_fp8(x, r, w, inv_scale, cell.eps, cell.weight_offset, y=y)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us, ring_mode(cell.bytes_algorithmic(), R)


def adarms_fp8_cold_us(torch, mbt, W, cell, launches=2000):
    """Adaptive RMSNorm -> FP8 (gated residual) over a ring of buffer sets;
    the scale comes from the GPU's own calibration pass over seed data.
    Returns (us, ring mode)."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: None if b is None else W.to_torch(b, cell.dtype, dev)
    g, sc, sh = t(i["gate"]), t(i["scale"]), t(i["shift"])
    cal = cell.calibration_inputs()
    amax = mbt.adarms_amax(t(cal["x"]), t(cal["residual"]), g, sc, sh, cell.eps)
    inv_scale = W.fp8_inv_scale(float(amax.item()))
    R = ring_slots(cell.bytes_algorithmic(), cache_resident_ok=True)
    x0, r0 = t(i["x"]), t(i["residual"])
    ring = [(x0.clone(), r0.clone(), torch.empty(x0.shape, dtype=torch.uint8, device=dev))
            for _ in range(R)]

    def call(j):
        x, r, y = ring[j]
        mbt.adarms_fp8(x, r, g, sc, sh, inv_scale, cell.eps, y=y)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us, ring_mode(cell.bytes_algorithmic(), R)


def norm_cold_us(torch, mbt, W, cell, launches=1500):
    """Residual RMSNorm in place (dtype output) over a ring of buffer sets.
    Returns (us, ring mode)."""
    dev = "cuda:0"
    i = cell.inputs()
    t = lambda b: W.to_torch(b, cell.dtype, dev)
    w = t(i["w"])
    R = ring_slots(cell.bytes_algorithmic(), cache_resident_ok=True)
    x0, r0 = t(i["x"]), t(i["residual"])
    ring = [(x0.clone(), r0.clone()) for _ in range(R)]

    def call(j):
        x, r = ring[j]
        mbt.fused_add_rmsnorm(x, r, w, cell.eps, cell.weight_offset)

    us = kernel_time_us(torch, call, R, launches)
    del ring
    torch.cuda.empty_cache()
    return us, ring_mode(cell.bytes_algorithmic(), R)


def act_cold_us(torch, mbt, W, cell, inv_scale=1.0, launches=1500):
    """Gated activation, dtype or FP8 output, over a ring of buffer sets.
    Returns (us, ring mode)."""
    dev = "cuda:0"
    gu0 = W.to_torch(cell.inputs()["gate_up"], cell.dtype, dev)
    R = ring_slots(cell.bytes_algorithmic(), cache_resident_ok=True)
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
    return us, ring_mode(cell.bytes_algorithmic(), R)


# the streaming copy's forms: (16-byte chunks per lane, block barrier between
# a block's loads and its stores), labelled "C" or "C+sync"
COPY_FORMS = [(c, s) for s in (False, True) for c in (1, 2, 4, 8)]


def copy_form_label(form):
    c, s = form
    return f"{c}+sync" if s else str(c)


def stream_copy_us(torch, mbt, nbytes, launches=1000, forms=COPY_FORMS):
    """Cold µs per launch of the library's streaming copy moving nbytes
    (nbytes/2 read, nbytes/2 written) in each of its forms."""
    half = max(16, nbytes // 2 // 16 * 16)
    # callers ask only for byte counts whose own ring is cold; rounding down
    # to 16 bytes may add a slot, which must not turn into a refusal
    R = ring_slots(2 * half, cache_resident_ok=True)
    src = [torch.empty(half, dtype=torch.uint8, device="cuda:0") for _ in range(R)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda:0") for _ in range(R)]
    out = {}
    for c, sy in forms:
        out[copy_form_label((c, sy))] = kernel_time_us(
            torch, lambda j, c=c, sy=sy: mbt.stream_copy(src[j], dst[j], c, block_sync=sy), R,
            launches)
    del src, dst
    torch.cuda.empty_cache()
    return out


def copy_warm_us(torch, mbt, nbytes, samples=200, inner=32):
    """The streaming copy of nbytes (nbytes/2 read, nbytes/2 written) by the
    T = 1 method: a graph of 32 calls on one buffer set, 20 warm-up replays,
    the median of `samples` replays.  The floor for a decode-width call that
    moves those bytes."""
    half = max(16, nbytes // 2 // 16 * 16)
    src = torch.empty(half, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(half, dtype=torch.uint8, device="cuda:0")
    g = capture(torch, lambda _: mbt.stream_copy(src, dst, 1), inner)
    for _ in range(20):
        g.replay()
    xs = [1000.0 * timed_replays(torch, [g]) / inner for _ in range(samples)]
    return median(xs)


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


# ---------------------------------------------------------------------------
# committed profile summaries (profiles/), tied to the kernel sources
# ---------------------------------------------------------------------------

def source_digest(kernel):
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "memory_bound_transformer_amd")
    # the compiler flags (build.py) shape the kernel as much as its source;
    # comments and layout do not, so they are left out of the digest
    for path in (os.path.join(pkg, "csrc", KERNEL_SOURCES[kernel]),
                 os.path.join(pkg, "csrc", "mbt_device.hpp"),
                 os.path.join(pkg, "csrc", "mbt_launch.hpp"), os.path.join(pkg, "build.py")):
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


def _profile_record(name, key, kernel):
    """Entry `key` of profiles/<name>, or None once the kernel's source has
    changed since it was taken."""
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec


def traffic_for(key, kernel):
    """HBM bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a
    plain copy's reading) from profiles/traffic.json."""
    rec = _profile_record("traffic.json", key, kernel)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def rocprof_us_for(cell_name):
    """rocprofv3 kernel-trace average and median duration of a prefill
    cell's launch, from profiles/prologue_prefill_cells.json."""
    rec = _profile_record("prologue_prefill_cells.json", cell_name, "qknorm_rope")
    return (None, None) if rec is None else (rec["average_us"], rec["median_us"])


def headline_rocprof_us():
    """rocprofv3 kernel-trace average and median duration of the headline
    launch in the default bench run (the command bench.py is), from
    profiles/bench_default_kernel_trace.json."""
    rec = _profile_record("bench_default_kernel_trace.json", "headline", "qknorm_rope")
    return (None, None) if rec is None else (rec["average_us"], rec["median_us"])


def _short(name):
    return name.replace("void mbt::(anonymous namespace)::", "").split("(")[0]


def trace_stats(src, dst):
    """Reduce a rocprofv3 kernel-trace CSV (tens of MB) to one row per
    kernel and launch size, plus the time-ordered runs of prologue launches
    (needed to tell the prefill cells apart)."""
    groups, runs = {}, []
    with open(src) as f:
        r = csv.DictReader(f)
        gcol = [c for c in r.fieldnames if c.startswith("Grid_Size")]
        rows = sorted(r, key=lambda row: int(row["Start_Timestamp"]))
    for row in rows:
        name = _short(row["Kernel_Name"])
        grid = "x".join(row[c] for c in gcol)
        d = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
        groups.setdefault((name, grid), []).append(d)
        if name.startswith("qknorm_rope"):
            if runs and runs[-1][0] == (name, grid):
                runs[-1][1].append(d)
            else:
                runs.append(((name, grid), [d]))
    with open(dst, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Name", "Grid", "Calls", "AverageNs", "MedianNs", "MinNs", "MaxNs"])
        for (n, g), d in sorted(groups.items(), key=lambda kv: -len(kv[1])):
            w.writerow(["group", n, g, len(d), sum(d) / len(d), statistics.median(d), min(d),
                        max(d)])
        for (n, g), d in runs:
            w.writerow(["run", n, g, len(d), sum(d) / len(d), statistics.median(d), min(d),
                        max(d)])


def _read_stats(path):
    with open(path) as f:
        rows = list(csv.DictReader(f))
    us = lambda r, k: float(r[k]) / 1000.0
    groups = {(r["Name"], r["Grid"]): r for r in rows if r["Kind"] == "group"}
    runs = [r for r in rows if r["Kind"] == "run"]
    return groups, runs, us


def write_profiles(d):
    """Write profiles/ from one profiling run's outputs in directory d:
      bench.json            python bench.py (unprofiled)
      default_stats.csv     --trace-stats of rocprofv3 --kernel-trace over
                            python bench.py --no-cpu (the same command)
      cells_stats.csv       --trace-stats of rocprofv3 --kernel-trace over
                            python bench.py --only prefill_cells
      cells.json            that run's stdout (the cells in launch order)
      pmc_<launch>_<counter>/pmc_counter_collection.csv
                            rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs"""
    import workloads as W
    P = os.path.join(ROOT, "profiles")
    repo = "$REPO"
    bj = json.loads(open(os.path.join(d, "bench.json")).read().strip().splitlines()[-1])
    cells_run = json.loads(open(os.path.join(d, "cells.json")).read().strip().splitlines()[-1])
    groups_c, runs_c, us = _read_stats(os.path.join(d, "cells_stats.csv"))
    names = cells_run["cells"]
    kept = [r for r in runs_c if int(r["Calls"]) >= 100]
    assert len(kept) == len(names), (len(kept), len(names))
    cells = {c.name: c for c in W.config3_cells()}
    digest = source_digest("qknorm_rope")
    cmd_cells = ("rocprofv3 --kernel-trace --output-format csv -d <out> -o cells -- "
                 f"python -u {repo}/bench.py --only prefill_cells")
    per_cell = {"_command": cmd_cells}
    lines = []
    event = {x["cell"]: x for x in bj["prefill"]}
    for name, r in zip(names, kept):
        c = cells[name]
        avg, med = us(r, "AverageNs"), us(r, "MedianNs")
        per_cell[name] = {"source_sha256": digest, "kernel": r["Name"],
                          "grid_work_items": r["Grid"], "launches": int(r["Calls"]),
                          "average_us": round(avg, 3), "median_us": round(med, 3),
                          "algorithmic_bytes": c.bytes_algorithmic()}
        ev = event.get(name, {}).get("event_us")
        gb = c.bytes_algorithmic() / avg / 1e3
        lines.append(f"| {name} | `{r['Name']}` | {r['Grid'].split('x')[0]} | {r['Calls']} | "
                     f"{avg:.3f} | {med:.3f} | {ev if ev is not None else '-'} | "
                     f"{gb:.0f} | {gb / PEAK_HBM_GBPS:.3f} |")
    with open(os.path.join(P, "prologue_prefill_cells.json"), "w") as f:
        json.dump(per_cell, f, indent=1)
    md = ["# Prologue launch durations per prefill cell: rocprofv3 --kernel-trace (MI355X, gfx950)",
          "", "Command (from /tmp with TMPDIR=/tmp; `$REPO` is the repository root):", "",
          "```", cmd_cells, f"python {repo}/bench.py --trace-stats <out>/cells_kernel_trace.csv "
          "cells_stats.csv", "```", "",
          "`--only prefill_cells` launches every configuration-3 cell in turn (T = 256 .. 2048,",
          "(24, 4) and (16, 2), bf16 / fp16 rotate-half with rot_dim 64, bf16 interleaved with full",
          "rotary), each over its own cold buffer ring (> 1 GiB).  Each cell's launches form one run",
          "of identical (kernel, grid) dispatches in the trace, matched to the cells in launch order.",
          "GB/s = algorithmic bytes / rocprofv3 average; fraction of 8 TB/s.  The event column is",
          "the unprofiled bench.py run's HIP-event average per launch (graphs over the same ring).",
          "Launches of a few microseconds read up to about 1.5 us longer under the tracer than in "
          "the unprofiled run, and vary more between runs; the streaming copy, which does no "
          "arithmetic, does the same (bench_default_kernel_trace.md, last section), so the event "
          "column is the figure for those cells.", "",
          "| cell | kernel | grid (work-items) | launches | average us | median us | "
          "bench.py events us | GB/s | of peak |",
          "|---|---|---|---|---|---|---|---|---|", *lines, "",
          "Kernel instantiation: `qknorm_rope_vec<dtype, lanes/row, chunks/lane, layout, general, "
          "load order>` (dtype 2 = bf16, 1 = fp16; layout 0 = rotate-half, 1 = interleaved).",
          "`profiles/prologue_prefill_cells.json` holds the same figures with a SHA-256 of the",
          "kernel source; bench.py reports them only while that digest matches."]
    with open(os.path.join(P, "prologue_prefill_cells_kernel_trace.md"), "w") as f:
        f.write("\n".join(md) + "\n")

    # the same command as the headline: the whole default run under the profiler
    groups_d, _, _ = _read_stats(os.path.join(d, "default_stats.csv"))
    head = per_cell[bj["config"]["cell"]]
    hk = groups_d[(head["kernel"], head["grid_work_items"])]
    cmd_d = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o bench -- "
             f"python -u {repo}/bench.py --no-cpu")
    top = sorted(groups_d.values(), key=lambda r: -int(r["Calls"]) * float(r["AverageNs"]))[:30]
    tl = [f"| `{r['Name']}` | {r['Grid'].split('x')[0]} | {r['Calls']} | "
          f"{us(r, 'AverageNs'):.3f} | {us(r, 'MedianNs'):.3f} |" for r in top]
    ev_us = bj["roofline"]["avg_launch_us"]
    av = us(hk, "AverageNs")
    md = ["# Kernel durations of the default bench run: rocprofv3 --kernel-trace --stats "
          "(MI355X, gfx950)", "",
          "Command (from /tmp with TMPDIR=/tmp; `$REPO` is the repository root):", "",
          "```", cmd_d, f"python {repo}/bench.py --trace-stats <out>/bench_kernel_trace.csv "
          "default_stats.csv", "```", "",
          "`--no-cpu` drops only the host-CPU oracle leg, which launches nothing on the GPU.", "",
          "## The headline launch", "",
          f"Cell `{bj['config']['cell']}`: `{head['kernel']}`, grid {head['grid_work_items']} "
          "work-items.", "",
          "| figure | us per launch |", "|---|---|",
          f"| rocprofv3 average over every launch of it in the run ({hk['Calls']} launches) | "
          f"{av:.3f} |",
          f"| rocprofv3 median | {us(hk, 'MedianNs'):.3f} |",
          f"| bench.py HIP events over the timed steps (unprofiled run, "
          f"{bj['steps']} steps) | {ev_us} |",
          f"| difference (rocprofv3 average / events - 1) | {100 * (av / ev_us - 1):+.1f} % |", "",
          f"Algorithmic bytes per launch {bj['roofline']['algorithmic_bytes_per_launch']}: "
          f"{bj['roofline']['algorithmic_bytes_per_launch'] / av / 1e3:.0f} GB/s by the rocprofv3 "
          f"average, {bj['roofline']['achieved']} GB/s by the events.", "",
          "## Launches with the most total time in the run", "",
          "| kernel | grid (work-items) | launches | average us | median us |",
          "|---|---|---|---|---|", *tl]
    # the copy ceilings: every launch shape of the streaming copy in the run
    cp = sorted((r for r in groups_d.values() if "stream_copy" in r["Name"]),
                key=lambda r: (int(r["Grid"].split("x")[0]), r["Name"]))
    if cp:
        # the unprofiled run's event time of each copy launch shape: a copy of
        # b bytes (b/2 read, b/2 written) at C chunks per lane has a grid of
        # ceil(b/2 / 16 / (256 C)) blocks of 256 work-items
        ev = {}
        for b, forms in bj.get("copy_ceilings_us", {}).items():
            half = int(b) // 2 // 16 * 16
            for k, v in forms.items():
                c, sync = int(k.split("+")[0]), k.endswith("+sync")
                g = -(-half // 16 // (256 * c)) * 256
                ev[(f"stream_copy<{c}, {'true' if sync else 'false'}>", str(g))] = (int(b), v)
        rows_cp = []
        for r in cp:
            b, e = ev.get((r["Name"], r["Grid"].split("x")[0]), (None, None))
            rows_cp.append(f"| `{r['Name']}` | {r['Grid'].split('x')[0]} | "
                           f"{'' if b is None else b} | {r['Calls']} | "
                           f"{us(r, 'AverageNs'):.3f} | {us(r, 'MedianNs'):.3f} | "
                           f"{'' if e is None else e} |")
        md += ["", "## The streaming copy (copy ceilings of the prefill cells)", "",
               "`stream_copy<C, sync>`: C 16-byte chunks per lane, with or without a block "
               "barrier between a block's loads and its stores; one launch copies half a cell's "
               "bytes into the other half.  The last column is the unprofiled run's HIP-event "
               "average for the same launch shape.  The copy does no arithmetic, so where the "
               "traced average exceeds the event time (launches of a few microseconds), the "
               "difference is the tracer's, and the prologue's short launches read long under "
               "it by about as much.", "",
               "| kernel | grid (work-items) | bytes moved | launches | average us | median us "
               "| bench.py events us |",
               "|---|---|---|---|---|---|---|", *rows_cp]
    # the gated activation and the residual norm: every launch shape of them
    # in the run (the configuration 4 and 5 sweeps, the decode-layer step,
    # the split route's norms, the no-weight and adaptive norms)
    for fam, title in (("gated_", "The gated activation"), ("rmsnorm_", "The residual norm")):
        rs = sorted((r for r in groups_d.values() if fam in r["Name"]),
                    key=lambda r: (r["Name"], int(r["Grid"].split("x")[0])))
        if rs:
            md += ["", f"## {title}: every launch shape in the run", "",
                   "| kernel | grid (work-items) | launches | average us | median us |",
                   "|---|---|---|---|---|",
                   *[f"| `{r['Name']}` | {r['Grid'].split('x')[0]} | {r['Calls']} | "
                     f"{us(r, 'AverageNs'):.3f} | {us(r, 'MedianNs'):.3f} |" for r in rs]]
    with open(os.path.join(P, "bench_default_kernel_trace.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(os.path.join(P, "bench_default_kernel_trace.json"), "w") as f:
        json.dump({"headline": {"source_sha256": digest, "cell": bj["config"]["cell"],
                                "kernel": head["kernel"],
                                "grid_work_items": head["grid_work_items"],
                                "launches": int(hk["Calls"]), "average_us": round(av, 3),
                                "median_us": round(us(hk, "MedianNs"), 3),
                                "events_us_unprofiled_run": ev_us, "command": cmd_d}},
                  f, indent=1)
        f.write("\n")

    # HBM traffic from the counter runs, scaled by a plain copy's reading
    def pmc(tag, ctr):
        path = os.path.join(d, f"pmc_{tag}_{ctr}", "pmc_counter_collection.csv")
        with open(path) as f:
            rows = list(csv.DictReader(f))
        v = [float(r["Counter_Value"]) for r in rows
             if ("mbt::" in r["Kernel_Name"]) or (tag == "copy" and "copyBuffer" in r["Kernel_Name"])]
        return statistics.median(v), len(v)
    copy_f, _ = pmc("copy", "FETCH_SIZE")
    copy_w, _ = pmc("copy", "WRITE_SIZE")
    half_kib = 67108864 // 2 / 1024
    ff, wf = half_kib / copy_f, half_kib / copy_w
    cmd_p = ("rocprofv3 --pmc {ctr} --output-format csv -d <out> -o pmc -- "
             f"python -u {repo}/bench.py --only {{only}}")
    traffic = {"_calibration": {"copy_bytes_read": 33554432, "copy_bytes_written": 33554432,
                                "FETCH_SIZE_KiB": copy_f, "WRITE_SIZE_KiB": copy_w,
                                "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
                                "command": cmd_p.replace("--only {only}", "--copy-probe 67108864")
                                .format(ctr="{FETCH_SIZE|WRITE_SIZE}")}}
    step = bj.get("decode_layer_step", {}).get("kernels", {})
    launches = {"prologue_prefill": ("prologue_prefill", "qknorm_rope",
                                     bj["roofline"]["algorithmic_bytes_per_launch"])}
    for k, src in (("norm_fp8", "rmsnorm"), ("prologue", "qknorm_rope"), ("act_fp8", "gated_act")):
        if k in step and os.path.exists(os.path.join(d, f"pmc_{k}_FETCH_SIZE")):
            launches[f"{k}_T128"] = (k, src, step[k]["bytes"])
    for k, src in (("act_prefill", "gated_act"), ("norm_prefill", "rmsnorm")):
        if os.path.exists(os.path.join(d, f"pmc_{k}_FETCH_SIZE")):
            launches[k] = (k, src, prefill_traffic_cell(W, k).bytes_algorithmic())
    tl = []
    for key, (only, src, algo) in launches.items():
        f_, n = pmc(only, "FETCH_SIZE")
        w_, _ = pmc(only, "WRITE_SIZE")
        hbm = f_ * 1024 * ff + w_ * 1024 * wf
        traffic[key] = {"source_sha256": source_digest(src), "FETCH_SIZE_KiB": f_,
                        "WRITE_SIZE_KiB": w_, "hbm_bytes_per_launch": round(hbm),
                        "algorithmic_bytes_per_launch": algo,
                        "traffic_over_algorithmic": round(hbm / algo, 4), "dispatches": n,
                        "command": cmd_p.format(ctr="{FETCH_SIZE|WRITE_SIZE}", only=only)}
        tl.append(f"| {key} | {f_:.3f} | {w_:.3f} | {hbm / 1e6:.3f} | {algo / 1e6:.3f} | "
                  f"{hbm / algo:.3f} |")
    with open(os.path.join(P, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    md = ["# HBM traffic per launch from rocprofv3 counters (MI355X, gfx950)", "",
          "Counters are taken one per run (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`), each over",
          "launches that stream through a buffer ring larger than 1 GiB (so every launch misses the",
          "256 MB Infinity Cache); the median per-dispatch value is used.", "",
          "Calibration: a plain device copy of 32 MiB -> 32 MiB (torch `copy_`, HIP's",
          f"`__amd_rocclr_copyBuffer`) reads FETCH_SIZE = {copy_f:.1f} KiB and WRITE_SIZE = "
          f"{copy_w:.1f} KiB per dispatch against 32768 KiB each, so FETCH_SIZE is scaled by "
          f"{ff:.4f} and WRITE_SIZE by {wf:.4f}.", "",
          "| launch | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB (scaled) | algorithmic MB | ratio |",
          "|---|---|---|---|---|---|", *tl, "",
          "`prologue_prefill` is the headline launch: the prologue at (Q, K) = (24, 4), head_dim 256,",
          "rot_dim 64, T = 2048, bf16.  `*_T128` are the kernels of the decode-layer step at T = 128.",
          "`act_prefill` is configuration 5's SiLU-gate -> FP8 at d = 10240, T = 512; `norm_prefill`",
          "configuration 4's bf16 residual norm in place at H = 2560, T = 512.",
          "", "Commands (from /tmp with TMPDIR=/tmp; `$REPO` is the repository root):", "", "```",
          *[cmd_p.format(ctr=c, only=o) for o in [v[0] for v in launches.values()]
            for c in ("FETCH_SIZE", "WRITE_SIZE")],
          *[cmd_p.replace("--only {only}", "--copy-probe 67108864").format(ctr=c)
            for c in ("FETCH_SIZE", "WRITE_SIZE")], "```", "",
          "`profiles/traffic.json` holds the same figures with a SHA-256 of each kernel's source;",
          "bench.py reports `traffic` only while that digest still matches."]
    with open(os.path.join(P, "hbm_traffic_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")


# ---------------------------------------------------------------------------
# the oracle on the host CPU (a reported baseline, not the target)
# ---------------------------------------------------------------------------

def _cpu_model():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return model


def cpu_baseline(W, cell, threads=1, tokens_per_call=32):
    """The oracle, as it stands, on the headline cell's inputs, following the
    measurement protocol of "thox-edge-ops v2" (section 7.1): 20 warm-up
    calls, then 30 trials of up to 50 calls each, as many as make a trial
    last about 0.2 s; median and quartiles of tokens/s over the trials.

    threads = 1: one call is the prologue on `tokens_per_call` tokens, on
    one thread pinned to one core (restored afterwards).  threads = n: one
    call runs n host threads at once, each on its own `tokens_per_call`
    tokens (the token-parallel CPU structure of its section 5.3; ctypes
    releases the interpreter lock inside the oracle)."""
    import concurrent.futures as cf
    import oracle
    orc = oracle.default()
    i = cell.inputs()
    n = tokens_per_call
    slices = [(a * n, (a + 1) * n) for a in range(threads)]

    def work(b):
        a, e = b
        orc.qknorm_rope(i["q"][a:e], i["k"][a:e], i["w_q"], i["w_k"], i["cos_sin"],
                        i["pos"][a:e], cell.rot, cell.eps, cell.weight_offset, cell.layout,
                        cell.dtype)

    old = os.sched_getaffinity(0)
    ex = None
    try:
        if threads == 1:
            os.sched_setaffinity(0, {min(old)})
            call = lambda: work(slices[0])
        else:
            ex = cf.ThreadPoolExecutor(threads)
            call = lambda: list(ex.map(work, slices))
        for _ in range(20):
            call()
        t0 = time.perf_counter()
        call()
        per_call = time.perf_counter() - t0
        m = max(1, min(50, int(round(0.2 / max(per_call, 1e-9)))))
        rates = []
        for _ in range(30):
            t0 = time.perf_counter()
            for _ in range(m):
                call()
            rates.append(m * n * threads / (time.perf_counter() - t0))
    finally:
        if ex is not None:
            ex.shutdown()
        os.sched_setaffinity(0, old)
    where = ("one thread pinned to one core" if threads == 1
             else f"{threads} threads, each on its own {n} tokens")
    return {"value": round(median(rates), 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "p25": round(pct(rates, 25), 1), "p75": round(pct(rates, 75), 1),
            "sample": f"the prologue on {n * threads} of the headline cell's {cell.T} tokens per "
                      f"call ({cell.Q}x{cell.K} heads, head_dim {cell.D}), {where}; 20 warm-up "
                      f"calls, 30 trials of {m} calls, median",
            "cpu_model": _cpu_model(), "cores_visible": len(old)}


# ---------------------------------------------------------------------------

def prefill_traffic_cell(W, what):
    """The bandwidth-bound cells whose HBM traffic the counter runs record
    beside the headline's: configuration 5's SiLU-gate -> FP8 at T = 512 and
    configuration 4's bf16 residual norm at H = 2560, T = 512."""
    if what == "act_prefill":
        return [c for c in W.config5_cells() if isinstance(c, W.ActCell) and c.T == 512
                and c.act == W.SILU and c.fp8][0]
    return [c for c in W.config4_cells() if c.dtype == W.BF16 and c.H == 2560 and c.T == 512
            and c.weight_offset == 0][0]


def only_mode(torch, mbt, W, what, steps):
    """Profiling aids: launch one thing repeatedly, print a JSON line, exit."""
    if what == "prologue_prefill":
        h = Headline(torch, mbt, W)
        n = max(steps, h.R)
        for j in range(n):
            h.step(j)
        torch.cuda.synchronize()
        return {"only": what, "cell": h.cell.name, "launches": n}
    if what == "prefill_cells":
        names = []
        for c in W.config3_cells():
            prologue_cold_us(torch, mbt, W, c, launches=500)
            names.append(c.name)
        return {"only": what, "cells": names}
    if what in ("act_prefill", "norm_prefill"):
        # configuration 5's SiLU-gate -> FP8 at T = 512, or configuration 4's
        # bf16 residual norm at H = 2560, T = 512, over a cold buffer ring
        c = prefill_traffic_cell(W, what)
        dev = "cuda:0"
        R = ring_slots(c.bytes_algorithmic())
        if what == "act_prefill":
            gu0 = W.to_torch(c.inputs()["gate_up"], c.dtype, dev)
            ring = [(gu0.clone(), torch.empty((c.T, c.d), dtype=torch.uint8, device=dev))
                    for _ in range(R)]

            def call(j):
                mbt.gated_act_fp8(ring[j][0], 1.0 / 16, c.act, out=ring[j][1])
        else:
            i = c.inputs()
            w = W.to_torch(i["w"], c.dtype, dev)
            x0, r0 = W.to_torch(i["x"], c.dtype, dev), W.to_torch(i["residual"], c.dtype, dev)
            ring = [(x0.clone(), r0.clone()) for _ in range(R)]

            def call(j):
                mbt.fused_add_rmsnorm(ring[j][0], ring[j][1], w, c.eps, c.weight_offset)
        n = max(steps, R)
        for j in range(n):
            call(j % R)
        torch.cuda.synchronize()
        return {"only": what, "cell": c.name, "launches": n}
    st = DecodeStep(torch, mbt, W, 128)
    fn = st.kernels()[what][0]
    n = max(steps, st.R)
    for j in range(n):
        fn(st.slots[j % st.R])
    torch.cuda.synchronize()
    return {"only": what, "tokens": 128, "launches": n}


def main():
    args = parse_args()
    if args.trace_stats:
        trace_stats(*args.trace_stats)
        return
    if args.write_profiles:
        write_profiles(args.write_profiles)
        return
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
    if args.only:
        print(json.dumps(only_mode(torch, mbt, W, args.only, args.steps)), flush=True)
        return

    # ---- the headline: K steps of the prologue at the widest prefill cell
    phase("headline buffers")
    h = Headline(torch, mbt, W)
    c = h.cell
    run = Steps(torch, h.step, h.R)
    phase("headline graphs: captured and replayed once, then one pass over the ring")
    run.prepare([args.warmup, args.steps, args.steps, args.steps])
    phase("headline warm-up and timed steps")
    run.run(args.warmup)                                    # untimed
    ms = run.run(args.steps)                                # timed: exactly K steps
    ms_per_step = ms / args.steps
    # the same measurement twice more, on the slots that follow (a null arm:
    # how far identical runs of K steps differ; `value` is the first)
    repeats = [ms_per_step] + [run.run(args.steps) / args.steps for _ in range(2)]
    us_launch = 1000.0 * ms_per_step
    achieved = h.bytes / us_launch / 1e3
    rp_avg, rp_med = headline_rocprof_us()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic_for("prologue_prefill", "qknorm_rope"),
                "kernel": f"qknorm_rope {c.Q}x{c.K} D{c.D} rot{c.rot} T={c.T} bf16",
                "algorithmic_bytes_per_launch": h.bytes, "avg_launch_us": round(us_launch, 3),
                "rocprof_avg_us": rp_avg, "rocprof_median_us": rp_med}
    phase("copy ceilings")
    copies = {}                  # bytes -> {form: µs}, the streaming copy

    def best_copy(nbytes):
        if nbytes not in copies:
            copies[nbytes] = stream_copy_us(torch, mbt, nbytes)
        k = min(copies[nbytes], key=copies[nbytes].get)
        return copies[nbytes][k], k

    cu, ck = best_copy(h.bytes)
    roofline["copy_ceiling_GBps"] = round(h.bytes / cu / 1e3, 1)
    roofline["copy_ceiling_us"] = round(cu, 3)
    roofline["copy_ceiling_kernel"] = f"mbt_stream_copy, form {ck} (chunks per lane, block sync), cold"
    roofline["of_copy"] = round(cu / us_launch, 4)
    roofline["torch_copy_GBps"] = round(copy_ceiling_gbps(torch, h.bytes), 1)
    del run, h
    torch.cuda.empty_cache()

    phase("T = 1")
    t1 = [x for x in W.config2_cells() if x.T == 1][0]
    w1 = prologue_warm_us(torch, mbt, W, t1)
    us_t1 = {k: round(v, 3) for k, v in w1.items()}
    us_t1["method"] = ("(16,2) D256 rot64 bf16, graph of 32 calls on one buffer set, 20 warm-up "
                       "replays, median / quartiles of 200 replays; stream = direct launches")
    # the same method on the library's streaming copy of the call's bytes,
    # and on its smallest launch (one 16-byte chunk): what any kernel node
    # in a graph costs here, whatever it moves
    us_t1["copy_floor_us"] = round(copy_warm_us(torch, mbt, t1.bytes_algorithmic()), 3)
    us_t1["launch_floor_us"] = round(copy_warm_us(torch, mbt, 32), 3)

    # configuration 1: the Qwen3-style cell (head_dim 128, full rotary,
    # (16, 8) heads, T = 4, one token outside the cache), same method
    config1 = []
    for x in W.config1_cells():
        w = prologue_warm_us(torch, mbt, W, x, samples=100)
        config1.append({"cell": x.name, "T": x.T, "warm_us": round(w["median"], 3),
                        "p25": round(w["p25"], 3), "p75": round(w["p75"], 3)})

    phase("prefill cells")
    prefill = []
    for x in W.config3_cells():
        us = prologue_cold_us(torch, mbt, W, x)
        gbps = x.bytes_algorithmic() / us / 1e3
        ra, rm = rocprof_us_for(x.name)
        cu, ck = best_copy(x.bytes_algorithmic())
        prefill.append({
            "cell": x.name, "QK": f"{x.Q}x{x.K}", "T": x.T, "dtype": W.DTYPE_NAMES[x.dtype],
            "layout": "interleaved" if x.layout == W.INTERLEAVED else "rotate_half",
            "rot_dim": x.rot, "bytes": x.bytes_algorithmic(), "event_us": round(us, 3),
            "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "tokens_per_s": round(x.T / us * 1e6, 1), "rocprof_avg_us": ra,
            "rocprof_frac_peak": None if ra is None else
            round(x.bytes_algorithmic() / ra / 1e3 / PEAK_HBM_GBPS, 4),
            "copy_us": round(cu, 3), "copy_form": ck,
            "of_copy": round(cu / us, 4)})

    out = {
        "metric": METRIC, "value": round(c.T / ms_per_step * 1e3, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"fused QK-RMSNorm+RoPE prologue, (Q,K)=({c.Q},{c.K}) heads, "
                               f"head_dim {c.D}, rot_dim {c.rot} rotate-half, 1+w weights, "
                               f"theta 1e7, T={c.T} tokens at positions 0..{c.T - 1}, bf16 "
                               f"storage, fp32 arithmetic, out of place, cold HBM ring",
                   "cell": c.name, "tokens": c.T, "heads_q": c.Q, "heads_kv": c.K,
                   "head_dim": c.D, "rot_dim": c.rot, "io_dtype": "bf16", "arithmetic": "fp32",
                   "ring_slots": ring_slots(c.bytes_algorithmic()),
                   "ring_bytes": ring_slots(c.bytes_algorithmic()) * c.bytes_algorithmic(),
                   "mode": "cold, hipGraph replays", "parallelism": "none (1 GPU)"},
        "achieved_GBps": roofline["achieved"], "frac_peak": roofline["frac"],
        "repeats_us_per_step": [round(1000.0 * x, 3) for x in repeats],
        "repeat_spread": round(max(repeats) / min(repeats) - 1.0, 4),
        "us_per_call_T1": us_t1,
        "config1_us_per_call": config1,
        "roofline": roofline,
        "prefill": prefill,
        "prefill_frac_min": min(x["frac_peak"] for x in prefill),
        "prefill_of_copy_min": min(x["of_copy"] for x in prefill),
    }

    if not args.no_sweep:
        # the headline geometry past configuration 3's widest batch (positions
        # 0 .. T - 1 with a cache of T rows, so every token rotates)
        phase("large prefill widths")
        large = []
        for T in (4096, 8192, 16384):
            x = W.PrologueCell(name=f"prefill24x4_bf16_T{T}", config=3, cell=900 + T, T=T, Q=24,
                               K=4, D=256, rot=64, theta=1e7, layout=W.ROTATE_HALF, dtype=W.BF16,
                               weight_offset=1, w_mean=0.0, w_std=0.05, x_std=2.0,
                               positions="arange", max_pos=T)
            us = prologue_cold_us(torch, mbt, W, x, launches=400)
            nb = x.bytes_algorithmic()
            cu, ck = best_copy(nb)
            large.append({"T": T, "bytes": nb, "event_us": round(us, 3),
                          "GBps": round(nb / us / 1e3, 1),
                          "frac_peak": round(nb / us / 1e3 / PEAK_HBM_GBPS, 4),
                          "tokens_per_s": round(T / us * 1e6, 1), "copy_us": round(cu, 3),
                          "copy_form": ck, "of_copy": round(cu / us, 4)})
        out["prefill_large_24x4"] = large
        phase("decode sweep")
        sweep = []
        for x in W.config2_cells():
            w = prologue_warm_us(torch, mbt, W, x, samples=50)
            sweep.append({"T": x.T, "warm_us": round(w["median"], 3),
                          "tokens_per_s": round(x.T / w["median"] * 1e6, 1),
                          "logical_GBps_warm": round(x.bytes_logical() / w["median"] / 1e3, 1)})
        out["decode_sweep_16x2"] = sweep
        phase("decode-layer step")
        out["decode_layer_step"] = decode_layer_step(torch, mbt, W)
        # the residual norm (configuration 4, bf16 and fp32, direct weights)
        # and the gated activation (configuration 5), as rows/s and GB/s
        phase("norm sweep (configuration 4)")
        nsweep = []
        for x in W.config4_cells():
            if x.weight_offset != 0 or x.dtype == W.F16:
                continue
            us, mode = norm_cold_us(torch, mbt, W, x)
            gbps = x.bytes_algorithmic() / us / 1e3
            row = {"dtype": W.DTYPE_NAMES[x.dtype], "H": x.H, "T": x.T, "us": round(us, 3),
                   "ring": mode, "rows_per_s": round(x.T / us * 1e6, 1),
                   "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_HBM_GBPS, 4)}
            if mode == "cold":
                # the in-place norm reads and writes equal bytes, like a copy
                cu, ck = best_copy(x.bytes_algorithmic())
                row.update({"copy_us": round(cu, 3), "copy_form": ck,
                            "of_copy": round(cu / us, 4)})
            if x.name == prefill_traffic_cell(W, "norm_prefill").name:
                row["traffic"] = traffic_for("norm_prefill", "rmsnorm")
            nsweep.append(row)
        out["norm_sweep_config4"] = nsweep
        phase("activation sweep (configuration 5)")
        asweep = []
        for x in W.config5_cells():
            if not isinstance(x, W.ActCell):
                continue
            us, mode = act_cold_us(torch, mbt, W, x)
            gbps = x.bytes_algorithmic() / us / 1e3
            arow = {"act": "silu" if x.act == W.SILU else "gelu_tanh", "T": x.T,
                    "out": "fp8" if x.fp8 else "bf16", "d": x.d, "us": round(us, 3),
                    "ring": mode, "rows_per_s": round(x.T / us * 1e6, 1),
                    "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_HBM_GBPS, 4)}
            if x.name == prefill_traffic_cell(W, "act_prefill").name:
                arow["traffic"] = traffic_for("act_prefill", "gated_act")
            asweep.append(arow)
        out["act_sweep_config5"] = asweep
        phase("routes")
        out["routes"] = {"warm": [route_us(torch, mbt, W, x, cold=False)
                                  for x in W.config2_cells() if x.T in (1, 8, 32, 128)],
                         "cold": [route_us(torch, mbt, W, x, cold=True)
                                  for x in W.config3_cells()
                                  if x.dtype == W.BF16 and x.layout == W.ROTATE_HALF]}
        phase("extended prologue forms")
        ext = []
        step_pro = W.PrologueCell(name="step_prologue", config=2, cell=4, T=128, Q=16, K=2,
                                  D=256, rot=64, theta=1e7, layout=W.ROTATE_HALF, dtype=W.BF16,
                                  weight_offset=1, w_mean=0.0, w_std=0.05, x_std=2.0)
        for x in (step_pro, c):
            row = {"QK": f"{x.Q}x{x.K}", "T": x.T,
                   "contract_us": round(prologue_cold_us(torch, mbt, W, x), 3)}
            for form in ("once", "qkv_cache"):
                us, nb = extended_cold_us(torch, mbt, W, x, form)
                row[form + "_us"] = round(us, 3)
                row[form + "_GBps"] = round(nb / us / 1e3, 1)
            ext.append(row)
        out["extended_forms"] = ext
        # RMSNorm -> FP8 with the weight against the no-weight form (the scale
        # folded into the next GEMM), H = 2048, bf16
        phase("no-weight norm")
        noweight = []
        for T in (128, 512):
            row = {"T": T, "H": 2048}
            for wt in (True, False):
                x = W.NormCell(name="nw", config=5, cell=60 + T, T=T, H=2048, dtype=W.BF16,
                               weight_offset=0 if not wt else 1, w_mean=0.0, w_std=0.05,
                               fp8=True, weight=wt)
                xi, cal = x.inputs(), x.calibration_inputs()
                t = lambda b: None if b is None else W.to_torch(b, W.BF16, "cuda:0")
                amax = mbt.fused_add_rmsnorm_amax(t(cal["x"]), t(cal["residual"]), t(xi["w"]),
                                                  x.eps, x.weight_offset)
                inv = W.fp8_inv_scale(float(amax.item()))
                us, mode = norm_fp8_cold_us(torch, mbt, W, x, inv)
                key = "weighted" if wt else "no_weight"
                row[key + "_us"] = round(us, 3)
                row[key + "_GBps"] = round(x.bytes_algorithmic() / us / 1e3, 1)
                row["ring"] = mode
            noweight.append(row)
        out["norm_fp8_weight_vs_none"] = noweight
        # adaptive RMSNorm -> FP8 with a gated residual (style vector per
        # call): the Pi0.5 decoder's 10-token rows and a 512-token batch
        phase("adaptive norm")
        ada = []
        for T in (10, 512):
            x = W.AdaCell(name="ada", config=5, cell=70 + T, T=T, H=2048, dtype=W.BF16, fp8=True)
            us, mode = adarms_fp8_cold_us(torch, mbt, W, x)
            ada.append({"T": T, "H": 2048, "us": round(us, 3), "ring": mode,
                        "GBps": round(x.bytes_algorithmic() / us / 1e3, 1),
                        "frac_peak": round(x.bytes_algorithmic() / us / 1e3 / PEAK_HBM_GBPS, 4)})
        out["adarms_fp8_gated"] = ada
    if args.sustained:
        # the headline held for about a quarter of a second: twelve runs of
        # 2000 steps back to back (after every other GPU figure, so a machine
        # that lowers its clocks under sustained streaming slows nothing else)
        phase("sustained headline")
        hs = Headline(torch, mbt, W)
        rs = Steps(torch, hs.step, hs.R)
        rs.prepare([2000] * 12)
        per = [1000.0 * rs.run(2000) / 2000 for _ in range(12)]
        out["headline_sustained"] = {
            "us_per_step_by_run": [round(x, 3) for x in per],
            "first_over_last": round(per[0] / per[-1], 4),
            "method": "12 back-to-back timed runs of 2000 headline steps on the same ring"}
        del rs, hs
        torch.cuda.empty_cache()

    if not args.no_cpu:
        phase("oracle on the host CPU")
        out["cpu_baseline"] = cpu_baseline(W, c, threads=1)
        n_thr = max(1, min(len(os.sched_getaffinity(0)), 16))
        out["cpu_baseline_threads"] = cpu_baseline(W, c, threads=n_thr)
    # every streaming-copy ceiling taken above: bytes -> {form: µs}
    out["copy_ceilings_us"] = {str(b): {k: round(v, 3) for k, v in d.items()}
                               for b, d in sorted(copies.items())}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
