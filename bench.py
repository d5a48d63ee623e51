"""Benchmark of the TIDE placement collectives on one MI355X.

One step = one pass of the whole hot path over the Llama-3.1-70B-shaped
decoder layer with 8 emulated ranks in this GPU's HBM:
  tide_rs  : rank R's fp32 block of the reduce-scatter of the 8 ranks' bf16
             per-parameter gradients (R rotates over the ranks, so every
             step streams gradient slices the previous step did not touch),
             written into its block of the flat rank-major [8, S] buffer;
  tide_ag  : the rank-major gathered bf16 buffer placed into the full
             per-parameter bf16 tensors.
Inputs are resident in HBM before the timed region starts.

Reported (one JSON line on stdout, progress on stderr):
  value       effective HBM GB/s of the step: algorithmic bytes of both
              calls / wall time per step;
  roofline    the dominant kernel's algorithmic bytes per launch / its mean
              launch time (HIP events on the launch stream) against the
              8 TB/s HBM peak, plus counter-measured traffic when a
              committed counter profile of the current kernel source exists;
  corun       slowdown of a bf16 8192^3 GEMM on another stream while
              tide_rs runs (default and small-footprint launch) on the
              64-rank 70B layer;
  corun_rs_step_workload  the same on the step's 8-rank workload;
  corun_ag    the same for tide_ag on the step's workload: kernel (default,
              small footprint) and SDMA copy engine;
  small_footprint_alone   small-footprint launches with nothing beside them;
  tiny_gpu_latency        the tiny workload's step on the GPU, in microseconds
              (per call, back to back, and per HIP-graph replay);
  tide_rs_variants        the bf16 shard and the mean;
  two_stage_rs            tide_pack + tide_rs_slots (one GPU's share);
  layout_conversion       a decoder-layer step's forward+backward beside
              FSDP2's layout copies (which TIDE removes) and this rank's
              tide_rs + tide_ag;
  copy ceilings           torch's device copy and the library's own copy;
  cpu_baseline the CPU oracle on the same step's inputs (host cores), and
              the tiny workload's step on one thread.

Algorithmic bytes (what the method must move; the fp32 pack buffer and the
copy-out pass it avoids are not counted):
  tide_rs:  2 * N * sum_i L(R,i)  (bf16 reads)  +  4 * S  (fp32 writes)
  tide_ag:  2 * Psi (bf16 reads)  +  2 * Psi (bf16 writes)
"""
import argparse
import dataclasses
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import parameter_layout_collectives_amd as tide  # noqa: E402
import parameter_layout_collectives_amd._lib as tide_lib  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# The kernels' machine code depends on these two files only (the runtime and
# the plan code around them do not change what a launch executes).
KERNEL_SRCS = [os.path.join(ROOT, "parameter_layout_collectives_amd", "csrc", f)
               for f in ("kernels.hip", "kernel_abi.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic_llama31_70b_layer.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fmt(x):
    return "n/a" if x is None else f"{x:.2f}"


def kernel_source_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def rs_bytes(plan, R):
    real = sum(plan.real(R, i)[1] for i in range(plan.P))
    return 2 * plan.world * real + 4 * plan.S


def ag_bytes(plan):
    psi = sum(plan.real(r, i)[1] for r in range(plan.world) for i in range(plan.P))
    return 2 * psi + 2 * psi


def timed_events(n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def copy_ceiling(nbytes=2 << 30, reps=10, library=True):
    """Device-to-device copies of nbytes (read + write) as measured ceilings
    next to the 8 TB/s spec: torch's copy, and this library's own 16-byte
    vector copy (tide_ag with one rank and one parameter: the rank block is
    the whole tensor).  Returns (torch GB/s, library GB/s)."""
    n = nbytes // 2
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    plan = tide.Plan([(n,)], 1)
    tables = tide.ag_tables(plan, a, [b])

    def timed(fn):
        for _ in range(3):
            fn()
        ev = timed_events(reps)
        for s, e in ev:
            s.record()
            fn()
            e.record()
        torch.cuda.synchronize()
        return 2 * nbytes / (statistics.median(s.elapsed_time(e) for s, e in ev) * 1e-3) / 1e9

    g_torch = timed(lambda: b.copy_(a))
    g_lib = None
    if library:
        b.zero_()
        g_lib = timed(lambda: tide.ag(plan, None, None, tables=tables))
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del a, b, tables
    return g_torch, g_lib


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------

class Step:
    def __init__(self, w, small=False):
        self.w = w
        self.small = small
        N = w.world
        log(f"generating {w.name}: {N} ranks x {len(w.shapes)} params on the device")
        self.grads = workloads.all_grads(w, device="cuda")
        self.plan = tide.Plan(w.shapes, N)
        S = self.plan.S
        self.table = tide.grad_table(self.plan, self.grads)
        self.blocks = torch.zeros(N, S, dtype=torch.float32, device="cuda")
        self.gathered = workloads.random_bf16(N * S, seed=4242, sigma=w.sigma, device="cuda")
        self.params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in w.shapes]
        self.agt = tide.ag_tables(self.plan, self.gathered, self.params)
        self.b_rs = rs_bytes(self.plan, 0)
        self.b_ag = ag_bytes(self.plan)
        torch.cuda.synchronize()

    def rs(self, R):
        tide.rs(self.plan, R, self.table, self.blocks[R], small=self.small)

    def ag(self):
        tide.ag(self.plan, None, None, small=self.small, tables=self.agt)

    def run(self, steps, warmup):
        """Wall time of exactly `steps` back-to-back steps (synchronised on both
        sides, nothing else on the stream), then the same steps again with a
        HIP event pair around every launch for the per-kernel statistics."""
        N = self.w.world
        for k in range(warmup):
            self.rs(k % N)
            self.ag()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            self.rs(k % N)
            self.ag()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_rs = timed_events(steps)
        ev_ag = timed_events(steps)
        torch.cuda.synchronize()
        for k in range(steps):
            ev_rs[k][0].record()
            self.rs(k % N)
            ev_rs[k][1].record()
            ev_ag[k][0].record()
            self.ag()
            ev_ag[k][1].record()
        torch.cuda.synchronize()
        t_rs = [s.elapsed_time(e) * 1e-3 for s, e in ev_rs]
        t_ag = [s.elapsed_time(e) * 1e-3 for s, e in ev_ag]
        return wall, t_rs, t_ag


def tiny_latency(reps=200, warmup=20, replays=200):
    """The tiny workload's step on the GPU (tide_rs for its rank, then tide_ag
    of the fp32 blocks): a few hundred bytes, so it is latency-bound and
    reported in microseconds, with no roofline.  Three figures: the median
    event-timed duration of each call, the wall time per step launched back
    to back from Python (bound by the host cost of the calls), and the wall
    time per replay of a HIP graph holding the step, replayed back to back
    (the graph launch path instead of two kernel launches)."""
    w = workloads.WORKLOADS["tiny"]
    N, R = w.world, w.rank
    grads = workloads.all_grads(w, device="cuda")
    plan = tide.Plan(w.shapes, N)
    table = tide.grad_table(plan, grads)
    blocks = torch.zeros(N, plan.S, dtype=torch.float32, device="cuda")
    params = [torch.empty(s, dtype=torch.float32, device="cuda") for s in w.shapes]
    agt = tide.ag_tables(plan, blocks, params)

    def rs():
        tide.rs(plan, R, table, blocks[R])

    def ag():
        tide.ag(plan, None, None, tables=agt)

    for _ in range(warmup):
        rs()
        ag()
    torch.cuda.synchronize()
    ev_rs, ev_ag = timed_events(reps), timed_events(reps)
    for k in range(reps):
        ev_rs[k][0].record()
        rs()
        ev_rs[k][1].record()
        ev_ag[k][0].record()
        ag()
        ev_ag[k][1].record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        rs()
        ag()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    res = {
        "workload": w.name,
        "rank": R,
        "tide_rs_event_us_median": statistics.median(s.elapsed_time(e) for s, e in ev_rs) * 1e3,
        "tide_ag_event_us_median": statistics.median(s.elapsed_time(e) for s, e in ev_ag) * 1e3,
        "step_wall_us_back_to_back": wall * 1e6,
    }
    # the same step captured once (its pointer tables are already uploaded)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rs()
        ag()
    torch.cuda.synchronize()
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    res["step_us_graph_replay"] = (time.perf_counter() - t0) / replays * 1e6
    del g
    log(f"tiny step: rs {res['tide_rs_event_us_median']:.1f} us, ag "
        f"{res['tide_ag_event_us_median']:.1f} us (events), {res['step_wall_us_back_to_back']:.1f} "
        f"us back to back, {res['step_us_graph_replay']:.1f} us per graph replay")
    return res


def small_footprint_alone(step, reps=20, warmup=3):
    """Event-timed small-footprint launches with nothing beside them, R
    rotating (median, p10, p90 as for the default launch)."""
    plan, N = step.plan, step.w.world
    res = {}
    for name, fn, nbytes in (
            ("tide_rs", lambda k: tide.rs(plan, k % N, step.table, step.blocks[k % N], small=True),
             step.b_rs),
            ("tide_ag", lambda k: tide.ag(plan, None, None, small=True, tables=step.agt),
             step.b_ag)):
        for k in range(warmup):
            fn(k)
        ev = timed_events(reps)
        torch.cuda.synchronize()
        for k in range(reps):
            ev[k][0].record()
            fn(k)
            ev[k][1].record()
        torch.cuda.synchronize()
        res[name] = kernel_stats(f"{name} (small footprint)", nbytes,
                                 [a.elapsed_time(b) * 1e-3 for a, b in ev])
        log(f"{name} small footprint alone: {res[name]['GBps']:.1f} GB/s")
    return res


def rs_variants(step, reps=20, warmup=3):
    """Event-timed tide_rs launches of the flag variants on the step's
    workload, R rotating: the bf16 shard (fp32 sum rounded once; half the
    write bytes) and the mean.  Bytes per launch: 2*N*sum_i L(R,i) reads
    plus S * (4 or 2) writes."""
    plan, N = step.plan, step.w.world
    out16 = torch.zeros(N, plan.S, dtype=torch.bfloat16, device="cuda")
    res = {}
    for name, out, kw, nbytes in (
            ("bf16_out", out16, {}, step.b_rs - 2 * plan.S),
            ("mean", step.blocks, {"avg": True}, step.b_rs)):
        for k in range(warmup):
            tide.rs(plan, k % N, step.table, out[k % N], **kw)
        ev = timed_events(reps)
        torch.cuda.synchronize()
        for k in range(reps):
            ev[k][0].record()
            tide.rs(plan, k % N, step.table, out[k % N], **kw)
            ev[k][1].record()
        torch.cuda.synchronize()
        res[name] = kernel_stats(f"tide_rs ({name})", nbytes, [a.elapsed_time(b) * 1e-3
                                                              for a, b in ev])
        log(f"tide_rs {name}: {res[name]['GBps']:.1f} GB/s")
    del out16
    return res


def two_stage_leg(step, reps=16, warmup=2):
    """One GPU's share of the two-stage TIDE-RS on the step's workload, R
    rotating: stage 1 packs rank R's gradients into its rank-major slot
    (2*Psi bytes read, 2*N*S written), stage 2 reduces block R of the N
    slots (the peers' slots are packed beforehand, untimed).  Staging needs
    N*S*2 bytes per rank, or none with Slot-Reuse (the vacated all-gather
    buffer has exactly that size)."""
    plan, N, S = step.plan, step.w.world, step.plan.S
    slots = torch.empty(N, N * S, dtype=torch.bfloat16, device="cuda")
    tables = [tide.PointerTable(step.grads[r], torch.bfloat16) for r in range(N)]
    for r in range(N):
        tide.pack(plan, tables[r], slots[r])
    stable = tide.slot_table(plan, slots)
    out = step.blocks
    for k in range(warmup):
        tide.pack(plan, tables[k % N], slots[k % N])
        tide.rs_slots(plan, k % N, stable, out[k % N])
    ev1, ev2 = timed_events(reps), timed_events(reps)
    torch.cuda.synchronize()
    for k in range(reps):
        R = k % N
        ev1[k][0].record()
        tide.pack(plan, tables[R], slots[R])
        ev1[k][1].record()
        ev2[k][0].record()
        tide.rs_slots(plan, R, stable, out[R])
        ev2[k][1].record()
    torch.cuda.synchronize()
    b1 = 2 * step.w.psi + 2 * N * S
    st1 = kernel_stats("tide_pack", b1, [a.elapsed_time(b) * 1e-3 for a, b in ev1])
    st2 = kernel_stats("tide_rs_slots", step.b_rs, [a.elapsed_time(b) * 1e-3 for a, b in ev2])
    t = st1["mean_us"] + st2["mean_us"]
    log(f"two-stage: pack {st1['GBps']:.1f} GB/s, rs_slots {st2['GBps']:.1f} GB/s, "
        f"{t:.1f} us per rank vs one-pass")
    del slots, stable, tables
    return {"stage1_pack": st1, "stage2_rs_slots": st2, "total_us": t,
            "rs_effective_GBps": step.b_rs / (t * 1e-6) / 1e9,
            "staging_bytes_per_rank": 2 * N * S, "staging_bytes_with_slot_reuse": 0}


def _rmsnorm(x, w, eps=1e-5):
    xf = x.float()
    return (xf * torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)).to(x.dtype) * w


def decoder_layer_fwd_bwd(p, x, n_heads, n_kv):
    """Forward and backward of one Llama-shaped decoder layer on one
    micro-batch x [T, D] with bf16 weights p = (q, k, v, o, gate, up, down,
    norm1, norm2).  Every product is a plain 2-D GEMM: the attention core is
    an elementwise stand-in (sigmoid(q * k) * v per head, k and v shared by
    groups of heads) with the real parameters and gradient shapes, so no
    batched bf16 product (or its transposed-operand backward) runs."""
    q_w, k_w, v_w, o_w, g_w, u_w, d_w, n1, n2 = p
    T = x.shape[0]
    hd = q_w.shape[0] // n_heads
    h = _rmsnorm(x, n1)
    q = torch.nn.functional.linear(h, q_w).view(T, n_kv, n_heads // n_kv, hd)
    k = torch.nn.functional.linear(h, k_w).view(T, n_kv, 1, hd)
    v = torch.nn.functional.linear(h, v_w).view(T, n_kv, 1, hd)
    a = (torch.sigmoid(q * k) * v).reshape(T, q_w.shape[0])
    x1 = x + torch.nn.functional.linear(a, o_w)
    h2 = _rmsnorm(x1, n2)
    m = torch.nn.functional.silu(torch.nn.functional.linear(h2, g_w)) * \
        torch.nn.functional.linear(h2, u_w)
    y = x1 + torch.nn.functional.linear(m, d_w)
    y.float().square().mean().backward()


def layout_conversion_leg(step, tokens=8192, reps=3):
    """One GPU's share of a data-parallel step of the workload's decoder layer
    (8K tokens per GPU, as in the pages' 70B runs): forward and backward of
    one micro-batch, then this rank's tide_rs and tide_ag.  Beside it, the
    layout copies TIDE removes, timed as FSDP2 makes them with torch ops:
    the gradient pack (per-parameter bf16 -> padded rank-major fp32 buffer)
    and the all-gather copy-out (rank-major bf16 buffer -> per-parameter
    tensors).  Their share of the step is the analogue of the pages' 6.4%."""
    w, plan, N, S = step.w, step.plan, step.w.world, step.plan.S
    if len(w.shapes) != 9:
        return None                       # dense decoder layers only
    D = w.shapes[0][1]
    n_heads, n_kv = w.shapes[0][0] // 128, w.shapes[1][0] // 128
    gen = torch.Generator(device="cuda").manual_seed(77)
    params = [(torch.randn(s, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
              .requires_grad_() for s in w.shapes]
    x = torch.randn(tokens, D, generator=gen, device="cuda").to(torch.bfloat16)
    segs = [(plan.param(i)[0], plan.param(i)[2]) for i in range(plan.P)]

    def fwd_bwd():
        for t in params:
            t.grad = None
        decoder_layer_fwd_bwd(params, x, n_heads, n_kv)

    def stock_pack():
        parts = []
        for t, (off, seg) in zip(params, segs):
            d0, inner = (t.shape[0], t.numel() // t.shape[0])
            c = seg // inner
            g = t.grad.view(d0, inner)
            if N * c > d0:
                g = torch.nn.functional.pad(g, (0, 0, 0, N * c - d0))
            parts.append(g.reshape(N, seg))
        return torch.cat(parts, dim=1).float()

    def stock_copy_out():
        gb = step.gathered.view(N, S)
        for t, (off, seg) in zip(params, segs):
            d0, inner = (t.shape[0], t.numel() // t.shape[0])
            t.data.copy_(gb[:, off:off + seg].reshape(-1, inner)[:d0].view(t.shape))

    fwd_bwd()
    torch.cuda.synchronize()
    assert all(t.grad is not None for t in params)
    res = {}
    for name, fn in (("fwd_bwd", fwd_bwd), ("stock_grad_pack", stock_pack),
                     ("stock_copy_out", stock_copy_out),
                     ("tide_rs", lambda: step.rs(0)), ("tide_ag", step.ag)):
        fn()
        ev = timed_events(reps)
        torch.cuda.synchronize()
        for k in range(reps):
            ev[k][0].record()
            fn()
            ev[k][1].record()
        torch.cuda.synchronize()
        res[name + "_ms"] = statistics.median(a.elapsed_time(b) for a, b in ev)
    copies = res["stock_grad_pack_ms"] + res["stock_copy_out_ms"]
    stock_step = res["fwd_bwd_ms"] + copies
    res.update({
        "tokens": tokens,
        "attention_core": "elementwise stand-in (no batched bf16 products)",
        "stock_layout_copies_ms": copies,
        "stock_layout_share_pct": 100.0 * copies / stock_step,
        "tide_layout_copies_ms": 0.0,
        "tide_local_collective_share_pct":
            100.0 * (res["tide_rs_ms"] + res["tide_ag_ms"]) /
            (res["fwd_bwd_ms"] + res["tide_rs_ms"] + res["tide_ag_ms"]),
    })
    log(f"layout conversion: fwd+bwd {res['fwd_bwd_ms']:.2f} ms, stock copies {copies:.2f} ms "
        f"({res['stock_layout_share_pct']:.1f}% of the step), tide rs+ag "
        f"{res['tide_rs_ms'] + res['tide_ag_ms']:.2f} ms")
    del params, x
    return res


def kernel_stats(name, nbytes, times):
    mean = statistics.fmean(times)
    q = sorted(times)
    return {
        "kernel": name,
        "bytes_per_launch": nbytes,
        "launches": len(times),
        "mean_us": mean * 1e6,
        "median_us": statistics.median(times) * 1e6,
        "p10_us": q[len(q) // 10] * 1e6,
        "p90_us": q[(9 * len(q)) // 10] * 1e6,
        "GBps": nbytes / mean / 1e9,
        "pct_of_peak": 100.0 * nbytes / mean / 1e9 / HBM_PEAK_GBPS,
    }


def counter_traffic(kernel, workload, small, other_lib):
    """HBM bytes per launch from the committed counter profile, if it was
    taken on the current kernel source, on this workload and launch mode,
    with the in-tree library (else None)."""
    if other_lib:
        return None
    try:
        with open(PMC_SUMMARY) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if doc.get("workload") != workload or doc.get("launch") != ("small" if small else "default"):
        return None
    k = doc.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# co-run with a bf16 GEMM
# ---------------------------------------------------------------------------

class Gemm:
    """The co-running compute kernel: a bf16 GEMM on its own stream."""

    def __init__(self, shape, reps=30):
        M, K, Nn = shape
        g = torch.Generator(device="cuda").manual_seed(77)
        self.A = torch.randn(M, K, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        self.B = torch.randn(K, Nn, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        self.C = torch.empty(M, Nn, dtype=torch.bfloat16, device="cuda")
        self.flop = 2.0 * M * K * Nn
        self.name = f"bf16 {M}x{K}x{Nn} torch.matmul"
        self.reps = reps
        # Two streams for the whole co-run phase: the process has few hardware
        # queues, and a stream created later can land on the GEMM's queue,
        # which would serialise the two instead of running them together.
        self.stream = torch.cuda.Stream()
        self.side = torch.cuda.Stream()
        torch.cuda.synchronize()
        ev = timed_events(reps)
        with torch.cuda.stream(self.stream):
            for _ in range(5):
                self.run()
            for s, e in ev:
                s.record()
                self.run()
                e.record()
        torch.cuda.synchronize()
        self.alone_ms = statistics.median(s.elapsed_time(e) for s, e in ev)

    def run(self):
        torch.matmul(self.A, self.B, out=self.C)


def corun_chain(gemm, launch, nbytes, repeats=2):
    """GEMMs on their stream while `launch(k, stream)` calls run back to back
    on another stream (started first, long enough to cover every GEMM).
    Returns the median GEMM slowdown over `repeats` runs and per-run detail;
    only GEMMs that start and end inside the collective's window count."""
    sb = gemm.side
    ev = timed_events(6)
    with torch.cuda.stream(sb):
        for k in range(2):
            launch(k, sb)
        for k, (s, e) in enumerate(ev):
            s.record()
            launch(k, sb)
            e.record()
    torch.cuda.synchronize()
    t_alone = statistics.median(s.elapsed_time(e) for s, e in ev)
    runs = []
    for _ in range(repeats):
        n = int(1.5 * (gemm.reps + 4) * gemm.alone_ms / t_alone) + 4
        base = torch.cuda.Event(enable_timing=True)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        first_done = torch.cuda.Event()
        ev = timed_events(gemm.reps)
        torch.cuda.synchronize()
        base.record()
        sb.wait_stream(torch.cuda.current_stream())
        gemm.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sb):
            c0.record()
            launch(0, sb)
            first_done.record()
            for k in range(1, n):
                launch(k, sb)
            c1.record()
        with torch.cuda.stream(gemm.stream):
            gemm.stream.wait_event(first_done)
            for _ in range(2):
                gemm.run()
            for s, e in ev:
                s.record()
                gemm.run()
                e.record()
        torch.cuda.synchronize()
        lo, hi = base.elapsed_time(c0), base.elapsed_time(c1)
        starts = [base.elapsed_time(s) for s, _ in ev]
        ends = [base.elapsed_time(e) for _, e in ev]
        inside = [e - s for s, e in zip(starts, ends) if s >= lo and e <= hi]
        if len(inside) < gemm.reps // 2:
            log(f"co-run: only {len(inside)} of {gemm.reps} GEMMs ran inside the collective's "
                f"window {lo:.1f}-{hi:.1f} ms (GEMMs {min(starts):.1f}-{max(ends):.1f} ms); "
                "this run does not measure concurrency")
            inside = []
        med = statistics.median(inside) if inside else None
        runs.append({
            "gemm_corun_ms": med,
            "gemms_fully_overlapped": len(inside),
            "gemm_slowdown_pct": None if med is None else 100.0 * (med / gemm.alone_ms - 1.0),
            "corun_GBps": n * nbytes / ((hi - lo) * 1e-3) / 1e9,
            "calls": n,
            "window_ms": [lo, hi],
            "gemms_ms": [min(starts), max(ends)],
        })
    slow = [r["gemm_slowdown_pct"] for r in runs if r["gemm_slowdown_pct"] is not None]
    return {
        "alone_us": t_alone * 1e3,
        "alone_GBps": nbytes / (t_alone * 1e-3) / 1e9,
        "corun_GBps": statistics.median(r["corun_GBps"] for r in runs),
        "gemm_slowdown_pct": statistics.median(slow) if slow else None,
        "runs": runs,
    }


CORUN_METHOD = ("stream A runs the GEMMs, stream B a chain of collective calls started first and "
                "long enough to cover them; slowdown = median GEMM time while the chain runs / "
                "median GEMM time alone - 1, counting only GEMMs that start and end inside the "
                "chain's window; median of 2 runs")


def corun_rs(w, gemm):
    """tide_rs beside the GEMM, default and small-footprint launch."""
    N = w.world
    log(f"co-run: generating {w.name} ({N} ranks) beside a {gemm.name}")
    grads = workloads.all_grads(w, device="cuda")
    plan = tide.Plan(w.shapes, N)
    table = tide.grad_table(plan, grads)
    out = torch.empty(N, plan.S, dtype=torch.float32, device="cuda")
    b_rs = rs_bytes(plan, 0)
    res = {"gemm": gemm.name, "gemm_alone_ms": gemm.alone_ms,
           "gemm_tflops_alone": gemm.flop / (gemm.alone_ms * 1e-3) / 1e12,
           "workload": w.name, "world": N, "method": CORUN_METHOD}
    for small in (False, True):
        key = "small_footprint" if small else "default"
        r = corun_chain(gemm, lambda k, st: tide.rs(plan, k % N, table, out[k % N], small=small,
                                                     stream=st), b_rs)
        res[key] = {"tide_rs_alone_us": r["alone_us"], "tide_rs_alone_GBps": r["alone_GBps"],
                    "tide_rs_corun_GBps": r["corun_GBps"],
                    "gemm_slowdown_pct": r["gemm_slowdown_pct"], "runs": r["runs"]}
        log(f"co-run tide_rs {key}: slowdown {fmt(r['gemm_slowdown_pct'])}% runs {r['runs']}, "
            f"{r['corun_GBps']:.0f} GB/s during, {r['alone_GBps']:.0f} GB/s alone")
    del grads, table, out
    return res


def corun_rs_step(step, gemm):
    """tide_rs beside the GEMM on the step's workload (its gradients are
    already resident), default and small-footprint launch."""
    plan, N = step.plan, step.w.world
    res = {"gemm": gemm.name, "gemm_alone_ms": gemm.alone_ms, "workload": step.w.name,
           "world": N, "method": CORUN_METHOD}
    for small in (False, True):
        key = "small_footprint" if small else "default"
        r = corun_chain(gemm, lambda k, st: tide.rs(plan, k % N, step.table, step.blocks[k % N],
                                                     small=small, stream=st), step.b_rs)
        res[key] = {"tide_rs_alone_us": r["alone_us"], "tide_rs_alone_GBps": r["alone_GBps"],
                    "tide_rs_corun_GBps": r["corun_GBps"],
                    "gemm_slowdown_pct": r["gemm_slowdown_pct"], "runs": r["runs"]}
        log(f"co-run tide_rs ({step.w.name}) {key}: slowdown {fmt(r['gemm_slowdown_pct'])}%, "
            f"{r['corun_GBps']:.0f} GB/s during, {r['alone_GBps']:.0f} GB/s alone")
    return res


def corun_ag(step, gemm):
    """tide_ag beside the GEMM: kernel (default, small footprint) and SDMA copy engine."""
    res = {"gemm": gemm.name, "gemm_alone_ms": gemm.alone_ms, "workload": step.w.name,
           "world": step.w.world, "method": CORUN_METHOD}
    for key, kw in (("default", {}), ("small_footprint", {"small": True}),
                    ("copy_engine", {"copy_engine": True})):
        r = corun_chain(gemm, lambda k, st: tide.ag(step.plan, None, None, stream=st,
                                                     tables=step.agt, **kw), step.b_ag)
        res[key] = {"tide_ag_alone_us": r["alone_us"], "tide_ag_alone_GBps": r["alone_GBps"],
                    "tide_ag_corun_GBps": r["corun_GBps"],
                    "gemm_slowdown_pct": r["gemm_slowdown_pct"], "runs": r["runs"]}
        log(f"co-run tide_ag {key}: slowdown {fmt(r['gemm_slowdown_pct'])}% runs {r['runs']}, "
            f"{r['corun_GBps']:.0f} GB/s during, {r['alone_GBps']:.0f} GB/s alone")
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the same step
# ---------------------------------------------------------------------------

def cpu_baseline(step, min_reps=3, max_reps=40, budget_s=10.0):
    import numpy as np

    import oracle

    orc = oracle.default()
    w, plan = step.w, step.plan
    N, S, R = w.world, plan.S, 0
    log("cpu baseline: copying rank-0 gradient slices and the gathered buffer to the host")
    slices = []
    for rank in step.grads:
        row = []
        for i, g in enumerate(rank):
            src, L = plan.real(R, i)
            row.append(g.reshape(-1)[src:src + L].view(torch.int16).cpu().numpy().view(np.uint16))
        slices.append(row)
    host = step.gathered.view(torch.int16).cpu().numpy().view(np.uint16)
    blocks = [host[r * S:(r + 1) * S] for r in range(N)]
    t_rs, t_ag = [], []
    start = time.perf_counter()
    for k in range(max_reps):
        if k >= min_reps and time.perf_counter() - start > budget_s:
            break
        t0 = time.perf_counter()
        orc.rs_slices(w.shapes, N, R, slices)
        t1 = time.perf_counter()
        orc.ag(w.shapes, N, blocks, elem_bytes=2)
        t2 = time.perf_counter()
        t_rs.append(t1 - t0)
        t_ag.append(t2 - t1)
        if k < 3:
            log(f"cpu baseline rep {k}: rs {t1 - t0:.3f} s, ag {t2 - t1:.3f} s")
    trs, tag = statistics.median(t_rs), statistics.median(t_ag)
    # the tiny workload on one thread (latency, not bandwidth)
    tw = workloads.WORKLOADS["tiny"]
    tg = [[workloads.bf16_bits(t).reshape(-1) for t in rank] for rank in workloads.all_grads(tw)]
    tplan = orc.geometry(tw.shapes, tw.world)
    tblocks = [np.zeros(tplan.S, np.uint16) for _ in range(tw.world)]
    threads = orc.threads()
    orc.set_threads(1)
    try:
        t_tiny = []
        for _ in range(200):
            t0 = time.perf_counter()
            orc.rs(tw.shapes, tw.world, 1, tg)
            orc.ag(tw.shapes, tw.world, tblocks, elem_bytes=2)
            t_tiny.append(time.perf_counter() - t0)
    finally:
        orc.set_threads(threads)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": (step.b_rs + step.b_ag) / (trs + tag) / 1e9,
        "unit": "GB/s",
        "cores": orc.threads(),
        "kind": "oracle",
        "sample": (f"one full step of {w.name} (tide_rs for rank 0 from host copies of its "
                   f"{N}x{plan.P} gradient slices + tide_ag of the {N}x{S} gathered buffer), "
                   f"median of {len(t_rs)} repetitions (~{budget_s:.0f} s); host copies not timed"),
        "rs_s": trs,
        "ag_s": tag,
        "tiny_step_us_1_thread": statistics.median(t_tiny) * 1e6,
        "cpu_model": cpu,
    }


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama31_70b_layer")
    ap.add_argument("--small", action="store_true", help="time the small-footprint launch")
    ap.add_argument("--corun", default="llama31_70b_layer_n64",
                    help="workload for the co-run GEMM measurement, or 'none'")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-copy", action="store_true", help="skip the copy-ceiling measurement")
    ap.add_argument("--no-lib-copy", action="store_true",
                    help="measure the copy ceiling with torch's copy only (profiled runs: the "
                         "library's copy is an all-gather launch)")
    ap.add_argument("--world", type=int, default=0,
                    help="number of emulated ranks, overriding the workload's (same shapes)")
    ap.add_argument("--lib", default="",
                    help="load the libtide.so at this path instead of the in-tree one (e.g. one "
                         "built with other tuning macros)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the tide_rs flag variants (bf16 shard, mean) and the "
                         "two-stage reduce-scatter")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (--gpus {args.gpus} requested); "
              "the N emulated ranks of the workload live in that GPU's memory.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no HIP device", file=sys.stderr, flush=True)
        sys.exit(1)
    if args.lib:
        tide_lib.LIB_PATH = os.path.abspath(args.lib)
    tide.lib()   # fails loudly if the HIP library is missing

    w = workloads.WORKLOADS[args.workload]
    if args.world and args.world != w.world:
        w = dataclasses.replace(w, name=f"{w.name}_n{args.world}", world=args.world)
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name}, {props.multi_processor_count} CUs")

    step = Step(w, small=args.small)
    log(f"plan: N={w.world} P={step.plan.P} S={step.plan.S} "
        f"B_rs={step.b_rs} B_ag={step.b_ag}")
    wall, t_rs, t_ag = step.run(args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    value = (step.b_rs + step.b_ag) * args.steps / wall / 1e9
    rs_k = kernel_stats("tide_rs", step.b_rs, t_rs)
    ag_k = kernel_stats("tide_ag", step.b_ag, t_ag)
    log(f"step {ms_per_step:.3f} ms, {value:.1f} GB/s; rs {rs_k['GBps']:.1f} GB/s, "
        f"ag {ag_k['GBps']:.1f} GB/s")

    dom = rs_k if sum(t_rs) >= sum(t_ag) else ag_k
    traffic = counter_traffic(dom["kernel"], w.name, args.small, bool(args.lib))
    roofline = {
        "bound": "hbm",
        "kernel": dom["kernel"],
        "achieved": dom["GBps"],
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": dom["GBps"] / HBM_PEAK_GBPS,
        "traffic": traffic,
        "bytes_per_launch": dom["bytes_per_launch"],
        "mean_launch_us": dom["mean_us"],
    }

    variants = None if args.no_variants else rs_variants(step)
    small_alone = None if args.no_variants else small_footprint_alone(step)
    tiny = None if args.no_variants else tiny_latency()
    two_stage = None if args.no_variants else two_stage_leg(step)
    layout = None if args.no_variants else layout_conversion_leg(step)
    copy_gbps, copy_lib_gbps = (None, None) if args.no_copy else \
        copy_ceiling(library=not args.no_lib_copy)
    if copy_gbps:
        log(f"copy ceiling {copy_gbps:.1f} GB/s (torch), {fmt(copy_lib_gbps)} GB/s (library)")
    cpu = None if args.no_cpu else cpu_baseline(step)
    corun_res = corun_ag_res = corun_rs_step_res = None
    gemm = None
    if args.corun != "none":
        cw = workloads.WORKLOADS[args.corun]
        gemm = Gemm(cw.corun_gemm or (8192, 8192, 8192))
        corun_ag_res = corun_ag(step, gemm)
        corun_rs_step_res = corun_rs_step(step, gemm)
    P, S = step.plan.P, step.plan.S
    del step
    gc.collect()
    torch.cuda.empty_cache()
    if gemm is not None:
        corun_res = corun_rs(cw, gemm)
        gc.collect()
        torch.cuda.empty_cache()

    line = {
        "metric": "tide_rs/tide_ag effective HBM GB/s + % of peak; co-run GEMM slowdown %",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "description": w.description,
            "world": w.world,
            "params": P,
            "psi": w.psi,
            "shard_numel": S,
            "grad_dtype": "bf16",
            "shard_dtype": "f32",
            "ag_dtype": "bf16",
            "launch": "small_footprint" if args.small else "default",
            "parallelism": "1 GPU, emulated ranks in one HBM",
        },
        "pct_of_peak": 100.0 * value / HBM_PEAK_GBPS,
        # the measured ceiling is this library's own 16-byte copy kernel over
        # 2 GiB; torch's copy (lower) is reported beside it
        "pct_of_copy_ceiling": None if not copy_lib_gbps else 100.0 * value / copy_lib_gbps,
        "copy_ceiling_library_GBps": copy_lib_gbps,
        "pct_of_torch_copy": None if not copy_gbps else 100.0 * value / copy_gbps,
        "torch_copy_GBps": copy_gbps,
        "tide_rs": rs_k,
        "tide_ag": ag_k,
        "tide_rs_variants": variants,
        "small_footprint_alone": small_alone,
        "tiny_gpu_latency": tiny,
        "two_stage_rs": two_stage,
        "layout_conversion": layout,
        "corun": corun_res,
        "corun_ag": corun_ag_res,
        "corun_rs_step_workload": corun_rs_step_res,
        "gemm_slowdown_pct": None if not corun_res else {
            k: corun_res[k]["gemm_slowdown_pct"] for k in ("default", "small_footprint")
            if k in corun_res},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if args.lib:
        line["library"] = args.lib
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
