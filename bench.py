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
  corun       tide_rs (default and small-footprint launch) on the 64-rank
              70B layer beside a bf16 8192^3 GEMM on another stream: the
              GEMM's slowdown, the bytes the collective moves while the GEMMs
              run (per-call events), and the exposed time of a fixed amount
              of collective work run beside a fixed GEMM chain;
  corun_rs_step_workload  the same on the step's 8-rank workload;
  corun_ag    the same for tide_ag on the step's workload: kernel (default,
              small footprint) and SDMA copy engine;
  corun_layer_step  tide_rs and tide_ag beside the decoder layer's own
              forward+backward (8K tokens) instead of the GEMM;
  corun_summary     one row per co-run leg and mode;
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
The printed line leaves out the per-repeat lists of the co-run experiments
(their medians stay); --detail FILE writes the full result as well.

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


# The pages' own figures (NVIDIA hardware, up to 64 GPUs), quoted in the
# bench line as context, never as targets: TIDE article ("FSDP通信终局：TIDE零
# 拷贝集合通信优化") §"FSDP2通信开销的根源" (layout conversion share; NCCL
# reduce-scatter slowing a single-wave GEMM) and §"性能表现" (step time,
# reduce-scatter SM time, peak memory).
PAGES_CONTEXT = {
    "source": "TIDE article, kongchang.com: sections on the roots of FSDP2's communication "
              "cost and on performance; NVIDIA hardware at up to 64 GPUs; context, not targets",
    "layout_conversion_pct_of_step_llama31_70b_8k_tokens": 6.4,
    "nccl_reduce_scatter_single_wave_gemm_slowdown_pct_max": 69.0,
    "step_time_reduction_vs_stock_fsdp2_pct_max": 27.1,
    "step_time_reduction_vs_fsdp2_symmmem_pct_max": 6.0,
    "reduce_scatter_sm_time_reduction_factor": [12.5, 14.5],
    "peak_memory_reduction_vs_fsdp2_symmmem_gib_max": 4.7,
}


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


def rs_bytes_mean(plan):
    """Mean of rs_bytes over the ranks: the bytes per call of a chain whose
    rank R rotates through 0..N-1 (equal to every rank's when every dim 0
    divides by N; below it when the last ranks hold padding rows)."""
    total = sum(rs_bytes(plan, r) for r in range(plan.world))
    return total // plan.world if total % plan.world == 0 else total / plan.world


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
        self.b_rs = rs_bytes_mean(self.plan)
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


def two_stage_leg(step, streams, reps=16, warmup=2, buckets=8):
    """One GPU's share of the two-stage TIDE-RS on the step's workload.

    Stage times, R rotating: stage 1 packs rank R's gradients into its
    rank-major slot (2*Psi bytes read, 2*N*S written), stage 2 reduces block
    R of the N slots (the peers' slots are packed beforehand, untimed).

    Peak memory of rank R's reduce-scatter (torch.cuda.max_memory_allocated
    above what is allocated before it): one-pass tide_rs; two-stage with a
    staging slot of its own (allocated for the call); two-stage with
    Slot-Reuse, where the slot is the vacated all-gather buffer.  The peers'
    slots stand for other GPUs' memory and are allocated beforehand.

    Pipelined bandwidth: `buckets` buckets (rank R = k mod N), two slot sets
    used in turn, stage 1 of bucket k+1 on one stream while stage 2 of
    bucket k runs on the other, against the same buckets one after the
    other on one stream."""
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

    # -- peak memory of rank R's reduce-scatter -----------------------------
    R = 0

    def extra_peak(fn):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() - base

    def one_pass():
        tide.rs(plan, R, step.table, out[R])

    def with_slot(own):
        tide.pack(plan, tables[R], own)
        tbl = tide.slot_table(plan, [own if r == R else slots[r] for r in range(N)])
        tide.rs_slots(plan, R, tbl, out[R])

    def separate():
        own = torch.empty(N * S, dtype=torch.bfloat16, device="cuda")
        with_slot(own)
        del own

    mem = {
        "peak_bytes_one_pass": extra_peak(one_pass),
        "peak_bytes_separate": extra_peak(separate),
        "peak_bytes_slot_reuse": extra_peak(lambda: with_slot(step.gathered)),
        "staging_bytes_per_rank": 2 * N * S,
        "method": "torch.cuda.max_memory_allocated() minus memory_allocated() before one "
                  "rank's reduce-scatter; Slot-Reuse packs into the all-gather buffer",
    }
    log(f"two-stage peak memory: one-pass {mem['peak_bytes_one_pass']}, separate slot "
        f"{mem['peak_bytes_separate']}, Slot-Reuse {mem['peak_bytes_slot_reuse']} bytes")

    # -- pipelined: stage 1 of bucket k+1 beside stage 2 of bucket k --------
    sets = [slots, slots.clone()]
    stabs = [stable, tide.slot_table(plan, sets[1])]
    sa, sb = streams
    cur = torch.cuda.current_stream()

    def run_buckets(pipelined):
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        if not pipelined:
            for k in range(buckets):
                Rk = k % N
                tide.pack(plan, tables[Rk], sets[k % 2][Rk])
                tide.rs_slots(plan, Rk, stabs[k % 2], out[Rk])
        else:
            sa.wait_stream(cur)
            sb.wait_stream(cur)
            packed = [torch.cuda.Event() for _ in range(buckets)]
            reduced = [torch.cuda.Event() for _ in range(buckets)]
            for k in range(buckets):
                Rk = k % N
                with torch.cuda.stream(sa):
                    if k >= 2:
                        sa.wait_event(reduced[k - 2])   # its slot set is read by bucket k-2
                    tide.pack(plan, tables[Rk], sets[k % 2][Rk], stream=sa)
                    packed[k].record(sa)
                with torch.cuda.stream(sb):
                    sb.wait_event(packed[k])
                    tide.rs_slots(plan, Rk, stabs[k % 2], out[Rk], stream=sb)
                    reduced[k].record(sb)
            cur.wait_stream(sa)
            cur.wait_stream(sb)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    run_buckets(False)
    run_buckets(True)
    seq = statistics.median(run_buckets(False) for _ in range(3))
    pipe = statistics.median(run_buckets(True) for _ in range(3))
    nbytes = buckets * (b1 + step.b_rs)
    pipeline = {
        "buckets": buckets,
        "bytes_per_bucket": b1 + step.b_rs,
        "sequential_ms": seq,
        "pipelined_ms": pipe,
        "sequential_GBps": nbytes / (seq * 1e-3) / 1e9,
        "pipelined_GBps": nbytes / (pipe * 1e-3) / 1e9,
    }
    log(f"two-stage pipeline over {buckets} buckets: sequential {seq:.2f} ms "
        f"({pipeline['sequential_GBps']:.0f} GB/s), pipelined {pipe:.2f} ms "
        f"({pipeline['pipelined_GBps']:.0f} GB/s)")
    del slots, stable, tables, sets, stabs
    return {"stage1_pack": st1, "stage2_rs_slots": st2, "total_us": t,
            "rs_effective_GBps": step.b_rs / (t * 1e-6) / 1e9,
            "peak_memory": mem, "pipeline": pipeline,
            "pipelined_GBps": pipeline["pipelined_GBps"],
            "peak_bytes_separate": mem["peak_bytes_separate"],
            "peak_bytes_slot_reuse": mem["peak_bytes_slot_reuse"]}


def _rmsnorm(x, w, eps=1e-5):
    xf = x.float()
    return (xf * torch.rsqrt(xf.square().mean(-1, keepdim=True) + eps)).to(x.dtype) * w


def _attention(q, k, v):
    """Causal attention of q [1, H, T, hd] over k, v [1, H, T, hd] through
    PyTorch's fused SDPA kernels only (memory-efficient, else flash): the
    unfused math path, which runs batched bf16 products, is never allowed."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    try:
        with sdpa_kernel([SDPBackend.EFFICIENT_ATTENTION]):
            return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    except RuntimeError:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)


def decoder_layer_fwd_bwd(p, x, n_heads, n_kv):
    """Forward and backward of one Llama-shaped decoder layer on one
    micro-batch x [T, D] with bf16 weights p = (q, k, v, o, gate, up, down,
    norm1, norm2): RMSNorm, q/k/v projections, causal attention (fused SDPA
    with each k/v head shared by a group of query heads), output projection,
    RMSNorm, SwiGLU MLP, residuals.  Rotary embeddings are left out (they
    move no weights and add only elementwise work)."""
    q_w, k_w, v_w, o_w, g_w, u_w, d_w, n1, n2 = p
    T = x.shape[0]
    hd = q_w.shape[0] // n_heads
    grp = n_heads // n_kv
    h = _rmsnorm(x, n1)
    q = torch.nn.functional.linear(h, q_w).view(T, n_heads, hd).transpose(0, 1).unsqueeze(0)
    k = torch.nn.functional.linear(h, k_w).view(T, n_kv, hd).transpose(0, 1).unsqueeze(0)
    v = torch.nn.functional.linear(h, v_w).view(T, n_kv, hd).transpose(0, 1).unsqueeze(0)
    k = k.repeat_interleave(grp, dim=1)
    v = v.repeat_interleave(grp, dim=1)
    a = _attention(q, k, v).squeeze(0).transpose(0, 1).reshape(T, q_w.shape[0])
    x1 = x + torch.nn.functional.linear(a, o_w)
    h2 = _rmsnorm(x1, n2)
    m = torch.nn.functional.silu(torch.nn.functional.linear(h2, g_w)) * \
        torch.nn.functional.linear(h2, u_w)
    y = x1 + torch.nn.functional.linear(m, d_w)
    y.float().square().mean().backward()


def layer_inputs(w, tokens, seed=77):
    """Random bf16 weights of the workload's dense decoder layer (requires
    grad) and one micro-batch x [tokens, D]; None for other workloads."""
    if len(w.shapes) != 9:
        return None
    D = w.shapes[0][1]
    gen = torch.Generator(device="cuda").manual_seed(seed)
    params = [(torch.randn(s, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
              .requires_grad_() for s in w.shapes]
    x = torch.randn(tokens, D, generator=gen, device="cuda").to(torch.bfloat16)
    return params, x, w.shapes[0][0] // 128, w.shapes[1][0] // 128


def layout_conversion_leg(step, tokens=8192, reps=3):
    """One GPU's share of a data-parallel step of the workload's decoder layer
    (8K tokens per GPU, as in the pages' 70B runs): forward and backward of
    one micro-batch, then this rank's tide_rs and tide_ag through the
    torch.ops.tide custom operators.  Beside it, the layout copies TIDE
    removes, timed as FSDP2 makes them with torch ops: the gradient pack
    (per-parameter bf16 -> padded rank-major fp32 buffer) and the all-gather
    copy-out (rank-major bf16 buffer -> per-parameter tensors).  Their share
    of the step is the analogue of the pages' 6.4%."""
    import parameter_layout_collectives_amd.torch_ops as tops

    w, plan, N, S = step.w, step.plan, step.w.world, step.plan.S
    li = layer_inputs(w, tokens)
    if li is None:
        return None                       # dense decoder layers only
    params, x, n_heads, n_kv = li
    segs = [(plan.param(i)[0], plan.param(i)[2]) for i in range(plan.P)]
    pid = tops.register_plan(plan)
    grads_flat = [t for rank in step.grads for t in rank]

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

    def tide_rs_op():
        torch.ops.tide.rs(pid, 0, grads_flat, step.blocks[0], False, False)

    def tide_ag_op():
        torch.ops.tide.ag(pid, step.gathered, step.params, False, False)

    fwd_bwd()
    torch.cuda.synchronize()
    assert all(t.grad is not None for t in params)
    res = {}
    for name, fn in (("fwd_bwd", fwd_bwd), ("stock_grad_pack", stock_pack),
                     ("stock_copy_out", stock_copy_out),
                     ("tide_rs", tide_rs_op), ("tide_ag", tide_ag_op)):
        fn()
        ev = timed_events(reps)
        torch.cuda.synchronize()
        for k in range(reps):
            ev[k][0].record()
            fn()
            ev[k][1].record()
        torch.cuda.synchronize()
        res[name + "_ms"] = statistics.median(a.elapsed_time(b) for a, b in ev)
    tops.unregister_plan(pid)
    copies = res["stock_grad_pack_ms"] + res["stock_copy_out_ms"]
    stock_step = res["fwd_bwd_ms"] + copies
    res.update({
        "tokens": tokens,
        "attention_core": "sdpa",
        "attention_detail": "causal torch scaled_dot_product_attention (fused memory-efficient "
                            "kernel, flash as fallback), k/v heads expanded to the query heads",
        "tide_calls": "torch.ops.tide.rs / torch.ops.tide.ag",
        "stock_layout_copies_ms": copies,
        "stock_layout_share_pct": 100.0 * copies / stock_step,
        "tide_layout_copies_ms": 0.0,
        "tide_local_collective_share_pct":
            100.0 * (res["tide_rs_ms"] + res["tide_ag_ms"]) /
            (res["fwd_bwd_ms"] + res["tide_rs_ms"] + res["tide_ag_ms"]),
        "pages_figure_pct": 6.4,
    })
    log(f"layout conversion: fwd+bwd {res['fwd_bwd_ms']:.2f} ms, stock copies {copies:.2f} ms "
        f"({res['stock_layout_share_pct']:.1f}% of the step), tide rs+ag "
        f"{res['tide_rs_ms'] + res['tide_ag_ms']:.2f} ms")
    del params, x
    return res


def fit_fixed_cost(*points):
    """Least-squares line t = t0 + B / r through two or more (bytes,
    microseconds) points: (t0 in us, r in GB/s)."""
    n = len(points)
    mb = sum(b for b, _ in points) / n
    mt = sum(t for _, t in points) / n
    slope = sum((b - mb) * (t - mt) for b, t in points) / sum((b - mb) ** 2 for b, _ in points)
    return mt - slope * mb, 1.0 / slope / 1e3


def fit_leg(w, repeats=(1, 2, 4), reps=40, warmup=3):
    """Per-launch fixed cost and in-kernel rate of tide_rs and tide_ag on the
    workload's shapes: each call is timed on a bucket of K copies of the
    layer (K in `repeats`, separate gradients and buffers for every copy, so
    nothing is re-read from a cache), and the least-squares line
    t = t0 + B / r is fitted through the (B, t) points; the residuals show
    how far the points are from one line."""
    res = {"workload": w.name, "repeats": list(repeats)}
    pts = {"tide_rs": [], "tide_ag": []}
    for K in repeats:
        wk = dataclasses.replace(w, name=f"{w.name}_x{K}",
                                 params=[(f"{n}#{k}", s) for k in range(K) for n, s in w.params])
        grads = workloads.all_grads(wk, device="cuda")
        plan = tide.Plan(wk.shapes, wk.world)
        table = tide.grad_table(plan, grads)
        N = wk.world
        out = torch.empty(N, plan.S, dtype=torch.float32, device="cuda")
        gathered = workloads.random_bf16(N * plan.S, seed=4242, sigma=w.sigma, device="cuda")
        params = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in wk.shapes]
        agt = tide.ag_tables(plan, gathered, params)
        for name, fn, nbytes in (
                ("tide_rs", lambda k: tide.rs(plan, k % N, table, out[k % N]),
                 rs_bytes_mean(plan)),
                ("tide_ag", lambda k: tide.ag(plan, None, None, tables=agt), ag_bytes(plan))):
            for k in range(warmup):
                fn(k)
            ev = timed_events(reps)
            torch.cuda.synchronize()
            for k in range(reps):
                ev[k][0].record()
                fn(k)
                ev[k][1].record()
            torch.cuda.synchronize()
            t = statistics.fmean(a.elapsed_time(b) for a, b in ev) * 1e3   # us
            pts[name].append((nbytes, t))
            log(f"fit: {name} x{K}: {nbytes / 1e9:.3f} GB in {t:.1f} us "
                f"({nbytes / t / 1e3:.0f} GB/s)")
        del grads, table, out, gathered, params, agt
        gc.collect()
        torch.cuda.empty_cache()
    for name, p in pts.items():
        (b1, t1) = p[0]
        t0, r = fit_fixed_cost(*p)
        resid = [t - (t0 + b / (r * 1e3)) for b, t in p]
        res[name] = {"points_bytes_us": p, "fixed_us": t0, "in_kernel_GBps": r,
                     "in_kernel_pct_of_peak": 100.0 * r / HBM_PEAK_GBPS,
                     "residuals_us": resid, "single_GBps": b1 / t1 / 1e3}
        log(f"fit: {name}: fixed cost {t0:.1f} us per launch, in-kernel {r:.0f} GB/s "
            f"({100 * r / HBM_PEAK_GBPS:.1f}% of peak), residuals "
            f"{', '.join(f'{x:+.1f}' for x in resid)} us")
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
# co-run: a compute job on one stream, the collectives on another
# ---------------------------------------------------------------------------
#
# The overlap page ("分析通信重叠", stream overlap and trace analysis) splits
# a step into compute plus the communication time that compute does not
# hide: T_step = T_compute + T_exposed.  Two experiments per collective and
# launch mode measure that directly:
#   progress  - the partner runs `reps` units (after two untimed ones)
#               while a chain of collective calls, each with its own event
#               pair, runs on the other stream; both start behind one gate
#               and the chain is sized to outlast the partner.  The
#               bytes the collective completes inside the partner's window
#               (each call's bytes pro-rated by the share of its time spent
#               inside) over that window give its rate beside the partner;
#               the partner's units that ran wholly inside the chain give
#               its slowdown.
#   makespan  - a fixed partner chain (`reps` units) and a fixed number of
#               collective calls (fixed_calls: the same bytes for every
#               launch mode) start together behind one gate.  exposed =
#               makespan - partner chain alone; serial = partner alone +
#               collective alone; saving = serial - makespan.

def bytes_in_window(calls, nbytes, lo, hi):
    """Bytes a chain of calls moved inside [lo, hi] (ms): each call's
    `nbytes` pro-rated by the share of its [start, end] inside the window."""
    total = 0.0
    for s, e in calls:
        if e <= s:
            continue
        ov = min(e, hi) - max(s, lo)
        if ov > 0:
            total += nbytes * ov / (e - s)
    return total


class Partner:
    """A compute job that the collectives run beside, on its own stream;
    run() enqueues one unit of it on the current stream.  Every co-run leg
    uses the same two streams, created once: the process has few hardware
    queues, and a stream created later can share the partner's queue, which
    would serialise the two instead of running them together."""

    def __init__(self, name, unit, reps, streams, flop=None, kind="gemm"):
        self.name, self.unit, self.reps, self.flop, self.kind = name, unit, reps, flop, kind
        self.stream, self.side = streams
        torch.cuda.synchronize()
        ev = timed_events(reps)
        with torch.cuda.stream(self.stream):
            for _ in range(3):
                self.run()
            for s, e in ev:
                s.record()
                self.run()
                e.record()
        torch.cuda.synchronize()
        self.alone_ms = statistics.median(s.elapsed_time(e) for s, e in ev)

    def run(self):
        self.unit()

    def describe(self):
        d = {"partner": self.name, "partner_alone_ms": self.alone_ms, "partner_units": self.reps}
        if self.flop:
            d["partner_tflops_alone"] = self.flop / (self.alone_ms * 1e-3) / 1e12
        return d


def gemm_partner(shape, streams, reps=30):
    """bf16 M x K x N torch.matmul (hipBLASLt), the single-wave GEMM case."""
    M, K, Nn = shape
    g = torch.Generator(device="cuda").manual_seed(77)
    A = torch.randn(M, K, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    B = torch.randn(K, Nn, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    C = torch.empty(M, Nn, dtype=torch.bfloat16, device="cuda")
    return Partner(f"bf16 {M}x{K}x{Nn} torch.matmul", lambda: torch.matmul(A, B, out=C), reps,
                   streams, flop=2.0 * M * K * Nn)


def layer_partner(w, streams, tokens=8192, reps=4):
    """Forward + backward of the workload's decoder layer on one 8K-token
    micro-batch (its own GEMMs, fused attention and elementwise kernels)."""
    li = layer_inputs(w, tokens, seed=78)
    if li is None:
        return None
    params, x, n_heads, n_kv = li

    def unit():
        for t in params:
            t.grad = None
        decoder_layer_fwd_bwd(params, x, n_heads, n_kv)

    flop = 6.0 * tokens * w.psi
    return Partner(f"{w.name} decoder layer forward+backward, {tokens} tokens", unit, reps,
                   streams, flop=flop, kind="layer")


_GATE_CYCLES = None


def gate():
    """Holds the current stream long enough (~25 ms) for the work enqueued
    behind it on other streams to be queued before any of it starts."""
    global _GATE_CYCLES
    if _GATE_CYCLES is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(10_000_000)
        b.record()
        torch.cuda.synchronize()
        _GATE_CYCLES = int(10_000_000 * 25.0 / max(a.elapsed_time(b), 1e-3))
    torch.cuda._sleep(_GATE_CYCLES)


def collective_alone(partner, launch, nbytes, reps=8):
    sb = partner.side
    ev = timed_events(reps)
    with torch.cuda.stream(sb):
        for k in range(2):
            launch(k, sb)
        for k, (s, e) in enumerate(ev):
            s.record()
            launch(k, sb)
            e.record()
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) for s, e in ev)


def corun_progress(partner, launch, nbytes, t_alone, repeats=3):
    """The progress experiment (see above); one dict per repeat."""
    sb, cur = partner.side, torch.cuda.current_stream()
    runs = []
    for _ in range(repeats):
        n = int(2.0 * (partner.reps + 2) * partner.alone_ms / t_alone) + 4
        base = torch.cuda.Event(enable_timing=True)
        cev, pev = timed_events(n), timed_events(partner.reps)
        torch.cuda.synchronize()
        # Both streams start behind one gate.  The partner is enqueued first:
        # copy-engine calls block the host while they are queued, and the
        # partner must not wait for that.  Its two untimed units give the
        # chain time to get going before the timed ones.
        gate()
        base.record()
        sb.wait_stream(cur)
        partner.stream.wait_stream(cur)
        with torch.cuda.stream(partner.stream):
            for _ in range(2):
                partner.run()
            for s, e in pev:
                s.record()
                partner.run()
                e.record()
        with torch.cuda.stream(sb):
            for k, (s, e) in enumerate(cev):
                s.record()
                launch(k, sb)
                e.record()
        torch.cuda.synchronize()
        calls = [(base.elapsed_time(s), base.elapsed_time(e)) for s, e in cev]
        units = [(base.elapsed_time(s), base.elapsed_time(e)) for s, e in pev]
        c0, c1 = calls[0][0], calls[-1][1]
        g0, g1 = units[0][0], units[-1][1]
        inside = [e - s for s, e in units if s >= c0 and e <= c1]
        lo, hi = max(g0, c0), min(g1, c1)
        moved = bytes_in_window(calls, nbytes, lo, hi) if hi > lo else 0.0
        med = statistics.median(inside) if len(inside) >= max(1, partner.reps // 2) else None
        runs.append({
            "partner_unit_corun_ms": med,
            "units_inside_chain": len(inside),
            "partner_slowdown_pct": None if med is None else 100.0 * (med / partner.alone_ms - 1),
            "during_partner_GBps": moved / ((hi - lo) * 1e-3) / 1e9 if hi > lo else None,
            "partner_window_covered": c0 <= g0 and c1 >= g1,
            "calls": n,
            "chain_ms": [c0, c1],
            "partner_ms": [g0, g1],
            "calls_completed_in_partner_window": sum(1 for s, e in calls if s >= g0 and e <= g1),
        })
    return runs


def corun_makespan(partner, launch, nbytes, n, repeats=3):
    """The makespan experiment (see above) with `n` collective calls: partner
    chain alone, collective chain alone, both together behind one gate;
    medians over `repeats`."""
    sb, cur = partner.side, torch.cuda.current_stream()

    def timed(do_partner, do_coll):
        torch.cuda.synchronize()
        gate()
        t0 = torch.cuda.Event(enable_timing=True)
        t0.record()
        ep = ec = None
        cev = timed_events(n) if do_coll else []
        if do_partner:
            partner.stream.wait_stream(cur)
            with torch.cuda.stream(partner.stream):
                for _ in range(partner.reps):
                    partner.run()
                ep = torch.cuda.Event(enable_timing=True)
                ep.record()
        if do_coll:
            sb.wait_stream(cur)
            with torch.cuda.stream(sb):
                for k, (s, e) in enumerate(cev):
                    s.record()
                    launch(k, sb)
                    e.record()
                ec = torch.cuda.Event(enable_timing=True)
                ec.record()
        torch.cuda.synchronize()
        calls = [(t0.elapsed_time(s), t0.elapsed_time(e)) for s, e in cev]
        return (None if ep is None else t0.elapsed_time(ep),
                None if ec is None else t0.elapsed_time(ec), calls)

    rows = []
    for _ in range(repeats):
        tp = timed(True, False)[0]
        tc = timed(False, True)[1]
        tpb, tcb, calls = timed(True, True)
        makespan = max(tpb, tcb)
        rows.append({
            "partner_chain_alone_ms": tp, "collective_chain_alone_ms": tc,
            "serial_ms": tp + tc, "makespan_ms": makespan, "exposed_ms": makespan - tp,
            "overlap_saving_ms": tp + tc - makespan,
            "partner_chain_together_ms": tpb, "collective_chain_together_ms": tcb,
            "during_partner_GBps_same_run":
                bytes_in_window(calls, nbytes, 0.0, tpb) / (tpb * 1e-3) / 1e9,
        })
    med = {k: statistics.median(r[k] for r in rows) for k in rows[0]}
    med.update({"collective_calls": n, "collective_bytes": n * nbytes,
                "hidden_pct": 100.0 * med["overlap_saving_ms"] / med["collective_chain_alone_ms"],
                "partner_slowdown_in_makespan_pct":
                    100.0 * (med["partner_chain_together_ms"] / med["partner_chain_alone_ms"] - 1),
                "runs": rows})
    return med


def fixed_calls(partner, t_ref):
    """The collective work of the makespan experiment, the same for every
    launch mode of one collective: beside a GEMM, calls whose time alone in
    the default launch (t_ref ms) is half the GEMM chain's; beside the layer
    step, one call per forward+backward (one layer's share of a step)."""
    if partner.kind == "layer":
        return partner.reps
    return max(1, int(round(0.5 * partner.reps * partner.alone_ms / t_ref)))


def corun_leg(partner, launch, nbytes, label, n_calls=None, t_alone=None):
    """Both experiments for one collective and launch mode beside `partner`;
    the makespan experiment runs `n_calls` calls (default: fixed_calls from
    this mode's own time alone)."""
    if t_alone is None:
        t_alone = collective_alone(partner, launch, nbytes)
    prog = corun_progress(partner, launch, nbytes, t_alone)
    if n_calls is None:
        n_calls = fixed_calls(partner, t_alone)
    mk = corun_makespan(partner, launch, nbytes, n_calls)
    slow = [r["partner_slowdown_pct"] for r in prog if r["partner_slowdown_pct"] is not None]
    during = [r["during_partner_GBps"] for r in prog if r["during_partner_GBps"] is not None]
    alone_gbps = nbytes / (t_alone * 1e-3) / 1e9
    res = {
        "alone_us": t_alone * 1e3,
        "alone_GBps": alone_gbps,
        "partner_slowdown_pct": statistics.median(slow) if slow else None,
        "during_partner_GBps": statistics.median(during) if during else None,
        "progress_share_of_alone": (statistics.median(during) / alone_gbps) if during else None,
        "serial_ms": mk["serial_ms"],
        "makespan_ms": mk["makespan_ms"],
        "exposed_ms": mk["exposed_ms"],
        "overlap_saving_ms": mk["overlap_saving_ms"],
        "hidden_pct": mk["hidden_pct"],
        "makespan_collective_bytes": mk["collective_bytes"],
        "partner_slowdown_in_makespan_pct": mk["partner_slowdown_in_makespan_pct"],
        "progress_runs": prog,
        "makespan": mk,
    }
    log(f"co-run {label}: partner slowdown {fmt(res['partner_slowdown_pct'])}%, "
        f"{fmt(res['during_partner_GBps'])} GB/s during the partner "
        f"({fmt(res['alone_GBps'])} alone); {n_calls} calls: serial {mk['serial_ms']:.2f} ms, "
        f"makespan {mk['makespan_ms']:.2f} ms, exposed {mk['exposed_ms']:.2f} ms "
        f"({mk['hidden_pct']:.0f}% of the collective hidden)")
    return res


CORUN_METHOD = (
    "progress: the partner's units run while a longer chain of collective calls (an event pair "
    "per call) runs on the other stream; during_partner_GBps = bytes completed inside the "
    "partner's window (calls pro-rated by their share inside) / that window; slowdown = median "
    "unit time inside the chain / median unit time alone - 1 (median of 3 runs). makespan: a "
    "fixed partner chain and a fixed number of collective calls, the same for every launch mode "
    "(beside a GEMM: calls whose default-launch time alone is half the GEMM chain's; beside the "
    "layer step: one call per forward+backward), start together behind one gate; exposed = "
    "makespan - partner chain alone, serial = sum of the two alone, saving = serial - makespan "
    "(median of 3 runs)")


def _with_keys(partner_kind, leg):
    """Names the partner in the rate key: during_gemm_GBps beside a GEMM,
    during_step_GBps beside the layer step."""
    key = "during_gemm_GBps" if partner_kind == "gemm" else "during_step_GBps"
    slow = "gemm_slowdown_pct" if partner_kind == "gemm" else "step_slowdown_pct"
    leg[key] = leg["during_partner_GBps"]
    leg[slow] = leg["partner_slowdown_pct"]
    return leg


def corun_modes(grids, copy_engine):
    """(name, launch keywords) of the co-run launch modes: default, small
    footprint, small footprint on a persistent grid of g workgroups for each
    g in `grids` (max_workgroups = g: each workgroup loops over tiles), and
    the copy engines (tide_ag)."""
    modes = [("default", {}), ("small_footprint", {"small": True})]
    modes += [(f"small_footprint_wg{g}", {"small": True, "max_workgroups": g}) for g in grids]
    if copy_engine:
        modes.append(("copy_engine", {"copy_engine": True}))
    return modes


def corun_rs(partner, kind, w=None, step=None, grids=()):
    """tide_rs beside `partner` in each launch mode of corun_modes, on the
    step's resident workload or on workload `w` (generated here)."""
    if step is not None:
        plan, table, out, N, name = step.plan, step.table, step.blocks, step.w.world, step.w.name
        b_rs = step.b_rs
    else:
        N, name = w.world, w.name
        log(f"co-run: generating {name} ({N} ranks) beside {partner.name}")
        grads = workloads.all_grads(w, device="cuda")
        plan = tide.Plan(w.shapes, N)
        table = tide.grad_table(plan, grads)
        out = torch.empty(N, plan.S, dtype=torch.float32, device="cuda")
        b_rs = rs_bytes_mean(plan)
    res = dict(partner.describe(), workload=name, world=N, bytes_per_call=b_rs,
               method=CORUN_METHOD)
    n_calls = None
    for key, kw in corun_modes(grids, copy_engine=False):

        def launch(k, st, kw=kw):
            tide.rs(plan, k % N, table, out[k % N], stream=st, **kw)

        t_alone = collective_alone(partner, launch, b_rs)
        if n_calls is None:   # the default launch's time sets the work for every mode
            n_calls = fixed_calls(partner, t_alone)
        res[key] = _with_keys(kind, corun_leg(partner, launch, b_rs,
                                              f"tide_rs {name} {key} beside {partner.name}",
                                              n_calls=n_calls, t_alone=t_alone))
    if step is None:
        del grads, table, out
    return res


def corun_ag(partner, kind, step, grids=()):
    """tide_ag beside `partner` in each launch mode of corun_modes, the SDMA
    copy engines included."""
    res = dict(partner.describe(), workload=step.w.name, world=step.w.world,
               bytes_per_call=step.b_ag, method=CORUN_METHOD)
    n_calls = None
    for key, kw in corun_modes(grids, copy_engine=True):

        def launch(k, st, kw=kw):
            tide.ag(step.plan, None, None, stream=st, tables=step.agt, **kw)

        t_alone = collective_alone(partner, launch, step.b_ag)
        if n_calls is None:
            n_calls = fixed_calls(partner, t_alone)
        res[key] = _with_keys(kind, corun_leg(
            partner, launch, step.b_ag, f"tide_ag {step.w.name} {key} beside {partner.name}",
            n_calls=n_calls, t_alone=t_alone))
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
    trs, tag = statistics.median(t_rs), statistics.median(t_ag)
    log(f"cpu baseline over {len(t_rs)} reps: rs min/median/max {min(t_rs):.3f}/{trs:.3f}/"
        f"{max(t_rs):.3f} s, ag {min(t_ag):.3f}/{tag:.3f}/{max(t_ag):.3f} s; per rep rs "
        + " ".join(f"{x:.3f}" for x in t_rs) + "; ag " + " ".join(f"{x:.3f}" for x in t_ag))
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
        "rs_s_min_median_max": [min(t_rs), trs, max(t_rs)],
        "ag_s_min_median_max": [min(t_ag), tag, max(t_ag)],
        "reps": len(t_rs),
        "tiny_step_us_1_thread": statistics.median(t_tiny) * 1e6,
        "cpu_model": cpu,
    }


# ---------------------------------------------------------------------------

LEGS = ("variants", "small_alone", "tiny", "two_stage", "layout", "copy", "cpu", "corun_gemm",
        "corun_layer", "corun_n64", "partner_gemm", "fit")


def corun_summary(results):
    """One row per (collective, workload, partner, mode) of the co-run legs."""
    rows = []
    for coll, res in results:
        if not res:
            continue
        for mode, leg in res.items():
            if not isinstance(leg, dict) or "exposed_ms" not in leg:
                continue
            rows.append({
                "collective": coll, "workload": res["workload"], "partner": res["partner"],
                "mode": mode,
                "partner_slowdown_pct": leg["partner_slowdown_pct"],
                "during_partner_GBps": leg["during_partner_GBps"],
                "alone_GBps": leg["alone_GBps"],
                "progress_share_of_alone": leg["progress_share_of_alone"],
                "serial_ms": leg["serial_ms"], "makespan_ms": leg["makespan_ms"],
                "exposed_ms": leg["exposed_ms"], "hidden_pct": leg["hidden_pct"],
                "makespan_collective_bytes": leg.get("makespan_collective_bytes"),
                "partner_slowdown_in_makespan_pct": leg.get("partner_slowdown_in_makespan_pct"),
            })
    return rows


def compact(obj):
    """The bench line without the per-repeat lists of the co-run experiments
    (their medians stay); --detail FILE keeps everything."""
    if isinstance(obj, dict):
        return {k: compact(v) for k, v in obj.items() if k not in ("progress_runs", "runs")}
    if isinstance(obj, list):
        return [compact(v) for v in obj]
    return obj


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
                    help="skip the tide_rs flag variants (bf16 shard, mean), the small-footprint "
                         "alone timing, the tiny workload, the two-stage reduce-scatter and the "
                         "layout-conversion leg")
    ap.add_argument("--detail", default="",
                    help="also write the full result, per-repeat co-run figures included, to "
                         "this JSON file")
    ap.add_argument("--corun-grids", default="128",
                    help="comma-separated persistent grid sizes (max_workgroups) for extra "
                         "small-footprint co-run modes, or 'none'")
    ap.add_argument("--legs", default="all",
                    help="comma-separated subset of the sections after the step: "
                         + ",".join(LEGS) + "; 'all' (the default) is every one but fit; "
                         "'none' runs the step only")
    args = ap.parse_args()
    grids = () if args.corun_grids == "none" else tuple(
        int(g) for g in args.corun_grids.split(",") if g)
    legs = set(LEGS) - {"fit"} if args.legs == "all" else \
        set() if args.legs == "none" else set(args.legs.split(","))
    unknown = legs - set(LEGS)
    if unknown:
        ap.error(f"--legs: unknown {sorted(unknown)}; choose from {','.join(LEGS)}")
    if args.no_variants:
        legs -= {"variants", "small_alone", "tiny", "two_stage", "layout"}
    if args.no_cpu:
        legs.discard("cpu")
    if args.no_copy:
        legs.discard("copy")
    if args.corun == "none":
        legs -= {"corun_gemm", "corun_layer", "corun_n64", "partner_gemm"}

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

    streams = (torch.cuda.Stream(), torch.cuda.Stream())   # every two-stream leg uses these
    variants = rs_variants(step) if "variants" in legs else None
    small_alone = small_footprint_alone(step) if "small_alone" in legs else None
    tiny = tiny_latency() if "tiny" in legs else None
    two_stage = two_stage_leg(step, streams) if "two_stage" in legs else None
    layout = layout_conversion_leg(step) if "layout" in legs else None
    copy_gbps, copy_lib_gbps = copy_ceiling(library=not args.no_lib_copy) if "copy" in legs \
        else (None, None)
    if copy_gbps:
        log(f"copy ceiling {copy_gbps:.1f} GB/s (torch), {fmt(copy_lib_gbps)} GB/s (library)")
    cpu = cpu_baseline(step) if "cpu" in legs else None
    fit = None
    corun_res = corun_ag_res = corun_rs_step_res = corun_layer_res = None
    gemm = None
    cw = workloads.WORKLOADS[args.corun] if args.corun != "none" else None
    if legs & {"corun_gemm", "corun_n64"}:
        gemm = gemm_partner(cw.corun_gemm or (8192, 8192, 8192), streams)
        log(f"partner: {gemm.name}, {gemm.alone_ms:.3f} ms alone")
    if "corun_gemm" in legs:
        corun_ag_res = corun_ag(gemm, "gemm", step, grids)
        corun_rs_step_res = corun_rs(gemm, "gemm", step=step, grids=grids)
    if "corun_layer" in legs:
        layer = layer_partner(step.w, streams)
        if layer is not None:
            log(f"partner: {layer.name}, {layer.alone_ms:.2f} ms alone")
            corun_layer_res = {"tide_rs": corun_rs(layer, "layer", step=step, grids=grids),
                               "tide_ag": corun_ag(layer, "layer", step, grids)}
            del layer
    if "partner_gemm" in legs and gemm is None:
        gemm = gemm_partner(cw.corun_gemm or (8192, 8192, 8192), streams)
        log(f"partner: {gemm.name}, {gemm.alone_ms:.3f} ms alone")
    P, S = step.plan.P, step.plan.S
    del step
    gc.collect()
    torch.cuda.empty_cache()
    if "corun_n64" in legs:
        corun_res = corun_rs(gemm, "gemm", w=cw, grids=grids)
        gc.collect()
        torch.cuda.empty_cache()
    if "fit" in legs:
        fit = fit_leg(w)
    summary = corun_summary([("tide_rs", corun_res), ("tide_ag", corun_ag_res),
                             ("tide_rs", corun_rs_step_res)] +
                            ([("tide_rs", corun_layer_res["tide_rs"]),
                              ("tide_ag", corun_layer_res["tide_ag"])] if corun_layer_res
                             else []))

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
        "corun_layer_step": corun_layer_res,
        "corun_summary": summary,
        "corun_partner_gemm": gemm.describe() if gemm is not None else None,
        "fixed_cost_fit": fit,
        "gemm_slowdown_pct": None if not corun_res else {
            k: corun_res[k]["gemm_slowdown_pct"] for k in ("default", "small_footprint")
            if k in corun_res},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "pages_context": PAGES_CONTEXT,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if args.lib:
        line["library"] = args.lib
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(line, f)
    print(json.dumps(compact(line)), flush=True)


if __name__ == "__main__":
    main()
