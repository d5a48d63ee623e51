"""The allocation-free TIDE-RS entry point (tide_rs_noalloc), called through
the C ABI and compared bit for bit with tide_rs on the same inputs.

tide_rs_noalloc keeps its tables in one fixed per-device scratch array that
every call rewrites on its stream, so the cases run back to back on one
stream without a synchronisation in between: a larger plan first (many
parameters, so its tables take several table-writing launches), then a
smaller one, whose tables overwrite the first's while the first call's
results are still to be checked.  The first call's output is also checked
against the CPU oracle for one rank.  Under HIP graph capture, where tide_rs
refuses a pointer set its plan has not uploaded, tide_rs_noalloc captures
such a set (its tables travel as kernel arguments) and every replay equals
the oracle.
"""
import numpy as np
import pytest
import torch

import parameter_layout_collectives_amd as tide
import workloads
from gpu_helpers import F32_SENTINEL, bits16, bits32, expected_rs, note, same_f32

pytestmark = pytest.mark.gpu


def _ragged_shapes(count, seed):
    g = np.random.default_rng(seed)
    shapes = []
    for k in range(count):
        d0 = int(g.integers(1, 300))
        if k % 7 == 3:
            shapes.append((d0,))
        else:
            shapes.append((d0, int(g.integers(1, 700))))
    return shapes


def _sentinel(n, dtype=torch.float32):
    if dtype == torch.float32:
        return torch.full((n,), F32_SENTINEL, dtype=torch.int32, device="cuda").view(torch.float32)
    return torch.full((n,), 0x7FBD, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _same(a, b):
    if a.dtype == torch.float32:
        return np.array_equal(bits32(a), bits32(b))
    return np.array_equal(bits16(a), bits16(b))


CASES = [
    # (name, shapes, N, ranks, kwargs)
    ("ragged 160 params, 12 ranks", _ragged_shapes(160, 5), 12, [0, 5, 11], {}),
    ("ragged 160 params, 12 ranks, small footprint, mean, bf16 out", _ragged_shapes(160, 5), 12,
     [3], {"small": True, "avg": True, "out_bf16": True}),
    ("ragged 40 params, 24 ranks, small footprint", _ragged_shapes(40, 9), 24, [0, 23],
     {"small": True}),
    ("ragged 40 params, 20 ranks (2-rank batches)", _ragged_shapes(40, 11), 20, [0, 19], {}),
    ("tiny, 4 ranks", workloads.WORKLOADS["tiny"].shapes, 4, [0, 1, 2, 3], {}),
    ("ragged 50 params, 8 ranks, fp16 grads, mean (x 1/8), persistent grid of 7",
     _ragged_shapes(50, 13), 8, [0, 7], {"dtype": torch.float16, "avg": True,
                                          "max_workgroups": 7}),
    ("ragged 30 params, 3 ranks, fp32 grads", _ragged_shapes(30, 15), 3, [1],
     {"dtype": torch.float32}),
    ("ragged 30 params, 1 rank", _ragged_shapes(30, 17), 1, [0], {}),
    ("ragged 30 params, 6 ranks, gradients 2 bytes off 16-byte alignment",
     _ragged_shapes(30, 19), 6, [2, 5], {"misalign": True}),
]


def _prepare(grads, dtype, misalign):
    """The cases' gradient variants: another element type (converted from
    the seeded bf16 values), or every tensor one element into a buffer of its
    own, so no gradient pointer is 16-byte aligned."""
    if dtype is not None:
        grads = [[t.to(dtype) for t in rank] for rank in grads]
    if misalign:
        moved = []
        for rank in grads:
            row = []
            for t in rank:
                buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
                v = buf[1:].view(t.shape)
                v.copy_(t)
                assert v.data_ptr() % 16 != 0
                row.append(v)
            moved.append(row)
        grads = moved
    return grads


def test_noalloc_matches_tide_rs_back_to_back(orc):
    torch.manual_seed(0)
    runs = []
    # Every case's inputs and tide_rs reference first, then every
    # tide_rs_noalloc call back to back on the current stream.
    for name, shapes, N, ranks, kw in CASES:
        grads = workloads.random_grads_for_shapes(shapes, N, seed_base=100 + N, device="cuda")
        grads = _prepare(grads, kw.get("dtype"), kw.get("misalign", False))
        plan = tide.Plan(shapes, N)
        table = tide.grad_table(plan, grads)
        odt = torch.bfloat16 if kw.get("out_bf16") else torch.float32
        opts = {k: v for k, v in kw.items() if k not in ("out_bf16", "dtype", "misalign")}
        for R in ranks:
            want = _sentinel(plan.S, odt)
            got = _sentinel(plan.S, odt)
            note(f"tide_rs reference: {name}, rank {R}")
            tide.rs(plan, R, table, want, **opts)
            runs.append((name, shapes, N, R, plan, grads, table, opts, want, got))
    torch.cuda.synchronize()
    for name, shapes, N, R, plan, grads, table, opts, want, got in runs:
        note(f"tide_rs_noalloc: {name}, rank {R}, S={plan.S}")
        tide.rs_noalloc(plan, R, table, got, **opts)
    torch.cuda.synchronize()
    for name, shapes, N, R, plan, grads, table, opts, want, got in runs:
        assert _same(got, want), f"{name}, rank {R}: tide_rs_noalloc differs from tide_rs"
    # the first call also against the oracle (sum, fp32 shard)
    name, shapes, N, R, plan, grads, table, opts, want, got = runs[0]
    exp = expected_rs(orc, shapes, N, R, grads, plan)
    assert np.array_equal(bits32(got), exp.view(np.uint32)), f"{name}: differs from the oracle"


def test_noalloc_repeated_calls_smaller_second():
    """Two calls in a row, the second with a smaller plan: the second call's
    tables overwrite the first's, and both results stay those of tide_rs."""
    w = workloads.WORKLOADS["tiny"]
    shapes_a = _ragged_shapes(60, 21)
    grads_a = workloads.random_grads_for_shapes(shapes_a, 8, seed_base=7, device="cuda")
    grads_b = workloads.all_grads(w, device="cuda")
    plan_a, plan_b = tide.Plan(shapes_a, 8), tide.Plan(w.shapes, w.world)
    ta, tb = tide.grad_table(plan_a, grads_a), tide.grad_table(plan_b, grads_b)
    want_a, want_b = _sentinel(plan_a.S), _sentinel(plan_b.S)
    note("tide_rs references (60 ragged params x 8 ranks; tiny)")
    tide.rs(plan_a, 6, ta, want_a)
    tide.rs(plan_b, 1, tb, want_b)
    torch.cuda.synchronize()
    for rep in range(2):
        got_a, got_b = _sentinel(plan_a.S), _sentinel(plan_b.S)
        note(f"tide_rs_noalloc pair {rep}: 60 params x 8 ranks, then tiny")
        tide.rs_noalloc(plan_a, 6, ta, got_a)
        tide.rs_noalloc(plan_b, 1, tb, got_b)
        torch.cuda.synchronize()
        assert _same(got_a, want_a), f"pair {rep}: the larger call differs from tide_rs"
        assert _same(got_b, want_b), f"pair {rep}: the smaller call differs from tide_rs"


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")   # the refused capture
def test_noalloc_captured_with_a_new_pointer_set(orc):
    """A pointer set tide_rs has never uploaded, captured into a HIP graph
    through tide_rs_noalloc for every rank (default and small footprint) and
    replayed three times, with the program's own eager work between the
    replays; every replay equals the oracle."""
    shapes = [(37, 5), (4100,), (3, 3), (9000,), (129, 33)]
    N = 4
    plan = tide.Plan(shapes, N)
    S = plan.S
    grads = workloads.random_grads_for_shapes(shapes, N, seed_base=61, device="cuda")
    table = tide.grad_table(plan, grads)
    out = torch.empty(N, S, dtype=torch.float32, device="cuda")
    out_small = torch.empty(N, S, dtype=torch.float32, device="cuda")
    # the first call on the device (it looks up the scratch address) runs
    # eagerly, on another plan, before the capture
    warm = tide.Plan([(5, 7)], 2)
    warm_grads = workloads.random_grads_for_shapes([(5, 7)], 2, seed_base=3, device="cuda")
    tide.rs_noalloc(warm, 0, tide.grad_table(warm, warm_grads),
                    torch.empty(warm.S, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()

    # tide_rs cannot take this pointer set inside a capture (its plan would
    # have to upload it)
    g0 = torch.cuda.CUDAGraph()
    err = None
    note("tide_rs: capture refused for a pointer set never uploaded")
    with torch.cuda.graph(g0):
        try:
            tide.rs(plan, 0, table, out[0])
        except tide.TideError as e:
            err = e
    assert err is not None and "capture" in str(err)
    del g0

    g = torch.cuda.CUDAGraph()
    note("tide_rs_noalloc: capture, 5 params x 4 ranks, a pointer set never uploaded")
    with torch.cuda.graph(g):
        for R in range(N):
            tide.rs_noalloc(plan, R, table, out[R])
            tide.rs_noalloc(plan, R, table, out_small[R], small=True)
    torch.cuda.synchronize()

    rng = np.random.default_rng(17)
    for rep in range(3):
        for rank in grads:
            for t in rank:
                t.copy_(torch.from_numpy(rng.standard_normal(t.numel()).astype(np.float32))
                        .to(torch.bfloat16).view(t.shape))
        out.view(torch.int32).fill_(F32_SENTINEL)
        out_small.view(torch.int32).fill_(F32_SENTINEL)
        torch.cuda.synchronize()
        note(f"tide_rs_noalloc: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for R in range(N):
            want = expected_rs(orc, shapes, N, R, grads, plan)
            assert same_f32(out[R].cpu().numpy(), want), (rep, R)
            assert same_f32(out_small[R].cpu().numpy(), want), (rep, R, "small")
    del g
