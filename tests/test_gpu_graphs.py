"""The collectives captured into a HIP graph (torch.cuda.graph) and replayed.

One step (tide_rs for every rank in both launch modes, tide_ag as a kernel
and on the copy engines, tide_pack and tide_rs_slots) is captured once and
replayed three times.  Between
replays the program does eager work of its own (new gradient and gathered
values written in place, outputs refilled) and synchronises; every replay
is checked against the oracle.  A pointer set the plan has not cached is
refused inside a capture without enqueueing anything.
"""
import numpy as np
import pytest
import torch

import parameter_layout_collectives_amd as tide
import workloads
from gpu_helpers import BF16_SENTINEL, F32_SENTINEL, bits16, expected_rs, note, same_f32

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")   # the refused capture
def test_step_captured_and_replayed(orc):
    shapes = [(37, 5), (4100,), (3, 3), (9000,)]
    N = 4
    plan = tide.Plan(shapes, N)
    S = plan.S
    grads = [[t.to(DEV) for t in rank]
             for rank in workloads.random_grads_for_shapes(shapes, N, seed_base=41)]
    table = tide.grad_table(plan, grads)
    out = torch.empty(N, S, dtype=torch.float32, device=DEV)
    out_small = torch.empty(N, S, dtype=torch.float32, device=DEV)
    gathered = torch.empty(N * S, dtype=torch.bfloat16, device=DEV)
    params = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    agt = tide.ag_tables(plan, gathered, params)
    params_ce = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    agt_ce = tide.ag_tables(plan, gathered, params_ce)
    slots = torch.empty(N, N * S, dtype=torch.bfloat16, device=DEV)
    stable = tide.slot_table(plan, slots)
    ptabs = [tide.PointerTable(grads[r], torch.bfloat16) for r in range(N)]
    out_slots = torch.empty(S, dtype=torch.float32, device=DEV)

    def step():
        for R in range(N):
            tide.rs(plan, R, table, out[R])
            tide.rs(plan, R, table, out_small[R], small=True)
        tide.ag(plan, None, None, tables=agt)
        tide.ag(plan, None, None, tables=agt_ce, copy_engine=True)
        for r in range(N):
            tide.pack(plan, ptabs[r], slots[r])
        tide.rs_slots(plan, 2, stable, out_slots)

    note("graph: eager warm-up")
    for _ in range(2):
        step()
        torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph: capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    for rep in range(3):
        # eager work of the program between replays
        for rank in grads:
            for t in rank:
                t.copy_(torch.from_numpy(rng.standard_normal(t.numel()).astype(np.float32))
                        .to(torch.bfloat16).view(t.shape))
        gathered.copy_(torch.from_numpy(rng.standard_normal(N * S).astype(np.float32))
                       .to(torch.bfloat16))
        out.view(torch.int32).fill_(F32_SENTINEL)
        out_small.view(torch.int32).fill_(F32_SENTINEL)
        out_slots.view(torch.int32).fill_(F32_SENTINEL)
        for p in params + params_ce:
            p.view(torch.int16).fill_(BF16_SENTINEL)
        torch.cuda.synchronize()
        note(f"graph: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for R in range(N):
            want = expected_rs(orc, shapes, N, R, grads, plan)
            assert same_f32(out[R].cpu().numpy(), want), (rep, R)
            assert same_f32(out_small[R].cpu().numpy(), want), (rep, R, "small")
            if R == 2:
                assert same_f32(out_slots.cpu().numpy(), want), (rep, "slots")
        host = bits16(gathered)
        want_p = orc.ag(shapes, N, [host[r * S:(r + 1) * S] for r in range(N)])
        for i, p in enumerate(params):
            assert np.array_equal(bits16(p).reshape(-1), want_p[i]), (rep, i)
        for i, p in enumerate(params_ce):
            assert np.array_equal(bits16(p).reshape(-1), want_p[i]), (rep, i, "copy engine")

    # a new pointer set cannot be uploaded inside a capture
    other = [[t.to(DEV) for t in rank]
             for rank in workloads.random_grads_for_shapes(shapes, N, seed_base=99)]
    otable = tide.grad_table(plan, other)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g2):
        try:
            tide.rs(plan, 0, otable, out[0])
        except tide.TideError as e:
            err = e
    assert err is not None and err.status == 2 and "capture" in str(err)
    # outside a capture the same call works
    tide.rs(plan, 0, otable, out[0])
    torch.cuda.synchronize()
    assert same_f32(out[0].cpu().numpy(), expected_rs(orc, shapes, N, 0, other, plan))
    del g, g2
