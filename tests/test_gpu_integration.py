"""The collectives inside a data-parallel step, through the PyTorch
custom operators and the FSDP-unit helper.

* torch.ops.tide.{rs, ag, pack, rs_slots} give the same bits as the plain
  binding, also inside a torch.compile'd step;
* one optimizer step of a TideUnit (shard, reduce-scatter the mean of the
  ranks' gradients, SGD on the fp32 master shards, all-gather into bf16
  parameter storage) equals the same step composed from the oracle's
  pack, reduce-scatter, bf16 rounding and all-gather, bit for bit.
"""
import numpy as np
import pytest
import torch

import parameter_layout_collectives_amd as tide
import parameter_layout_collectives_amd.torch_ops as tops
import workloads
from gpu_helpers import bits16, bits32, note, same_f32
from parameter_layout_collectives_amd.fsdp import TideUnit

pytestmark = pytest.mark.gpu

DEV = "cuda"
# a decoder layer in miniature: q, k, v, o, gate, up, down, two norms; dim 0
# of k and v (and of the ragged ones) is not a multiple of the world size
LAYER = [(64, 48), (18, 48), (18, 48), (48, 64), (161, 48), (161, 48), (48, 161), (48,), (48,)]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def test_custom_ops_match_binding(orc):
    shapes = LAYER
    N = 4
    plan = tide.Plan(shapes, N)
    pid = tops.register_plan(plan)
    try:
        g = [[t.to(DEV) for t in rank]
             for rank in workloads.random_grads_for_shapes(shapes, N, seed_base=5)]
        flat = [t for rank in g for t in rank]
        for R in range(N):
            for small, avg in ((False, False), (True, True)):
                a = torch.empty(plan.S, device=DEV)
                b = torch.empty(plan.S, device=DEV)
                note(f"custom op tide::rs R={R} small={small} avg={avg}")
                torch.ops.tide.rs(pid, R, flat, a, small, avg)
                tide.rs(plan, R, g, b, small=small, avg=avg)
                torch.cuda.synchronize()
                assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        gathered = workloads.random_bf16(N * plan.S, seed=6, device=DEV)
        p1 = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
        p2 = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
        note("custom op tide::ag")
        torch.ops.tide.ag(pid, gathered, p1, False, False)
        tide.ag(plan, gathered, p2)
        slots = torch.empty(N, N * plan.S, dtype=torch.bfloat16, device=DEV)
        note("custom ops tide::pack, tide::rs_slots")
        for r in range(N):
            torch.ops.tide.pack(pid, g[r], slots[r], False)
        out = torch.empty(plan.S, device=DEV)
        torch.ops.tide.rs_slots(pid, 1, slots, out, False, False)
        ref = torch.empty(plan.S, device=DEV)
        tide.rs(plan, 1, g, ref)
        torch.cuda.synchronize()
        for x, y in zip(p1, p2):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    finally:
        tops.unregister_plan(pid)


def test_custom_ops_under_torch_compile():
    """A compiled step (dynamo + AOT functionalization, eager kernels) that
    reduce-scatters, all-gathers and reads the shard gives the eager bits."""
    shapes = LAYER
    N = 4
    plan = tide.Plan(shapes, N)
    pid = tops.register_plan(plan)
    try:
        g = [[t.to(DEV) for t in rank]
             for rank in workloads.random_grads_for_shapes(shapes, N, seed_base=9)]
        flat = [t for rank in g for t in rank]
        gathered = workloads.random_bf16(N * plan.S, seed=10, device=DEV)

        def step(flat, out, gathered, params):
            torch.ops.tide.rs(pid, 2, flat, out, False, True)
            torch.ops.tide.ag(pid, gathered, params, False, False)
            return out * 2.0

        compiled = torch.compile(step, backend="aot_eager", fullgraph=True)
        res = {}
        for name, fn in (("eager", step), ("compiled", compiled)):
            out = torch.full((plan.S,), float("nan"), device=DEV)
            params = [torch.zeros(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
            note(f"tide::rs + tide::ag, {name}")
            y = fn(flat, out, gathered, params)
            torch.cuda.synchronize()
            res[name] = (out, params, y)
        (o1, p1, y1), (o2, p2, y2) = res["eager"], res["compiled"]
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
        for a, b in zip(p1, p2):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    finally:
        tops.unregister_plan(pid)


def test_tide_unit_sgd_step(orc):
    shapes = LAYER
    N = 4
    lr = 2.0 ** -4                     # a power of two: lr * g is exact
    rng = np.random.default_rng(17)
    full = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    unit = TideUnit(shapes, N)
    note("TideUnit: load")
    unit.load([torch.from_numpy(f) for f in full])
    torch.cuda.synchronize()
    g = orc.geometry(shapes, N)

    # sharding: master rows = the oracle's fp32 pack; params = bf16 of it
    master0 = orc.pack(shapes, N, [f.view(np.uint32) for f in full], elem_bytes=4)
    assert np.array_equal(bits32(unit.master).reshape(-1), master0)

    def placed(master_bits):
        b16 = orc.round_bf16(master_bits.view(np.float32))
        return orc.ag(shapes, N, [b16[r * g.S:(r + 1) * g.S] for r in range(N)])

    want_p = placed(master0)
    for i, p in enumerate(unit.params):
        assert np.array_equal(bits16(p).reshape(-1), want_p[i]), i

    # backward on every rank -> reduce-scatter of the mean
    grads = [[t.to(DEV) for t in rank]
             for rank in workloads.random_grads_for_shapes(shapes, N, seed_base=23)]
    note("TideUnit: reduce_scatter")
    unit.reduce_scatter(grads)
    torch.cuda.synchronize()
    host = [[bits16(t) for t in rank] for rank in grads]
    want_g = [orc.rs(shapes, N, R, host, avg=True) for R in range(N)]
    for R in range(N):
        assert same_f32(unit.grad[R].cpu().numpy(), want_g[R]), R

    # SGD on the shards, then the all-gather into parameter storage
    unit.master.add_(unit.grad, alpha=-lr)
    note("TideUnit: all_gather")
    unit.all_gather()
    torch.cuda.synchronize()
    m1 = master0.view(np.float32).reshape(N, g.S) + np.float32(-lr) * np.stack(want_g)
    m1 = m1.astype(np.float32)
    assert np.array_equal(bits32(unit.master).reshape(-1), m1.reshape(-1).view(np.uint32))
    want_p = placed(m1.reshape(-1).view(np.uint32))
    for i, p in enumerate(unit.params):
        assert np.array_equal(bits16(p).reshape(-1), want_p[i]), i
