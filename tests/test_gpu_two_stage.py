"""GPU parity of the two-stage TIDE-RS (tide_pack, then tide_rs_slots)
against the CPU oracle.

* tide_pack: the whole staging slot equals the oracle's rank-major pack bit
  for bit (real elements copied, padding and gaps zero), for 2- and 4-byte
  elements, ragged shapes, alignment gaps, unaligned tensors and both launch
  modes;
* tide_rs_slots over the N ranks' slots equals the oracle's reduce-scatter of
  the gradients they were packed from, and the one-pass tide_rs, bit for bit
  (bf16 / fp16 / fp32 slots, sum and mean, fp32 and bf16 shards);
* Slot-Reuse: the slot is the all-gather buffer after its shards were placed
  into the parameters;
* full workloads: the 70B-shaped layer (8 ranks) and the MoE layer (16 ranks).
"""
import gc

import numpy as np
import pytest
import torch

import parameter_layout_collectives_amd as tide
import workloads
from gpu_helpers import (BF16_SENTINEL, F32_SENTINEL, bits16, bits32, expected_rs,
                         first_mismatch, first_mismatch16, note, same_bf16, same_f32)

pytestmark = pytest.mark.gpu

DEV = "cuda"
_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}

RAGGED = [
    [(4099, 3), (8191,), (1, 5), (12345, 2), (0, 4), (64, 64), ()],
    [(33, 4), (2,), (70000,), (5, 1023)],
]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def typed_grads(shapes, N, seed, dtype):
    g = workloads.random_grads_for_shapes(shapes, N, seed_base=seed)
    return [[t.float().to(_TORCH[dtype]).to(DEV) for t in rank] for rank in g]


def host_bits(t):
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def sentinel_slot(plan, dtype):
    n = plan.world * plan.S
    if torch.tensor([], dtype=dtype).element_size() == 2:
        return torch.full((n,), BF16_SENTINEL, dtype=torch.int16, device=DEV).view(dtype)
    return torch.full((n,), F32_SENTINEL, dtype=torch.int32, device=DEV).view(dtype)


def check_pack(orc, shapes, N, tensors, align=1, **kw):
    plan = tide.Plan(shapes, N, align)
    dtype = tensors[0].dtype
    slot = sentinel_slot(plan, dtype)
    note(f"tide_pack shapes={shapes} N={N} align={align} dtype={dtype} {kw}")
    tide.pack(plan, tensors, slot, **kw)
    torch.cuda.synchronize()
    e = slot.element_size()
    want = orc.pack(shapes, N, [host_bits(t).reshape(-1) for t in tensors], elem_bytes=e,
                    align=align)
    got = host_bits(slot)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (shapes, N, align, kw, int(bad[0]), bad.size)
    return plan, slot


def test_pack_tiny_every_mode(orc):
    w = workloads.WORKLOADS["tiny"]
    g = [[t.to(DEV) for t in rank] for rank in workloads.all_grads(w)]
    for r in range(w.world):
        for kw in ({}, {"small": True}, {"max_workgroups": 1}):
            check_pack(orc, w.shapes, w.world, g[r], **kw)


@pytest.mark.parametrize("N", [1, 3, 8, 16])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_ragged_and_gaps(orc, N, dtype):
    g = typed_grads(RAGGED[0], N, 40 + N, dtype)
    check_pack(orc, RAGGED[0], N, g[0])
    check_pack(orc, RAGGED[0], N, g[N - 1], small=True)
    g1 = typed_grads(RAGGED[1], N, 50 + N, dtype)
    check_pack(orc, RAGGED[1], N, g1[0], align=8)


def test_pack_unaligned_tensors(orc):
    """Tensors at odd element offsets: narrower vectors or element copies."""
    shapes = [(1031, 3), (9000,), (5, 5)]
    N = 4
    for dtype in ("bf16", "f32"):
        base = typed_grads(shapes, N, 60, dtype)[0]
        odd = []
        for shift, t in zip((1, 3, 2), base):
            buf = torch.empty(t.numel() + shift, dtype=t.dtype, device=DEV)
            buf[shift:].copy_(t.reshape(-1))
            odd.append(buf[shift:].view(t.shape))
        check_pack(orc, shapes, N, odd)


def two_stage(plan, grads, R, out, **kw):
    """Pack every rank's gradients into its own slot, then reduce block R."""
    N = plan.world
    slots = torch.empty(N, N * plan.S, dtype=grads[0][0].dtype, device=DEV)
    for r in range(N):
        tide.pack(plan, grads[r], slots[r])
    tide.rs_slots(plan, R, slots, out, **kw)
    torch.cuda.synchronize()
    return slots


def fresh(plan, bf16_out):
    if bf16_out:
        return torch.full((plan.S,), BF16_SENTINEL, dtype=torch.int16,
                          device=DEV).view(torch.bfloat16)
    return torch.full((plan.S,), F32_SENTINEL, dtype=torch.int32,
                      device=DEV).view(torch.float32)


def check_two_stage(orc, shapes, N, grads, R, dtype="bf16", avg=False, bf16_out=False,
                    align=1, **kw):
    plan = tide.Plan(shapes, N, align)
    out2 = fresh(plan, bf16_out)
    note(f"two-stage shapes={shapes} N={N} R={R} {dtype} avg={avg} bf16_out={bf16_out} "
         f"align={align} {kw}")
    two_stage(plan, grads, R, out2, avg=avg, **kw)
    out1 = fresh(plan, bf16_out)
    tide.rs(plan, R, grads, out1, avg=avg, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16 if bf16_out else torch.int32),
                       out2.view(torch.int16 if bf16_out else torch.int32))
    slices = [[host_bits(g.reshape(-1)[plan.real(R, i)[0]:plan.real(R, i)[0] +
                                       plan.real(R, i)[1]]) for i, g in enumerate(rank)]
              for rank in grads]
    if dtype == "f32":
        slices = [[a.view(np.float32) for a in row] for row in slices]
    want = orc.rs_slices(shapes, N, R, slices, align=align, dtype=dtype, avg=avg)
    if bf16_out:
        want16 = orc.round_bf16(want)
        got = bits16(out2)
        assert same_bf16(got, want16), first_mismatch16(got, want16)
    else:
        got = out2.cpu().numpy()
        assert same_f32(got, want), first_mismatch(got, want)


def test_two_stage_tiny_every_rank(orc):
    w = workloads.WORKLOADS["tiny"]
    g = [[t.to(DEV) for t in rank] for rank in workloads.all_grads(w)]
    for R in range(w.world):
        check_two_stage(orc, w.shapes, w.world, g, R)
        check_two_stage(orc, w.shapes, w.world, g, R, avg=True, small=True)
        check_two_stage(orc, w.shapes, w.world, g, R, bf16_out=True, max_workgroups=1)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N", [1, 3, 8])
def test_two_stage_ragged(orc, dtype, N):
    g = typed_grads(RAGGED[0], N, 70 + N, dtype)
    for R in sorted({0, N // 2, N - 1}):
        check_two_stage(orc, RAGGED[0], N, g, R, dtype=dtype)
    check_two_stage(orc, RAGGED[0], N, g, N - 1, dtype=dtype, avg=True, bf16_out=True,
                    small=True)
    g1 = typed_grads(RAGGED[1], N, 80 + N, dtype)
    check_two_stage(orc, RAGGED[1], N, g1, 0, dtype=dtype, align=8)


def test_slot_reuse_round_trip(orc):
    """Forward: tide_ag places the gathered buffer into the parameters.  The
    buffer is then vacated and holds this rank's packed gradients; with the
    peers' slots, tide_rs_slots gives the oracle's reduce-scatter, and the
    parameters keep the gathered values."""
    shapes = [(37, 5), (4100,), (7, 3, 2)]
    N = 4
    plan = tide.Plan(shapes, N)
    rng = np.random.default_rng(31)
    host = rng.integers(0, 65535, size=N * plan.S).astype(np.uint16)
    gathered = torch.from_numpy(host.view(np.int16)).to(DEV).view(torch.bfloat16)
    params = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    note("slot reuse: all-gather, then pack into the vacated buffer")
    tide.ag(plan, gathered, params)
    grads = [[t.to(DEV) for t in rank]
             for rank in workloads.random_grads_for_shapes(shapes, N, seed_base=90)]
    slots = [gathered] + [torch.empty(N * plan.S, dtype=torch.bfloat16, device=DEV)
                          for _ in range(N - 1)]
    for r in range(N):
        tide.pack(plan, grads[r], slots[r])
    for R in range(N):
        out = fresh(plan, False)
        tide.rs_slots(plan, R, slots, out)
        torch.cuda.synchronize()
        want = expected_rs(orc, shapes, N, R, grads, plan)
        got = out.cpu().numpy()
        assert same_f32(got, want), (R, first_mismatch(got, want))
    want_p = orc.ag(shapes, N, [host[r * plan.S:(r + 1) * plan.S] for r in range(N)])
    for i, p in enumerate(params):
        assert np.array_equal(bits16(p).reshape(-1), want_p[i]), i


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama31_70b_layer", "qwen3_30b_a3b_moe_layer"])
def test_two_stage_workloads(orc, name):
    """Full size: every rank's slot packed on the device; rank 0's slot
    checked against the oracle's pack; ranks 0 and N-1 reduced from the
    slots and compared with the one-pass tide_rs and (rank N-1) the oracle."""
    w = workloads.WORKLOADS[name]
    N = w.world
    note(f"{name}: generating {N} ranks of gradients on the device")
    grads = workloads.all_grads(w, device=DEV)
    plan = tide.Plan(w.shapes, N)
    slots = torch.empty(N, N * plan.S, dtype=torch.bfloat16, device=DEV)
    for r in range(N):
        note(f"{name}: tide_pack rank {r}")
        tide.pack(plan, grads[r], slots[r])
    torch.cuda.synchronize()
    want0 = orc.pack(w.shapes, N, [host_bits(t).reshape(-1) for t in grads[0]])
    got0 = host_bits(slots[0])
    assert np.array_equal(got0, want0), int(np.nonzero(got0 != want0)[0][0])
    del want0, got0
    out1 = torch.empty(plan.S, dtype=torch.float32, device=DEV)
    out2 = torch.empty(plan.S, dtype=torch.float32, device=DEV)
    for R in (0, N - 1):
        for small in (False, True):
            note(f"{name}: tide_rs_slots R={R} small={small}")
            tide.rs_slots(plan, R, slots, out2, small=small)
            tide.rs(plan, R, grads, out1)
            torch.cuda.synchronize()
            assert torch.equal(out1.view(torch.int32), out2.view(torch.int32)), (R, small)
    want = expected_rs(orc, w.shapes, N, N - 1, grads, plan)
    got = out2.cpu().numpy()
    assert same_f32(got, want), first_mismatch(got, want)
    del grads, slots, out1, out2
    _free()
