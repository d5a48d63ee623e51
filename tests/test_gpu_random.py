"""Randomised GPU parity (hypothesis, derandomised: the same examples every
run).  Each example draws a parameter list (0-dim, empty, 1-3 dims, sizes
across tile boundaries), a world size, an alignment, a gradient type, the
mean and bf16-shard flags and the launch mode, then compares tide_rs for
three ranks, tide_ag and tide_pack with the oracle bit for bit."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import parameter_layout_collectives_amd as tide
import workloads
from gpu_helpers import (BF16_SENTINEL, F32_SENTINEL, bits16, note, same_bf16, same_f32)

pytestmark = pytest.mark.gpu

DEV = "cuda"
_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}

shape = st.one_of(
    st.just(()),
    st.tuples(st.integers(0, 9000)),
    st.tuples(st.integers(0, 300), st.integers(1, 40)),
    st.tuples(st.integers(1, 20), st.integers(1, 9), st.integers(1, 7)),
)
example = st.fixed_dictionaries({
    "shapes": st.lists(shape, min_size=1, max_size=6),
    "N": st.sampled_from([1, 2, 3, 4, 7, 8, 16, 24]),
    "align": st.sampled_from([1, 2, 8, 64]),
    "dtype": st.sampled_from(["bf16", "f16", "f32"]),
    "avg": st.booleans(),
    "bf16_out": st.booleans(),
    "small": st.booleans(),
    "seed": st.integers(0, 2 ** 31),
})


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _host(t):
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.function_scoped_fixture,
                                 HealthCheck.too_slow, HealthCheck.data_too_large])
@given(example)
def test_random_parity(orc, ex):
    shapes, N, align, dtype = ex["shapes"], ex["N"], ex["align"], ex["dtype"]
    note(f"random parity {ex}")
    plan = tide.Plan(shapes, N, align)
    S = plan.S
    g = workloads.random_grads_for_shapes(shapes, N, seed_base=ex["seed"] % 100000)
    grads = [[t.float().to(_TORCH[dtype]).to(DEV) for t in rank] for rank in g]
    host = [[_host(t).reshape(-1) for t in rank] for rank in grads]
    if dtype == "f32":
        host = [[a.view(np.float32) for a in rank] for rank in host]
    # reduce-scatter
    for R in sorted({0, N - 1, N // 2}):
        if ex["bf16_out"]:
            out = torch.full((max(S, 1),), BF16_SENTINEL, dtype=torch.int16,
                             device=DEV).view(torch.bfloat16)[:S]
        else:
            out = torch.full((max(S, 1),), F32_SENTINEL, dtype=torch.int32,
                             device=DEV).view(torch.float32)[:S]
        tide.rs(plan, R, grads, out, small=ex["small"], avg=ex["avg"])
        torch.cuda.synchronize()
        want = orc.rs(shapes, N, R, host, align=align, dtype=dtype, avg=ex["avg"])
        if ex["bf16_out"]:
            assert same_bf16(bits16(out), orc.round_bf16(want)), (ex, R)
        else:
            assert same_f32(out.cpu().numpy(), want), (ex, R)
    # all-gather of a random gathered buffer (same element type as the grads)
    e = 4 if dtype == "f32" else 2
    rng = np.random.default_rng(ex["seed"])
    gh = rng.integers(0, 2 ** (8 * e) - 1, size=N * S, dtype=np.uint64).astype(
        np.uint16 if e == 2 else np.uint32)
    gathered = torch.from_numpy(gh.view(np.int16 if e == 2 else np.int32)).to(DEV)
    params = [torch.full(s, 0, dtype=gathered.dtype, device=DEV) for s in shapes]
    if N * S:
        tide.ag(plan, gathered, params, small=ex["small"])
        torch.cuda.synchronize()
        want_p = orc.ag(shapes, N, [gh[r * S:(r + 1) * S] for r in range(N)], elem_bytes=e,
                        align=align)
        for i, p in enumerate(params):
            assert np.array_equal(_host(p).reshape(-1), want_p[i]), (ex, i)
    # pack of rank 0's gradients
    slot = torch.full((max(N * S, 1),), -1, dtype=torch.int16 if e == 2 else torch.int32,
                      device=DEV).view(_TORCH[dtype])[:N * S]
    tide.pack(plan, grads[0], slot, small=ex["small"])
    torch.cuda.synchronize()
    want_s = orc.pack(shapes, N, [a.view(np.uint16 if e == 2 else np.uint32) for a in host[0]],
                      elem_bytes=e, align=align)
    assert np.array_equal(_host(slot), want_s), ex
