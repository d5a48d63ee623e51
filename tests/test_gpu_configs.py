"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times (default grid and small-footprint grid).

Workloads (architecture shapes only, synthetic seeded bf16 gradients):
  * Llama-3-8B-shaped decoder layer, 8 ranks;
  * Llama-3.1-70B-shaped decoder layer, 8 ranks;
  * Qwen3-30B-A3B-shaped MoE layer (391 parameters, 6256 gradient
    pointers), 16 ranks, 10% of experts all-zero per rank;
  * Llama-3.1-70B-shaped layer at 64 ranks (~110 GB of gradients in HBM),
    also with bf16 8192^3 GEMMs running on another stream (the co-run).

The whole fp32 output block of each checked rank is compared bit for bit
with the oracle, which reads host copies of exactly the gradient slices the
rank reduces; so is the bf16 block (the fp32 result rounded once, the
oracle's rounding applied to its fp32 block).  The all-gather placement is compared on every element of
every parameter.
"""
import gc

import numpy as np
import pytest
import torch

import parameter_layout_collectives_amd as tide
import workloads
from gpu_helpers import (BF16_SENTINEL, F32_SENTINEL, bits16, expected_rs, first_mismatch,
                         first_mismatch16, note, same_bf16, same_f32)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rs_cases(orc, w, grads, plan, table, ranks, modes):
    out = torch.empty(plan.S, dtype=torch.float32, device=DEV)
    out16 = torch.empty(plan.S, dtype=torch.bfloat16, device=DEV)
    for R in ranks:
        want = expected_rs(orc, w.shapes, w.world, R, grads, plan)
        want16 = orc.round_bf16(want)
        for small in modes:
            out.view(torch.int32).fill_(F32_SENTINEL)
            note(f"{w.name}: tide_rs R={R} small={small}")
            tide.rs(plan, R, table, out, small=small)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            assert same_f32(got, want), (w.name, R, small, first_mismatch(got, want))
            out16.view(torch.int16).fill_(BF16_SENTINEL)
            note(f"{w.name}: tide_rs bf16 out R={R} small={small}")
            tide.rs(plan, R, table, out16, small=small)
            torch.cuda.synchronize()
            got16 = bits16(out16)
            assert same_bf16(got16, want16), (w.name, R, small, first_mismatch16(got16, want16))
    del out16
    return out


def _ag_case(orc, w, plan):
    N, S = w.world, plan.S
    gathered = workloads.random_bf16(N * S, seed=4242, sigma=w.sigma, device=DEV)
    host = bits16(gathered)
    want = orc.ag(w.shapes, N, [host[r * S:(r + 1) * S] for r in range(N)], elem_bytes=2)
    for kw in ({}, {"small": True}, {"copy_engine": True}):
        params = [torch.full(s, 0, dtype=torch.int16, device=DEV).fill_(BF16_SENTINEL)
                  .view(torch.bfloat16) for s in w.shapes]
        note(f"{w.name}: tide_ag N={N} S={S} {kw}")
        tide.ag(plan, gathered, params, **kw)
        torch.cuda.synchronize()
        for i, p in enumerate(params):
            got = bits16(p).reshape(-1)
            bad = np.nonzero(got != want[i])[0]
            assert bad.size == 0, (w.name, kw, i, int(bad[0]) if bad.size else None, bad.size)
        del params


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama3_8b_layer", "llama31_70b_layer",
                                  "qwen3_30b_a3b_moe_layer"])
def test_workload_rs_ag(orc, name):
    w = workloads.WORKLOADS[name]
    note(f"{name}: generating {w.world} ranks of gradients on the device")
    grads = workloads.all_grads(w, device=DEV)
    plan = tide.Plan(w.shapes, w.world)
    table = tide.grad_table(plan, grads)
    out = _rs_cases(orc, w, grads, plan, table, sorted({0, 1, w.world - 1}), (False, True))
    # determinism: the same call again gives the same bits
    first = out.clone()
    tide.rs(plan, w.world - 1, table, out)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int32), out.view(torch.int32))
    del grads, table, out, first
    _free()
    _ag_case(orc, w, plan)
    _free()


@pytest.mark.timeout(900)
def test_llama70b_layer_64_ranks(orc):
    w = workloads.WORKLOADS["llama31_70b_layer_n64"]
    note(f"{w.name}: generating {w.world} ranks of gradients on the device (~110 GB)")
    grads = workloads.all_grads(w, device=DEV)
    plan = tide.Plan(w.shapes, w.world)
    table = tide.grad_table(plan, grads)
    _rs_cases(orc, w, grads, plan, table, (0, 63), (False,))
    _rs_cases(orc, w, grads, plan, table, (1,), (True,))
    # the co-run configuration: tide_rs on one stream while bf16 8192^3
    # GEMMs run on another (the bench's co-run), results checked
    M, K, Nn = w.corun_gemm
    a = torch.randn(M, K, device=DEV).to(torch.bfloat16)
    b = torch.randn(K, Nn, device=DEV).to(torch.bfloat16)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {R: torch.empty(plan.S, dtype=torch.float32, device=DEV) for R in (5, 40)}
    wants = {R: expected_rs(orc, w.shapes, w.world, R, grads, plan) for R in outs}
    torch.cuda.synchronize()
    note(f"{w.name}: tide_rs beside bf16 GEMMs")
    with torch.cuda.stream(sa):
        for _ in range(12):
            torch.matmul(a, b)
    for small in (True, False):
        for R, o in outs.items():
            o.view(torch.int32).fill_(F32_SENTINEL)
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            for _ in range(12):
                torch.matmul(a, b)
        for R, o in outs.items():
            tide.rs(plan, R, table, o, small=small, stream=sb)
        torch.cuda.synchronize()
        for R, o in outs.items():
            got = o.cpu().numpy()
            assert same_f32(got, wants[R]), (R, small, first_mismatch(got, wants[R]))
    del grads, table, a, b, outs
    _free()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_llama8b_layer_typed_gradients_and_mean(orc, dtype):
    """The gradient-type and mean variants at full size: the 8B-shaped layer
    with fp16 or fp32 gradients (the bf16 draws widened), sum and mean,
    both launch modes, whole blocks of ranks 0 and 7 against the oracle."""
    w = workloads.WORKLOADS["llama3_8b_layer"]
    N = w.world
    tdt = {"f16": torch.float16, "f32": torch.float32}[dtype]
    note(f"{w.name}: {dtype} gradients on the device")
    grads = [[t.to(tdt) for t in rank] for rank in workloads.all_grads(w, device=DEV)]
    plan = tide.Plan(w.shapes, N)
    table = tide.grad_table(plan, grads)
    out = torch.empty(plan.S, dtype=torch.float32, device=DEV)
    for R in (0, N - 1):
        slices = []
        for rank in grads:
            row = []
            for i, g in enumerate(rank):
                src, L = plan.real(R, i)
                h = g.reshape(-1)[src:src + L].cpu()
                row.append(h.numpy() if dtype == "f32" else
                           h.view(torch.int16).numpy().view(np.uint16))
            slices.append(row)
        for avg in (False, True):
            want = orc.rs_slices(w.shapes, N, R, slices, dtype=dtype, avg=avg)
            for small in (False, True):
                out.view(torch.int32).fill_(F32_SENTINEL)
                note(f"{w.name}: tide_rs {dtype} R={R} avg={avg} small={small}")
                tide.rs(plan, R, table, out, small=small, avg=avg)
                torch.cuda.synchronize()
                got = out.cpu().numpy()
                assert same_f32(got, want), (dtype, R, avg, small, first_mismatch(got, want))
    del grads, table, out
    _free()
