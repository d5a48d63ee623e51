"""GPU parity at the size limits of the boundary.

* one parameter of 2^31 + 37 elements (4.3 GB of bf16 per rank), 2 ranks:
  every element and byte offset past 2^31 takes 64-bit arithmetic.  The
  reduce-scatter, all-gather and pack outputs are checked on sampled
  elements (edges, tile boundaries, the 2^31 crossing, random ones), each
  computed by the oracle from the same inputs;
* 1024 ranks with small ragged parameters: whole outputs against the oracle;
* the largest world a plan takes, 65,536 ranks: whole outputs of ranks that
  own real rows, against the oracle.
"""
import gc

import numpy as np
import pytest
import torch

import parameter_layout_collectives_amd as tide
import workloads
from gpu_helpers import F32_SENTINEL, bits16, first_mismatch, note, same_f32

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


def _sample(n, rng, tile, extra=()):
    """Sorted unique indices in [0, n): both ends, both sides of every
    `tile`-th boundary among the first few, random ones, and `extra`."""
    pts = [0, 1, 2, 3, n - 4, n - 3, n - 2, n - 1]
    for b in range(1, 64):
        pts += [b * tile - 1, b * tile]
    for x in extra:
        pts += [x - 2, x - 1, x, x + 1]
    pts += list(rng.integers(0, n, size=200000))
    a = np.unique(np.array([p for p in pts if 0 <= p < n], np.int64))
    return a


@pytest.mark.timeout(900)
def test_parameter_over_2g_elements(orc):
    n = 2 ** 31 + 37
    shapes = [(n,)]
    N = 2
    plan = tide.Plan(shapes, N)
    c = (n + N - 1) // N
    assert plan.S == c
    note(f"max size: generating 2 x {n} bf16 gradient elements")
    grads = [[workloads.random_bf16(n, seed=5000 + r, device=DEV)] for r in range(N)]
    rng = np.random.default_rng(1)
    out = torch.empty(plan.S, dtype=torch.float32, device=DEV)
    for R in range(N):
        src, L = plan.real(R, 0)
        k = _sample(L, rng, 4096, extra=(2 ** 31 - src,))
        for small in (False, True):
            out.view(torch.int32).fill_(F32_SENTINEL)
            note(f"max size: tide_rs R={R} small={small}")
            tide.rs(plan, R, grads, out, small=small)
            torch.cuda.synchronize()
            kt = torch.from_numpy(k).to(DEV)
            got = out[kt].cpu().numpy()
            # the oracle on the sampled elements: a problem of one parameter
            # of 2*K elements whose rank-0 shard is exactly the samples
            slices = [[bits16(grads[r][0][src + kt])] for r in range(N)]
            want = orc.rs_slices([(2 * k.size,)], N, 0, slices)
            assert same_f32(got, want), (R, small, first_mismatch(got, want))
            if L < plan.S:                       # padding of the short rank
                assert torch.all(out[L:] == 0).item()
        del kt
    del out, grads
    _free()

    # all-gather of a 2^32-element gathered buffer into the one parameter
    note("max size: tide_ag")
    gathered = workloads.random_bf16(N * plan.S, seed=5100, device=DEV)
    param = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for kw in ({}, {"small": True}):
        param.view(torch.int16).fill_(0x7FBD)
        tide.ag(plan, gathered, [param], **kw)
        torch.cuda.synchronize()
        j = _sample(n, rng, 2048, extra=(2 ** 31, c))
        g = orc.geometry(shapes, N)
        owner = j // c
        pos = owner * plan.S + g.off[0] + (j - owner * c)
        jt, pt = torch.from_numpy(j).to(DEV), torch.from_numpy(pos).to(DEV)
        assert torch.equal(param[jt].view(torch.int16), gathered[pt].view(torch.int16)), kw
        del jt, pt
    del gathered
    _free()

    # pack of the parameter into a 2^32-element slot
    note("max size: tide_pack")
    slot = torch.empty(N * plan.S, dtype=torch.bfloat16, device=DEV)
    tide.pack(plan, [param], slot)
    torch.cuda.synchronize()
    q = _sample(N * plan.S, rng, 2048, extra=(2 ** 31, plan.S))
    blk, kk = q // plan.S, q % plan.S
    src_idx = blk * c + kk
    real = src_idx < n
    qt = torch.from_numpy(q).to(DEV)
    got = bits16(slot[qt])
    want = np.zeros(q.size, np.uint16)
    want[real] = bits16(param[torch.from_numpy(src_idx[real]).to(DEV)])
    assert np.array_equal(got, want)
    del slot, param, qt
    _free()


def _views(shapes, N, seed):
    """Rank r's gradient of param i = row r of one [N, numel_i] buffer."""
    bufs = []
    for i, s in enumerate(shapes):
        n = int(np.prod(s)) if len(s) else 1
        bufs.append(workloads.random_bf16(N * n, seed=seed + i, device=DEV).view(N, n))
    return [[bufs[i][r].view(s) for i, s in enumerate(shapes)] for r in range(N)], bufs


def _expected_from_views(orc, shapes, N, R, bufs, plan):
    slices = []
    host = []
    for i in range(len(shapes)):
        src, L = plan.real(R, i)
        host.append(bits16(bufs[i][:, src:src + L]).reshape(N, L))
    for r in range(N):
        slices.append([host[i][r] for i in range(len(shapes))])
    return orc.rs_slices(shapes, N, R, slices)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N,ranks", [(1024, (0, 511, 1023)), (65536, (0, 2, 34999))])
def test_many_ranks(orc, N, ranks):
    shapes = [(70000,), (3, 5), (1025, 3)]
    plan = tide.Plan(shapes, N)
    note(f"many ranks: N={N} S={plan.S}")
    grads, bufs = _views(shapes, N, 7000)
    table = tide.grad_table(plan, grads)
    out = torch.empty(plan.S, dtype=torch.float32, device=DEV)
    for R in ranks:
        for small in (False, True):
            out.view(torch.int32).fill_(F32_SENTINEL)
            note(f"many ranks: tide_rs N={N} R={R} small={small}")
            tide.rs(plan, R, table, out, small=small)
            torch.cuda.synchronize()
            want = _expected_from_views(orc, shapes, N, R, bufs, plan)
            got = out.cpu().numpy()
            assert same_f32(got, want), (N, R, small, first_mismatch(got, want))
    # all-gather of the whole N*S buffer, every element checked
    gathered = workloads.random_bf16(N * plan.S, seed=7100, device=DEV)
    params = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    note(f"many ranks: tide_ag N={N}")
    tide.ag(plan, gathered, params)
    torch.cuda.synchronize()
    host = bits16(gathered)
    want = orc.ag(shapes, N, [host[r * plan.S:(r + 1) * plan.S] for r in range(N)])
    for i, p in enumerate(params):
        assert np.array_equal(bits16(p).reshape(-1), want[i]), i
    del grads, bufs, table, out, gathered, params
    _free()
