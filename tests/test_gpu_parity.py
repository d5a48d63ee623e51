"""GPU parity of tide_rs / tide_ag against the CPU oracle at small sizes.

Every case compares the HIP path with the oracle element by element on the
same seeded inputs: bit-exact for the reduce-scatter (rank-order fp32 sum;
NaN compared by class) and for the all-gather placement (a byte copy).
Outputs are pre-filled with a sentinel so unwritten elements show up.

Sizes span several tiles (4096 elements per reduce-scatter tile, 8192 per
all-gather tile) with ragged tails, and cover the degenerate cases: empty
parameters, 0-dim parameters, dim0 < N (ranks with no rows), N = 1, a single
workgroup, unaligned pointers (scalar paths), alignment gaps, fp32 elements.
"""
import numpy as np
import pytest
import torch

import parameter_layout_collectives_amd as tide
import workloads
from gpu_helpers import (BF16_SENTINEL, F32_SENTINEL, bits16, bits32, expected_rs,
                         first_mismatch, first_mismatch16, note, run_rs, same_bf16, same_f32)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def to_dev(grads):
    return [[g.to(DEV) for g in rank] for rank in grads]


def fresh_out(S):
    return torch.full((S,), F32_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)


def check_rs(orc, shapes, N, grads_dev, R, align=1, **kw):
    plan = tide.Plan(shapes, N, align)
    out = fresh_out(plan.S)
    note(f"tide_rs shapes={shapes} N={N} R={R} align={align} {kw}")
    run_rs(plan, R, grads_dev, out, **kw)
    want = expected_rs(orc, shapes, N, R, grads_dev, plan, align)
    got = out.cpu().numpy()
    assert same_f32(got, want), first_mismatch(got, want)
    return got


# ---------------------------------------------------------------------------
# reduce-scatter
# ---------------------------------------------------------------------------

def test_tiny_every_rank(orc):
    w = workloads.WORKLOADS["tiny"]
    g = to_dev(workloads.all_grads(w))
    for R in range(w.world):
        for kw in ({}, {"small": True}, {"max_workgroups": 1}, {"max_workgroups": 3}):
            check_rs(orc, w.shapes, w.world, g, R, **kw)


RAGGED = [
    [(4099, 3), (8191,), (1, 5), (12345, 2), (0, 4), (64, 64), ()],
    [(33, 4), (2,), (70000,), (5, 1023)],
]


@pytest.mark.parametrize("case", range(len(RAGGED)))
@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 13, 16])
def test_ragged_shapes(orc, case, N):
    shapes = RAGGED[case]
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=100 * N + case))
    for R in sorted({0, 1 % N, N // 2, N - 1}):
        check_rs(orc, shapes, N, g, R)


@pytest.mark.parametrize("align", [4, 6, 64])
def test_alignment_gaps(orc, align):
    shapes = [(37, 3), (16,), (9, 9), (3,)]
    N = 4
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=7))
    for R in range(N):
        check_rs(orc, shapes, N, g, R, align=align)


def test_many_ranks_and_tiny_params(orc):
    shapes = [(1,), (3,), (200, 7), (64,)]
    N = 64
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=3))
    for R in (0, 1, 2, 63):
        check_rs(orc, shapes, N, g, R)
        check_rs(orc, shapes, N, g, R, small=True)


def test_unaligned_pointers(orc):
    """Gradients at odd element offsets inside bigger buffers (2-byte
    aligned, not 16), with every rank at a different offset, and an output
    that is 4-byte but not 16-byte aligned: all scalar paths."""
    shapes = [(513, 5), (4100,), (7, 3)]
    N = 5
    host = workloads.random_grads_for_shapes(shapes, N, seed_base=55)
    grads = []
    for r, rank in enumerate(host):
        row = []
        for i, t in enumerate(rank):
            n = t.numel()
            buf = torch.zeros(n + 16, dtype=torch.bfloat16, device=DEV)
            shift = (r + 3 * i) % 8 + 1
            view = buf[shift:shift + n]
            view.copy_(t.reshape(-1).to(DEV))
            row.append(view.view(t.shape))
        grads.append(row)
    plan = tide.Plan(shapes, N)
    for R in range(N):
        big = fresh_out(plan.S + 3)
        out = big[1:1 + plan.S]
        note(f"tide_rs unaligned R={R}")
        run_rs(plan, R, grads, out)
        want = expected_rs(orc, shapes, N, R, grads, plan)
        got = out.cpu().numpy()
        assert same_f32(got, want), first_mismatch(got, want)
        assert bits32(big[0:1])[0] == F32_SENTINEL
        assert bits32(big[-2:])[1] == F32_SENTINEL


def test_aligned_inputs_unaligned_output(orc):
    shapes = [(1000, 8), (4096,)]
    N = 4
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=9))
    plan = tide.Plan(shapes, N)
    big = fresh_out(plan.S + 2)
    out = big[1:1 + plan.S]
    for R in range(N):
        run_rs(plan, R, g, out)
        want = expected_rs(orc, shapes, N, R, g, plan)
        got = out.cpu().numpy()
        assert same_f32(got, want), first_mismatch(got, want)


def test_special_values(orc):
    """-0.0, bf16 subnormals, +-Inf and NaN go through the vector path."""
    N = 4
    n = 4096 + 24
    pool = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x7F80, 0xFF80,
                     0x7FC0, 0x3F80, 0xBF80, 0x4B80, 0xCB80, 0x7F7F, 0xFF7F], np.uint16)
    rng = np.random.default_rng(1)
    grads = []
    for r in range(N):
        bits = pool[rng.integers(0, len(pool), size=n)]
        bits[:64] = 0x8000                      # columns of -0.0 only
        bits[64:128] = 0x0001                   # subnormal sums, exact
        t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(DEV)
        grads.append([t.reshape(n // 4, 4)])
    for R in range(N):
        got = check_rs(orc, [(n // 4, 4)], N, grads, R)
        if R == 0:
            assert np.all(got[:64].view(np.uint32) == 0x80000000)
            assert np.all(got[64:128].view(np.uint32) == (N << 16))


def test_integer_values_exact(orc):
    N = 16
    shapes = [(300, 17), (4096,)]
    rng = np.random.default_rng(3)
    ints = [[rng.integers(-8, 9, size=s) for s in shapes] for _ in range(N)]
    grads = [[torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(DEV) for a in rank]
             for rank in ints]
    plan = tide.Plan(shapes, N)
    for R in (0, 7, 15):
        out = fresh_out(plan.S)
        run_rs(plan, R, grads, out)
        got = out.cpu().numpy()
        for i, s in enumerate(shapes):
            src, L = plan.real(R, i)
            off = plan.param(i)[0]
            want = sum(ints[r][i].reshape(-1)[src:src + L].astype(np.int64) for r in range(N))
            assert np.array_equal(got[off:off + L].astype(np.int64), want)


def test_deterministic_and_streams(orc):
    shapes = [(4096, 33), (77,)]
    N = 8
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=21))
    plan = tide.Plan(shapes, N)
    table = tide.grad_table(plan, g)
    a = fresh_out(plan.S)
    b = fresh_out(plan.S)
    s = torch.cuda.Stream()
    tide.rs(plan, 3, table, a)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tide.rs(plan, 3, table, b, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    want = expected_rs(orc, shapes, N, 3, g, plan)
    assert same_f32(a.cpu().numpy(), want)


# ---------------------------------------------------------------------------
# gradient element types and the mean
# ---------------------------------------------------------------------------

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def typed_grads(shapes, N, seed, dtype):
    g = workloads.random_grads_for_shapes(shapes, N, seed_base=seed)
    return [[t.float().to(_TORCH[dtype]).to(DEV) for t in rank] for rank in g]


def host_elems(t, dtype):
    t = t.detach().contiguous().cpu()
    return t.numpy() if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def check_rs_typed(orc, shapes, N, grads, R, dtype, avg, align=1, **kw):
    plan = tide.Plan(shapes, N, align)
    out = fresh_out(plan.S)
    note(f"tide_rs typed {dtype} avg={avg} shapes={shapes} N={N} R={R} {kw}")
    run_rs(plan, R, grads, out, avg=avg, **kw)
    slices = [[host_elems(g.reshape(-1)[plan.real(R, i)[0]:plan.real(R, i)[0] +
                                        plan.real(R, i)[1]], dtype)
               for i, g in enumerate(rank)] for rank in grads]
    want = orc.rs_slices(shapes, N, R, slices, align=align, dtype=dtype, avg=avg)
    got = out.cpu().numpy()
    assert same_f32(got, want), (dtype, avg, R, first_mismatch(got, want))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N", [1, 3, 8, 16])
def test_typed_and_mean(orc, dtype, N):
    shapes = RAGGED[0]
    g = typed_grads(shapes, N, 300 + N, dtype)
    for R in sorted({0, N // 2, N - 1}):
        for avg in (False, True):
            check_rs_typed(orc, shapes, N, g, R, dtype, avg)
        check_rs_typed(orc, shapes, N, g, R, dtype, True, small=True)


def test_typed_unaligned_and_gaps(orc):
    """fp16/fp32 gradients at odd element offsets (scalar path) and with
    alignment gaps in the block."""
    shapes = [(513, 5), (4100,), (7, 3)]
    N = 4
    for dtype in ("f16", "f32"):
        base = typed_grads(shapes, N, 77, dtype)
        grads = []
        for r, rank in enumerate(base):
            row = []
            for i, t in enumerate(rank):
                n = t.numel()
                buf = torch.zeros(n + 8, dtype=t.dtype, device=DEV)
                shift = (r + i) % 3 + 1
                buf[shift:shift + n].copy_(t.reshape(-1))
                row.append(buf[shift:shift + n].view(t.shape))
            grads.append(row)
        for R in range(N):
            check_rs_typed(orc, shapes, N, grads, R, dtype, R % 2 == 1)
        for R in range(N):
            check_rs_typed(orc, shapes, N, base, R, dtype, False, align=6)


def test_f16_special_values(orc):
    """fp16 subnormals, -0.0, +-Inf and NaN through the vector path."""
    N = 4
    n = 4096 + 40
    pool = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x7C00,
                     0xFC00, 0x7E00, 0x3C00, 0xBC00], np.uint16)
    rng = np.random.default_rng(5)
    grads = []
    for r in range(N):
        bits = pool[rng.integers(0, len(pool), size=n)]
        bits[:64] = 0x8000
        bits[64:128] = 0x0001           # 2^-24: sums exact in fp32
        grads.append([torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(DEV)
                      .reshape(n // 4, 4)])
    for R in range(N):
        for avg in (False, True):
            check_rs_typed(orc, [(n // 4, 4)], N, grads, R, "f16", avg)


@pytest.mark.parametrize("N", [2, 6, 8, 16])
def test_f32_mean_subnormal_and_special_results(orc, N):
    """The mean of fp32 gradients whose sums are subnormal, tiny normal,
    huge (overflowing to infinity), signed zeros, infinities and NaNs.  At
    power-of-two N the kernel multiplies by 1/N, otherwise it divides; the
    oracle always divides, and the bits must agree either way."""
    n = 4096 + 36
    pool = np.array([0x00000001, 0x80000001, 0x00000003, 0x007FFFFF, 0x807FFFFF, 0x00800000,
                     0x00800001, 0x80800000, 0x01000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F000000,
                     0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000,
                     0x00400000, 0x00000010], np.uint32)
    rng = np.random.default_rng(17 + N)
    grads = []
    for r in range(N):
        bits = pool[rng.integers(0, len(pool), size=n)]
        bits[:256] = pool[rng.integers(0, 7, size=256)]     # subnormal sums
        grads.append([torch.from_numpy(bits.view(np.int32)).view(torch.float32).to(DEV)
                      .reshape(n // 4, 4)])
    for R in sorted({0, N - 1}):
        check_rs_typed(orc, [(n // 4, 4)], N, grads, R, "f32", True)
        check_rs_typed(orc, [(n // 4, 4)], N, grads, R, "f32", True, small=True)


# ---------------------------------------------------------------------------
# reduce-scatter with a bf16 shard (the fp32 result rounded once)
# ---------------------------------------------------------------------------

def check_rs_bf16(orc, shapes, N, grads, R, dtype="bf16", avg=False, align=1, out_shift=0,
                  **kw):
    """tide_rs into a bf16 block `out_shift` elements into a sentinel-filled
    buffer; compared with the oracle's fp32 block rounded by the oracle."""
    plan = tide.Plan(shapes, N, align)
    base = torch.full((plan.S + out_shift + 1,), BF16_SENTINEL, dtype=torch.int16,
                      device=DEV).view(torch.bfloat16)
    out = base[out_shift:out_shift + plan.S]
    note(f"tide_rs bf16 out {dtype} avg={avg} shapes={shapes} N={N} R={R} align={align} "
         f"out_shift={out_shift} {kw}")
    run_rs(plan, R, grads, out, avg=avg, **kw)
    slices = [[host_elems(g.reshape(-1)[plan.real(R, i)[0]:plan.real(R, i)[0] +
                                        plan.real(R, i)[1]], dtype)
               for i, g in enumerate(rank)] for rank in grads]
    want = orc.round_bf16(orc.rs_slices(shapes, N, R, slices, align=align, dtype=dtype, avg=avg))
    got = bits16(out)
    assert same_bf16(got, want), (dtype, avg, R, first_mismatch16(got, want))
    whole = bits16(base)
    assert np.all(whole[:out_shift] == BF16_SENTINEL) and whole[-1] == BF16_SENTINEL


def test_bf16_out_tiny_every_rank(orc):
    w = workloads.WORKLOADS["tiny"]
    g = to_dev(workloads.all_grads(w))
    for R in range(w.world):
        for kw in ({}, {"small": True}, {"max_workgroups": 1}):
            for avg in (False, True):
                check_rs_bf16(orc, w.shapes, w.world, g, R, avg=avg, **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("N", [1, 3, 8, 16])
def test_bf16_out_ragged(orc, dtype, N):
    g = typed_grads(RAGGED[0], N, 500 + N, dtype)
    for R in sorted({0, N // 2, N - 1}):
        check_rs_bf16(orc, RAGGED[0], N, g, R, dtype=dtype)
        check_rs_bf16(orc, RAGGED[0], N, g, R, dtype=dtype, avg=True, small=True)
    g1 = typed_grads(RAGGED[1], N, 600 + N, dtype)
    check_rs_bf16(orc, RAGGED[1], N, g1, N - 1, dtype=dtype, align=8)


@pytest.mark.parametrize("out_shift", [1, 4, 8])
def test_bf16_out_unaligned(orc, out_shift):
    """Outputs 2-, 8- and 16-byte aligned (scalar and vector stores), and
    gradients at odd element offsets (scalar loads)."""
    shapes = [(1031, 3), (9000,), (5, 5)]
    N = 4
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=700))
    check_rs_bf16(orc, shapes, N, g, 1, out_shift=out_shift)
    bufs = [[torch.empty(t.numel() + 1, dtype=torch.bfloat16, device=DEV) for t in rank]
            for rank in g]
    odd = []
    for rank, brank in zip(g, bufs):
        row = []
        for t, b in zip(rank, brank):
            b[1:].copy_(t.reshape(-1))
            row.append(b[1:].view(t.shape))
        odd.append(row)
    check_rs_bf16(orc, shapes, N, odd, 2, out_shift=out_shift, avg=True)


def test_bf16_out_rounding_edges(orc):
    """Sums on rounding ties (integer values past 256, where bf16 steps by
    2 and 4), sums that round to infinity, subnormal sums, NaN and Inf."""
    N = 3
    shapes = [(4096,), (517,)]
    rng = np.random.default_rng(808)
    ints = [[torch.from_numpy(rng.integers(-300, 301, size=s).astype(np.float32))
             .to(torch.bfloat16).to(DEV) for s in shapes] for _ in range(N)]
    for R in range(N):
        check_rs_bf16(orc, shapes, N, ints, R)
    big = 3.3999e38        # above the largest bf16 by more than half its unit
    vals = np.array([big, -big, 3.3895e38, 1e-39, 3e-40, -5e-41, np.inf, -np.inf, np.nan,
                     1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 0.0], np.float32)
    # rank 0 cycles through the values, rank 1 adds zeros, rank 2 a rotation
    # of them, so every pair of values meets somewhere
    f32 = [[torch.from_numpy(np.resize(vals, 4096)).to(DEV),
            torch.from_numpy(np.resize(vals[::-1].copy(), 517)).to(DEV)],
           [torch.zeros(4096, device=DEV), torch.zeros(517, device=DEV)],
           [torch.from_numpy(np.resize(np.roll(vals, 5), 4096)).to(DEV),
            torch.from_numpy(np.resize(np.roll(vals, 3), 517)).to(DEV)]]
    for R in range(N):
        check_rs_bf16(orc, shapes, N, f32, R, dtype="f32")


# ---------------------------------------------------------------------------
# all-gather placement
# ---------------------------------------------------------------------------

def check_ag(orc, shapes, N, e=2, align=1, src_shift=0, dst_shift=0, **kw):
    plan = tide.Plan(shapes, N, align)
    S = plan.S
    dt = torch.bfloat16 if e == 2 else torch.float32
    ft = torch.int16 if e == 2 else torch.int32
    sentinel = BF16_SENTINEL if e == 2 else F32_SENTINEL
    rng = np.random.default_rng(N * 7 + e + align)
    flat_bits = rng.integers(0, 2 ** (8 * e) - 1, size=N * S + src_shift, dtype=np.uint64)
    flat_bits = flat_bits.astype(np.uint16 if e == 2 else np.uint32)
    buf = torch.from_numpy(flat_bits.view(np.int16 if e == 2 else np.int32)).to(DEV).view(dt)
    gathered = buf[src_shift:src_shift + N * S]
    blocks = [gathered[r * S:(r + 1) * S] for r in range(N)]
    params, bases = [], []
    for s in shapes:
        n = int(np.prod(s)) if len(s) else 1
        base = torch.full((n + dst_shift + 1,), sentinel, dtype=ft, device=DEV).view(dt)
        bases.append(base)
        params.append(base[dst_shift:dst_shift + n].view(s if len(s) else ()))
    note(f"tide_ag shapes={shapes} N={N} e={e} align={align} shifts={src_shift},{dst_shift} {kw}")
    tide.ag(plan, blocks, params, **kw)
    torch.cuda.synchronize()
    host_blocks = [flat_bits[src_shift + r * S: src_shift + (r + 1) * S] for r in range(N)]
    want = orc.ag(shapes, N, host_blocks, elem_bytes=e, align=align)
    for i, p in enumerate(params):
        got = (bits16(p) if e == 2 else bits32(p)).reshape(-1)
        bad = np.nonzero(got != want[i])[0]
        assert bad.size == 0, (i, int(bad[0]), bad.size)
        tail = (bits16(bases[i]) if e == 2 else bits32(bases[i]))
        assert np.all(tail[:dst_shift] == sentinel) and tail[-1] == sentinel


def test_ag_tiny(orc):
    w = workloads.WORKLOADS["tiny"]
    for kw in ({}, {"small": True}, {"max_workgroups": 1}, {"copy_engine": True}):
        check_ag(orc, w.shapes, w.world, **kw)


@pytest.mark.parametrize("N", [1, 3, 8, 16])
@pytest.mark.parametrize("e", [2, 4])
def test_ag_ragged(orc, N, e):
    check_ag(orc, RAGGED[0], N, e=e)
    check_ag(orc, RAGGED[1], N, e=e, align=8)
    check_ag(orc, RAGGED[0], N, e=e, small=True)


@pytest.mark.parametrize("N", [1, 2, 5, 16])
@pytest.mark.parametrize("e", [2, 4])
def test_ag_copy_engine(orc, N, e):
    """SDMA placement: 2-D copies over the full ranks, 1-D for the short rank."""
    check_ag(orc, RAGGED[0], N, e=e, copy_engine=True)
    check_ag(orc, RAGGED[1], N, e=e, align=8, copy_engine=True)
    check_ag(orc, [(1031, 3), (9000,), (5, 5)], N, e=e, src_shift=1, dst_shift=3,
             copy_engine=True)


def test_ag_copy_engine_separate_blocks(orc):
    """Rank blocks in separate allocations (not equally spaced): one copy per
    (parameter, rank)."""
    shapes = [(37, 3), (4100,), (2, 2)]
    N = 5
    plan = tide.Plan(shapes, N)
    rng = np.random.default_rng(12)
    host = [rng.integers(0, 65535, size=plan.S).astype(np.uint16) for _ in range(N)]
    blocks = [torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16) for h in host]
    params = [torch.full(s, 0, dtype=torch.int16, device=DEV).fill_(BF16_SENTINEL)
              .view(torch.bfloat16) for s in shapes]
    tide.ag(plan, blocks, params, copy_engine=True)
    torch.cuda.synchronize()
    want = orc.ag(shapes, N, host, elem_bytes=2)
    for i, p in enumerate(params):
        assert np.array_equal(bits16(p).reshape(-1), want[i]), i


@pytest.mark.parametrize("src_shift,dst_shift", [(1, 0), (0, 3), (5, 5), (2, 6), (4, 0)])
@pytest.mark.parametrize("e", [2, 4])
def test_ag_unaligned(orc, src_shift, dst_shift, e):
    check_ag(orc, [(1031, 3), (9000,), (5, 5)], 4, e=e, src_shift=src_shift,
             dst_shift=dst_shift)


def test_ag_inverts_rs_layout(orc):
    """AG of the fp32 blocks tide_rs wrote for every rank equals the
    rank-order all-reduce of the gradients (reduce-scatter + all-gather)."""
    shapes = [(5, 7), (16,), (33, 4), (4097,)]
    N = 4
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=31))
    plan = tide.Plan(shapes, N)
    blocks = torch.empty(N, plan.S, dtype=torch.float32, device=DEV)
    for R in range(N):
        tide.rs(plan, R, g, blocks[R])
    params = [torch.empty(s, dtype=torch.float32, device=DEV) for s in shapes]
    tide.ag(plan, blocks, params)
    torch.cuda.synchronize()
    host = [[bits16(t) for t in rank] for rank in g]
    want_blocks = [orc.rs(shapes, N, R, host).view(np.uint32) for R in range(N)]
    want = orc.ag(shapes, N, want_blocks, elem_bytes=4)
    for i in range(len(shapes)):
        assert np.array_equal(bits32(params[i]).reshape(-1), want[i]), i


def test_ag_destinations_inside_unread_parts_of_blocks(orc):
    """Destinations may lie in the gaps of the gathered buffer, which are
    never read: the call is accepted and every read element is placed."""
    shapes = [(3, 4), (5,)]
    N, align = 2, 64          # S = 128; rank blocks read [0,8), [64,67) / [0,4), [64,66)
    plan = tide.Plan(shapes, N, align)
    assert plan.S == 128
    rng = np.random.default_rng(77)
    host = rng.integers(0, 65535, size=N * plan.S).astype(np.uint16)
    gathered = torch.from_numpy(host.view(np.int16)).to(DEV).view(torch.bfloat16)
    blocks = [gathered[r * plan.S:(r + 1) * plan.S] for r in range(N)]
    params = [gathered[plan.S + 10:plan.S + 22].view(3, 4),   # in rank 1's gap [8, 64)
              gathered[16:21]]                                # in rank 0's gap
    note("tide_ag destinations inside block gaps")
    tide.ag(plan, blocks, params)
    torch.cuda.synchronize()
    want = orc.ag(shapes, N, [host[r * plan.S:(r + 1) * plan.S] for r in range(N)],
                  elem_bytes=2, align=align)
    got_all = bits16(gathered)
    for i, p in enumerate(params):
        assert np.array_equal(bits16(p).reshape(-1), want[i]), i
    untouched = np.ones(N * plan.S, bool)
    untouched[plan.S + 10:plan.S + 22] = False
    untouched[16:21] = False
    assert np.array_equal(got_all[untouched], host[untouched])


def test_rs_output_inside_unread_rows_of_a_gradient(orc):
    """`out` may overlap gradient elements the call does not read (rows of
    other ranks' shards)."""
    shapes = [(256, 4), (10,)]
    N, R = 4, 3               # rank 3 reads rows 192..255 of param 0, element 9 of param 1
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=55))
    plan = tide.Plan(shapes, N)
    assert plan.S == 259
    out = g[1][0].reshape(-1)[0:2 * plan.S].view(torch.float32)   # rank 1's rows 0..129
    note("tide_rs out inside unread gradient rows")
    run_rs(plan, R, g, out)
    want = expected_rs(orc, shapes, N, R, g, plan)
    got = out.cpu().numpy()
    assert same_f32(got, want), first_mismatch(got, want)


# ---------------------------------------------------------------------------
# runtime behaviour
# ---------------------------------------------------------------------------

def test_pointer_table_cache_eviction(orc):
    """More gradient sets than the plan caches (8): tables are evicted and
    re-uploaded, and every call still reads the right tensors."""
    shapes = [(33, 5), (4100,)]
    N = 3
    plan = tide.Plan(shapes, N)
    sets = [to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=1000 + 10 * j))
            for j in range(11)]
    out = fresh_out(plan.S)
    for sweep in range(2):
        for j, g in enumerate(sets):
            R = (j + sweep) % N
            note(f"cache eviction: set {j} R={R} sweep {sweep}")
            run_rs(plan, R, g, out)
            want = expected_rs(orc, shapes, N, R, g, plan)
            got = out.cpu().numpy()
            assert same_f32(got, want), (j, R, first_mismatch(got, want))


def test_concurrent_calls_on_one_plan(orc):
    """Several host threads use one plan at once (each with its own stream
    and output); results equal the oracle's."""
    import threading
    shapes = [(257, 9), (4096,), (3, 3)]
    N = 4
    plan = tide.Plan(shapes, N)
    g = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=77))
    outs = [fresh_out(plan.S) for _ in range(8)]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for k in range(5):
                    tide.rs(plan, t % N, g, outs[t], stream=s, small=(k % 2 == 1))
            s.synchronize()
        except Exception as exc:  # noqa: BLE001 - reported below
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(8):
        want = expected_rs(orc, shapes, N, t % N, g, plan)
        assert same_f32(outs[t].cpu().numpy(), want), t


def test_table_upload_ordered_across_streams(orc):
    """A new pointer set is uploaded by an async copy on the caller's stream.
    Here that stream is held back by a spin kernel; a second call with the
    same set on another stream must wait for the upload.  Every slot first
    holds a valid set, so reading the slot too early would give another
    set's sums, not a fault."""
    shapes = [(37, 5), (4100,)]
    N = 3
    plan = tide.Plan(shapes, N)
    sets = [to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=2000 + 10 * j))
            for j in range(9)]
    scratch = fresh_out(plan.S)
    for j in range(8):                       # fill the 8 slots of the cache
        run_rs(plan, 0, sets[j], scratch)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    out_a, out_b = fresh_out(plan.S), fresh_out(plan.S)
    torch.cuda.synchronize()
    note("upload on a held-back stream, hit on another stream")
    with torch.cuda.stream(a):
        torch.cuda._sleep(20_000_000)        # bounded spin: holds stream a back
    tide.rs(plan, 1, sets[8], out_a, stream=a)   # replaces slot of set 0; upload queued on a
    tide.rs(plan, 1, sets[8], out_b, stream=b)   # hit: must wait for that upload
    torch.cuda.synchronize()
    want = expected_rs(orc, shapes, N, 1, sets[8], plan)
    for out in (out_a, out_b):
        got = out.cpu().numpy()
        assert same_f32(got, want), first_mismatch(got, want)


def test_table_slots_under_concurrent_eviction(orc):
    """Two host threads, each with its own stream, cycle through 12 pointer
    sets (more than the 8 cached slots), so slots are replaced while the
    other stream may still read them: every result still equals the oracle."""
    import threading
    shapes = [(33, 5), (4100,)]
    N = 3
    plan = tide.Plan(shapes, N)
    sets = [to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=3000 + 10 * j))
            for j in range(12)]
    outs = [[fresh_out(plan.S) for _ in range(len(sets))] for _ in range(2)]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            for sweep in range(3):
                for j in range(len(sets)):
                    jj = (j * (t + 1) + sweep) % len(sets)
                    tide.rs(plan, jj % N, sets[jj], outs[t][jj], stream=s)
            s.synchronize()
        except Exception as exc:  # noqa: BLE001 - reported below
            errors.append(exc)

    note("pointer-table slots: two streams, 12 sets, 8 slots")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for j, g in enumerate(sets):
        want = expected_rs(orc, shapes, N, j % N, g, plan)
        for t in range(2):
            got = outs[t][j].cpu().numpy()
            assert same_f32(got, want), (t, j, first_mismatch(got, want))


def _sleep_cycles_for(ms):
    """torch.cuda._sleep cycle count for about `ms` milliseconds (measured)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(5_000_000)
    b.record()
    torch.cuda.synchronize()
    return int(5_000_000 * ms / max(a.elapsed_time(b), 1e-3))


def test_slot_reuse_waits_only_for_its_readers(orc):
    """Every cached pointer set is read on two streams; replacing one then
    waits for those two streams' events only, not for a long (bounded) spin
    on a third stream that never read it."""
    import time
    shapes = [(29, 7), (4100,)]
    N = 3
    plan = tide.Plan(shapes, N)
    sets = [to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=4000 + 10 * j))
            for j in range(9)]
    a, b, c = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    scratch = fresh_out(plan.S)
    for j in range(8):                       # 8 slots, each read on a and b
        tide.rs(plan, 0, sets[j], scratch, stream=a)
        tide.rs(plan, 0, sets[j], scratch, stream=b)
    torch.cuda.synchronize()
    spin = _sleep_cycles_for(800.0)
    out = fresh_out(plan.S)
    note("slot reuse beside an 800 ms spin on an unrelated stream")
    with torch.cuda.stream(c):
        torch.cuda._sleep(spin)
    t0 = time.perf_counter()
    tide.rs(plan, 2, sets[8], out, stream=a)  # replaces the slot of set 0
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    assert host_s < 0.4, f"replacing a slot waited {host_s:.3f} s (the unrelated spin)"
    want = expected_rs(orc, shapes, N, 2, sets[8], plan)
    got = out.cpu().numpy()
    assert same_f32(got, want), first_mismatch(got, want)


def test_one_set_read_on_many_streams(orc):
    """20 streams read one cached set (more than the 16 tracked per slot),
    then 9 other sets replace every slot: every result equals the oracle."""
    shapes = [(31, 6), (2049,)]
    N = 4
    plan = tide.Plan(shapes, N)
    base = to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=5000))
    others = [to_dev(workloads.random_grads_for_shapes(shapes, N, seed_base=5100 + 10 * j))
              for j in range(9)]
    streams = [torch.cuda.Stream() for _ in range(20)]
    outs = [fresh_out(plan.S) for _ in streams]
    note("one pointer set on 20 streams, then 9 evicting sets")
    for k, (s, o) in enumerate(zip(streams, outs)):
        tide.rs(plan, k % N, base, o, stream=s)
    outs2 = [fresh_out(plan.S) for _ in others]
    for j, (g, o) in enumerate(zip(others, outs2)):
        tide.rs(plan, j % N, g, o, stream=streams[j])
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        want = expected_rs(orc, shapes, N, k % N, base, plan)
        assert same_f32(o.cpu().numpy(), want), k
    for j, o in enumerate(outs2):
        want = expected_rs(orc, shapes, N, j % N, others[j], plan)
        assert same_f32(o.cpu().numpy(), want), j
