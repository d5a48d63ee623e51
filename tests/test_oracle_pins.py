"""Pins of the CPU oracle against things other than itself.

Every ``pin_*`` function takes an oracle handle and raises AssertionError on
a mismatch.  The tests below run them on the real oracle;
``test_oracle_mutants.py`` runs them on builds of oracle.c with planted
mistakes and requires each mistake to be caught.

Pins used (none of them re-types the oracle's formulas):
  * brute force: shards cut with torch.chunk and rank blocks built by
    concatenation (tests/brute.py), on tiny shapes, every rank;
  * a worked layout derived by hand for the tiny workload;
  * closed forms and page figures (tests/golden/page_figures.json):
    S = Psi/N when N divides every dim 0 (1/N per GPU, 12.5% at 8), traffic
    (N-1)/N*Psi per rank, 420 GB per step for a 70B model at 16 bit;
  * special cases that reduce to exact arithmetic or a library routine:
    integer-valued bf16 inputs (int64 sum), N=1 (plain cast), N=2 (torch
    sum), rank order fixed by a cancellation case, -0.0, subnormals, Inf/NaN;
  * the recursive-summation error bound against an exact rational sum;
  * all-gather invariants: AG of the shards is the identity, and RS for
    every rank followed by AG is the per-element rank-order all-reduce;
  * gradient element types and the mean: every binary16 pattern widened as
    numpy does, N=2 and integer-valued sums of fp16/fp32 gradients, the mean
    as an exact power-of-two scaling (N = 2^k) or as the exact rational
    sum/N rounded to nearest even (other N);
  * staging for the two-stage reduce-scatter: the packed slot equals the
    brute-force rank blocks of the tensors (zero padding), the all-gather
    of a packed slot gives the tensors back, and the reduce-scatter of the
    staged blocks equals the one-pass reduce-scatter of the gradients;
  * fp32 -> bf16 rounding of a shard: torch's own conversion over millions
    of patterns (every low half under chosen high halves), a search over all
    65,536 bf16 values for the nearest one, worked ties, and an N=2 shard
    equal to torch's (a + b) in fp32 converted to bf16.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import brute
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TINY = workloads.WORKLOADS["tiny"]

# Small shape sweep: ragged dim 0 around N, several inner sizes, 1-D/2-D/3-D,
# empty parameters.
SWEEP = [
    [(5, 7), (16,), (33, 4)],
    [(1,), (2, 3)],
    [(0, 5), (7,), (3, 2, 2)],
    [(9, 1), (8, 8), (11, 3)],
    [()],
    [(13, 7), (1, 1), (4,)],
]


def bits_f32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def random_bits(shape, rng):
    """bf16 bit patterns of N(0,1) draws (round to nearest even)."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    return workloads.bf16_bits(x.to(torch.bfloat16)).reshape(shape)


def bits_of(vals):
    return workloads.bf16_bits(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16))


# --------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------
def pin_tiny_worked_layout(orc):
    # Worked by hand from "ceil(d0/N) rows per rank, shards padded to that
    # many rows, parameters packed in order":
    #   a [5,7]:  c=2, seg=14, off=0;  rows 2,2,1,0 -> L 14,14,7,0;  src 0,14,28,42
    #   b [16]:   c=4, seg=4,  off=14; rows 4,4,4,4 -> L 4,4,4,4;    src 0,4,8,12
    #   c [33,4]: c=9, seg=36, off=18; rows 9,9,9,6 -> L 36,36,36,24; src 0,36,72,108
    #   S = 54, N*S = 216, Psi = 35+16+132 = 183, padding = 33.
    g = orc.geometry(TINY.shapes, 4)
    assert g.c == [2, 4, 9]
    assert g.seg == [14, 4, 36]
    assert g.off == [0, 14, 18]
    assert g.S == 54
    L = [[g.run(r, i)[1] for r in range(4)] for i in range(3)]
    src = [[g.run(r, i)[0] for r in range(4)] for i in range(3)]
    assert L == [[14, 14, 7, 0], [4, 4, 4, 4], [36, 36, 36, 24]]
    assert src == [[0, 14, 28, 42], [0, 4, 8, 12], [0, 36, 72, 108]]
    assert 4 * g.S - g.psi == 33


def pin_geometry_vs_brute(orc):
    for shapes in SWEEP:
        for N in (1, 2, 3, 4, 5, 8):
            for align in (1, 4):
                g = orc.geometry(shapes, N, align)
                pos, S = brute.segment_positions(shapes, N, align)
                assert g.S == S, (shapes, N, align)
                assert [p for p, _ in pos] == g.off, (shapes, N, align)
                assert [n for _, n in pos] == g.seg, (shapes, N, align)
                for i, s in enumerate(shapes):
                    t = torch.zeros(s if len(s) else (), dtype=torch.int8)
                    chunks, c = brute.shard_rows(t, N)
                    inner = g.inner[i]
                    for r in range(N):
                        src, L = g.run(r, i)
                        assert L == chunks[r].numel(), (shapes, N, r, i)
                        if L:
                            # first element of the chunk inside the full tensor
                            start = sum(chunks[q].numel() for q in range(r))
                            assert src == start, (shapes, N, r, i)
                        assert orc.shard_run(N, s, r) == (src, L)
                    assert g.c[i] * inner == g.seg[i]


def pin_layout_bijection(orc):
    for shapes in SWEEP:
        for N in (1, 3, 4, 8):
            g = orc.geometry(shapes, N)
            where, total = brute.layout_map(shapes, N)
            assert total == N * g.S
            # oracle's map: element j of param i -> r*S + off_i + (j - src)
            seen = set()
            for i in range(len(shapes)):
                for r in range(N):
                    src, L = g.run(r, i)
                    for k in range(L):
                        pos = r * g.S + g.off[i] + k
                        assert where[(i, src + k)] == pos
                        seen.add(pos)
            assert len(seen) == g.psi == len(where)
            assert total - len(seen) == N * g.S - g.psi   # padding count


def pin_divisible_closed_form(orc):
    golden = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    for name in ("llama3_8b_layer", "llama31_70b_layer", "qwen3_30b_a3b_moe_layer",
                 "llama31_70b_layer_n64"):
        w = workloads.WORKLOADS[name]
        g = orc.geometry(w.shapes, w.world)
        assert g.S * w.world == w.psi, name
    w = workloads.WORKLOADS["llama31_70b_layer"]
    g = orc.geometry(w.shapes, 8)
    assert g.S / g.psi == golden["per_rank_fraction_at_8"]["value"]


# --------------------------------------------------------------------------
# traffic
# --------------------------------------------------------------------------
def pin_traffic(orc):
    # tiny, by hand: (N-1)*S = 162 padded per rank; real 162,162,141,84.
    real = [orc.rs_traffic(TINY.shapes, 4, R) for R in range(4)]
    assert [p for _, p in real] == [162] * 4
    assert [x for x, _ in real] == [162, 162, 141, 84]
    for shapes in SWEEP:
        for N in (1, 2, 5, 8):
            g = orc.geometry(shapes, N)
            tot = sum(orc.rs_traffic(shapes, N, R)[0] for R in range(N))
            assert tot == (N - 1) * g.psi          # mean (N-1)/N * Psi per rank
            for R in range(N):
                assert orc.rs_traffic(shapes, N, R)[1] == (N - 1) * g.S


def pin_traffic_page_figure(orc):
    golden = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    f = golden["fsdp_step_bytes_70b_16bit"]
    shapes = [(70000, 1000000)]                    # Psi = 7e10
    N = 1000
    psi = 70000 * 1000000
    assert psi == f["psi"]
    per_rank = [orc.rs_traffic(shapes, N, R)[0] for R in range(N)]
    mean = sum(per_rank) / N
    assert sum(per_rank) == (N - 1) * psi
    # forward all-gather + backward all-gather + reduce-scatter, 2 bytes each
    step_bytes = 3 * mean * f["bytes_per_elem"]
    assert abs(step_bytes - f["value"]) / f["value"] < 1.1e-3
    # all-reduce = reduce-scatter + all-gather: FSDP/DDP = 3/2
    assert (3 * mean) / (2 * mean) == golden["fsdp_over_ddp"]["value"]


# --------------------------------------------------------------------------
# reduce-scatter arithmetic
# --------------------------------------------------------------------------
def _rand_case(shapes, N, seed):
    rng = np.random.default_rng(seed)
    return [[random_bits(s if len(s) else (), rng) for s in shapes] for _ in range(N)]


def pin_rs_vs_brute(orc):
    cases = [(TINY.shapes, 4), ([(3, 2, 2), (7,)], 3), ([(9, 1), (11, 3)], 5),
             ([(1,), (2, 3)], 2), ([(0, 5), (6,)], 4)]
    for idx, (shapes, N) in enumerate(cases):
        grads = _rand_case(shapes, N, 100 + idx)
        for align in (1, 4):
            for R in range(N):
                got = orc.rs(shapes, N, R, grads, align=align)
                want = brute.rs_rank_order(grads, shapes, N, R, align)
                assert np.array_equal(bits_f32(got), bits_f32(want)), (shapes, N, R, align)


def pin_rs_integer_exact(orc):
    rng = np.random.default_rng(7)
    shapes = [(13, 3), (8,), (5, 2, 3)]
    for N in (1, 2, 3, 8, 16):
        ints = [[rng.integers(-8, 9, size=s) for s in shapes] for _ in range(N)]
        grads = [[bits_of(a.astype(np.float32).reshape(-1)) for a in rank] for rank in ints]
        g = orc.geometry(shapes, N)
        for R in range(N):
            out = orc.rs(shapes, N, R, grads)
            for i, s in enumerate(shapes):
                src, L = g.run(R, i)
                want = sum(ints[r][i].reshape(-1)[src:src + L].astype(np.int64) for r in range(N))
                seg = out[g.off[i]:g.off[i] + g.seg[i]]
                assert np.array_equal(seg[:L].astype(np.int64), want), (N, R, i)
                assert np.all(bits_f32(seg[L:]) == 0)


def pin_rs_n1_is_cast(orc):
    shapes = [(7, 3), (5,)]
    grads = _rand_case(shapes, 1, 3)
    out = orc.rs(shapes, 1, 0, grads)
    want = torch.cat([torch.from_numpy(g.reshape(-1).astype(np.int16)).view(torch.bfloat16).float()
                      for g in grads[0]])
    assert np.array_equal(bits_f32(out), bits_f32(want.numpy()))


def pin_rs_n2_is_library_sum(orc):
    shapes = [(9, 5), (4,), (3, 3)]
    grads = _rand_case(shapes, 2, 4)
    g = orc.geometry(shapes, 2)
    for R in range(2):
        out = orc.rs(shapes, 2, R, grads)
        for i in range(len(shapes)):
            src, L = g.run(R, i)
            ts = [torch.from_numpy(grads[r][i].reshape(-1)[src:src + L].astype(np.int16))
                  .view(torch.bfloat16) for r in range(2)]
            want = torch.stack(ts).float().sum(0).numpy()
            got = out[g.off[i]:g.off[i] + L]
            assert np.array_equal(bits_f32(got), bits_f32(want)), (R, i)


def pin_rs_rank_order(orc):
    # ranks hold 2^24, 1, -2^24 at the same position.  In rank order:
    # fl(2^24 + 1) = 2^24 (tie, round to even), then 2^24 - 2^24 = +0.
    # Any other order (reverse, pairwise) gives 1.
    vals = [2.0 ** 24, 1.0, -(2.0 ** 24)]
    grads = [[bits_of([v])] for v in vals]
    out = orc.rs([(1,)], 3, 0, grads)
    assert bits_f32(out)[0] == 0x00000000
    grads_rev = [[bits_of([v])] for v in reversed(vals)]
    out_rev = orc.rs([(1,)], 3, 0, grads_rev)
    assert out_rev[0] == np.float32(1.0)


def pin_rs_negative_zero(orc):
    # All ranks -0.0: the sum starts from rank 0's value, so -0.0 survives.
    grads = [[np.array([0x8000, 0x8000], np.uint16)] for _ in range(4)]
    out = orc.rs([(2,)], 4, 0, grads)   # c = 1: rank 0 owns element 0
    assert bits_f32(out)[0] == 0x80000000


def pin_rs_subnormals(orc):
    # bf16 0x0001 = 2^-133 (subnormal).  Sum of N such values is N*2^-133,
    # exactly representable in binary32 (subnormal): bits N << 16.
    for N in (2, 3, 8):
        grads = [[np.array([0x0001], np.uint16)] for _ in range(N)]
        out = orc.rs([(1,)], N, 0, grads)
        assert bits_f32(out)[0] == (N << 16), N
    # mixed sign subnormals cancel exactly
    grads = [[np.array([0x0003], np.uint16)], [np.array([0x8001], np.uint16)]]
    out = orc.rs([(1,)], 2, 0, grads)
    assert bits_f32(out)[0] == (2 << 16)


def pin_rs_special_values(orc):
    inf, ninf, nan, one = 0x7F80, 0xFF80, 0x7FC0, 0x3F80
    out = orc.rs([(1,)], 2, 0, [[np.array([inf], np.uint16)], [np.array([one], np.uint16)]])
    assert np.isposinf(out[0])
    out = orc.rs([(1,)], 2, 0, [[np.array([inf], np.uint16)], [np.array([ninf], np.uint16)]])
    assert np.isnan(out[0])
    out = orc.rs([(1,)], 3, 0, [[np.array([one], np.uint16)], [np.array([nan], np.uint16)],
                                [np.array([one], np.uint16)]])
    assert np.isnan(out[0])


def pin_rs_error_bound(orc):
    # |rank-order sum - exact sum| <= (N-1) * 2^-24 * sum_r |g_r|
    shapes = [(16, 3)]
    for N in (3, 8):
        grads = _rand_case(shapes, N, 11 + N)
        g = orc.geometry(shapes, N)
        for R in (0, N - 1):
            out = orc.rs(shapes, N, R, grads)
            src, L = g.run(R, 0)
            for k in range(L):
                col = [int(grads[r][0].reshape(-1)[src + k]) for r in range(N)]
                exact = brute.exact_sum(col)
                absum = sum(abs(float(brute.widen(b))) for b in col)
                err = abs(float(out[k]) - float(exact))
                assert err <= (N - 1) * 2.0 ** -24 * absum, (N, R, k)


def pin_rs_slices_match_full(orc):
    shapes = [(5, 7), (16,), (33, 4)]
    grads = _rand_case(shapes, 4, 21)
    g = orc.geometry(shapes, 4)
    for R in range(4):
        slices = [[grads[r][i].reshape(-1)[g.run(R, i)[0]:g.run(R, i)[0] + g.run(R, i)[1]]
                   for i in range(3)] for r in range(4)]
        a = orc.rs(shapes, 4, R, grads)
        b = orc.rs_slices(shapes, 4, R, slices)
        assert np.array_equal(bits_f32(a), bits_f32(b))


# --------------------------------------------------------------------------
# gradient element types and the mean
# --------------------------------------------------------------------------
def _rand_typed(shapes, N, seed, dtype):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(N):
        row = []
        for s in shapes:
            x = rng.standard_normal(s).astype(np.float32)
            row.append(x.astype(np.float16).view(np.uint16) if dtype == "f16" else x)
        out.append(row)
    return out


def pin_f16_widening_exhaustive(orc):
    # every binary16 pattern against numpy's float16 -> float32 conversion
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    out = orc.rs([(65536,)], 1, 0, [[bits]], dtype="f16")
    want = bits.view(np.float16).astype(np.float32)
    assert np.array_equal(bits_f32(out), bits_f32(want))


def pin_typed_n2_is_library_sum(orc):
    shapes = [(9, 5), (4,)]
    for dtype in ("f16", "f32"):
        grads = _rand_typed(shapes, 2, 8, dtype)
        g = orc.geometry(shapes, 2)
        for R in range(2):
            out = orc.rs(shapes, 2, R, grads, dtype=dtype)
            for i in range(len(shapes)):
                src, L = g.run(R, i)
                ts = [torch.from_numpy(grads[r][i].reshape(-1)[src:src + L].copy())
                      for r in range(2)]
                if dtype == "f16":
                    ts = [t.view(torch.float16) for t in ts]
                want = torch.stack(ts).float().sum(0).numpy()
                assert np.array_equal(bits_f32(out[g.off[i]:g.off[i] + L]), bits_f32(want)), \
                    (dtype, R, i)


def pin_typed_integer_exact(orc):
    rng = np.random.default_rng(17)
    shapes = [(11, 3), (7,)]
    for dtype in ("f16", "f32"):
        for N in (3, 16):
            ints = [[rng.integers(-64, 65, size=s) for s in shapes] for _ in range(N)]
            grads = [[a.astype(np.float16).view(np.uint16) if dtype == "f16" else
                      a.astype(np.float32) for a in row] for row in ints]
            g = orc.geometry(shapes, N)
            for R in range(N):
                out = orc.rs(shapes, N, R, grads, dtype=dtype)
                for i in range(len(shapes)):
                    src, L = g.run(R, i)
                    want = sum(ints[r][i].reshape(-1)[src:src + L].astype(np.int64)
                               for r in range(N))
                    got = out[g.off[i]:g.off[i] + L]
                    assert np.array_equal(got.astype(np.int64), want), (dtype, N, R, i)


def pin_mean_power_of_two(orc):
    # N = 2^k: the mean is the sum scaled by 2^-k, which is exact here
    shapes = [(40, 3), (9,)]
    for N, k in ((2, 1), (4, 2), (8, 3), (16, 4)):
        grads = _rand_case(shapes, N, 30 + N)
        for R in (0, N - 1):
            s_ = orc.rs(shapes, N, R, grads)
            m = orc.rs(shapes, N, R, grads, avg=True)
            assert np.array_equal(bits_f32(m), bits_f32(np.ldexp(s_, -k).astype(np.float32)))


def pin_mean_exact_rounding(orc):
    # other N: the mean is the exact rational sum/N rounded to nearest even
    shapes = [(17, 3)]
    for N in (3, 5, 7, 13):
        grads = _rand_case(shapes, N, 50 + N)
        for R in (0, N - 1):
            s_ = orc.rs(shapes, N, R, grads)
            m = orc.rs(shapes, N, R, grads, avg=True)
            g = orc.geometry(shapes, N)
            src, L = g.run(R, 0)
            for k in range(L):
                want = brute.round_f32(Fraction(float(s_[k])) / N)
                assert bits_f32([m[k]])[0] == bits_f32([want])[0], (N, R, k)
            assert np.all(bits_f32(m[L:g.seg[0]]) == 0)          # padding stays +0


# --------------------------------------------------------------------------
# staging (two-stage reduce-scatter)
# --------------------------------------------------------------------------

def pin_pack_vs_brute(orc):
    rng = np.random.default_rng(910)
    for shapes in SWEEP:
        for N in (1, 2, 3, 5, 8):
            for align in (1, 4):
                ts = []
                for s in shapes:
                    n = int(np.prod(s)) if len(s) else 1
                    ts.append(rng.integers(1, 65535, size=n).astype(np.uint16))
                got = orc.pack(shapes, N, ts, align=align)
                tt = [torch.from_numpy(t.astype(np.int64)).reshape(s) for t, s in zip(ts, shapes)]
                want = torch.cat([brute.rank_block(tt, N, q, align, pad_value=0)
                                  for q in range(N)]).numpy().astype(np.uint16)
                assert np.array_equal(got, want), (shapes, N, align)


def pin_ag_inverts_pack(orc):
    rng = np.random.default_rng(911)
    for shapes in SWEEP:
        for N in (1, 3, 8):
            for e, dt in ((2, np.uint16), (4, np.uint32)):
                ts = [rng.integers(0, 2 ** (8 * e) - 1, size=int(np.prod(s)) if len(s) else 1,
                                   dtype=np.uint64).astype(dt) for s in shapes]
                slot = orc.pack(shapes, N, ts, elem_bytes=e, align=3)
                g = orc.geometry(shapes, N, 3)
                back = orc.ag(shapes, N, [slot[q * g.S:(q + 1) * g.S] for q in range(N)],
                              elem_bytes=e, align=3)
                for i in range(len(shapes)):
                    assert np.array_equal(back[i], ts[i]), (shapes, N, e, i)


def pin_two_stage_is_one_pass(orc):
    # reduce-scatter of block R of every rank's staged slot == reduce-scatter
    # of the gradients themselves, for every rank R
    for shapes in SWEEP[:4]:
        for N in (2, 3, 4):
            grads = _rand_case(shapes, N, 920 + N)
            g = orc.geometry(shapes, N)
            slots = [orc.pack(shapes, N, grads[r]) for r in range(N)]
            for R in range(N):
                slices = [[slots[r][R * g.S + g.off[i]:R * g.S + g.off[i] + g.run(R, i)[1]]
                           for i in range(len(shapes))] for r in range(N)]
                a = orc.rs_slices(shapes, N, R, slices)
                b = orc.rs(shapes, N, R, grads)
                assert np.array_equal(bits_f32(a), bits_f32(b)), (shapes, N, R)


# --------------------------------------------------------------------------
# fp32 -> bf16 rounding of a shard
# --------------------------------------------------------------------------

def _torch_bf16_bits(x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _check_rounding(orc, pats):
    """Oracle vs torch's fp32 -> bf16 conversion (round to nearest even):
    bitwise for non-NaN inputs; NaN inputs must give a NaN."""
    x = np.ascontiguousarray(pats, np.uint32).view(np.float32)
    got = orc.round_bf16(x)
    want = _torch_bf16_bits(x)
    nan = np.isnan(x)
    bad = np.nonzero((got != want) & ~nan)[0]
    assert bad.size == 0, [(hex(int(pats[k])), hex(int(got[k])), hex(int(want[k]))) for k in bad[:5]]
    got_f = (got[nan].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(got_f))


def pin_round_bf16_library(orc):
    rng = np.random.default_rng(404)
    _check_rounding(orc, rng.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32))
    low = np.arange(1 << 16, dtype=np.uint32)
    # every low half under: zero/subnormal, smallest normal, 1.0, largest
    # finite (overflow to inf), their negatives, and an infinity (NaNs).
    for hi in (0x0000, 0x0001, 0x0080, 0x3F80, 0x3F81, 0x7F7F, 0x7F80, 0x8000, 0xBF80, 0xFF7F,
               0xFF80):
        _check_rounding(orc, (np.uint32(hi) << 16) | low)


def _nearest_bf16_by_search(x):
    """The bf16 nearest to the finite float32 x, ties to the even pattern,
    by comparing x with every finite bf16 value and both infinities
    (counted as +-2^128 for the distance).  float64 distances are exact for
    the two nearest candidates."""
    pats = np.arange(1 << 16, dtype=np.uint32)
    keep = ((pats & 0x7F80) != 0x7F80) | ((pats & 0x7F) == 0)     # drop the NaNs
    pats = pats[keep]
    vals = (pats << 16).view(np.float32).astype(np.float64)
    vals = np.where(np.isinf(vals), np.sign(vals) * 2.0 ** 128, vals)
    d = np.abs(vals - float(x))
    best = np.nonzero(d == d.min())[0]
    cands = [int(pats[b]) for b in best]
    if len(cands) > 1:
        nonzero = [c for c in cands if c & 0x7FFF]
        if not nonzero:                      # +0 and -0: keep x's sign
            return 0x8000 if np.signbit(x) else 0
        cands = [c for c in cands if c % 2 == 0] or cands
    return cands[0]


def pin_round_bf16_global_nearest(orc):
    rng = np.random.default_rng(405)
    xs = [rng.standard_normal() * 10.0 ** rng.integers(-40, 39) for _ in range(120)]
    xs = np.array(xs, np.float32)
    ties = (rng.integers(0, 1 << 16, size=60).astype(np.uint32) << 16) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000].view(np.float32)
    xs = np.concatenate([xs, ties, np.array([3.4028235e38, -3.39e38, 1e-45, -1e-41], np.float32)])
    got = orc.round_bf16(xs)
    for x, g in zip(xs, got):
        assert int(g) == _nearest_bf16_by_search(x), (float(x), hex(int(g)))


def pin_round_bf16_worked_ties(orc):
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: to the even one, 1.
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: to 1 + 2^-6.
    # 2^-134 is half the smallest bf16 subnormal 2^-133: to +0.
    # 3*2^-134 lies between 2^-133 (odd) and 2^-132 (even): to 2^-132.
    # The largest finite float exceeds the largest bf16 by more than half
    # a unit of it: to infinity.
    xs = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 2.0 ** -134, 3 * 2.0 ** -134,
                   -(1 + 2.0 ** -8), 3.4028235e38], np.float32)
    want = [0x3F80, 0x3F82, 0x0000, 0x0002, 0xBF80, 0x7F80]
    assert [int(v) for v in orc.round_bf16(xs)] == want


def pin_bf16_shard_n2_is_library_sum(orc):
    # N = 2: the shard is fl32(g0 + g1) rounded once to bf16, which torch
    # computes as (a.float() + b.float()).to(bfloat16).
    shapes = [(37, 5), (64,)]
    grads = _rand_case(shapes, 2, 77)
    g = orc.geometry(shapes, 2)
    for R in (0, 1):
        got = orc.round_bf16(orc.rs(shapes, 2, R, grads))
        for i in range(len(shapes)):
            src, L = g.run(R, i)
            a = torch.from_numpy(grads[0][i].reshape(-1)[src:src + L].view(np.int16)).view(torch.bfloat16)
            b = torch.from_numpy(grads[1][i].reshape(-1)[src:src + L].view(np.int16)).view(torch.bfloat16)
            want = (a.float() + b.float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(got[g.off[i]:g.off[i] + L], want), (R, i)
            assert np.all(got[g.off[i] + L:g.off[i] + g.seg[i]] == 0)


# --------------------------------------------------------------------------
# all-gather placement
# --------------------------------------------------------------------------
def pin_ag_inverts_sharding(orc):
    for shapes in SWEEP:
        for N in (1, 2, 4, 5):
            for align in (1, 8):
                rng = np.random.default_rng(N * 31 + align)
                full = [rng.integers(1, 65535, size=int(np.prod(s)) if len(s) else 1)
                        .astype(np.uint16).reshape(s if len(s) else ()) for s in shapes]
                blocks = [brute.rank_block([torch.from_numpy(f.astype(np.int32)) for f in full],
                                           N, r, align).numpy().astype(np.uint16)
                          for r in range(N)]
                out = orc.ag(shapes, N, blocks, elem_bytes=2, align=align)
                for i in range(len(shapes)):
                    assert np.array_equal(out[i], full[i].reshape(-1)), (shapes, N, align, i)
                # slicing the gathered buffer at rank r gives shard r
                g = orc.geometry(shapes, N, align)
                for r in range(N):
                    for i in range(len(shapes)):
                        src, L = g.run(r, i)
                        blk = blocks[r][g.off[i]:g.off[i] + L]
                        assert np.array_equal(blk, full[i].reshape(-1)[src:src + L])


def pin_ag_fp32_and_untouched(orc):
    shapes = [(5, 7), (16,), (33, 4)]
    N = 4
    g = orc.geometry(shapes, N)
    rng = np.random.default_rng(5)
    blocks = [rng.integers(0, 2 ** 32 - 1, size=g.S, dtype=np.uint32) for _ in range(N)]
    # poison the padding: the placement must never read it
    for r in range(N):
        for i in range(3):
            src, L = g.run(r, i)
            blocks[r][g.off[i] + L:g.off[i] + g.seg[i]] = 0xDEADBEEF
    out = orc.ag(shapes, N, blocks, elem_bytes=4, fill=0xFFFFFFFF)
    want = brute.ag_by_concat(blocks, shapes, N)
    for i in range(3):
        assert np.array_equal(out[i], want[i].astype(np.uint32))
        assert not np.any(out[i] == 0xDEADBEEF)
        assert not np.any(out[i] == 0xFFFFFFFF)   # every element written


def pin_rs_then_ag_is_allreduce(orc):
    shapes = [(5, 7), (16,), (33, 4)]
    N = 4
    grads = _rand_case(shapes, N, 77)
    blocks = [orc.rs(shapes, N, R, grads).view(np.uint32) for R in range(N)]
    full = orc.ag(shapes, N, blocks, elem_bytes=4)
    for i, s in enumerate(shapes):
        n = int(np.prod(s))
        want = np.zeros(n, np.float32)
        for j in range(n):
            acc = brute.widen(int(grads[0][i].reshape(-1)[j]))
            for r in range(1, N):
                acc = np.float32(acc + brute.widen(int(grads[r][i].reshape(-1)[j])))
            want[j] = acc
        assert np.array_equal(full[i], want.view(np.uint32)), i


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_does_not_change_bits(orc):
    shapes = [(257, 9), (1000,)]
    grads = _rand_case(shapes, 8, 9)
    n = orc.threads()
    try:
        orc.set_threads(1)
        a = orc.rs(shapes, 8, 3, grads)
        orc.set_threads(max(2, n))
        b = orc.rs(shapes, 8, 3, grads)
    finally:
        orc.set_threads(n)
    assert np.array_equal(bits_f32(a), bits_f32(b))


def test_tiny_golden(orc):
    """Stored tiny-workload inputs and oracle outputs (written by
    tests/golden/make_golden.py, which calls only the oracle) still hold:
    guards the input generator and the oracle against silent drift."""
    gold = json.load(open(os.path.join(GOLDEN, "tiny_expected.json")))
    grads = workloads.all_grads(TINY)
    for r in range(TINY.world):
        for i in range(len(TINY.shapes)):
            assert workloads.bf16_bits(grads[r][i]).reshape(-1).tolist() == gold["grads"][r][i]
    gb = [[np.array(x, np.uint16) for x in rank] for rank in gold["grads"]]
    for R in range(TINY.world):
        out = orc.rs(TINY.shapes, TINY.world, R, gb)
        assert bits_f32(out).tolist() == gold["rs"][R]
        mean = orc.rs(TINY.shapes, TINY.world, R, gb, avg=True)
        assert bits_f32(mean).tolist() == gold["rs_mean"][R]
        assert orc.round_bf16(out).tolist() == gold["rs_bf16"][R]
        assert orc.pack(TINY.shapes, TINY.world, gb[R]).tolist() == gold["pack"][R]
