"""Randomised pins of the oracle (hypothesis), beside the fixed sweeps of
test_oracle_pins.py: random shape lists, world sizes and alignments.

* geometry and the layout map equal the brute-force construction of
  tests/brute.py (shards cut with torch.chunk, blocks built by concatenation);
* the padding count is N*S - Psi, and the real elements biject onto the
  non-padding slots;
* pack equals the brute-force rank blocks (zero padding), and the
  all-gather of a packed slot gives the tensors back;
* the reduce-scatter of integer-valued gradients equals the exact int64 sum.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import brute

shape = st.one_of(
    st.just(()),
    st.tuples(st.integers(0, 40)),
    st.tuples(st.integers(0, 25), st.integers(1, 6)),
    st.tuples(st.integers(1, 9), st.integers(1, 4), st.integers(1, 3)),
)
case = st.tuples(st.lists(shape, min_size=1, max_size=5), st.integers(1, 9), st.integers(1, 8))
SETTINGS = settings(max_examples=60, deadline=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])


def _numel(s):
    return int(np.prod(s)) if len(s) else 1


@SETTINGS
@given(case)
def test_geometry_and_layout_match_brute_force(orc, c):
    shapes, N, align = c
    g = orc.geometry(shapes, N, align)
    pos, S = brute.segment_positions(shapes, N, align)
    assert g.S == S
    assert [(g.off[i], g.seg[i]) for i in range(len(shapes))] == pos
    where, total = brute.layout_map(shapes, N, align)
    assert total == N * g.S
    psi = sum(_numel(s) for s in shapes)
    assert len(where) == psi and len(set(where.values())) == psi     # a bijection
    for (i, j), flat in where.items():
        rows = g.inner[i]
        r = (j // rows) // g.c[i]
        src, L = g.run(r, i)
        assert flat == r * g.S + g.off[i] + (j - src) and j - src < L


@SETTINGS
@given(case, st.integers(0, 2 ** 31))
def test_pack_and_ag_match_brute_force(orc, c, seed):
    shapes, N, align = c
    rng = np.random.default_rng(seed)
    ts = [rng.integers(1, 65535, size=_numel(s)).astype(np.uint16) for s in shapes]
    slot = orc.pack(shapes, N, ts, align=align)
    tt = [torch.from_numpy(t.astype(np.int64)).reshape(s) for t, s in zip(ts, shapes)]
    want = torch.cat([brute.rank_block(tt, N, q, align, pad_value=0) for q in range(N)])
    assert np.array_equal(slot, want.numpy().astype(np.uint16))
    g = orc.geometry(shapes, N, align)
    back = orc.ag(shapes, N, [slot[q * g.S:(q + 1) * g.S] for q in range(N)], align=align)
    for i in range(len(shapes)):
        assert np.array_equal(back[i], ts[i])


@SETTINGS
@given(case, st.integers(0, 2 ** 31))
def test_rs_integer_values_are_exact(orc, c, seed):
    # integer values in [-8, 8] are exact in bf16 and in every partial fp32
    # sum of up to 9 ranks, so every order gives the int64 sum
    shapes, N, align = c
    rng = np.random.default_rng(seed)
    ints = [[rng.integers(-8, 9, size=_numel(s)) for s in shapes] for _ in range(N)]
    bits = [[(torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
              .numpy().view(np.uint16)) for a in rank] for rank in ints]
    g = orc.geometry(shapes, N, align)
    for R in {0, N - 1, N // 2}:
        out = orc.rs(shapes, N, R, bits, align=align)
        want = np.zeros(g.S, np.float32)
        for i in range(len(shapes)):
            src, L = g.run(R, i)
            tot = sum(ints[r][i][src:src + L] for r in range(N))
            want[g.off[i]:g.off[i] + L] = tot
        assert np.array_equal(out.view(np.uint32), want.view(np.uint32))
