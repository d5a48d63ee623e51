"""Host-side checks of libtide.so that need no GPU.

* the library loads and exports every function include/tide.h declares;
* tide_plan_* geometry equals the CPU oracle's on a sweep of shapes
  (the plan code and the oracle share no code);
* every argument error returns its status and message before anything is
  enqueued (these calls never reach the HIP runtime).
"""
import ctypes
import os
import re

import pytest

import parameter_layout_collectives_amd as tide
from parameter_layout_collectives_amd._lib import SIGNATURES, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tide.h")

E_INVALID, E_UNSUPPORTED = 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tide_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(SIGNATURES)


def test_status_strings():
    L = lib()
    assert L.tide_status_string(0) == b"TIDE_OK"
    assert L.tide_status_string(4) == b"TIDE_E_HIP"


SHAPE_SWEEP = [
    [(5, 7), (16,), (33, 4)],
    [(0, 5), (7,), (3, 2, 2), ()],
    [(9, 1), (8, 8), (11, 3)],
    [(4096, 4096), (1024, 4096), (14336, 4096), (4096,)],
]


@pytest.mark.parametrize("shapes", SHAPE_SWEEP)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 8, 64])
@pytest.mark.parametrize("align", [1, 4, 64])
def test_plan_matches_oracle(orc, shapes, N, align):
    plan = tide.Plan(shapes, N, align)
    g = orc.geometry(shapes, N, align)
    assert plan.S == g.S
    for i in range(len(shapes)):
        assert plan.param(i) == (g.off[i], g.c[i], g.seg[i])
        for r in range(N):
            assert plan.real(r, i) == g.run(r, i)


def _create(world, dims, align=1):
    P = len(dims)
    d0 = (ctypes.c_int64 * max(P, 1))(*[d for d, _ in dims])
    inner = (ctypes.c_int64 * max(P, 1))(*[n for _, n in dims])
    h = ctypes.c_void_p(1234)
    st = lib().tide_plan_create(world, P, d0, inner, align, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("world,dims,align,needle", [
    (0, [(4, 4)], 1, "world"),
    (70000, [(4, 4)], 1, "world"),
    (2, [], 1, "nparams"),
    (2, [(-1, 4)], 1, "negative"),
    (2, [(4, -4)], 1, "negative"),
    (2, [(4, 4)], 0, "align"),
    (2, [(2 ** 62, 4)], 1, "overflow"),
    (2, [(2 ** 40, 2 ** 20), (2 ** 40, 2 ** 20)], 1, "overflow"),
])
def test_plan_create_errors(world, dims, align, needle):
    st, h = _create(world, dims, align)
    assert st == E_INVALID
    assert h.value is None
    assert needle in lib().tide_last_error().decode()


def test_plan_query_errors():
    plan = tide.Plan([(4, 4)], 2)
    x = ctypes.c_int64()
    L = lib()
    assert L.tide_plan_param(plan.handle, 1, ctypes.byref(x), None, None) == E_INVALID
    assert L.tide_plan_param(plan.handle, -1, None, None, None) == E_INVALID
    assert L.tide_plan_real(plan.handle, 2, 0, None, None) == E_INVALID
    assert L.tide_plan_real(None, 0, 0, None, None) == E_INVALID
    assert L.tide_plan_shard_numel(None) == -1
    assert L.tide_plan_world(plan.handle) == 2
    assert L.tide_plan_nparams(plan.handle) == 1
    L.tide_plan_destroy(None)


def _ptrs(vals):
    return (ctypes.c_void_p * len(vals))(*vals)


# Fake, never-dereferenced device addresses: every call below must be
# rejected by validation before the library touches the HIP runtime.
A = 0x7F0000000000


def _rs(plan, rank, grads, out, flags=0, max_wg=0):
    return lib().tide_rs(plan.handle if plan else None, rank, grads,
                         ctypes.c_void_p(out), flags, max_wg, None)


def test_rs_argument_errors():
    plan = tide.Plan([(4, 4), (8,)], 2)        # S = 8 + 4 = 12
    good = _ptrs([A, A + 0x10000, A + 0x20000, A + 0x30000])
    out = A + 0x100000
    L = lib()
    assert _rs(None, 0, good, out) == E_INVALID
    assert _rs(plan, 2, good, out) == E_INVALID and b"rank" in L.tide_last_error()
    assert _rs(plan, -1, good, out) == E_INVALID
    assert _rs(plan, 0, good, out, flags=0x2) == E_UNSUPPORTED   # copy engine: AG only
    assert b"tide_ag" in L.tide_last_error()
    assert _rs(plan, 0, good, out, max_wg=-1) == E_INVALID
    assert _rs(plan, 0, None, out) == E_INVALID and b"grads" in L.tide_last_error()
    assert _rs(plan, 0, good, 0) == E_INVALID and b"out is NULL" in L.tide_last_error()
    assert _rs(plan, 0, good, out + 2) == E_INVALID and b"aligned" in L.tide_last_error()
    assert _rs(plan, 0, _ptrs([A, None, A + 0x20000, A + 0x30000]), out) == E_INVALID
    assert _rs(plan, 0, _ptrs([A + 1, A + 0x10000, A + 0x20000, A + 0x30000]), out) == E_INVALID
    # out overlaps what rank 0 reads of rank 1's first gradient (elements 0..7)
    assert _rs(plan, 0, good, A + 0x20000 + 8) == E_INVALID
    assert b"overlaps" in L.tide_last_error()
    # gradient element types: both type flags, fp32 pointers 2- but not 4-aligned
    assert _rs(plan, 0, good, out, flags=0x18) == E_INVALID
    assert b"both" in L.tide_last_error()
    assert _rs(plan, 0, _ptrs([A, A + 0x10002, A + 0x20000, A + 0x30000]), out,
               flags=0x10) == E_INVALID
    assert b"element size" in L.tide_last_error()
    # fp32 gradients read 4 bytes per element: out at 16 bytes into rank 1's
    # first gradient overlaps elements 4..7 only when they are 4 bytes wide
    assert _rs(plan, 0, good, A + 0x20000 + 16, flags=0x10) == E_INVALID
    assert _rs(plan, 0, good, out, flags=0x40) == E_UNSUPPORTED
    # bf16 output: 2-byte elements, so an odd address is misaligned; the
    # written span is 2*S = 24 bytes, so out 8 bytes before the elements read
    # from rank 1's first gradient overlaps them.
    assert _rs(plan, 0, good, out + 1, flags=0x20) == E_INVALID
    assert b"aligned" in L.tide_last_error()
    assert _rs(plan, 0, good, A + 0x20000 - 8, flags=0x20) == E_INVALID
    assert b"overlaps" in L.tide_last_error()


def test_rs_empty_plan_is_a_noop():
    # S = 0: nothing to write, so nothing is launched and no HIP call is made.
    plan = tide.Plan([(0, 3)], 4)
    assert plan.S == 0
    assert _rs(plan, 3, None, 0) == 0


def _ag(plan, srcs, dsts, e=2, flags=0, max_wg=0):
    return lib().tide_ag(plan.handle if plan else None, srcs, dsts, e, flags, max_wg, None)


def test_ag_argument_errors():
    plan = tide.Plan([(4, 4), (8,)], 2)        # S = 12; param sizes 16, 8
    srcs = _ptrs([A, A + 0x1000])
    dsts = _ptrs([A + 0x10000, A + 0x20000])
    L = lib()
    assert _ag(None, srcs, dsts) == E_INVALID
    assert _ag(plan, srcs, dsts, e=3) == E_INVALID and b"elem_bytes" in L.tide_last_error()
    assert _ag(plan, srcs, dsts, flags=0x8) == E_UNSUPPORTED
    assert _ag(plan, srcs, dsts, flags=0x3) == E_UNSUPPORTED   # small + copy engine
    assert b"exclude" in L.tide_last_error()
    assert _ag(plan, srcs, dsts, max_wg=-5) == E_INVALID
    assert _ag(plan, None, dsts) == E_INVALID
    assert _ag(plan, srcs, None) == E_INVALID
    assert _ag(plan, _ptrs([A, None]), dsts) == E_INVALID
    assert _ag(plan, _ptrs([A + 1, A + 0x1000]), dsts) == E_INVALID
    assert _ag(plan, srcs, _ptrs([A + 0x10000, A + 0x20002]), e=4) == E_INVALID
    # destinations overlapping each other
    assert _ag(plan, srcs, _ptrs([A + 0x10000, A + 0x10000 + 30])) == E_INVALID
    assert b"overlaps" in L.tide_last_error()
    # destination overlapping a source element that is read
    assert _ag(plan, srcs, _ptrs([A + 0x10000, A + 0x1000 + 4])) == E_INVALID


def test_ag_empty_plan_is_a_noop():
    plan = tide.Plan([(0, 3), (0,)], 4)
    assert _ag(plan, None, None) == 0


def _pack(plan, tensors, slot, e=2, flags=0, max_wg=0):
    return lib().tide_pack(plan.handle if plan else None, tensors, ctypes.c_void_p(slot), e,
                           flags, max_wg, None)


def test_pack_argument_errors():
    plan = tide.Plan([(4, 4), (8,)], 2)        # S = 12; tensor sizes 16, 8
    ts = _ptrs([A, A + 0x1000])
    slot = A + 0x10000
    L = lib()
    assert _pack(None, ts, slot) == E_INVALID
    assert _pack(plan, ts, slot, e=8) == E_INVALID and b"elem_bytes" in L.tide_last_error()
    assert _pack(plan, ts, slot, flags=0x2) == E_UNSUPPORTED
    assert _pack(plan, ts, slot, flags=0x4) == E_UNSUPPORTED
    assert _pack(plan, ts, slot, max_wg=-1) == E_INVALID
    assert _pack(plan, None, slot) == E_INVALID
    assert _pack(plan, ts, 0) == E_INVALID and b"slot is NULL" in L.tide_last_error()
    assert _pack(plan, ts, slot + 1) == E_INVALID and b"aligned" in L.tide_last_error()
    assert _pack(plan, ts, slot + 2, e=4) == E_INVALID
    assert _pack(plan, _ptrs([A, None]), slot) == E_INVALID
    assert _pack(plan, _ptrs([A + 1, A + 0x1000]), slot) == E_INVALID
    # the slot (2*12 elements = 48 bytes) overlaps tensor 1 (bytes 0x1000..0x1010)
    assert _pack(plan, ts, A + 0x1000 - 40) == E_INVALID
    assert b"overlaps" in L.tide_last_error()


def test_pack_empty_plan_is_a_noop():
    plan = tide.Plan([(0, 3)], 4)
    assert _pack(plan, None, 0) == 0


def _rss(plan, rank, slots, out, flags=0, max_wg=0):
    return lib().tide_rs_slots(plan.handle if plan else None, rank, slots, ctypes.c_void_p(out),
                               flags, max_wg, None)


def test_rs_slots_argument_errors():
    plan = tide.Plan([(4, 4), (8,)], 2)        # S = 12; block 1 of a slot = bytes 24..48
    slots = _ptrs([A, A + 0x1000])
    out = A + 0x100000
    L = lib()
    assert _rss(None, 0, slots, out) == E_INVALID
    assert _rss(plan, 2, slots, out) == E_INVALID and b"rank" in L.tide_last_error()
    assert _rss(plan, 0, slots, out, flags=0x2) == E_UNSUPPORTED
    assert _rss(plan, 0, slots, out, flags=0x40) == E_UNSUPPORTED
    assert _rss(plan, 0, slots, out, flags=0x18) == E_INVALID
    assert _rss(plan, 0, slots, out, max_wg=-1) == E_INVALID
    assert _rss(plan, 0, None, out) == E_INVALID
    assert _rss(plan, 0, slots, 0) == E_INVALID and b"out is NULL" in L.tide_last_error()
    assert _rss(plan, 0, slots, out + 2) == E_INVALID and b"aligned" in L.tide_last_error()
    assert _rss(plan, 0, slots, out + 1, flags=0x20) == E_INVALID
    assert _rss(plan, 0, _ptrs([A, None]), out) == E_INVALID
    assert _rss(plan, 0, _ptrs([A + 1, A + 0x1000]), out) == E_INVALID
    assert _rss(plan, 0, _ptrs([A, A + 0x1002]), out, flags=0x10) == E_INVALID
    # out overlaps the real elements of block 1 of slot 1 (read for rank 1)
    assert _rss(plan, 1, slots, A + 0x1000 + 24) == E_INVALID
    assert b"overlaps" in L.tide_last_error()


def test_python_binding_rejects_bad_tensors():
    import torch
    plan = tide.Plan([(4, 4)], 2)
    cpu = [[torch.zeros(4, 4, dtype=torch.bfloat16)] for _ in range(2)]
    with pytest.raises(ValueError):
        tide.grad_table(plan, cpu)                   # not device tensors
    with pytest.raises(TypeError):
        tide.grad_table(plan, [[torch.zeros(4, 4, dtype=torch.int32)] for _ in range(2)])
    with pytest.raises(TypeError):   # one dtype for all gradients
        tide.grad_table(plan, [[torch.zeros(4, 4, dtype=torch.bfloat16)],
                               [torch.zeros(4, 4, dtype=torch.float16)]])
    with pytest.raises(ValueError):
        tide.grad_table(plan, cpu[:1])


class _DeviceStub:
    """Passes the binding's tensor checks (device, contiguous, size, dtype)
    but points at address 0, which the library refuses before enqueuing
    anything: a check that wrongly let it through still launches nothing."""

    is_cuda = True

    def __init__(self, n, dtype):
        self.n, self.dtype = n, dtype

    def is_contiguous(self):
        return True

    def numel(self):
        return self.n

    def data_ptr(self):
        return 0


def test_pointer_tables_are_checked_against_each_plan():
    """A table whose tensors fit one plan is refused by another plan with
    the same numbers of ranks and parameters but larger shapes: the kernels
    would read past the ends of its tensors.  With its own plan it passes
    the table checks and stops at the next check (a host `out`)."""
    import torch
    bf = torch.bfloat16
    small = tide.Plan([(4, 4), (8,)], 2)
    large = tide.Plan([(400, 400), (8,)], 2)
    host_out = torch.zeros(large.S)

    grads = tide.PointerTable([_DeviceStub(16, bf), _DeviceStub(8, bf)] * 2, bf)
    with pytest.raises(ValueError, match="elements"):
        tide.rs(large, 0, grads, host_out)
    with pytest.raises(ValueError, match="out must be"):
        tide.rs(small, 0, grads, torch.zeros(small.S))
    with pytest.raises(ValueError, match="elements"):      # checked again for the other plan
        tide.rs(large, 0, grads, host_out)
    wrong_dtype = tide.PointerTable([_DeviceStub(16, bf), _DeviceStub(8, bf)] * 2, torch.float32)
    with pytest.raises(TypeError):
        tide.rs(small, 0, wrong_dtype, torch.zeros(small.S))

    blocks = tide.PointerTable([_DeviceStub(small.S, bf)] * 2)
    params = tide.PointerTable([_DeviceStub(16, bf), _DeviceStub(8, bf)])
    with pytest.raises(ValueError):
        tide.ag(large, None, None, tables=(blocks, params, 2))
    with pytest.raises(TypeError):                          # 2-byte tensors, 4-byte elements
        tide.ag(small, None, None, tables=(blocks, params, 4))

    with pytest.raises(ValueError, match="elements"):
        tide.pack(large, params, torch.zeros(2 * large.S, dtype=bf))
    slots = tide.PointerTable([_DeviceStub(2 * small.S, bf)] * 2, bf)
    with pytest.raises(ValueError, match="elements"):
        tide.rs_slots(large, 0, slots, host_out)


def test_custom_ops_registered():
    """The PyTorch operators exist and declare the tensors they write."""
    import torch
    import parameter_layout_collectives_amd.torch_ops  # noqa: F401 - registers the ops
    schemas = {n: str(getattr(torch.ops.tide, n).default._schema)
               for n in ("rs", "ag", "pack", "rs_slots")}
    assert "Tensor(a3!) out" in schemas["rs"]
    assert "Tensor(a2!)[] params" in schemas["ag"]
    assert "Tensor(a2!) slot" in schemas["pack"]
    assert "Tensor(a3!) out" in schemas["rs_slots"]


@pytest.mark.filterwarnings("ignore:.*LeafSpec.*:FutureWarning")   # torch.export's own pytree use
def test_custom_ops_trace_with_their_mutations():
    """torch.export traces a step that calls tide::rs then tide::ag and reads
    the reduce-scatter's output (fake tensors only: no kernel runs).  After
    functionalization the graph records `out` and every parameter as mutated
    inputs, and the read after the reduce-scatter takes its result."""
    import torch
    import parameter_layout_collectives_amd.torch_ops as tops
    shapes = [(5, 7), (16,), (33, 4)]
    plan = tide.Plan(shapes, 4)
    pid = tops.register_plan(plan)
    try:
        class Step(torch.nn.Module):
            def forward(self, flat, out, gathered, params):
                torch.ops.tide.rs(pid, 1, flat, out, False, False)
                torch.ops.tide.ag(pid, gathered, params, False, False)
                return out * 2.0

        flat = [torch.zeros(s, dtype=torch.bfloat16) for _ in range(4) for s in shapes]
        out = torch.zeros(plan.S)
        gathered = torch.zeros(4 * plan.S, dtype=torch.bfloat16)
        params = [torch.zeros(s, dtype=torch.bfloat16) for s in shapes]
        ep = torch.export.export(Step(), (flat, out, gathered, params)).run_decompositions()
        mutated = ep.graph_signature.user_inputs_to_mutate
        assert sorted(mutated.values()) == ["out", "params_0", "params_1", "params_2"]
        code = ep.graph_module.code
        assert "tide.rs.default" in code and "tide.ag.default" in code
        rs_result = [k for k, v in mutated.items() if v == "out"][0]
        assert f"aten.mul.Tensor({rs_result}, 2.0)" in code
    finally:
        tops.unregister_plan(pid)


def test_binding_refuses_pointer_tables_of_another_plan():
    """A table built for another plan would make the library read past the
    end of the host array: the binding refuses it before any call."""
    import torch
    plan = tide.Plan([(4, 4), (8,)], 2)                 # N*P = 4
    other = tide.PointerTable([torch.zeros(1)] * 6)      # 6 entries (CPU tensors, never read)
    out = torch.zeros(plan.S)
    with pytest.raises(ValueError, match="pointer table"):
        tide.rs(plan, 0, other, out)
    with pytest.raises(ValueError, match="pointer table"):
        tide.ag(plan, None, None, tables=(other, other, 2))
    with pytest.raises(ValueError, match="pointer table"):
        tide.pack(plan, other, torch.zeros(2 * plan.S))
    with pytest.raises(ValueError, match="pointer table"):
        tide.rs_slots(plan, 0, other, out)


def _rs_noalloc(plan, rank, grads, out, flags=0, max_wg=0):
    return lib().tide_rs_noalloc(plan.handle if plan else None, rank, grads,
                                 ctypes.c_void_p(out), flags, max_wg, None)


def test_rs_noalloc_validates_like_tide_rs():
    # the same checks as tide_rs, before anything reaches the HIP runtime
    plan = tide.Plan([(4, 4), (8,)], 2)
    good = _ptrs([A, A + 0x10000, A + 0x20000, A + 0x30000])
    out = A + 0x100000
    L = lib()
    assert _rs_noalloc(None, 0, good, out) == E_INVALID
    assert _rs_noalloc(plan, 2, good, out) == E_INVALID and b"rank" in L.tide_last_error()
    assert _rs_noalloc(plan, 0, good, out, flags=0x2) == E_UNSUPPORTED
    assert _rs_noalloc(plan, 0, None, out) == E_INVALID
    assert _rs_noalloc(plan, 0, good, A + 0x20000 + 8) == E_INVALID
    assert b"overlaps" in L.tide_last_error()
    empty = tide.Plan([(0, 3)], 4)
    assert _rs_noalloc(empty, 3, None, 0) == 0


def test_rs_noalloc_rejects_tables_beyond_its_scratch():
    L = lib()
    # 2^32 elements in one parameter: 2^20 tiles of 4096 elements need 16 MiB
    # of tile list, beyond the 8 MiB scratch array.
    big = tide.Plan([(1 << 32,)], 1)
    assert _rs_noalloc(big, 0, _ptrs([A]), A + (1 << 40)) == E_INVALID
    msg = L.tide_last_error()
    assert b"scratch" in msg and b"8388608" in msg
    # 4096 ranks x 300 parameters: a 9.8 MB pointer table alone
    N, P = 4096, 300
    plan = tide.Plan([(N,)] * P, N)
    ptrs = _ptrs([A + 16 * k for k in range(N * P)])
    assert _rs_noalloc(plan, 0, ptrs, A + (1 << 36)) == E_INVALID
    assert b"scratch" in L.tide_last_error()


def test_rs_noalloc_limit_counts_small_footprint_tiles():
    # Above 16 ranks the small footprint walks 1024-element tiles.  One
    # [17, 2^29 + 64] parameter over 17 ranks: 2^17 + 1 default tiles (2 MiB
    # of tile list) but 2^19 + 1 small-footprint tiles (8 MiB + 16 B), so only
    # the small-footprint call exceeds the scratch array, by its exact need:
    # 512 bytes of tables (440 rounded up to 256) plus 16 bytes per tile.
    L = lib()
    N = 17
    plan = tide.Plan([(N, (1 << 29) + 64)], N)
    assert plan.S == (1 << 29) + 64
    ptrs = _ptrs([A + r * (1 << 35) for r in range(N)])
    assert _rs_noalloc(plan, 0, ptrs, A + (1 << 40), flags=0x1) == E_INVALID
    need = 512 + 16 * ((1 << 19) + 1)
    assert f"need {need} bytes".encode() in L.tide_last_error()
