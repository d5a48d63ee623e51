"""Python binding of the TIDE placement collectives (libtide.so).

Argument marshalling only: every step of tide_rs / tide_ag runs in the HIP
kernels of libtide.so.  PyTorch supplies device memory and streams.

    plan = Plan(shapes, world)                  # tide_plan_create
    rs(plan, rank, grads, out)                  # tide_rs  (TIDE-RS)
    ag(plan, rank_src, params)                  # tide_ag  (TIDE-AG placement)

TIDE-RS and TIDE-AG are described in "FSDP通信终局：TIDE零拷贝集合通信优化"
(kongchang.com), §"TIDE的设计思路：布局感知的零拷贝通信".
"""
import ctypes
import sys

import torch

from ._lib import lib

SMALL_FOOTPRINT = 0x1
COPY_ENGINE = 0x2
AVG = 0x4
GRAD_F16 = 0x8
GRAD_F32 = 0x10
OUT_BF16 = 0x20

# gradient dtype -> tide_rs flag selecting it
_GRAD_FLAG = {torch.bfloat16: 0, torch.float16: GRAD_F16, torch.float32: GRAD_F32}

_STATUS = {0: "TIDE_OK", 1: "TIDE_E_INVALID", 2: "TIDE_E_UNSUPPORTED", 3: "TIDE_E_NOMEM",
           4: "TIDE_E_HIP"}


class TideError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def _check(status):
    if status != 0:
        msg = lib().tide_last_error()
        raise TideError(status, msg.decode() if msg else "")


def _rows_inner(shape):
    shape = tuple(int(s) for s in shape)
    if not shape:
        return 1, 1
    inner = 1
    for s in shape[1:]:
        inner *= s
    return shape[0], inner


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """Shard geometry of a parameter list for `world` ranks (tide_plan)."""

    def __init__(self, shapes, world, align=1):
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        self.world = int(world)
        P = len(self.shapes)
        d0 = (ctypes.c_int64 * max(P, 1))(*[_rows_inner(s)[0] for s in self.shapes])
        inner = (ctypes.c_int64 * max(P, 1))(*[_rows_inner(s)[1] for s in self.shapes])
        h = ctypes.c_void_p()
        self._h = None
        self._destroy = lib().tide_plan_destroy
        _check(lib().tide_plan_create(self.world, P, d0, inner, int(align), ctypes.byref(h)))
        self._h = h
        self.S = int(lib().tide_plan_shard_numel(h))
        self.P = P
        # what a pointer table is checked against (compared by identity)
        self._sig = (self.world, tuple(self.shapes), self.S)

    def __del__(self, _finalizing=sys.is_finalizing):
        # At interpreter exit the HIP runtime may already be torn down (and
        # module globals cleared); the process is ending, so the plan's device
        # tables go with it.
        if getattr(self, "_h", None) is not None and not _finalizing():
            self._destroy(self._h)
        self._h = None

    @property
    def handle(self):
        return self._h

    def param(self, i):
        """(off_i, rows per rank c_i, seg_i)."""
        off, c, seg = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().tide_plan_param(self._h, i, ctypes.byref(off), ctypes.byref(c),
                                     ctypes.byref(seg)))
        return off.value, c.value, seg.value

    def real(self, rank, i):
        """(src, L): rank's shard of param i starts at element src, L real elements."""
        src, L = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().tide_plan_real(self._h, rank, i, ctypes.byref(src), ctypes.byref(L)))
        return src.value, L.value


class PointerTable:
    """A host array of device pointers kept alive with the tensors it names.
    Build it once and pass it to rs/ag repeatedly to skip re-marshalling.

    The kernels read as many bytes behind each pointer as the plan says, so
    a table is checked against the plan (element counts, dtype, device,
    contiguity) the first time it is used with that plan for a given call;
    later calls with the same plan skip the check."""

    def __init__(self, tensors, dtype=None):
        self.tensors = list(tensors)
        self.dtype = dtype
        self.array = (ctypes.c_void_p * max(len(self.tensors), 1))(
            *[t.data_ptr() if t is not None else None for t in self.tensors])
        self._checked = {}   # role -> signature of the plan it was checked against

    def check_len(self, n, what):
        """The library reads exactly n entries: refuse a table of another size."""
        if len(self.tensors) != n:
            raise ValueError(f"{what}: pointer table has {len(self.tensors)} entries, "
                             f"the plan needs {n}")

    def _ensure(self, plan, role, check):
        """Runs check() unless this table already passed it for this plan."""
        if self._checked.get(role) is not plan._sig:
            check()
            self._checked[role] = plan._sig


def _check_grads(plan, flat, dtype):
    """flat[r*P + i] is rank r's gradient of param i: all of `dtype`."""
    if dtype not in _GRAD_FLAG:
        raise TypeError(f"gradients must be bfloat16, float16 or float32, got {dtype}")
    for k, t in enumerate(flat):
        if t.dtype != dtype:
            r, i = divmod(k, plan.P)
            raise TypeError(f"grads[{r}][{i}] is {t.dtype}, the others are {dtype}")
    for k, t in enumerate(flat):
        r, i = divmod(k, plan.P)
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"grads[{r}][{i}] must be a contiguous device tensor")
        if t.numel() != _numel(plan.shapes[i]):
            raise ValueError(f"grads[{r}][{i}] has {t.numel()} elements, "
                             f"expected {_numel(plan.shapes[i])}")


def grad_table(plan, grads):
    """PointerTable for tide_rs: grads[r][i] = rank r's gradient of param i,
    all bf16, all fp16 or all fp32."""
    if len(grads) != plan.world:
        raise ValueError(f"expected {plan.world} ranks of gradients, got {len(grads)}")
    for r, rank in enumerate(grads):
        if len(rank) != plan.P:
            raise ValueError(f"rank {r}: expected {plan.P} gradients, got {len(rank)}")
    flat = [t for rank in grads for t in rank]
    dtype = flat[0].dtype if flat else torch.bfloat16
    table = PointerTable(flat, dtype)
    table._ensure(plan, "rs", lambda: _check_grads(plan, flat, dtype))
    return table


def _numel(shape):
    n = 1
    for s in shape:
        n *= s
    return n


def _rs_flags(plan, grads, out, small, avg):
    """Checks rs()'s arguments and returns (pointer table, flags)."""
    if not isinstance(grads, PointerTable):
        grads = grad_table(plan, grads)
    grads.check_len(plan.world * plan.P, "rs")
    grads._ensure(plan, "rs", lambda: _check_grads(plan, grads.tensors, grads.dtype))
    if out.dtype not in (torch.float32, torch.bfloat16) or not out.is_cuda \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 or bfloat16 device tensor")
    if out.numel() != plan.S:
        raise ValueError(f"out has {out.numel()} elements, expected S = {plan.S}")
    flags = _GRAD_FLAG.get(grads.dtype, 0)
    flags |= (SMALL_FOOTPRINT if small else 0) | (AVG if avg else 0)
    flags |= OUT_BF16 if out.dtype == torch.bfloat16 else 0
    return grads, flags


def rs(plan, rank, grads, out, small=False, max_workgroups=0, stream=None, avg=False):
    """TIDE-RS: write rank `rank`'s block (plan.S elements) into `out`.

    grads: list over ranks of lists over params of device tensors (bf16,
    fp16 or fp32, one dtype for all), or a PointerTable from grad_table().
    out: contiguous device tensor with plan.S elements (e.g. a row of an
    [N, S] buffer): float32 for the fp32 shard, bfloat16 for the fp32 result
    rounded once to bf16.  avg: write the mean (sum / N) instead of the sum."""
    grads, flags = _rs_flags(plan, grads, out, small, avg)
    _check(lib().tide_rs(plan.handle, int(rank), grads.array, ctypes.c_void_p(out.data_ptr()),
                         flags, int(max_workgroups), _stream_handle(stream)))


def rs_noalloc(plan, rank, grads, out, small=False, max_workgroups=0, stream=None, avg=False):
    """tide_rs_noalloc: rs() without any device allocation - its tables go
    into the library's fixed per-device scratch array, rewritten on `stream`
    by every call.  Same arguments and bit-identical result as rs().  Calls
    that overlap on one device (other streams, unordered) race on that
    array."""
    grads, flags = _rs_flags(plan, grads, out, small, avg)
    _check(lib().tide_rs_noalloc(plan.handle, int(rank), grads.array,
                                 ctypes.c_void_p(out.data_ptr()), flags, int(max_workgroups),
                                 _stream_handle(stream)))


_ELEM = {torch.bfloat16: 2, torch.float16: 2, torch.int16: 2, torch.float32: 4, torch.int32: 4}


def _check_ag(plan, blocks, params, e):
    """N rank blocks of at least S elements and P parameters of their sizes,
    all contiguous device tensors of one dtype of e bytes."""
    dt = blocks[0].dtype if blocks else None
    if dt not in _ELEM or _ELEM[dt] != e:
        raise TypeError(f"unsupported element type {dt} for {e}-byte elements")
    for r, b in enumerate(blocks):
        if b.dtype != dt or not b.is_cuda or not b.is_contiguous() or b.numel() < plan.S:
            raise ValueError(f"rank block {r} must be a contiguous {dt} device tensor "
                             f"of at least S elements")
    for i, t in enumerate(params):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"params[{i}] must be a contiguous {dt} device tensor")
        if t.numel() != _numel(plan.shapes[i]):
            raise ValueError(f"params[{i}] has {t.numel()} elements, "
                             f"expected {_numel(plan.shapes[i])}")


def ag_tables(plan, rank_src, params):
    """(PointerTable of rank blocks, PointerTable of params, element bytes)."""
    if isinstance(rank_src, torch.Tensor):
        if rank_src.numel() != plan.world * plan.S:
            raise ValueError(f"gathered buffer has {rank_src.numel()} elements, "
                             f"expected N*S = {plan.world * plan.S}")
        if not rank_src.is_contiguous():
            raise ValueError("gathered buffer must be contiguous")
        flat = rank_src.reshape(-1)
        blocks = [flat[r * plan.S:(r + 1) * plan.S] for r in range(plan.world)]
    else:
        blocks = list(rank_src)
    params = list(params)
    if len(blocks) != plan.world or len(params) != plan.P:
        raise ValueError("need one block per rank and one tensor per parameter")
    dt = blocks[0].dtype
    if dt not in _ELEM:
        raise TypeError(f"unsupported element type {dt}")
    e = _ELEM[dt]
    _check_ag(plan, blocks, params, e)
    src_t, dst_t = PointerTable(blocks), PointerTable(params)
    src_t._checked["ag"] = plan._sig
    dst_t._checked["ag"] = plan._sig
    return src_t, dst_t, e


def ag(plan, rank_src, params, small=False, max_workgroups=0, stream=None, tables=None,
       copy_engine=False):
    """TIDE-AG placement: scatter N rank blocks into full parameter tensors.

    rank_src: one contiguous N*S buffer (rank-major) or a list of N blocks.
    params: list of P full tensors of the same dtype (2- or 4-byte elements).
    tables: optional result of ag_tables() to skip re-marshalling.
    copy_engine: place the shards with SDMA copies instead of a kernel."""
    src_t, dst_t, e = tables if tables is not None else ag_tables(plan, rank_src, params)
    src_t.check_len(plan.world, "ag (rank blocks)")
    dst_t.check_len(plan.P, "ag (parameters)")
    if src_t._checked.get("ag") is not plan._sig or dst_t._checked.get("ag") is not plan._sig:
        _check_ag(plan, src_t.tensors, dst_t.tensors, e)
        src_t._checked["ag"] = dst_t._checked["ag"] = plan._sig
    flags = (SMALL_FOOTPRINT if small else 0) | (COPY_ENGINE if copy_engine else 0)
    _check(lib().tide_ag(plan.handle, src_t.array, dst_t.array, e, flags, int(max_workgroups),
                         _stream_handle(stream)))


def _slot_size_ok(plan, slot, what):
    if not slot.is_cuda or not slot.is_contiguous():
        raise ValueError(f"{what} must be a contiguous device tensor")
    if slot.numel() != plan.world * plan.S:
        raise ValueError(f"{what} has {slot.numel()} elements, expected N*S = "
                         f"{plan.world * plan.S}")


def _check_pack(plan, tensors, dtype):
    for i, t in enumerate(tensors):
        if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"tensors[{i}] must be a contiguous {dtype} device tensor")
        if t.numel() != _numel(plan.shapes[i]):
            raise ValueError(f"tensors[{i}] has {t.numel()} elements, "
                             f"expected {_numel(plan.shapes[i])}")


def pack(plan, tensors, slot, small=False, max_workgroups=0, stream=None):
    """Stage 1 of the two-stage TIDE-RS: lay one rank's per-parameter tensors
    out rank-major in `slot` (N*S elements of the tensors' dtype; for
    Slot-Reuse, the vacated all-gather buffer).  Padding and gaps become 0.

    tensors: list of P device tensors of one 2- or 4-byte dtype, or a
    PointerTable of them."""
    if slot.dtype not in _ELEM:
        raise TypeError(f"unsupported element type {slot.dtype}")
    if not isinstance(tensors, PointerTable):
        if len(tensors) != plan.P:
            raise ValueError(f"expected {plan.P} tensors, got {len(tensors)}")
        tensors = PointerTable(tensors, slot.dtype)
    tensors.check_len(plan.P, "pack")
    if tensors.dtype is not None and tensors.dtype != slot.dtype:
        raise TypeError(f"pack: tensors are {tensors.dtype}, the slot is {slot.dtype}")
    tensors._ensure(plan, ("pack", slot.dtype), lambda: _check_pack(plan, tensors.tensors,
                                                                    slot.dtype))
    _slot_size_ok(plan, slot, "slot")
    flags = SMALL_FOOTPRINT if small else 0
    _check(lib().tide_pack(plan.handle, tensors.array, ctypes.c_void_p(slot.data_ptr()),
                           _ELEM[slot.dtype], flags, int(max_workgroups),
                           _stream_handle(stream)))


def _check_slots(plan, slots, dtype):
    if dtype not in _GRAD_FLAG:
        raise TypeError(f"slots must be bfloat16, float16 or float32, got {dtype}")
    for r, t in enumerate(slots):
        if t.dtype != dtype:
            raise TypeError(f"slots[{r}] is {t.dtype}, the others are {dtype}")
        _slot_size_ok(plan, t, f"slots[{r}]")


def slot_table(plan, slots):
    """PointerTable for rs_slots: slots[r] = rank r's slot (N*S elements,
    bf16, fp16 or fp32, one dtype for all), or one [N, N*S] tensor."""
    if isinstance(slots, torch.Tensor):
        if slots.dim() != 2 or slots.shape[0] != plan.world:
            raise ValueError("a slot tensor must have shape [N, N*S]")
        slots = list(slots)
    if len(slots) != plan.world:
        raise ValueError(f"expected {plan.world} slots, got {len(slots)}")
    dtype = slots[0].dtype
    _check_slots(plan, slots, dtype)
    table = PointerTable(slots, dtype)
    table._checked["rs_slots"] = plan._sig
    return table


def rs_slots(plan, rank, slots, out, small=False, max_workgroups=0, stream=None, avg=False):
    """Stage 2 of the two-stage TIDE-RS: rank `rank`'s block from the N staged
    slots (see slot_table), bit-identical to rs() over the gradients they
    were packed from.  out, small, avg: as for rs()."""
    if not isinstance(slots, PointerTable):
        slots = slot_table(plan, slots)
    slots.check_len(plan.world, "rs_slots")
    slots._ensure(plan, "rs_slots", lambda: _check_slots(plan, slots.tensors, slots.dtype))
    if out.dtype not in (torch.float32, torch.bfloat16) or not out.is_cuda \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 or bfloat16 device tensor")
    if out.numel() != plan.S:
        raise ValueError(f"out has {out.numel()} elements, expected S = {plan.S}")
    flags = _GRAD_FLAG.get(slots.dtype, 0)
    flags |= (SMALL_FOOTPRINT if small else 0) | (AVG if avg else 0)
    flags |= OUT_BF16 if out.dtype == torch.bfloat16 else 0
    _check(lib().tide_rs_slots(plan.handle, int(rank), slots.array,
                               ctypes.c_void_p(out.data_ptr()), flags, int(max_workgroups),
                               _stream_handle(stream)))


__all__ = ["Plan", "PointerTable", "TideError", "SMALL_FOOTPRINT", "COPY_ENGINE", "AVG",
           "GRAD_F16", "GRAD_F32", "OUT_BF16", "grad_table",
           "ag_tables", "slot_table",
           "rs", "rs_noalloc", "ag", "pack", "rs_slots", "lib"]
