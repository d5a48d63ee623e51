"""TIDE collectives as PyTorch custom operators (torch.library).

    import parameter_layout_collectives_amd.torch_ops as tops
    pid = tops.register_plan(plan)
    torch.ops.tide.rs(pid, rank, grads_flat, out, small, avg)
    torch.ops.tide.ag(pid, gathered, params, small, copy_engine)
    torch.ops.tide.pack(pid, tensors, slot, small)
    torch.ops.tide.rs_slots(pid, rank, slots, out, small, avg)

They are how a training framework calls the collectives in place of
FSDP2's gradient pack and all-gather copy-out ("FSDP通信终局：TIDE零拷贝集合
通信优化", §"TIDE的设计思路": TIDE sits under FSDP2 and keeps its
per-parameter storage).  Each operator declares the tensors it writes, so
autograd and torch.compile see the mutation; the work itself runs in the
library's kernels on the current stream.  grads_flat is rank-major: entry
r*P + i is rank r's gradient of parameter i.  Marshalling walks the tensor
lists on every call; hot loops that reuse the same tensors call the plain
binding with a PointerTable instead.
"""
import itertools
import threading
from typing import List

import torch

from . import Plan, ag, pack, rs, rs_slots

_PLANS = {}
_LOCK = threading.Lock()
_IDS = itertools.count(1)


def register_plan(plan: Plan) -> int:
    """An integer id for `plan` that the operators accept (kept until
    unregister_plan)."""
    with _LOCK:
        pid = next(_IDS)
        _PLANS[pid] = plan
    return pid


def unregister_plan(pid: int) -> None:
    with _LOCK:
        _PLANS.pop(pid, None)


def _plan(pid):
    try:
        return _PLANS[pid]
    except KeyError:
        raise ValueError(f"no plan registered under id {pid}") from None


def _by_rank(flat, plan):
    if len(flat) != plan.world * plan.P:
        raise ValueError(f"expected N*P = {plan.world * plan.P} gradients, got {len(flat)}")
    P = plan.P
    return [list(flat[r * P:(r + 1) * P]) for r in range(plan.world)]


@torch.library.custom_op("tide::rs", mutates_args=("out",))
def rs_op(pid: int, rank: int, grads: List[torch.Tensor], out: torch.Tensor,
          small: bool = False, avg: bool = False) -> None:
    plan = _plan(pid)
    rs(plan, rank, _by_rank(grads, plan), out, small=small, avg=avg)


@rs_op.register_fake
def _(pid, rank, grads, out, small=False, avg=False):
    return None


@torch.library.custom_op("tide::ag", mutates_args=("params",))
def ag_op(pid: int, gathered: torch.Tensor, params: List[torch.Tensor], small: bool = False,
          copy_engine: bool = False) -> None:
    ag(_plan(pid), gathered, list(params), small=small, copy_engine=copy_engine)


@ag_op.register_fake
def _(pid, gathered, params, small=False, copy_engine=False):
    return None


@torch.library.custom_op("tide::pack", mutates_args=("slot",))
def pack_op(pid: int, tensors: List[torch.Tensor], slot: torch.Tensor,
            small: bool = False) -> None:
    pack(_plan(pid), list(tensors), slot, small=small)


@pack_op.register_fake
def _(pid, tensors, slot, small=False):
    return None


@torch.library.custom_op("tide::rs_slots", mutates_args=("out",))
def rs_slots_op(pid: int, rank: int, slots: torch.Tensor, out: torch.Tensor,
                small: bool = False, avg: bool = False) -> None:
    rs_slots(_plan(pid), rank, slots, out, small=small, avg=avg)


@rs_slots_op.register_fake
def _(pid, rank, slots, out, small=False, avg=False):
    return None
