"""Helpers shared by the GPU parity tests: host copies of device data and
the oracle's expected values for them.  Inputs always come from the seeded
generators in workloads.py; expected values always come from the oracle."""
import sys

import numpy as np
import torch

import parameter_layout_collectives_amd as tide

F32_SENTINEL = 0x7FBADBAD      # a NaN pattern no kernel produces
BF16_SENTINEL = 0x7FBD


def note(msg):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def bits16(t):
    """Device or host bf16/int16 tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits32(t):
    return t.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def rank_slices(geom, grads, R):
    """slices[r][i] = host copy of the elements of rank r's gradient of param
    i that fall in rank R's shard (what tide_rs reads).  The shard offsets
    come from the oracle's geometry `geom`, not from the library's plan."""
    out = []
    for rank in grads:
        row = []
        for i, g in enumerate(rank):
            src, L = geom.run(R, i)
            row.append(bits16(g.reshape(-1)[src:src + L]))
        out.append(row)
    return out


def expected_rs(orc, shapes, N, R, grads, plan=None, align=1):
    """The oracle's block R of the reduce-scatter of `grads` (device or host
    bf16 tensors).  `plan` is accepted for the callers' convenience and not
    used: every offset comes from the oracle."""
    geom = orc.geometry(shapes, N, align)
    return orc.rs_slices(shapes, N, R, rank_slices(geom, grads, R), align=align)


def same_f32(got, want):
    """Bitwise equality, except that NaNs compare by class only.  An output
    word still holding the exact sentinel pattern (never written) fails even
    where a NaN is expected, unless the oracle expects that very pattern."""
    g = np.asarray(got, np.float32)
    w = np.asarray(want, np.float32)
    if np.any((g.view(np.uint32) == F32_SENTINEL) & (w.view(np.uint32) != F32_SENTINEL)):
        return False
    gn, wn = np.isnan(g), np.isnan(w)
    if not np.array_equal(gn, wn):
        return False
    return np.array_equal(g[~gn].view(np.uint32), w[~wn].view(np.uint32))


def same_bf16(got, want):
    """Bitwise equality of bf16 bit patterns (uint16), NaNs by class only; an
    unwritten word (the exact sentinel) fails as in same_f32."""
    g = np.asarray(got, np.uint16)
    w = np.asarray(want, np.uint16)
    if np.any((g == BF16_SENTINEL) & (w != BF16_SENTINEL)):
        return False
    gn = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    wn = ((w & 0x7F80) == 0x7F80) & ((w & 0x7F) != 0)
    return np.array_equal(gn, wn) and np.array_equal(g[~gn], w[~wn])


def first_mismatch16(got, want):
    g = np.asarray(got, np.uint16)
    w = np.asarray(want, np.uint16)
    idx = np.nonzero(g != w)[0]
    if idx.size == 0:
        return None
    k = int(idx[0])
    return k, hex(int(g[k])), hex(int(w[k])), int(idx.size)


def first_mismatch(got, want):
    g = np.asarray(got, np.float32).view(np.uint32)
    w = np.asarray(want, np.float32).view(np.uint32)
    idx = np.nonzero(g != w)[0]
    if idx.size == 0:
        return None
    k = int(idx[0])
    return k, hex(int(g[k])), hex(int(w[k])), int(idx.size)


def run_rs(plan, R, grads_or_table, out, **kw):
    """tide_rs, then wait for it."""
    tide.rs(plan, R, grads_or_table, out, **kw)
    torch.cuda.synchronize()
