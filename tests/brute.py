"""Brute-force construction of the rank-major layout, used to pin the oracle.

This is deliberately a different route to the same definitions than the
oracle takes.  The oracle computes offsets and run lengths in closed form;
here every shard is cut with ``torch.chunk`` along dim 0 (the rows of a
parameter split into ceil-sized groups, one per rank, trailing ranks short
or empty), padded by concatenation, and rank blocks are built by
concatenating padded shards in parameter order.  Pure Python / torch on tiny
inputs only.

Layout definition: "FSDP通信终局：TIDE零拷贝集合通信优化" §"FSDP2通信开销的根源"
(rank-major: one rank's elements contiguous, rank blocks in sequence);
tqpw.cn "FSDP技术演进全景图" §2.1 (each of N ranks keeps 1/N).
"""
from fractions import Fraction

import numpy as np
import torch


def _as_rows(t: torch.Tensor):
    """View a tensor as [d0, inner] (0-dim -> [1, 1])."""
    if t.dim() == 0:
        return t.reshape(1, 1)
    inner = 1
    for d in t.shape[1:]:
        inner *= d
    return t.reshape(t.shape[0], inner)


def shard_rows(t: torch.Tensor, N: int):
    """The N dim-0 shards of t (each [rows, inner]) and the padded row count."""
    rows = _as_rows(t)
    d0 = rows.shape[0]
    if d0 == 0:
        return [rows[0:0] for _ in range(N)], 0
    chunks = list(torch.chunk(rows, N, dim=0))
    c = chunks[0].shape[0]
    while len(chunks) < N:
        chunks.append(rows[0:0])
    return chunks, c


def padded_shard(t: torch.Tensor, N: int, r: int, pad_value=0):
    """Rank r's shard of t, flattened and padded with `pad_value` to c rows."""
    chunks, c = shard_rows(t, N)
    s = chunks[r]
    inner = _as_rows(t).shape[1]
    pad = torch.full(((c - s.shape[0]) * inner,), pad_value, dtype=t.dtype)
    return torch.cat([s.reshape(-1), pad])


def rank_block(tensors, N: int, r: int, align: int = 1, pad_value=0):
    """Rank r's block: its padded shards of every tensor, in order, each
    starting at a multiple of `align` elements (gaps and tail filled)."""
    parts = []
    pos = 0
    for t in tensors:
        gap = (-pos) % align
        if gap:
            parts.append(torch.full((gap,), pad_value, dtype=t.dtype))
            pos += gap
        s = padded_shard(t, N, r, pad_value)
        parts.append(s)
        pos += s.numel()
    gap = (-pos) % align
    if gap:
        parts.append(torch.full((gap,), pad_value, dtype=tensors[0].dtype))
    if not parts:
        return torch.zeros(0, dtype=tensors[0].dtype)
    return torch.cat(parts)


def segment_positions(shapes, N: int, align: int = 1):
    """(start, padded length) of each parameter inside a rank block, found
    by walking the padded shards in order (no closed form)."""
    out = []
    pos = 0
    for s in shapes:
        t = torch.zeros(s, dtype=torch.int8)
        pos += (-pos) % align
        seg = padded_shard(t, N, 0).numel()
        out.append((pos, seg))
        pos += seg
    pos += (-pos) % align
    return out, pos


def layout_map(shapes, N: int, align: int = 1):
    """Enumerate every element: returns {(i, j): flat position in the N*S
    rank-major buffer}.  Built by tagging each element with a unique id and
    reading the ids back out of the brute-force rank blocks."""
    tagged = []
    next_id = 1
    ids = {}
    for i, s in enumerate(shapes):
        n = int(np.prod(s)) if len(s) else 1
        t = torch.arange(next_id, next_id + n, dtype=torch.int64).reshape(s)
        for j in range(n):
            ids[next_id + j] = (i, j)
        next_id += n
        tagged.append(t)
    flat = torch.cat([rank_block(tagged, N, r, align, pad_value=0) for r in range(N)])
    where = {}
    for pos, v in enumerate(flat.tolist()):
        if v:
            where[ids[v]] = pos
    return where, flat.numel()


def widen(bits: int) -> np.float32:
    return np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]


def rs_rank_order(grads_bits, shapes, N: int, R: int, align: int = 1):
    """Rank R's fp32 block: per element, rank-order binary32 sum of the
    widened bf16 values (numpy float32 scalar adds, one at a time)."""
    blocks = []
    for r in range(N):
        ts = [torch.from_numpy(np.asarray(g, dtype=np.uint16).astype(np.int64)).reshape(s)
              for g, s in zip(grads_bits[r], shapes)]
        blocks.append(rank_block(ts, N, R, align, pad_value=-1).tolist())
    S = len(blocks[0])
    out = np.zeros(S, dtype=np.float32)
    with np.errstate(all="ignore"):
        for k in range(S):
            if blocks[0][k] < 0:          # padding or alignment gap
                out[k] = np.float32(0.0)
                continue
            acc = widen(blocks[0][k])
            for r in range(1, N):
                acc = np.float32(acc + widen(blocks[r][k]))
            out[k] = acc
    return out


def exact_sum(values_bits):
    """Exact rational sum of bf16 values given as bit patterns (finite)."""
    total = Fraction(0)
    for b in values_bits:
        f = float(widen(int(b)))
        total += Fraction(f)
    return total


def ag_by_concat(rank_blocks, shapes, N: int, align: int = 1):
    """Full tensors rebuilt from rank blocks by cutting each block at the
    walked segment positions and concatenating the real rows of the ranks."""
    pos, _ = segment_positions(shapes, N, align)
    out = []
    for i, s in enumerate(shapes):
        probe = torch.zeros(s, dtype=torch.int8)
        chunks, c = shard_rows(probe, N)
        start, seg = pos[i]
        pieces = []
        for r in range(N):
            n_real = chunks[r].numel()
            pieces.append(torch.as_tensor(rank_blocks[r][start:start + n_real]))
        full = torch.cat(pieces) if pieces else torch.zeros(0)
        out.append(full.numpy())
    return out


def round_f32(q: Fraction) -> np.float32:
    """The binary32 value nearest to the rational q, ties to even (normal
    range), found by exact comparison of the neighbours of a first guess."""
    c = np.float32(float(q))
    with np.errstate(all="ignore"):
        cands = (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf)))
    best = None
    for cand in cands:
        d = abs(Fraction(float(cand)) - q)
        even = (int(np.array([cand], np.float32).view(np.uint32)[0]) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, cand)
    return np.float32(best[1])
