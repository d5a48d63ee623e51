"""CPU oracle for the TIDE placement collectives (numpy front end over oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library and its Python
binding never import it, and it imports nothing from them.

What it computes (cited by page title and section):
  * ``geometry``: dim-0 shards with ceil padding laid out rank-major
    ("FSDP通信终局：TIDE零拷贝集合通信优化", §"FSDP2通信开销的根源";
    tqpw.cn "FSDP技术演进全景图" §2.1).
  * ``rs``: this rank's fp32 block of the rank-order binary32 sum of the
    ranks' bf16 gradients (TIDE article §"TIDE的设计思路", TIDE-RS).
  * ``ag``: rank blocks placed straight into full per-parameter tensors
    (TIDE article §"TIDE的设计思路", TIDE-AG; apxml "Communication volume
    analysis" §"分片中的通信原语").
  * ``rs_traffic``: elements pulled from peers, (N-1)/N*Psi per rank on
    average (apxml "Communication volume analysis" §"带宽饱和和节点扩展").
  * ``pack``: one rank's per-parameter tensors laid out rank-major (the
    all-gather buffer's layout), padding and gaps zero: the staging of the
    two-stage reduce-scatter (TIDE article §"TIDE的设计思路", two-stage
    pipeline and Slot-Reuse).
  * ``round_bf16``: fp32 -> bf16, round to nearest, ties to even; a bf16
    shard is the fp32 block from ``rs`` rounded once (the reduction itself
    stays fp32: tqpw.cn blog §3.2, TIDE article §"TIDE的设计思路").

Arrays of bf16 values are carried as numpy ``uint16`` bit patterns.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

# gradient element types of the reduce-scatter (codes of oracle.c)
DTYPES = {"bf16": 0, "f16": 1, "f32": 2}

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def rows_inner(shape):
    """(d0, inner) of a row-major tensor: dim 0 and the product of the rest.

    A 0-dim tensor counts as shape [1]."""
    shape = tuple(int(s) for s in shape)
    if len(shape) == 0:
        return 1, 1
    inner = 1
    for s in shape[1:]:
        inner *= s
    return shape[0], inner


class Geometry:
    """Shard geometry of a parameter list for N ranks."""

    def __init__(self, shapes, N, align, c, seg, off, S):
        self.shapes = [tuple(int(x) for x in s) for s in shapes]
        self.N = int(N)
        self.align = int(align)
        self.d0 = [rows_inner(s)[0] for s in self.shapes]
        self.inner = [rows_inner(s)[1] for s in self.shapes]
        self.c = list(c)
        self.seg = list(seg)
        self.off = list(off)
        self.S = int(S)

    @property
    def P(self):
        return len(self.shapes)

    @property
    def psi(self):
        return sum(d * n for d, n in zip(self.d0, self.inner))

    def numel(self, i):
        return self.d0[i] * self.inner[i]

    def run(self, r, i):
        """(src, L): rank r's shard of param i starts at element src of the
        full tensor and holds L real elements."""
        rows = min(self.c[i], max(0, self.d0[i] - r * self.c[i]))
        return r * self.c[i] * self.inner[i], rows * self.inner[i]


class Oracle:
    """Handle on one build of oracle.c (tests may load planted-mistake builds)."""

    def __init__(self, path=DEFAULT_LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with `python oracle/build_oracle.py`")
        lib = ctypes.CDLL(path)
        lib.oracle_geometry.argtypes = [_i32, _i32, _p, _p, _i64, _p, _p, _p, _p]
        lib.oracle_shard_run.argtypes = [_i32, _i64, _i64, _i32, _p, _p]
        lib.oracle_rs.argtypes = [_i32, _i32, _p, _p, _i64, _i32, _p, _p]
        lib.oracle_rs_slices.argtypes = [_i32, _i32, _p, _p, _i64, _i32, _p, _p]
        lib.oracle_rs_typed.argtypes = [_i32, _i32, _p, _p, _i64, _i32, ctypes.c_int,
                                        ctypes.c_int, _p, _p]
        lib.oracle_rs_slices_typed.argtypes = [_i32, _i32, _p, _p, _i64, _i32, ctypes.c_int,
                                               ctypes.c_int, _p, _p]
        lib.oracle_ag.argtypes = [_i32, _i32, _p, _p, _i64, _i32, _p, _p]
        lib.oracle_rs_traffic.argtypes = [_i32, _i32, _p, _p, _i64, _i32, _p, _p]
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_round_bf16.argtypes = [_p, _p, _i64]
        lib.oracle_pack.argtypes = [_i32, _i32, _p, _p, _i64, _i32, _p, _p]
        for fn in (lib.oracle_geometry, lib.oracle_shard_run, lib.oracle_rs,
                   lib.oracle_rs_slices, lib.oracle_rs_typed, lib.oracle_rs_slices_typed,
                   lib.oracle_ag, lib.oracle_rs_traffic, lib.oracle_threads,
                   lib.oracle_round_bf16, lib.oracle_pack):
            fn.restype = ctypes.c_int
        lib.oracle_set_threads.restype = None
        self.lib = lib
        self.path = path

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _dims(shapes):
        d0 = np.array([rows_inner(s)[0] for s in shapes], dtype=np.int64)
        inner = np.array([rows_inner(s)[1] for s in shapes], dtype=np.int64)
        return d0, inner

    @staticmethod
    def _ptrs(arrays):
        return (ctypes.c_void_p * len(arrays))(
            *[a.ctypes.data if a is not None and a.size else None for a in arrays])

    # -- API ---------------------------------------------------------------
    def geometry(self, shapes, N, align=1):
        P = len(shapes)
        d0, inner = self._dims(shapes)
        c = np.zeros(P, np.int64)
        seg = np.zeros(P, np.int64)
        off = np.zeros(P, np.int64)
        S = np.zeros(1, np.int64)
        rc = self.lib.oracle_geometry(N, P, d0.ctypes.data, inner.ctypes.data, align,
                                      c.ctypes.data, seg.ctypes.data, off.ctypes.data,
                                      S.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_geometry: invalid arguments")
        return Geometry(shapes, N, align, c.tolist(), seg.tolist(), off.tolist(), int(S[0]))

    def shard_run(self, N, shape, r):
        d0, inner = rows_inner(shape)
        src = np.zeros(1, np.int64)
        L = np.zeros(1, np.int64)
        if self.lib.oracle_shard_run(N, d0, inner, r, src.ctypes.data, L.ctypes.data) != 0:
            raise ValueError("oracle_shard_run: invalid arguments")
        return int(src[0]), int(L[0])

    @staticmethod
    def _elems(a, dtype):
        """Flat contiguous element array: uint16 bit patterns for bf16/f16,
        float32 (or uint32 bit patterns, viewed as float32) for f32."""
        if dtype == "f32":
            a = np.ascontiguousarray(a)
            if a.dtype != np.float32:
                a = a.astype(np.uint32).view(np.float32) if a.dtype == np.uint32 else \
                    np.ascontiguousarray(a, dtype=np.float32)
            return a.reshape(-1)
        return np.ascontiguousarray(a, dtype=np.uint16).reshape(-1)

    def rs(self, shapes, N, R, grads, align=1, dtype="bf16", avg=False):
        """grads[r][i]: rank r's gradient of param i (any shape with d0*inner
        elements; uint16 bits for bf16/f16, float32 for f32).  Returns rank
        R's fp32 block (S,): rank-order sum, or its mean if avg."""
        P = len(shapes)
        g = self.geometry(shapes, N, align)
        flat = []
        for r in range(N):
            for i in range(P):
                a = self._elems(grads[r][i], dtype)
                assert a.size == g.numel(i), (r, i, a.size, g.numel(i))
                flat.append(a)
        d0, inner = self._dims(shapes)
        out = np.empty(g.S, np.float32)
        rc = self.lib.oracle_rs_typed(N, P, d0.ctypes.data, inner.ctypes.data, align, R,
                                      DTYPES[dtype], int(bool(avg)), self._ptrs(flat),
                                      out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_rs_typed: invalid arguments")
        return out

    def round_bf16(self, x):
        """fp32 values (float32 array, or uint32 bit patterns) -> uint16 bf16
        bit patterns, each rounded to nearest with ties to even."""
        x = np.asarray(x)
        if x.dtype == np.uint32:
            x = x.view(np.float32)
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, np.uint16)
        if self.lib.oracle_round_bf16(x.ctypes.data, out.ctypes.data, x.size) != 0:
            raise ValueError("oracle_round_bf16: invalid arguments")
        return out

    def rs_slices(self, shapes, N, R, slices, align=1, dtype="bf16", avg=False):
        """slices[r][i]: the L(R,i) elements of rank r's gradient of param i
        that fall in rank R's shard.  Returns rank R's block (S,)."""
        P = len(shapes)
        g = self.geometry(shapes, N, align)
        flat = []
        for r in range(N):
            for i in range(P):
                a = self._elems(slices[r][i], dtype)
                assert a.size == g.run(R, i)[1], (r, i, a.size)
                flat.append(a)
        d0, inner = self._dims(shapes)
        out = np.empty(g.S, np.float32)
        rc = self.lib.oracle_rs_slices_typed(N, P, d0.ctypes.data, inner.ctypes.data, align, R,
                                             DTYPES[dtype], int(bool(avg)), self._ptrs(flat),
                                             out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_rs_slices_typed: invalid arguments")
        return out

    def ag(self, shapes, N, rank_blocks, elem_bytes=2, align=1, fill=None):
        """rank_blocks[r]: rank r's block of S elements (uint16 for 2-byte,
        uint32 for 4-byte elements).  Returns the list of full tensors (flat).

        `fill` pre-sets every output element (default 0) so a test can see
        which elements the placement never wrote."""
        P = len(shapes)
        g = self.geometry(shapes, N, align)
        dt = {2: np.uint16, 4: np.uint32}[elem_bytes]
        src = []
        for r in range(N):
            b = np.ascontiguousarray(rank_blocks[r]).view(dt).reshape(-1)
            assert b.size >= g.S, (r, b.size, g.S)
            src.append(b)
        params = [np.full(g.numel(i), 0 if fill is None else fill, dtype=dt) for i in range(P)]
        d0, inner = self._dims(shapes)
        rc = self.lib.oracle_ag(N, P, d0.ctypes.data, inner.ctypes.data, align, elem_bytes,
                                self._ptrs(src), self._ptrs(params))
        if rc != 0:
            raise ValueError("oracle_ag: invalid arguments")
        return params

    def pack(self, shapes, N, tensors, elem_bytes=2, align=1):
        """tensors[i]: one rank's tensor of param i (uint16 bits for 2-byte,
        uint32 for 4-byte elements).  Returns its rank-major slot (N*S,)."""
        P = len(shapes)
        g = self.geometry(shapes, N, align)
        dt = {2: np.uint16, 4: np.uint32}[elem_bytes]
        src = []
        for i in range(P):
            a = np.ascontiguousarray(tensors[i]).view(dt).reshape(-1)
            assert a.size == g.numel(i), (i, a.size, g.numel(i))
            src.append(a)
        slot = np.empty(N * g.S, dt)
        d0, inner = self._dims(shapes)
        rc = self.lib.oracle_pack(N, P, d0.ctypes.data, inner.ctypes.data, align, elem_bytes,
                                  self._ptrs(src), slot.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_pack: invalid arguments")
        return slot

    def rs_traffic(self, shapes, N, R, align=1):
        """(real, padded) element counts rank R pulls from its N-1 peers."""
        P = len(shapes)
        d0, inner = self._dims(shapes)
        real = np.zeros(1, np.int64)
        padded = np.zeros(1, np.int64)
        rc = self.lib.oracle_rs_traffic(N, P, d0.ctypes.data, inner.ctypes.data, align, R,
                                        real.ctypes.data, padded.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_rs_traffic: invalid arguments")
        return int(real[0]), int(padded[0])

    def threads(self):
        return int(self.lib.oracle_threads())

    def set_threads(self, n):
        self.lib.oracle_set_threads(int(n))


_default = None


def default():
    """The oracle built from oracle.c in this directory."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
