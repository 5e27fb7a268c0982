"""CPU oracle of the Atom copy/reduce collectives.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. It shares no code
with the GPU library: its C core (``oracle.c``) has its own element helpers,
offsets and loops, and ``brute.py`` is an independent pure-Python version
for tiny inputs.

Semantics (arXiv 2609.36954, "Purlin: Separating Orchestration from the
Datapath of Collectives"):

* ReduceScatter (Figure 4, top): y_k = sum over ranks r of partition k of x_r.
* AllGather (Figure 4, top): every rank receives all y_k in rank order.
* AllToAll (Figure 4, bottom): rank j receives partition j of every source.
* AllToAllV (Table 2, the variable-length variant): per-pair row counts.
* AllReduce (Figure 6): AllGather composed with ReduceScatter.
* MoE dispatch and combine (Table 2, expert parallelism): an AllToAllV
  whose destinations are experts chosen per token by routing ids, and its
  way back as a weighted sum over each token's k choices.

The sum is binary32 accumulation in rank order, rounded once to the element
type with round-to-nearest-even. Arrays are numpy: bf16 as raw ``uint16``,
fp32 as ``float32``.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, F32 = 0, 1
_NP = {BF16: np.uint16, F32: np.float32}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        vpp = ctypes.POINTER(ctypes.c_void_p)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        i64p = ctypes.POINTER(ctypes.c_int64)
        sig = {
            "orc_reduce": [i32, i64, i32, vpp, ctypes.c_void_p],
            "orc_reduce_scatter": [i32, i64, i32, vpp, vpp],
            "orc_all_gather": [i32, i64, i64, vpp, vpp],
            "orc_all_to_all": [i32, i64, i64, vpp, vpp],
            "orc_all_to_all_v": [i32, i64p, i64, vpp, vpp],
            "orc_all_reduce": [i32, i64, i32, vpp, vpp],
            "orc_reduce_scatter_v": [i32, i64p, i32, vpp, vpp],
            "orc_all_gather_v": [i32, i64p, i64, vpp, vpp],
            "orc_moe_route": [i32, i32, i32, i64, vpp, vpp, ctypes.c_void_p, ctypes.c_void_p],
            "orc_moe_dispatch": [i32, i32, i32, i64, vpp, vpp, i64, i64, vpp, vpp],
            "orc_moe_combine": [i32, i32, i32, i64, vpp, vpp, vpp, i64, i64, i32, vpp, vpp],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.orc_threads.argtypes = []
        lib.orc_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle arrays are uint16 (bf16 bits) or float32, not {a.dtype}")


def _ptrs(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _contig(arrays):
    return [np.ascontiguousarray(a).reshape(-1) for a in arrays]


def threads() -> int:
    return int(_load().orc_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for later calls; every result is independent of it
    (each output element is computed by one thread, in the fixed order)."""
    _check(_load().orc_set_threads(int(n)), "set_threads")


def reduce(srcs) -> np.ndarray:
    """dst[i] = round(sum_r srcs[r][i]) in rank order."""
    srcs = _contig(srcs)
    dt = _dtype_code(srcs[0])
    m = srcs[0].size
    assert all(s.size == m and s.dtype == srcs[0].dtype for s in srcs)
    dst = np.empty(m, dtype=_NP[dt])
    _check(_load().orc_reduce(len(srcs), m, dt, _ptrs(srcs), dst.ctypes.data),
           "reduce")
    return dst


def reduce_scatter(xs):
    """P inputs of P*n elements -> P outputs y_k of n elements."""
    xs = _contig(xs)
    P = len(xs)
    dt = _dtype_code(xs[0])
    assert xs[0].size % P == 0
    n = xs[0].size // P
    ys = [np.empty(n, dtype=_NP[dt]) for _ in range(P)]
    _check(_load().orc_reduce_scatter(P, n, dt, _ptrs(xs), _ptrs(ys)),
           "reduce_scatter")
    return ys


def all_gather(zs):
    """P inputs of n elements -> P outputs of P*n elements."""
    zs = _contig(zs)
    P = len(zs)
    n = zs[0].size
    outs = [np.empty(P * n, dtype=zs[0].dtype) for _ in range(P)]
    _check(_load().orc_all_gather(P, n, zs[0].itemsize, _ptrs(zs), _ptrs(outs)),
           "all_gather")
    return outs


def all_to_all(xs):
    """P inputs of P*n elements -> P outputs of P*n elements."""
    xs = _contig(xs)
    P = len(xs)
    assert xs[0].size % P == 0
    n = xs[0].size // P
    outs = [np.empty(P * n, dtype=xs[0].dtype) for _ in range(P)]
    _check(_load().orc_all_to_all(P, n, xs[0].itemsize, _ptrs(xs), _ptrs(outs)),
           "all_to_all")
    return outs


def all_to_all_v(xs, counts, row_elems: int):
    """AllToAllV over rows of ``row_elems`` elements; counts[r][j] rows r -> j."""
    xs = _contig(xs)
    P = len(xs)
    C = np.ascontiguousarray(np.asarray(counts, dtype=np.int64).reshape(P, P))
    dtype = xs[0].dtype
    R = C.sum(axis=0)
    outs = [np.empty(int(R[j]) * row_elems, dtype=dtype) for j in range(P)]
    _check(_load().orc_all_to_all_v(
        P, C.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        row_elems * xs[0].itemsize, _ptrs(xs), _ptrs(outs)), "all_to_all_v")
    return outs


def all_reduce(xs):
    """P inputs of P*n elements -> P identical outputs of P*n elements."""
    xs = _contig(xs)
    P = len(xs)
    dt = _dtype_code(xs[0])
    assert xs[0].size % P == 0
    n = xs[0].size // P
    outs = [np.empty(P * n, dtype=_NP[dt]) for _ in range(P)]
    _check(_load().orc_all_reduce(P, n, dt, _ptrs(xs), _ptrs(outs)), "all_reduce")
    return outs


def reduce_scatter_v(xs, cnt):
    """Partition k has cnt[k] elements on every rank -> y_k of cnt[k] elements."""
    xs = _contig(xs)
    P = len(xs)
    dt = _dtype_code(xs[0])
    c = np.ascontiguousarray(np.asarray(cnt, dtype=np.int64).reshape(P))
    ys = [np.empty(int(c[k]), dtype=_NP[dt]) for k in range(P)]
    _check(_load().orc_reduce_scatter_v(
        P, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), dt, _ptrs(xs),
        _ptrs(ys)), "reduce_scatter_v")
    return ys


def all_gather_v(zs):
    """z_k of any length -> P outputs holding all z_k in rank order."""
    zs = _contig(zs)
    P = len(zs)
    c = np.ascontiguousarray(np.array([z.size for z in zs], dtype=np.int64))
    T = int(c.sum())
    outs = [np.empty(T, dtype=zs[0].dtype) for _ in range(P)]
    _check(_load().orc_all_gather_v(
        P, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), zs[0].itemsize,
        _ptrs(zs), _ptrs(outs)), "all_gather_v")
    return outs


# ---------------------------------------------------------------- MoE (Table 2)

def _i32(arrays, n):
    out = [np.ascontiguousarray(a, dtype=np.int32).reshape(-1) for a in arrays]
    assert all(a.size == n for a in out)
    return out


def moe_route(ids, E: int, k: int):
    """ids: P arrays of T*k expert ids (token-major). Returns (pos, counts,
    recv): pos P arrays of T*k int32 rows (-1: invalid id), counts (P, E)
    int32, recv (P,) int64 rows each rank receives."""
    P = len(ids)
    n = np.asarray(ids[0]).size
    assert n % k == 0
    T = n // k
    ids = _i32(ids, n)
    pos = [np.empty(n, dtype=np.int32) for _ in range(P)]
    counts = np.zeros((P, E), dtype=np.int32)
    recv = np.zeros(P, dtype=np.int64)
    _check(_load().orc_moe_route(P, E, k, T, _ptrs(ids), _ptrs(pos), counts.ctypes.data,
                                 recv.ctypes.data), "moe_route")
    return pos, counts, recv


def moe_dispatch(xs, ids, pos, E: int, k: int, row_elems: int, cap: int, fill=None):
    """xs: P arrays of T*row_elems; returns P arrays of cap*row_elems
    (rows no entry lands on hold ``fill``, default zeros)."""
    P = len(xs)
    xs = _contig(xs)
    n = pos[0].size
    T = n // k
    ids = _i32(ids, n)
    pos = _i32(pos, n)
    outs = [np.zeros(cap * row_elems, dtype=xs[0].dtype) if fill is None else
            np.full(cap * row_elems, fill, dtype=xs[0].dtype) for _ in range(P)]
    _check(_load().orc_moe_dispatch(P, E, k, T, _ptrs(ids), _ptrs(pos), cap,
                                    row_elems * xs[0].itemsize, _ptrs(xs), _ptrs(outs)),
           "moe_dispatch")
    return outs


def moe_combine(ys, ids, pos, w, E: int, k: int, H: int, cap: int):
    """ys: P arrays of cap*H (expert outputs in dispatch layout); w: P arrays
    of T*k float32 weights. Returns P arrays of T*H."""
    P = len(ys)
    ys = _contig(ys)
    dt = _dtype_code(ys[0])
    n = pos[0].size
    T = n // k
    ids = _i32(ids, n)
    pos = _i32(pos, n)
    w = [np.ascontiguousarray(a, dtype=np.float32).reshape(-1) for a in w]
    outs = [np.empty(T * H, dtype=_NP[dt]) for _ in range(P)]
    _check(_load().orc_moe_combine(P, E, k, T, _ptrs(ids), _ptrs(pos), _ptrs(w), cap, H, dt,
                                   _ptrs(ys), _ptrs(outs)), "moe_combine")
    return outs
