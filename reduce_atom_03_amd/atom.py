"""Python binding of libatom (include/atom.h): argument marshalling only.

Every entry point of the C ABI is exposed under the same name. Tensors are
accepted where the C side takes device pointers; the default stream is
torch's current stream on the tensors' device. There is no fallback: if the
shared library is missing or fails to load, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libatom.so")

MAX_RANKS = 16

# atom_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_TIMEOUT, ERR_NOMEM, ERR_LIMIT = range(7)
# ATOM_NOALLOC_RING_BYTES: ring of atom_collective_noalloc's fixed workspace
NOALLOC_RING_BYTES = 16 << 20
# atom_dtype
DT_BF16, DT_F32 = 0, 1
# atom_op
OP_COPY, OP_SUM = 0, 1
# atom_layout_kind
PARTITIONED, SHARD, GATHERED, TRANSPOSED = 0, 1, 2, 3
# atom_config flags
F_STAGED, F_NO_NT, F_XCD_ORDER, F_COUNTED = 0x1, 0x2, 0x4, 0x8
# atom_collective_kind
COLL_NONE, COLL_REDUCE_SCATTER, COLL_ALL_GATHER, COLL_ALL_TO_ALL, \
    COLL_ALL_TO_ALL_V, COLL_ALL_REDUCE, COLL_REDUCE_SCATTER_V, \
    COLL_ALL_GATHER_V = range(8)


class AtomLayout(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int),
        ("nranks", ctypes.c_int32),
        ("bufs", ctypes.POINTER(ctypes.c_void_p)),
        ("part_elems", ctypes.c_int64),
        ("counts", ctypes.POINTER(ctypes.c_int64)),
        ("row_elems", ctypes.c_int64),
        ("dtype", ctypes.c_int),
    ]


class AtomConfig(ctypes.Structure):
    _fields_ = [
        ("chunk_bytes", ctypes.c_int64),
        ("stages", ctypes.c_int32),
        ("num_wgs", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("ring_slots", ctypes.c_int32),
        ("piece_bytes", ctypes.c_int32),
        ("wait_us", ctypes.c_int32),
        ("lanes", ctypes.c_int32),
        ("jitter_us", ctypes.c_int32),
        ("jitter_seed", ctypes.c_uint32),
        ("snac_lead", ctypes.c_int32),
        ("trace", ctypes.c_void_p),
    ]


class AtomPlanInfo(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int),
        ("nranks", ctypes.c_int32),
        ("staged", ctypes.c_int32),
        ("vector_path", ctypes.c_int32),
        ("elems_per_rank_in", ctypes.c_int64),
        ("elems_per_rank_out", ctypes.c_int64 * MAX_RANKS),
        ("credited_bytes", ctypes.c_int64),
        ("chunk_bytes", ctypes.c_int64),
        ("num_chunks", ctypes.c_int64),
        ("ring_slots", ctypes.c_int32),
        ("num_wgs", ctypes.c_int32),
        ("lanes", ctypes.c_int32),
        ("stages", ctypes.c_int32),
        ("streaming_stores", ctypes.c_int32),
        ("grid_rows", ctypes.c_int32),
        ("shifted", ctypes.c_int32),
        ("snac_lead", ctypes.c_int32),
        ("snac_tasks", ctypes.c_int64),
        ("snac_tagged", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_ENTRIES = 1024, 16, 1 << 20


class AtomMoeRouting(ctypes.Structure):
    _fields_ = [
        ("nranks", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("tokens", ctypes.c_int64),
        ("expert_ids", ctypes.POINTER(ctypes.c_void_p)),
        ("positions", ctypes.POINTER(ctypes.c_void_p)),
        ("counts", ctypes.c_void_p),
        ("recv_rows", ctypes.c_void_p),
        ("scratch", ctypes.c_void_p),
    ]


EXPORTS = ("atom_copy", "atom_reduce", "atom_collective", "atom_collective_noalloc",
           "atom_plan_query",
           "atom_sync_status", "atom_bdp_chunk_bytes", "atom_status_string",
           "atom_last_error", "atom_version", "atom_moe_scratch_bytes",
           "atom_moe_route", "atom_moe_dispatch", "atom_moe_combine", "atom_device_clock_khz")


def _hip_runtimes() -> set:
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libatom not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    # torch ships its own HIP runtime. Load it first so that libatom binds to
    # that same runtime (same soname); loaded the other way round, the process
    # would map two HIP/HSA runtimes and the second sees no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    if len(_hip_runtimes()) > 1:
        raise ImportError("two HIP runtimes are mapped into this process: "
                          + ", ".join(sorted(_hip_runtimes())))
    vp = ctypes.c_void_p
    lib.atom_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.atom_copy.restype = ctypes.c_int
    lib.atom_reduce.argtypes = [vp, ctypes.POINTER(vp), ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_int, ctypes.c_int, vp]
    lib.atom_reduce.restype = ctypes.c_int
    lp = ctypes.POINTER(AtomLayout)
    lib.atom_collective.argtypes = [lp, lp, ctypes.c_int, ctypes.POINTER(AtomConfig), vp]
    lib.atom_collective.restype = ctypes.c_int
    lib.atom_collective_noalloc.argtypes = [lp, lp, ctypes.c_int, ctypes.POINTER(AtomConfig), vp]
    lib.atom_collective_noalloc.restype = ctypes.c_int
    lib.atom_plan_query.argtypes = [lp, lp, ctypes.c_int, ctypes.POINTER(AtomConfig),
                                    ctypes.POINTER(AtomPlanInfo)]
    lib.atom_plan_query.restype = ctypes.c_int
    lib.atom_sync_status.argtypes = [vp]
    lib.atom_sync_status.restype = ctypes.c_int
    lib.atom_bdp_chunk_bytes.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.atom_bdp_chunk_bytes.restype = ctypes.c_int64
    lib.atom_status_string.argtypes = [ctypes.c_int]
    lib.atom_status_string.restype = ctypes.c_char_p
    lib.atom_last_error.argtypes = []
    lib.atom_last_error.restype = ctypes.c_char_p
    lib.atom_version.argtypes = []
    lib.atom_version.restype = ctypes.c_int32
    lib.atom_device_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    lib.atom_device_clock_khz.restype = ctypes.c_int
    rp = ctypes.POINTER(AtomMoeRouting)
    vpp = ctypes.POINTER(vp)
    lib.atom_moe_scratch_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64]
    lib.atom_moe_scratch_bytes.restype = ctypes.c_int64
    lib.atom_moe_route.argtypes = [rp, vp]
    lib.atom_moe_route.restype = ctypes.c_int
    lib.atom_moe_dispatch.argtypes = [rp, vpp, vpp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                      ctypes.POINTER(AtomConfig), vp]
    lib.atom_moe_dispatch.restype = ctypes.c_int
    lib.atom_moe_combine.argtypes = [rp, vpp, vpp, vpp, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int, ctypes.POINTER(AtomConfig), vp]
    lib.atom_moe_combine.restype = ctypes.c_int
    return lib


lib = _load()


class AtomError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = f" [{atom_last_error()}]" if status == ERR_HIP else ""
        super().__init__(f"{what}: {atom_status_string(status)} ({status}){detail}")
        self.status = status


# ------------------------------------------------------------- marshalling

def _ptr(x) -> int:
    """Device address of a tensor (or an int address as given)."""
    if isinstance(x, int):
        return x
    if x is None:
        return 0
    return int(x.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise TypeError(f"libatom handles bfloat16 and float32, not {t.dtype}")


def _stream(stream, like=None) -> int:
    if stream is None:
        import torch
        dev = like.device if like is not None and hasattr(like, "device") else None
        return int(torch.cuda.current_stream(dev).cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int, what: str, check: bool) -> int:
    if check and status != OK:
        raise AtomError(status, what)
    return status


def layout(kind: int, bufs: Sequence, part_elems: int = 0, counts=None,
           row_elems: int = 1, dtype: Optional[int] = None) -> AtomLayout:
    """An atom_layout over P buffers (tensors or int device addresses).
    The returned structure keeps its pointer and count arrays alive."""
    P = len(bufs)
    arr = (ctypes.c_void_p * max(P, 1))(*[_ptr(b) for b in bufs])
    if dtype is None:
        dtype = _dtype_code(bufs[0])
    lay = AtomLayout(kind=kind, nranks=P,
                     bufs=ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
                     part_elems=int(part_elems), row_elems=int(row_elems), dtype=dtype)
    lay._keep = [arr]
    if counts is not None:
        flat = [int(c) for c in (counts.reshape(-1).tolist() if hasattr(counts, "reshape")
                                 else _flatten(counts))]
        carr = (ctypes.c_int64 * len(flat))(*flat)
        lay.counts = ctypes.cast(carr, ctypes.POINTER(ctypes.c_int64))
        lay._keep.append(carr)
    return lay


def _flatten(c):
    out = []
    for x in c:
        if isinstance(x, (list, tuple)):
            out.extend(x)
        else:
            out.append(x)
    return out


def config(chunk_bytes: int = 0, stages: int = 0, num_wgs: int = 0, flags: int = 0,
           ring_slots: int = 0, piece_bytes: int = 0, wait_us: int = 0,
           lanes: int = 0, jitter_us: int = 0, jitter_seed: int = 0,
           snac_lead: int = 0, trace: int = 0) -> AtomConfig:
    return AtomConfig(chunk_bytes=chunk_bytes, stages=stages, num_wgs=num_wgs,
                      flags=flags, ring_slots=ring_slots, piece_bytes=piece_bytes,
                      wait_us=wait_us, lanes=lanes, jitter_us=jitter_us,
                      jitter_seed=jitter_seed, snac_lead=snac_lead, trace=trace or None)


# --------------------------------------------------------- the C entry points

def atom_status_string(status: int) -> str:
    return lib.atom_status_string(int(status)).decode()


def atom_last_error() -> str:
    return lib.atom_last_error().decode()


def atom_version() -> int:
    return int(lib.atom_version())


def atom_device_clock_khz() -> int:
    """Rate of the clock behind atom_config.trace stamps (kHz)."""
    v = ctypes.c_int32(0)
    st = int(lib.atom_device_clock_khz(ctypes.byref(v)))
    if st != OK:
        raise RuntimeError(f"atom_device_clock_khz: {atom_status_string(st)}")
    return int(v.value)


def atom_bdp_chunk_bytes(bytes_per_s: float, round_trip_s: float) -> int:
    return int(lib.atom_bdp_chunk_bytes(float(bytes_per_s), float(round_trip_s)))


def atom_copy(dst, src, nbytes: Optional[int] = None, stream=None, check: bool = True) -> int:
    """Copy nbytes (default: all of src) from src to dst."""
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    st = lib.atom_copy(_ptr(dst), _ptr(src), int(nbytes), _stream(stream, dst))
    return _check(st, "atom_copy", check)


def atom_reduce(dst, srcs: Sequence, count: Optional[int] = None, dtype: Optional[int] = None,
                op: int = OP_SUM, stream=None, check: bool = True) -> int:
    """dst[i] = sum over r of srcs[r][i] (binary32, rank order, one rounding)."""
    n = len(srcs)
    arr = (ctypes.c_void_p * max(n, 1))(*[_ptr(s) for s in srcs])
    if count is None:
        count = dst.numel()
    if dtype is None:
        dtype = _dtype_code(dst)
    st = lib.atom_reduce(_ptr(dst), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), n,
                         int(count), dtype, op, _stream(stream, dst))
    return _check(st, "atom_reduce", check)


def atom_collective(inp: AtomLayout, out: AtomLayout, op: int, cfg: Optional[AtomConfig] = None,
                    stream=None, check: bool = True) -> int:
    st = lib.atom_collective(ctypes.byref(inp), ctypes.byref(out), op,
                             ctypes.byref(cfg) if cfg is not None else None,
                             _stream(stream))
    return _check(st, "atom_collective", check)


def atom_collective_noalloc(inp: AtomLayout, out: AtomLayout, op: int,
                            cfg: Optional[AtomConfig] = None, stream=None,
                            check: bool = True) -> int:
    """atom_collective whose staged calls use the library's fixed workspace
    (no device allocation)."""
    st = lib.atom_collective_noalloc(ctypes.byref(inp), ctypes.byref(out), op,
                                     ctypes.byref(cfg) if cfg is not None else None,
                                     _stream(stream))
    return _check(st, "atom_collective_noalloc", check)


def atom_plan_query(inp: AtomLayout, out: AtomLayout, op: int,
                    cfg: Optional[AtomConfig] = None):
    """(status, AtomPlanInfo) without touching the GPU."""
    info = AtomPlanInfo()
    st = lib.atom_plan_query(ctypes.byref(inp), ctypes.byref(out), op,
                             ctypes.byref(cfg) if cfg is not None else None,
                             ctypes.byref(info))
    return st, info


def atom_sync_status(stream=None) -> int:
    return int(lib.atom_sync_status(_stream(stream)))


# ------------------------------------------------- collectives by layout name

def reduce_scatter(xs: Sequence, ys: Sequence, cfg=None, stream=None, check=True) -> int:
    """Figure 4 (top): y_k = sum over r of partition k of x_r."""
    n = ys[0].numel()
    return atom_collective(layout(PARTITIONED, xs, n), layout(SHARD, ys, n), OP_SUM, cfg,
                           _stream(stream, ys[0]), check)


def all_gather(zs: Sequence, outs: Sequence, cfg=None, stream=None, check=True) -> int:
    """Figure 4 (top): every output holds all z_k in rank order."""
    n = zs[0].numel()
    return atom_collective(layout(SHARD, zs, n), layout(GATHERED, outs, n), OP_COPY, cfg,
                           _stream(stream, outs[0]), check)


def all_to_all(xs: Sequence, outs: Sequence, cfg=None, stream=None, check=True) -> int:
    """Figure 4 (bottom): output j holds partition j of every source."""
    n = xs[0].numel() // len(xs)
    return atom_collective(layout(PARTITIONED, xs, n), layout(TRANSPOSED, outs, n), OP_COPY,
                           cfg, _stream(stream, outs[0]), check)


def all_to_all_v(xs: Sequence, outs: Sequence, counts, row_elems: int, cfg=None, stream=None,
                 check=True) -> int:
    """Table 2 (V): counts[r][j] rows of row_elems elements from r to j."""
    return atom_collective(layout(PARTITIONED, xs, 0, counts, row_elems),
                           layout(TRANSPOSED, outs, 0, None, row_elems), OP_COPY, cfg,
                           _stream(stream, outs[0]), check)


def all_reduce(xs: Sequence, outs: Sequence, cfg=None, stream=None, check=True) -> int:
    """Figure 6: AllGather(ReduceScatter(x)); every output is the full sum."""
    n = xs[0].numel() // len(xs)
    return atom_collective(layout(PARTITIONED, xs, n), layout(GATHERED, outs, n), OP_SUM, cfg,
                           _stream(stream, outs[0]), check)


def reduce_scatter_v(xs: Sequence, ys: Sequence, counts, row_elems: int = 1, cfg=None,
                     stream=None, check=True) -> int:
    """Table 2 (V): partition k holds counts[k] rows on every rank."""
    return atom_collective(layout(PARTITIONED, xs, 0, counts, row_elems),
                           layout(SHARD, ys, 0, None, row_elems), OP_SUM, cfg,
                           _stream(stream, ys[0]), check)


def all_gather_v(zs: Sequence, outs: Sequence, counts, row_elems: int = 1, cfg=None,
                 stream=None, check=True) -> int:
    """Table 2 (V): z_k holds counts[k] rows; outputs hold all in rank order."""
    return atom_collective(layout(SHARD, zs, 0, counts, row_elems),
                           layout(GATHERED, outs, 0, None, row_elems), OP_COPY, cfg,
                           _stream(stream, outs[0]), check)


# ------------------------------------------- MoE dispatch / combine (Table 2)

def _ptr_array(xs):
    arr = (ctypes.c_void_p * max(len(xs), 1))(*[_ptr(x) for x in xs])
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))


def atom_moe_scratch_bytes(nranks: int, num_experts: int, topk: int, tokens: int) -> int:
    return int(lib.atom_moe_scratch_bytes(int(nranks), int(num_experts), int(topk), int(tokens)))


def moe_routing(expert_ids: Sequence, num_experts: int, topk: int, positions: Sequence,
                counts, recv_rows, scratch, tokens: Optional[int] = None) -> AtomMoeRouting:
    """An atom_moe_routing over caller-owned device arrays (tensors or int
    addresses). The structure keeps its pointer arrays alive."""
    P = len(expert_ids)
    if tokens is None:
        tokens = expert_ids[0].numel() // topk
    ids_arr, ids_p = _ptr_array(expert_ids)
    pos_arr, pos_p = _ptr_array(positions)
    rt = AtomMoeRouting(nranks=P, num_experts=int(num_experts), topk=int(topk), reserved=0,
                        tokens=int(tokens), expert_ids=ids_p, positions=pos_p,
                        counts=_ptr(counts), recv_rows=_ptr(recv_rows), scratch=_ptr(scratch))
    rt._keep = [ids_arr, pos_arr]
    return rt


def moe_alloc_routing(expert_ids: Sequence, num_experts: int, topk: int) -> AtomMoeRouting:
    """moe_routing with its positions, counts, recv_rows and scratch
    allocated by torch on the ids' device (kept alive by the structure as
    .positions_t, .counts_t, .recv_t)."""
    import torch
    P = len(expert_ids)
    dev = expert_ids[0].device
    T = expert_ids[0].numel() // topk
    pos = [torch.empty(T * topk, dtype=torch.int32, device=dev) for _ in range(P)]
    counts = torch.empty(P * num_experts, dtype=torch.int32, device=dev)
    recv = torch.empty(P, dtype=torch.int64, device=dev)
    nbytes = atom_moe_scratch_bytes(P, num_experts, topk, T)
    scratch = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    rt = moe_routing(expert_ids, num_experts, topk, pos, counts, recv, scratch, T)
    rt._keep += [list(expert_ids), scratch]
    rt.positions_t, rt.counts_t, rt.recv_t = pos, counts, recv
    return rt


def atom_moe_route(rt: AtomMoeRouting, stream=None, check: bool = True) -> int:
    st = lib.atom_moe_route(ctypes.byref(rt), _stream(stream))
    return _check(st, "atom_moe_route", check)


def atom_moe_dispatch(rt: AtomMoeRouting, x: Sequence, out: Sequence, capacity_rows: int,
                      row_elems: int, dtype: Optional[int] = None, stream=None,
                      check: bool = True, cfg: Optional[AtomConfig] = None) -> int:
    xa, xp = _ptr_array(x)
    oa, op = _ptr_array(out)
    if dtype is None:
        dtype = _dtype_code(x[0])
    st = lib.atom_moe_dispatch(ctypes.byref(rt), xp, op, int(capacity_rows), int(row_elems),
                               dtype, ctypes.byref(cfg) if cfg is not None else None,
                               _stream(stream, out[0] if out else None))
    return _check(st, "atom_moe_dispatch", check)


def atom_moe_combine(rt: AtomMoeRouting, y: Sequence, weights: Sequence, out: Sequence,
                     capacity_rows: int, row_elems: int, dtype: Optional[int] = None,
                     stream=None, check: bool = True, cfg: Optional[AtomConfig] = None) -> int:
    ya, yp = _ptr_array(y)
    wa, wp = _ptr_array(weights)
    oa, op = _ptr_array(out)
    if dtype is None:
        dtype = _dtype_code(out[0])
    st = lib.atom_moe_combine(ctypes.byref(rt), yp, wp, op, int(capacity_rows), int(row_elems),
                              dtype, ctypes.byref(cfg) if cfg is not None else None,
                              _stream(stream, out[0] if out else None))
    return _check(st, "atom_moe_combine", check)
