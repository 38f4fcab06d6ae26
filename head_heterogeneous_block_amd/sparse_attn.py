"""ctypes binding of libsparse_attn.so (argument marshalling only).

Each function has the name of the C entry point it calls and does no compute of
its own: it turns torch tensors into device pointers, shapes into an
``sa_attn_desc``, per-head budgets into ``sa_head_budget[]``, and passes the
current HIP stream.  Every step of the method runs in the library's kernels.
Importing this module fails loudly if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_SANITIZE=1 loads the AddressSanitizer / UBSan build of the host code
# (build_sanitize.py; needs the sanitizer runtime preloaded)
LIB_PATH = os.path.join(_HERE, "libsparse_attn_san.so" if os.environ.get("SA_SANITIZE") == "1"
                        else "libsparse_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                      "or `python head_heterogeneous_block_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP, SA_ERR_NO_DEVICE, SA_ERR_ARCH = \
    0, -1, -2, -3, -4, -5, -6
SA_BF16, SA_F32 = 0, 1
MAX_HEADS = 128

EXPORTED = [
    "sa_version", "sa_last_error", "sa_set_debug_checks", "sa_lpt_schedule", "sa_lpt_schedule_grouped", "sa_lpt_order_bins",
    "sa_lpt_queue_order", "sa_lpt_queue_order_tiered", "sa_lpt_queue_partition",
    "sa_prefill_block_counts", "sa_decode_block_counts", "sa_prefill_schedule",
    "sa_decode_pooled_size", "sa_pool_keys_decode", "sa_select_workspace_size", "sa_select_blocks",
    "sa_prefill_workspace_size", "sa_sparse_attn_prefill", "sa_sparse_attn_prefill_queues",
    "sa_sparse_attn_prefill_timed",
    "sa_decode_workspace_size", "sa_sparse_attn_decode", "sa_sparse_attn_decode_noalloc",
    "sa_pool_keys_decode_paged", "sa_sparse_attn_decode_paged",
    "sa_block_attention_mass", "sa_budget_recovery", "sa_budget_shift", "sa_output_deviation",
    "sa_measure_mfma_peak", "sa_measure_hbm_read",
]


class SaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sparse_attn status {status}: {msg}")
        self.status = status


class sa_attn_desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("kernel_variant", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
    ]


class sa_head_budget(ctypes.Structure):
    _fields_ = [("min_blocks", ctypes.c_int32), ("ratio_q16", ctypes.c_uint32), ("n_sink", ctypes.c_int32),
                ("n_local", ctypes.c_int32), ("granularity", ctypes.c_int32)]


class sa_prefill_schedule_opts(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_bins", ctypes.c_int32), ("bin_order", ctypes.c_int32),
                ("xcd_groups", ctypes.c_int32), ("xcd_chunk", ctypes.c_int32), ("queue_group", ctypes.c_int32),
                ("n_queues", ctypes.c_int32), ("queue_chunk", ctypes.c_int32)]


SA_SCHED_GRID, SA_SCHED_BINS, SA_SCHED_BINS_XCD, SA_SCHED_QUEUE = 0, 1, 2, 3
QUEUE_GROUPS = {"kv_tiers": 0, "kv": 1, "head": 2, "flat": 3, "auto": 4}


class sa_kv_pages(ctypes.Structure):
    _fields_ = [("table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("pages_per_head", ctypes.c_int32)]


_P = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_descp = ctypes.POINTER(sa_attn_desc)
_budp = ctypes.POINTER(sa_head_budget)

_SIG = {
    "sa_version": (ctypes.c_int32, []),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_set_debug_checks": (ctypes.c_int32, [ctypes.c_int32]),
    "sa_lpt_schedule": (ctypes.c_int32, [_i64p, ctypes.c_int32, ctypes.c_int32, _i32p, _i32p, _i32p, _i64p]),
    "sa_lpt_order_bins": (ctypes.c_int32, [_i32p, ctypes.c_int32, _i32p]),
    "sa_lpt_queue_order": (ctypes.c_int32, [_i64p, _i32p, ctypes.c_int32, _i32p]),
    "sa_lpt_queue_order_tiered": (ctypes.c_int32, [_i64p, _i32p, ctypes.c_int32, ctypes.c_int32, _i32p]),
    "sa_lpt_queue_partition": (ctypes.c_int32, [_i64p, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, _i32p, _i32p]),
    "sa_lpt_schedule_grouped": (ctypes.c_int32, [_i64p, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, _i32p, _i32p, _i32p, _i64p]),
    "sa_prefill_block_counts": (ctypes.c_int32, [_descp, _budp, _i32p, _i32p]),
    "sa_decode_block_counts": (ctypes.c_int32, [_descp, _budp, _i32p, _i32p]),
    "sa_prefill_schedule": (ctypes.c_int32, [_descp, _budp, ctypes.POINTER(sa_prefill_schedule_opts), _i32p, _i32p,
                                             _i32p, _i64p]),
    "sa_decode_pooled_size": (ctypes.c_size_t, [_descp, _budp]),
    "sa_pool_keys_decode": (ctypes.c_int32, [_descp, _budp, _P, _P, _P]),
    "sa_select_workspace_size": (ctypes.c_size_t, [_descp, _budp, ctypes.c_int32]),
    "sa_select_blocks": (ctypes.c_int32, [_descp, _budp, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, ctypes.c_size_t,
                                          _P]),
    "sa_prefill_workspace_size": (ctypes.c_size_t, [_descp, ctypes.c_int32, ctypes.c_int32]),
    "sa_sparse_attn_prefill": (ctypes.c_int32, [_descp, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                                ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_size_t, _P]),
    "sa_sparse_attn_prefill_queues": (ctypes.c_int32, [_descp, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _i32p,
                                                       ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                                       ctypes.c_size_t, _P]),
    "sa_sparse_attn_prefill_timed": (ctypes.c_int32, [_descp, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                                      ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                                      ctypes.c_size_t, _P]),
    "sa_decode_workspace_size": (ctypes.c_size_t, [_descp, _budp, ctypes.c_int32]),
    "sa_sparse_attn_decode": (ctypes.c_int32, [_descp, _budp, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                               ctypes.c_int32, _P, ctypes.c_size_t, _P]),
    "sa_sparse_attn_decode_noalloc": (ctypes.c_int32, [_descp, _budp, _P, _P, _P, _P, _P, _P, _P,
                                                       ctypes.c_int32, ctypes.c_int32, _P]),
    "sa_pool_keys_decode_paged": (ctypes.c_int32, [_descp, _budp, _P, ctypes.POINTER(sa_kv_pages), _P, _P]),
    "sa_sparse_attn_decode_paged": (ctypes.c_int32, [_descp, _budp, _P, _P, _P, ctypes.POINTER(sa_kv_pages), _P,
                                                     _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P,
                                                     ctypes.c_size_t, _P]),
    "sa_block_attention_mass": (ctypes.c_int32, [_descp, _P, _P, _P, _P]),
    "sa_budget_recovery": (ctypes.c_int32, [ctypes.POINTER(ctypes.c_float), ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _budp, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_double)]),
    "sa_output_deviation": (ctypes.c_int32, [_descp, _P, _P, _P, _P]),
    "sa_budget_shift": (ctypes.c_int32, [ctypes.POINTER(ctypes.c_double), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.POINTER(ctypes.c_uint32)]),
    "sa_measure_mfma_peak": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "sa_measure_hbm_read": (ctypes.c_int32, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P]),
}
for _name, (_res, _args) in _SIG.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check(status: int) -> None:
    if status != SA_OK:
        raise SaError(status, _lib.sa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    if t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return None


def _match(name: str, t: Optional[torch.Tensor], shape, strides=None, dtype=None, contiguous: bool = False) -> None:
    """Raise ValueError unless t has this shape (and dtype, contiguity, and
    these strides on every axis longer than one).  The kernels address their
    tensors from the descriptor's sizes and strides alone, so a tensor laid out
    otherwise would be read or written outside its storage."""
    if t is None:
        raise ValueError(f"{name} is None")
    # fast path: everything as expected (plain tuples compare in one step)
    if (t.shape == shape and (dtype is None or t.dtype == dtype) and (strides is None or t.stride() == strides)
            and (not contiguous or t.is_contiguous())):
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if strides is not None:
        for n, got, want in zip(t.shape, t.stride(), strides):
            if n > 1 and got != int(want):
                raise ValueError(f"{name}: strides {tuple(t.stride())} differ from the descriptor's "
                                 f"{tuple(int(x) for x in strides)}")


def _check_outputs_prefill(desc: "sa_attn_desc", q, o, lse, out_f32: bool) -> None:
    """o and lse of a prefill call against the descriptor (what the kernels write)."""
    B, Hq, S, D = desc.batch, desc.n_q_heads, desc.q_len, desc.head_dim
    if _dtype_code(q) != desc.dtype:
        raise ValueError(f"q: dtype {q.dtype} does not match the descriptor")
    _match("o", o, (B, Hq, S, D), (*desc.o_stride, 1), torch.float32 if out_f32 else q.dtype)
    if lse is not None:
        _match("lse", lse, (B, Hq, S), dtype=torch.float32, contiguous=True)


def _check_outputs_decode(desc: "sa_attn_desc", q, o, lse, out_f32: bool) -> None:
    """o and lse of a decode call against the descriptor (what the kernels write)."""
    B, Hq, D = desc.batch, desc.n_q_heads, desc.head_dim
    if _dtype_code(q) != desc.dtype:
        raise ValueError(f"q: dtype {q.dtype} does not match the descriptor")
    _match("o", o, (B, Hq, D), (desc.o_stride[0], desc.o_stride[1], 1), torch.float32 if out_f32 else q.dtype)
    if lse is not None:
        _match("lse", lse, (B, Hq), dtype=torch.float32, contiguous=True)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_budgets(budget: dict) -> ctypes.Array:
    """``sa_head_budget[H]`` from a dict of per-head integer arrays
    (min_blocks, ratio_q16, n_sink, n_local, granularity)."""
    H = len(budget["min_blocks"])
    arr = (sa_head_budget * H)()
    for h in range(H):
        arr[h].min_blocks = int(budget["min_blocks"][h])
        arr[h].ratio_q16 = int(budget["ratio_q16"][h])
        arr[h].n_sink = int(budget["n_sink"][h])
        arr[h].n_local = int(budget["n_local"][h])
        arr[h].granularity = int(budget["granularity"][h]) if "granularity" in budget else 0
    return arr


def make_prefill_desc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: Optional[torch.Tensor], block: int,
                      scale: float = 0.0, kernel_variant: int = 0) -> sa_attn_desc:
    """Descriptor for q/o ``[b, Hq, S, D]`` and k/v ``[b, Hkv, S, D]`` (any strides
    with a contiguous last axis)."""
    b, hq, S, D = q.shape
    d = sa_attn_desc()
    d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim = b, hq, k.shape[1], D
    d.q_len, d.kv_len, d.block_size, d.dtype = S, k.shape[2], block, _dtype_code(q)
    d.softmax_scale, d.kernel_variant = scale, kernel_variant
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o if o is not None else q)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: last axis must be contiguous")
        getattr(d, name)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    return d


def make_decode_desc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: Optional[torch.Tensor],
                     scale: float = 0.0) -> sa_attn_desc:
    """Descriptor for q/o ``[b, Hq, D]`` and the KV cache k/v ``[b, Hkv, L, D]``."""
    b, hq, D = q.shape
    d = sa_attn_desc()
    d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim = b, hq, k.shape[1], D
    d.q_len, d.kv_len, d.block_size, d.dtype = 1, k.shape[2], 0, _dtype_code(q)
    d.softmax_scale = scale
    oo = o if o is not None else q
    d.q_stride[:] = [q.stride(0), q.stride(1), 0]
    d.o_stride[:] = [oo.stride(0), oo.stride(1), 0]
    d.k_stride[:] = [k.stride(0), k.stride(1), k.stride(2)]
    d.v_stride[:] = [v.stride(0), v.stride(1), v.stride(2)]
    return d


def make_paged_decode_desc(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, kv_len: int,
                           o: Optional[torch.Tensor] = None, scale: float = 0.0) -> sa_attn_desc:
    """Descriptor for q/o ``[b, Hq, D]`` and a paged cache whose pools k_pages /
    v_pages are ``[Hkv, pages_per_head, page_size, D]`` (row-contiguous pages)."""
    b, hq, D = q.shape
    d = sa_attn_desc()
    d.batch, d.n_q_heads, d.n_kv_heads, d.head_dim = b, hq, k_pages.shape[0], D
    d.q_len, d.kv_len, d.block_size, d.dtype = 1, kv_len, 0, _dtype_code(q)
    d.softmax_scale = scale
    oo = o if o is not None else q
    d.q_stride[:] = [q.stride(0), q.stride(1), 0]
    d.o_stride[:] = [oo.stride(0), oo.stride(1), 0]
    for t, st in ((k_pages, d.k_stride), (v_pages, d.v_stride)):
        if t.stride(1) != t.shape[2] * t.stride(2):
            raise ValueError("the pages of a pool must follow each other row by row")
        st[:] = [0, t.stride(0), t.stride(2)]
    return d


def make_pages(table: torch.Tensor, page_size: int, pages_per_head: int) -> sa_kv_pages:
    """Page description for a device int32 table ``[b, Hkv, max_pages]``."""
    if table.dtype != torch.int32 or not table.is_contiguous():
        raise ValueError("the page table must be a contiguous int32 tensor")
    p = sa_kv_pages()
    p.table = table.data_ptr()
    p.page_size, p.max_pages, p.pages_per_head = page_size, table.shape[2], pages_per_head
    return p


# ---------------------------------------------------------------- host calls


def sa_version() -> int:
    return int(_lib.sa_version())


def sa_set_debug_checks(on: bool) -> bool:
    """Switch the library's host-side index-table checks before every attention
    launch on or off (process-wide); returns the previous setting."""
    return bool(_lib.sa_set_debug_checks(1 if on else 0))


def sa_lpt_schedule(loads: Sequence[int], n_bins: int):
    """Greedy longest-load-first placement (host).  Returns numpy
    ``(bin_of_item, bin_offsets, items_by_bin, bin_load)``."""
    ld = np.ascontiguousarray(np.asarray(loads, dtype=np.int64))
    n = ld.size
    bin_of = np.empty(n, np.int32)
    off = np.empty(n_bins + 1 if n_bins > 0 else 1, np.int32)
    items = np.empty(n, np.int32)
    bl = np.empty(max(n_bins, 1), np.int64)
    _check(_lib.sa_lpt_schedule(ld.ctypes.data_as(_i64p), n, n_bins, bin_of.ctypes.data_as(_i32p),
                                off.ctypes.data_as(_i32p), items.ctypes.data_as(_i32p), bl.ctypes.data_as(_i64p)))
    return bin_of, off, items, bl


def sa_lpt_schedule_grouped(loads: Sequence[int], chunk_of_item: Sequence[int], n_chunks: int, n_groups: int,
                            n_bins: int):
    """Two-level placement (chunks onto groups, then items onto each group's
    bins).  Returns numpy ``(bin_of_item, bin_offsets, items_by_bin, bin_load)``."""
    ld = np.ascontiguousarray(np.asarray(loads, dtype=np.int64))
    ch = np.ascontiguousarray(np.asarray(chunk_of_item, dtype=np.int32))
    n = ld.size
    bin_of = np.empty(n, np.int32)
    off = np.empty(n_bins + 1 if n_bins > 0 else 1, np.int32)
    items = np.empty(n, np.int32)
    bl = np.empty(max(n_bins, 1), np.int64)
    _check(_lib.sa_lpt_schedule_grouped(ld.ctypes.data_as(_i64p), ch.ctypes.data_as(_i32p), n, n_chunks, n_groups,
                                        n_bins, bin_of.ctypes.data_as(_i32p), off.ctypes.data_as(_i32p),
                                        items.ctypes.data_as(_i32p), bl.ctypes.data_as(_i64p)))
    return bin_of, off, items, bl


def sa_lpt_order_bins(bin_offsets: np.ndarray, items_by_bin: np.ndarray) -> np.ndarray:
    """Copy of ``items_by_bin`` with every bin's items in ascending item order."""
    off = np.ascontiguousarray(bin_offsets, dtype=np.int32)
    items = np.array(items_by_bin, dtype=np.int32, copy=True)
    _check(_lib.sa_lpt_order_bins(off.ctypes.data_as(_i32p), off.size - 1, items.ctypes.data_as(_i32p)))
    return items


def sa_lpt_queue_order_tiered(loads: Sequence[int], group_of_item: Optional[Sequence[int]] = None,
                              tiers_per_octave: int = 4) -> np.ndarray:
    """Item order for the work queue in load tiers (see the C header)."""
    ld = np.ascontiguousarray(loads, dtype=np.int64)
    n = ld.size
    gp = None if group_of_item is None else np.ascontiguousarray(group_of_item, dtype=np.int32)
    order = np.zeros(n, dtype=np.int32)
    _check(_lib.sa_lpt_queue_order_tiered(ld.ctypes.data_as(_i64p), gp.ctypes.data_as(_i32p) if gp is not None
                                          else None, n, tiers_per_octave, order.ctypes.data_as(_i32p)))
    return order


def sa_lpt_queue_partition(loads: Sequence[int], group_of_item: Sequence[int], n_groups: int, n_queues: int,
                           tiers_per_octave: int = 4, chunk_items: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Work queue cut into ``n_queues`` partitions of (tier, group) units of at
    most ``chunk_items`` items, 0 = no limit (see the C header): returns
    (order, queue_offsets)."""
    ld = np.ascontiguousarray(loads, dtype=np.int64)
    gp = np.ascontiguousarray(group_of_item, dtype=np.int32)
    if gp.size != ld.size:
        raise ValueError("group_of_item must have one entry per item")
    order = np.zeros(ld.size, dtype=np.int32)
    off = np.zeros(max(n_queues, 0) + 1, dtype=np.int32)
    _check(_lib.sa_lpt_queue_partition(ld.ctypes.data_as(_i64p), gp.ctypes.data_as(_i32p), ld.size, n_groups,
                                       n_queues, tiers_per_octave, chunk_items, order.ctypes.data_as(_i32p),
                                       off.ctypes.data_as(_i32p)))
    return order, off


def sa_lpt_queue_order(loads: Sequence[int], group_of_item: Optional[Sequence[int]] = None) -> np.ndarray:
    """Item order for the work queue: groups ascending, largest load first inside a group."""
    ld = np.ascontiguousarray(loads, dtype=np.int64)
    n = ld.size
    order = np.empty(n, dtype=np.int32)
    gp = None
    if group_of_item is not None:
        gp = np.ascontiguousarray(group_of_item, dtype=np.int32)
        if gp.size != n:
            raise ValueError("group_of_item must have one entry per item")
    _check(_lib.sa_lpt_queue_order(ld.ctypes.data_as(_i64p), gp.ctypes.data_as(_i32p) if gp is not None else None, n,
                                   order.ctypes.data_as(_i32p)))
    return order


def sa_prefill_block_counts(desc: sa_attn_desc, budgets) -> tuple[np.ndarray, int]:
    nb = -(-desc.q_len // desc.block_size)
    counts = np.empty((desc.batch, desc.n_q_heads, nb), np.int32)
    kmax = ctypes.c_int32(0)
    _check(_lib.sa_prefill_block_counts(ctypes.byref(desc), budgets, counts.ctypes.data_as(_i32p),
                                        ctypes.byref(kmax)))
    return counts, int(kmax.value)


def sa_prefill_schedule(desc: sa_attn_desc, budgets, kind: int, n_bins: int = 0, bin_order: int = 0,
                        xcd_groups: int = 0, xcd_chunk: int = 0, queue_group: int = 0, n_queues: int = 1,
                        queue_chunk: int = 0):
    """The host schedule of the prefill tiles: (items, offsets, bin_load) as
    numpy arrays (bin_load None for the queue; all None for the natural grid)."""
    opts = sa_prefill_schedule_opts(kind, n_bins, bin_order, xcd_groups, xcd_chunk, queue_group, n_queues,
                                    queue_chunk)
    if kind == SA_SCHED_GRID:
        n_off = ctypes.c_int32(0)
        _check(_lib.sa_prefill_schedule(ctypes.byref(desc), budgets, ctypes.byref(opts), None, None,
                                        ctypes.byref(n_off), None))
        return None, None, None
    nb = -(-desc.q_len // desc.block_size)
    n = desc.batch * desc.n_q_heads * nb
    items = np.zeros(max(n, 1), dtype=np.int32)
    offsets = np.zeros(max(n_bins, n_queues, 1) + 1, dtype=np.int32)
    is_bins = kind in (SA_SCHED_BINS, SA_SCHED_BINS_XCD)
    load = np.zeros(max(n_bins, 1), dtype=np.int64) if is_bins else None
    n_off = ctypes.c_int32(0)
    _check(_lib.sa_prefill_schedule(ctypes.byref(desc), budgets, ctypes.byref(opts), items.ctypes.data_as(_i32p),
                                    offsets.ctypes.data_as(_i32p), ctypes.byref(n_off),
                                    load.ctypes.data_as(_i64p) if is_bins else None))
    return items[:n], offsets[:n_off.value], load


def sa_decode_block_counts(desc: sa_attn_desc, budgets) -> tuple[np.ndarray, int]:
    counts = np.empty(desc.n_q_heads, np.int32)
    kmax = ctypes.c_int32(0)
    _check(_lib.sa_decode_block_counts(ctypes.byref(desc), budgets, counts.ctypes.data_as(_i32p),
                                       ctypes.byref(kmax)))
    return counts, int(kmax.value)


def sa_select_workspace_size(desc: sa_attn_desc, budgets, kmax: int) -> int:
    return int(_lib.sa_select_workspace_size(ctypes.byref(desc), budgets, kmax))


def sa_prefill_workspace_size(desc: sa_attn_desc, kmax: int, n_bins: int) -> int:
    return int(_lib.sa_prefill_workspace_size(ctypes.byref(desc), kmax, n_bins))


def sa_decode_workspace_size(desc: sa_attn_desc, budgets, kmax: int) -> int:
    return int(_lib.sa_decode_workspace_size(ctypes.byref(desc), budgets, kmax))


def sa_decode_pooled_size(desc: sa_attn_desc, budgets) -> int:
    return int(_lib.sa_decode_pooled_size(ctypes.byref(desc), budgets))


# ---------------------------------------------------------------- device calls


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def sa_pool_keys_decode(desc: sa_attn_desc, budgets, k: torch.Tensor, k_pooled: torch.Tensor) -> None:
    _check(_lib.sa_pool_keys_decode(ctypes.byref(desc), budgets, _ptr(k), _ptr(k_pooled), _stream(k)))


def sa_select_blocks(desc: sa_attn_desc, budgets, q: torch.Tensor, k: torch.Tensor,
                     k_pooled: Optional[torch.Tensor], block_idx: torch.Tensor, block_cnt: torch.Tensor,
                     kmax: int, workspace: torch.Tensor, key_norms: Optional[torch.Tensor] = None,
                     check: bool = True) -> None:
    if check:  # (the plans validate their own tables once and pass check=False)
        B, Hq = desc.batch, desc.n_q_heads
        if desc.block_size == 0:  # decode
            rows = (B, Hq)
        else:
            rows = (B, Hq, -(-desc.q_len // desc.block_size))
            if key_norms is not None:
                _match("key_norms", key_norms, (B, desc.n_kv_heads, rows[2]), dtype=torch.float32, contiguous=True)
        _match("block_idx", block_idx, (*rows, kmax), dtype=torch.int32, contiguous=True)
        _match("block_cnt", block_cnt, rows, dtype=torch.int32, contiguous=True)
    _check(_lib.sa_select_blocks(ctypes.byref(desc), budgets, _ptr(q), _ptr(k), _ptr(k_pooled), _ptr(block_idx),
                                 _ptr(block_cnt), kmax, _ptr(key_norms), _ptr(workspace), workspace.numel(),
                                 _stream(q)))


def sa_sparse_attn_prefill(desc: sa_attn_desc, q, k, v, o, lse, block_idx, block_cnt, kmax: int,
                           bin_offsets=None, items_by_bin=None, n_bins: int = 0, out_f32: bool = False,
                           workspace: Optional[torch.Tensor] = None, key_norms: Optional[torch.Tensor] = None,
                           check: bool = True) -> None:
    if check:
        _check_outputs_prefill(desc, q, o, lse, out_f32)
    ws = workspace
    _check(_lib.sa_sparse_attn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       _ptr(block_idx), _ptr(block_cnt), kmax, _ptr(key_norms), _ptr(bin_offsets),
                                       _ptr(items_by_bin), n_bins, 1 if out_f32 else 0, _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(q)))


def sa_sparse_attn_prefill_queues(desc: sa_attn_desc, q, k, v, o, lse, block_idx, block_cnt, kmax: int,
                                  queue_offsets: np.ndarray, order, n_workgroups: int, out_f32: bool = False,
                                  workspace: Optional[torch.Tensor] = None,
                                  key_norms: Optional[torch.Tensor] = None, check: bool = True) -> None:
    if check:
        _check_outputs_prefill(desc, q, o, lse, out_f32)
    off = np.ascontiguousarray(queue_offsets, dtype=np.int32)
    ws = workspace
    _check(_lib.sa_sparse_attn_prefill_queues(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              _ptr(block_idx), _ptr(block_cnt), kmax, _ptr(key_norms),
                                              off.ctypes.data_as(_i32p),
                                              off.size - 1, _ptr(order), n_workgroups, 1 if out_f32 else 0,
                                              _ptr(ws), 0 if ws is None else ws.numel(), _stream(q)))


def sa_sparse_attn_prefill_timed(desc: sa_attn_desc, q, k, v, o, lse, block_idx, block_cnt, kmax: int,
                                 bin_offsets, items_by_bin, n_bins: int, queue_offsets: Optional[np.ndarray],
                                 out_f32: bool, wg_times: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                                 key_norms: Optional[torch.Tensor] = None, check: bool = True) -> None:
    """A prefill launch recording each workgroup's start and end on the constant
    clock into wg_times (int64 [2 * grid])."""
    if check:
        _check_outputs_prefill(desc, q, o, lse, out_f32)
    off = None if queue_offsets is None else np.ascontiguousarray(queue_offsets, dtype=np.int32)
    ws = workspace
    _check(_lib.sa_sparse_attn_prefill_timed(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(block_idx), _ptr(block_cnt), kmax,
        _ptr(key_norms), _ptr(bin_offsets), _ptr(items_by_bin), n_bins, None if off is None else off.ctypes.data_as(_i32p),
        0 if off is None else off.size - 1, 1 if out_f32 else 0, _ptr(wg_times), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(q)))


def sa_sparse_attn_decode(desc: sa_attn_desc, budgets, q, k, v, o, lse, block_idx, block_cnt, kmax: int,
                          workspace: torch.Tensor, out_f32: bool = False, check: bool = True) -> None:
    if check:
        _check_outputs_decode(desc, q, o, lse, out_f32)
    _check(_lib.sa_sparse_attn_decode(ctypes.byref(desc), budgets, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _ptr(block_idx), _ptr(block_cnt), kmax, 1 if out_f32 else 0, _ptr(workspace),
                                      workspace.numel(), _stream(q)))


def sa_sparse_attn_decode_noalloc(desc: sa_attn_desc, budgets, q, k, v, o, lse, block_idx, block_cnt, kmax: int,
                                  out_f32: bool = False) -> None:
    """sa_sparse_attn_decode with the library's fixed per-GPU scratch array
    instead of a workspace (no allocation; calls on one GPU must not overlap)."""
    _check_outputs_decode(desc, q, o, lse, out_f32)
    _check(_lib.sa_sparse_attn_decode_noalloc(ctypes.byref(desc), budgets, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                              _ptr(lse), _ptr(block_idx), _ptr(block_cnt), kmax,
                                              1 if out_f32 else 0, _stream(q)))


def sa_pool_keys_decode_paged(desc: sa_attn_desc, budgets, k_pages: torch.Tensor, pages: sa_kv_pages,
                              k_pooled: torch.Tensor) -> None:
    _check(_lib.sa_pool_keys_decode_paged(ctypes.byref(desc), budgets, _ptr(k_pages), ctypes.byref(pages),
                                          _ptr(k_pooled), _stream(k_pages)))


def sa_sparse_attn_decode_paged(desc: sa_attn_desc, budgets, q, k_pages, v_pages, pages: sa_kv_pages, o, lse,
                                block_idx, block_cnt, kmax: int, workspace: torch.Tensor,
                                out_f32: bool = False, check: bool = True) -> None:
    if check:
        _check_outputs_decode(desc, q, o, lse, out_f32)
    _check(_lib.sa_sparse_attn_decode_paged(ctypes.byref(desc), budgets, _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                            ctypes.byref(pages), _ptr(o), _ptr(lse), _ptr(block_idx),
                                            _ptr(block_cnt), kmax, 1 if out_f32 else 0, _ptr(workspace),
                                            workspace.numel(), _stream(q)))


def sa_block_attention_mass(desc: sa_attn_desc, q: torch.Tensor, k: torch.Tensor, mass: torch.Tensor) -> None:
    _check(_lib.sa_block_attention_mass(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(mass), _stream(q)))


def sa_budget_recovery(mass: np.ndarray, budget: dict, step_q16: int) -> np.ndarray:
    """Host recovery table ``[H, 65536 // step_q16]`` from a host fp32 mass
    array ``[b, H, NB, NB]``."""
    m = np.ascontiguousarray(mass, dtype=np.float32)
    b, H, nb, _ = m.shape
    rec = np.zeros((H, 65536 // step_q16), dtype=np.float64)
    _check(_lib.sa_budget_recovery(m.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), b, H, nb,
                                   make_budgets(budget), step_q16,
                                   rec.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return rec


def sa_output_deviation(desc: sa_attn_desc, o_approx: torch.Tensor, o_ref: torch.Tensor, dev: torch.Tensor) -> None:
    """dev [n_q_heads] float64 on the device: relative output distance per head."""
    if dev.dtype != torch.float64 or dev.numel() < desc.n_q_heads:
        raise ValueError("dev must be a float64 tensor of n_q_heads entries")
    _check(_lib.sa_output_deviation(ctypes.byref(desc), _ptr(o_approx), _ptr(o_ref), _ptr(dev), _stream(o_ref)))


def sa_measure_mfma_peak(n_workgroups: int, iters: int, sink: torch.Tensor, operands: int = 0) -> int:
    """Launch the bf16 MFMA rate probe on sink's device and stream; returns the
    flops it does.  operands 0: ones (every sink entry becomes 128 * iters);
    1: pseudo-random bf16 operands (the sink entries follow the header's
    formula)."""
    if sink.dtype != torch.float32 or sink.numel() < n_workgroups * 256:
        raise ValueError("sink must be fp32 with n_workgroups * 256 entries")
    _check(_lib.sa_measure_mfma_peak(n_workgroups, iters, operands, _ptr(sink), _stream(sink)))
    return n_workgroups * 4 * 8 * iters * 32768


def sa_measure_hbm_read(buf: torch.Tensor, n_workgroups: int, sink: torch.Tensor) -> int:
    """Launch the HBM streaming-read probe over buf (all of its bytes); returns
    the bytes read.  The XOR of sink's entries equals that of buf's 32-bit words."""
    if not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < n_workgroups * 256:
        raise ValueError("buf must be contiguous, sink int32 with n_workgroups * 256 entries")
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.sa_measure_hbm_read(_ptr(buf), nbytes, n_workgroups, _ptr(sink), _stream(sink)))
    return nbytes


def deviation_table(q, k, v, budget: dict, block: int, step_q16: int, n_bins: int = 512) -> np.ndarray:
    """dev[h, i]: output deviation of head h when every head runs at ratio
    (i + 1) * step_q16, against ratio 1 (every block), each output from the
    library's selection and prefill attention (fp32 out), each deviation from
    sa_output_deviation."""
    H = q.shape[1]
    n_grid = 65536 // step_q16
    if n_grid * step_q16 != 65536:
        raise ValueError("step_q16 must divide 65536")

    def run(ratio):
        b = dict(budget)
        b["ratio_q16"] = [ratio] * H
        plan = PrefillPlan(q, k, v, b, block, n_bins=n_bins, out_f32=True, queue=True)
        o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        plan.select(q, k)
        plan.attend(q, k, v, o)
        return plan, o

    plan, o_ref = run(65536)
    dev = torch.empty((n_grid, H), dtype=torch.float64, device=q.device)
    for i in range(n_grid):
        _, o = run((i + 1) * step_q16)
        sa_output_deviation(plan.desc, o, o_ref, dev[i])
    torch.cuda.synchronize(q.device)
    return dev.cpu().numpy().T.copy()


def sa_budget_shift(recovery: np.ndarray, step_q16: int, total_q16: int) -> np.ndarray:
    """Max-min shifted ratios (uint32 ``[H]``, units 2^-16) from a recovery table."""
    rec = np.ascontiguousarray(recovery, dtype=np.float64)
    out = np.zeros(rec.shape[0], dtype=np.uint32)
    _check(_lib.sa_budget_shift(rec.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), rec.shape[0], step_q16,
                                int(total_q16), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))))
    return out


# ---------------------------------------------------------------- conveniences
# (allocation + the calls above, in order; still no compute outside the library)


class PrefillPlan:
    """Everything a prefill layer needs that depends only on shapes and budgets:
    descriptor, per-head budgets, block counts (LPT loads), kmax and the LPT
    schedule over ``n_bins`` persistent workgroups (uploaded to the device).
    ``bin_order``: "index" walks each bin in item order (sa_lpt_order_bins),
    "lpt" in assignment order.  ``xcd_groups`` > 0 uses the two-level placement
    (sa_lpt_schedule_grouped): chunks of ``xcd_chunk`` query blocks of one
    (sequence, KV head) onto ``xcd_groups`` cache partitions, then LPT inside.
    ``queue``: instead of fixed bins, the ``n_bins`` workgroups take the tiles
    longest first from a shared counter (the greedy rule applied online).
    ``queue_group`` orders the queue: "kv_tiers" in load tiers of a quarter
    octave, heaviest first, grouped by (sequence, KV head) inside a tier; "kv"
    grouped by (sequence, KV head) only; "head" grouped by query head,
    heaviest head first; "flat" plain longest first; "auto" (default) the
    library's choice by size (SA_QUEUE_AUTO: "flat" on one queue up to 256
    query blocks per head, else "kv_tiers" in partitions).  ``queues`` > 1
    (default 8, one per XCD of MI355X) cuts the "kv_tiers" queue into that many
    partitions (sa_lpt_queue_partition): runs of one (load tier, sequence, KV
    head), of at most ``queue_chunk`` tiles (0: no limit), placed by LPT, each
    partition in the tiered order; other ``queue_group`` orders use one queue.
    ``key_norms``: the selection also writes each key block's largest key-row
    norm, and the attention uses it to skip the per-step row max where the
    scores cannot overflow (False: every step takes the row max).  ``scale``:
    the softmax scale (0: 1/sqrt(D))."""

    def __init__(self, q, k, v, budget: dict, block: int, n_bins: int = 0, out_f32: bool = False,
                 kernel_variant: int = 0, bin_order: str = "index", xcd_groups: int = 0, xcd_chunk: int = 64,
                 queue: bool = False, queue_group: str = "auto", queues: int = 8, queue_chunk: int = 0,
                 key_norms: bool = True, scale: float = 0.0):
        self.desc = make_prefill_desc(q, k, v, q, block, scale=scale, kernel_variant=kernel_variant)
        self.budgets = make_budgets(budget)
        self.counts, self.kmax = sa_prefill_block_counts(self.desc, self.budgets)
        self.block = block
        self.n_bins = n_bins
        self.out_f32 = out_f32
        dev = q.device
        self.nb = -(-q.shape[2] // block)
        self.block_idx = torch.empty((q.shape[0], q.shape[1], self.nb, self.kmax), dtype=torch.int32, device=dev)
        self.block_cnt = torch.empty((q.shape[0], q.shape[1], self.nb), dtype=torch.int32, device=dev)
        self.select_ws = _workspace(sa_select_workspace_size(self.desc, self.budgets, self.kmax), dev)
        self.attn_ws = _workspace(sa_prefill_workspace_size(self.desc, self.kmax, n_bins), dev)
        self.key_norms = (torch.empty((q.shape[0], k.shape[1], self.nb), dtype=torch.float32, device=dev)
                          if key_norms else None)
        # the layouts the descriptor was built for (every later q, k, v must
        # have them); o may differ from q, and the descriptor follows it
        self._lay = {n: (tuple(t.shape), tuple(t.stride()), q.dtype) for n, t in (("q", q), ("k", k), ("v", v))}
        self._o_dtype = torch.float32 if out_f32 else q.dtype
        self._o_stride = tuple(q.stride())
        self.queue = queue
        self.queue_offsets = None
        self.bin_load = None
        self.bin_offsets = self.items_by_bin = None
        if queue:
            if n_bins < 1:
                raise ValueError("the work queue needs n_bins >= 1 workgroups")
            if queue_group not in QUEUE_GROUPS:
                raise ValueError(f"queue_group {queue_group!r}")
            nq = queues if queue_group in ("kv_tiers", "auto") else 1
            items, off, _ = sa_prefill_schedule(self.desc, self.budgets, SA_SCHED_QUEUE,
                                                queue_group=QUEUE_GROUPS[queue_group], n_queues=nq,
                                                queue_chunk=queue_chunk)
            if off.size > 2:  # partitions
                self.queue_offsets = off
            self.items_by_bin = torch.from_numpy(items).to(dev)
        elif n_bins > 0:
            if bin_order not in ("index", "lpt"):
                raise ValueError(bin_order)
            items, off, load = sa_prefill_schedule(self.desc, self.budgets,
                                                   SA_SCHED_BINS_XCD if xcd_groups > 0 else SA_SCHED_BINS,
                                                   n_bins=n_bins, bin_order=0 if bin_order == "index" else 1,
                                                   xcd_groups=xcd_groups, xcd_chunk=xcd_chunk)
            self.bin_load = load
            self.bin_offsets = torch.from_numpy(off).to(dev)
            self.items_by_bin = torch.from_numpy(items).to(dev)

    def select(self, q, k) -> None:
        _match("q", q, *self._lay["q"])
        _match("k", k, *self._lay["k"])
        sa_select_blocks(self.desc, self.budgets, q, k, None, self.block_idx, self.block_cnt, self.kmax,
                         self.select_ws, self.key_norms, check=False)

    def _set_out(self, q, k, v, o, lse) -> None:
        """Check q, k and v against the plan's layouts and o and lse against its
        shapes, and take o's strides (o may be laid out differently from q)."""
        for n, t in (("q", q), ("k", k), ("v", v)):
            _match(n, t, *self._lay[n])
        if o is None or o.dim() != 4:
            raise ValueError("o must be a [b, Hq, S, D] tensor")
        _match("o", o, self._lay["q"][0], dtype=self._o_dtype)
        if lse is not None:
            _match("lse", lse, self._lay["q"][0][:3], dtype=torch.float32, contiguous=True)
        st = o.stride()
        if st != self._o_stride:
            if st[3] != 1:
                raise ValueError("o: last axis must be contiguous")
            self.desc.o_stride[:] = [st[0], st[1], st[2]]
            self._o_stride = st

    def attend(self, q, k, v, o, lse=None) -> None:
        self._set_out(q, k, v, o, lse)
        if self.queue and self.queue_offsets is not None:
            sa_sparse_attn_prefill_queues(self.desc, q, k, v, o, lse, self.block_idx, self.block_cnt, self.kmax,
                                          self.queue_offsets, self.items_by_bin, self.n_bins, self.out_f32,
                                          self.attn_ws, self.key_norms, check=False)
            return
        sa_sparse_attn_prefill(self.desc, q, k, v, o, lse, self.block_idx, self.block_cnt, self.kmax,
                               self.bin_offsets, self.items_by_bin, self.n_bins, self.out_f32, self.attn_ws,
                               self.key_norms, check=False)

    def share_tables(self, other: "PrefillPlan") -> None:
        """Use the selection outputs of another plan of the same shape and
        budgets (block lists, counts and key-norm table) instead of this plan's
        own, e.g. to run the same selection under another schedule."""
        if other.block_idx.shape != self.block_idx.shape:
            raise ValueError("plans of different shapes")
        self.block_idx = other.block_idx
        self.block_cnt = other.block_cnt
        self.key_norms = other.key_norms

    def grid(self) -> int:
        """Workgroups of a launch: the persistent workgroups, or one per tile."""
        return self.n_bins if self.items_by_bin is not None else int(self.counts.size)

    def attend_timed(self, q, k, v, o, lse=None, stamps: Optional[torch.Tensor] = None) -> torch.Tensor:
        """attend(), also recording each workgroup's start and end on the GPU's
        constant clock into ``stamps`` (int64 [grid, 2], allocated if None);
        returns it."""
        self._set_out(q, k, v, o, lse)
        t = stamps if stamps is not None else torch.zeros((self.grid(), 2), dtype=torch.int64, device=q.device)
        if t.dtype != torch.int64 or t.numel() < 2 * self.grid():
            raise ValueError("stamps must be int64 with 2 * grid entries")
        sa_sparse_attn_prefill_timed(self.desc, q, k, v, o, lse, self.block_idx, self.block_cnt, self.kmax,
                                     self.bin_offsets, self.items_by_bin, self.n_bins if self.items_by_bin is not None
                                     else 0, self.queue_offsets if self.queue else None, self.out_f32, t,
                                     self.attn_ws, self.key_norms, check=False)
        return t


class DecodePlan:
    """Descriptor, budgets, kmax, index buffers and workspaces for one decode
    shape; ``pool`` builds the pooled-key cache once per KV cache."""

    def __init__(self, q, k, v, budget: dict, out_f32: bool = False, desc: Optional[sa_attn_desc] = None,
                 scale: float = 0.0):
        # scale: the softmax scale (0: 1/sqrt(D)); ignored when desc is given
        self.desc = desc if desc is not None else make_decode_desc(q, k, v, q, scale=scale)
        self.budgets = make_budgets(budget)
        self.counts, self.kmax = sa_decode_block_counts(self.desc, self.budgets)
        self.out_f32 = out_f32
        dev = q.device
        self.block_idx = torch.empty((q.shape[0], q.shape[1], self.kmax), dtype=torch.int32, device=dev)
        self.block_cnt = torch.empty((q.shape[0], q.shape[1]), dtype=torch.int32, device=dev)
        self.k_pooled = torch.empty(max(sa_decode_pooled_size(self.desc, self.budgets) // 4, 4),
                                    dtype=torch.float32, device=dev)
        self.select_ws = _workspace(sa_select_workspace_size(self.desc, self.budgets, self.kmax), dev)
        self.attn_ws = _workspace(sa_decode_workspace_size(self.desc, self.budgets, self.kmax), dev)
        # the layouts the descriptor was built for (k and v: the cache, or the
        # page pools of a paged plan); o may differ from q
        self._lay = {n: (tuple(t.shape), tuple(t.stride()), q.dtype) for n, t in (("q", q), ("k", k), ("v", v))}
        self._o_dtype = torch.float32 if out_f32 else q.dtype
        self._o_stride = (int(self.desc.o_stride[0]), int(self.desc.o_stride[1]), 1)

    def pool(self, k) -> None:
        _match("k", k, *self._lay["k"])
        self._pool(k)

    def _pool(self, k) -> None:
        sa_pool_keys_decode(self.desc, self.budgets, k, self.k_pooled)

    def select(self, q, k) -> None:
        # (the selection reads the pooled-key cache, not k)
        _match("q", q, *self._lay["q"])
        sa_select_blocks(self.desc, self.budgets, q, k, self.k_pooled, self.block_idx, self.block_cnt, self.kmax,
                         self.select_ws, check=False)

    def _set_out(self, q, k, v, o, lse) -> None:
        for n, t in (("q", q), ("k", k), ("v", v)):
            _match(n, t, *self._lay[n])
        if o is None or o.dim() != 3:
            raise ValueError("o must be a [b, Hq, D] tensor")
        _match("o", o, self._lay["q"][0], dtype=self._o_dtype)
        if lse is not None:
            _match("lse", lse, self._lay["q"][0][:2], dtype=torch.float32, contiguous=True)
        st = o.stride()
        if st != self._o_stride:
            if st[2] != 1:
                raise ValueError("o: last axis must be contiguous")
            self.desc.o_stride[:] = [st[0], st[1], 0]
            self._o_stride = st

    def attend(self, q, k, v, o, lse=None) -> None:
        self._set_out(q, k, v, o, lse)
        sa_sparse_attn_decode(self.desc, self.budgets, q, k, v, o, lse, self.block_idx, self.block_cnt, self.kmax,
                              self.attn_ws, self.out_f32, check=False)


class PagedDecodePlan(DecodePlan):
    """DecodePlan over a paged cache: pools ``[Hkv, pages_per_head, page_size,
    D]`` and a page table ``[b, Hkv, max_pages]`` (``table``).  Selection reads
    the pooled-key cache built by ``pool``, as for a contiguous cache."""

    def __init__(self, q, k_pages, v_pages, table, kv_len: int, budget: dict, out_f32: bool = False):
        super().__init__(q, k_pages, v_pages, budget, out_f32,
                         desc=make_paged_decode_desc(q, k_pages, v_pages, kv_len))
        self.pages = make_pages(table, k_pages.shape[2], k_pages.shape[1])
        self.table = table  # keeps the table alive while the plan holds its address

    def _pool(self, k_pages) -> None:
        sa_pool_keys_decode_paged(self.desc, self.budgets, k_pages, self.pages, self.k_pooled)

    def attend(self, q, k_pages, v_pages, o, lse=None) -> None:
        self._set_out(q, k_pages, v_pages, o, lse)
        sa_sparse_attn_decode_paged(self.desc, self.budgets, q, k_pages, v_pages, self.pages, o, lse,
                                    self.block_idx, self.block_cnt, self.kmax, self.attn_ws, self.out_f32,
                                    check=False)
