"""R-KV decode-time KV-cache compression on MI355X: Python binding of librkv.so.

Argument marshalling only. Every step of the compression (importance,
redundancy, joint score, selection, compaction, page return) runs in the HIP
kernels behind the C ABI in ``include/rkv.h``; torch provides device memory
and the stream. There is no CPU fallback: if the library is not built, or
the tensors are not on a GPU, these functions raise.

Keyword names follow the R-KV entry point described on the pages
(``kv_budget``, ``window_size``, ``mix_lambda``). The reading variants are
keyword flags: ``symmetric`` (R over every other candidate), ``causal``
(False: every window query sees all candidates), ``pool`` ("max" or "mean"
over the GQA heads), and ``select_group`` (head-shared selection over runs of
that many consecutive units).
"""
from __future__ import annotations

import ctypes
from typing import NamedTuple, Optional

from . import _lib
from ._lib import RkvError  # noqa: F401

HEAD_DIM = 128


class CompressResult(NamedTuple):
    kept_idx: object      # int32 [Bh, B]
    K_out: object         # [Bh, B, 128]
    V_out: object
    I: Optional[object]   # float32 [Bh, N] when debug
    R: Optional[object]
    Z: Optional[object]


class PagedResult(NamedTuple):
    kept_idx: object      # int32, ragged (see rkv.h)
    free_count: int
    Z: Optional[object]


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.RKV_BF16
    if t.dtype == torch.float32:
        return _lib.RKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on a GPU (the library has no CPU path)")
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors must share one GPU (got {sorted(str(d) for d in devs)})")


def _check_rows_out(name, t, dtype, bh, rows):
    """An output of [bh, >= rows, 128] rows of `dtype`, rows contiguous: the
    library writes rows * 128 elements per unit at the tensor's unit stride."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if t.dim() != 3 or t.shape[0] != bh or t.shape[1] < rows or t.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} must be [{bh}, >= {rows}, {HEAD_DIM}] (got {tuple(t.shape)})")


def _check_index_out(name, t, numel, shape=None):
    """A contiguous int32 index output of exactly `shape`, or (shape None)
    holding at least `numel` entries."""
    import torch
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)} (got {list(t.shape)})")
    if t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} entries (got {t.numel()})")


def variant_bits(symmetric: bool = False, causal: bool = True, pool: str = "max") -> int:
    """RKV_VARIANT_* bits of the reading variants (0 = the default readings)."""
    if pool not in ("max", "mean"):
        raise ValueError(f"pool must be 'max' or 'mean' (got {pool!r})")
    return ((_lib.RKV_VARIANT_SYMMETRIC if symmetric else 0)
            | (0 if causal else _lib.RKV_VARIANT_NO_CAUSAL)
            | (_lib.RKV_VARIANT_POOL_MEAN if pool == "mean" else 0))


def dense_desc(num_heads, n_cand, gqa, window, budget, lam, dtype_code, kv_stride=0, out_stride=0,
               variant=0, select_group=0):
    return _lib.DenseDesc(num_heads, n_cand, HEAD_DIM, gqa, window, budget, float(lam), dtype_code,
                          kv_stride, out_stride, variant, select_group)


def workspace_size(num_heads, n_cand, gqa_group, window_size, kv_budget, dtype="bf16",
                   select_group: int = 0) -> int:
    code = _lib.RKV_BF16 if dtype in ("bf16", "bfloat16") else _lib.RKV_F32
    d = dense_desc(num_heads, n_cand, gqa_group, window_size, kv_budget, 0.0, code,
                   select_group=select_group)
    n = _lib.load().rkv_workspace_size(ctypes.byref(d))
    if n == 0:
        raise _lib.RkvError(_lib.RKV_EINVAL, _lib.last_error())
    return int(n)


def compress(K, V, Q_win, kv_budget: int, window_size: int = 8, mix_lambda: float = 0.1, *,
             K_out=None, V_out=None, kept_idx=None, debug: bool = False, workspace=None,
             stream=None, symmetric: bool = False, causal: bool = True, pool: str = "max",
             select_group: int = 1) -> CompressResult:
    """Compress every unit of a dense cache (out of place).

    K, V: [Bh, N, 128] (rows contiguous; the unit stride may exceed N*128, as
    in a cache buffer with spare capacity, and must match between K and V).
    Q_win: [Bh, G, w, 128] contiguous, the last w queries of each of the G
    query heads sharing the KV head. Returns kept indices (ascending) and the
    compacted rows; with ``debug`` also I, R and Z.
    """
    import torch
    _require_cuda(K, V, Q_win)
    if K.dim() != 3 or V.shape != K.shape or K.shape[2] != HEAD_DIM:
        raise ValueError(f"K and V must be [Bh, N, {HEAD_DIM}] with equal shapes")
    if K.stride(2) != 1 or K.stride(1) != HEAD_DIM or V.stride() != K.stride():
        raise ValueError("K and V rows must be contiguous with equal strides")
    if Q_win.dim() != 4 or Q_win.shape[0] != K.shape[0] or Q_win.shape[2] != window_size \
            or Q_win.shape[3] != HEAD_DIM or not Q_win.is_contiguous():
        raise ValueError("Q_win must be a contiguous [Bh, G, window_size, 128] tensor")
    if not (K.dtype == V.dtype == Q_win.dtype):
        raise TypeError("K, V and Q_win must share a dtype")
    bh, n = int(K.shape[0]), int(K.shape[1])
    g = int(Q_win.shape[1])
    b = int(kv_budget)
    dev = K.device
    if K_out is None:
        K_out = torch.empty((bh, b, HEAD_DIM), dtype=K.dtype, device=dev)
    if V_out is None:
        V_out = torch.empty((bh, b, HEAD_DIM), dtype=K.dtype, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((bh, b), dtype=torch.int32, device=dev)
    _require_cuda(K, K_out, V_out, kept_idx)
    # the library writes min(N, B) rows per unit (kept indices: B per unit)
    _check_rows_out("K_out", K_out, K.dtype, bh, min(n, b))
    _check_rows_out("V_out", V_out, K.dtype, bh, min(n, b))
    if K_out.stride() != V_out.stride() or K_out.stride(2) != 1 or K_out.stride(1) != HEAD_DIM:
        raise ValueError("K_out and V_out rows must be contiguous with equal strides")
    _check_index_out("kept_idx", kept_idx, bh * b, shape=(bh, b))
    dbg = [torch.empty((bh, n), dtype=torch.float32, device=dev) for _ in range(3)] if debug \
        else [None, None, None]
    d = dense_desc(bh, n, g, window_size, b, mix_lambda, _dtype_code(K),
                   K.stride(0) if bh > 1 else 0, K_out.stride(0) if bh > 1 else 0,
                   variant_bits(symmetric, causal, pool), int(select_group))
    lib = _lib.load()
    need = lib.rkv_workspace_size(ctypes.byref(d))
    if need == 0:
        raise _lib.RkvError(_lib.RKV_EINVAL, _lib.last_error())
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _lib.check(lib.rkv_compress(ctypes.byref(d), _ptr(K), _ptr(V), _ptr(Q_win), _ptr(kept_idx),
                                _ptr(K_out), _ptr(V_out), _ptr(dbg[0]), _ptr(dbg[1]), _ptr(dbg[2]),
                                _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return CompressResult(kept_idx, K_out, V_out, *dbg)


def compress_static(K, V, Q_win, kv_budget: int, window_size: int = 8, mix_lambda: float = 0.1,
                    *, K_out, V_out, kept_idx, I=None, R=None, Z=None, stream=None,
                    symmetric: bool = False, causal: bool = True, pool: str = "max",
                    select_group: int = 1) -> CompressResult:
    """:func:`compress` through rkv_compress_static: no workspace and no
    allocation, neither here nor in the library, so every output (and any
    debug score buffer, float32 [Bh, N]) is the caller's. The call must need
    at most the library's static scratch (64 MiB per GPU); calls on one GPU
    must not overlap."""
    import torch
    _require_cuda(K, V, Q_win, K_out, V_out, kept_idx, I, R, Z)
    if K.dim() != 3 or V.shape != K.shape or K.shape[2] != HEAD_DIM:
        raise ValueError(f"K and V must be [Bh, N, {HEAD_DIM}] with equal shapes")
    if K.stride(2) != 1 or K.stride(1) != HEAD_DIM or V.stride() != K.stride():
        raise ValueError("K and V rows must be contiguous with equal strides")
    if Q_win.dim() != 4 or Q_win.shape[0] != K.shape[0] or Q_win.shape[2] != window_size \
            or Q_win.shape[3] != HEAD_DIM or not Q_win.is_contiguous():
        raise ValueError("Q_win must be a contiguous [Bh, G, window_size, 128] tensor")
    if not (K.dtype == V.dtype == Q_win.dtype):
        raise TypeError("K, V and Q_win must share a dtype")
    bh, n, b = int(K.shape[0]), int(K.shape[1]), int(kv_budget)
    _check_rows_out("K_out", K_out, K.dtype, bh, min(n, b))
    _check_rows_out("V_out", V_out, K.dtype, bh, min(n, b))
    if K_out.stride() != V_out.stride() or K_out.stride(2) != 1 or K_out.stride(1) != HEAD_DIM:
        raise ValueError("K_out and V_out rows must be contiguous with equal strides")
    _check_index_out("kept_idx", kept_idx, bh * b, shape=(bh, b))
    for name, t in (("I", I), ("R", R), ("Z", Z)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (bh, n)
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [{bh}, {n}] tensor")
    d = dense_desc(bh, n, int(Q_win.shape[1]), window_size, b, mix_lambda, _dtype_code(K),
                   K.stride(0) if bh > 1 else 0, K_out.stride(0) if bh > 1 else 0,
                   variant_bits(symmetric, causal, pool), int(select_group))
    _lib.check(_lib.load().rkv_compress_static(ctypes.byref(d), _ptr(K), _ptr(V), _ptr(Q_win),
                                               _ptr(kept_idx), _ptr(K_out), _ptr(V_out), _ptr(I),
                                               _ptr(R), _ptr(Z), _stream_ptr(stream)))
    return CompressResult(kept_idx, K_out, V_out, I, R, Z)


def paged_desc(num_seqs, kv_heads, gqa, window, page_size, max_pages, num_pages, lam, dtype_code,
               page_stride=0, head_stride=0, slot_stride=0, variant=0):
    return _lib.PagedDesc(num_seqs, kv_heads, HEAD_DIM, gqa, window, page_size, max_pages, num_pages,
                          float(lam), dtype_code, page_stride, head_stride, slot_stride, variant)


def _host_i32(x):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def compress_paged(K_pages, V_pages, page_table, seq_len, budget, Q_win, free_list, free_count: int,
                   window_size: int = 8, mix_lambda: float = 0.1, *, kept_idx=None,
                   debug: bool = False, workspace=None, stream=None, symmetric: bool = False,
                   causal: bool = True, pool: str = "max", shared_heads: bool = False) -> PagedResult:
    """Compress a paged cache in place and return freed pages to ``free_list``.

    K_pages, V_pages: [P, H, page_size, 128] device tensors (any page/head/slot
    strides with contiguous rows); page_table: int32 [S, max_pages] on the
    device, updated in place; seq_len, budget: host sequences of S ints;
    Q_win: [S, H, G, w, 128]; free_list: int32 device tensor of capacity
    free_list.numel() holding ``free_count`` ids. Returns the ragged kept
    indices and the new free count. ``shared_heads``: the H heads of each
    sequence keep one token set, chosen on the sum of their scores
    (RKV_VARIANT_SHARED_HEADS).
    """
    import torch
    _require_cuda(K_pages, V_pages, page_table, Q_win, free_list, kept_idx)
    if not (K_pages.dtype == V_pages.dtype == Q_win.dtype):
        raise TypeError("K_pages, V_pages and Q_win must share a dtype")
    if K_pages.dim() != 4 or K_pages.shape[3] != HEAD_DIM or V_pages.shape != K_pages.shape \
            or K_pages.stride() != V_pages.stride() or K_pages.stride(3) != 1:
        raise ValueError("K_pages and V_pages must be [P, H, page_size, 128] with equal strides")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 [S, max_pages] tensor")
    if free_list.dtype != torch.int32 or not free_list.is_contiguous():
        raise ValueError("free_list must be a contiguous int32 tensor")
    P, H, ps = int(K_pages.shape[0]), int(K_pages.shape[1]), int(K_pages.shape[2])
    S = int(page_table.shape[0])
    g = int(Q_win.shape[2])
    if tuple(Q_win.shape) != (S, H, g, window_size, HEAD_DIM) or not Q_win.is_contiguous():
        raise ValueError("Q_win must be a contiguous [S, H, G, window_size, 128] tensor")
    sl, sl_p = _host_i32(seq_len)
    bu, bu_p = _host_i32(budget)
    if len(sl) != S or len(bu) != S:
        raise ValueError("seq_len and budget need one entry per sequence")
    d = paged_desc(S, H, g, window_size, ps, int(page_table.shape[1]), P, mix_lambda,
                   _dtype_code(K_pages), K_pages.stride(0), K_pages.stride(1), K_pages.stride(2),
                   variant_bits(symmetric, causal, pool)
                   | (_lib.RKV_VARIANT_SHARED_HEADS if shared_heads else 0))
    lib = _lib.load()
    need = lib.rkv_paged_workspace_size(ctypes.byref(d), sl_p, bu_p)
    if need == 0:
        raise _lib.RkvError(_lib.RKV_EINVAL, _lib.last_error())
    dev = K_pages.device
    total_kept = H * int(sum(min(int(a), int(b)) for a, b in zip(sl, bu)))
    if kept_idx is None:
        kept_idx = torch.empty(max(total_kept, 1), dtype=torch.int32, device=dev)
    _check_index_out("kept_idx", kept_idx, total_kept)
    zbuf = torch.empty(max(H * int(sl.sum()), 1), dtype=torch.float32, device=dev) if debug else None
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    cnt = ctypes.c_int32(int(free_count))
    _lib.check(lib.rkv_compress_paged(ctypes.byref(d), _ptr(K_pages), _ptr(V_pages), _ptr(page_table),
                                      sl_p, bu_p, _ptr(Q_win), _ptr(kept_idx), _ptr(free_list),
                                      int(free_list.numel()), ctypes.byref(cnt), _ptr(zbuf),
                                      _ptr(workspace), workspace.numel(), _stream_ptr(stream)))
    return PagedResult(kept_idx, int(cnt.value), zbuf)


class PagePlanResult(NamedTuple):
    pages_now: object       # numpy int32 [S]
    pages_peak: object      # -1 where compression is off
    pages_after: object
    pages_freed: object
    steps_to_event: object  # -1 where compression is off
    totals: dict            # sums over the sequences with compression on


def page_plan(seq_len, budget, page_size: int = 16, divide_length: int = 128) -> PagePlanResult:
    """Page accounting of a paged cache under periodic compression, for a
    scheduler that admits requests on the compressed footprint (host only;
    see rkv_paged_plan in rkv.h)."""
    import numpy as np
    sl, sl_p = _host_i32(seq_len)
    bu, bu_p = _host_i32(budget)
    if sl.shape != bu.shape or sl.ndim != 1:
        raise ValueError("seq_len and budget need one entry per sequence")
    S = int(sl.shape[0])
    plan = (_lib.PagePlan * max(S, 1))()
    tot = (ctypes.c_int64 * 4)()
    _lib.check(_lib.load().rkv_paged_plan(S, sl_p, bu_p, int(page_size), int(divide_length), plan,
                                          tot))
    cols = {f: np.array([getattr(plan[i], f) for i in range(S)], dtype=np.int32)
            for f, _ in _lib.PagePlan._fields_}
    totals = dict(zip(("pages_now", "pages_peak", "pages_after", "pages_freed"), map(int, tot)))
    return PagePlanResult(**cols, totals=totals)


def timing_enable(on: bool = True) -> None:
    _lib.check(_lib.load().rkv_timing_enable(1 if on else 0))


def timing_read(max_kernels: int = 32) -> dict:
    """{kernel name: (timed launches, summed ms)} since timing was enabled."""
    lib = _lib.load()
    names = (ctypes.c_char_p * max_kernels)()
    cnt = (ctypes.c_int32 * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    n = lib.rkv_timing_read(names, cnt, ms, max_kernels)
    if n < 0:
        _lib.check(n)
    return {names[i].decode(): (int(cnt[i]), float(ms[i])) for i in range(min(n, max_kernels))}
