"""ctypes binding of libmxfa.so (include/mxfa.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  PyTorch supplies device memory and the current HIP stream.
If the library has not been built this module raises on first use; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxfa.so")

MXFA_OK, MXFA_ERR_INVALID_ARG, MXFA_ERR_UNSUPPORTED, MXFA_ERR_WORKSPACE, MXFA_ERR_HIP = range(5)
NOALLOC_SCRATCH_BYTES = 32 << 20      # MXFA_NOALLOC_SCRATCH_BYTES in include/mxfa.h
MXFA_FP16, MXFA_BF16 = 0, 1
PATH_NAMES = {0: "valu", 1: "mfma"}

# every symbol include/mxfa.h declares
EXPORTS = ("mxfa_fwd_kvcache", "mxfa_fwd_kvcache_ws", "mxfa_workspace_size",
           "mxfa_fwd_kvcache_noalloc",
           "mxfa_fwd_kvcache_paged", "mxfa_fwd_kvcache_paged_ws", "mxfa_workspace_size_paged",
           "mxfa_fwd_kvcache_append", "mxfa_fwd_kvcache_paged_append", "mxfa_fwd_varlen",
           "mxfa_fwd_kvcache_dkdv", "mxfa_workspace_size_dkdv",
           "mxfa_plan", "mxfa_last_plan", "mxfa_set_timing_events",
           "mxfa_read_probe", "mxfa_status_string", "mxfa_version")


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("layout", ctypes.c_int), ("schedule", ctypes.c_int),
                ("rows", ctypes.c_int),
                ("row_block", ctypes.c_int), ("head_block", ctypes.c_int),
                ("num_splits", ctypes.c_int),
                ("chunk", ctypes.c_int), ("grid_x", ctypes.c_int),
                ("grid_y", ctypes.c_int), ("grid_z", ctypes.c_int),
                ("combine", ctypes.c_int), ("num_cus", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["path"] = PATH_NAMES.get(self.path, str(self.path))
        return d


class PreparedCall:
    """An attention call whose arguments were checked and marshalled once
    (``fwd_kvcache(..., prepare=True)``, ``fwd_kvcache_paged(...,
    prepare=True)``).  ``run()`` enqueues it again on the same stream with the
    same tensors, whose contents may change between runs (a decode loop
    writes the next query into ``q`` and bumps ``cache_seqlens`` in place);
    it returns (out, lse).  The object keeps every tensor it points to alive;
    the stream it was prepared for must outlive it.  Runs on one stream are
    ordered like any other work there; the same PreparedCall must not run on
    two streams at once (they would share its output and scratch)."""
    __slots__ = ("_fn", "_args", "_name", "_dev", "out", "lse", "_keep")

    def __init__(self, fn, args, name, dev, out, lse, keep):
        self._fn, self._args, self._name, self._dev = fn, args, name, dev
        self.out, self.lse, self._keep = out, lse, keep

    def run(self):
        import torch
        if torch.cuda.current_device() != self._dev:
            with torch.cuda.device(self._dev):
                st = self._fn(*self._args)
        else:
            st = self._fn(*self._args)
        if st != MXFA_OK:
            raise MxfaError(st, self._name)
        return self.out, self.lse


class MxfaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = status_string(status)
        super().__init__(f"{what}: {msg}" if what else msg)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmxfa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python split_kv_decode_amd/build.py)")
    # torch ships its own HIP runtime, and a process holds one copy of it:
    # libamdhip64.so.7 is resolved by its soname to whichever copy is loaded
    # first.  Loading this library before torch would install the system
    # copy, and torch would then find no GPU; importing torch first makes its
    # copy the one this library calls (as the tensors it is given require).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.mxfa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp] + [ci] * 8 + [vp]
    L.mxfa_fwd_kvcache.restype = ci
    L.mxfa_fwd_kvcache_ws.argtypes = [vp, vp, vp, vp, vp, vp] + [ci] * 9 + [vp, sz, vp]
    L.mxfa_fwd_kvcache_ws.restype = ci
    L.mxfa_fwd_kvcache_noalloc.argtypes = [vp, vp, vp, vp, vp, vp] + [ci] * 9 + [vp]
    L.mxfa_fwd_kvcache_noalloc.restype = ci
    L.mxfa_workspace_size.argtypes = [ci] * 9 + [ctypes.POINTER(sz)]
    L.mxfa_workspace_size.restype = ci
    L.mxfa_fwd_kvcache_paged.argtypes = [vp] * 7 + [ci] * 10 + [vp]
    L.mxfa_fwd_kvcache_paged.restype = ci
    L.mxfa_fwd_kvcache_paged_ws.argtypes = [vp] * 7 + [ci] * 11 + [vp, sz, vp]
    L.mxfa_fwd_kvcache_paged_ws.restype = ci
    L.mxfa_workspace_size_paged.argtypes = [ci] * 10 + [ctypes.POINTER(sz)]
    L.mxfa_workspace_size_paged.restype = ci
    L.mxfa_fwd_kvcache_append.argtypes = [vp] * 8 + [ci] * 10 + [vp, sz, vp]
    L.mxfa_fwd_kvcache_append.restype = ci
    L.mxfa_fwd_kvcache_paged_append.argtypes = [vp] * 9 + [ci] * 12 + [vp, sz, vp]
    L.mxfa_fwd_kvcache_paged_append.restype = ci
    L.mxfa_fwd_varlen.argtypes = [vp] * 7 + [ci] * 11 + [vp, sz, vp]
    L.mxfa_fwd_varlen.restype = ci
    L.mxfa_fwd_kvcache_dkdv.argtypes = [vp] * 6 + [ci] * 10 + [vp, sz, vp]
    L.mxfa_fwd_kvcache_dkdv.restype = ci
    L.mxfa_workspace_size_dkdv.argtypes = [ci] * 10 + [ctypes.POINTER(sz)]
    L.mxfa_workspace_size_dkdv.restype = ci
    L.mxfa_plan.argtypes = [ci] * 10 + [ctypes.POINTER(Plan)]
    L.mxfa_plan.restype = ci
    L.mxfa_last_plan.argtypes = [ctypes.POINTER(Plan)]
    L.mxfa_last_plan.restype = ci
    L.mxfa_set_timing_events.argtypes = [vp, vp]
    L.mxfa_set_timing_events.restype = ci
    L.mxfa_read_probe.argtypes = [vp, sz, ci, vp, ci, vp]
    L.mxfa_read_probe.restype = ci
    L.mxfa_status_string.argtypes = [ci]
    L.mxfa_status_string.restype = ctypes.c_char_p
    L.mxfa_version.argtypes = []
    L.mxfa_version.restype = ci
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().mxfa_status_string(int(status)).decode()


def version() -> int:
    return lib().mxfa_version()


def plan(B, Hq, Hkv, D, qLen, kv_cap, causal=False, dtype=MXFA_FP16, num_splits=0,
         num_cus=0) -> Plan:
    p = Plan()
    st = lib().mxfa_plan(B, Hq, Hkv, D, qLen, kv_cap, int(causal), int(dtype),
                         int(num_splits), int(num_cus), ctypes.byref(p))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_plan")
    return p


def last_plan() -> Plan:
    p = Plan()
    st = lib().mxfa_last_plan(ctypes.byref(p))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_last_plan")
    return p


def set_timing_events(before=None, after=None) -> None:
    """Record raw HIP events (handles as ints, e.g. torch.cuda.Event.cuda_event)
    around the split kernel of every later call on this thread; None, None
    turns it off."""
    vp = lambda e: None if e is None else ctypes.c_void_p(int(e))
    st = lib().mxfa_set_timing_events(vp(before), vp(after))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_set_timing_events")


def workspace_size(B, Hq, Hkv, D, qLen, kv_cap, causal=False, dtype=MXFA_FP16,
                   num_splits=0) -> int:
    n = ctypes.c_size_t(0)
    st = lib().mxfa_workspace_size(B, Hq, Hkv, D, qLen, kv_cap, int(causal), int(dtype),
                                   int(num_splits), ctypes.byref(n))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_workspace_size")
    return n.value


def workspace_size_paged(B, Hq, Hkv, D, qLen, page_size, max_pages, causal=False,
                         dtype=MXFA_FP16, num_splits=0) -> int:
    n = ctypes.c_size_t(0)
    st = lib().mxfa_workspace_size_paged(B, Hq, Hkv, D, qLen, page_size, max_pages,
                                         int(causal), int(dtype), int(num_splits),
                                         ctypes.byref(n))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_workspace_size_paged")
    return n.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return MXFA_FP16
    if t.dtype == torch.bfloat16:
        return MXFA_BF16
    raise TypeError(f"q must be float16 or bfloat16, got {t.dtype}")


def fwd_kvcache(q, k_cache, v_cache, cache_seqlens=None, causal: bool = False,
                out=None, lse=None, return_lse: bool = True, num_splits: int = 0,
                workspace=None, stream=None, prepare: bool = False, noalloc: bool = False):
    """Decode attention on the current HIP stream; returns (out, lse), or with
    prepare=True a PreparedCall that enqueues the call on each run().

    q [B, qLen, Hq, D]; k_cache, v_cache [B, kv_cap, Hkv, D] (fp16 or bf16,
    contiguous, on one GPU); cache_seqlens int32 [B] or None.  With
    num_splits > 0 or an explicit workspace (a uint8 tensor), the
    caller-workspace entry point is used; with noalloc=True the
    allocation-free one (the library's fixed scratch array; no workspace);
    otherwise the library allocates its scratch on the stream.
    """
    import torch
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, qLen, Hq, D = q.shape
    Bk, kv_cap, Hkv, Dk = k_cache.shape
    if Bk != B or Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache must be [B, kv_cap, Hkv, D] matching q")
    dt = _dtype_code(q)
    if cache_seqlens is not None:
        if (cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda
                or tuple(cache_seqlens.shape) != (B,) or not cache_seqlens.is_contiguous()):
            raise ValueError("cache_seqlens must be a contiguous int32 GPU tensor of shape [B]")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, qLen), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, qLen)
                              or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, qLen]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = (ptr(q), ptr(k_cache), ptr(v_cache), ptr(cache_seqlens), ptr(out), ptr(lse),
            B, Hq, Hkv, D, qLen, kv_cap, int(bool(causal)), dt)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc=True uses the library's own scratch: pass no workspace")
        fn = lib().mxfa_fwd_kvcache_noalloc
        full = (*args, int(num_splits), ctypes.c_void_p(stream))
    elif workspace is None and num_splits == 0:
        fn, full = lib().mxfa_fwd_kvcache, (*args, ctypes.c_void_p(stream))
    else:
        if workspace is None:
            with torch.cuda.device(q.device):
                need = workspace_size(B, Hq, Hkv, D, qLen, kv_cap, causal, dt, num_splits)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        fn = lib().mxfa_fwd_kvcache_ws
        full = (*args, int(num_splits), ptr(workspace),
                workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream))
    name = "mxfa_fwd_kvcache_noalloc" if noalloc else "mxfa_fwd_kvcache"
    call = PreparedCall(fn, full, name, q.device.index, out, lse,
                        (q, k_cache, v_cache, cache_seqlens, workspace))
    return call if prepare else call.run()


def fwd_kvcache_paged(q, k_pages, v_pages, block_table, cache_seqlens=None,
                      causal: bool = False, out=None, lse=None, return_lse: bool = True,
                      num_splits: int = 0, workspace=None, stream=None,
                      prepare: bool = False):
    """Decode attention over a paged cache on the current HIP stream.

    q [B, qLen, Hq, D]; k_pages, v_pages [num_pages, page_size, Hkv, D];
    block_table int32 [B, max_pages] (token j of sequence b is row
    j % page_size of page block_table[b, j // page_size]); cache_seqlens
    int32 [B] or None.  Returns (out, lse), or with prepare=True a
    PreparedCall."""
    import torch
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, qLen, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_pages.shape
    if Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages / v_pages must be [num_pages, page_size, Hkv, D] matching q")
    if (not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32
            or not block_table.is_cuda or block_table.dim() != 2
            or block_table.shape[0] != B or not block_table.is_contiguous()):
        raise ValueError("block_table must be a contiguous int32 GPU tensor [B, max_pages]")
    max_pages = block_table.shape[1]
    dt = _dtype_code(q)
    if cache_seqlens is not None:
        if (cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda
                or tuple(cache_seqlens.shape) != (B,) or not cache_seqlens.is_contiguous()):
            raise ValueError("cache_seqlens must be a contiguous int32 GPU tensor of shape [B]")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, qLen), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, qLen)
                              or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, qLen]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    args = (ptr(q), ptr(k_pages), ptr(v_pages), ptr(block_table), ptr(cache_seqlens),
            ptr(out), ptr(lse), B, Hq, Hkv, D, qLen, num_pages, page_size, max_pages,
            int(bool(causal)), dt)
    if workspace is None and num_splits == 0:
        fn, full = lib().mxfa_fwd_kvcache_paged, (*args, ctypes.c_void_p(stream))
    else:
        if workspace is None:
            with torch.cuda.device(q.device):
                need = workspace_size_paged(B, Hq, Hkv, D, qLen, page_size, max_pages, causal,
                                            dt, num_splits)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        fn = lib().mxfa_fwd_kvcache_paged_ws
        full = (*args, int(num_splits), ptr(workspace),
                workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream))
    call = PreparedCall(fn, full, "mxfa_fwd_kvcache_paged", q.device.index, out, lse,
                        (q, k_pages, v_pages, block_table, cache_seqlens, workspace))
    return call if prepare else call.run()


def fwd_kvcache_append(q, k_cache, v_cache, k_new, v_new, cache_seqlens, causal: bool = False,
                       out=None, lse=None, return_lse: bool = True, num_splits: int = 0,
                       workspace=None, block_table=None,
                       stream=None) -> Tuple[object, Optional[object]]:
    """Write k_new / v_new [B, new_len, Hkv, D] into the cache at
    cache_seqlens[b] + t, then attend over cache_seqlens + new_len keys.

    Contiguous cache [B, kv_cap, Hkv, D], or with ``block_table`` a paged
    pool [num_pages, page_size, Hkv, D].  The cache is updated in place;
    cache_seqlens is not."""
    import torch
    paged = block_table is not None
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new),
                    ("v_new", v_new)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, qLen, Hq, D = q.shape
    C0, C1, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache must match each other and q's head dim")
    if not paged and C0 != B:
        raise ValueError("a contiguous cache must be [B, kv_cap, Hkv, D]")
    Bn, new_len, Hn, Dn = k_new.shape
    if (Bn, Hn, Dn) != (B, Hkv, D) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new / v_new must be [B, new_len, Hkv, D]")
    if (not isinstance(cache_seqlens, torch.Tensor) or cache_seqlens.dtype != torch.int32
            or not cache_seqlens.is_cuda or tuple(cache_seqlens.shape) != (B,)
            or not cache_seqlens.is_contiguous()):
        raise ValueError("cache_seqlens must be a contiguous int32 GPU tensor of shape [B]")
    if paged and (block_table.dtype != torch.int32 or not block_table.is_cuda
                  or block_table.dim() != 2 or block_table.shape[0] != B
                  or not block_table.is_contiguous()):
        raise ValueError("block_table must be a contiguous int32 GPU tensor [B, max_pages]")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, qLen), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, qLen)
                              or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, qLen]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        if paged:
            st = lib().mxfa_fwd_kvcache_paged_append(
                ptr(q), ptr(k_cache), ptr(v_cache), ptr(block_table), ptr(k_new), ptr(v_new),
                ptr(cache_seqlens), ptr(out), ptr(lse), B, Hq, Hkv, D, qLen, new_len, C0, C1,
                block_table.shape[1], int(bool(causal)), dt, int(num_splits), ptr(workspace),
                wsb, ctypes.c_void_p(stream))
        else:
            st = lib().mxfa_fwd_kvcache_append(
                ptr(q), ptr(k_cache), ptr(v_cache), ptr(k_new), ptr(v_new), ptr(cache_seqlens),
                ptr(out), ptr(lse), B, Hq, Hkv, D, qLen, new_len, C1, int(bool(causal)), dt,
                int(num_splits), ptr(workspace), wsb, ctypes.c_void_p(stream))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_fwd_kvcache_append")
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
               causal: bool = False, out=None, lse=None, return_lse: bool = True,
               num_splits: int = 0, workspace=None,
               stream=None) -> Tuple[object, Optional[object]]:
    """Attention over a packed batch: q [total_q, Hq, D], k / v [total_k, Hkv, D],
    cu_seqlens_q / cu_seqlens_k int32 [B + 1] on the GPU.  Returns (out
    [total_q, Hq, D], lse [Hq, total_q])."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 3:
            raise ValueError(f"{name} must be 3-D")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k / v must be [total_k, Hkv, D] matching q")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda
                or t.dim() != 1 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor [B + 1]")
    if cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.shape[0] < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1]")
    B = cu_seqlens_q.shape[0] - 1
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q)
                              or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [Hq, total_q]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptr = lambda t: None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib().mxfa_fwd_varlen(ptr(q), ptr(k), ptr(v), ptr(cu_seqlens_q),
                                   ptr(cu_seqlens_k), ptr(out), ptr(lse), B, Hq, Hkv, D,
                                   total_q, total_k, int(max_seqlen_q), int(max_seqlen_k),
                                   int(bool(causal)), dt, int(num_splits), ptr(workspace),
                                   wsb, ctypes.c_void_p(stream))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_fwd_varlen")
    return out, lse


def fwd_kvcache_dkdv(q, k_cache, v_cache, cache_seqlens=None, causal: bool = False,
                     out=None, lse=None, return_lse: bool = True, num_splits: int = 0,
                     workspace=None, stream=None) -> Tuple[object, Optional[object]]:
    """Decode attention with different key and value head dims: q [B, qLen,
    Hq, Dk], k_cache [B, kv_cap, Hkv, Dk], v_cache [B, kv_cap, Hkv, Dv];
    returns out [B, qLen, Hq, Dv] and lse [B, Hq, qLen]."""
    import torch
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    B, qLen, Hq, Dk = q.shape
    Bk, kv_cap, Hkv, Dk2 = k_cache.shape
    Dv = v_cache.shape[3]
    if Bk != B or Dk2 != Dk or tuple(v_cache.shape[:3]) != (B, kv_cap, Hkv):
        raise ValueError("k_cache [B, kv_cap, Hkv, Dk] and v_cache [B, kv_cap, Hkv, Dv] must "
                         "match q")
    dt = _dtype_code(q)
    if cache_seqlens is not None:
        if (cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda
                or tuple(cache_seqlens.shape) != (B,) or not cache_seqlens.is_contiguous()):
            raise ValueError("cache_seqlens must be a contiguous int32 GPU tensor of shape [B]")
    if out is None:
        out = torch.empty((B, qLen, Hq, Dv), dtype=q.dtype, device=q.device)
    elif (tuple(out.shape) != (B, qLen, Hq, Dv) or out.dtype != q.dtype
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor [B, qLen, Hq, Dv] of q's dtype")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, qLen), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, qLen)
                              or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, qLen]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib().mxfa_fwd_kvcache_dkdv(ptr(q), ptr(k_cache), ptr(v_cache), ptr(cache_seqlens),
                                         ptr(out), ptr(lse), B, Hq, Hkv, Dk, Dv, qLen, kv_cap,
                                         int(bool(causal)), dt, int(num_splits), ptr(workspace),
                                         wsb, ctypes.c_void_p(stream))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_fwd_kvcache_dkdv")
    return out, lse


def workspace_size_dkdv(B, Hq, Hkv, Dk, Dv, qLen, kv_cap, causal=False, dtype=MXFA_FP16,
                        num_splits=0) -> int:
    n = ctypes.c_size_t(0)
    st = lib().mxfa_workspace_size_dkdv(B, Hq, Hkv, Dk, Dv, qLen, kv_cap, int(causal),
                                        int(dtype), int(num_splits), ctypes.byref(n))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_workspace_size_dkdv")
    return n.value


def read_probe(src, nontemporal: bool, sink, num_cus: int = 0, stream=None) -> None:
    """Enqueue one streaming read of the whole device tensor `src` (the
    practical read-ceiling kernel); `sink` is a device int32/uint32 tensor of
    at least one element.  Time it with events on `stream`."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    nbytes = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        st = lib().mxfa_read_probe(ctypes.c_void_p(src.data_ptr()), nbytes, int(bool(nontemporal)),
                                   ctypes.c_void_p(sink.data_ptr()), int(num_cus),
                                   ctypes.c_void_p(stream))
    if st != MXFA_OK:
        raise MxfaError(st, "mxfa_read_probe")
