"""fp64 CPU oracle for decode attention (ctypes binding of ``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code
with the GPU library and never imports it.

``attention`` evaluates softmax(Q K^T / sqrt(D)) V per output row in double
precision, directly from the definition (see ``oracle.c`` for the readings
taken: GQA head mapping, bottom-right causal alignment, empty rows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "libmxfa_oracle.so")

FP16, BF16 = 0, 1


def compile_oracle(out_path: str = LIB_PATH, mutant: int = 0) -> str:
    """Compile oracle.c with gcc (OpenMP, -O2, IEEE semantics kept).

    The library is written under a temporary name and renamed into place, so
    a process loading it (another test worker, say) never sees a partial file."""
    tmp = f"{out_path}.{os.getpid()}.tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", f"-DMXO_MUTANT={int(mutant)}",
           _SRC, "-o", tmp, "-lm"]
    try:
        subprocess.run(cmd, check=True)
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return out_path


def build() -> None:
    compile_oracle(LIB_PATH, 0)


_lib_cache = {}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path == LIB_PATH:
            compile_oracle(path, 0)
        else:
            raise FileNotFoundError(path)
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    ci = ctypes.c_int
    lib.mxo_fp16_to_f64.argtypes = [ctypes.c_uint16]
    lib.mxo_fp16_to_f64.restype = ctypes.c_double
    lib.mxo_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.mxo_bf16_to_f64.restype = ctypes.c_double
    lib.mxo_attention.argtypes = [u16p, u16p, u16p, i32p] + [ci] * 8 + [f64p, f64p, ci]
    lib.mxo_attention.restype = ci
    lib.mxo_attention_dkdv.argtypes = [u16p, u16p, u16p, i32p] + [ci] * 9 + [f64p, f64p, ci]
    lib.mxo_attention_dkdv.restype = ci
    lib.mxo_attention_rows.argtypes = ([u16p, u16p, u16p, i32p] + [ci] * 8 +
                                       [i32p, ci, f64p, f64p, ci])
    lib.mxo_attention_rows.restype = ci
    lib.mxo_mutant_id.argtypes = []
    lib.mxo_mutant_id.restype = ci
    _lib_cache[path] = lib
    return lib


def _as_u16(x) -> np.ndarray:
    """Bit patterns of a 16-bit float array (torch fp16/bf16 or numpy)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype in (torch.float16, torch.bfloat16):
                x = x.view(torch.int16)
            return x.numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype in (np.uint16, np.int16):
        return a.view(np.uint16)
    raise TypeError(f"unsupported array dtype {a.dtype}")


def _dtype_code(x, dtype: Optional[str]) -> int:
    if dtype is not None:
        return {"fp16": FP16, "bf16": BF16}[dtype]
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return BF16 if x.dtype == torch.bfloat16 else FP16
    except ImportError:  # pragma: no cover
        pass
    return FP16


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _seqlens(cache_seqlens, B: int):
    if cache_seqlens is None:
        return None
    try:
        import torch
        if isinstance(cache_seqlens, torch.Tensor):
            cache_seqlens = cache_seqlens.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    s = np.ascontiguousarray(np.asarray(cache_seqlens, dtype=np.int32))
    assert s.shape == (B,)
    return s


def attention(q, k_cache, v_cache, cache_seqlens=None, causal: bool = False,
              dtype: Optional[str] = None, nthreads: int = 0,
              lib_path: str = LIB_PATH) -> Tuple[np.ndarray, np.ndarray]:
    """Return (out [B,qLen,Hq,Dv] float64, lse [B,Hq,qLen] float64).

    q and k_cache share the head dim Dk; v_cache may have another, Dv."""
    qa, ka, va = _as_u16(q), _as_u16(k_cache), _as_u16(v_cache)
    B, qLen, Hq, D = qa.shape
    Bk, kv_cap, Hkv, Dk = ka.shape
    Dv = va.shape[3]
    assert Bk == B and Dk == D and va.shape[:3] == ka.shape[:3]
    sl = _seqlens(cache_seqlens, B)
    out = np.empty((B, qLen, Hq, Dv), dtype=np.float64)
    lse = np.empty((B, Hq, qLen), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.mxo_attention_dkdv(_ptr(qa, ctypes.c_uint16), _ptr(ka, ctypes.c_uint16),
                                _ptr(va, ctypes.c_uint16),
                                None if sl is None else _ptr(sl, ctypes.c_int32),
                                B, Hq, Hkv, Dk, Dv, qLen, kv_cap, int(bool(causal)),
                                _dtype_code(q, dtype), _ptr(out, ctypes.c_double),
                                _ptr(lse, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (rc={rc})")
    return out, lse


def attention_rows(q, k_cache, v_cache, rows: Sequence[Tuple[int, int, int]],
                   cache_seqlens=None, causal: bool = False,
                   dtype: Optional[str] = None, nthreads: int = 0,
                   lib_path: str = LIB_PATH) -> Tuple[np.ndarray, np.ndarray]:
    """Selected output rows (b, h, i): returns (out [n, D], lse [n])."""
    qa, ka, va = _as_u16(q), _as_u16(k_cache), _as_u16(v_cache)
    B, qLen, Hq, D = qa.shape
    _, kv_cap, Hkv, _ = ka.shape
    sl = _seqlens(cache_seqlens, B)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    n = r.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    lib = load(lib_path)
    rc = lib.mxo_attention_rows(_ptr(qa, ctypes.c_uint16), _ptr(ka, ctypes.c_uint16),
                                _ptr(va, ctypes.c_uint16),
                                None if sl is None else _ptr(sl, ctypes.c_int32),
                                B, Hq, Hkv, D, qLen, kv_cap, int(bool(causal)),
                                _dtype_code(q, dtype), _ptr(r, ctypes.c_int32), n,
                                _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double),
                                int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (rc={rc})")
    return out, lse


def gather_pages(k_pages, v_pages, block_table, cache_seqlens=None):
    """The contiguous cache a paged cache stands for.

    A paged KV cache is among the layouts the MXFlashAttn sdist README lists
    (capability matrix); the pages give no layout, and the FlashAttention
    block-table convention is read: token j of sequence b is row j % P of
    page block_table[b, j // P], P the page size.  Returns (k, v) bit patterns
    [B, max_pages * P, Hkv, D] and the lengths; rows at or past a sequence's
    length are zero and are never read.  Every block-table entry that is read
    must name a page of the pool."""
    kp, vp = _as_u16(k_pages), _as_u16(v_pages)
    num_pages, P, Hkv, D = kp.shape
    assert vp.shape == kp.shape
    try:
        import torch
        if isinstance(block_table, torch.Tensor):
            block_table = block_table.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    bt = np.asarray(block_table, dtype=np.int64)
    B, max_pages = bt.shape
    cap = max_pages * P
    sl = _seqlens(cache_seqlens, B)
    lens = [cap] * B if sl is None else [max(0, min(int(x), cap)) for x in sl]
    k = np.zeros((B, cap, Hkv, D), dtype=np.uint16)
    v = np.zeros((B, cap, Hkv, D), dtype=np.uint16)
    for b, n in enumerate(lens):
        j = np.arange(n)
        pages = bt[b, j // P]
        if n and (pages.min() < 0 or pages.max() >= num_pages):
            raise ValueError(f"block table of sequence {b} names a page outside the pool")
        k[b, :n] = kp[pages, j % P]
        v[b, :n] = vp[pages, j % P]
    return k, v, np.asarray(lens, dtype=np.int32)


def attention_paged(q, k_pages, v_pages, block_table, cache_seqlens=None,
                    causal: bool = False, dtype: Optional[str] = None, nthreads: int = 0,
                    lib_path: str = LIB_PATH) -> Tuple[np.ndarray, np.ndarray]:
    """``attention`` over the contiguous cache ``gather_pages`` forms."""
    k, v, lens = gather_pages(k_pages, v_pages, block_table, cache_seqlens)
    return attention(q, k, v, lens, causal, dtype, nthreads, lib_path)


def _lens_for_append(cache_seqlens, B: int, cap: int):
    sl = _seqlens(cache_seqlens, B)
    if sl is None:
        raise ValueError("an append needs cache_seqlens")
    return [max(0, min(int(x), cap)) for x in sl]


def append_kv(k_cache, v_cache, k_new, v_new, cache_seqlens):
    """The cache after an in-call KV append, and the lengths attention sees.

    The MXFlashAttn package page names a FlashAttention-compatible
    attention-with-KV-cache entry point (Python API section) and its sdist
    README lists paged KV append (capability matrix); the FlashAttention rule
    is read: token t of k_new / v_new [B, new_len, Hkv, D] goes to position
    n_b + t of sequence b (n_b = cache_seqlens[b] clamped to [0, kv_cap]),
    positions at or past kv_cap are dropped, and attention then sees
    min(n_b + new_len, kv_cap) keys.  Returns copies (bit patterns) and the
    lengths; the inputs are not modified."""
    k, v = _as_u16(k_cache).copy(), _as_u16(v_cache).copy()
    kn, vn = _as_u16(k_new), _as_u16(v_new)
    B, cap = k.shape[:2]
    new_len = kn.shape[1]
    lens0 = _lens_for_append(cache_seqlens, B, cap)
    for b in range(B):
        for t in range(new_len):
            pos = lens0[b] + t
            if pos < cap:
                k[b, pos] = kn[b, t]
                v[b, pos] = vn[b, t]
    return k, v, np.asarray([min(n + new_len, cap) for n in lens0], dtype=np.int32)


def append_kv_paged(k_pages, v_pages, block_table, k_new, v_new, cache_seqlens):
    """``append_kv`` for a paged cache (layout as in ``gather_pages``):
    position pos of sequence b is row pos % P of page block_table[b, pos // P].
    Returns the updated pool copies and the lengths."""
    kp, vp = _as_u16(k_pages).copy(), _as_u16(v_pages).copy()
    kn, vn = _as_u16(k_new), _as_u16(v_new)
    num_pages, P = kp.shape[:2]
    try:
        import torch
        if isinstance(block_table, torch.Tensor):
            block_table = block_table.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    bt = np.asarray(block_table, dtype=np.int64)
    B, max_pages = bt.shape
    cap = max_pages * P
    new_len = kn.shape[1]
    lens0 = _lens_for_append(cache_seqlens, B, cap)
    for b in range(B):
        for t in range(new_len):
            pos = lens0[b] + t
            if pos < cap:
                page = int(bt[b, pos // P])
                if not 0 <= page < num_pages:
                    raise ValueError(f"block table of sequence {b} names a page outside the pool")
                kp[page, pos % P] = kn[b, t]
                vp[page, pos % P] = vn[b, t]
    return kp, vp, np.asarray([min(n + new_len, cap) for n in lens0], dtype=np.int32)


def _int_array(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                     max_seqlen_k: int, causal: bool = False, dtype: Optional[str] = None,
                     nthreads: int = 0,
                     lib_path: str = LIB_PATH) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over a packed batch (q [total_q, Hq, D], k / v [total_k, Hkv,
    D], offsets [B + 1]): the flash_attn_varlen_func layout the MXFlashAttn
    package page names (Python API section), read the FlashAttention way.

    Each sequence is placed in a padded batch [B, max_seqlen_q, Hq, D] with
    its q_b queries in the LAST q_b rows, so the padded problem's bottom-right
    causal alignment (row i sees key j iff j <= i + n_b - max_seqlen_q) is
    the sequence's own (query i sees j iff j <= i + n_b - q_b); the output
    rows are read back from there.  Returns (out [total_q, Hq, D] float64,
    lse [Hq, total_q] float64); rows outside every sequence stay NaN."""
    qa, ka, va = _as_u16(q), _as_u16(k), _as_u16(v)
    total_q, Hq, D = qa.shape
    total_k, Hkv, _ = ka.shape
    cq, ck = _int_array(cu_seqlens_q), _int_array(cu_seqlens_k)
    assert cq.shape == ck.shape and cq.ndim == 1
    B = cq.shape[0] - 1
    qpad = np.zeros((B, max_seqlen_q, Hq, D), dtype=np.uint16)
    kpad = np.zeros((B, max(max_seqlen_k, 1), Hkv, D), dtype=np.uint16)
    vpad = np.zeros_like(kpad)
    spans, lens = [], []
    for b in range(B):
        q0 = min(max(int(cq[b]), 0), total_q)
        qb = min(min(max(int(cq[b + 1]), q0), total_q) - q0, max_seqlen_q)
        k0 = min(max(int(ck[b]), 0), total_k)
        nb = min(min(max(int(ck[b + 1]), k0), total_k) - k0, max_seqlen_k)
        qpad[b, max_seqlen_q - qb:] = qa[q0:q0 + qb]
        kpad[b, :nb] = ka[k0:k0 + nb]
        vpad[b, :nb] = va[k0:k0 + nb]
        spans.append((q0, qb))
        lens.append(nb)
    code = {FP16: "fp16", BF16: "bf16"}[_dtype_code(q, dtype)]
    o, l = attention(qpad, kpad, vpad, np.asarray(lens, dtype=np.int32), causal, code,
                     nthreads, lib_path)
    out = np.full((total_q, Hq, D), np.nan)
    lse = np.full((Hq, total_q), np.nan)
    for b, (q0, qb) in enumerate(spans):
        if qb:
            out[q0:q0 + qb] = o[b, max_seqlen_q - qb:]
            lse[:, q0:q0 + qb] = l[b, :, max_seqlen_q - qb:]
    return out, lse


def decode16(bits: np.ndarray, dtype: str, lib_path: str = LIB_PATH) -> np.ndarray:
    """Decode an array of 16-bit patterns to float64 with the oracle's decoder."""
    lib = load(lib_path)
    fn = lib.mxo_bf16_to_f64 if dtype == "bf16" else lib.mxo_fp16_to_f64
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([fn(int(x)) for x in flat], dtype=np.float64).reshape(np.shape(bits))
