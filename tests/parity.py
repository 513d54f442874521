"""Comparison of the GPU path with the fp64 oracle.

Tolerances (decode attention over fp16/bf16 inputs, fp32 accumulation):
  * out: max |out - O_ref| <= 4e-3 (fp16) / 2e-2 (bf16);
  * lse: max |lse - lse_ref| <= 1e-3 over finite entries (plus 2^-22 |lse|
    where scores are huge, since fp32 cannot hold 1e-3 absolute there);
    -inf must match -inf exactly;
  * a stricter diagnostic gate, also asserted: max |out - O_ref| must not
    exceed 2 units in the last place of the output dtype at max |O_ref|.  A
    correct fp32 kernel is limited by the final rounding to 16 bits (half an
    ulp), so this catches errors that the absolute tolerance would let pass
    when |O| is small (e.g. an all-zero output at |O| ~ 1e-2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import workloads

OUT_TOL = {"fp16": 4e-3, "bf16": 2e-2}
LSE_TOL = 1e-3
MANT_BITS = {"fp16": 10, "bf16": 7}


def ulp(x: float, dtype: str) -> float:
    if x <= 0:
        x = 2.0 ** -14
    return 2.0 ** (math.floor(math.log2(x)) - MANT_BITS[dtype])


@dataclass
class Report:
    max_err: float
    max_ref: float
    lse_err: float
    rows: int

    def __str__(self):
        return (f"rows={self.rows} max|dO|={self.max_err:.3e} max|O|={self.max_ref:.3e} "
                f"max|dlse|={self.lse_err:.3e}")


def compare(out_gpu: np.ndarray, lse_gpu: np.ndarray, out_ref: np.ndarray,
            lse_ref: np.ndarray, dtype: str, lse_rel: float = 0.0) -> Report:
    """out arrays [..., D] float64, lse arrays [...] float64 (matching order)."""
    assert out_gpu.shape == out_ref.shape, (out_gpu.shape, out_ref.shape)
    assert lse_gpu.shape == lse_ref.shape
    assert np.isfinite(out_gpu).all(), "non-finite output"
    err = np.abs(out_gpu - out_ref)
    max_err = float(err.max()) if err.size else 0.0
    max_ref = float(np.abs(out_ref).max()) if out_ref.size else 0.0
    assert max_err <= OUT_TOL[dtype], f"max|dO|={max_err:.3e} > {OUT_TOL[dtype]}"
    gate = 2 * ulp(max_ref, dtype)
    assert max_err <= gate, f"max|dO|={max_err:.3e} > 2 ulp ({gate:.3e}) at max|O|={max_ref:.3e}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), "lse finiteness differs"
    assert np.all(lse_gpu[~fin] == -np.inf), "empty rows must have lse = -inf"
    lerr = np.abs(lse_gpu[fin] - lse_ref[fin])
    lse_err = float(lerr.max()) if lerr.size else 0.0
    bound = LSE_TOL + lse_rel * np.abs(lse_ref[fin])
    assert np.all(lerr <= bound), f"max|dlse|={lse_err:.3e}"
    return Report(max_err, max_ref, lse_err, int(np.prod(lse_ref.shape)))


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def run_gpu(inp, num_splits: int = 0, use_workspace: bool = True, device="cuda"):
    """Inputs (CPU) -> (out [B,qLen,Hq,D] f64, lse [B,Hq,qLen] f64, plan dict)."""
    import split_kv_decode_amd as mx
    w = inp.workload
    g = inp.to(device)
    if use_workspace or num_splits:
        dt = 1 if w.dtype == "bf16" else 0
        need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt,
                                 num_splits)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        out, lse = mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, g.cache_seqlens, w.causal,
                                  num_splits=num_splits, workspace=ws)
    else:
        out, lse = mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, g.cache_seqlens, w.causal)
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()
    return to_f64(out), lse.detach().cpu().double().numpy(), plan


def oracle_full(inp):
    w = inp.workload
    return oracle.attention(inp.q, inp.k_cache, inp.v_cache, inp.cache_seqlens, w.causal,
                            w.dtype)


def sample_rows(w, lengths, count: int, seed: int = 0):
    """Rows (b, h, i) that include the shortest and longest sequences, the
    first and last head and the first and last query position."""
    rng = np.random.default_rng(seed)
    bmin, bmax = int(np.argmin(lengths)), int(np.argmax(lengths))
    rows = {(bmin, 0, 0), (bmax, w.Hq - 1, w.qLen - 1), (bmin, w.Hq - 1, w.qLen - 1),
            (bmax, 0, 0)}
    while len(rows) < count:
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.qLen))))
    return sorted(rows)


def check_rows(inp, out_gpu, lse_gpu, rows, lse_rel=0.0):
    w = inp.workload
    ref_o, ref_l = oracle.attention_rows(inp.q, inp.k_cache, inp.v_cache, rows,
                                         inp.cache_seqlens, w.causal, w.dtype)
    go = np.stack([out_gpu[b, i, h] for (b, h, i) in rows])
    gl = np.array([lse_gpu[b, h, i] for (b, h, i) in rows])
    return compare(go, gl, ref_o, ref_l, w.dtype, lse_rel)


def run_gpu_paged(paged, inp, num_splits: int = 0, use_workspace: bool = True,
                  device="cuda"):
    """A paged cache (workloads.PagedCache, CPU) with the queries of ``inp``
    -> (out f64, lse f64, plan dict)."""
    import split_kv_decode_amd as mx
    w = inp.workload
    g = paged.to(device)
    q = inp.q.to(device)
    if use_workspace or num_splits:
        dt = 1 if w.dtype == "bf16" else 0
        need = mx.workspace_size_paged(w.B, w.Hq, w.Hkv, w.D, w.qLen, paged.page_size,
                                       paged.block_table.shape[1], w.causal, dt, num_splits)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        out, lse = mx.fwd_kvcache_paged(q, g.k_pages, g.v_pages, g.block_table,
                                        g.cache_seqlens, w.causal, num_splits=num_splits,
                                        workspace=ws)
    else:
        out, lse = mx.fwd_kvcache_paged(q, g.k_pages, g.v_pages, g.block_table,
                                        g.cache_seqlens, w.causal)
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()
    return to_f64(out), lse.detach().cpu().double().numpy(), plan


def oracle_paged(paged, inp):
    w = inp.workload
    return oracle.attention_paged(inp.q, paged.k_pages, paged.v_pages, paged.block_table,
                                  paged.cache_seqlens, w.causal, w.dtype)


def bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def new_tokens(w, new_len, seed):
    """k_new, v_new [B, new_len, Hkv, D] drawn N(0, sigma^2), rounded to the dtype."""
    g = torch.Generator().manual_seed(seed)
    mk = lambda: (torch.randn(w.B, new_len, w.Hkv, w.D, generator=g) * w.sigma).to(
        w.torch_dtype)
    return mk(), mk()


def run_append(inp, new_len, P=0, num_splits=0, use_ws=False, seed=1):
    """In-call KV append on the GPU (contiguous, or paged with pages of P)
    checked against the oracle: the updated cache bit for bit, cache_seqlens
    untouched, attention to tolerance.  Returns the grown lengths."""
    import split_kv_decode_amd as mx
    w = inp.workload
    kn, vn = new_tokens(w, new_len, seed)
    dev = "cuda"
    dt = 1 if w.dtype == "bf16" else 0
    if P:
        pg = workloads.to_paged(inp, P, reserve=True)
        kc, vc, bt, sl = (pg.k_pages.to(dev), pg.v_pages.to(dev), pg.block_table.to(dev),
                          pg.cache_seqlens.to(dev))
        k_ref, v_ref, lens = oracle.append_kv_paged(pg.k_pages, pg.v_pages, pg.block_table,
                                                    kn, vn, pg.cache_seqlens)
        if w.qLen:
            ref_o, ref_l = oracle.attention_paged(inp.q, k_ref, v_ref, pg.block_table, lens,
                                                  w.causal, w.dtype)
        need = mx.workspace_size_paged(w.B, w.Hq, w.Hkv, w.D, w.qLen, P, bt.shape[1],
                                       w.causal, dt, num_splits)
    else:
        kc, vc, bt = inp.k_cache.to(dev), inp.v_cache.to(dev), None
        sl = inp.cache_seqlens.to(dev)
        k_ref, v_ref, lens = oracle.append_kv(inp.k_cache, inp.v_cache, kn, vn,
                                              inp.cache_seqlens)
        if w.qLen:
            ref_o, ref_l = oracle.attention(inp.q, k_ref, v_ref, lens, w.causal, w.dtype)
        need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt,
                                 num_splits)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev) if use_ws else None
    sl_before = sl.clone()
    out, lse = mx.fwd_kvcache_append(inp.q.to(dev), kc, vc, kn.to(dev), vn.to(dev), sl,
                                     w.causal, num_splits=num_splits, workspace=ws,
                                     block_table=bt)
    torch.cuda.synchronize()
    # the cache is updated bit for bit; cache_seqlens is left alone
    assert np.array_equal(bits16(kc), k_ref.view(np.int16))
    assert np.array_equal(bits16(vc), v_ref.view(np.int16))
    assert torch.equal(sl, sl_before)
    if w.qLen:
        rep = compare(to_f64(out), lse.cpu().double().numpy(), ref_o, ref_l, w.dtype)
        print(w.name, new_len, P, mx.last_plan().as_dict(), rep, flush=True)
    return lens
