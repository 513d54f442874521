"""Seeded synthetic decode-attention workloads.

This module only draws inputs: it holds none of the attention arithmetic, so
both the fp64 CPU oracle and the GPU path can be fed from it without sharing
any part of the computation.

The five workload families follow the shapes the source pages talk about:

* the FlashAttention-style example call on the MXFlashAttn package page
  (section "Python API": q of shape (1, 32, 8, 64), k/v of shape (1, 128, 2, 64),
  causal=True) -> ``tiny_causal``;
* the SmallQ FlashAttention README (section on supported range and tests:
  qLen 1..8, non power-of-two kvLen such as 1023 and 3000, 32 heads of 128)
  -> ``smallq_mha_q{q}_kv{kv}``;
* Qwen3-8B / Qwen3-4B shaped long-KV decode (MXFlashAttn sdist README, C500
  re-test tables; the 15,000-token prompt with max_model_len 16384)
  -> ``qwen3_8b_decode`` and ``qwen3_4b_long_decode``;
* Llama-70B shaped decode at 32K context (ops-transformer article, measured
  data section) with a multi-token (qLen 8) draft -> ``llama70b_mtp_decode``;
* a packed batch of Llama-70B shaped chunked-prefill steps (query chunks of
  128-512 tokens against 4K-32K caches, the varlen entry point the
  MXFlashAttn package page names) -> ``llama70b_chunked_prefill``
  (``VARLEN_WORKLOADS``, drawn by ``make_varlen_inputs``).

Recipe (identical on every machine for a given torch version):

1. ``g = torch.Generator().manual_seed(seed)`` on the CPU.
2. Per-sequence valid lengths ``cache_seqlens`` are drawn first (integer
   uniform, both ends inclusive) when the workload has a length range;
   otherwise every sequence uses the full cache capacity.
3. Outlier channels (only where the workload has them): for every kv head,
   ``n_outlier`` distinct channel indices from ``torch.randperm(D)``.
4. ``q`` is drawn as fp32 N(0, sigma^2) and rounded to the storage dtype (RNE).
5. For each batch row b in order: K rows for tokens ``[0, len_b)`` then V rows,
   fp32 N(0, sigma^2); the K outlier channels are multiplied by
   ``outlier_scale`` in fp32 (a power of two, so exact) before rounding.
6. Cache slots at or beyond ``len_b`` are filled with NaN ("poisoned"): the
   method must never read them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    qLen: int
    Hq: int
    Hkv: int
    D: int
    kv_cap: int
    dtype: str  # "fp16" | "bf16"
    causal: bool
    sigma: float
    seed: int
    len_range: Optional[Tuple[int, int]] = None  # inclusive; None -> all kv_cap
    n_outlier: int = 0
    outlier_scale: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16

    @property
    def elt(self) -> int:
        return 2

    def describe(self) -> str:
        lens = (f"cache_seqlens~U[{self.len_range[0]},{self.len_range[1]}]"
                if self.len_range else f"kvLen={self.kv_cap}")
        extra = (f", {self.n_outlier} K channels/head x{self.outlier_scale:g}"
                 if self.n_outlier else "")
        return (f"B={self.B} qLen={self.qLen} Hq={self.Hq} Hkv={self.Hkv} "
                f"D={self.D} kv_cap={self.kv_cap} {lens} {self.dtype} "
                f"{'causal(bottom-right)' if self.causal else 'non-causal'} "
                f"N(0,{self.sigma:g}^2){extra} seed={self.seed}")


def _smallq() -> Dict[str, Workload]:
    out = {}
    for qi, q in enumerate((1, 2, 4, 8)):
        for kj, kv in enumerate((1023, 3000, 4096)):
            name = f"smallq_mha_q{q}_kv{kv}"
            out[name] = Workload(name, B=1, qLen=q, Hq=32, Hkv=32, D=128,
                                 kv_cap=kv, dtype="fp16", causal=False,
                                 sigma=1.0, seed=200 + 10 * qi + kj)
    return out


WORKLOADS: Dict[str, Workload] = {
    "tiny_causal": Workload("tiny_causal", B=1, qLen=32, Hq=8, Hkv=2, D=64,
                            kv_cap=128, dtype="fp16", causal=True, sigma=1.0,
                            seed=101),
    **_smallq(),
    "qwen3_8b_decode": Workload("qwen3_8b_decode", B=64, qLen=1, Hq=32, Hkv=8,
                                D=128, kv_cap=16384, dtype="bf16",
                                causal=False, sigma=1.0, seed=301,
                                len_range=(1024, 16384), n_outlier=2,
                                outlier_scale=8.0),
    "qwen3_4b_long_decode": Workload("qwen3_4b_long_decode", B=16, qLen=1,
                                     Hq=32, Hkv=8, D=128, kv_cap=16384,
                                     dtype="fp16", causal=False, sigma=1.0,
                                     seed=401, len_range=(15000, 16384)),
    "llama70b_mtp_decode": Workload("llama70b_mtp_decode", B=4, qLen=8,
                                    Hq=64, Hkv=8, D=128, kv_cap=32768,
                                    dtype="bf16", causal=True, sigma=0.5,
                                    seed=501),
}

SMALLQ_NAMES: List[str] = [n for n in WORKLOADS if n.startswith("smallq_")]
LONG_KV_NAMES: List[str] = ["qwen3_8b_decode", "qwen3_4b_long_decode",
                            "llama70b_mtp_decode"]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller test variants)."""
    return dataclasses.replace(w, **changes)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: torch.Tensor            # [B, qLen, Hq, D] fp16/bf16
    k_cache: torch.Tensor      # [B, kv_cap, Hkv, D]
    v_cache: torch.Tensor      # [B, kv_cap, Hkv, D]
    cache_seqlens: Optional[torch.Tensor]  # int32 [B] or None (all kv_cap)
    outlier_channels: Optional[torch.Tensor]  # int64 [Hkv, n_outlier]

    def lengths(self) -> List[int]:
        if self.cache_seqlens is None:
            return [self.workload.kv_cap] * self.workload.B
        return [int(x) for x in self.cache_seqlens.tolist()]

    def to(self, device) -> "Inputs":
        mv = lambda t: None if t is None else t.to(device)
        return Inputs(self.workload, mv(self.q), mv(self.k_cache),
                      mv(self.v_cache), mv(self.cache_seqlens),
                      self.outlier_channels)


def make_inputs(w: Workload, seed: Optional[int] = None,
                poison_tail: bool = True,
                lengths: Optional[List[int]] = None) -> Inputs:
    """Draw one batch of inputs for ``w`` on the CPU (see module recipe).

    ``lengths`` overrides the drawn cache_seqlens (used by edge-case tests);
    it is still materialised as an int32 tensor.
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    td = w.torch_dtype
    if lengths is not None:
        seqlens = torch.tensor(lengths, dtype=torch.int32)
    elif w.len_range is not None:
        lo, hi = w.len_range
        seqlens = torch.randint(lo, hi + 1, (w.B,), generator=g,
                                dtype=torch.int64).to(torch.int32)
    else:
        seqlens = None
    outl = None
    if w.n_outlier:
        outl = torch.stack([torch.randperm(w.D, generator=g)[:w.n_outlier]
                            for _ in range(w.Hkv)])
    q = (torch.randn(w.B, w.qLen, w.Hq, w.D, generator=g) * w.sigma).to(td)
    fill = float("nan") if poison_tail else 0.0
    k = torch.full((w.B, w.kv_cap, w.Hkv, w.D), fill, dtype=td)
    v = torch.full((w.B, w.kv_cap, w.Hkv, w.D), fill, dtype=td)
    for b in range(w.B):
        n = w.kv_cap if seqlens is None else int(seqlens[b])
        n = max(0, min(n, w.kv_cap))
        if n == 0:
            continue
        kb = torch.randn(n, w.Hkv, w.D, generator=g) * w.sigma
        if outl is not None:
            for h in range(w.Hkv):
                kb[:, h, outl[h]] *= w.outlier_scale
        vb = torch.randn(n, w.Hkv, w.D, generator=g) * w.sigma
        k[b, :n] = kb.to(td)
        v[b, :n] = vb.to(td)
    return Inputs(w, q, k, v, seqlens, outl)


def kv_bytes(w: Workload, lengths: List[int]) -> int:
    """K and V bytes the method must read: every visible cache row, once."""
    return sum(max(0, min(n, w.kv_cap)) for n in lengths) * w.Hkv * w.D * 2 * w.elt


def algorithmic_bytes(w: Workload, lengths: List[int]) -> int:
    """Q + visible K/V rows + out + lse (fp32) + cache_seqlens (int32)."""
    qo = 2 * w.B * w.qLen * w.Hq * w.D * w.elt
    lse = w.B * w.Hq * w.qLen * 4
    sl = w.B * 4 if w.len_range is not None else 0
    return kv_bytes(w, lengths) + qo + lse + sl


def visible_pairs(w: Workload, lengths: List[int]) -> int:
    """Number of (query row, key) pairs inside the mask, over all heads."""
    tot = 0
    for n in lengths:
        n = max(0, min(n, w.kv_cap))
        for i in range(w.qLen):
            last = (i + n - w.qLen) if w.causal else (n - 1)
            tot += max(0, min(last, n - 1) + 1)
    return tot * w.Hq


def flops(w: Workload, lengths: List[int]) -> int:
    """2*D for QK^T plus 2*D for PV per visible (row, key) pair."""
    return 4 * w.D * visible_pairs(w, lengths)


@dataclasses.dataclass
class PagedCache:
    """A paged copy of a contiguous cache (see ``to_paged``)."""
    page_size: int
    k_pages: torch.Tensor          # [num_pages, page_size, Hkv, D]
    v_pages: torch.Tensor
    block_table: torch.Tensor      # int32 [B, max_pages]
    cache_seqlens: torch.Tensor    # int32 [B]

    def to(self, device) -> "PagedCache":
        return PagedCache(self.page_size, self.k_pages.to(device), self.v_pages.to(device),
                          self.block_table.to(device), self.cache_seqlens.to(device))


def to_paged(inp: Inputs, page_size: int, seed: int = 0, spare_pages: int = 3,
             poison: bool = True, reserve: bool = False) -> PagedCache:
    """Scatter the contiguous cache of ``inp`` into a pool of pages.

    Block i of sequence b (its tokens [i * page_size, (i + 1) * page_size))
    goes to a page drawn from a seeded random permutation of the pool; the
    pool has ``spare_pages`` extra pages.  max_pages = ceil(kv_cap /
    page_size).  Pages and page rows that hold no valid token are filled with
    NaN (``poison``), and the block-table entries past a sequence's last
    block hold out-of-pool values (-1, num_pages, large), so any read of them
    shows.  The lengths are the contiguous cache's (kv_cap when it has none),
    so the logical sequences are the same.  ``reserve``: every block below
    kv_cap gets its own page (for appends), none holds junk.  No arithmetic:
    a data layout."""
    w = inp.workload
    P = page_size
    max_pages = -(-w.kv_cap // P)
    num_pages = w.B * max_pages + spare_pages
    g = torch.Generator().manual_seed(10007 * (seed + 1) + P)
    perm = torch.randperm(num_pages, generator=g)
    fill = float("nan") if poison else 0.0
    kp = torch.full((num_pages, P, w.Hkv, w.D), fill, dtype=w.torch_dtype)
    vp = torch.full((num_pages, P, w.Hkv, w.D), fill, dtype=w.torch_dtype)
    bt = torch.empty((w.B, max_pages), dtype=torch.int32)
    junk = torch.tensor([-1, num_pages, 1 << 30], dtype=torch.int32)
    lens = inp.lengths()
    for b in range(w.B):
        n = max(0, min(lens[b], w.kv_cap))
        nblk = -(-n // P)
        for i in range(max_pages):
            if reserve and i >= nblk:
                bt[b, i] = int(perm[b * max_pages + i])
            elif i < nblk:
                page = int(perm[b * max_pages + i])
                bt[b, i] = page
                t0, t1 = i * P, min((i + 1) * P, n)
                kp[page, : t1 - t0] = inp.k_cache[b, t0:t1]
                vp[page, : t1 - t0] = inp.v_cache[b, t0:t1]
            else:
                bt[b, i] = junk[(b + i) % 3]
    seqlens = torch.tensor([max(0, min(n, w.kv_cap)) for n in lens], dtype=torch.int32)
    return PagedCache(P, kp, vp, bt, seqlens)


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch: sequence b has qlens[b] queries and klens[b] keys."""
    name: str
    qlens: Tuple[int, ...]
    klens: Tuple[int, ...]
    Hq: int
    Hkv: int
    D: int
    dtype: str
    causal: bool
    sigma: float
    seed: int

    @property
    def B(self) -> int:
        return len(self.qlens)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float16 if self.dtype == "fp16" else torch.bfloat16

    def describe(self) -> str:
        return (f"packed B={self.B} q lengths {list(self.qlens)} kv lengths "
                f"{list(self.klens)} Hq={self.Hq} Hkv={self.Hkv} D={self.D} {self.dtype} "
                f"{'causal(bottom-right)' if self.causal else 'non-causal'} "
                f"N(0,{self.sigma:g}^2) seed={self.seed}")


VARLEN_WORKLOADS: Dict[str, VarlenWorkload] = {
    "llama70b_chunked_prefill": VarlenWorkload(
        "llama70b_chunked_prefill", qlens=(512, 512, 256, 128),
        klens=(8192, 16384, 4096, 32768), Hq=64, Hkv=8, D=128, dtype="bf16", causal=True,
        sigma=0.5, seed=601),
}


def make_varlen_inputs(w: VarlenWorkload):
    """(q [total_q, Hq, D], k, v [total_k, Hkv, D], cu_q, cu_k int32 [B + 1]) on
    the CPU: q first, then K and V of each sequence in order, N(0, sigma^2)
    rounded to the storage dtype."""
    g = torch.Generator().manual_seed(w.seed)
    td = w.torch_dtype
    q = (torch.randn(sum(w.qlens), w.Hq, w.D, generator=g) * w.sigma).to(td)
    ks, vs = [], []
    for n in w.klens:
        ks.append((torch.randn(n, w.Hkv, w.D, generator=g) * w.sigma).to(td))
        vs.append((torch.randn(n, w.Hkv, w.D, generator=g) * w.sigma).to(td))
    cu_q = torch.tensor([0] + list(itertools_accumulate(w.qlens)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(itertools_accumulate(w.klens)), dtype=torch.int32)
    return q, torch.cat(ks), torch.cat(vs), cu_q, cu_k


def itertools_accumulate(xs):
    tot = 0
    for x in xs:
        tot += x
        yield tot


def varlen_visible_pairs(w: VarlenWorkload) -> int:
    """(query row, key) pairs inside the mask, over all query heads."""
    tot = 0
    for qb, n in zip(w.qlens, w.klens):
        for i in range(qb):
            last = (i + n - qb) if w.causal else (n - 1)
            tot += max(0, min(last, n - 1) + 1)
    return tot * w.Hq


def varlen_flops(w: VarlenWorkload) -> int:
    """2*D for QK^T plus 2*D for PV per visible (row, key) pair."""
    return 4 * w.D * varlen_visible_pairs(w)


def varlen_bytes(w: VarlenWorkload) -> int:
    """Q, K, V once, out, lse (fp32) and the two offset arrays."""
    tq, tk = sum(w.qlens), sum(w.klens)
    return (2 * tq * w.Hq * w.D * 2 + 2 * tk * w.Hkv * w.D * 2 + tq * w.Hq * 4
            + 2 * (w.B + 1) * 4)


def make_inputs_dkdv(B: int, qLen: int, Hq: int, Hkv: int, Dk: int, Dv: int, kv_cap: int,
                     lengths: List[int], dtype: str, sigma: float, seed: int):
    """Inputs with different key and value head dims, drawn like make_inputs
    (q, then K and V rows per sequence, N(0, sigma^2) rounded to the dtype;
    cache rows at or past a length are NaN): q [B, qLen, Hq, Dk],
    k [B, kv_cap, Hkv, Dk], v [B, kv_cap, Hkv, Dv], cache_seqlens int32 [B]."""
    g = torch.Generator().manual_seed(seed)
    td = torch.float16 if dtype == "fp16" else torch.bfloat16
    q = (torch.randn(B, qLen, Hq, Dk, generator=g) * sigma).to(td)
    k = torch.full((B, kv_cap, Hkv, Dk), float("nan"), dtype=td)
    v = torch.full((B, kv_cap, Hkv, Dv), float("nan"), dtype=td)
    for b in range(B):
        n = max(0, min(lengths[b], kv_cap))
        k[b, :n] = (torch.randn(n, Hkv, Dk, generator=g) * sigma).to(td)
        v[b, :n] = (torch.randn(n, Hkv, Dv, generator=g) * sigma).to(td)
    return q, k, v, torch.tensor(lengths, dtype=torch.int32)
