"""The oracle's in-call KV append, pinned on the CPU (hand-placed tokens,
capacity drops, equality with a cache built directly, paged == contiguous)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build()


def _tagged(B, n, Hkv, D, base):
    """Rows tagged with (base + b, position) in their first two channels."""
    x = np.zeros((B, n, Hkv, D), dtype=np.uint16)
    for b in range(B):
        for j in range(n):
            x[b, j, :, 0] = base + b
            x[b, j, :, 1] = j
    return x


def test_append_places_tokens_by_hand():
    cap = 6
    k = _tagged(3, cap, 1, 4, 100)
    kn = _tagged(3, 2, 1, 4, 200)
    k2, v2, lens = oracle.append_kv(k, k.copy(), kn, kn.copy(), [2, 5, 9])
    assert list(lens) == [4, 6, 6]
    # sequence 0: new tokens 0, 1 at rows 2, 3; the rest untouched
    assert [tuple(k2[0, j, 0, :2]) for j in range(cap)] == \
        [(100, 0), (100, 1), (200, 0), (200, 1), (100, 4), (100, 5)]
    # sequence 1: new token 0 at row 5, token 1 dropped (past kv_cap)
    assert tuple(k2[1, 5, 0, :2]) == (201, 0)
    assert [tuple(k2[1, j, 0, :2]) for j in range(5)] == [(101, j) for j in range(5)]
    # sequence 2 (length clamped to kv_cap): nothing written
    assert np.array_equal(k2[2], k[2])
    assert np.array_equal(k2, v2)
    # inputs are not modified
    assert tuple(k[0, 2, 0, :2]) == (100, 2)


def test_negative_lengths_append_at_the_start():
    k = _tagged(1, 4, 1, 4, 100)
    kn = _tagged(1, 1, 1, 4, 200)
    k2, _, lens = oracle.append_kv(k, k, kn, kn, [-3])
    assert list(lens) == [1] and tuple(k2[0, 0, 0, :2]) == (200, 0)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_after_append_equals_the_cache_built_directly(causal):
    new_len = 3
    w = wl.Workload("ap", B=3, qLen=3, Hq=8, Hkv=2, D=64, kv_cap=40, dtype="bf16",
                    causal=causal, sigma=1.0, seed=12, len_range=(0, 40))
    full = wl.make_inputs(w, lengths=[40, 20, 3])
    n0 = [37, 17, 0]
    kn = torch.stack([full.k_cache[b, n0[b]:n0[b] + new_len] for b in range(3)])
    vn = torch.stack([full.v_cache[b, n0[b]:n0[b] + new_len] for b in range(3)])
    kc, vc = full.k_cache.clone(), full.v_cache.clone()
    for b in range(3):
        kc[b, n0[b]:] = float("nan")
        vc[b, n0[b]:] = float("nan")
    k2, v2, lens = oracle.append_kv(kc, vc, kn, vn, n0)
    assert list(lens) == [40, 20, 3]
    o1, l1 = oracle.attention(full.q, full.k_cache, full.v_cache, full.cache_seqlens, causal)
    o2, l2 = oracle.attention(full.q, k2, v2, lens, causal, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_append_equals_contiguous_append():
    w = wl.Workload("pa", B=3, qLen=2, Hq=4, Hkv=2, D=64, kv_cap=64, dtype="fp16",
                    causal=True, sigma=1.0, seed=13, len_range=(0, 64))
    inp = wl.make_inputs(w, lengths=[10, 63, 0])
    pg = wl.to_paged(inp, 16, poison=False)
    g = torch.Generator().manual_seed(4)
    kn = torch.randn(3, 5, 2, 64, generator=g).to(torch.float16)
    vn = torch.randn(3, 5, 2, 64, generator=g).to(torch.float16)
    # the appended tokens land in blocks the table must name: give every
    # block below kv_cap a page (the junk entries of to_paged would not do)
    bt = pg.block_table.clone()
    npages = pg.k_pages.shape[0]
    used = {int(x) for x in bt.flatten() if 0 <= int(x) < npages}
    spare = sorted(set(range(npages)) - used)
    for b in range(3):
        for i in range(bt.shape[1]):
            if not 0 <= int(bt[b, i]) < npages:
                bt[b, i] = spare.pop()
    kc = torch.zeros_like(inp.k_cache).copy_(inp.k_cache.nan_to_num(0.0))
    vc = torch.zeros_like(inp.v_cache).copy_(inp.v_cache.nan_to_num(0.0))
    k2, v2, lens = oracle.append_kv(kc, vc, kn, vn, inp.cache_seqlens)
    kp2, vp2, lens_p = oracle.append_kv_paged(pg.k_pages, pg.v_pages, bt, kn, vn,
                                              pg.cache_seqlens)
    assert list(lens) == list(lens_p) == [15, 64, 5]
    kg, vg, _ = oracle.gather_pages(kp2, vp2, bt, lens_p)
    for b, n in enumerate(lens):
        assert np.array_equal(kg[b, :n], k2[b, :n]) and np.array_equal(vg[b, :n], v2[b, :n])
