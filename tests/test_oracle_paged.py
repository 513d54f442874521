"""The oracle's reading of a paged cache, pinned on the CPU.

A paged KV cache is listed among the layouts of the MXFlashAttn sdist
README (capability matrix) without a layout; the FlashAttention block-table
convention is read (token j of sequence b is row j % P of page
block_table[b, j // P]).  These pins fix that index mapping by hand-worked
placements and tie the paged oracle to the contiguous one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build()


def _pool(num_pages, P, Hkv, D):
    """Pages whose every row is tagged with (page, row) in its first two channels."""
    kp = np.zeros((num_pages, P, Hkv, D), dtype=np.uint16)
    for p in range(num_pages):
        for r in range(P):
            kp[p, r, :, 0] = p
            kp[p, r, :, 1] = r
    return kp


def test_gather_places_each_token_by_hand():
    # P = 2, two sequences of 5 and 3 tokens; pages named in a scrambled order
    P = 2
    kp = _pool(7, P, 1, 4)
    bt = np.array([[5, 0, 3], [6, 2, 1]], dtype=np.int32)
    k, v, lens = oracle.gather_pages(kp, kp.copy(), bt, [5, 3])
    assert list(lens) == [5, 3]
    # sequence 0: tokens 0,1 -> page 5 rows 0,1; 2,3 -> page 0; 4 -> page 3 row 0
    want0 = [(5, 0), (5, 1), (0, 0), (0, 1), (3, 0)]
    want1 = [(6, 0), (6, 1), (2, 0)]
    assert [tuple(k[0, j, 0, :2]) for j in range(5)] == want0
    assert [tuple(k[1, j, 0, :2]) for j in range(3)] == want1
    # past the length nothing is taken from the pool
    assert not k[1, 3:].any() and not v[1, 3:].any()


def test_gather_ignores_entries_past_the_length_and_rejects_bad_ones():
    P = 4
    kp = _pool(3, P, 1, 4)
    bt = np.array([[2, -1, 99]], dtype=np.int32)      # only block 0 is read for n <= 4
    k, _, _ = oracle.gather_pages(kp, kp, bt, [4])
    assert [tuple(k[0, j, 0, :2]) for j in range(4)] == [(2, 0), (2, 1), (2, 2), (2, 3)]
    with pytest.raises(ValueError):
        oracle.gather_pages(kp, kp, bt, [5])          # block 1 names page -1


@pytest.mark.parametrize("P", [16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_paged_attention_equals_the_contiguous_cache(P, causal):
    w = wl.Workload("pg", B=3, qLen=4, Hq=8, Hkv=2, D=64, kv_cap=150, dtype="bf16",
                    causal=causal, sigma=1.0, seed=5, len_range=(0, 150))
    inp = wl.make_inputs(w, lengths=[150, 37, 0])
    pg = wl.to_paged(inp, P, seed=1)
    o1, l1 = oracle.attention(inp.q, inp.k_cache, inp.v_cache, inp.cache_seqlens, causal)
    o2, l2 = oracle.attention_paged(inp.q, pg.k_pages, pg.v_pages, pg.block_table,
                                    pg.cache_seqlens, causal)
    assert np.array_equal(o1, o2)
    assert np.array_equal(l1, l2)


def test_shared_pages_give_equal_rows():
    # two sequences whose block tables name the same pages see the same keys
    P = 16
    g = torch.Generator().manual_seed(3)
    kp = torch.randn(4, P, 1, 64, generator=g).to(torch.float16)
    vp = torch.randn(4, P, 1, 64, generator=g).to(torch.float16)
    q1 = torch.randn(1, 1, 2, 64, generator=g).to(torch.float16)
    q = torch.cat([q1, q1])
    bt = torch.tensor([[2, 0], [2, 0]], dtype=torch.int32)
    o, l = oracle.attention_paged(q, kp, vp, bt, torch.tensor([20, 20], dtype=torch.int32))
    assert np.array_equal(o[0], o[1]) and np.array_equal(l[0], l[1])
    # and a table that names other pages does not
    bt2 = torch.tensor([[2, 0], [0, 2]], dtype=torch.int32)
    o2, _ = oracle.attention_paged(q, kp, vp, bt2, torch.tensor([20, 20], dtype=torch.int32))
    assert not np.array_equal(o2[0], o2[1])


def test_to_paged_keeps_every_valid_token():
    w = wl.Workload("tp", B=2, qLen=1, Hq=2, Hkv=2, D=64, kv_cap=70, dtype="fp16",
                    causal=False, sigma=1.0, seed=9, len_range=(1, 70))
    inp = wl.make_inputs(w, lengths=[70, 33])
    pg = wl.to_paged(inp, 16)
    k, v, lens = oracle.gather_pages(pg.k_pages, pg.v_pages, pg.block_table, pg.cache_seqlens)
    ku = inp.k_cache.view(torch.int16).numpy().view(np.uint16)
    vu = inp.v_cache.view(torch.int16).numpy().view(np.uint16)
    for b, n in enumerate(lens):
        assert np.array_equal(k[b, :n], ku[b, :n]) and np.array_equal(v[b, :n], vu[b, :n])
    # the pool holds NaN wherever no valid token lives
    nan_rows = torch.isnan(pg.k_pages.float()).all(dim=-1).all(dim=-1).sum().item()
    assert nan_rows == pg.k_pages.shape[0] * 16 - (70 + 33)
