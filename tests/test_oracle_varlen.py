"""The oracle's packed (varlen) batch, pinned on the CPU against separate
single-sequence calls of the contiguous oracle (each with its own qLen and
cache), so the right-aligned padding and the per-sequence causal alignment
are checked by an independent path."""
import numpy as np
import pytest
import torch

import oracle


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build()


def _packed(qlens, klens, Hq, Hkv, D, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(sum(qlens), Hq, D, generator=g).to(dtype)
    k = torch.randn(sum(klens), Hkv, D, generator=g).to(dtype)
    v = torch.randn(sum(klens), Hkv, D, generator=g).to(dtype)
    cq = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(klens)]).astype(np.int32)
    return q, k, v, cq, ck


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_one_call_per_sequence(causal):
    qlens, klens = [3, 1, 0, 5], [10, 0, 4, 5]
    q, k, v, cq, ck = _packed(qlens, klens, 4, 2, 64, 1)
    o, l = oracle.attention_varlen(q, k, v, cq, ck, 5, 10, causal)
    for b, (qb, nb) in enumerate(zip(qlens, klens)):
        if qb == 0:
            continue
        q1 = q[cq[b]:cq[b + 1]].unsqueeze(0)
        k1 = k[ck[b]:ck[b + 1]].unsqueeze(0) if nb else torch.zeros(1, 1, 2, 64, dtype=q.dtype)
        v1 = v[ck[b]:ck[b + 1]].unsqueeze(0) if nb else torch.zeros(1, 1, 2, 64, dtype=q.dtype)
        o1, l1 = oracle.attention(q1, k1, v1, np.array([nb], np.int32), causal)
        assert np.array_equal(o[cq[b]:cq[b + 1]], o1[0])
        assert np.array_equal(l[:, cq[b]:cq[b + 1]], l1[0])


def test_causal_rows_before_the_keys_see_nothing():
    # 5 queries against 2 keys: rows 0..2 see no key (j <= i + 2 - 5)
    q, k, v, cq, ck = _packed([5], [2], 2, 1, 64, 2)
    o, l = oracle.attention_varlen(q, k, v, cq, ck, 5, 2, True)
    assert np.all(np.isneginf(l[:, :3])) and np.all(o[:3] == 0)
    assert np.all(np.isfinite(l[:, 3:]))
    # row 3 sees key 0 only: its output is v[0] exactly
    vd = oracle.decode16(v.view(torch.int16).numpy().view(np.uint16), "bf16")
    for h in range(2):
        assert np.array_equal(o[3, h], vd[0, 0])
