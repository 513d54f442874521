"""Packed (varlen) batches on the GPU vs the fp64 oracle (needs an MI355X).

Queries and keys of all sequences are packed back to back with int32
offsets; lengths are ragged and include empty sequences, sequences with
more queries than keys (causal rows that see nothing) and long query chunks
(hundreds of rows per kv head, the matrix-core path with many row blocks).
"""
import numpy as np
import pytest
import torch

import oracle
import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import split_kv_decode_amd as mx
    mx.lib()
    oracle.build()


def _packed(qlens, klens, Hq, Hkv, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    td = torch.float16 if dtype == "fp16" else torch.bfloat16
    q = torch.randn(sum(qlens), Hq, D, generator=g).to(td)
    k = torch.randn(max(sum(klens), 1), Hkv, D, generator=g).to(td)
    v = torch.randn(max(sum(klens), 1), Hkv, D, generator=g).to(td)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(klens)]), dtype=torch.int32)
    return q, k, v, cq, ck


def _check(qlens, klens, Hq, Hkv, D, dtype, causal, seed=0, num_splits=0, use_ws=False):
    import split_kv_decode_amd as mx
    q, k, v, cq, ck = _packed(qlens, klens, Hq, Hkv, D, dtype, seed)
    mq, mk = max(qlens), max(klens)
    ws = None
    if use_ws:
        dt = 1 if dtype == "bf16" else 0
        need = mx.workspace_size(len(qlens), Hq, Hkv, D, mq, mk, causal, dt, num_splits)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out, lse = mx.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), mq, mk,
                             causal, num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()
    ref_o, ref_l = oracle.attention_varlen(q, k, v, cq, ck, mq, mk, causal, dtype)
    # per query token: out [total_q, Hq, D], lse [Hq, total_q] -> [total_q, Hq]
    rep = parity.compare(parity.to_f64(out), lse.cpu().double().numpy().T, ref_o, ref_l.T,
                         dtype)
    print(qlens, klens, plan, rep, flush=True)
    return plan


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    # (Hq, Hkv, D, dtype): VALU rows (G * max q < 32) and matrix-core rows
    (8, 2, 128, "bf16"), (4, 4, 64, "fp16"), (32, 4, 128, "bf16"), (16, 1, 64, "fp16"),
], ids=lambda s: f"H{s[0]}_{s[1]}_D{s[2]}")
def test_varlen_ragged(shape, causal):
    Hq, Hkv, D, dt = shape
    qlens = [1, 4, 0, 3, 2]
    klens = [700, 1, 50, 0, 1500]
    _check(qlens, klens, Hq, Hkv, D, dt, causal, seed=Hq + D)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_long_query_chunks(causal):
    # chunked prefill: 200 and 37 queries per sequence, 8 query heads per kv head
    _check([200, 37, 1], [900, 37, 3000], 16, 2, 128, "bf16", causal, seed=5)


@pytest.mark.parametrize("num_splits", [1, 4])
def test_varlen_forced_splits_and_workspace(num_splits):
    _check([3, 8], [333, 2049], 16, 2, 128, "fp16", True, seed=7, num_splits=num_splits,
           use_ws=True)


def test_varlen_single_sequence_equals_padded_call():
    import split_kv_decode_amd as mx
    q, k, v, cq, ck = _packed([4], [500], 8, 2, 128, "bf16", 9)
    o1, l1 = mx.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), 4, 500, True)
    o2, l2 = mx.fwd_kvcache(q.unsqueeze(0).cuda(), k.unsqueeze(0).cuda(),
                            v.unsqueeze(0).cuda(), None, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[0])
    assert torch.equal(l1, l2[0].reshape(8, 4))


def test_varlen_chunked_prefill_full_size_sampled():
    """The Llama-70B-shaped chunked-prefill batch at full size (512/512/256/128
    queries against 8K/16K/4K/32K keys, 64/8 heads): fixed partitions with 64
    row blocks per kv head, numbered head block fastest so that each XCD
    serves whole kv heads.  Sampled rows of every sequence (first, last and
    random queries, every head) against the fp64 oracle, each sequence taken
    on its own as a causal (bottom-right) problem; every output finite."""
    import split_kv_decode_amd as mx
    import workloads as wl
    w = wl.VARLEN_WORKLOADS["llama70b_chunked_prefill"]
    q, k, v, cq, ck = wl.make_varlen_inputs(w)
    mq, mk = max(w.qlens), max(w.klens)
    print("case llama70b_chunked_prefill full size", flush=True)
    out, lse = mx.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), mq, mk, True)
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()
    assert plan["schedule"] == 0 and plan["row_block"] == 64 and plan["head_block"] == 1, plan
    assert plan["grid_y"] == w.Hkv * (-(-plan["rows"] // 64)), plan
    out64 = parity.to_f64(out)
    lse64 = lse.cpu().double().numpy()
    assert np.isfinite(out64).all() and np.isfinite(lse64).all()
    r = np.random.default_rng(601)
    for b, (ql, kl) in enumerate(zip(w.qlens, w.klens)):
        q0, k0 = int(cq[b]), int(ck[b])
        qs = sorted({0, ql - 1, *[int(x) for x in r.integers(0, ql, size=3)]})
        rows = [(0, h, i) for i in qs for h in range(w.Hq)]
        ref_o, ref_l = oracle.attention_rows(q[q0:q0 + ql].unsqueeze(0), k[k0:k0 + kl].unsqueeze(0),
                                             v[k0:k0 + kl].unsqueeze(0), rows, None, True, w.dtype)
        go = np.stack([out64[q0 + i, h] for (_, h, i) in rows])
        gl = np.array([lse64[h, q0 + i] for (_, h, i) in rows])
        print(b, ql, kl, parity.compare(go, gl, ref_o, ref_l, w.dtype), flush=True)
