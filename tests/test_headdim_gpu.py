"""Head dims other than 64 / 128, and different key and value dims, on the
GPU vs the fp64 oracle (needs an MI355X).

The SmallQ README's support range allows any head dim and lists 64, 256 and
the DeepSeek V3 MLA split (K side 192, V side 128); here every multiple of 8
up to 256 is accepted.  They run on the matrix-core kernel's padded tiles
(64, 128, 192 x 128, 256): the cases cover each tile, dims just above and
below a tile width, few and many query rows, causal masks, forced splits, a
paged cache and a packed batch.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import split_kv_decode_amd as mx
    mx.lib()
    oracle.build()


@pytest.mark.parametrize("D", [8, 32, 96, 136, 160, 192, 200, 256])
@pytest.mark.parametrize("G,qLen,causal", [(4, 1, False), (8, 8, True)])
def test_equal_head_dims(D, G, qLen, causal):
    w = wl.Workload("hd", B=3, qLen=qLen, Hq=2 * G, Hkv=2, D=D, kv_cap=700, dtype="bf16",
                    causal=causal, sigma=1.0, seed=D + G, len_range=(1, 700))
    inp = wl.make_inputs(w, lengths=[700, 333, 1])
    out, lse, plan = parity.run_gpu(inp)
    ref_o, ref_l = parity.oracle_full(inp)
    rep = parity.compare(out, lse, ref_o, ref_l, "bf16")
    print(D, G, qLen, plan, rep, flush=True)
    assert plan["path"] == "mfma"


def _dkdv(B, qLen, Hq, Hkv, Dk, Dv, cap, lens, dt, causal, num_splits=0, seed=0):
    import split_kv_decode_amd as mx
    q, k, v, sl = wl.make_inputs_dkdv(B, qLen, Hq, Hkv, Dk, Dv, cap, lens, dt, 1.0, seed)
    ws = None
    if num_splits:
        d = 1 if dt == "bf16" else 0
        need = mx.workspace_size_dkdv(B, Hq, Hkv, Dk, Dv, qLen, cap, causal, d, num_splits)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out, lse = mx.fwd_kvcache_dkdv(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), causal,
                                   num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, sl, causal, dt)
    rep = parity.compare(parity.to_f64(out), lse.cpu().double().numpy(), ref_o, ref_l, dt)
    print(Dk, Dv, mx.last_plan().as_dict(), rep, flush=True)


@pytest.mark.parametrize("Dk,Dv", [(192, 128), (128, 64), (64, 128), (256, 64), (24, 200),
                                   (136, 136)])
@pytest.mark.parametrize("qLen,causal", [(1, False), (4, True)])
def test_separate_key_and_value_dims(Dk, Dv, qLen, causal):
    # MLA-like: many query heads on one kv head
    _dkdv(2, qLen, 16, 1, Dk, Dv, 900, [900, 257], "bf16", causal, seed=Dk + Dv)


@pytest.mark.parametrize("num_splits", [1, 5])
def test_separate_dims_forced_splits(num_splits):
    _dkdv(2, 2, 8, 2, 192, 128, 1000, [1000, 40], "fp16", True, num_splits, seed=3)


def test_wide_head_paged_and_packed():
    import split_kv_decode_amd as mx
    w = wl.Workload("hdp", B=3, qLen=2, Hq=8, Hkv=2, D=256, kv_cap=600, dtype="bf16",
                    causal=True, sigma=1.0, seed=11, len_range=(1, 600))
    inp = wl.make_inputs(w, lengths=[600, 75, 16])
    pg = wl.to_paged(inp, 16)
    out, lse, _ = parity.run_gpu_paged(pg, inp)
    ref_o, ref_l = parity.oracle_paged(pg, inp)
    parity.compare(out, lse, ref_o, ref_l, "bf16")
    # packed: the same three sequences, 96-wide heads
    g = torch.Generator().manual_seed(5)
    qlens, klens = [2, 1, 5], [300, 1, 64]
    q = torch.randn(sum(qlens), 8, 96, generator=g).to(torch.bfloat16)
    k = torch.randn(sum(klens), 2, 96, generator=g).to(torch.bfloat16)
    v = torch.randn(sum(klens), 2, 96, generator=g).to(torch.bfloat16)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(klens)]), dtype=torch.int32)
    o2, l2 = mx.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), 5, 300, True)
    torch.cuda.synchronize()
    r_o, r_l = oracle.attention_varlen(q, k, v, cq, ck, 5, 300, True, "bf16")
    parity.compare(parity.to_f64(o2), l2.cpu().double().numpy().T, r_o, r_l.T, "bf16")


def test_head_dim_256_decode_sampled():
    # a Qwen3.5-9B-like decode batch (head_dim 256, GQA 4) at 8K context
    w = wl.Workload("hd256", B=16, qLen=1, Hq=16, Hkv=4, D=256, kv_cap=8192, dtype="bf16",
                    causal=False, sigma=1.0, seed=21, len_range=(1024, 8192))
    inp = wl.make_inputs(w)
    out, lse, plan = parity.run_gpu(inp)
    rows = parity.sample_rows(w, inp.lengths(), 48)
    rep = parity.check_rows(inp, out, lse, rows)
    print(plan, rep, flush=True)
