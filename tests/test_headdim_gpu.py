"""Head dims other than 64 / 128, and different key and value dims, on the
GPU vs the fp64 oracle (needs an MI355X).

The SmallQ README's support range allows any head dim and lists 64, 256 and
the DeepSeek V3 MLA split (K side 192, V side 128); here every head dim from 1
to 256 is accepted.  They run on the matrix-core kernel's padded tiles
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


# ------------------------------------------- head dims not multiples of 8
#
# The SmallQ README's support range allows any head dim of at least 1; such
# rows are only 2-byte aligned, so the matrix-core kernel assembles every
# 16-byte chunk from 16-bit loads, zeroes the elements past the head (the
# next head's values, or a poisoned NaN slot, must not leak in) and stores
# outputs element by element (nothing past the head may be written: out is
# pre-filled with a sentinel and checked).

ODD_DIMS = [1, 3, 17, 36, 100, 129, 130, 255]


def _run_sentinel(inp, num_splits=0, paged=None):
    """The contiguous (or paged) call with out pre-filled with a sentinel
    past the tensor's own elements; returns out, lse as float64 arrays."""
    import split_kv_decode_amd as mx
    w = inp.workload
    g = inp.to("cuda")
    # a buffer one row longer than out, filled with a sentinel; out is a view
    # of its first elements, so a store past the last head row would show
    n = w.B * w.qLen * w.Hq * w.D
    buf = torch.full((n + 64,), 7.0, dtype=w.torch_dtype, device="cuda")
    out = buf[:n].view(w.B, w.qLen, w.Hq, w.D)
    ws = None
    if num_splits:
        dt = 1 if w.dtype == "bf16" else 0
        if paged is None:
            need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt,
                                     num_splits)
        else:
            need = mx.workspace_size_paged(w.B, w.Hq, w.Hkv, w.D, w.qLen, paged.page_size,
                                           paged.block_table.shape[1], w.causal, dt, num_splits)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    if paged is None:
        _, lse = mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, g.cache_seqlens, w.causal, out=out,
                                num_splits=num_splits, workspace=ws)
    else:
        pg = paged.to("cuda")
        _, lse = mx.fwd_kvcache_paged(g.q, pg.k_pages, pg.v_pages, pg.block_table,
                                      pg.cache_seqlens, w.causal, out=out,
                                      num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    assert bool((buf[n:] == 7.0).all()), "a store went past the output"
    return parity.to_f64(out), lse.cpu().double().numpy(), mx.last_plan().as_dict()


@pytest.mark.parametrize("D", ODD_DIMS)
@pytest.mark.parametrize("G,qLen,causal,dtype", [(4, 1, False, "bf16"), (8, 8, True, "fp16"),
                                                (1, 3, True, "bf16")])
def test_odd_head_dims(D, G, qLen, causal, dtype):
    w = wl.Workload("odd", B=3, qLen=qLen, Hq=2 * G, Hkv=2, D=D, kv_cap=700, dtype=dtype,
                    causal=causal, sigma=1.0, seed=500 + D + G, len_range=(0, 700))
    inp = wl.make_inputs(w, lengths=[700, 333, 1])
    out, lse, plan = _run_sentinel(inp)
    ref_o, ref_l = parity.oracle_full(inp)
    rep = parity.compare(out, lse, ref_o, ref_l, dtype)
    print(D, G, qLen, plan, rep, flush=True)
    assert (plan["path"], plan["row_block"], plan["head_block"]) == ("mfma", 16, 1)


@pytest.mark.parametrize("D,P,num_splits", [(3, 16, 0), (100, 64, 0), (129, 16, 3), (255, 32, 0),
                                            (17, 64, 7)])
def test_odd_head_dims_paged_and_forced_splits(D, P, num_splits):
    w = wl.Workload("oddp", B=3, qLen=2, Hq=8, Hkv=2, D=D, kv_cap=500, dtype="bf16",
                    causal=True, sigma=1.0, seed=600 + D, len_range=(0, 500))
    inp = wl.make_inputs(w, lengths=[500, 0, 77])
    pg = wl.to_paged(inp, P)
    out, lse, plan = _run_sentinel(inp, num_splits, paged=pg)
    ref_o, ref_l = parity.oracle_paged(pg, inp)
    parity.compare(out, lse, ref_o, ref_l, "bf16")
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    out, lse, _ = _run_sentinel(inp, num_splits)
    parity.compare(out, lse, *parity.oracle_full(inp), "bf16")


@pytest.mark.parametrize("Dk,Dv", [(1, 7), (3, 5), (17, 100), (129, 64), (255, 129), (100, 130),
                                   (36, 250), (192, 127), (191, 3), (150, 121)])
@pytest.mark.parametrize("qLen,causal", [(1, False), (4, True)])
def test_odd_separate_key_and_value_dims(Dk, Dv, qLen, causal):
    _dkdv(2, qLen, 16, 1, Dk, Dv, 900, [900, 257], "bf16", causal, seed=Dk * 7 + Dv)


def test_odd_head_dims_packed_and_appended():
    import split_kv_decode_amd as mx
    g = torch.Generator().manual_seed(9)
    qlens, klens, D = [2, 1, 5], [300, 1, 64], 45
    q = torch.randn(sum(qlens), 8, D, generator=g).to(torch.float16)
    k = torch.randn(sum(klens), 2, D, generator=g).to(torch.float16)
    v = torch.randn(sum(klens), 2, D, generator=g).to(torch.float16)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(klens)]), dtype=torch.int32)
    o2, l2 = mx.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), 5, 300, True)
    torch.cuda.synchronize()
    r_o, r_l = oracle.attention_varlen(q, k, v, cq, ck, 5, 300, True, "fp16")
    parity.compare(parity.to_f64(o2), l2.cpu().double().numpy().T, r_o, r_l.T, "fp16")
    # in-call append with an odd head dim, contiguous and paged: the cache bit
    # for bit, the attention to tolerance
    for P in (0, 16):
        w = wl.Workload("odda", B=3, qLen=2, Hq=8, Hkv=2, D=D, kv_cap=300, dtype="fp16",
                        causal=True, sigma=1.0, seed=31 + P, len_range=(0, 300))
        inp = wl.make_inputs(w, lengths=[298, 0, 120])
        parity.run_append(inp, 2, P, seed=P)


@pytest.mark.parametrize("case", range(16))
def test_random_any_head_dims(case):
    """Random key and value head dims anywhere in 1 .. 256, ragged lengths,
    forced partitions and dtypes."""
    import split_kv_decode_amd as mx
    r = np.random.default_rng([20261204, case])
    B, qLen, G, Hkv = int(r.integers(1, 4)), int(r.choice([1, 2, 4, 8])), \
        int(r.choice([1, 2, 4, 8])), int(r.integers(1, 3))
    Dk = int(r.integers(1, 257))
    Dv = Dk if r.random() < 0.4 else int(r.integers(1, 257))
    dt = str(r.choice(["fp16", "bf16"]))
    causal = bool(r.integers(0, 2))
    cap = int(r.integers(1, 900))
    lens = [int(x) for x in r.integers(0, cap + 1, size=B)]
    num_splits = int(r.choice([0, 0, 1, 3, 9]))
    print(f"case {case}: B={B} qLen={qLen} G={G} Hkv={Hkv} Dk={Dk} Dv={Dv} {dt} causal={causal} "
          f"cap={cap} lens={lens} splits={num_splits}", flush=True)
    q, k, v, sl = wl.make_inputs_dkdv(B, qLen, G * Hkv, Hkv, Dk, Dv, cap, lens, dt, 1.0,
                                      20261204 + case)
    ws = None
    if num_splits:
        d = 1 if dt == "bf16" else 0
        need = mx.workspace_size_dkdv(B, G * Hkv, Hkv, Dk, Dv, qLen, cap, causal, d, num_splits)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out, lse = mx.fwd_kvcache_dkdv(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), causal,
                                   num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, sl, causal, dt)
    rep = parity.compare(parity.to_f64(out), lse.cpu().double().numpy(), ref_o, ref_l, dt)
    print(case, mx.last_plan().as_dict(), rep, flush=True)
