"""GPU path vs the fp64 oracle (needs an MI355X).

Small and medium shapes are compared element by element over every output
(the full-size long-KV workloads, every row, are in test_headline_gpu.py).  Every cache slot past a sequence's valid length is NaN (see
workloads.py), so any read of it would show up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
import pins
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import split_kv_decode_amd as mx
    mx.lib()
    oracle.build()


def _full_check(inp, num_splits=0, use_workspace=True, lse_rel=0.0):
    out, lse, plan = parity.run_gpu(inp, num_splits, use_workspace)
    ref_o, ref_l = parity.oracle_full(inp)
    rep = parity.compare(out, lse, ref_o, ref_l, inp.workload.dtype, lse_rel)
    print(inp.workload.name, plan, rep, flush=True)
    return out, lse, plan


# ------------------------------------------------------------ named workloads

def test_tiny_causal_full():
    inp = wl.make_inputs(wl.WORKLOADS["tiny_causal"])
    _full_check(inp)
    _full_check(inp, use_workspace=False)


@pytest.mark.parametrize("name", wl.SMALLQ_NAMES)
def test_smallq_mha_full(name):
    _full_check(wl.make_inputs(wl.WORKLOADS[name]))


@pytest.mark.parametrize("name", wl.LONG_KV_NAMES)
def test_long_kv_reduced_full(name):
    """Same structure at a size the oracle checks completely: several
    partitions, a ragged tail and (for the ragged workloads) varied lengths."""
    w = wl.WORKLOADS[name]
    cap = 2500 if w.len_range else 3000
    small = wl.scaled(w, B=min(w.B, 5), kv_cap=cap,
                      len_range=(cap // 4, cap) if w.len_range else None)
    _full_check(wl.make_inputs(small))


# ------------------------------------------------------------ partitioning

@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 64, 10 ** 6])
def test_forced_splits(num_splits):
    w = wl.Workload("splits", B=3, qLen=2, Hq=8, Hkv=2, D=128, kv_cap=777, dtype="bf16",
                    causal=True, sigma=1.0, seed=17, len_range=(1, 777))
    inp = wl.make_inputs(w, lengths=[777, 300, 1])
    out, lse, plan = _full_check(inp, num_splits=num_splits)
    assert 1 <= plan["num_splits"] <= min(num_splits, 777)


def test_splits_agree_with_each_other():
    """Different partition counts change only the fp32 summation order."""
    w = wl.Workload("agree", B=2, qLen=1, Hq=8, Hkv=2, D=128, kv_cap=4096, dtype="fp16",
                    causal=False, sigma=1.0, seed=23)
    inp = wl.make_inputs(w)
    outs = [parity.run_gpu(inp, s)[:2] for s in (1, 4, 16, 64)]
    for o, l in outs[1:]:
        assert np.abs(o - outs[0][0]).max() <= 2 * 2 ** -10 * np.abs(outs[0][0]).max()
        assert np.abs(l - outs[0][1]).max() <= 1e-5


def test_deterministic_run_to_run():
    inp = wl.make_inputs(wl.scaled(wl.WORKLOADS["qwen3_8b_decode"], B=8, kv_cap=4096,
                                   len_range=(1000, 4096)))
    o1, l1, _ = parity.run_gpu(inp)
    o2, l2, _ = parity.run_gpu(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------ shapes and edges

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("G,qLen,causal", [(1, 1, False), (2, 1, False), (4, 1, False),
                                          (8, 1, False), (1, 3, True), (3, 1, False),
                                          (5, 2, True), (4, 4, True), (8, 8, True),
                                          (16, 2, False), (16, 8, True)])
def test_shape_sweep(D, dtype, G, qLen, causal):
    Hkv = 2
    w = wl.Workload("sweep", B=2, qLen=qLen, Hq=G * Hkv, Hkv=Hkv, D=D, kv_cap=1100,
                    dtype=dtype, causal=causal, sigma=1.0, seed=1000 + G * 10 + qLen,
                    len_range=(1, 1100))
    inp = wl.make_inputs(w, lengths=[1100, 613])
    _full_check(inp)


@pytest.mark.parametrize("Hkv,num_splits", [(1, 0), (3, 0), (2, 0), (6, 0), (4, 3), (5, 2)])
def test_matrix_core_head_blocks(Hkv, num_splits):
    """The matrix-core kernel with one kv head per workgroup (odd Hkv) and two
    (even Hkv: two waves per head, merged per head), under the balanced and
    forced partitions, ragged lengths and a causal draft."""
    G = 8
    w = wl.Workload("heads", B=3, qLen=2, Hq=G * Hkv, Hkv=Hkv, D=128, kv_cap=900, dtype="bf16",
                    causal=True, sigma=1.0, seed=900 + Hkv, len_range=(1, 900))
    inp = wl.make_inputs(w, lengths=[900, 333, 2])
    _, _, plan = _full_check(inp, num_splits=num_splits)
    assert plan["path"] == "mfma" and plan["head_block"] == (2 if Hkv % 2 == 0 else 1)


@pytest.mark.parametrize("num_splits,rb", [(0, 16), (3, 64)])
def test_matrix_core_many_rows_keep_one_head_per_workgroup(num_splits, rb):
    """Several row blocks per kv head (a prefill chunk): one kv head per
    workgroup, whatever Hkv.  On this short cache the planner takes 16-row
    blocks (64-row ones would leave most CUs idle); forced partitions keep
    the 64-row tile."""
    w = wl.Workload("rows", B=2, qLen=20, Hq=16, Hkv=2, D=128, kv_cap=900, dtype="bf16",
                    causal=True, sigma=1.0, seed=950, len_range=(1, 900))
    inp = wl.make_inputs(w, lengths=[900, 25])
    _, _, plan = _full_check(inp, num_splits=num_splits)
    assert plan["path"] == "mfma" and plan["head_block"] == 1 and plan["rows"] == 160
    assert plan["row_block"] == rb, plan


@pytest.mark.parametrize("num_splits", [2, 0])
@pytest.mark.parametrize("Hkv,qLen", [(3, 8), (3, 5), (5, 6)])
def test_matrix_core_one_block_one_head(Hkv, qLen, num_splits):
    """One block per kv head (64 rows, or 48 for 40-48 rows) with an odd Hkv:
    one kv head per workgroup, K loaded straight into the operand layout,
    ragged lengths and a causal draft (forced partitions); with the
    planner's own partitions this short cache takes 16-row blocks instead."""
    R = 8 * qLen
    rb = 16 if num_splits == 0 else (48 if R <= 48 else 64)
    w = wl.Workload("onehead", B=3, qLen=qLen, Hq=8 * Hkv, Hkv=Hkv, D=128, kv_cap=800,
                    dtype="bf16", causal=True, sigma=1.0, seed=960 + Hkv + qLen,
                    len_range=(1, 800))
    inp = wl.make_inputs(w, lengths=[800, 217, 3])
    _, _, plan = _full_check(inp, num_splits=num_splits)
    assert plan["path"] == "mfma" and plan["head_block"] == 1 and plan["row_block"] == rb


@pytest.mark.parametrize("kvlen", [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1023, 1025])
def test_kv_length_sweep(kvlen):
    w = wl.Workload("lens", B=1, qLen=1, Hq=4, Hkv=1, D=128, kv_cap=kvlen, dtype="fp16",
                    causal=False, sigma=1.0, seed=kvlen)
    _full_check(wl.make_inputs(w))


def test_single_key_output_is_the_v_row_exactly():
    for dt in ("fp16", "bf16"):
        w = wl.Workload("one", B=3, qLen=1, Hq=8, Hkv=2, D=128, kv_cap=1, dtype=dt,
                        causal=False, sigma=1.0, seed=5)
        inp = wl.make_inputs(w)
        out, lse, _ = parity.run_gpu(inp)
        v = inp.v_cache.double().numpy()
        for h in range(8):
            assert np.array_equal(out[:, 0, h], v[:, 0, h // 4])


def test_empty_rows_and_zero_lengths():
    w = wl.Workload("empty", B=4, qLen=4, Hq=4, Hkv=2, D=64, kv_cap=50, dtype="bf16",
                    causal=True, sigma=1.0, seed=9, len_range=(0, 50))
    inp = wl.make_inputs(w, lengths=[0, 2, 50, 3])
    out, lse, _ = _full_check(inp)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isneginf(lse[1][:, :2]))           # rows 0,1 see nothing with n=2
    for ns in (1, 5):
        _full_check(inp, num_splits=ns)


@pytest.mark.parametrize("G,qLen,Hkv,D,cap,lengths", [
    (1, 6, 2, 64, 3, [0, 1, 3]),          # VALU path, one row block of 8
    (4, 4, 2, 64, 3, [0, 1, 3]),          # matrix-core path, 16-row blocks
    (8, 16, 1, 128, 5, [0, 2, 5]),        # matrix-core path, two row blocks of 64
])
def test_causal_draft_longer_than_the_cache(G, qLen, Hkv, D, cap, lengths):
    # rows whose causal bound lies before the first key see nothing; whole
    # row blocks can be empty while the sequence is not
    w = wl.Workload("draft", B=len(lengths), qLen=qLen, Hq=G * Hkv, Hkv=Hkv, D=D,
                    kv_cap=cap, dtype="bf16", causal=True, sigma=1.0, seed=77,
                    len_range=(0, cap))
    inp = wl.make_inputs(w, lengths=lengths)
    out, lse, _ = _full_check(inp)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    for ns in (1, 3):
        _full_check(inp, num_splits=ns)


def test_zero_capacity_cache():
    w = wl.Workload("cap0", B=2, qLen=1, Hq=2, Hkv=1, D=128, kv_cap=0, dtype="fp16",
                    causal=False, sigma=1.0, seed=1)
    inp = wl.make_inputs(w)
    out, lse, _ = parity.run_gpu(inp)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_out_of_range_seqlens_are_clamped():
    w = wl.Workload("clamp", B=3, qLen=1, Hq=4, Hkv=2, D=128, kv_cap=40, dtype="fp16",
                    causal=False, sigma=1.0, seed=3, len_range=(0, 40))
    inp = wl.make_inputs(w, lengths=[40, 40, 0])
    inp.cache_seqlens = torch.tensor([1000, 40, -7], dtype=torch.int32)
    out, lse, _ = parity.run_gpu(inp)
    ref_o, ref_l = parity.oracle_full(inp)
    parity.compare(out, lse, ref_o, ref_l, "fp16")


@pytest.mark.parametrize("qLen,Hq,Hkv,D,path,rb", [
    (1, 4, 4, 128, "valu", 1),      # one row per kv head
    (1, 8, 4, 128, "valu", 2),      # two rows
    (2, 4, 1, 128, "mfma", 16),     # the 16-row matrix-core tiles
    (4, 16, 1, 128, "mfma", 64),    # the 64-row tiles
    (1, 4, 1, 100, "mfma", 16),     # a head dim that is not a multiple of 8
])
@pytest.mark.parametrize("num_splits", [0, 3])
def test_fp16_large_scores_do_not_overflow(qLen, Hq, Hkv, D, path, rb, num_splits):
    """Scores far beyond the fp16 range (|s| ~ 1e4) must stay finite, on every
    kernel variant and through the merge of partitions."""
    g = torch.Generator().manual_seed(31 + D + Hq)
    w = wl.Workload("ovf", B=1, qLen=qLen, Hq=Hq, Hkv=Hkv, D=D, kv_cap=300, dtype="fp16",
                    causal=True, sigma=1.0, seed=31)
    inp = wl.make_inputs(w)
    inp.q = (torch.randn(1, qLen, Hq, D, generator=g) * 200).to(torch.float16)
    inp.k_cache = (torch.randn(1, 300, Hkv, D, generator=g) * 200).to(torch.float16)
    out, lse, plan = parity.run_gpu(inp, num_splits)
    # on this one-sequence cache the planner's own partitions take 16-row
    # blocks for the 64-row shape (64-row tiles would leave most CUs idle);
    # forced partitions keep the 64-row tile
    want = 16 if (rb == 64 and num_splits == 0) else rb
    assert (plan["path"], plan["row_block"]) == (path, want), plan
    ref_o, ref_l = parity.oracle_full(inp)
    assert np.abs(ref_l).max() > 1e4
    parity.compare(out, lse, ref_o, ref_l, "fp16", lse_rel=2 ** -22)


def test_identical_keys_give_the_mean_of_v():
    w = wl.Workload("ident", B=1, qLen=1, Hq=4, Hkv=1, D=128, kv_cap=3000, dtype="bf16",
                    causal=False, sigma=1.0, seed=41)
    inp = wl.make_inputs(w)
    inp.k_cache = inp.k_cache[:, :1].expand(1, 3000, 1, 128).contiguous()
    out, lse, _ = parity.run_gpu(inp)
    mean = inp.v_cache.double().numpy()[0, :, 0].mean(axis=0)
    assert np.abs(out[0, 0] - mean).max() <= 2 * parity.ulp(np.abs(mean).max(), "bf16")
    s = inp.q.double().numpy()[0, 0] @ inp.k_cache.double().numpy()[0, 0, 0] / math.sqrt(128)
    assert np.abs(lse[0, :, 0] - (s + math.log(3000))).max() <= 1e-3


def test_golden_examples_on_gpu():
    """The hand-worked D=4 examples, embedded in D=64: the extra channels are
    zero and q is multiplied by 4 (exact), so that q.k/sqrt(64) equals the
    original q.k/sqrt(4) and the expected outputs and lse are unchanged."""
    import split_kv_decode_amd as mx
    for ex in pins.load_golden():
        q, k, v, sl = pins.golden_inputs(ex)
        eo, el = pins.golden_expected(ex)
        pad = lambda t: torch.nn.functional.pad(t, (0, 64 - t.shape[-1]))
        q64, k64, v64 = pad(q * 4), pad(k), pad(v)
        assert torch.equal((q64[..., :4] / 4), q)
        dev = lambda t: t.contiguous().to("cuda")
        sld = None if sl is None else torch.from_numpy(sl).to("cuda")
        for ns in (0, 2):
            out, lse = mx.fwd_kvcache(dev(q64), dev(k64), dev(v64), sld, ex["causal"],
                                      num_splits=ns)
            torch.cuda.synchronize()
            o = parity.to_f64(out)
            assert np.all(o[..., 4:] == 0)
            parity.compare(o[..., :4], lse.cpu().double().numpy(), eo, el, ex["dtype"])


def test_workspace_errors_on_gpu():
    import split_kv_decode_amd as mx
    w = wl.Workload("ws", B=2, qLen=1, Hq=8, Hkv=2, D=128, kv_cap=4096, dtype="fp16",
                    causal=False, sigma=1.0, seed=2)
    g = wl.make_inputs(w).to("cuda")
    need = mx.workspace_size(2, 8, 2, 128, 1, 4096, False, 0, 8)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    out = torch.full_like(g.q, 7.0)
    with pytest.raises(mx.MxfaError) as e:
        mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, None, False, out=out, num_splits=8,
                       workspace=small)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())          # untouched on error


def test_prepared_call_reruns_with_new_contents():
    """A PreparedCall enqueues the same call again: after the query and the
    lengths change in place, its output equals a fresh call's, bit for bit,
    and the oracle's; the paged variant likewise."""
    import split_kv_decode_amd as mx
    w = wl.Workload("prep", B=2, qLen=2, Hq=16, Hkv=2, D=128, kv_cap=700, dtype="bf16",
                    causal=True, sigma=1.0, seed=61, len_range=(1, 700))
    inp = wl.make_inputs(w, lengths=[700, 300])
    g = inp.to("cuda")
    call = mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, g.cache_seqlens, True, prepare=True)
    o1, l1 = call.run()
    torch.cuda.synchronize()
    first = o1.clone()
    g.q.mul_(-1.0)
    g.cache_seqlens.copy_(torch.tensor([650, 123], dtype=torch.int32))
    o2, l2 = call.run()
    f_o, f_l = mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, g.cache_seqlens, True)
    torch.cuda.synchronize()
    assert o2.data_ptr() == o1.data_ptr() and not torch.equal(first, o2)
    assert torch.equal(o2, f_o) and torch.equal(l2, f_l)
    inp2 = wl.Inputs(w, g.q.cpu(), inp.k_cache, inp.v_cache,
                     torch.tensor([650, 123], dtype=torch.int32), None)
    ref_o, ref_l = parity.oracle_full(inp2)
    parity.compare(o2.float().cpu().double().numpy(), l2.cpu().double().numpy(),
                   ref_o, ref_l, "bf16", 0.0)
    pg = wl.to_paged(inp2, 64).to("cuda")
    pcall = mx.fwd_kvcache_paged(g.q, pg.k_pages, pg.v_pages, pg.block_table,
                                 pg.cache_seqlens, True, prepare=True)
    for _ in range(2):
        po, pl = pcall.run()
    fpo, fpl = mx.fwd_kvcache_paged(g.q, pg.k_pages, pg.v_pages, pg.block_table,
                                    pg.cache_seqlens, True)
    torch.cuda.synchronize()
    assert torch.equal(po, fpo) and torch.equal(pl, fpl)
    parity.compare(po.float().cpu().double().numpy(), pl.cpu().double().numpy(),
                   ref_o, ref_l, "bf16", 0.0)
