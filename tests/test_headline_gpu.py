"""The kernel variants that run the long-KV decode batches, compared with the
fp64 oracle over every output row (needs an MI355X).

The planner routes decode with 4 query rows per kv head at head dim 128 (GQA
4, one query token) to the vector-ALU kernel with 4 rows and 8 kv heads per
workgroup only when the caches (contiguous or paged) hold at least 256 MiB;
below that the matrix-core kernel's 16-row variant runs.  So these tests use caches of
at least that size, short ragged lengths (the route depends on capacity, not
on lengths, and the oracle then finishes in seconds), both dtypes, the
balanced schedule and forced partition counts, and assert the plan.  The
full-size batches are compared over every row in the launch configuration
the benchmark times.  A dominant-key closed form places the selected key
late in a long sequence, so that the matrix-core kernel's lazily moved
softmax reference must jump far after many tiles.
"""
import math

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


def _headline_shape(dtype, seed, outliers):
    # B=8 sequences of capacity 8192, 32 query / 8 kv heads of 128: the K and V
    # caches hold 8 * 8192 * 8 * 128 * 2 * 2 bytes = 256 MiB
    return wl.Workload("valu4x8", B=8, qLen=1, Hq=32, Hkv=8, D=128, kv_cap=8192, dtype=dtype,
                       causal=False, sigma=1.0, seed=seed, len_range=(0, 8192),
                       n_outlier=2 if outliers else 0, outlier_scale=8.0 if outliers else 1.0)


# ragged lengths with an empty sequence, a single key, the full capacity and
# lengths around tile and share boundaries
HEADLINE_LENGTHS = [0, 1, 8192, 777, 2, 4095, 31, 1500]


def _assert_headline_plan(plan, schedule):
    assert plan["path"] == "valu", plan
    assert plan["row_block"] == 4 and plan["head_block"] == 8 and plan["layout"] == 0, plan
    assert plan["schedule"] == schedule, plan


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 7, 64])
def test_valu_four_row_variant_every_row(dtype, num_splits):
    w = _headline_shape(dtype, 7100 + num_splits, outliers=dtype == "bf16")
    inp = wl.make_inputs(w, lengths=HEADLINE_LENGTHS)
    out, lse, plan = parity.run_gpu(inp, num_splits)
    _assert_headline_plan(plan, 1 if num_splits == 0 else 0)
    ref_o, ref_l = parity.oracle_full(inp)
    rep = parity.compare(out, lse, ref_o, ref_l, dtype)
    print(w.name, dtype, num_splits, plan, rep, flush=True)
    # the empty sequence: O = 0 and lse = -inf; one key: O = that V row exactly
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    v = inp.v_cache.double().numpy()
    for h in range(w.Hq):
        assert np.array_equal(out[1, 0, h], v[1, 0, h // w.G])


def test_valu_four_row_variant_library_scratch():
    """The same variant with the library's own stream-ordered scratch."""
    w = _headline_shape("bf16", 7200, outliers=True)
    inp = wl.make_inputs(w, lengths=[8192, 3, 0, 6000, 1, 2049, 4096, 100])
    out, lse, plan = parity.run_gpu(inp, use_workspace=False)
    _assert_headline_plan(plan, 1)
    ref_o, ref_l = parity.oracle_full(inp)
    print(parity.compare(out, lse, ref_o, ref_l, "bf16"), flush=True)


@pytest.mark.parametrize("P", [16, 64, 256])
def test_valu_four_row_variant_paged(P):
    """The same route through a paged cache (the page lookups run a step
    ahead of the loads), scattered into a random page order with poisoned
    spare pages and out-of-pool block-table entries past each sequence."""
    w = _headline_shape("bf16", 7400 + P, outliers=True)
    inp = wl.make_inputs(w, lengths=HEADLINE_LENGTHS)
    pg = wl.to_paged(inp, P)
    out, lse, plan = parity.run_gpu_paged(pg, inp)
    _assert_headline_plan(plan, 1)
    ref_o, ref_l = oracle.attention(inp.q, inp.k_cache, inp.v_cache, inp.cache_seqlens,
                                    w.causal, w.dtype)
    rep = parity.compare(out, lse, ref_o, ref_l, w.dtype)
    print(w.name, P, plan, rep, flush=True)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("rows", [1, 2])
@pytest.mark.parametrize("dtype,num_splits,paged", [("bf16", 0, False), ("fp16", 0, False),
                                                    ("bf16", 5, False), ("fp16", 0, True)])
def test_valu_whole_row_variants_every_row(rows, dtype, num_splits, paged):
    """One and two query rows per kv head on caches of 256 MiB and more run the
    VALU kernel with 8 kv heads per workgroup (whole 2 KiB token rows); below
    that size the planner takes 4.  16 kv heads, 8 x 8192 tokens: 512 MiB."""
    w = wl.Workload("valu_rows", B=8, qLen=1, Hq=16 * rows, Hkv=16, D=128, kv_cap=8192,
                    dtype=dtype, causal=False, sigma=1.0, seed=7500 + 10 * rows + num_splits,
                    len_range=(0, 8192))
    inp = wl.make_inputs(w, lengths=[3000, 0, 1, 8192, 17, 513, 64, 2])
    if paged:
        out, lse, plan = parity.run_gpu_paged(wl.to_paged(inp, 64), inp)
    else:
        out, lse, plan = parity.run_gpu(inp, num_splits)
    assert plan["path"] == "valu" and plan["head_block"] == 8 and plan["layout"] == 0, plan
    assert plan["row_block"] == rows, plan
    ref_o, ref_l = oracle.attention(inp.q, inp.k_cache, inp.v_cache, inp.cache_seqlens,
                                    w.causal, w.dtype)
    rep = parity.compare(out, lse, ref_o, ref_l, dtype)
    print(w.name, rows, dtype, num_splits, paged, plan, rep, flush=True)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("name", wl.LONG_KV_NAMES)
def test_long_kv_full_size_every_row(name):
    """The full-size batch in the benchmark's launch configuration (planner's
    choice, caller workspace), every output row against the oracle."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    out, lse, plan = parity.run_gpu(inp)
    if name != "llama70b_mtp_decode":
        _assert_headline_plan(plan, 1)
    else:
        assert plan["path"] == "mfma" and plan["row_block"] == 64, plan
    ref_o, ref_l = parity.oracle_full(inp)
    rep = parity.compare(out, lse, ref_o, ref_l, w.dtype)
    print(name, plan, rep, flush=True)


@pytest.mark.parametrize("name,P", [("qwen3_8b_decode", 16), ("llama70b_mtp_decode", 64),
                                    ("qwen3_4b_long_decode", 256)])
def test_paged_full_size_every_row(name, P):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    pg = wl.to_paged(inp, P)
    out, lse, plan = parity.run_gpu_paged(pg, inp)
    if name != "llama70b_mtp_decode":
        _assert_headline_plan(plan, 1)
    ref_o, ref_l = oracle.attention(inp.q, inp.k_cache, inp.v_cache, inp.cache_seqlens,
                                    w.causal, w.dtype)
    rep = parity.compare(out, lse, ref_o, ref_l, w.dtype)
    print(name, P, plan, rep, flush=True)


# ------------------------------------------------------------ dominant key

def _dominant_inputs(w, lengths, jstar):
    """q has only channel 0 set (16 in every row); every K row has channel 0
    equal to 0 except key jstar[b] of sequence b, whose channel 0 is 32.  The
    score of every other key is exactly 0 and that of the selected key is
    16 * 32 / sqrt(D) (45.3 at D = 128, a margin of e^-45)."""
    inp = wl.make_inputs(w, lengths=lengths)
    q = torch.zeros_like(inp.q)
    q[..., 0] = 16.0
    k = inp.k_cache.clone()
    for b, n in enumerate(lengths):
        k[b, :n, :, 0] = 0.0
        if jstar[b] is not None:
            k[b, jstar[b], :, 0] = 32.0
    inp.q, inp.k_cache = q, k
    return inp


def _check_dominant(inp, lengths, jstar, num_splits=0):
    w = inp.workload
    out, lse, plan = parity.run_gpu(inp, num_splits)
    v = inp.v_cache.double().numpy()
    s_star = 16.0 * 32.0 / math.sqrt(w.D)
    for b, n in enumerate(lengths):
        for i in range(w.qLen):
            last = min(n - 1, i + n - w.qLen) if w.causal else n - 1
            for h in range(w.Hq):
                hk = h // w.G
                if last < 0:
                    assert np.all(out[b, i, h] == 0) and np.isneginf(lse[b, h, i])
                elif jstar[b] is not None and jstar[b] <= last:
                    # the selected key: O is its V row, bit for bit, and
                    # lse = s* + ln(1 + (count - 1) e^-s*) = s* to far below 1e-3
                    assert np.array_equal(out[b, i, h], v[b, jstar[b], hk]), (b, i, h)
                    assert abs(lse[b, h, i] - s_star) <= 1e-3
                else:
                    # all visible scores 0: O = mean of the visible V rows,
                    # lse = ln(count)
                    mean = v[b, :last + 1, hk].mean(axis=0)
                    gate = 2 * parity.ulp(np.abs(mean).max(), w.dtype)
                    assert np.abs(out[b, i, h] - mean).max() <= gate, (b, i, h)
                    assert abs(lse[b, h, i] - math.log(last + 1)) <= 1e-3
    return plan


@pytest.mark.parametrize("num_splits", [0, 5])
@pytest.mark.parametrize("kind", ["valu4x8", "valu2", "mfma64", "mfma16"])
def test_dominant_key_arrives_late(kind, num_splits):
    # late in the longest sequences (after ~190 tiles of 32 keys), near the
    # end of a ragged one, at the very first key, and none at all
    jstar = [8189, 6000 - 3, 0, None]
    if kind == "valu4x8":
        # the 256 MiB cache that routes to the 4-row vector-ALU variant
        w = _headline_shape("bf16", 7300, outliers=False)
        lengths = [8192, 6000, 4097, 1, 0, 300, 8192, 2]
        jstar = jstar + [None, 150, None, 1]
        plan_want = ("valu", 4)
    elif kind == "valu2":
        w = wl.Workload("dom", B=4, qLen=1, Hq=4, Hkv=2, D=128, kv_cap=8192, dtype="fp16",
                        causal=False, sigma=1.0, seed=7301, len_range=(0, 8192))
        lengths = [8192, 6000, 4097, 1]
        plan_want = ("valu", 2)
    elif kind == "mfma64":
        w = wl.Workload("dom", B=4, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=8192, dtype="bf16",
                        causal=True, sigma=0.5, seed=7302, len_range=(0, 8192))
        lengths = [8192, 6000, 4097, 5]
        plan_want = ("mfma", 64)
    else:
        w = wl.Workload("dom", B=4, qLen=1, Hq=64, Hkv=8, D=128, kv_cap=8192, dtype="fp16",
                        causal=False, sigma=1.0, seed=7303, len_range=(0, 8192))
        lengths = [8192, 6000, 4097, 1]
        plan_want = ("mfma", 16)
    inp = _dominant_inputs(w, lengths, jstar)
    plan = _check_dominant(inp, lengths, jstar, num_splits)
    assert (plan["path"], plan["row_block"]) == plan_want, plan
    print(kind, num_splits, plan, flush=True)
