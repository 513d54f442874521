"""The allocation-free entry point (mxfa_fwd_kvcache_noalloc) on the GPU: its
output equals that of the caller-workspace entry point (mxfa_fwd_kvcache_ws)
bit for bit and the fp64 oracle's within the parity tolerances, on two calls
in a row whose second problem is smaller (the shared scratch keeps the first
call's contents), on both split kernels; a problem whose plan needs more
scratch than the fixed array holds is rejected before anything runs."""
import ctypes

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


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call_noalloc(g, w, out, lse, num_splits):
    import split_kv_decode_amd as mx
    dt = 1 if w.dtype == "bf16" else 0
    stream = torch.cuda.current_stream().cuda_stream
    return mx.lib().mxfa_fwd_kvcache_noalloc(
        _p(g.q), _p(g.k_cache), _p(g.v_cache), _p(g.cache_seqlens), _p(out), _p(lse), w.B, w.Hq,
        w.Hkv, w.D, w.qLen, w.kv_cap, int(w.causal), dt, num_splits, ctypes.c_void_p(stream))


def _check(w, lengths, num_splits, path):
    import split_kv_decode_amd as mx
    inp = wl.make_inputs(w, lengths=lengths)
    g = inp.to("cuda")
    out = torch.full_like(g.q, 3.0)
    lse = torch.full((w.B, w.Hq, w.qLen), 3.0, dtype=torch.float32, device="cuda")
    st = _call_noalloc(g, w, out, lse, num_splits)
    assert st == mx.MXFA_OK, mx.status_string(st)
    plan = mx.last_plan().as_dict()
    assert plan["path"] == path and plan["combine"] == 1, plan
    assert plan["workspace_bytes"] <= mx.NOALLOC_SCRATCH_BYTES
    ref_out, ref_lse = mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, g.cache_seqlens, w.causal,
                                      num_splits=num_splits,
                                      workspace=torch.empty(max(plan["workspace_bytes"], 256),
                                                            dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    ro, rl = parity.oracle_full(inp)
    rep = parity.compare(parity.to_f64(out), lse.cpu().double().numpy(), ro, rl, w.dtype)
    print(w.name, num_splits, plan, rep, flush=True)


def test_two_calls_in_a_row_second_smaller():
    # first: a 4-row GQA decode batch on a 256 MiB cache (vector-ALU kernel,
    # balanced schedule), then a small causal draft batch (matrix-core kernel)
    big = wl.Workload("na1", B=8, qLen=1, Hq=32, Hkv=8, D=128, kv_cap=8192, dtype="bf16",
                      causal=False, sigma=1.0, seed=811, len_range=(0, 8192))
    _check(big, [8192, 1, 0, 5000, 300, 8000, 2, 4097], 0, "valu")
    small = wl.Workload("na2", B=3, qLen=4, Hq=16, Hkv=2, D=128, kv_cap=900, dtype="fp16",
                        causal=True, sigma=1.0, seed=812, len_range=(0, 900))
    _check(small, [900, 17, 0], 0, "mfma")
    # and once more with forced partitions (fixed schedule), smaller again
    tiny = wl.Workload("na3", B=2, qLen=2, Hq=8, Hkv=2, D=64, kv_cap=300, dtype="bf16",
                       causal=True, sigma=1.0, seed=813, len_range=(0, 300))
    _check(tiny, [300, 5], 7, "mfma")


def test_problem_beyond_the_scratch_is_rejected():
    import split_kv_decode_amd as mx
    # forced 64 partitions of a 64-sequence draft batch: about 1 GiB of partials
    w = wl.Workload("na4", B=64, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=2048, dtype="bf16",
                    causal=True, sigma=0.5, seed=814)
    need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, 1, 64)
    assert need > mx.NOALLOC_SCRATCH_BYTES
    g = wl.Inputs(w, torch.zeros(w.B, w.qLen, w.Hq, w.D, dtype=torch.bfloat16),
                  torch.zeros(w.B, w.kv_cap, w.Hkv, w.D, dtype=torch.bfloat16),
                  torch.zeros(w.B, w.kv_cap, w.Hkv, w.D, dtype=torch.bfloat16), None,
                  None).to("cuda")
    out = torch.full_like(g.q, 3.0)
    lse = torch.full((w.B, w.Hq, w.qLen), 3.0, dtype=torch.float32, device="cuda")
    assert _call_noalloc(g, w, out, lse, 64) == mx.MXFA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((lse == 3.0).all())      # untouched
