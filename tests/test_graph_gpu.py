"""Attention calls captured in a HIP graph and replayed (needs an MI355X).

The caller-workspace and allocation-free entry points enqueue kernels only
(no allocation, no memset), so a decode loop can capture one call and replay
it with new contents in the same tensors.  Each replay is compared with an
eager call on the same inputs (bit for bit) and with the fp64 oracle, with
the program's own eager work and synchronisations between the replays.
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


CASES = [
    # the 4-row vector-ALU variant on a 256 MiB cache, balanced schedule
    ("valu", wl.Workload("gv", B=8, qLen=1, Hq=32, Hkv=8, D=128, kv_cap=8192, dtype="bf16",
                         causal=False, sigma=1.0, seed=901, len_range=(0, 8192))),
    # a causal draft on the 64-row matrix-core kernel with its merge kernel
    ("mfma64", wl.Workload("gm", B=16, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=1100, dtype="bf16",
                           causal=True, sigma=0.5, seed=902, len_range=(0, 1100))),
    # the same draft on a short cache for three sequences: 16-row blocks
    ("mfma16rows", wl.Workload("gr", B=3, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=3000,
                               dtype="bf16", causal=True, sigma=0.5, seed=904,
                               len_range=(0, 3000))),
    # 4- and 6-token drafts on GQA 8: 32- and 48-row blocks
    ("mfma32", wl.Workload("g32", B=16, qLen=4, Hq=64, Hkv=8, D=128, kv_cap=2048, dtype="bf16",
                           causal=True, sigma=0.5, seed=905, len_range=(0, 2048))),
    ("mfma48", wl.Workload("g48", B=16, qLen=6, Hq=64, Hkv=8, D=128, kv_cap=2048, dtype="fp16",
                           causal=True, sigma=0.5, seed=906, len_range=(0, 2048))),
    # the 16-row matrix-core variant, fp16
    ("mfma16", wl.Workload("gs", B=2, qLen=1, Hq=64, Hkv=8, D=128, kv_cap=2000, dtype="fp16",
                           causal=False, sigma=1.0, seed=903, len_range=(0, 2000))),
]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("kind,w", CASES, ids=[c[0] for c in CASES])
def test_captured_call_replays(kind, w, noalloc):
    import split_kv_decode_amd as mx
    g = torch.Generator().manual_seed(w.seed + 7)
    lengths = [int(x) for x in torch.randint(1, w.kv_cap + 1, (w.B,), generator=g)]
    inp = wl.make_inputs(w, lengths=lengths)
    dev = inp.to("cuda")
    q, k, v, sl = dev.q, dev.k_cache, dev.v_cache, dev.cache_seqlens
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.qLen), dtype=torch.float32, device="cuda")
    dt = 1 if w.dtype == "bf16" else 0
    ws = None
    if not noalloc:
        need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt, 0)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")

    def call():
        if noalloc:
            return mx.fwd_kvcache(q, k, v, sl, w.causal, out=out, lse=lse, noalloc=True)
        return mx.fwd_kvcache(q, k, v, sl, w.causal, out=out, lse=lse, workspace=ws)

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    plan = mx.last_plan().as_dict()
    assert plan["schedule"] == 1, plan
    want_rb = {"valu": 4, "mfma64": 64, "mfma16rows": 16, "mfma32": 32, "mfma48": 48,
               "mfma16": 16}[kind]
    assert plan["row_block"] == want_rb, plan
    for rep in range(4):
        # new queries and lengths in the captured tensors (eager work between replays)
        g2 = torch.Generator().manual_seed(w.seed + 100 + rep)
        new_q = (torch.randn(q.shape, generator=g2) * w.sigma).to(w.torch_dtype)
        new_len = [int(x) for x in torch.randint(0, w.kv_cap + 1, (w.B,), generator=g2)]
        new_len = [min(n, lengths[b]) for b, n in enumerate(new_len)]    # rows past are NaN
        q.copy_(new_q.cuda())
        sl.copy_(torch.tensor(new_len, dtype=torch.int32).cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_out, ref_lse = mx.fwd_kvcache(q, k, v, sl, w.causal, workspace=torch.empty(
            max(plan["workspace_bytes"], 256), dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_out) and torch.equal(got_l, ref_lse), rep
        inp_r = wl.Inputs(w, new_q, inp.k_cache, inp.v_cache,
                          torch.tensor(new_len, dtype=torch.int32), None)
        ro, rl = parity.oracle_full(inp_r)
        rep_ = parity.compare(parity.to_f64(got_o), got_l.cpu().double().numpy(), ro, rl,
                              w.dtype)
        print(kind, noalloc, rep, plan["path"], rep_, flush=True)

