"""Batches without per-sequence lengths (cache_seqlens NULL: every sequence
holds kv_cap keys) under the balanced schedule (needs an MI355X).  The
planner then gives every stream shares of its own when shares of the
concatenated layout's width fit the grid stream by stream, else keeps the
streams concatenated.  The shapes below were chosen, from the plans the
planner makes for them, so that every case occurs: several shares per
stream with a shorter last share (both kernels, the 64-row tile, a padded
head dim), exactly one share per stream (each workgroup writes its final
output), and the concatenated layout with shares that straddle streams.
Every row is compared with the fp64 oracle."""
import pytest
import torch

import parity
import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [
    # (name, B, qLen, Hq, Hkv, D, kv_cap, dtype, causal) -> layout the planner picks
    ("aligned_valu_mha_q1", 1, 1, 32, 32, 128, 1023, "bf16", False),      # 32 shares/stream
    ("aligned_mfma16_gqa4_q2", 3, 2, 16, 4, 128, 777, "fp16", True),     # 13 shares/stream
    ("aligned_mfma16_mtp8", 2, 8, 64, 8, 128, 5000, "bf16", True),       # 16-row blocks, 8 shares/stream
    ("aligned_mfma64_mtp8", 16, 8, 64, 8, 128, 1100, "bf16", True),      # 64-row tiles, 3 shares/stream
    ("aligned_mfma16_mha_q8_d64", 1, 8, 16, 16, 64, 3000, "fp16", True), # 47 shares/stream
    ("aligned_d96", 7, 3, 12, 4, 96, 1337, "bf16", True),                # 14 shares/stream
    ("one_share_per_stream", 256, 1, 8, 8, 64, 1000, "fp16", False),     # 256 streams, 256 shares
    ("concatenated_b200", 200, 1, 8, 8, 64, 700, "bf16", False),         # 200 streams on 256
    ("concatenated_gqa2_q4", 5, 4, 16, 8, 128, 2500, "fp16", True),      # 20 streams on 512
    ("concatenated_b48", 48, 1, 32, 8, 128, 3000, "bf16", False),        # 48 streams on 256
]


def _workload(case):
    name, B, qLen, Hq, Hkv, D, cap, dtype, causal = case
    return wl.Workload(name, B=B, qLen=qLen, Hq=Hq, Hkv=Hkv, D=D, kv_cap=cap, dtype=dtype,
                       causal=causal, sigma=1.0, seed=61)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_equal_lengths_balanced(case):
    w = _workload(case)
    inp = wl.make_inputs(w)
    assert inp.cache_seqlens is None
    print(f"case {w.name}", flush=True)
    out, lse, plan = parity.run_gpu(inp)
    assert plan["schedule"] == 1, plan            # balanced
    ro, rl = parity.oracle_full(inp)
    print(w.name, plan, parity.compare(out, lse, ro, rl, w.dtype), flush=True)


PAGED = [
    # kv_cap a multiple of the page: without lengths every page row is a key
    ("aligned_paged16_gqa4_q2", 3, 2, 16, 4, 128, 784, "fp16", True, 16),
    ("aligned_paged64_mtp8", 2, 8, 64, 8, 128, 4992, "bf16", True, 64),
    ("concatenated_paged32_b48", 48, 1, 32, 8, 128, 2976, "bf16", False, 32),
]


@pytest.mark.parametrize("case", PAGED, ids=[c[0] for c in PAGED])
def test_equal_lengths_balanced_paged(case):
    import split_kv_decode_amd as mx
    *shape, page = case
    w = _workload(tuple(shape))
    inp = wl.make_inputs(w)
    paged = wl.to_paged(inp, page, seed=5)
    g = inp.to("cuda")
    pg = paged.to("cuda")
    print(f"case {w.name}", flush=True)
    out, lse = mx.fwd_kvcache_paged(g.q, pg.k_pages, pg.v_pages, pg.block_table, None, w.causal)
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()
    assert plan["schedule"] == 1, plan
    ro, rl = parity.oracle_paged(paged, inp)
    print(w.name, plan, parity.compare(parity.to_f64(out), lse.cpu().double().numpy(), ro, rl,
                                       w.dtype), flush=True)
