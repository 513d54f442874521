"""Paged KV cache on the GPU vs the fp64 oracle (needs an MI355X).

The cache is scattered into a pool of pages in a seeded random order
(workloads.to_paged): pool rows that hold no valid token and block-table
entries past a sequence's last block are poisoned (NaN rows, out-of-pool
page numbers), so a read of either shows up as a non-finite output or a
fault-free mismatch.  Every shape is compared element by element (the
full-size paged workloads are in test_headline_gpu.py).
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


def _check(inp, P, num_splits=0, use_workspace=True, seed=0):
    pg = wl.to_paged(inp, P, seed=seed)
    out, lse, plan = parity.run_gpu_paged(pg, inp, num_splits, use_workspace)
    ref_o, ref_l = parity.oracle_paged(pg, inp)
    rep = parity.compare(out, lse, ref_o, ref_l, inp.workload.dtype)
    print(inp.workload.name, P, plan, rep, flush=True)
    return out, lse, plan


# (name, B, qLen, Hq, Hkv, D, kv_cap, dtype, causal): every kernel layout
SHAPES = [
    ("valu_heads", 3, 1, 16, 8, 128, 1100, "bf16", False),     # all-heads slots
    ("valu_tokens128", 3, 2, 2, 2, 128, 1100, "fp16", True),    # one head per workgroup
    ("mfma_small128", 3, 1, 32, 8, 128, 1100, "bf16", False),  # 4 rows: 16-row tiles
    ("valu_tokens64_r1", 2, 1, 2, 2, 64, 1100, "bf16", False),  # the capped load step
    ("valu_tokens64_r8", 2, 3, 4, 2, 64, 900, "fp16", True),
    ("mfma128", 2, 8, 16, 2, 128, 1100, "bf16", True),
    ("mfma64", 2, 2, 16, 1, 64, 1000, "fp16", False),
    # several row blocks per kv head: K loaded straight into operand layout
    ("mfma_rowblocks128", 2, 12, 16, 2, 128, 1000, "bf16", True),
    ("mfma_rowblocks64", 2, 20, 8, 2, 64, 900, "fp16", False),
    ("mfma_rowblocks256", 2, 4, 16, 2, 256, 700, "bf16", True),
    ("mfma128_oddkv", 2, 8, 24, 3, 128, 900, "bf16", True),    # 64 rows, one head per workgroup
]


@pytest.mark.parametrize("P", [16, 64, 256])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s[0])
def test_paged_shapes(shape, P):
    name, B, qLen, Hq, Hkv, D, cap, dt, causal = shape
    w = wl.Workload(name, B=B, qLen=qLen, Hq=Hq, Hkv=Hkv, D=D, kv_cap=cap, dtype=dt,
                    causal=causal, sigma=1.0, seed=len(name) * 31 + P, len_range=(1, cap))
    lens = [cap, cap // 2 + 7, 1] if B > 2 else [cap, min(cap, 13 * P + 5)]
    inp = wl.make_inputs(w, lengths=lens)
    _, _, plan = _check(inp, P)
    if plan["path"] == "mfma" and plan["rows"] > 16 and plan["row_block"] == 16 and D <= 128:
        # the planner took 16-row blocks for this short cache: the 32-, 48-
        # or 64-row tile of the same shape, through forced partitions
        _, _, plan = _check(inp, P, num_splits=2)
        assert plan["row_block"] == (32 if plan["rows"] <= 32 else 48 if plan["rows"] <= 48 else 64), plan


@pytest.mark.parametrize("num_splits", [1, 3, 7])
@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_paged_forced_splits(path, num_splits):
    if path == "valu":
        w = wl.Workload("ps", B=3, qLen=2, Hq=2, Hkv=2, D=128, kv_cap=777, dtype="bf16",
                        causal=True, sigma=1.0, seed=17, len_range=(1, 777))
    else:
        w = wl.Workload("ps", B=3, qLen=4, Hq=16, Hkv=2, D=128, kv_cap=777, dtype="bf16",
                        causal=True, sigma=1.0, seed=18, len_range=(1, 777))
    inp = wl.make_inputs(w, lengths=[777, 300, 1])
    _, _, plan = _check(inp, 16, num_splits=num_splits)
    assert plan["schedule"] == 0 and plan["path"] == path


@pytest.mark.parametrize("num_splits", [40, 64, 100, 777])
@pytest.mark.parametrize("kind", ["mfma64rows", "mfma16rows", "valu"])
def test_paged_partitions_shorter_than_a_tile(kind, num_splits):
    """Forced partitions of 1-20 keys.  The matrix-core kernel reads a paged
    cache in 32-key tiles and its segments start on tile boundaries: most of
    these partitions round to nothing and write empty partials, the others
    to whole tiles; the merge must count both.  The VALU kernel keeps its own
    bounds (masked to the key)."""
    if kind == "mfma64rows":
        w = wl.Workload("tiny_parts", B=3, qLen=8, Hq=16, Hkv=2, D=128, kv_cap=777,
                        dtype="bf16", causal=True, sigma=1.0, seed=61, len_range=(1, 777))
    elif kind == "mfma16rows":
        w = wl.Workload("tiny_parts", B=3, qLen=1, Hq=32, Hkv=4, D=64, kv_cap=777,
                        dtype="fp16", causal=False, sigma=1.0, seed=62, len_range=(1, 777))
    else:
        w = wl.Workload("tiny_parts", B=3, qLen=1, Hq=8, Hkv=8, D=128, kv_cap=777,
                        dtype="bf16", causal=False, sigma=1.0, seed=63, len_range=(1, 777))
    inp = wl.make_inputs(w, lengths=[777, 45, 1])
    _, _, plan = _check(inp, 16, num_splits=num_splits)
    assert plan["schedule"] == 0 and plan["path"] == ("valu" if kind == "valu" else "mfma")


@pytest.mark.parametrize("P", [16, 32, 64])
def test_paged_balanced_shares_start_inside_tiles(P):
    """Balanced shares of 64 keys laid over sequences whose lengths are not
    multiples of 32, so share bounds fall inside tiles and are rounded (one
    16-row tile per kv head: the matrix-core kernel's small variant)."""
    w = wl.Workload("odd_shares", B=7, qLen=2, Hq=16, Hkv=2, D=128, kv_cap=1000, dtype="bf16",
                    causal=True, sigma=1.0, seed=64 + P, len_range=(1, 1000))
    inp = wl.make_inputs(w, lengths=[1000, 33, 999, 31, 65, 517, 2])
    _, _, plan = _check(inp, P)
    assert plan["schedule"] == 1 and plan["path"] == "mfma", plan


def test_paged_library_scratch_and_whole_pages():
    # lengths at, just below and just above page boundaries; no caller workspace
    w = wl.Workload("edges", B=5, qLen=1, Hq=16, Hkv=4, D=128, kv_cap=512, dtype="fp16",
                    causal=False, sigma=1.0, seed=41, len_range=(0, 512))
    inp = wl.make_inputs(w, lengths=[512, 64, 63, 65, 0])
    out, lse, _ = _check(inp, 64, use_workspace=False)
    assert np.all(out[4] == 0) and np.all(np.isneginf(lse[4]))


def test_paged_without_lengths_uses_every_page():
    # cache_seqlens NULL: every sequence holds max_pages * page_size tokens
    import split_kv_decode_amd as mx
    w = wl.Workload("full", B=2, qLen=2, Hq=8, Hkv=2, D=64, kv_cap=256, dtype="bf16",
                    causal=True, sigma=1.0, seed=43)
    inp = wl.make_inputs(w)
    pg = wl.to_paged(inp, 32).to("cuda")
    out, lse = mx.fwd_kvcache_paged(inp.q.cuda(), pg.k_pages, pg.v_pages, pg.block_table,
                                    None, True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(inp.q, inp.k_cache, inp.v_cache, None, True)
    parity.compare(parity.to_f64(out), lse.cpu().double().numpy(), ref_o, ref_l, "bf16")


def test_shared_prefix_pages():
    # sequences 1 and 2 reuse sequence 0's first two pages (a shared prompt)
    import split_kv_decode_amd as mx
    w = wl.Workload("shared", B=3, qLen=1, Hq=8, Hkv=2, D=128, kv_cap=160, dtype="bf16",
                    causal=False, sigma=1.0, seed=47, len_range=(1, 160))
    inp = wl.make_inputs(w, lengths=[160, 100, 40])
    pg = wl.to_paged(inp, 32)
    bt = pg.block_table.clone()
    bt[1, :2] = bt[0, :2]
    bt[2, :2] = bt[0, :2]
    pg.block_table = bt
    out, lse, _ = parity.run_gpu_paged(pg, inp)
    ref_o, ref_l = parity.oracle_paged(pg, inp)
    parity.compare(out, lse, ref_o, ref_l, "bf16")


def test_paged_agrees_with_the_contiguous_path():
    w = wl.scaled(wl.WORKLOADS["qwen3_8b_decode"], B=6, kv_cap=4096, len_range=(100, 4096))
    inp = wl.make_inputs(w)
    o1, l1, _ = parity.run_gpu(inp)
    o2, l2, _ = parity.run_gpu_paged(wl.to_paged(inp, 256), inp)
    assert np.abs(o1 - o2).max() <= 2 * 2 ** -8 * np.abs(o1).max()
    assert np.abs(l1 - l2).max() <= 1e-5
