"""Head-group and batch shapes at the edges of the planner (needs an MI355X).

Grouped-query groups larger than 8 (multi-query attention with one kv head
and 64 or 128 query heads; 16, 24 or 32 query heads per kv head), where a kv
head carries up to 512 query rows, split into several 64-row blocks with a
ragged last block, or fit one 16-row tile; and batches on both sides of the
1024-sequence limit of the balanced schedule (more sequences take fixed
partitions); and the 32- and 48-row tiles (two or three 16-row tiles per
wave) that 17 to 48 rows per kv head take.  Every row is compared with the fp64 oracle.
"""
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


GROUPS = [
    # (name, B, qLen, Hq, Hkv, D, kv_cap, dtype, causal)
    ("mqa64_q1", 3, 1, 64, 1, 128, 2000, "bf16", False),       # 64 rows: one 64-row block
    ("mqa128_q2", 2, 2, 128, 1, 128, 1500, "fp16", True),      # 256 rows: 4 blocks
    ("mqa32_q8_d64", 2, 8, 32, 1, 64, 1200, "bf16", True),     # 256 rows at head dim 64
    ("g16_q1", 4, 1, 32, 2, 128, 1800, "fp16", False),         # 16 rows: one 16-row tile
    ("g24_q3", 2, 3, 96, 4, 128, 900, "bf16", True),           # 72 rows: a ragged second block
    ("g32_q4_d96", 2, 4, 64, 2, 96, 700, "fp16", True),        # 128 rows, padded head dim
    ("mqa128_q4", 1, 4, 128, 1, 128, 3000, "bf16", True),      # 512 rows: 8 blocks
]


@pytest.mark.parametrize("forced", [0, 4], ids=["planned", "forced4"])
@pytest.mark.parametrize("case", GROUPS, ids=[c[0] for c in GROUPS])
def test_large_query_head_groups(case, forced):
    name, B, qLen, Hq, Hkv, D, cap, dtype, causal = case
    w = wl.Workload(name, B=B, qLen=qLen, Hq=Hq, Hkv=Hkv, D=D, kv_cap=cap, dtype=dtype,
                    causal=causal, sigma=1.0, seed=Hq + qLen + D, len_range=(0, cap))
    lengths = [cap] + [int(x) for x in torch.randint(0, cap + 1, (B - 1,),
                                                      generator=torch.Generator().manual_seed(B))]
    inp = wl.make_inputs(w, lengths=lengths)
    print(f"case {name} forced={forced} lengths={lengths}", flush=True)
    out, lse, plan = parity.run_gpu(inp, num_splits=forced)
    assert plan["path"] == "mfma" and plan["rows"] == Hq // Hkv * qLen, plan
    ref_o, ref_l = parity.oracle_full(inp)
    print(name, forced, plan, parity.compare(out, lse, ref_o, ref_l, dtype), flush=True)


@pytest.mark.parametrize("B,schedule", [(1024, 1), (1025, 0), (1500, 0)])
@pytest.mark.parametrize("qLen,Hq,Hkv,cap", [(1, 8, 8, 96), (4, 8, 2, 600)],
                         ids=["valu", "mfma"])
def test_batches_around_the_balanced_limit(B, schedule, qLen, Hq, Hkv, cap):
    w = wl.Workload(f"b{B}", B=B, qLen=qLen, Hq=Hq, Hkv=Hkv, D=64, kv_cap=cap, dtype="bf16",
                    causal=True, sigma=1.0, seed=B + qLen, len_range=(0, cap))
    inp = wl.make_inputs(w)
    print(f"case B={B} qLen={qLen} Hq={Hq} Hkv={Hkv}", flush=True)
    out, lse, plan = parity.run_gpu(inp)
    assert plan["schedule"] == schedule, plan
    ref_o, ref_l = parity.oracle_full(inp)
    print(B, plan, parity.compare(out, lse, ref_o, ref_l, "bf16"), flush=True)


MID_PLANNED = [
    # 17-48 rows per kv head on batches that keep every CU busy: the planner's
    # balanced schedule on two or three 16-row tiles per wave
    ("gqa8_q4", 16, 4, 64, 8, 128, 2048, "bf16", True),          # 32 rows
    ("gqa16_q2", 4, 2, 128, 8, 128, 3000, "fp16", True),         # 32 rows
    ("gqa8_q6", 16, 6, 64, 8, 128, 2048, "bf16", True),          # 48 rows
    ("gqa16_q3", 8, 3, 128, 8, 128, 2500, "fp16", True),         # 48 rows
]
MID_FORCED = [
    # small caches (the planner would take 16-row blocks): forced partitions
    ("gqa8_q3_even_kv", 3, 3, 48, 6, 128, 500, "fp16", True),     # 24 rows, two heads per workgroup
    ("gqa8_q4_odd_kv_d64", 2, 4, 24, 3, 64, 900, "bf16", True),   # 32 rows, one head, head dim 64
    ("mha_q17", 1, 17, 8, 8, 128, 300, "fp16", False),             # 17 rows
    ("gqa8_q5_even_kv", 3, 5, 48, 6, 128, 500, "bf16", True),     # 40 rows in a 48-row block
    ("gqa8_q6_odd_kv_d64", 2, 6, 24, 3, 64, 900, "fp16", True),   # 48 rows, one head, head dim 64
    ("mha_q33", 1, 33, 8, 8, 128, 300, "bf16", False),             # 33 rows
]


def _mid_workload(case):
    name, B, qLen, Hq, Hkv, D, cap, dtype, causal = case
    return wl.Workload(name, B=B, qLen=qLen, Hq=Hq, Hkv=Hkv, D=D, kv_cap=cap, dtype=dtype,
                       causal=causal, sigma=1.0, seed=B + qLen + D, len_range=(0, cap))


def _mid_rows(w):
    R = w.Hq // w.Hkv * w.qLen
    return -(-R // 16) * 16


@pytest.mark.parametrize("case", MID_PLANNED, ids=[c[0] for c in MID_PLANNED])
def test_mid_row_tiles_planned(case):
    w = _mid_workload(case)
    inp = wl.make_inputs(w)
    print(f"case {w.name}", flush=True)
    out, lse, plan = parity.run_gpu(inp)
    assert plan["row_block"] == _mid_rows(w) and plan["schedule"] == 1, plan
    ref_o, ref_l = parity.oracle_full(inp)
    print(w.name, plan, parity.compare(out, lse, ref_o, ref_l, w.dtype), flush=True)


@pytest.mark.parametrize("page", [0, 32])
@pytest.mark.parametrize("case", MID_FORCED, ids=[c[0] for c in MID_FORCED])
def test_mid_row_tiles_forced_and_paged(case, page):
    w = _mid_workload(case)
    inp = wl.make_inputs(w)
    print(f"case {w.name} page={page}", flush=True)
    if page:
        pg = wl.to_paged(inp, page, seed=3)
        out, lse, plan = parity.run_gpu_paged(pg, inp, num_splits=3)
        ref_o, ref_l = parity.oracle_paged(pg, inp)
    else:
        out, lse, plan = parity.run_gpu(inp, num_splits=3)
        ref_o, ref_l = parity.oracle_full(inp)
    assert plan["row_block"] == _mid_rows(w) and plan["schedule"] == 0, plan
    assert plan["head_block"] == (2 if w.Hkv % 2 == 0 else 1), plan
    print(w.name, page, plan, parity.compare(out, lse, ref_o, ref_l, w.dtype), flush=True)
