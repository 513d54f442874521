"""In-call KV append on the GPU vs the fp64 oracle (needs an MI355X).

The new keys and values are written into the cache (contiguous or paged)
before attention: the updated cache must equal the oracle's append bit for
bit (a copy), and the attention over the grown sequences must match the
oracle's.  Cache rows past the lengths are NaN, so a misplaced or missing
write, or a read past the new length, shows.
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
    # (name, B, qLen, Hq, Hkv, D, cap, dtype, causal, lengths, new_len)
    ("valu_decode", 3, 1, 32, 8, 128, 1000, "bf16", False, [999, 500, 0], 1),
    ("gqa_draft", 3, 2, 8, 2, 64, 700, "fp16", True, [690, 33, 5], 5),
    ("mfma_mtp", 2, 8, 64, 8, 128, 2048, "bf16", True, [2040, 100], 8),
    ("mfma_drop", 2, 8, 64, 8, 128, 2048, "bf16", True, [2045, 0], 8),
]


@pytest.mark.parametrize("P", [0, 16, 64])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_append_then_attend(case, P):
    name, B, qLen, Hq, Hkv, D, cap, dt, causal, lens, new_len = case
    w = wl.Workload(name, B=B, qLen=qLen, Hq=Hq, Hkv=Hkv, D=D, kv_cap=cap, dtype=dt,
                    causal=causal, sigma=1.0, seed=7 + P, len_range=(0, cap))
    inp = wl.make_inputs(w, lengths=lens)
    got = parity.run_append(inp, new_len, P)
    if P == 0:
        assert list(got) == [min(n + new_len, cap) for n in lens]


@pytest.mark.parametrize("num_splits", [1, 3])
def test_append_forced_splits_and_caller_workspace(num_splits):
    w = wl.Workload("ws", B=2, qLen=4, Hq=32, Hkv=4, D=128, kv_cap=600, dtype="bf16",
                    causal=True, sigma=1.0, seed=31, len_range=(0, 600))
    inp = wl.make_inputs(w, lengths=[300, 596])
    parity.run_append(inp, 4, 0, num_splits=num_splits, use_ws=True)
    parity.run_append(inp, 4, 32, num_splits=num_splits, use_ws=True)


def test_append_with_no_query_only_updates_the_cache():
    w = wl.Workload("q0", B=2, qLen=0, Hq=8, Hkv=2, D=64, kv_cap=64, dtype="fp16",
                    causal=False, sigma=1.0, seed=33, len_range=(0, 64))
    inp = wl.make_inputs(w, lengths=[10, 63])
    parity.run_append(inp, 3, 0)
    parity.run_append(inp, 3, 16)


def test_append_nothing_is_plain_attention():
    w = wl.Workload("n0", B=2, qLen=2, Hq=8, Hkv=2, D=128, kv_cap=300, dtype="bf16",
                    causal=True, sigma=1.0, seed=35, len_range=(0, 300))
    inp = wl.make_inputs(w, lengths=[300, 7])
    parity.run_append(inp, 0, 0)
