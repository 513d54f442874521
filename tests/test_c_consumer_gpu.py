"""The C ABI driven by a plain C99 program (needs an MI355X): no Python or
torch in the calling process.  The program queries the scratch size, runs
the call on its own stream, and, with the planner's partitions, also runs the
library-managed entry point and requires the same bits; its results must
match the fp64 oracle like the binding's."""
import os

import pytest

import c_consumer
import parity
import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [
    # (name, B, qLen, Hq, Hkv, D, kv_cap, dtype, causal, lengths, num_splits, page)
    ("gqa4_causal_ragged", 3, 2, 16, 4, 128, 1500, "bf16", True, [1500, 777, 0], 0, 0),
    ("gqa4_forced_splits", 3, 1, 16, 4, 128, 1500, "fp16", False, [1, 1500, 640], 7, 0),
    ("mha_d64_paged16", 2, 1, 8, 8, 64, 1000, "fp16", False, [1000, 33], 0, 16),
    ("gqa8_mtp_paged64", 2, 8, 32, 4, 128, 2048, "bf16", True, [2048, 900], 0, 64),
    ("odd_d100", 2, 3, 6, 2, 100, 600, "bf16", True, [600, 5], 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plain_c_caller_matches_oracle(case, tmp_path):
    name, B, qLen, Hq, Hkv, D, cap, dtype, causal, lengths, splits, page = case
    assert os.path.exists(c_consumer.BIN_PATH), "the C caller is not built: run build()"
    w = wl.Workload(name, B=B, qLen=qLen, Hq=Hq, Hkv=Hkv, D=D, kv_cap=cap, dtype=dtype,
                    causal=causal, sigma=1.0, seed=31)
    inp = wl.make_inputs(w, lengths=lengths)
    paged = wl.to_paged(inp, page, seed=3) if page else None
    prob, res = tmp_path / "problem.bin", tmp_path / "result.bin"
    c_consumer.write_problem(str(prob), inp, num_splits=splits, paged=paged)
    print(f"case {name}: running the C caller", flush=True)
    r = c_consumer.run(str(prob), str(res))
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, (r.returncode, r.stderr)
    status, plan, ws, out, lse = c_consumer.read_result(str(res), inp)
    assert status == 0
    if splits:
        assert plan["num_splits"] == splits and plan["schedule"] == 0, plan
    ro, rl = parity.oracle_paged(paged, inp) if paged else parity.oracle_full(inp)
    print(name, plan, ws, parity.compare(out, lse, ro, rl, dtype), flush=True)
