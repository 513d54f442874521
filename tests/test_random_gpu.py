"""Seeded random configurations on the GPU vs the fp64 oracle (needs an
MI355X).  A second, wider draw (up to 32 kv heads, any head dim, longer
caches) adds 200 cases, and a third, 48 cases of grouped-query drafts with
16 to 128 rows per kv head on batches large enough for the planner to keep
the 32-, 48- and 64-row matrix-core tiles under either schedule.

Each case draws a shape (batch, query length, GQA group, kv heads, head dim
64 or 128, dtype, causal mask, capacity), ragged lengths including empty
sequences, the partitioning (planner's choice or a forced count) and the
cache layout (contiguous, or paged with a random page size), so the cases
spread over both kernels, both schedules and the paged addressing.  The
draws are fixed by the seed; a failure names its case index.  Values are
N(0, 1) or N(0, 0.5^2), the distributions of the workloads the tolerances
are stated for: with wider values a row's output can reach |O| ~ 8, where
one bf16 unit in the last place (0.031) already exceeds the absolute bf16
tolerance of 2e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import workloads as wl

pytestmark = pytest.mark.gpu

N_CASES = 64
SEED = 20261203


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import split_kv_decode_amd as mx
    mx.lib()
    oracle.build()


def draw(case):
    r = np.random.default_rng([SEED, case])
    B = int(r.integers(1, 5))
    qLen = int(r.choice([1, 1, 2, 3, 5, 8, 12]))
    G = int(r.choice([1, 2, 3, 4, 8]))
    Hkv = int(r.integers(1, 4))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["fp16", "bf16"]))
    causal = bool(r.integers(0, 2))
    cap = int(r.integers(1, 1600))
    lengths = [int(x) for x in r.integers(0, cap + 1, size=B)]
    if r.random() < 0.3:
        lengths[int(r.integers(0, B))] = 0
    num_splits = int(r.choice([0, 0, 1, 2, 3, 7, 50]))
    page = int(r.choice([0, 0, 16, 32, 64, 128]))
    w = wl.Workload(f"random{case}", B=B, qLen=qLen, Hq=G * Hkv, Hkv=Hkv, D=D, kv_cap=cap,
                    dtype=dtype, causal=causal, sigma=float(r.choice([0.5, 1.0])),
                    seed=SEED + case, len_range=(0, cap))
    return w, lengths, num_splits, page


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(case):
    w, lengths, num_splits, page = draw(case)
    inp = wl.make_inputs(w, lengths=lengths)
    print(f"case {case}: {w.describe()} lengths={lengths} splits={num_splits} page={page}",
          flush=True)
    if page:
        pg = wl.to_paged(inp, page, seed=case)
        out, lse, plan = parity.run_gpu_paged(pg, inp, num_splits)
        ref_o, ref_l = parity.oracle_paged(pg, inp)
    else:
        out, lse, plan = parity.run_gpu(inp, num_splits)
        ref_o, ref_l = parity.oracle_full(inp)
    rep = parity.compare(out, lse, ref_o, ref_l, w.dtype)
    print(case, plan, rep, flush=True)


@pytest.mark.parametrize("case", range(16))
def test_random_head_dims(case):
    """Random key and value head dims (multiples of 8 up to 256, equal or
    not), ragged lengths and partitions: the matrix-core kernel's padded
    tiles."""
    import split_kv_decode_amd as mx
    r = np.random.default_rng([SEED, 1000 + case])
    B, qLen, G, Hkv = int(r.integers(1, 4)), int(r.choice([1, 2, 4, 8])), \
        int(r.choice([1, 2, 4, 8])), int(r.integers(1, 3))
    Dk = 8 * int(r.integers(1, 33))
    Dv = Dk if r.random() < 0.4 else 8 * int(r.integers(1, 33))
    dt = str(r.choice(["fp16", "bf16"]))
    causal = bool(r.integers(0, 2))
    cap = int(r.integers(1, 900))
    lens = [int(x) for x in r.integers(0, cap + 1, size=B)]
    num_splits = int(r.choice([0, 0, 1, 3, 9]))
    print(f"case {case}: B={B} qLen={qLen} G={G} Hkv={Hkv} Dk={Dk} Dv={Dv} {dt} causal={causal} "
          f"cap={cap} lens={lens} splits={num_splits}", flush=True)
    q, k, v, sl = wl.make_inputs_dkdv(B, qLen, G * Hkv, Hkv, Dk, Dv, cap, lens, dt, 1.0,
                                      SEED + case)
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


@pytest.mark.parametrize("case", range(16))
def test_random_packed_batches(case):
    """Random packed (varlen) batches: per-sequence query and key counts
    (empty ones included, queries beyond keys allowed), both kernels."""
    import split_kv_decode_amd as mx
    r = np.random.default_rng([SEED, 2000 + case])
    B = int(r.integers(1, 6))
    qlens = tuple(int(x) for x in r.choice([0, 1, 2, 3, 7, 16, 40], size=B))
    if sum(qlens) == 0:
        qlens = (1,) + qlens[1:]
    klens = tuple(int(x) for x in r.integers(0, 1200, size=B))
    G, Hkv = int(r.choice([1, 2, 4, 8])), int(r.integers(1, 3))
    D = int(r.choice([64, 128]))
    w = wl.VarlenWorkload(f"rv{case}", qlens, klens, G * Hkv, Hkv, D,
                          str(r.choice(["fp16", "bf16"])), bool(r.integers(0, 2)), 1.0,
                          SEED + 2000 + case)
    print(f"case {case}: {w}", flush=True)
    q, k, v, cq, ck = wl.make_varlen_inputs(w)
    mq, mk = max(qlens), max(max(klens), 1)
    out, lse = mx.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cq.cuda(), ck.cuda(), mq, mk,
                             w.causal)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention_varlen(q, k, v, cq, ck, mq, mk, w.causal, w.dtype)
    rep = parity.compare(parity.to_f64(out), lse.cpu().double().numpy().T, ref_o, ref_l.T,
                         w.dtype)
    print(case, mx.last_plan().as_dict(), rep, flush=True)


@pytest.mark.parametrize("case", range(12))
def test_random_in_call_append(case):
    """Random in-call appends (contiguous or paged caches, drafts of 1-8 new
    tokens, sequences near capacity so some new tokens are dropped): the
    cache bit for bit and the attention to tolerance."""
    r = np.random.default_rng([SEED, 3000 + case])
    B, G, Hkv = int(r.integers(1, 4)), int(r.choice([1, 4, 8])), int(r.integers(1, 3))
    new_len = int(r.choice([1, 2, 5, 8]))
    qLen = int(r.choice([0, 1, new_len]))
    cap = int(r.integers(8, 1000))
    lens = [int(x) for x in r.integers(0, cap + 1, size=B)]
    w = wl.Workload(f"ra{case}", B=B, qLen=qLen, Hq=G * Hkv, Hkv=Hkv, D=int(r.choice([64, 128])),
                    kv_cap=cap, dtype=str(r.choice(["fp16", "bf16"])),
                    causal=bool(r.integers(0, 2)), sigma=1.0, seed=SEED + 3000 + case,
                    len_range=(0, cap))
    P = int(r.choice([0, 16, 64]))
    print(f"case {case}: {w.describe()} lens={lens} new_len={new_len} page={P}", flush=True)
    inp = wl.make_inputs(w, lengths=lens)
    parity.run_append(inp, new_len, P, num_splits=int(r.choice([0, 0, 2])), seed=case)


def draw_wide(case):
    """A wider space: up to 32 kv heads (every VALU slot layout, caches from a
    few KB to ~0.5 GB), head dims 64, 128 or any in 1..256, 16-token query
    drafts, caches up to 5000 keys, page sizes up to 256."""
    r = np.random.default_rng([SEED + 1, case])
    B = int(r.integers(1, 7))
    qLen = int(r.choice([1, 1, 1, 2, 3, 4, 8, 16]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2, 3, 4, 8, 12, 16, 32]))
    D = int(r.choice([64, 128, 128, int(r.integers(1, 257))]))
    dtype = str(r.choice(["fp16", "bf16"]))
    causal = bool(r.integers(0, 2))
    cap = int(r.choice([int(r.integers(1, 600)), int(r.integers(600, 5000))]))
    lengths = [int(x) for x in r.integers(0, cap + 1, size=B)]
    if r.random() < 0.3:
        lengths[int(r.integers(0, B))] = cap
    num_splits = int(r.choice([0, 0, 0, 1, 2, 5, 33]))
    page = int(r.choice([0, 0, 16, 64, 256]))
    G = min(G, max(1, 64 // Hkv))
    w = wl.Workload(f"wide{case}", B=B, qLen=qLen, Hq=G * Hkv, Hkv=Hkv, D=D, kv_cap=cap,
                    dtype=dtype, causal=causal, sigma=float(r.choice([0.5, 1.0])),
                    seed=SEED + 7000 + case, len_range=(0, cap))
    return w, lengths, num_splits, page


@pytest.mark.parametrize("case", range(200))
def test_random_wide_configuration(case):
    w, lengths, num_splits, page = draw_wide(case)
    inp = wl.make_inputs(w, lengths=lengths)
    print(f"case {case}: {w.describe()} lengths={lengths} splits={num_splits} page={page}",
          flush=True)
    if page:
        pg = wl.to_paged(inp, page, seed=case)
        out, lse, plan = parity.run_gpu_paged(pg, inp, num_splits)
        ref_o, ref_l = parity.oracle_paged(pg, inp)
    else:
        out, lse, plan = parity.run_gpu(inp, num_splits)
        ref_o, ref_l = parity.oracle_full(inp)
    rep = parity.compare(out, lse, ref_o, ref_l, w.dtype)
    print(case, plan, rep, flush=True)


def draw_tiles(case):
    """GQA groups of 4-16 with 3-8 query tokens (12-128 rows per kv head), 1-8
    kv heads, 6-24 sequences of 1000-3000 keys: the planner's 32-, 48- and
    64-row tiles with one or two kv heads per workgroup, balanced and fixed."""
    r = np.random.default_rng([SEED + 2, case])
    B = int(r.integers(6, 25))
    G = int(r.choice([4, 6, 8, 12, 16]))
    qLen = int(r.choice([3, 4, 5, 6, 8]))
    Hkv = int(r.choice([1, 2, 3, 4, 8]))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["fp16", "bf16"]))
    cap = int(r.integers(1000, 3001))
    lengths = [int(x) for x in r.integers(0, cap + 1, size=B)]
    lengths[int(r.integers(0, B))] = cap
    if r.random() < 0.3:
        lengths[int(r.integers(0, B))] = 0
    num_splits = int(r.choice([0, 0, 0, 4]))
    page = int(r.choice([0, 0, 16, 64]))
    w = wl.Workload(f"tiles{case}", B=B, qLen=qLen, Hq=G * Hkv, Hkv=Hkv, D=D, kv_cap=cap,
                    dtype=dtype, causal=bool(r.integers(0, 4)), sigma=float(r.choice([0.5, 1.0])),
                    seed=SEED + 9000 + case, len_range=(0, cap))
    return w, lengths, num_splits, page


N_TILE_CASES = 48


@pytest.mark.parametrize("case", range(N_TILE_CASES))
def test_random_tile_configuration(case):
    w, lengths, num_splits, page = draw_tiles(case)
    inp = wl.make_inputs(w, lengths=lengths)
    print(f"case {case}: {w.describe()} lengths={lengths} splits={num_splits} page={page}",
          flush=True)
    if page:
        pg = wl.to_paged(inp, page, seed=case)
        out, lse, plan = parity.run_gpu_paged(pg, inp, num_splits)
        ref_o, ref_l = parity.oracle_paged(pg, inp)
    else:
        out, lse, plan = parity.run_gpu(inp, num_splits)
        ref_o, ref_l = parity.oracle_full(inp)
    assert plan["path"] == "mfma", plan
    rep = parity.compare(out, lse, ref_o, ref_l, w.dtype)
    print(case, plan, rep, flush=True)
