"""The seeded random GPU cases reach every kernel layout (CPU only).

The planner is pure host code, so the layouts the random parity cases run
on can be listed without a GPU: every draw of the three families in
test_random_gpu.py is planned here, and the union must hold each
matrix-core row tile (16, 32, 48, 64 rows) with one and with two kv heads
per workgroup under both schedules, each vector-ALU row count with both
schedules, and both contiguous and paged caches on each kernel.  A change
to the draws or to the planner that drops a layout from the random cases
fails here rather than silently narrowing the GPU coverage.
"""
import collections

import split_kv_decode_amd as mx
from test_random_gpu import N_CASES, N_TILE_CASES, draw, draw_tiles, draw_wide


def _layouts():
    seen = collections.Counter()
    for fn, n in ((draw, N_CASES), (draw_wide, 200), (draw_tiles, N_TILE_CASES)):
        for case in range(n):
            w, _lengths, num_splits, page = fn(case)
            dt = mx.MXFA_BF16 if w.dtype == "bf16" else mx.MXFA_FP16
            p = mx.plan(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt,
                        num_splits).as_dict()
            seen[(p["path"], p["row_block"], p["head_block"], p["schedule"], bool(page))] += 1
    return seen


def test_random_cases_cover_every_matrix_core_tile():
    seen = _layouts()
    for rb in (16, 32, 48, 64):
        for hb in (1, 2):
            for sched in (0, 1):
                n = seen[("mfma", rb, hb, sched, False)] + seen[("mfma", rb, hb, sched, True)]
                assert n > 0, (rb, hb, sched, sorted(seen))
        for paged in (False, True):
            assert sum(v for k, v in seen.items()
                       if k[0] == "mfma" and k[1] == rb and k[4] == paged) > 0, (rb, paged)


def test_random_cases_cover_every_vector_alu_layout():
    seen = _layouts()
    for rows in (1, 2, 4, 8):
        for sched in (0, 1):
            assert sum(v for k, v in seen.items()
                       if k[0] == "valu" and k[1] == rows and k[3] == sched) > 0, (rows, sched)
        for paged in (False, True):
            assert sum(v for k, v in seen.items()
                       if k[0] == "valu" and k[1] == rows and k[4] == paged) > 0, (rows, paged)
    for hb in (1, 4, 8):
        assert sum(v for k, v in seen.items() if k[0] == "valu" and k[2] == hb) > 0, hb
