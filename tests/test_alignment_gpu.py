"""Buffers at every alignment the boundary accepts (needs an MI355X).

The C ABI takes q, k, v and out at any 16-byte boundary and lse,
cache_seqlens and the block table at any 4-byte boundary; torch allocations
are aligned far more strictly, so the other tests never see such pointers.
Here every buffer is a view that starts a few bytes into an allocation of its
own (q +16 B, k +48 B, v +80 B, out +16 B, lse +4 B, lengths +4 B, block table
+4 B), on each kernel layout: the 4-row vector-ALU variant that streams whole
token rows (a cache of 256 MiB), the 4-head vector-ALU layout, head dim 64,
the 64-row and 16-row matrix-core tiles, head dims that are not multiples of
8, separate key and value dims, and paged caches.  The kernels' arithmetic
does not depend on addresses, so each result must equal, bit for bit, the
same call on aligned tensors, and match the fp64 oracle.
"""
import pytest
import torch

import oracle
import parity
import workloads as wl

pytestmark = pytest.mark.gpu

OFF = {"q": 16, "k": 48, "v": 80, "out": 16, "lse": 4, "lens": 4, "table": 4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    import split_kv_decode_amd as mx
    mx.lib()
    oracle.build()


def placed(t, off, fill=None):
    """A GPU copy of t (or a tensor of t's shape filled with `fill`) that
    starts `off` bytes into an allocation of its own; returns (keep, view)."""
    nbytes = t.numel() * t.element_size()
    buf = torch.empty(nbytes + off + 256, dtype=torch.uint8, device="cuda")
    v = buf[off:off + nbytes].view(t.dtype).view(t.shape)
    if fill is None:
        v.copy_(t.to("cuda"))
    else:
        v.fill_(fill)
    assert v.data_ptr() % 256 == off % 256
    return buf, v


def _check(out, lse, out_ref_bits, lse_ref, ref_o, ref_l, dtype):
    assert torch.equal(out.view(torch.int16), out_ref_bits), "output differs from the aligned call"
    assert torch.equal(lse, lse_ref), "lse differs from the aligned call"
    return parity.compare(parity.to_f64(out), lse.cpu().double().numpy(), ref_o, ref_l, dtype)


CONTIGUOUS = [
    # (name, workload, expected path, expected row block, expected head block)
    ("valu_rows_256MiB", wl.Workload("al1", B=8, qLen=1, Hq=32, Hkv=8, D=128, kv_cap=8192,
                                     dtype="bf16", causal=False, sigma=1.0, seed=71,
                                     len_range=(0, 8192)), "valu", 4, 8),
    ("valu_heads4", wl.Workload("al2", B=1, qLen=1, Hq=32, Hkv=32, D=128, kv_cap=1000,
                                dtype="fp16", causal=False, sigma=1.0, seed=72,
                                len_range=(1000, 1000)), "valu", 1, 4),
    ("valu_d64", wl.Workload("al3", B=3, qLen=2, Hq=16, Hkv=8, D=64, kv_cap=1500,
                             dtype="bf16", causal=True, sigma=1.0, seed=73,
                             len_range=(0, 1500)), "valu", None, None),
    ("mfma64", wl.Workload("al4", B=16, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=1100,
                           dtype="bf16", causal=True, sigma=0.5, seed=74,
                           len_range=(1, 1100)), "mfma", 64, 2),
    # the same draft on a short cache for two sequences: 16-row blocks
    ("mfma16_rowblocks", wl.Workload("al4s", B=2, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=3000,
                                     dtype="bf16", causal=True, sigma=0.5, seed=78,
                                     len_range=(1, 3000)), "mfma", 16, 1),
    ("mfma16", wl.Workload("al5", B=1, qLen=8, Hq=16, Hkv=16, D=128, kv_cap=2000,
                           dtype="fp16", causal=False, sigma=1.0, seed=75,
                           len_range=(2000, 2000)), "mfma", 16, 2),
    ("odd_d100", wl.Workload("al6", B=2, qLen=2, Hq=8, Hkv=2, D=100, kv_cap=700,
                             dtype="fp16", causal=True, sigma=1.0, seed=76,
                             len_range=(1, 700)), "mfma", 16, 1),
    ("odd_d37", wl.Workload("al7", B=2, qLen=3, Hq=8, Hkv=4, D=37, kv_cap=500,
                            dtype="bf16", causal=False, sigma=1.0, seed=77,
                            len_range=(0, 500)), "mfma", 16, 1),
]


@pytest.mark.parametrize("forced", [0, 3], ids=["planned", "forced3"])
@pytest.mark.parametrize("name,w,path,rb,hb", CONTIGUOUS, ids=[c[0] for c in CONTIGUOUS])
def test_offset_buffers_contiguous(name, w, path, rb, hb, forced):
    import split_kv_decode_amd as mx
    inp = wl.make_inputs(w)
    dt = 1 if w.dtype == "bf16" else 0
    need = mx.workspace_size(w.B, w.Hq, w.Hkv, w.D, w.qLen, w.kv_cap, w.causal, dt, forced)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    g = inp.to("cuda")
    print(f"case {name} forced={forced}", flush=True)
    o_ref, l_ref = mx.fwd_kvcache(g.q, g.k_cache, g.v_cache, g.cache_seqlens, w.causal,
                                  num_splits=forced, workspace=ws)
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()
    assert plan["path"] == path, plan
    if rb is not None and not forced:
        assert plan["row_block"] == rb and plan["head_block"] == hb, plan
    if forced and path == "mfma" and plan["rows"] > 16 and w.D % 8 == 0:
        # forced partitions keep the tile the head shape selects
        assert plan["row_block"] == (32 if plan["rows"] <= 32 else 48 if plan["rows"] <= 48 else 64), plan
    keep = []
    views = {}
    for key, t in (("q", inp.q), ("k", inp.k_cache), ("v", inp.v_cache)):
        b_, views[key] = placed(t, OFF[key])
        keep.append(b_)
    b_, out = placed(inp.q, OFF["out"], fill=float("nan"))
    keep.append(b_)
    b_, lse = placed(torch.empty((w.B, w.Hq, w.qLen), dtype=torch.float32), OFF["lse"],
                     fill=float("nan"))
    keep.append(b_)
    sl = None
    if inp.cache_seqlens is not None:
        b_, sl = placed(inp.cache_seqlens, OFF["lens"])
        keep.append(b_)
    mx.fwd_kvcache(views["q"], views["k"], views["v"], sl, w.causal, out=out, lse=lse,
                   num_splits=forced, workspace=ws)
    torch.cuda.synchronize()
    ref_o, ref_l = parity.oracle_full(inp)
    rep = _check(out, lse, o_ref.view(torch.int16), l_ref, ref_o, ref_l, w.dtype)
    print(name, forced, plan, rep, flush=True)


@pytest.mark.parametrize("Dk,Dv,qLen", [(192, 128, 4), (24, 200, 1)])
def test_offset_buffers_separate_dims(Dk, Dv, qLen):
    import split_kv_decode_amd as mx
    B, Hq, Hkv, cap = 2, 16, 2, 800
    q, k, v, sl = wl.make_inputs_dkdv(B, qLen, Hq, Hkv, Dk, Dv, cap, [800, 131], "bf16", 1.0,
                                      Dk + Dv)
    print(f"case dkdv {Dk}x{Dv} q{qLen}", flush=True)
    o_ref, l_ref = mx.fwd_kvcache_dkdv(q.cuda(), k.cuda(), v.cuda(), sl.cuda(), True)
    torch.cuda.synchronize()
    keep = []
    b1, qv = placed(q, OFF["q"])
    b2, kv_ = placed(k, OFF["k"])
    b3, vv = placed(v, OFF["v"])
    b4, slv = placed(sl, OFF["lens"])
    b5, out = placed(torch.empty((B, qLen, Hq, Dv), dtype=q.dtype), OFF["out"],
                     fill=float("nan"))
    b6, lse = placed(torch.empty((B, Hq, qLen), dtype=torch.float32), OFF["lse"],
                     fill=float("nan"))
    keep += [b1, b2, b3, b4, b5, b6]
    mx.fwd_kvcache_dkdv(qv, kv_, vv, slv, True, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, sl, True, "bf16")
    rep = _check(out, lse, o_ref.view(torch.int16), l_ref, ref_o, ref_l, "bf16")
    print("dkdv", Dk, Dv, mx.last_plan().as_dict(), rep, flush=True)


PAGED = [
    ("paged16_mfma64", wl.Workload("alp1", B=16, qLen=8, Hq=64, Hkv=8, D=128, kv_cap=1104,
                                   dtype="bf16", causal=True, sigma=0.5, seed=81,
                                   len_range=(1, 1104)), 16, "mfma", 64),
    ("paged64_valu", wl.Workload("alp2", B=4, qLen=1, Hq=16, Hkv=8, D=128, kv_cap=2048,
                                 dtype="fp16", causal=False, sigma=1.0, seed=82,
                                 len_range=(0, 2048)), 64, "valu", 2),
    ("paged32_odd_d50", wl.Workload("alp3", B=2, qLen=2, Hq=4, Hkv=2, D=50, kv_cap=512,
                                    dtype="bf16", causal=True, sigma=1.0, seed=83,
                                    len_range=(1, 512)), 32, "mfma", 16),
]


@pytest.mark.parametrize("name,w,P,path,rb", PAGED, ids=[c[0] for c in PAGED])
def test_offset_buffers_paged(name, w, P, path, rb):
    import split_kv_decode_amd as mx
    inp = wl.make_inputs(w)
    pg = wl.to_paged(inp, P, seed=9)
    g = pg.to("cuda")
    q = inp.q.to("cuda")
    print(f"case {name}", flush=True)
    o_ref, l_ref = mx.fwd_kvcache_paged(q, g.k_pages, g.v_pages, g.block_table, g.cache_seqlens,
                                        w.causal)
    torch.cuda.synchronize()
    plan = mx.last_plan().as_dict()
    assert plan["path"] == path and plan["row_block"] == rb and plan["combine"] == 1, plan
    keep = []
    b1, qv = placed(inp.q, OFF["q"])
    b2, kp = placed(pg.k_pages, OFF["k"])
    b3, vp = placed(pg.v_pages, OFF["v"])
    b4, bt = placed(pg.block_table, OFF["table"])
    b5, sl = placed(pg.cache_seqlens, OFF["lens"])
    b6, out = placed(inp.q, OFF["out"], fill=float("nan"))
    b7, lse = placed(torch.empty((w.B, w.Hq, w.qLen), dtype=torch.float32), OFF["lse"],
                     fill=float("nan"))
    keep += [b1, b2, b3, b4, b5, b6, b7]
    mx.fwd_kvcache_paged(qv, kp, vp, bt, sl, w.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = parity.oracle_paged(pg, inp)
    rep = _check(out, lse, o_ref.view(torch.int16), l_ref, ref_o, ref_l, w.dtype)
    print(name, mx.last_plan().as_dict(), rep, flush=True)
