"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes the path of an oracle build so the same checks can be run
against deliberately broken builds (see test_oracle_mutants.py).  A pin
raises AssertionError when the oracle disagrees with:

* the IEEE binary16 / bfloat16 bit layouts (exhaustive decode),
* a whole-matrix NumPy brute force on tiny shapes,
* PyTorch's scaled_dot_product_attention in float64 (a third-party library
  routine for the same definition, with an explicit bottom-right mask and its
  own GQA head expansion),
* closed forms: one key -> O = V row; identical keys -> O = mean of V and
  lse = s + ln n; one dominant score -> O = that V row,
* invariants: causal with qLen = 1 equals non-causal; causal row i equals
  non-causal attention over the prefix of length n - qLen + i + 1; GQA equals
  MHA with repeated kv heads; values past the valid length never matter;
  convexity of O and the lse bounds,
* the log-sum-exp merge of two disjoint key ranges (the algebra the split-KV
  GPU path relies on) reproducing the single-range result,
* hand-worked examples under tests/golden/.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
import brute_force

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _rand(shape, dtype, g, sigma=1.0):
    td = torch.float16 if dtype == "fp16" else torch.bfloat16
    return (torch.randn(*shape, generator=g) * sigma).to(td)


def _dec(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# decoders


def pin_fp16_decode_exhaustive(lib_path):
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode16(bits, "fp16", lib_path)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16_decode_exhaustive(lib_path):
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode16(bits, "bf16", lib_path)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# --------------------------------------------------------------------------
# brute force and library routine

_TINY = [
    # B, qLen, Hq, Hkv, D, cap, lens, causal, dtype
    (1, 1, 1, 1, 4, 5, None, False, "fp16"),
    (2, 3, 4, 2, 4, 7, [7, 3], True, "fp16"),
    (2, 5, 4, 1, 64, 33, [33, 17], True, "bf16"),
    (2, 4, 2, 2, 64, 9, [0, 9], False, "bf16"),
    (1, 5, 8, 2, 16, 12, [3], True, "fp16"),    # causal with n < qLen: empty rows
    (2, 2, 8, 8, 8, 6, [6, 5], True, "bf16"),
    # head dims that are not multiples of 8 (the support range allows any)
    (2, 3, 4, 2, 1, 8, [8, 2], True, "fp16"),
    (1, 2, 6, 3, 5, 11, None, False, "bf16"),
    (2, 4, 4, 1, 17, 10, [10, 4], True, "bf16"),
]


def pin_brute_force_tiny(lib_path):
    g = torch.Generator().manual_seed(7)
    for (B, qLen, Hq, Hkv, D, cap, lens, causal, dt) in _TINY:
        q = _rand((B, qLen, Hq, D), dt, g)
        k = _rand((B, cap, Hkv, D), dt, g)
        v = _rand((B, cap, Hkv, D), dt, g)
        sl = None if lens is None else np.array(lens, np.int32)
        o1, l1 = oracle.attention(q, k, v, sl, causal, dt, lib_path=lib_path)
        o2, l2 = brute_force.attention(_bits(q), _bits(k), _bits(v), sl, causal, dt)
        assert np.allclose(o1, o2, rtol=0, atol=1e-12), (B, qLen, Hq, Hkv, D, causal)
        fin = np.isfinite(l2)
        assert np.array_equal(np.isfinite(l1), fin)
        assert np.array_equal(l1[~fin], l2[~fin])
        assert np.allclose(l1[fin], l2[fin], rtol=0, atol=1e-12)


def pin_torch_sdpa_fp64(lib_path):
    """torch SDPA in float64 with its own GQA expansion and an explicit mask."""
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(11)
    for (B, qLen, Hq, Hkv, D, cap, n, causal, dt) in [
            (1, 4, 8, 2, 64, 40, 40, True, "bf16"),
            (2, 8, 8, 1, 128, 70, 70, True, "fp16"),
            (1, 3, 4, 4, 32, 50, 50, False, "fp16"),
            (1, 2, 6, 3, 16, 30, 30, True, "bf16"),
            (1, 3, 4, 2, 3, 20, 20, True, "fp16"),
            (1, 2, 4, 1, 129, 25, 25, False, "bf16")]:
        q = _rand((B, qLen, Hq, D), dt, g)
        k = _rand((B, cap, Hkv, D), dt, g)
        v = _rand((B, cap, Hkv, D), dt, g)
        o1, l1 = oracle.attention(q, k, v, None, causal, dt, lib_path=lib_path)
        qt = q.to(torch.float64).permute(0, 2, 1, 3)        # B, Hq, qLen, D
        kt = k.to(torch.float64).permute(0, 2, 1, 3)        # B, Hkv, n, D
        vt = v.to(torch.float64).permute(0, 2, 1, 3)
        ii = torch.arange(qLen)[:, None]
        jj = torch.arange(n)[None, :]
        mask = (jj <= ii + n - qLen) if causal else torch.ones(qLen, n, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                             enable_gqa=True).permute(0, 2, 1, 3)
        assert np.allclose(o1, ref.numpy(), rtol=0, atol=1e-12)
        # lse from the library's own logsumexp of the scaled, masked scores
        kr = kt.repeat_interleave(Hq // Hkv, dim=1)
        s = (qt @ kr.transpose(-1, -2)) / math.sqrt(D)
        s = s.masked_fill(~mask, float("-inf"))
        lref = torch.logsumexp(s, dim=-1).numpy()
        assert np.allclose(l1, lref, rtol=0, atol=1e-12)


def pin_separate_key_and_value_dims(lib_path):
    """Dk != Dv (the MLA heads of the SmallQ README's support range): the
    brute force and torch SDPA in float64 (which also takes a V of another
    width, scale 1/sqrt(Dk)), and the value-slicing identity: each output
    channel depends on its V channel alone, so a V of Dv channels gives the
    first Dv channels of the output for a wider V."""
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(13)
    for (B, qLen, Hq, Hkv, Dk, Dv, cap, lens, causal, dt) in [
            (2, 3, 4, 2, 24, 16, 9, [9, 4], True, "bf16"),
            (1, 2, 2, 1, 16, 40, 7, None, False, "fp16"),
            (1, 4, 8, 2, 192, 128, 30, [30], True, "bf16"),
            (2, 2, 4, 2, 3, 13, 8, [8, 3], True, "fp16"),
            (1, 3, 2, 1, 17, 9, 6, None, False, "bf16")]:
        q = _rand((B, qLen, Hq, Dk), dt, g)
        k = _rand((B, cap, Hkv, Dk), dt, g)
        v = _rand((B, cap, Hkv, Dv), dt, g)
        sl = None if lens is None else np.array(lens, np.int32)
        o1, l1 = oracle.attention(q, k, v, sl, causal, dt, lib_path=lib_path)
        assert o1.shape == (B, qLen, Hq, Dv)
        o2, l2 = brute_force.attention(_bits(q), _bits(k), _bits(v), sl, causal, dt)
        assert np.allclose(o1, o2, rtol=0, atol=1e-12)
        assert np.array_equal(l1, l2) or np.allclose(l1, l2, rtol=0, atol=1e-12)
        if sl is None:
            qt = q.to(torch.float64).permute(0, 2, 1, 3)
            kt = k.to(torch.float64).permute(0, 2, 1, 3)
            vt = v.to(torch.float64).permute(0, 2, 1, 3)
            ii = torch.arange(qLen)[:, None]
            jj = torch.arange(cap)[None, :]
            mask = (jj <= ii + cap - qLen) if causal else torch.ones(qLen, cap, dtype=torch.bool)
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                 enable_gqa=True).permute(0, 2, 1, 3)
            assert np.allclose(o1, ref.numpy(), rtol=0, atol=1e-12)
        # slicing V to its first 8 channels slices the output, lse unchanged
        o3, l3 = oracle.attention(q, k, v[..., :8].contiguous(), sl, causal, dt,
                                  lib_path=lib_path)
        assert np.array_equal(o3, o1[..., :8]) and np.array_equal(l3, l1)


# --------------------------------------------------------------------------
# closed forms


def pin_single_key(lib_path):
    """kvLen = 1: the softmax weight is exactly 1, O is the V row, lse = s0."""
    g = torch.Generator().manual_seed(3)
    for dt in ("fp16", "bf16"):
        B, qLen, Hq, Hkv, D = 2, 1, 4, 2, 64
        q = _rand((B, qLen, Hq, D), dt, g)
        k = _rand((B, 1, Hkv, D), dt, g)
        v = _rand((B, 1, Hkv, D), dt, g)
        o, l = oracle.attention(q, k, v, None, False, dt, lib_path=lib_path)
        qd, kd, vd = _dec(q), _dec(k), _dec(v)
        for b in range(B):
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                assert np.array_equal(o[b, 0, h], vd[b, 0, hk])
                s0 = float(np.dot(qd[b, 0, h], kd[b, 0, hk])) / math.sqrt(D)
                assert abs(l[b, h, 0] - s0) <= 1e-12 * max(1.0, abs(s0))
    # causal with qLen > 1 and one key: only the last row sees it
    q = _rand((1, 3, 2, 16), "fp16", g)
    k = _rand((1, 1, 2, 16), "fp16", g)
    v = _rand((1, 1, 2, 16), "fp16", g)
    o, l = oracle.attention(q, k, v, None, True, "fp16", lib_path=lib_path)
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(l[0, :, :2]))
    assert np.array_equal(o[0, 2], _dec(v)[0, 0])


def pin_identical_keys(lib_path):
    """All visible K rows equal: uniform weights, O = mean V, lse = s + ln n."""
    g = torch.Generator().manual_seed(5)
    for dt, n, cap in (("fp16", 37, 40), ("bf16", 300, 300)):
        D, Hkv, Hq = 64, 2, 4
        q = _rand((1, 1, Hq, D), dt, g)
        krow = _rand((1, 1, Hkv, D), dt, g)
        k = krow.expand(1, cap, Hkv, D).contiguous()
        v = _rand((1, cap, Hkv, D), dt, g)
        o, l = oracle.attention(q, k, v, np.array([n], np.int32), False, dt,
                                lib_path=lib_path)
        vd = _dec(v)
        for h in range(Hq):
            hk = h // 2
            assert np.allclose(o[0, 0, h], vd[0, :n, hk].mean(axis=0), rtol=0, atol=1e-13)
            s = float(np.dot(_dec(q)[0, 0, h], _dec(krow)[0, 0, hk])) / math.sqrt(D)
            assert abs(l[0, h, 0] - (s + math.log(n))) < 1e-12 * max(1, abs(s))


def pin_dominant_key(lib_path):
    """One key scores >= 40 above every other: O is that V row within e^-40."""
    D, cap, jstar = 64, 50, 17
    for dt in ("fp16", "bf16"):
        g = torch.Generator().manual_seed(9)
        q = torch.zeros(1, 1, 1, D)
        q[..., 0] = 16.0
        k = torch.randn(1, cap, 1, D, generator=g)
        k[..., 0] = 0.0                   # every key orthogonal to q ...
        k[0, jstar, 0, 0] = 32.0          # ... except j*: s* = 16*32/8 = 64
        v = torch.randn(1, cap, 1, D, generator=g)
        td = torch.float16 if dt == "fp16" else torch.bfloat16
        q, k, v = q.to(td), k.to(td), v.to(td)
        o, l = oracle.attention(q, k, v, None, False, dt, lib_path=lib_path)
        vd = _dec(v)
        err = np.abs(o[0, 0, 0] - vd[0, jstar, 0]).max()
        assert err <= cap * math.exp(-60) * np.abs(vd).max() + 1e-15
        assert abs(l[0, 0, 0] - 64.0) <= cap * math.exp(-60) + 1e-12


# --------------------------------------------------------------------------
# invariants


def pin_causal_qlen1_is_noncausal(lib_path):
    g = torch.Generator().manual_seed(12)
    q = _rand((2, 1, 4, 64), "bf16", g)
    k = _rand((2, 20, 2, 64), "bf16", g)
    v = _rand((2, 20, 2, 64), "bf16", g)
    sl = np.array([20, 7], np.int32)
    o1, l1 = oracle.attention(q, k, v, sl, True, "bf16", lib_path=lib_path)
    o2, l2 = oracle.attention(q, k, v, sl, False, "bf16", lib_path=lib_path)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_causal_row_is_prefix(lib_path):
    """Causal row i == non-causal attention over the first n - qLen + i + 1 keys."""
    g = torch.Generator().manual_seed(13)
    B, qLen, Hq, Hkv, D, cap = 2, 6, 4, 2, 32, 30
    q = _rand((B, qLen, Hq, D), "fp16", g)
    k = _rand((B, cap, Hkv, D), "fp16", g)
    v = _rand((B, cap, Hkv, D), "fp16", g)
    sl = np.array([30, 11], np.int32)
    oc, lc = oracle.attention(q, k, v, sl, True, "fp16", lib_path=lib_path)
    for b in range(B):
        n = int(sl[b])
        for i in range(qLen):
            pre = np.array([n - qLen + i + 1 if bb == b else 0 for bb in range(B)], np.int32)
            qi = q[:, i:i + 1].contiguous()
            on, ln = oracle.attention(qi, k, v, pre, False, "fp16", lib_path=lib_path)
            assert np.allclose(oc[b, i], on[b, 0], rtol=0, atol=1e-14)
            assert np.allclose(lc[b, :, i], ln[b, :, 0], rtol=0, atol=1e-13)


def pin_gqa_is_repeated_mha(lib_path):
    g = torch.Generator().manual_seed(14)
    for G in (2, 4, 8):
        Hkv = 2
        Hq = G * Hkv
        q = _rand((1, 2, Hq, 32), "bf16", g)
        k = _rand((1, 25, Hkv, 32), "bf16", g)
        v = _rand((1, 25, Hkv, 32), "bf16", g)
        og, lg = oracle.attention(q, k, v, None, True, "bf16", lib_path=lib_path)
        kr = k.repeat_interleave(G, dim=2).contiguous()
        vr = v.repeat_interleave(G, dim=2).contiguous()
        om, lm = oracle.attention(q, kr, vr, None, True, "bf16", lib_path=lib_path)
        assert np.array_equal(og, om) and np.array_equal(lg, lm)


def pin_tail_never_read(lib_path):
    """Cache slots >= valid length (poisoned with NaN/Inf) never matter, and
    a longer capacity gives the same result as a cache truncated to n."""
    g = torch.Generator().manual_seed(15)
    q = _rand((2, 2, 4, 64), "fp16", g)
    k = _rand((2, 40, 2, 64), "fp16", g)
    v = _rand((2, 40, 2, 64), "fp16", g)
    sl = np.array([23, 40], np.int32)
    kp, vp = k.clone(), v.clone()
    kp[0, 23:] = float("nan")
    vp[0, 23:] = float("inf")
    o1, l1 = oracle.attention(q, k, v, sl, True, "fp16", lib_path=lib_path)
    o2, l2 = oracle.attention(q, kp, vp, sl, True, "fp16", lib_path=lib_path)
    assert np.isfinite(o2).all() and np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle.attention(q[:1], k[:1, :23].contiguous(), v[:1, :23].contiguous(),
                              None, True, "fp16", lib_path=lib_path)
    assert np.array_equal(o1[:1], o3) and np.array_equal(l1[:1], l3)


def pin_seqlens_clamped(lib_path):
    g = torch.Generator().manual_seed(16)
    q = _rand((3, 1, 2, 16), "bf16", g)
    k = _rand((3, 10, 1, 16), "bf16", g)
    v = _rand((3, 10, 1, 16), "bf16", g)
    o1, l1 = oracle.attention(q, k, v, np.array([99, -5, 0], np.int32), False, "bf16",
                              lib_path=lib_path)
    o2, l2 = oracle.attention(q, k, v, np.array([10, 0, 0], np.int32), False, "bf16",
                              lib_path=lib_path)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.all(o1[1:] == 0) and np.all(np.isneginf(l1[1:]))


def pin_convexity_and_lse_bounds(lib_path):
    g = torch.Generator().manual_seed(17)
    B, qLen, Hq, Hkv, D, cap = 2, 3, 4, 2, 64, 60
    q = _rand((B, qLen, Hq, D), "bf16", g, sigma=2.0)
    k = _rand((B, cap, Hkv, D), "bf16", g)
    v = _rand((B, cap, Hkv, D), "bf16", g)
    sl = np.array([60, 21], np.int32)
    o, l = oracle.attention(q, k, v, sl, True, "bf16", lib_path=lib_path)
    qd, kd, vd = _dec(q), _dec(k), _dec(v)
    for b in range(B):
        n = int(sl[b])
        for h in range(Hq):
            hk = h // 2
            for i in range(qLen):
                last = i + n - qLen
                vis = vd[b, :last + 1, hk]
                assert np.all(o[b, i, h] >= vis.min(axis=0) - 1e-12)
                assert np.all(o[b, i, h] <= vis.max(axis=0) + 1e-12)
                s = kd[b, :last + 1, hk] @ qd[b, i, h] / math.sqrt(D)
                assert s.max() - 1e-12 <= l[b, h, i] <= s.max() + math.log(last + 1) + 1e-12


def pin_lse_merge_of_key_ranges(lib_path):
    """Attention over keys [0, n) equals the log-sum-exp merge of the results
    over [0, a) and [a, n) -- the combine step of the split-KV method."""
    g = torch.Generator().manual_seed(18)
    B, qLen, Hq, Hkv, D, n = 1, 2, 4, 2, 64, 90
    q = _rand((B, qLen, Hq, D), "fp16", g)
    k = _rand((B, n, Hkv, D), "fp16", g)
    v = _rand((B, n, Hkv, D), "fp16", g)
    o, l = oracle.attention(q, k, v, None, False, "fp16", lib_path=lib_path)
    for a in (1, 33, 64, 89):
        oa, la = oracle.attention(q, k[:, :a].contiguous(), v[:, :a].contiguous(),
                                  None, False, "fp16", lib_path=lib_path)
        ob, lb = oracle.attention(q, k[:, a:].contiguous(), v[:, a:].contiguous(),
                                  None, False, "fp16", lib_path=lib_path)
        M = np.maximum(la, lb)
        wa, wb = np.exp(la - M), np.exp(lb - M)
        lm = M + np.log(wa + wb)
        om = ((wa.transpose(0, 2, 1)[..., None] * oa + wb.transpose(0, 2, 1)[..., None] * ob)
              / (wa + wb).transpose(0, 2, 1)[..., None])
        assert np.allclose(lm, l, rtol=0, atol=1e-12)
        assert np.allclose(om, o, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# hand-worked examples


def load_golden():
    with open(os.path.join(GOLDEN_DIR, "worked_examples.json")) as f:
        return json.load(f)["examples"]


def golden_inputs(ex):
    td = torch.float16 if ex["dtype"] == "fp16" else torch.bfloat16
    q = torch.tensor(ex["q"], dtype=torch.float64).to(td)
    k = torch.tensor(ex["k"], dtype=torch.float64).to(td)
    v = torch.tensor(ex["v"], dtype=torch.float64).to(td)
    for name, src, t in (("q", ex["q"], q), ("k", ex["k"], k), ("v", ex["v"], v)):
        # every fixture value is exactly representable in the storage dtype
        assert np.array_equal(t.to(torch.float64).numpy(), np.array(src, np.float64)), name
    if ex.get("poison_from") is not None:
        b, j0 = ex["poison_from"]
        k[b, j0:] = float("nan")
        v[b, j0:] = float("nan")
    sl = None if ex["cache_seqlens"] is None else np.array(ex["cache_seqlens"], np.int32)
    return q, k, v, sl


def _closed_form(expr):
    """Evaluate a hand-derived closed form such as "1 + log(1 + exp(-1))"."""
    if isinstance(expr, (int, float)):
        return float(expr)
    if expr == "-inf":
        return -math.inf
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log": math.log}))


def golden_expected(ex):
    eo = np.vectorize(_closed_form, otypes=[np.float64])(np.array(ex["expected_out"], dtype=object))
    el = np.vectorize(_closed_form, otypes=[np.float64])(np.array(ex["expected_lse"], dtype=object))
    return eo, el


def pin_golden_examples(lib_path):
    for ex in load_golden():
        q, k, v, sl = golden_inputs(ex)
        o, l = oracle.attention(q, k, v, sl, ex["causal"], ex["dtype"], lib_path=lib_path)
        eo, el = golden_expected(ex)
        assert np.allclose(o, eo, rtol=0, atol=1e-14), ex["name"]
        fin = np.isfinite(el)
        assert np.array_equal(np.isfinite(l), fin), ex["name"]
        assert np.allclose(l[fin], el[fin], rtol=0, atol=1e-14), ex["name"]


ALL_PINS = [
    pin_fp16_decode_exhaustive,
    pin_bf16_decode_exhaustive,
    pin_brute_force_tiny,
    pin_torch_sdpa_fp64,
    pin_separate_key_and_value_dims,
    pin_single_key,
    pin_identical_keys,
    pin_dominant_key,
    pin_causal_qlen1_is_noncausal,
    pin_causal_row_is_prefix,
    pin_gqa_is_repeated_mha,
    pin_tail_never_read,
    pin_seqlens_clamped,
    pin_convexity_and_lse_bounds,
    pin_lse_merge_of_key_ranges,
    pin_golden_examples,
]
