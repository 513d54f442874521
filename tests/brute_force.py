"""Whole-matrix float64 attention in NumPy, for tiny shapes only.

An independent check of the oracle: it decodes the 16-bit inputs with its own
decoders (NumPy's float16 cast; bfloat16 as the upper half of a float32) and
materialises the full score matrix, masks it, and applies softmax with array
operations instead of the oracle's per-row loops.
"""
import numpy as np


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention(q_bits, k_bits, v_bits, seqlens, causal, dtype):
    q = decode(q_bits, dtype)
    k = decode(k_bits, dtype)
    v = decode(v_bits, dtype)
    B, qLen, Hq, D = q.shape
    _, cap, Hkv, _ = k.shape
    Dv = v.shape[3]                                    # may differ from D (= Dk)
    G = Hq // Hkv
    out = np.zeros((B, qLen, Hq, Dv))
    lse = np.full((B, Hq, qLen), -np.inf)
    for b in range(B):
        n = cap if seqlens is None else int(np.clip(seqlens[b], 0, cap))
        Kb = np.repeat(k[b, :n], G, axis=1)           # [n, Hq, D]
        Vb = np.repeat(v[b, :n], G, axis=1)
        S = np.einsum("ihd,jhd->hij", q[b], Kb) / np.sqrt(D)   # [Hq, qLen, n]
        ii = np.arange(qLen)[:, None]
        jj = np.arange(n)[None, :]
        vis = np.ones((qLen, n), bool) if not causal else (jj <= ii + n - qLen)
        S = np.where(vis[None], S, -np.inf)
        for h in range(Hq):
            for i in range(qLen):
                row = S[h, i]
                if not np.isfinite(row).any():
                    continue
                mx = row.max()
                P = np.exp(row - mx)
                L = P.sum()
                out[b, i, h] = P @ Vb[:, h] / L
                lse[b, h, i] = mx + np.log(L)
    return out, lse
