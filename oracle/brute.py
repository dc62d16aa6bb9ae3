"""Brute-force attention over the contiguous *logical* K/V arrays (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  This never looks at a block pool or a block table: it
is ordinary decode attention, softmax(scale * q K^T) V, over the sequence laid out
as one contiguous array from token 0 to n-1 -- the logical view the page
"显存虚拟化革命：PagedAttention 内存池管理与显存碎片终结" (blog.llmgo.top), §二.1
("逻辑块"), says PagedAttention must reproduce.  Query head h reads KV head
h // (Hq/Hkv) (consecutive grouping of query heads onto KV heads).

It pins the paged oracle: both must agree to 1e-12 on small inputs.
"""
from __future__ import annotations

import numpy as np


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """fp16/bf16 bit patterns -> float64, written independently of the generator."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        sign = np.where(bits >> 15, -1.0, 1.0)
        e = ((bits >> 10) & 0x1F).astype(np.int64)
        m = (bits & 0x3FF).astype(np.float64)
        val = np.where(e == 0, np.ldexp(m, -24), np.ldexp(m + 1024.0, (e - 25).astype(np.int32)))
        val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
        return sign * val
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def attention_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """q [D], K/V [n, D] float64 -> [D]; n == 0 gives zeros."""
    if K.shape[0] == 0:
        return np.zeros(q.shape[-1])
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def attention(w, scale: float) -> np.ndarray:
    """Decode attention of a workload over its logical arrays: [S, Hq, D] float64."""
    c = w.cfg
    G = c.num_q_heads // c.num_kv_heads
    out = np.zeros((c.num_seqs, c.num_q_heads, c.head_dim))
    q = widen(w.q, c.dtype)
    for s in range(c.num_seqs):
        Kb, Vb = w.logical_kv(s)
        K, V = widen(Kb, c.dtype), widen(Vb, c.dtype)
        for h in range(c.num_q_heads):
            out[s, h] = attention_one(q[s, h], K[:, h // G], V[:, h // G], scale)
    return out
