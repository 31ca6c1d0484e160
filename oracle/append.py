"""Paged KV-cache append, float64 — TEST INFRASTRUCTURE (oracle side).

The new token of sequence s at position pos lives in physical page
block_tables[s][pos // bs], slot pos % bs (vllm-metal kernels page,
cf-1.com/news/5525226, section "什么是 Paged Attention").  Rotary position
embedding of K (voxtral.c page, dpshk.com/news/5521762, section
"下一步优化方向" names it as part of the KV write; the pages do not define
it), read here in the rotate-half form: for j < D/2 the pair
(k[j], k[j + D/2]) is rotated by the angle pos * theta^(-2j/D).
Everything is float64; the stored K is rounded once to fp16 (numpy's
round-to-nearest-even conversion).
"""
from __future__ import annotations

import numpy as np


def rope(k: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """float64 rotate-half rotary embedding of one head vector."""
    k = np.asarray(k, dtype=np.float64)
    D = k.shape[-1]
    H = D // 2
    j = np.arange(H, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * j / D)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(k)
    out[..., :H] = k[..., :H] * c - k[..., H:] * s
    out[..., H:] = k[..., :H] * s + k[..., H:] * c
    return out


def kv_append(k_cache, v_cache, block_tables, positions, k_new, v_new, rope_theta=0.0):
    """Return new (k_cache, v_cache) with each sequence's token written.
    Positions < 0 or past the page table, and page ids outside the pool,
    write nothing."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    nb, Hkv, bs, D = kc.shape
    S, mb = np.asarray(block_tables).shape
    for s in range(S):
        pos = int(positions[s])
        if pos < 0 or pos >= mb * bs:
            continue
        blk = int(block_tables[s][pos // bs])
        if blk < 0 or blk >= nb:
            continue
        for g in range(Hkv):
            k = np.asarray(k_new[s, g], dtype=np.float64)
            if rope_theta > 0:
                k = rope(k, pos, rope_theta)
            kc[blk, g, pos % bs] = k.astype(np.float16)
            vc[blk, g, pos % bs] = v_new[s, g]
    return kc, vc
