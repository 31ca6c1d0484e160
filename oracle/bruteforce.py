"""Exact-arithmetic brute force for tiny paged-attention inputs — TEST
INFRASTRUCTURE.

A second, independent statement of the same definition as oracle.c (see that
file's header for the pages it follows), in pure Python for tiny inputs only:
dot products are exact rationals (fp16 values are dyadic rationals), and the
exponentials are evaluated with `decimal` at 60 significant digits, so the
result is the true value to far below float64 resolution.

The K and V rows are looked up through `block_tables` with explicit integer
index arithmetic on the flat pool, not through numpy indexing.
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

_PREC = 60


def _exp(x: Fraction) -> Decimal:
    getcontext().prec = _PREC
    return (Decimal(x.numerator) / Decimal(x.denominator)).exp()


def attention_exact(q, k_cache, v_cache, block_tables, seq_lens, scale):
    """Return a nested list out[s][h][d] of Decimal values (60 digits)."""
    getcontext().prec = _PREC
    q = np.asarray(q, dtype=np.float16)
    kf = np.asarray(k_cache, dtype=np.float16).reshape(-1)
    vf = np.asarray(v_cache, dtype=np.float16).reshape(-1)
    nb, Hkv, bs, D = np.asarray(k_cache).shape
    S, Hq, _ = q.shape
    G = Hq // Hkv
    sc = Fraction(float(np.float32(scale)))
    out = []
    for s in range(S):
        L = int(seq_lens[s])
        rows = []
        for h in range(Hq):
            g = h // G
            qv = [Fraction(float(x)) for x in q[s, h]]
            z = []
            vrows = []
            for t in range(L):
                b = int(block_tables[s][t // bs])
                base = ((b * Hkv + g) * bs + (t % bs)) * D
                kr = [Fraction(float(kf[base + d])) for d in range(D)]
                vrows.append([Fraction(float(vf[base + d])) for d in range(D)])
                z.append(sc * sum(a * b_ for a, b_ in zip(qv, kr)))
            zmax = max(z)
            e = [_exp(zt - zmax) for zt in z]
            tot = sum(e)
            res = []
            for d in range(D):
                num = sum(e[t] * Decimal(vrows[t][d].numerator) / Decimal(vrows[t][d].denominator)
                          for t in range(L))
                res.append(num / tot)
            rows.append(res)
        out.append(rows)
    return out
