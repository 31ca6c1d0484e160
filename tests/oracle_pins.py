"""Pins of the float64 oracle against facts that do not come from the oracle.

Each pin takes an `Oracle` binding and raises AssertionError when the oracle
disagrees with:
  * a library routine (numpy's fp16 decoding, torch's float64
    scaled_dot_product_attention and logsumexp) on dense K/V that the test
    builds first and only then scatters into shuffled pages itself;
  * closed forms (L = 1, uniform keys, one dominant score, hand-worked z);
  * invariants (page permutation, split vs unsplit, score shift, GQA -> MHA);
  * exact-arithmetic brute force stored under tests/golden/;
  * the one-hot page-table probe.

test_oracle_pins.py runs them on the real oracle; test_oracle_mutants.py runs
them on deliberately broken builds and requires that each break is caught.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from paged_gqa_kv_decode_amd.workloads import make_custom, make_onehot_probe

LOG2E = 1.4426950408889634
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# Independent construction: dense K/V first, then scattered into pages here.
# ----------------------------------------------------------------------------
def dense_case(seed, lens, Hq, Hkv, D, bs, pool_factor=2.0, sigma_k=1.0, pad=-1):
    rng = np.random.default_rng(seed)
    S = len(lens)
    q = (rng.standard_normal((S, Hq, D), dtype=np.float32)).astype(np.float16)
    dk = [(rng.standard_normal((Hkv, L, D), dtype=np.float32) * sigma_k).astype(np.float16)
          for L in lens]
    dv = [rng.standard_normal((Hkv, L, D), dtype=np.float32).astype(np.float16) for L in lens]
    npages = [-(-L // bs) for L in lens]
    pool = max(1, int(math.ceil(pool_factor * sum(npages))))
    ids = rng.permutation(pool)
    kc = np.full((pool, Hkv, bs, D), np.nan, dtype=np.float16)
    vc = np.full((pool, Hkv, bs, D), np.nan, dtype=np.float16)
    bt = np.full((S, max(npages) + 1), pad, dtype=np.int32)
    pos = 0
    for s, L in enumerate(lens):
        for p in range(npages[s]):
            b = int(ids[pos]); pos += 1
            bt[s, p] = b
            n = min(bs, L - p * bs)
            kc[b, :, :n, :] = dk[s][:, p * bs:p * bs + n, :]
            vc[b, :, :n, :] = dv[s][:, p * bs:p * bs + n, :]
    scale = float(np.float32(1.0 / math.sqrt(D)))
    return dict(q=q, dk=dk, dv=dv, k_cache=kc, v_cache=vc, block_tables=bt,
                seq_lens=np.asarray(lens, dtype=np.int32), scale=scale, Hkv=Hkv)


def sdpa_dense(c):
    """torch float64 SDPA on the dense tensors, one sequence at a time, with
    the KV heads repeated to the query heads (head h reads KV head h // G)."""
    q = c["q"]
    S, Hq, D = q.shape
    G = Hq // c["Hkv"]
    out = np.empty((S, Hq, D))
    for s in range(S):
        qs = torch.from_numpy(q[s].astype(np.float64))[:, None, :]           # [Hq,1,D]
        ks = torch.from_numpy(c["dk"][s].astype(np.float64)).repeat_interleave(G, 0)
        vs = torch.from_numpy(c["dv"][s].astype(np.float64)).repeat_interleave(G, 0)
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=c["scale"])
        out[s] = o[:, 0, :].numpy()
    return out


def dense_scores(c, s):
    """[Hq, L] float64 scores from the dense K (numpy matmul)."""
    q = c["q"][s].astype(np.float64)
    G = q.shape[0] // c["Hkv"]
    k = np.repeat(c["dk"][s].astype(np.float64), G, axis=0)
    return c["scale"] * np.einsum("hd,htd->ht", q, k)


def run(orc, c):
    return orc.paged_attention_arrays(c["q"], c["k_cache"], c["v_cache"], c["block_tables"],
                                      c["seq_lens"], c["scale"])


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert np.all(np.isfinite(a)), f"{what}: non-finite oracle output"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


SDPA_CASES = [
    # (lens, Hq, Hkv, D, bs)
    ([5, 17, 1, 33], 8, 2, 16, 4),
    ([64], 32, 8, 128, 16),
    ([40, 7], 24, 4, 256, 32),
    ([3, 9, 1], 16, 2, 128, 8),
    ([70], 16, 2, 256, 32),
]


def pin_half_decode(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "fp16 decode differs from numpy"


def pin_sdpa(orc):
    for i, (lens, Hq, Hkv, D, bs) in enumerate(SDPA_CASES):
        c = dense_case(100 + i, lens, Hq, Hkv, D, bs)
        _close(run(orc, c), sdpa_dense(c), 1e-12, f"sdpa case {i}")


def pin_closed_forms(orc):
    # L = 1: the single V row, exactly, whatever q and K are.
    c = dense_case(7, [1, 1, 1], 16, 2, 32, 8)
    out = run(orc, c)
    G = 8
    for s in range(3):
        for h in range(16):
            assert np.array_equal(out[s, h], c["dv"][s][h // G, 0].astype(np.float64)), "L=1"
    # q = 0 and scale = 0: the exact mean of the V rows.
    for kind in ("q0", "scale0", "samek"):
        c = dense_case(8, [13, 5], 8, 2, 16, 4)
        if kind == "q0":
            c["q"][:] = 0
        elif kind == "scale0":
            c["scale"] = 0.0
        else:                                   # all K rows of a head identical
            for s in range(2):
                c["dk"][s][:] = c["dk"][s][:, :1, :]
            c = _rescatter(c, 4, seed=9)
        out = run(orc, c)
        for s in range(2):
            for h in range(8):
                rows = c["dv"][s][h // 4]
                mean = [float(sum(Fraction(float(x)) for x in rows[:, d]) / rows.shape[0])
                        for d in range(rows.shape[1])]
                _close(out[s, h], mean, 1e-14, f"mean-of-V ({kind})")
    # Hand-worked: scores (0, 1, 2), V rows (1,0), (0,1), (1,1) ->
    # out = ((1 + e^2), (e + e^2)) / (1 + e + e^2); tokens 0,1 in block 1, 2 in block 0.
    q = np.array([[[1.0, 0.0]]], dtype=np.float16)
    kc = np.zeros((2, 1, 2, 2), dtype=np.float16)
    vc = np.zeros((2, 1, 2, 2), dtype=np.float16)
    kc[1, 0, 0] = (0, 5); kc[1, 0, 1] = (1, 7); kc[0, 0, 0] = (2, -3); kc[0, 0, 1] = (np.nan, np.nan)
    vc[1, 0, 0] = (1, 0); vc[1, 0, 1] = (0, 1); vc[0, 0, 0] = (1, 1); vc[0, 0, 1] = (np.nan, np.nan)
    bt = np.array([[1, 0]], dtype=np.int32)
    out = orc.paged_attention_arrays(q, kc, vc, bt, np.array([3], dtype=np.int32), 1.0)
    e = math.e
    den = 1 + e + e * e
    _close(out[0, 0], [(1 + e * e) / den, (e + e * e) / den], 1e-15, "hand-worked z=(0,1,2)")
    # One score ahead of all others by > 745 nats: exactly that V row.
    c = dense_case(11, [9], 2, 1, 8, 4)
    c["q"][:] = 0
    c["q"][0, :, 0] = 60.0
    c["dk"][0][:] = 0
    c["dk"][0][0, 5, 0] = 60.0          # z_5 = 3600 * scale = 1272.8 nats
    c = _rescatter(c, 4, seed=12)
    out = run(orc, c)
    assert np.array_equal(out[0, 0], c["dv"][0][0, 5].astype(np.float64)), "dominant score"


def _rescatter(c, bs, seed):
    lens = [int(x) for x in c["seq_lens"]]
    Hq, D = c["q"].shape[1], c["q"].shape[2]
    nc = dense_case(seed, lens, Hq, c["Hkv"], D, bs)
    nc["q"], nc["dk"], nc["dv"], nc["scale"] = c["q"], c["dk"], c["dv"], c["scale"]
    # re-scatter the given dense tensors into nc's page placement
    kc = np.full_like(nc["k_cache"], np.nan)
    vc = np.full_like(nc["v_cache"], np.nan)
    for s, L in enumerate(lens):
        for p in range(-(-L // bs)):
            b = nc["block_tables"][s, p]
            n = min(bs, L - p * bs)
            kc[b, :, :n] = c["dk"][s][:, p * bs:p * bs + n]
            vc[b, :, :n] = c["dv"][s][:, p * bs:p * bs + n]
    nc["k_cache"], nc["v_cache"] = kc, vc
    return nc


def pin_large_scores(orc):
    """Scores of thousands of nats: subtracting the maximum keeps the result finite
    and equal to the float64 library softmax."""
    c = dense_case(13, [21, 4], 8, 2, 16, 4, sigma_k=1000.0)
    _close(run(orc, c), sdpa_dense(c), 1e-9, "large scores")


def pin_permutation(orc):
    wl = make_custom(seq_lens=[37, 5, 64], num_q_heads=16, num_kv_heads=2, head_dim=32,
                     block_size=8, seed=21, pool_factor=1.5)
    base = orc.paged_attention(wl)
    rng = np.random.default_rng(22)
    perm = rng.permutation(wl.num_blocks)          # new id of old block b is perm[b]
    k2 = np.empty_like(wl.k_cache)
    v2 = np.empty_like(wl.v_cache)
    k2[perm] = wl.k_cache
    v2[perm] = wl.v_cache
    bt2 = wl.block_tables.copy()
    valid = bt2 >= 0
    bt2[valid] = perm[bt2[valid]]
    out = orc.paged_attention_arrays(wl.q, k2, v2, bt2, wl.seq_lens, wl.scale)
    assert np.array_equal(out, base), "page permutation changed the output"


def pin_split_merge(orc):
    wl = make_custom(seq_lens=[1100, 1, 513, 256, 257], num_q_heads=16, num_kv_heads=2,
                     head_dim=16, block_size=8, seed=31)
    direct = orc.paged_attention(wl)
    for P in (8, 256, 512):
        m, l, o = orc.partials(wl, P)
        _close(orc.merge(m, l, o, wl.seq_lens, P), direct, 1e-12, f"split/merge P={P}")
        # partitions past each sequence's end are untouched
        for s, L in enumerate(wl.seq_lens):
            n = -(-int(L) // P)
            assert np.all(np.isnan(m[s, :, n:])), "wrote past the last partition"
            assert np.all(np.isfinite(m[s, :, :n])), "missing partition"


def pin_partials_closed(orc):
    c = dense_case(41, [6, 3], 4, 1, 8, 2)
    # P = 1: each partition is one token: m = log2e z_t, l = 1, o = v_t.
    m, l, o = orc.partials_arrays(c["q"], c["k_cache"], c["v_cache"], c["block_tables"],
                                  c["seq_lens"], c["scale"], 1)
    for s, L in enumerate([6, 3]):
        z = dense_scores(c, s)
        for h in range(4):
            _close(m[s, h, :L], LOG2E * z[h], 1e-13, "P=1 max")
            assert np.array_equal(l[s, h, :L], np.ones(L)), "P=1 exp-sum"
            assert np.array_equal(o[s, h, :L], c["dv"][s][0].astype(np.float64)), "P=1 out"
    # One partition covering everything: m + log2 l = log2e * logsumexp(z),
    # o = library softmax attention.
    c = dense_case(42, [30, 17], 8, 2, 16, 8)
    m, l, o = orc.partials_arrays(c["q"], c["k_cache"], c["v_cache"], c["block_tables"],
                                  c["seq_lens"], c["scale"], 256)
    ref = sdpa_dense(c)
    for s in range(2):
        lse = torch.logsumexp(torch.from_numpy(dense_scores(c, s)), dim=1).numpy()
        _close(m[s, :, 0] + np.log2(l[s, :, 0]), LOG2E * lse, 1e-12, "log-sum-exp")
        _close(o[s, :, 0], ref[s], 1e-12, "single partition output")


def pin_merge_closed(orc):
    S, Hq, NP, D = 1, 2, 3, 4
    seq = np.array([3 * 256], dtype=np.int32)
    rng = np.random.default_rng(5)
    o = rng.standard_normal((S, Hq, NP, D))
    m = np.full((S, Hq, NP), 1.5)
    l = np.full((S, Hq, NP), 7.0)
    out = orc.merge(m, l, o, seq, 256)
    _close(out, o.mean(axis=2), 1e-15, "equal weights -> mean")
    m2 = m.copy()
    m2[0, :, 1] += 200.0
    out = orc.merge(m2, np.full_like(l, 4.0), o, seq, 256)   # w = 4: scaling is exact
    assert np.array_equal(out, o[:, :, 1, :]), "dominant partition"
    # weights l_i 2^(m_i - M): exact ratio check with two partitions
    m3 = np.array([[[0.0, 1.0, 0.0]] * Hq])
    l3 = np.array([[[3.0, 1.0, 0.0]] * Hq])
    out = orc.merge(m3, l3, o, np.array([2 * 256], dtype=np.int32), 256)
    _close(out, (3 * o[:, :, 0] + 2 * o[:, :, 1]) / 5, 1e-15, "weights l*2^(m-M)")


def pin_shift_invariance(orc):
    """A constant first K column adds q[0]*c*scale to every score of a head;
    changing q[0] shifts all its scores equally and must not change out."""
    c = dense_case(51, [25, 9], 8, 2, 16, 4)
    for s in range(2):
        c["dk"][s][:, :, 0] = 1.0
    c = _rescatter(c, 4, seed=52)
    base = run(orc, c)
    c["q"][:, :, 0] = np.float16(3.0)
    _close(run(orc, c), base, 1e-13, "score shift")


def pin_gqa_to_mha(orc):
    wl = make_custom(seq_lens=[19, 40], num_q_heads=16, num_kv_heads=2, head_dim=16,
                     block_size=8, seed=61)
    base = orc.paged_attention(wl)
    G = 8
    k2 = np.repeat(wl.k_cache, G, axis=1)
    v2 = np.repeat(wl.v_cache, G, axis=1)
    out = orc.paged_attention_arrays(wl.q, k2, v2, wl.block_tables, wl.seq_lens, wl.scale)
    assert np.array_equal(out, base), "GQA != MHA with repeated KV heads"


def pin_onehot(orc):
    base = make_custom(seq_lens=[70, 1, 33], num_q_heads=24, num_kv_heads=4, head_dim=16,
                       block_size=8, seed=71, pool_factor=3.0, canaries=True)
    wl, targets = make_onehot_probe(base, seed=72, amplitude=60.0)  # 900-nat gap: e^-900 = 0 in float64
    out = orc.paged_attention(wl)
    G = 6
    for s in range(wl.num_seqs):
        for h in range(wl.num_q_heads):
            t = int(targets[s, h])
            blk = int(wl.block_tables[s, t // wl.block_size])
            want = [blk % 2048, blk // 2048, t % wl.block_size, h // G]
            assert list(out[s, h, :4]) == want, f"probe ({s},{h}): {out[s, h, :4]} != {want}"
            assert np.all(out[s, h, 4:] == 0.0)


def pin_golden(orc):
    for name in sorted(os.listdir(GOLDEN)):
        if not name.endswith(".json"):
            continue
        with open(os.path.join(GOLDEN, name)) as f:
            case = json.load(f)
        sh = case["shapes"]
        q = np.array(case["q_bits"], dtype=np.uint16).view(np.float16).reshape(sh["q"])
        k = np.array(case["k_bits"], dtype=np.uint16).view(np.float16).reshape(sh["kv"])
        v = np.array(case["v_bits"], dtype=np.uint16).view(np.float16).reshape(sh["kv"])
        bt = np.array(case["block_tables"], dtype=np.int32)
        sl = np.array(case["seq_lens"], dtype=np.int32)
        out = orc.paged_attention_arrays(q, k, v, bt, sl, case["scale"])
        want = np.array([float(x) for x in case["expected"]]).reshape(out.shape)
        _close(out, want, 1e-13, f"golden {name}")


# ----------------------------------------------------------------------------
# Several query tokens per sequence (causal, packed rows).
# ----------------------------------------------------------------------------
def varlen_case(seed, lens, qlens, Hq, Hkv, D, bs):
    c = dense_case(seed, lens, Hq, Hkv, D, bs)
    rng = np.random.default_rng(seed + 1000)
    T = int(sum(qlens))
    c["qv"] = rng.standard_normal((T, Hq, D), dtype=np.float32).astype(np.float16)
    c["cu"] = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    c["qlens"] = list(qlens)
    return c


def run_varlen(orc, c):
    return orc.paged_varlen_arrays(c["qv"], c["k_cache"], c["v_cache"], c["block_tables"],
                                   c["seq_lens"], c["cu"], c["scale"])


def sdpa_varlen(c):
    """torch float64 SDPA per sequence with an explicit boolean mask: query j
    of a sequence of L tokens whose last qlen are the queries sees the tokens
    t <= L - qlen + j.  Rows that see no token are zeros."""
    Hq, D = c["qv"].shape[1], c["qv"].shape[2]
    G = Hq // c["Hkv"]
    out = np.zeros((c["qv"].shape[0], Hq, D))
    for s, (L, ql) in enumerate(zip(c["seq_lens"], c["qlens"])):
        L, ql = int(L), int(ql)
        if ql == 0:
            continue
        rows = c["qv"][c["cu"][s]:c["cu"][s + 1]].astype(np.float64)      # [ql, Hq, D]
        qs = torch.from_numpy(rows.transpose(1, 0, 2).copy())              # [Hq, ql, D]
        ks = torch.from_numpy(c["dk"][s].astype(np.float64)).repeat_interleave(G, 0)
        vs = torch.from_numpy(c["dv"][s].astype(np.float64)).repeat_interleave(G, 0)
        mask = torch.zeros((ql, L), dtype=torch.bool)
        for j in range(ql):
            mask[j, :max(0, L - ql + j + 1)] = True
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask,
                                                             scale=c["scale"])
        o = o.numpy().transpose(1, 0, 2)
        for j in range(ql):
            if L - ql + j + 1 > 0:
                out[c["cu"][s] + j] = o[j]
    return out


VARLEN_CASES = [([40, 7, 100, 3], [5, 7, 1, 5], 8, 2, 16, 4),
                ([33, 64, 1], [33, 16, 1], 24, 4, 8, 8)]


def pin_varlen_sdpa(orc):
    for i, (lens, qlens, Hq, Hkv, D, bs) in enumerate(VARLEN_CASES):
        c = varlen_case(200 + i, lens, qlens, Hq, Hkv, D, bs)
        got = run_varlen(orc, c)
        _close(got, sdpa_varlen(c), 1e-12, f"varlen sdpa case {i}")


def pin_varlen_rows_are_truncated_decodes(orc):
    """Query row j of sequence s is a one-token decode over the first
    L - qlen + j + 1 tokens of the same pages: same value to the last bit."""
    c = varlen_case(211, [50, 9, 30], [6, 9, 2], 8, 2, 16, 4)
    got = run_varlen(orc, c)
    for s, (L, ql) in enumerate(zip(c["seq_lens"], c["qlens"])):
        for j in range(ql):
            lim = int(L) - ql + j + 1
            row = c["cu"][s] + j
            ref = orc.paged_attention_arrays(c["qv"][row:row + 1], c["k_cache"], c["v_cache"],
                                             c["block_tables"][s:s + 1],
                                             np.array([lim], dtype=np.int32), c["scale"])
            assert np.array_equal(got[row], ref[0]), f"row {row} != decode over {lim} tokens"


def pin_varlen_one_token_is_decode(orc):
    c = varlen_case(221, [17, 1, 64], [1, 1, 1], 16, 2, 32, 8)
    got = run_varlen(orc, c)
    ref = orc.paged_attention_arrays(c["qv"], c["k_cache"], c["v_cache"], c["block_tables"],
                                     c["seq_lens"], c["scale"])
    assert np.array_equal(got, ref), "qlen = 1 must be the decode oracle"


# ----------------------------------------------------------------------------
# Other element types of q, K and V (bf16 bit patterns, fp32).
# ----------------------------------------------------------------------------
def pin_bf16_decode(orc):
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):          # signalling NaN patterns
        ref = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([orc.bf16_to_double(int(b)) for b in bits[::97]] +
                   [orc.bf16_to_double(int(b)) for b in (0x0000, 0x8000, 0x0001, 0x7F80, 0xFF80,
                                                        0x7F7F, 0x3F80, 0x7FC0)])
    want = np.concatenate([ref[::97], ref[[0x0000, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x7F7F,
                                           0x3F80, 0x7FC0]]])
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert np.all(same), "bf16 decode"


def _dtype_case(seed, lens, Hq, Hkv, D, bs, dtype):
    """Dense values in the element type; torch builds the float64 copies the
    reference uses from the stored bits itself."""
    c = dense_case(seed, lens, Hq, Hkv, D, bs)
    rng = np.random.default_rng(seed + 7)

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if dtype == "f32":
            return x, torch.from_numpy(x.copy()).double()
        u = x.view(np.uint32)
        b = (((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16)).astype(np.uint16)
        t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).double()
        return b, t

    S = len(lens)
    q, tq = draw((S, Hq, D))
    dk, tk, dv, tv = [], [], [], []
    for L in lens:
        a, ta = draw((Hkv, L, D))
        b_, tb = draw((Hkv, L, D))
        dk.append(a); tk.append(ta); dv.append(b_); tv.append(tb)
    st = np.float32 if dtype == "f32" else np.uint16
    kc = np.zeros(c["k_cache"].shape, dtype=st)
    vc = np.zeros(c["v_cache"].shape, dtype=st)
    for s, L in enumerate(lens):
        for p in range(-(-L // bs)):
            blk = c["block_tables"][s, p]
            n = min(bs, L - p * bs)
            kc[blk, :, :n, :] = dk[s][:, p * bs:p * bs + n, :]
            vc[blk, :, :n, :] = dv[s][:, p * bs:p * bs + n, :]
    G = Hq // Hkv
    ref = np.empty((S, Hq, D))
    for s in range(S):
        o = torch.nn.functional.scaled_dot_product_attention(
            tq[s][:, None, :], tk[s].repeat_interleave(G, 0), tv[s].repeat_interleave(G, 0),
            scale=c["scale"])
        ref[s] = o[:, 0, :].numpy()
    return q, kc, vc, c["block_tables"], c["seq_lens"], c["scale"], ref


def pin_other_element_types(orc):
    for dtype in ("bf16", "f32"):
        q, kc, vc, bt, sl, scale, ref = _dtype_case(301, [37, 1, 70], 16, 2, 32, 8, dtype)
        got = orc.paged_attention_arrays(q, kc, vc, bt, sl, scale, dtype=dtype)
        _close(got, ref, 1e-12, f"sdpa {dtype}")
        m, l, o = orc.partials_arrays(q, kc, vc, bt, sl, scale, 16, dtype=dtype)
        _close(orc.merge(m, l, o, sl, 16), ref, 1e-12, f"split/merge {dtype}")


def pin_varlen_bf16(orc):
    """bf16 q/K/V through the causal multi-token path: the oracle against torch
    float64 SDPA with a causal mask on the values torch itself decodes from
    the bf16 bits."""
    for i, (lens, qlens, Hq, Hkv, D, bs) in enumerate(VARLEN_CASES):
        c = varlen_case(230 + i, lens, qlens, Hq, Hkv, D, bs)
        rng = np.random.default_rng(240 + i)

        def bf16(shape):
            u = rng.standard_normal(shape, dtype=np.float32).view(np.uint32)
            bits = (((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16)).astype(np.uint16)
            vals = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
            return bits, vals

        qb, c["qv"] = bf16(c["qv"].shape)
        kc = np.zeros(c["k_cache"].shape, dtype=np.uint16)
        vc = np.zeros(c["v_cache"].shape, dtype=np.uint16)
        for s, L in enumerate(lens):
            kb_, c["dk"][s] = bf16((Hkv, L, D))
            vb_, c["dv"][s] = bf16((Hkv, L, D))
            for p in range(-(-L // bs)):
                blk = c["block_tables"][s, p]
                n = min(bs, L - p * bs)
                kc[blk, :, :n, :] = kb_[:, p * bs:p * bs + n, :]
                vc[blk, :, :n, :] = vb_[:, p * bs:p * bs + n, :]
        got = orc.paged_varlen_arrays(qb, kc, vc, c["block_tables"], c["seq_lens"], c["cu"],
                                      c["scale"], dtype="bf16")
        _close(got, sdpa_varlen(c), 1e-12, f"varlen bf16 case {i}")


ALL_PINS = [pin_half_decode, pin_sdpa, pin_closed_forms, pin_large_scores, pin_permutation,
            pin_split_merge, pin_partials_closed, pin_merge_closed, pin_shift_invariance,
            pin_gqa_to_mha, pin_onehot, pin_golden, pin_varlen_sdpa,
            pin_varlen_rows_are_truncated_decodes, pin_varlen_one_token_is_decode,
            pin_bf16_decode, pin_other_element_types, pin_varlen_bf16]
