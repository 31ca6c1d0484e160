"""Seeded synthetic inputs for paged GQA decode attention.

This module only draws random numbers and lays them out in the paged-cache
format; it holds none of the attention arithmetic.  Both the float64 oracle
and the HIP path are fed from here, so they always see identical bytes.

Paged-cache format (vllm-metal kernels page, cf-1.com/news/5525226, section
"什么是 Paged Attention" — the KV cache is cut into fixed-size pages and a
`block_tables` page table maps each logical page of a sequence to a physical
page of a shared pool):

  q            fp16  [S, Hq, D]
  k_cache      fp16  [num_blocks, Hkv, block_size, D]
  v_cache      fp16  [num_blocks, Hkv, block_size, D]
  block_tables int32 [S, max_blocks_per_seq]   logical page -> physical page
  seq_lens     int32 [S]

Entries of `block_tables` past ceil(L/bs) are padding (default -1); they are
never meant to be dereferenced.

Values are `standard_normal(float32) * sigma`, rounded to fp16 with
round-to-nearest-even.  Each named workload i draws from
`numpy.random.SeedSequence(1000 + i).spawn(5)`: independent PCG64 streams for
(seq_lens, page placement, q, K, V).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_workload",
    "make_custom",
    "make_onehot_probe",
    "kv_read_bytes",
    "VARLEN_WORKLOADS",
    "make_varlen",
    "make_varlen_custom",
    "varlen_pairs",
]


@dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seq_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray      # int32 [S, max_blocks_per_seq]
    num_blocks: int
    q: np.ndarray                 # float16 [S, Hq, D]
    k_cache: np.ndarray           # float16 [num_blocks, Hkv, bs, D]
    v_cache: np.ndarray           # float16 [num_blocks, Hkv, bs, D]
    scale: float                  # an exactly representable float32 value
    partition_sizes: tuple = (512,)   # -1 = planner, 0 = unsplit, 256 / 512
    meta: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


# Named workloads: the shapes, length mixes and value distributions that the
# bench and the parity tests run.  Geometries are the four admitted (Hq, Hkv, D)
# triples; block sizes are the 8/16/32 page sizes; partitions 256 / 512.
WORKLOADS = {
    # 1 seq, (32q, 8kv, 128), L=64, bs 16: 4 pages at random ids of an 8-page pool.
    "tiny_1x64": dict(index=1, S=1, Hq=32, Hkv=8, D=128, bs=16, parts=(0,)),
    # 8 seqs, (32q, 8kv, 128), L uniform in [1, 2048], bs 16, 1024-page pool.
    "batch8_2k": dict(index=2, S=8, Hq=32, Hkv=8, D=128, bs=16, parts=(512,)),
    # 32 seqs, (24q, 4kv, 256), L uniform in [4096, 16384], bs 32, K x3.
    "long32_16k": dict(index=3, S=32, Hq=24, Hkv=4, D=256, bs=32, parts=(256, 512)),
    # 64 seqs, (16q, 2kv, 128), mixed lengths up to 32768, bs 8.
    "mixed64_32k": dict(index=4, S=64, Hq=16, Hkv=2, D=128, bs=8, parts=(512,)),
    # 4 seqs, (16q, 2kv, 256), L = 131072 each, bs 32, pool 2x needed, sigma 0.5.
    "long4_128k": dict(index=5, S=4, Hq=16, Hkv=2, D=256, bs=32, parts=(-1,)),
}


def _rngs(index: int):
    seqs = np.random.SeedSequence(1000 + index).spawn(5)
    return [np.random.Generator(np.random.PCG64(s)) for s in seqs]


def _draw_fp16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)
    # Draw in chunks to bound the float32 temporary.
    chunk = 1 << 26
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[lo:hi] = x.astype(np.float16)
    return out.reshape(shape)


def _seq_lens(name: str, S: int, rng: np.random.Generator) -> np.ndarray:
    if name == "tiny_1x64":
        return np.full(S, 64, dtype=np.int32)
    if name == "batch8_2k":
        return rng.integers(1, 2048, size=S, endpoint=True).astype(np.int32)
    if name == "long32_16k":
        return rng.integers(4096, 16384, size=S, endpoint=True).astype(np.int32)
    if name == "mixed64_32k":
        q = S // 4
        ones = np.ones(q, dtype=np.int64)
        u = rng.integers(0, 4095, size=q, endpoint=True)
        r = rng.integers(1, 3, size=q, endpoint=True)
        tails = 8 * u + r                      # 1-3 token tail pages (bs 8)
        rest = rng.integers(1, 32768, size=S - 2 * q, endpoint=True)
        lens = np.concatenate([ones, tails, rest])
        rng.shuffle(lens)
        return lens.astype(np.int32)
    if name == "long4_128k":
        return np.full(S, 131072, dtype=np.int32)
    raise KeyError(name)


def _place_pages(pages_per_seq, pool_blocks: int, rng, max_blocks: int,
                 pad_value: int, take_prefix: bool):
    """Assign physical pages sequence-major, in logical order, from a
    permutation of the pool."""
    need = int(sum(pages_per_seq))
    if need > pool_blocks:
        raise ValueError("pool too small")
    perm = rng.permutation(pool_blocks)
    ids = perm[:need] if take_prefix else perm
    S = len(pages_per_seq)
    bt = np.full((S, max_blocks), pad_value, dtype=np.int32)
    pos = 0
    for s, n in enumerate(pages_per_seq):
        bt[s, :n] = ids[pos:pos + n]
        pos += n
    return bt


def kv_read_bytes(seq_lens, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Algorithmic K+V bytes of one decode step: each element (fp16 unless
    elem_bytes says otherwise) of every valid token's K and V row is read
    once, for every KV head."""
    return int(2 * elem_bytes * num_kv_heads * head_dim *
               int(np.asarray(seq_lens, dtype=np.int64).sum()))


# Element types of q, K and V: numpy storage (bf16 as its uint16 bit pattern)
# and the value that stands for NaN in canaries.
ELEM_TYPES = {"f16": (np.float16, np.float16(np.nan)),
              "bf16": (np.uint16, np.uint16(0x7FC0)),
              "f32": (np.float32, np.float32(np.nan))}


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def _draw(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    """standard_normal(float32) * sigma in the element type (fp16 / bf16 round
    to nearest even; fp32 as drawn)."""
    if dtype == "f16":
        return _draw_fp16(rng, shape, sigma)
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    x = x.reshape(shape)
    return _to_bf16_bits(x) if dtype == "bf16" else x


def _fill_canaries(wl: Workload) -> None:
    """NaN in every pool block no sequence uses, and in the slots past L of
    each sequence's last page."""
    used = np.zeros(wl.num_blocks, dtype=bool)
    bs = wl.block_size
    nan = ELEM_TYPES[wl.meta.get("dtype", "f16")][1]
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        n = -(-L // bs)
        ids = wl.block_tables[s, :n]
        used[ids] = True
        tail = L - (n - 1) * bs
        if tail < bs:
            last = ids[n - 1]
            wl.k_cache[last, :, tail:, :] = nan
            wl.v_cache[last, :, tail:, :] = nan
    wl.k_cache[~used] = nan
    wl.v_cache[~used] = nan
    wl.meta["unused_blocks"] = int((~used).sum())


def make_workload(name: str, *, canaries: bool = False, pad_value: int = -1) -> Workload:
    """Build one named workload deterministically.

    canaries: fill unused pool blocks and the slots past L with NaN.
    pad_value: value of `block_tables` entries past ceil(L/bs); a non-negative
      value names a physical block (use it with canaries=True so that the
      block holds NaN if it is unused).
    """
    spec = WORKLOADS[name]
    i, S, Hq, Hkv, D, bs = (spec[k] for k in ("index", "S", "Hq", "Hkv", "D", "bs"))
    r_len, r_place, r_q, r_k, r_v = _rngs(i)
    seq_lens = _seq_lens(name, S, r_len)
    pages = [-(-int(L) // bs) for L in seq_lens]
    max_blocks = max(pages)
    sig_q, sig_k, sig_v = 1.0, 1.0, 1.0
    if name == "tiny_1x64":
        pool = 8
        bt = _place_pages(pages, pool, r_place, max_blocks, pad_value, take_prefix=True)
    elif name == "batch8_2k":
        pool = 1024
        bt = _place_pages(pages, pool, r_place, max_blocks, pad_value, take_prefix=True)
    elif name in ("long32_16k", "mixed64_32k"):
        pool = int(sum(pages))                # exact fit
        bt = _place_pages(pages, pool, r_place, max_blocks, pad_value, take_prefix=True)
        if name == "long32_16k":
            sig_k = 3.0                       # peaky softmax
    elif name == "long4_128k":
        pool = 2 * int(sum(pages))            # pages scattered in a 2x pool
        bt = _place_pages(pages, pool, r_place, max_blocks, pad_value, take_prefix=True)
        sig_q = sig_k = sig_v = 0.5
    else:
        raise KeyError(name)
    q = _draw_fp16(r_q, (S, Hq, D), sig_q)
    k = _draw_fp16(r_k, (pool, Hkv, bs, D), sig_k)
    v = _draw_fp16(r_v, (pool, Hkv, bs, D), sig_v)
    wl = Workload(name=name, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                  block_size=bs, seq_lens=seq_lens, block_tables=bt, num_blocks=pool,
                  q=q, k_cache=k, v_cache=v, scale=float(np.float32(1.0 / math.sqrt(D))),
                  partition_sizes=tuple(spec["parts"]))
    if canaries:
        _fill_canaries(wl)
    return wl


def make_custom(*, seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, seed: int, pool_factor: float = 1.0,
                sigma_q: float = 1.0, sigma_k: float = 1.0, sigma_v: float = 1.0,
                scale: float | None = None, canaries: bool = False, pad_value: int = -1,
                extra_blocks_per_seq: int = 0, name: str = "custom",
                dtype: str = "f16") -> Workload:
    """A seeded workload of any shape (for tests): pages shuffled in a pool of
    ceil(pool_factor * needed) blocks; `extra_blocks_per_seq` widens the page
    table beyond the longest sequence.  dtype: element type of q, K and V
    ("f16", "bf16" as uint16 bit patterns, "f32"); meta["dtype"] records it."""
    r_place, r_q, r_k, r_v = [np.random.Generator(np.random.PCG64(s))
                              for s in np.random.SeedSequence(seed).spawn(4)]
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    S = len(seq_lens)
    bs = block_size
    pages = [-(-int(L) // bs) for L in seq_lens]
    need = int(sum(pages))
    pool = max(1, int(math.ceil(pool_factor * need)))
    max_blocks = max(1, max(pages) + extra_blocks_per_seq)
    bt = _place_pages(pages, pool, r_place, max_blocks, pad_value, take_prefix=True)
    q = _draw(r_q, (S, num_q_heads, head_dim), sigma_q, dtype)
    k = _draw(r_k, (pool, num_kv_heads, bs, head_dim), sigma_k, dtype)
    v = _draw(r_v, (pool, num_kv_heads, bs, head_dim), sigma_v, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    wl = Workload(name=name, num_seqs=S, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                  head_dim=head_dim, block_size=bs, seq_lens=seq_lens, block_tables=bt,
                  num_blocks=pool, q=q, k_cache=k, v_cache=v, scale=float(np.float32(scale)))
    wl.meta["dtype"] = dtype
    if canaries:
        _fill_canaries(wl)
    return wl


def make_onehot_probe(base: Workload, seed: int, amplitude: float | None = None) -> tuple:
    """Page-table indexing probe built on `base`'s pool and page table.

    For every (s, kv head g) one target token t*_j per query head j of the
    group is drawn.  Query head j of the group is a*e_j; the target row has
    K[t*_j][j] = a and every other K element is 0, so the target's score
    exceeds every other score by a*a*scale.  V of every row encodes its own
    location in dims 0..3: (block mod 2048, block // 2048, slot, g), all exact
    in fp16; the other dims are 0.  Unused blocks and padding keep whatever
    `base` holds (NaN when built with canaries).

    Returns (workload, targets) where targets[s, h] is the logical target
    token of query head h.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S, Hq, Hkv, D, bs = (base.num_seqs, base.num_q_heads, base.num_kv_heads,
                         base.head_dim, base.block_size)
    G = Hq // Hkv
    if amplitude is None:
        amplitude = 40.0 if D <= 128 else 48.0
    a = np.float16(amplitude)
    q = np.zeros((S, Hq, D), dtype=np.float16)
    k = base.k_cache.copy()
    v = base.v_cache.copy()
    targets = np.zeros((S, Hq), dtype=np.int64)
    for s in range(S):
        L = int(base.seq_lens[s])
        n = -(-L // bs)
        ids = base.block_tables[s, :n].astype(np.int64)
        # zero K and write the location code into V for every valid token
        for g in range(Hkv):
            for p in range(n):
                blk = int(ids[p])
                valid = min(bs, L - p * bs)
                k[blk, g, :valid, :] = 0
                v[blk, g, :valid, :] = 0
                v[blk, g, :valid, 0] = np.float16(blk % 2048)
                v[blk, g, :valid, 1] = np.float16(blk // 2048)
                v[blk, g, :valid, 2] = np.arange(valid, dtype=np.float16)
                v[blk, g, :valid, 3] = np.float16(g)
            for j in range(G):
                h = g * G + j
                t = int(rng.integers(0, L))
                targets[s, h] = t
                q[s, h, j] = a
                blk = int(ids[t // bs])
                k[blk, g, t % bs, j] = a
    wl = Workload(name=base.name + "_probe", num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv,
                  head_dim=D, block_size=bs, seq_lens=base.seq_lens.copy(),
                  block_tables=base.block_tables.copy(), num_blocks=base.num_blocks,
                  q=q, k_cache=k, v_cache=v, scale=base.scale,
                  partition_sizes=base.partition_sizes)
    return wl, targets


# ----------------------------------------------------------------------------
# Several query tokens per sequence (speculative-decode verification, chunked
# prefill).  The cache holds L tokens per sequence, the last q_len of them the
# new ones; q is packed [total_q, Hq, D] with cu_q [S + 1] row offsets.
# ----------------------------------------------------------------------------
VARLEN_WORKLOADS = {
    # 32 seqs, (32q, 8kv, 128), bs 16, L uniform in [4096, 16384], 4 query
    # tokens each (3 drafted + 1).
    "verify32_q4": dict(index=6, S=32, Hq=32, Hkv=8, D=128, bs=16, L=(4096, 16384), q=(4, 4)),
    # 4 seqs, (24q, 4kv, 256), bs 32, a 1024-token chunk on a context uniform
    # in [1024, 8192] (L = context + 1024).
    "prefill4_chunk1k": dict(index=7, S=4, Hq=24, Hkv=4, D=256, bs=32, ctx=(1024, 8192), q=(1024, 1024)),
}


def varlen_pairs(seq_lens, q_lens) -> int:
    """(query, key) pairs of a causal varlen batch: sum over rows of the keys
    each query sees."""
    n = 0
    for L, ql in zip(seq_lens, q_lens):
        L, ql = int(L), int(ql)
        for j in range(ql):
            n += max(0, L - ql + j + 1)
    return n


def make_varlen_custom(*, seq_lens, q_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                       block_size: int, seed: int, pool_factor: float = 1.0,
                       sigma_q: float = 1.0, sigma_k: float = 1.0, sigma_v: float = 1.0,
                       canaries: bool = False, extra_blocks_per_seq: int = 0,
                       name: str = "varlen", dtype: str = "f16") -> Workload:
    """A seeded cache as make_custom builds it, with packed query rows: q is
    [sum q_lens, Hq, D]; meta holds cu_q (int32 [S + 1]) and q_lens.  dtype:
    "f16" or "bf16" (uint16 bit patterns), as for make_custom."""
    wl = make_custom(seq_lens=seq_lens, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                     head_dim=head_dim, block_size=block_size, seed=seed,
                     pool_factor=pool_factor, sigma_q=sigma_q, sigma_k=sigma_k, sigma_v=sigma_v,
                     canaries=canaries, extra_blocks_per_seq=extra_blocks_per_seq, name=name,
                     dtype=dtype)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    r_q = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(5)[4]))
    total = int(q_lens.sum())
    wl.q = _draw(r_q, (total, num_q_heads, head_dim), sigma_q, dtype)
    wl.meta["cu_q"] = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    wl.meta["q_lens"] = q_lens
    return wl


def make_varlen(name: str, *, canaries: bool = False, dtype: str = "f16") -> Workload:
    """Build one named variable-length workload deterministically (dtype:
    element type of q, K and V, "f16" or "bf16")."""
    spec = VARLEN_WORKLOADS[name]
    i, S = spec["index"], spec["S"]
    r_len = _rngs(i)[0]
    q_lens = r_len.integers(spec["q"][0], spec["q"][1], size=S, endpoint=True)
    if "L" in spec:
        lens = r_len.integers(spec["L"][0], spec["L"][1], size=S, endpoint=True)
    else:
        lens = r_len.integers(spec["ctx"][0], spec["ctx"][1], size=S, endpoint=True) + q_lens
    wl = make_varlen_custom(seq_lens=lens, q_lens=q_lens, num_q_heads=spec["Hq"],
                            num_kv_heads=spec["Hkv"], head_dim=spec["D"], block_size=spec["bs"],
                            seed=1000 + i, canaries=canaries, name=name, dtype=dtype)
    wl.partition_sizes = (-1,)
    return wl
