"""Host-side checks of libvkpaged that need no GPU: the library loads, exports
every function include/vk_paged.h declares, its planner agrees with the
oracle's planner rule, and argument validation rejects bad calls before any
HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from paged_gqa_kv_decode_amd import binding as vb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vk_paged.h")
CODES = {v: k for k, v in vb.STATUS_NAMES.items()}


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vk_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = vb.lib()
    names = declared_functions()
    assert set(names) == set(vb.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings():
    for code in range(9):
        assert vb.status_string(code)
    assert vb.status_string(99) == "unknown status"


def test_select_decode_kernel_roundtrip():
    prev = vb.select_decode_kernel(vb.KERNEL_DOT)
    assert vb.select_decode_kernel(prev) == vb.KERNEL_DOT
    with pytest.raises(ValueError):
        vb.select_decode_kernel(77)


def _c_plan(lens, Hq, Hkv, D, bs, mb, req, cu, per_cu=0, cap=0):
    try:
        p = vb.plan_partitions(lens, Hq, Hkv, D, bs, mb, req, cu, per_cu, cap)
        return dict(partition_size=p.partition_size, max_num_partitions=p.max_num_partitions,
                    work_full_parts=p.work_full_parts, budget=p.budget, cu_count=p.cu_count,
                    scratch_bytes=p.scratch_bytes)
    except vb.VkError as e:
        return e.name


def _o_plan(lens, Hq, Hkv, D, bs, mb, req, cu, per_cu=0, cap=0):
    try:
        return oracle.plan(lens, Hq, Hkv, D, bs, mb, req, cu, per_cu, cap, wave_slots_per_cu=8)
    except oracle.PlanError as e:
        return e.code


GEOMS = [(32, 8, 128), (24, 4, 256), (16, 2, 128), (16, 2, 256)]
# with the multi-head and multi-query triples (G = 1 and 16), where the
# default budget of 4 * G per CU and the 1024-first step differ most
ALL_GEOMS = GEOMS + [(16, 16, 128), (8, 8, 256), (16, 1, 128), (16, 1, 256)]


def test_planner_matches_oracle_rule_random():
    rng = np.random.default_rng(2024)
    for it in range(4000):
        Hq, Hkv, D = ALL_GEOMS[rng.integers(len(ALL_GEOMS))]
        bs = int(rng.choice([8, 16, 32]))
        S = int(rng.integers(1, 70))
        hi = int(rng.choice([300, 3000, 40000, 200000]))
        lens = rng.integers(1, hi, size=S).tolist()
        mb = -(-max(lens) // bs) + int(rng.integers(0, 3))
        req = int(rng.choice([-1, -1, -1, 0, 256, 512, 1024]))
        cu = int(rng.choice([1, 8, 80, 256, 304]))
        per_cu = int(rng.choice([0, 0, 1, 33, 64]))
        cap = int(rng.choice([0, 0, 1 << 20, 64 << 20]))
        if it % 50 == 0:
            lens[0] = 0 if it % 100 == 0 else mb * bs + 1       # invalid lengths
        a = _c_plan(lens, Hq, Hkv, D, bs, mb, req, cu, per_cu, cap)
        b = _o_plan(lens, Hq, Hkv, D, bs, mb, req, cu, per_cu, cap)
        assert a == b, (lens, Hq, Hkv, D, bs, mb, req, cu, per_cu, cap, a, b)


def test_planner_long_context_decisions():
    # 4 x 131072 tokens (16q, 2kv, 256), bs 32 on 256 CUs: W(512) = 16384 >=
    # the default budget 4 * G * 256 = 8192 -> 512; its 4 * 2 * 256 = 2048
    # workgroups would fill the 2048 wave slots (8 per CU) once with one wave
    # each, and 4 * 2 * 128 = 1024 workgroups of two waves over 1024-token
    # partitions fill them too -> 1024, W(1024) = 16 * 4 * 128.
    p = vb.plan_partitions([131072] * 4, 16, 2, 256, 32, 4096, -1, 256)
    assert (p.partition_size, p.max_num_partitions, p.work_full_parts, p.budget) == (1024, 128, 8192, 8192)
    # the default budget is 4 * G query-head units per CU: 4 workgroups per CU
    for (Hq, Hkv, D), bs in (((32, 8, 128), 16), ((24, 4, 256), 32), ((16, 1, 128), 16),
                             ((16, 16, 128), 16)):
        assert vb.plan_partitions([4096], Hq, Hkv, D, bs, 4096 // bs, -1, 80).budget == 4 * (Hq // Hkv) * 80
    # both sides of 4 workgroups per CU on 16 CUs, (32q, 8kv, 128): W(512) =
    # 32 * floor(L / 512) against 4 * 4 * 16 = 256, i.e. 8 full partitions
    # (512, and one round of 1024-token partitions: 32 workgroups <= 128 / 2 slots -> 1024)
    assert vb.plan_partitions([8 * 512], 32, 8, 128, 16, 256, -1, 16).partition_size == 1024
    assert vb.plan_partitions([8 * 512 - 1], 32, 8, 128, 16, 256, -1, 16).partition_size == 256
    # the pages' budget, 33 units per CU, on request
    assert vb.plan_partitions([8 * 512], 32, 8, 128, 16, 256, -1, 16, 33).partition_size == 256
    # 304 CUs (2432 slots): 2 * 2048 > 2432 and 2 * 1024 <= 2432 -> 1024
    assert vb.plan_partitions([131072] * 4, 16, 2, 256, 32, 4096, -1, 304).partition_size == 1024
    # 32 x 16k (24q, 4kv, 256): full 1024-token partitions 4 * 32 * 16 = 2048
    # workgroups >= 2 per CU (512) -> 1024 first (the default budget's rule)
    assert vb.plan_partitions([16384] * 32, 24, 4, 256, 32, 512, -1, 256).partition_size == 1024
    # under the pages' budget (33 per CU) the same batch takes 512: its 2048
    # two-wave 1024-token workgroups would not fit one round of 2048 slots
    assert vb.plan_partitions([16384] * 32, 24, 4, 256, 32, 512, -1, 256, 33).partition_size == 512
    # no full 1024-token partition, 300 * 4 = 1200 full 512-token ones
    # (>= 4 per CU) and 1024-token workgroups of two waves over 2048 slots -> 512
    assert vb.plan_partitions([1000] * 300, 24, 4, 256, 32, 32, -1, 256).partition_size == 512
    # both sides of 2 full 1024-token workgroups per CU (16 CUs, Hkv = 2):
    # 2 * floor(L / 1024) >= 32 <=> L >= 16 * 1024
    assert vb.plan_partitions([16 * 1024], 16, 2, 256, 32, 512, -1, 16).partition_size == 1024
    # (one token less: 2 * 15 = 30 < 32, and W(512) = 16 * 31 = 496 < 4 * 8 * 16 -> 256)
    assert vb.plan_partitions([16 * 1024 - 1], 16, 2, 256, 32, 512, -1, 16).partition_size == 256
    # multi-query 16 x 32768 (16q, 1kv, 256): W(512) = 16 * 16 * 64 >= 8448 ->
    # 512, whose 1024 workgroups would still get four waves each; 1024-token
    # partitions, 512 workgroups, fit the slots twice over -> 1024
    assert vb.plan_partitions([32768] * 16, 16, 1, 256, 32, 1024, -1, 256).partition_size == 1024
    # both sides of the regime on 1 CU (8 slots), budget 1 per CU, Hkv = 2:
    # 512 needs W(512) = 16 * floor(L / 512) >= 1, i.e. L >= 512, and 1024 then
    # needs 2 * 2 * ceil(L / 1024) <= 8, i.e. L <= 2048
    for L, P in ((511, 256), (512, 1024), (1024, 1024), (2048, 1024), (2049, 512)):
        assert vb.plan_partitions([L], 16, 2, 128, 16, 129, -1, 1, 1).partition_size == P, L
    # a forced 1024 is taken as it is
    p = vb.plan_partitions([5000, 3000], 32, 8, 128, 16, 313, 1024, 256)
    assert (p.partition_size, p.max_num_partitions) == (1024, 5)
    # 8 seqs up to 2048 tokens: too few full 512 partitions -> 256.
    p = vb.plan_partitions([2048, 1, 100, 1500, 2000, 512, 513, 7], 32, 8, 128, 16, 128, -1, 256)
    assert p.partition_size == 256 and p.max_num_partitions == 8
    assert vb.last_plan().partition_size == 256


@pytest.mark.parametrize("args,code", [
    (dict(geom=(32, 8, 64)), "GEOMETRY"),
    (dict(geom=(30, 8, 128)), "GEOMETRY"),
    (dict(geom=(0, 8, 128)), "BAD_DIM"),
    (dict(bs=4), "BLOCK_SIZE"),
    (dict(req=128), "PARTITION"),
    (dict(lens=[0]), "SEQ_LEN"),
    (dict(lens=[10 ** 6]), "SEQ_LEN"),
    (dict(cap=1000, req=512, lens=[5000] * 8), "SCRATCH_CAP"),
])
def test_planner_rejections(args, code):
    geom = args.get("geom", (32, 8, 128))
    lens = args.get("lens", [100, 200])
    got = _c_plan(lens, *geom, args.get("bs", 16), 1000, args.get("req", -1), 256, 0,
                  args.get("cap", 0))
    assert got == code


def test_planner_null_args():
    L = vb.lib()
    assert L.vk_plan_partitions(None, 1, 32, 8, 128, 16, 4, -1, 256, 0, 0, None) == CODES["NULL_ARG"]
    p = vb._Plan()
    assert L.vk_last_plan(None) == CODES["NULL_ARG"]
    assert L.vk_last_plan(ctypes.byref(p)) == 0


# ---- decode / reduce validation (fake device pointers; CPU tier only) -------
FAKE = 0x1000


def _decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=32, Hkv=8, D=128, bs=16, mb=8,
             nb=64, scale=0.088, P=512, NP=1, out=FAKE, ml=FAKE, es=FAKE, to=FAKE)
    a.update(kw)
    return vb.lib().vk_paged_gqa_decode(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["S"],
                                        a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"],
                                        a["scale"], a["P"], a["NP"], a["out"], a["ml"], a["es"],
                                        a["to"], None)


@pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation runs only without a GPU")
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), "NULL_ARG"), (dict(k=None), "NULL_ARG"), (dict(v=None), "NULL_ARG"),
    (dict(bt=None), "NULL_ARG"), (dict(sl=None), "NULL_ARG"),
    (dict(P=0, NP=1, out=None), "NULL_ARG"), (dict(P=512, ml=None), "NULL_ARG"),
    (dict(P=256, to=None), "NULL_ARG"), (dict(P=512, es=None), "NULL_ARG"),
    (dict(S=0), "BAD_DIM"), (dict(mb=0), "BAD_DIM"), (dict(nb=0), "BAD_DIM"),
    (dict(S=70000), "BAD_DIM"), (dict(scale=float("nan")), "BAD_DIM"),
    (dict(Hq=24, Hkv=8), "GEOMETRY"), (dict(Hq=16, Hkv=2, D=64), "GEOMETRY"),
    (dict(bs=64), "BLOCK_SIZE"), (dict(P=128), "PARTITION"), (dict(P=512, NP=0), "PARTITION"),
    (dict(P=0, NP=2), "PARTITION"), (dict(P=512, NP=5_000_000), "PARTITION"),
    (dict(mb=200_000_000), "BAD_DIM"), (dict(P=768), "PARTITION"),
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == CODES[code]


@pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation runs only without a GPU")
@pytest.mark.parametrize("kw", [dict(q=FAKE + 8), dict(k=FAKE + 4), dict(v=FAKE + 2),
                                dict(P=0, NP=1, out=FAKE + 4), dict(to=FAKE + 12),
                                dict(bt=FAKE + 2), dict(sl=FAKE + 1), dict(ml=FAKE + 2),
                                dict(es=FAKE + 3)])
def test_decode_rejects_misaligned_pointers(kw):
    """16-byte vectors for q, K, V, out and tmp_out; 4 bytes for the int32 and
    fp32 arrays: anything else is refused on the host."""
    assert _decode(**kw) == CODES["ALIGN"]
    # a 16-byte aligned address that is not 256-byte aligned is fine
    # (validation then stops at the first real check: none here, so the call
    # would launch; only check that alignment alone is not the reason)
    assert _decode(q=FAKE + 16, S=0) == CODES["BAD_DIM"]


@pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation runs only without a GPU")
def test_reduce_validation():
    R = vb.lib().vk_paged_gqa_reduce
    assert R(None, FAKE, FAKE, FAKE, 1, 32, 128, 512, 4, FAKE, None) == CODES["NULL_ARG"]
    assert R(FAKE, FAKE, FAKE, FAKE, 1, 32, 128, 512, 4, None, None) == CODES["NULL_ARG"]
    assert R(FAKE, FAKE, FAKE, FAKE, 0, 32, 128, 512, 4, FAKE, None) == CODES["BAD_DIM"]
    assert R(FAKE, FAKE, FAKE, FAKE, 1, 32, 96, 512, 4, FAKE, None) == CODES["GEOMETRY"]
    assert R(FAKE, FAKE, FAKE, FAKE, 1, 32, 128, 0, 4, FAKE, None) == CODES["PARTITION"]
    assert R(FAKE, FAKE, FAKE, FAKE, 1, 32, 128, 512, 0, FAKE, None) == CODES["PARTITION"]
    assert R(FAKE, FAKE, FAKE, FAKE, 1, 32, 128, 768, 4, FAKE, None) == CODES["PARTITION"]
    assert R(FAKE, FAKE, FAKE + 4, FAKE, 1, 32, 128, 512, 4, FAKE, None) == CODES["ALIGN"]
    assert R(FAKE, FAKE, FAKE, FAKE, 1, 32, 128, 512, 4, FAKE + 8, None) == CODES["ALIGN"]
    assert R(FAKE + 2, FAKE, FAKE, FAKE, 1, 32, 128, 512, 4, FAKE, None) == CODES["ALIGN"]


def _noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, S=2, Hq=32, Hkv=8, D=128, bs=16, mb=8,
             nb=64, scale=0.088, P=512, NP=1, out=FAKE)
    a.update(kw)
    return vb.lib().vk_paged_gqa_decode_noalloc(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["S"],
                                                a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"],
                                                a["nb"], a["scale"], a["P"], a["NP"], a["out"],
                                                None)


NOALLOC_BYTES = 64 << 20   # VK_NOALLOC_SCRATCH_BYTES


def _noalloc_need(S, Hq, D, NP):
    rows = S * Hq * NP
    vec = (rows * 4 + 255) // 256 * 256
    return 2 * vec + rows * D * 4


@pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation runs only without a GPU")
@pytest.mark.parametrize("kw,code", [
    (dict(out=None), "NULL_ARG"), (dict(P=0, NP=1, out=None), "NULL_ARG"),
    (dict(S=0), "BAD_DIM"), (dict(S=70000), "BAD_DIM"),
    (dict(Hq=24, Hkv=8), "GEOMETRY"), (dict(P=128), "PARTITION"), (dict(NP=0), "PARTITION"),
    (dict(NP=5_000_000), "PARTITION"),
    # partials over the library's 64 MiB array: 2 x 32 x 3000 x 130 x 4 bytes = 99.8 MB
    (dict(NP=3000), "SCRATCH_CAP"),
    (dict(S=32, Hq=24, Hkv=4, D=256, bs=32, P=256, NP=100), "SCRATCH_CAP"),
    # unsplit: the decode's own checks
    (dict(P=0, NP=2), "PARTITION"), (dict(P=0, NP=1, q=None), "NULL_ARG"),
])
def test_noalloc_validation(kw, code):
    """The no-allocation entry point refuses, on the host, what the decode
    refuses and any split call whose partials exceed its array."""
    assert _noalloc(**kw) == CODES[code]


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_noalloc_cap_boundary():
    """The largest partition count whose partials fit passes the size check
    (and then fails only at the device lookup, there being no GPU here); one
    more is refused."""
    S, Hq, D = 2, 32, 128
    np_fit = max(n for n in range(1, 5000) if _noalloc_need(S, Hq, D, n) <= NOALLOC_BYTES)
    assert _noalloc_need(S, Hq, D, np_fit + 1) > NOALLOC_BYTES
    assert _noalloc(S=S, Hq=Hq, D=D, NP=np_fit + 1) == CODES["SCRATCH_CAP"]
    assert _noalloc(S=S, Hq=Hq, D=D, NP=np_fit) == CODES["HIP"]
    # every named long-context workload's partials fit: (S, Hq, D, P, max L)
    for S_, Hq_, D_, P_, Lmax in ((32, 24, 256, 256, 16384), (64, 16, 128, 512, 32768),
                                   (4, 16, 256, 512, 131072), (8, 32, 128, 512, 2048)):
        assert _noalloc_need(S_, Hq_, D_, -(-Lmax // P_)) <= NOALLOC_BYTES


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine without a GPU")
def test_planner_device_query_without_gpu_is_hip_error():
    code = _c_plan([100], 32, 8, 128, 16, 8, -1, 0)
    assert code == "HIP"


# ----------------------------------------------------------------------------
# vk_plan_varlen: hand-computed decisions (host only; cu_count given).
# ----------------------------------------------------------------------------
@pytest.fixture
def columns():
    prev = vb.select_varlen_kernel(vb.KERNEL_VARLEN_COLUMNS)
    yield
    vb.select_varlen_kernel(prev)


def _pv(lens, qlens, geom, bs=16, P=-1, cu=256, cap=0, mb=None):
    Hq, Hkv, D = geom
    mb = mb or max(-(-L // bs) for L in lens)
    return vb.plan_varlen(lens, qlens, Hq, Hkv, D, bs, mb, P, cu, cap)


def test_plan_varlen_split_small_work(columns):
    # G = 4: 4 query tokens per tile; tiles 1 + 1, units 8 * 2 = 16 < 8 * 4.
    # Full-512 work 32 * (1 + 1) = 64 < 33 * 4 -> 256; NP = ceil(1000 / 256) = 4.
    p = _pv([1000, 600], [4, 1], (32, 8, 128), cu=4)
    assert (p.partition_size, p.max_num_partitions) == (256, 4)
    assert p.scratch_bytes == 5 * 32 * 4 * 130 * 4
    assert p.budget == 33 * 4


def test_plan_varlen_unsplit_when_tiles_fill_the_slots(columns):
    # G = 8: 2 tokens per tile; tiles 4 + 4 + 2 = 10, units 2 * 10 = 20 >= 8 * 1.
    p = _pv([100, 100, 100], [8, 8, 4], (16, 2, 128), cu=1)
    assert (p.partition_size, p.max_num_partitions, p.scratch_bytes) == (0, 1, 0)
    assert p.work_full_parts == 20


def test_plan_varlen_large_partition_at_the_budget(columns):
    # G = 8, tiles 1 + 1 -> units 4 < 8.  Two query tokens: full-1024 units
    # 16 * (8 + 4) = 192 >= 33 -> 1024.
    p = _pv([8192, 4096], [2, 2], (16, 2, 256), bs=32, cu=1)
    assert (p.partition_size, p.max_num_partitions) == (1024, 8)
    # 16 * (1 + 1) = 32 < 33 -> 256
    p = _pv([1023, 600], [2, 2], (16, 2, 256), bs=32, cu=1)
    assert (p.partition_size, p.max_num_partitions) == (256, 4)
    # both sides of W(512) = budget: 16 CUs, budget 528 = 16 heads * 33 full partitions
    p = _pv([33 * 512], [2], (16, 2, 256), bs=32, cu=16)
    assert (p.partition_size, p.work_full_parts, p.budget) == (512, 528, 528)
    p = _pv([33 * 512 - 1], [2], (16, 2, 256), bs=32, cu=16)
    assert (p.partition_size, p.work_full_parts) == (256, 16 * 65)
    # one query token per sequence: the decode planner's choice, except its
    # one-round upgrade to 1024 (two waves per partition, which the one-wave
    # column kernel does not have): there 512
    for lens in ([8192, 4096], [1023, 600], [33 * 512], [33 * 512 - 1]):
        for cu in (1, 16):
            a = _pv(lens, [1] * len(lens), (16, 2, 256), bs=32, cu=cu)
            # (the multi-token planner keeps the pages' budget of 33 per CU)
            d = vb.plan_partitions(np.array(lens, dtype=np.int32), 16, 2, 256, 32, 600, -1, cu, 33)
            if d.partition_size == 1024:
                assert (a.partition_size, a.work_full_parts) == (512, 16 * sum(L // 512 for L in lens))
            else:
                assert (a.partition_size, a.work_full_parts) == (d.partition_size, d.work_full_parts)
    # 16 * (4 + 2) = 96 full 1024-token units >= 33
    p = _pv([4096, 2048], [2, 2], (16, 2, 256), bs=32, cu=1)
    assert (p.partition_size, p.max_num_partitions) == (1024, 4)
    # forced sizes and unsplit
    assert _pv([4096, 2048], [2, 2], (16, 2, 256), bs=32, P=512, cu=1).max_num_partitions == 8
    assert _pv([4096, 2048], [2, 2], (16, 2, 256), bs=32, P=0, cu=1).partition_size == 0


def test_plan_varlen_xlarge_partition_rule(columns):
    # Column tiles with several query tokens try 1024 first, under the same
    # budget rule: both sides of W(1024) = budget (16 CUs: 528 = 16 heads x
    # 33 full 1024-token partitions).
    p = _pv([33 * 1024], [2], (16, 2, 256), bs=32, cu=16)
    assert (p.partition_size, p.work_full_parts, p.max_num_partitions) == (1024, 528, 33)
    assert p.scratch_bytes == 2 * 16 * 33 * 258 * 4
    p = _pv([33 * 1024 - 1], [2], (16, 2, 256), bs=32, cu=16)
    assert (p.partition_size, p.work_full_parts) == (512, 16 * 65)
    # one query token per sequence: the decode planner's sizes only
    p = _pv([33 * 1024], [1], (16, 2, 256), bs=32, cu=16)
    # (against the decode planner under the same, pages' budget of 33 per CU)
    d = vb.plan_partitions(np.array([33 * 1024], dtype=np.int32), 16, 2, 256, 32, 1100, -1, 16, 33)
    assert p.partition_size == d.partition_size == 512
    # the verification shape: 32 x 4 tokens (32, 8, 128) on 4k-16k contexts
    lens = [4096 + 384 * k for k in range(32)]
    p = _pv(lens, [4] * 32, (32, 8, 128), cu=256)
    full1024 = sum(L // 1024 for L in lens)
    assert 32 * full1024 >= 33 * 256 and p.partition_size == 1024
    assert p.max_num_partitions == -(-max(lens) // 1024)
    # forced 1024, and its scratch
    p = _pv([5000, 3000], [4, 4], (32, 8, 128), P=1024, cu=4)
    assert (p.partition_size, p.max_num_partitions) == (1024, 5)
    assert p.scratch_bytes == 8 * 32 * 5 * 130 * 4
    # 3 CUs (budget 99): full-1024 units 32 * 2 = 64 < 99, full-512 units
    # 32 * 4 = 128 >= 99 -> 512; with the cap one byte under its scratch
    # (8 rows x 32 heads x 3 partitions) the next size up, 1024, before unsplit
    assert _pv([1500, 1500], [4, 4], (32, 8, 128), cu=3).partition_size == 512
    p = _pv([1500, 1500], [4, 4], (32, 8, 128), cu=3, cap=8 * 32 * 3 * 130 * 4 - 1)
    assert (p.partition_size, p.max_num_partitions) == (1024, 2)
    p = _pv([1500, 1500], [4, 4], (32, 8, 128), cu=3, cap=8 * 32 * 2 * 130 * 4 - 1)
    assert p.partition_size == 0
    # the decode planner takes 1024 only when asked, or in its one-round regime
    assert vb.plan_partitions(np.array([4096], dtype=np.int32), 32, 8, 128, 16, 256, 1024, 4).partition_size == 1024


@pytest.mark.parametrize("lens,qlens,name", [([100, 50], [101, 1], "SEQ_LEN"),
                                             ([100, 50], [-1, 1], "SEQ_LEN"),
                                             ([0, 50], [0, 1], "SEQ_LEN")])
def test_plan_varlen_rejects(lens, qlens, name):
    with pytest.raises(vb.VkError) as e:
        _pv(lens, qlens, (32, 8, 128), cu=4)
    assert e.value.name == name


def test_plan_varlen_scratch_cap():
    with pytest.raises(vb.VkError) as e:
        _pv([4096], [4], (32, 8, 128), P=256, cu=4, cap=1000)
    assert e.value.name == "SCRATCH_CAP"


@pytest.mark.parametrize("geom,fits", [((32, 8, 128), 4), ((24, 4, 256), 2), ((16, 2, 128), 2),
                                       ((16, 2, 256), 2), ((16, 16, 128), 16), ((16, 1, 128), 1)])
def test_plan_varlen_kernel_choice_rule(geom, fits):
    # The longest query run decides: while it fits one 16-column tile of the
    # column kernel (16 / G tokens) -> columns, above -> LDS tiles.
    C, T = vb.KERNEL_VARLEN_COLUMNS, vb.KERNEL_VARLEN_TILES
    assert _pv([2000, 1500], [fits, 1], geom, cu=4).kernel == C
    assert _pv([2000, 1500], [1, fits], geom, cu=4).kernel == C
    assert _pv([2000, 1500], [fits + 1, 1], geom, cu=4).kernel == T


def test_plan_varlen_kernel_choice():
    assert _pv([2000, 1500], [3, 1], (32, 8, 128), cu=4).kernel == vb.KERNEL_VARLEN_COLUMNS
    assert _pv([2000, 1500], [5, 1], (32, 8, 128), cu=4).kernel == vb.KERNEL_VARLEN_TILES
    prev = vb.select_varlen_kernel(vb.KERNEL_VARLEN_COLUMNS)
    try:
        assert _pv([2000, 1500], [100, 1], (32, 8, 128), cu=4).kernel == vb.KERNEL_VARLEN_COLUMNS
        vb.select_varlen_kernel(vb.KERNEL_VARLEN_TILES)
        assert _pv([2000, 1500], [2, 1], (32, 8, 128), cu=4).kernel == vb.KERNEL_VARLEN_TILES
    finally:
        assert vb.select_varlen_kernel(prev) == vb.KERNEL_VARLEN_TILES
    with pytest.raises(ValueError):
        vb.select_varlen_kernel(vb.KERNEL_MFMA_W1)


def test_plan_varlen_tiles_split_rule():
    # G = 4: 128 / 4 = 32 tokens per tile; tiles 4 + 2 = 6, n = 8 * 6 = 48
    # (KV head, tile) workgroups of 4 waves = 192 waves.
    p = _pv([2000, 1500], [100, 64], (32, 8, 128), cu=24)          # 192 >= 8 * 24
    assert (p.partition_size, p.max_num_partitions, p.scratch_bytes) == (0, 1, 0)
    assert p.work_full_parts == 48
    # 192 < 8 * 25 -> split; full-512 units 8 * (4 * 3 + 2 * 2) = 128 < 33 * 25 -> 256
    p = _pv([2000, 1500], [100, 64], (32, 8, 128), cu=25)
    assert (p.partition_size, p.max_num_partitions) == (256, 8)
    assert p.scratch_bytes == 164 * 32 * 8 * 130 * 4
    # one 16k sequence, 64 query tokens: 2 tiles, 64 waves < 8 * 10 -> split;
    # full-512 units 8 * 2 * 32 = 512 >= 33 * 10 -> 512; LDS tiles never
    # take 1024
    p = _pv([16384], [64], (32, 8, 128), cu=10)
    assert (p.partition_size, p.max_num_partitions) == (512, 32)
    # a 64k context: full-1024 units 32 * 2 * 64 = 4096 >= 330, yet 512
    p = _pv([65536], [64], (32, 8, 128), cu=10)
    assert p.kernel == vb.KERNEL_VARLEN_TILES
    assert (p.partition_size, p.max_num_partitions) == (512, 128)
    # G = 6, D = 256: a tile is 128 consecutive (token, head) columns, so
    # 1024 query tokens are 1024 * 6 / 128 = 48 tiles (whole tokens per tile
    # would need 49); 4 chunks -> 4 * 4 * 48 = 768 workgroups, 6144 waves
    # >= 8 * 256: the chunked-prefill shape runs unsplit.
    p = _pv([3000, 5000, 8000, 2048], [1024] * 4, (24, 4, 256), bs=32, cu=256)
    assert (p.kernel, p.partition_size, p.work_full_parts) == (vb.KERNEL_VARLEN_TILES, 0, 768)
    # tile counts at G = 6: ceil(q_len * 6 / 128) per sequence, times Hkv = 4
    for ql, tiles in ((22, 2), (64, 3), (65, 4), (128, 6), (129, 7)):
        p = _pv([5000], [ql], (24, 4, 256), bs=32, cu=1)
        assert (p.kernel, p.partition_size, p.work_full_parts) == (vb.KERNEL_VARLEN_TILES, 0, 4 * tiles)


def test_plan_varlen_auto_falls_back_under_the_scratch_cap():
    # 32 sequences x 32 query tokens of (32, 8, 128) on 16k contexts: one tile
    # per sequence, 4 * 8 * 32 = 1024 waves < 8 * 256 -> split; at 256 the
    # partials need 1024 * 32 * 64 * 130 * 4 = 1.09 GB > 512 MiB, at 512
    # 545 MB > 512 MiB -> unsplit.  An explicit 256 is refused.
    lens, ql = [16384] * 32, [32] * 32
    p = _pv(lens, ql, (32, 8, 128), cu=256)
    assert (p.kernel, p.partition_size, p.scratch_bytes) == (vb.KERNEL_VARLEN_TILES, 0, 0)
    with pytest.raises(vb.VkError) as e:
        _pv(lens, ql, (32, 8, 128), P=256, cu=256)
    assert e.value.name == "SCRATCH_CAP"
    # with a larger cap the rule's own choice stands
    p = _pv(lens, ql, (32, 8, 128), cu=256, cap=2 << 30)
    assert p.partition_size in (256, 512)


def _varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, S=2, T=8, mq=4, Hq=32, Hkv=8,
             D=128, bs=16, mb=8, nb=64, scale=0.088, P=256, NP=2, out=FAKE, ml=FAKE, es=FAKE,
             to=FAKE)
    a.update(kw)
    return vb.lib().vk_paged_gqa_varlen(a["q"], a["k"], a["v"], a["bt"], a["sl"], a["cu"], a["S"],
                                        a["T"], a["mq"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                        a["mb"], a["nb"], a["scale"], a["P"], a["NP"], a["out"],
                                        a["ml"], a["es"], a["to"], None)


@pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation runs only without a GPU")
@pytest.mark.parametrize("kw", [dict(q=FAKE + 8), dict(k=FAKE + 4), dict(v=FAKE + 2),
                                dict(to=FAKE + 12), dict(P=0, NP=1, out=FAKE + 4),
                                dict(cu=FAKE + 2), dict(bt=FAKE + 1), dict(ml=FAKE + 2)])
def test_varlen_rejects_misaligned_pointers(kw):
    assert _varlen(**kw) == CODES["ALIGN"]
    assert _varlen(q=FAKE + 16, S=0) == CODES["BAD_DIM"]


@pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation runs only without a GPU")
def test_varlen_reduce_rejects_misaligned_pointers():
    R = vb.lib().vk_paged_gqa_varlen_reduce
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 32, 128, 256, 2, FAKE, None)
    for pos, off in [(2, 4), (11, 8), (0, 2), (4, 1)]:
        args = list(ok)
        args[pos] = FAKE + off
        assert R(*args) == CODES["ALIGN"], (pos, off)


def test_varlen_dt_rejects_other_element_types():
    """fp32 (and unknown) element types are refused on the host, before any
    pointer is looked at or any HIP call is made."""
    L = vb.lib()
    for dtype in (vb.DTYPE_F32, 7, -1):
        code = L.vk_paged_gqa_varlen_dt(dtype, None, None, None, None, None, None, 1, 1, 1, 32, 8,
                                        128, 16, 1, 1, 1.0, 0, 1, None, None, None, None, None)
        assert vb.STATUS_NAMES[code] == "DTYPE"


def test_trace_switch_loads_roctx():
    """VK_TRACE=1 turns on roctx ranges around the entry points that enqueue
    work (a roctx library loaded at the first call); unset or "0", tracing is off.
    A traced call still validates and returns as usual (checked on a call
    refused on the host)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from paged_gqa_kv_decode_amd import binding as vb\n"
            "L = vb.lib()\n"
            "r = L.vk_paged_gqa_reduce(None, None, None, None, 1, 32, 128, 512, 4, None, None)\n"
            "print(L.vk_trace_enabled(), r)\n") % ROOT
    outs = {}
    for val in ("1", "0", None):
        env = {k: v for k, v in os.environ.items() if k != "VK_TRACE"}
        if val is not None:
            env["VK_TRACE"] = val
        p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=120)
        assert p.returncode == 0, p.stderr
        outs[val] = p.stdout.split()
    null_arg = str(CODES["NULL_ARG"])
    assert outs["1"] == ["1", null_arg]
    assert outs["0"] == ["0", null_arg] and outs[None] == ["0", null_arg]
