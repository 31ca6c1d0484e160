"""GPU parity of the HIP path (through the C ABI) against the float64 oracle,
plus bit-exact indexing, invariants, canaries and edge cases.

Tolerance of fp32 outputs against the oracle: max |gpu - ref| <= 2e-3 and,
per (sequence, head) row, ||gpu - ref||_2 / ||ref||_2 <= 1e-2.  Page-table
indexing (the one-hot probe), L = 1 rows, page permutation, V scaling by 2,
repeated runs and canaries are bit-exact.
"""
import numpy as np
import pytest

from gpu_helpers import assert_parity, named, oracle_ref, run_hip, say, to_device
from paged_gqa_kv_decode_amd import binding as vb
from paged_gqa_kv_decode_amd.workloads import make_custom, make_onehot_probe

pytestmark = pytest.mark.gpu

KERNELS = [vb.KERNEL_DOT, vb.KERNEL_MFMA_W1, vb.KERNEL_MFMA_W2, vb.KERNEL_MFMA_W4,
           vb.KERNEL_MFMA_W4P2]
FAMILIES = [vb.KERNEL_DOT, vb.KERNEL_MFMA]

NAMED = [("tiny_1x64", 0), ("batch8_2k", 512), ("long32_16k", 256), ("long32_16k", 512),
         ("mixed64_32k", 512), ("long4_128k", -1)]

_probes = {}


def _probe(name, seed):
    key = (name, seed)
    if key not in _probes:
        if len(_probes) >= 2:
            _probes.pop(next(iter(_probes)))
        _probes[key] = make_onehot_probe(named(name, canaries=True), seed=seed)
    return _probes[key]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name,P", NAMED, ids=[f"{n}-P{p}" for n, p in NAMED])
def test_named_workload_parity(orc, name, P, kernel):
    say(f"[parity] {name} P={P} kernel={kernel}")
    wl = named(name)
    ref = oracle_ref(orc, name)
    gpu, plan, last, _ = run_hip(wl, P, kernel=kernel)
    if P == -1:   # one round of two-wave 1024-token partitions on 256 CUs
        assert plan.partition_size == 1024, "planner should pick 1024 for 4 x 131072 tokens"
    if kernel == vb.KERNEL_MFMA_W4P2 and plan.partition_size == 0:
        assert last.kernel == vb.KERNEL_MFMA_W4    # two partitions per workgroup need a split
    else:
        assert last.kernel == kernel
    assert_parity(gpu, ref, f"{name} P={plan.partition_size}")


@pytest.mark.parametrize("kernel", [vb.KERNEL_DOT, vb.KERNEL_MFMA_W1, vb.KERNEL_MFMA_W4,
                                    vb.KERNEL_MFMA_W4P2])
@pytest.mark.parametrize("name,P", [("batch8_2k", 512), ("mixed64_32k", 512), ("long32_16k", 256),
                                    ("batch8_2k", 1024), ("mixed64_32k", 1024)])
def test_partials_match_oracle(orc, name, P, kernel):
    say(f"[partials] {name} P={P} kernel={kernel}")
    wl = named(name)
    _, plan, _, (m, l, o) = run_hip(wl, P, keep_partials=True, kernel=kernel)
    NP = plan.max_num_partitions
    om, ol, oo = orc.partials(wl, P, NP)
    for s, L in enumerate(wl.seq_lens):
        n = -(-int(L) // P)
        assert np.all(np.isnan(m[s, :, n:])), "decode wrote past the last partition"
        assert np.all(np.isnan(o[s, :, n:])), "decode wrote past the last partition"
        assert np.all(np.isfinite(m[s, :, :n])) and np.all(np.isfinite(o[s, :, :n]))
        dm = np.max(np.abs(m[s, :, :n] - om[s, :, :n]))
        assert dm <= 1e-3, f"max_logits off by {dm}"
        rl = np.max(np.abs(l[s, :, :n] / ol[s, :, :n] - 1))
        assert rl <= 1e-3, f"exp_sums rel err {rl}"
    valid = np.isfinite(om)
    assert_parity(o[valid], oo[valid], f"{name} tmp_out")


@pytest.mark.parametrize("name,P", [("tiny_1x64", 0), ("batch8_2k", 512), ("batch8_2k", 0),
                                    ("long32_16k", 256), ("mixed64_32k", 512),
                                    ("long4_128k", 512), ("long4_128k", 0)])
@pytest.mark.parametrize("kernel", FAMILIES)
def test_onehot_probe_bit_exact(name, P, kernel):
    """Page-table indexing: every output decodes to exactly the (block, slot,
    KV head) the page table names for the target token."""
    say(f"[probe] {name} P={P} kernel={kernel}")
    wl, targets = _probe(name, 7 + P)
    gpu, _, _, _ = run_hip(wl, P, kernel=kernel)
    bs, G = wl.block_size, wl.group
    for s in range(wl.num_seqs):
        t = targets[s]
        blk = wl.block_tables[s, t // bs].astype(np.int64)
        want = np.stack([blk % 2048, blk // 2048, t % bs, np.arange(wl.num_q_heads) // G], 1)
        got = gpu[s, :, :4]
        assert np.array_equal(got, want.astype(np.float64)), f"seq {s}: {got} != {want}"
        assert np.all(gpu[s, :, 4:] == 0.0)


@pytest.mark.parametrize("kernel", [vb.KERNEL_DOT, vb.KERNEL_MFMA])
def test_single_token_rows_bit_exact(kernel):
    wl = named("mixed64_32k")
    gpu, _, _, _ = run_hip(wl, 512, kernel=kernel)
    ones = np.nonzero(wl.seq_lens == 1)[0]
    assert len(ones) == 16
    for s in ones:
        blk = wl.block_tables[s, 0]
        for h in range(wl.num_q_heads):
            v0 = wl.v_cache[blk, h // wl.group, 0].astype(np.float32).astype(np.float64)
            assert np.array_equal(gpu[s, h], v0)


@pytest.mark.parametrize("kernel", [vb.KERNEL_DOT, vb.KERNEL_MFMA])
@pytest.mark.parametrize("name,P", [("batch8_2k", 512), ("mixed64_32k", 512)])
def test_page_permutation_bit_identical(name, P, kernel):
    wl = named(name)
    base, _, _, _ = run_hip(wl, P, kernel=kernel)
    rng = np.random.default_rng(99)
    perm = rng.permutation(wl.num_blocks)
    import copy
    w2 = copy.copy(wl)
    w2.k_cache = np.empty_like(wl.k_cache)
    w2.v_cache = np.empty_like(wl.v_cache)
    w2.k_cache[perm] = wl.k_cache
    w2.v_cache[perm] = wl.v_cache
    bt = wl.block_tables.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    w2.block_tables = bt
    out, _, _, _ = run_hip(w2, P, kernel=kernel)
    assert np.array_equal(out, base)


@pytest.mark.parametrize("kernel", FAMILIES)
@pytest.mark.parametrize("name,Pa,Pb", [("batch8_2k", 0, 512), ("long32_16k", 256, 512),
                                        ("batch8_2k", 256, 512)])
def test_split_vs_unsplit(name, Pa, Pb, kernel):
    wl = named(name)
    a, _, _, _ = run_hip(wl, Pa, kernel=kernel)
    b, _, _, _ = run_hip(wl, Pb, kernel=kernel)
    assert_parity(a, b, f"{name} P={Pa} vs P={Pb}")


@pytest.mark.parametrize("kernel", [vb.KERNEL_DOT, vb.KERNEL_MFMA])
def test_v_scaled_by_two_is_exact(kernel):
    import copy
    wl = named("batch8_2k")
    base, _, _, _ = run_hip(wl, 512, kernel=kernel)
    w2 = copy.copy(wl)
    w2.v_cache = (wl.v_cache.astype(np.float32) * 2).astype(np.float16)
    out, _, _, _ = run_hip(w2, 512, kernel=kernel)
    assert np.array_equal(out, 2 * base)


@pytest.mark.parametrize("kernel", [vb.KERNEL_DOT, vb.KERNEL_MFMA])
@pytest.mark.parametrize("name,P", [("batch8_2k", 512), ("mixed64_32k", 512)])
def test_repeat_runs_bit_identical(name, P, kernel):
    wl = named(name)
    dev = to_device(wl)
    a, _, _, _ = run_hip(wl, P, dev=dev, kernel=kernel)
    b, _, _, _ = run_hip(wl, P, dev=dev, kernel=kernel)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,P", [("batch8_2k", 512), ("tiny_1x64", 0), ("long4_128k", 512),
                                    ("mixed64_32k", 512)])
@pytest.mark.parametrize("pad", ["minus1", "block"])
@pytest.mark.parametrize("kernel", FAMILIES)
def test_canaries_never_read(name, P, pad, kernel):
    """NaN in unused blocks and in the slots past L; padding entries of the
    page table -1 or the id of a block that is unused (NaN) where one exists.
    The output must be bit-identical to the run without canaries."""
    say(f"[canary] {name} P={P} pad={pad}")
    plain = named(name)
    base, _, _, _ = run_hip(plain, P, kernel=kernel)
    pad_value = -1
    if pad == "block":
        used = np.zeros(plain.num_blocks, bool)
        for s, L in enumerate(plain.seq_lens):
            used[plain.block_tables[s, :-(-int(L) // plain.block_size)]] = True
        unused = np.nonzero(~used)[0]
        pad_value = int(unused[0]) if len(unused) else 0
    wl = named(name, canaries=True, pad_value=pad_value)
    out, _, _, _ = run_hip(wl, P, prefill_nan=True, kernel=kernel)
    assert np.all(np.isfinite(out)), "a canary leaked into the output"
    assert np.array_equal(out, base)


def test_uniform_keys_mean_of_v(orc):
    import copy
    wl = copy.copy(named("batch8_2k"))
    wl.q = np.zeros_like(wl.q)
    ref = orc.paged_attention(wl)
    gpu, _, _, _ = run_hip(wl, 512)
    assert_parity(gpu, ref, "q = 0")


def test_reduce_synthetic_closed_forms():
    import torch
    S, Hq, NP, D, P = 2, 16, 5, 256, 512
    rng = np.random.default_rng(3)
    o = torch.from_numpy(rng.standard_normal((S, Hq, NP, D)).astype(np.float32)).cuda()
    m = torch.full((S, Hq, NP), 3.0, device="cuda")
    l = torch.full((S, Hq, NP), 4.0, device="cuda")
    sl = torch.tensor([NP * P, NP * P - 7], dtype=torch.int32, device="cuda")
    out = torch.empty((S, Hq, D), device="cuda")
    vb.paged_gqa_reduce(m, l, o, sl, P, out)
    torch.cuda.synchronize()
    ref = o.double().mean(dim=2)
    assert torch.max(torch.abs(out.double() - ref)).item() <= 1e-6
    m2 = m.clone()
    m2[:, :, 2] += 200.0
    vb.paged_gqa_reduce(m2, l, o, sl, P, out)
    torch.cuda.synchronize()
    assert torch.equal(out, o[:, :, 2, :])
    # one partition: copied exactly; L <= 0: zeros
    sl1 = torch.tensor([P, -5], dtype=torch.int32, device="cuda")
    vb.paged_gqa_reduce(m, l, o, sl1, P, out)
    torch.cuda.synchronize()
    assert torch.equal(out[0], o[0, :, 0, :])
    assert torch.equal(out[1], torch.zeros_like(out[1]))


SWEEP = [((32, 8, 128), 8), ((32, 8, 128), 16), ((32, 8, 128), 32),
         ((24, 4, 256), 8), ((24, 4, 256), 16), ((24, 4, 256), 32),
         ((16, 2, 128), 8), ((16, 2, 128), 16), ((16, 2, 128), 32),
         ((16, 2, 256), 8), ((16, 2, 256), 16), ((16, 2, 256), 32)]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("geom,bs", SWEEP, ids=[f"{g[0]}-{g[1]}-{g[2]}-bs{b}" for g, b in SWEEP])
def test_all_specialisations_ragged(orc, geom, bs, kernel):
    """Every (geometry, page size) instance, lengths around page, step and
    partition boundaries, split (256 and 512) and unsplit, canaries on."""
    Hq, Hkv, D = geom
    lens = [1, bs - 1, bs, bs + 1, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1025, 1537, 2100]
    wl = make_custom(seq_lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                     seed=Hq * 1000 + D + bs, pool_factor=1.7, canaries=True,
                     extra_blocks_per_seq=2, sigma_k=2.0)
    ref = orc.paged_attention(wl)
    for P in (0, 256, 512):
        gpu, _, _, _ = run_hip(wl, P, kernel=kernel)
        assert_parity(gpu, ref, f"{geom} bs{bs} P{P}")


@pytest.mark.parametrize("order", [vb.ORDER_GRID, vb.ORDER_LONGEST_FIRST])
@pytest.mark.parametrize("kernel", [vb.KERNEL_DOT, vb.KERNEL_MFMA_W1, vb.KERNEL_MFMA_W4,
                                    vb.KERNEL_MFMA_W4P2])
@pytest.mark.parametrize("head_dim", [128, 256])
def test_device_side_guards(kernel, head_dim, order):
    """Values the host cannot validate: a length <= 0 gives zeros; a page id
    outside the pool or a length beyond the page table gives NaN for that
    sequence only, without reading out of bounds."""
    import torch
    wl = make_custom(seq_lens=[40, 40, 40, 40], num_q_heads=16, num_kv_heads=2,
                     head_dim=head_dim,
                     block_size=16, seed=5, pool_factor=2.0)
    q, k, v, bt, sl = to_device(wl)
    sl_dev = torch.tensor([40, 0, 40, 40 + 16 * 10], dtype=torch.int32, device="cuda")
    bt_h = wl.block_tables.copy()
    bt_h[2, 1] = wl.num_blocks + 5          # out of the pool
    bt_dev = torch.from_numpy(bt_h).cuda()
    prev = vb.select_decode_kernel(kernel)
    prev_order = vb.select_work_order(order)
    for P in (0, 512):
        D = wl.head_dim
        out = torch.full((4, 16, D), 7.0, device="cuda")
        if P == 0:
            vb.paged_gqa_decode(q, k, v, bt_dev, sl_dev, wl.scale, 0, 1, out)
        else:
            NP = 1
            ml = torch.empty((4, 16, NP), device="cuda")
            es = torch.empty((4, 16, NP), device="cuda")
            to = torch.empty((4, 16, NP, D), device="cuda")
            vb.paged_gqa_decode(q, k, v, bt_dev, sl_dev, wl.scale, P, NP, None, ml, es, to)
            vb.paged_gqa_reduce(ml, es, to, sl_dev, P, out)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(np.isfinite(o[0])), f"P={P}"
        assert np.all(o[1] == 0.0), f"P={P}: empty sequence must be zeros"
        assert np.all(np.isnan(o[2])), f"P={P}: bad page id must poison its sequence"
        assert np.all(np.isnan(o[3])), f"P={P}: length beyond the page table must poison"
    vb.select_decode_kernel(prev)
    vb.select_work_order(prev_order)


def test_errors_on_real_tensors():
    import torch
    wl = named("tiny_1x64")
    q, k, v, bt, sl = to_device(wl)
    out = torch.empty((1, 32, 128), device="cuda")
    with pytest.raises(vb.VkError) as e:
        vb.paged_gqa_decode(q, k, v, bt, sl, wl.scale, 128, 1, out)
    assert e.value.name == "PARTITION"
    with pytest.raises(vb.VkError) as e:
        vb.paged_gqa_decode(q, k, v, bt, sl, wl.scale, 0, 2, out)
    assert e.value.name == "PARTITION"


def test_last_plan_reports_launch():
    wl = named("batch8_2k")
    _, plan, last, _ = run_hip(wl, 512)
    assert last.partition_size == 512 and last.max_num_partitions == plan.max_num_partitions
    assert tuple(last.grid) == (plan.max_num_partitions, wl.num_kv_heads, wl.num_seqs)
    assert last.block > 0


WORK_LENS = [1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2100, 4097, 5000]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("kernel", [vb.KERNEL_MFMA_W1, vb.KERNEL_MFMA_W2, vb.KERNEL_MFMA_W4,
                                    vb.KERNEL_MFMA_W4P2])
@pytest.mark.parametrize("geom,bs,S", [((24, 4, 256), 32, 32), ((16, 2, 128), 8, 64),
                                       ((32, 8, 128), 16, 3)])
def test_work_orders_bit_identical(orc, geom, bs, S, kernel, fused):
    """Grid order and longest-first order hand the same (partition, KV head,
    sequence) items to different workgroups: partials and outputs are
    bit-identical (NaN-prefilled scratch shows a missed or extra partial),
    and both match the oracle."""
    Hq, Hkv, D = geom
    lens = (WORK_LENS * 4)[:S]
    wl = make_custom(seq_lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                     seed=Hq + D + bs + S, pool_factor=1.3, canaries=True, sigma_k=2.0)
    ref = orc.paged_attention(wl)
    for P in (256, 512, 1024):
        a, _, la, pa = run_hip(wl, P, kernel=kernel, keep_partials=True, fused=fused,
                               order=vb.ORDER_GRID)
        b, _, lb, pb = run_hip(wl, P, kernel=kernel, keep_partials=True, fused=fused,
                               order=vb.ORDER_LONGEST_FIRST)
        assert la.work_order == vb.ORDER_GRID and lb.work_order == vb.ORDER_LONGEST_FIRST
        assert np.array_equal(a, b)
        for x, y in zip(pa, pb):
            assert np.array_equal(x, y, equal_nan=True)
        assert_parity(b, ref, f"{geom} S={S} P={P} longest-first")
