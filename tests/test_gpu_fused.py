"""GPU parity of the single-launch decode (vk_paged_gqa_decode_fused): the
last workgroup of each (sequence, KV head) merges the split partials in place,
so one launch writes the final output.

Against the float64 oracle at the stated tolerance (max |gpu - ref| <= 2e-3,
per-row relative L2 <= 1e-2); against the two-launch path (decode + reduce):
the partials are bit-identical and the merged output agrees to fp32 rounding
of a different summation order; page-table indexing (one-hot probe),
unsplit calls and repeated calls are bit-exact; the arrival counters are zero
after every call.
"""
import ctypes

import numpy as np
import pytest

from gpu_helpers import assert_parity, named, oracle_ref, run_hip, say, to_device
from paged_gqa_kv_decode_amd import binding as vb
from paged_gqa_kv_decode_amd.workloads import make_custom, make_onehot_probe

pytestmark = pytest.mark.gpu

FUSED_MAX_PARTITIONS = 8   # above this the single-launch entry point runs decode + reduce
NAMED = [("tiny_1x64", 0), ("batch8_2k", 512), ("long32_16k", 256), ("long32_16k", 512),
         ("mixed64_32k", 512), ("long4_128k", -1)]
WAVES = [vb.KERNEL_MFMA, vb.KERNEL_MFMA_W1, vb.KERNEL_MFMA_W2, vb.KERNEL_MFMA_W4]


@pytest.mark.parametrize("kernel", WAVES)
@pytest.mark.parametrize("name,P", NAMED, ids=[f"{n}-P{p}" for n, p in NAMED])
def test_fused_named_workload_parity(orc, name, P, kernel):
    say(f"[fused] {name} P={P} kernel={kernel}")
    wl = named(name)
    ref = oracle_ref(orc, name)
    gpu, plan, last, _ = run_hip(wl, P, kernel=kernel, fused=True)
    if kernel != vb.KERNEL_MFMA:
        assert last.kernel == kernel
    assert_parity(gpu, ref, f"fused {name} P={plan.partition_size}")


@pytest.mark.parametrize("name,P", [("batch8_2k", 512), ("batch8_2k", 256), ("mixed64_32k", 512),
                                    ("long32_16k", 256), ("long4_128k", 512)])
def test_fused_matches_two_launch(name, P):
    """Same kernel body: partials bit-identical where written; the merged
    output within fp32 rounding of the separate reduce; single-partition
    sequences go straight to `out` and leave their scratch rows untouched.
    Above 8 partitions per sequence the call is decode + reduce itself: every
    partial and the output bit-identical."""
    wl = named(name)
    dev = to_device(wl)
    two, _, _, (m2, l2, o2) = run_hip(wl, P, dev=dev, keep_partials=True)
    one, plan, _, (m1, l1, o1) = run_hip(wl, P, dev=dev, keep_partials=True, fused=True)
    d = float(np.max(np.abs(one - two)))
    say(f"  fused vs two-launch {name} P={P} NP={plan.max_num_partitions}: max |diff| {d:.3e}")
    if plan.max_num_partitions > FUSED_MAX_PARTITIONS:
        assert np.array_equal(one, two)
        for a, b in ((m1, m2), (l1, l2), (o1, o2)):
            assert np.array_equal(a, b, equal_nan=True)
        return
    assert d <= 2e-5
    for s, L in enumerate(wl.seq_lens):
        n = -(-int(L) // P)
        if n == 1:
            assert np.all(np.isnan(o1[s])) and np.all(np.isnan(m1[s])), "scratch written for n == 1"
            assert np.array_equal(one[s], o2[s, :, 0, :]), "direct write must equal the partial"
        else:
            assert np.array_equal(m1[s, :, :n], m2[s, :, :n])
            assert np.array_equal(l1[s, :, :n], l2[s, :, :n])
            assert np.array_equal(o1[s, :, :n], o2[s, :, :n])
            assert np.all(np.isnan(o1[s, :, n:]))


@pytest.mark.parametrize("name", ["tiny_1x64", "batch8_2k"])
def test_fused_unsplit_is_the_unsplit_kernel(name):
    wl = named(name)
    dev = to_device(wl)
    a, _, _, _ = run_hip(wl, 0, dev=dev)
    b, _, _, _ = run_hip(wl, 0, dev=dev, fused=True)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,P", [("batch8_2k", 512), ("long32_16k", 256), ("mixed64_32k", 512)])
def test_fused_onehot_probe_bit_exact(name, P):
    wl, targets = make_onehot_probe(named(name, canaries=True), seed=11 + P)
    gpu, _, _, _ = run_hip(wl, P, fused=True)
    bs, G = wl.block_size, wl.group
    for s in range(wl.num_seqs):
        t = targets[s]
        blk = wl.block_tables[s, t // bs].astype(np.int64)
        want = np.stack([blk % 2048, blk // 2048, t % bs, np.arange(wl.num_q_heads) // G], 1)
        assert np.array_equal(gpu[s, :, :4], want.astype(np.float64)), f"seq {s}"
        assert np.all(gpu[s, :, 4:] == 0.0)


@pytest.mark.parametrize("name,P", [("batch8_2k", 512), ("mixed64_32k", 512)])
def test_fused_repeat_calls_bit_identical(name, P):
    """One step object called three times: the counters it zeroed once are
    back at zero after each call, and the results do not change."""
    import torch
    wl = named(name)
    q, k, v, bt, sl = to_device(wl)
    step = vb.DecodeStep(q, k, v, bt, sl, wl.seq_lens, wl.scale, P, fused=True)
    outs = []
    for _ in range(3):
        step.out.fill_(float("nan"))
        step.run()
        torch.cuda.synchronize()
        assert int(step.counters.abs().sum().item()) == 0
        outs.append(step.out.cpu().numpy().copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_fused_counter_buffer_reused_across_shapes(orc):
    """One counter buffer for a 16-sequence call and then a 5-sequence call
    (up to 8 partitions of 256: the in-place merge)."""
    import torch
    counters = torch.zeros(16 * 8, dtype=torch.int32, device="cuda")
    for S, seed in ((16, 1), (5, 2)):
        lens = list(np.random.default_rng(seed).integers(1, 2049, S))
        wl = make_custom(seq_lens=lens, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                         seed=seed, pool_factor=1.3, canaries=True)
        q, k, v, bt, sl = to_device(wl)
        NP = -(-max(lens) // 256)
        out = torch.full((S, 32, 128), float("nan"), device="cuda")
        ml = torch.empty((S, 32, NP), device="cuda")
        es = torch.empty((S, 32, NP), device="cuda")
        to = torch.empty((S, 32, NP, 128), device="cuda")
        vb.paged_gqa_decode_fused(q, k, v, bt, sl, wl.scale, 256, NP, out, ml, es, to, counters)
        torch.cuda.synchronize()
        assert int(counters.abs().sum().item()) == 0
        assert_parity(out.cpu().numpy().astype(np.float64), orc.paged_attention(wl), f"S={S}")


SWEEP = [((32, 8, 128), 8), ((32, 8, 128), 16), ((32, 8, 128), 32),
         ((24, 4, 256), 8), ((24, 4, 256), 16), ((24, 4, 256), 32),
         ((16, 2, 128), 8), ((16, 2, 128), 16), ((16, 2, 128), 32),
         ((16, 2, 256), 8), ((16, 2, 256), 16), ((16, 2, 256), 32)]


@pytest.mark.parametrize("kernel", WAVES[1:])
@pytest.mark.parametrize("geom,bs", SWEEP, ids=[f"{g[0]}-{g[1]}-{g[2]}-bs{b}" for g, b in SWEEP])
def test_fused_all_specialisations_ragged(orc, geom, bs, kernel):
    """Every (geometry, page size, waves) instance with lengths around page,
    step and partition boundaries (1 to 9 partitions), canaries on."""
    Hq, Hkv, D = geom
    lens = [1, bs - 1, bs, bs + 1, 255, 256, 257, 511, 512, 513, 1025, 1537, 2100, 4097]
    wl = make_custom(seq_lens=lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                     seed=Hq * 1000 + D + bs + 7, pool_factor=1.7, canaries=True,
                     extra_blocks_per_seq=2, sigma_k=2.0)
    ref = orc.paged_attention(wl)
    for P in (256, 512, 1024):
        gpu, _, _, _ = run_hip(wl, P, kernel=kernel, fused=True)
        assert_parity(gpu, ref, f"fused {geom} bs{bs} P{P}")


@pytest.mark.parametrize("order", [vb.ORDER_GRID, vb.ORDER_LONGEST_FIRST])
@pytest.mark.parametrize("kernel", [vb.KERNEL_MFMA_W1, vb.KERNEL_MFMA_W4])
@pytest.mark.parametrize("head_dim", [128, 256])
def test_fused_device_side_guards(kernel, head_dim, order):
    """Lengths and page ids the host cannot see: L <= 0 gives zeros; a bad
    page id, a length beyond the page table or beyond NP * P gives NaN for
    that sequence only, in both the merged (several partitions) and the
    direct (one partition) case; every counter ends at zero."""
    import torch
    S, bs, P, NP = 7, 16, 256, 3
    wl = make_custom(seq_lens=[600, 600, 600, 900, 600, 100, 100], num_q_heads=16, num_kv_heads=2,
                     head_dim=head_dim,
                     block_size=bs, seed=8, pool_factor=2.0, extra_blocks_per_seq=20)
    cap = wl.block_tables.shape[1] * bs
    assert 768 < 900 < cap < 2000
    q, k, v, bt, sl = to_device(wl)
    sl_dev = torch.tensor([600, 0, 600, 900, 2000, 100, 100], dtype=torch.int32, device="cuda")
    bt_h = wl.block_tables.copy()
    bt_h[2, 20] = wl.num_blocks + 5     # partition 1 of sequence 2
    bt_h[5, 2] = -3                     # the only partition of sequence 5
    bt_dev = torch.from_numpy(bt_h).cuda()
    counters = torch.zeros(S * 2, dtype=torch.int32, device="cuda")
    D = head_dim
    out = torch.full((S, 16, D), 7.0, device="cuda")
    ml = torch.empty((S, 16, NP), device="cuda")
    es = torch.empty((S, 16, NP), device="cuda")
    to = torch.empty((S, 16, NP, D), device="cuda")
    prev = vb.select_decode_kernel(kernel)
    prev_order = vb.select_work_order(order)
    try:
        vb.paged_gqa_decode_fused(q, k, v, bt_dev, sl_dev, wl.scale, P, NP, out, ml, es, to,
                                  counters)
        torch.cuda.synchronize()
        assert vb.last_plan().work_order == order
    finally:
        vb.select_decode_kernel(prev)
        vb.select_work_order(prev_order)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o[0])) and np.all(np.isfinite(o[6]))
    assert np.all(o[1] == 0.0), "empty sequence must be zeros"
    for s, why in ((2, "bad page id"), (3, "length beyond NP * P"), (4, "length beyond the table"),
                   (5, "bad page id, one partition")):
        assert np.all(np.isnan(o[s])), f"{why} must poison sequence {s}"
    assert int(counters.abs().sum().item()) == 0


def test_fused_argument_errors():
    """Through the C ABI: `out` and (split) `counters` are required; the VALU
    family selection falls back to the matrix-core kernels."""
    import torch
    wl = named("batch8_2k")
    q, k, v, bt, sl = to_device(wl)
    S, Hq, D = wl.q.shape
    NP = -(-int(wl.seq_lens.max()) // 512)
    out = torch.empty((S, Hq, D), device="cuda")
    ml = torch.empty((S, Hq, NP), device="cuda")
    es = torch.empty((S, Hq, NP), device="cuda")
    to = torch.empty((S, Hq, NP, D), device="cuda")
    cnt = torch.zeros(S * wl.num_kv_heads, dtype=torch.int32, device="cuda")
    L = vb.lib()

    def call(o, c, P=512, np_=NP):
        return L.vk_paged_gqa_decode_fused(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), bt.data_ptr(), sl.data_ptr(), S, Hq,
            wl.num_kv_heads, D, wl.block_size, bt.shape[1], wl.num_blocks,
            ctypes.c_float(wl.scale), P, np_, o, ml.data_ptr(), es.data_ptr(), to.data_ptr(), c,
            None)

    assert call(out.data_ptr(), None) == 1          # VK_ERR_NULL_ARG
    assert call(None, cnt.data_ptr()) == 1
    assert call(None, None, 0, 1) == 1
    assert call(out.data_ptr(), None, 0, 1) == 0    # unsplit: no counters needed
    prev = vb.select_decode_kernel(vb.KERNEL_DOT)
    try:
        assert call(out.data_ptr(), cnt.data_ptr()) == 0
        assert vb.last_plan().kernel != vb.KERNEL_DOT
    finally:
        vb.select_decode_kernel(prev)
    torch.cuda.synchronize()
    assert int(cnt.abs().sum().item()) == 0


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays_match_eager(fused):
    """The step captured in a HIP graph and replayed three times, with eager
    work (another decode, a fill of the output) between replays: every replay
    equals the eager result bit for bit, and the counters stay at zero."""
    import torch
    wl = named("batch8_2k")
    q, k, v, bt, sl = to_device(wl)
    step = vb.DecodeStep(q, k, v, bt, sl, wl.seq_lens, wl.scale, 512, fused=fused)
    step.run()
    torch.cuda.synchronize()
    eager = step.out.cpu().numpy().copy()
    other = named("tiny_1x64")
    oq, ok_, ov, obt, osl = to_device(other)
    side = vb.DecodeStep(oq, ok_, ov, obt, osl, other.seq_lens, other.scale, 0)
    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        step.run(stream=cap)
    for rep in range(3):
        step.out.fill_(float("nan"))
        side.run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(step.out.cpu().numpy(), eager), f"replay {rep}"
        if step.counters is not None:
            assert int(step.counters.abs().sum().item()) == 0
