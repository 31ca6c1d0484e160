"""GPU parity of several query tokens per sequence (vk_paged_gqa_varlen,
causal, packed rows) against the float64 oracle.

Tolerance as for the decode: max |gpu - ref| <= 2e-3 and per-row relative L2
<= 1e-2.  One query token per sequence is bit-identical to the decode kernel
(one wave per workgroup, grid order) for both unsplit and split launches;
causality is checked structurally (changing keys past a row's position leaves
that row bit-identical); guards and empty rows as documented.
"""
import numpy as np
import pytest

from gpu_helpers import assert_parity, say
from paged_gqa_kv_decode_amd import binding as vb
from paged_gqa_kv_decode_amd.workloads import make_varlen, make_varlen_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def column_kernel():
    """These tests cover the column kernel (auto picks the LDS-tiled one when
    a sequence has more than 16 / G query tokens; that kernel has its own
    tests)."""
    prev = vb.select_varlen_kernel(vb.KERNEL_VARLEN_COLUMNS)
    yield
    vb.select_varlen_kernel(prev)


def _dev(wl):
    import torch
    return (torch.from_numpy(wl.q).cuda(), torch.from_numpy(wl.k_cache).cuda(),
            torch.from_numpy(wl.v_cache).cuda(), torch.from_numpy(wl.block_tables).cuda(),
            torch.from_numpy(wl.seq_lens).cuda(), torch.from_numpy(wl.meta["cu_q"]).cuda())


def run_varlen(wl, P=-1, dev=None, keep_partials=False, cu_count=0):
    import torch
    q, k, v, bt, sl, cu = dev if dev is not None else _dev(wl)
    out = torch.full(tuple(wl.q.shape), float("nan"), dtype=torch.float32, device="cuda")
    step = vb.VarlenStep(q, k, v, bt, sl, cu, wl.seq_lens, wl.meta["q_lens"], wl.scale, P,
                         cu_count=cu_count, out=out)
    if step.tmp_out is not None:
        step.max_logits.fill_(float("nan"))
        step.exp_sums.fill_(float("nan"))
        step.tmp_out.fill_(float("nan"))
    step.run()
    torch.cuda.synchronize()
    parts = None
    if keep_partials and step.tmp_out is not None:
        parts = tuple(t.cpu().numpy() for t in (step.max_logits, step.exp_sums, step.tmp_out))
    return out.cpu().numpy().astype(np.float64), step.plan, parts


def oracle_varlen(orc, wl):
    return orc.paged_varlen_arrays(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                   wl.meta["cu_q"], wl.scale)


def sampled_rows_ref(orc, wl, rows_per_seq, seed):
    """Oracle values of sampled query rows, each as a one-token decode over the
    keys it sees (the oracle pins this equivalence)."""
    rng = np.random.default_rng(seed)
    cu, ql = wl.meta["cu_q"], wl.meta["q_lens"]
    rows, lims, seqs = [], [], []
    for s in range(wl.num_seqs):
        js = np.unique(np.concatenate([[0, ql[s] - 1], rng.integers(0, ql[s], rows_per_seq)]))
        for j in js:
            rows.append(int(cu[s] + j))
            lims.append(int(wl.seq_lens[s] - ql[s] + j + 1))
            seqs.append(s)
    ref = orc.paged_attention_arrays(wl.q[rows], wl.k_cache, wl.v_cache, wl.block_tables[seqs],
                                     np.array(lims, dtype=np.int32), wl.scale)
    return np.array(rows), ref


@pytest.mark.parametrize("P", [-1, 0, 256, 512, 1024])
def test_verify_workload_parity(orc, P):
    wl = make_varlen("verify32_q4")
    ref = oracle_varlen(orc, wl)
    gpu, plan, _ = run_varlen(wl, P)
    say(f"[varlen] verify32_q4 P={plan.partition_size} NP={plan.max_num_partitions}")
    assert_parity(gpu, ref, f"verify32_q4 P={plan.partition_size}")


def test_prefill_split_scratch_over_the_cap():
    """A split launch would need 4096 rows x 24 heads x 18 partitions x 258
    floats = 1.8 GB of partials: the planner refuses it (the unsplit path,
    which the planner picks itself, needs none)."""
    wl = make_varlen("prefill4_chunk1k")
    with pytest.raises(vb.VkError) as e:
        vb.plan_varlen(wl.seq_lens, wl.meta["q_lens"], 24, 4, 256, 32, wl.max_blocks_per_seq, 512)
    assert e.value.name == "SCRATCH_CAP"


@pytest.mark.parametrize("P", [-1, 0])
def test_prefill_workload_sampled_parity(orc, P):
    wl = make_varlen("prefill4_chunk1k")
    gpu, plan, _ = run_varlen(wl, P)
    say(f"[varlen] prefill4_chunk1k P={plan.partition_size}")
    assert np.all(np.isfinite(gpu))
    rows, ref = sampled_rows_ref(orc, wl, 48, seed=5)
    assert_parity(gpu[rows], ref, f"prefill4_chunk1k P={plan.partition_size} ({len(rows)} rows)",
                  dtype="f16_tiles")


SWEEP = [((32, 8, 128), 8), ((32, 8, 128), 16), ((32, 8, 128), 32),
         ((24, 4, 256), 8), ((24, 4, 256), 16), ((24, 4, 256), 32),
         ((16, 2, 128), 8), ((16, 2, 128), 16), ((16, 2, 128), 32),
         ((16, 2, 256), 8), ((16, 2, 256), 16), ((16, 2, 256), 32)]


@pytest.mark.parametrize("geom,bs", SWEEP, ids=[f"{g[0]}-{g[1]}-{g[2]}-bs{b}" for g, b in SWEEP])
def test_all_specialisations_mixed_batch(orc, geom, bs):
    """Decode rows, verification rows, prefill chunks, a whole prompt (q_len =
    L) and an empty sequence in one batch, around page / step / partition
    boundaries; unsplit and every partition size; canaries on."""
    Hq, Hkv, D = geom
    lens = [1, 17, 300, 513, 1030, 257, 64, 2100, 40]
    qlens = [1, 1, 3, 8, 300, 257, 0, 5, 40]
    wl = make_varlen_custom(seq_lens=lens, q_lens=qlens, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim=D, block_size=bs, seed=Hq * 100 + D + bs, pool_factor=1.5,
                            canaries=True, sigma_k=2.0)
    ref = oracle_varlen(orc, wl)
    for P in (0, 256, 512, 1024):
        gpu, _, _ = run_varlen(wl, P)
        assert_parity(gpu, ref, f"{geom} bs{bs} P{P}", dtype="f16_tiles")


@pytest.mark.parametrize("P", [0, 512])
@pytest.mark.parametrize("geom,bs", [((32, 8, 128), 16), ((24, 4, 256), 32), ((16, 2, 128), 8)])
def test_one_token_rows_equal_the_decode_kernel(geom, bs, P):
    """q_len = 1 everywhere: the same matrix-core steps as the one-wave decode
    kernel in grid order, so the outputs are bit-identical."""
    import torch
    Hq, Hkv, D = geom
    lens = [1, 15, 16, 17, 500, 513, 1100, 3000]
    wl = make_varlen_custom(seq_lens=lens, q_lens=[1] * len(lens), num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim=D, block_size=bs, seed=3, canaries=True)
    gpu, _, _ = run_varlen(wl, P)
    q, k, v, bt, sl, cu = _dev(wl)
    NP = -(-max(lens) // 512)
    prev = vb.select_decode_kernel(vb.KERNEL_MFMA_W1)
    prev_order = vb.select_work_order(vb.ORDER_GRID)
    try:
        step = vb.DecodeStep(q, k, v, bt, sl, wl.seq_lens, wl.scale, P)
        dec = step.run()
        torch.cuda.synchronize()
    finally:
        vb.select_decode_kernel(prev)
        vb.select_work_order(prev_order)
    assert step.plan.max_num_partitions == (NP if P else 1)
    assert np.array_equal(gpu, dec.cpu().numpy().astype(np.float64))


def test_causality_is_structural():
    """Changing the K/V of the last token of every sequence leaves every row
    that does not see it bit-identical, and changes the last row."""
    wl = make_varlen_custom(seq_lens=[600, 90], q_lens=[40, 90], num_q_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=16, seed=12)
    a, _, _ = run_varlen(wl, 0)
    import copy
    w2 = copy.copy(wl)
    w2.k_cache = wl.k_cache.copy()
    w2.v_cache = wl.v_cache.copy()
    for s, L in enumerate(wl.seq_lens):
        b = wl.block_tables[s, (L - 1) // 16]
        w2.k_cache[b, :, (L - 1) % 16] *= np.float16(-1)
        w2.v_cache[b, :, (L - 1) % 16] += np.float16(3)
    b_, _, _ = run_varlen(w2, 0)
    cu = wl.meta["cu_q"]
    for s in range(2):
        last = cu[s + 1] - 1
        assert np.array_equal(a[cu[s]:last], b_[cu[s]:last]), "a row saw a later token"
        assert not np.array_equal(a[last], b_[last])


@pytest.mark.parametrize("P", [0, 256])
def test_varlen_device_side_guards(P):
    """Sequence 1: a page id outside the pool (NaN rows); sequence 2: length
    beyond the page table (NaN rows, nothing read); sequence 3: q_len > L
    (its first rows see nothing: zeros); sequence 4: q_len = 0 (no rows)."""
    import torch
    lens, qlens = [300, 300, 300, 4, 20], [5, 5, 5, 6, 0]
    wl = make_varlen_custom(seq_lens=lens, q_lens=qlens, num_q_heads=16, num_kv_heads=2,
                            head_dim=128, block_size=16, seed=4, pool_factor=2.0)
    q, k, v, bt, sl, cu = _dev(wl)
    bt_h = wl.block_tables.copy()
    bt_h[1, 3] = wl.num_blocks + 7
    bt = torch.from_numpy(bt_h).cuda()
    sl_h = wl.seq_lens.copy()
    sl_h[2] = bt_h.shape[1] * 16 + 100
    sl = torch.from_numpy(sl_h).cuda()
    T = wl.q.shape[0]
    NP = -(-int(sl_h.max()) // P) if P else 1
    out = torch.full((T, 16, 128), 7.0, device="cuda")
    if P:
        ml = torch.empty((T, 16, NP), device="cuda")
        es = torch.empty((T, 16, NP), device="cuda")
        to = torch.empty((T, 16, NP, 128), device="cuda")
        vb.paged_gqa_varlen(q, k, v, bt, sl, cu, 6, wl.scale, P, NP, None, ml, es, to)
        vb.paged_gqa_varlen_reduce(ml, es, to, sl, cu, 6, P, out)
    else:
        vb.paged_gqa_varlen(q, k, v, bt, sl, cu, 6, wl.scale, 0, 1, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    c = wl.meta["cu_q"]
    assert np.all(np.isfinite(o[c[0]:c[1]]))
    assert np.all(np.isnan(o[c[1]:c[2]])), "bad page id must poison its sequence"
    assert np.all(np.isnan(o[c[2]:c[3]])), "length beyond the table must poison"
    # sequence 3: L = 4, q_len = 6: rows 0, 1 see nothing, rows 2.. see 1..4 tokens
    assert np.all(o[c[3]:c[3] + 2] == 0.0)
    assert np.all(np.isfinite(o[c[3] + 2:c[4]]))


def test_varlen_argument_errors():
    import torch
    wl = make_varlen_custom(seq_lens=[40], q_lens=[4], num_q_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=16, seed=1)
    q, k, v, bt, sl, cu = _dev(wl)
    out = torch.empty((4, 32, 128), device="cuda")
    with pytest.raises(vb.VkError) as e:
        vb.paged_gqa_varlen(q, k, v, bt, sl, cu, 5, wl.scale, 0, 1, out)   # max_q_len > total_q
    assert e.value.name == "BAD_DIM"
    with pytest.raises(vb.VkError) as e:
        vb.paged_gqa_varlen(q, k, v, bt, sl, cu, 4, wl.scale, 128, 1, out)
    assert e.value.name == "PARTITION"


@pytest.mark.parametrize("P", [256, 512, 1024])
def test_single_tile_longest_first_matches_grid_order(orc, P):
    """Every sequence's queries fit one column tile (<= 16 / G tokens): the
    split launch takes the decode's longest-first order over (partition,
    KV head, sequence) when the grid takes several rounds, with its partials
    written through L2.  Same partials as grid order, so bit-identical, and
    both within the oracle's bar; rows with q_len = 0 and L = 1 included."""
    lens = [4000, 9000, 300, 1, 7000, 2048, 513, 12000] * 4
    qlens = [4, 1, 3, 1, 4, 2, 0, 4] * 4
    wl = make_varlen_custom(seq_lens=lens, q_lens=qlens, num_q_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=16, seed=21, canaries=True)
    ref = oracle_varlen(orc, wl)
    outs = {}
    for order in (vb.ORDER_GRID, vb.ORDER_LONGEST_FIRST):
        prev = vb.select_work_order(order)
        try:
            outs[order], plan, _ = run_varlen(wl, P)
            ran = vb.last_plan().work_order
        finally:
            vb.select_work_order(prev)
        assert plan.kernel == vb.KERNEL_VARLEN_COLUMNS and ran == order
        say(f"[columns] single tile P={P} order={order}")
        assert_parity(outs[order], ref, f"single tile P{P} order {order}")
    assert np.array_equal(outs[vb.ORDER_GRID], outs[vb.ORDER_LONGEST_FIRST])


def test_varlen_reduce_row_and_chunk_merges_bit_identical(orc):
    """The variable-length reduce merges one row per wave when there are many
    rows of few partitions, and 32 dims per wave otherwise; per dim both take
    the same fold steps in the same order, so the same partials give
    bit-identical rows.  max_q_len (an upper bound that only sizes the grid)
    picks the mode here: 4 -> 8 x 4 x 32 = 1024 rows (32 dims per wave),
    8 -> 2048 rows (one row per wave); P = 1024, at most 7 partitions."""
    import torch
    lens = [3000, 5000, 1200, 7000, 4100, 2500, 6000, 800]
    qlens = [4, 4, 3, 4, 1, 4, 2, 4]
    wl = make_varlen_custom(seq_lens=lens, q_lens=qlens, num_q_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=16, seed=31)
    q, k, v, bt, sl, cu = _dev(wl)
    step = vb.VarlenStep(q, k, v, bt, sl, cu, wl.seq_lens, wl.meta["q_lens"], wl.scale, 1024)
    assert (step.plan.partition_size, step.plan.max_num_partitions) == (1024, 7)
    step.run()
    outs = []
    for mq in (4, 8):
        o = torch.full_like(step.out, float("nan"))
        vb.paged_gqa_varlen_reduce(step.max_logits, step.exp_sums, step.tmp_out, sl, cu, mq, 1024, o)
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy())
    say("[varlen] reduce row vs chunk merge, P=1024")
    assert np.array_equal(outs[0], outs[1])
    assert_parity(outs[1].astype(np.float64), oracle_varlen(orc, wl), "reduce row merge P1024")
