"""GPU parity of bf16 q/K/V through both multi-token kernels (the column
kernel and the LDS-tiled one) against the float64 oracle on the same bf16
bits.  Same tolerance as the decode: max |gpu - ref| <= 2e-3 and per-row
relative L2 <= 1e-2.
"""
import numpy as np
import pytest

from gpu_helpers import assert_parity, say
from paged_gqa_kv_decode_amd import binding as vb
from paged_gqa_kv_decode_amd.workloads import make_varlen_custom

pytestmark = pytest.mark.gpu


def _t(x):
    import torch
    if x.dtype == np.uint16:   # bf16 bit patterns
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def run(wl, kernel, P):
    import torch
    prev = vb.select_varlen_kernel(kernel)
    try:
        q, k, v = _t(wl.q), _t(wl.k_cache), _t(wl.v_cache)
        bt, sl = _t(wl.block_tables), _t(wl.seq_lens)
        cu = _t(wl.meta["cu_q"])
        out = torch.full(tuple(wl.q.shape), float("nan"), dtype=torch.float32, device="cuda")
        st = vb.VarlenStep(q, k, v, bt, sl, cu, wl.seq_lens, wl.meta["q_lens"], wl.scale, P,
                           out=out)
        st.run()
        torch.cuda.synchronize()
        assert st.plan.kernel == kernel
        return out.cpu().numpy().astype(np.float64)
    finally:
        vb.select_varlen_kernel(prev)


def oracle_bf16(orc, wl):
    return orc.paged_varlen_arrays(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                   wl.meta["cu_q"], wl.scale, dtype="bf16")


CASES = [((32, 8, 128), 16), ((24, 4, 256), 32), ((16, 1, 128), 8), ((8, 8, 256), 16)]


@pytest.mark.parametrize("kernel", [vb.KERNEL_VARLEN_COLUMNS, vb.KERNEL_VARLEN_TILES],
                         ids=["columns", "tiles"])
@pytest.mark.parametrize("geom,bs", CASES, ids=[f"{g[0]}-{g[1]}-{g[2]}-bs{b}" for g, b in CASES])
def test_bf16_mixed_batch(orc, geom, bs, kernel):
    Hq, Hkv, D = geom
    bq = 128 // (Hq // Hkv)
    lens = [1, 100, 700, 64, 1100, 40]
    qlens = [1, 40, bq + 1, 0, 2 * bq, 33]
    wl = make_varlen_custom(seq_lens=lens, q_lens=qlens, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim=D, block_size=bs, seed=Hq * 3 + D + bs, pool_factor=1.5,
                            canaries=True, sigma_k=2.0, dtype="bf16")
    assert wl.q.dtype == np.uint16
    ref = oracle_bf16(orc, wl)
    for P in (0, 256, 1024):
        gpu = run(wl, kernel, P)
        say(f"[bf16 varlen] {geom} bs{bs} kernel {kernel} P{P}")
        assert_parity(gpu, ref, f"bf16 {geom} bs{bs} k{kernel} P{P}", dtype="bf16")


def test_bf16_is_not_the_fp16_result(orc):
    """The kernels read the bf16 bits as bf16: the same bits read as fp16 give
    a different answer, the bf16 one matches the oracle."""
    wl = make_varlen_custom(seq_lens=[300, 90], q_lens=[70, 9], num_q_heads=32, num_kv_heads=8,
                            head_dim=128, block_size=16, seed=5, dtype="bf16")
    ref = oracle_bf16(orc, wl)
    gpu = run(wl, vb.KERNEL_VARLEN_TILES, 0)
    assert_parity(gpu, ref, "bf16 tiles", dtype="bf16")
    as_f16 = orc.paged_varlen_arrays(wl.q.view(np.float16), wl.k_cache.view(np.float16),
                                     wl.v_cache.view(np.float16), wl.block_tables, wl.seq_lens,
                                     wl.meta["cu_q"], wl.scale)
    assert np.nanmax(np.abs(np.nan_to_num(as_f16) - ref)) > 1e-2
