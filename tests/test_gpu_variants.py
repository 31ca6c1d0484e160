"""GPU parity of the geometry and element-type variants against the float64
oracle: multi-head (Hkv = Hq) and multi-query (Hkv = 1) geometries on the
decode (every wave count, split and unsplit, the single launch) and on the
multi-token kernel; bf16 and fp32 q / K / V on the decode.

Tolerance as everywhere: max |gpu - ref| <= 2e-3, per-row relative L2 <= 1e-2
(bf16 and fp32 scores are exact products accumulated in fp32; bf16 weights
enter PV as a rounded value plus its residual, fp32 weights unrounded).
"""
import numpy as np
import pytest

from gpu_helpers import assert_parity, run_hip, say, to_device
from paged_gqa_kv_decode_amd import binding as vb
from paged_gqa_kv_decode_amd.workloads import make_custom, make_varlen_custom

pytestmark = pytest.mark.gpu

MHQ = [((16, 16, 128), 16), ((8, 8, 256), 32), ((16, 1, 128), 8), ((16, 1, 256), 32)]
LENS = [1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1025, 2100, 4097]
WAVES = [vb.KERNEL_MFMA, vb.KERNEL_MFMA_W1, vb.KERNEL_MFMA_W2, vb.KERNEL_MFMA_W4]


@pytest.mark.parametrize("kernel", WAVES)
@pytest.mark.parametrize("geom,bs", MHQ, ids=[f"{g[0]}-{g[1]}-{g[2]}-bs{b}" for g, b in MHQ])
def test_mha_mqa_decode(orc, geom, bs, kernel):
    Hq, Hkv, D = geom
    wl = make_custom(seq_lens=LENS, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                     seed=Hq + 7 * Hkv + D, pool_factor=1.5, canaries=True, sigma_k=2.0)
    ref = orc.paged_attention(wl)
    for P in (0, 256, 512):
        gpu, _, last, _ = run_hip(wl, P, kernel=kernel)
        assert_parity(gpu, ref, f"{geom} P{P} kernel {last.kernel}")
        fused, _, _, _ = run_hip(wl, P, kernel=kernel, fused=True)
        assert_parity(fused, ref, f"{geom} P{P} single launch")


@pytest.mark.parametrize("geom,bs", MHQ, ids=[f"{g[0]}-{g[1]}-{g[2]}-bs{b}" for g, b in MHQ])
def test_mha_mqa_varlen(orc, geom, bs):
    Hq, Hkv, D = geom
    lens, qlens = [1, 300, 513, 1030, 40, 2100], [1, 3, 17, 300, 40, 5]
    wl = make_varlen_custom(seq_lens=lens, q_lens=qlens, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim=D, block_size=bs, seed=Hq * 3 + D, pool_factor=1.5,
                            canaries=True)
    ref = orc.paged_varlen_arrays(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.seq_lens,
                                  wl.meta["cu_q"], wl.scale)
    import torch
    q, k, v, bt, sl = vb.device_inputs(wl)
    cu = torch.from_numpy(wl.meta["cu_q"]).cuda()
    for P in (0, 512):
        step = vb.VarlenStep(q, k, v, bt, sl, cu, wl.seq_lens, wl.meta["q_lens"], wl.scale, P)
        out = step.run()
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy().astype(np.float64), ref, f"varlen {geom} P{P}",
                      dtype="f16_tiles")


GEOMS = [((32, 8, 128), 16), ((24, 4, 256), 32), ((16, 2, 128), 8), ((16, 2, 256), 32),
         ((16, 16, 128), 16), ((16, 1, 256), 32)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kernel", WAVES)
@pytest.mark.parametrize("geom,bs", GEOMS, ids=[f"{g[0]}-{g[1]}-{g[2]}-bs{b}" for g, b in GEOMS])
def test_element_types_decode(orc, geom, bs, kernel, dtype):
    Hq, Hkv, D = geom
    wl = make_custom(seq_lens=LENS, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                     seed=Hq + D + bs, pool_factor=1.5, canaries=True, sigma_k=2.0, dtype=dtype)
    ref = orc.paged_attention(wl)
    for P in (0, 512, 1024):
        gpu, _, last, _ = run_hip(wl, P, kernel=kernel)
        assert_parity(gpu, ref, f"{dtype} {geom} P{P} kernel {last.kernel}", dtype=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_element_types_long_sequences(orc, dtype):
    """A long-context shape per type: 8 sequences of 2k-16k tokens, planner."""
    lens = list(np.random.default_rng(4).integers(2048, 16384, 8))
    wl = make_custom(seq_lens=lens, num_q_heads=24, num_kv_heads=4, head_dim=256, block_size=32,
                     seed=17, dtype=dtype)
    ref = orc.paged_attention(wl)
    gpu, plan, _, _ = run_hip(wl, -1)
    say(f"  {dtype} long: P={plan.partition_size}")
    assert_parity(gpu, ref, f"{dtype} long", dtype=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_element_types_v_times_two_is_exact(dtype):
    """Doubling V (exact in both types) doubles the output bit for bit."""
    import copy
    wl = make_custom(seq_lens=[100, 700, 1500], num_q_heads=32, num_kv_heads=8, head_dim=128,
                     block_size=16, seed=23, dtype=dtype)
    base, _, _, _ = run_hip(wl, 512)
    w2 = copy.copy(wl)
    if dtype == "f32":
        w2.v_cache = wl.v_cache * np.float32(2)
    else:   # bf16 bit patterns: add one to the exponent field (values are normal)
        w2.v_cache = (wl.v_cache.astype(np.uint32) + (1 << 7)).astype(np.uint16)
    out, _, _, _ = run_hip(w2, 512)
    assert np.array_equal(out, 2 * base)


def test_element_type_errors():
    import torch
    wl = make_custom(seq_lens=[40], num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                     seed=1, dtype="bf16")
    q, k, v, bt, sl = to_device(wl)
    out = torch.empty((1, 32, 128), device="cuda")
    with pytest.raises(vb.VkError) as e:
        vb.lib()   # an unknown element type
        code = vb.lib().vk_paged_gqa_decode_dt(7, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               bt.data_ptr(), sl.data_ptr(), 1, 32, 8, 128, 16,
                                               bt.shape[1], wl.num_blocks, wl.scale, 0, 1,
                                               out.data_ptr(), None, None, None, None)
        vb._check("vk_paged_gqa_decode_dt", code)
    assert e.value.name == "DTYPE"
    with pytest.raises(TypeError):   # fp16 entry point with bf16 tensors
        vb.paged_gqa_decode(q, k, v, bt, sl, wl.scale, 0, 1, out)
    cnt = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):   # the single launch is fp16 only
        vb.paged_gqa_decode_fused(q, k, v, bt, sl, wl.scale, 512, 1, out, out, out, out, cnt)
