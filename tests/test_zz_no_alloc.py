"""The no-allocation decode entry point (vk_paged_gqa_decode_noalloc) against
the existing split decode + reduce entry points on the same inputs: same
kernels and launch choices, so the outputs must agree bit for bit, and both
must match the float64 oracle within the stated tolerance.  Two calls in a
row on the library's one array per GPU, the second with a smaller input (its
partials overwrite only the front of what the first left)."""
import numpy as np
import pytest

from gpu_helpers import assert_parity, say, to_device

pytestmark = pytest.mark.gpu


def _existing(wl, dev, P):
    """decode + reduce through the entry points that take caller scratch."""
    import torch
    from paged_gqa_kv_decode_amd import binding as vb
    q, k, v, bt, sl = dev
    step = vb.DecodeStep(q, k, v, bt, sl, wl.seq_lens, wl.scale, P)
    out = step.run()
    torch.cuda.synchronize()
    return out.cpu().numpy(), step.plan


def _noalloc(wl, dev, P, NP):
    import torch
    from paged_gqa_kv_decode_amd import binding as vb
    q, k, v, bt, sl = dev
    out = torch.full((wl.num_seqs, wl.num_q_heads, wl.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    vb.paged_gqa_decode_noalloc(q, k, v, bt, sl, wl.scale, P, NP, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("P", [512, 256, 0])
def test_noalloc_matches_decode_and_reduce(orc, P):
    from paged_gqa_kv_decode_amd.workloads import make_custom
    big = make_custom(seq_lens=[3000, 17, 5200, 1, 4097, 800, 2600, 1024], num_q_heads=32,
                      num_kv_heads=8, head_dim=128, block_size=16, seed=31, pool_factor=1.5,
                      canaries=True)
    small = make_custom(seq_lens=[700, 1300, 9], num_q_heads=16, num_kv_heads=2, head_dim=256,
                        block_size=32, seed=32, pool_factor=1.5, canaries=True)
    for name, wl in (("first (8 seqs, (32,8,128))", big), ("second, smaller (3 seqs, (16,2,256))", small)):
        say(f"noalloc P={P} {name}")
        dev = to_device(wl)
        want, plan = _existing(wl, dev, P)
        got = _noalloc(wl, dev, P, plan.max_num_partitions)
        assert np.array_equal(got, want, equal_nan=False), \
            f"P={P} {name}: differs from decode + reduce (max |diff| " \
            f"{np.nanmax(np.abs(got - want)):.3e})"
        assert_parity(got.astype(np.float64), orc.paged_attention(wl), f"noalloc P={P} {name}")


def test_noalloc_named_long_context_workload(orc):
    """long4_128k at the planner's partition size (1024 on 256 CUs: 8.5 MB of partials):
    bit-identical to decode + reduce."""
    from gpu_helpers import named
    wl = named("long4_128k")
    dev = to_device(wl)
    want, plan = _existing(wl, dev, -1)
    got = _noalloc(wl, dev, plan.partition_size, plan.max_num_partitions)
    assert np.array_equal(got, want)
    say(f"  long4_128k P={plan.partition_size}: noalloc == decode + reduce")
