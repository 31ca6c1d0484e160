"""The planner rule (oracle/planner.py) against hand-computed decisions.

Rule (vllm-metal kernels page, section on the dispatch layer): budget =
33 simdgroups per core x cores; try 512-token partitions first, then 256;
only full partitions count as work; GQA scratch capped at 512 MiB."""
import pytest

from oracle.planner import plan, PlanError


def test_long_context_picks_512():
    # 4 x 131072 tokens, Hq 16: W(512) = 16 * 4 * 256 = 16384 >= 33 * 256 = 8448.
    p = plan([131072] * 4, 16, 2, 256, 32, 4096, -1, 256)
    assert p["partition_size"] == 512 and p["work_full_parts"] == 16384
    assert p["budget"] == 8448 and p["max_num_partitions"] == 256
    assert p["scratch_bytes"] == 4 * 16 * 256 * 258 * 4


def test_boundary_both_sides():
    # Hq 16, one sequence: W(512) = 16 * floor(L / 512); budget 33 * 16 = 528 = W at L = 33*512.
    L = 33 * 512
    assert plan([L], 16, 2, 128, 16, L // 16, -1, 16)["partition_size"] == 512
    assert plan([L - 1], 16, 2, 128, 16, L // 16, -1, 16)["partition_size"] == 256


def test_ragged_tails_do_not_count():
    # 100 sequences of 511 tokens: no full 512 partition at all -> 256.
    p = plan([511] * 100, 32, 8, 128, 16, 32, -1, 1, budget_per_cu=1)
    assert p["partition_size"] == 256
    # one full 512 partition per sequence, 32 heads, 100 seqs = 3200 >= 33 * 96 = 3168
    p = plan([1023] * 100, 32, 8, 128, 16, 64, -1, 96)
    assert p["partition_size"] == 512 and p["work_full_parts"] == 3200
    p = plan([1023] * 100, 32, 8, 128, 16, 64, -1, 97)
    assert p["partition_size"] == 256 and p["work_full_parts"] == 32 * 100 * 3


def test_forced_and_unsplit():
    p = plan([64], 32, 8, 128, 16, 4, 0, 256)
    assert p["partition_size"] == 0 and p["max_num_partitions"] == 1 and p["scratch_bytes"] == 0
    p = plan([2048, 1], 32, 8, 128, 16, 128, 512, 256)
    assert p["partition_size"] == 512 and p["max_num_partitions"] == 4
    assert p["scratch_bytes"] == 2 * 32 * 4 * 130 * 4
    p = plan([513], 24, 4, 256, 32, 17, 256, 256)
    assert p["partition_size"] == 256 and p["max_num_partitions"] == 3


def test_scratch_cap():
    # 64 seqs x 24 heads x 64 partitions(256) x 258 x 4 = 101449728 B (96.75 MiB).
    with pytest.raises(PlanError) as e:
        plan([16384] * 64, 24, 4, 256, 32, 512, 256, 256, scratch_cap_bytes=101449727)
    assert e.value.code == "SCRATCH_CAP"
    p = plan([16384] * 64, 24, 4, 256, 32, 512, 256, 256, scratch_cap_bytes=101449728)
    assert p["scratch_bytes"] == 101449728
    # the default cap is 512 MiB: the same request at 512 partitions of 2048 seqs is over
    with pytest.raises(PlanError):
        plan([16384] * 2048, 24, 4, 256, 32, 512, 256, 256)


@pytest.mark.parametrize("args,code", [
    (([64], 32, 8, 64, 16, 4), "GEOMETRY"),        # head_dim not admitted
    (([64], 30, 8, 128, 16, 4), "GEOMETRY"),       # Hq not a multiple of Hkv
    (([64], 32, 8, 128, 64, 4), "BLOCK_SIZE"),
    (([0], 32, 8, 128, 16, 4), "SEQ_LEN"),
    (([65], 32, 8, 128, 16, 4), "SEQ_LEN"),        # beyond 4 pages of 16
    (([], 32, 8, 128, 16, 4), "BAD_DIM"),
])
def test_rejections(args, code):
    with pytest.raises(PlanError) as e:
        plan(*args, -1, 256)
    assert e.value.code == code


def test_bad_partition_request():
    with pytest.raises(PlanError) as e:
        plan([64], 32, 8, 128, 16, 4, 128, 256)
    assert e.value.code == "PARTITION"
