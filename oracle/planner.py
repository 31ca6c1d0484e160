"""Partition-size planner rule, written from the pages — oracle side.

TEST INFRASTRUCTURE: the GPU library has its own planner; this one exists so
tests can check it.  Source: vllm-metal kernels page (cf-1.com/news/5525226),
section "分发层" (the dispatch layer), and section "GQA 解码内核的四个提速技巧"
item 4 (split-KV partitions of 256 or 512 tokens):

  * the work budget is a fixed number of simdgroups per GPU core (33) times
    the core count read from the hardware;
  * 512-token partitions are tried first, then 256;
  * only *full* partitions count as work, so ragged tails are not counted;
  * the GQA scratch of one call is capped at 512 MiB.

Not from the pages: the MI355X library adds a third partition size, 1024,
in one regime (plan(..., wave_slots_per_cu=8) models it; without that
argument this is the pages' rule alone), and its default budget is 4 * G
query-head units per CU (four workgroups of one KV head's G query heads)
instead of the pages' 33 (an MI355X calibration); when the rule picks 512 and
1024-token partitions fit in a single round of cu_count * wave_slots_per_cu
resident waves with at least two waves each, the launch takes 1024: the
same work with half the partials; and with the default budget 1024 is taken
first once its full partitions give 2 workgroups per CU.

Readings where the page is silent (each stated in the design notes):
  * work W(P) = Hq * sum_s floor(L_s / P): one unit per (query head, full
    partition), since the page runs one simdgroup per query head;
  * P = 512 when W(512) >= budget, else 256 (the page does not say what
    happens when neither reaches the budget; 256 gives more parallelism);
  * scratch = S * Hq * NP * (D + 2) * 4 bytes (max, exp-sum, and D outputs,
    fp32), with NP = ceil(max L / P); over the cap is an error because no
    fallback path exists.
"""
from __future__ import annotations

ADMITTED_GEOMETRIES = {(32, 8, 128), (24, 4, 256), (16, 2, 128), (16, 2, 256),
                       # multi-head and multi-query triples
                       (16, 16, 128), (8, 8, 256), (16, 1, 128), (16, 1, 256)}
BLOCK_SIZES = (8, 16, 32)
PARTITION_SIZES = (256, 512)
DEFAULT_BUDGET_PER_CU = 33
DEFAULT_SCRATCH_CAP = 512 * 1024 * 1024


class PlanError(ValueError):
    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


def work_full_partitions(seq_lens, num_q_heads: int, P: int) -> int:
    return num_q_heads * sum(int(L) // P for L in seq_lens)


def plan(seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
         max_blocks_per_seq: int, partition_request: int = -1, cu_count: int = 256,
         budget_per_cu: int = 0, scratch_cap_bytes: int = 0, wave_slots_per_cu: int = 0) -> dict:
    """Return dict(partition_size, max_num_partitions, work_full_parts, budget,
    cu_count, scratch_bytes) or raise PlanError(code, ...)."""
    S = len(seq_lens)
    if S < 1 or num_q_heads < 1 or num_kv_heads < 1 or head_dim < 1 or max_blocks_per_seq < 1:
        raise PlanError("BAD_DIM", "non-positive dimension")
    if num_q_heads % num_kv_heads:
        raise PlanError("GEOMETRY", "Hq not a multiple of Hkv")
    if (num_q_heads, num_kv_heads, head_dim) not in ADMITTED_GEOMETRIES:
        raise PlanError("GEOMETRY", "geometry not admitted")
    if block_size not in BLOCK_SIZES:
        raise PlanError("BLOCK_SIZE", "block size not 8/16/32")
    sizes = PARTITION_SIZES + ((1024,) if wave_slots_per_cu else ())
    if partition_request not in (-1, 0) + sizes:
        raise PlanError("PARTITION", "partition request not -1/0 or a partition size")
    if cu_count < 1:
        raise PlanError("BAD_DIM", "cu_count must be positive here")
    cap_tokens = max_blocks_per_seq * block_size
    for L in seq_lens:
        if int(L) < 1 or int(L) > cap_tokens:
            raise PlanError("SEQ_LEN", f"seq_len {L} outside [1, {cap_tokens}]")
    per_cu = budget_per_cu if budget_per_cu > 0 else DEFAULT_BUDGET_PER_CU
    if wave_slots_per_cu and budget_per_cu <= 0:   # the MI355X default above
        per_cu = 4 * (num_q_heads // num_kv_heads)
    budget = per_cu * cu_count
    cap = scratch_cap_bytes if scratch_cap_bytes > 0 else DEFAULT_SCRATCH_CAP
    max_len = max(int(L) for L in seq_lens)
    if partition_request == 0:
        return dict(partition_size=0, max_num_partitions=1, work_full_parts=0, budget=budget,
                    cu_count=cu_count, scratch_bytes=0)
    if partition_request == -1:
        P = 512 if work_full_partitions(seq_lens, num_q_heads, 512) >= budget else 256
        if wave_slots_per_cu and P == 512:   # the MI355X regime above
            slots = wave_slots_per_cu * cu_count
            items = lambda p: S * num_kv_heads * -(-max_len // p)
            if 2 * items(1024) <= slots:
                P = 1024
        # MI355X default budget: 1024 first once its full partitions give 2
        # workgroups (KV head, partition) per CU
        if wave_slots_per_cu and budget_per_cu <= 0 and \
                num_kv_heads * sum(int(L) // 1024 for L in seq_lens) >= 2 * cu_count:
            P = 1024
    else:
        P = partition_request
    NP = -(-max_len // P)
    scratch = S * num_q_heads * NP * (head_dim + 2) * 4
    if scratch > cap:
        raise PlanError("SCRATCH_CAP", f"{scratch} bytes over cap {cap}")
    return dict(partition_size=P, max_num_partitions=NP,
                work_full_parts=work_full_partitions(seq_lens, num_q_heads, P),
                budget=budget, cu_count=cu_count, scratch_bytes=scratch)
