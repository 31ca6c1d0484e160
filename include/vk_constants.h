/*
 * Compile-time constants shared by the host library and the HIP kernels of
 * libvkpaged, so that the two sides cannot drift apart.
 *
 * Sources (vllm-metal kernels page, cf-1.com/news/5525226):
 *  - section "三大 Metal 内核": a default KV partition of 512 tokens and page
 *    sizes 32, 16 and 8 are shared constants baked into both host and kernel;
 *  - section "GQA 解码内核的四个提速技巧", item 4: split-KV partitions of 256
 *    or 512 tokens;
 *  - section "分发层": the admitted (query heads, KV heads, head dim) triples,
 *    a fixed work budget of 33 simdgroups per GPU core, and a 512 MiB cap on
 *    the scratch of one attention call.
 */
#ifndef VK_CONSTANTS_H
#define VK_CONSTANTS_H

#define VK_PARTITION_LARGE 512
#define VK_PARTITION_SMALL 256
/* A third, larger partition (an MI355X addition: half the partials of 512).
 * vk_plan_partitions takes it first under its default budget once the full
 * 1024-token partitions give VK_DECODE_XLARGE_WG_PER_CU workgroups per CU,
 * and upgrades 512 to it when the 1024-token launch fits one round of the
 * wave slots with two or more waves per partition; vk_plan_varlen tries it
 * first for column tiles of several query tokens.  Every split entry point
 * accepts it. */
#define VK_PARTITION_XLARGE 1024

#define VK_DEFAULT_BUDGET_PER_CU 33
/* The decode planner's default budget, an MI355X calibration (not from the
 * pages): 4 workgroups per CU, one workgroup serving the G = Hq / Hkv query
 * heads of a KV head, i.e. 4 * G query-head units per CU in the pages' rule.
 * Timed over 56 grouped-query batches (two runs) it lost 28-32 us against
 * the faster partition size in all, the pages' 33 units per CU 43-45 us;
 * over 36 multi-head and multi-query batches 158 us against 231 us. */
#define VK_DECODE_BUDGET_WG_PER_CU 4
/* With the default budget the decode planner tries 1024-token partitions
 * first: taken once their full partitions give this many workgroups per CU
 * (MI355X calibration, not from the pages). */
#define VK_DECODE_XLARGE_WG_PER_CU 2
#define VK_DEFAULT_SCRATCH_CAP (512ull * 1024ull * 1024ull)

/* Admitted geometries (Hq, Hkv, D): the four grouped-query triples of the
 * dispatch layer, then multi-head (Hkv = Hq) and multi-query (Hkv = 1)
 * triples (the vllm-metal page's prefill path names MHA, GQA and MQA).
 * Eight geometries x three page sizes give 24 kernel specialisations. */
#define VK_NUM_GEOMETRIES 8
#define VK_GEOMETRY_LIST {{32, 8, 128}, {24, 4, 256}, {16, 2, 128}, {16, 2, 256}, \
                          {16, 16, 128}, {8, 8, 256}, {16, 1, 128}, {16, 1, 256}}
#define VK_NUM_BLOCK_SIZES 3
#define VK_BLOCK_SIZE_LIST {8, 16, 32}

/* Size of the device array that holds the split-KV partials of
 * vk_paged_gqa_decode_noalloc (one per GPU, for the life of the process):
 * 64 MiB, enough for num_seqs * num_q_heads * max_num_partitions * (head_dim
 * + 2) * 4 bytes of scratch up to about 16 M floats (e.g. 32 sequences of 16k
 * tokens at (24, 4, 256) and partition 256: 51 MB). */
#define VK_NOALLOC_SCRATCH_BYTES (64ull * 1024ull * 1024ull)

/* A KV page id outside [0, num_blocks), or a device seq_len the page table
 * cannot hold, never reaches memory: the kernel reads page 0 instead and the
 * affected (sequence, head) results become NaN. */

#endif /* VK_CONSTANTS_H */
