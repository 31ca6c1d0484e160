/*
 * libvkpaged — single-token (decode) grouped-query attention over a paged fp16
 * KV cache, for AMD Instinct MI355X (gfx950).  Plain C ABI: raw pointers and
 * sizes, no C++ or framework types.
 *
 * What is computed (vllm-metal kernels page, cf-1.com/news/5525226):
 *  - section "什么是 Paged Attention": the KV cache is split into fixed-size
 *    pages; block_tables maps each logical page of a sequence to a physical
 *    page of a shared pool;
 *  - section "Metal 并行模型": one workgroup per (partition, KV head,
 *    sequence), holding every query head of that KV head's group, so a K/V
 *    page is fetched once for the whole group;
 *  - section "GQA 解码内核的四个提速技巧": (1) online softmax in log2 space
 *    (log2 e folded into the scale, every exponential an exp2, running max
 *    and exp-sum kept in registers, one pass over K/V); (2) the loop advances
 *    page by page with the page id read once and shared by the wave, and K/V
 *    are read straight from device memory; (3) several tokens in flight per
 *    loop step, with a masked tail; (4) split-KV partitions of 256 or 512
 *    tokens whose partial results are (max in log2 units, exp-sum, output
 *    normalised by that exp-sum), merged by a separate reduce step;
 *  - section "分发层": admitted geometries, a partition-size choice against a
 *    work budget of 33 per core that counts only full partitions, and a
 *    512 MiB scratch cap.
 * For each sequence s, query head h (KV head g = h / (Hq/Hkv)) and the
 * L = seq_lens[s] tokens t < L:
 *     z_t = scale * (q[s,h,:] . K[block_tables[s][t/bs], g, t%bs, :])
 *     out[s,h,:] = sum_t softmax(z)_t * V[block_tables[s][t/bs], g, t%bs, :]
 *
 * Memory layouts (all row-major, element strides implied by the sizes):
 *   q             fp16  [num_seqs, num_q_heads, head_dim]
 *   k_cache       fp16  [num_blocks, num_kv_heads, block_size, head_dim]
 *   v_cache       fp16  [num_blocks, num_kv_heads, block_size, head_dim]
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; only the first
 *                 ceil(L/block_size) entries of a row are ever read
 *   seq_lens      int32 [num_seqs]
 *   out           fp32  [num_seqs, num_q_heads, head_dim]
 *   max_logits    fp32  [num_seqs, num_q_heads, max_num_partitions]
 *   exp_sums      fp32  [num_seqs, num_q_heads, max_num_partitions]
 *   tmp_out       fp32  [num_seqs, num_q_heads, max_num_partitions, head_dim]
 *   counters      uint32 [num_seqs, num_kv_heads] (single-launch form only)
 *
 * Ownership and asynchrony: every tensor pointer is device memory owned by the
 * caller.  The library allocates nothing, frees nothing and keeps no pointer
 * after a call returns.  GPU calls only enqueue work on `stream` (a
 * hipStream_t; NULL = the default stream) and never synchronise; the caller
 * keeps buffers alive until that work has finished and must enqueue
 * vk_paged_gqa_reduce on the same stream after vk_paged_gqa_decode.
 *
 * Alignment: q, k_cache, v_cache, out and tmp_out are read and written in
 * 16-byte vectors and must be 16-byte aligned; the int32 and fp32 arrays
 * (block_tables, seq_lens, cu_seqlens_q, max_logits, exp_sums, counters)
 * 4-byte aligned; VK_ERR_ALIGN otherwise.  (torch allocations are 256-byte
 * aligned; a view that starts mid-row may not be.)
 *
 * Errors: every function returns a vk_status.  All argument validation is
 * host-only and happens before any HIP call, so a rejected call launches
 * nothing and writes nothing.  A failed launch returns VK_ERR_HIP and
 * vk_last_hip_error() returns the HIP error code.  Device-side values the
 * host cannot see (seq_lens and block_tables contents) are guarded in the
 * kernels: an entry outside [0, num_blocks), or a length above
 * max_blocks_per_seq*block_size or above max_num_partitions*partition_size,
 * makes the affected outputs NaN instead of reading out of bounds; a length
 * <= 0 yields zeros.
 *
 * Thread safety: all functions are re-entrant; the only state is
 * thread-local diagnostics (vk_last_plan, vk_last_hip_error).
 */
#ifndef VK_PAGED_H
#define VK_PAGED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vk_status;
enum {
    VK_OK = 0,
    VK_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
    VK_ERR_BAD_DIM = 2,     /* a size is non-positive or inconsistent */
    VK_ERR_GEOMETRY = 3,    /* (Hq, Hkv, D) is not an admitted geometry */
    VK_ERR_BLOCK_SIZE = 4,  /* block_size not in {8, 16, 32} */
    VK_ERR_PARTITION = 5,   /* partition size or count not allowed */
    VK_ERR_SEQ_LEN = 6,     /* a host seq_len is < 1 or beyond the page table */
    VK_ERR_SCRATCH_CAP = 7, /* split-KV scratch would exceed the cap */
    VK_ERR_HIP = 8,         /* a HIP runtime call or launch failed */
    VK_ERR_DTYPE = 9,       /* element type not supported by this entry point */
    VK_ERR_ALIGN = 10       /* a device pointer is not aligned as its kernel reads it */
};

/* Element type of q, K and V (vk_paged_gqa_decode_dt). */
enum {
    VK_DTYPE_F16 = 0,
    VK_DTYPE_BF16 = 1,
    VK_DTYPE_F32 = 2
};

/* Decode kernel families; see vk_select_decode_kernel. */
enum {
    VK_KERNEL_AUTO = 0,
    VK_KERNEL_DOT = 1,      /* VALU: lane-sliced fp16 dot2 products, DPP reductions */
    VK_KERNEL_MFMA = 2,     /* matrix cores for QK and PV; waves per workgroup chosen */
    VK_KERNEL_MFMA_W1 = 3,  /* matrix cores, 1 wave64 per workgroup (A/B tuning) */
    VK_KERNEL_MFMA_W2 = 4,  /* matrix cores, 2 wave64s per workgroup (A/B tuning) */
    VK_KERNEL_MFMA_W4 = 5,  /* matrix cores, 4 wave64s per workgroup (A/B tuning) */
    VK_KERNEL_MFMA_W4P2 = 6, /* matrix cores, 4 wave64s per workgroup over two
                               consecutive partitions, two waves each (split
                               launches; A/B tuning) */
    /* vk_paged_gqa_varlen kernels; see vk_select_varlen_kernel */
    VK_KERNEL_VARLEN_COLUMNS = 7, /* one wave per 16 (token, head) columns, keys
                                     streamed through registers */
    VK_KERNEL_VARLEN_TILES = 8    /* four waves per 128 columns, keys staged in
                                     LDS tiles shared by all of them */
};

/* Work order of the matrix-core decode (and of the multi-token column kernel
 * when every sequence's queries fit one of its tiles); see
 * vk_select_work_order. */
enum {
    VK_ORDER_AUTO = 0,           /* longest first when the split grid over <= 64
                                    sequences takes more than one round of the
                                    device's resident wave slots; else grid
                                    order */
    VK_ORDER_GRID = 1,           /* (partition, KV head, sequence) in launch order */
    VK_ORDER_LONGEST_FIRST = 2   /* split, <= 64 sequences: full partitions, then
                                    ragged ones by decreasing length */
};

typedef struct vk_plan {
    int32_t  partition_size;     /* 0 = unsplit, else 256, 512 or 1024 */
    int32_t  max_num_partitions; /* NP = ceil(max_s L_s / P); 1 when unsplit */
    int64_t  work_full_parts;    /* W(P) = Hq * sum_s floor(L_s / P) at the chosen P */
    int64_t  budget;             /* budget_per_cu * cu_count */
    int32_t  cu_count;           /* compute units the budget was sized for */
    int32_t  kernel;             /* decode: VK_KERNEL_DOT or VK_KERNEL_MFMA_W* that ran; planner: 0 */
    uint64_t scratch_bytes;      /* S * Hq * NP * (D + 2) * 4 */
    int32_t  grid[3];            /* decode: launch grid (partitions, Hkv, S); partitions
                                    halved (rounded up) for VK_KERNEL_MFMA_W4P2 */
    int32_t  block;              /* decode: threads per workgroup */
    int32_t  work_order;         /* decode: VK_ORDER_GRID or VK_ORDER_LONGEST_FIRST used */
} vk_plan;

/*
 * vk_plan_partitions — choose the split-KV partition size for one call.
 * Host-only: makes no HIP call when cu_count > 0.
 *
 * Rule (vllm-metal kernels page, section "分发层", read as stated in the
 * design notes): budget B = budget_per_cu * cu_count.  Work W(P) =
 * Hq * sum_s floor(L_s / P) counts only full partitions.  With
 * partition_request == -1 the planner picks P = 512 when W(512) >= B, else
 * P = 256.  The default budget is an MI355X calibration, not the pages' 33:
 * 4 * G units per CU (G = Hq / Hkv), i.e. P = 512 once the full 512-token
 * partitions give 4 workgroups per CU.  Then, not from the pages (MI355X
 * additions): 512 becomes VK_PARTITION_XLARGE = 1024 when the 1024 launch
 * fits in a single round of the device's 8 * cu_count resident waves with
 * at least two waves per partition (2 * S * Hkv * ceil(max L / 1024) <=
 * 8 * cu_count): half the partials, longer streams per wave; and with the
 * default budget 1024 is taken first whenever Hkv * sum_s floor(L_s / 1024)
 * >= 2 * cu_count (two workgroups of full 1024-token partitions per CU).
 * 0 asks for the unsplit path; 256, 512 or 1024 forces that size.  NP = ceil(max L / P); scratch = S*Hq*NP*(D+2)*4 bytes, which must not
 * exceed the cap (no fallback path exists).
 *
 *   seq_lens_host       host int32 [num_seqs], each in [1, max_blocks_per_seq*block_size]
 *   cu_count            compute units; 0 = query the current HIP device
 *   budget_per_cu       query-head units per CU; 0 = 4 * Hq / Hkv (four
 *                       workgroups of full 512-token partitions per CU, an
 *                       MI355X calibration; the pages' constant is 33)
 *   scratch_cap_bytes   0 = 512 MiB
 *   plan_out            host struct, written on VK_OK only
 * Also recorded as this thread's vk_last_plan.
 */
vk_status vk_plan_partitions(const int32_t* seq_lens_host, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq,
                             int32_t partition_request, int32_t cu_count,
                             int32_t budget_per_cu, uint64_t scratch_cap_bytes,
                             vk_plan* plan_out);

/*
 * vk_paged_gqa_decode — the decode kernel: for every (partition, KV head,
 * sequence) one workgroup reads that KV head's pages of the partition once and
 * serves all its query heads.
 *
 * partition_size == 0 (unsplit): each workgroup covers a whole sequence and
 *   writes out[s, h, :] directly; max_logits/exp_sums/tmp_out may be NULL and
 *   max_num_partitions must be 1.
 * partition_size == 256, 512 or 1024 (split): partition i covers tokens
 *   [i*P, min(L, (i+1)*P)); for each i < ceil(L/P) it writes
 *     max_logits[s,h,i] = max over the partition of z_t * log2(e)
 *     exp_sums[s,h,i]   = sum over the partition of 2^(z_t*log2(e) - max)
 *     tmp_out[s,h,i,:]  = (sum 2^(z_t*log2(e) - max) * v_t) / exp_sums
 *   and nothing for i >= ceil(L/P); `out` is not touched (may be NULL).
 *   Requires max_num_partitions >= ceil(max L / P) (see vk_plan_partitions).
 * scale is the softmax scale (usually 1/sqrt(head_dim)); the kernel applies
 * scale*log2(e) (rounded once to fp32) to the fp32 dot products.
 */
vk_status vk_paged_gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size,
                              int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                              int32_t partition_size, int32_t max_num_partitions,
                              float* out, float* max_logits, float* exp_sums, float* tmp_out,
                              void* stream);

/*
 * vk_paged_gqa_decode_dt — vk_paged_gqa_decode for another element type of
 * q, k_cache and v_cache (one type for all three; the partials and `out` stay
 * fp32 and are merged by the same vk_paged_gqa_reduce).  The voxtral.c page,
 * dpshk.com/news/5521762, keeps fp32 as the fallback of its fp16 KV cache.
 *   VK_DTYPE_F16   the fp16 path of vk_paged_gqa_decode
 *   VK_DTYPE_BF16  bfloat16: the matrix-core family, scores exact products
 *                  accumulated in fp32 as for fp16; each softmax weight enters
 *                  the PV product as a bf16 value plus its bf16 residual
 *   VK_DTYPE_F32   fp32: the fp32 matrix-core products (v_mfma 16x16x4 f32)
 * Layouts as for fp16 with the element size of the type.  VK_ERR_DTYPE for
 * any other value.  Non-fp16 types always run the matrix-core family with
 * one partition per workgroup (a VALU or two-partition selection is ignored).
 */
vk_status vk_paged_gqa_decode_dt(int32_t dtype, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                 int32_t partition_size, int32_t max_num_partitions, float* out,
                                 float* max_logits, float* exp_sums, float* tmp_out,
                                 void* stream);

/*
 * vk_paged_gqa_reduce — merge the split-KV partials (vllm-metal kernels page,
 * section "GQA 解码内核的四个提速技巧", item 4: the GQA path reuses the
 * split-KV reducer).  For each (s, h) with n = ceil(L/P) partitions:
 *     M = max_i max_logits[i];  w_i = exp_sums[i] * 2^(max_logits[i] - M)
 *     out[s,h,:] = sum_i w_i * tmp_out[i,:] / sum_i w_i
 * reading only i < n (n == 1 copies tmp_out[0] exactly).  L <= 0 writes
 * zeros.  head_dim must be 128 or 256; partition_size 256, 512 or 1024.
 */
vk_status vk_paged_gqa_reduce(const float* max_logits, const float* exp_sums,
                              const float* tmp_out, const int32_t* seq_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t head_dim, int32_t partition_size,
                              int32_t max_num_partitions, float* out, void* stream);

/*
 * vk_paged_gqa_decode_fused — decode and reduce in one launch (the voxtral.c
 * page, dpshk.com/news/5521762, sections "模型结构与解码瓶颈" and "融合内核如何
 * 工作": a token-by-token decode step pays per launch, and fusing small
 * kernels cuts launches and buffer round trips; vllm-metal kernels page,
 * section "GQA 解码内核的四个提速技巧", item 4: the partials are merged by the
 * same split-KV reduction).
 *
 * Arguments are those of vk_paged_gqa_decode, plus
 *   counters   uint32 [num_seqs * num_kv_heads], device, owned by the caller;
 *              required when partition_size > 0, ignored (may be NULL) when 0.
 *              Must be all zero before the first call; every completed call
 *              leaves it all zero again, so one buffer serves any number of
 *              later calls on the same stream without clearing.  Calls that
 *              overlap in time on one counter buffer (different streams) race.
 * and `out` is always required: it receives the final normalised result
 *   out[s,h,:] for every (s, h), as after vk_paged_gqa_decode followed by
 *   vk_paged_gqa_reduce (same formula; the summation order differs).
 * Split: each workgroup writes its partial triple to max_logits/exp_sums/
 *   tmp_out as in vk_paged_gqa_decode, then counts itself in
 *   counters[s * num_kv_heads + g]; the last of the ceil(L/P) workgroups of
 *   (s, g) merges them into out.  A sequence with one partition writes out
 *   directly and leaves its scratch rows untouched.  L <= 0 writes zeros.
 * The merge is done by one workgroup per (s, KV head), so the form suits few
 * partitions per sequence (short and medium contexts, where the second
 * launch is a large share of the step).  With max_num_partitions > 8 the
 * call enqueues vk_paged_gqa_decode and vk_paged_gqa_reduce instead (two
 * launches, the same partials and the same output; counters untouched), since
 * the separate reduce spreads the merge over more workgroups.  Always runs
 * the matrix-core family (VK_KERNEL_DOT selects the automatic choice here).  Errors and
 * device-side guards are those of vk_paged_gqa_decode; additionally
 * VK_ERR_NULL_ARG if out is NULL, or counters is NULL with partition_size > 0.
 */
vk_status vk_paged_gqa_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                    int32_t partition_size, int32_t max_num_partitions,
                                    float* out, float* max_logits, float* exp_sums,
                                    float* tmp_out, uint32_t* counters, void* stream);

/*
 * vk_paged_gqa_decode_noalloc — vk_paged_gqa_decode followed by
 * vk_paged_gqa_reduce (same kernels, same launch choices, same result bit for
 * bit) with the split-KV partials held in a device array of the library
 * instead of caller buffers, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The call allocates and frees nothing.
 *
 * Arguments are those of vk_paged_gqa_decode without the three scratch
 * pointers; `out` (fp32 [num_seqs, num_q_heads, head_dim]) is always required
 * and receives the final normalised result.  partition_size 0 runs the
 * unsplit decode into out (no scratch); 256, 512 or 1024 writes the partials into
 * the array and merges them into out.  The partials (num_seqs * num_q_heads *
 * max_num_partitions * (head_dim + 2) * 4 bytes, plus alignment) must fit
 * VK_NOALLOC_SCRATCH_BYTES (64 MiB, vk_constants.h): larger calls return
 * VK_ERR_SCRATCH_CAP before any HIP call.
 * The array is one per GPU, held until the process ends, and shared by every
 * call on that GPU: calls that overlap in time on one GPU (other streams,
 * other threads) race on it and must be serialised by the caller.  Nothing in
 * it needs clearing between calls (every partial the merge reads is written
 * by the same call).  The first call on a device looks up that device's copy
 * (VK_ERR_HIP if the lookup fails).  Other errors and device-side guards are
 * those of vk_paged_gqa_decode and vk_paged_gqa_reduce.
 */
vk_status vk_paged_gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                      int32_t partition_size, int32_t max_num_partitions,
                                      float* out, void* stream);

/*
 * vk_plan_varlen — plan a vk_paged_gqa_varlen call (host only; no HIP call
 * when cu_count > 0).  seq_lens_host[s] (>= 1, within the page table) counts
 * all of sequence s's cached tokens including its q_lens_host[s] new query
 * tokens (0 <= q_len <= seq_len).  The kernel follows vk_select_varlen_kernel
 * and is reported in plan_out->kernel.  A tile covers (query token, head)
 * columns of one KV head's G heads and runs on w waves: for
 * VK_KERNEL_VARLEN_COLUMNS T = 16 / G whole tokens, w = 1, so a sequence has
 * t_s = ceil(q_len / T) tiles; for VK_KERNEL_VARLEN_TILES 128 consecutive
 * columns in token-major order (across token boundaries where G does not
 * divide 128), w = 4 at head_dim 128 and 8 at head_dim 256, so
 * t_s = ceil(q_len * G / 128).
 * With n = Hkv * sum t_s tiles and partition_request == -1 the
 * call is unsplit when the tiles alone give one wave per wave slot
 * (w * n >= 8 * cu_count), otherwise split at the largest P whose full-
 * partition work W(P) = Hq * sum_s t_s * floor(L_s / P)
 * reaches 33 * cu_count, else at 256 (vk_plan_partitions' rule, whose unit
 * is a (query head, full partition) pair, counted for every tile).  The
 * sizes tried are 512 and, for column tiles when some sequence brings more
 * than one query token, first VK_PARTITION_XLARGE = 1024 (an MI355X
 * addition: half the partials of 512); with one query token per sequence
 * the two planners agree, except where vk_plan_partitions upgrades 512 to
 * 1024 for two-wave partitions (the column kernel keeps 512).  When that
 * split's scratch would exceed the cap,
 * the next larger size, and failing that unsplit.  partition_request may
 * force 256, 512 or 1024.
 * NP = ceil(max L / P); scratch = total_q * Hq * NP * (D + 2) * 4 bytes
 * against the cap (an explicit partition request over it is an error).  Errors: those of vk_plan_partitions; VK_ERR_SEQ_LEN for a
 * q_len outside [0, seq_len]; VK_ERR_BAD_DIM if a q_len exceeds 65535.
 */
vk_status vk_plan_varlen(const int32_t* seq_lens_host, const int32_t* q_lens_host,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int32_t partition_request, int32_t cu_count, uint64_t scratch_cap_bytes,
                         vk_plan* plan_out);

/*
 * vk_paged_gqa_varlen — several query tokens per sequence, causal, over the
 * paged cache: speculative-decode verification and chunked prefill (the
 * vllm-metal kernels page, section "什么是 Paged Attention": a unified paged
 * variable-length kernel serves prefill and speculative decoding).
 *
 *   q              fp16 [total_q, Hq, D], the query rows of all sequences
 *                  packed in sequence order
 *   cu_seqlens_q   int32 [num_seqs + 1], device: sequence s owns rows
 *                  cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 (non-decreasing,
 *                  first 0, last total_q)
 *   seq_lens       int32 [num_seqs], device: cached tokens of s, its new
 *                  query tokens included (they are the last q_len of them,
 *                  written beforehand, e.g. with vk_paged_kv_append)
 *   max_q_len      host: the largest q_len (sets the grid; rows of a longer
 *                  sequence would not be computed)
 *   out            fp32 [total_q, Hq, D] (unsplit)
 *   max_logits, exp_sums  fp32 [total_q, Hq, NP]; tmp_out fp32
 *                  [total_q, Hq, NP, D] (split), as for vk_paged_gqa_decode
 * Query j of sequence s attends to tokens t < L_s - q_len_s + j + 1 with the
 * decode's scores and log2-space softmax; a row that sees no token is zeros.
 * Split (partition_size 256, 512 or 1024): partition i of row j is written
 * for i < ceil((L - q_len + j + 1) / P) and merged by
 * vk_paged_gqa_varlen_reduce on the same stream.  Geometries,
 * block sizes, errors and device-side guards as for vk_paged_gqa_decode (a
 * sequence longer than the page table gives NaN rows and reads nothing);
 * VK_ERR_BAD_DIM for total_q or max_q_len outside [1, 65535] or max_q_len >
 * total_q.
 */
vk_status vk_paged_gqa_varlen(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t total_q,
                              int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, int32_t partition_size,
                              int32_t max_num_partitions, float* out, float* max_logits,
                              float* exp_sums, float* tmp_out, void* stream);

/*
 * vk_paged_gqa_varlen_dt — vk_paged_gqa_varlen with the element type of q,
 * k_cache and v_cache given by dtype: VK_DTYPE_F16 or VK_DTYPE_BF16 (bf16 as
 * in vk_paged_gqa_decode_dt: the same steps on the bf16 matrix instructions,
 * each softmax weight taken through PV as a bf16 value plus its bf16
 * residual).  Same layouts in elements, outputs and partials fp32.  Errors:
 * those of vk_paged_gqa_varlen; VK_ERR_DTYPE for any other dtype (fp32
 * q/K/V run only through the single-token decode).
 */
vk_status vk_paged_gqa_varlen_dt(int32_t dtype, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                                 int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                                 float scale, int32_t partition_size, int32_t max_num_partitions,
                                 float* out, float* max_logits, float* exp_sums, float* tmp_out,
                                 void* stream);

/*
 * vk_paged_gqa_varlen_reduce — the merge of vk_paged_gqa_reduce for
 * variable-length rows: row cu_seqlens_q[s] + j merges its
 * n = min(ceil((L - q_len + j + 1) / P), NP) partitions into out
 * [total_q, Hq, D]; a row that sees no token is zeros.  P is 256, 512 or
 * 1024 (VK_ERR_PARTITION otherwise).
 */
vk_status vk_paged_gqa_varlen_reduce(const float* max_logits, const float* exp_sums,
                                     const float* tmp_out, const int32_t* seq_lens,
                                     const int32_t* cu_seqlens_q, int32_t num_seqs,
                                     int32_t max_q_len, int32_t num_q_heads, int32_t head_dim,
                                     int32_t partition_size, int32_t max_num_partitions,
                                     float* out, void* stream);

/*
 * vk_paged_kv_append — write each sequence's new token into the paged cache
 * (vllm-metal kernels page, section "什么是 Paged Attention": the token at
 * position pos of sequence s lives in physical page block_tables[s][pos/bs],
 * slot pos % bs; the voxtral.c page, dpshk.com/news/5521762, sections
 * "模型结构与解码瓶颈" and "下一步优化方向": every decode step writes the new
 * K/V, and rotary embedding of K is fused into that write).
 *
 *   k_new, v_new   fp16 [num_seqs, num_kv_heads, head_dim], device
 *   positions      int32 [num_seqs], device: the token's index in its
 *                  sequence (the sequence length before the append); a
 *                  negative position skips the sequence
 *   rope_theta     <= 0: K is copied as is; > 0: each pair (d, d + D/2) of K
 *                  is rotated by pos * rope_theta^(-2d/D) (rotate-half form),
 *                  computed in float64 and rounded once to fp16
 *   k_cache, v_cache  the pools of vk_paged_gqa_decode, written in place
 * Only slot (block_tables[s][pos/bs], pos % bs) of each KV head is written.
 * Device-side values the host cannot see are guarded: a position at or past
 * max_blocks_per_seq*block_size, or a page id outside [0, num_blocks),
 * writes nothing for that sequence.  head_dim must be even and at most 256;
 * the geometry need not be one of the decode's admitted ones.
 */
vk_status vk_paged_kv_append(const void* k_new, const void* v_new, const int32_t* block_tables,
                             const int32_t* positions, int32_t num_seqs, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, double rope_theta, void* k_cache, void* v_cache,
                             void* stream);

/*
 * vk_select_decode_kernel — A/B switch for this thread's later decode calls
 * (vllm-metal kernels page, cf-1.com/news/5525226, section "上手实践：如何验证
 * 内核生效": an environment switch sends eligible requests back to the
 * classic path so the two can be compared; here the switch is a call, per
 * thread, and selects a kernel family or a wave count).  VK_KERNEL_AUTO
 * picks the fastest family for the geometry.  Returns the previous setting,
 * or -1 for an unknown value (setting kept).
 */
int32_t vk_select_decode_kernel(int32_t kernel);

/*
 * vk_select_work_order — A/B switch (as vk_select_decode_kernel: vllm-metal
 * kernels page, section "上手实践：如何验证内核生效") for the order in which this thread's
 * later matrix-core decode launches hand out their (partition, KV head,
 * sequence) items.  Longest first applies only to split launches over at most
 * 64 sequences (others run in grid order whatever the setting), and to the
 * multi-token column kernel's split launches when one tile holds every
 * sequence's queries (the same items; write-through partials come with it
 * there).  VK_ORDER_LONGEST_FIRST also puts unsplit LDS-tiled multi-token
 * launches over at most 64 sequences in global longest-first order of their
 * (sequence, tile) items (decreasing key range; VK_ORDER_AUTO keeps grid
 * order there, measured faster).  It changes
 * which workgroup computes which partial or row, never a result.  Returns the
 * previous setting, or -1 for an unknown value (setting kept).
 */
int32_t vk_select_work_order(int32_t order);

/*
 * vk_select_varlen_kernel — A/B switch (as vk_select_decode_kernel: vllm-metal
 * kernels page, section "上手实践：如何验证内核生效") for this thread's later
 * vk_plan_varlen and vk_paged_gqa_varlen calls: VK_KERNEL_AUTO (columns
 * when the longest query run of the batch fits one 16-column tile, i.e. is
 * at most 16 / G tokens for G = Hq / Hkv, so every K/V step is read once;
 * tiles above that: measured on MI355X for G = 4, 6, 8),
 * VK_KERNEL_VARLEN_COLUMNS or VK_KERNEL_VARLEN_TILES.
 * Both kernels compute the same rows to the same tolerance; the planner's
 * split rule depends on the kernel, so plan and launch under the same
 * setting.  Returns the previous setting, or -1 for an unknown value
 * (setting kept).
 */
int32_t vk_select_varlen_kernel(int32_t kernel);

/* Human-readable name of a status code (static storage). */
const char* vk_status_string(vk_status s);

/* HIP error code of this thread's last VK_ERR_HIP (0 if none). */
int32_t vk_last_hip_error(void);

/* 1 when the environment variable VK_TRACE is set (and not "0") and a
 * roctx library could be loaded, else 0.  Then every entry point that enqueues
 * work (the decode, reduce, multi-token and append calls) opens a roctx range
 * named after itself for the length of the call, which rocprofv3
 * --marker-trace records beside the kernels (the vllm-metal kernels page,
 * section "上手实践：如何验证内核生效": confirm in a trace which kernels a
 * request ran).  The library does not link a roctx library: the
 * rocprofiler-sdk one (librocprofiler-sdk-roctx.so.1), else libroctx64, is
 * loaded at the first call, and without either tracing stays off (VK_LOG
 * reports that once).  The setting is read once per process. */
int32_t vk_trace_enabled(void);

/* This thread's last plan: from vk_plan_partitions or vk_plan_varlen, or
 * the launch shape of the last decode or multi-token launch (vllm-metal
 * kernels page, section "上手实践：如何验证内核生效": after a request the
 * runtime reports which path the last dispatch took and the partition size,
 * 256 or 512, it actually ran; here partition_size, kernel, grid, block and
 * work_order).  Copied into *out, a caller-owned host struct; returns
 * VK_ERR_NULL_ARG if out is NULL (the status return keeps every call of this
 * ABI on one error convention).  Before any plan or launch on this thread,
 * *out is all zero. */
vk_status vk_last_plan(vk_plan* out);

#ifdef __cplusplus
}
#endif

#endif /* VK_PAGED_H */
