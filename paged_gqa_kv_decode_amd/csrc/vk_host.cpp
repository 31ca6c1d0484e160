// C-ABI entry points of libvkpaged: validation, partition planning and kernel
// dispatch.  Everything here is host code; it launches on the caller's stream
// and never synchronises.  Validation is complete before the first HIP call.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <initializer_list>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "vk_constants.h"
#include "vk_kernels.h"
#include "vk_paged.h"

namespace {

thread_local vk_plan t_last_plan = {};
thread_local int32_t t_last_hip_error = 0;
thread_local int32_t t_kernel_choice = VK_KERNEL_AUTO;
thread_local int32_t t_order_choice = VK_ORDER_AUTO;
thread_local int32_t t_varlen_choice = VK_KERNEL_AUTO;

// The multi-token kernel for a batch whose longest query run is max_q tokens,
// G = `group` query heads per KV head.  Measured on MI355X (32 sequences of
// 4k-16k tokens, G = 4, 6, 8): the column kernel is faster while one of its
// 16-column tiles (16 / G tokens x G heads) holds every sequence's queries,
// so each K/V step is read once and used straight from the prefetch slots
// (G = 4, 4 tokens: 281 vs 344 us); with more tokens it reads the keys once
// per tile and the LDS-tiled kernel, which shares them among 128 columns,
// wins (G = 6, 4 tokens: 531 vs 365 us).
int32_t varlen_kernel(int64_t max_q, int group) {
    if (t_varlen_choice != VK_KERNEL_AUTO) return t_varlen_choice;
    return max_q > vk::varlen_tokens_per_tile(group) ? VK_KERNEL_VARLEN_TILES
                                                     : VK_KERNEL_VARLEN_COLUMNS;
}

struct Geometry {
    int hq, hkv, d;
};
constexpr Geometry kGeometries[VK_NUM_GEOMETRIES] = VK_GEOMETRY_LIST;
constexpr int kBlockSizes[VK_NUM_BLOCK_SIZES] = VK_BLOCK_SIZE_LIST;

bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("VK_LOG");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

// VK_TRACE=1: every entry point that enqueues work opens a roctx range named
// after itself for the length of the call (rocprofv3 --marker-trace lists the
// ranges beside the kernels they launched).  The roctx library is looked up
// at the first call, so the library has no link-time dependency on it; if it cannot
// be loaded, tracing stays off (and VK_LOG says so once).
struct Roctx {
    int (*push)(const char*) = nullptr;
    int (*pop)() = nullptr;
};

const Roctx& roctx() {
    static const Roctx r = [] {
        Roctx x;
        const char* e = std::getenv("VK_TRACE");
        if (!e || !e[0] || e[0] == '0') return x;
        // rocprofv3 records the rocprofiler-sdk roctx library's ranges; the
        // older libroctx64 (same two functions) serves older tools.
        void* h = nullptr;
        for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so",
                                "libroctx64.so.4", "libroctx64.so"})
            if (!h) h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
        if (h) {
            x.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
            x.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
            if (!x.push || !x.pop) x = Roctx();
        }
        if (!x.push && log_enabled()) std::fprintf(stderr, "[vk] VK_TRACE: no roctx library found, tracing off\n");
        return x;
    }();
    return r;
}

class TraceRange {
public:
    explicit TraceRange(const char* name) : on_(roctx().push != nullptr) {
        if (on_) roctx().push(name);
    }
    ~TraceRange() {
        if (on_) roctx().pop();
    }
    TraceRange(const TraceRange&) = delete;
    TraceRange& operator=(const TraceRange&) = delete;

private:
    bool on_;
};

// Null pointers pass (their own checks decide whether they are allowed).
bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

bool vectors_aligned(std::initializer_list<const void*> v16, std::initializer_list<const void*> v4) {
    for (const void* p : v16)
        if (!aligned(p, 16)) return false;
    for (const void* p : v4)
        if (!aligned(p, 4)) return false;
    return true;
}

vk_status geometry_status(int32_t hq, int32_t hkv, int32_t d) {
    if (hq <= 0 || hkv <= 0 || d <= 0) return VK_ERR_BAD_DIM;
    if (hq % hkv != 0) return VK_ERR_GEOMETRY;
    for (const Geometry& g : kGeometries)
        if (g.hq == hq && g.hkv == hkv && g.d == d) return VK_OK;
    return VK_ERR_GEOMETRY;
}

bool block_size_ok(int32_t bs) {
    for (int b : kBlockSizes)
        if (b == bs) return true;
    return false;
}

vk_status hip_fail(hipError_t e) {
    t_last_hip_error = static_cast<int32_t>(e);
    return VK_ERR_HIP;
}

// Resident wave slots of the current device for the matrix-core decode:
// CUs x 4 SIMDs x 2 waves (its register budget allows two waves per SIMD).
// The CU count is queried once per device; 2048 (256 CUs) if the query fails.
// Largest partition count per sequence that the single-launch form merges in
// place (the merge's few-partition path: all loads of a piece in flight).
constexpr int32_t kFusedMaxPartitions = 8;

int64_t wave_slots() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 2048;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            return 2048;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return (int64_t)n * 8;
}

}  // namespace

extern "C" {

const char* vk_status_string(vk_status s) {
    switch (s) {
        case VK_OK: return "ok";
        case VK_ERR_NULL_ARG: return "null argument";
        case VK_ERR_BAD_DIM: return "bad dimension";
        case VK_ERR_GEOMETRY: return "geometry not admitted (Hq, Hkv, head_dim)";
        case VK_ERR_BLOCK_SIZE: return "block size not in {8, 16, 32}";
        case VK_ERR_PARTITION: return "partition size or count not allowed";
        case VK_ERR_SEQ_LEN: return "sequence length outside [1, max_blocks_per_seq * block_size]";
        case VK_ERR_SCRATCH_CAP: return "split-KV scratch over the cap";
        case VK_ERR_HIP: return "HIP error";
        case VK_ERR_DTYPE: return "element type not supported";
        case VK_ERR_ALIGN: return "device pointer not aligned (16 bytes for q, K, V, out, tmp_out; 4 for int32/fp32 arrays)";
        default: return "unknown status";
    }
}

int32_t vk_last_hip_error(void) { return t_last_hip_error; }

int32_t vk_trace_enabled(void) { return roctx().push != nullptr ? 1 : 0; }

vk_status vk_last_plan(vk_plan* out) {
    if (!out) return VK_ERR_NULL_ARG;
    *out = t_last_plan;
    return VK_OK;
}

int32_t vk_select_decode_kernel(int32_t kernel) {
    if (kernel < VK_KERNEL_AUTO || kernel > VK_KERNEL_MFMA_W4P2) return -1;
    const int32_t prev = t_kernel_choice;
    t_kernel_choice = kernel;
    return prev;
}

int32_t vk_select_varlen_kernel(int32_t kernel) {
    if (kernel != VK_KERNEL_AUTO && kernel != VK_KERNEL_VARLEN_COLUMNS &&
        kernel != VK_KERNEL_VARLEN_TILES)
        return -1;
    const int32_t prev = t_varlen_choice;
    t_varlen_choice = kernel;
    return prev;
}

int32_t vk_select_work_order(int32_t order) {
    if (order < VK_ORDER_AUTO || order > VK_ORDER_LONGEST_FIRST) return -1;
    const int32_t prev = t_order_choice;
    t_order_choice = order;
    return prev;
}

vk_status vk_plan_partitions(const int32_t* seq_lens_host, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int32_t partition_request,
                             int32_t cu_count, int32_t budget_per_cu, uint64_t scratch_cap_bytes,
                             vk_plan* plan_out) {
    if (!seq_lens_host || !plan_out) return VK_ERR_NULL_ARG;
    if (num_seqs <= 0 || max_blocks_per_seq <= 0) return VK_ERR_BAD_DIM;
    vk_status gs = geometry_status(num_q_heads, num_kv_heads, head_dim);
    if (gs != VK_OK) return gs;
    if (!block_size_ok(block_size)) return VK_ERR_BLOCK_SIZE;
    if (partition_request != -1 && partition_request != 0 && partition_request != VK_PARTITION_SMALL &&
        partition_request != VK_PARTITION_LARGE && partition_request != VK_PARTITION_XLARGE)
        return VK_ERR_PARTITION;
    if (cu_count < 0 || budget_per_cu < 0) return VK_ERR_BAD_DIM;
    const int64_t cap_tokens = (int64_t)max_blocks_per_seq * block_size;
    if (cap_tokens > INT32_MAX) return VK_ERR_BAD_DIM;

    int64_t max_len = 0;
    int64_t full1024 = 0, full512 = 0, full256 = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t L = seq_lens_host[s];
        if (L < 1 || L > cap_tokens) return VK_ERR_SEQ_LEN;
        if (L > max_len) max_len = L;
        full1024 += L / VK_PARTITION_XLARGE;
        full512 += L / VK_PARTITION_LARGE;
        full256 += L / VK_PARTITION_SMALL;
    }

    if (cu_count == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e);
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e);
        cu_count = n;
    }
    // Default budget: 4 workgroups of full 512-token partitions per CU, each
    // workgroup serving the G query heads of one KV head (MI355X calibration).
    const int64_t per_cu = budget_per_cu > 0
                               ? budget_per_cu
                               : (int64_t)VK_DECODE_BUDGET_WG_PER_CU * (num_q_heads / num_kv_heads);
    const uint64_t cap = scratch_cap_bytes > 0 ? scratch_cap_bytes : VK_DEFAULT_SCRATCH_CAP;

    vk_plan p = {};
    p.cu_count = cu_count;
    p.budget = per_cu * cu_count;
    if (partition_request == 0) {
        p.partition_size = 0;
        p.max_num_partitions = 1;
        p.work_full_parts = 0;
        p.scratch_bytes = 0;
    } else {
        int32_t P = partition_request;
        if (P == -1) {
            // Largest partition first; it is kept only if its full partitions
            // alone reach the budget, otherwise the smaller size is used.
            P = ((int64_t)num_q_heads * full512 >= p.budget) ? VK_PARTITION_LARGE : VK_PARTITION_SMALL;
            // MI355X: when 1024-token partitions fit in one round of the
            // wave slots (8 per CU) with at least two waves each, the launch
            // takes them instead of 512: half the partials to write and
            // merge, longer streams per wave.  Measured: 4 x 131072 tokens
            // (16, 2, 256), decode 176.0 -> 170.6 us, reduce 10.1 -> 7.7;
            // multi-query (16, 1, 256) on 16 x 32768 and 4 x 131072 tokens
            // 95.5 -> 90.5 us, (16, 1, 128) on 6 x 65536 41.1 -> 39.9 us.
            if (P == VK_PARTITION_LARGE) {
                const int64_t slots = 8 * (int64_t)cu_count;
                const int64_t wgs1024 = (int64_t)num_seqs * num_kv_heads * ((max_len + 1023) / 1024);
                if (2 * wgs1024 <= slots) P = VK_PARTITION_XLARGE;
            }
            // MI355X default (no caller budget): 1024-token partitions first,
            // once their full partitions give 2 workgroups per CU (launched
            // with four waves each): over 84 timed batches of the eight
            // geometries this lost 65 us against the fastest size, the 512 /
            // 256 rule above 460 us.
            if (budget_per_cu == 0 &&
                (int64_t)num_kv_heads * full1024 >= (int64_t)VK_DECODE_XLARGE_WG_PER_CU * cu_count)
                P = VK_PARTITION_XLARGE;
        }
        p.partition_size = P;
        p.max_num_partitions = (int32_t)((max_len + P - 1) / P);
        p.work_full_parts = (int64_t)num_q_heads * (P == VK_PARTITION_XLARGE ? full1024
                                                    : P == VK_PARTITION_LARGE ? full512 : full256);
        p.scratch_bytes = (uint64_t)num_seqs * (uint64_t)num_q_heads *
                          (uint64_t)p.max_num_partitions * (uint64_t)(head_dim + 2) * 4u;
        if (p.scratch_bytes > cap) return VK_ERR_SCRATCH_CAP;
    }
    *plan_out = p;
    t_last_plan = p;
    if (log_enabled())
        std::fprintf(stderr, "[vkpaged] plan: P=%d NP=%d W=%lld budget=%lld cu=%d scratch=%llu\n",
                     p.partition_size, p.max_num_partitions, (long long)p.work_full_parts,
                     (long long)p.budget, p.cu_count, (unsigned long long)p.scratch_bytes);
    return VK_OK;
}

}  // extern "C"

namespace {

// Shared by the two decode entry points; `fused` selects the single-launch
// form (split partials merged in place by the last workgroup per KV head).
vk_status decode_impl(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                      float scale, int32_t partition_size, int32_t max_num_partitions, float* out,
                      float* max_logits, float* exp_sums, float* tmp_out, uint32_t* counters,
                      bool fused, int32_t dtype, void* stream) {
    if (dtype != VK_DTYPE_F16 && dtype != VK_DTYPE_BF16 && dtype != VK_DTYPE_F32)
        return VK_ERR_DTYPE;
    if (fused && dtype != VK_DTYPE_F16) return VK_ERR_DTYPE;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens) return VK_ERR_NULL_ARG;
    if (fused && (!out || (partition_size != 0 && !counters))) return VK_ERR_NULL_ARG;
    if (!vectors_aligned({q, k_cache, v_cache, out, tmp_out},
                         {block_tables, seq_lens, max_logits, exp_sums, counters}))
        return VK_ERR_ALIGN;
    if (num_seqs <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0) return VK_ERR_BAD_DIM;
    if (num_seqs > 65535) return VK_ERR_BAD_DIM;  // grid.z limit
    vk_status gs = geometry_status(num_q_heads, num_kv_heads, head_dim);
    if (gs != VK_OK) return gs;
    if (!block_size_ok(block_size)) return VK_ERR_BLOCK_SIZE;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return VK_ERR_BAD_DIM;
    if (!std::isfinite(scale)) return VK_ERR_BAD_DIM;
    if (partition_size == 0) {
        if (!out) return VK_ERR_NULL_ARG;
        if (max_num_partitions != 1) return VK_ERR_PARTITION;
    } else if (partition_size == VK_PARTITION_SMALL || partition_size == VK_PARTITION_LARGE ||
               partition_size == VK_PARTITION_XLARGE) {
        if (!max_logits || !exp_sums || !tmp_out) return VK_ERR_NULL_ARG;
        if (max_num_partitions < 1) return VK_ERR_PARTITION;
        if ((int64_t)max_num_partitions * partition_size > (int64_t)INT32_MAX) return VK_ERR_PARTITION;
    } else {
        return VK_ERR_PARTITION;
    }

    // The single launch merges the partials of a (sequence, KV head) in the
    // workgroup that finishes last.  With more than kFusedMaxPartitions
    // partitions that one workgroup folds them alone and becomes the launch's
    // tail (measured on MI355X: 4 sequences of 131072 tokens at P = 512,
    // 256 partitions, 483.8 us against 183.3 us for decode + reduce), so the
    // call then enqueues the decode and the reduce instead: same kernels,
    // same partials, the counters untouched.
    const bool fused_split = fused && partition_size > 0 && max_num_partitions > kFusedMaxPartitions;
    if (fused_split) {
        fused = false;
        counters = nullptr;
    }

    vk::DecodeArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_cache);
    a.v = static_cast<const uint16_t*>(v_cache);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.out = out;
    a.max_logits = max_logits;
    a.exp_sums = exp_sums;
    a.tmp_out = tmp_out;
    a.counters = fused ? counters : nullptr;
    a.num_blocks = num_blocks;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.num_seqs = num_seqs;
    a.partition_size = partition_size;
    a.max_num_partitions = max_num_partitions;
    // log2(e) folded into the scale once, in double, then rounded to fp32.
    a.scale_log2e = (float)((double)scale * 1.4426950408889634073599246810019);

    const int group = num_q_heads / num_kv_heads;
    dim3 grid(partition_size == 0 ? 1u : (unsigned)max_num_partitions, (unsigned)num_kv_heads,
              (unsigned)num_seqs);
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool ok = false;
    int block = 0;
    int32_t kernel = t_kernel_choice;
    // The in-place merge, the multi-head / multi-query geometries and the
    // other element types exist only in the matrix-core family; two
    // partitions per workgroup need an fp16 split without the in-place merge.
    const bool mhq = group == 1 || group == 16;
    if (kernel == VK_KERNEL_DOT && (fused || fused_split || mhq || dtype != VK_DTYPE_F16))
        kernel = VK_KERNEL_AUTO;
    if (kernel == VK_KERNEL_MFMA_W4P2 &&
        (fused || fused_split || partition_size == 0 || dtype != VK_DTYPE_F16))
        kernel = VK_KERNEL_MFMA_W4;
    const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
    const int64_t slots = kernel == VK_KERNEL_DOT ? 0 : wave_slots();
    const bool auto_waves = kernel == VK_KERNEL_AUTO || kernel == VK_KERNEL_MFMA;
    if (auto_waves) {
        // Waves per workgroup from the grid size (measured on MI355X, 256
        // CUs = 2048 wave slots): small grids (few sequences or unsplit)
        // spread a workgroup's tokens over 4 waves; a grid that fills the
        // slots about once keeps 1 wave per workgroup; larger grids balance
        // better with 2.
        kernel = 2 * wgs <= slots ? VK_KERNEL_MFMA_W4 : wgs <= slots ? VK_KERNEL_MFMA_W1 : VK_KERNEL_MFMA_W2;
        // 1024-token partitions in one round of two waves each (the
        // planner's choice in place of one wave per 512): 512 tokens per wave.
        // fp32 at head dim 256 holds one wave per SIMD (half the slots the
        // planner counts): one wave per 1024-token partition keeps that one
        // round (two waves per partition measured 514 vs 365 us at 512).
        // Other 1024-token launches: four waves of 256 tokens per partition.
        // The grid counts every (partition, KV head, sequence) slot, empty
        // ones included, so on mixed lengths it can fit one round while few
        // partitions exist; one wave each then left the CUs short of loads
        // (e.g. 16 sequences of 1-32768 tokens, (24, 4, 256): 194 vs 136 us).
        if (partition_size == VK_PARTITION_XLARGE)
            kernel = (2 * wgs <= slots && 4 * wgs > slots)
                         ? ((dtype == VK_DTYPE_F32 && head_dim == 256) ? VK_KERNEL_MFMA_W1 : VK_KERNEL_MFMA_W2)
                         : VK_KERNEL_MFMA_W4;
    }
    a.work_order = 0;
    a.write_through = 0;
    hipError_t e;
    if (kernel == VK_KERNEL_DOT) {
        e = vk::launch_decode_dot(a, group, head_dim, block_size, grid, st, &ok, &block);
    } else {
        int waves = kernel == VK_KERNEL_MFMA_W1 ? 1 : kernel == VK_KERNEL_MFMA_W2 ? 2 : 4;
        // fp32 at head dim 256 holds one wave per SIMD (its registers): a
        // split grid of at least two workgroups per CU runs one wave per
        // partition, the work order decided for that (32 sequences of
        // 4k-16k tokens, (24, 4, 256): four waves 822 / 817 us at P = 512 /
        // 1024, one wave 452.6 / 488 us; 512 workgroups: one wave 65.9 vs
        // four 87.4 us); at one workgroup per CU four waves still win
        // (46.6 vs 55.9 us).
        const bool f32_wide = auto_waves && dtype == VK_DTYPE_F32 && head_dim == 256 &&
                              partition_size > 0 && 4 * wgs >= slots;
        if (f32_wide) {
            waves = 1;
            kernel = VK_KERNEL_MFMA_W1;
        }
        int parts_per_wg = kernel == VK_KERNEL_MFMA_W4P2 ? 2 : 1;
        // Longest-first work order when the split grid takes more than one
        // round of the wave slots, so the order decides the tail.  Measured on
        // MI355X at P = 512: 9-20% faster for 16-64 sequences of 2k-32k
        // tokens with 16- and 32-token pages, 3% for 64 mixed-length
        // sequences with 8-token pages.
        const bool lf_ok = partition_size > 0 && num_seqs <= 64;
        if (lf_ok && (t_order_choice == VK_ORDER_LONGEST_FIRST ||
                      (t_order_choice == VK_ORDER_AUTO && wgs * waves > slots)))
            a.work_order = 1;
        // In longest-first order, waves of 8 steps (P / 128 waves per
        // partition) balanced best: 4 waves at P = 512, 2 at P = 256.
        // Partials written through L2 in the same case: measured on MI355X,
        // longest-first launches of several rounds lose 3% to partials kept
        // dirty in L2 until the launch ends; single-round and grid-order
        // launches gained nothing from writing through.
        a.write_through = a.work_order;
        if (auto_waves && a.work_order == 1 && !f32_wide) {
            waves = partition_size >= VK_PARTITION_LARGE ? 4 : 2;
            kernel = waves == 4 ? VK_KERNEL_MFMA_W4 : VK_KERNEL_MFMA_W2;
        }

        if (parts_per_wg == 2) grid.x = (grid.x + 1) / 2;
        e = vk::launch_decode_mfma(a, dtype, group, head_dim, block_size, waves, parts_per_wg,
                                   grid, st, &ok, &block);
    }
    if (!ok) return VK_ERR_GEOMETRY;
    if (e != hipSuccess) return hip_fail(e);
    if (fused_split) {
        const vk_status rs = vk_paged_gqa_reduce(max_logits, exp_sums, tmp_out, seq_lens, num_seqs,
                                                 num_q_heads, head_dim, partition_size,
                                                 max_num_partitions, out, stream);
        if (rs != VK_OK) return rs;
    }

    vk_plan p = {};
    p.partition_size = partition_size;
    p.max_num_partitions = max_num_partitions;
    p.kernel = kernel;
    p.scratch_bytes = partition_size == 0 ? 0
                      : (uint64_t)num_seqs * num_q_heads * (uint64_t)max_num_partitions *
                            (uint64_t)(head_dim + 2) * 4u;
    p.grid[0] = (int32_t)grid.x;
    p.grid[1] = (int32_t)grid.y;
    p.grid[2] = (int32_t)grid.z;
    p.block = block;
    p.work_order = a.work_order ? VK_ORDER_LONGEST_FIRST : VK_ORDER_GRID;
    t_last_plan = p;
    return VK_OK;
}

}  // namespace

extern "C" {

vk_status vk_paged_gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, int32_t partition_size,
                              int32_t max_num_partitions, float* out, float* max_logits,
                              float* exp_sums, float* tmp_out, void* stream) {
    TraceRange trace("vk_paged_gqa_decode");
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       partition_size, max_num_partitions, out, max_logits, exp_sums, tmp_out,
                       nullptr, false, VK_DTYPE_F16, stream);
}

vk_status vk_paged_gqa_decode_dt(int32_t dtype, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                 int32_t partition_size, int32_t max_num_partitions, float* out,
                                 float* max_logits, float* exp_sums, float* tmp_out,
                                 void* stream) {
    TraceRange trace("vk_paged_gqa_decode_dt");
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       partition_size, max_num_partitions, out, max_logits, exp_sums, tmp_out,
                       nullptr, false, dtype, stream);
}

vk_status vk_paged_gqa_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                    int32_t partition_size, int32_t max_num_partitions,
                                    float* out, float* max_logits, float* exp_sums,
                                    float* tmp_out, uint32_t* counters, void* stream) {
    TraceRange trace("vk_paged_gqa_decode_fused");
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       partition_size, max_num_partitions, out, max_logits, exp_sums, tmp_out,
                       counters, true, VK_DTYPE_F16, stream);
}

vk_status vk_plan_varlen(const int32_t* seq_lens_host, const int32_t* q_lens_host,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int32_t partition_request, int32_t cu_count, uint64_t scratch_cap_bytes,
                         vk_plan* plan_out) {
    if (!seq_lens_host || !q_lens_host || !plan_out) return VK_ERR_NULL_ARG;
    if (num_seqs <= 0 || num_seqs > 65535 || max_blocks_per_seq <= 0) return VK_ERR_BAD_DIM;
    vk_status gs = geometry_status(num_q_heads, num_kv_heads, head_dim);
    if (gs != VK_OK) return gs;
    if (!block_size_ok(block_size)) return VK_ERR_BLOCK_SIZE;
    if (partition_request != -1 && partition_request != 0 && partition_request != VK_PARTITION_SMALL &&
        partition_request != VK_PARTITION_LARGE && partition_request != VK_PARTITION_XLARGE)
        return VK_ERR_PARTITION;
    if (cu_count < 0) return VK_ERR_BAD_DIM;
    const int64_t cap_tokens = (int64_t)max_blocks_per_seq * block_size;
    if (cap_tokens > INT32_MAX) return VK_ERR_BAD_DIM;
    int64_t max_q = 0;
    for (int32_t s = 0; s < num_seqs; ++s) max_q = std::max<int64_t>(max_q, q_lens_host[s]);
    const int group = num_q_heads / num_kv_heads;
    const int32_t kernel = varlen_kernel(max_q, group);
    const bool tiled = kernel == VK_KERNEL_VARLEN_TILES;
    const int tpt = vk::varlen_tokens_per_tile(group);   // column kernel
    const int waves_per_tile = tiled ? vk::varlen_tile_threads(head_dim) / 64 : 1;
    int64_t max_len = 0, total_q = 0, tiles = 0, full1024 = 0, full512 = 0, full256 = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t L = seq_lens_host[s], ql = q_lens_host[s];
        if (L < 1 || L > cap_tokens) return VK_ERR_SEQ_LEN;
        if (ql < 0 || ql > L) return VK_ERR_SEQ_LEN;
        if (L > max_len) max_len = L;
        total_q += ql;
        const int64_t t = tiled ? vk::varlen_tile_count(ql, group) : (ql + tpt - 1) / tpt;
        tiles += t;
        full1024 += t * (L / VK_PARTITION_XLARGE);
        full512 += t * (L / VK_PARTITION_LARGE);
        full256 += t * (L / VK_PARTITION_SMALL);
    }
    if (max_q > 65535 || total_q > INT32_MAX) return VK_ERR_BAD_DIM;
    if (cu_count == 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e);
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e);
        cu_count = n;
    }
    const uint64_t cap = scratch_cap_bytes > 0 ? scratch_cap_bytes : VK_DEFAULT_SCRATCH_CAP;
    vk_plan p = {};
    p.cu_count = cu_count;
    p.budget = (int64_t)VK_DEFAULT_BUDGET_PER_CU * cu_count;
    p.kernel = kernel;
    int32_t P = partition_request;
    const auto scratch_at = [&](int32_t Pc) -> uint64_t {
        return (uint64_t)total_q * (uint64_t)num_q_heads * (uint64_t)((max_len + Pc - 1) / Pc) *
               (uint64_t)(head_dim + 2) * 4u;
    };
    if (P == -1) {
        // Unsplit when the (tile, KV head) workgroups fill the wave slots
        // once (8 per CU); otherwise the decode's rule, its unit a (query
        // head, full partition) pair, counted for every tile: W(P) =
        // Hq * sum_s tiles_s * floor(L_s / P), which is the decode's W(P)
        // when each sequence brings one query token.  Many query rows can
        // make the partials outgrow the cap: then 512, and failing that
        // unsplit (which needs none).
        // Column tiles of several query tokens also take the next size up,
        // 1024, under the same rule (largest first); measured on MI355X
        // (verification, 32 sequences x 4 tokens on 4k-16k contexts): 4%
        // faster than 512, with half the partials to merge.  Rows of one
        // query token keep the decode's sizes.
        const bool xl = !tiled && max_q > 1;
        if ((int64_t)waves_per_tile * num_kv_heads * tiles >= 8 * (int64_t)cu_count)
            P = 0;
        else if (xl && (int64_t)num_q_heads * full1024 >= p.budget)
            P = VK_PARTITION_XLARGE;
        else
            P = ((int64_t)num_q_heads * full512 >= p.budget) ? VK_PARTITION_LARGE : VK_PARTITION_SMALL;
        if (P == VK_PARTITION_SMALL && scratch_at(P) > cap) P = VK_PARTITION_LARGE;
        if (P == VK_PARTITION_LARGE && scratch_at(P) > cap) P = xl ? VK_PARTITION_XLARGE : 0;
        if (P == VK_PARTITION_XLARGE && scratch_at(P) > cap) P = 0;
    }
    p.partition_size = P;
    if (P == 0) {
        p.max_num_partitions = 1;
        p.work_full_parts = (int64_t)num_kv_heads * tiles;
    } else {
        p.max_num_partitions = (int32_t)((max_len + P - 1) / P);
        p.work_full_parts = (int64_t)num_q_heads * (P == VK_PARTITION_XLARGE ? full1024
                                                    : P == VK_PARTITION_LARGE ? full512 : full256);
        p.scratch_bytes = scratch_at(P);
        if (p.scratch_bytes > cap) return VK_ERR_SCRATCH_CAP;
    }
    *plan_out = p;
    t_last_plan = p;
    return VK_OK;
}

static vk_status varlen_impl(int32_t dtype, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t total_q,
                             int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, float scale, int32_t partition_size,
                             int32_t max_num_partitions, float* out, float* max_logits,
                             float* exp_sums, float* tmp_out, void* stream) {
    if (dtype != VK_DTYPE_F16 && dtype != VK_DTYPE_BF16) return VK_ERR_DTYPE;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !cu_seqlens_q)
        return VK_ERR_NULL_ARG;
    if (!vectors_aligned({q, k_cache, v_cache, out, tmp_out},
                         {block_tables, seq_lens, cu_seqlens_q, max_logits, exp_sums}))
        return VK_ERR_ALIGN;
    if (num_seqs <= 0 || num_seqs > 65535 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        total_q <= 0 || max_q_len <= 0 || max_q_len > 65535 || max_q_len > total_q)
        return VK_ERR_BAD_DIM;
    vk_status gs = geometry_status(num_q_heads, num_kv_heads, head_dim);
    if (gs != VK_OK) return gs;
    if (!block_size_ok(block_size)) return VK_ERR_BLOCK_SIZE;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return VK_ERR_BAD_DIM;
    if (!std::isfinite(scale)) return VK_ERR_BAD_DIM;
    if (partition_size == 0) {
        if (!out) return VK_ERR_NULL_ARG;
        if (max_num_partitions != 1) return VK_ERR_PARTITION;
    } else if (partition_size == VK_PARTITION_SMALL || partition_size == VK_PARTITION_LARGE ||
               partition_size == VK_PARTITION_XLARGE) {
        if (!max_logits || !exp_sums || !tmp_out) return VK_ERR_NULL_ARG;
        if (max_num_partitions < 1) return VK_ERR_PARTITION;
        if ((int64_t)max_num_partitions * partition_size > (int64_t)INT32_MAX) return VK_ERR_PARTITION;
    } else {
        return VK_ERR_PARTITION;
    }
    const int group = num_q_heads / num_kv_heads;
    const int32_t kernel = varlen_kernel(max_q_len, group);
    const bool tiled = kernel == VK_KERNEL_VARLEN_TILES;
    const int tpt = vk::varlen_tokens_per_tile(group);
    const int64_t tiles = tiled ? vk::varlen_tile_count(max_q_len, group) : (max_q_len + tpt - 1) / tpt;
    const int64_t gx = tiles * (partition_size == 0 ? 1 : max_num_partitions);
    if (gx > INT32_MAX) return VK_ERR_BAD_DIM;

    vk::VarlenArgs va = {};
    vk::DecodeArgs& a = va.d;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_cache);
    a.v = static_cast<const uint16_t*>(v_cache);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.out = out;
    a.max_logits = max_logits;
    a.exp_sums = exp_sums;
    a.tmp_out = tmp_out;
    a.counters = nullptr;
    a.num_blocks = num_blocks;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.num_seqs = num_seqs;
    a.partition_size = partition_size;
    a.max_num_partitions = max_num_partitions;
    a.scale_log2e = (float)((double)scale * 1.4426950408889634073599246810019);
    a.work_order = 0;
    a.write_through = 0;
    // The column kernel with one tile per sequence, split, over <= 64
    // sequences has the decode's items: its longest-first order and
    // write-through partials apply when the grid takes more than one round
    // of the wave slots (measured on 32 sequences of 4k-16k tokens, 4 query
    // tokens at G = 4).
    if (!tiled && tiles == 1 && partition_size > 0 && num_seqs <= 64 &&
        (t_order_choice == VK_ORDER_LONGEST_FIRST ||
         (t_order_choice == VK_ORDER_AUTO &&
          gx * num_kv_heads * (int64_t)num_seqs > wave_slots()))) {
        a.work_order = 1;
        a.write_through = 1;
    }
    // The LDS-tiled kernel, unsplit, over <= 64 sequences, on request only:
    // its items in global longest-first order (decreasing key range).  Grid
    // order stays the default: on the chunked prefill of 4 x 1024 tokens
    // (768 workgroups) longest-first measured 1049 vs 1007 us on MI355X — it
    // spreads each (sequence, KV head)'s tiles over the XCDs, whose L2s the
    // grid order's runs of 8 share, and that outweighed the better balance.
    if (tiled && partition_size == 0 && num_seqs <= 64 && t_order_choice == VK_ORDER_LONGEST_FIRST)
        a.work_order = 1;
    va.cu_q = cu_seqlens_q;
    va.tiles = (int32_t)tiles;
    const dim3 grid((unsigned)gx, (unsigned)num_kv_heads, (unsigned)num_seqs);
    bool ok = false;
    hipError_t e = tiled ? vk::launch_varlen_tile(va, dtype, group, head_dim, block_size, grid,
                                                  static_cast<hipStream_t>(stream), &ok)
                         : vk::launch_decode_varlen(va, dtype, group, head_dim, block_size, grid,
                                                    static_cast<hipStream_t>(stream), &ok);
    if (!ok) return VK_ERR_GEOMETRY;
    if (e != hipSuccess) return hip_fail(e);
    vk_plan p = {};
    p.partition_size = partition_size;
    p.max_num_partitions = max_num_partitions;
    p.kernel = kernel;
    p.scratch_bytes = partition_size == 0 ? 0
                      : (uint64_t)total_q * num_q_heads * (uint64_t)max_num_partitions *
                            (uint64_t)(head_dim + 2) * 4u;
    p.grid[0] = (int32_t)grid.x;
    p.grid[1] = (int32_t)grid.y;
    p.grid[2] = (int32_t)grid.z;
    p.block = tiled ? vk::varlen_tile_threads(head_dim) : 64;
    p.work_order = a.work_order ? VK_ORDER_LONGEST_FIRST : VK_ORDER_GRID;
    t_last_plan = p;
    return VK_OK;
}

vk_status vk_paged_gqa_varlen(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t total_q,
                              int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, float scale, int32_t partition_size,
                              int32_t max_num_partitions, float* out, float* max_logits,
                              float* exp_sums, float* tmp_out, void* stream) {
    TraceRange trace("vk_paged_gqa_varlen");
    return varlen_impl(VK_DTYPE_F16, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q,
                       num_seqs, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, scale, partition_size,
                       max_num_partitions, out, max_logits, exp_sums, tmp_out, stream);
}

vk_status vk_paged_gqa_varlen_dt(int32_t dtype, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                                 int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                                 float scale, int32_t partition_size, int32_t max_num_partitions,
                                 float* out, float* max_logits, float* exp_sums, float* tmp_out,
                                 void* stream) {
    TraceRange trace("vk_paged_gqa_varlen_dt");
    return varlen_impl(dtype, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, num_seqs,
                       total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, scale, partition_size, max_num_partitions,
                       out, max_logits, exp_sums, tmp_out, stream);
}

vk_status vk_paged_gqa_varlen_reduce(const float* max_logits, const float* exp_sums,
                                     const float* tmp_out, const int32_t* seq_lens,
                                     const int32_t* cu_seqlens_q, int32_t num_seqs,
                                     int32_t max_q_len, int32_t num_q_heads, int32_t head_dim,
                                     int32_t partition_size, int32_t max_num_partitions,
                                     float* out, void* stream) {
    TraceRange trace("vk_paged_gqa_varlen_reduce");
    if (!max_logits || !exp_sums || !tmp_out || !seq_lens || !cu_seqlens_q || !out)
        return VK_ERR_NULL_ARG;
    if (!vectors_aligned({tmp_out, out}, {max_logits, exp_sums, seq_lens, cu_seqlens_q}))
        return VK_ERR_ALIGN;
    if (num_seqs <= 0 || num_seqs > 65535 || num_q_heads <= 0 || num_q_heads > 256 ||
        max_q_len <= 0 || max_q_len > 65535)
        return VK_ERR_BAD_DIM;
    if (head_dim != 128 && head_dim != 256) return VK_ERR_GEOMETRY;
    if (partition_size != VK_PARTITION_SMALL && partition_size != VK_PARTITION_LARGE &&
        partition_size != VK_PARTITION_XLARGE)
        return VK_ERR_PARTITION;
    if (max_num_partitions < 1) return VK_ERR_PARTITION;
    vk::ReduceArgs a;
    a.max_logits = max_logits;
    a.exp_sums = exp_sums;
    a.tmp_out = tmp_out;
    a.seq_lens = seq_lens;
    a.out = out;
    a.num_q_heads = num_q_heads;
    a.partition_size = partition_size;
    a.max_num_partitions = max_num_partitions;
    bool ok = false;
    hipError_t e = vk::launch_reduce_varlen(a, cu_seqlens_q, head_dim, max_q_len, num_seqs,
                                            static_cast<hipStream_t>(stream), &ok);
    if (!ok) return VK_ERR_GEOMETRY;
    if (e != hipSuccess) return hip_fail(e);
    return VK_OK;
}

vk_status vk_paged_kv_append(const void* k_new, const void* v_new, const int32_t* block_tables,
                             const int32_t* positions, int32_t num_seqs, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, double rope_theta, void* k_cache, void* v_cache,
                             void* stream) {
    TraceRange trace("vk_paged_kv_append");
    if (!k_new || !v_new || !block_tables || !positions || !k_cache || !v_cache)
        return VK_ERR_NULL_ARG;
    if (num_seqs <= 0 || num_seqs > 65535 || num_kv_heads <= 0 || num_kv_heads > 65535 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return VK_ERR_BAD_DIM;
    if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > 256) return VK_ERR_BAD_DIM;
    if (!block_size_ok(block_size)) return VK_ERR_BLOCK_SIZE;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return VK_ERR_BAD_DIM;
    if (!std::isfinite(rope_theta)) return VK_ERR_BAD_DIM;
    vk::AppendArgs a;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.block_tables = block_tables;
    a.positions = positions;
    a.k_cache = static_cast<uint16_t*>(k_cache);
    a.v_cache = static_cast<uint16_t*>(v_cache);
    a.num_blocks = num_blocks;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.rope_theta = rope_theta;
    hipError_t e = vk::launch_kv_append(a, num_seqs, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e);
    return VK_OK;
}

vk_status vk_paged_gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                      int32_t partition_size, int32_t max_num_partitions,
                                      float* out, void* stream) {
    TraceRange trace("vk_paged_gqa_decode_noalloc");
    // Host checks of the sizes first (decode_impl repeats the rest before
    // its launch): the partials must fit the library's array.
    if (!out) return VK_ERR_NULL_ARG;
    if (num_seqs <= 0 || num_seqs > 65535) return VK_ERR_BAD_DIM;
    vk_status gs = geometry_status(num_q_heads, num_kv_heads, head_dim);
    if (gs != VK_OK) return gs;
    if (partition_size == 0) {
        return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                           num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                           scale, 0, max_num_partitions, out, nullptr, nullptr, nullptr, nullptr,
                           false, VK_DTYPE_F16, stream);
    }
    if (partition_size != VK_PARTITION_SMALL && partition_size != VK_PARTITION_LARGE &&
        partition_size != VK_PARTITION_XLARGE)
        return VK_ERR_PARTITION;
    if (max_num_partitions < 1 ||
        (int64_t)max_num_partitions * partition_size > (int64_t)INT32_MAX)
        return VK_ERR_PARTITION;
    // Layout in the array: max_logits, exp_sums, tmp_out, each at a 256-byte
    // boundary (at most 2^16 * 32 * 2^23 * 258 * 4 bytes: no overflow).
    const uint64_t rows = (uint64_t)num_seqs * (uint64_t)num_q_heads * (uint64_t)max_num_partitions;
    const uint64_t vec = (rows * 4u + 255u) & ~(uint64_t)255u;
    const uint64_t need = 2u * vec + rows * (uint64_t)head_dim * 4u;
    if (need > VK_NOALLOC_SCRATCH_BYTES) return VK_ERR_SCRATCH_CAP;
    void* base = nullptr;
    hipError_t e = vk::noalloc_scratch(&base);
    if (e != hipSuccess) return hip_fail(e);
    char* b = static_cast<char*>(base);
    float* ml = reinterpret_cast<float*>(b);
    float* es = reinterpret_cast<float*>(b + vec);
    float* to = reinterpret_cast<float*>(b + 2u * vec);
    vk_status st = decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                               num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                               scale, partition_size, max_num_partitions, nullptr, ml, es, to,
                               nullptr, false, VK_DTYPE_F16, stream);
    if (st != VK_OK) return st;
    const vk_plan launched = t_last_plan;   // the decode's launch shape, reported afterwards
    st = vk_paged_gqa_reduce(ml, es, to, seq_lens, num_seqs, num_q_heads, head_dim,
                             partition_size, max_num_partitions, out, stream);
    if (st == VK_OK) t_last_plan = launched;
    return st;
}

vk_status vk_paged_gqa_reduce(const float* max_logits, const float* exp_sums, const float* tmp_out,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t head_dim, int32_t partition_size, int32_t max_num_partitions,
                              float* out, void* stream) {
    TraceRange trace("vk_paged_gqa_reduce");
    if (!max_logits || !exp_sums || !tmp_out || !seq_lens || !out) return VK_ERR_NULL_ARG;
    if (!vectors_aligned({tmp_out, out}, {max_logits, exp_sums, seq_lens})) return VK_ERR_ALIGN;
    if (num_seqs <= 0 || num_q_heads <= 0 || num_seqs > 65535) return VK_ERR_BAD_DIM;
    if (head_dim != 128 && head_dim != 256) return VK_ERR_GEOMETRY;
    if (partition_size != VK_PARTITION_SMALL && partition_size != VK_PARTITION_LARGE &&
        partition_size != VK_PARTITION_XLARGE)
        return VK_ERR_PARTITION;
    if (max_num_partitions < 1) return VK_ERR_PARTITION;
    vk::ReduceArgs a;
    a.max_logits = max_logits;
    a.exp_sums = exp_sums;
    a.tmp_out = tmp_out;
    a.seq_lens = seq_lens;
    a.out = out;
    a.num_q_heads = num_q_heads;
    a.partition_size = partition_size;
    a.max_num_partitions = max_num_partitions;
    bool ok = false;
    hipError_t e = vk::launch_reduce(a, head_dim, dim3((unsigned)num_q_heads, (unsigned)num_seqs),
                                     static_cast<hipStream_t>(stream), &ok);
    if (!ok) return VK_ERR_GEOMETRY;
    if (e != hipSuccess) return hip_fail(e);
    return VK_OK;
}

}  // extern "C"
