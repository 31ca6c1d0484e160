// Split-KV partition reduce for gfx950: the merge of merge_ops.h (vllm-metal
// kernels page, cf-1.com/news/5525226, section "GQA 解码内核的四个提速技巧",
// item 4) as its own launch.
//
// Grid (D / 32, Hq, S), one wave64 per 32 output dims (one 128-byte line of
// every partial row, so no line is split between waves on different XCDs)
// of one (sequence, query head).
#include "merge_ops.h"
#include "vk_kernels.h"

namespace vk {
namespace merge {

// All NCH * 32 dims of one row in one wave: per 32-dim chunk the lanes,
// partition order and fold steps of merge_columns (so the same results),
// with each partition's (max, exp-sum) loaded once for the whole row and the
// loads of every chunk in flight together (merge_columns over the chunks in
// turn would wait for one chunk's loads at a time).
template <int NCH>
__device__ __forceinline__ void merge_row(const float* ml, const float* es, const float4* to,
                                          int row4, int n, int lane, float4* dst) {
    constexpr int KB = 16 / NCH > 0 ? 16 / NCH : 1;   // partitions per lane loaded ahead
    const int c = lane % kCols, grp = lane / kCols;
    if (n == 1) {
        if (lane < kCols) {
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) dst[ch * kCols + lane] = to[ch * kCols + lane];
        }
        return;
    }
    State st[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        st[ch].m = -INFINITY;
        st[ch].l = 0.f;
        st[ch].acc = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int i0 = grp; i0 < n; i0 += KB * kGroups) {
        float m[KB], l[KB];
        float4 o[KB][NCH];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int i = i0 + k * kGroups;
            const bool ok = i < n;
            m[k] = ok ? ml[i] : -INFINITY;
            l[k] = ok ? es[i] : 0.f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
                o[k][ch] = ok ? to[(int64_t)i * row4 + ch * kCols + c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < KB; ++k)
            if (m[k] != -INFINITY) {
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) fold(st[ch], m[k], l[k], o[k][ch]);
            }
    }
#pragma unroll
    for (int off = kCols; off < 64; off <<= 1) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            State t;
            t.m = __shfl_xor(st[ch].m, off);
            t.l = __shfl_xor(st[ch].l, off);
            t.acc.x = __shfl_xor(st[ch].acc.x, off);
            t.acc.y = __shfl_xor(st[ch].acc.y, off);
            t.acc.z = __shfl_xor(st[ch].acc.z, off);
            t.acc.w = __shfl_xor(st[ch].acc.w, off);
            fold_state(st[ch], t);
        }
    }
    if (lane < kCols) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
            dst[ch * kCols + lane] = make_float4(st[ch].acc.x / st[ch].l, st[ch].acc.y / st[ch].l,
                                                 st[ch].acc.z / st[ch].l, st[ch].acc.w / st[ch].l);
    }
}

}  // namespace merge

namespace {

template <int D>
__global__ __launch_bounds__(64) void reduce_kernel(ReduceArgs a) {
    const int chunk = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int lane = threadIdx.x;
    const int Hq = a.num_q_heads, P = a.partition_size, NP = a.max_num_partitions;
    const int64_t r = (int64_t)s * Hq + h;
    const int L = a.seq_lens[s];
    float4* dst = reinterpret_cast<float4*>(a.out + r * D + chunk * merge::kDims);
    if (L <= 0) {
        if (lane < merge::kCols) dst[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int n = (int)min(((int64_t)L + P - 1) / P, (int64_t)NP);
    merge::merge_columns(a.max_logits + r * NP, a.exp_sums + r * NP,
                         reinterpret_cast<const float4*>(a.tmp_out + r * NP * D + chunk * merge::kDims),
                         D / 4, n, lane, dst);
}

// Variable-length rows: grid ((D / 32) * Hq, max_q_len, S), one wave per 32
// dims, or with ROW grid (Hq, max_q_len, S), one wave per row (merge_row:
// each partition's max and exp-sum loaded once and every dim's loads in
// flight together; for many rows of few partitions).  Query j of sequence s
// (row cu_q[s] + j) merges the partitions its causal range
// [0, L - qlen + j + 1) covers; a row that sees no key is zeros.
template <int D, bool ROW>
__global__ __launch_bounds__(64) void reduce_varlen_kernel(ReduceArgs a, const int32_t* __restrict__ cu_q) {
    constexpr int kChunks = ROW ? 1 : D / merge::kDims;
    const int chunk = blockIdx.x % kChunks, h = blockIdx.x / kChunks;
    const int j = blockIdx.y, s = blockIdx.z;
    const int lane = threadIdx.x;
    const int q0 = cu_q[s], qlen = cu_q[s + 1] - q0;
    if (j >= qlen) return;
    const int Hq = a.num_q_heads, P = a.partition_size, NP = a.max_num_partitions;
    const int64_t r = ((int64_t)q0 + j) * Hq + h;
    const int lim = a.seq_lens[s] - qlen + j + 1;
    float4* dst = reinterpret_cast<float4*>(a.out + r * D + chunk * merge::kDims);
    if (lim <= 0) {
        if (lane < (ROW ? D / 4 : merge::kCols)) dst[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int n = (int)min(((int64_t)lim + P - 1) / P, (int64_t)NP);
    if constexpr (ROW)
        merge::merge_row<D / merge::kDims>(a.max_logits + r * NP, a.exp_sums + r * NP,
                                           reinterpret_cast<const float4*>(a.tmp_out + r * NP * D), D / 4,
                                           n, lane, dst);
    else
        merge::merge_columns(a.max_logits + r * NP, a.exp_sums + r * NP,
                             reinterpret_cast<const float4*>(a.tmp_out + r * NP * D + chunk * merge::kDims),
                             D / 4, n, lane, dst);
}

}  // namespace

hipError_t launch_reduce_varlen(const ReduceArgs& a, const int32_t* cu_q, int head_dim,
                                int max_q_len, int num_seqs, hipStream_t stream,
                                bool* geometry_ok) {
    *geometry_ok = true;
    // One wave per row when the rows alone fill the wave slots about once
    // (>= 2048 waves) and each merges at most 16 partitions; otherwise one
    // wave per 32 dims, which keeps few long rows spread over many waves.
    // Measured on MI355X: 32 sequences x 4 query tokens at (32, 8, 128),
    // 4096 rows of <= 16 partitions: 13.7 vs 16.3 us (HIP events).
    const int64_t rows = (int64_t)max_q_len * num_seqs * a.num_q_heads;
    const bool row = rows >= 2048 && a.max_num_partitions <= 16;
    const dim3 g((unsigned)((row ? 1 : head_dim / merge::kDims) * a.num_q_heads), (unsigned)max_q_len,
                 (unsigned)num_seqs);
    if (head_dim == 128) {
        if (row)
            hipLaunchKernelGGL((reduce_varlen_kernel<128, true>), g, dim3(64), 0, stream, a, cu_q);
        else
            hipLaunchKernelGGL((reduce_varlen_kernel<128, false>), g, dim3(64), 0, stream, a, cu_q);
    } else if (head_dim == 256) {
        if (row)
            hipLaunchKernelGGL((reduce_varlen_kernel<256, true>), g, dim3(64), 0, stream, a, cu_q);
        else
            hipLaunchKernelGGL((reduce_varlen_kernel<256, false>), g, dim3(64), 0, stream, a, cu_q);
    } else {
        *geometry_ok = false;
        return hipSuccess;
    }
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, dim3 grid, hipStream_t stream,
                         bool* geometry_ok) {
    *geometry_ok = true;
    const dim3 g(head_dim / merge::kDims, grid.x, grid.y);
    if (head_dim == 128) {
        hipLaunchKernelGGL(reduce_kernel<128>, g, dim3(64), 0, stream, a);
    } else if (head_dim == 256) {
        hipLaunchKernelGGL(reduce_kernel<256>, g, dim3(64), 0, stream, a);
    } else {
        *geometry_ok = false;
        return hipSuccess;
    }
    return hipGetLastError();
}

}  // namespace vk
