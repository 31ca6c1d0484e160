// Split-KV partition reduce for gfx950 (vllm-metal kernels page,
// cf-1.com/news/5525226, section "GQA 解码内核的四个提速技巧", item 4: partials
// are (max in log2 units, exp-sum, normalised output) and a shared reducer
// merges them).
//
// Grid (D / 64, Hq, S): a workgroup of 256 threads owns 64 output dims of one
// (sequence, query head).  With n partitions:
//   M   = max_i m_i                        (block max over the n values)
//   w_i = l_i * 2^(m_i - M),  W = sum w_i  (block sum)
//   out = sum_i w_i o_i / W
// For the weighted sum, thread t handles float4 column t % 16 of the 64-dim
// chunk for partitions i = t / 16 (mod 16).  Its first 16 partitions' values
// are loaded before the statistics are read, so every load of a workgroup is
// in flight at once; the 16 partition groups are then summed in LDS.
#include "vk_kernels.h"

namespace vk {
namespace {

constexpr int kChunk = 64;                 // output dims per workgroup
constexpr int kLanes = kChunk / 4;         // float4 columns
constexpr int kGroups = 256 / kLanes;      // partition groups
constexpr int kPre = 16;                   // partitions per thread loaded up front

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ void fma4(float4& acc, float w, const float4& o) {
    acc.x = fmaf(w, o.x, acc.x);
    acc.y = fmaf(w, o.y, acc.y);
    acc.z = fmaf(w, o.z, acc.z);
    acc.w = fmaf(w, o.w, acc.w);
}

template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
    __shared__ float s_red[4];
    __shared__ float4 s_part[kGroups][kLanes];

    const int chunk = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int Hq = a.num_q_heads, P = a.partition_size, NP = a.max_num_partitions;
    const int64_t r = (int64_t)s * Hq + h;
    const int L = a.seq_lens[s];
    float4* dst = reinterpret_cast<float4*>(a.out + r * D + chunk * kChunk);
    if (L <= 0) {
        if (tid < kLanes) dst[tid] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int n = min((int)(((int64_t)L + P - 1) / P), NP);
    const float* ml = a.max_logits + r * NP;
    const float* es = a.exp_sums + r * NP;
    // row i of this workgroup's 64-dim slice of tmp_out
    const float4* to = reinterpret_cast<const float4*>(a.tmp_out + r * NP * D + chunk * kChunk);
    constexpr int kRow4 = D / 4;  // float4 stride between partitions
    if (n == 1) {  // a single partition is already normalised
        if (tid < kLanes) dst[tid] = to[tid];
        return;
    }

    // Issue every load first: the first kPre partitions' float4 of this
    // thread (they do not depend on the weights), then the statistics.
    const int c = tid % kLanes, grp = tid / kLanes;
    float4 pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int i = grp + k * kGroups;
        pre[k] = i < n ? to[(int64_t)i * kRow4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mx = -INFINITY;
    for (int i = tid; i < n; i += 256) mx = fmaxf(mx, ml[i]);
    mx = wave_max(mx);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();

    float ws = 0.f;
    for (int i = tid; i < n; i += 256) ws += es[i] * __builtin_amdgcn_exp2f(ml[i] - M);
    ws = wave_sum(ws);
    if (lane == 0) s_red[wave] = ws;
    __syncthreads();
    const float W = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int i = grp + k * kGroups;
        if (i < n) fma4(acc, es[i] * __builtin_amdgcn_exp2f(ml[i] - M), pre[k]);
    }
    int i = grp + kPre * kGroups;
    for (; i + 3 * kGroups < n; i += 4 * kGroups) {
        const float4 o0 = to[(int64_t)i * kRow4 + c];
        const float4 o1 = to[(int64_t)(i + kGroups) * kRow4 + c];
        const float4 o2 = to[(int64_t)(i + 2 * kGroups) * kRow4 + c];
        const float4 o3 = to[(int64_t)(i + 3 * kGroups) * kRow4 + c];
        fma4(acc, es[i] * __builtin_amdgcn_exp2f(ml[i] - M), o0);
        fma4(acc, es[i + kGroups] * __builtin_amdgcn_exp2f(ml[i + kGroups] - M), o1);
        fma4(acc, es[i + 2 * kGroups] * __builtin_amdgcn_exp2f(ml[i + 2 * kGroups] - M), o2);
        fma4(acc, es[i + 3 * kGroups] * __builtin_amdgcn_exp2f(ml[i + 3 * kGroups] - M), o3);
    }
    for (; i < n; i += kGroups)
        fma4(acc, es[i] * __builtin_amdgcn_exp2f(ml[i] - M), to[(int64_t)i * kRow4 + c]);
    s_part[grp][c] = acc;
    __syncthreads();
    if (tid < kLanes) {
        float4 t = s_part[0][tid];
#pragma unroll
        for (int gi = 1; gi < kGroups; ++gi) {
            const float4 u = s_part[gi][tid];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        dst[tid] = make_float4(t.x / W, t.y / W, t.z / W, t.w / W);
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, dim3 grid, hipStream_t stream,
                         bool* geometry_ok) {
    *geometry_ok = true;
    const dim3 g(head_dim / kChunk, grid.x, grid.y);
    if (head_dim == 128) {
        hipLaunchKernelGGL(reduce_kernel<128>, g, dim3(256), 0, stream, a);
    } else if (head_dim == 256) {
        hipLaunchKernelGGL(reduce_kernel<256>, g, dim3(256), 0, stream, a);
    } else {
        *geometry_ok = false;
        return hipSuccess;
    }
    return hipGetLastError();
}

}  // namespace vk
