// Split-KV partition reduce for gfx950 (vllm-metal kernels page,
// cf-1.com/news/5525226, section "GQA 解码内核的四个提速技巧", item 4: partials
// are (max in log2 units, exp-sum, normalised output) and a shared reducer
// merges them).
//
// One workgroup of 256 threads per (query head, sequence).  With n partitions:
//   M   = max_i m_i                       (block max)
//   w_i = l_i * 2^(m_i - M),  W = sum w_i (block sum)
//   out = sum_i w_i o_i / W               (float4 lanes over the head dims,
//                                          groups of lanes over partitions,
//                                          LDS sum of the groups)
#include "vk_kernels.h"

namespace vk {
namespace {

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

template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
    constexpr int LANES = D / 4;            // float4 lanes per head row
    constexpr int GROUPS = 256 / LANES;     // partition groups
    __shared__ float s_red[4];
    __shared__ float4 s_part[GROUPS][LANES];

    const int h = blockIdx.x, s = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int Hq = a.num_q_heads, P = a.partition_size, NP = a.max_num_partitions;
    const int64_t r = (int64_t)s * Hq + h;
    float* dst = a.out + r * D;
    const int L = a.seq_lens[s];
    if (L <= 0) {
        for (int d = tid; d < D; d += 256) dst[d] = 0.f;
        return;
    }
    const int n = min((int)(((int64_t)L + P - 1) / P), NP);
    const float* ml = a.max_logits + r * NP;
    const float* es = a.exp_sums + r * NP;
    const float4* to = reinterpret_cast<const float4*>(a.tmp_out + r * NP * D);
    float4* dst4 = reinterpret_cast<float4*>(dst);
    if (n == 1) {  // a single partition is already normalised
        if (tid < LANES) dst4[tid] = to[tid];
        return;
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

    const int dl = tid % LANES, grp = tid / LANES;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = grp; i < n; i += GROUPS) {
        const float w = es[i] * __builtin_amdgcn_exp2f(ml[i] - M);
        const float4 o = to[(int64_t)i * LANES + dl];
        acc.x = fmaf(w, o.x, acc.x);
        acc.y = fmaf(w, o.y, acc.y);
        acc.z = fmaf(w, o.z, acc.z);
        acc.w = fmaf(w, o.w, acc.w);
    }
    s_part[grp][dl] = acc;
    __syncthreads();
    if (tid < LANES) {
        float4 t = s_part[0][tid];
#pragma unroll
        for (int gi = 1; gi < GROUPS; ++gi) {
            const float4 u = s_part[gi][tid];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
        }
        dst4[tid] = make_float4(t.x / W, t.y / W, t.z / W, t.w / W);
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, dim3 grid, hipStream_t stream,
                         bool* geometry_ok) {
    *geometry_ok = true;
    if (head_dim == 128) {
        hipLaunchKernelGGL(reduce_kernel<128>, grid, dim3(256), 0, stream, a);
    } else if (head_dim == 256) {
        hipLaunchKernelGGL(reduce_kernel<256>, grid, dim3(256), 0, stream, a);
    } else {
        *geometry_ok = false;
        return hipSuccess;
    }
    return hipGetLastError();
}

}  // namespace vk
