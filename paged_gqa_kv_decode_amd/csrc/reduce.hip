// Split-KV partition reduce for gfx950 (vllm-metal kernels page,
// cf-1.com/news/5525226, section "GQA 解码内核的四个提速技巧", item 4: partials
// are (max in log2 units, exp-sum, normalised output) and a shared reducer
// merges them into
//   out = sum_i l_i 2^(m_i - M) o_i / sum_i l_i 2^(m_i - M),  M = max_i m_i).
//
// Grid (D / 32, Hq, S), one wave64 per 32 output dims (one 128-byte line of
// every partial row, so no line is split between waves on different XCDs)
// of one (sequence, query head).  Lane l owns float4 column l % 8 and
// partitions i = l / 8 (mod 8).
// It folds its partitions into a running (max, exp-sum, weighted sum) in one
// pass (the same log2-space merge the decode uses between tokens), with the
// loads of up to 16 partitions issued ahead of the arithmetic; the 8 lane
// states of a column are then merged with lane shuffles.  No LDS, no
// barriers: the wave's whole working set is in flight at once.
#include "vk_kernels.h"

namespace vk {
namespace {

constexpr int kDims = 32;        // output dims per wave
constexpr int kCols = kDims / 4; // float4 columns
constexpr int kGroups = 64 / kCols;  // partition groups (lanes per column)
constexpr int kBatch = 16;       // partitions per lane loaded ahead

struct Merge {
    float m, l;
    float4 acc;
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold partial (m, l, o) into s: everything is rescaled to the larger max.
__device__ __forceinline__ void fold(Merge& s, float m, float l, const float4& o) {
    const float M = fmaxf(s.m, m);
    const float a = (s.m == -INFINITY) ? 0.f : exp2_fast(s.m - M);
    const float w = l * exp2_fast(m - M);
    s.l = s.l * a + w;
    s.acc.x = s.acc.x * a + w * o.x;
    s.acc.y = s.acc.y * a + w * o.y;
    s.acc.z = s.acc.z * a + w * o.z;
    s.acc.w = s.acc.w * a + w * o.w;
    s.m = M;
}

// Fold another lane's running state (whose acc is a weighted sum, not a mean).
__device__ __forceinline__ void fold_state(Merge& s, const Merge& t) {
    const float M = fmaxf(s.m, t.m);
    const float a = (s.m == -INFINITY) ? 0.f : exp2_fast(s.m - M);
    const float b = (t.m == -INFINITY) ? 0.f : exp2_fast(t.m - M);
    s.l = s.l * a + t.l * b;
    s.acc.x = s.acc.x * a + t.acc.x * b;
    s.acc.y = s.acc.y * a + t.acc.y * b;
    s.acc.z = s.acc.z * a + t.acc.z * b;
    s.acc.w = s.acc.w * a + t.acc.w * b;
    s.m = M;
}

template <int D>
__global__ __launch_bounds__(64) void reduce_kernel(ReduceArgs a) {
    const int chunk = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int lane = threadIdx.x;
    const int c = lane % kCols, grp = lane / kCols;
    const int Hq = a.num_q_heads, P = a.partition_size, NP = a.max_num_partitions;
    const int64_t r = (int64_t)s * Hq + h;
    const int L = a.seq_lens[s];
    float4* dst = reinterpret_cast<float4*>(a.out + r * D + chunk * kDims);
    if (L <= 0) {
        if (lane < kCols) dst[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int n = min((int)(((int64_t)L + P - 1) / P), NP);
    const float* ml = a.max_logits + r * NP;
    const float* es = a.exp_sums + r * NP;
    const float4* to = reinterpret_cast<const float4*>(a.tmp_out + r * NP * D + chunk * kDims);
    constexpr int kRow4 = D / 4;   // float4 stride between partitions
    if (n == 1) {                  // a single partition is already normalised
        if (lane < kCols) dst[lane] = to[lane];
        return;
    }

    Merge st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = grp; i0 < n; i0 += kBatch * kGroups) {
        float m[kBatch], l[kBatch];
        float4 o[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * kGroups;
            const bool ok = i < n;
            m[k] = ok ? ml[i] : -INFINITY;
            l[k] = ok ? es[i] : 0.f;
            o[k] = ok ? to[(int64_t)i * kRow4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (m[k] != -INFINITY) fold(st, m[k], l[k], o[k]);
    }
#pragma unroll
    for (int off = kCols; off < 64; off <<= 1) {
        Merge t;
        t.m = __shfl_xor(st.m, off);
        t.l = __shfl_xor(st.l, off);
        t.acc.x = __shfl_xor(st.acc.x, off);
        t.acc.y = __shfl_xor(st.acc.y, off);
        t.acc.z = __shfl_xor(st.acc.z, off);
        t.acc.w = __shfl_xor(st.acc.w, off);
        fold_state(st, t);
    }
    if (lane < kCols)
        dst[lane] = make_float4(st.acc.x / st.l, st.acc.y / st.l, st.acc.z / st.l, st.acc.w / st.l);
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, dim3 grid, hipStream_t stream,
                         bool* geometry_ok) {
    *geometry_ok = true;
    const dim3 g(head_dim / kDims, grid.x, grid.y);
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
