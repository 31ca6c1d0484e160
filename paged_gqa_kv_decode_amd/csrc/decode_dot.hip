// Paged GQA decode attention, VALU kernel family for gfx950 (VK_KERNEL_DOT).
//
// One workgroup per (partition, KV head, sequence); all G query heads of the
// group live in the workgroup, so every K/V page of the partition is read from
// HBM once and serves the whole group (vllm-metal kernels page,
// cf-1.com/news/5525226, section "Metal 并行模型").
//
// Work split inside the workgroup (4 wave64s = 16 rows of 16 lanes):
//  * each 16-lane row owns one token at a time; lane `col` of the row owns
//    head dims [8 col, 8 col + 8) (and [128 + 8 col, ...) for D = 256), i.e.
//    one 16-byte load per 128 dims, so a row reads whole 256-byte K/V rows;
//  * q . k is 4 (8) packed fp16 dot2 instructions per lane and a 4-step DPP
//    butterfly over the row; every lane of the row ends with the same sum;
//  * each row keeps its own online-softmax state per head (running max m in
//    log2 units, exp-sum l, fp32 accumulator), updated once per step of N
//    tokens per row (section "GQA 解码内核的四个提速技巧", items 1 and 3);
//  * the 16 row states are merged at the end of the partition: across the 4
//    rows of a wave with lane shuffles, across the 4 waves through LDS.
// The partition's page ids are staged once in LDS (at most 64 per chunk) and
// read per token, so page-id latency never sits in front of each K/V load
// (item 2 of the same section).  Tokens past the end are masked by select:
// their K/V registers are zero and their scores -inf.
#include "vk_kernels.h"
#include "vk_constants.h"

namespace vk {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8(const uint4& k, const uint4& q, float acc) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, k.x), __builtin_bit_cast(half2v, q.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, k.y), __builtin_bit_cast(half2v, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, k.z), __builtin_bit_cast(half2v, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, k.w), __builtin_bit_cast(half2v, q.w), acc, false);
    return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; all 16 lanes get bit-identical totals.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A product that is rounded to fp32 and never fused into a later add.
__device__ __forceinline__ float mul_rounded(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

__device__ __forceinline__ float half_at(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (float)__builtin_bit_cast(half2v, w)[e & 1];
}

template <int D, int G, int BS>
struct DotKernel {
    static constexpr int NV = D / 128;               // 16-byte chunks per lane per row
    static constexpr int N = (D == 128) ? 4 : 2;     // tokens per row per step
    static constexpr int STEP = 16 * N;              // tokens per workgroup step
    static constexpr int CH_PAGES = 64;
    static constexpr int CH = CH_PAGES * BS;         // tokens per staged page chunk
    static constexpr int E = 8 * NV;                 // dims per lane

    struct State {
        float m[G], l[G], acc[G][E];
    };

    template <bool FULL>
    static __device__ __forceinline__ void step(const DecodeArgs& a, State& st,
                                                const uint4 (&qv)[G][NV], const int* s_pages,
                                                int g, int c0, int c1, int t0, int slot, int col) {
        const int64_t head_stride = (int64_t)BS * D;
        uint4 kr[N][NV], vr[N][NV];
        bool valid[N];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int t = t0 + slot + 16 * n;
            valid[n] = FULL || t < c1;
            if (valid[n]) {
                const int pid = s_pages[(t - c0) / BS];
                const int64_t off = ((int64_t)pid * a.num_kv_heads + g) * head_stride +
                                    (int64_t)(t % BS) * D + col * 8;
#pragma unroll
                for (int nv = 0; nv < NV; ++nv) {
                    kr[n][nv] = *reinterpret_cast<const uint4*>(a.k + off + nv * 128);
                    vr[n][nv] = *reinterpret_cast<const uint4*>(a.v + off + nv * 128);
                }
            } else {
#pragma unroll
                for (int nv = 0; nv < NV; ++nv) {
                    kr[n][nv] = make_uint4(0, 0, 0, 0);
                    vr[n][nv] = make_uint4(0, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float x[N];
#pragma unroll
            for (int n = 0; n < N; ++n) {
                float d = 0.f;
#pragma unroll
                for (int nv = 0; nv < NV; ++nv) d = dot8(kr[n][nv], qv[h][nv], d);
                // Round the score once (no contraction into the later x - m):
                // the running max and the exponent see the same value, so the
                // maximal token gets a weight of exactly 1.
                d = mul_rounded(row16_sum(d), a.scale_log2e);
                x[n] = valid[n] ? d : -INFINITY;
            }
            float mx = x[0];
#pragma unroll
            for (int n = 1; n < N; ++n) mx = fmaxf(mx, x[n]);
            const float mnew = fmaxf(st.m[h], mx);
            const float mref = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = exp2_fast(st.m[h] - mref);
            float p[N];
            float ps = 0.f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                p[n] = exp2_fast(x[n] - mref);
                ps += p[n];
            }
            st.l[h] = st.l[h] * alpha + ps;
            st.m[h] = mnew;
#pragma unroll
            for (int nv = 0; nv < NV; ++nv) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float v = st.acc[h][nv * 8 + e] * alpha;
#pragma unroll
                    for (int n = 0; n < N; ++n) v = fmaf(p[n], half_at(vr[n][nv], e), v);
                    st.acc[h][nv * 8 + e] = v;
                }
            }
        }
    }

    static __device__ void run(const DecodeArgs& a) {
        __shared__ int s_pages[CH_PAGES];
        __shared__ int s_poison;
        __shared__ float s_acc[4][G][D];
        __shared__ float s_m[4][G];
        __shared__ float s_l[4][G];

        const int part = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
        const int row = lane >> 4, col = lane & 15;
        const int slot = wave * 4 + row;
        const int Hq = a.num_q_heads;
        const int P = a.partition_size, NP = a.max_num_partitions;

        int L = a.seq_lens[s];
        bool poison = false;
        const int cap = a.max_blocks_per_seq * BS;
        if (L > cap) {
            L = cap;
            poison = true;
        }
        int t_begin = 0, t_end = L;
        if (P > 0) {
            t_begin = part * P;
            t_end = min(L, t_begin + P);
            if (part == NP - 1 && L > t_begin + P) poison = true;  // beyond the grid
        }
        if (t_end <= t_begin) {
            if (P == 0) {  // empty sequence, unsplit: zeros
                float* o = a.out + ((int64_t)s * Hq + g * G) * D;
                for (int i = tid; i < G * D; i += 256) o[i] = 0.f;
            }
            return;  // split: partitions past the end write nothing
        }
        if (tid == 0) s_poison = 0;

        uint4 qv[G][NV];
        const uint16_t* qb = a.q + ((int64_t)s * Hq + g * G) * D + col * 8;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int nv = 0; nv < NV; ++nv)
                qv[h][nv] = *reinterpret_cast<const uint4*>(qb + h * D + nv * 128);

        State st;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            st.m[h] = -INFINITY;
            st.l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) st.acc[h][e] = 0.f;
        }

        const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
        for (int c0 = t_begin; c0 < t_end; c0 += CH) {
            const int c1 = min(t_end, c0 + CH);
            __syncthreads();  // the previous chunk's page ids are no longer read
            if (tid < CH_PAGES) {
                const int np = (c1 - c0 + BS - 1) / BS;
                if (tid < np) {
                    int pid = bt[c0 / BS + tid];
                    if (pid < 0 || (int64_t)pid >= a.num_blocks) {
                        pid = 0;
                        s_poison = 1;
                    }
                    s_pages[tid] = pid;
                }
            }
            __syncthreads();
            int t0 = c0;
            for (; t0 + STEP <= c1; t0 += STEP) step<true>(a, st, qv, s_pages, g, c0, c1, t0, slot, col);
            if (t0 < c1) step<false>(a, st, qv, s_pages, g, c0, c1, t0, slot, col);
        }

        // Merge the 4 rows of the wave: lanes col, col+16, col+32, col+48 hold
        // the same dims for different token rows.
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float M = fmaxf(st.m[h], __shfl_xor(st.m[h], 16));
            M = fmaxf(M, __shfl_xor(M, 32));
            const float sc = (st.m[h] == -INFINITY) ? 0.f : exp2_fast(st.m[h] - M);
            float lh = st.l[h] * sc;
            lh += __shfl_xor(lh, 16);
            lh += __shfl_xor(lh, 32);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float v = st.acc[h][e] * sc;
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                st.acc[h][e] = v;
            }
            st.m[h] = M;
            st.l[h] = lh;
        }
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
#pragma unroll
                for (int nv = 0; nv < NV; ++nv)
#pragma unroll
                    for (int e = 0; e < 8; ++e) s_acc[wave][h][nv * 128 + col * 8 + e] = st.acc[h][nv * 8 + e];
                if (col == 0) {
                    s_m[wave][h] = st.m[h];
                    s_l[wave][h] = st.l[h];
                }
            }
        }
        __syncthreads();
        const bool bad = poison || s_poison;
        for (int idx = tid; idx < G * D; idx += 256) {
            const int h = idx / D, d = idx % D;
            float M = s_m[0][h];
#pragma unroll
            for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float mw = s_m[w][h];
                const float sc = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
                num += sc * s_acc[w][h][d];
                den += sc * s_l[w][h];
            }
            const float o = bad ? __builtin_nanf("") : num / den;
            const int64_t r = (int64_t)s * Hq + g * G + h;
            if (P == 0) {
                a.out[r * D + d] = o;
            } else {
                const int64_t pr = r * NP + part;
                a.tmp_out[pr * D + d] = o;
                if (d == 0) {
                    a.max_logits[pr] = M;
                    a.exp_sums[pr] = bad ? __builtin_nanf("") : den;
                }
            }
        }
    }
};

template <int D, int G, int BS>
__global__ __launch_bounds__(256) void decode_dot_kernel(DecodeArgs a) {
    DotKernel<D, G, BS>::run(a);
}

template <int D, int G>
hipError_t launch_bs(const DecodeArgs& a, int bs, dim3 grid, hipStream_t st, bool* ok) {
    *ok = true;
    switch (bs) {
        case 8: hipLaunchKernelGGL((decode_dot_kernel<D, G, 8>), grid, dim3(256), 0, st, a); break;
        case 16: hipLaunchKernelGGL((decode_dot_kernel<D, G, 16>), grid, dim3(256), 0, st, a); break;
        case 32: hipLaunchKernelGGL((decode_dot_kernel<D, G, 32>), grid, dim3(256), 0, st, a); break;
        default: *ok = false; return hipSuccess;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_dot(const DecodeArgs& a, int group, int head_dim, int block_size,
                             dim3 grid, hipStream_t stream, bool* geometry_ok, int* block) {
    *block = 256;
    if (group == 4 && head_dim == 128) return launch_bs<128, 4>(a, block_size, grid, stream, geometry_ok);
    if (group == 6 && head_dim == 256) return launch_bs<256, 6>(a, block_size, grid, stream, geometry_ok);
    if (group == 8 && head_dim == 128) return launch_bs<128, 8>(a, block_size, grid, stream, geometry_ok);
    if (group == 8 && head_dim == 256) return launch_bs<256, 8>(a, block_size, grid, stream, geometry_ok);
    *geometry_ok = false;
    return hipSuccess;
}

}  // namespace vk
