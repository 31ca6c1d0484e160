// The split-KV merge (vllm-metal kernels page, cf-1.com/news/5525226, section
// "GQA 解码内核的四个提速技巧", item 4: partials are (max in log2 units,
// exp-sum, normalised output), and the GQA path reuses one reducer that forms
//   out = sum_i l_i 2^(m_i - M) o_i / sum_i l_i 2^(m_i - M),  M = max_i m_i).
//
// One wave64 merges 32 output dims (one 128-byte line of every partial row)
// of one (sequence, query head): lane l owns float4 column l % 8 and
// partitions i = l / 8 (mod 8).  It folds its partitions into a running
// (max, exp-sum, weighted sum) in one pass (the log2-space merge the decode
// uses between tokens), with the loads of up to 16 partitions issued ahead of
// the arithmetic; the 8 lane states of a column are then merged with lane
// shuffles.  No LDS, no barriers.  Used by the separate reduce kernel and by
// the single-launch decode, whose last workgroup per KV head runs it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vk {
namespace merge {

constexpr int kDims = 32;            // output dims per wave
constexpr int kCols = kDims / 4;     // float4 columns
constexpr int kGroups = 64 / kCols;  // partition groups (lanes per column)
constexpr int kBatch = 16;           // partitions per lane loaded ahead

struct State {
    float m, l;
    float4 acc;
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold partial (m, l, o) into s: everything is rescaled to the larger max.
__device__ __forceinline__ void fold(State& s, float m, float l, const float4& o) {
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
__device__ __forceinline__ void fold_state(State& s, const State& t) {
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

// Merge partitions i < n (n >= 1) of one (sequence, head) for dims
// [chunk, chunk + 32): ml/es point at the row's max_logits/exp_sums, `to` at
// tmp_out[row][0][chunk], `row4` is the float4 stride between partitions
// (D / 4); dst receives the 32 merged dims.  n == 1 copies exactly.
__device__ __forceinline__ void merge_columns(const float* ml, const float* es, const float4* to,
                                              int row4, int n, int lane, float4* dst) {
    const int c = lane % kCols, grp = lane / kCols;
    if (n == 1) {   // a single partition is already normalised
        if (lane < kCols) dst[lane] = to[lane];
        return;
    }
    State st;
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
            o[k] = ok ? to[(int64_t)i * row4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (m[k] != -INFINITY) fold(st, m[k], l[k], o[k]);
    }
#pragma unroll
    for (int off = kCols; off < 64; off <<= 1) {
        State t;
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

// The same merge for NB pieces of work at once (one (sequence, head, 32 dims)
// each, `ok[b]` false for an unused piece) when every piece has n <= kGroups
// partitions: each lane holds at most one partition per piece, so all the
// pieces' loads are issued before the first fold, where merge_columns would
// wait for one piece's loads at a time.  Per piece the steps are those of
// merge_columns (one fold of partition lane / kCols into the empty state,
// then the same shuffle tree), so the results are bit-identical to it.
template <int NB>
__device__ __forceinline__ void merge_columns_few(const float* const (&ml)[NB],
                                                  const float* const (&es)[NB],
                                                  const float4* const (&to)[NB],
                                                  const bool (&ok)[NB], int row4, int n, int lane,
                                                  float4* const (&dst)[NB]) {
    const int c = lane % kCols, grp = lane / kCols;
    float m[NB], l[NB];
    float4 o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const bool ld = ok[b] && grp < n;
        m[b] = ld ? ml[b][grp] : -INFINITY;
        l[b] = ld ? es[b][grp] : 0.f;
        o[b] = ld ? to[b][(int64_t)grp * row4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        State st;
        st.m = -INFINITY;
        st.l = 0.f;
        st.acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m[b] != -INFINITY) fold(st, m[b], l[b], o[b]);
#pragma unroll
        for (int off = kCols; off < 64; off <<= 1) {
            State t;
            t.m = __shfl_xor(st.m, off);
            t.l = __shfl_xor(st.l, off);
            t.acc.x = __shfl_xor(st.acc.x, off);
            t.acc.y = __shfl_xor(st.acc.y, off);
            t.acc.z = __shfl_xor(st.acc.z, off);
            t.acc.w = __shfl_xor(st.acc.w, off);
            fold_state(st, t);
        }
        if (ok[b] && lane < kCols)
            dst[b][lane] = make_float4(st.acc.x / st.l, st.acc.y / st.l, st.acc.z / st.l,
                                       st.acc.w / st.l);
    }
}

}  // namespace merge
}  // namespace vk
