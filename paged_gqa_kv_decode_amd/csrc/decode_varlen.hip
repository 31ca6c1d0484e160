// Several query tokens per sequence over the paged KV cache, causal, on the
// gfx950 matrix cores: speculative-decode verification (a few draft tokens)
// and chunked prefill (a chunk of new tokens) in one kernel (the vllm-metal
// kernels page, cf-1.com/news/5525226, section "什么是 Paged Attention",
// names a unified paged variable-length kernel for both).  Sequence s owns
// the packed query rows cu_q[s] .. cu_q[s+1]-1; its cache already holds all
// L tokens, the new ones last, so query j (position L - qlen + j) sees the
// tokens t < L - qlen + j + 1.
//
// The decode kernel's matrix-core step is reused unchanged (MfmaKernel in
// decode_mfma_impl.h: 16-token steps, K as the A operand, V transposed in
// registers, the next step's K/V loaded straight into the wave's LDS slots
// while the current one computes).  What changes is the meaning of the 16
// MFMA columns: in the
// decode they are the G heads of a KV group; here they are (query token,
// head) pairs, 16 / G tokens x G heads per tile, so every K/V load of a step
// serves that many queries.  Each column carries its own causal limit; the
// scores past it are masked by select.  One wave per workgroup = one column
// tile of one (sequence, KV head) over one partition of the keys (split-KV,
// merged by the variable-length reduce) or over all of them (unsplit).
#include "decode_mfma_impl.h"

namespace vk {
namespace {

// DT: element type of q, K and V (0 fp16, 1 bf16; the decode's bf16 steps,
// weights split into a bf16 value and its residual for PV).
template <int D, int G, int BS, int DT>
struct VarlenKernel {
    using M = MfmaKernel<D, G, BS, 1, 1, 16, false, DT>;
    using Buf = typename M::Buf;
    using State = typename M::State;
    static constexpr int TPT = 16 / G;    // query tokens per column tile
    static constexpr int NC = TPT * G;    // columns in use
    static constexpr int NKC = M::NKC, NDH = M::NDH, NPT = M::NPT, CH = M::CH;
    static_assert(M::PF, "16-bit types: LDS prefetch");
    static_assert(16 * D * 4 <= M::WAVE_LDS, "output staging fits the prefetch slots");

    // Column col of the tile: its row, and whether and what it writes for
    // this launch item (0 nothing, 1 zeros: unsplit and no visible key,
    // 2 its result); `cbad` poisons a written result.
    struct Col {
        int64_t row;
        int mode;
        bool cbad;
    };
    static __device__ __forceinline__ Col column(const VarlenArgs& va, int col, int tile, int part,
                                                 int g, int q0, int qlen, int L, int t_begin,
                                                 bool wave_bad) {
        const DecodeArgs& a = va.d;
        const int P = a.partition_size, NP = a.max_num_partitions;
        const int jt = tile * TPT + col / G;
        const bool valid = col < NC && jt < qlen;
        const int lim = valid ? L - qlen + jt + 1 : 0;
        Col r;
        r.row = ((int64_t)q0 + jt) * a.num_q_heads + g * G + col % G;
        r.mode = !valid ? 0 : (P == 0 && lim <= 0) ? 1 : (lim <= t_begin) ? 0 : 2;
        r.cbad = wave_bad || (P > 0 && part == NP - 1 && lim > t_begin + P);
        return r;
    }

    // QK of one 16-key step and the online-softmax update per column; `rem`
    // is how many of the step's keys this lane's column may see (<= 0: none).
    static __device__ __forceinline__ uint4 qk_softmax(const DecodeArgs& a, State& st, const Buf& b,
                                                       const uint4 (&qb)[NKC], int rem, int c) {
        floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) sc = M::qk_mma(b.kr[0][kk], qb[kk], sc);
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = mul_rounded(sc[r], a.scale_log2e);
            x[r] = (4 * c + r) < rem ? v : -INFINITY;
        }
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(st.m, mx);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2_fast(st.m - mref);
        float p[4];
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = exp2_fast(x[r] - mref) * M::kPScale;
            ps += p[r];
        }
        st.l = st.l * alpha + ps;
        st.m = mnew;
#pragma unroll
        for (int t = 0; t < NPT; ++t) st.acc[t] *= alpha;
        return M::pack_weights(p[0], p[1], p[2], p[3]);
    }

    static __device__ void run(const VarlenArgs& va) {
        const DecodeArgs& a = va.d;
        const int lane = threadIdx.x, i = lane & 15, c = lane >> 4;
        int tile, part, g, s;
        if (a.work_order == 1) {
            // One tile per sequence (the host's condition for this order):
            // the items are the decode's (partition, KV head, sequence), so
            // its longest-first mapping applies as it is.
            if (!M::longest_first(a, part, g, s)) return;
            tile = 0;
        } else {
            tile = (int)(blockIdx.x % (unsigned)va.tiles);
            part = (int)(blockIdx.x / (unsigned)va.tiles);
            g = blockIdx.y;
            s = blockIdx.z;
        }
        const int q0 = va.cu_q[s], qlen = va.cu_q[s + 1] - q0;
        if (qlen <= 0 || tile * TPT >= qlen) return;
        const int Hq = a.num_q_heads, P = a.partition_size, NP = a.max_num_partitions;

        // A length beyond the page table poisons the whole sequence: its rows
        // that see keys become NaN and nothing of it is read.
        const int L = a.seq_lens[s];
        const bool poison = L > a.max_blocks_per_seq * BS;
        // Column i: query token jt of the sequence, head h.
        const int jt = tile * TPT + i / G;
        const int h = g * G + i % G;
        const bool valid = i < NC && jt < qlen;
        const int lim = valid ? L - qlen + jt + 1 : 0;           // keys this column sees
        int kv_end = lim;                                        // the wave's key range
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) kv_end = max(kv_end, __shfl_xor(kv_end, off));
        int t_begin = 0, t_end = kv_end;
        if (P > 0) {
            t_begin = part * P;
            t_end = min(kv_end, t_begin + P);
        }
        const int64_t row = ((int64_t)q0 + jt) * Hq + h;
        if (t_end <= t_begin || poison) {
            if (valid && P == 0) {            // no visible key: zeros; poisoned: NaN
                const float z = (poison && lim > 0) ? __builtin_nanf("") : 0.f;
                float* o = a.out + row * D;
                for (int d = 4 * c; d < D; d += 16) *reinterpret_cast<float4*>(o + d) = make_float4(z, z, z, z);
            } else if (valid && poison && lim > t_begin) {   // the partials the reduce will read
                const int64_t pr = row * NP + part;
                if (c == 0) a.max_logits[pr] = a.exp_sums[pr] = __builtin_nanf("");
                const float z = __builtin_nanf("");
                float* o = a.tmp_out + pr * D;
                for (int d = 4 * c; d < D; d += 16) *reinterpret_cast<float4*>(o + d) = make_float4(z, z, z, z);
            }
            return;
        }
        // The first chunk's page ids (clamped into the table row), then the
        // query columns: one round trip before the first K/V loads.
        const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
        const int32_t pg_first = bt[min(t_begin / BS + lane, a.max_blocks_per_seq - 1)];
        uint4 qb[NKC];
        {
            const uint4* qp = reinterpret_cast<const uint4*>(a.q + (valid ? row : 0) * D);
#pragma unroll
            for (int kk = 0; kk < NKC; ++kk) qb[kk] = valid ? qp[4 * kk + c] : make_uint4(0, 0, 0, 0);
        }
        const int e_lim = min(lim, t_end);   // this column's last visible key + 1 here

        __shared__ __attribute__((aligned(16))) char lds[M::WAVE_LDS];
        State st;
#pragma unroll
        for (int t = 0; t < NPT; ++t) st.acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.f;
        bool bad = false;
        for (int c0 = t_begin; c0 < t_end; c0 += CH) {
            const int c1 = min(t_end, c0 + CH);
            const int np = (c1 - c0 + BS - 1) / BS;
            int pg = 0;
            if (lane < np) {
                pg = (c0 == t_begin) ? pg_first : bt[c0 / BS + lane];
                if (pg < 0 || (int64_t)pg >= a.num_blocks) {
                    pg = 0;
                    bad = true;
                }
            }
            // Full 16-key steps, then at most one partial step; step k + 1
            // is in flight to LDS while step k computes.
            const int nfull = (c1 - c0) / 16;
            const int tl = c0 + 16 * nfull;
            if (nfull > 0)
                M::template issue_lds<true>(a, lds, M::step_pages(pg, 0), g, 16, i, c);
            else if (tl < c1)
                M::template issue_lds<false>(a, lds, M::step_pages(pg, tl - c0), g, c1 - tl, i, c);
            for (int k = 0; k < nfull; ++k) {
                Buf b;
                M::wait_lds_loads();
                M::template read_lds<true>(b, lds, 16, lane, i, c);
                M::wait_lds_reads();
                if (k + 1 < nfull)
                    M::template issue_lds<true>(a, lds, M::step_pages(pg, 16 * (k + 1)), g, 16, i, c);
                else if (tl < c1)
                    M::template issue_lds<false>(a, lds, M::step_pages(pg, tl - c0), g, c1 - tl, i, c);
                const int t0 = c0 + 16 * k;
                M::pv(st, b, qk_softmax(a, st, b, qb, e_lim - t0, c));
            }
            if (tl < c1) {
                Buf b;
                M::wait_lds_loads();
                M::template read_lds<false>(b, lds, c1 - tl, lane, i, c);
                M::wait_lds_reads();
                M::pv(st, b, qk_softmax(a, st, b, qb, min(e_lim, c1) - tl, c));
            }
        }
        float lsum = st.l + __shfl_xor(st.l, 16);
        lsum += __shfl_xor(lsum, 32);
        const bool wave_bad = __ballot(bad) != 0;

        // The accumulator layout scatters a column's dims over the lanes; the
        // normalised columns go through the (now idle) prefetch slots and
        // leave as 16-byte stores, one row of D floats per column.
        float* stage = reinterpret_cast<float*>(lds);
        if (valid) {
#pragma unroll
            for (int dh = 0; dh < NDH; ++dh)
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        stage[i * D + 128 * dh + 8 * (4 * c + rr) + e] = st.acc[dh * 8 + e][rr] / lsum;
        }
        if (c == 0) {
            const Col me = column(va, i, tile, part, g, q0, qlen, L, t_begin, wave_bad);
            if (P > 0 && me.mode == 2) {
                const int64_t pr = me.row * NP + part;
                M::store_partial1(a, a.max_logits + pr, st.m);
                M::store_partial1(a, a.exp_sums + pr, me.cbad ? __builtin_nanf("") : lsum * M::kInvPScale);
            }
        }
        __syncthreads();
        const float nanv = __builtin_nanf("");
        for (int e = lane; e < 16 * (D / 4); e += 64) {
            const int col = e / (D / 4), d = 4 * (e % (D / 4));
            const Col cl = column(va, col, tile, part, g, q0, qlen, L, t_begin, wave_bad);
            if (cl.mode == 0) continue;
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (cl.mode == 2)
                o = cl.cbad ? make_float4(nanv, nanv, nanv, nanv)
                            : *reinterpret_cast<const float4*>(stage + col * D + d);
            if (P == 0)
                *reinterpret_cast<float4*>(a.out + cl.row * D + d) = o;
            else
                M::store_partial(a, a.tmp_out + (cl.row * NP + part) * D + d, o);
        }
    }
};

template <int D, int G, int BS, int DT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(VK_MFMA_WAVES_PER_EU)))
void decode_varlen_kernel(VarlenArgs a) {
    VarlenKernel<D, G, BS, DT>::run(a);
}

template <int D, int G, int DT>
hipError_t launch_bs_dt(const VarlenArgs& a, int bs, dim3 grid, hipStream_t st, bool* ok) {
    *ok = true;
    switch (bs) {
        case 8: hipLaunchKernelGGL((decode_varlen_kernel<D, G, 8, DT>), grid, dim3(64), 0, st, a); break;
        case 16: hipLaunchKernelGGL((decode_varlen_kernel<D, G, 16, DT>), grid, dim3(64), 0, st, a); break;
        case 32: hipLaunchKernelGGL((decode_varlen_kernel<D, G, 32, DT>), grid, dim3(64), 0, st, a); break;
        default: *ok = false; return hipSuccess;
    }
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_bs(const VarlenArgs& a, int dtype, int bs, dim3 grid, hipStream_t st, bool* ok) {
    if (dtype == 1) return launch_bs_dt<D, G, 1>(a, bs, grid, st, ok);
    return launch_bs_dt<D, G, 0>(a, bs, grid, st, ok);
}

}  // namespace

int varlen_tokens_per_tile(int group) { return group > 0 && group <= 16 ? 16 / group : 0; }

hipError_t launch_decode_varlen(const VarlenArgs& a, int dtype, int group, int head_dim,
                                int block_size, dim3 grid, hipStream_t stream, bool* geometry_ok) {
    if (group == 4 && head_dim == 128) return launch_bs<128, 4>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 6 && head_dim == 256) return launch_bs<256, 6>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 8 && head_dim == 128) return launch_bs<128, 8>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 8 && head_dim == 256) return launch_bs<256, 8>(a, dtype, block_size, grid, stream, geometry_ok);
    // multi-head: 16 query tokens of one head per tile; multi-query: 1 token x 16 heads
    if (group == 1 && head_dim == 128) return launch_bs<128, 1>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 1 && head_dim == 256) return launch_bs<256, 1>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 16 && head_dim == 128) return launch_bs<128, 16>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 16 && head_dim == 256) return launch_bs<256, 16>(a, dtype, block_size, grid, stream, geometry_ok);
    *geometry_ok = false;
    return hipSuccess;
}

}  // namespace vk
