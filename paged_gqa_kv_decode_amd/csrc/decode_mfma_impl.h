// The matrix-core decode's workgroup code (MfmaKernel) and its tuning knobs,
// shared by the decode kernels (decode_mfma.hip) and the multi-token query
// kernels (decode_varlen.hip), which reuse its K/V step loads and PV product.
//
// Paged GQA decode attention on the gfx950 matrix cores (VK_KERNEL_MFMA).
//
// Why matrix cores: with G query heads per KV head the path does G flops per
// KV byte (4, 6 or 8).  With packed fp32 off, the VALU ridge is ~9.8 flop/B,
// so a VALU kernel spends most of its issue slots on arithmetic.  Both
// contractions of a KV-group step are small dense products:
//   S[t, h]  = sum_d K[t, d] Q[h, d]      (16 tokens x 16 heads x D)
//   O^T[d,h] += sum_t V^T[d, t] P^T[t, h]   (16 dims  x 16 heads x T tokens)
// and one v_mfma_f32_16x16x32_f16 (16x16x16 for T = 16) does each block,
// leaving the VALU only the softmax.  The G <= 8 heads fill half (or less) of
// the 16 columns; the matrix cores are far from busy either way.
//
// Workgroup = W wave64s per (partition, KV head, sequence) (vllm-metal
// kernels page, cf-1.com/news/5525226, section "Metal 并行模型": all query
// heads of the group share one pass over the group's K/V pages).  Each wave
// takes every W-th step of T = 16 tokens.  Per step and lane l
// (i = l % 16, c = l / 16):
//  * K: lane l holds token i, dims [32 kk + 8 c, +8) for kk < D/32: exactly
//    the MFMA A operand.  16-bit types load it through the wave's LDS slots
//    in whole 128-byte lines and read it back in this layout (issue_lds /
//    read_lds); fp32 loads it directly.  The B operand is Q^T: head i, the
//    same dims (zero for i >= G), held in registers for the whole partition.
//  * The QK output tile gives lane l head i and tokens 4c + r (r < 4): that
//    is exactly the B operand (P^T) of the 16x16x16 PV product, so P needs
//    no data movement, only packing to the element type.  16-bit types take
//    each weight as a rounded value plus its rounded residual (two PV
//    products), so the weights keep ~2^-22 (fp16) or ~2^-16 (bf16) relative
//    precision instead of the operand format's 2^-11 or 2^-8.
//  * V: lane l loads its 4 tokens' dims [128 dh + 8 i, +8) (whole 256-byte
//    half-rows per 16 lanes) and transposes the 4x8 block in registers with
//    v_perm_b32 into the PV A operands: tile (dh, e) holds d = 128 dh + 8 i + e.
//  * Online softmax in log2 space (section "GQA 解码内核的四个提速技巧",
//    item 1): per head, max over the step's tokens (in-lane, then across the
//    4 lane groups), one rescale of the accumulators per step, exp2 of
//    x - max, per-lane partial exp-sums (summed once at the end).
// Page ids: each wave holds up to 64 page ids of the current chunk in one
// register (lane k = page k, one coalesced load) and reads the step's 1-4 ids
// with readlane, so no dependent table load precedes each K/V load (item 2).
// Tokens past the end are masked by select (zeroed K/V registers, score -inf).

#pragma once

#include "merge_ops.h"
#include "mfma_ops.h"
#include "vk_constants.h"
#include "vk_kernels.h"

// Compile-time tuning knobs (defaults are the measured best on MI355X).
#ifndef VK_MFMA_WAVES_PER_EU
#define VK_MFMA_WAVES_PER_EU 2   // minimum resident waves per SIMD
#endif
#ifndef VK_MFMA_LDS_PF
#define VK_MFMA_LDS_PF 1         // 16-bit types: next step's K/V loaded straight into LDS
#endif
#ifndef VK_MFMA_ORDER
#define VK_MFMA_ORDER 1          // split launches of <= 64 sequences: longest-first work order
#endif

namespace vk {
namespace {

using namespace mfma;

// DT: element type of q, K and V (0 fp16, 1 bf16, 2 fp32).
//
// fp32 (DT = 2) runs the same steps on v_mfma_f32_16x16x4_f32: in QK product
// kk the k-slot of lane group c is dim c * D/4 + kk, so lane (token i, c)
// reads D/4 contiguous floats of its K row and the Q^T operand the same dims
// of head i; the QK output (lane: head i, tokens 4c + r) is again the PV B
// operand, one fp32 weight per product r.  In PV the A-operand row of lane i
// is dim 64 t' + 4 i + e in tile 4 t' + e, so one 16-byte read of V[token
// 4c + r][64 t' + 4 i, +4) feeds four products; accumulator tile 4 t' + e
// then holds dims 64 t' + 16 c + 4 rr + e in row rr of lane group c.
template <int D, int G, int BS, int W, int WP, int T, bool FUSED, int DT = 0>
struct MfmaKernel {
    static_assert(T == 16, "16 tokens per wave step");
    // WP waves share one partition; a workgroup covers PPW = W / WP
    // consecutive partitions (split launches only, not the single launch).
    static constexpr int PPW = W / WP;
    static_assert(W % WP == 0 && (PPW == 1 || !FUSED), "waves per partition");
    static constexpr int NT = T / 16;     // 16-token QK tiles per step
    static constexpr int NJ = T / 4;      // tokens per lane in the PV product
    static constexpr int NKC = D / 32;    // QK k-chunks of 32 dims
    static constexpr int NDH = D / 128;   // 128-dim halves of a V row
    static constexpr int NPT = D / 16;    // PV output tiles (16 dims each)
    static constexpr int CHP = 64;        // page ids per chunk (one per lane)
    static constexpr int CH = CHP * BS;   // tokens per chunk
    // fp16 weights are computed as 2^15 * 2^(x - m): the largest is 2^15, so
    // the residual of each weight's fp16 rounding stays a normal fp16 number
    // (pack_half2_split).  The exp-sums carry the same factor (a power of
    // two: exact), the normalised outputs cancel it, and the stored
    // partials' exp-sums are divided by it.
    static constexpr float kPScale = DT == 0 ? 32768.f : 1.f;
    static constexpr float kInvPScale = 1.f / kPScale;

    struct State {
        floatx4 acc[NPT];
        float m, l;
    };

    // A split partial (16 bytes of tmp_out).  With a.write_through, and
    // always in the single-launch form, it is stored at device scope (`sc1`),
    // i.e. written through this XCD's L2.
    // Measured on MI355X: in longest-first launches of several rounds,
    // partials kept dirty in L2 until the kernel ends cost about 3% of the
    // launch (32 sequences of 4k-16k tokens, (24, 4, 256): 222.8 -> 215.5 us
    // at P = 512, 230.0 -> 223.4 us at P = 256; the reduce that reads them
    // is unchanged); single-round and grid-order launches gained nothing
    // and keep plain stores.  Nontemporal stores did not help.  The merge
    // that reads partials runs in a later launch, or after the single-launch
    // form's own device-scope release.
    static __device__ __forceinline__ void store_partial(const DecodeArgs& a, float* p,
                                                         const float4& v) {
        if (FUSED || a.write_through) {
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v x = {v.x, v.y, v.z, v.w};
            asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(x) : "memory");
        } else {
            *reinterpret_cast<float4*>(p) = v;
        }
    }
    // A partial's max or exp-sum, under the same rule.
    static __device__ __forceinline__ void store_partial1(const DecodeArgs& a, float* p, float v) {
        if (FUSED || a.write_through)
            asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
        else
            *p = v;
    }

    // Page id of token `tok` (0..31 within the step) from the step's ids.
    static __device__ __forceinline__ int page_of(int tok, const int (&pid)[T / BS < 1 ? 1 : T / BS]) {
        if constexpr (BS >= T) {
            return pid[0];
        } else {
            int p = pid[0];
#pragma unroll
            for (int k = 1; k < T / BS; ++k) p = (tok >= k * BS) ? pid[k] : p;
            return p;
        }
    }

    // K/V registers of one step.
    static constexpr int KQ = DT == 2 ? D / 16 : NKC;   // uint4 of K per token tile, and of Q
    static constexpr int NVQ = DT == 2 ? D / 64 : 1;    // fp32: uint4 of V per token per lane
    using QReg = uint4[KQ];

    // Dim of accumulator tile t, row rr, for lane group c.
    static __device__ __forceinline__ int acc_dim(int t, int c, int rr) {
        if constexpr (DT == 2)
            return 64 * (t / 4) + 16 * c + 4 * rr + t % 4;
        else
            return 128 * (t / 8) + 8 * (4 * c + rr) + t % 8;
    }

    struct Buf {
        uint4 kr[NT][KQ];
        uint4 vr[NDH][NJ];
        uint4 vq[4][NVQ];   // fp32: V[4c + r][64 t' + 4 i, +4)
    };

    // Page ids of the step at chunk offset `off`, read from the chunk's page
    // list (lane k = page k) with readlane: wave-uniform, no memory access.
    struct StepPages {
        int pid[T / BS < 1 ? 1 : T / BS];
        int off_slot;   // step start within its page (BS > T only)
    };
    static __device__ __forceinline__ StepPages step_pages(int pg, int off) {
        StepPages sp;
        const int k0 = off / BS;
#pragma unroll
        for (int k = 0; k < (T / BS < 1 ? 1 : T / BS); ++k)
            sp.pid[k] = __builtin_amdgcn_readlane(pg, k0 + k);
        sp.off_slot = off % BS;
        return sp;
    }

    // Issue the K loads of a step (`remain` valid tokens when not FULL).
    template <bool FULL>
    static __device__ __forceinline__ void issue_k(const DecodeArgs& a, Buf& b, const StepPages& sp,
                                                   int g, int remain, int i, int c) {
        const int64_t page_stride = (int64_t)a.num_kv_heads * BS * D;   // elements
        if constexpr (DT == 2) {
            const float* kbase = reinterpret_cast<const float*>(a.k) + (int64_t)g * BS * D;
            const int tok = i;
            const bool ok = FULL || tok < remain;
            const uint4* kp = reinterpret_cast<const uint4*>(
                kbase + (int64_t)page_of(tok, sp.pid) * page_stride +
                (int64_t)((sp.off_slot + tok) % BS) * D);
#pragma unroll
            for (int u = 0; u < KQ; ++u)
                b.kr[0][u] = ok ? load_stream(kp + c * KQ + u) : make_uint4(0, 0, 0, 0);
            return;
        }
        const uint16_t* kbase = a.k + (int64_t)g * BS * D;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int tok = 16 * tt + i;
            const bool ok = FULL || tok < remain;
            const uint4* kp = reinterpret_cast<const uint4*>(
                kbase + (int64_t)page_of(tok, sp.pid) * page_stride +
                (int64_t)((sp.off_slot + tok) % BS) * D);
#pragma unroll
            for (int kk = 0; kk < NKC; ++kk)
                b.kr[tt][kk] = ok ? load_stream(kp + 4 * kk + c) : make_uint4(0, 0, 0, 0);
        }
    }

    // Issue the V loads of a step: this lane's NJ tokens, dims [128 dh + 8 i, +8).
    template <bool FULL>
    static __device__ __forceinline__ void issue_v(const DecodeArgs& a, Buf& b, const StepPages& sp,
                                                   int g, int remain, int i, int c) {
        const int64_t page_stride = (int64_t)a.num_kv_heads * BS * D;   // elements
        if constexpr (DT == 2) {
            const float* vbase = reinterpret_cast<const float*>(a.v) + (int64_t)g * BS * D;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 4 * c + r;
                const bool ok = FULL || tok < remain;
                const uint4* vp = reinterpret_cast<const uint4*>(
                    vbase + (int64_t)page_of(tok, sp.pid) * page_stride +
                    (int64_t)((sp.off_slot + tok) % BS) * D);
#pragma unroll
                for (int t = 0; t < NVQ; ++t)
                    b.vq[r][t] = ok ? load_stream(vp + 16 * t + i) : make_uint4(0, 0, 0, 0);
            }
            return;
        }
        const uint16_t* vbase = a.v + (int64_t)g * BS * D;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int tok = (j < 4) ? 4 * c + j : 16 + 4 * c + (j - 4);
            const bool ok = FULL || tok < remain;
            const uint4* vp = reinterpret_cast<const uint4*>(
                vbase + (int64_t)page_of(tok, sp.pid) * page_stride +
                (int64_t)((sp.off_slot + tok) % BS) * D);
#pragma unroll
            for (int dh = 0; dh < NDH; ++dh)
                b.vr[dh][j] = ok ? load_stream(vp + 16 * dh + i) : make_uint4(0, 0, 0, 0);
        }
    }

    template <bool FULL>
    static __device__ __forceinline__ void issue(const DecodeArgs& a, Buf& b, int pg, int g,
                                                 int off, int remain, int i, int c) {
        const StepPages sp = step_pages(pg, off);
        issue_k<FULL>(a, b, sp, g, remain, i, c);
        issue_v<FULL>(a, b, sp, g, remain, i, c);
    }

    // QK and the online-softmax update of one step; returns the fp16 weights
    // packed as the PV B operand (x, y used for 16-token steps).
    template <bool FULL>
    static __device__ __forceinline__ uint4 qk_softmax(const DecodeArgs& a, State& st, const Buf& b,
                                                       const QReg& qb, int remain, int c) {
        const auto& kr = b.kr;
        // ---- S = K Q^T on the matrix cores ----
        floatx4 sc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            sc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if constexpr (DT == 2) {
#pragma unroll
                for (int u = 0; u < KQ; ++u) {
                    sc[tt] = mfma4_f32(kr[tt][u].x, qb[u].x, sc[tt]);
                    sc[tt] = mfma4_f32(kr[tt][u].y, qb[u].y, sc[tt]);
                    sc[tt] = mfma4_f32(kr[tt][u].z, qb[u].z, sc[tt]);
                    sc[tt] = mfma4_f32(kr[tt][u].w, qb[u].w, sc[tt]);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NKC; ++kk) sc[tt] = qk_mma(kr[tt][kk], qb[kk], sc[tt]);
            }
        }

        // ---- online softmax (log2 units) for head i, tokens of this lane ----
        float x[NJ];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = mul_rounded(sc[tt][r], a.scale_log2e);
                if (!FULL && (16 * tt + 4 * c + r) >= remain) v = -INFINITY;
                x[4 * tt + r] = v;
            }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < NJ; ++j) mx = fmaxf(mx, x[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(st.m, mx);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2_fast(st.m - mref);
        float p[NJ];
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            p[j] = exp2_fast(x[j] - mref) * kPScale;
            ps += p[j];
        }
        st.l = st.l * alpha + ps;
        st.m = mnew;
#pragma unroll
        for (int t = 0; t < NPT; ++t) st.acc[t] *= alpha;
        return pack_weights(p[0], p[1], p[2], p[3]);
    }

    // S = K Q^T product of one 32-dim chunk in the element type.
    static __device__ __forceinline__ floatx4 qk_mma(const uint4& a, const uint4& b, const floatx4& c) {
        if constexpr (DT == 1)
            return mfma32_bf16(a, b, c);
        else
            return mfma32(a, b, c);
    }

    // Four weights of a 16-token step as the PV B operand: for 16-bit types
    // the rounded pairs in .x/.y and their residuals in .z/.w.
    static __device__ __forceinline__ uint4 pack_weights(float p0, float p1, float p2, float p3) {
        uint4 pb;
        if constexpr (DT == 2) {   // fp32 weights as they are
            pb = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                            __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
        } else if constexpr (DT == 1) {
            pack_bf16_split(p0, p1, pb.x, pb.z);
            pack_bf16_split(p2, p3, pb.y, pb.w);
        } else {
            pack_half2_split(p0, p1, pb.x, pb.z);
            pack_half2_split(p2, p3, pb.y, pb.w);
        }
        return pb;
    }

    // One 16-dim PV output tile of a 16-token step (dims e of the lane
    // group's 4 tokens): the rounded weights' product, then the residuals'.
    template <int E>
    static __device__ __forceinline__ void pv16(floatx4& acc, const uint4 (&v)[4], const uint4& pb) {
        const uint2 a = vt_operand4<E>(v);
        if constexpr (DT == 1) {
            acc = mfma16_bf16(a, make_uint2(pb.x, pb.y), acc);
            acc = mfma16_bf16(a, make_uint2(pb.z, pb.w), acc);
        } else {
            acc = mfma16(a, make_uint2(pb.x, pb.y), acc);
            acc = mfma16(a, make_uint2(pb.z, pb.w), acc);
        }
    }

    // ---- O^T += V^T P^T on the matrix cores ----
    static __device__ __forceinline__ void pv(State& st, const Buf& b, const uint4& pb) {
        if constexpr (DT == 2) {
            const uint32_t pw[4] = {pb.x, pb.y, pb.z, pb.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < NVQ; ++t) {
                    st.acc[4 * t + 0] = mfma4_f32(b.vq[r][t].x, pw[r], st.acc[4 * t + 0]);
                    st.acc[4 * t + 1] = mfma4_f32(b.vq[r][t].y, pw[r], st.acc[4 * t + 1]);
                    st.acc[4 * t + 2] = mfma4_f32(b.vq[r][t].z, pw[r], st.acc[4 * t + 2]);
                    st.acc[4 * t + 3] = mfma4_f32(b.vq[r][t].w, pw[r], st.acc[4 * t + 3]);
                }
            return;
        }
        const auto& vr = b.vr;
#pragma unroll
        for (int dh = 0; dh < NDH; ++dh) {
            pv16<0>(st.acc[dh * 8 + 0], vr[dh], pb);
            pv16<1>(st.acc[dh * 8 + 1], vr[dh], pb);
            pv16<2>(st.acc[dh * 8 + 2], vr[dh], pb);
            pv16<3>(st.acc[dh * 8 + 3], vr[dh], pb);
            pv16<4>(st.acc[dh * 8 + 4], vr[dh], pb);
            pv16<5>(st.acc[dh * 8 + 5], vr[dh], pb);
            pv16<6>(st.acc[dh * 8 + 6], vr[dh], pb);
            pv16<7>(st.acc[dh * 8 + 7], vr[dh], pb);
        }
    }

    template <bool FULL>
    static __device__ __forceinline__ void compute(const DecodeArgs& a, State& st, const Buf& b,
                                                   const QReg& qb, int remain, int c) {
        const uint4 pb = qk_softmax<FULL>(a, st, b, qb, remain, c);
        pv(st, b, pb);
    }

    // ---- Loads of the next step straight into LDS (16-bit types) ----
    // While a wave computes a step, the next step's K/V are already on their
    // way: global_load_lds_dwordx4 puts lane l's 16 bytes at base + 16 l of a
    // per-wave LDS slot (one slot per 16-byte register of a Buf), so no
    // registers hold them in flight; the step then reads its Buf back with
    // ds_read_b128.  Lanes past the valid tokens load a clamped (valid) row
    // and are zeroed on the way back.
    //
    // K is loaded in whole 128-byte lines: the operand of QK chunk kk (row i,
    // 16-byte piece 4 kk + c for lane (i, c)) touches 16 rows at 64 bytes
    // each, half a line per row, so loading it as it is used costs two
    // requests per line.  Instead, chunks 2m and 2m + 1 (line m of every row)
    // come in as two loads of 8 full rows: slot 2m + hf holds rows 8 hf..8 hf+7,
    // lane l taking row 8 hf + l / 8 and piece (l % 8) ^ f(l / 8) of the line,
    // with f(r) = r for hf = 0 and r ^ 1 for hf = 1.  The read-back of chunk
    // kk by lane (i, c) then finds piece 4 (kk % 2) + c of row i at position
    // 8 (i % 8) + (piece ^ f(i % 8)) of slot 2 (kk / 2) + i / 8; the swizzle
    // puts the 16 lanes of one read (rows 0..15, same piece) on 16 distinct
    // 16-byte bank groups.  Registers end up holding exactly the operands of
    // the direct loads.
    //
    // fp32 rows are 4D bytes (one or two rows per 1 KiB slot): K and V land
    // in whole rows, K rows in slots 0 .. F_KSL - 1, V rows after them.  Lane
    // l of a slot load takes row r = slot * F_RPS + l / F_LPR and piece
    // (l % F_LPR) ^ (r % 16) of it, so piece p of row r sits at position
    // (r % F_RPS) * F_LPR + (p ^ (r % 16)) of slot r / F_RPS: the 16 lanes of
    // each read-back (16 rows at one piece for K, 16 pieces of one row for V)
    // fall on 16 distinct 16-byte bank groups.
    static constexpr bool PF = VK_MFMA_LDS_PF && T == 16;
    static constexpr int F_RPS = DT == 2 ? 1024 / (4 * D) : 1;   // fp32: rows per slot
    static constexpr int F_LPR = 64 / F_RPS;                     // fp32: 16-byte pieces per row
    static constexpr int F_KSL = 16 / F_RPS;                     // fp32: slots of the K rows
    static constexpr int SLOTS = DT == 2 ? 2 * F_KSL : NT * NKC + NDH * NJ;   // 1 KiB slots per wave
    static constexpr int WAVE_LDS = PF ? SLOTS * 64 * 16 : 0;   // bytes per wave
    typedef __attribute__((address_space(3))) void* lds_ptr_t;

    template <bool FULL>
    static __device__ __forceinline__ void issue_lds(const DecodeArgs& a, char* lds,
                                                     const StepPages& sp, int g, int remain, int i,
                                                     int c) {
        const int64_t page_stride = (int64_t)a.num_kv_heads * BS * D;   // elements
        if constexpr (DT == 2) {
            static_assert(F_RPS * 4 * D == 1024 && F_LPR * 4 == D, "fp32 rows fill the slots");
            const float* kbase = reinterpret_cast<const float*>(a.k) + (int64_t)g * BS * D;
            const float* vbase = reinterpret_cast<const float*>(a.v) + (int64_t)g * BS * D;
            const int l = i + 16 * c;
#pragma unroll
            for (int sl = 0; sl < F_KSL; ++sl) {
                const int row = sl * F_RPS + l / F_LPR;
                const int tok = FULL ? row : min(row, remain - 1);
                const int64_t off = (int64_t)page_of(tok, sp.pid) * page_stride +
                                    (int64_t)((sp.off_slot + tok) % BS) * D;
                const int piece = (l % F_LPR) ^ (row & 15);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(kbase + off) + piece,
                                                 (lds_ptr_t)(lds + sl * 1024), 16, 0, 2);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(vbase + off) + piece,
                                                 (lds_ptr_t)(lds + (F_KSL + sl) * 1024), 16, 0, 2);
            }
            return;
        }
        const uint16_t* kbase = a.k + (int64_t)g * BS * D;
        const uint16_t* vbase = a.v + (int64_t)g * BS * D;
        static_assert(NT == 1 && NKC % 2 == 0, "LDS prefetch: 16-token steps, whole K lines");
        {
            const int l = i + 16 * c, r0 = l >> 3;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = r0 + 8 * hf;
                const int tok = FULL ? row : min(row, remain - 1);
                const uint4* kp = reinterpret_cast<const uint4*>(
                    kbase + (int64_t)page_of(tok, sp.pid) * page_stride +
                    (int64_t)((sp.off_slot + tok) % BS) * D);
                const int piece = (l & 7) ^ (hf ? (r0 ^ 1) : r0);
#pragma unroll
                for (int m = 0; m < NKC / 2; ++m)
                    __builtin_amdgcn_global_load_lds(kp + 8 * m + piece,
                                                     (lds_ptr_t)(lds + (2 * m + hf) * 1024), 16, 0, 2);
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int t0 = (j < 4) ? 4 * c + j : 16 + 4 * c + (j - 4);
            const int tok = FULL ? t0 : min(t0, remain - 1);
            const uint4* vp = reinterpret_cast<const uint4*>(
                vbase + (int64_t)page_of(tok, sp.pid) * page_stride +
                (int64_t)((sp.off_slot + tok) % BS) * D);
#pragma unroll
            for (int dh = 0; dh < NDH; ++dh)
                __builtin_amdgcn_global_load_lds(vp + 16 * dh + i,
                                                 (lds_ptr_t)(lds + (NT * NKC + dh * NJ + j) * 1024),
                                                 16, 0, 2);
        }
    }

    template <bool FULL>
    static __device__ __forceinline__ void read_lds(Buf& b, const char* lds, int remain, int lane,
                                                    int i, int c) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        if constexpr (DT == 2) {
            // K: row i, pieces c KQ + u (dims [c D/4 + 4u, +4)).
#pragma unroll
            for (int u = 0; u < KQ; ++u) {
                const int pos = (i % F_RPS) * F_LPR + ((c * KQ + u) ^ (i & 15));
                const uint4 v = *reinterpret_cast<const uint4*>(lds + (i / F_RPS) * 1024 + 16 * pos);
                b.kr[0][u] = (FULL || i < remain) ? v : z;
            }
            // V: row 4c + r, pieces 16 t + i (dims [64 t + 4 i, +4)).
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < NVQ; ++t) {
                    const int row = 4 * c + r;
                    const int pos = (row % F_RPS) * F_LPR + ((16 * t + i) ^ (row & 15));
                    const uint4 v = *reinterpret_cast<const uint4*>(
                        lds + (F_KSL + row / F_RPS) * 1024 + 16 * pos);
                    b.vq[r][t] = (FULL || row < remain) ? v : z;
                }
            return;
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int kk = 0; kk < NKC; ++kk) {
                const int r = i & 7, hf = i >> 3;
                const int pos = 8 * r + ((4 * (kk & 1) + c) ^ (hf ? (r ^ 1) : r));
                const uint4 v = *reinterpret_cast<const uint4*>(lds + ((kk >> 1) * 2 + hf) * 1024 + 16 * pos);
                b.kr[tt][kk] = (FULL || 16 * tt + i < remain) ? v : z;
            }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int dh = 0; dh < NDH; ++dh) {
                const int tok = (j < 4) ? 4 * c + j : 16 + 4 * c + (j - 4);
                const uint4 v = *reinterpret_cast<const uint4*>(lds + (NT * NKC + dh * NJ + j) * 1024 + 16 * lane);
                b.vr[dh][j] = (FULL || tok < remain) ? v : z;
            }
    }

    // The compiler tracks neither order below (the loads into LDS go through
    // M0, not through a pointer it follows), so both waits are explicit and
    // are also compiler barriers:
    //  * the step's loads into LDS have landed before it is read back;
    //  * the read-back is done before the slot is loaded again.
    static __device__ __forceinline__ void wait_lds_loads() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    static __device__ __forceinline__ void wait_lds_reads() {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    static __device__ __forceinline__ void scan(const DecodeArgs& a, State& st, const QReg& qb,
                                                int t_begin, int t_end, int g, int s, int wsub,
                                                int lane, int i, int c, int pg_first, bool& bad,
                                                char* lds) {
        const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
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
            // Full steps of this wave, then at most one partial step.
            const int first = c0 + wsub * T;
            constexpr int stride = WP * T;
            const int nfull = (first + T <= c1) ? (c1 - T - first) / stride + 1 : 0;
            const int tl = first + nfull * stride;
            if constexpr (PF) {
                // step k + 1 is in flight to LDS while step k computes
                if (nfull > 0)
                    issue_lds<true>(a, lds, step_pages(pg, first - c0), g, T, i, c);
                else if (tl < c1)
                    issue_lds<false>(a, lds, step_pages(pg, tl - c0), g, c1 - tl, i, c);
                for (int k = 0; k < nfull; ++k) {
                    Buf b;
                    wait_lds_loads();
                    read_lds<true>(b, lds, T, lane, i, c);
                    wait_lds_reads();
                    if (k + 1 < nfull)
                        issue_lds<true>(a, lds, step_pages(pg, first + (k + 1) * stride - c0), g, T, i, c);
                    else if (tl < c1)
                        issue_lds<false>(a, lds, step_pages(pg, tl - c0), g, c1 - tl, i, c);
                    compute<true>(a, st, b, qb, T, c);
                }
                if (tl < c1) {
                    Buf bl;
                    wait_lds_loads();
                    read_lds<false>(bl, lds, c1 - tl, lane, i, c);
                    wait_lds_reads();
                    compute<false>(a, st, bl, qb, c1 - tl, c);
                }
            } else {
                for (int k = 0; k < nfull; ++k) {
                    Buf b;
                    issue<true>(a, b, pg, g, first + k * stride - c0, T, i, c);
                    compute<true>(a, st, b, qb, T, c);
                }
                if (tl < c1) {
                    Buf bl;
                    issue<false>(a, bl, pg, g, tl - c0, c1 - tl, i, c);
                    compute<false>(a, st, bl, qb, c1 - tl, c);
                }
            }
        }
    }

    // Workgroup `unit` of (KV head g, sequence s): partitions
    // [unit * PPW, unit * PPW + PPW), WP waves each.
    static __device__ void item(const DecodeArgs& a, const int unit, const int g, const int s) {
        // The per-wave prefetch slots and the end-of-partition merge area
        // are never live together: one allocation holds both.
        constexpr int MERGE_BYTES = (W > 1 ? W * G * D : 1) * 4;
        constexpr int RAW_BYTES = W * WAVE_LDS > MERGE_BYTES ? W * WAVE_LDS : MERGE_BYTES;
        __shared__ __attribute__((aligned(16))) char s_raw[RAW_BYTES];
        auto& s_acc = *reinterpret_cast<float (*)[W > 1 ? W : 1][W > 1 ? G : 1][W > 1 ? D : 1]>(s_raw);
        __shared__ float s_m[W][G];
        __shared__ float s_l[W][G];
        __shared__ int s_bad[W];

        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
        const int i = lane & 15, c = lane >> 4;
        const int wsub = wave % WP;                     // this wave's index within its partition
        const int part = unit * PPW + wave / WP;        // this wave's partition
        const int Hq = a.num_q_heads;
        const int P = a.partition_size, NP = a.max_num_partitions;

        // Issue the independent loads together: the sequence length, the
        // first chunk's page ids (its start does not depend on the length;
        // the index is clamped into the table row and the ids are used only
        // below ceil(L/bs)) and the query.  The first K/V loads then wait for
        // one round trip, not for the length and then the table.
        const int t_first = P > 0 ? part * P : 0;
        const int32_t pg_first =
            a.block_tables[(int64_t)s * a.max_blocks_per_seq +
                           min(t_first / BS + lane, a.max_blocks_per_seq - 1)];
        // Q^T operand: head i of the group, dims [32 kk + 8 c, +8) (fp32:
        // [c D/4, +D/4)); zero for i >= G.
        QReg qb;
        {
            const int64_t qrow = ((int64_t)s * Hq + g * G + (i < G ? i : 0)) * D;
            if constexpr (DT == 2) {
                const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.q) + qrow);
#pragma unroll
                for (int u = 0; u < KQ; ++u) qb[u] = (i < G) ? qp[c * KQ + u] : make_uint4(0, 0, 0, 0);
            } else {
                const uint4* qp = reinterpret_cast<const uint4*>(a.q + qrow);
#pragma unroll
                for (int kk = 0; kk < NKC; ++kk) qb[kk] = (i < G) ? qp[4 * kk + c] : make_uint4(0, 0, 0, 0);
            }
        }
        int L = a.seq_lens[s];
        bool poison = false;
        const int cap = a.max_blocks_per_seq * BS;
        if (L > cap) {
            L = cap;
            poison = true;
        }
        int t_begin = 0, t_end = L;
        int nparts = 1;   // partitions of this sequence that write a result
        if (P > 0) {
            t_begin = part * P;
            t_end = min(L, t_begin + P);
            if (part == NP - 1 && L > t_begin + P) poison = true;  // beyond the grid
            if (part >= NP) t_end = t_begin;   // a workgroup's spare partition slot
            nparts = L > 0 ? (int)min(((int64_t)L + P - 1) / P, (int64_t)NP) : 0;
        }
        const bool active = t_end > t_begin;
        if constexpr (PPW == 1) {
            if (!active) {
                if (P == 0 || (FUSED && part == 0)) {  // empty sequence: zeros
                    float* o = a.out + ((int64_t)s * Hq + g * G) * D;
                    for (int k = tid; k < G * D; k += 64 * W) o[k] = 0.f;
                }
                return;  // split: partitions past the end write nothing
            }
        }
        // Unsplit, or fused with a single partition: the normalised result
        // goes straight to `out`.
        const bool direct = (P == 0) || (FUSED && nparts == 1);

        State st;
#pragma unroll
        for (int t = 0; t < NPT; ++t) st.acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.f;
        bool bad = false;

        // (With PPW > 1 the waves of an empty partition skip the scan but
        // still meet the others at the barrier below.)
        if (PPW == 1 || active)
            scan(a, st, qb, t_begin, t_end, g, s, wsub, lane, i, c, pg_first, bad,
                 s_raw + wave * WAVE_LDS);

        // Sum the per-lane exp-sums over the 4 lane groups (same head, same m).
        float lsum = st.l + __shfl_xor(st.l, 16);
        lsum += __shfl_xor(lsum, 32);
        const bool wave_bad = __ballot(bad) != 0;

        const int64_t row0 = (int64_t)s * Hq + g * G;   // first query head of the group
        if constexpr (W == 1 && PF) {
            // The accumulator layout scatters a head's dims over the lanes
            // (64 four-byte stores per wave, each touching 24 lines); the
            // normalised rows go through this wave's (now idle) prefetch
            // slots instead and leave as one 16-byte store per lane and row.
            static_assert(G * D * 4 <= WAVE_LDS, "staging fits the prefetch slots");
            const bool out_bad = poison || wave_bad;
            float* stage = reinterpret_cast<float*>(s_raw);
            if (i < G) {
#pragma unroll
                for (int t = 0; t < NPT; ++t)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        stage[i * D + acc_dim(t, c, rr)] = st.acc[t][rr] / lsum;
            }
            __syncthreads();
            const float nanv = __builtin_nanf("");
            for (int e = lane; e < G * D / 4; e += 64) {
                const int h = e / (D / 4), d = 4 * (e % (D / 4));
                const int64_t r = row0 + h;
                float4 o = *reinterpret_cast<const float4*>(stage + 4 * e);
                if (out_bad) o = make_float4(nanv, nanv, nanv, nanv);
                if (direct)
                    *reinterpret_cast<float4*>(a.out + r * D + d) = o;
                else
                    store_partial(a, a.tmp_out + (r * NP + part) * D + d, o);
            }
            if (!direct && i < G && c == 0) {
                const int64_t pr = (row0 + i) * NP + part;
                store_partial1(a, a.max_logits + pr, st.m);
                store_partial1(a, a.exp_sums + pr, out_bad ? nanv : lsum * kInvPScale);
            }
        } else if constexpr (W == 1) {
            // (fp32, or built without the LDS prefetch.)  Plain stores: the
            // single launch's release needs every partial at device scope.
            static_assert(!FUSED, "the single launch stages its partials through the prefetch slots");
            const bool out_bad = poison || wave_bad;
            if (i < G) {
                const int64_t r = row0 + i;
                float* dst;
                if (direct) {
                    dst = a.out + r * D;
                } else {
                    const int64_t pr = r * NP + part;
                    dst = a.tmp_out + pr * D;
                    if (c == 0) {
                        store_partial1(a, a.max_logits + pr, st.m);
                        store_partial1(a, a.exp_sums + pr, out_bad ? __builtin_nanf("") : lsum * kInvPScale);
                    }
                }
#pragma unroll
                for (int t = 0; t < NPT; ++t)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        dst[acc_dim(t, c, rr)] = out_bad ? __builtin_nanf("") : st.acc[t][rr] / lsum;
            }
        } else {
            // the merge area overlaps other waves' prefetch slots: all scans first
            if constexpr (PF) __syncthreads();
            if (i < G) {
#pragma unroll
                for (int t = 0; t < NPT; ++t)
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        s_acc[wave][i][acc_dim(t, c, rr)] = st.acc[t][rr];
                if (c == 0) {
                    s_m[wave][i] = st.m;
                    s_l[wave][i] = lsum;
                }
            }
            if (lane == 0) s_bad[wave] = wave_bad || poison;
            __syncthreads();
            // Four dims per thread, one 16-byte store each.
            const float nanv = __builtin_nanf("");
            for (int idx = 4 * tid; idx < PPW * G * D; idx += 4 * 64 * W) {
                const int b = idx / (G * D), h = (idx / D) % G, d = idx % D;
                const int pb = unit * PPW + b;        // partition of wave group b
                if constexpr (PPW > 1) {
                    if (pb >= NP || pb * P >= L) continue;   // empty slot: nothing written
                }
                const int w0 = b * WP;
                bool out_bad = false;
#pragma unroll
                for (int w = 0; w < WP; ++w) out_bad = out_bad || s_bad[w0 + w];
                float M = s_m[w0][h];
#pragma unroll
                for (int w = 1; w < WP; ++w) M = fmaxf(M, s_m[w0 + w][h]);
                float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
                float den = 0.f;
#pragma unroll
                for (int w = 0; w < WP; ++w) {
                    const float mw = s_m[w0 + w][h];
                    const float sc = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
                    const float4 x = *reinterpret_cast<const float4*>(&s_acc[w0 + w][h][d]);
                    num.x += sc * x.x;
                    num.y += sc * x.y;
                    num.z += sc * x.z;
                    num.w += sc * x.w;
                    den += sc * s_l[w0 + w][h];
                }
                const float4 o = out_bad ? make_float4(nanv, nanv, nanv, nanv)
                                         : make_float4(num.x / den, num.y / den, num.z / den,
                                                       num.w / den);
                const int64_t r = row0 + h;
                if (direct) {
                    *reinterpret_cast<float4*>(a.out + r * D + d) = o;
                } else {
                    const int64_t pr = r * NP + pb;
                    store_partial(a, a.tmp_out + pr * D + d, o);
                    if (d == 0) {
                        store_partial1(a, a.max_logits + pr, M);
                        store_partial1(a, a.exp_sums + pr, out_bad ? nanv : den * kInvPScale);
                    }
                }
            }
        }
        if constexpr (FUSED) {
            if (!direct) merge_if_last(a, g, s, nparts, row0, tid);
        }
    }

    // Single-launch split-KV: the workgroup that writes the last of the
    // sequence's `n` partials for KV head g merges all of them into `out`
    // with the reduce kernel's merge (merge_ops.h), one wave per 32 dims of a
    // head.  Arrival is counted in counters[s * Hkv + g] with a device-scope
    // atomic increment that wraps to zero at n - 1: the last arrival sees
    // n - 1 and leaves the counter at zero for the next call.
    // Ordering across XCDs (each has its own L2): the partials were stored
    // at device scope (written through L2), so once every wave has waited
    // for its stores to be acknowledged they are visible to every XCD; the
    // barrier gathers the workgroup and one lane increments.  No L2
    // write-back per workgroup (that release, measured: 2-3x the launch time
    // at thousands of workgroups).  The last arrival acquires (L2
    // invalidate: its XCD may hold stale lines of these buffers from an
    // earlier call) before the barrier that lets its waves read the other
    // partials: one acquire per (sequence, KV head).
    static __device__ void merge_if_last(const DecodeArgs& a, int g, int s, int n, int64_t row0,
                                         int tid) {
        __shared__ int s_last;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const unsigned old = atomicInc(a.counters + (int64_t)s * a.num_kv_heads + g, (unsigned)(n - 1));
            const bool last = old == (unsigned)(n - 1);
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_last = last;
        }
        __syncthreads();
        if (!s_last) return;
        const int NP = a.max_num_partitions;
        const int wave = tid >> 6, lane = tid & 63;
        constexpr int kChunks = D / merge::kDims;
        if (n <= merge::kGroups) {
            // Few partitions: NB pieces per wave with all their loads in flight.
            constexpr int NB = 4;
            for (int it0 = wave * NB; it0 < G * kChunks; it0 += W * NB) {
                const float* ml[NB];
                const float* es[NB];
                const float4* to[NB];
                float4* dst[NB];
                bool ok[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int it = min(it0 + b, G * kChunks - 1);
                    ok[b] = it0 + b < G * kChunks;
                    const int h = it / kChunks, chunk = it % kChunks;
                    const int64_t r = row0 + h;
                    ml[b] = a.max_logits + r * NP;
                    es[b] = a.exp_sums + r * NP;
                    to[b] = reinterpret_cast<const float4*>(a.tmp_out + r * NP * D + chunk * merge::kDims);
                    dst[b] = reinterpret_cast<float4*>(a.out + r * D + chunk * merge::kDims);
                }
                merge::merge_columns_few<NB>(ml, es, to, ok, D / 4, n, lane, dst);
            }
            return;
        }
        for (int it = wave; it < G * kChunks; it += W) {
            const int h = it / kChunks, chunk = it % kChunks;
            const int64_t r = row0 + h;
            merge::merge_columns(a.max_logits + r * NP, a.exp_sums + r * NP,
                                 reinterpret_cast<const float4*>(a.tmp_out + r * NP * D + chunk * merge::kDims),
                                 D / 4, n, lane,
                                 reinterpret_cast<float4*>(a.out + r * D + chunk * merge::kDims));
        }
    }

    // Work order of a split launch over at most 64 sequences, used when the
    // grid takes several rounds of the resident wave slots.  Workgroups
    // start in linear-id order as slots free up, so the order of the items
    // decides the tail: every full partition first, then the ragged last
    // partitions by decreasing length (longest-first list scheduling); the
    // ids past the last item (partitions past the end of a sequence) exit
    // after one load.  Every wave derives the same mapping from the sequence
    // lengths (lane j holds sequence j), without LDS or barriers.  Lengths
    // are taken as the kernel guards them (<= 0: none; at most the table
    // capacity and NP * P), so each partition index the guarded item code
    // accepts is covered exactly once.  The single-launch form adds one
    // item per (sequence, KV head) of length <= 0, whose output is zeros.
    static __device__ __forceinline__ bool longest_first(const DecodeArgs& a, int& part, int& g,
                                                         int& s) {
        const int lane = threadIdx.x & 63;
        const int S = a.num_seqs, Hkv = a.num_kv_heads, P = a.partition_size;
        const int64_t k = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
        const int lim = min(a.max_blocks_per_seq * BS, a.max_num_partitions * P);
        const int L = lane < S ? a.seq_lens[lane] : 0;
        const int Le = min(max(L, 0), lim);
        const int PU = P * PPW;     // tokens per workgroup unit
        const int F = Le / PU;      // full units of sequence `lane`
        const int r = Le % PU;      // tokens of its ragged last unit (0: none)
        int pf = F;                 // inclusive prefix sum of F over the lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(pf, off);
            if (lane >= off) pf += t;
        }
        const int64_t nfull = (int64_t)__shfl(pf, 63) * Hkv;
        if (k < nfull) {
            s = __ffsll((unsigned long long)__ballot((int64_t)pf * Hkv > k)) - 1;
            const int Fs = __shfl(F, s);
            const int64_t rem = k - (int64_t)(__shfl(pf, s) - Fs) * Hkv;
            g = (int)(rem / Fs);
            part = (int)(rem % Fs);
            return true;
        }
        const bool ragged = lane < S && r > 0;
        const unsigned long long rmask = __ballot(ragged);
        const int64_t nrag = (int64_t)__popcll(rmask) * Hkv;
        const int64_t q = k - nfull;
        if (q >= nrag) {
            if constexpr (FUSED) {
                const unsigned long long zmask = __ballot(lane < S && Le == 0);
                const int64_t qz = q - nrag;
                if (qz >= (int64_t)__popcll(zmask) * Hkv) return false;
                const int want = (int)(qz / Hkv);
                const int idx = __popcll(zmask & ((1ull << lane) - 1ull));
                s = __ffsll((unsigned long long)__ballot(((zmask >> lane) & 1ull) && idx == want)) - 1;
                g = (int)(qz % Hkv);
                part = 0;
                return true;
            }
            return false;
        }
        // Rank of each ragged partition: longer first, ties by sequence.
        int rank = 0;
        for (int j = 0; j < S; ++j) {
            const int rj = __builtin_amdgcn_readlane(r, j);
            rank += (rj > r) || (rj == r && j < lane);
        }
        s = __ffsll((unsigned long long)__ballot(ragged && rank == (int)(q / Hkv))) - 1;
        g = (int)(q % Hkv);
        part = __shfl(F, s);
        return true;
    }

    static __device__ void run(const DecodeArgs& a) {
#if VK_MFMA_ORDER
        if (a.work_order == 1) {
            int part, g, s;
            if (longest_first(a, part, g, s)) item(a, part, g, s);
            return;
        }
#endif
        item(a, blockIdx.x, blockIdx.y, blockIdx.z);
    }
};

// At least two resident waves per SIMD (a lane gets at most 256 registers),
// except fp32 at D = 256, whose K, V, Q and accumulators take 64 registers
// each: one wave per SIMD, 512 registers.
template <int D, int G, int BS, int W, int WP, bool FUSED, int DT>
__global__ __launch_bounds__(64 * W)
__attribute__((amdgpu_waves_per_eu((DT == 2 && D == 256) ? 1 : VK_MFMA_WAVES_PER_EU)))
void decode_mfma_kernel(DecodeArgs a) {
    MfmaKernel<D, G, BS, W, WP, 16, FUSED, DT>::run(a);
}

template <int D, int G, int W, int WP, bool FUSED, int DT>
hipError_t launch_bs(const DecodeArgs& a, int bs, dim3 grid, hipStream_t st, bool* ok) {
    *ok = true;
    const dim3 block(64 * W);
    switch (bs) {
        case 8: hipLaunchKernelGGL((decode_mfma_kernel<D, G, 8, W, WP, FUSED, DT>), grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL((decode_mfma_kernel<D, G, 16, W, WP, FUSED, DT>), grid, block, 0, st, a); break;
        case 32: hipLaunchKernelGGL((decode_mfma_kernel<D, G, 32, W, WP, FUSED, DT>), grid, block, 0, st, a); break;
        default: *ok = false; return hipSuccess;
    }
    return hipGetLastError();
}

// Geometry sets, one translation unit each: 0 = grouped-query heads
// (G = 4, 6, 8); 1 = multi-head (G = 1) and multi-query (G = 16).
template <int SET, int W, int WP, bool FUSED, int DT>
hipError_t launch_w(const DecodeArgs& a, int group, int head_dim, int bs, dim3 grid,
                    hipStream_t st, bool* ok) {
    if constexpr (SET == 0) {
        if (group == 4 && head_dim == 128) return launch_bs<128, 4, W, WP, FUSED, DT>(a, bs, grid, st, ok);
        if (group == 6 && head_dim == 256) return launch_bs<256, 6, W, WP, FUSED, DT>(a, bs, grid, st, ok);
        if (group == 8 && head_dim == 128) return launch_bs<128, 8, W, WP, FUSED, DT>(a, bs, grid, st, ok);
        if (group == 8 && head_dim == 256) return launch_bs<256, 8, W, WP, FUSED, DT>(a, bs, grid, st, ok);
    } else {
        if (group == 1 && head_dim == 128) return launch_bs<128, 1, W, WP, FUSED, DT>(a, bs, grid, st, ok);
        if (group == 1 && head_dim == 256) return launch_bs<256, 1, W, WP, FUSED, DT>(a, bs, grid, st, ok);
        if (group == 16 && head_dim == 128) return launch_bs<128, 16, W, WP, FUSED, DT>(a, bs, grid, st, ok);
        if (group == 16 && head_dim == 256) return launch_bs<256, 16, W, WP, FUSED, DT>(a, bs, grid, st, ok);
    }
    *ok = false;
    return hipSuccess;
}

// Waves per workgroup (1, 2, 4), partitions per workgroup (1, or 2 with four
// waves, split only) and the single-launch form (fp16 only) for one geometry
// set and element type.
template <int SET, int DT>
hipError_t launch_mfma_set(const DecodeArgs& a, int group, int head_dim, int bs, int waves,
                           int parts_per_wg, dim3 grid, hipStream_t st, bool* ok) {
    *ok = false;
    if (a.counters != nullptr && a.partition_size > 0) {
        if constexpr (DT == 0) {
            if (parts_per_wg != 1) return hipSuccess;
            switch (waves) {
                case 1: return launch_w<SET, 1, 1, true, DT>(a, group, head_dim, bs, grid, st, ok);
                case 2: return launch_w<SET, 2, 2, true, DT>(a, group, head_dim, bs, grid, st, ok);
                case 4: return launch_w<SET, 4, 4, true, DT>(a, group, head_dim, bs, grid, st, ok);
                default: return hipSuccess;
            }
        }
        return hipSuccess;
    }
    if (parts_per_wg == 2) {
        if constexpr (DT == 0) {
            if (waves == 4 && a.partition_size > 0)
                return launch_w<SET, 4, 2, false, DT>(a, group, head_dim, bs, grid, st, ok);
        }
        return hipSuccess;
    }
    if (parts_per_wg != 1) return hipSuccess;
    switch (waves) {
        case 1: return launch_w<SET, 1, 1, false, DT>(a, group, head_dim, bs, grid, st, ok);
        case 2: return launch_w<SET, 2, 2, false, DT>(a, group, head_dim, bs, grid, st, ok);
        case 4: return launch_w<SET, 4, 4, false, DT>(a, group, head_dim, bs, grid, st, ok);
        default: return hipSuccess;
    }
}

}  // namespace
}  // namespace vk
