// Many query tokens per sequence over the paged KV cache, causal: the
// chunked-prefill shape of the variable-length attention (the vllm-metal
// kernels page, cf-1.com/news/5525226, section "什么是 Paged Attention",
// names one paged variable-length kernel for prefill and speculative decode;
// the scores, masking and log2-space softmax are those of the column kernel
// in decode_varlen.hip and of the decode).
//
// The column kernel gives each wave 16 (token, head) columns and streams the
// keys through that wave's own prefetch slots, so every 16 / G query tokens
// re-read the whole context.  Here a workgroup owns 128 consecutive columns
// of one (sequence, KV head) — columns are (token, head) pairs in token-major
// order, so a workgroup covers 128 / G query tokens and, where G does not
// divide 128, runs across token boundaries — and streams the keys through LDS
// in 64-key tiles: each tile is fetched once per workgroup and serves all 128
// columns.  At G = 6, 1024 query tokens are then exactly 48 workgroups (whole
// tokens per workgroup would take 49, the last one partial; on the chunked
// prefill of 4 x 1024 tokens that is 768 workgroups, three full rounds of the
// 256 CUs, instead of 784).
//
//  * Loads: the tile's K and V go straight from the paged cache into LDS
//    (global_load_lds_dwordx4: lane l's 16 bytes land at slot base + 16 l),
//    two buffers, tile t + 1 in flight while tile t is computed (a build
//    option takes 32-key tiles through four buffers, three in flight; at
//    D = 256 either fills 128 KiB).  Measured on MI355X, 64-key tiles: chunked
//    prefill fp16 1046 -> 958 us, bf16 1198 -> 1118 us (half the barriers and
//    per-tile softmax reductions); D = 128 unsplit verification 501 -> 392 us.
//    K: a slot is one matrix-core operand register of the whole wave, so
//    every K read is one conflict-free ds_read_b128 of 1 KiB; K slot
//    (kb, kk): lane (i, c) holds K[16 kb + i][32 kk + 8 c, +8).  V: rows in
//    order, 16-byte chunks permuted per row against bank conflicts, read with
//    the transposing ds_read_b64_tr_b16, which hands each lane four keys of
//    one dim, so V^T needs no register shuffles.
//  * Per wave and tile: S^T = K Q^T for its 16-column blocks (16x16x32
//    products, Q^T held in registers), log2 online softmax per column with
//    the causal limit applied by select on the diagonal tiles only, then
//    O^T += V^T P^T (16x16x32).  The softmax's exponent reference trails the
//    running max by up to 2^8, so the accumulators are rescaled only on the
//    rare tiles that move it.
//  * Waves whose columns see none of a tile's keys skip its arithmetic but
//    still take part in its loads and barriers.
//  * Page ids of a tile go into a per-wave LDS ring NBUF - 1 tiles ahead of
//    its K/V loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_ops.h"
#include "vk_kernels.h"

#ifndef VK_TILE_D256_ONE_BLOCK
#define VK_TILE_D256_ONE_BLOCK 1   // D = 256: eight waves of one column block
#endif
#ifndef VK_TILE_PV_AHEAD
#define VK_TILE_PV_AHEAD 4         // PV: V reads kept this many products ahead (0: compiler's order)
#endif
#ifndef VK_TILE_QK_AHEAD
#define VK_TILE_QK_AHEAD 2         // QK: K reads kept this many 32-dim chunks ahead (0: compiler's order)
#endif
#ifndef VK_TILE_KEYS
#define VK_TILE_KEYS 64            // keys per tile: 64 (two LDS buffers) or 32 (four)
#endif
#ifndef VK_TILE_SPLIT_WEIGHTS
#define VK_TILE_SPLIT_WEIGHTS 0    // fp16 residual PV product: 0 never, 1 on heavy tiles, 2 always
#endif

namespace vk {
namespace {

using namespace mfma;

// 16-column blocks per wave and waves per workgroup (128 columns in all):
// at D = 128 four waves of two blocks (two workgroups per CU, two waves per
// SIMD); at D = 256 eight waves of one block, so that a wave fits in 256
// registers and two share each SIMD (with two blocks a wave needs ~300 and
// runs alone).
constexpr int tile_blocks(int D) { return (D == 256 && VK_TILE_D256_ONE_BLOCK) ? 1 : 2; }
constexpr int tile_waves(int D) { return 8 / tile_blocks(D); }

// DT: element type of q, K and V (0 fp16, 1 bf16).  bf16 runs the same
// steps on the bf16 matrix instructions, with each softmax weight split into
// a bf16 value and its bf16 residual and both taken through PV (as the bf16
// decode does), so the weights keep ~2^-16 relative precision.
template <int D, int G, int BS, int DT>
struct TileKernel {
    static constexpr int CB = tile_blocks(D);    // 16-column blocks per wave
    static constexpr int NW = tile_waves(D);     // waves per workgroup
    static constexpr int NC = NW * CB * 16;      // columns per workgroup (128)
    static constexpr int KT = VK_TILE_KEYS;      // keys per tile
    static constexpr int KB = KT / 16;           // 16-key blocks per tile
    static constexpr int KH = KT / 32;           // 32-key PV steps per tile
    static constexpr int NKC = D / 32;           // QK k-chunks of 32 dims
    static constexpr int NDH = D / 128;          // 128-dim halves of a V row
    static constexpr int NACC = D / 16;          // PV output tiles per column block (dims 16 m + 4 c + rr)
    static constexpr int KSLOTS = KB * NKC;      // [key block][dim chunk]
    static constexpr int VSLOTS = (KT / 4) * NDH;   // V: KT rows of 2D bytes
    static constexpr int SLOTS = KSLOTS + VSLOTS;
    static constexpr int RB = 2 * D;             // bytes of a V row
    static constexpr int RPI = 1024 / RB;        // V rows per slot
    static constexpr int CPR = RB / 16;          // 16-byte chunks of a V row
    static constexpr int BUF = SLOTS * 1024;     // bytes of one tile in LDS
    static constexpr int NPG = KT / BS;          // pages per tile
    // tiles in LDS: with 32 keys 3 in flight while 1 is computed, with 64
    // keys 1 (both 128 KiB at D = 256)
    static constexpr int NBUF = KT == 32 ? 4 : 2;
    static constexpr int ISSUE = SLOTS / NW;     // loads into LDS per wave and tile
    static_assert(KSLOTS % NW == 0 && VSLOTS % NW == 0, "slots split evenly over the waves");
    static_assert(RPI <= BS, "the rows of a V slot sit in one page");
    static_assert(BS <= KT && KT % BS == 0, "a tile covers whole pages");
    static_assert(KT == 32 || KT == 64, "tile of 32 or 64 keys");
    typedef __attribute__((address_space(3))) void* lds_ptr_t;

    // Per column: m is the running max score (log2 units); the weights are
    // exp2(score - r) against a reference r that trails m by at most kTau, and
    // l sums them.  r moves (and acc, l are rescaled) only when m outgrows it
    // by more than kTau, so after the first tiles of a row the rescale is
    // skipped; the weights stay <= 2^kTau, well inside fp16.
    static constexpr float kTau = 8.f;
    // fp16 weights.  By default PV takes each weight's fp16 rounding alone
    // and l sums exactly those rounded values, so every output is the convex
    // combination sum_t w'_t v_t / sum_t w'_t of V rows with weights w'_t
    // within 2^-11 relative of the softmax's: the error is at most 2^-11
    // times the largest |v_t - o| of the row, and in practice far less where
    // many keys share the weight (their rounding errors average out; a row
    // dominated by one key is exact).  Measured on MI355X: 2.8e-5 max abs on
    // the chunked-prefill workload, up to 5.6e-4 on rows of mixed test
    // batches that see few keys or a peaked softmax.
    // Two build options take the rounded residual through a second PV
    // product as well (weights 2^7 * 2^(score - r) <= 2^15, so the residual
    // stays a normal fp16 number; l and the stored exp-sum carry the same
    // power of two), which brings the weights to ~2^-22:
    //  * VK_TILE_SPLIT_WEIGHTS 2, on every tile: largest error ~1e-6, chunked
    //    prefill 1528 us against 1270 us (the products are this kernel's
    //    critical path);
    //  * VK_TILE_SPLIT_WEIGHTS 1, only on tiles where some lane's share of
    //    the tile's weights is at least 1/16 of that lane's exp-sum so far (a
    //    row's first tiles, a tile that brings a new dominant key): largest
    //    error 2.9e-5, 1410 us.  The waves of a workgroup meet at a barrier
    //    on every tile, so one wave's extra pass holds all eight.
    static constexpr int kSplitMode = DT == 1 ? 2 : VK_TILE_SPLIT_WEIGHTS;
    static constexpr float kSplitShare = 1.f / 16.f;
    static constexpr float kPScale = (DT == 0 && kSplitMode > 0) ? 128.f : 1.f;
    struct Col {
        floatx4 acc[NACC];
        float m, r, l;
    };

    // Loads into LDS (lane l's 4 or 16 bytes land at lds + 4 l or + 16 l).
    // Issued as inline assembly so that the compiler does not see them: it
    // would otherwise wait for every one of them (vmcnt(0)) before each LDS
    // read, since it cannot tell which buffer they fill; the kernel orders
    // them itself (wait_tile, lds_barrier).  M0 holds the LDS address and is
    // restored afterwards.
    static __device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
    }
    // Scalar base + 32-bit lane offset (bytes): no per-lane address arithmetic.
    static __device__ __forceinline__ void dma16_s(const void* base, uint32_t off, uint32_t lds) {
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
    }
    static __device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                     "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
    }
    static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
        return (uint32_t)(uintptr_t)(lds_ptr_t)p;
    }

    // Page id of key offset x of the tile (lane k of `ids` holds page k);
    // readlane keeps the ids in scalar registers rather than in an array.
    static __device__ __forceinline__ int page_of(int x, int ids) {
        int p = __builtin_amdgcn_readlane(ids, 0);
#pragma unroll
        for (int k = 1; k < NPG; ++k) p = (x >= k * BS) ? __builtin_amdgcn_readlane(ids, k) : p;
        return p;
    }

    // Loads of the tile at key k0 into LDS buffer `lb`: this wave's share of
    // the slots.  `last` is the tile's last valid key offset; later keys load
    // that row again (their scores are masked).
    static __device__ __forceinline__ void issue_tile(const DecodeArgs& a, char* lbuf, int ids, int last,
                                                      int g, int wave, int i, int c) {
        const uint32_t lb = lds_addr(lbuf);
        const int lane = 16 * c + i;
        const int64_t page_stride = (int64_t)a.num_kv_heads * BS * D;
        const int64_t head_off = (int64_t)g * BS * D;
        if (last == KT - 1) {
            // A whole tile: each V slot's rows, and with pages of >= 16
            // tokens each K slot's 16 keys, sit in one page, so the page base
            // is wave-uniform (scalar registers) and each lane adds a fixed
            // in-page offset.
#pragma unroll
            for (int u = 0; u < VSLOTS / NW; ++u) {
                const int v = wave + NW * u;
                const int t = v * RPI + lane / CPR;
                const int page = __builtin_amdgcn_readlane(ids, (v * RPI) / BS);
                const uint16_t* pb = a.v + (int64_t)page * page_stride + head_off;
                const int off = (t % BS) * D + 8 * vchunk(t, lane % CPR);
                dma16_s(pb, 2u * (uint32_t)off, lb + (KSLOTS + v) * 1024);
            }
            if constexpr (BS >= 16) {
#pragma unroll
                for (int u = 0; u < KSLOTS / NW; ++u) {
                    const int s = wave + NW * u;
                    const int kb = s / NKC, kk = s % NKC;
                    const int page = __builtin_amdgcn_readlane(ids, (16 * kb) / BS);
                    const uint16_t* pb = a.k + (int64_t)page * page_stride + head_off;
                    const int off = ((16 * kb + i) % BS) * D + 32 * kk + 8 * c;
                    dma16_s(pb, 2u * (uint32_t)off, lb + s * 1024);
                }
                return;
            }
        } else {
#pragma unroll
            for (int u = 0; u < VSLOTS / NW; ++u) {
                const int v = wave + NW * u;
                const int t = v * RPI + lane / CPR;
                const int x = min(t, last);
                const uint16_t* p = a.v + (int64_t)page_of(x, ids) * page_stride + head_off +
                                    (int64_t)(x % BS) * D + 8 * vchunk(t, lane % CPR);
                dma16(p, lb + (KSLOTS + v) * 1024);
            }
        }
#pragma unroll
        for (int u = 0; u < KSLOTS / NW; ++u) {
            const int s = wave + NW * u;
            const int kb = s / NKC, kk = s % NKC;
            const int x = min(16 * kb + i, last);
            const uint16_t* p = a.k + (int64_t)page_of(x, ids) * page_stride + head_off +
                                (int64_t)(x % BS) * D + 32 * kk + 8 * c;
            dma16(p, lb + s * 1024);
        }
    }

    // V row t of a tile sits in LDS at t * RB with its 16-byte chunks
    // permuted (chunk ch at position ch ^ 2 (t & 7)), so that the eight rows
    // that 32 lanes of one transposing read touch fall in different banks.
    static __device__ __forceinline__ int vchunk(int t, int pos) { return pos ^ ((t & 7) << 1); }

    // Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
    // lanes, lane i receives, for e = 0..3, 16-bit element i % 4 of the 8
    // bytes addressed by lane 4 e + i / 4 of the group.  When lane 4 e + r of
    // group c addresses V[row0 + e][16 m + 4 r ...], lane (i, c) receives
    // V[row0 + e][16 m + i] for e = 0..3: four keys of one dim, a quarter of
    // the PV product's V^T operand.
    static __device__ __forceinline__ uint2 read_vt(const char* p) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
        const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)p);
        return __builtin_bit_cast(uint2, r);
    }

    static __device__ __forceinline__ floatx4 qk_mma(const uint4& a, const uint4& b, const floatx4& c) {
        if constexpr (DT == 1)
            return mfma32_bf16(a, b, c);
        else
            return mfma32(a, b, c);
    }

    static __device__ __forceinline__ uint4 lds16(const char* lb, int slot, int lane) {
        return *reinterpret_cast<const uint4*>(lb + slot * 1024 + 16 * lane);
    }

    // Instruction order of a run of STEPS matrix-product steps fed from LDS
    // (READS operand reads and MFMAS products per step): the reads of the
    // first AH steps, then per step its products and the reads of the step
    // AH later.  Left to itself the compiler issued the PV product's V reads
    // just one product ahead, so every product waited out the LDS latency.
    template <int STEPS, int READS, int MFMAS, int AHEAD>
    static __device__ __forceinline__ void lds_ahead() {
        constexpr int AH = AHEAD < STEPS ? AHEAD : STEPS;
        if constexpr (AH > 0) {
            __builtin_amdgcn_sched_group_barrier(0x100, AH * READS, 0);   // LDS reads
#pragma unroll
            for (int j = 0; j < STEPS - AH; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, MFMAS, 0);    // matrix products
                __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, AH * MFMAS, 0);
        }
    }

    // One tile for this wave's column blocks; rem[cb]: keys of the tile the
    // lane's column sees (MASK: some column sees fewer than KT).
    template <bool MASK>
    static __device__ __forceinline__ void compute(const DecodeArgs& a, Col (&st)[CB], const char* lb,
                                                   const uint4 (&qb)[CB][NKC], const int (&rem)[CB],
                                                   const int (&voff)[8], int lane, int c) {
        floatx4 sc[CB][KB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sc[cb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKC; ++kk) {
            uint4 kv[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kv[kb] = lds16(lb, kb * NKC + kk, lane);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sc[cb][kb] = qk_mma(kv[kb], qb[cb][kk], sc[cb][kb]);
        }
        // the compiler issued most of the tile's K reads before the first
        // product; two chunks ahead: 855 vs 862 us on the chunked prefill
        lds_ahead<NKC, KB, KB * CB, VK_TILE_QK_AHEAD>();
        // weights and their residuals, per 32-key PV step h: keys 32 h + 4c + e,
        // then 32 h + 16 + 4c + e
        uint4 pb[CB][KH], pl[CB][KH];
        float s_hi[CB], s_full[CB];   // fp16: the lane's sum of the rounded / exact weights
        bool heavy = false;           // fp16: some column block of this lane needs the residual
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            constexpr int NX = 4 * KB;
            float x[NX];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = mul_rounded(sc[cb][kb][r], a.scale_log2e);
                    x[4 * kb + r] = (!MASK || 16 * kb + 4 * c + r < rem[cb]) ? v : -INFINITY;
                }
            float mx = x[0];
#pragma unroll
            for (int j = 1; j < NX; ++j) mx = fmaxf(mx, x[j]);
            mx = max_rows4(mx);
            const float mnew = fmaxf(st[cb].m, mx);
            st[cb].m = mnew;
            const bool grow = mnew > st[cb].r + kTau;
            if (__ballot(grow) != 0) {   // some column of the block moves its reference
                const float rnew = grow ? mnew : st[cb].r;
                const float alpha = grow ? exp2_fast(st[cb].r - rnew) : 1.f;   // r = -inf: 0
                st[cb].r = rnew;
                st[cb].l *= alpha;
#pragma unroll
                for (int t = 0; t < NACC; ++t) st[cb].acc[t] *= alpha;
            }
            const float rref = (st[cb].r == -INFINITY) ? 0.f : st[cb].r;
            float p[NX];
#pragma unroll
            for (int j = 0; j < NX; ++j) p[j] = exp2_fast(x[j] - rref) * kPScale;
            if constexpr (DT == 1) {
                float ps = 0.f;
#pragma unroll
                for (int j = 0; j < NX; ++j) ps += p[j];
                st[cb].l += ps;
#pragma unroll
                for (int h = 0; h < KH; ++h) {
                    const float* ph = p + 8 * h;
                    pack_bf16_split(ph[0], ph[1], pb[cb][h].x, pl[cb][h].x);
                    pack_bf16_split(ph[2], ph[3], pb[cb][h].y, pl[cb][h].y);
                    pack_bf16_split(ph[4], ph[5], pb[cb][h].z, pl[cb][h].z);
                    pack_bf16_split(ph[6], ph[7], pb[cb][h].w, pl[cb][h].w);
                }
            } else if constexpr (kSplitMode == 0) {
                // the rounded weights (round to nearest even) and their sum:
                // v_dot2_f32_f16 of each packed pair with (1, 1) adds the two
                // fp16 values exactly as converted back to fp32 (four
                // instructions instead of eight conversions each way and
                // eight adds)
                typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
                const half2_t one2 = {(_Float16)1.f, (_Float16)1.f};
                float hs = 0.f;
#pragma unroll
                for (int h = 0; h < KH; ++h) {
                    const float* ph = p + 8 * h;
                    uint4& w = pb[cb][h];
                    w.x = pack_half2(ph[0], ph[1]);
                    w.y = pack_half2(ph[2], ph[3]);
                    w.z = pack_half2(ph[4], ph[5]);
                    w.w = pack_half2(ph[6], ph[7]);
                    hs = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.x), one2, hs, false);
                    hs = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.y), one2, hs, false);
                    hs = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.z), one2, hs, false);
                    hs = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.w), one2, hs, false);
                }
                s_hi[cb] = s_full[cb] = hs;
            } else {
                // the rounded weights, their sum and the rounded residuals
                float h[NX];
                float hs = 0.f, fs = 0.f;
#pragma unroll
                for (int j = 0; j < NX; ++j) {
                    h[j] = (float)(_Float16)p[j];
                    hs += h[j];
                    fs += p[j];
                }
#pragma unroll
                for (int u = 0; u < KH; ++u) {
                    const float* hu = h + 8 * u;
                    const float* pu = p + 8 * u;
                    pb[cb][u].x = pack_half2(hu[0], hu[1]);
                    pb[cb][u].y = pack_half2(hu[2], hu[3]);
                    pb[cb][u].z = pack_half2(hu[4], hu[5]);
                    pb[cb][u].w = pack_half2(hu[6], hu[7]);
                    if constexpr (kSplitMode > 0) {
                        pl[cb][u].x = pack_half2(pu[0] - hu[0], pu[1] - hu[1]);
                        pl[cb][u].y = pack_half2(pu[2] - hu[2], pu[3] - hu[3]);
                        pl[cb][u].z = pack_half2(pu[4] - hu[4], pu[5] - hu[5]);
                        pl[cb][u].w = pack_half2(pu[6] - hu[6], pu[7] - hu[7]);
                    }
                }
                if constexpr (kSplitMode > 0) heavy = heavy || hs >= kSplitShare * (st[cb].l + hs);
                s_hi[cb] = hs;
                s_full[cb] = fs;
            }
        }
        // fp16: one decision per wave (the products are the wave's).
        bool split = DT == 1 || kSplitMode == 2;
        if constexpr (DT == 0 && kSplitMode == 1) split = __ballot(heavy) != 0;
        if constexpr (DT == 0) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) st[cb].l += split ? s_full[cb] : s_hi[cb];
        }
        // O^T += V^T P^T, 16 dims at a time: in 32-key step h the k-slots of
        // lane group c are keys 32 h + 4c + e, then 32 h + 16 + 4c + e (the
        // order of the weights in pb).  fp16:
        // the residual weights' product, on the tiles that need it, is a
        // second pass over V (its own loop: a branch among the products would
        // keep the compiler from scheduling them together).
        if constexpr (DT == 1 || kSplitMode == 2) {
            pv<2>(st, lb, pb, pl, voff);
        } else {
            pv<0>(st, lb, pb, pl, voff);
            if constexpr (kSplitMode == 1) {
                if (split) pv<1>(st, lb, pb, pl, voff);
            }
        }
    }

    // PV of one tile: W = 0 the rounded weights, 1 the residuals, 2 both.
    // The 32-key steps run outermost, so consecutive products update
    // different accumulators.
    template <int W>
    static __device__ __forceinline__ void pv(Col (&st)[CB], const char* lb, const uint4 (&pb)[CB][KH],
                                              const uint4 (&pl)[CB][KH], const int (&voff)[8]) {
        const char* vb = lb + KSLOTS * 1024;
#pragma unroll
        for (int h = 0; h < KH; ++h)
#pragma unroll
            for (int m = 0; m < NACC; ++m) {
                const char* p = vb + voff[m & 7] + 256 * (m >> 3) + 32 * h * RB;
                const uint2 lo = read_vt(p), hi = read_vt(p + 16 * RB);
                const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    if constexpr (DT == 1) {
                        st[cb].acc[m] = mfma32_bf16(av, pb[cb][h], st[cb].acc[m]);
                        st[cb].acc[m] = mfma32_bf16(av, pl[cb][h], st[cb].acc[m]);
                    } else {
                        if constexpr (W != 1) st[cb].acc[m] = mfma32(av, pb[cb][h], st[cb].acc[m]);
                        if constexpr (W != 0) st[cb].acc[m] = mfma32(av, pl[cb][h], st[cb].acc[m]);
                    }
                }
            }
        lds_ahead<KH * NACC, 2, CB * ((DT == 1 || W == 2) ? 2 : 1), VK_TILE_PV_AHEAD>();
    }

    // Page ids of the tile at k0 into a 256-byte LDS slot: lane k holds page
    // k / BS + k of the tile, clamped to the range's last page (only lanes
    // k < NPG are used).
    static __device__ __forceinline__ void load_ids(const int32_t* bt, int k0, int t_end, int lane,
                                                    int* slot) {
        dma4(bt + min(k0 / BS + lane, (t_end - 1) / BS), lds_addr(slot));
    }
    // Out-of-pool ids read page 0 instead and flag the tile.
    static __device__ __forceinline__ int checked_ids(const DecodeArgs& a, int ids, int lane, bool& bad) {
        const bool b = lane < NPG && (ids < 0 || (int64_t)ids >= a.num_blocks);
        bad = __ballot(b) != 0;
        return b ? 0 : ids;
    }

    // This wave's loads of a tile have landed once at most `n` of its later
    // loads are outstanding (loads complete in issue order).
    template <int N>
    static __device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
    // Workgroup barrier for the LDS pipeline.  __syncthreads() would also wait
    // for every outstanding global load (its fence covers global memory),
    // i.e. for the tiles still in flight; here only this wave's LDS reads are
    // drained (the buffer loaded next is free once every wave is past), and
    // the memory clobber keeps the compiler from moving LDS accesses across.
    static __device__ __forceinline__ void lds_barrier() {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    static __device__ __forceinline__ void wait_tile(int later_tiles) {
        // (two buffers: no later tile is in flight, later_tiles is 0)
        static_assert((NBUF == 4 || NBUF == 2) && 2 * (ISSUE + 1) < 64, "vmcnt range");
        // each later tile: its page-id load and its K/V loads
        if (later_tiles >= 2)
            wait_vm<2 * (ISSUE + 1)>();
        else if (later_tiles == 1)
            wait_vm<ISSUE + 1>();
        else
            wait_vm<0>();
    }

    // Workgroup order across the XCDs.  Workgroups are dealt to the eight
    // XCDs in turn by linear id, each XCD with its own L2, and the query tiles
    // of one (sequence, KV head) stream the same key tiles.  Here each XCD
    // takes runs of 8 consecutive items (8 query tiles of one (sequence, KV
    // head), read through one L2) while the runs are still dealt round-robin,
    // so every XCD keeps a share of every sequence (contiguous quarters of
    // the launch per XCD unbalanced the XCDs: 10% slower).  Measured on the
    // chunked prefill: L2 hit rate 75% -> 83%, bytes fetched past L2
    // 1.49 -> 1.00 GB, 1.8% faster.  A bijection of the ids (the tail of
    // fewer than 64 keeps its order), so only the speed depends on it.
    static __device__ __forceinline__ void xcd_order(unsigned& bx, unsigned& by, unsigned& bz) {
        constexpr uint64_t kXcds = 8, kRun = 8;
        const uint64_t gx = gridDim.x, gy = gridDim.y;
        const uint64_t n = gx * gy * gridDim.z;
        uint64_t i = blockIdx.x + gx * (blockIdx.y + gy * (uint64_t)blockIdx.z);
        if (i < n / (kXcds * kRun) * (kXcds * kRun)) {
            const uint64_t x = i % kXcds, slot = i / kXcds;
            i = ((slot / kRun) * kXcds + x) * kRun + slot % kRun;
        }
        bx = (unsigned)(i % gx);
        by = (unsigned)((i / gx) % gy);
        bz = (unsigned)(i / (gx * gy));
    }

    // Tiles of the (sequence, KV head) with at most key-range end y relative
    // to the sequence's first new token (key-range end = L - q + the tile's
    // last token + 1): tile t ends at token min(q, ((t + 1) NC - 1) / G + 1),
    // so the first T - 1 tiles end by y < q exactly when (t + 1) NC <= y G,
    // and the last one (and a second-to-last that reaches the last token)
    // only when y >= q.
    static __device__ __forceinline__ int tiles_ending_by(int64_t y, int q, int T) {
        if (T == 0 || y < 1) return 0;
        if (y >= q) return T;
        return (int)min((int64_t)T - 1, (y * G) / NC);
    }
    static __device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
        return v;
    }

    // Global longest-first order of an unsplit launch over at most 64
    // sequences (lane s holds sequence s): the (sequence, tile) items by
    // decreasing key-range end, ties by sequence then tile, the Hkv KV heads
    // of an item consecutive.  Launch index k is item k / Hkv: its key-range
    // end x is found by a binary search over the tiles that end after x,
    // counted per sequence in closed form; then the rank among the items
    // ending exactly at x picks the sequence and tile.  Indices past the last
    // item return false.  Selected on request only: on the chunked prefill
    // it lost the L2 reuse of the grid order's runs of 8 (xcd_order) and was
    // 4% slower.
    static __device__ bool longest_first(const VarlenArgs& va, int& tile, int& g, int& s) {
        const DecodeArgs& a = va.d;
        const int lane = threadIdx.x & 63;
        const int S = a.num_seqs, Hkv = a.num_kv_heads;
        const int64_t k = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
        const int q = lane < S ? va.cu_q[lane + 1] - va.cu_q[lane] : 0;
        const int T = q > 0 ? (int)(((int64_t)q * G + NC - 1) / NC) : 0;
        const int64_t base = lane < S ? (int64_t)a.seq_lens[lane] - q : 0;
        const int64_t j = k / Hkv;
        if (j >= wave_sum(T)) return false;
        g = (int)(k % Hkv);
        // key-range ends lie in [base + first tile's end, base + q]
        int64_t lo = T > 0 ? base + min(q, (NC - 1) / G + 1) - 1 : INT64_MAX;
        int64_t hi = T > 0 ? base + q : INT64_MIN;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            lo = min(lo, (int64_t)__shfl_xor(lo, off));
            hi = max(hi, (int64_t)__shfl_xor(hi, off));
        }
        // invariant: more than j items end after lo, at most j after hi
        while (hi - lo > 1) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (wave_sum(T - tiles_ending_by(mid - base, q, T)) <= j)
                hi = mid;
            else
                lo = mid;
        }
        const int r = (int)(j - wave_sum(T - tiles_ending_by(hi - base, q, T)));
        const int below = tiles_ending_by(hi - 1 - base, q, T);
        const int m = tiles_ending_by(hi - base, q, T) - below;   // this sequence's items ending at hi
        int pre = m;                                              // inclusive prefix over the lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(pre, off);
            if (lane >= off) pre += t;
        }
        pre -= m;
        const unsigned long long own = __ballot(m > 0 && r >= pre && r < pre + m);
        if (own == 0) return false;   // unreachable when the counts agree
        s = __ffsll(own) - 1;
        tile = __shfl(below + (r - pre), s);
        return true;
    }

    static __device__ void run(const VarlenArgs& va) {
        __shared__ __attribute__((aligned(16))) char lds[NBUF * BUF];
        __shared__ int ring[NW][NBUF][64];   // per wave: page ids of tile u in slot u % NBUF
        const DecodeArgs& a = va.d;
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i = lane & 15, c = lane >> 4;
        int tile, part, g, s;
        if (a.work_order == 1) {
            if (!longest_first(va, tile, g, s)) return;
            part = 0;
        } else {
            unsigned bx, by, bz;
            xcd_order(bx, by, bz);
            // Later tiles see more keys: they start first.
            tile = va.tiles - 1 - (int)(bx % (unsigned)va.tiles);
            part = (int)(bx / (unsigned)va.tiles);
            g = (int)by;
            s = (int)bz;
        }
        const int q0 = va.cu_q[s], qlen = va.cu_q[s + 1] - q0;
        if (qlen <= 0 || tile * NC >= qlen * G) return;
        const int Hq = a.num_q_heads, P = a.partition_size, NP = a.max_num_partitions;
        const int L = a.seq_lens[s];
        const bool poison = L > a.max_blocks_per_seq * BS;
        // The workgroup's key range ends where its last query token's does.
        const int kv_end = L - qlen + min(qlen, (tile * NC + NC - 1) / G + 1);
        int t_begin = 0, t_end = kv_end;
        if (P > 0) {
            t_begin = part * P;
            t_end = min(kv_end, t_begin + P);
        }

        // Columns: lane column i of block cb is workgroup column 16 (CB wave + cb) + i,
        // column tile * NC + that of the (sequence, KV head): token / G, head % G.
        bool valid[CB], col_poison[CB];
        int lim[CB];
        int64_t row[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int cg = tile * NC + 16 * CB * wave + 16 * cb + i;
            const int jt = cg / G;
            valid[cb] = jt < qlen;
            lim[cb] = valid[cb] ? L - qlen + jt + 1 : 0;
            row[cb] = ((int64_t)q0 + jt) * Hq + g * G + cg % G;
            col_poison[cb] = P > 0 && part == NP - 1 && lim[cb] > t_begin + P;
        }
        if (t_end <= t_begin || poison) {   // uniform over the workgroup
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                if (valid[cb] && P == 0) {   // no visible key: zeros; poisoned: NaN
                    const float z = (poison && lim[cb] > 0) ? __builtin_nanf("") : 0.f;
                    float* o = a.out + row[cb] * D;
                    for (int d = 4 * c; d < D; d += 16) *reinterpret_cast<float4*>(o + d) = make_float4(z, z, z, z);
                } else if (valid[cb] && poison && lim[cb] > t_begin) {   // the partials the reduce reads
                    const int64_t pr = row[cb] * NP + part;
                    if (c == 0) a.max_logits[pr] = a.exp_sums[pr] = __builtin_nanf("");
                    const float z = __builtin_nanf("");
                    float* o = a.tmp_out + pr * D;
                    for (int d = 4 * c; d < D; d += 16) *reinterpret_cast<float4*>(o + d) = make_float4(z, z, z, z);
                }
            }
            return;
        }

        const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
        // Page ids of tiles 0 .. NBUF - 2; later ones are loaded NBUF - 1
        // tiles ahead of their K/V, ahead of the loads of the tile that frees
        // their slot, so they have landed whenever that tile has.
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u) load_ids(bt, t_begin + u * KT, t_end, lane, ring[wave][u]);
        uint4 qb[CB][NKC];
        int e_lim[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint4* qp = reinterpret_cast<const uint4*>(a.q + (valid[cb] ? row[cb] : 0) * D);
#pragma unroll
            for (int kk = 0; kk < NKC; ++kk) qb[cb][kk] = valid[cb] ? qp[4 * kk + c] : make_uint4(0, 0, 0, 0);
            // keys of the range this column sees (other columns: all, harmlessly)
            e_lim[cb] = valid[cb] ? min(lim[cb], t_end) : t_end;
        }
        // The wave's key span: tiles past its largest limit are skipped, tiles
        // below its smallest need no mask.
        int w_max = t_begin, w_min = t_end;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (valid[cb]) w_max = max(w_max, e_lim[cb]);
            w_min = min(w_min, e_lim[cb]);
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            w_max = max(w_max, __shfl_xor(w_max, off));
            w_min = min(w_min, __shfl_xor(w_min, off));
        }

        Col st[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int t = 0; t < NACC; ++t) st[cb].acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
            st[cb].m = st[cb].r = -INFINITY;
            st[cb].l = 0.f;
        }
        // Transposing-read addresses of dims 16 m .. 16 m + 15 (m % 8 = mm;
        // + 256 (m / 8) bytes), keys 4c + e: lane 4e + r of group c points at
        // V[4c + e][16 m + 4 r], its chunk permuted as stored (row t = 4c + e,
        // also for the keys 16 + 4c + e, read 16 rows further).
        int voff[8];
        {
            const int e = (lane & 15) >> 2, r = lane & 3, t = 4 * c + e;
#pragma unroll
            for (int mm = 0; mm < 8; ++mm) voff[mm] = t * RB + 32 * (mm ^ (t & 7)) + 8 * r;
        }
        const int nt = (t_end - t_begin + KT - 1) / KT;
        // Tile u goes to buffer u % NBUF; bit u % NBUF of tbad flags a page id
        // of tile u that was outside the pool.
        bool bad = false;
        unsigned tbad = 0;
        // Every issue makes ISSUE + 1 loads (the page-id load is clamped past
        // the range), which wait_tile counts on.
        auto issue = [&](int u) {
            bool b = false;
            const int ids = checked_ids(a, ring[wave][u % NBUF][lane], lane, b);
            const int k0 = t_begin + u * KT;
            load_ids(bt, k0 + (NBUF - 1) * KT, t_end, lane, ring[wave][(u + NBUF - 1) % NBUF]);
            issue_tile(a, lds + (u % NBUF) * BUF, ids, min(KT, t_end - k0) - 1, g, wave, i, c);
            tbad = b ? (tbad | (1u << (u % NBUF))) : (tbad & ~(1u << (u % NBUF)));
        };
        wait_vm<0>();
        // Mark the query registers as used here, so the compiler's own wait
        // for their loads falls before the loop rather than inside it.
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int kk = 0; kk < NKC; ++kk)
                asm volatile("" ::"v"(qb[cb][kk].x), "v"(qb[cb][kk].y), "v"(qb[cb][kk].z), "v"(qb[cb][kk].w));
#pragma unroll
        for (int u = 0; u < NBUF - 1; ++u)
            if (u < nt) issue(u);
        for (int t = 0; t < nt; ++t) {
            const int k0 = t_begin + t * KT;
            // This wave's loads of tile t have landed; the barrier makes every
            // wave's visible and closes the reads of tile t - 1, whose buffer
            // is loaded next.
            wait_tile(min(nt - 1 - t, NBUF - 2));
            lds_barrier();
            if (t + NBUF - 1 < nt) issue(t + NBUF - 1);
            if (k0 < w_max) {
                bad = bad || ((tbad >> (t % NBUF)) & 1u);
                const char* lb = lds + (t % NBUF) * BUF;
                if (k0 + KT <= w_min) {
                    int rem[CB];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) rem[cb] = KT;
                    compute<false>(a, st, lb, qb, rem, voff, lane, c);
                } else {
                    int rem[CB];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) rem[cb] = e_lim[cb] - k0;
                    compute<true>(a, st, lb, qb, rem, voff, lane, c);
                }
            }
        }

#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            float lsum = st[cb].l + __shfl_xor(st[cb].l, 16);
            lsum += __shfl_xor(lsum, 32);
            // the partial's exp-sum is taken against the max itself
            const float lmax = (st[cb].r == -INFINITY ? lsum : lsum * exp2_fast(st[cb].r - st[cb].m)) *
                               (1.f / kPScale);
            if (!valid[cb]) continue;
            if (P == 0 && lim[cb] <= 0) {   // a query that sees no key: zeros
                float* o = a.out + row[cb] * D;
                for (int d = 4 * c; d < D; d += 16) *reinterpret_cast<float4*>(o + d) = make_float4(0.f, 0.f, 0.f, 0.f);
                continue;
            }
            if (lim[cb] <= t_begin) continue;   // this column does not see this partition
            const bool out_bad = bad || col_poison[cb];
            float* dst;
            if (P == 0) {
                dst = a.out + row[cb] * D;
            } else {
                const int64_t pr = row[cb] * NP + part;
                dst = a.tmp_out + pr * D;
                if (c == 0) {
                    a.max_logits[pr] = st[cb].m;
                    a.exp_sums[pr] = out_bad ? __builtin_nanf("") : lmax;
                }
            }
            const float inv = 1.f / lsum;
#pragma unroll
            for (int m = 0; m < NACC; ++m) {
                float v[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = out_bad ? __builtin_nanf("") : st[cb].acc[m][rr] * inv;
                *reinterpret_cast<float4*>(dst + 16 * m + 4 * c) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
};

template <int D, int G, int BS, int DT>
__global__ __launch_bounds__(64 * tile_waves(D))
__attribute__((amdgpu_waves_per_eu(tile_blocks(D) == 2 && D == 256 ? 1 : 2)))
void varlen_tile_kernel(VarlenArgs a) {
    TileKernel<D, G, BS, DT>::run(a);
}

template <int D, int G, int DT>
hipError_t launch_bs_dt(const VarlenArgs& a, int bs, dim3 grid, hipStream_t st, bool* ok) {
    *ok = true;
    const dim3 block(64 * tile_waves(D));
    switch (bs) {
        case 8: hipLaunchKernelGGL((varlen_tile_kernel<D, G, 8, DT>), grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL((varlen_tile_kernel<D, G, 16, DT>), grid, block, 0, st, a); break;
        case 32: hipLaunchKernelGGL((varlen_tile_kernel<D, G, 32, DT>), grid, block, 0, st, a); break;
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

int64_t varlen_tile_count(int64_t q_len, int group) { return (q_len * group + 127) / 128; }
int varlen_tile_threads(int head_dim) { return 64 * tile_waves(head_dim); }

hipError_t launch_varlen_tile(const VarlenArgs& a, int dtype, int group, int head_dim,
                              int block_size, dim3 grid, hipStream_t stream, bool* geometry_ok) {
    if (group == 4 && head_dim == 128) return launch_bs<128, 4>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 6 && head_dim == 256) return launch_bs<256, 6>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 8 && head_dim == 128) return launch_bs<128, 8>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 8 && head_dim == 256) return launch_bs<256, 8>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 1 && head_dim == 128) return launch_bs<128, 1>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 1 && head_dim == 256) return launch_bs<256, 1>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 16 && head_dim == 128) return launch_bs<128, 16>(a, dtype, block_size, grid, stream, geometry_ok);
    if (group == 16 && head_dim == 256) return launch_bs<256, 16>(a, dtype, block_size, grid, stream, geometry_ok);
    *geometry_ok = false;
    return hipSuccess;
}

}  // namespace vk
