// Paged KV-cache append for gfx950: write each sequence's new token's K and V
// rows into the page slot the page table names (vllm-metal kernels page,
// cf-1.com/news/5525226, section "什么是 Paged Attention": logical page
// pos / bs of sequence s is physical page block_tables[s][pos / bs]; the
// voxtral.c page, dpshk.com/news/5521762, sections "模型结构与解码瓶颈" and
// "下一步优化方向": each decode step writes the new K/V, and rotary position
// embedding of K belongs in the same pass).
//
// Rotary embedding (when theta > 0), rotate-half convention: for
// j < D/2 the pair (k[j], k[j + D/2]) is rotated by the angle
// pos * theta^(-2j/D).  The angle, its sine and cosine and the rotation are
// evaluated in float64 (positions reach 1e5+, where an fp32 angle would
// already be off by ~1e-2 rad), then rounded once to fp16.
//
// Grid (S, Hkv), D/2 threads: thread j owns the pair (j, j + D/2) of K and V.
#include "vk_kernels.h"

namespace vk {
namespace {

__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
    // double -> fp16 with one rounding (round to nearest even), overflow to inf.
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
    return (double)__builtin_bit_cast(_Float16, h);
}

__global__ __launch_bounds__(128) void kv_append_kernel(AppendArgs a) {
    const int s = blockIdx.x, g = blockIdx.y, j = threadIdx.x;
    const int D = a.head_dim, H = D / 2;
    if (j >= H) return;
    const int pos = a.positions[s];
    if (pos < 0 || pos >= a.max_blocks_per_seq * a.block_size) return;   // padding / out of table
    const int32_t blk = a.block_tables[(int64_t)s * a.max_blocks_per_seq + pos / a.block_size];
    if (blk < 0 || (int64_t)blk >= a.num_blocks) return;                 // no such page
    const int64_t src = ((int64_t)s * a.num_kv_heads + g) * D;
    const int64_t dst = (((int64_t)blk * a.num_kv_heads + g) * a.block_size + pos % a.block_size) * D;
    const uint16_t k0 = a.k_new[src + j], k1 = a.k_new[src + j + H];
    uint16_t o0 = k0, o1 = k1;
    if (a.rope_theta > 0.0) {
        const double inv_freq = pow(a.rope_theta, -2.0 * (double)j / (double)D);
        double sn, cs;
        sincos((double)pos * inv_freq, &sn, &cs);
        const double x0 = f16_bits_to_f64(k0), x1 = f16_bits_to_f64(k1);
        o0 = f64_to_f16_bits(x0 * cs - x1 * sn);
        o1 = f64_to_f16_bits(x0 * sn + x1 * cs);
    }
    a.k_cache[dst + j] = o0;
    a.k_cache[dst + j + H] = o1;
    a.v_cache[dst + j] = a.v_new[src + j];
    a.v_cache[dst + j + H] = a.v_new[src + j + H];
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, int num_seqs, hipStream_t stream) {
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)num_seqs, (unsigned)a.num_kv_heads),
                       dim3((unsigned)(a.head_dim / 2)), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vk
