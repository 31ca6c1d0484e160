// Paged GQA decode attention on the gfx950 matrix cores (VK_KERNEL_MFMA):
// kernel instantiations and launchers; the workgroup code is MfmaKernel in
// decode_mfma_impl.h.
#include "decode_mfma_impl.h"

namespace vk {
namespace {

// At least two resident waves per SIMD: caps a lane at 256 registers.
template <int D, int G, int BS, int W, int WP, bool FUSED>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(VK_MFMA_WAVES_PER_EU)))
void decode_mfma_kernel(DecodeArgs a) {
    MfmaKernel<D, G, BS, W, WP, (D == 256 ? VK_MFMA_T256 : VK_MFMA_T128), FUSED>::run(a);
}

template <int D, int G, int W, int WP, bool FUSED>
hipError_t launch_bs(const DecodeArgs& a, int bs, dim3 grid, hipStream_t st, bool* ok) {
    *ok = true;
    const dim3 block(64 * W);
    switch (bs) {
        case 8: hipLaunchKernelGGL((decode_mfma_kernel<D, G, 8, W, WP, FUSED>), grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL((decode_mfma_kernel<D, G, 16, W, WP, FUSED>), grid, block, 0, st, a); break;
        case 32: hipLaunchKernelGGL((decode_mfma_kernel<D, G, 32, W, WP, FUSED>), grid, block, 0, st, a); break;
        default: *ok = false; return hipSuccess;
    }
    return hipGetLastError();
}

template <int W, int WP, bool FUSED>
hipError_t launch_w(const DecodeArgs& a, int group, int head_dim, int bs, dim3 grid,
                    hipStream_t st, bool* ok) {
    if (group == 4 && head_dim == 128) return launch_bs<128, 4, W, WP, FUSED>(a, bs, grid, st, ok);
    if (group == 6 && head_dim == 256) return launch_bs<256, 6, W, WP, FUSED>(a, bs, grid, st, ok);
    if (group == 8 && head_dim == 128) return launch_bs<128, 8, W, WP, FUSED>(a, bs, grid, st, ok);
    if (group == 8 && head_dim == 256) return launch_bs<256, 8, W, WP, FUSED>(a, bs, grid, st, ok);
    *ok = false;
    return hipSuccess;
}

template <bool FUSED>
hipError_t launch_waves(const DecodeArgs& a, int group, int head_dim, int block_size, int waves,
                        dim3 grid, hipStream_t stream, bool* geometry_ok) {
    switch (waves) {
        case 1: return launch_w<1, 1, FUSED>(a, group, head_dim, block_size, grid, stream, geometry_ok);
        case 2: return launch_w<2, 2, FUSED>(a, group, head_dim, block_size, grid, stream, geometry_ok);
        case 4: return launch_w<4, 4, FUSED>(a, group, head_dim, block_size, grid, stream, geometry_ok);
        default: *geometry_ok = false; return hipSuccess;
    }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int group, int head_dim, int block_size,
                              int waves, int parts_per_wg, dim3 grid, hipStream_t stream,
                              bool* geometry_ok, int* block) {
    *block = 64 * waves;
    // Split launches with a counter array merge their partitions in place.
    if (a.counters != nullptr && a.partition_size > 0) {
        if (parts_per_wg != 1) {
            *geometry_ok = false;
            return hipSuccess;
        }
        return launch_waves<true>(a, group, head_dim, block_size, waves, grid, stream, geometry_ok);
    }
    if (parts_per_wg == 2) {
        // four waves over two consecutive partitions, two waves each (split only)
        if (waves != 4 || a.partition_size == 0) {
            *geometry_ok = false;
            return hipSuccess;
        }
        return launch_w<4, 2, false>(a, group, head_dim, block_size, grid, stream, geometry_ok);
    }
    if (parts_per_wg != 1) {
        *geometry_ok = false;
        return hipSuccess;
    }
    return launch_waves<false>(a, group, head_dim, block_size, waves, grid, stream, geometry_ok);
}

}  // namespace vk
