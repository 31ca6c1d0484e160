// Paged GQA decode attention on the gfx950 matrix cores (VK_KERNEL_MFMA):
// the grouped-query fp16 instantiations and the dispatch across geometry
// sets and element types; the workgroup code is MfmaKernel in
// decode_mfma_impl.h, the other instantiations are in decode_mfma_mhq.hip
// (multi-head / multi-query fp16), decode_mfma_bf16.hip (bf16) and
// decode_mfma_f32.hip (fp32).
#include "decode_mfma_impl.h"

namespace vk {

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int group, int head_dim,
                              int block_size, int waves, int parts_per_wg, dim3 grid,
                              hipStream_t stream, bool* geometry_ok, int* block) {
    *block = 64 * waves;
    const bool mhq = group == 1 || group == 16;
    if (dtype == 1)
        return launch_decode_mfma_bf16(a, mhq, group, head_dim, block_size, waves, parts_per_wg,
                                       grid, stream, geometry_ok);
    if (dtype == 2)
        return launch_decode_mfma_f32(a, mhq, group, head_dim, block_size, waves, parts_per_wg,
                                      grid, stream, geometry_ok);
    if (dtype != 0) {
        *geometry_ok = false;
        return hipSuccess;
    }
    if (mhq)
        return launch_decode_mfma_mhq(a, group, head_dim, block_size, waves, parts_per_wg, grid,
                                      stream, geometry_ok);
    return launch_mfma_set<0, 0>(a, group, head_dim, block_size, waves, parts_per_wg, grid,
                                 stream, geometry_ok);
}

}  // namespace vk
