// Matrix-core decode instantiations for bf16 q, K and V (MfmaKernel with
// DT = 1, decode_mfma_impl.h): QK on v_mfma_f32_16x16x32_bf16, PV on
// v_mfma_f32_16x16x16_bf16 with every softmax weight carried as a rounded
// bf16 value plus its bf16 residual (two products), all geometries, the
// two-launch split and the unsplit forms.
#include "decode_mfma_impl.h"

namespace vk {

hipError_t launch_decode_mfma_bf16(const DecodeArgs& a, bool mhq, int group, int head_dim,
                                   int block_size, int waves, int parts_per_wg, dim3 grid,
                                   hipStream_t stream, bool* geometry_ok) {
    if (mhq)
        return launch_mfma_set<1, 1>(a, group, head_dim, block_size, waves, parts_per_wg, grid,
                                     stream, geometry_ok);
    return launch_mfma_set<0, 1>(a, group, head_dim, block_size, waves, parts_per_wg, grid,
                                 stream, geometry_ok);
}

}  // namespace vk
