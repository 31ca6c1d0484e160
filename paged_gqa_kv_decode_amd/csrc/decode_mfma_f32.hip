// Matrix-core decode instantiations for fp32 q, K and V (MfmaKernel with
// DT = 2, decode_mfma_impl.h): QK and PV on v_mfma_f32_16x16x4_f32, so scores
// and weights stay fp32 end to end; all geometries, the two-launch split and
// the unsplit forms.  (The fp32 KV cache is the fallback of the fp16 one.)
#include "decode_mfma_impl.h"

namespace vk {

hipError_t launch_decode_mfma_f32(const DecodeArgs& a, bool mhq, int group, int head_dim,
                                  int block_size, int waves, int parts_per_wg, dim3 grid,
                                  hipStream_t stream, bool* geometry_ok) {
    if (mhq)
        return launch_mfma_set<1, 2>(a, group, head_dim, block_size, waves, parts_per_wg, grid,
                                     stream, geometry_ok);
    return launch_mfma_set<0, 2>(a, group, head_dim, block_size, waves, parts_per_wg, grid,
                                 stream, geometry_ok);
}

}  // namespace vk
