// Matrix-core decode instantiations for the multi-head (G = 1) and
// multi-query (G = 16) geometries, fp16 (MfmaKernel, decode_mfma_impl.h).
// With G = 16 the sixteen MFMA columns are all query heads; with G = 1 one
// column is used and the kernel stays bound by the K/V reads.
#include "decode_mfma_impl.h"

namespace vk {

hipError_t launch_decode_mfma_mhq(const DecodeArgs& a, int group, int head_dim, int block_size,
                                  int waves, int parts_per_wg, dim3 grid, hipStream_t stream,
                                  bool* geometry_ok) {
    return launch_mfma_set<1, 0>(a, group, head_dim, block_size, waves, parts_per_wg, grid,
                                 stream, geometry_ok);
}

}  // namespace vk
