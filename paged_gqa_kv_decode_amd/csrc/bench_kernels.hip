// Measurement-only kernels for the benchmark harness (libvkbench.so; the
// attention library does not contain them):
//   vkb_stream_read   read a buffer once with 16-byte loads (HBM read ceiling);
//                     vkb_stream_read_nt with nontemporal loads
//   vkb_page_read     read whole KV pages named by a page list, one workgroup
//                     per run of `pages_per_group` pages (the page pattern of
//                     the decode kernel without its arithmetic)
//   vkb_fill          write a buffer
// Every read value is folded into a per-thread xor that is stored to `sink`
// (one uint32 per thread), so no load can be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
    if constexpr (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t x = 0;
    int64_t i = tid;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4 a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = load16<NT>(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[tid] = x;
}

// Workgroup g reads pages ids[g * ppg + k] (k < ppg) of `page_bytes` each.
// mode 0: each load instruction of a wave reads 1 KiB contiguous;
// mode 1: each reads 64 B from each of 16 rows of `row_bytes` (the shape of
//         the decode kernel's K loads).
template <int MODE, bool NT = false>
__global__ __launch_bounds__(256) void page_read_kernel(const uint8_t* __restrict__ pool,
                                                        int64_t pool_pages,
                                                        const int32_t* __restrict__ ids,
                                                        int64_t n_pages, int ppg, int64_t page_bytes,
                                                        int64_t row_bytes,
                                                        uint32_t* __restrict__ sink) {
    const int64_t first = (int64_t)blockIdx.x * ppg;
    const int t = threadIdx.x;
    const int64_t n16 = page_bytes / 16;
    uint32_t x = 0;
    for (int k = 0; k < ppg && first + k < n_pages; ++k) {
        const int64_t id = ids[first + k];
        if (id < 0 || id >= pool_pages) continue;
        const uint4* pg = reinterpret_cast<const uint4*>(pool + id * page_bytes);
        if constexpr (MODE == 1) {
            // wave w, lane l: row 16 * (w + 4 q) + l % 16, chunk 4 kk + l / 16
            const int w = t >> 6, l = t & 63;
            const int64_t row16 = row_bytes / 16, nrows = page_bytes / row_bytes;
            for (int64_t r0 = 16 * w; r0 < nrows; r0 += 64) {
                if (r0 + (l & 15) >= nrows) continue;
                const uint4* rp = pg + (r0 + (l & 15)) * row16;
                for (int64_t kk = 0; 4 * kk < row16; kk += 4) {
                    uint4 v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        v[u] = (4 * (kk + u) + (l >> 4) < row16) ? rp[4 * (kk + u) + (l >> 4)] : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < 4; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
                }
            }
            continue;
        }
        int64_t i = t;
        for (; i + 3 * 256 < n16; i += 4 * 256) {
            const uint4 a = load16<NT>(pg + i), b = load16<NT>(pg + i + 256),
                        c = load16<NT>(pg + i + 512), d = load16<NT>(pg + i + 768);
            x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
        }
        for (; i < n16; i += 256) {
            const uint4 a = pg[i];
            x ^= a.x ^ a.y ^ a.z ^ a.w;
        }
    }
    sink[(int64_t)blockIdx.x * 256 + t] = x;
}

__global__ __launch_bounds__(256) void fill_kernel(uint4* __restrict__ p, int64_t n16, uint32_t v) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(v, v, v, v);
}

}  // namespace

extern "C" {

// bytes must be a multiple of 16; sink holds blocks*256 uint32.
int vkb_stream_read(const void* p, int64_t bytes, void* sink, int blocks, void* stream) {
    if (!p || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return 1;
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)p, bytes / 16, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Same with nontemporal (streaming) loads.
int vkb_stream_read_nt(const void* p, int64_t bytes, void* sink, int blocks, void* stream) {
    if (!p || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return 1;
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const uint4*)p, bytes / 16, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// ids: n_pages int32 page indices into pool (each < pool_pages); sink holds
// ceil(n_pages/ppg)*256 uint32.  Ids outside [0, pool_pages) are skipped.
int vkb_page_read(const void* pool, int64_t pool_pages, const int32_t* ids_dev, int64_t n_pages,
                  int ppg, int64_t page_bytes, void* sink, void* stream) {
    if (!pool || !ids_dev || !sink || n_pages <= 0 || ppg <= 0 || page_bytes <= 0 ||
        page_bytes % 16 || pool_pages <= 0)
        return 1;
    const int64_t groups = (n_pages + ppg - 1) / ppg;
    hipLaunchKernelGGL(page_read_kernel<0>, dim3((unsigned)groups), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)pool, pool_pages, ids_dev, n_pages, ppg, page_bytes,
                       page_bytes, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Mode-0 page read with nontemporal loads.
int vkb_page_read_nt(const void* pool, int64_t pool_pages, const int32_t* ids_dev, int64_t n_pages,
                     int ppg, int64_t page_bytes, void* sink, void* stream) {
    if (!pool || !ids_dev || !sink || n_pages <= 0 || ppg <= 0 || page_bytes <= 0 ||
        page_bytes % 16 || pool_pages <= 0)
        return 1;
    const int64_t groups = (n_pages + ppg - 1) / ppg;
    hipLaunchKernelGGL((page_read_kernel<0, true>), dim3((unsigned)groups), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t*)pool, pool_pages, ids_dev, n_pages, ppg,
                       page_bytes, page_bytes, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Mode-1 page read: rows of row_bytes (a multiple of 64 dividing page_bytes).
int vkb_page_read_rows(const void* pool, int64_t pool_pages, const int32_t* ids_dev,
                       int64_t n_pages, int ppg, int64_t page_bytes, int64_t row_bytes,
                       void* sink, void* stream) {
    if (!pool || !ids_dev || !sink || n_pages <= 0 || ppg <= 0 || page_bytes <= 0 ||
        page_bytes % 16 || pool_pages <= 0 || row_bytes <= 0 || row_bytes % 64 ||
        page_bytes % row_bytes)
        return 1;
    const int64_t groups = (n_pages + ppg - 1) / ppg;
    hipLaunchKernelGGL(page_read_kernel<1>, dim3((unsigned)groups), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)pool, pool_pages, ids_dev, n_pages, ppg, page_bytes,
                       row_bytes, (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int vkb_fill(void* p, int64_t bytes, uint32_t value, void* stream) {
    if (!p || bytes <= 0 || bytes % 16) return 1;
    hipLaunchKernelGGL(fill_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, (uint4*)p,
                       bytes / 16, value);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
