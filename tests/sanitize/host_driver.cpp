// Host sanitizer driver for the library's host code (csrc/vk_host.cpp):
// linked with stand-ins for the kernel launchers and for the two HIP device
// queries it makes, so every host path (argument validation, both planners,
// the decode / multi-token / reduce / append dispatch and the no-allocation
// entry point's sizing) runs under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU.  The launcher stand-ins check
// the launch shapes the host code hands the kernels.  Built and run by
// tests/test_sanitizers.py; exits 0 when every check holds.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "vk_kernels.h"
#include "vk_paged.h"

static int g_fail = 0;
static int g_launches = 0;
#define CHECK(c)                                                           \
    do {                                                                   \
        if (!(c)) {                                                        \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

// ---- stand-ins: HIP device queries (256 CUs) ----
extern "C" hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t a, int) {
    *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

// ---- stand-ins: kernel launchers ----
namespace vk {
static void check_grid(dim3 g) { CHECK(g.x >= 1 && g.y >= 1 && g.z >= 1 && g.y <= 65535 && g.z <= 65535); }
static void check_decode(const DecodeArgs& a) {
    CHECK(a.q && a.k && a.v && a.block_tables && a.seq_lens);
    CHECK(a.num_seqs >= 1 && a.num_q_heads >= a.num_kv_heads && a.num_kv_heads >= 1);
    if (a.partition_size == 0) CHECK(a.out != nullptr && a.max_num_partitions == 1);
    else CHECK(a.max_logits && a.exp_sums && a.tmp_out && a.max_num_partitions >= 1);
}
static char g_scratch[64];
hipError_t noalloc_scratch(void** out) { *out = g_scratch; return hipSuccess; }
hipError_t launch_decode_dot(const DecodeArgs& a, int, int, int, dim3 grid, hipStream_t, bool* ok,
                             int* block) {
    check_decode(a); check_grid(grid); ++g_launches; *ok = true; *block = 256; return hipSuccess;
}
hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int, int, int, int waves, int ppw,
                              dim3 grid, hipStream_t, bool* ok, int* block) {
    check_decode(a); check_grid(grid);
    CHECK(dtype >= 0 && dtype <= 2 && (waves == 1 || waves == 2 || waves == 4) && (ppw == 1 || ppw == 2));
    ++g_launches; *ok = true; *block = 64 * waves; return hipSuccess;
}
int varlen_tokens_per_tile(int group) { return group > 0 && group <= 16 ? 16 / group : 0; }
int64_t varlen_tile_count(int64_t q_len, int group) { return (q_len * group + 127) / 128; }
int varlen_tile_threads(int head_dim) { return head_dim == 256 ? 512 : 256; }
hipError_t launch_decode_varlen(const VarlenArgs& a, int, int, int, int, dim3 grid, hipStream_t,
                                bool* ok) {
    check_decode(a.d); check_grid(grid); CHECK(a.cu_q && a.tiles >= 1);
    ++g_launches; *ok = true; return hipSuccess;
}
hipError_t launch_varlen_tile(const VarlenArgs& a, int, int, int, int, dim3 grid, hipStream_t,
                              bool* ok) {
    check_decode(a.d); check_grid(grid); CHECK(a.cu_q && a.tiles >= 1);
    ++g_launches; *ok = true; return hipSuccess;
}
hipError_t launch_kv_append(const AppendArgs& a, int num_seqs, hipStream_t) {
    CHECK(a.k_new && a.v_new && a.positions && num_seqs >= 1); ++g_launches; return hipSuccess;
}
hipError_t launch_reduce(const ReduceArgs& a, int, dim3 grid, hipStream_t, bool* ok) {
    CHECK(a.max_logits && a.exp_sums && a.tmp_out && a.out); check_grid(grid);
    ++g_launches; *ok = true; return hipSuccess;
}
hipError_t launch_reduce_varlen(const ReduceArgs& a, const int32_t* cu_q, int, int max_q_len,
                                int num_seqs, hipStream_t, bool* ok) {
    CHECK(a.out && cu_q && max_q_len >= 1 && num_seqs >= 1); ++g_launches; *ok = true;
    return hipSuccess;
}
}  // namespace vk

int main() {
    std::mt19937 rng(7);
    const int geo[][3] = {{32, 8, 128}, {24, 4, 256}, {16, 2, 128}, {16, 2, 256},
                          {16, 16, 128}, {8, 8, 256}, {16, 1, 128}, {16, 1, 256}};
    // device pointers are never dereferenced on the host: aligned stand-ins
    alignas(256) static char fake[4096];
    void* F = fake;
    for (int it = 0; it < 400; ++it) {
        const int* g = geo[it % 8];
        const int Hq = g[0], Hkv = g[1], D = g[2], bs = 8 << (it % 3);
        const int S = 1 + (int)(rng() % 64);
        std::vector<int32_t> lens(S), ql(S);
        int maxL = 1;
        for (int s = 0; s < S; ++s) {
            lens[s] = 1 + (int)(rng() % (it % 5 == 0 ? 140000 : 9000));
            ql[s] = (int)(rng() % (lens[s] < 40 ? lens[s] + 1 : 41));
            maxL = lens[s] > maxL ? lens[s] : maxL;
        }
        const int mb = (maxL + bs - 1) / bs;
        for (int req : {-1, 0, 256, 512}) {
            vk_plan p{};
            const vk_status st = vk_plan_partitions(lens.data(), S, Hq, Hkv, D, bs, mb, req, 256, 0, 0, &p);
            CHECK(st == VK_OK || st == VK_ERR_SCRATCH_CAP);
            if (st != VK_OK) continue;
            const int P = p.partition_size, NP = p.max_num_partitions;
            float* out = (float*)F;
            CHECK(vk_paged_gqa_decode(F, F, F, (int32_t*)F, (int32_t*)F, S, Hq, Hkv, D, bs, mb, 1000, 0.1f,
                                      P, NP, out, P ? out : nullptr, P ? out : nullptr, P ? out : nullptr,
                                      nullptr) == VK_OK);
            for (int dt : {1, 2})
                CHECK(vk_paged_gqa_decode_dt(dt, F, F, F, (int32_t*)F, (int32_t*)F, S, Hq, Hkv, D, bs, mb, 1000,
                                             0.1f, P, NP, out, out, out, out, nullptr) == VK_OK);
            CHECK(vk_paged_gqa_decode_fused(F, F, F, (int32_t*)F, (int32_t*)F, S, Hq, Hkv, D, bs, mb, 1000,
                                            0.1f, P, NP, out, out, out, out, (uint32_t*)F, nullptr) == VK_OK);
            const vk_status na = vk_paged_gqa_decode_noalloc(F, F, F, (int32_t*)F, (int32_t*)F, S, Hq, Hkv, D,
                                                             bs, mb, 1000, 0.1f, P, NP, out, nullptr);
            CHECK(na == VK_OK || na == VK_ERR_SCRATCH_CAP);
            if (P) CHECK(vk_paged_gqa_reduce(out, out, out, (int32_t*)F, S, Hq, D, P, NP, out, nullptr) == VK_OK);
            vk_plan lp{};
            CHECK(vk_last_plan(&lp) == VK_OK);
        }
        // several query tokens per sequence
        int32_t total_q = 0, max_q = 0;
        for (int s = 0; s < S; ++s) { total_q += ql[s]; max_q = ql[s] > max_q ? ql[s] : max_q; }
        for (int kern : {VK_KERNEL_AUTO, VK_KERNEL_VARLEN_COLUMNS, VK_KERNEL_VARLEN_TILES}) {
            vk_select_varlen_kernel(kern);
            for (int req : {-1, 0, 256, 512}) {
                vk_plan p{};
                const vk_status st = vk_plan_varlen(lens.data(), ql.data(), S, Hq, Hkv, D, bs, mb, req, 256, 0, &p);
                CHECK(st == VK_OK || st == VK_ERR_SCRATCH_CAP);
                if (st != VK_OK || total_q == 0) continue;
                float* out = (float*)F;
                for (int dt : {0, 1})
                    CHECK(vk_paged_gqa_varlen_dt(dt, F, F, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, S, total_q,
                                                 max_q, Hq, Hkv, D, bs, mb, 1000, 0.1f, p.partition_size,
                                                 p.max_num_partitions, out, out, out, out, nullptr) == VK_OK);
                if (p.partition_size)
                    CHECK(vk_paged_gqa_varlen_reduce(out, out, out, (int32_t*)F, (int32_t*)F, S, max_q, Hq, D,
                                                     p.partition_size, p.max_num_partitions, out, nullptr) == VK_OK);
            }
        }
        vk_select_varlen_kernel(VK_KERNEL_AUTO);
        CHECK(vk_paged_kv_append(F, F, (int32_t*)F, (int32_t*)F, S, Hkv, D, bs, mb, 1000, it % 2 ? 1e4 : 0.0,
                                 F, F, nullptr) == VK_OK);
        // every kernel family and order switch through the same dispatch
        vk_select_decode_kernel(VK_KERNEL_DOT + it % 6);
        vk_select_work_order(it % 3);
    }
    // rejected arguments never reach a launcher
    const int before = g_launches;
    CHECK(vk_paged_gqa_decode(nullptr, F, F, (int32_t*)F, (int32_t*)F, 1, 32, 8, 128, 16, 4, 10, 0.1f, 0, 1,
                              (float*)F, nullptr, nullptr, nullptr, nullptr) == VK_ERR_NULL_ARG);
    CHECK(vk_paged_gqa_decode((char*)F + 8, F, F, (int32_t*)F, (int32_t*)F, 1, 32, 8, 128, 16, 4, 10, 0.1f, 0, 1,
                              (float*)F, nullptr, nullptr, nullptr, nullptr) == VK_ERR_ALIGN);
    CHECK(vk_paged_gqa_decode_noalloc(F, F, F, (int32_t*)F, (int32_t*)F, 2, 32, 8, 128, 16, 4, 10, 0.1f, 512,
                                      3000, (float*)F, nullptr) == VK_ERR_SCRATCH_CAP);
    CHECK(g_launches == before);
    for (int s = -3; s < 14; ++s) CHECK(vk_status_string(s) != nullptr);
    std::printf("host sanitizer driver: %d launches checked, %d failures\n", g_launches, g_fail);
    return g_fail != 0;
}
