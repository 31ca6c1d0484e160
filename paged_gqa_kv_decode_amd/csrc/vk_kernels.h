// Internal interface between the C-ABI host code (vk_host.cpp) and the HIP
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vk {

struct DecodeArgs {
    const uint16_t* q;            // fp16 [S, Hq, D]
    const uint16_t* k;            // fp16 [num_blocks, Hkv, BS, D]
    const uint16_t* v;            // fp16 [num_blocks, Hkv, BS, D]
    const int32_t* block_tables;  // [S, max_blocks_per_seq]
    const int32_t* seq_lens;      // [S]
    float* out;                   // [S, Hq, D]          (unsplit)
    float* max_logits;            // [S, Hq, NP]         (split)
    float* exp_sums;              // [S, Hq, NP]         (split)
    float* tmp_out;               // [S, Hq, NP, D]      (split)
    uint32_t* counters;           // [S, Hkv] arrival counters (split, single launch); else null
    int64_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_seqs;
    int32_t partition_size;       // 0 = unsplit
    int32_t max_num_partitions;
    float scale_log2e;            // scale * log2(e), rounded once to fp32
    int32_t work_order;           // 0: grid order; 1: longest first (split, <= 64 sequences)
    int32_t write_through;        // 1: split partials stored through L2 (device scope)
};

// Several query tokens per sequence (causal): `d` as for the decode, with
// d.q the packed query rows [total_q, Hq, D], d.out [total_q, Hq, D] and the
// partials [total_q, Hq, NP(, D)]; sequence s owns rows cu_q[s] .. cu_q[s+1]-1.
struct VarlenArgs {
    DecodeArgs d;
    const int32_t* cu_q;          // [S + 1]
    int32_t tiles;                // column tiles per (sequence, KV head): grid.x = tiles * NP
};

struct ReduceArgs {
    const float* max_logits;
    const float* exp_sums;
    const float* tmp_out;
    const int32_t* seq_lens;
    float* out;
    int32_t num_q_heads;
    int32_t partition_size;
    int32_t max_num_partitions;
};

struct AppendArgs {
    const uint16_t* k_new;        // fp16 [S, Hkv, D]
    const uint16_t* v_new;        // fp16 [S, Hkv, D]
    const int32_t* block_tables;  // [S, max_blocks_per_seq]
    const int32_t* positions;     // [S]
    uint16_t* k_cache;            // fp16 [num_blocks, Hkv, BS, D]
    uint16_t* v_cache;
    int64_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    double rope_theta;            // <= 0: no rotary embedding
};

// Device address of this device's copy of the library-held scratch array
// (VK_NOALLOC_SCRATCH_BYTES; noalloc.hip), looked up once per device.
hipError_t noalloc_scratch(void** out);

// Each launcher returns hipSuccess or the launch error; `geometry_ok` is
// false when no specialisation exists for the shape (host code checks first).
hipError_t launch_decode_dot(const DecodeArgs& a, int group, int head_dim, int block_size,
                             dim3 grid, hipStream_t stream, bool* geometry_ok, int* block);
// dtype: element type of q, K and V (0 fp16, 1 bf16, 2 fp32); waves: 1, 2 or 4
// wave64s per workgroup; parts_per_wg: partitions per workgroup (1, or 2 with
// 4 waves in a split fp16 launch: grid.x = ceil(NP / 2)).  geometry_ok is
// false when no instantiation matches (including the single-launch form or
// two partitions per workgroup with bf16).
hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int group, int head_dim,
                              int block_size, int waves, int parts_per_wg, dim3 grid,
                              hipStream_t stream, bool* geometry_ok, int* block);
hipError_t launch_decode_mfma_mhq(const DecodeArgs& a, int group, int head_dim, int block_size,
                                  int waves, int parts_per_wg, dim3 grid, hipStream_t stream,
                                  bool* geometry_ok);
hipError_t launch_decode_mfma_bf16(const DecodeArgs& a, bool mhq, int group, int head_dim,
                                   int block_size, int waves, int parts_per_wg, dim3 grid,
                                   hipStream_t stream, bool* geometry_ok);
hipError_t launch_decode_mfma_f32(const DecodeArgs& a, bool mhq, int group, int head_dim,
                                  int block_size, int waves, int parts_per_wg, dim3 grid,
                                  hipStream_t stream, bool* geometry_ok);
// One wave per workgroup; grid (tiles * max(NP, 1), Hkv, S).  tokens_per_tile
// receives 16 / G (query tokens per 16-column tile) for the caller's grid.
// dtype: element type of q, K and V (0 fp16, 1 bf16).
hipError_t launch_decode_varlen(const VarlenArgs& a, int dtype, int group, int head_dim,
                                int block_size, dim3 grid, hipStream_t stream, bool* geometry_ok);
int varlen_tokens_per_tile(int group);
// Workgroups of 128 consecutive (token, head) columns; grid (tiles * max(NP, 1),
// Hkv, S) with tiles = varlen_tile_count(max_q_len, G) = ceil(max_q_len * G / 128).
hipError_t launch_varlen_tile(const VarlenArgs& a, int dtype, int group, int head_dim,
                              int block_size, dim3 grid, hipStream_t stream, bool* geometry_ok);
int64_t varlen_tile_count(int64_t q_len, int group);
int varlen_tile_threads(int head_dim);
hipError_t launch_kv_append(const AppendArgs& a, int num_seqs, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int head_dim, dim3 grid, hipStream_t stream,
                         bool* geometry_ok);
// Variable-length rows: grid (Hq, max_q_len, S) before the split into 32-dim chunks.
hipError_t launch_reduce_varlen(const ReduceArgs& a, const int32_t* cu_q, int head_dim,
                                int max_q_len, int num_seqs, hipStream_t stream,
                                bool* geometry_ok);

}  // namespace vk
