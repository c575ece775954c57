// pa_internal.hpp -- argument blocks and launchers shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// The attention kernels work in units of 16 tokens of one kv head: a 16-token block, or one
// half of a 32-token block (the pool layout puts a 32-token block's two halves at fixed
// offsets inside its tile).
constexpr int kUnitTokens = 16;
constexpr int kDecodeThreads = 256; // 4 waves per decode workgroup
constexpr int kDecodeWaves = 4;

struct KvWriteArgs {
    const void* key;
    const void* value;
    void* k_pool;
    void* v_pool;
    int64_t num_blocks;
    const int64_t* slots;
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    const float* k_scale;
    const float* v_scale;
};

// Decode: the streaming kernel (phase 1) and the merge kernel (phase 2).
constexpr int kSimds = 1024;         // 256 CUs x 4 SIMDs
constexpr int kStreamWavesMax = 3 * kSimds;  // largest persistent grid (3 waves per SIMD)
constexpr int kMinChunkBlocks = 8;   // smallest automatic chunk, in (block, kv head) units
constexpr int kMaxDecodeSeqs = 16384;  // context lengths of a call are staged in 64 KiB of LDS
constexpr int kMaxDecodeSeqsShared = 8192;  // ... and the shared-block counts beside them

struct DecodeArgs {
    void* out;
    const void* query;
    void* k_pool;     // written only by the fused append
    void* v_pool;
    const void* new_key;    // fused append: [num_seqs][Hkv][D] rows in the query dtype, or null
    const void* new_value;
    int64_t num_blocks;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    const int32_t* shared_blocks;  // [S] leading blocks of each sequence shared with other
                                   // sequences (read with cached loads), or null
    int32_t max_context_len;  // context lengths are clamped to this bound
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t block_size;  // 16 or 32 tokens
    float scale_log2;  // softmax scale times log2(e): scores are kept in base 2
    const float* k_scale;
    const float* v_scale;
    int32_t chunk_blocks;     // units per chunk; 0 = ceil(U / waves), at least kMinChunkBlocks;
                              // -1 = one chunk per run (no split, no merge)
    int32_t grid_workgroups;  // workgroups of the streaming grid (4 waves each)
    int64_t max_chunks;       // chunks the workspace has room for
    int64_t max_pieces;       // pieces the workspace has room for (runs + max_chunks)
    float* o_part;            // [max_pieces][G][D]  normalised partial rows
    float* ml_part;           // [max_pieces][G][2]  (running max in base 2, softmax sum)
    int32_t* run_info;        // [Hkv * S][2]        (first chunk, number of pieces) of run g S + s
};

// Chunked prefill: MFMA attention kernel (+ merge kernel when the keys are split).
// Prefill: 8 waves per workgroup (two groups that alternate matrix and vector phases on each
// SIMD), one workgroup per CU.
constexpr int kPrefillThreads = 512;
constexpr int kPrefillRowTiles = 2;   // 16-row MFMA tiles per wave

struct PrefillArgs {
    void* out;                     // [num_query_rows][Hq][D], bf16
    const void* query;             // [num_query_rows][Hq][D], bf16
    const int32_t* cu_query_lens;  // [num_seqs + 1]
    const void* k_pool;
    const void* v_pool;
    int64_t num_blocks;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t max_context_len;  // context lengths are clamped to this bound
    int32_t num_seqs;
    int32_t num_query_rows;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t block_size;  // 16 or 32 tokens
    int32_t row_blocks;  // workgroup row blocks per (sequence, kv head)
    int32_t num_splits;  // key ranges per row block
    int32_t split_keys;  // keys per range; 0 = each row block's keys cut into num_splits parts
    float scale_log2;
    const float* k_scale;
    const float* v_scale;
    float* o_part;   // [num_splits][num_query_rows][Hq][D]  unnormalised rows times v_scale
    float* ml_part;  // [num_splits][num_query_rows][Hq][2]  (running max in base 2, softmax sum)
};

hipError_t launch_kv_write(int src_dtype, int cache_dtype, const KvWriteArgs& a, hipStream_t stream);

// Waves per SIMD the streaming kernel of this variant is built for (2 or 3); the persistent
// grid has that many waves per SIMD.
int decode_waves_per_simd(int q_dtype, int cache_dtype, int head_dim, int gqa, bool fused = false);

// phase 1 = streaming kernel, 2 = merge kernel, 3 = both.  Returns hipErrorInvalidValue when
// no kernel exists for the combination.
hipError_t launch_decode(int phase, int q_dtype, int cache_dtype, int head_dim, int gqa,
                         const DecodeArgs& a, hipStream_t stream);

// The streaming kernel's fused-append instances (a.new_key set), one launch.
hipError_t launch_decode_stream_fused(int q_dtype, int cache_dtype, int head_dim, int gqa, const DecodeArgs& a,
                                      hipStream_t stream);

// Per (query dtype, cache dtype) launchers, one translation unit each (decode_<dtype>.hip and
// decode_fused_<dtype>.hip).
hipError_t launch_decode_f32(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_e4m3(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_e5m2(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_i8(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_fused_f32(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_fused_bf16(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_fused_e4m3(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_fused_e5m2(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_fused_i8(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream);

// grid = num_seqs * num_kv_heads * row_blocks * num_splits workgroups.
hipError_t launch_prefill(int cache_dtype, int head_dim, int gqa, const PrefillArgs& a, int64_t grid,
                          hipStream_t stream);

// Measurement helper: num_reads 4 KiB tiles of buf in the order given, grid x 256 threads.
hipError_t launch_tile_read(const void* buf, int64_t buf_tiles, int64_t num_reads, const int32_t* order, int grid,
                            uint32_t* sink, hipStream_t stream);

}  // namespace pa
