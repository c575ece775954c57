// pa_internal.hpp -- argument blocks and launchers shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;      // tokens per KV block handled by the kernels
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

struct DecodeArgs {
    void* out;
    const void* query;
    const void* k_pool;
    const void* v_pool;
    int64_t num_blocks;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    float scale_log2;  // softmax scale times log2(e): scores are kept in base 2
    const float* k_scale;
    const float* v_scale;
    int32_t partition_size;  // tokens per partition (multiple of kBlockSize)
    int32_t max_partitions;  // partitions of the longest sequence
    float* o_part;           // [S][Hq][max_partitions][D]  normalised partial rows
    float* m_part;           // [S][Hq][max_partitions]     running max (base 2)
    float* l_part;           // [S][Hq][max_partitions]     softmax denominator
};

hipError_t launch_kv_write(int src_dtype, int cache_dtype, const KvWriteArgs& a, hipStream_t stream);

// Returns hipErrorInvalidValue when no kernel exists for the combination.
hipError_t launch_decode_partitions(int q_dtype, int cache_dtype, int head_dim, int gqa,
                                    const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_reduce(int q_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream);

}  // namespace pa
