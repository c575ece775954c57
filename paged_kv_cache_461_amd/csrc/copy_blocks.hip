// copy_blocks.hip -- copy whole pool blocks (every kv head, K and V): the copy-on-write step
// of the block manager, run before a sequence writes into a block it shared.
//
// Workgroup (pair, pool, part) copies one contiguous share of a block's bytes with 16-byte
// loads and stores; a pair whose ids fall outside the pool is skipped.
#include "pa_copy.hpp"
#include "pa_device.hpp"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyPartBytes = 16384;  // bytes per workgroup (16 per thread x 4 steps)

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(unsigned char* k_pool, unsigned char* v_pool,
                                                                   int64_t num_blocks, int64_t block_bytes,
                                                                   const int32_t* pairs)
{
    const int p = blockIdx.x;
    const int src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || dst < 0 || (int64_t)src >= num_blocks || (int64_t)dst >= num_blocks) return;
    unsigned char* pool = blockIdx.y ? v_pool : k_pool;
    const int64_t begin = (int64_t)blockIdx.z * kCopyPartBytes;
    const int64_t end = begin + kCopyPartBytes < block_bytes ? begin + kCopyPartBytes : block_bytes;
    const unsigned char* s = pool + (int64_t)src * block_bytes;
    unsigned char* d = pool + (int64_t)dst * block_bytes;
    for (int64_t o = begin + (int64_t)threadIdx.x * 16; o < end; o += kCopyThreads * 16)
        *reinterpret_cast<uint4*>(d + o) = load16(s + o);
}

}  // namespace

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks, int64_t block_bytes,
                              const int32_t* pairs, int32_t num_pairs, hipStream_t stream)
{
    if (num_pairs <= 0) return hipSuccess;
    const int64_t parts = (block_bytes + kCopyPartBytes - 1) / kCopyPartBytes;
    if (parts > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, 2, (unsigned)parts), dim3(kCopyThreads), 0,
                       stream, static_cast<unsigned char*>(k_pool), static_cast<unsigned char*>(v_pool), num_blocks,
                       block_bytes, pairs);
    return hipGetLastError();
}

}  // namespace pa
