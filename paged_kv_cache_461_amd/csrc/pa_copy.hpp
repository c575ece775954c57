// pa_copy.hpp -- launcher of the block-copy kernel (copy-on-write of shared blocks).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// For each pair i: pool block pairs[2i] -> block pairs[2i+1] (block_bytes each), in both pools.
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks, int64_t block_bytes,
                              const int32_t* pairs, int32_t num_pairs, hipStream_t stream);

}  // namespace pa
