// decode_fused_i8.hip -- fused-append decode instances for bf16 queries over an INT8 cache.
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_fused_i8(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_fused_d<kBF16, kI8>(head_dim, gqa, a, stream);
}

}  // namespace pa
