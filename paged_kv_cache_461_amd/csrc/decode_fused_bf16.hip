// decode_fused_bf16.hip -- fused-append decode instances for bf16 queries over a bf16 cache.
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_fused_bf16(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_fused_d<kBF16, kBF16>(head_dim, gqa, a, stream);
}

}  // namespace pa
