// decode_fused_e4m3.hip -- fused-append decode instances for bf16 queries over an OCP E4M3 cache.
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_fused_e4m3(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_fused_d<kBF16, kFP8>(head_dim, gqa, a, stream);
}

}  // namespace pa
