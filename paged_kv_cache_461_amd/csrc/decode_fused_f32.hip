// decode_fused_f32.hip -- fused-append decode instances for fp32 queries over an fp32 cache.
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_fused_f32(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_fused_d<kF32, kF32>(head_dim, gqa, a, stream);
}

}  // namespace pa
