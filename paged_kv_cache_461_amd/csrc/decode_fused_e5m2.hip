// decode_fused_e5m2.hip -- fused-append decode instances for bf16 queries over an OCP E5M2 cache.
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_fused_e5m2(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_fused_d<kBF16, kE5M2>(head_dim, gqa, a, stream);
}

}  // namespace pa
