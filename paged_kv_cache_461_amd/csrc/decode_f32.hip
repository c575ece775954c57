// decode_f32.hip -- decode instances for fp32 queries over an fp32 cache (streaming and merge kernels).
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_decode_f32(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_d<kF32, kF32>(phase, head_dim, gqa, a, stream);
}

}  // namespace pa
