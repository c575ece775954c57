// decode_e4m3.hip -- decode instances for bf16 queries over an OCP E4M3 cache (streaming and merge kernels).
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_decode_e4m3(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_d<kBF16, kFP8>(phase, head_dim, gqa, a, stream);
}

}  // namespace pa
