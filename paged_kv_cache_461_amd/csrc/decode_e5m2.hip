// decode_e5m2.hip -- decode instances for bf16 queries over an OCP E5M2 cache (streaming and merge kernels).
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_decode_e5m2(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_d<kBF16, kE5M2>(phase, head_dim, gqa, a, stream);
}

}  // namespace pa
