// decode_bf16.hip -- decode instances for bf16 queries over a bf16 cache (streaming and merge kernels).
#include "decode_launch.hpp"

namespace pa {

hipError_t launch_decode_bf16(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    return launch_d<kBF16, kBF16>(phase, head_dim, gqa, a, stream);
}

}  // namespace pa
