// decode_fused.hip -- the fused-append instances of the decode streaming kernel
// (decode_kernel.hpp): the kernel stores each sequence's new token and attends it in the same
// launch.  Compiled apart from decode.hip so that the two build in parallel.
#include "decode_kernel.hpp"

namespace pa {
namespace {

template <int QT, int KT, int D, int G>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)a.grid_workgroups), block(kDecodeThreads);
    const size_t lds = (size_t)a.num_seqs * sizeof(int) * (a.shared_blocks ? 2 : 1);
    if (a.chunk_blocks < 0)
        hipLaunchKernelGGL((decode_stream_kernel<QT, KT, D, G, true, true>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((decode_stream_kernel<QT, KT, D, G, false, true>), grid, block, lds, stream, a);
    return hipGetLastError();
}

template <int QT, int KT, int D>
hipError_t launch_g(int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (gqa) {
    case 1: return launch_t<QT, KT, D, 1>(a, stream);
    case 2: return launch_t<QT, KT, D, 2>(a, stream);
    case 4: return launch_t<QT, KT, D, 4>(a, stream);
    case 8: return launch_t<QT, KT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int QT, int KT>
hipError_t launch_d(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (head_dim) {
    case 64: return launch_g<QT, KT, 64>(gqa, a, stream);
    case 128: return launch_g<QT, KT, 128>(gqa, a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_stream_fused(int q_dtype, int cache_dtype, int head_dim, int gqa, const DecodeArgs& a,
                                      hipStream_t stream)
{
    if (q_dtype == kF32 && cache_dtype == kF32) return launch_d<kF32, kF32>(head_dim, gqa, a, stream);
    if (q_dtype == kBF16 && cache_dtype == kBF16) return launch_d<kBF16, kBF16>(head_dim, gqa, a, stream);
    if (q_dtype == kBF16 && cache_dtype == kFP8) return launch_d<kBF16, kFP8>(head_dim, gqa, a, stream);
    if (q_dtype == kBF16 && cache_dtype == kE5M2) return launch_d<kBF16, kE5M2>(head_dim, gqa, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
