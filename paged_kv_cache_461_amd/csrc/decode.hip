// decode.hip -- PagedAttention decode for gfx950: dispatch over the (query dtype, cache dtype)
// pairs, whose launchers are compiled one cache dtype per translation unit (decode_<dtype>.hip,
// from decode_launch.hpp; the fused-append instances are in decode_fused_<dtype>.hip), and the
// occupancy each streaming-kernel variant is built for.
#include "decode_kernel.hpp"

namespace pa {

namespace {
template <int KT, int D, bool FUSED>
int waves_g(int gqa)
{
    switch (gqa) {
    case 1: return stream_waves_per_simd<KT, D, 1, FUSED>();
    case 2: return stream_waves_per_simd<KT, D, 2, FUSED>();
    case 4: return stream_waves_per_simd<KT, D, 4, FUSED>();
    default: return stream_waves_per_simd<KT, D, 8, FUSED>();
    }
}
template <int KT>
int waves_d(int head_dim, int gqa, bool fused)
{
    if (fused) return head_dim == 64 ? waves_g<KT, 64, true>(gqa) : waves_g<KT, 128, true>(gqa);
    return head_dim == 64 ? waves_g<KT, 64, false>(gqa) : waves_g<KT, 128, false>(gqa);
}
}  // namespace

int decode_waves_per_simd(int q_dtype, int cache_dtype, int head_dim, int gqa, bool fused)
{
    (void)q_dtype;  // fp32 queries go with an fp32 cache, bf16 with the others
    switch (cache_dtype) {
    case kF32: return waves_d<kF32>(head_dim, gqa, fused);
    case kBF16: return waves_d<kBF16>(head_dim, gqa, fused);
    case kFP8: return waves_d<kFP8>(head_dim, gqa, fused);
    case kE5M2: return waves_d<kE5M2>(head_dim, gqa, fused);
    case kI8: return waves_d<kI8>(head_dim, gqa, fused);
    default: return 2;
    }
}

hipError_t launch_decode(int phase, int q_dtype, int cache_dtype, int head_dim, int gqa, const DecodeArgs& a,
                         hipStream_t stream)
{
    if (q_dtype == kF32 && cache_dtype == kF32) return launch_decode_f32(phase, head_dim, gqa, a, stream);
    if (q_dtype != kBF16) return hipErrorInvalidValue;
    switch (cache_dtype) {
    case kBF16: return launch_decode_bf16(phase, head_dim, gqa, a, stream);
    case kFP8: return launch_decode_e4m3(phase, head_dim, gqa, a, stream);
    case kE5M2: return launch_decode_e5m2(phase, head_dim, gqa, a, stream);
    case kI8: return launch_decode_i8(phase, head_dim, gqa, a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_stream_fused(int q_dtype, int cache_dtype, int head_dim, int gqa, const DecodeArgs& a,
                                      hipStream_t stream)
{
    if (q_dtype == kF32 && cache_dtype == kF32) return launch_fused_f32(head_dim, gqa, a, stream);
    if (q_dtype != kBF16) return hipErrorInvalidValue;
    switch (cache_dtype) {
    case kBF16: return launch_fused_bf16(head_dim, gqa, a, stream);
    case kFP8: return launch_fused_e4m3(head_dim, gqa, a, stream);
    case kE5M2: return launch_fused_e5m2(head_dim, gqa, a, stream);
    case kI8: return launch_fused_i8(head_dim, gqa, a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
