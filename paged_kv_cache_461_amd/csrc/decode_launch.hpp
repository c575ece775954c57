// decode_launch.hpp -- the split-K merge kernel of PagedAttention decode and the launchers of
// the streaming kernel (decode_kernel.hpp) for one (query dtype, cache dtype) pair.  Each cache
// dtype's instances are compiled in a translation unit of their own (decode_<dtype>.hip), so
// the units build in parallel.
#pragma once

#include "decode_kernel.hpp"

namespace pa {
namespace {

// Merge the pieces of one run (sequence s, kv head g), one wave per run: output row h =
// sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - M), M = max_p m_p (flash-decoding's
// combination of partial softmax results), times v_scale for an fp8 cache.  Lane p holds
// piece p's (max, sum) for the G heads, so maxima, weights and sums come from one round of
// loads and two wave reductions; each lane then owns D / 64 channels and reads the pieces'
// rows UN at a time (up to 64 loads per lane in flight per round trip).  The kernel is
// latency-bound (a few MB), so the chain of dependent loads is what it is built to keep short:
// context length and run record, then (max, sum), then rows.  Also writes the zero rows of
// empty sequences, which no streaming wave visits.
constexpr int kMergeWaves = 4;  // runs per merge workgroup

template <int QT, int KT, int D, int G>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(const DecodeArgs a)
{
    constexpr int PER = D / 64;
    constexpr int UN = G * PER >= 8 ? 64 / (G * PER) : 8;  // pieces whose rows are loaded together
    const int lane = threadIdx.x & 63;
    // runs are numbered as the streaming kernel lists them: run g S + s
    const int64_t run = (int64_t)blockIdx.x * kMergeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (run >= (int64_t)a.num_seqs * a.num_kv_heads) return;
    const int s = (int)(run % a.num_seqs), g = (int)(run / a.num_seqs);
    const int ctx = seq_ctx(a, s);
    const int64_t k0 = a.run_info[2 * run];
    const int np = a.run_info[2 * run + 1];
    float acc[G][PER];
    float L[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        L[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < PER; j++) acc[h][j] = 0.0f;
    }
    if (ctx > 0) {
        // whole run: written by the streaming kernel (the other checks only reject a workspace
        // the streaming kernel has not filled)
        if (np <= 1 || k0 < 0 || run + k0 + np > a.max_pieces) return;
        const int64_t p0 = run + k0;
        auto load_ml = [&](int base, float (&m)[G], float (&l)[G]) {
            const bool valid = base + lane < np;
            const int64_t p = p0 + (valid ? base + lane : 0);
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float2 v = *reinterpret_cast<const float2*>(a.ml_part + (p * G + h) * 2);
                m[h] = valid ? v.x : -FLT_MAX;
                l[h] = valid ? v.y : 0.0f;
            }
        };
        float m[G], l[G], M[G];
        load_ml(0, m, l);
#pragma unroll
        for (int h = 0; h < G; h++) M[h] = wave_max(m[h]);
        for (int base = 64; base < np; base += 64) {  // more than 64 pieces: small partitions
            float m2[G], l2[G];
            load_ml(base, m2, l2);
#pragma unroll
            for (int h = 0; h < G; h++) M[h] = __builtin_fmaxf(M[h], wave_max(m2[h]));
        }
        for (int base = 0; base < np; base += 64) {
            if (base > 0) load_ml(base, m, l);
            float w[G];
#pragma unroll
            for (int h = 0; h < G; h++) {
                w[h] = l[h] * fast_exp2(m[h] - M[h]);
                L[h] += wave_sum(w[h]);
            }
            const int n = min(64, np - base);
            for (int i = 0; i < n; i += UN) {
                float x[UN][G][PER];
#pragma unroll
                for (int u = 0; u < UN; u++) {
                    const int64_t p = p0 + base + min(i + u, n - 1);  // past the end: re-read, weight 0
#pragma unroll
                    for (int h = 0; h < G; h++)
#pragma unroll
                        for (int j = 0; j < PER; j++) x[u][h][j] = a.o_part[(p * G + h) * D + lane + 64 * j];
                }
#pragma unroll
                for (int u = 0; u < UN; u++) {
                    const bool in = i + u < n;
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        const float wt = in ? as_float(__builtin_amdgcn_readlane(as_uint(w[h]), min(i + u, 63))) : 0.0f;
#pragma unroll
                        for (int j = 0; j < PER; j++) acc[h][j] = __builtin_fmaf(wt, x[u][h][j], acc[h][j]);
                    }
                }
            }
        }
    }
    const float vs = kIsQuant<KT> ? a.v_scale[g] : 1.0f;
#pragma unroll
    for (int h = 0; h < G; h++) {
        const int64_t row = (int64_t)s * a.num_heads + (int64_t)g * G + h;
#pragma unroll
        for (int j = 0; j < PER; j++) {
            const float v = L[h] > 0.0f ? acc[h][j] / L[h] * vs : 0.0f;
            if constexpr (QT == kBF16)
                static_cast<uint16_t*>(a.out)[row * D + lane + 64 * j] = f32_to_bf16_bits(v);
            else
                static_cast<float*>(a.out)[row * D + lane + 64 * j] = v;
        }
    }
}

template <int QT, int KT, int D, int G>
hipError_t launch_phase_t(int phase, const DecodeArgs& a, hipStream_t stream)
{
    if ((phase & 1) && a.grid_workgroups > 0) {
        const dim3 grid((unsigned)a.grid_workgroups), block(kDecodeThreads);
        const size_t lds = (size_t)a.num_seqs * sizeof(int) * (a.shared_blocks ? 2 : 1);
        hipError_t e = hipSuccess;
        if (a.new_key != nullptr)
            e = launch_decode_stream_fused(QT, KT, D, G, a, stream);
        else if (a.chunk_blocks < 0)  // short contexts: the shared-block hint is not used
            hipLaunchKernelGGL((decode_stream_kernel<QT, KT, D, G, true, false>), grid, block, lds, stream, a);
        else if (a.shared_blocks != nullptr)
            hipLaunchKernelGGL((decode_stream_kernel<QT, KT, D, G, false, false, true>), grid, block, lds, stream, a);
        else
            hipLaunchKernelGGL((decode_stream_kernel<QT, KT, D, G, false, false>), grid, block, lds, stream, a);
        if (e == hipSuccess) e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((phase & 2) && a.chunk_blocks >= 0) {  // one chunk per run: nothing to merge
        const int64_t grid = ((int64_t)a.num_seqs * a.num_kv_heads + kMergeWaves - 1) / kMergeWaves;
        if (grid <= 0) return hipSuccess;
        if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL((decode_merge_kernel<QT, KT, D, G>), dim3((unsigned)grid), dim3(64 * kMergeWaves), 0,
                           stream, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int QT, int KT, int D>
hipError_t launch_g(int phase, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (gqa) {
    case 1: return launch_phase_t<QT, KT, D, 1>(phase, a, stream);
    case 2: return launch_phase_t<QT, KT, D, 2>(phase, a, stream);
    case 4: return launch_phase_t<QT, KT, D, 4>(phase, a, stream);
    case 8: return launch_phase_t<QT, KT, D, 8>(phase, a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int QT, int KT>
hipError_t launch_d(int phase, int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (head_dim) {
    case 64: return launch_g<QT, KT, 64>(phase, gqa, a, stream);
    case 128: return launch_g<QT, KT, 128>(phase, gqa, a, stream);
    default: return hipErrorInvalidValue;
    }
}

// ---- fused-append instances (the kernel stores each sequence's new token and attends it in
// the same launch) -----------------------------------------------------------------------------

template <int QT, int KT, int D, int G>
hipError_t launch_fused_t(const DecodeArgs& a, hipStream_t stream)
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
hipError_t launch_fused_g(int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (gqa) {
    case 1: return launch_fused_t<QT, KT, D, 1>(a, stream);
    case 2: return launch_fused_t<QT, KT, D, 2>(a, stream);
    case 4: return launch_fused_t<QT, KT, D, 4>(a, stream);
    case 8: return launch_fused_t<QT, KT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int QT, int KT>
hipError_t launch_fused_d(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (head_dim) {
    case 64: return launch_fused_g<QT, KT, 64>(gqa, a, stream);
    case 128: return launch_fused_g<QT, KT, 128>(gqa, a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace pa
