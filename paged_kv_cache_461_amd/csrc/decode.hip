// decode.hip -- PagedAttention decode for gfx950: split-K partition kernel + merge kernel.
//
// One workgroup (4 waves) attends one (sequence, kv head, context partition).  The GQA
// group's G query rows are staged once through LDS into registers; every K/V block is read
// from HBM once and reused by all G heads.  Each wave walks every 4th block of the
// partition through the block table (page 1, section 4; page 3, section 2.1: the cache is
// read block by block via the table, never assumed contiguous).
//
// Per 16-token block (layout in include/pagedattn.h) a wave issues NCH K loads and NCH V
// loads of 16 bytes per lane, each one contiguous 1 KiB slice:
//   QK^T: lane l holds channels of token l/4; bf16/fp8 K is multiplied with the bf16 query
//         pairs by v_dot2c_f32_bf16 (fp8 first widened exactly to bf16 pairs), fp32 K with
//         FMAs; the 4 lanes of a token finish the dot product with two DPP quad moves.
//   softmax: online, in base 2.  The running max is wave-uniform and only moved when a score
//         exceeds it by more than 8 (then o and l are rescaled), so most blocks skip the
//         rescale; weights stay below 2^8, and normalisation happens once at the end.
//   PV:   lane l holds channels of the token pair l/8; the pair's two weights come from the
//         quad of the other token by one ds_swizzle, are packed to bf16 and contracted with
//         the pair-interleaved V by v_dot2c_f32_bf16 (fp32 V: FMAs).
// The 4 waves' (m, l, o) are merged through LDS.  A sequence that fits one partition writes
// its output row directly; otherwise the partition's normalised row and (m, l) go to the
// workspace and decode_reduce merges them (flash-decoding split-K).
#include <float.h>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr float kRescaleMargin = 8.0f;  // log2 units: weights are kept <= 2^8

template <int QT, int KT, int D, int G>
struct Shape {
    static constexpr int EB = DtypeBytes<KT>::value;
    static constexpr int W = 64 / EB;      // channels per 64-byte slice
    static constexpr int NCH = D / W;      // 1 KiB slices per (block, kv head) tile
    static constexpr int KE = W / 4;       // K channels per lane per slice
    static constexpr int VE = W / 8;       // V channels per lane per slice (x 2 tokens)
    static constexpr int TILE = kBlockSize * D * EB;
    static constexpr int QB = DtypeBytes<QT>::value;
    static constexpr int QP = (QT == kBF16) ? KE / 2 : 1;  // bf16 query pairs per slice
    static constexpr int QF = (QT == kF32) ? KE : 1;       // fp32 query values per slice
    static_assert(TILE == NCH * 1024, "a tile is a whole number of 1 KiB slices");
    static_assert((QT == kF32) == (KT == kF32), "fp32 queries go with an fp32 cache");
};

template <int QT, int KT, int D, int G>
struct WaveState {
    using S = Shape<QT, KT, D, G>;
    uint32_t qp[S::NCH][S::QP][G];
    float qf[S::NCH][S::QF][G];
    float o[S::NCH][S::VE][G];
    float l[G];
    float m[G];
};

// Partial dot products of this lane's K channels with the G query rows.
template <int QT, int KT, int D, int G>
__device__ __forceinline__ void qk_slice(const WaveState<QT, KT, D, G>& st, int c, const uint4& kv,
                                         float (&acc)[G])
{
    if constexpr (KT == kBF16) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int h = 0; h < G; h++) acc[h] = dot2_bf16(u4_get(kv, i), st.qp[c][i][h], acc[h]);
    } else if constexpr (KT == kFP8) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = u4_get(kv, i);
            const uint32_t lo = e4m3x2_to_bf16x2<false>(w);
            const uint32_t hi = e4m3x2_to_bf16x2<true>(w);
#pragma unroll
            for (int h = 0; h < G; h++) {
                acc[h] = dot2_bf16(lo, st.qp[c][2 * i][h], acc[h]);
                acc[h] = dot2_bf16(hi, st.qp[c][2 * i + 1][h], acc[h]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float k = as_float(u4_get(kv, i));
#pragma unroll
            for (int h = 0; h < G; h++) acc[h] = __builtin_fmaf(k, st.qf[c][i][h], acc[h]);
        }
    }
}

// o += p_even * V[even token] + p_odd * V[odd token] for this lane's V channels.
template <int QT, int KT, int D, int G>
__device__ __forceinline__ void pv_slice(WaveState<QT, KT, D, G>& st, int c, const uint4& vv,
                                         const uint32_t (&pp)[G], const float (&pe)[G],
                                         const float (&po)[G])
{
    if constexpr (KT == kBF16) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int h = 0; h < G; h++) st.o[c][i][h] = dot2_bf16(u4_get(vv, i), pp[h], st.o[c][i][h]);
    } else if constexpr (KT == kFP8) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = u4_get(vv, i);
            const uint32_t lo = e4m3x2_to_bf16x2<false>(w);
            const uint32_t hi = e4m3x2_to_bf16x2<true>(w);
#pragma unroll
            for (int h = 0; h < G; h++) {
                st.o[c][2 * i][h] = dot2_bf16(lo, pp[h], st.o[c][2 * i][h]);
                st.o[c][2 * i + 1][h] = dot2_bf16(hi, pp[h], st.o[c][2 * i + 1][h]);
            }
        }
    } else {
        const float v0 = as_float(vv.x), v1 = as_float(vv.y), v2 = as_float(vv.z), v3 = as_float(vv.w);
#pragma unroll
        for (int h = 0; h < G; h++) {
            st.o[c][0][h] = __builtin_fmaf(po[h], v1, __builtin_fmaf(pe[h], v0, st.o[c][0][h]));
            st.o[c][1][h] = __builtin_fmaf(po[h], v3, __builtin_fmaf(pe[h], v2, st.o[c][1][h]));
        }
    }
}

// Zero the V elements of tokens past the end of the context (they may hold anything,
// including NaN, and 0 * NaN would leak into the sum).
template <int KT>
__device__ __forceinline__ uint4 mask_pair(uint4 v, bool even_ok, bool odd_ok)
{
    uint32_t m;
    if constexpr (KT == kBF16)
        m = (even_ok ? 0x0000FFFFu : 0u) | (odd_ok ? 0xFFFF0000u : 0u);
    else if constexpr (KT == kFP8)
        m = (even_ok ? 0x00FF00FFu : 0u) | (odd_ok ? 0xFF00FF00u : 0u);
    else {
        uint4 r;
        r.x = even_ok ? v.x : 0u;
        r.y = odd_ok ? v.y : 0u;
        r.z = even_ok ? v.z : 0u;
        r.w = odd_ok ? v.w : 0u;
        return r;
    }
    v.x &= m;
    v.y &= m;
    v.z &= m;
    v.w &= m;
    return v;
}

template <int QT, int KT, int D, int G>
__device__ __forceinline__ void attend_block(WaveState<QT, KT, D, G>& st, const uint4 (&kb)[Shape<QT, KT, D, G>::NCH],
                                             const uint4 (&vb)[Shape<QT, KT, D, G>::NCH], int n_valid,
                                             float c2, int lane)
{
    using S = Shape<QT, KT, D, G>;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; h++) acc[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < S::NCH; c++) qk_slice<QT, KT, D, G>(st, c, kb[c], acc);

    const int tok = lane >> 2;  // this lane's token within the block
    float s2[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        s2[h] = quad_sum(acc[h]) * c2;
        if (n_valid < kBlockSize) s2[h] = tok < n_valid ? s2[h] : -__builtin_inff();
    }

    bool need = false;
#pragma unroll
    for (int h = 0; h < G; h++) need |= s2[h] > st.m[h] + kRescaleMargin;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float mn = __builtin_fmaxf(st.m[h], wave_max(s2[h]));
            const float alpha = fast_exp2(st.m[h] - mn);
            st.m[h] = mn;
            st.l[h] *= alpha;
#pragma unroll
            for (int c = 0; c < S::NCH; c++)
#pragma unroll
                for (int i = 0; i < S::VE; i++) st.o[c][i][h] *= alpha;
        }
    }

    const bool odd = (tok & 1) != 0;
    float pe[G], po[G];
    uint32_t pp[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float mine = fast_exp2(s2[h] - st.m[h]);
        const float other = swizzle_xor4(mine);
        pe[h] = odd ? other : mine;
        po[h] = odd ? mine : other;
        if constexpr (KT == kF32) {
            st.l[h] += pe[h] + po[h];
            pp[h] = 0;
        } else {
            pp[h] = pack_bf16x2(pe[h], po[h]);
            st.l[h] = dot2_bf16(pp[h], kBf16OnePair, st.l[h]);
        }
    }

    if (n_valid < kBlockSize) {
        const int pr = lane >> 3;
        const bool even_ok = 2 * pr < n_valid, odd_ok = 2 * pr + 1 < n_valid;
#pragma unroll
        for (int c = 0; c < S::NCH; c++) pv_slice<QT, KT, D, G>(st, c, mask_pair<KT>(vb[c], even_ok, odd_ok), pp, pe, po);
    } else {
#pragma unroll
        for (int c = 0; c < S::NCH; c++) pv_slice<QT, KT, D, G>(st, c, vb[c], pp, pe, po);
    }
}

template <int QT, int KT, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(const DecodeArgs a)
{
    using S = Shape<QT, KT, D, G>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    // blockIdx -> (kv head fastest, then sequence, then partition): consecutive workgroups
    // go to different XCDs, so with 8 kv heads each XCD serves one kv head.
    int bid = blockIdx.x;
    const int Hkv = a.num_kv_heads;
    const int g = bid % Hkv;
    bid /= Hkv;
    const int s = bid % a.num_seqs;
    const int part = bid / a.num_seqs;
    const int ctx = a.context_lens[s];
    const int P = a.partition_size;
    const int t_begin = part * P;
    if (part > 0 && t_begin >= ctx) return;

    __shared__ __align__(16) unsigned char q_lds[G * D * S::QB];
    __shared__ __align__(16) float red_o[kDecodeWaves * 4][G][D];
    __shared__ float red_l[kDecodeWaves * 4][G];
    __shared__ float red_m[kDecodeWaves][G];

    // Stage the GQA group's query rows (contiguous G*D elements) through LDS.
    {
        const uint4* src = reinterpret_cast<const uint4*>(
            static_cast<const unsigned char*>(a.query) + ((int64_t)s * a.num_heads + (int64_t)g * G) * D * S::QB);
        uint4* dst = reinterpret_cast<uint4*>(q_lds);
        for (int i = threadIdx.x; i < G * D * S::QB / 16; i += kDecodeThreads) dst[i] = src[i];
    }
    __syncthreads();

    WaveState<QT, KT, D, G> st;
    {
        const int kp = lane & 3;
#pragma unroll
        for (int c = 0; c < S::NCH; c++) {
#pragma unroll
            for (int h = 0; h < G; h++) {
                const int base = h * D + c * S::W + kp * S::KE;
                if constexpr (QT == kBF16) {
#pragma unroll
                    for (int i = 0; i < S::QP; i++)
                        st.qp[c][i][h] = reinterpret_cast<const uint32_t*>(q_lds)[(base >> 1) + i];
                } else {
#pragma unroll
                    for (int i = 0; i < S::QF; i++) st.qf[c][i][h] = reinterpret_cast<const float*>(q_lds)[base + i];
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            st.m[h] = -FLT_MAX;
            st.l[h] = 0.0f;
#pragma unroll
            for (int c = 0; c < S::NCH; c++)
#pragma unroll
                for (int i = 0; i < S::VE; i++) st.o[c][i][h] = 0.0f;
        }
    }

    const float c2 = a.scale_log2 * (KT == kFP8 ? a.k_scale[g] : 1.0f);
    const int nblk_ctx = ctx > 0 ? (ctx + kBlockSize - 1) / kBlockSize : 0;
    const int blk_begin = t_begin / kBlockSize;
    const int blk_end = min(nblk_ctx, (t_begin + P) / kBlockSize);
    const int nblk = blk_end - blk_begin;
    const int nk = nblk > wave ? (nblk - wave + kDecodeWaves - 1) / kDecodeWaves : 0;

    const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k_pool) + (int64_t)g * S::TILE + lane * 16;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v_pool) + (int64_t)g * S::TILE + lane * 16;
    const int64_t block_stride = (int64_t)Hkv * S::TILE;

    // Blocks of this wave: partition block wave + 4k, k = 0..nk-1.  Lane j of `entry` holds
    // the physical id of k = seg + j.
    for (int seg = 0; seg < nk; seg += 64) {
        const int nseg = min(64, nk - seg);
        const int my_blk = blk_begin + wave + kDecodeWaves * (seg + lane);
        const int entry = (lane < nseg && my_blk < a.max_blocks_per_seq) ? table[my_blk] : -1;

        auto issue = [&](int k, uint4 (&kb)[S::NCH], uint4 (&vb)[S::NCH]) -> bool {
            int phys = __builtin_amdgcn_readlane(entry, k);
            const bool bad = phys < 0 || (int64_t)phys >= a.num_blocks;
            phys = bad ? 0 : phys;
            const unsigned char* kp = kbase + (int64_t)phys * block_stride;
            const unsigned char* vp = vbase + (int64_t)phys * block_stride;
#pragma unroll
            for (int c = 0; c < S::NCH; c++) kb[c] = load16(kp + c * 1024);
#pragma unroll
            for (int c = 0; c < S::NCH; c++) vb[c] = load16(vp + c * 1024);
            return bad;
        };
        auto valid_tokens = [&](int k, bool bad) -> int {
            const int blk = blk_begin + wave + kDecodeWaves * (seg + k);
            return bad ? 0 : min(kBlockSize, ctx - blk * kBlockSize);
        };

        uint4 ka[S::NCH], va[S::NCH], kb2[S::NCH], vb2[S::NCH];
        bool bad_a = issue(0, ka, va), bad_b = false;
        for (int k = 0; k < nseg; k += 2) {
            if (k + 1 < nseg) bad_b = issue(k + 1, kb2, vb2);
            attend_block<QT, KT, D, G>(st, ka, va, valid_tokens(k, bad_a), c2, lane);
            if (k + 1 < nseg) {
                if (k + 2 < nseg) bad_a = issue(k + 2, ka, va);
                attend_block<QT, KT, D, G>(st, kb2, vb2, valid_tokens(k + 1, bad_b), c2, lane);
            }
        }
    }

    // Merge inside the wave: the two token pairs of every 16-lane row.
#pragma unroll
    for (int h = 0; h < G; h++) {
        st.l[h] += dpp_f32<kDppRowRor8>(st.l[h]);
#pragma unroll
        for (int c = 0; c < S::NCH; c++)
#pragma unroll
            for (int i = 0; i < S::VE; i++) st.o[c][i][h] += dpp_f32<kDppRowRor8>(st.o[c][i][h]);
    }
    const int row = lane >> 4;
    if ((lane & 8) == 0) {
        const int vp = lane & 7;
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int c = 0; c < S::NCH; c++)
#pragma unroll
                for (int i = 0; i < S::VE; i++) red_o[wave * 4 + row][h][c * S::W + vp * S::VE + i] = st.o[c][i][h];
    }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int h = 0; h < G; h++) red_l[wave * 4 + row][h] = st.l[h];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; h++) red_m[wave][h] = st.m[h];
    }
    __syncthreads();

    // Merge the 4 waves and write this partition's result.
    // (clamped: a context longer than max_context_len breaks the caller's contract, and
    // must not send the merge past the workspace)
    const int np_seq = min(ctx > 0 ? (ctx + P - 1) / P : 1, a.max_partitions);
    for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
        const int h = idx / D, d = idx % D;
        float M = red_m[0][h];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; w++) M = __builtin_fmaxf(M, red_m[w][h]);
        float acc = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; w++) {
            const float f = fast_exp2(red_m[w][h] - M);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                acc += f * red_o[w * 4 + r][h][d];
                L += f * red_l[w * 4 + r][h];
            }
        }
        const float v = L > 0.0f ? acc / L : 0.0f;
        const int64_t row_id = (int64_t)s * a.num_heads + (int64_t)g * G + h;
        if (np_seq == 1) {
            const float vs = KT == kFP8 ? a.v_scale[g] : 1.0f;
            if constexpr (QT == kBF16)
                static_cast<uint16_t*>(a.out)[row_id * D + d] = f32_to_bf16_bits(v * vs);
            else
                static_cast<float*>(a.out)[row_id * D + d] = v * vs;
        } else {
            const int64_t pi = row_id * a.max_partitions + part;
            a.o_part[pi * D + d] = v;
            if (d == 0) {
                a.m_part[pi] = M;
                a.l_part[pi] = L;
            }
        }
    }
}

// Merge the partitions of one (sequence, query head): weights l_p * 2^(m_p - M).
template <int QT, int KT, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(const DecodeArgs a)
{
    const int row_id = blockIdx.x;  // s * Hq + h
    const int s = row_id / a.num_heads;
    const int ctx = a.context_lens[s];
    const int P = a.partition_size;
    const int np = min(ctx > 0 ? (ctx + P - 1) / P : 1, a.max_partitions);
    if (np <= 1) return;
    const int lane = threadIdx.x;
    const int64_t base = (int64_t)row_id * a.max_partitions;
    float M = -FLT_MAX;
    for (int p = 0; p < np; p++) M = __builtin_fmaxf(M, a.m_part[base + p]);
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; j++) acc[j] = 0.0f;
    float L = 0.0f;
    for (int p = 0; p < np; p++) {
        const float w = a.l_part[base + p] * fast_exp2(a.m_part[base + p] - M);
        L += w;
        const float* op = a.o_part + (base + p) * D;
#pragma unroll
        for (int j = 0; j < PER; j++) acc[j] = __builtin_fmaf(w, op[lane + 64 * j], acc[j]);
    }
    const int g = (row_id % a.num_heads) / (a.num_heads / a.num_kv_heads);
    const float vs = KT == kFP8 ? a.v_scale[g] : 1.0f;
#pragma unroll
    for (int j = 0; j < PER; j++) {
        const float v = L > 0.0f ? acc[j] / L * vs : 0.0f;
        if constexpr (QT == kBF16)
            static_cast<uint16_t*>(a.out)[(int64_t)row_id * D + lane + 64 * j] = f32_to_bf16_bits(v);
        else
            static_cast<float*>(a.out)[(int64_t)row_id * D + lane + 64 * j] = v;
    }
}

template <int QT, int KT, int D, int G>
hipError_t launch_partitions_t(const DecodeArgs& a, hipStream_t stream)
{
    const int64_t grid = (int64_t)a.max_partitions * a.num_seqs * a.num_kv_heads;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_partition_kernel<QT, KT, D, G>), dim3((unsigned)grid), dim3(kDecodeThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int QT, int KT, int D>
hipError_t launch_partitions_g(int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (gqa) {
    case 1: return launch_partitions_t<QT, KT, D, 1>(a, stream);
    case 2: return launch_partitions_t<QT, KT, D, 2>(a, stream);
    case 4: return launch_partitions_t<QT, KT, D, 4>(a, stream);
    case 8: return launch_partitions_t<QT, KT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int QT, int KT>
hipError_t launch_partitions_d(int head_dim, int gqa, const DecodeArgs& a, hipStream_t stream)
{
    switch (head_dim) {
    case 64: return launch_partitions_g<QT, KT, 64>(gqa, a, stream);
    case 128: return launch_partitions_g<QT, KT, 128>(gqa, a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int QT, int KT, int D>
hipError_t launch_reduce_t(const DecodeArgs& a, hipStream_t stream)
{
    const int64_t grid = (int64_t)a.num_seqs * a.num_heads;
    if (grid <= 0 || a.max_partitions <= 1) return hipSuccess;
    hipLaunchKernelGGL((decode_reduce_kernel<QT, KT, D>), dim3((unsigned)grid), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_partitions(int q_dtype, int cache_dtype, int head_dim, int gqa, const DecodeArgs& a,
                                    hipStream_t stream)
{
    if (q_dtype == kF32 && cache_dtype == kF32) return launch_partitions_d<kF32, kF32>(head_dim, gqa, a, stream);
    if (q_dtype == kBF16 && cache_dtype == kBF16) return launch_partitions_d<kBF16, kBF16>(head_dim, gqa, a, stream);
    if (q_dtype == kBF16 && cache_dtype == kFP8) return launch_partitions_d<kBF16, kFP8>(head_dim, gqa, a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_reduce(int q_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream)
{
    // The merge only differs by output dtype, head dim and whether a v_scale applies.
    const bool fp8 = a.v_scale != nullptr;
    if (q_dtype == kF32) {
        if (head_dim == 64) return launch_reduce_t<kF32, kF32, 64>(a, stream);
        if (head_dim == 128) return launch_reduce_t<kF32, kF32, 128>(a, stream);
    } else if (q_dtype == kBF16) {
        if (head_dim == 64) return fp8 ? launch_reduce_t<kBF16, kFP8, 64>(a, stream) : launch_reduce_t<kBF16, kBF16, 64>(a, stream);
        if (head_dim == 128) return fp8 ? launch_reduce_t<kBF16, kFP8, 128>(a, stream) : launch_reduce_t<kBF16, kBF16, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
