// decode_kernel.hpp -- PagedAttention decode for gfx950: the balanced streaming kernel.
//
// Included by decode.hip (the plain instances, the merge kernel and the launchers) and by
// decode_fused.hip (the fused-append instances), which compile in parallel.
//
// The attention of one decode query over its sequence's cache is softmax(q K^T * scale) V
// (page 1, section 2), read block by block through the sequence's block table (page 1,
// section 4; page 3, section 2.1), with the G query heads of a GQA group sharing one KV head
// (page 1, section 10).
//
// Work decomposition.  The K/V blocks of every (sequence, kv head) pair -- a "run" -- are
// laid end to end, kv head by kv head and in sequence order within a kv head, into one list of
// U units (one unit = one 16-token block of one kv head); run (s, g) is run number g S + s.
// The list is cut into chunks of C units and the waves of a persistent grid take one chunk
// each, or chunks w, w + NW, ... for a caller-given size (by default C = ceil(U / NW): one chunk
// per wave, so every wave moves the same number of bytes and the kernel has no tail).  Chunk k
// runs on XCD k mod 8; with the shared-block hint the chunks are dealt to the XCDs in 8
// contiguous ranges instead, so the sharers of a prefix block of one kv head (whose runs lie in
// one stretch of the list) read it through one L2.
// A chunk that covers runs r1..r2 attends each covered piece of a run on its own (online
// softmax state reset per piece) and stores the piece's normalised row and (max, sum) as a
// partial result; a run covered by one piece writes its output row directly.  The merge
// kernel combines the pieces of every split run (flash-decoding split-K).  Piece ids are
// run + chunk, which is one-to-one over non-empty pieces (a later run can only meet a later
// chunk), so the workspace size depends only on the numbers of runs and chunks.
//
// Inside a wave, per 16-token block (pool layout in include/pagedattn.h), the K loads read one
// contiguous 1 KiB slice each and the V loads whole 16-channel tiles or 1 KiB slices, with the
// nontemporal hint (every K/V byte is read once per launch).
//   bf16 and 8-bit caches (the matrix-core form, described beside attend_mfma): S^T = K Q^T and
//     O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x16_bf16 with the GQA heads as
//     the tile columns, an 8-bit cache widened exactly to bf16 first, the online softmax on the
//     accumulator, whose lanes already hold the next product's weights.
//   fp32 caches (the vector form): lane l holds channels of token l/4, multiplied with the query
//     (in LDS) by FMAs and finished with two DPP quad moves; the weights are read into scalar
//     registers and each V load gives every lane one channel of 4 consecutive tokens.
//   softmax: online, in base 2.  The running max only moves when a score exceeds it by more than
//     8 (then o and l are rescaled), so most blocks skip the rescale; weights stay below 2^8, and
//     normalisation happens once per piece.
// An NST-deep ring of register buffers keeps NST-1 blocks of K and V in flight while one is
// attended; all loop bounds are wave-uniform, so the waits on the ring stay counted.  Results of
// pieces that end inside a chunk wait in LDS until the chunk's last unit (deferred stores).
#pragma once

#include <float.h>

#include <type_traits>

#include "kv_store.hpp"
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
    static constexpr int TPC = 16 / EB;    // V: tokens of one channel per 16-byte piece
    static constexpr int NQ = kUnitTokens / TPC;  // V: token groups per unit
    static constexpr int CG = D / 64;      // V: 64-channel groups (one channel per lane)
    static constexpr int TILE = kUnitTokens * D * EB;  // bytes of one unit (16 tokens, one kv head)
    static constexpr int QB = DtypeBytes<QT>::value;
    static constexpr int QBYTES = G * D * QB;  // one GQA group's query rows
    static_assert(TILE == NCH * 1024, "a tile is a whole number of 1 KiB slices");
    static_assert(NQ * CG == NCH, "V: one 1 KiB load per (token group, channel group)");
    static_assert((QT == kF32) == (KT == kF32), "fp32 queries go with an fp32 cache");
    static_assert(QBYTES % 16 == 0, "query staging in whole 16-byte pieces");
};

template <int QT, int KT, int D, int G>
struct Acc {
    using S = Shape<QT, KT, D, G>;
    float o[S::CG][G];  // channel cg * 64 + lane
    float l[G];
    float m[G];
};

// The lane's query channels for every slice: the 16 (fp8 cache: 32) bytes of each (slice c,
// head h) that meet this lane's K elements.  Held in VGPRs for the whole piece.
template <int QT, int KT, int D, int G>
struct QRegs {
    using S = Shape<QT, KT, D, G>;
    static constexpr int NQW = kIsQuant<KT> ? 8 : 4;  // dwords per (slice, head)
    uint32_t w[S::NCH][G][NQW];
};

template <int QT, int KT, int D, int G>
__device__ __forceinline__ void load_q(QRegs<QT, KT, D, G>& q, const unsigned char* qrow, int kp)
{
    using S = Shape<QT, KT, D, G>;
#pragma unroll
    for (int c = 0; c < S::NCH; c++)
#pragma unroll
        for (int h = 0; h < G; h++) {
            const unsigned char* src = qrow + (h * D + c * S::W + kp * S::KE) * S::QB;
#pragma unroll
            for (int i = 0; i < QRegs<QT, KT, D, G>::NQW; i += 4) {
                const uint4 v = load16(src + i * 4);
                q.w[c][h][i] = v.x;
                q.w[c][h][i + 1] = v.y;
                q.w[c][h][i + 2] = v.z;
                q.w[c][h][i + 3] = v.w;
            }
        }
}

// The query kept in the wave's LDS copy instead: the same dwords are read per slice as
// they are needed.  The copy's LDS offset is made opaque to the compiler once per block --
// otherwise the loop-invariant reads are hoisted back into VGPRs -- with an empty asm on a
// scalar register, which (unlike a volatile access) adds no memory wait that would drain the
// K/V ring.
struct QLds {
    const unsigned char* base;
    int off;
};

__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+s"(x));
    return x;
}

template <int QT, int KT, int D, int G>
__device__ __forceinline__ void q_dwords(const QRegs<QT, KT, D, G>& q, int c, int h, int kp, uint32_t (&qw)[QRegs<QT, KT, D, G>::NQW])
{
#pragma unroll
    for (int i = 0; i < QRegs<QT, KT, D, G>::NQW; i++) qw[i] = q.w[c][h][i];
    (void)kp;
}

template <int QT, int KT, int D, int G>
__device__ __forceinline__ void q_dwords(const QLds& q, int c, int h, int kp, uint32_t (&qw)[QRegs<QT, KT, D, G>::NQW])
{
    using S = Shape<QT, KT, D, G>;
    const unsigned char* p = q.base + q.off + (h * D + c * S::W + kp * S::KE) * S::QB;
#pragma unroll
    for (int i = 0; i < QRegs<QT, KT, D, G>::NQW; i += 4) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p + i * 4);
        qw[i] = v.x;
        qw[i + 1] = v.y;
        qw[i + 2] = v.z;
        qw[i + 3] = v.w;
    }
}

// Partial dot products of this lane's K channels with the G query rows.
template <int QT, int KT, int D, int G, class QSrc>
__device__ __forceinline__ void qk_slice(const QSrc& q, int kp, int c, const uint4& kv, float (&acc)[G])
{
#pragma unroll
    for (int h = 0; h < G; h++) {
        uint32_t qw[QRegs<QT, KT, D, G>::NQW];
        q_dwords<QT, KT, D, G>(q, c, h, kp, qw);
        if constexpr (KT == kBF16) {
            acc[h] = dot2_bf16(kv.x, qw[0], acc[h]);
            acc[h] = dot2_bf16(kv.y, qw[1], acc[h]);
            acc[h] = dot2_bf16(kv.z, qw[2], acc[h]);
            acc[h] = dot2_bf16(kv.w, qw[3], acc[h]);
        } else if constexpr (kIsQuant<KT>) {
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, false>(kv.x), qw[0], acc[h]);
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, true>(kv.x), qw[1], acc[h]);
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, false>(kv.y), qw[2], acc[h]);
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, true>(kv.y), qw[3], acc[h]);
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, false>(kv.z), qw[4], acc[h]);
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, true>(kv.z), qw[5], acc[h]);
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, false>(kv.w), qw[6], acc[h]);
            acc[h] = dot2_bf16(q8x2_to_bf16x2<KT, true>(kv.w), qw[7], acc[h]);
        } else {
            acc[h] = __builtin_fmaf(as_float(kv.x), as_float(qw[0]), acc[h]);
            acc[h] = __builtin_fmaf(as_float(kv.y), as_float(qw[1]), acc[h]);
            acc[h] = __builtin_fmaf(as_float(kv.z), as_float(qw[2]), acc[h]);
            acc[h] = __builtin_fmaf(as_float(kv.w), as_float(qw[3]), acc[h]);
        }
    }
}

// o[cg] += sum over the TPC tokens of V load c of p[token] * V[token][channel]: the weights
// are wave-uniform (scalar registers), each lane owns one channel.  bf16 / fp8 weights come
// as bf16 pairs (tokens 2i, 2i+1) and meet V pairs of the same tokens in v_dot2c_f32_bf16;
// fp32 uses one FMA per token.
template <int QT, int KT, int D, int G>
__device__ __forceinline__ void pv_load(Acc<QT, KT, D, G>& st, int c, const uint4& vv, const uint32_t (&pps)[G][8],
                                        const float (&ps)[G][16])
{
    using S = Shape<QT, KT, D, G>;
    const int q = c / S::CG, cg = c % S::CG;
    if constexpr (KT == kBF16) {
#pragma unroll
        for (int h = 0; h < G; h++) {
            st.o[cg][h] = dot2_bf16(vv.x, pps[h][q * 4 + 0], st.o[cg][h]);
            st.o[cg][h] = dot2_bf16(vv.y, pps[h][q * 4 + 1], st.o[cg][h]);
            st.o[cg][h] = dot2_bf16(vv.z, pps[h][q * 4 + 2], st.o[cg][h]);
            st.o[cg][h] = dot2_bf16(vv.w, pps[h][q * 4 + 3], st.o[cg][h]);
        }
    } else if constexpr (kIsQuant<KT>) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = u4_get(vv, i);
            const uint32_t lo = q8x2_to_bf16x2<KT, false>(w);
            const uint32_t hi = q8x2_to_bf16x2<KT, true>(w);
#pragma unroll
            for (int h = 0; h < G; h++) {
                st.o[cg][h] = dot2_bf16(lo, pps[h][2 * i], st.o[cg][h]);
                st.o[cg][h] = dot2_bf16(hi, pps[h][2 * i + 1], st.o[cg][h]);
            }
        }
    } else {
#pragma unroll
        for (int h = 0; h < G; h++) {
            st.o[cg][h] = __builtin_fmaf(ps[h][q * 4 + 0], as_float(vv.x), st.o[cg][h]);
            st.o[cg][h] = __builtin_fmaf(ps[h][q * 4 + 1], as_float(vv.y), st.o[cg][h]);
            st.o[cg][h] = __builtin_fmaf(ps[h][q * 4 + 2], as_float(vv.z), st.o[cg][h]);
            st.o[cg][h] = __builtin_fmaf(ps[h][q * 4 + 3], as_float(vv.w), st.o[cg][h]);
        }
    }
}

// Zero the V elements of tokens at or past n_valid in V load c (they may hold anything,
// including NaN, and 0 * NaN would leak into the sum).
template <int QT, int KT, int D, int G>
__device__ __forceinline__ uint4 mask_tail(uint4 v, int c, int n_valid)
{
    using S = Shape<QT, KT, D, G>;
    constexpr int EPD = 4 / S::EB;  // elements (tokens) per dword
    const int t0 = (c / S::CG) * S::TPC;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < EPD; e++)
            if (t0 + i * EPD + e < n_valid) m |= (EPD == 1 ? 0xFFFFFFFFu : ((1u << (32 / EPD)) - 1u) << (e * 32 / EPD));
        w[i] &= m;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int QT, int KT, int D, int G, class QSrc>
__device__ __forceinline__ void attend_block(Acc<QT, KT, D, G>& st, const QSrc& q,
                                             const uint4 (&kb)[Shape<QT, KT, D, G>::NCH],
                                             const uint4 (&vb)[Shape<QT, KT, D, G>::NCH], int n_valid, float c2,
                                             int lane)
{
    using S = Shape<QT, KT, D, G>;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; h++) acc[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < S::NCH; c++) qk_slice<QT, KT, D, G>(q, lane & 3, c, kb[c], acc);

    const int tok = lane >> 2;  // this lane's token within the block
    float s2[G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        s2[h] = quad_sum(acc[h]) * c2;
        if (n_valid < kUnitTokens) s2[h] = tok < n_valid ? s2[h] : -__builtin_inff();
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
            for (int cg = 0; cg < S::CG; cg++) st.o[cg][h] *= alpha;
        }
    }

    const bool odd = (tok & 1) != 0;
    uint32_t pps[G][8];  // bf16 weight pairs of tokens (2i, 2i+1), wave-uniform
    float ps[G][16];     // fp32 weight of token t, wave-uniform
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float mine = fast_exp2(s2[h] - st.m[h]);
        const float other = swizzle_xor4(mine);  // weight of the other token of the pair
        // l gathers each pair's weights once per lane; the 8 lanes of a pair are folded at
        // the end of the piece
        if constexpr (KT == kF32) {
            st.l[h] += mine + other;
#pragma unroll
            for (int t = 0; t < kUnitTokens; t++) ps[h][t] = as_float(__builtin_amdgcn_readlane(as_uint(mine), 4 * t));
        } else {
            const uint32_t pp = pack_bf16x2(odd ? other : mine, odd ? mine : other);
            st.l[h] = dot2_bf16(pp, kBf16OnePair, st.l[h]);
#pragma unroll
            for (int i = 0; i < 8; i++) pps[h][i] = __builtin_amdgcn_readlane(pp, 8 * i);
        }
    }

    if (n_valid < kUnitTokens) {
#pragma unroll
        for (int c = 0; c < S::NCH; c++) pv_load<QT, KT, D, G>(st, c, mask_tail<QT, KT, D, G>(vb[c], c, n_valid), pps, ps);
    } else {
#pragma unroll
        for (int c = 0; c < S::NCH; c++) pv_load<QT, KT, D, G>(st, c, vb[c], pps, ps);
    }
}

// ---- the matrix-core form (bf16 and 8-bit caches) ----------------------------------------
//
// Per 16-token unit, with the GQA group's G heads as the columns of 16 x 16 MFMA tiles
// (columns G..15 repeat them and are never read):
//   S^T (16 tokens x 16 heads) = K Q^T in D/32 steps of v_mfma_f32_16x16x32_bf16: A = K, lane l
//     holding token l % 16 and 8 channels (an 8-bit cache: a 16-byte piece of 16 channels,
//     widened exactly to bf16, feeds two steps); B = the query, lane l holding head l % 16 and
//     the same channels, in VGPRs for the piece.
//   Softmax on the accumulator: lane l holds the scores of head l % 16 for tokens
//     4 (l / 16) .. + 3, which -- rounded to bf16 -- is the B operand of the next product, so
//     the weights never leave the lane.  The running max of a head is the same in its 4 lanes.
//   O^T (16 channels x 16 heads) += V^T P^T in D/16 tiles of v_mfma_f32_16x16x16_bf16: A = V,
//     lane l holding channel l % 16 of the tile and tokens 4 (l / 16) .. + 3 (8 bytes of bf16,
//     4 bytes of an 8-bit cache: one load per tile, read straight from the pool layout).
// The accumulator of lane l holds head l % 16, channels 16 t + 4 (l / 16) .. + 3 of tile t.
typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef short mf_s16x4 __attribute__((ext_vector_type(4)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));

template <int QT, int KT, int D, int G>
struct MShape {
    static constexpr int EB = DtypeBytes<KT>::value;
    static constexpr int NCH = D * EB / 64;  // 1 KiB K slices per unit
    static constexpr int KS = D / 32;        // S^T steps
    static constexpr int NT = D / 16;        // O^T tiles
    using VP = std::conditional_t<EB == 2, uint2, uint32_t>;  // a lane's V piece of one tile
    static_assert(QT == kBF16 && (EB == 2 || EB == 1), "bf16 queries over a bf16 or 8-bit cache");
    static_assert(G <= 16, "the GQA group fits the 16 columns of a tile");
};

template <int QT, int KT, int D, int G>
struct MQ {
    mf_bf16x8 w[MShape<QT, KT, D, G>::KS];
};

template <int QT, int KT, int D, int G>
struct MAcc {
    mf_f32x4 o[MShape<QT, KT, D, G>::NT];
    float m, l;  // of head lane % 16
};

// Channel c of step st for lane group grp (lanes 16 grp .. 16 grp + 15), element e: the
// channels that lane's K piece holds (a bf16 slice is 32 channels, 8 per lane group; an 8-bit
// slice 64, 16 per lane group, split over two steps).
template <int EB>
__device__ __forceinline__ int mf_channel(int st, int grp)
{
    return EB == 2 ? st * 32 + 8 * grp : (st >> 1) * 64 + 16 * grp + 8 * (st & 1);
}

// Columns G..15 of the tile repeat heads 0..G-1 (lane l loads head (l % 16) mod G): a product
// column depends on its own B column only, so they cost nothing but are never read, and the
// loaded values go straight into the operand -- a select on them would make the wave wait for
// the load at once, and with it for every K/V load in flight.
template <int QT, int KT, int D, int G>
__device__ __forceinline__ void load_q_mf(MQ<QT, KT, D, G>& q, const unsigned char* qrow, int lane)
{
    using M = MShape<QT, KT, D, G>;
    const int hh = (lane & 15) % G, grp = lane >> 4;
#pragma unroll
    for (int st = 0; st < M::KS; st++)
        q.w[st] = __builtin_bit_cast(mf_bf16x8, load16(qrow + (hh * D + mf_channel<M::EB>(st, grp)) * 2));
}

// One step of a sum (sum_or_max = false) or max over the four 16-lane groups holding one
// head: v_permlane16_swap pairs each 16-lane row with its neighbour, v_permlane32_swap each
// half of the wave with the other.
__device__ __forceinline__ float mf_swap(float x, bool halves, bool is_max)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto p = halves ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                          : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t p0 = p[0], p1 = p[1];  // (a bit_cast of the vector elements themselves reads
                                          // element 0 twice with this compiler)
    const float a = __builtin_bit_cast(float, p0), b = __builtin_bit_cast(float, p1);
    return is_max ? __builtin_fmaxf(a, b) : a + b;
}

// Four bf16 (or four 8-bit codes widened to bf16) of lane's V piece.
template <int KT>
__device__ __forceinline__ uint2 mf_v_operand(const typename MShape<kBF16, KT, 64, 1>::VP& v)
{
    if constexpr (DtypeBytes<KT>::value == 2)
        return v;
    else
        return make_uint2(q8x2_to_bf16x2<KT, false>(v), q8x2_to_bf16x2<KT, true>(v));
}

template <int QT, int KT, int D, int G>
__device__ __forceinline__ void attend_mfma(MAcc<QT, KT, D, G>& st, const MQ<QT, KT, D, G>& q,
                                            const uint4 (&kb)[MShape<QT, KT, D, G>::NCH],
                                            const typename MShape<QT, KT, D, G>::VP (&vb)[MShape<QT, KT, D, G>::NT],
                                            int n_valid, float c2, int lane)
{
    using M = MShape<QT, KT, D, G>;
    mf_f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < M::NCH; c++) {
        if constexpr (M::EB == 2) {
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, kb[c]), q.w[c], sacc, 0, 0, 0);
        } else {
            const uint4 k = kb[c];
            const uint4 lo = make_uint4(q8x2_to_bf16x2<KT, false>(k.x), q8x2_to_bf16x2<KT, true>(k.x),
                                        q8x2_to_bf16x2<KT, false>(k.y), q8x2_to_bf16x2<KT, true>(k.y));
            const uint4 hi = make_uint4(q8x2_to_bf16x2<KT, false>(k.z), q8x2_to_bf16x2<KT, true>(k.z),
                                        q8x2_to_bf16x2<KT, false>(k.w), q8x2_to_bf16x2<KT, true>(k.w));
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, lo), q.w[2 * c], sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, hi), q.w[2 * c + 1], sacc, 0, 0, 0);
        }
    }
    const int tb = 4 * (lane >> 4);  // this lane's first token
    float s2[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};
#pragma unroll
    for (int r = 0; r < 4; r++) {
        s2[r] *= c2;
        if (__builtin_amdgcn_readfirstlane(n_valid) < kUnitTokens) s2[r] = tb + r < n_valid ? s2[r] : -__builtin_inff();
    }
    bool need = false;
#pragma unroll
    for (int r = 0; r < 4; r++) need |= s2[r] > st.m + kRescaleMargin;
    if (__builtin_amdgcn_ballot_w64(need && (lane & 15) < G) != 0) {
        float mx = __builtin_fmaxf(__builtin_fmaxf(s2[0], s2[1]), __builtin_fmaxf(s2[2], s2[3]));
        mx = mf_swap(mx, false, true);
        mx = mf_swap(mx, true, true);
        const float mn = __builtin_fmaxf(st.m, mx);
        const float alpha = fast_exp2(st.m - mn);
        st.m = mn;
        st.l *= alpha;
#pragma unroll
        for (int t = 0; t < M::NT; t++) st.o[t] *= alpha;
    }
    const uint32_t pp0 = pack_bf16x2(fast_exp2(s2[0] - st.m), fast_exp2(s2[1] - st.m));
    const uint32_t pp1 = pack_bf16x2(fast_exp2(s2[2] - st.m), fast_exp2(s2[3] - st.m));
    // l sums the weights as rounded for the product (each lane its 4 tokens; the 4 lane
    // groups of a head are folded at the end of the piece)
    st.l = dot2_bf16(pp0, kBf16OnePair, st.l);
    st.l = dot2_bf16(pp1, kBf16OnePair, st.l);
    const mf_s16x4 pb = __builtin_bit_cast(mf_s16x4, make_uint2(pp0, pp1));
    // V elements of tokens at or past n_valid are zeroed: in a ragged unit they may hold anything,
    // including NaN, and 0 * NaN would leak into the sum.  The lane's tokens tb..tb+3 are the four
    // bf16 of its operand; the masks are worked out once per unit, and only for a ragged one.
    uint32_t kx = 0xFFFFFFFFu, ky = 0xFFFFFFFFu;
    if (__builtin_amdgcn_readfirstlane(n_valid) < kUnitTokens) {
        const int keep = n_valid - tb;
        kx = keep >= 2 ? 0xFFFFFFFFu : keep == 1 ? 0xFFFFu : 0u;
        ky = keep >= 4 ? 0xFFFFFFFFu : keep == 3 ? 0xFFFFu : 0u;
    }
#pragma unroll
    for (int t = 0; t < M::NT; t++) {
        uint2 av = mf_v_operand<KT>(vb[t]);
        av.x &= kx;
        av.y &= ky;
        st.o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mf_s16x4, av), pb, st.o[t], 0, 0, 0);
    }
}

// ---- work-list arithmetic ---------------------------------------------------------------

// Context length the kernels use for sequence s: clamped to [0, max_context_len], so a
// length beyond the caller's bound can never send a table read or a workspace write out of
// range (the caller's contract is context_lens[s] <= max_context_len).
__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int c)
{
    return c < 0 ? 0 : (c > a.max_context_len ? a.max_context_len : c);
}

__device__ __forceinline__ int seq_ctx(const DecodeArgs& a, int s) { return clamp_ctx(a, a.context_lens[s]); }

// Tokens per work unit, as a shift: 16, or 8 for 8-token blocks (one block per unit, the unit's
// upper half empty).
__device__ __forceinline__ int unit_shift(int block_size) { return block_size < kUnitTokens ? 3 : 4; }
__device__ __forceinline__ int nunits(int ctx, int ush) { return (ctx + (1 << ush) - 1) >> ush; }

__device__ __forceinline__ int wave_incl_scan(int x, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        x += lane >= d ? y : 0;
    }
    return x;
}

constexpr int kScanPerLane = 16;  // sequences per lane in one pass over the context lengths
constexpr int kScanWindow = 64 * kScanPerLane;

struct Pos {
    int s, g, j;        // run (sequence s, kv head g), block j of the run
    int64_t run_start;  // unit index of the run's block 0
};

// The list's total U and the position of unit chunk_start(U), from the clamped context
// lengths in LDS.  Lane l holds sequences base + 16 l .. base + 16 l + 15 of each
// 1024-sequence window.  Every kv head lists the same T units (the sum over the sequences),
// so unit u is in kv head u / T at offset u mod T of the sequences' units.
struct Plan {
    int64_t U;
    Pos p;
};

template <class ChunkStart>
__device__ __forceinline__ Plan plan_wave(const DecodeArgs& a, const int* lctx, int lane, ChunkStart chunk_start)
{
    const int Hkv = a.num_kv_heads, S = a.num_seqs;
    const int ush = unit_shift(a.block_size);
    // total
    int64_t total = 0;
    for (int base = 0; base < S; base += kScanWindow) {
        int part = 0;
#pragma unroll
        for (int i = 0; i < kScanPerLane; i++) {
            const int s = base + lane * kScanPerLane + i;
            part += s < S ? nunits(lctx[s], ush) : 0;
        }
        total += __builtin_amdgcn_readlane(wave_incl_scan(part, lane), 63);
    }
    Plan pl;
    pl.U = total * Hkv;
    const int64_t u0 = chunk_start(pl.U);
    pl.p.s = S;
    pl.p.g = pl.p.j = 0;
    pl.p.run_start = pl.U;
    if (u0 >= pl.U) return pl;
    // locate u0: kv head g0, offset r0 in the sequences' units
    const int g0 = (int)(u0 / total);
    const int64_t r0 = u0 - (int64_t)g0 * total;
    int64_t before = 0;
    for (int base = 0; base < S; base += kScanWindow) {
        int nb[kScanPerLane];
        int part = 0;
#pragma unroll
        for (int i = 0; i < kScanPerLane; i++) {
            const int s = base + lane * kScanPerLane + i;
            nb[i] = s < S ? nunits(lctx[s], ush) : 0;
            part += nb[i];
        }
        const int incl = wave_incl_scan(part, lane);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(before + incl > r0);
        if (hit) {
            const int L = __builtin_ctzll(hit);
            int64_t u = before + (__builtin_amdgcn_readlane(incl, L) - __builtin_amdgcn_readlane(part, L));
#pragma unroll
            for (int i = 0; i < kScanPerLane; i++) {
                const int n = __builtin_amdgcn_readlane(nb[i], L);
                if (r0 < u + n) {
                    pl.p.s = base + L * kScanPerLane + i;
                    pl.p.g = g0;
                    pl.p.j = (int)(r0 - u);
                    pl.p.run_start = (int64_t)g0 * total + u;
                    return pl;
                }
                u += n;
            }
        }
        before += __builtin_amdgcn_readlane(incl, 63);
    }
    return pl;  // not reached
}

// A position in the work list that moves block by block: (sequence, kv head, block) with
// the run's context length.  Sequences with no context are skipped; past the list's end the
// cursor rests at (num_seqs, num_kv_heads) with no context.
struct Cursor {
    int s, g, j, ctx, nbs;
    int ush;  // unit_shift of the block size
    int64_t run_start;
};

__device__ __forceinline__ Cursor cursor_at(const Pos& p, const int* lctx, int ush)
{
    Cursor c;
    c.ush = ush;
    c.s = p.s;
    c.g = p.g;
    c.j = p.j;
    c.ctx = lctx[p.s];
    c.nbs = nunits(c.ctx, c.ush);
    c.run_start = p.run_start;
    return c;
}

// Move the cursor to block 0 of the next run: the next non-empty sequence of this kv head, else
// the first non-empty one of the next kv head.
__device__ __forceinline__ void next_run(Cursor& c, const int* lctx, int num_seqs, int num_kv_heads)
{
    c.run_start += c.nbs;
    c.j = 0;
    for (;;) {
        if (++c.s == num_seqs) {
            if (++c.g == num_kv_heads) {
                c.ctx = 0;
                break;
            }
            c.s = 0;
        }
        c.ctx = lctx[c.s];
        if (c.ctx != 0) break;
    }
    c.nbs = nunits(c.ctx, c.ush);
}

__device__ __forceinline__ void cursor_next(Cursor& c, const int* lctx, int num_seqs, int num_kv_heads)
{
    if (++c.j < c.nbs) return;
    next_run(c, lctx, num_seqs, num_kv_heads);
}

// Fused append.  The chunk that holds a run's last unit is the only one that reads the new
// token's slot (position ctx - 1).  When its wave issues that unit's K/V loads it also loads the
// run's new K and V rows (source [s][g] of new_key / new_value, in the query dtype), one
// 16-byte piece per lane.  When it attends the unit, the lanes encode their pieces in the
// cache dtype, store them into the slot and stage them in a per-wave LDS row, and the token's
// K and V are patched from that row into the unit's loaded registers: the ring's copy of the
// slot may or may not include the store, and either way the attention sees the same values in
// the same places as after a separate append.  The row travels with the unit's loads, so
// nothing waits for it.  Nothing in the launch waits for the store either; the pool bytes are
// those of the append kernel (encode_elem, store_piece_bytes -> store_piece_codes).
template <int QT, int KT, int D>
struct NewRow {
    static constexpr int ES = DtypeBytes<QT>::value;  // source element bytes (query dtype)
    static constexpr int EC = DtypeBytes<KT>::value;  // cache element bytes
    static constexpr int N = 16 / ES;                 // source elements per 16-byte piece
    static constexpr int P = D / N;                   // pieces per source row
    static constexpr int ROW = D * EC;                // encoded row bytes
    static_assert(2 * P <= 64, "the K and V rows of a token fit one wave");
};

// Deferred stores.  A store counts on the same wait counter as the ring's loads, so a store
// issued in the middle of a chunk makes the next wait on the ring wait for it to be written as
// well (the ring runs dry meanwhile).  The results of pieces that end inside the chunk -- and,
// with the fused append, the new rows -- are kept in a per-wave LDS stage and written after
// the chunk's last unit; a piece that finds the stage full is written at once.
template <int G, int CG>
constexpr int defer_slots()
{
    return G * CG >= 16 ? 1 : 2;
}

template <int G>
struct PieceMeta {
    int64_t dst;    // whole run: its first output row; partial: the piece id; -1: nothing
    int64_t run;    // the run whose chunk range is recorded for the merge, or -1
    int64_t rtile;  // fused append: element offset of the new token's tile, or -1
    int32_t k0, kn; // the chunk range
    int32_t ro;     // fused append: the token's offset in its block
    int32_t whole;
    float ml[G][2]; // partial: (max, sum) per head
};

template <int QT, int KT, int D, int G, bool FUSED, int SLOTS>
struct WaveStage {
    using S = Shape<QT, KT, D, G>;
    static constexpr int NS = SLOTS > 0 ? SLOTS : 1;
    float v[NS][G * D];  // the piece's output rows (head-major), normalised
    PieceMeta<G> meta[NS];
    // fused append: the new row of each slot, and one more for a piece written at once
    unsigned char row[FUSED ? SLOTS + 1 : 1][FUSED ? 2 * NewRow<QT, KT, D>::ROW : 16];
};

// The kernel's arguments read again from the kernarg segment at a point of use (scalar loads
// behind an empty asm the compiler cannot see through), for the paths that run once per piece:
// it keeps their pointers out of the registers the streaming loop holds.
typedef const __attribute__((address_space(4))) DecodeArgs KernArgs;
__device__ __forceinline__ KernArgs& kernel_args()
{
    KernArgs* p = (KernArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
    asm volatile("" : "+s"(p));
    return *p;
}

__device__ __forceinline__ int64_t uniform64(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---- the streaming kernel ---------------------------------------------------------------

// Per (cache dtype): where the query lives and how deep the K/V ring is.  Measured on the
// Llama-3-8B-shaped bf16 batch: query in VGPRs with a 2-deep ring beats query in LDS with a
// 3-deep ring (118 vs 121 us); an fp32 query does not fit in VGPRs beside the ring.
template <int KT>
struct Variant {
    static constexpr bool kQueryInLds = KT == kF32;
    static constexpr int kDepth = kQueryInLds ? 3 : 2;
};

// Chunks of the unit list: chunk k = units [k*C, (k+1)*C).
struct ChunkMap {
    int64_t C;
    __device__ int64_t start(int64_t k) const { return k * C; }
    __device__ int64_t size(int64_t) const { return C; }
    __device__ int64_t of_unit(int64_t u) const { return u / C; }
};

// Occupancy of the streaming kernel, chosen per variant from measurements on MI355X (stream
// kernel alone, Llama-shaped batch with the variant's heads):
//   3 waves per SIMD (at most 168 VGPRs, no spills) where that measured faster: fp8 with G <= 4
//     (70.3 -> 66.4 us at D 128) and D 64 with G <= 4 (bf16: 60.0 -> 55.5 us);
//   2 forced for bf16 D 128 G 8, which otherwise takes 296 registers and runs one wave per
//     SIMD (157 -> 139 us despite a few spills), and for fp8 G 8 (it fits 256 registers);
//   otherwise the compiler's choice: 2 waves per SIMD for most variants (bf16 G 1 / 2 measured
//     slower at 3), one for fp32 D 128, which measured slower when forced to 2 with spills.
// The fused-append instances of the 8-bit caches at D 128 run 2 waves per SIMD: the append's
// registers do not fit beside the ring in 168 (at 3 they spilled 14 VGPRs, and scratch traffic
// is HBM traffic).
// The persistent grid has max(2, this) waves per SIMD.
template <int KT, int D, int G, bool FUSED = false>
constexpr int stream_min_waves()
{
    if constexpr (KT == kF32) return 1;
    else if constexpr (KT == kBF16) return D == 64 && G <= 4 ? 3 : D == 128 && G == 8 ? 2 : 1;
    else if constexpr (FUSED && D == 128) return 2;
    else return G <= 4 ? 3 : 2;
}

template <int KT, int D, int G, bool FUSED = false>
constexpr int stream_waves_per_simd()
{
    return stream_min_waves<KT, D, G, FUSED>() > 2 ? stream_min_waves<KT, D, G, FUSED>() : 2;
}

// PER_RUN: the one-chunk-per-run form (chunk_blocks < 0); FUSED: the fused append (new_key set);
// HINT: cached loads for the leading blocks a.shared_blocks marks as shared.  Separate instances,
// so that their extra paths leave the plain balanced form's registers alone.
template <int QT, int KT, int D, int G, bool PER_RUN, bool FUSED, bool HINT = false>
__global__ __launch_bounds__(kDecodeThreads, (stream_min_waves<KT, D, G, FUSED>())) void decode_stream_kernel(
    const DecodeArgs a)
{
    using S = Shape<QT, KT, D, G>;
    constexpr bool QL = Variant<KT>::kQueryInLds;
    constexpr int NST = Variant<KT>::kDepth;
    constexpr bool MF = KT != kF32;  // the matrix-core form (bf16 and 8-bit caches)
    constexpr int KM = MF ? KT : kBF16;
    using M = MShape<kBF16, KM, D, G>;
    const int lane = threadIdx.x & 63;
    const int wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t NW = (int64_t)gridDim.x * kDecodeWaves;
    const int64_t w = (int64_t)blockIdx.x * kDecodeWaves + wave_in_wg;
    const int Hkv = a.num_kv_heads, NS = a.num_seqs;

    __shared__ __align__(16) unsigned char q_lds[QL ? kDecodeWaves * S::QBYTES : 16];
    constexpr int SLOTS = PER_RUN ? 0 : defer_slots<G, S::CG>();  // one run per chunk: nothing to defer
    using Stage = WaveStage<QT, KT, D, G, FUSED, SLOTS>;
    __shared__ __align__(16) Stage stage_lds[kDecodeWaves];
    extern __shared__ int lctx[];  // clamped context length of every sequence

    // All cursor moves read context lengths from LDS, so inside the stream the only global
    // loads are the ring's K/V loads and one block-table entry per step, a fixed count per
    // step that keeps every wait on the ring exact.
    for (int i = threadIdx.x; i < NS; i += kDecodeThreads) lctx[i] = seq_ctx(a, i);
    // shared-block counts, when given, follow the context lengths
    constexpr bool hint = HINT;
    if (hint)
        for (int i = threadIdx.x; i < NS; i += kDecodeThreads) lctx[NS + i] = a.shared_blocks[i];
    __syncthreads();

    // Chunk size: one chunk of ceil(U / NW) units per wave (at least kMinChunkBlocks), or the
    // caller's chunk size with chunks dealt round-robin to the waves.  Workgroups are dealt to
    // the 8 XCDs round-robin; the wave's first chunk is chosen so that chunk k runs on XCD
    // k mod 8, which gives every XCD the same mix of sequences, kv heads and block ranges (with
    // 4 consecutive chunks per workgroup, an XCD would see a fixed part of every run).
    const bool xcd8 = (gridDim.x & 7) == 0;
    const int64_t first =
        xcd8 ? 8 * kDecodeWaves * (int64_t)(blockIdx.x >> 3) + 8 * wave_in_wg + (blockIdx.x & 7) : w;
    // with the hint, slot kk (on XCD kk mod 8) takes chunk (kk mod 8) q + kk / 8, q = ceil(chunks / 8):
    // XCD x runs chunks x q .. x q + q - 1
    auto chunk_of = [&](int64_t kk, int64_t nch) -> int64_t {
        if (!hint || !xcd8) return kk;
        return (kk & 7) * ((nch + 7) >> 3) + (kk >> 3);
    };
    // chunk_blocks < 0: one chunk per run.  The host picks it when every run fits in one
    // minimum chunk, so no run is split, nothing is merged and the merge launch is skipped
    // (small batches, where a launch costs more than the work).  Chunk k is then the run of
    // sequence k / Hkv and kv head k mod Hkv (no run records, so the numbering is free).
    constexpr bool per_run = PER_RUN;
    ChunkMap cm{};
    auto count_chunks = [&](int64_t U) { return U > 0 ? min(cm.of_unit(U - 1) + 1, a.max_chunks) : (int64_t)0; };
    const Plan pl = per_run ? Plan{0, Pos{NS, 0, 0, 0}} : plan_wave(a, lctx, lane, [&](int64_t U) {
        cm.C = a.chunk_blocks > 0 ? (int64_t)a.chunk_blocks : max((U + NW - 1) / NW, (int64_t)kMinChunkBlocks);
        return cm.start(chunk_of(first, count_chunks(U)));
    });
    const int64_t U = pl.U;
    const int64_t nchunks = per_run ? (int64_t)NS * Hkv : count_chunks(U);
    // slots kk = first, first + NW, ... below kk_end map onto the chunks (the hint's dealing
    // leaves up to 7 slots without a chunk)
    const int64_t kk_end = hint && xcd8 ? 8 * ((nchunks + 7) >> 3) : nchunks;

    const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool);
    const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool);
    // A block of B = 16 << ub tokens is 1 << ub units.  Unit `sub` of a block: its K slices are
    // 1 KiB pieces at sub * 1 KiB + c * (B * 64) of the block's tile, its V loads the
    // sub-th run of TILE bytes (the pool layout of include/pagedattn.h).
    // An 8-token block is one unit whose upper 8 tokens are empty: lanes 32..63 of its K loads
    // and its V loads past the block's bytes fall outside the window and read nothing.
    const int ub = a.block_size > kUnitTokens ? 1 : 0;
    const int ush = unit_shift(a.block_size);
    const int btile = a.block_size * D * S::EB;  // bytes of one (block, kv head) tile
    const int vwin = btile < S::TILE ? btile : S::TILE;
    // K: lane l reads token l / 4 (matrix-core form: token l % 16), 16 bytes of each slice
    const int ktok = MF ? (lane & 15) : (lane >> 2);
    const int kvoff = a.block_size < kUnitTokens && ktok >= 8 ? 0x40000000
                      : MF                                   ? ktok * 64 + (lane >> 4) * 16
                                                             : lane * 16;
    // matrix-core form, V: lane l reads tokens 4 (l / 16) .. + 3 of channel l % 16 of each
    // 16-channel tile: element (token o, channel d) of a unit's V is at ((o / T) D + d) T + o % T
    // with T = min(16 / e, B) tokens per channel piece, so tile t starts 16 T e bytes after tile
    // t - 1.  With 8-token blocks of an 8-bit cache (T = 8) the lanes of tokens 8..15 fall past
    // the block's bytes, outside the window, and read nothing.
    const int vT = 16 / M::EB < a.block_size ? 16 / M::EB : a.block_size;
    const int mtok = 4 * (lane >> 4);
    const int mvoff = ((mtok / vT) * D + (lane & 15)) * vT * M::EB + (mtok % vT) * M::EB;
    const int mvtile = 16 * vT * M::EB;
    const int kstride = a.block_size * 64;
    const int64_t block_stride = (int64_t)Hkv * btile;
    const int32_t* tables = a.block_tables;
    const int mbps = a.max_blocks_per_seq;

    if constexpr (per_run) {  // the zero rows of empty sequences, before (and apart from) the stream
        for (int64_t k = first; k < nchunks; k += NW) {
            const int s = (int)(k / Hkv), g = (int)(k % Hkv);
            if (lctx[s] != 0) continue;
#pragma unroll
            for (int h = 0; h < G; h++) {
                const int64_t row = (int64_t)s * a.num_heads + (int64_t)g * G + h;
#pragma unroll
                for (int cg = 0; cg < S::CG; cg++) {
                    if constexpr (QT == kBF16)
                        static_cast<uint16_t*>(a.out)[row * D + cg * 64 + lane] = 0;
                    else
                        static_cast<float*>(a.out)[row * D + cg * 64 + lane] = 0.0f;
                }
            }
        }
    }

    for (int64_t kk = first; kk < kk_end; kk += NW) {
        const int64_t k = chunk_of(kk, nchunks);  // the chunk
        if (k >= nchunks) continue;
        int n;           // units of this chunk
        Pos p0;          // its first unit
        if constexpr (per_run) {
            p0 = Pos{(int)(k / Hkv), (int)(k % Hkv), 0, 0};
            n = __builtin_amdgcn_readfirstlane(nunits(lctx[p0.s], ush));  // uniform: keeps loop control scalar
            if (n == 0) {  // empty sequence: its zero rows were written above
                continue;
            }
        } else {
            n = (int)min(cm.size(k), U - cm.start(k));  // >= 1
            p0 = kk == first ? pl.p : plan_wave(a, lctx, lane, [&](int64_t) { return cm.start(k); }).p;
        }

        // table cursor: the block whose table entry is fetched next (it stops at the chunk's
        // last block, whose entry then feeds the fill-in loads past the end)
        Cursor tc = cursor_at(p0, lctx, ush);
        int tcount = 0;
        constexpr bool fused = FUSED;
        auto fetch_entry = [&](int& e, int& nv, int& g, int& sub, int& cached, int& es, int& last) {
            e = tables[(int64_t)tc.s * mbps + (tc.j >> ub)];
            nv = min(1 << ush, tc.ctx - (tc.j << ush));
            g = tc.g;
            sub = tc.j & ub;
            if constexpr (hint) cached = (tc.j >> ub) < lctx[NS + tc.s];
            if constexpr (fused) {
                es = tc.s;
                last = tc.j == tc.nbs - 1;
            }
            if (tcount + 1 < n) {
                cursor_next(tc, lctx, NS, Hkv);
                ++tcount;
            }
        };
        // compute cursor: the block attended next, with its piece's bookkeeping
        Cursor cc = cursor_at(p0, lctx, ush);
        int piece_j0 = cc.j;

        // entry ring: physical id, valid tokens, kv head and unit of the block (with the fused
        // append: its sequence and whether it is its run's last unit), for units t .. t+NST-1
        int ent[NST], ent_nv[NST], ent_g[NST], ent_sub[NST], ent_cached[NST] = {}, ent_s[NST] = {}, ent_last[NST] = {};
#pragma unroll
        for (int i = 0; i < NST; i++)
            fetch_entry(ent[i], ent_nv[i], ent_g[i], ent_sub[i], ent_cached[i], ent_s[i], ent_last[i]);

        auto query_row = [&](const Cursor& c) {
            KernArgs& a = kernel_args();
            return static_cast<const unsigned char*>(a.query) + ((int64_t)c.s * a.num_heads + (int64_t)c.g * G) * D * S::QB;
        };
        std::conditional_t<MF, MQ<kBF16, KM, D, G>, QRegs<QT, KT, D, G>> qr;
        const int q_off = wave_in_wg * S::QBYTES;
        auto load_query = [&](const Cursor& c) {
            if constexpr (QL) {
#pragma unroll
                for (int off = 0; off < S::QBYTES; off += 1024)
                    if (off + lane * 16 < S::QBYTES)
                        *reinterpret_cast<uint4*>(q_lds + q_off + off + lane * 16) = load16(query_row(c) + off + lane * 16);
            } else if constexpr (MF) {
                load_q_mf(qr, query_row(c), lane);
            } else {
                load_q<QT, KT, D, G>(qr, query_row(c), lane & 3);
            }
        };
        Stage& ws = stage_lds[wave_in_wg];
        using R = NewRow<QT, KT, D>;
        int npend = 0;  // pieces in the stage
        load_query(cc);
        float c2 = a.scale_log2 * (kIsQuant<KT> ? a.k_scale[cc.g] : 1.0f);

        std::conditional_t<MF, MAcc<kBF16, KM, D, G>, Acc<QT, KT, D, G>> st;
        auto reset = [&]() {
            if constexpr (MF) {
                st.m = -FLT_MAX;
                st.l = 0.0f;
#pragma unroll
                for (int t = 0; t < M::NT; t++) st.o[t] = mf_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            } else {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    st.m[h] = -FLT_MAX;
                    st.l[h] = 0.0f;
#pragma unroll
                    for (int cg = 0; cg < S::CG; cg++) st.o[cg][h] = 0.0f;
                }
            }
        };
        reset();

        // ---- end of a piece: fold l over the lanes that summed parts of it (the 8 token-pair
        // lane groups; matrix-core form: the 4 lane groups of a head), then write the row (a run
        // covered whole) or the partial result ----
        const int mh = lane & 15, mtb = 4 * (lane >> 4);  // matrix-core form: lane's head, first channel
        auto finish_piece = [&](bool defer) {
            KernArgs& a = kernel_args();
            if constexpr (MF) {
                st.l = mf_swap(st.l, false, false);
                st.l = mf_swap(st.l, true, false);
            } else {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    float x = st.l[h];
                    x += dpp_f32<kDppRowRor8>(x);
                    x += swizzle_xor16(x);
                    x += __shfl_xor(x, 32, 64);
                    st.l[h] = x;
                }
            }
            const int64_t run = (int64_t)cc.g * NS + cc.s;  // the run's number in list order
            const bool first = piece_j0 == 0, whole = first && cc.j == cc.nbs - 1;
            // every run with blocks is entered at its block 0 by exactly one wave, which records
            // the chunk range covering it for the merge
            const bool rec = first && !per_run;
            const int64_t k_last = rec ? cm.of_unit(cc.run_start + cc.nbs - 1) : k;
            const int64_t piece = run + k;
            const int64_t row0 = (int64_t)cc.s * a.num_heads + (int64_t)cc.g * G;
            const float vs = whole && kIsQuant<KT> ? a.v_scale[cc.g] : 1.0f;
            if constexpr (SLOTS > 0) {
                if (defer) {
                    PieceMeta<G>& me = ws.meta[npend];
                    if (lane == 0) {
                        me.dst = whole ? row0 : piece < a.max_pieces ? piece : -1;
                        me.run = rec ? run : -1;
                        me.rtile = -1;
                        me.k0 = (int32_t)k;
                        me.kn = (int32_t)(k_last - k + 1);
                        me.whole = whole;
                    }
                    float* v = ws.v[npend];
                    if constexpr (MF) {
                        if (lane < G) {
                            me.ml[lane][0] = st.m;
                            me.ml[lane][1] = st.l;
                        }
                        if (mh < G) {
                            const float f = st.l > 0.0f ? vs / st.l : 0.0f;
#pragma unroll
                            for (int t = 0; t < M::NT; t++)
                                *reinterpret_cast<mf_f32x4*>(v + mh * D + 16 * t + mtb) = st.o[t] * f;
                        }
                    } else {
                        if (lane == 0) {
#pragma unroll
                            for (int h = 0; h < G; h++) {
                                me.ml[h][0] = st.m[h];
                                me.ml[h][1] = st.l[h];
                            }
                        }
#pragma unroll
                        for (int h = 0; h < G; h++) {
                            const float f = st.l[h] > 0.0f ? vs / st.l[h] : 0.0f;
#pragma unroll
                            for (int cg = 0; cg < S::CG; cg++) v[h * D + cg * 64 + lane] = st.o[cg][h] * f;
                        }
                    }
                    ++npend;
                    return;
                }
            }
            if (rec && lane == 0) {
                a.run_info[2 * run] = (int32_t)k;
                a.run_info[2 * run + 1] = (int32_t)(k_last - k + 1);
            }
            if constexpr (MF) {
                if (mh < G) {
                    if (whole) {
                        const float f = st.l > 0.0f ? vs / st.l : 0.0f;
                        uint16_t* orow = static_cast<uint16_t*>(a.out) + (row0 + mh) * D + mtb;
#pragma unroll
                        for (int t = 0; t < M::NT; t++) {
                            const mf_f32x4 x = st.o[t] * f;
                            *reinterpret_cast<uint2*>(orow + 16 * t) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
                        }
                    } else if (piece < a.max_pieces) {
                        const float f = st.l > 0.0f ? 1.0f / st.l : 0.0f;
                        float* op = a.o_part + (piece * G + mh) * D + mtb;
#pragma unroll
                        for (int t = 0; t < M::NT; t++) *reinterpret_cast<mf_f32x4*>(op + 16 * t) = st.o[t] * f;
                        if (lane < G) {
                            a.ml_part[(piece * G + mh) * 2] = st.m;
                            a.ml_part[(piece * G + mh) * 2 + 1] = st.l;
                        }
                    }
                }
            } else if (whole) {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float f = st.l[h] > 0.0f ? vs / st.l[h] : 0.0f;
#pragma unroll
                    for (int cg = 0; cg < S::CG; cg++) {
                        const float v = st.o[cg][h] * f;
                        if constexpr (QT == kBF16)
                            static_cast<uint16_t*>(a.out)[(row0 + h) * D + cg * 64 + lane] = f32_to_bf16_bits(v);
                        else
                            static_cast<float*>(a.out)[(row0 + h) * D + cg * 64 + lane] = v;
                    }
                }
            } else if (piece < a.max_pieces) {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float f = st.l[h] > 0.0f ? 1.0f / st.l[h] : 0.0f;
                    float* op = a.o_part + (piece * G + h) * D;
#pragma unroll
                    for (int cg = 0; cg < S::CG; cg++) op[cg * 64 + lane] = st.o[cg][h] * f;
                    if (lane == 0) {
                        a.ml_part[(piece * G + h) * 2] = st.m[h];
                        a.ml_part[(piece * G + h) * 2 + 1] = st.l[h];
                    }
                }
            }
        };

        // fused append: store the new row staged in slot r into the pool (lanes 0..2P-1)
        auto store_row = [&](int r, int64_t tile, int o) {
            KernArgs& a = kernel_args();
            if constexpr (fused) {
                if (lane < 2 * R::P) {
                    const int kv = lane / R::P, piece = lane % R::P;
                    store_piece_bytes<KT, R::N>(ws.row[r] + kv * R::ROW + piece * R::N * R::EC,
                                                static_cast<unsigned char*>(kv ? a.v_pool : a.k_pool), tile,
                                                piece * R::N, o, kv, D, a.block_size);
                }
            }
        };

        // write what the stage holds (after the chunk's last unit)
        auto flush = [&]() {
            KernArgs& a = kernel_args();
            if constexpr (SLOTS > 0) {
                for (int i = 0; i < npend; i++) {
                    const PieceMeta<G>& me = ws.meta[i];
                    const int64_t dst = uniform64(me.dst), run = uniform64(me.run);
                    const bool whole = __builtin_amdgcn_readfirstlane(me.whole) != 0;
                    const float* v = ws.v[i];
                    if (run >= 0 && lane == 0) {
                        a.run_info[2 * run] = me.k0;
                        a.run_info[2 * run + 1] = me.kn;
                    }
                    if constexpr (MF) {
                        if (mh < G) {
                            if (whole) {
                                uint16_t* orow = static_cast<uint16_t*>(a.out) + (dst + mh) * D + mtb;
#pragma unroll
                                for (int t = 0; t < M::NT; t++) {
                                    const mf_f32x4 x = *reinterpret_cast<const mf_f32x4*>(v + mh * D + 16 * t + mtb);
                                    *reinterpret_cast<uint2*>(orow + 16 * t) =
                                        make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
                                }
                            } else if (dst >= 0) {
                                float* op = a.o_part + (dst * G + mh) * D + mtb;
#pragma unroll
                                for (int t = 0; t < M::NT; t++)
                                    *reinterpret_cast<mf_f32x4*>(op + 16 * t) =
                                        *reinterpret_cast<const mf_f32x4*>(v + mh * D + 16 * t + mtb);
                                if (lane < G) {
                                    a.ml_part[(dst * G + mh) * 2] = me.ml[mh][0];
                                    a.ml_part[(dst * G + mh) * 2 + 1] = me.ml[mh][1];
                                }
                            }
                        }
                    } else if (whole) {
#pragma unroll
                        for (int h = 0; h < G; h++)
#pragma unroll
                            for (int cg = 0; cg < S::CG; cg++) {
                                const float x = v[h * D + cg * 64 + lane];
                                if constexpr (QT == kBF16)
                                    static_cast<uint16_t*>(a.out)[(dst + h) * D + cg * 64 + lane] = f32_to_bf16_bits(x);
                                else
                                    static_cast<float*>(a.out)[(dst + h) * D + cg * 64 + lane] = x;
                            }
                    } else if (dst >= 0) {
#pragma unroll
                        for (int h = 0; h < G; h++) {
#pragma unroll
                            for (int cg = 0; cg < S::CG; cg++)
                                a.o_part[(dst * G + h) * D + cg * 64 + lane] = v[h * D + cg * 64 + lane];
                            if (lane == 0) {
                                a.ml_part[(dst * G + h) * 2] = me.ml[h][0];
                                a.ml_part[(dst * G + h) * 2 + 1] = me.ml[h][1];
                            }
                        }
                    }
                    if constexpr (fused) {
                        const int64_t rtile = uniform64(me.rtile);
                        if (rtile >= 0) store_row(i, rtile, me.ro);
                    }
                }
                npend = 0;
            }
        };

        // ---- the stream: step t issues block t into ring slot t % NST (blocks past the end
        // re-read the chunk's last block and are never attended), refills the entry ring with
        // block t + NST, and attends block t - (NST - 1) ----
        uint4 kb[NST][S::NCH];
        // V: 16 bytes per slice; matrix-core form: one piece per 16-channel tile
        std::conditional_t<MF, typename M::VP, uint4> vb[NST][MF ? M::NT : S::NCH];
        int kv_nv[NST];
        uint4 nrw[NST];     // fused append: the new row piece loaded with the run's last unit
        int kv_phys[NST];   // fused append: the unit's physical block
        for (int t0 = 0; t0 < n + NST - 1; t0 += NST) {
#pragma unroll
            for (int i = 0; i < NST; i++) {
                const int t = t0 + i;
                {
                    // A step past the chunk's end, or a block id outside the pool, loads through
                    // an empty buffer window: the loads return zeros without touching memory,
                    // and the instruction stream (hence every wait count) stays the same.
                    int phys = __builtin_amdgcn_readfirstlane(ent[i]);
                    const bool bad = phys < 0 || (int64_t)phys >= a.num_blocks;
                    phys = bad ? 0 : phys;
                    kv_nv[i] = bad ? 0 : ent_nv[i];
                    const bool none = bad || t >= n;
                    // kv head and unit are wave-uniform; saying so keeps the buffer descriptors
                    // in SGPRs (otherwise every load is wrapped in a readfirstlane loop)
                    const int sub = __builtin_amdgcn_readfirstlane(ent_sub[i]);
                    const int gu = __builtin_amdgcn_readfirstlane(ent_g[i]);
                    const int64_t off = (int64_t)phys * block_stride + (int64_t)gu * btile;
                    const TileWindow kw(kpool + off + sub * 1024, none ? 0 : btile - sub * 1024);
                    const TileWindow vw(vpool + off + sub * S::TILE, none ? 0 : vwin);
                    // a block shared with other sequences keeps the default cache policy, so its
                    // other readers find it cached; the rest are read once and streamed (nt)
                    if constexpr (MF) {
                        const bool cached = hint && __builtin_amdgcn_readfirstlane(ent_cached[i]);
                        if (cached) {
#pragma unroll
                            for (int c = 0; c < S::NCH; c++) kb[i][c] = kw.load_cached(kvoff, c * kstride);
#pragma unroll
                            for (int t = 0; t < M::NT; t++) vb[i][t] = vw.template load_piece<typename M::VP>(mvoff, t * mvtile, true);
                        } else {
#pragma unroll
                            for (int c = 0; c < S::NCH; c++) kb[i][c] = kw.load_stream(kvoff, c * kstride);
#pragma unroll
                            for (int t = 0; t < M::NT; t++) vb[i][t] = vw.template load_piece<typename M::VP>(mvoff, t * mvtile, false);
                        }
                    } else if (hint && __builtin_amdgcn_readfirstlane(ent_cached[i])) {
#pragma unroll
                        for (int c = 0; c < S::NCH; c++) kb[i][c] = kw.load_cached(kvoff, c * kstride);
#pragma unroll
                        for (int c = 0; c < S::NCH; c++) vb[i][c] = vw.load_cached(lane * 16 + c * 1024);
                    } else {
#pragma unroll
                        for (int c = 0; c < S::NCH; c++) kb[i][c] = kw.load_stream(kvoff, c * kstride);
#pragma unroll
                        for (int c = 0; c < S::NCH; c++) vb[i][c] = vw.load_stream(lane * 16 + c * 1024);
                    }
                    if constexpr (fused) {
                        // with its run's last unit (a valid block): lanes 0..P-1 load the K row's
                        // pieces, P..2P-1 the V row's; every other lane and step loads the first 16
                        // bytes of new_key, so the instruction stream stays the same
                        const int sn = __builtin_amdgcn_readfirstlane(ent_s[i]);
                        const bool want = !none && __builtin_amdgcn_readfirstlane(ent_last[i]);
                        const int64_t roff = (((int64_t)sn * Hkv + gu) * D) * R::ES;
                        const unsigned char* src = static_cast<const unsigned char*>(a.new_key);
                        if (want && lane < 2 * R::P)
                            src = lane < R::P ? src + roff + lane * 16
                                              : static_cast<const unsigned char*>(a.new_value) + roff + (lane - R::P) * 16;
                        nrw[i] = load16(src);
                        kv_phys[i] = phys;
                    }
                }
                fetch_entry(ent[i], ent_nv[i], ent_g[i], ent_sub[i], ent_cached[i], ent_s[i], ent_last[i]);

                const int ta = t - (NST - 1);
                if (ta >= 0 && ta < n) {
                    const int j = (i + 1) % NST;  // the slot issued NST-1 steps ago
                    if (ta > 0 && cc.j == 0) {       // a new run: start its piece
                        load_query(cc);
                        c2 = a.scale_log2 * (kIsQuant<KT> ? a.k_scale[cc.g] : 1.0f);
                        reset();
                        piece_j0 = 0;
                    }
                    // fused append: the run's last unit holds the new token at index nv - 1.  Its
                    // row pieces are encoded and staged in LDS; the ring's copy of the slot may
                    // predate this launch's store, so the token's K and V are patched in from
                    // the staged row before the unit is attended.
                    if constexpr (fused) {
                        if (cc.j == cc.nbs - 1 && kv_nv[j] > 0) {
                            const int tn = kv_nv[j] - 1;  // the new token's index in the unit
                            unsigned char* const nrow = ws.row[npend];  // the slot this piece takes
                            if (lane < 2 * R::P) {
                                const int kv = lane / R::P, piece = lane % R::P;
                                unsigned char* dst = nrow + kv * R::ROW + piece * R::N * R::EC;
                                if constexpr (R::EC == R::ES) {
                                    *reinterpret_cast<uint4*>(dst) = nrw[j];
                                } else {
                                    static_assert(R::EC == 1 && R::N == 8, "bf16 source, 8-bit cache");
                                    const int gc = __builtin_amdgcn_readfirstlane(cc.g);
                                    const float sc = kv ? a.v_scale[gc] : a.k_scale[gc];
                                    const uint32_t words[4] = {nrw[j].x, nrw[j].y, nrw[j].z, nrw[j].w};
                                    uint32_t code[R::N];
#pragma unroll
                                    for (int e = 0; e < R::N; e++) code[e] = encode_elem<QT, KT>(words, e, sc);
                                    *reinterpret_cast<uint2*>(dst) =
                                        make_uint2(code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24,
                                                   code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24);
                                }
                            }
                            // K: the lanes of token tn (lane / 4; matrix-core form: lane % 16) take
                            // their channels of each slice from the row
                            const bool mine = ktok == tn;
                            const int kq = MF ? (lane >> 4) : (lane & 3);
#pragma unroll
                            for (int c = 0; c < S::NCH; c++) {
                                const uint4 kn = *reinterpret_cast<const uint4*>(nrow + (c * S::W + kq * S::KE) * S::EB);
                                if (mine) kb[j][c] = kn;
                            }
                            if constexpr (MF) {
                                // V: lane l holds tokens 4 (l / 16) .. + 3 of channel 16 t + l % 16;
                                // the lanes of token tn replace element tn % 4
                                const bool vmine = (lane >> 4) == (tn >> 2);
                                const int en = tn & 3;
#pragma unroll
                                for (int t = 0; t < M::NT; t++) {
                                    const unsigned char* e = nrow + R::ROW + (16 * t + (lane & 15)) * M::EB;
                                    if constexpr (M::EB == 2) {
                                        const uint32_t v = *reinterpret_cast<const uint16_t*>(e);
                                        const uint32_t sh = 16 * (en & 1), keep = ~(0xFFFFu << sh);
                                        uint2& w = vb[j][t];
                                        w.x = vmine && en < 2 ? (w.x & keep) | (v << sh) : w.x;
                                        w.y = vmine && en >= 2 ? (w.y & keep) | (v << sh) : w.y;
                                    } else {
                                        const uint32_t v = *e;
                                        const uint32_t sh = 8 * en, keep = ~(0xFFu << sh);
                                        vb[j][t] = vmine ? (vb[j][t] & keep) | (v << sh) : vb[j][t];
                                    }
                                }
                            } else {
                                // V: lane l holds channel cg * 64 + l; token tn is element tn % TPC
                                // of the channel's 16-byte piece in token group tn / TPC
                                const int qn = tn / S::TPC, en = tn % S::TPC;
                                const int wn = en * S::EB / 4, sh = (en * S::EB % 4) * 8;
                                constexpr uint32_t emask = S::EB == 4 ? 0xFFFFFFFFu : (1u << (8 * S::EB)) - 1u;
#pragma unroll
                                for (int c = 0; c < S::NCH; c++) {  // constant indices keep the ring in VGPRs
                                    const int cg = c % S::CG;
                                    if (c / S::CG != qn) continue;
                                    const unsigned char* e = nrow + R::ROW + (cg * 64 + lane) * S::EB;
                                    uint32_t v;
                                    if constexpr (S::EB == 4)
                                        v = *reinterpret_cast<const uint32_t*>(e);
                                    else if constexpr (S::EB == 2)
                                        v = *reinterpret_cast<const uint16_t*>(e);
                                    else
                                        v = *e;
                                    auto& w = vb[j][c];
                                    const uint32_t put = v << sh, keep = ~(emask << sh);
                                    w.x = wn == 0 ? (w.x & keep) | put : w.x;
                                    w.y = wn == 1 ? (w.y & keep) | put : w.y;
                                    w.z = wn == 2 ? (w.z & keep) | put : w.z;
                                    w.w = wn == 3 ? (w.w & keep) | put : w.w;
                                }
                            }
                        }
                    }
                    if constexpr (QL) {
                        const QLds qo{q_lds, opaque(q_off)};
                        attend_block<QT, KT, D, G>(st, qo, kb[j], vb[j], kv_nv[j], c2, lane);
                    } else if constexpr (MF) {
                        attend_mfma<kBF16, KM, D, G>(st, qr, kb[j], vb[j], kv_nv[j], c2, lane);
                    } else {
                        attend_block<QT, KT, D, G>(st, qr, kb[j], vb[j], kv_nv[j], c2, lane);
                    }
                    if (cc.j == cc.nbs - 1 || ta == n - 1) {
                        // a piece ending inside the chunk goes to the stage while it has room
                        const bool defer = SLOTS > 0 && ta < n - 1 && npend < SLOTS;
                        const int r = npend;  // its slot (the fused append staged its row there)
                        finish_piece(defer);
                        // fused append: the staged row goes into the slot, token
                        // ((unit & ub) * 16 + tn) of the block
                        if constexpr (fused) {
                            if (cc.j == cc.nbs - 1 && kv_nv[j] > 0) {
                                const int gc = __builtin_amdgcn_readfirstlane(cc.g);
                                const int64_t tile = ((int64_t)kv_phys[j] * Hkv + gc) * (int64_t)a.block_size * D;
                                const int o = ((cc.j & ub) << 4) + kv_nv[j] - 1;
                                if (defer) {
                                    if (lane == 0) {
                                        ws.meta[r].rtile = tile;
                                        ws.meta[r].ro = o;
                                    }
                                } else {
                                    store_row(r, tile, o);
                                }
                            }
                        }
                    }
                    if (ta < n - 1) cursor_next(cc, lctx, NS, Hkv);
                }
            }
        }
        flush();
    }
}

}  // namespace
}  // namespace pa
