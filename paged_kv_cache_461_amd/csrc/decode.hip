// decode.hip -- PagedAttention decode for gfx950: balanced streaming kernel + merge kernel.
//
// The attention of one decode query over its sequence's cache is softmax(q K^T * scale) V
// (page 1, section 2), read block by block through the sequence's block table (page 1,
// section 4; page 3, section 2.1), with the G query heads of a GQA group sharing one KV head
// (page 1, section 10).
//
// Work decomposition.  The K/V blocks of every (sequence, kv head) pair -- a "run" -- are
// laid end to end, sequence-major then kv head, into one list of U units (one unit = one
// 16-token block of one kv head).  The list is cut into equal chunks of C units and the
// waves of a persistent grid take chunks w, w + NW, ... (by default C = ceil(U / NW): one
// chunk per wave, so every wave moves the same number of bytes and the kernel has no tail).
// A chunk that covers runs r1..r2 attends each covered piece of a run on its own (online
// softmax state reset per piece) and stores the piece's normalised row and (max, sum) as a
// partial result; a run covered by one piece writes its output row directly.  The merge
// kernel combines the pieces of every split run (flash-decoding split-K).  Piece ids are
// run + chunk, which is one-to-one over non-empty pieces (a later run can only meet a later
// chunk), so the workspace size depends only on the numbers of runs and chunks.
//
// Inside a wave, per 16-token block (pool layout in include/pagedattn.h) NCH K loads and NCH V
// loads of 16 bytes per lane each read one contiguous 1 KiB slice:
//   QK^T: lane l holds channels of token l/4; bf16/fp8 K is multiplied with bf16 query pairs
//         (staged per wave in LDS) by v_dot2c_f32_bf16 (fp8 first widened exactly to bf16
//         pairs), fp32 K with FMAs; the 4 lanes of a token finish the dot product with two DPP
//         quad moves.
//   softmax: online, in base 2.  The running max is wave-uniform and only moved when a score
//         exceeds it by more than 8 (then o and l are rescaled), so most blocks skip the
//         rescale; weights stay below 2^8, and normalisation happens once per piece.
//   PV:   the block's weights are packed to bf16 pairs (the partner token's weight comes from
//         the neighbouring quad by one ds_swizzle) and read into scalar registers; each V load
//         gives every lane one channel of 8 (bf16) or 16 (fp8) consecutive tokens, contracted
//         with the pairs by v_dot2c_f32_bf16 (fp32: FMAs).  The accumulator is one fp32 per
//         (channel group, head) per lane.
// An NST-deep ring of register buffers keeps NST-1 blocks of K and V in flight while one is
// attended; all loop bounds are wave-uniform, so the waits on the ring stay counted.
#include <float.h>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

constexpr float kRescaleMargin = 8.0f;  // log2 units: weights are kept <= 2^8
#ifndef PA_PIPELINE_DEPTH
#define PA_PIPELINE_DEPTH 3
#endif
constexpr int kPipelineDepth = PA_PIPELINE_DEPTH;  // blocks per wave in the register ring

template <int QT, int KT, int D, int G>
struct Shape {
    static constexpr int EB = DtypeBytes<KT>::value;
    static constexpr int W = 64 / EB;      // channels per 64-byte slice
    static constexpr int NCH = D / W;      // 1 KiB slices per (block, kv head) tile
    static constexpr int KE = W / 4;       // K channels per lane per slice
    static constexpr int TPC = 16 / EB;    // V: tokens of one channel per 16-byte piece
    static constexpr int NQ = kBlockSize / TPC;  // V: token groups per block
    static constexpr int CG = D / 64;      // V: 64-channel groups (one channel per lane)
    static constexpr int TILE = kBlockSize * D * EB;
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

// Four dwords of this wave's query copy in LDS.
__device__ __forceinline__ u32x4_t lds_q16(const unsigned char* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// The query copy's LDS offset, made opaque to the compiler once per block: otherwise the
// loop-invariant query reads are hoisted out of the block loop and the query occupies 64 more
// VGPRs per lane (half the waves per SIMD).  An empty asm on a scalar register costs nothing
// and, unlike a volatile access, adds no memory wait that would drain the K/V ring.
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// Partial dot products of this lane's K channels with the G query rows (query in LDS).
template <int QT, int KT, int D, int G>
__device__ __forceinline__ void qk_slice(const unsigned char* q_lds, int kp, int c, const uint4& kv,
                                         float (&acc)[G])
{
    using S = Shape<QT, KT, D, G>;
#pragma unroll
    for (int h = 0; h < G; h++) {
        const unsigned char* qp = q_lds + (h * D + c * S::W + kp * S::KE) * S::QB;
        if constexpr (KT == kBF16) {
            const u32x4_t q = lds_q16(qp);
            acc[h] = dot2_bf16(kv.x, q.x, acc[h]);
            acc[h] = dot2_bf16(kv.y, q.y, acc[h]);
            acc[h] = dot2_bf16(kv.z, q.z, acc[h]);
            acc[h] = dot2_bf16(kv.w, q.w, acc[h]);
        } else if constexpr (KT == kFP8) {
            const u32x4_t q0 = lds_q16(qp);
            const u32x4_t q1 = lds_q16(qp + 16);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<false>(kv.x), q0.x, acc[h]);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<true>(kv.x), q0.y, acc[h]);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<false>(kv.y), q0.z, acc[h]);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<true>(kv.y), q0.w, acc[h]);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<false>(kv.z), q1.x, acc[h]);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<true>(kv.z), q1.y, acc[h]);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<false>(kv.w), q1.z, acc[h]);
            acc[h] = dot2_bf16(e4m3x2_to_bf16x2<true>(kv.w), q1.w, acc[h]);
        } else {
            const u32x4_t q = lds_q16(qp);
            acc[h] = __builtin_fmaf(as_float(kv.x), as_float(q.x), acc[h]);
            acc[h] = __builtin_fmaf(as_float(kv.y), as_float(q.y), acc[h]);
            acc[h] = __builtin_fmaf(as_float(kv.z), as_float(q.z), acc[h]);
            acc[h] = __builtin_fmaf(as_float(kv.w), as_float(q.w), acc[h]);
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
    } else if constexpr (KT == kFP8) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w = u4_get(vv, i);
            const uint32_t lo = e4m3x2_to_bf16x2<false>(w);
            const uint32_t hi = e4m3x2_to_bf16x2<true>(w);
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

template <int QT, int KT, int D, int G>
__device__ __forceinline__ void attend_block(Acc<QT, KT, D, G>& st, const unsigned char* q_lds_base, int q_off,
                                             const uint4 (&kb)[Shape<QT, KT, D, G>::NCH],
                                             const uint4 (&vb)[Shape<QT, KT, D, G>::NCH], int n_valid, float c2,
                                             int lane)
{
    using S = Shape<QT, KT, D, G>;
    const unsigned char* q_lds = q_lds_base + opaque(q_off);
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; h++) acc[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < S::NCH; c++) qk_slice<QT, KT, D, G>(q_lds, lane & 3, c, kb[c], acc);

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
            for (int t = 0; t < kBlockSize; t++) ps[h][t] = as_float(__builtin_amdgcn_readlane(as_uint(mine), 4 * t));
        } else {
            const uint32_t pp = pack_bf16x2(odd ? other : mine, odd ? mine : other);
            st.l[h] = dot2_bf16(pp, kBf16OnePair, st.l[h]);
#pragma unroll
            for (int i = 0; i < 8; i++) pps[h][i] = __builtin_amdgcn_readlane(pp, 8 * i);
        }
    }

    if (n_valid < kBlockSize) {
#pragma unroll
        for (int c = 0; c < S::NCH; c++) pv_load<QT, KT, D, G>(st, c, mask_tail<QT, KT, D, G>(vb[c], c, n_valid), pps, ps);
    } else {
#pragma unroll
        for (int c = 0; c < S::NCH; c++) pv_load<QT, KT, D, G>(st, c, vb[c], pps, ps);
    }
}

// ---- work-list arithmetic ---------------------------------------------------------------

// Context length the kernels use for sequence s: clamped to [0, max_context_len], so a
// length beyond the caller's bound can never send a table read or a workspace write out of
// range (the caller's contract is context_lens[s] <= max_context_len).
__device__ __forceinline__ int seq_ctx(const DecodeArgs& a, int s)
{
    const int c = a.context_lens[s];
    return c < 0 ? 0 : (c > a.max_context_len ? a.max_context_len : c);
}

__device__ __forceinline__ int seq_blocks(const DecodeArgs& a, int s)
{
    return (seq_ctx(a, s) + kBlockSize - 1) / kBlockSize;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        x += lane >= d ? y : 0;
    }
    return x;
}

constexpr int kScanPerLane = 16;  // sequences per lane in one pass over context_lens
constexpr int kScanWindow = 64 * kScanPerLane;

// Total units U = num_kv_heads * sum_s ceil(ctx_s / B).
__device__ int64_t total_units(const DecodeArgs& a, int lane)
{
    int64_t total = 0;
    for (int base = 0; base < a.num_seqs; base += kScanWindow) {
        int part = 0;
#pragma unroll
        for (int i = 0; i < kScanPerLane; i++) {
            // unconditional (clamped) loads: all of them are in flight before the first wait
            const int s = base + i * 64 + lane;
            const int n = seq_blocks(a, min(s, a.num_seqs - 1));
            part += s < a.num_seqs ? n : 0;
        }
        total += __builtin_amdgcn_readlane(wave_incl_scan(part, lane), 63);
    }
    return total * a.num_kv_heads;
}

struct Pos {
    int s, g, j;        // run (sequence s, kv head g), block j of the run
    int64_t run_start;  // unit index of the run's block 0
};

// Position of unit u0 in the work list (s = num_seqs when u0 >= U).
__device__ Pos locate(const DecodeArgs& a, int64_t u0, int lane)
{
    const int Hkv = a.num_kv_heads;
    int64_t before = 0;  // units of the sequences before this window
    for (int base = 0; base < a.num_seqs; base += kScanWindow) {
        int nb[kScanPerLane];
        int part = 0;
#pragma unroll
        for (int i = 0; i < kScanPerLane; i++) {
            const int s = base + lane * kScanPerLane + i;  // lane holds consecutive sequences
            const int n = seq_blocks(a, min(s, a.num_seqs - 1));
            nb[i] = s < a.num_seqs ? n : 0;
            part += nb[i];
        }
        const int incl = wave_incl_scan(part, lane);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(before + (int64_t)incl * Hkv > u0);
        if (hit) {
            const int L = __builtin_ctzll(hit);
            int64_t u = before + (int64_t)(__builtin_amdgcn_readlane(incl, L) - __builtin_amdgcn_readlane(part, L)) * Hkv;
#pragma unroll
            for (int i = 0; i < kScanPerLane; i++) {
                const int n = __builtin_amdgcn_readlane(nb[i], L);
                const int64_t span = (int64_t)n * Hkv;
                if (u0 < u + span) {
                    const int64_t off = u0 - u;
                    Pos p;
                    p.s = base + L * kScanPerLane + i;
                    p.g = (int)(off / n);
                    p.j = (int)(off % n);
                    p.run_start = u + (int64_t)p.g * n;
                    return p;
                }
                u += span;
            }
        }
        before += (int64_t)__builtin_amdgcn_readlane(incl, 63) * Hkv;
    }
    Pos p;
    p.s = a.num_seqs;
    p.g = p.j = 0;
    p.run_start = before;
    return p;
}

// ---- the streaming kernel ---------------------------------------------------------------

template <int QT, int KT, int D, int G, int NST>
__global__ __launch_bounds__(kDecodeThreads) void decode_stream_kernel(const DecodeArgs a)
{
    using S = Shape<QT, KT, D, G>;
    const int lane = threadIdx.x & 63;
    const int wave_in_wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t NW = (int64_t)gridDim.x * kDecodeWaves;
    const int64_t w = (int64_t)blockIdx.x * kDecodeWaves + wave_in_wg;
    const int Hkv = a.num_kv_heads;

    __shared__ __align__(16) unsigned char q_lds_all[kDecodeWaves * S::QBYTES];
    const int q_off = wave_in_wg * S::QBYTES;
    unsigned char* q_lds = q_lds_all + q_off;

    const int64_t U = total_units(a, lane);
    const int64_t C = a.chunk_blocks > 0 ? a.chunk_blocks : max((U + NW - 1) / NW, (int64_t)kMinChunkBlocks);
    const int64_t nchunks = min((U + C - 1) / C, a.max_chunks);

    const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool) + lane * 16;
    const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool) + lane * 16;
    const int64_t block_stride = (int64_t)Hkv * S::TILE;

    for (int64_t k = w; k < nchunks; k += NW) {
        const int64_t u0 = k * C;
        const int64_t uend = min(u0 + C, U);
        Pos p = locate(a, u0, lane);
        int64_t u = u0;
        while (u < uend && p.s < a.num_seqs) {
            // ---- one piece: blocks j0 .. j0+len-1 of run (s, g) ----
            const int s = p.s, g = p.g, j0 = p.j;
            const int ctx = seq_ctx(a, s);
            const int nbs = (ctx + kBlockSize - 1) / kBlockSize;
            const int len = (int)min((int64_t)(nbs - j0), uend - u);
            const int64_t run = (int64_t)s * Hkv + g;
            const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

            // the group's query rows into this wave's LDS copy
            {
                const unsigned char* qsrc = static_cast<const unsigned char*>(a.query) +
                                            ((int64_t)s * a.num_heads + (int64_t)g * G) * D * S::QB;
#pragma unroll
                for (int off = 0; off < S::QBYTES; off += 1024)
                    if (off + lane * 16 < S::QBYTES)
                        *reinterpret_cast<uint4*>(q_lds + off + lane * 16) = load16(qsrc + off + lane * 16);
            }
            const float c2 = a.scale_log2 * (KT == kFP8 ? a.k_scale[g] : 1.0f);
            const unsigned char* kbase = kpool + (int64_t)g * S::TILE;
            const unsigned char* vbase = vpool + (int64_t)g * S::TILE;

            Acc<QT, KT, D, G> st;
#pragma unroll
            for (int h = 0; h < G; h++) {
                st.m[h] = -FLT_MAX;
                st.l[h] = 0.0f;
#pragma unroll
                for (int cg = 0; cg < S::CG; cg++) st.o[cg][h] = 0.0f;
            }

            // Segments of up to 64 blocks: lane i of `entry` holds the physical id of the
            // segment's block i.  Every ring refill is issued, also past the end of the segment
            // (then it re-reads the last block, which is in cache, and is never attended), so the
            // number of loads between a block's issue and its use is fixed and the compiler
            // waits for exactly that block.
            for (int sj = 0; sj < len; sj += 64) {
                const int slen = min(64, len - sj);
                const int jb = j0 + sj;
                int entry = table[jb + min(lane, slen - 1)];
                entry = lane < slen ? entry : -1;

                uint4 kb[NST][S::NCH], vb[NST][S::NCH];
                int nv[NST];  // valid tokens of the block in each ring slot (0 = unusable block)
                auto issue = [&](int t, uint4 (&kd)[S::NCH], uint4 (&vd)[S::NCH]) -> int {
                    t = min(t, slen - 1);
                    int phys = __builtin_amdgcn_readlane(entry, t);
                    const bool bad = phys < 0 || (int64_t)phys >= a.num_blocks;
                    phys = bad ? 0 : phys;
                    const unsigned char* kp = kbase + (int64_t)phys * block_stride;
                    const unsigned char* vp = vbase + (int64_t)phys * block_stride;
#pragma unroll
                    for (int c = 0; c < S::NCH; c++) kd[c] = load16(kp + c * 1024);
#pragma unroll
                    for (int c = 0; c < S::NCH; c++) vd[c] = load16(vp + c * 1024);
                    return bad ? 0 : min(kBlockSize, ctx - (jb + t) * kBlockSize);
                };

#pragma unroll
                for (int i = 0; i < NST - 1; i++) nv[i] = issue(i, kb[i], vb[i]);
                for (int t0 = 0; t0 < slen; t0 += NST) {
#pragma unroll
                    for (int i = 0; i < NST; i++) {
                        const int nx = (i + NST - 1) % NST;  // the slot freed by the previous step
                        nv[nx] = issue(t0 + i + NST - 1, kb[nx], vb[nx]);
                        if (t0 + i < slen)
                            attend_block<QT, KT, D, G>(st, q_lds_all, q_off, kb[i], vb[i], nv[i], c2, lane);
                    }
                }
            }

            // ---- finish the piece ----
            // every lane of a token pair's 8 lanes added that pair's weights to l: add the 8
            // pairs once each (lanes differing in bits 3, 4, 5)
#pragma unroll
            for (int h = 0; h < G; h++) {
                float x = st.l[h];
                x += dpp_f32<kDppRowRor8>(x);
                x += swizzle_xor16(x);
                x += __shfl_xor(x, 32, 64);
                st.l[h] = x;
            }
            const bool first = j0 == 0, whole = first && len == nbs;
            if (first && lane == 0) {
                // every run with blocks is entered at its block 0 by exactly one wave, which
                // records the chunk range covering it for the merge
                const int64_t k_last = (p.run_start + nbs - 1) / C;
                a.run_info[2 * run] = (int32_t)k;
                a.run_info[2 * run + 1] = (int32_t)(k_last - k + 1);
            }
            const int64_t piece = run + k;
            if (whole) {
                const float vs = KT == kFP8 ? a.v_scale[g] : 1.0f;
#pragma unroll
                for (int h = 0; h < G; h++) {
                    const float f = st.l[h] > 0.0f ? vs / st.l[h] : 0.0f;
                    const int64_t row = (int64_t)s * a.num_heads + (int64_t)g * G + h;
#pragma unroll
                    for (int cg = 0; cg < S::CG; cg++) {
                        const float v = st.o[cg][h] * f;
                        if constexpr (QT == kBF16)
                            static_cast<uint16_t*>(a.out)[row * D + cg * 64 + lane] = f32_to_bf16_bits(v);
                        else
                            static_cast<float*>(a.out)[row * D + cg * 64 + lane] = v;
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

            // ---- next run ----
            u += len;
            p.run_start = u;
            p.j = 0;
            if (++p.g == Hkv) {
                p.g = 0;
                do {
                    ++p.s;
                } while (p.s < a.num_seqs && seq_ctx(a, p.s) == 0);
            }
        }
    }
}

// Merge the pieces of one (sequence, query head): weights l_p * 2^(m_p - M).  Also writes
// the zero rows of empty sequences, which no wave visits.
template <int QT, int KT, int D, int G>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeArgs a)
{
    const int row_id = blockIdx.x;  // s * Hq + h
    const int s = row_id / a.num_heads;
    const int h = row_id % a.num_heads;
    const int g = h / G, hg = h % G;
    const int lane = threadIdx.x;
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; j++) acc[j] = 0.0f;
    float L = 0.0f;
    if (seq_ctx(a, s) > 0) {
        const int64_t run = (int64_t)s * a.num_kv_heads + g;
        const int64_t k0 = a.run_info[2 * run];
        const int np = a.run_info[2 * run + 1];
        // whole run: written by the streaming kernel (the other checks only reject a workspace
        // the streaming kernel has not filled)
        if (np <= 1 || k0 < 0 || run + k0 + np > a.max_pieces) return;
        const int64_t p0 = run + k0;
        float M = -FLT_MAX;
        for (int p = 0; p < np; p++) M = __builtin_fmaxf(M, a.ml_part[((p0 + p) * G + hg) * 2]);
        for (int p = 0; p < np; p++) {
            const float* ml = a.ml_part + ((p0 + p) * G + hg) * 2;
            const float wgt = ml[1] * fast_exp2(ml[0] - M);
            L += wgt;
            const float* op = a.o_part + ((p0 + p) * G + hg) * D;
#pragma unroll
            for (int j = 0; j < PER; j++) acc[j] = __builtin_fmaf(wgt, op[lane + 64 * j], acc[j]);
        }
    }
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
hipError_t launch_phase_t(int phase, const DecodeArgs& a, hipStream_t stream)
{
    if ((phase & 1) && a.grid_workgroups > 0) {
        hipLaunchKernelGGL((decode_stream_kernel<QT, KT, D, G, kPipelineDepth>), dim3((unsigned)a.grid_workgroups),
                           dim3(kDecodeThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 2) {
        const int64_t grid = (int64_t)a.num_seqs * a.num_heads;
        if (grid <= 0) return hipSuccess;
        if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL((decode_merge_kernel<QT, KT, D, G>), dim3((unsigned)grid), dim3(64), 0, stream, a);
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

}  // namespace

hipError_t launch_decode(int phase, int q_dtype, int cache_dtype, int head_dim, int gqa, const DecodeArgs& a,
                         hipStream_t stream)
{
    if (q_dtype == kF32 && cache_dtype == kF32) return launch_d<kF32, kF32>(phase, head_dim, gqa, a, stream);
    if (q_dtype == kBF16 && cache_dtype == kBF16) return launch_d<kBF16, kBF16>(phase, head_dim, gqa, a, stream);
    if (q_dtype == kBF16 && cache_dtype == kFP8) return launch_d<kBF16, kFP8>(phase, head_dim, gqa, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
