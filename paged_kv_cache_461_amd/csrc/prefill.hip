// prefill.hip -- chunked-prefill PagedAttention on the gfx950 matrix cores.
//
// A chunk of q_len new positions of a sequence attends causally over that sequence's paged
// cache: row i sits at position p_i = context_len - q_len + i (the chunk is the last q_len
// positions of the context) and sees positions 0..p_i.  Pages: page 1, section 12 (chunked
// prefill: a long prompt is split into chunks that are scheduled together with decode rows);
// page 3, section 2.3 (chunked prefill batched with decode); the attention itself is the
// softmax(QK^T * scale)V of page 1, section 2, read block by block through the block table
// (page 1, section 4; page 3, section 2.1).
//
// Unlike decode, a chunk makes QK^T and PV real dense tiles, so this path runs on MFMA:
//   * Rows are "stacked": for kv head g the G query heads of every position form G rows, so a
//     16-row MFMA tile is 16/G positions x G heads and every K/V element loaded serves all
//     G heads.
//   * One workgroup = 4 waves = 128 stacked rows of one (sequence, kv head), over one key
//     range (split).  Each iteration stages 64 keys (4 blocks) of K and V in LDS as bf16
//     (an fp8 cache is widened exactly: every E4M3 value is a bf16 value), double-buffered, with
//     the next iteration's global loads in flight during the math.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 channels from LDS, B = the
//     wave's query rows held in VGPRs).  Keys are laid out in LDS so that the S^T accumulator
//     of lane l already holds the 8 keys that lane needs as the B operand of
//     O^T += V^T P^T, so P never leaves the registers.
//   * Online softmax in base 2 (scores times scale*log2(e), times k_scale for fp8), with the
//     running max only moved when a row's max grows by more than 8 (p stays <= 256).
//   * Keys split over several workgroups (split-K) when the grid would otherwise not fill the
//     GPU; a merge kernel combines the partial rows.
#include <type_traits>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = kPrefillThreads / 64;
constexpr int kPfKeys = 64;           // keys per iteration: 4 blocks of 16
constexpr float kPfInitMax = -1e30f;  // running max before any visible key (finite: no inf-inf)
constexpr float kPfMargin = 8.0f;     // lazy rescale threshold, base 2

template <int D>
struct PfLds {
    static constexpr int KS = D + 8;         // K row stride in bf16 (16 B pad against bank conflicts)
    static constexpr int VS = kPfKeys + 8;   // V^T row stride in bf16
    static constexpr int K_ELEMS = kPfKeys * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
};

__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Keep the first n bf16 of an 8-element group (n may be <= 0 or >= 8), zero the rest.
__device__ __forceinline__ u32x4_t keep_bf16(u32x4_t v, int n)
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int t = 2 * i;
        v[i] = t + 1 < n ? v[i] : t < n ? (v[i] & 0xFFFFu) : 0u;
    }
    return v;
}

// Channel order inside an LDS K row, in chunks of 8 channels.  The products read chunk
// position 4*st + grp (step st, lane group grp) and the query fragments follow the same
// order, so any permutation is valid; for head_dim 128 it is chosen so that the 16 lanes of
// a staging store (4 tokens x 4 pieces) hit distinct LDS banks: pieces of one token land 4
// positions (64 bytes) apart.  fp8: lane piece = 16 channels 64*slice + 16*q .. (two chunks);
// bf16: lane piece = 8 channels 32*slice + 8*q.
template <int KT, int D>
__device__ __forceinline__ int k_pos_of_chunk(int c8)
{
    if constexpr (D != 128) return c8;
    else if constexpr (kIsQuant<KT>) return 4 * ((c8 & 7) >> 1) + 2 * (c8 >> 3) + (c8 & 1);
    else return 4 * (c8 & 3) + (c8 >> 2);
}
template <int KT, int D>
__device__ __forceinline__ int k_chunk_of_pos(int p)
{
    if constexpr (D != 128) return p;
    else if constexpr (kIsQuant<KT>) return 8 * ((p & 3) >> 1) + 2 * (p >> 2) + (p & 1);
    else return 4 * (p & 3) + (p >> 2);
}

// LDS fragments of a product loop are read kRing ahead of the MFMAs that use them.
constexpr int kRing = 4;

// Scheduling hint for such a loop over N fragments with R products each: kRing reads, then
// (R products, one read) while reads remain, then the last kRing x R products.
template <int N, int R>
__device__ __forceinline__ void ring_schedule()
{
    __builtin_amdgcn_sched_group_barrier(0x100, kRing, 0);
#pragma unroll
    for (int i = 0; i < N - kRing; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, R, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < kRing; i++) __builtin_amdgcn_sched_group_barrier(0x008, R, 0);
}

// LDS row of key o of block b (0..3) of an iteration: tile u = o / 4 of the S^T product reads
// rows 16u .. 16u+15, and its row 4q + j is key 16q + 4u + j (block q, token 4u + j).
__device__ __forceinline__ int k_lds_row(int b, int o) { return 16 * (o >> 2) + 4 * b + (o & 3); }

// B8: the 8-token-block form (bf16 cache only), a separate instance so that its second table
// entry per unit costs the other block sizes nothing.
template <int KT, int D, int G, int R, bool B8>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillArgs a)
{
    using L = PfLds<D>;
    constexpr int EB = kIsQuant<KT> ? 1 : 2;
    constexpr int TILE_BYTES = kUnitTokens * D * EB;  // one 16-token unit of one kv head
    constexpr int CH_PER_TILE = TILE_BYTES / 16;     // 16-byte pieces per tile
    constexpr int NCH = 4 * CH_PER_TILE / kPrefillThreads;  // K (and V) pieces per thread per iteration
    constexpr int ROWS = kPfWaves * R * 16;          // stacked rows per workgroup
    constexpr int POS = ROWS / G;                    // positions per workgroup
    constexpr int ND = D / 16;                       // 16-channel tiles of O^T
    constexpr int NS = D / 32;                       // 32-channel steps of Q K^T
    static_assert(NCH >= 1 && 4 * CH_PER_TILE % kPrefillThreads == 0, "tile split");
    static_assert(16 % G == 0, "a 16-row tile holds whole positions");

    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * L::STAGE];

    // ---- work item: (sequence, kv head, row block, split); items of one (sequence, kv head)
    // are consecutive, and with a grid that is a multiple of 8 consecutive items go to one XCD
    // (workgroups are dealt round-robin over the 8 XCDs), so they share that XCD's L2.
    const int nwg = gridDim.x;
    int t = (nwg & 7) == 0 ? (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int split = t % a.num_splits;
    t /= a.num_splits;
    const int rb = t % a.row_blocks;
    t /= a.row_blocks;
    const int g = t % a.num_kv_heads;
    const int s = t / a.num_kv_heads;

    // values loaded once per workgroup: readfirstlane keeps them (and all loop control derived
    // from them) in scalar registers
    const int q0 = __builtin_amdgcn_readfirstlane(a.cu_query_lens[s]);
    int qlen = __builtin_amdgcn_readfirstlane(a.cu_query_lens[s + 1]) - q0;
    if (q0 < 0 || qlen < 0 || q0 > a.num_query_rows - qlen) qlen = 0;  // rows outside the query array
    const int i_first = rb * POS;
    if (i_first >= qlen) return;  // uniform over the workgroup
    const int i_last = min(i_first + POS, qlen) - 1;
    const int ctx = min(max(__builtin_amdgcn_readfirstlane(a.context_lens[s]), 0), a.max_context_len);
    const int past = ctx - qlen;  // positions before the chunk
    const int kend = max(past + i_last + 1, 0);  // keys any row of the workgroup sees

    // key range of this split: fixed-size partitions, or kend cut into num_splits equal parts
    int per = a.split_keys;
    if (per <= 0) per = ((kend + a.num_splits - 1) / a.num_splits + kPfKeys - 1) / kPfKeys * kPfKeys;
    const int kbeg = __builtin_amdgcn_readfirstlane(min(split * per, kend));
    const int kstop = __builtin_amdgcn_readfirstlane(min(kbeg + per, kend));
    const int niter = (kstop - kbeg + kPfKeys - 1) / kPfKeys;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;  // query row of the lane inside a 16-row tile
    const int grp = lane >> 4;  // lane group: 8-element k slice of the MFMA operands

    // ---- the wave's rows: tile rho, lane col -> stacked row, position, head
    const int Hq = a.num_heads;
    int prow[R];
    int64_t orow[R];  // (query row * Hq + head) of the lane's row, -1 if it is padding
    bf16x8_t qb[R][NS];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int rst = 16 * (R * w + r) + col;
        const int i = i_first + rst / G;
        const int h = g * G + rst % G;
        const bool valid = i <= i_last;
        prow[r] = valid ? past + i : -1;
        orow[r] = valid ? (int64_t)(q0 + i) * Hq + h : -1;
        const __bf16* qp = static_cast<const __bf16*>(a.query) + (valid ? orow[r] : 0) * D;
#pragma unroll
        for (int st = 0; st < NS; st++)
            qb[r][st] = as_bf16x8(valid ? load16(qp + 8 * k_chunk_of_pos<KT, D>(4 * st + grp)) : make_uint4(0, 0, 0, 0));
    }
    // wave-uniform bounds of the rows' visible keys (padding rows count as seeing nothing)
    const int wi_lo = i_first + (16 * R * w) / G, wi_hi = i_first + (16 * R * w + 16 * R - 1) / G;
    const int pw_max = wi_lo <= i_last ? past + min(wi_hi, i_last) : -1;
    const int pw_min = wi_hi <= i_last ? past + wi_lo : -1;
    // last key each row may use: its causal limit, and never past this split's range
    int klim[R];
#pragma unroll
    for (int r = 0; r < R; r++) klim[r] = min(prow[r], kstop - 1);
    const int kw_min = min(pw_min, kstop - 1);

    const float sc = a.scale_log2 * (kIsQuant<KT> ? a.k_scale[g] : 1.0f);
    const float vsc = kIsQuant<KT> ? a.v_scale[g] : 1.0f;

    f32x4_t o[R][ND];
    float m[R], l[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        m[r] = kPfInitMax;
        l[r] = 0.0f;
#pragma unroll
        for (int d = 0; d < ND; d++) o[r][d] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // ---- staging: thread tid owns pieces tid + 256 j of the iteration's 4 K tiles and 4 V tiles
    const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool);
    const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool);
    const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // NSET register sets: the loads for iteration it + NSET are in flight while it is computed
    // (two sets measured no faster than one on the 512-row fp8 chunk, so one)
    constexpr int NSET = 1;
    uint4 kr[NSET][NCH], vr[NSET][NCH];
    uint32_t okbits[NSET] = {};  // bit j: piece j comes from a block that holds tokens of the range
    __shared__ int blk_ok[2][4];  // per buffer: block b of the iteration has a valid table entry

    // The block of piece j is the same for all 64 lanes of a wave (a tile is a whole number of
    // 1 KiB wave loads), so its checks are uniform.  Each load() fetches the table entries the
    // next load() needs, unconditionally (the index is clamped to the range's last block), so
    // a K/V load never waits on a table read.
    static_assert(CH_PER_TILE % 64 == 0, "wave-uniform block per piece");
    // A block of 16 << ub tokens holds 1 << ub units; unit u of the range is unit u & ub of
    // table entry u >> ub.  Inside a 32-token block's tile, unit `sub` has its K slices at
    // sub * 1 KiB + slice * (B * 64) and its V at sub * TILE_BYTES (include/pagedattn.h).
    // 8-token blocks (bf16 cache only): unit u is blocks 2u (tokens 0..7) and 2u+1 (8..15).
    const int ub = a.block_size > kUnitTokens ? 1 : 0;
    constexpr bool b8 = B8;
    static_assert(!B8 || KT == kBF16, "8-token blocks with a bf16 cache only");
    const int kstride = a.block_size * 64;
    const int64_t btile = (int64_t)a.block_size * D * EB;  // bytes of one (block, kv head) tile
    const int last_unit = kstop > 0 ? (kstop - 1) >> 4 : 0;
    const int last_b8 = kstop > 0 ? (kstop - 1) >> 3 : 0;
    int ent[NCH], ent8[B8 ? NCH : 1];  // ent8: the unit's second 8-token block
    auto fetch_entries = [&](int kbase) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NCH; j++) {
            const int b = __builtin_amdgcn_readfirstlane((tid + kPrefillThreads * j) / CH_PER_TILE);
            const int u = (kbase >> 4) + b;
            if constexpr (b8) {
                ent[j] = table[min(2 * u, last_b8)];
                ent8[j] = table[min(2 * u + 1, last_b8)];
            } else {
                ent[j] = table[min(u, last_unit) >> ub];
            }
        }
    };
    auto load = [&](auto set_tag, int kbase) __attribute__((always_inline)) {
        constexpr int SET = decltype(set_tag)::value;
        okbits[SET] = 0;
#pragma unroll
        for (int j = 0; j < NCH; j++) {
            const int c = tid + kPrefillThreads * j;
            const int b = __builtin_amdgcn_readfirstlane(c / CH_PER_TILE);
            const int off = (c % CH_PER_TILE) * 16;
            const int phys = __builtin_amdgcn_readfirstlane(ent[j]);
            const bool ok = kbase + 16 * b < kstop && phys >= 0 && (int64_t)phys < a.num_blocks;
            // a block with no valid entry still reads block 0 (the pool has one); store() zeroes it
            if constexpr (b8) {
                const int phys2 = __builtin_amdgcn_readfirstlane(ent8[j]);
                const bool ok2 = kbase + 16 * b + 8 < kstop && phys2 >= 0 && (int64_t)phys2 < a.num_blocks;
                const int64_t t1 = ((int64_t)(ok ? phys : 0) * a.num_kv_heads + g) * btile;
                const int64_t t2 = ((int64_t)(ok2 ? phys2 : 0) * a.num_kv_heads + g) * btile;
                // K: the piece's token (off >> 6 within its 1 KiB slice) picks the block
                const int tok = (off & 1023) >> 6;
                kr[SET][j] = load16(kpool + (tok < 8 ? t1 : t2) + (off >> 10) * kstride + (tok & 7) * 64 + (off & 63));
                // V: 8-token group og of the unit is block og; the piece is channel (off >> 4) % D
                const int og = (off >> 4) / D;
                vr[SET][j] = load16(vpool + (og ? t2 : t1) + (off - og * D * 16));
            } else {
                const int sub = ((kbase >> 4) + b) & ub;
                const int64_t tile = ((int64_t)(ok ? phys : 0) * a.num_kv_heads + g) * btile;
                kr[SET][j] = load16(kpool + tile + sub * 1024 + (off >> 10) * kstride + (off & 1023));
                vr[SET][j] = load16(vpool + tile + sub * TILE_BYTES + off);
            }
            okbits[SET] |= ok ? 1u << j : 0u;
        }
        fetch_entries(kbase + kPfKeys);  // for the next load, one compute phase away
    };

    // Convert and place piece j.  MASK: zero tokens at or past nval of the piece's block (the
    // range end, or the whole block when its table entry is invalid).
    auto put = [&](auto mask_tag, auto set_tag, int j, __bf16* kl, __bf16* vl, int buf, int kbase) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int SET = decltype(set_tag)::value;
        const int c = tid + kPrefillThreads * j;
        const int b = c / CH_PER_TILE;
        const int off = (c % CH_PER_TILE) * 16;
        const bool blk = okbits[SET] >> j & 1u;
        if (off == 0) blk_ok[buf][b] = blk;  // one piece per block starts it
        const int nval = MASK ? (blk ? min(kstop - (kbase + 16 * b), 16) : 0) : 16;  // valid tokens
        // K: 64-byte channel slices, token-major: a piece is 16 bytes of one token
        const int slice = off >> 10;
        const int tok = (off & 1023) >> 6;
        __bf16* krow = kl + k_lds_row(b, tok) * L::KS;
        const bool kzero = MASK && tok >= nval;
        if constexpr (kIsQuant<KT>) {
            const int c8 = (64 * slice + (off & 63)) >> 3;
            const uint4 w = kr[SET][j];
            u32x4_t lo = {q8x2_to_bf16x2<KT, false>(w.x), q8x2_to_bf16x2<KT, true>(w.x), q8x2_to_bf16x2<KT, false>(w.y),
                          q8x2_to_bf16x2<KT, true>(w.y)};
            u32x4_t hi = {q8x2_to_bf16x2<KT, false>(w.z), q8x2_to_bf16x2<KT, true>(w.z), q8x2_to_bf16x2<KT, false>(w.w),
                          q8x2_to_bf16x2<KT, true>(w.w)};
            if (kzero) lo = hi = u32x4_t{0, 0, 0, 0};
            *reinterpret_cast<u32x4_t*>(krow + 8 * k_pos_of_chunk<KT, D>(c8)) = lo;
            *reinterpret_cast<u32x4_t*>(krow + 8 * k_pos_of_chunk<KT, D>(c8 + 1)) = hi;
            // V: 16 tokens of channel d side by side
            const int d = off >> 4;
            const uint4 v = vr[SET][j];
            u32x4_t vlo = {q8x2_to_bf16x2<KT, false>(v.x), q8x2_to_bf16x2<KT, true>(v.x), q8x2_to_bf16x2<KT, false>(v.y),
                           q8x2_to_bf16x2<KT, true>(v.y)};
            u32x4_t vhi = {q8x2_to_bf16x2<KT, false>(v.z), q8x2_to_bf16x2<KT, true>(v.z), q8x2_to_bf16x2<KT, false>(v.w),
                           q8x2_to_bf16x2<KT, true>(v.w)};
            if constexpr (MASK) {
                vlo = keep_bf16(vlo, nval);
                vhi = keep_bf16(vhi, nval - 8);
            }
            *reinterpret_cast<u32x4_t*>(vl + d * L::VS + 16 * b) = vlo;
            *reinterpret_cast<u32x4_t*>(vl + d * L::VS + 16 * b + 8) = vhi;
        } else {
            const int c8 = (32 * slice + ((off & 63) >> 1)) >> 3;
            u32x4_t k = __builtin_bit_cast(u32x4_t, kr[SET][j]);
            if (kzero) k = u32x4_t{0, 0, 0, 0};
            *reinterpret_cast<u32x4_t*>(krow + 8 * k_pos_of_chunk<KT, D>(c8)) = k;
            // V: groups of 8 tokens, channel-major
            const int gi = off >> 4;
            const int og = gi / D, d = gi % D;
            u32x4_t v = __builtin_bit_cast(u32x4_t, vr[SET][j]);
            if constexpr (MASK) v = keep_bf16(v, nval - 8 * og);
            *reinterpret_cast<u32x4_t*>(vl + d * L::VS + 16 * b + 8 * og) = v;
        }
    };
    auto store = [&](auto set_tag, int buf, int kbase) __attribute__((always_inline)) {
        constexpr int SET = decltype(set_tag)::value;
        __bf16* kl = lds + buf * L::STAGE;
        __bf16* vl = kl + L::K_ELEMS;
        // all four blocks valid and inside the range: no token to zero (wave-uniform)
        if (kbase + kPfKeys <= kstop && okbits[SET] == (1u << NCH) - 1) {
#pragma unroll
            for (int j = 0; j < NCH; j++) put(std::false_type{}, set_tag, j, kl, vl, buf, kbase);
        } else {
#pragma unroll
            for (int j = 0; j < NCH; j++) put(std::true_type{}, set_tag, j, kl, vl, buf, kbase);
        }
    };

    // Iteration it: stage set it % NSET into LDS buffer it % 2, barrier, issue the loads of
    // iteration it + NSET into the freed set (unconditionally: past the range they read block 0
    // and are never stored), then compute on the buffer.
    auto compute = [&](int buf, int kbase) __attribute__((always_inline)) {
        if (kbase > pw_max) return;  // every row of this wave is done (uniform)
        // keys of block grp that have no valid table entry are masked like causal ones
        const bool blk_valid = blk_ok[buf][grp] != 0;
        const bool need_mask = kbase + kPfKeys - 1 > kw_min || __builtin_amdgcn_ballot_w64(!blk_valid) != 0;
        const int key0 = kbase + 16 * grp;  // the lane's keys are key0 + 4u + j
        const __bf16* kl = lds + buf * L::STAGE;
        const __bf16* vl = kl + L::K_ELEMS;

        // S^T tiles: sacc[r][u] = keys of tile u x query rows of tile r.  Fragment i = (step
        // i / 4, tile i % 4) is read kRing fragments ahead of its products.
        f32x4_t sacc[R][4];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int u = 0; u < 4; u++) sacc[r][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        auto kread = [&](int i) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8_t*>(kl + (16 * (i & 3) + col) * L::KS + 32 * (i >> 2) + 8 * grp);
        };
        {
            bf16x8_t kf[kRing];
#pragma unroll
            for (int i = 0; i < kRing; i++) kf[i] = kread(i);
#pragma unroll
            for (int i = 0; i < 4 * NS; i++) {
#pragma unroll
                for (int r = 0; r < R; r++) sacc[r][i & 3] = mfma_16x16x32(kf[i % kRing], qb[r][i >> 2], sacc[r][i & 3]);
                if (i + kRing < 4 * NS) kf[i % kRing] = kread(i + kRing);
            }
            ring_schedule<4 * NS, R>();
        }

        // online softmax; lane holds keys 16*grp + 4u + j of its row
        bf16x8_t pb[R][2];
#pragma unroll
        for (int r = 0; r < R; r++) {
            // raw scores; the scale (> 0) is applied to the max and inside the exponent's FMA
            float z[4][4];
            if (need_mask) {
                const int lim = blk_valid ? klim[r] - key0 : -1;  // last visible key offset
#pragma unroll
                for (int u = 0; u < 4; u++)
#pragma unroll
                    for (int j = 0; j < 4; j++) z[u][j] = 4 * u + j > lim ? -__builtin_inff() : sacc[r][u][j];
            } else {
#pragma unroll
                for (int u = 0; u < 4; u++)
#pragma unroll
                    for (int j = 0; j < 4; j++) z[u][j] = sacc[r][u][j];
            }
            float mx = -__builtin_inff();
#pragma unroll
            for (int u = 0; u < 4; u++)
                mx = __builtin_fmaxf(__builtin_fmaxf(mx, __builtin_fmaxf(z[u][0], z[u][1])),
                                     __builtin_fmaxf(z[u][2], z[u][3]));
            mx = __builtin_fmaxf(mx, swizzle_xor16(mx));
            mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
            mx *= sc;
            const bool up = mx > m[r] + kPfMargin;
            if (__builtin_amdgcn_ballot_w64(up)) {
                const float mn = up ? mx : m[r];
                const float alpha = fast_exp2(m[r] - mn);
                m[r] = mn;
                l[r] *= alpha;
#pragma unroll
                for (int d = 0; d < ND; d++) o[r][d] *= alpha;
            }
            uint32_t pw[2][4];
            float ls = l[r];
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                for (int v2 = 0; v2 < 2; v2++) {
                    const int u = 2 * h2 + v2;
                    const float nm = -m[r];
                    const uint32_t p01 = pack_bf16x2(fast_exp2(__builtin_fmaf(z[u][0], sc, nm)),
                                                     fast_exp2(__builtin_fmaf(z[u][1], sc, nm)));
                    const uint32_t p23 = pack_bf16x2(fast_exp2(__builtin_fmaf(z[u][2], sc, nm)),
                                                     fast_exp2(__builtin_fmaf(z[u][3], sc, nm)));
                    pw[h2][2 * v2] = p01;
                    pw[h2][2 * v2 + 1] = p23;
                    ls = dot2_bf16(p01, kBf16OnePair, ls);
                    ls = dot2_bf16(p23, kBf16OnePair, ls);
                }
            l[r] = ls;
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
                pb[r][h2] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[h2][0], pw[h2][1], pw[h2][2], pw[h2][3]));
        }

        // O^T += V^T P^T: V^T rows = channels, k = keys 16*grp + 8*h2 + 0..7; fragment
        // i = (half i / ND, channel tile i % ND), read kRing ahead.
        auto vread = [&](int i) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8_t*>(vl + (16 * (i % ND) + col) * L::VS + 16 * grp + 8 * (i / ND));
        };
        {
            bf16x8_t vf[kRing];
#pragma unroll
            for (int i = 0; i < kRing; i++) vf[i] = vread(i);
#pragma unroll
            for (int i = 0; i < 2 * ND; i++) {
#pragma unroll
                for (int r = 0; r < R; r++) o[r][i % ND] = mfma_16x16x32(vf[i % kRing], pb[r][i / ND], o[r][i % ND]);
                if (i + kRing < 2 * ND) vf[i % kRing] = vread(i + kRing);
            }
            ring_schedule<2 * ND, R>();
        }
    };
    auto iteration = [&](auto set_tag, int it) __attribute__((always_inline)) {
        const int kbase = kbeg + it * kPfKeys;
        store(set_tag, it & 1, kbase);
        __syncthreads();
        load(set_tag, kbase + NSET * kPfKeys);
        compute(it & 1, kbase);
    };
    fetch_entries(kbeg);
    if (niter > 0) {
        load(std::integral_constant<int, 0>{}, kbeg);
        if constexpr (NSET > 1) load(std::integral_constant<int, 1>{}, kbeg + kPfKeys);
    }
    for (int it = 0; it < niter; it += NSET) {
        iteration(std::integral_constant<int, 0>{}, it);
        if constexpr (NSET > 1)
            if (it + 1 < niter) iteration(std::integral_constant<int, 1>{}, it + 1);
    }

    // ---- epilogue: lane holds channels 16d + 4*grp + 0..3 of its row
#pragma unroll
    for (int r = 0; r < R; r++) {
        float lt = l[r];
        lt += swizzle_xor16(lt);
        lt += __shfl_xor(lt, 32, 64);
        if (orow[r] < 0) continue;
        if (a.num_splits == 1) {
            const float inv = lt > 0.0f ? vsc / lt : 0.0f;
            __bf16* op = static_cast<__bf16*>(a.out) + orow[r] * D + 4 * grp;
#pragma unroll
            for (int d = 0; d < ND; d++) {
                const uint2 v = make_uint2(pack_bf16x2(o[r][d][0] * inv, o[r][d][1] * inv),
                                           pack_bf16x2(o[r][d][2] * inv, o[r][d][3] * inv));
                *reinterpret_cast<uint2*>(op + 16 * d) = v;
            }
        } else {
            const int64_t prow_idx = (int64_t)split * a.num_query_rows * Hq + orow[r];
            float* op = a.o_part + prow_idx * D + 4 * grp;
#pragma unroll
            for (int d = 0; d < ND; d++) {
                const f32x4_t v = o[r][d] * vsc;
                *reinterpret_cast<f32x4_t*>(op + 16 * d) = v;
            }
            if (grp == 0) *reinterpret_cast<f32x2_t*>(a.ml_part + 2 * prow_idx) = f32x2_t{m[r], lt};
        }
    }
}

// Combine the splits of every (query row, head): M = max_k m_k, w_k = 2^(m_k - M),
// out = sum_k w_k o_k / sum_k w_k l_k (o_k already times v_scale).  One wave per row-head.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a)
{
    const int64_t n = (int64_t)a.num_query_rows * a.num_heads;
    const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (idx >= n) return;
    const int lane = threadIdx.x & 63;
    constexpr int PER = D / 64;
    float mm = -__builtin_inff();
    for (int k = 0; k < a.num_splits; k++) mm = __builtin_fmaxf(mm, a.ml_part[2 * (k * n + idx)]);
    float lsum = 0.0f, acc[PER] = {};
    for (int k = 0; k < a.num_splits; k++) {
        const float* ml = a.ml_part + 2 * (k * n + idx);
        const float wk = fast_exp2(ml[0] - mm);
        lsum += wk * ml[1];
        const float* op = a.o_part + (k * n + idx) * D;
#pragma unroll
        for (int e = 0; e < PER; e++) acc[e] += wk * op[lane + 64 * e];
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    __bf16* out = static_cast<__bf16*>(a.out) + idx * D;
#pragma unroll
    for (int e = 0; e < PER; e++) out[lane + 64 * e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(acc[e] * inv));
}

template <int KT, int D, int G>
hipError_t launch_one(const PrefillArgs& a, int grid, hipStream_t stream)
{
    if (a.block_size < kUnitTokens) {
        if constexpr (KT == kBF16)
            hipLaunchKernelGGL((prefill_kernel<KT, D, G, kPrefillRowTiles, true>), dim3((unsigned)grid),
                               dim3(kPrefillThreads), 0, stream, a);
        else
            return hipErrorInvalidValue;  // rejected by the host checks before this point
    } else {
        hipLaunchKernelGGL((prefill_kernel<KT, D, G, kPrefillRowTiles, false>), dim3((unsigned)grid),
                           dim3(kPrefillThreads), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits == 1) return e;
    const int64_t n = (int64_t)a.num_query_rows * a.num_heads;
    hipLaunchKernelGGL((prefill_merge_kernel<D>), dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int KT, int D>
hipError_t launch_g(int gqa, const PrefillArgs& a, int grid, hipStream_t stream)
{
    switch (gqa) {
    case 1: return launch_one<KT, D, 1>(a, grid, stream);
    case 2: return launch_one<KT, D, 2>(a, grid, stream);
    case 4: return launch_one<KT, D, 4>(a, grid, stream);
    case 8: return launch_one<KT, D, 8>(a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(int cache_dtype, int head_dim, int gqa, const PrefillArgs& a, int64_t grid,
                          hipStream_t stream)
{
    if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (cache_dtype == kFP8) {
        if (head_dim == 128) return launch_g<kFP8, 128>(gqa, a, (int)grid, stream);
        if (head_dim == 64) return launch_g<kFP8, 64>(gqa, a, (int)grid, stream);
    } else if (cache_dtype == kE5M2) {
        if (head_dim == 128) return launch_g<kE5M2, 128>(gqa, a, (int)grid, stream);
        if (head_dim == 64) return launch_g<kE5M2, 64>(gqa, a, (int)grid, stream);
    } else if (cache_dtype == kI8) {
        if (head_dim == 128) return launch_g<kI8, 128>(gqa, a, (int)grid, stream);
        if (head_dim == 64) return launch_g<kI8, 64>(gqa, a, (int)grid, stream);
    } else if (cache_dtype == kBF16) {
        if (head_dim == 128) return launch_g<kBF16, 128>(gqa, a, (int)grid, stream);
        if (head_dim == 64) return launch_g<kBF16, 64>(gqa, a, (int)grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
