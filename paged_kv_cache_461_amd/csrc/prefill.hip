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
//   * One workgroup = 8 waves = 256 stacked rows of one (sequence, kv head), over one key
//     range (split), one workgroup per CU.  Each iteration stages 64 keys (4 blocks) of K and V
//     in LDS as bf16 (an 8-bit cache is widened exactly: every E4M3, E5M2 and INT8 value is a
//     bf16 value), in three stages, with the loads of later tiles in flight.
//   * The waves form two groups, one wave of each per SIMD, that alternate a matrix phase (the
//     PV product of the previous tile and the QK^T product of this one, then the staging) and a
//     vector phase (the softmax), one phase apart: while one wave of a SIMD issues MFMAs the
//     other runs its exponentials.
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

// LDS layouts, chosen from measured gfx950 bank behaviour: a ds_read_b128 is conflict-free when
// the 32 lanes of each half-wave hit distinct 16-byte chunks modulo 32 (a 512-byte window), a
// ds_write_b128 when each 16 lanes hit distinct chunks modulo 16.  K rows of D + 16 bf16 (288 B
// for D = 128) put the 16 rows x 2 lane groups of a half-wave's fragment read on 32 distinct
// chunks.  V^T rows are 64 keys (128 B) unpadded, with the 8-key chunks of row d permuted by
// v_pos so that both the fragment reads (16 rows x 2 chunks) and the staging stores (16
// consecutive rows, one chunk) spread over distinct banks.
template <int D>
struct PfLds {
    static constexpr int KS = D + 16;    // K row stride in bf16
    static constexpr int VS = kPfKeys;   // V^T row stride in bf16
    static constexpr int K_ELEMS = kPfKeys * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
};
static_assert(kPfKeys == 64, "v_pos permutes the 8 key chunks of a 64-key V^T row");

// Position (in 8-key chunks) of V^T key chunk kc of channel row d.  Lane group grp reads keys
// 16 grp + 8 h .. + 7 for k-step h; the chunks of one k-step sit side by side so that the two
// lane groups of a half-wave read adjacent positions, and the XOR with bits 1..3 of d turns
// the 128-byte row stride into distinct banks for 16 consecutive rows.
__device__ __forceinline__ int v_pos(int kc, int d) { return ((kc >> 1) + 4 * (kc & 1)) ^ ((d >> 1) & 7); }

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
// a staging store (4 tokens x 4 pieces, rows 18 chunks apart) hit distinct chunks modulo 16:
// the 4 pieces q of one token land on chunks {0, 8, 1, 9} + const.  bf16: lane piece = chunk
// c8 = 4 slice + q; 8-bit caches: lane piece = chunks c8 = 8 slice + 2 q + h, h = 0, 1.
template <int KT, int D>
__device__ __forceinline__ int k_pos_of_chunk(int c8)
{
    if constexpr (D != 128) {
        return c8;
    } else if constexpr (kIsQuant<KT>) {
        const int sl = c8 >> 3, q = (c8 >> 1) & 3, h = c8 & 1;
        return 8 * (q & 1) + (q >> 1) + 4 * sl + 2 * h;
    } else {
        const int sl = c8 >> 2, q = c8 & 3;
        return 8 * (q & 1) + (q >> 1) + 2 * sl;
    }
}
template <int KT, int D>
__device__ __forceinline__ int k_chunk_of_pos(int p)
{
    if constexpr (D != 128) {
        return p;
    } else if constexpr (kIsQuant<KT>) {
        const int q = 2 * (p & 1) + (p >> 3), h = (p >> 1) & 1, sl = (p >> 2) & 1;
        return 8 * sl + 2 * q + h;
    } else {
        const int q = 2 * (p & 1) + (p >> 3), sl = (p >> 1) & 3;
        return 4 * sl + q;
    }
}

// One step of a max over the four 16-lane groups (lanes l, l^16, l^32, l^48), on the VALU:
// v_permlane16_swap pairs each 16-lane row with its neighbour (halves = false), then
// v_permlane32_swap each half of the wave with the other (halves = true); after a swap of two copies of x, one copy holds each lane's own value and
// the other its partner's.  (A ds_swizzle / ds_bpermute round trip would queue behind the
// other waves' fragment reads in the LDS.)
__device__ __forceinline__ float swap_max(float x, bool halves)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto p = halves ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                          : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t p0 = p[0], p1 = p[1];  // (a bit_cast of the vector elements themselves
                                          // reads element 0 twice with this compiler)
    return __builtin_fmaxf(__builtin_bit_cast(float, p0), __builtin_bit_cast(float, p1));
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

// LDS stages of K/V tiles: tile t sits in stage t % kPfStages (see the slot schedule below).
constexpr int kPfStages = 3;

// s_waitcnt immediate that waits for vector memory only: vmcnt = 0 (bits 3:0 and 15:14),
// expcnt and lgkmcnt at their maxima; OR a count of at most 15 into bits 3:0 to leave that many
// of the newest loads in flight.
constexpr int kWaitVm = 0x0F70;

// Workgroup barrier that orders LDS only: the release waits for this wave's LDS stores, the
// acquire keeps later LDS reads behind the barrier, and global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// B8: the 8-token-block form, a separate instance so that its second table entry per unit costs
// the other block sizes nothing.
//
// Ping-pong schedule.  The 8 waves form two groups, A = waves 0..3 and B = waves 4..7, one wave
// of each per SIMD.  Each wave alternates two phases per iteration it: M(it) on the matrix
// cores (PV of tile it - 1, QK of tile it, then the staging of tile it + 1 into LDS and the
// global loads of tile it + 3) and S(it) on the vector ALUs (the online softmax of tile it).
// Phases end at a workgroup barrier and group B runs one phase behind group A:
//     slot 2it:   A M(it)   B S(it-1)
//     slot 2it+1: A S(it)   B M(it)
// Tile t is written by A in slot 2t-2 and by B in slot 2t-1 and read (K by QK, V by PV) in
// slots 2t .. 2t+3, so three LDS stages never hold a tile that is read while it is rewritten.
template <int KT, int D, int G, int R, bool B8>
__global__ __launch_bounds__(kPrefillThreads, 1) void prefill_kernel(PrefillArgs a)
{
    using L = PfLds<D>;
    constexpr int EB = kIsQuant<KT> ? 1 : 2;
    constexpr int TILE_BYTES = kUnitTokens * D * EB;  // one 16-token unit of one kv head
    constexpr int CH_PER_TILE = TILE_BYTES / 16;     // 16-byte pieces per tile
    constexpr int PIECES = 4 * CH_PER_TILE;          // K (and V) pieces per iteration
    // pieces per thread; with fewer pieces than threads only the first PIECES threads stage
    constexpr int NCH = PIECES >= kPrefillThreads ? PIECES / kPrefillThreads : 1;
    constexpr int ROWS = kPfWaves * R * 16;          // stacked rows per workgroup
    constexpr int POS = ROWS / G;                    // positions per workgroup
    constexpr int ND = D / 16;                       // 16-channel tiles of O^T
    constexpr int NS = D / 32;                       // 32-channel steps of Q K^T
    static_assert(PIECES % kPrefillThreads == 0 || (kPrefillThreads % PIECES == 0 && PIECES % 64 == 0),
                  "tile split");
    static_assert(16 % G == 0, "a 16-row tile holds whole positions");

    __shared__ __attribute__((aligned(16))) __bf16 lds[kPfStages * L::STAGE];
    __shared__ int blk_ok[kPfStages][4];  // per stage: block b of the tile has a valid table entry

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
    const bool group_a = w < kPfWaves / 2;
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
    const int kw_min = __builtin_amdgcn_readfirstlane(min(pw_min, kstop - 1));

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

    // ---- staging: thread tid owns pieces tid + 512 j of a tile's 4 K units and 4 V units
    const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool);
    const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool);
    // the block table is read-only here: reading it through the constant address space makes
    // its (wave-uniform) reads scalar loads, which the vector-load waits below do not count
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const_i32* table = (const_i32*)(a.block_tables + (int64_t)s * a.max_blocks_per_seq);
    const bool stager = PIECES >= kPrefillThreads || tid < PIECES;  // wave-uniform
    // Register sets of loaded pieces: with two, set t % 2 holds tile t from
    // its load (staging of iteration t - 3) to its LDS store (staging of iteration t - 1); a bf16
    // cache with head_dim 128 has twice the pieces per thread and keeps one set (tile t loaded
    // in the staging of iteration t - 2), which fits its registers.
    constexpr int NSETS = (KT == kBF16 && D == 128) ? 1 : 2;
    uint4 kr[NSETS][NCH], vr[NSETS][NCH];
    uint32_t okbits[NSETS] = {};  // bit j: piece j comes from a block that holds tokens of the range

    // The block of piece j is the same for all 64 lanes of a wave (a tile is a whole number of
    // 1 KiB wave loads), so its checks are uniform.  The table entries a load() needs are read
    // one iteration ahead by fetch_entries() (index clamped to the range's last block).
    static_assert(CH_PER_TILE % 64 == 0, "wave-uniform block per piece");
    // A block of 16 << ub tokens holds 1 << ub units; unit u of the range is unit u & ub of
    // table entry u >> ub.  Inside a 32-token block's tile, unit `sub` has its K slices at
    // sub * 1 KiB + slice * (B * 64) and its V at sub * TILE_BYTES (include/pagedattn.h).
    // 8-token blocks: unit u is blocks 2u (tokens 0..7) and 2u+1 (8..15).
    const int ub = a.block_size > kUnitTokens ? 1 : 0;
    constexpr bool b8 = B8;
    const int kstride = a.block_size * 64;
    const int64_t btile = (int64_t)a.block_size * D * EB;  // bytes of one (block, kv head) tile
    const int last_unit = kstop > 0 ? (kstop - 1) >> 4 : 0;
    const int last_b8 = kstop > 0 ? (kstop - 1) >> 3 : 0;
    int ent[NCH], ent8[B8 ? NCH : 1];  // ent8: the unit's second 8-token block
    auto fetch_entries = [&](int kbase) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NCH; j++) {
            const int b = __builtin_amdgcn_readfirstlane((tid + kPrefillThreads * j) / CH_PER_TILE) & 3;
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
        constexpr int SET = decltype(set_tag)::value % NSETS;
        okbits[SET] = 0;
#pragma unroll
        for (int j = 0; j < NCH; j++) {
            const int c = tid + kPrefillThreads * j;
            const int b = __builtin_amdgcn_readfirstlane(c / CH_PER_TILE) & 3;
            const int off = (c % CH_PER_TILE) * 16;
            const int phys = __builtin_amdgcn_readfirstlane(ent[j]);
            const bool ok = kbase + 16 * b < kstop && phys >= 0 && (int64_t)phys < a.num_blocks;
            // a block with no valid entry still reads block 0 (the pool has one); put() zeroes it
            if constexpr (b8) {
                const int phys2 = __builtin_amdgcn_readfirstlane(ent8[j]);
                const bool ok2 = kbase + 16 * b + 8 < kstop && phys2 >= 0 && (int64_t)phys2 < a.num_blocks;
                const int64_t t1 = ((int64_t)(ok ? phys : 0) * a.num_kv_heads + g) * btile;
                const int64_t t2 = ((int64_t)(ok2 ? phys2 : 0) * a.num_kv_heads + g) * btile;
                // K: the piece's token (off >> 6 within its 1 KiB slice) picks the block
                const int tok = (off & 1023) >> 6;
                kr[SET][j] = load16(kpool + (tok < 8 ? t1 : t2) + (off >> 10) * kstride + (tok & 7) * 64 + (off & 63));
                if constexpr (kIsQuant<KT>) {
                    // V: the 16-token piece of channel d is 8 bytes (8 tokens) of each block
                    const int d = off >> 4;
                    const uint2 lo = *reinterpret_cast<const uint2*>(vpool + t1 + d * 8);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vpool + t2 + d * 8);
                    vr[SET][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                } else {
                    // V: a piece is one 8-token group; the first D pieces are block 1's
                    const int og = (off >> 4) / D;
                    vr[SET][j] = load16(vpool + (og ? t2 : t1) + (off - og * D * 16));
                }
            } else {
                const int sub = ((kbase >> 4) + b) & ub;
                const int64_t tile = ((int64_t)(ok ? phys : 0) * a.num_kv_heads + g) * btile;
                kr[SET][j] = load16(kpool + tile + sub * 1024 + (off >> 10) * kstride + (off & 1023));
                vr[SET][j] = load16(vpool + tile + sub * TILE_BYTES + off);
            }
            okbits[SET] |= ok ? 1u << j : 0u;
        }
    };

    // Convert and place piece j.  MASK: zero tokens at or past nval of the piece's block (the
    // range end, or the whole block when its table entry is invalid).
    auto put = [&](auto mask_tag, auto set_tag, int j, __bf16* kl, __bf16* vl, int stage, int kbase) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int SET = decltype(set_tag)::value % NSETS;
        const int c = tid + kPrefillThreads * j;
        const int b = (c / CH_PER_TILE) & 3;
        const int off = (c % CH_PER_TILE) * 16;
        const bool blk = okbits[SET] >> j & 1u;
        if (off == 0) blk_ok[stage][b] = blk;  // one piece per block starts it
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
            *reinterpret_cast<u32x4_t*>(vl + d * L::VS + 8 * v_pos(2 * b, d)) = vlo;
            *reinterpret_cast<u32x4_t*>(vl + d * L::VS + 8 * v_pos(2 * b + 1, d)) = vhi;
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
            *reinterpret_cast<u32x4_t*>(vl + d * L::VS + 8 * v_pos(2 * b + og, d)) = v;
        }
    };
    auto store = [&](auto set_tag, int kbase) __attribute__((always_inline)) {
        constexpr int SET = decltype(set_tag)::value % NSETS;
        const int stage = (kbase - kbeg) / kPfKeys % kPfStages;
        __bf16* kl = lds + stage * L::STAGE;
        __bf16* vl = kl + L::K_ELEMS;
        // all four blocks valid and inside the range: no token to zero (wave-uniform)
        if (kbase + kPfKeys <= kstop && okbits[SET] == (1u << NCH) - 1) {
#pragma unroll
            for (int j = 0; j < NCH; j++) put(std::false_type{}, set_tag, j, kl, vl, stage, kbase);
        } else {
#pragma unroll
            for (int j = 0; j < NCH; j++) put(std::true_type{}, set_tag, j, kl, vl, stage, kbase);
        }
    };
    // Staging of iteration it: tile it + 1 from its register set into its
    // LDS stage, then the loads of tile it + 1 + NSETS into the same set and the table entries
    // of the tile after.  The loads are issued whatever it is (past the range they read block 0
    // and are never stored), so that every path has the same loads in flight and one explicit
    // wait -- for this set, the older one -- serves all of them: the other set's loads stay in
    // flight.
    auto stage_phase = [&](auto set_tag, int it) __attribute__((always_inline)) {
        if (!stager) return;
        __builtin_amdgcn_s_waitcnt(kWaitVm | (NSETS == 2 ? 2 * NCH : 0));
        if (it + 1 < niter) store(set_tag, kbeg + (it + 1) * kPfKeys);
        load(set_tag, kbeg + (it + 1 + NSETS) * kPfKeys);
        fetch_entries(kbeg + (it + 2 + NSETS) * kPfKeys);
    };

    // ---- compute phases of iteration it on LDS stage it % 3
    f32x4_t sacc[R][4];  // S^T tiles: sacc[r][u] = keys of tile u x query rows of tile r
    bool blk_valid_next = true;  // block grp of the tile in sacc has a valid table entry
    bf16x8_t pb[R][2];   // P as the B operand of the PV product
    auto qk_phase = [&](int it) __attribute__((always_inline)) {
        const int kbase = kbeg + it * kPfKeys;
        if (kbase > pw_max) return;  // every row of this wave is done (uniform)
        const __bf16* kl = lds + (it % kPfStages) * L::STAGE;
        // the tile's block flags, read here so that the softmax phase does not wait on the LDS
        blk_valid_next = blk_ok[it % kPfStages][grp] != 0;
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int u = 0; u < 4; u++) sacc[r][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        // fragment i = (step i / 4, tile i % 4) is read kRing fragments ahead of its products
        auto kread = [&](int i) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8_t*>(kl + (16 * (i & 3) + col) * L::KS + 32 * (i >> 2) + 8 * grp);
        };
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
    };
    auto softmax_phase = [&](int it) __attribute__((always_inline)) {
        const int kbase = kbeg + it * kPfKeys;
        if (kbase > pw_max) return;
        // keys of block grp that have no valid table entry are masked like causal ones
        const bool blk_valid = blk_valid_next;
        const bool need_mask = kbase + kPfKeys - 1 > kw_min || __builtin_amdgcn_ballot_w64(!blk_valid) != 0;
        const int key0 = kbase + 16 * grp;  // the lane's keys are key0 + 4u + j
        // Both row tiles go through each step together (one basic block per step), so that
        // their independent dependency chains interleave.
        // raw scores, masked in place; the scale (> 0) is applied to the max and inside the
        // exponent's FMA
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int lim = blk_valid ? klim[r] - key0 : -1;  // last visible key offset
#pragma unroll
                for (int u = 0; u < 4; u++)
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        if (4 * u + j > lim) sacc[r][u][j] = -__builtin_inff();
            }
        }
        const auto& z = sacc;
        float mx[R];
        bool up[R];
        bool any_up = false;
#pragma unroll
        for (int r = 0; r < R; r++) {
            float t[4];
#pragma unroll
            for (int u = 0; u < 4; u++)
                t[u] = __builtin_fmaxf(__builtin_fmaxf(z[r][u][0], z[r][u][1]), __builtin_fmaxf(z[r][u][2], z[r][u][3]));
            mx[r] = __builtin_fmaxf(__builtin_fmaxf(t[0], t[1]), __builtin_fmaxf(t[2], t[3]));
        }
#pragma unroll
        for (int r = 0; r < R; r++) mx[r] = swap_max(mx[r], false);
#pragma unroll
        for (int r = 0; r < R; r++) {
            mx[r] = swap_max(mx[r], true) * sc;
            up[r] = mx[r] > m[r] + kPfMargin;
            any_up |= up[r];
        }
        if (__builtin_amdgcn_ballot_w64(any_up)) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float mn = up[r] ? mx[r] : m[r];
                const float alpha = fast_exp2(m[r] - mn);
                m[r] = mn;
                l[r] *= alpha;
#pragma unroll
                for (int d = 0; d < ND; d++) o[r][d] *= alpha;
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            const float nm = -m[r];
            uint32_t pw[4][2];
            float ls[2] = {0.0f, 0.0f};  // two partial sums: shorter dependency chains
#pragma unroll
            for (int u = 0; u < 4; u++) {
                pw[u][0] = pack_bf16x2(fast_exp2(__builtin_fmaf(z[r][u][0], sc, nm)),
                                       fast_exp2(__builtin_fmaf(z[r][u][1], sc, nm)));
                pw[u][1] = pack_bf16x2(fast_exp2(__builtin_fmaf(z[r][u][2], sc, nm)),
                                       fast_exp2(__builtin_fmaf(z[r][u][3], sc, nm)));
                ls[u & 1] = dot2_bf16(pw[u][0], kBf16OnePair, ls[u & 1]);
                ls[u & 1] = dot2_bf16(pw[u][1], kBf16OnePair, ls[u & 1]);
            }
            l[r] += ls[0] + ls[1];
            // k-step h2 of the PV product takes keys 16 grp + 8 h2 + 0..7 = S^T tiles 2 h2, 2 h2 + 1
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
                pb[r][h2] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[2 * h2][0], pw[2 * h2][1], pw[2 * h2 + 1][0],
                                                                    pw[2 * h2 + 1][1]));
        }
    };
    auto pv_phase = [&](int it) __attribute__((always_inline)) {
        const int kbase = kbeg + it * kPfKeys;
        if (kbase > pw_max) return;
        const __bf16* vl = lds + (it % kPfStages) * L::STAGE + L::K_ELEMS;
        // O^T += V^T P^T: V^T rows = channels, k = keys 16*grp + 8*h2 + 0..7; fragment
        // i = (half i / ND, channel tile i % ND), read kRing ahead.
        auto vread = [&](int i) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8_t*>(vl + (16 * (i % ND) + col) * L::VS +
                                                      8 * v_pos(2 * grp + i / ND, 16 * (i % ND) + col));
        };
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
    };

    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;
    // ---- prologue: tile 0 into LDS, the next NSETS tiles in flight
    if (stager) {
        fetch_entries(kbeg);
        load(Set0{}, kbeg);
        fetch_entries(kbeg + kPfKeys);
        if constexpr (NSETS == 2) load(Set1{}, kbeg + kPfKeys);
        // the queries and tile 0 have landed
        __builtin_amdgcn_s_waitcnt(kWaitVm | (NSETS == 2 ? 2 * NCH : 0));
        if (niter > 0) store(Set0{}, kbeg);
        if constexpr (NSETS == 2) {
            fetch_entries(kbeg + 2 * kPfKeys);
            load(Set0{}, kbeg + 2 * kPfKeys);
            fetch_entries(kbeg + 3 * kPfKeys);
        } else {
            load(Set0{}, kbeg + kPfKeys);
            fetch_entries(kbeg + 2 * kPfKeys);
        }
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm);
    }
    lds_barrier();

    // ---- main loop: phase M(it) = PV(it - 1), QK(it) and the staging of tile it + 1 on
    // the matrix cores, phase S(it) = the softmax of tile it on the vector ALUs, a barrier
    // after each.  Group B passes one barrier first and group A one last, which puts B one
    // phase behind A: in every slot one wave of each SIMD runs an M phase and the other an
    // S phase.  M(it) reads stages it - 1 and it (mod 3) and writes stage it + 1, and the
    // two groups' M phases are one slot apart, so no stage is written while it is read.
    // Two iterations per trip so that the register set is a constant.
    if (!group_a) lds_barrier();
    // M(it) and S(it) for 0 < it < niter; M(0) and the last M, which have no PV or no QK,
    // are peeled off so that this body is one straight path
    auto iteration = [&](auto set_tag, int it) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);  // keep the matrix cores fed before the other wave's VALU
        pv_phase(it - 1);
        // P dies in PV before the scores are born in QK: keep the two apart so that they
        // share registers
        __builtin_amdgcn_sched_barrier(0);
        qk_phase(it);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        stage_phase(set_tag, it);
        lds_barrier();
        softmax_phase(it);
        lds_barrier();
    };
    if (niter > 0) {
        __builtin_amdgcn_s_setprio(1);
        qk_phase(0);
        __builtin_amdgcn_s_setprio(0);
        stage_phase(Set1{}, 0);
        lds_barrier();
        softmax_phase(0);
        lds_barrier();
        int it = 1;
        for (; it + 1 < niter; it += 2) {
            iteration(Set0{}, it);
            iteration(Set1{}, it + 1);
        }
        if (it < niter) iteration(Set0{}, it);
        __builtin_amdgcn_s_setprio(1);
        pv_phase(niter - 1);
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();
        lds_barrier();
    }
    if (group_a) lds_barrier();

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
// out = sum_k w_k o_k / sum_k w_k l_k (o_k already times v_scale).  D / 4 lanes per row-head,
// 4 channels each (one 16-byte load per split), so a wave merges 64 / (D / 4) row-heads and
// every lane has all of its splits' loads in flight at once.
constexpr int kMergeThreads = 256;
template <int D>
constexpr int merge_rows_per_wg()
{
    return kMergeThreads / (D / 4);
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillArgs a)
{
    constexpr int LPR = D / 4;  // lanes per row-head
    const int64_t n = (int64_t)a.num_query_rows * a.num_heads;
    const int64_t idx = (int64_t)blockIdx.x * merge_rows_per_wg<D>() + threadIdx.x / LPR;
    if (idx >= n) return;
    const int c4 = (threadIdx.x % LPR) * 4;
    const int ns = a.num_splits;
    float mm = -__builtin_inff();
    for (int k = 0; k < ns; k++) mm = __builtin_fmaxf(mm, a.ml_part[2 * (k * n + idx)]);
    float lsum = 0.0f;
    f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < ns; k++) {
        const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(a.ml_part + 2 * (k * n + idx));
        const float wk = fast_exp2(ml[0] - mm);
        lsum += wk * ml[1];
        const f32x4_t o = *reinterpret_cast<const f32x4_t*>(a.o_part + (k * n + idx) * D + c4);
        acc += wk * o;
    }
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    *reinterpret_cast<uint2*>(static_cast<__bf16*>(a.out) + idx * D + c4) =
        make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
}

template <int KT, int D, int G>
hipError_t launch_one(const PrefillArgs& a, int grid, hipStream_t stream)
{
    if (a.block_size < kUnitTokens) {
        hipLaunchKernelGGL((prefill_kernel<KT, D, G, kPrefillRowTiles, true>), dim3((unsigned)grid),
                           dim3(kPrefillThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL((prefill_kernel<KT, D, G, kPrefillRowTiles, false>), dim3((unsigned)grid),
                           dim3(kPrefillThreads), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits == 1) return e;
    const int64_t n = (int64_t)a.num_query_rows * a.num_heads;
    constexpr int rpw = merge_rows_per_wg<D>();
    hipLaunchKernelGGL((prefill_merge_kernel<D>), dim3((unsigned)((n + rpw - 1) / rpw)), dim3(kMergeThreads), 0,
                       stream, a);
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
