// api.hip -- C ABI entry points of libpagedattn.so (declared in include/pagedattn.h).
//
// Host-side validation, workspace sizing and kernel dispatch.  Every argument check
// happens before anything is enqueued; the library allocates nothing and keeps no state
// beyond a per-thread error message and, for the no-allocation decode, the device address of
// each GPU's static scratch array.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/pagedattn.h"
#include "pa_internal.hpp"
#include "pa_copy.hpp"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int32_t ok()
{
    g_last_error.clear();
    return PA_OK;
}

int elem_bytes(int32_t dt)
{
    switch (dt) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    case PA_FP8_E5M2: return 1;
    case PA_INT8: return 1;
    default: return 0;
    }
}

// A quantised cache: 8-bit codes (OCP E4M3 / E5M2 floats or INT8) times per-head scales.
bool is_quant(int32_t dt) { return dt == PA_FP8_E4M3 || dt == PA_FP8_E5M2 || dt == PA_INT8; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kWorkspaceAlign = 256;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct DecodePlan {
    int32_t chunk_blocks;  // 0 = balanced over the grid, -1 = one chunk per run
    int32_t grid_workgroups;
    int64_t max_chunks, max_pieces;
    int64_t o_bytes, ml_bytes, info_bytes;  // workspace regions, in this order
    int64_t total;
};

// Tokens per work unit of the attention kernels: 16, or one 8-token block.
int32_t unit_tokens(int32_t block_size) { return block_size < pa::kUnitTokens ? block_size : pa::kUnitTokens; }

// Work units (unit_tokens tokens of one kv head) of the largest batch these arguments allow.
int64_t max_units(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len, int32_t utok)
{
    return (int64_t)num_seqs * num_kv_heads * ((max_context_len + utok - 1) / utok);
}

// stream_waves: waves of the full persistent grid for the kernel variant.
DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t max_context_len, int32_t partition_size, int64_t stream_waves)
{
    DecodePlan pl{};
    const int32_t utok = unit_tokens(block_size);
    const int64_t umax = max_units(num_seqs, num_kv_heads, max_context_len, utok);
    int64_t waves;
    if (partition_size > 0) {
        pl.chunk_blocks = partition_size / utok;
        pl.max_chunks = (umax + pl.chunk_blocks - 1) / pl.chunk_blocks;
        waves = pl.max_chunks < stream_waves ? pl.max_chunks : stream_waves;
    } else if ((max_context_len + utok - 1) / utok <= pa::kMinChunkBlocks) {
        // every run fits in one minimum chunk: one chunk per run, no split, no merge, no workspace
        pl.chunk_blocks = -1;
        const int64_t runs = (int64_t)num_seqs * num_kv_heads;
        waves = runs < stream_waves ? runs : stream_waves;
        pl.grid_workgroups = (int32_t)((waves + pa::kDecodeWaves - 1) / pa::kDecodeWaves);
        pl.max_chunks = runs;
        return pl;
    } else {
        pl.chunk_blocks = 0;
        const int64_t need = (umax + pa::kMinChunkBlocks - 1) / pa::kMinChunkBlocks;
        waves = need < stream_waves ? need : stream_waves;
    }
    pl.grid_workgroups = (int32_t)((waves + pa::kDecodeWaves - 1) / pa::kDecodeWaves);
    // automatic chunks: C >= ceil(U / NW) gives at most NW chunks
    if (partition_size <= 0) pl.max_chunks = (int64_t)pl.grid_workgroups * pa::kDecodeWaves;
    if (num_seqs == 0) return pl;
    const int64_t runs = (int64_t)num_seqs * num_kv_heads;
    const int64_t gqa = num_heads / num_kv_heads;
    pl.max_pieces = runs + pl.max_chunks;
    pl.o_bytes = align_up(pl.max_pieces * gqa * head_dim * 4, kWorkspaceAlign);
    pl.ml_bytes = align_up(pl.max_pieces * gqa * 2 * 4, kWorkspaceAlign);
    pl.info_bytes = align_up(runs * 2 * 4, kWorkspaceAlign);
    pl.total = pl.o_bytes + pl.ml_bytes + pl.info_bytes;
    return pl;
}

int32_t check_decode_shape(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_context_len, int32_t partition_size, int32_t q_dtype,
                           int32_t cache_dtype)
{
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_context_len < 0 || partition_size < 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_seqs=%d num_heads=%d num_kv_heads=%d "
                    "head_dim=%d block_size=%d max_context_len=%d partition_size=%d)", num_seqs, num_heads,
                    num_kv_heads, head_dim, block_size, max_context_len, partition_size);
    if (num_heads % num_kv_heads)
        return fail(PA_ERR_INVALID_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads, num_kv_heads);
    if (!elem_bytes(q_dtype) || !elem_bytes(cache_dtype) || is_quant(q_dtype))
        return fail(PA_ERR_INVALID_ARG, "unknown dtype (q %d, cache %d)", q_dtype, cache_dtype);
    const int32_t g = num_heads / num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(PA_ERR_UNSUPPORTED, "GQA group %d (supported: 1, 2, 4, 8)", g);
    if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size != 8 && block_size != 16 && block_size != 32)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d (supported: 8, 16, 32)", block_size);
    const bool combo = (q_dtype == PA_F32 && cache_dtype == PA_F32) || (q_dtype == PA_BF16 && cache_dtype == PA_BF16) ||
                       (q_dtype == PA_BF16 && is_quant(cache_dtype));
    if (!combo) return fail(PA_ERR_UNSUPPORTED, "(q dtype %d, cache dtype %d) not supported", q_dtype, cache_dtype);
    if (partition_size > 0 && partition_size % block_size)
        return fail(PA_ERR_INVALID_ARG, "partition_size %d is not a multiple of block_size %d", partition_size, block_size);
    return PA_OK;
}

struct PrefillPlan {
    int32_t row_blocks, num_splits, split_keys;
    int64_t grid;
    int64_t o_bytes, ml_bytes;  // workspace regions, in this order
    int64_t total;
};

// Workgroups the prefill grid should reach before splitting keys: one per CU of 256 CUs (a
// prefill workgroup fills a CU: 8 waves and 102 KiB of LDS).
constexpr int64_t kPrefillTargetWorkgroups = 256;
// Automatic splits keep at least this many keys per split.
constexpr int32_t kPrefillMinSplitKeys = 256;

PrefillPlan plan_prefill(int32_t num_query_rows, int32_t num_seqs, int32_t max_query_len, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len, int32_t partition_size)
{
    PrefillPlan pl{};
    const int32_t gqa = num_heads / num_kv_heads;
    const int32_t rows_per_wg = pa::kPrefillThreads / 64 * pa::kPrefillRowTiles * 16;
    pl.row_blocks = (int32_t)(((int64_t)max_query_len * gqa + rows_per_wg - 1) / rows_per_wg);
    const int64_t base = (int64_t)num_seqs * num_kv_heads * pl.row_blocks;
    if (partition_size > 0) {
        // key ranges start on 16-token units (an 8-token-block partition is rounded up)
        pl.split_keys = (partition_size + pa::kUnitTokens - 1) / pa::kUnitTokens * pa::kUnitTokens;
        pl.num_splits = max_context_len > 0 ? (max_context_len + pl.split_keys - 1) / pl.split_keys : 1;
    } else {
        pl.split_keys = 0;
        int64_t ns = base > 0 ? (kPrefillTargetWorkgroups + base - 1) / base : 1;
        const int64_t cap = max_context_len / kPrefillMinSplitKeys;
        if (ns > cap) ns = cap;
        pl.num_splits = ns < 1 ? 1 : (int32_t)ns;
    }
    pl.grid = base * pl.num_splits;
    if (pl.num_splits > 1 && num_query_rows > 0) {
        const int64_t rh = (int64_t)num_query_rows * num_heads;
        pl.o_bytes = align_up(pl.num_splits * rh * head_dim * 4, kWorkspaceAlign);
        pl.ml_bytes = align_up(pl.num_splits * rh * 2 * 4, kWorkspaceAlign);
    }
    pl.total = pl.o_bytes + pl.ml_bytes;
    return pl;
}

int32_t check_prefill_shape(int32_t num_query_rows, int32_t num_seqs, int32_t max_query_len, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_context_len,
                            int32_t partition_size, int32_t q_dtype, int32_t cache_dtype)
{
    int32_t st = check_decode_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                    partition_size, q_dtype, cache_dtype);
    if (st != PA_OK) return st;
    if (num_query_rows < 0 || max_query_len < 0)
        return fail(PA_ERR_INVALID_ARG, "num_query_rows %d / max_query_len %d negative", num_query_rows,
                    max_query_len);
    if (num_query_rows > 0 && max_query_len < 1)
        return fail(PA_ERR_INVALID_ARG, "max_query_len %d with %d query rows", max_query_len, num_query_rows);
    if (max_query_len > num_query_rows)
        return fail(PA_ERR_INVALID_ARG, "max_query_len %d exceeds num_query_rows %d", max_query_len, num_query_rows);
    if (q_dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "chunked prefill runs on bf16 matrix cores: q dtype must be BF16 (got %d)",
                    q_dtype);
    return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(int32_t status)
{
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
    case PA_ERR_NO_BLOCKS: return "no free or evictable block";
    default: return "unknown status";
    }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int64_t pa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim, int32_t cache_dtype)
{
    const int e = elem_bytes(cache_dtype);
    if (!e || num_layers < 0 || num_kv_heads < 0 || head_dim < 0) return -1;
    return (int64_t)num_layers * num_kv_heads * head_dim * 2 * e;
}

int64_t pa_pool_bytes(int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t cache_dtype)
{
    const int e = elem_bytes(cache_dtype);
    if (!e || num_blocks < 0 || num_kv_heads < 0 || head_dim < 0 || block_size < 0) return -1;
    return num_blocks * num_kv_heads * (int64_t)block_size * head_dim * e;
}

int32_t pa_validate_tables(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t max_context_len, int32_t block_size, int64_t num_blocks,
                           const int64_t* slots, int32_t num_slots, const int32_t* block_refcounts)
{
    if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || block_size < 1 || num_blocks < 0 ||
        num_slots < 0)
        return fail(PA_ERR_INVALID_ARG, "negative size (num_seqs=%d max_blocks_per_seq=%d max_context_len=%d "
                    "block_size=%d num_blocks=%lld num_slots=%d)", num_seqs, max_blocks_per_seq, max_context_len,
                    block_size, (long long)num_blocks, num_slots);
    if (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_tables)))
        return fail(PA_ERR_INVALID_ARG, "null block_tables or context_lens");
    for (int32_t s = 0; s < num_seqs; s++) {
        const int32_t ctx = context_lens[s];
        if (ctx < 0 || ctx > max_context_len)
            return fail(PA_ERR_INVALID_ARG, "sequence %d: context length %d outside [0, %d]", s, ctx,
                        max_context_len);
        const int64_t nb = ((int64_t)ctx + block_size - 1) / block_size;
        if (nb > max_blocks_per_seq)
            return fail(PA_ERR_INVALID_ARG, "sequence %d: context length %d needs %lld blocks, the table holds %d",
                        s, ctx, (long long)nb, max_blocks_per_seq);
        for (int64_t j = 0; j < nb; j++) {
            const int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + j];
            if (b < 0 || b >= num_blocks)
                return fail(PA_ERR_INVALID_ARG, "sequence %d: table entry %lld is block %d, outside [0, %lld)", s,
                            (long long)j, b, (long long)num_blocks);
        }
    }
    if (slots && num_slots > 0) {
        const int64_t cap = num_blocks * block_size;
        std::vector<std::pair<int64_t, int32_t>> used;  // (slot, token)
        used.reserve((size_t)num_slots);
        for (int32_t t = 0; t < num_slots; t++) {
            const int64_t sl = slots[t];
            if (sl < 0) continue;  // a skipped token
            if (sl >= cap)
                return fail(PA_ERR_INVALID_ARG, "token %d: slot %lld outside [0, %lld)", t, (long long)sl,
                            (long long)cap);
            if (block_refcounts && block_refcounts[sl / block_size] != 1)
                return fail(PA_ERR_INVALID_ARG, "token %d: slot %lld is in block %lld with reference count %d "
                            "(only a block its sequence alone holds may be written)", t, (long long)sl,
                            (long long)(sl / block_size), block_refcounts[sl / block_size]);
            used.emplace_back(sl, t);
        }
        std::sort(used.begin(), used.end());
        for (size_t i = 1; i < used.size(); i++)
            if (used[i].first == used[i - 1].first)
                return fail(PA_ERR_INVALID_ARG, "tokens %d and %d write the same slot %lld", used[i - 1].second,
                            used[i].second, (long long)used[i].first);
    }
    return ok();
}

int32_t pa_kv_cache_write(const void* key, const void* value, int32_t src_dtype, void* k_pool, void* v_pool,
                          int64_t num_blocks, int32_t cache_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, const float* k_scale,
                          const float* v_scale, void* stream)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
        return fail(PA_ERR_INVALID_ARG, "negative or zero size (num_tokens=%d num_kv_heads=%d head_dim=%d "
                    "block_size=%d num_blocks=%lld)", num_tokens, num_kv_heads, head_dim, block_size,
                    (long long)num_blocks);
    if (!elem_bytes(src_dtype) || !elem_bytes(cache_dtype) || is_quant(src_dtype))
        return fail(PA_ERR_INVALID_ARG, "unknown dtype (src %d, cache %d)", src_dtype, cache_dtype);
    if (!(src_dtype == cache_dtype || is_quant(cache_dtype)))
        return fail(PA_ERR_UNSUPPORTED, "append from dtype %d into a dtype %d cache", src_dtype, cache_dtype);
    if (head_dim % (64 / elem_bytes(cache_dtype)) || head_dim % (16 / elem_bytes(src_dtype)))
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d is not a whole number of 64-byte cache slices", head_dim);
    {
        const int t = 16 / elem_bytes(cache_dtype) < block_size ? 16 / elem_bytes(cache_dtype) : block_size;
        if (block_size % t)
            return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a whole number of %d-token V groups", block_size, t);
    }
    if (num_tokens == 0) return ok();
    if (!key || !value || !k_pool || !v_pool || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null pointer (key %p value %p k_pool %p v_pool %p slot_mapping %p)", key,
                    value, k_pool, v_pool, (const void*)slot_mapping);
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PA_ERR_INVALID_ARG, "key, value and pools must be 16-byte aligned");
    if (is_quant(cache_dtype) && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID_ARG, "a quantised (fp8 / INT8) cache needs k_scale and v_scale");
    pa::KvWriteArgs a{key, value, k_pool, v_pool, num_blocks, slot_mapping, num_tokens, num_kv_heads, head_dim,
                      block_size, is_quant(cache_dtype) ? k_scale : nullptr,
                      is_quant(cache_dtype) ? v_scale : nullptr};
    hipError_t e = pa::launch_kv_write(src_dtype, cache_dtype, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "kv_cache_write launch: %s", hipGetErrorString(e));
    return ok();
}

int64_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_context_len, int32_t partition_size)
{
    if (check_decode_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                           partition_size, PA_BF16, PA_BF16) != PA_OK)
        return -1;
    // sized for the largest grid any dtype's kernel uses
    return plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len, partition_size,
                       pa::kStreamWavesMax)
        .total;
}

}  // extern "C"

// ---- decode without a caller workspace -------------------------------------------------------
//
// For callers that cannot allocate (code under graph capture, tight serving loops): the split-K
// partial results live in this file-scope device array instead of a caller workspace.  Every
// GPU the library runs on holds its own copy until the process ends.  In host code the array's
// name is only a stand-in; its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what the kernels get.
// Every call on one GPU shares the array: calls that overlap on one GPU (two streams, two
// threads) race.  The kernels need no part of it zeroed (the merge reads only what the
// streaming kernel of the same call wrote), so nothing is cleared between calls.

namespace {

constexpr int64_t kNoAllocScratchBytes = 64ll << 20;  // 64 MiB per GPU
constexpr int kMaxScratchDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// Device address of this device's scratch, looked up on the first call on the device.
int32_t scratch_for_current_device(void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(PA_ERR_UNSUPPORTED, "device %d (the scratch table covers devices 0..%d)", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

namespace {

// Decode, with the fused append when new_key is not null.
int32_t decode_call(int32_t phase, void* out, const void* query, int32_t q_dtype, const void* new_key,
                    const void* new_value, const void* k_pool, const void* v_pool, int64_t num_blocks,
                    int32_t cache_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, const int32_t* shared_blocks, int32_t max_context_len,
                    int32_t num_seqs, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale, const float* k_scale,
                    const float* v_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                    void* stream, bool use_scratch = false)
{
    if (phase < 1 || phase > 3) return fail(PA_ERR_INVALID_ARG, "phase %d (1, 2 or 3)", phase);
    int32_t st = check_decode_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                    partition_size, q_dtype, cache_dtype);
    if (st != PA_OK) return st;
    if (num_blocks < 0 || max_blocks_per_seq < 0)
        return fail(PA_ERR_INVALID_ARG, "num_blocks %lld / max_blocks_per_seq %d negative", (long long)num_blocks,
                    max_blocks_per_seq);
    if (num_seqs > pa::kMaxDecodeSeqs)
        return fail(PA_ERR_UNSUPPORTED, "num_seqs %d above %d (context lengths are staged in LDS)", num_seqs,
                    pa::kMaxDecodeSeqs);
    if (shared_blocks && num_seqs > pa::kMaxDecodeSeqsShared)
        return fail(PA_ERR_UNSUPPORTED, "num_seqs %d above %d with shared-block counts (staged in LDS beside the "
                    "context lengths)", num_seqs, pa::kMaxDecodeSeqsShared);
    if ((int64_t)max_blocks_per_seq * block_size < max_context_len)
        return fail(PA_ERR_INVALID_ARG, "max_context_len %d exceeds the table capacity %d x %d", max_context_len,
                    max_blocks_per_seq, block_size);
    if (num_seqs == 0) return ok();
    if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "the pool has no blocks (num_blocks %lld)", (long long)num_blocks);
    if (!out || !query || !k_pool || !v_pool || !block_tables || !context_lens)
        return fail(PA_ERR_INVALID_ARG, "null pointer (out %p query %p k_pool %p v_pool %p block_tables %p "
                    "context_lens %p)", out, query, k_pool, v_pool, (const void*)block_tables,
                    (const void*)context_lens);
    if (!aligned16(query) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PA_ERR_INVALID_ARG, "query and pools must be 16-byte aligned");
    if (is_quant(cache_dtype) && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID_ARG, "a quantised (fp8 / INT8) cache needs k_scale and v_scale");
    if (!(scale > 0.0f && scale <= 3.402823466e38f))
        return fail(PA_ERR_INVALID_ARG, "scale %g: the softmax scale must be positive and finite", (double)scale);
    if ((new_key == nullptr) != (new_value == nullptr))
        return fail(PA_ERR_INVALID_ARG, "new_key and new_value must both be given");
    if (new_key && (!aligned16(new_key) || !aligned16(new_value)))
        return fail(PA_ERR_INVALID_ARG, "new_key and new_value must be 16-byte aligned");
    const int64_t stream_waves =
        (int64_t)pa::kSimds *
        pa::decode_waves_per_simd(q_dtype, cache_dtype, head_dim, num_heads / num_kv_heads, new_key != nullptr);
    const DecodePlan pl = plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                      partition_size, stream_waves);
    if (use_scratch) {  // the no-allocation form: this GPU's static scratch array is the workspace
        if (pl.total > kNoAllocScratchBytes)
            return fail(PA_ERR_WORKSPACE, "this decode needs %lld bytes of split-K scratch, above the %lld bytes the "
                        "no-allocation entry point holds per GPU (use pa_paged_attention_decode with a workspace)",
                        (long long)pl.total, (long long)kNoAllocScratchBytes);
        const int32_t sst = scratch_for_current_device(&workspace);
        if (sst != PA_OK) return sst;
        workspace_bytes = (size_t)kNoAllocScratchBytes;
    }
    if (pl.total > 0) {
        if (!workspace || (int64_t)workspace_bytes < pl.total)
            return fail(PA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %lld", workspace_bytes, workspace,
                        (long long)pl.total);
        if (reinterpret_cast<uintptr_t>(workspace) % kWorkspaceAlign)
            return fail(PA_ERR_WORKSPACE, "workspace must be %d-byte aligned", (int)kWorkspaceAlign);
    }
    const bool quant = is_quant(cache_dtype);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    pa::DecodeArgs a{};
    a.out = out;
    a.query = query;
    a.k_pool = const_cast<void*>(k_pool);  // written only by the fused append
    a.v_pool = const_cast<void*>(v_pool);
    a.new_key = new_key;
    a.new_value = new_value;
    a.num_blocks = num_blocks;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.shared_blocks = shared_blocks;
    a.max_context_len = max_context_len;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.k_scale = quant ? k_scale : nullptr;
    a.v_scale = quant ? v_scale : nullptr;
    a.chunk_blocks = pl.chunk_blocks;
    a.grid_workgroups = pl.grid_workgroups;
    a.max_chunks = pl.max_chunks;
    a.max_pieces = pl.max_pieces;
    a.o_part = reinterpret_cast<float*>(ws);
    a.ml_part = reinterpret_cast<float*>(ws + pl.o_bytes);
    a.run_info = reinterpret_cast<int32_t*>(ws + pl.o_bytes + pl.ml_bytes);
    hipError_t e = pa::launch_decode(phase, q_dtype, cache_dtype, head_dim, num_heads / num_kv_heads, a,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "decode launch (phase %d): %s", phase, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int32_t pa_paged_attention_decode_phase(int32_t phase, void* out, const void* query, int32_t q_dtype,
                                        const void* k_pool, const void* v_pool, int64_t num_blocks,
                                        int32_t cache_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                                        int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, float scale, const float* k_scale,
                                        const float* v_scale, int32_t partition_size, void* workspace,
                                        size_t workspace_bytes, void* stream)
{
    return decode_call(phase, out, query, q_dtype, nullptr, nullptr, k_pool, v_pool, num_blocks, cache_dtype,
                       block_tables, max_blocks_per_seq, context_lens, nullptr, max_context_len, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, scale, k_scale, v_scale, partition_size, workspace,
                       workspace_bytes, stream);
}

int32_t pa_paged_attention_decode_shared(int32_t phase, void* out, const void* query, int32_t q_dtype,
                                         const void* k_pool, const void* v_pool, int64_t num_blocks,
                                         int32_t cache_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, const int32_t* shared_blocks,
                                         int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                                         const float* k_scale, const float* v_scale, int32_t partition_size,
                                         void* workspace, size_t workspace_bytes, void* stream)
{
    return decode_call(phase, out, query, q_dtype, nullptr, nullptr, k_pool, v_pool, num_blocks, cache_dtype,
                       block_tables, max_blocks_per_seq, context_lens, shared_blocks, max_context_len, num_seqs,
                       num_heads, num_kv_heads, head_dim, block_size, scale, k_scale, v_scale, partition_size,
                       workspace, workspace_bytes, stream);
}

int32_t pa_paged_attention_decode_append(int32_t phase, void* out, const void* query, int32_t q_dtype,
                                         const void* new_key, const void* new_value, void* k_pool, void* v_pool,
                                         int64_t num_blocks, int32_t cache_dtype, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                                         const float* k_scale, const float* v_scale, int32_t partition_size,
                                         void* workspace, size_t workspace_bytes, void* stream)
{
    if (num_seqs > 0 && (!new_key || !new_value))
        return fail(PA_ERR_INVALID_ARG, "null new_key / new_value");
    return decode_call(phase, out, query, q_dtype, num_seqs > 0 ? new_key : nullptr,
                       num_seqs > 0 ? new_value : nullptr, k_pool, v_pool, num_blocks, cache_dtype, block_tables,
                       max_blocks_per_seq, context_lens, nullptr, max_context_len, num_seqs, num_heads, num_kv_heads,
                       head_dim, block_size, scale, k_scale, v_scale, partition_size, workspace, workspace_bytes,
                       stream);
}

}  // extern "C"

extern "C" {

int64_t pa_decode_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

int32_t pa_paged_attention_decode_noalloc(void* out, const void* query, int32_t q_dtype, const void* k_pool,
                                          const void* v_pool, int64_t num_blocks, int32_t cache_dtype,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, float scale, const float* k_scale,
                                          const float* v_scale, int32_t partition_size, void* stream)
{
    return decode_call(3, out, query, q_dtype, nullptr, nullptr, k_pool, v_pool, num_blocks, cache_dtype,
                       block_tables, max_blocks_per_seq, context_lens, nullptr, max_context_len, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, scale, k_scale, v_scale, partition_size, nullptr, 0, stream,
                       true);
}

int32_t pa_paged_attention_decode(void* out, const void* query, int32_t q_dtype, const void* k_pool,
                                  const void* v_pool, int64_t num_blocks, int32_t cache_dtype,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, float scale, const float* k_scale,
                                  const float* v_scale, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream)
{
    return pa_paged_attention_decode_phase(3, out, query, q_dtype, k_pool, v_pool, num_blocks, cache_dtype,
                                           block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                                           num_heads, num_kv_heads, head_dim, block_size, scale, k_scale, v_scale,
                                           partition_size, workspace, workspace_bytes, stream);
}

int64_t pa_chunked_prefill_workspace_size(int32_t num_query_rows, int32_t num_seqs, int32_t max_query_len,
                                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_context_len, int32_t partition_size)
{
    if (check_prefill_shape(num_query_rows, num_seqs, max_query_len, num_heads, num_kv_heads, head_dim, block_size,
                            max_context_len, partition_size, PA_BF16, PA_BF16) != PA_OK)
        return -1;
    return plan_prefill(num_query_rows, num_seqs, max_query_len, num_heads, num_kv_heads, head_dim, max_context_len,
                        partition_size)
        .total;
}

int32_t pa_paged_attention_chunked_prefill(void* out, const void* query, int32_t q_dtype,
                                           const int32_t* cu_query_lens, int32_t num_query_rows,
                                           int32_t max_query_len, const void* k_pool, const void* v_pool,
                                           int64_t num_blocks, int32_t cache_dtype, const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                                           int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                                           const float* k_scale, const float* v_scale, int32_t partition_size,
                                           void* workspace, size_t workspace_bytes, void* stream)
{
    int32_t st = check_prefill_shape(num_query_rows, num_seqs, max_query_len, num_heads, num_kv_heads, head_dim,
                                     block_size, max_context_len, partition_size, q_dtype, cache_dtype);
    if (st != PA_OK) return st;
    if (num_blocks < 0 || max_blocks_per_seq < 0)
        return fail(PA_ERR_INVALID_ARG, "num_blocks %lld / max_blocks_per_seq %d negative", (long long)num_blocks,
                    max_blocks_per_seq);
    if ((int64_t)max_blocks_per_seq * block_size < max_context_len)
        return fail(PA_ERR_INVALID_ARG, "max_context_len %d exceeds the table capacity %d x %d", max_context_len,
                    max_blocks_per_seq, block_size);
    if (num_seqs == 0 || num_query_rows == 0) return ok();
    if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "the pool has no blocks (num_blocks %lld)", (long long)num_blocks);
    if (!out || !query || !cu_query_lens || !k_pool || !v_pool || !block_tables || !context_lens)
        return fail(PA_ERR_INVALID_ARG, "null pointer (out %p query %p cu_query_lens %p k_pool %p v_pool %p "
                    "block_tables %p context_lens %p)", out, query, (const void*)cu_query_lens, k_pool, v_pool,
                    (const void*)block_tables, (const void*)context_lens);
    if (!aligned16(query) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PA_ERR_INVALID_ARG, "query, out and pools must be 16-byte aligned");
    if (is_quant(cache_dtype) && (!k_scale || !v_scale))
        return fail(PA_ERR_INVALID_ARG, "a quantised (fp8 / INT8) cache needs k_scale and v_scale");
    if (!(scale > 0.0f && scale <= 3.402823466e38f))
        return fail(PA_ERR_INVALID_ARG, "scale %g: the softmax scale must be positive and finite", (double)scale);
    const PrefillPlan pl = plan_prefill(num_query_rows, num_seqs, max_query_len, num_heads, num_kv_heads, head_dim,
                                        max_context_len, partition_size);
    if (pl.grid > 0x7FFFFFFF)
        return fail(PA_ERR_UNSUPPORTED, "prefill grid of %lld workgroups", (long long)pl.grid);
    if (pl.total > 0) {
        if (!workspace || (int64_t)workspace_bytes < pl.total)
            return fail(PA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %lld", workspace_bytes, workspace,
                        (long long)pl.total);
        if (reinterpret_cast<uintptr_t>(workspace) % kWorkspaceAlign)
            return fail(PA_ERR_WORKSPACE, "workspace must be %d-byte aligned", (int)kWorkspaceAlign);
    }
    if (pl.grid == 0) return ok();
    const bool quant = is_quant(cache_dtype);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    pa::PrefillArgs a{};
    a.out = out;
    a.query = query;
    a.cu_query_lens = cu_query_lens;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.num_blocks = num_blocks;
    a.block_tables = block_tables;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.context_lens = context_lens;
    a.max_context_len = max_context_len;
    a.num_seqs = num_seqs;
    a.num_query_rows = num_query_rows;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.row_blocks = pl.row_blocks;
    a.num_splits = pl.num_splits;
    a.split_keys = pl.split_keys;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.k_scale = quant ? k_scale : nullptr;
    a.v_scale = quant ? v_scale : nullptr;
    a.o_part = pl.total > 0 ? reinterpret_cast<float*>(ws) : nullptr;
    a.ml_part = pl.total > 0 ? reinterpret_cast<float*>(ws + pl.o_bytes) : nullptr;
    hipError_t e = pa::launch_prefill(cache_dtype, head_dim, num_heads / num_kv_heads, a, pl.grid,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "chunked prefill launch: %s", hipGetErrorString(e));
    return ok();
}

int32_t pa_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks, int64_t block_bytes, const int32_t* pairs,
                       int32_t num_pairs, void* stream)
{
    if (num_pairs < 0 || num_blocks < 0 || block_bytes <= 0 || block_bytes % 16)
        return fail(PA_ERR_INVALID_ARG, "num_pairs %d, num_blocks %lld, block_bytes %lld (a positive multiple of 16)",
                    num_pairs, (long long)num_blocks, (long long)block_bytes);
    if (num_pairs == 0) return ok();
    if (!k_pool || !v_pool || !pairs || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PA_ERR_INVALID_ARG, "null or misaligned pointer (k_pool %p v_pool %p pairs %p)", k_pool, v_pool,
                    (const void*)pairs);
    hipError_t e = pa::launch_copy_blocks(k_pool, v_pool, num_blocks, block_bytes, pairs, num_pairs,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "copy_blocks launch: %s", hipGetErrorString(e));
    return ok();
}

int32_t pa_probe_tile_read(const void* buf, int64_t buf_bytes, const int32_t* order, int64_t num_reads,
                           int32_t grid_workgroups, void* sink, void* stream)
{
    if (!buf || !order || !sink) return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(buf)) return fail(PA_ERR_INVALID_ARG, "buf must be 16-byte aligned");
    if (buf_bytes < 4096 || num_reads < 0 || grid_workgroups < 1 || grid_workgroups > 65535)
        return fail(PA_ERR_INVALID_ARG, "buf_bytes %lld, num_reads %lld, grid %d", (long long)buf_bytes,
                    (long long)num_reads, grid_workgroups);
    if (num_reads == 0) return ok();
    hipError_t e = pa::launch_tile_read(buf, buf_bytes / 4096, num_reads, order, grid_workgroups,
                                        static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
