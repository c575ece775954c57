/*
 * pagedattn.h -- C ABI of libpagedattn.so: paged KV append and PagedAttention for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (from the four pages on paged KV caches):
 *   - attention of a query over its sequence's cached keys and values is
 *     softmax(q K^T * scale) V with scale = 1/sqrt(head_dim)   (page 1, section 2, the
 *     Attention(Q,K,V) formula);
 *   - the KV cache of every sequence is cut into fixed-size physical blocks (16 tokens by
 *     default) held in one pool; a per-sequence block table maps logical block i to a
 *     physical block, and the attention reads the cache block by block through that table
 *     rather than assuming contiguous storage (page 1, section 4 and its worked mapping
 *     0->7, 1->2, 2->19, 3->4; page 3, section 2.1);
 *   - several query heads share one KV head (grouped-query attention; page 1, section 10);
 *   - each decode step writes the new token's K and V into its block slot before attending
 *     (page 1, section 1, the prefill/decode diagram);
 *   - the cache may be stored as 8-bit floats, E4M3 or E5M2, with per-head scales (page 1,
 *     section 15; page 2, quantisation, which also names per-tensor scales -- pass one value
 *     repeated per head; page 3, section 2.4, which prefers E4M3 because E5M2 can drift on
 *     long sequences), or as 8-bit integers (page 4, section 4.5, step 4: the KV cache brought
 *     from FP16 down to INT8; page 2, quantisation, KV-cache quantisation);
 *   - a long prompt may be processed in chunks that run alongside decode rows (page 1,
 *     section 12; page 3, section 2.3).
 *
 * Conventions for every entry point
 *   - Pointers named "device" point to GPU memory (hipMalloc / torch CUDA tensors) that the
 *     caller owns; the library keeps no reference after the call returns and allocates
 *     nothing on these paths.  Host scalars are passed by value.
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is enqueued
 *     asynchronously on it; nothing synchronises.
 *   - The return value is a pa_status.  Argument errors are detected on the host before any
 *     GPU work is enqueued, so they leave every buffer untouched.  PA_ERR_HIP means a launch
 *     failed (the HIP error is in pa_last_error()).  Errors raised by earlier asynchronous
 *     work are not reported here.
 *   - Device-resident data is the caller's contract and is not validated: block ids in
 *     [0, num_blocks), context_lens[s] <= max_context_len and
 *     ceil(context_lens[s] / block_size) <= max_blocks_per_seq, distinct write slots.  The
 *     kernels still bounds-check every block id and slot they dereference: an out-of-range
 *     block is treated as holding no valid token and an out-of-range slot is skipped, so bad
 *     data gives wrong numbers, never an out-of-bounds access.
 *   - Functions are stateless and may be called from several host threads at once.
 *
 * Element types (pa_dtype):  PA_F32 IEEE binary32; PA_BF16 bfloat16; PA_FP8_E4M3 the OCP
 * 8-bit float E4M3 (bias 7, no infinities, S.1111.111 = NaN, largest finite 448);
 * PA_FP8_E5M2 the OCP 8-bit float E5M2 (bias 15, S.11111.00 = +-inf, S.11111.mm with mm != 0
 * = NaN, largest finite 57344); PA_INT8 a two's-complement 8-bit integer code.  The three 8-bit
 * types are "quantised" caches: the cached value is code * scale with one fp32 scale per kv
 * head (k_scale for K, v_scale for V).
 *
 * Pool layout.  k_pool and v_pool are each [num_blocks][num_kv_heads][block_size*head_dim]
 * elements of cache_dtype.  With e = element bytes, W = 64/e and T = min(16/e, block_size),
 * token o of a block and channel d sit inside their (block, kv head) tile at
 *     K:  (d / W) * (block_size * W) + o * W + (d % W)
 *     V:  ((o / T) * head_dim + d) * T + (o % T)
 * K is stored as 64-byte channel slices, token-major; V as groups of T consecutive tokens,
 * channel-major, so the T tokens of one channel fill one 16-byte piece.  One (block, kv head)
 * tile of a 16-token bf16 block with head_dim 128 is 4 KiB; one 64-lane 16-byte-per-lane load
 * reads a whole 1 KiB K slice (16 tokens x 32 channels) or a 1 KiB V piece (8 tokens x 64
 * channels).
 *
 * Supported shapes: head_dim 64 or 128; block_size 8, 16 or 32 for attention (the pages weigh
 * block size against fragmentation and access efficiency: page 2, the PagedAttention section;
 * the append takes any block size the layout allows); num_heads / num_kv_heads in
 * {1, 2, 4, 8}; (q dtype, cache dtype) in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 * (BF16, FP8_E5M2), (BF16, INT8)};
 * up to 16384 sequences per decode call; chunked prefill with BF16 queries only.
 * Anything else returns PA_ERR_UNSUPPORTED.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent sizes          */
    PA_ERR_UNSUPPORTED = 2, /* valid request outside the support matrix above            */
    PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the required size       */
    PA_ERR_HIP = 4,         /* a HIP launch failed                                       */
    PA_ERR_NO_BLOCKS = 5    /* the block manager has no free or evictable block left      */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2, PA_FP8_E5M2 = 3, PA_INT8 = 4 } pa_dtype;

/*
 * Paged KV append (the step that stores each new token's K and V in its block slot).
 *   key, value     device, [num_tokens][num_kv_heads][head_dim] of src_dtype, contiguous.
 *   k_pool, v_pool device, pools of cache_dtype in the layout above, num_blocks blocks.
 *   slot_mapping   device int64 [num_tokens]; token i goes to physical block
 *                  slot / block_size at offset slot % block_size.  A negative slot skips the
 *                  token; a slot >= num_blocks*block_size is also skipped.
 *   k_scale, v_scale  device fp32 [num_kv_heads] for a quantised cache, else NULL.
 * src_dtype == cache_dtype copies the bits.  A BF16 or F32 source into an FP8_E4M3 cache
 * stores e4m3(fl32(x / scale[h])): one binary32 division (round to nearest even), then
 * round-to-nearest-even to E4M3 saturating at +-448, NaN kept as NaN with its sign.  An
 * FP8_E5M2 cache stores e5m2(fl32(x / scale[h])) by the same rule, saturating at +-57344
 * (infinities included) and storing NaN as S.11111.11.  An INT8 cache stores the nearest
 * integer to fl32(x / scale[h]) (ties to even), saturated to [-127, 127] (the symmetric
 * range; infinities saturate), NaN stored as 0.  Only
 * the addressed slots are written; every other byte of the pools is left unchanged.  Slots
 * must be distinct within one call.
 */
int32_t pa_kv_cache_write(const void* key, const void* value, int32_t src_dtype,
                          void* k_pool, void* v_pool, int64_t num_blocks, int32_t cache_dtype,
                          const int64_t* slot_mapping, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          const float* k_scale, const float* v_scale, void* stream);

/*
 * Bytes of device workspace that pa_paged_attention_decode needs for these arguments
 * (partition_size 0 = automatic work split).  Depends only on the shapes, never on the
 * context lengths' values.  0 for an empty batch, and for an automatic split when
 * max_context_len <= 128 (64 with 8-token blocks): every sequence then fits in one work chunk,
 * nothing is split and no merge runs.  Returns -1 for arguments the decode call would reject.
 */
int64_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size);

/*
 * PagedAttention decode: one query row per sequence attends over all context_lens[s]
 * cached positions of its sequence (the token appended this step included).
 *   out            device [num_seqs][num_heads][head_dim] of q_dtype (written).
 *   query          device [num_seqs][num_heads][head_dim] of q_dtype.
 *   k_pool, v_pool device pools (layout above) of num_blocks >= 1 blocks.
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                  ceil(context_lens[s] / block_size) are never read.
 *   context_lens   device int32 [num_seqs]; a sequence with 0 positions gets zeros.
 *   max_context_len  host bound on context_lens (sizes the launch and the workspace).
 *   scale          softmax scale applied to q.k (1/sqrt(head_dim) for standard attention);
 *                  positive and finite, else PA_ERR_INVALID_ARG.
 *   k_scale, v_scale device fp32 [num_kv_heads] for a quantised cache (the stored code times
 *                  the scale is the cached value), else NULL.  Exactly num_kv_heads values are
 *                  read from each; a per-tensor scale is passed repeated per head.
 *   partition_size 0 = automatic, else a multiple of block_size.  The work is the list of
 *                  every (sequence, kv head) pair's units (16 tokens, or one 8-token block)
 *                  laid end to end; it is cut into chunks of partition_size tokens' units
 *                  (automatic: equal chunks, one per wave of a grid sized to fill the GPU; or,
 *                  when every sequence fits in 8 units, one chunk per (sequence, kv head)),
 *                  each chunk is attended independently per
 *                  sequence piece, and the pieces of a sequence are merged (split-K).  The
 *                  result does not depend on the split beyond rounding.
 *   workspace      device scratch of at least pa_decode_workspace_size(...) bytes, 256-byte
 *                  aligned.  Contents need no initialisation and are undefined afterwards.
 *                  Two calls that run concurrently need separate workspaces.
 * Context lengths above max_context_len are treated as max_context_len.
 * query head h reads kv head h / (num_heads / num_kv_heads).
 */
int32_t pa_paged_attention_decode(void* out, const void* query, int32_t q_dtype,
                                  const void* k_pool, const void* v_pool, int64_t num_blocks,
                                  int32_t cache_dtype, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  float scale, const float* k_scale, const float* v_scale,
                                  int32_t partition_size, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * The same decode as two separately enqueued phases, for callers that time or overlap
 * them: phase 1 runs the attention over the work chunks (it writes the final rows of
 * sequences that one chunk covers whole and the partial results of the others into the
 * workspace); phase 2 merges the partial results and writes the zero rows of empty
 * sequences.  Calling phase 1 then phase 2 with identical
 * arguments on one stream equals pa_paged_attention_decode.  phase 3 runs both.
 */
int32_t pa_paged_attention_decode_phase(int32_t phase, void* out, const void* query,
                                        int32_t q_dtype, const void* k_pool, const void* v_pool,
                                        int64_t num_blocks, int32_t cache_dtype,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, float scale,
                                        const float* k_scale, const float* v_scale,
                                        int32_t partition_size, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace that pa_paged_attention_chunked_prefill needs for these arguments
 * (0 when the keys are not split; partition_size as there).  Depends only on the shapes.
 * Returns -1 for shapes the prefill call would reject.
 */
int64_t pa_chunked_prefill_workspace_size(int32_t num_query_rows, int32_t num_seqs, int32_t max_query_len,
                                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_context_len,
                                          int32_t partition_size);

/*
 * Chunked-prefill PagedAttention (page 1, section 12: a long prompt is processed as chunks
 * scheduled alongside decode rows; page 3, section 2.3).  Sequence s contributes
 * q_len = cu_query_lens[s+1] - cu_query_lens[s] query rows, rows cu_query_lens[s] .. +q_len-1
 * of query/out; they are the LAST q_len positions of its context_lens[s] cached positions
 * (their K and V are already in the cache), so row i sits at position
 * p = context_lens[s] - q_len + i and attends causally to positions 0..p.  A sequence with
 * q_len 1 is a decode row; q_len 0 contributes nothing.  A row whose position would be
 * negative (q_len > context_lens[s]) gets zeros.
 *   out            device [num_query_rows][num_heads][head_dim] bf16 (written).
 *   query          device [num_query_rows][num_heads][head_dim] bf16.
 *   q_dtype        PA_BF16 (the products run on bf16 matrix cores with fp32 accumulation; an
 *                  fp8 or INT8 cache is widened to bf16 exactly).  Other types: PA_ERR_UNSUPPORTED.
 *   cu_query_lens  device int32 [num_seqs + 1], non-decreasing, cu_query_lens[0] = 0 and
 *                  cu_query_lens[num_seqs] = num_query_rows.  A sequence whose rows fall
 *                  outside [0, num_query_rows) is skipped.
 *   max_query_len  host bound on q_len (sizes the launch).
 *   k_pool .. v_scale, scale  as for pa_paged_attention_decode.
 *   partition_size 0 = automatic, else a multiple of block_size (rounded up to a multiple of
 *                  16 for 8-token blocks): the visible keys of each group
 *                  of rows are cut into ranges of partition_size keys that run on separate
 *                  workgroups and are merged (split-K).  Automatic splits only when the rows
 *                  alone do not fill the GPU.
 *   workspace      device scratch of pa_chunked_prefill_workspace_size(...) bytes, 256-byte
 *                  aligned (NULL when that size is 0).  Contents need no initialisation.
 * Rows not owned by any sequence are left unchanged when the keys are not split and are
 * undefined otherwise.
 */
int32_t pa_paged_attention_chunked_prefill(void* out, const void* query, int32_t q_dtype,
                                           const int32_t* cu_query_lens, int32_t num_query_rows,
                                           int32_t max_query_len, const void* k_pool, const void* v_pool,
                                           int64_t num_blocks, int32_t cache_dtype,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t max_context_len,
                                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, float scale,
                                           const float* k_scale, const float* v_scale,
                                           int32_t partition_size, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * pa_paged_attention_decode_phase with a hint about blocks shared between sequences: sequences
 * that share a prefix hold the same physical blocks in their tables (page 1, section 4; page 2,
 * the PagedAttention section), so every sharer reads those blocks:
 *   shared_blocks  device int32 [num_seqs], or NULL (= pa_paged_attention_decode_phase): block j
 *                  of sequence s with j < shared_blocks[s] is read with the default cache policy,
 *                  so the sequence's other readers of that block can find it cached; every other
 *                  block is read once per call and streamed past the caches.  With the hint the
 *                  work chunks are also placed so that the sharers of one kv head's blocks run on
 *                  one XCD (one L2).  The hint changes only the loads' cache policy and where the
 *                  chunks run: the output is the same, bit for bit, for any values (an
 *                  inaccurate hint only costs time).  The host knows the counts from its block
 *                  refcounts (the leading blocks with refcount > 1).
 * num_seqs must be <= 8192 when shared_blocks is given (the counts are staged in LDS beside the
 * context lengths).  Other arguments, errors and the workspace as for
 * pa_paged_attention_decode_phase.
 */
int32_t pa_paged_attention_decode_shared(int32_t phase, void* out, const void* query, int32_t q_dtype,
                                         const void* k_pool, const void* v_pool, int64_t num_blocks,
                                         int32_t cache_dtype, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         const int32_t* shared_blocks, int32_t max_context_len,
                                         int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, float scale,
                                         const float* k_scale, const float* v_scale,
                                         int32_t partition_size, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Decode with the step's append fused in (one launch instead of pa_kv_cache_write followed by
 * pa_paged_attention_decode_phase).  Every sequence s with context_lens[s] >= 1 first stores its
 * new token -- new_key[s] and new_value[s] -- at position context_lens[s] - 1, i.e. slot
 * block_tables[s][(ctx - 1) / block_size] * block_size + (ctx - 1) % block_size, exactly as
 * pa_kv_cache_write would (same bytes, including the fp8 encode); then the decode runs as
 * pa_paged_attention_decode_phase with the same arguments (the same output bits).
 *   new_key, new_value  device [num_seqs][num_kv_heads][head_dim] in q_dtype (the source dtype
 *                  of the append), 16-byte aligned.
 *   k_pool, v_pool device pools, written at the new tokens' slots.
 * Phase 1 does both: the wave that attends the token's block takes the new token from its
 * input row (encoded as the cache stores it) into the block it has loaded, and stores the row
 * into the slot, so no wait orders the store before a read.  A new token's block must not be shared with another
 * sequence (the same rule as for pa_kv_cache_write's distinct slots).  Other arguments, errors
 * and the workspace as for pa_paged_attention_decode_phase; phase 2 alone appends nothing.
 */
int32_t pa_paged_attention_decode_append(int32_t phase, void* out, const void* query, int32_t q_dtype,
                                         const void* new_key, const void* new_value, void* k_pool,
                                         void* v_pool, int64_t num_blocks, int32_t cache_dtype,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t max_context_len,
                                         int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, float scale,
                                         const float* k_scale, const float* v_scale,
                                         int32_t partition_size, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Decode that allocates nothing and takes no workspace, for callers that cannot allocate device
 * memory at all: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It equals pa_paged_attention_decode (phase 3, the same kernels, the same output
 * bits) with the split-K partial results held in a static device array inside the library:
 * pa_decode_noalloc_max_workspace() bytes (64 MiB) per GPU, reserved when the library's code is
 * loaded on that GPU and held until the process ends.  The first call on a device looks the
 * array's address up (hipGetSymbolAddress); no call allocates.
 *   Arguments as for pa_paged_attention_decode, without workspace and workspace_bytes.
 *   Returns PA_ERR_WORKSPACE, before any GPU work, when these arguments need more than that many
 *   bytes of workspace (pa_decode_workspace_size(...) gives an upper bound of the need).
 * All calls on one GPU share the array, whose contents are left from the last call: two calls
 * that overlap on one GPU (different streams or host threads without ordering) race and give
 * undefined results.  Calls ordered on one stream are safe.
 */
int32_t pa_paged_attention_decode_noalloc(void* out, const void* query, int32_t q_dtype,
                                          const void* k_pool, const void* v_pool, int64_t num_blocks,
                                          int32_t cache_dtype, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          float scale, const float* k_scale, const float* v_scale,
                                          int32_t partition_size, void* stream);

/* Bytes of the static scratch array pa_paged_attention_decode_noalloc uses per GPU. */
int64_t pa_decode_noalloc_max_workspace(void);

/* KV bytes one token occupies over num_layers layers: layers x kv_heads x head_dim x 2 (K and
 * V) x element bytes (page 1, section 2.1: 131072 for 32 x 8 x 128 bf16).  -1 on bad input. */
int64_t pa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                              int32_t cache_dtype);

/* Bytes of one pool (K or V) of num_blocks blocks.  -1 on bad input. */
int64_t pa_pool_bytes(int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t cache_dtype);

/*
 * Debug check, on host copies, of the device-resident data the calls above take on trust
 * (the block table and slot mapping of page 1, section 4).  No GPU work; host pointers.
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]; context_lens int32 [num_seqs].
 *   Every sequence must have 0 <= context_lens[s] <= max_context_len and
 *   ceil(context_lens[s] / block_size) <= max_blocks_per_seq, and each of those table entries
 *   must be a block id in [0, num_blocks) (entries past them are not looked at).
 *   slots           int64 [num_slots] or NULL: the write slots of a pa_kv_cache_write call.
 *                   A negative slot (a skipped token) is allowed; the others must be below
 *                   num_blocks * block_size and distinct.
 *   block_refcounts int32 [num_blocks] or NULL (only with slots): the block manager's reference
 *                   counts; a slot in a block whose count is not 1 is a write into an unowned
 *                   or shared block (a missed copy-on-write).
 * Returns PA_OK, or PA_ERR_INVALID_ARG naming the first offending sequence, entry or slot in
 * pa_last_error().
 */
int32_t pa_validate_tables(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t max_context_len, int32_t block_size, int64_t num_blocks,
                           const int64_t* slots, int32_t num_slots, const int32_t* block_refcounts);

/*
 * Measurement helper (not part of the attention path): read num_reads 4 KiB tiles of buf, tile
 * order[i] for i = 0 .. num_reads-1, with grid_workgroups x 256 threads (two tiles per wave and
 * iteration, 16-byte nontemporal loads, each wave load one contiguous 1 KiB).  Timing it with a random
 * order gives the HBM read bandwidth this GPU delivers for the scattered 4 KiB (block, kv head)
 * tiles of a paged pool, the practical ceiling the decode kernel is compared with.
 *   buf    device, buf_bytes bytes (16-byte aligned; whole tiles are used).
 *   order  device int32 [num_reads]; an entry outside [0, buf_bytes / 4096) reads tile 0.
 *   sink   device, at least 4 * grid_workgroups bytes; written only in a case that does not occur.
 */
int32_t pa_probe_tile_read(const void* buf, int64_t buf_bytes, const int32_t* order, int64_t num_reads,
                           int32_t grid_workgroups, void* sink, void* stream);

/*
 * Copy whole blocks inside the pools: for each pair i, block pairs[2i] -> block pairs[2i+1],
 * every kv head, in both k_pool and v_pool (the copy-on-write of a shared tail block before a
 * sequence appends into it; see the block manager below).
 *   k_pool, v_pool  device pools (layout above) of num_blocks blocks of block_bytes each,
 *                   block_bytes = num_kv_heads * block_size * head_dim * element bytes (a
 *                   multiple of 16; pools 16-byte aligned).
 *   pairs           device int32 [num_pairs][2] (source, destination).  A pair with an id
 *                   outside [0, num_blocks) is skipped.  Destinations must be distinct and no
 *                   destination may be a source of the same call.
 */
int32_t pa_copy_blocks(void* k_pool, void* v_pool, int64_t num_blocks, int64_t block_bytes, const int32_t* pairs,
                       int32_t num_pairs, void* stream);

/*
 * Block manager (host only; no GPU work): the allocator of a pool's blocks, with reference
 * counts, prefix caching and copy-on-write.
 *   - Sequences reference blocks through their block tables (page 1, section 4); a block is
 *     shared by every sequence whose table holds it and returns to the allocator when the
 *     last one lets go (sharing across requests: page 2, the PagedAttention section).
 *   - Prefix caching is block-granular (page 1, section 11; page 3, section 2.3): every full
 *     block is keyed by a hash chained over the previous block and its own token ids, and a new
 *     prompt whose leading full blocks match reuses them, so only the rest needs prefill.  A
 *     partly filled block is never taken from the cache.  A hit is confirmed by comparing the
 *     token ids and the chain's previous block, so a hash collision cannot share a block.
 *   - Cached blocks nobody references stay cached until an allocation finds no never-used or
 *     released block; then the one released longest ago is evicted.
 *   - Appending into a partly filled block that other sequences also reference (after
 *     pa_bm_fork) first moves the sequence to a private copy: the call returns the (source,
 *     destination) pair, which the caller copies with pa_copy_blocks before writing the token.
 * The manager is not thread-safe: one host thread at a time per manager.
 */
typedef struct pa_block_manager pa_block_manager;

typedef struct {
    int64_t free_blocks;       /* never used or released uncached blocks */
    int64_t evictable_blocks;  /* cached blocks no sequence references */
    int64_t used_blocks;       /* blocks referenced by at least one sequence */
    int64_t cached_blocks;     /* entries of the prefix cache (in use or evictable) */
    int64_t lookups;           /* full prompt blocks looked up in the cache */
    int64_t hits;              /* of those, found (prefix hit rate = hits / lookups) */
    int64_t evictions;         /* cached blocks reused for other data */
    int64_t cow_copies;        /* copy-on-write copies handed out */
} pa_bm_stats;

/* A manager for num_blocks blocks (ids 0 .. num_blocks-1) of block_size tokens; NULL for
 * num_blocks outside [1, 2^31) or block_size < 1.  Blocks are handed out from id 0 upwards. */
pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* New sequence seq_id (>= 0, not already present) holding the prompt tokens[0 .. num_tokens).
 * Leading full blocks found in the prefix cache are shared, at most (num_tokens - 1) /
 * block_size of them so that at least one prompt token is computed; *cached_tokens (may be
 * NULL) receives their token count.  The other blocks are allocated and the full ones
 * registered in the cache.  The caller writes the K/V of tokens cached_tokens .. num_tokens-1
 * (slots from pa_bm_block_table) before a later call attends over them.  PA_ERR_NO_BLOCKS
 * leaves the manager unchanged. */
int32_t pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                           int32_t* cached_tokens);

/* Append one token to seq_id: *slot receives its pool slot (block * block_size + offset).  If
 * the token lands in a partly filled block other sequences also reference, the sequence first
 * moves to a fresh block: *copy_src / *copy_dst (may be NULL) receive the pair to copy with
 * pa_copy_blocks before the token's K/V are written, else -1.  A block that becomes full is
 * registered in the prefix cache.  PA_ERR_NO_BLOCKS leaves the manager unchanged. */
int32_t pa_bm_append_token(pa_block_manager* bm, int64_t seq_id, int32_t token, int64_t* slot, int32_t* copy_src,
                           int32_t* copy_dst);

/* child_id (>= 0, new) shares every block of parent_id (parallel sampling, beam search). */
int32_t pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Drop seq_id: every block loses one reference; unreferenced cached blocks become evictable,
 * other unreferenced blocks free. */
int32_t pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);

/* seq_id's block table row (table may be NULL; PA_ERR_INVALID_ARG if it holds more than
 * max_blocks blocks), its block count and token count (either may be NULL). */
int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* table, int32_t max_blocks,
                          int32_t* num_blocks, int32_t* num_tokens);

/* References held on block (-1 for an id outside the pool). */
int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block);

int32_t pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* out);

/* Static name of a status code. */
const char* pa_status_string(int32_t status);

/* Detail of the most recent failing call on this host thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
