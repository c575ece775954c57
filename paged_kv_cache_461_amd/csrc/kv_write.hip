// kv_write.hip -- paged KV append: store each new token's K and V rows into its block slot.
//
// Each decode step produces the new token's K/V and stores it in the cache (page 1,
// section 1, the prefill/decode diagram); the slot is physical block * block_size + offset
// from the sequence's block table (page 1, section 4).  One thread moves one 16-byte piece of
// one source row (token, kv head, K or V); the piece store is kv_store.hpp's.
#include "kv_store.hpp"
#include "pa_internal.hpp"

namespace pa {
namespace {

template <int ST, int CT>
__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteArgs a)
{
    constexpr int ES = DtypeBytes<ST>::value;
    constexpr int EC = DtypeBytes<CT>::value;
    constexpr int N = 16 / ES;  // source elements per piece
    constexpr int W = 64 / EC;  // cache channels per 64-byte slice
    static_assert(W % N == 0, "a piece never straddles a slice");

    const int D = a.head_dim, Hkv = a.num_kv_heads, B = a.block_size;
    const int pieces = D / N;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)a.num_tokens * Hkv * 2 * pieces;
    if (gid >= total) return;
    const int piece = (int)(gid % pieces);
    int64_t r = gid / pieces;
    const int kv = (int)(r % 2);  // 0 = key, 1 = value
    r /= 2;
    const int h = (int)(r % Hkv);
    const int64_t tok = r / Hkv;

    const int64_t slot = a.slots[tok];
    if (slot < 0 || slot >= a.num_blocks * (int64_t)B) return;
    const int64_t blk = slot / B;
    const int o = (int)(slot % B);

    const unsigned char* src = static_cast<const unsigned char*>(kv ? a.value : a.key) +
                               (((tok * Hkv + h) * D) + (int64_t)piece * N) * ES;
    const int64_t tile = (blk * Hkv + h) * (int64_t)B * D;  // element offset of the tile
    unsigned char* pool = static_cast<unsigned char*>(kv ? a.v_pool : a.k_pool);
    const float sc = kIsQuant<CT> && ST != CT ? (kv ? a.v_scale : a.k_scale)[h] : 1.0f;
    store_kv_piece<ST, CT>(load16(src), pool, tile, piece * N, o, kv, D, B, sc);
}

template <int ST, int CT>
hipError_t launch_t(const KvWriteArgs& a, hipStream_t stream)
{
    constexpr int N = 16 / DtypeBytes<ST>::value;
    const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * 2 * (a.head_dim / N);
    if (total <= 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((kv_write_kernel<ST, CT>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(int src_dtype, int cache_dtype, const KvWriteArgs& a, hipStream_t stream)
{
    if (src_dtype == kF32 && cache_dtype == kF32) return launch_t<kF32, kF32>(a, stream);
    if (src_dtype == kBF16 && cache_dtype == kBF16) return launch_t<kBF16, kBF16>(a, stream);
    if (src_dtype == kBF16 && cache_dtype == kFP8) return launch_t<kBF16, kFP8>(a, stream);
    if (src_dtype == kF32 && cache_dtype == kFP8) return launch_t<kF32, kFP8>(a, stream);
    if (src_dtype == kBF16 && cache_dtype == kE5M2) return launch_t<kBF16, kE5M2>(a, stream);
    if (src_dtype == kF32 && cache_dtype == kE5M2) return launch_t<kF32, kE5M2>(a, stream);
    if (src_dtype == kBF16 && cache_dtype == kI8) return launch_t<kBF16, kI8>(a, stream);
    if (src_dtype == kF32 && cache_dtype == kI8) return launch_t<kF32, kI8>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
