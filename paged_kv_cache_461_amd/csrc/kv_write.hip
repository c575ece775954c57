// kv_write.hip -- paged KV append: store each new token's K and V rows into its block slot.
//
// Each decode step produces the new token's K/V and stores it in the cache (page 1,
// section 1, the prefill/decode diagram); the slot is physical block * block_size + offset
// from the sequence's block table (page 1, section 4).
//
// One thread moves one 16-byte piece of one source row (token, kv head, K or V).  A K piece
// lands contiguously inside one 64-byte channel slice of the tile; a V piece is spread over
// its channels' token groups (layout in include/pagedattn.h), so V is written with
// element-sized stores that touch only this token's bytes.  Same-dtype append copies bits.
// bf16/fp32 -> OCP E4M3 divides by the head's scale in binary32 (round to nearest even) and
// converts with v_cvt_pk_fp8_f32 after clamping to +-448 (saturation), NaN handled explicitly.
#include "pa_device.hpp"
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
    const uint4 raw = load16(src);
    const int d0 = piece * N;
    const int64_t tile = (blk * Hkv + h) * (int64_t)B * D;   // element offset of the tile
    const int64_t slice = tile + (int64_t)(d0 / W) * B * W;  // element offset of the slice
    unsigned char* pool = static_cast<unsigned char*>(kv ? a.v_pool : a.k_pool);

    uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
    // V: token group (o / T), channel d, position o % T inside the channel's 16-byte piece
    const int T = (16 / EC) < B ? (16 / EC) : B;
    const int64_t vbase = tile + ((int64_t)(o / T) * D + d0) * T + (o % T);
    if constexpr (ST == CT) {
        if (kv == 0) {
            *reinterpret_cast<uint4*>(pool + (slice + (int64_t)o * W + d0 % W) * EC) = raw;
        } else {
#pragma unroll
            for (int i = 0; i < N; i++) {
                const int64_t e = vbase + (int64_t)i * T;
                if constexpr (EC == 4)
                    reinterpret_cast<uint32_t*>(pool)[e] = words[i];
                else
                    reinterpret_cast<uint16_t*>(pool)[e] = (uint16_t)(words[i / 2] >> (16 * (i % 2)));
            }
        }
    } else {
        static_assert(CT == kFP8, "conversions go to E4M3 only");
        const float sc = (kv ? a.v_scale : a.k_scale)[h];
        uint32_t codes[N];
#pragma unroll
        for (int i = 0; i < N; i++) {
            float x;
            if constexpr (ST == kBF16)
                x = bf16_bits_to_f32((words[i / 2] >> (16 * (i % 2))) & 0xFFFFu);
            else
                x = as_float(words[i]);
            codes[i] = f32_to_e4m3(__fdiv_rn(x, sc));
        }
        if (kv == 0) {
            unsigned char* dst = pool + slice + (int64_t)o * W + d0 % W;
            if constexpr (N == 8) {
                uint2 packed;
                packed.x = codes[0] | codes[1] << 8 | codes[2] << 16 | codes[3] << 24;
                packed.y = codes[4] | codes[5] << 8 | codes[6] << 16 | codes[7] << 24;
                *reinterpret_cast<uint2*>(dst) = packed;
            } else {
                *reinterpret_cast<uint32_t*>(dst) = codes[0] | codes[1] << 8 | codes[2] << 16 | codes[3] << 24;
            }
        } else {
#pragma unroll
            for (int i = 0; i < N; i++) pool[vbase + (int64_t)i * T] = (unsigned char)codes[i];
        }
    }
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
    return hipErrorInvalidValue;
}

}  // namespace pa
