// kv_store.hpp -- store one 16-byte piece of a new token's K or V row into its pool slot.
//
// The append kernel stores with store_kv_piece; the decode kernel's fused append encodes with
// encode_elem, so both write the same bytes.  Each decode step stores the new token's K/V in
// the cache (page 1, section 1, the prefill/decode diagram) at its slot, the physical block from the sequence's block table and
// the offset inside it (page 1, section 4).  Layouts are those of include/pagedattn.h: a K
// piece lands contiguously inside one 64-byte channel slice of the (block, kv head) tile; a V
// piece is spread over its channels' token groups, so V is written with element-sized stores
// that touch only this token's bytes.  Same-dtype append copies bits; bf16/fp32 -> OCP E4M3 or
// E5M2 divides by the head's scale in binary32 (round to nearest even) and converts with
// v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 after clamping to the format's largest finite value
// (saturation), NaN handled explicitly.
#pragma once

#include "pa_device.hpp"

namespace pa {

// Element i of a 16-byte source piece in the cache's encoding (the low EC bytes of the result):
// the same bits for the same dtype; for an fp8 cache, x / scale in binary32 (round to nearest
// even) converted with saturation.
template <int ST, int CT>
__device__ __forceinline__ uint32_t encode_elem(const uint32_t (&words)[4], int i, float scale)
{
    constexpr int ES = DtypeBytes<ST>::value;
    if constexpr (ST == CT) {
        if constexpr (ES == 4)
            return words[i];
        else
            return (words[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
    } else {
        static_assert(kIsQuant<CT>, "conversions go to 8-bit codes only");
        float x;
        if constexpr (ST == kBF16)
            x = bf16_bits_to_f32((words[i / 2] >> (16 * (i % 2))) & 0xFFFFu);
        else
            x = as_float(words[i]);
        return f32_to_q8<CT>(__fdiv_rn(x, scale));
    }
}

// src: the piece's 16 source bytes (source elements d0 .. d0 + N - 1 of the row).
// pool: the K or V pool (kv = 0 or 1); tile: element offset of the (block, kv head) tile;
// o: token offset inside the block; scale: the head's fp8 scale (fp8 cache only).
template <int ST, int CT>
__device__ __forceinline__ void store_kv_piece(const uint4 raw, unsigned char* pool, int64_t tile, int d0, int o, int kv,
                                               int D, int B, float scale)
{
    constexpr int ES = DtypeBytes<ST>::value;
    constexpr int EC = DtypeBytes<CT>::value;
    constexpr int N = 16 / ES;  // source elements per piece
    constexpr int W = 64 / EC;  // cache channels per 64-byte slice
    static_assert(W % N == 0, "a piece never straddles a slice");
    const int64_t slice = tile + (int64_t)(d0 / W) * B * W;  // element offset of the slice
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
        static_assert(kIsQuant<CT>, "conversions go to 8-bit codes only");
        uint32_t codes[N];
#pragma unroll
        for (int i = 0; i < N; i++) codes[i] = encode_elem<ST, CT>(words, i, scale);
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

}  // namespace pa
