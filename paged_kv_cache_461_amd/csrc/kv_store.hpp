// kv_store.hpp -- store one 16-byte piece of a new token's K or V row into its pool slot.
//
// The append kernel stores with store_kv_piece; the decode kernel's fused append encodes with
// encode_elem and stores the encoded bytes with store_piece_bytes, and both end in
// store_piece_codes, so both write the same bytes.  Each decode step stores the new token's K/V
// in the cache (page 1, section 1, the prefill/decode diagram) at its slot, the physical block
// from the sequence's block table and the offset inside it (page 1, section 4).  Layouts are those of include/pagedattn.h: a K
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

// Store N elements already in the cache's encoding (codes[i]: the low EC bytes), source
// elements d0 .. d0 + N - 1 of a token's K or V row.  pool: the K or V pool (kv = 0 or 1);
// tile: element offset of the (block, kv head) tile; o: token offset inside the block.
template <int CT, int N>
__device__ __forceinline__ void store_piece_codes(const uint32_t (&codes)[N], unsigned char* pool, int64_t tile, int d0,
                                                  int o, int kv, int D, int B)
{
    constexpr int EC = DtypeBytes<CT>::value;
    constexpr int W = 64 / EC;  // cache channels per 64-byte slice
    static_assert(W % N == 0, "a piece never straddles a slice");
    static_assert(N * EC == 4 || N * EC == 8 || N * EC == 16, "a K piece is one 4-, 8- or 16-byte store");
    if (kv == 0) {  // K: contiguous inside the channel slice
        const int64_t slice = tile + (int64_t)(d0 / W) * B * W;  // element offset of the slice
        unsigned char* dst = pool + (slice + (int64_t)o * W + d0 % W) * EC;
        constexpr int PER = 4 / EC;  // elements per 32-bit word
        uint32_t w[N * EC / 4];
#pragma unroll
        for (int k = 0; k < N * EC / 4; k++) {
            w[k] = 0;
#pragma unroll
            for (int i = 0; i < PER; i++) w[k] |= codes[k * PER + i] << (8 * EC * i);
        }
        if constexpr (N * EC == 16)
            *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        else if constexpr (N * EC == 8)
            *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        else
            *reinterpret_cast<uint32_t*>(dst) = w[0];
    } else {
        // V: token group (o / T), channel d, position o % T inside the channel's 16-byte piece;
        // element-sized stores touch only this token's bytes
        const int T = (16 / EC) < B ? (16 / EC) : B;
        const int64_t vbase = tile + ((int64_t)(o / T) * D + d0) * T + (o % T);
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int64_t e = vbase + (int64_t)i * T;
            if constexpr (EC == 4)
                reinterpret_cast<uint32_t*>(pool)[e] = codes[i];
            else if constexpr (EC == 2)
                reinterpret_cast<uint16_t*>(pool)[e] = (uint16_t)codes[i];
            else
                pool[e] = (unsigned char)codes[i];
        }
    }
}

// The same store from the piece's N * EC bytes already encoded (in LDS or registers).
template <int CT, int N>
__device__ __forceinline__ void store_piece_bytes(const unsigned char* enc, unsigned char* pool, int64_t tile, int d0,
                                                  int o, int kv, int D, int B)
{
    constexpr int EC = DtypeBytes<CT>::value;
    constexpr int NW = N * EC / 4;  // 32-bit words of the piece
    uint32_t w[NW];
    if constexpr (NW == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(enc);
        w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
    } else if constexpr (NW == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(enc);
        w[0] = v.x, w[1] = v.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t*>(enc);
    }
    constexpr int PER = 4 / EC;  // elements per word
    uint32_t codes[N];
#pragma unroll
    for (int i = 0; i < N; i++) {
        if constexpr (EC == 4)
            codes[i] = w[i];
        else
            codes[i] = (w[i / PER] >> (8 * EC * (i % PER))) & ((1u << (8 * EC)) - 1u);
    }
    store_piece_codes<CT, N>(codes, pool, tile, d0, o, kv, D, B);
}

// src: the piece's 16 source bytes (source elements d0 .. d0 + N - 1 of the row), encoded
// with encode_elem and stored with store_piece_codes; scale: the head's scale (8-bit cache only).
template <int ST, int CT>
__device__ __forceinline__ void store_kv_piece(const uint4 raw, unsigned char* pool, int64_t tile, int d0, int o, int kv,
                                               int D, int B, float scale)
{
    constexpr int N = 16 / DtypeBytes<ST>::value;  // source elements per piece
    const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t codes[N];
#pragma unroll
    for (int i = 0; i < N; i++) codes[i] = encode_elem<ST, CT>(words, i, scale);
    store_piece_codes<CT, N>(codes, pool, tile, d0, o, kv, D, B);
}

}  // namespace pa
