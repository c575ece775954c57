// pa_device.hpp -- gfx950 device helpers shared by the paged-KV kernels.
//
// Element conversions and cross-lane primitives, written directly against CDNA4
// instructions through clang builtins: v_dot2c_f32_bf16, DPP row/quad moves, ds_swizzle,
// v_exp_f32, v_cvt_scalef32_pk_bf16_fp8 / _bf8 (OCP E4M3 / E5M2 -> bf16 pair),
// v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 (f32 -> OCP E4M3 / E5M2), v_cvt_f32_i32 with SDWA byte
// selects (INT8 -> f32), v_rndne_f32 (f32 -> INT8) and the gfx950 f32 -> bf16 pack.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// kFP8 is OCP fp8 E4M3, kE5M2 OCP fp8 E5M2 (AMD's "bf8"), kI8 a two's-complement 8-bit integer
// code (INT8 cache: value = code * scale).
enum Dtype : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kE5M2 = 3, kI8 = 4 };

template <int DT>
constexpr bool kIsFp8 = DT == kFP8 || DT == kE5M2;

// A quantised cache: 8-bit codes times a per-(layer, kv head) scale (fp8 or INT8).
template <int DT>
constexpr bool kIsQuant = kIsFp8<DT> || DT == kI8;

template <int DT>
struct DtypeBytes;
template <>
struct DtypeBytes<kF32> {
    static constexpr int value = 4;
};
template <>
struct DtypeBytes<kBF16> {
    static constexpr int value = 2;
};
template <>
struct DtypeBytes<kFP8> {
    static constexpr int value = 1;
};
template <>
struct DtypeBytes<kE5M2> {
    static constexpr int value = 1;
};
template <>
struct DtypeBytes<kI8> {
    static constexpr int value = 1;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kBf16OnePair = 0x3F803F80u;  // (1.0, 1.0) as two bf16

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

// c + a.lo*b.lo + a.hi*b.hi with a, b holding two bf16 each; products and sum in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two fp32 -> two bf16 (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x)
{
    return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return as_float(b << 16); }

// Two OCP E4M3 bytes (bits 0..15 if !hi, 16..31 if hi) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Two OCP E5M2 bytes -> two bf16, exact (every E5M2 value, infinities and NaN included, is a
// bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t e5m2x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}

// Two INT8 codes (bytes 0, 1 if !hi, bytes 2, 3 if hi) -> two bf16, exact (every integer in
// [-128, 127] is a bf16 value): each byte is sign-extended and converted to fp32 in one
// v_cvt_f32_i32 with an SDWA byte select, then the pair is packed with v_cvt_pk_bf16_f32.
template <bool HI>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w)
{
    const float lo = (float)(int8_t)(HI ? (w >> 16) & 0xFFu : w & 0xFFu);
    const float hi = (float)(int8_t)(HI ? w >> 24 : (w >> 8) & 0xFFu);
    return pack_bf16x2(lo, hi);
}

// Two 8-bit codes of quantised cache format KT -> two bf16 (exact for every format).
template <int KT, bool HI>
__device__ __forceinline__ uint32_t q8x2_to_bf16x2(uint32_t w)
{
    static_assert(kIsQuant<KT>, "8-bit cache formats only");
    if constexpr (KT == kFP8)
        return e4m3x2_to_bf16x2<HI>(w);
    else if constexpr (KT == kE5M2)
        return e5m2x2_to_bf16x2<HI>(w);
    else
        return i8x2_to_bf16x2<HI>(w);
}

// fp32 -> OCP E4M3 code: round to nearest even, finite overflow saturates to +-448, NaN
// keeps its sign and becomes S.1111.111.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y)
{
    if (__builtin_isnan(y)) return (as_uint(y) >> 24 & 0x80u) | 0x7Fu;
    float c = __builtin_fminf(__builtin_fmaxf(y, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// fp32 -> OCP E5M2 code: round to nearest even; finite overflow and the infinities saturate
// to +-57344 (the same saturating rule as E4M3), NaN keeps its sign and becomes S.11111.11.
__device__ __forceinline__ uint32_t f32_to_e5m2(float y)
{
    if (__builtin_isnan(y)) return (as_uint(y) >> 24 & 0x80u) | 0x7Fu;
    float c = __builtin_fminf(__builtin_fmaxf(y, -57344.0f), 57344.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, c, 0, false) & 0xFFu;
}

// fp32 -> INT8 code byte: the nearest integer, ties to even (v_rndne_f32), saturated to
// [-127, 127] (the symmetric range); NaN stores 0.
__device__ __forceinline__ uint32_t f32_to_i8(float y)
{
    if (__builtin_isnan(y)) return 0u;
    const float r = __builtin_rintf(__builtin_fminf(__builtin_fmaxf(y, -127.0f), 127.0f));
    return (uint32_t)(int32_t)r & 0xFFu;
}

template <int CT>
__device__ __forceinline__ uint32_t f32_to_q8(float y)
{
    static_assert(kIsQuant<CT>, "8-bit cache formats only");
    if constexpr (CT == kFP8)
        return f32_to_e4m3(y);
    else if constexpr (CT == kE5M2)
        return f32_to_e5m2(y);
    else
        return f32_to_i8(y);
}

// v_exp_f32: 2^x.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP move inside a row of 16 lanes; lanes whose source is outside the row read 0.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x)
{
    return as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_uint(x), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// Sum over the 4 lanes of a quad (every lane gets the sum).
__device__ __forceinline__ float quad_sum(float x)
{
    x += dpp_f32<kDppQuadSwap1>(x);
    x += dpp_f32<kDppQuadSwap2>(x);
    return x;
}

// Value held by lane ^ 4 (within 32-lane halves; ds_swizzle bitmask mode, xor 4).
__device__ __forceinline__ float swizzle_xor4(float x)
{
    return as_float((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_uint(x), 0x101F));
}

// Value held by lane ^ 16 (within 32-lane halves; ds_swizzle bitmask mode, xor 16).
__device__ __forceinline__ float swizzle_xor16(float x)
{
    return as_float((uint32_t)__builtin_amdgcn_ds_swizzle((int)as_uint(x), 0x401F));
}

// Maximum over all 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ float wave_max(float x)
{
    x = __builtin_fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
    x = __builtin_fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
    x = __builtin_fmaxf(x, dpp_f32<kDppRowRor4>(x));
    x = __builtin_fmaxf(x, dpp_f32<kDppRowRor8>(x));
    x = __builtin_fmaxf(x, __shfl_xor(x, 16, 64));
    x = __builtin_fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}

// Sum over all 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp_f32<kDppQuadSwap1>(x);
    x += dpp_f32<kDppQuadSwap2>(x);
    x += dpp_f32<kDppRowRor4>(x);
    x += dpp_f32<kDppRowRor8>(x);
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load with the nontemporal hint (global_load_dwordx4 ... nt): for data read once per
// launch, such as the K/V stream of decode.  Scattered 4 KiB tile reads run ~14% faster with
// it on MI355X (6.0 -> 6.8 TB/s in a random-order read probe).
__device__ __forceinline__ uint4 load16_stream(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A wave-uniform window of `bytes` bytes at `base`, read with buffer loads: an offset at or
// past the end (a window of 0 bytes makes every offset so) returns zeros without a memory
// access.  The descriptor is the raw-buffer form of the gfx9 family (stride 0, word 3
// 0x00020000); loads carry the nontemporal hint.
struct TileWindow {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ TileWindow(const void* base, int bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000))
    {
    }
    // bytes offset + soffset (offset per lane, soffset wave-uniform)
    __device__ __forceinline__ uint4 load_stream(int offset, int soffset = 0) const
    {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, offset, soffset, kBufferNontemporal);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    // the same load with the default cache policy: for bytes that other waves read again
    // (blocks shared between sequences)
    __device__ __forceinline__ uint4 load_cached(int offset, int soffset = 0) const
    {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, offset, soffset, 0);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    // 8- and 4-byte forms of the same loads
    __device__ __forceinline__ uint2 load_stream_b64(int offset, int soffset = 0) const
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, offset, soffset, kBufferNontemporal);
        const uint32_t v0 = v[0], v1 = v[1];
        return make_uint2(v0, v1);
    }
    __device__ __forceinline__ uint2 load_cached_b64(int offset, int soffset = 0) const
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, offset, soffset, 0);
        const uint32_t v0 = v[0], v1 = v[1];
        return make_uint2(v0, v1);
    }
    __device__ __forceinline__ uint32_t load_stream_b32(int offset, int soffset = 0) const
    {
        return __builtin_amdgcn_raw_buffer_load_b32(r, offset, soffset, kBufferNontemporal);
    }
    __device__ __forceinline__ uint32_t load_cached_b32(int offset, int soffset = 0) const
    {
        return __builtin_amdgcn_raw_buffer_load_b32(r, offset, soffset, 0);
    }
    // a uint2 or uint32_t piece, streamed or cached
    template <class T>
    __device__ __forceinline__ T load_piece(int offset, int soffset, bool cached) const
    {
        if constexpr (sizeof(T) == 8)
            return cached ? load_cached_b64(offset, soffset) : load_stream_b64(offset, soffset);
        else
            return cached ? load_cached_b32(offset, soffset) : load_stream_b32(offset, soffset);
    }
    static constexpr int kBufferNontemporal = 2;  // the cache-policy bit printed as "nt"
};

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace pa
