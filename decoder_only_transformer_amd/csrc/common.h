// Device-side helpers shared by the gfx950 kernels: storage types, bf16 / fp16 conversion,
// wave64 reductions, vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llk {

constexpr int kWave = 64;

// bf16 is handled as raw 16-bit storage; arithmetic is always fp32.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16: the conversion compiles to gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Value of x after storage in bf16.
__device__ __forceinline__ float round_bf16(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// Low / high bf16 of a packed pair -> fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// IEEE binary16 (fp16) is handled as raw 16-bit storage too; conversions go through clang's
// _Float16 (v_cvt_f16_f32 rounds to nearest even; v_cvt_f32_f16 is exact).
struct f16 {
    uint16_t bits;
};
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return static_cast<float>(__builtin_bit_cast(_Float16, h)); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }

// Element access for the storage types.  k16: a 16-bit type, whose values the method rounds
// where it stores them (round: the value after storage); lo / hi: the two elements of a
// packed 32-bit pair.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr bool k16 = false;
    __device__ __forceinline__ static float round(float x) { return x; }
    static constexpr int kPer16B = 4;
    __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
    // 16 bytes -> 4 floats
    __device__ __forceinline__ static void unpack(const uint4& v, float* out) {
        out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
    }
};
template <> struct Elem<bf16> {
    static constexpr bool k16 = true;
    __device__ __forceinline__ static float round(float x) { return round_bf16(x); }
    __device__ __forceinline__ static float lo(uint32_t w) { return bf16lo(w); }
    __device__ __forceinline__ static float hi(uint32_t w) { return bf16hi(w); }
    static constexpr int kPer16B = 8;
    __device__ __forceinline__ static float load(const bf16* p, size_t i) { return bf16_to_f32(p[i].bits); }
    __device__ __forceinline__ static void store(bf16* p, size_t i, float v) { p[i].bits = f32_to_bf16(v); }
    // 16 bytes -> 8 floats
    __device__ __forceinline__ static void unpack(const uint4& v, float* out) {
        out[0] = bf16lo(v.x); out[1] = bf16hi(v.x); out[2] = bf16lo(v.y); out[3] = bf16hi(v.y);
        out[4] = bf16lo(v.z); out[5] = bf16hi(v.z); out[6] = bf16lo(v.w); out[7] = bf16hi(v.w);
    }
};
template <> struct Elem<f16> {
    static constexpr bool k16 = true;
    __device__ __forceinline__ static float round(float x) { return f16_to_f32(f32_to_f16(x)); }
    __device__ __forceinline__ static float lo(uint32_t w) { return f16_to_f32(static_cast<uint16_t>(w & 0xffffu)); }
    __device__ __forceinline__ static float hi(uint32_t w) { return f16_to_f32(static_cast<uint16_t>(w >> 16)); }
    static constexpr int kPer16B = 8;
    __device__ __forceinline__ static float load(const f16* p, size_t i) { return f16_to_f32(p[i].bits); }
    __device__ __forceinline__ static void store(f16* p, size_t i, float v) { p[i].bits = f32_to_f16(v); }
    // 16 bytes -> 8 floats
    __device__ __forceinline__ static void unpack(const uint4& v, float* out) {
        out[0] = lo(v.x); out[1] = hi(v.x); out[2] = lo(v.y); out[3] = hi(v.y);
        out[4] = lo(v.z); out[5] = hi(v.z); out[6] = lo(v.w); out[7] = hi(v.w);
    }
};

// The 16-bit storage types on the MFMA path: the 16x16x32 product of that type with fp32
// accumulation, and the conversions the method's storage points use (round to nearest even).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <typename T16> struct Mma;
template <> struct Mma<bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    __device__ __forceinline__ static f32x4_t mma(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint16_t bits(float x) { return f32_to_bf16(x); }
    __device__ __forceinline__ static float value(uint16_t b) { return bf16_to_f32(b); }
    __device__ __forceinline__ static float round(float x) { return round_bf16(x); }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
};
template <> struct Mma<f16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    __device__ __forceinline__ static f32x4_t mma(v8 a, v8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint16_t bits(float x) { return f32_to_f16(x); }
    __device__ __forceinline__ static float value(uint16_t b) { return f16_to_f32(b); }
    __device__ __forceinline__ static float round(float x) { return f16_to_f32(f32_to_f16(x)); }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi) {
        return static_cast<uint32_t>(f32_to_f16(lo)) | (static_cast<uint32_t>(f32_to_f16(hi)) << 16);
    }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Streaming (read-once) 16-byte load: non-temporal hint so weights do not evict reused data.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
// x^2 exactly (a product of two fp32 values fits fp64's 53-bit significand)
__device__ __forceinline__ double sq64(float x) { return (double)x * (double)x; }
// x / d correctly rounded, given r = 1 / d from an IEEE division (correctly rounded) and a
// finite x and d with the quotient in the normal range: q0 = x r is within one ulp of x / d,
// the residual x - d q0 is exact in one FMA, and q0 + residual * r rounded once is the
// correctly rounded quotient (Markstein's correction step) -- three instructions per element
// where a row shares d, instead of the general division sequence.  With d = 1, r = 0 it
// returns 0 for any finite x.
__device__ __forceinline__ float div_rn(float x, float d, float r) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, d, x);
    return __builtin_fmaf(e, r, q0);
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
// Sum over aligned groups of `G` consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// v from another lane of the same DPP row (16 lanes) as selected by a DPP control word.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over each DPP row of 16 lanes, in every lane of the row, on DPP moves (VALU) rather
// than LDS permutes: pair swap, quad half swap, mirror within 8 lanes, mirror within 16.
template <>
__device__ __forceinline__ float group_sum<16>(float v) {
    v += dpp_f32<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_f32<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_f32<0x141>(v);   // row_half_mirror
    v += dpp_f32<0x140>(v);   // row_mirror
    return v;
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }


// Fragment-major position of element (m, k) of a bf16 activation matrix kept as mt tiles of
// 16 rows: the 16 x 32 block (row tile m / 16, k-step k / 32) is 1 KB laid out in the lane
// order of an MFMA 16x16x32 B operand, lane (m % 16) + 16 * ((k % 32) / 8) holding 8
// consecutive k.  Rows past the matrix inside the last tile are padding.
__device__ __forceinline__ size_t frag_index(int m, int k, int mt) {
    return ((size_t)(k >> 5) * mt + (m >> 4)) * 512 + ((k >> 3) & 3) * 128 + (m & 15) * 8 + (k & 7);
}

}  // namespace llk
