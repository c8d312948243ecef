// moe_device.h -- device-side helpers shared by the gfx950 kernels: element
// formats (fp32, bf16, MXFP4), 16-byte chunk dot products, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int WAVE = 64;

// ---- scalar conversions --------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even: the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32) in the default round-to-nearest-even mode
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// lo*lo' + hi*hi' + c on packed bf16 pairs, fp32 accumulate (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// E8M0 scale code -> fp32 multiplier 2^(code-127) (code 0 maps to 0, 255 to inf)
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) { return __uint_as_float(code << 23); }

// two E2M1 codes of byte `sel` of `packed` (low nibble first) times `scale`, as bf16x2
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t packed, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, SEL));
}

// silu(g) * u = g * u / (1 + e^-g), with the hardware reciprocal (v_rcp_f32, 1 ulp)
// instead of a correctly rounded division: the result is stored as bf16 (or compared at
// 1e-5 relative in fp32), far above that error.  g -> -inf gives g * rcp(inf) = -0.
__device__ __forceinline__ float swiglu(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// streaming (non-temporal) 16-byte load: weights are read once per call
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- wave64 reductions -----------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// DPP move of v (fp32 bits); lanes with no source read `fill`
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v, float fill) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v), CTRL, ROW_MASK, 0xf,
                                                      false));
}

// Sums of groups of 16 / 32 / 64 consecutive lanes through DPP row shifts and
// row broadcasts (no LDS traffic).  The group's total lands in its last lane
// (lane 15 of each row, lanes 31 and 63, or lane 63).
__device__ __forceinline__ float dpp_sum16(float v) {
    v += dpp_f<0x111>(v, 0.f);  // row_shr:1
    v += dpp_f<0x112>(v, 0.f);  // row_shr:2
    v += dpp_f<0x114>(v, 0.f);  // row_shr:4
    v += dpp_f<0x118>(v, 0.f);  // row_shr:8
    return v;
}
__device__ __forceinline__ float dpp_sum32(float v) {
    v = dpp_sum16(v);
    return v + dpp_f<0x142, 0xa>(v, 0.f);  // row_bcast:15 into rows 1 and 3
}
__device__ __forceinline__ float dpp_sum64(float v) {
    v = dpp_sum32(v);
    return v + dpp_f<0x143, 0xc>(v, 0.f);  // row_bcast:31 into rows 2 and 3
}
// wave-uniform total of v over the 64 lanes
__device__ __forceinline__ float wave_sum_u(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dpp_sum64(v)), 63));
}
__device__ __forceinline__ float wave_max_u(float v) {
    const float ninf = -__builtin_inff();
    v = fmaxf(v, dpp_f<0x111>(v, ninf));
    v = fmaxf(v, dpp_f<0x112>(v, ninf));
    v = fmaxf(v, dpp_f<0x114>(v, ninf));
    v = fmaxf(v, dpp_f<0x118>(v, ninf));
    v = fmaxf(v, dpp_f<0x142, 0xa>(v, ninf));
    v = fmaxf(v, dpp_f<0x143, 0xc>(v, ninf));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// order-preserving map of fp32 to uint32 (-0 and +0 map to the same key)
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- element formats -------------------------------------------------------------
// A "chunk" is 16 bytes of a weight row: 4 fp32, 8 bf16 or 32 MXFP4 codes (one
// scale block).  Dot products are taken chunk by chunk against the matching
// activation elements.

struct FmtF32 {  // fp32 weights with fp32 activations
    static constexpr int EPC = 4;          // elements per 16-byte weight chunk
    static constexpr int XB = 16;          // activation bytes per chunk
    static constexpr bool SCALED = false;
};
struct FmtBF16 {  // bf16 weights with bf16 activations
    static constexpr int EPC = 8;
    static constexpr int XB = 16;
    static constexpr bool SCALED = false;
};
struct FmtMX4 {  // MXFP4 weights with bf16 activations
    static constexpr int EPC = 32;
    static constexpr int XB = 64;
    static constexpr bool SCALED = true;
};

// partial dot of one weight chunk with the activation chunk at xp (XB bytes)
template <class F>
__device__ __forceinline__ float chunk_dot(const uint4 &w, uint32_t scale_code, const uint8_t *xp, float acc);

template <>
__device__ __forceinline__ float chunk_dot<FmtF32>(const uint4 &w, uint32_t, const uint8_t *xp, float acc) {
    const float4 xv = *reinterpret_cast<const float4 *>(xp);
    acc = fmaf(__uint_as_float(w.x), xv.x, acc);
    acc = fmaf(__uint_as_float(w.y), xv.y, acc);
    acc = fmaf(__uint_as_float(w.z), xv.z, acc);
    acc = fmaf(__uint_as_float(w.w), xv.w, acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<FmtBF16>(const uint4 &w, uint32_t, const uint8_t *xp, float acc) {
    const uint4 xv = *reinterpret_cast<const uint4 *>(xp);
    acc = dot2_bf16(w.x, xv.x, acc);
    acc = dot2_bf16(w.y, xv.y, acc);
    acc = dot2_bf16(w.z, xv.z, acc);
    acc = dot2_bf16(w.w, xv.w, acc);
    return acc;
}

__device__ __forceinline__ float mx4_word_dot(uint32_t codes, float s, const uint4 &xv, float acc) {
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(codes, s), xv.x, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(codes, s), xv.y, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(codes, s), xv.z, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(codes, s), xv.w, acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<FmtMX4>(const uint4 &w, uint32_t scale_code, const uint8_t *xp, float acc) {
    const float s = e8m0_to_f32(scale_code);
    const uint4 *x4 = reinterpret_cast<const uint4 *>(xp);
    acc = mx4_word_dot(w.x, s, x4[0], acc);
    acc = mx4_word_dot(w.y, s, x4[1], acc);
    acc = mx4_word_dot(w.z, s, x4[2], acc);
    acc = mx4_word_dot(w.w, s, x4[3], acc);
    return acc;
}

}  // namespace moe
