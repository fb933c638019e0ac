// device_common.hpp -- small gfx950 device helpers shared by the ConvRot HIP kernels.
// Internal to libconvrot; not part of the public C-ABI.
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

constexpr int kWave = 64;                 // CDNA wavefront width
constexpr float kMagicRound = 12582912.0f; // 1.5 * 2^23: adding it leaves round-to-nearest-even(x) in the low mantissa bits

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32); a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    v2bf16 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// Lane exchanges inside a quad (DPP quad_perm), all lanes enabled.
__device__ __forceinline__ float dpp_xor1(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)); // [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)); // [2,3,0,1]
}

// x[i] += c * x[i] of the partner lane (lane ^ 1 for QUAD_PERM "[1,0,3,2]", lane ^ 2 for
// "[2,3,0,1]"), for 8 values: one v_fmac_f32 per value with its first source read through DPP.
// (The compiler keeps a separate v_mov_b32_dpp for the tied-accumulator fmac.)  The leading
// s_nop covers the DPP read-after-VALU-write hazard for all eight: inside the block each
// instruction reads only the register it alone writes.
#define CONVROT_FMAC_DPP8(QUAD_PERM)                                                                        \
    __device__ __forceinline__ void fmac_dpp8_##QUAD_PERM##_(float (&x)[8], float c)                       \
    {                                                                                                       \
        asm volatile("s_nop 1\n\t"                                                                         \
                     "v_fmac_f32_dpp %0, %0, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                     "v_fmac_f32_dpp %1, %1, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                     "v_fmac_f32_dpp %2, %2, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                     "v_fmac_f32_dpp %3, %3, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                     "v_fmac_f32_dpp %4, %4, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                     "v_fmac_f32_dpp %5, %5, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                     "v_fmac_f32_dpp %6, %6, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
                     "v_fmac_f32_dpp %7, %7, %8 quad_perm:" QP_##QUAD_PERM " row_mask:0xf bank_mask:0xf bound_ctrl:1" \
                     : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),    \
                       "+v"(x[7])                                                                           \
                     : "v"(c));                                                                             \
    }
#define QP_xor1 "[1,0,3,2]"
#define QP_xor2 "[2,3,0,1]"
CONVROT_FMAC_DPP8(xor1)
CONVROT_FMAC_DPP8(xor2)
#undef CONVROT_FMAC_DPP8
#undef QP_xor1
#undef QP_xor2

// Exchange the upper 32 lanes of `a` with the lower 32 lanes of `b` (v_permlane32_swap):
// afterwards a = [a_lo | b_lo], b = [a_hi | b_hi].
__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b)
{
    auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap32f(float &a, float &b)
{
    uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    swap32(ua, ub);
    a = __uint_as_float(ua);
    b = __uint_as_float(ub);
}

// Round-to-nearest-even of x*m with a single rounding; the signed integer sits in the low
// bits of the returned float's bit pattern (valid for |x*m| < 2^22).
__device__ __forceinline__ uint32_t rne_bits(float x, float m) { return __float_as_uint(__builtin_fmaf(x, m, kMagicRound)); }

// fp16 nearest-even rounding of the exact quotient a / d (a >= 0, d > 0, both fp32) with a single
// rounding.  Rounding the fp32 quotient to fp16 would round twice; instead the fp32 quotient is
// first made round-to-odd (the correctly rounded q, moved one ulp towards the true value when it
// is inexact and its last bit is even; the remainder a - q*d is exact in one fma and gives the
// direction), and round-to-odd at 24 bits followed by nearest-even at 11 bits is exact rounding.
__device__ __forceinline__ __half f16_quotient_rne(float a, float d)
{
    const float q = a / d;
    const float r = __builtin_fmaf(-q, d, a);
    uint32_t b = __float_as_uint(q);
    if (r != 0.0f && !(b & 1u)) b += r > 0.0f ? 1u : (b ? 0xffffffffu : 0u);
    return __float2half_rn(__uint_as_float(b));
}

// Low bytes of four rne_bits() results -> one packed dword (byte 0 = t0).
__device__ __forceinline__ uint32_t pack4_i8(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3)
{
    uint32_t p01 = __builtin_amdgcn_perm(t1, t0, 0x0c0c0400u);
    uint32_t p23 = __builtin_amdgcn_perm(t3, t2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// Low nibbles of eight rne_bits() results -> one dword (nibble i = t[i]).
__device__ __forceinline__ uint32_t pack8_i4(const uint32_t *t)
{
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) r |= (t[i] & 0xFu) << (4 * i);
    return r;
}

} // namespace convrot
