// Device-side helpers for the MoE kernels (gfx950): number-format conversions,
// wave reductions and MFMA wrappers.
//
// Formats (sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark
// MXFP4 MoE on gfx950", Summary): OCP E4M3FN for block FP8, OCP MXFP4 = E2M1
// elements with one E8M0 scale per 32 elements.  The rounding conversions
// (fp32 -> e4m3 / E2M1 / bf16, E8M0 exponents) are written with integer and
// round-to-nearest-even arithmetic, so their results are fixed by
// construction; only exact widenings (e4m3 -> f16) use a hardware convert.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

// E4M3FN code of a finite fp32 value with |v| <= 448, rounded to nearest,
// ties to even; the sign bit is kept (also for zero and for values that round
// to zero).  This is the hardware conversion, which rounds exactly so on
// gfx950: the GPU quantiser tests hold its codes to the oracle's on every
// E4M3 value and midpoint and their fp32 neighbours, at several group scales,
// and on rows spanning fp32's range, subnormals and signed zeros included.
// One instruction instead of a branch per value.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

// E2M1 code of a finite fp32 value with |v| <= 6 (grid 0, .5, 1, 1.5, 2, 3,
// 4, 6), rounded to nearest, ties to the even code; sign in bit 3 (kept for
// zero).  The hardware conversion with scale 1, which rounds exactly so on
// gfx950: the GPU quantiser tests hold its codes to the oracle's on every
// grid value and midpoint and their fp32 neighbours, at several E8M0 scales.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu;
}

// E8M0 byte of an MX block: 2^(floor(log2 amax) - 2) biased by 127, clamped to
// [0, 254]; 0 for amax == 0.  floor(log2) comes from the exponent bits
// (subnormals included), never from a log instruction.
__device__ __forceinline__ uint32_t e8m0_byte(float amax) {
  uint32_t u = __float_as_uint(amax);
  if (u == 0u) return 0u;
  int e;
  uint32_t ef = u >> 23;
  if (ef) {
    e = (int)ef - 127;
  } else {
    e = (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;
  }
  int b = e - 2 + 127;
  return (uint32_t)(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// 2^(127 - b) as fp32 for b in [0, 252] (always a normal number).
__device__ __forceinline__ float e8m0_inverse(uint32_t b) {
  return __uint_as_float((254u - b) << 23);
}

// 2^(b - 127) as fp32 for an E8M0 byte b in [0, 254]; b = 0 is the fp32
// subnormal 2^-127.
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

// UE8M0 block scale ("[AMD] [GLM5] Opt-in prefill-only FP8 dense projection
// GEMM for MLA q_b/o_proj (gfx950)", Modifications: e4m3 with a 128x128 UE8M0
// scale): 2^e with e the smallest integer such that 448 * 2^e >= amax,
// biased by 127 and clamped to [0, 254]; 0 for amax == 0.  With amax =
// 1.m * 2^E, 448 * 2^e = 1.75 * 2^(e+8), so e = E - 8 when 1.m <= 1.75
// (mantissa field <= 0x600000), else E - 7.  Subnormal amax is normalised
// first.
__device__ __forceinline__ uint32_t ue8m0_byte(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0u) return 0u;
  int E;
  uint32_t mant;
  const uint32_t ef = u >> 23;
  if (ef) {
    E = (int)ef - 127;
    mant = u & 0x7FFFFFu;
  } else {
    const int p = 31 - __builtin_clz(u);
    E = p - 149;
    mant = (u << (23 - p)) & 0x7FFFFFu;
  }
  const int b = E - 8 + (mant > 0x600000u ? 1 : 0) + 127;
  return (uint32_t)(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// e4m3 code of v in a UE8M0 group with scale byte b (inv = 2^(127 - b)):
// the scaling is exact, and |v| * inv <= 448 by the choice of b.
__device__ __forceinline__ uint32_t fp8e8_quant(float v, float inv) {
  float r = v * inv;
  r = fminf(fmaxf(r, -kE4M3Max), kE4M3Max);
  return e4m3_code(r);
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Quantise one value of a block-FP8 group whose scale s = amax/448 > 0.
__device__ __forceinline__ uint32_t fp8_quant(float v, float s) {
  float r = v / s;  // IEEE division (built with correctly rounded fp32 divide)
  r = fminf(fmaxf(r, -kE4M3Max), kE4M3Max);
  return e4m3_code(r);
}

// E4M3FN code of v * inv, saturated to +-448: the re-quantisation of GEMM1's
// SwiGLU output, with inv = fl32(1/s) computed once per group.  v * inv is
// within 1.5 ulp of the IEEE quotient v / s, so a code can differ from
// fp8_quant's only where v / s lies that close to a rounding midpoint; the
// intermediate's codes already differ from a host computation at such ties,
// because GEMM1's fp32 sums run in another order.
__device__ __forceinline__ uint32_t fp8_quant_inv(float v, float inv) {
  float r = v * inv;
  r = fminf(fmaxf(r, -kE4M3Max), kE4M3Max);
  return e4m3_code(r);
}

// Quantise one value of an MX group with scale byte b (inv = 2^(127-b)).
__device__ __forceinline__ uint32_t mx_quant(float v, float inv) {
  float r = v * inv;  // exact scaling by a power of two
  r = fminf(fmaxf(r, -kE2M1Max), kE2M1Max);
  return e2m1_code(r);
}

// silu(g) = g / (1 + e^-g), with the hardware exp2 and reciprocal (each a
// few ulp; a relative error of ~1e-6 at |g| = 10): the value is re-quantised
// right after, where only codes at a rounding tie can move.  Large negative g
// gives e^-g = inf and silu = -0, as the exact formula in fp32.
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// Clamped SwiGLU (FreeToken PR #270, Summary): silu(min(g, L)) * clamp(u, -L, L).
__device__ __forceinline__ float swiglu_clamped(float g, float u, float L) {
  float gc = fminf(g, L);
  float uc = fminf(fmaxf(u, -L), L);
  return silu_f32(gc) * uc;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over aligned groups of WIDTH lanes (4 or 16), every lane of the
// group receives it.  DPP quad swaps, then half-row and row mirrors.
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
  static_assert(WIDTH == 4 || WIDTH == 16, "group of 4 or 16 lanes");
  v = fmaxf(v, dpp_f32<0xB1>(v));     // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));     // quad_perm [2,3,0,1]
  if constexpr (WIDTH == 16) {
    v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  }
  return v;
}

// 16x16x128 FP8 (e4m3 x e4m3) MFMA with unit E8M0 scales (byte 127 = 2^0).
// Lane l holds A row (l % 16), K bytes [32*(l/16), +32); B likewise for its
// column; the result lane l holds C[4*(l/16) + i][l % 16], i = 0..3.
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x128 FP8 MFMA with per-lane E8M0 scales: sa scales lane l's 32 A
// values (row l % 16), sb its 32 B values; a power-of-two block scale is
// applied exactly inside the instruction.
__device__ __forceinline__ v4f mfma_fp8_scaled(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Two e4m3 values (bytes 0,1 or 2,3 of w) to two f16 values.  Exact: every
// e4m3 value, subnormals included, is an f16 value (scale 1.0).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  v2h h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, h);
}

// 16x16x32 f16 MFMA, fp32 accumulation.  Lane l holds A row (l % 16), 8
// values of K; result layout as mfma_fp8.  Used where the sum must be exact
// to fp32 precision: the gfx950 FP8 MFMA drops low-order bits of small
// products inside its internal sum, the f16 one does not.
__device__ __forceinline__ v4f mfma_f16(const v8h& a, const v8h& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The lane's 32 FP8 bytes as four f16 operands: step st holds bytes
// 8st..8st+7, i.e. K = 32*(lane/16) + 8st + i for both A and B.
__device__ __forceinline__ void widen_fp8(const v8i& w, v8h (&h)[4]) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const uint32_t d0 = (uint32_t)w[2 * st], d1 = (uint32_t)w[2 * st + 1];
    const uint4 v = make_uint4(e4m3x2_to_f16x2<false>(d0), e4m3x2_to_f16x2<true>(d0),
                               e4m3x2_to_f16x2<false>(d1), e4m3x2_to_f16x2<true>(d1));
    h[st] = __builtin_bit_cast(v8h, v);
  }
}

// 16x16x128 FP4 (E2M1 x E2M1) MFMA with per-lane E8M0 scales: lane l's scale
// applies to its own 32 K-values (its A row / B column, K group l/16).  The A
// scale is byte 0 of sa; the B scale is byte OPB of sb.
template <int OPB>
__device__ __forceinline__ v4f mfma_fp4_scaled(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, OPB, sb);
}

}  // namespace moe
