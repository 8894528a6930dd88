// Row quantisers shared by the quantisation kernels and the fused small-batch
// front end (device code only).
//
// sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark MXFP4 MoE
// on gfx950", Summary: dynamic FP8 activations (1x128 groups here) and OCP
// MXFP4 1x32; UE8M0 scales: "[AMD] [GLM5] Opt-in prefill-only FP8 dense
// projection GEMM for MLA q_b/o_proj (gfx950)", Modifications.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Eight consecutive elements of one row as fp32 (zeros past `cols`).  VEC:
// the row start and stride allow 16-byte loads.
template <bool BF16, bool VEC>
__device__ __forceinline__ void load8(const void* in, int64_t row, int64_t ld, int col, int cols, float (&v)[8]) {
  if (BF16) {
    const uint16_t* p = (const uint16_t*)in + row * ld + col;
    if (VEC && col + 8 <= cols) {
      const uint4 w = *(const uint4*)p;
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (col + i < cols) ? bf16_to_f32(p[i]) : 0.0f;
    }
  } else {
    const float* p = (const float*)in + row * ld + col;
    if (VEC && col + 8 <= cols) {
      const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (col + i < cols) ? p[i] : 0.0f;
    }
  }
}

// One 128-column unit (16 lanes, 8 elements per lane) of the row
// quantisers, from its loaded values: FP8 (one group), UE8M0 FP8 (one
// group) or MX (four groups of 4 lanes).  Stores when `live`.
template <int MODE>
__device__ __forceinline__ void quant_unit(const float (&v)[8], bool live, int64_t row, int g, int col, int units,
                                           int cols_padded, uint8_t* __restrict__ q, void* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
  if constexpr (MODE == kQuantFp8) {
    a = group_max<16>(a);
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const float s = (a > 0.0f) ? a / kE4M3Max : 0.0f;
    if (a > 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = fp8_quant(v[i], s);
    }
    if (live) {
      *(uint2*)(q + row * (int64_t)cols_padded + col) =
          make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
      if ((lane & 15) == 0) ((float*)scales)[row * units + g] = s;
    }
  } else if constexpr (MODE == kQuantFp8E8) {
    a = group_max<16>(a);
    const uint32_t b = ue8m0_byte(a);
    const float inv = e8m0_inverse(b);
    uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (a > 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = fp8e8_quant(v[i], inv);
    }
    if (live) {
      *(uint2*)(q + row * (int64_t)cols_padded + col) =
          make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
      const int64_t lds = (units + 3) / 4 * 4;
      uint8_t* srow = (uint8_t*)scales + row * lds;
      if ((lane & 15) == 0) srow[g] = (uint8_t)b;
      if ((lane & 15) == 1 && g == units - 1) {
        for (int i = units; i < lds; ++i) srow[i] = 0;
      }
    }
  } else {
    a = group_max<4>(a);
    const uint32_t b = e8m0_byte(a);
    const float inv = e8m0_inverse(b);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= mx_quant(v[i], inv) << (4 * i);
    if (live) {
      *(uint32_t*)(q + row * (int64_t)(cols_padded / 2) + col / 2) = w;
      if ((lane & 3) == 0) ((uint8_t*)scales)[row * (int64_t)(cols_padded / 32) + col / 32] = (uint8_t)b;
    }
  }
}

// A wave quantises four 128-column units (16 lanes each, 8 elements per
// lane); a unit is one FP8 group or four MX groups of 4 lanes.  Wave `gw` of
// `nw` quantising waves takes units 4*gw .. +3, then every 4*nw-th.  A lane
// keeps its unit's (row, group) and steps both by the stride (one division
// at the start, none per unit).
// UE8M0 scale rows are e8_scale_ld(cols_padded) bytes long; the bytes past
// the last group are written as zero.  U: units per lane loaded before any
// is quantised (U loads in flight; the results do not depend on U).
template <bool BF16, bool VEC, int MODE, int U = 1>
__device__ __forceinline__ void quant_rows_body(const void* __restrict__ in, int64_t rows, int cols, int64_t ld_in,
                                                int cols_padded, uint8_t* __restrict__ q, void* __restrict__ scales,
                                                int64_t gw, int64_t nw) {
  const int lane = threadIdx.x & 63;
  const int units = cols_padded / 128;
  const int64_t total = rows * units;
  const int64_t stride = nw * 4;
  const int64_t drow = stride / units;
  const int dg = (int)(stride - drow * units);
  int64_t u = gw * 4 + (lane >> 4);
  int64_t row = u / units;
  int g = (int)(u - row * units);
  while (u - (lane >> 4) < total) {
    float v[U][8];
    int64_t ur[U], rr[U];
    int gr[U];
#pragma unroll
    for (int r = 0; r < U; ++r) {
      ur[r] = u;
      rr[r] = row;
      gr[r] = g;
      if (u < total) {
        load8<BF16, VEC>(in, row, ld_in, g * 128 + (lane & 15) * 8, cols, v[r]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[r][i] = 0.0f;
      }
      u += stride;
      row += drow;
      g += dg;
      if (g >= units) {
        g -= units;
        ++row;
      }
    }
#pragma unroll
    for (int r = 0; r < U; ++r) {
      // a pass whose units all lie past the end does nothing (its lanes
      // would only exchange zeros)
      if (ur[r] - (lane >> 4) >= total) break;
      const bool live = ur[r] < total;
      const int64_t row_r = live ? rr[r] : 0;
      const int g_r = live ? gr[r] : 0;
      quant_unit<MODE>(v[r], live, row_r, g_r, g_r * 128 + (lane & 15) * 8, units, cols_padded, q, scales);
    }
  }
}

}  // namespace moe
