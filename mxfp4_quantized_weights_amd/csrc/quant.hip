// Quantisers and the weight preshuffle.
//
// sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark MXFP4 MoE
// on gfx950", Summary: block FP8 [128,128] weights with dynamic FP8
// activations (per token, 1x128 groups here), and OCP MXFP4 1x32 for weights
// and activations; contract table: the runner that consumes a preshuffled
// layout owns it.
//
// Block FP8 group:  s = amax / 448 (fp32 division), q = RNE(clamp(v / s)),
//                   amax = 0 -> s = 0, all codes 0x00.
// MXFP4 group (32): b = clamp(floor(log2 amax) - 2 + 127, 0, 254) (0 for
//                   amax = 0), q = RNE_E2M1(clamp(v * 2^(127 - b), +-6)),
//                   element 2i in the low nibble of byte i.
// UE8M0 FP8 group:  ("[AMD] [GLM5] Opt-in prefill-only FP8 dense projection
//                   GEMM for MLA q_b/o_proj (gfx950)", Modifications) scale
//                   2^e, e smallest with 448 * 2^e >= amax, stored as the
//                   byte b = clamp(e + 127, 0, 254) (0 for amax = 0);
//                   q = RNE(v * 2^(127 - b)).
#include "moe_device.h"
#include "moe_internal.h"
#include "moe_quant_rows.h"

namespace moe {

template <bool BF16, bool VEC, int MODE>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ in, int64_t rows, int cols,
                                                         int64_t ld_in, int cols_padded,
                                                         uint8_t* __restrict__ q, void* __restrict__ scales) {
  quant_rows_body<BF16, VEC, MODE>(in, rows, cols, ld_in, cols_padded, q, scales,
                                   (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), (int64_t)gridDim.x * 4);
}

template <bool BF16, bool VEC>
static void launch_quant_rows_t(dim3 grid, hipStream_t s, const void* in, int64_t rows, int cols, int64_t ld_in,
                                int cols_padded, int mode, uint8_t* q, void* scales) {
  if (mode == kQuantFp8)
    hipLaunchKernelGGL((quant_rows_kernel<BF16, VEC, kQuantFp8>), grid, dim3(256), 0, s, in, rows, cols, ld_in,
                       cols_padded, q, scales);
  else if (mode == kQuantFp8E8)
    hipLaunchKernelGGL((quant_rows_kernel<BF16, VEC, kQuantFp8E8>), grid, dim3(256), 0, s, in, rows, cols, ld_in,
                       cols_padded, q, scales);
  else
    hipLaunchKernelGGL((quant_rows_kernel<BF16, VEC, kQuantMx>), grid, dim3(256), 0, s, in, rows, cols, ld_in,
                       cols_padded, q, scales);
}

hipError_t launch_quant_rows(const void* in, bool in_is_bf16, int64_t rows, int cols, int64_t ld_in,
                             int cols_padded, int mode, void* q, void* scales, hipStream_t s) {
  const int64_t units = rows * (cols_padded / 128);
  int64_t blocks = (units + 15) / 16;  // 16 units per workgroup
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  dim3 grid((unsigned)blocks);
  uint8_t* qb = (uint8_t*)q;
  const int esize = in_is_bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)in % 16 == 0) && ((ld_in * esize) % 16 == 0);
  if (in_is_bf16) {
    if (vec) launch_quant_rows_t<true, true>(grid, s, in, rows, cols, ld_in, cols_padded, mode, qb, scales);
    else launch_quant_rows_t<true, false>(grid, s, in, rows, cols, ld_in, cols_padded, mode, qb, scales);
  } else {
    if (vec) launch_quant_rows_t<false, true>(grid, s, in, rows, cols, ld_in, cols_padded, mode, qb, scales);
    else launch_quant_rows_t<false, false>(grid, s, in, rows, cols, ld_in, cols_padded, mode, qb, scales);
  }
  return hipGetLastError();
}

// One workgroup per [128, 128] block; thread t covers row t/2, columns
// 64*(t%2) .. +64.  E8: UE8M0 scale bytes instead of fp32 scales.
template <bool E8>
__global__ __launch_bounds__(256) void quant_weight_fp8_kernel(const float* __restrict__ w, int N, int K,
                                                               uint8_t* __restrict__ q, void* __restrict__ scales) {
  __shared__ float red[4];
  const int nbk = K / 128, nbn = N / 128;
  const int64_t blk = blockIdx.x;
  const int64_t e = blk / ((int64_t)nbn * nbk);
  const int bn = (int)((blk / nbk) % nbn), bk = (int)(blk % nbk);
  const int t = threadIdx.x;
  const int64_t r = (int64_t)bn * 128 + (t >> 1);
  const int c0 = bk * 128 + (t & 1) * 64;
  const float4* src = (const float4*)(w + (e * N + r) * (int64_t)K + c0);
  float4 v[16];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = src[i];
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  }
  a = group_max<16>(a);
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48)));
  if ((t & 63) == 0) red[t >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  uint32_t* dst = (uint32_t*)(q + (e * N + r) * (int64_t)K + c0);
  const int64_t si = (e * nbn + bn) * nbk + bk;
  if constexpr (E8) {
    const uint32_t b = ue8m0_byte(a);
    const float inv = e8m0_inverse(b);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t word = 0;
      if (a > 0.0f) {
        word = fp8e8_quant(v[i].x, inv) | (fp8e8_quant(v[i].y, inv) << 8) | (fp8e8_quant(v[i].z, inv) << 16) |
               (fp8e8_quant(v[i].w, inv) << 24);
      }
      dst[i] = word;
    }
    if (t == 0) ((uint8_t*)scales)[si] = (uint8_t)b;
  } else {
    const float s = (a > 0.0f) ? a / kE4M3Max : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t word = 0;
      if (a > 0.0f) {
        word = fp8_quant(v[i].x, s) | (fp8_quant(v[i].y, s) << 8) | (fp8_quant(v[i].z, s) << 16) |
               (fp8_quant(v[i].w, s) << 24);
      }
      dst[i] = word;
    }
    if (t == 0) ((float*)scales)[si] = s;
  }
}

hipError_t launch_quant_weight_fp8(int mode, const float* w, int E, int N, int K, uint8_t* q, void* scales,
                                   hipStream_t s) {
  int64_t blocks = (int64_t)E * (N / 128) * (K / 128);
  if (mode == kQuantFp8E8)
    hipLaunchKernelGGL(quant_weight_fp8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, w, N, K, q, scales);
  else
    hipLaunchKernelGGL(quant_weight_fp8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, w, N, K, q, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// TILED_V2 preshuffle.  For each expert, 16-row tile and 128-wide K block kb,
// the kernels' B operand is one MFMA 16x16x128 tile: lane l needs the tile's
// row l%16 and K values kb*128 + 32*(l/16) .. +32.
//   FP8: tile = 2048 bytes, [h (2)][lane (64)][16 bytes]: half h holds the
//        lane's K bytes 16h .. 16h+15, so each 16-byte wave load is 1 KB
//        contiguous.  Block scales stay canonical f32 [E, N/128, K/128].
//   UE8M0 FP8: the same tiles; the scale bytes are widened to their exact
//        fp32 values 2^(b-127) in the canonical [E, N/128, K/128] order.
//   MX:  tile = 1024 bytes, [lane (64)][16 bytes] (32 packed E2M1).  Scales:
//        per (expert, N tile, group of 4 K blocks, tile position) one
//        [lane (64)][4 bytes] word row, byte i = E8M0 of K block 4q+i for
//        the lane's row and 32-group; missing K blocks (K/128 not a multiple
//        of 4) hold 0.
// Tiles are ordered [E][N tile][16 / R][K block][R] for the matrix's tile
// run R (tiled_row_tile names the row tile at each position 0..15,
// tiled_index the storage order), so the tiles one GEMM item needs at one K
// block come in contiguous runs of R tiles.  MX scale word rows follow the
// same order with groups of 4 K blocks in place of K blocks.
// Positions without a row tile (a half last N tile of w2) hold zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void preshuffle_fp8_kernel(const uint8_t* __restrict__ w, int64_t total_chunks,
                                                             int N, int K, int gate_half, int R, uint8_t* __restrict__ out) {
  const int KB = K / 128, NG = tiled_n_groups(N);
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total_chunks; c += (int64_t)gridDim.x * 256) {
    const int within = (int)(c & 127);
    const int h = within >> 6, l = within & 63;
    int64_t rest = c >> 7;  // storage tile index
    const int ir = (int)(rest % R);
    rest /= R;
    const int kb = (int)(rest % KB);
    rest /= KB;
    const int i = (int)(rest % (16 / R)) * R + ir;
    rest /= 16 / R;
    const int g = (int)(rest % NG);
    const int64_t e = rest / NG;
    const int rt = tiled_row_tile(gate_half, N, g, i);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (rt >= 0) {
      const int64_t row = (int64_t)rt * 16 + (l & 15);
      const int64_t col = (int64_t)kb * 128 + 32 * (l >> 4) + 16 * h;
      v = *(const uint4*)(w + (e * N + row) * (int64_t)K + col);
    }
    *(uint4*)(out + c * 16) = v;
  }
}

__global__ __launch_bounds__(256) void preshuffle_mx_kernel(const uint8_t* __restrict__ w, int64_t total_chunks,
                                                            int N, int K, int gate_half, int R, uint8_t* __restrict__ out) {
  const int KB = K / 128, NG = tiled_n_groups(N);
  const int64_t ldw = K / 2;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total_chunks; c += (int64_t)gridDim.x * 256) {
    const int l = (int)(c & 63);
    int64_t rest = c >> 6;  // storage tile index
    const int ir = (int)(rest % R);
    rest /= R;
    const int kb = (int)(rest % KB);
    rest /= KB;
    const int i = (int)(rest % (16 / R)) * R + ir;
    rest /= 16 / R;
    const int g = (int)(rest % NG);
    const int64_t e = rest / NG;
    const int rt = tiled_row_tile(gate_half, N, g, i);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (rt >= 0) {
      const int64_t row = (int64_t)rt * 16 + (l & 15);
      const int64_t col = (int64_t)kb * 64 + 16 * (l >> 4);
      v = *(const uint4*)(w + (e * N + row) * ldw + col);
    }
    *(uint4*)(out + c * 16) = v;
  }
}

__global__ __launch_bounds__(256) void preshuffle_mx_scale_kernel(const uint8_t* __restrict__ s, int64_t total_words,
                                                                  int N, int K, int gate_half, int R,
                                                                  uint32_t* __restrict__ out) {
  const int KB = K / 128, KB4 = (KB + 3) / 4, NG = tiled_n_groups(N);
  const int64_t lds = K / 32;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total_words; c += (int64_t)gridDim.x * 256) {
    const int l = (int)(c & 63);
    int64_t rest = c >> 6;  // storage word-row index, ordered as the tiles with K groups of 4 blocks
    const int ir = (int)(rest % R);
    rest /= R;
    const int kq = (int)(rest % KB4);
    rest /= KB4;
    const int i = (int)(rest % (16 / R)) * R + ir;
    rest /= 16 / R;
    const int g = (int)(rest % NG);
    const int64_t e = rest / NG;
    const int rt = tiled_row_tile(gate_half, N, g, i);
    uint32_t word = 0;
    if (rt >= 0) {
      const int64_t row = (int64_t)rt * 16 + (l & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = kq * 4 + j;
        if (kb < KB) word |= (uint32_t)s[(e * N + row) * lds + kb * 4 + (l >> 4)] << (8 * j);
      }
    }
    out[c] = word;
  }
}

__global__ __launch_bounds__(256) void e8m0_to_f32_kernel(const uint8_t* __restrict__ in, int64_t n,
                                                          float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out[i] = e8m0_value(in[i]);
}

__global__ __launch_bounds__(256) void copy_words_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                         uint32_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) out[i] = in[i];
}

static unsigned grid_for(int64_t items) {
  int64_t b = (items + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

hipError_t launch_preshuffle(int mode, const uint8_t* w, const void* sc, int E, int N, int K, int gate_half, int R,
                             uint8_t* w_out, void* s_out, hipStream_t s) {
  const int64_t KB = K / 128, NG = tiled_n_groups(N);
  if (mode == kQuantFp8 || mode == kQuantFp8E8) {
    const int64_t chunks = (int64_t)E * NG * KB * 16 * 128;
    hipLaunchKernelGGL(preshuffle_fp8_kernel, dim3(grid_for(chunks)), dim3(256), 0, s, w, chunks, N, K, gate_half,
                       R, w_out);
    const int64_t words = (int64_t)E * (N / 128) * KB;
    if (mode == kQuantFp8E8)
      hipLaunchKernelGGL(e8m0_to_f32_kernel, dim3(grid_for(words)), dim3(256), 0, s, (const uint8_t*)sc, words,
                         (float*)s_out);
    else
      hipLaunchKernelGGL(copy_words_kernel, dim3(grid_for(words)), dim3(256), 0, s, (const uint32_t*)sc, words,
                         (uint32_t*)s_out);
  } else {
    const int64_t chunks = (int64_t)E * NG * KB * 16 * 64;
    hipLaunchKernelGGL(preshuffle_mx_kernel, dim3(grid_for(chunks)), dim3(256), 0, s, w, chunks, N, K, gate_half,
                       R, w_out);
    const int64_t words = (int64_t)E * NG * ((KB + 3) / 4) * 16 * 64;
    hipLaunchKernelGGL(preshuffle_mx_scale_kernel, dim3(grid_for(words)), dim3(256), 0, s, (const uint8_t*)sc,
                       words, N, K, gate_half, R, (uint32_t*)s_out);
  }
  return hipGetLastError();
}

}  // namespace moe
