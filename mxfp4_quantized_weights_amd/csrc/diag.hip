// Diagnostic: one 16x16 output tile of A . B^T over K = 128 from e4m3 codes,
// computed the way each grouped GEMM computes a K block, so that tests can
// compare the two matrix-core sums against an exact one.
//   kind 0: one FP8 MFMA (16x16x128, unit E8M0 scales), as GEMM2 does;
//   kind 1: the operands widened exactly to f16 and four chained 16x16x32
//           f16 MFMAs, as GEMM1 does (its output is re-quantised, so its sum
//           must stay within fp32 rounding of the exact one).
// Lane l holds row l % 16 of A and of B and K bytes 32*(l/16) .. +32, the
// fragment layout of the GEMM kernels; result lane l holds
// C[4*(l/16) + i][l % 16], i = 0..3.
#include "../../include/moe.h"
#include "moe_device.h"

namespace moe {

// One instance per kind: the result is read in the MFMA's own basic block,
// where the compiler inserts the wait states the instruction needs (read from
// a join block after a branch, the FP8 instruction's first result register
// was read too early).
template <int KIND>
__global__ __launch_bounds__(64) void mfma_tile_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                       float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int row = lane & 15, k0 = 32 * (lane >> 4);
  const uint4* pa = (const uint4*)(a + row * 128 + k0);
  const uint4* pb = (const uint4*)(b + row * 128 + k0);
  const uint4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  const v8i av{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const v8i bv{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  v4f c = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (KIND == 0) {
    c = mfma_fp8(av, bv, c);
  } else {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t ad0 = (uint32_t)av[2 * st], ad1 = (uint32_t)av[2 * st + 1];
      const uint32_t bd0 = (uint32_t)bv[2 * st], bd1 = (uint32_t)bv[2 * st + 1];
      const uint4 ah = make_uint4(e4m3x2_to_f16x2<false>(ad0), e4m3x2_to_f16x2<true>(ad0),
                                  e4m3x2_to_f16x2<false>(ad1), e4m3x2_to_f16x2<true>(ad1));
      const uint4 bh = make_uint4(e4m3x2_to_f16x2<false>(bd0), e4m3x2_to_f16x2<true>(bd0),
                                  e4m3x2_to_f16x2<false>(bd1), e4m3x2_to_f16x2<true>(bd1));
      c = mfma_f16(__builtin_bit_cast(v8h, ah), __builtin_bit_cast(v8h, bh), c);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) out[(4 * (lane >> 4) + i) * 16 + row] = c[i];
}

// Matrix-core rate: every wave runs `iters` rounds of 8 independent
// accumulator chains of one instruction (no memory traffic in the loop), so
// the launch time gives the part's MFMA throughput for that instruction.
//   kind 0: 16x16x32 f16 (GEMM1's block-FP8 path), 16384 FLOP each;
//   kind 1: 16x16x128 FP8 e4m3, unit E8M0 scales (GEMM2), 65536 FLOP each;
//   kind 2: 16x16x128 FP4 e2m1, unit E8M0 scales (the MXFP4 GEMMs), 65536.
// The instructions are written as inline assembly with each accumulator tied
// to its own registers: with the builtins the compiler keeps loop-carried
// accumulators in AGPRs and copies them between the MFMAs, which halves the
// rate.  (The GEMM kernels start each MFMA chain from zero inside the K loop
// and have no such copies.)  The wait states around the loop cover the
// VALU->MFMA and MFMA->VALU hazards the compiler cannot see in assembly.
// Each thread writes the sum of its accumulators to out (a sink).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* __restrict__ out) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const float f = (float)lane;
  v4f a0{f, 0, 0, 0}, a1{f + 1, 0, 0, 0}, a2{f + 2, 0, 0, 0}, a3{f + 3, 0, 0, 0};
  v4f a4{f + 4, 0, 0, 0}, a5{f + 5, 0, 0, 0}, a6{f + 6, 0, 0, 0}, a7{f + 7, 0, 0, 0};
  // small finite e4m3 / e2m1 bytes and f16 values from the lane id
  const int word = (0x08 + (lane & 7)) * 0x01010101;
  v8i q{word, word, word, word, word, word, word, word};
  v4i q4{word & 0x33333333, word & 0x33333333, word & 0x33333333, word & 0x33333333};
  const _Float16 hv = (_Float16)(0.0078125f * (float)(1 + (lane & 7)));
  v8h h{hv, hv, hv, hv, hv, hv, hv, hv};
  int one = 127;  // E8M0 2^0
  // the wait states take the registers as operands, so the compiler keeps
  // every VALU write of them before this point and every read after the last
  asm volatile("s_nop 7" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(one));
  if constexpr (KIND == 0) asm volatile("s_nop 7" : "+v"(h));
  if constexpr (KIND == 1) asm volatile("s_nop 7" : "+v"(q));
  if constexpr (KIND == 2) asm volatile("s_nop 7" : "+v"(q4));
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == 0) {
#define MOE_RATE_STEP(A) asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %1, %0" : "+v"(A) : "v"(h))
      MOE_RATE_STEP(a0); MOE_RATE_STEP(a1); MOE_RATE_STEP(a2); MOE_RATE_STEP(a3);
      MOE_RATE_STEP(a4); MOE_RATE_STEP(a5); MOE_RATE_STEP(a6); MOE_RATE_STEP(a7);
#undef MOE_RATE_STEP
    } else if constexpr (KIND == 1) {
#define MOE_RATE_STEP(A) \
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %1, %0, %2, %2 op_sel_hi:[0,0,0]" : "+v"(A) : "v"(q), "v"(one))
      MOE_RATE_STEP(a0); MOE_RATE_STEP(a1); MOE_RATE_STEP(a2); MOE_RATE_STEP(a3);
      MOE_RATE_STEP(a4); MOE_RATE_STEP(a5); MOE_RATE_STEP(a6); MOE_RATE_STEP(a7);
#undef MOE_RATE_STEP
    } else {
#define MOE_RATE_STEP(A)                                                                                   \
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %1, %0, %2, %2 op_sel_hi:[0,0,0] cbsz:4 blgp:4" \
               : "+v"(A)                                                                                   \
               : "v"(q4), "v"(one))
      MOE_RATE_STEP(a0); MOE_RATE_STEP(a1); MOE_RATE_STEP(a2); MOE_RATE_STEP(a3);
      MOE_RATE_STEP(a4); MOE_RATE_STEP(a5); MOE_RATE_STEP(a6); MOE_RATE_STEP(a7);
#undef MOE_RATE_STEP
    }
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
  const v4f s = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

// Read stream: each workgroup reads a contiguous share of the buffer, its
// lanes loading consecutive 16-byte words (non-temporal, as the GEMMs load
// their weights) with four loads in flight, and folds them into a checksum,
// one word per thread in sink.  (Of the forms measured on an MI355X --
// grid-stride or per-workgroup shares, 256 to 1024 threads, 4 or 8 loads in
// flight, 256 to 4096 workgroups -- this one read fastest: 7.2 TB/s against
// 5.8-6.0 for grid-stride loops.)
__global__ __launch_bounds__(512) void stream_read_kernel(const void* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  constexpr int NT = 512;
  const v4u* p = (const v4u*)src;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < n16 ? lo + per : n16;
  int64_t i = lo + threadIdx.x;
  v4u x = v4u{0u, 0u, 0u, 0u};
  for (; i + 3 * NT < hi; i += 4 * NT) {
    const v4u a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + NT);
    const v4u c = __builtin_nontemporal_load(p + i + 2 * NT), d = __builtin_nontemporal_load(p + i + 3 * NT);
    x ^= a ^ b ^ c ^ d;
  }
  for (; i < hi; i += NT) x ^= __builtin_nontemporal_load(p + i);
  sink[(int64_t)blockIdx.x * NT + threadIdx.x] = x.x ^ x.y ^ x.z ^ x.w;
}

}  // namespace moe

extern "C" moe_status_t moe_diag_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return MOE_ERR_NULL;
  if (bytes < 0) return MOE_ERR_SHAPE;
  if ((uintptr_t)src % 16 != 0 || bytes % 16 != 0) return MOE_ERR_ALIGN;
  hipLaunchKernelGGL(moe::stream_read_kernel, dim3(MOE_DIAG_STREAM_WORKGROUPS), dim3(512), 0, (hipStream_t)stream,
                     src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_diag_mfma_rate(int32_t kind, int32_t iters, float* out, void* stream) {
  if (kind < 0 || kind > 2 || iters < 1) return MOE_ERR_UNSUPPORTED;
  if (!out) return MOE_ERR_NULL;
  const dim3 grid(MOE_DIAG_MFMA_RATE_WORKGROUPS), block(256);
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(moe::mfma_rate_kernel<0>, grid, block, 0, s, iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(moe::mfma_rate_kernel<1>, grid, block, 0, s, iters, out);
  else
    hipLaunchKernelGGL(moe::mfma_rate_kernel<2>, grid, block, 0, s, iters, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_diag_mfma_tile(int32_t kind, const void* a, const void* b, float* out, void* stream) {
  if (kind != 0 && kind != 1) return MOE_ERR_UNSUPPORTED;
  if (!a || !b || !out) return MOE_ERR_NULL;
  if (((uintptr_t)a | (uintptr_t)b) % 16 != 0) return MOE_ERR_ALIGN;
  if (kind == 0)
    hipLaunchKernelGGL(moe::mfma_tile_kernel<0>, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a,
                       (const uint8_t*)b, out);
  else
    hipLaunchKernelGGL(moe::mfma_tile_kernel<1>, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a,
                       (const uint8_t*)b, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
