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

}  // namespace moe

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
