// Host-side launchers shared between the library's translation units.  Every
// launcher assumes its arguments were validated by the C ABI layer and returns
// the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kQuantFp8 = 1;
constexpr int kQuantMx = 2;
// GEMM operand mode: FP8 storage, operands widened to f16 for an MFMA whose
// internal sum is exact to fp32 precision (internal to the GEMM kernels).
constexpr int kQuantFp8F16 = 3;

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);

hipError_t launch_permute_align(const int32_t* ids, int T, int k, int E, int block_m, int nb,
                                int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                                int32_t* npp, hipStream_t s);

// in_is_bf16: element type of `in`; rows x cols valid, row stride ld_in elements.
hipError_t launch_quant_rows(const void* in, bool in_is_bf16, int64_t rows, int cols, int64_t ld_in,
                             int cols_padded, int mode, void* q, void* scales, hipStream_t s);

hipError_t launch_quant_weight_fp8(const float* w, int E, int N, int K, uint8_t* q, float* scales,
                                   hipStream_t s);

hipError_t launch_preshuffle(int mode, const uint8_t* w, const void* sc, int E, int N, int K,
                             uint8_t* w_out, void* s_out, hipStream_t s);

struct GemmArgs {
  const uint8_t* A;       // GEMM1: quantised x [T, ...]; GEMM2: aq [rows, ...]
  const void* As;         // activation scales
  int64_t lda;            // bytes per A row
  int64_t ldas;           // scale elements per A row (FP8: floats, MX: bytes)
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* npp;
  int32_t top_k;
  int32_t num_pairs;
  const uint8_t* B;       // TILED_V1 weights
  const void* Bs;         // FP8: canonical f32 block scales; MX: tiled scale dwords
  int32_t N;              // weight rows per expert (padded)
  int32_t K;              // reduction length (padded)
  int32_t n_tiles;        // N-tiles per M-block
  uint8_t* aq;            // GEMM1 outputs
  void* as;
  int32_t Ip;
  float limit;
  float* y;               // GEMM2 output: weighted per-pair rows [P, N]
  const float* topk_w;    // [P]
};

hipError_t launch_gemm1(int mode, int block_m, int nb, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm2(int mode, int block_m, int nb, const GemmArgs& a, hipStream_t s);

hipError_t launch_combine(const float* y, int T, int k, int H, int Hp, uint16_t* out, int64_t ld_out,
                          hipStream_t s);

}  // namespace moe
