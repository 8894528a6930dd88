// Host-side launchers shared between the library's translation units.  Every
// launcher assumes its arguments were validated by the C ABI layer and returns
// the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Quantisation contracts (the values of MOE_QUANT_* in include/moe.h).
constexpr int kQuantFp8 = 1;    // e4m3, fp32 scales (128x128 weights, 1x128 activations)
constexpr int kQuantMx = 2;     // E2M1 + E8M0 per 1x32
constexpr int kQuantFp8E8 = 3;  // e4m3, UE8M0 scale bytes (128x128 weights, 1x128 activations)

// Row stride in bytes of UE8M0 activation-scale rows: one byte per 128
// columns, rounded up to whole dwords so that the GEMMs load aligned words.
inline int64_t e8_scale_ld(int64_t cols_padded) { return (cols_padded / 128 + 3) / 4 * 4; }

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);

hipError_t launch_permute_align(const int32_t* ids, int T, int k, int E, int block_m, int nb,
                                int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                                int32_t* npp, hipStream_t s);

// in_is_bf16: element type of `in`; rows x cols valid, row stride ld_in elements.
hipError_t launch_quant_rows(const void* in, bool in_is_bf16, int64_t rows, int cols, int64_t ld_in,
                             int cols_padded, int mode, void* q, void* scales, hipStream_t s);

// Block FP8 weights, one scale per [128, 128] block: fp32 (kQuantFp8) or a
// UE8M0 byte (kQuantFp8E8).
hipError_t launch_quant_weight_fp8(int mode, const float* w, int E, int N, int K, uint8_t* q, void* scales,
                                   hipStream_t s);

hipError_t launch_preshuffle(int mode, const uint8_t* w, const void* sc, int E, int N, int K,
                             uint8_t* w_out, void* s_out, hipStream_t s);

struct GemmArgs {
  const uint8_t* A;       // GEMM1: quantised x [T, ...]; GEMM2: aq [rows, ...]
  const void* As;         // activation scales
  int64_t lda;            // bytes per A row
  int64_t ldas;           // scale elements per A row (FP8: floats; MX, UE8M0: bytes)
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* npp;
  int32_t top_k;
  int32_t num_pairs;
  const uint8_t* B;       // TILED_V1 weights
  const void* Bs;         // FP8, UE8M0: f32 block scales [E, N/128, K/128]; MX: tiled scale dwords
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
