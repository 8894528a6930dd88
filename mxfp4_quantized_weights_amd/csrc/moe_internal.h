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
__host__ __device__ inline int64_t e8_scale_ld(int64_t cols_padded) { return (cols_padded / 128 + 3) / 4 * 4; }

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);

hipError_t launch_permute_align(const int32_t* ids, int T, int k, int E, int block_m, int nb,
                                int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                                int32_t* npp, hipStream_t s);

// Routing (as launch_route_topk) and quantisation of bf16 x (as
// launch_quant_rows) in one launch, for any batch with E <= 1024.
hipError_t launch_route_and_quant(const float* logits, int T, int E, int k, int32_t* ids, float* w, const void* x_bf16,
                                  int H, int64_t ld_x, int Hp, int mode, void* xq, void* xs, hipStream_t s);

// Routing, permutation and quantisation of bf16 x in one launch (T <= 16)
// or two, for batches where front_small_ok(T, E, k) holds (same results as the three
// stage launchers for routing output, which never repeats an expert).
bool front_small_ok(int T, int E, int k);
hipError_t launch_front_small(const float* logits, int T, int E, int k, int32_t* ids, float* w, int block_m, int nb,
                              int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets, int32_t* npp,
                              const void* x_bf16, int H, int64_t ld_x, int Hp, int mode, void* xq, void* xs,
                              hipStream_t s);

// in_is_bf16: element type of `in`; rows x cols valid, row stride ld_in elements.
hipError_t launch_quant_rows(const void* in, bool in_is_bf16, int64_t rows, int cols, int64_t ld_in,
                             int cols_padded, int mode, void* q, void* scales, hipStream_t s);

// Block FP8 weights, one scale per [128, 128] block: fp32 (kQuantFp8) or a
// UE8M0 byte (kQuantFp8E8).
hipError_t launch_quant_weight_fp8(int mode, const float* w, int E, int N, int K, uint8_t* q, void* scales,
                                   hipStream_t s);

// TILED_V2 weight layout: a matrix's 16-row tiles are grouped into N tiles of
// 16 (the 256 weight rows one GEMM item multiplies), each K block of an N
// tile in contiguous runs of tiles (below).  For w13 (gate_half = Ip/16 > 0) N tile g holds gate row
// tiles 8g .. 8g+7 and then the matching up row tiles gate_half + 8g ..;
// for w2 (gate_half = 0) row tiles 16g .. 16g+15, the positions past N/16
// of a last, half N tile holding zeros.
__host__ __device__ inline int tiled_n_groups(int N) { return (N + 255) / 256; }
__host__ __device__ inline int tiled_row_tile(int gate_half, int N, int g, int i) {
  if (gate_half > 0) return i < 8 ? 8 * g + i : gate_half + 8 * g + (i - 8);
  const int t = 16 * g + i;
  return t < N / 16 ? t : -1;
}
// Within an N tile, runs of R positions (the tile run) are contiguous per K
// block: tiles are ordered [E][N tile][16 / R][K block][R], so tile position
// i of N tile g at K block kb sits at tile index
// (((e * NG + g) * (16 / R) + i / R) * KB + kb) * R + i % R, and stepping one
// K block moves every position by R tiles.  MX scale word rows follow the
// same order, groups of 4 K blocks taking the place of K blocks.
__host__ __device__ inline int64_t tiled_index(int R, int64_t e, int NG, int g, int i, int KB, int kb) {
  return ((((e * NG + g) * (16 / R) + i / R) * KB + kb) * R) + i % R;
}
// The tile run of each matrix, fixed by the quantisation mode and the matrix
// (13: w13, 2: w2); measured on the MI355X (all layouts give bit-identical
// results): whole 16-tile runs stream fastest for a purely streaming item
// list (block-FP8 w13 at small batches), runs of 4 suit w2 at every batch,
// and MXFP4 w13 at large batches is fastest with single tiles.
inline int tile_run(int mode, int which) {
  if (which == 2) return 4;
  return mode == kQuantMx ? 1 : 16;
}

// CANONICAL -> TILED_V2 (gate_half as above: Ip/16 for w13, 0 for w2; tile
// run R from tile_run).
hipError_t launch_preshuffle(int mode, const uint8_t* w, const void* sc, int E, int N, int K, int gate_half, int R,
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
  const uint8_t* B;       // TILED_V2 weights
  const void* Bs;         // FP8, UE8M0: f32 block scales [E, N/128, K/128]; MX: tiled scale dwords
  int32_t N;              // weight rows per expert (padded)
  int32_t K;              // reduction length (padded)
  int32_t n_tiles;        // N-tiles per M-block
  uint8_t* aq;            // GEMM1 outputs
  void* as;
  int32_t Ip;
  float limit;
  uint8_t* y;             // GEMM2 output: weighted per-pair rows, columns nt0*256 .. (plane 0; see y_plane_bytes)
  const float* topk_w;    // [P]
  int32_t nt0;            // GEMM2: first 256-column N tile of this launch (items cover n_tiles tiles)
  int64_t ldy;            // GEMM2: row stride of y in values (a multiple of 256)
  int32_t ks_log2;        // K split: each item covers K / 2^ks_log2 of the reduction
  float* part;            // GEMM1 with a K split: fp32 partial sums [2^ks_log2, P, 2*Ip], then int32 [P]
  int64_t yplane;         // GEMM2 with a K split: bytes between the y planes of the K pieces
  int64_t yexp;           // GEMM2: byte offset of the exponents within a plane
  int32_t tile_run;       // TILED_V2 tile run R of B (tile_run(mode, which))
  int32_t tail;           // GEMM1 with a K split: whole items in whole rounds, only the rest split (see below)
  int32_t ntg;            // N tiles per item (set by launch_gemm1 / launch_gemm2)
};

// K split of the grouped GEMMs for small batches.  When few (M block, N tile)
// items exist, each is cut into 2, 4 or 8 pieces along K so that every CU
// streams weights: GEMM1 pieces store fp32 partial sums that
// launch_swiglu_requant adds in piece order before the clamped SwiGLU and
// the re-quantisation; GEMM2 pieces store their own y plane and the combine
// adds the planes.  Only batches of at most kSplitMaxPairs pairs are split.
constexpr int kSplitMaxPairs = 1024;
constexpr int kSplitMax = 8;
// Largest split a GEMM with KB 128-wide K blocks can take (pieces of whole
// dwords of UE8M0/E8M0 scale bytes, i.e. multiples of 4 K blocks, for the MX
// and UE8M0 modes; at least 4 K blocks per piece).
int ksplit_cap(int mode, int KB);
bool ksplit_ok(int mode, int KB, int ks);
// The split the library uses for a GEMM of n_tiles N tiles per block and KB
// K blocks, for T tokens: the largest whose pieces do not outnumber the
// workgroups (one per CU), from the expected number of active experts under
// uniform routing.  Host-only; depends on the device's CU count.
int pick_ksplit(int mode, int T, int E, int k, int block_m, int KB, int n_tiles);

// Tail split of GEMM1 (every block_m): a launch over gemm_grid_max()
// workgroups runs the F = floor(items / W) whole rounds of (M block, N tile)
// items unsplit, with the fused epilogue, and cuts only the items past them
// into ks pieces, which store fp32 partial sums part[piece][r][block_m][256]
// (r < W: leftover item r; 128 gate then 128 up columns of its N tile).  A
// second kernel (one workgroup per possible r) adds the pieces in order and
// applies the clamped SwiGLU and the re-quantisation.  This evens out the last
// round of items without splitting the rest.
int gemm_grid_max();
// Whether the planner uses a tail split for a GEMM1 of n_tiles N tiles at T
// tokens (estimated leftover items at most 0.7 of a round).
bool tail_split_plan_ok(int T, int E, int k, int block_m, int n_tiles);
hipError_t launch_gemm1_tail_finish(int mode, int ks, int block_m, const float* part, const int32_t* sorted,
                                    const int32_t* npp, int n_tiles, int W, int P, int Ip, float limit, uint8_t* aq,
                                    void* as, hipStream_t s);

// GEMM1 with a K split (ks = 2, 4 or 8), second half: for each pair f < P,
// h = sum over pieces of part[piece, f], then the clamped SwiGLU and the
// re-quantisation of the fused GEMM1 epilogue, into the pair's sorted row
// (which GEMM1 stored after the partial sums; it also zeroed the pad rows).
hipError_t launch_swiglu_requant(int mode, const float* part, int ks, int P, int Ip, float limit, uint8_t* aq,
                                 void* as, hipStream_t s);

// GEMM2's weighted per-pair rows y are block floating point: one plane holds
// int16 values [pairs, cols] (256-byte aligned) and then one int8 exponent s
// per 64 columns [pairs, cols/64]; value v of a group is stored as
// q = rint(v * 2^-s), saturated to the int16 range, with s =
// max(floor(log2 max|v|) - 14, -128): |v| * 2^-s < 2^15, so v' = q * 2^s
// differs from v by at most 2^(s-1) (2^-15 of the group's largest |v|), or
// 2^s where the largest value rounds to 2^15 and saturates.  The combine
// decodes exactly and sums in fp32.  Half the bytes of fp32 rows, for the
// two passes over them.  Within each 64-column group the values are stored
// in GEMM2's lane order: position 16q + 4j + i holds column 16j + 4q + i
// (y_group_col), so each lane of GEMM2 writes 32 contiguous bytes.
__host__ __device__ inline int y_group_col(int pos) {
  const int u = pos & 63;
  return (pos & ~63) + 16 * ((u >> 2) & 3) + 4 * (u >> 4) + (u & 3);
}
inline int64_t y_values_bytes(int64_t pairs, int64_t cols) { return (pairs * cols * 2 + 255) / 256 * 256; }
inline int64_t y_plane_bytes(int64_t pairs, int64_t cols) {
  return y_values_bytes(pairs, cols) + (pairs * (cols / 64) + 255) / 256 * 256;
}

// Columns of y kept at once: all Hp when a plane of P rows fits in
// kYChunkBytes, else the largest multiple of 256 that does (at least 256).
// GEMM2 and the combine then run once per column chunk on the same y buffer,
// which bounds the workspace of very large batches.  Chunks cost time (each
// re-runs GEMM2's item list and its tail, and the memory-side cache does not
// keep a 64-128 MiB chunk between GEMM2 and the combine), so the cap is set
// high: a 4096-token, 288-expert top-8 layer (260 MiB of y) runs in one piece.
#ifndef MOE_Y_CHUNK_BYTES
#define MOE_Y_CHUNK_BYTES (1ll << 30)
#endif
constexpr int64_t kYChunkBytes = MOE_Y_CHUNK_BYTES;
inline int64_t y_chunk_cols(int64_t pairs, int64_t Hp) {
  if (pairs <= 0 || y_plane_bytes(pairs, Hp) <= kYChunkBytes) return Hp;
  // 2 bytes per value + 1 per 64 values, 512 bytes of alignment slack
  int64_t w = (kYChunkBytes - 512) * 64 / (pairs * 129) / 256 * 256;
  return w < 256 ? 256 : (w > Hp ? Hp : w);
}
// Bytes reserved for y: at least one plane of pairs x y_chunk_cols, and
// non-decreasing in `pairs`, so a workspace sized for T_max tokens fits every
// T <= T_max.
inline int64_t y_reserve_bytes(int64_t pairs, int64_t Hp) {
  const int64_t full = y_plane_bytes(pairs, Hp);
  const int64_t capped = full < kYChunkBytes ? full : kYChunkBytes;
  const int64_t used = y_plane_bytes(pairs, y_chunk_cols(pairs, Hp));
  return used > capped ? used : capped;
}

hipError_t launch_gemm1(int mode, int block_m, int nb, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm2(int mode, int block_m, int nb, const GemmArgs& a, hipStream_t s);

// out[t, c0 + h] for h < cols from the block-floating-point y rows (pair
// t*k + j; values and exponents as above, exponents `yexp` bytes after the
// values), summed over nplanes planes `plane` bytes apart.
hipError_t launch_combine(const uint8_t* y, int64_t yexp, int T, int k, int c0, int cols, int64_t ldy, int nplanes,
                          int64_t plane, uint16_t* out, int64_t ld_out, hipStream_t s);

// Decode micro-batches (T <= kDecodeMaxT tokens, block FP8 with fp32 or
// UE8M0 scales): M-tiled GEMV kernels, see decode.hip.
//   decode_gemm1: GEMM1 and the clamped SwiGLU from the routing and the
//     quantised x, a fp32 [T*k][Ip] in pair order f = t*k + j.
//   decode_gemm2: re-quantisation of a (1x128), GEMM2 and the weighted
//     combine into out; the intermediate codes and scales in pair order go
//     to aq [T*k][Ip], as [T*k][Ip/128] fp32 or [T*k][e8_scale_ld(Ip)]
//     UE8M0 bytes.  Up to kDecodeSmallT tokens every GEMM2 workgroup
//     re-quantises a itself (and workgroup 0 stores aq / as); above, one
//     launch re-quantises it once, into aq / as, before GEMM2.
constexpr int kDecodeMaxT = 16;
constexpr int kDecodeMaxPairs = 128;
constexpr int kDecodeWaves = 8;
constexpr int kDecodeSmallT = 4;
struct DecodeArgs {
  int32_t T, E, k, H, Hp, Ip;
  float limit;
  int32_t* ids;           // routing [T][k]
  float* topk_w;          // routing weights [T][k]
  const uint8_t* xq;      // quantised x [T][Hp] and its scales
  const void* xs;
  const uint8_t* w13;     // TILED_V2
  const float* s13;
  float* a;               // clamped SwiGLU output, fp32 [T*k][Ip]
  const uint8_t* w2;      // TILED_V2
  const float* s2;
  uint16_t* out;          // bf16 [T][ld_out]
  int64_t ld_out;
  uint8_t* aq;            // the intermediate in pair order (see above)
  void* as;
};
// Shapes the decode kernels take: quant mode block FP8, 1 <= T <= 16,
// T*k <= 128, E <= 1024, Hp in {1024, 2048, 4096}, Ip in {128, 256, 512,
// 1024}.
bool decode_ok(int mode, int T, int E, int k, int Hp, int Ip);
hipError_t launch_decode_gemm1(int mode, const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_gemm2(int mode, const DecodeArgs& a, hipStream_t s);

}  // namespace moe
