/*
 * moe.h -- C ABI of libmoe.so, a routed-expert MoE layer for AMD MI355X (gfx950).
 *
 * The layer (one call of moe_forward) computes, for T tokens x[T, H]:
 *   1. top-k routing over E experts with renormalised softmax weights;
 *   2. a stable expert permutation of the T*k (token, slot) pairs, each
 *      expert's segment padded to a multiple of block_m rows;
 *   3. dynamic activation quantisation (block FP8 1x128 or OCP MXFP4 1x32);
 *   4. a grouped gate/up GEMM over separate gate and up halves of w13, fused
 *      with the clamped SwiGLU silu(min(gate, L)) * clamp(up, -L, L) and the
 *      re-quantisation of the intermediate;
 *   5. a grouped down GEMM and the routing-weighted combine into bf16 out[T, H].
 *
 * Sources (page title and section):
 *   - sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark MXFP4
 *     MoE on gfx950": Summary (block FP8 [128,128] weights with dynamic FP8
 *     activations; OCP MXFP4 1x32 weights and activations; gate and up loaded
 *     as separate contiguous halves; clamped SwiGLU with swiglu_limit=10.0) and
 *     the contract table (explicit gate mode, limit always forwarded,
 *     preshuffle owned by the runner that consumes it, unsupported
 *     configurations rejected at construction, hidden/intermediate padding
 *     recorded and forwarded).
 *   - FreeToken PR #270 "glm5_next: support GLM-5.3-Flash (hybrid KDA + DSA,
 *     mHC, NVFP4 expert offload)": Summary (288-expert top-8 routing; the
 *     clamped SwiGLU formula, an infinite limit giving plain SwiGLU; backends
 *     that cannot apply the limit are rejected).
 *   - "[AMD] [GLM5] Opt-in prefill-only FP8 dense projection GEMM for MLA
 *     q_b/o_proj (gfx950)": Modifications (e4m3 weights with a 128x128 UE8M0,
 *     i.e. power-of-two, block scale).
 *
 * Conventions for every entry point:
 *   - Every pointer argument is DEVICE memory owned by the caller, except the
 *     moe_cfg_t pointer, which is host memory read during the call only.
 *     Device buffers must be 16-byte aligned (any hipMalloc / torch
 *     allocation is); row strides are in elements.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it; no call synchronises, allocates device memory or reads
 *     device memory back to the host, so moe_forward can be captured in a
 *     HIP graph.  Scratch memory is caller-provided (moe_workspace_bytes).
 *   - Every argument is validated before anything is enqueued: a call that
 *     returns an error has launched nothing.  MOE_ERR_HIP reports a failed
 *     launch; faults inside kernels surface at the caller's next sync.
 *   - The library keeps no state; calls on different streams are independent
 *     as long as their buffers do not overlap.
 *   - T = 0 (no tokens) is valid and launches nothing.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  MOE_ERR_ALIGN = 3,       /* a padded size is not a multiple of 128 */
  MOE_ERR_UNSUPPORTED = 4, /* quant mode, gate mode, block_m, limit or dtype not supported */
  MOE_ERR_LAYOUT = 5,      /* weight layout tag is not the one this call consumes */
  MOE_ERR_WORKSPACE = 6,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 7          /* a kernel launch failed */
} moe_status_t;

/* Weight/activation contracts (sglang PR #38546, Summary; UE8M0: "[AMD]
 * [GLM5] Opt-in prefill-only FP8 dense projection GEMM for MLA q_b/o_proj
 * (gfx950)", Modifications). */
enum {
  MOE_QUANT_FP8_BLOCK = 1, /* w: e4m3 + fp32 scale per [128,128] block; act: e4m3 + fp32 per 1x128 */
  MOE_QUANT_MXFP4 = 2,     /* w and act: E2M1 two per byte (low nibble = even index) + E8M0 per 1x32 */
  MOE_QUANT_FP8_UE8M0 = 3  /* w: e4m3 + UE8M0 byte per [128,128] block; act: e4m3 + UE8M0 byte per 1x128.
                              UE8M0 scale = 2^e, e the smallest integer with 448 * 2^e >= amax of the
                              group, stored as the byte clamp(e + 127, 0, 254) (0 when amax = 0) */
};

/* Physical order of the gate and up projections inside w13.  Only separate
 * contiguous halves (gate rows [0, Ip), up rows [Ip, 2Ip)) are accepted;
 * interleaved is rejected with MOE_ERR_UNSUPPORTED (sglang PR #38546, contract
 * table: gate mode is explicit, never inferred). */
enum { MOE_GATE_SEPARATED = 0, MOE_GATE_INTERLEAVED = 1 };

/* Weight layout tags.  CANONICAL is row-major [E, N, K] (what
 * moe_quant_weights writes).  TILED_V2 is the GEMM kernels' layout, written
 * only by moe_preshuffle_weights (the runner owns its preshuffle): 16-row x
 * 128-column MFMA tiles ordered [E][N tile][16/R][K block][R], an N tile
 * being the 256 weight rows one GEMM work item multiplies (w13: 128 gate
 * rows and the matching 128 up rows; w2: 256 rows, a half last N tile
 * zero-padded), so the tiles of one K block come in contiguous runs of R
 * (R fixed per matrix and mode: block FP8 w13 16, w2 4; MXFP4 w13 1). */
enum { MOE_LAYOUT_CANONICAL = 0, MOE_LAYOUT_TILED_V2 = 0x4D310002 };

/* Element types accepted by moe_quant_act / moe_quant_weights. */
enum { MOE_DTYPE_BF16 = 1, MOE_DTYPE_F32 = 2 };

/* Hidden/intermediate padding metadata (sglang PR #38546, contract table:
 * padding is recorded and forwarded).  `*_padded` must be multiples of 128 and
 * not below the real size.  x and out have `hidden` columns; weights are
 * stored padded with zeros: w13 [E, 2*inter_padded, hidden_padded] (each half
 * padded separately) and w2 [E, hidden_padded, inter_padded]. */
typedef struct {
  int32_t hidden, hidden_padded, inter, inter_padded;
} moe_pad_t;

typedef struct {
  int32_t num_experts;   /* E, 1..1024 */
  int32_t top_k;         /* k, 1..min(16, E) */
  int32_t quant_mode;    /* MOE_QUANT_* */
  int32_t gate_mode;     /* must be MOE_GATE_SEPARATED */
  int32_t weight_layout; /* must be MOE_LAYOUT_TILED_V2 for the GEMM entry points */
  int32_t block_m;       /* rows per expert block: 16, 32, 64 or 128 */
  float swiglu_limit;    /* L > 0; +inf gives plain SwiGLU; NaN rejected */
  moe_pad_t pad;
} moe_cfg_t;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status_t s);

/* Validates a configuration without touching the GPU ("fails at
 * construction, not later"). */
moe_status_t moe_validate_cfg(const moe_cfg_t* cfg);

/* Number of block_m-row blocks the padded permutation can need for
 * num_pairs = T*k pairs: min(P, (P + E*(block_m-1)) / block_m).  Returns -1
 * for invalid arguments. */
int32_t moe_max_blocks(int32_t num_pairs, int32_t num_experts, int32_t block_m);

/* Bytes of scratch that moe_forward needs for up to T_max tokens (0 if the
 * configuration is invalid; non-decreasing in T_max).  Also enough for
 * moe_grouped_gemm2_combine.  The per-pair GEMM2 rows it holds (2 bytes per
 * value plus one byte per 64) are capped near 1 GiB: larger batches run GEMM2
 * and the combine in column chunks over one reused buffer.  It also covers
 * the K-split scratch (see moe_plan_ksplit): at most 8 * min(T*k, 1024) fp32
 * rows of 2*Ip partial sums and y planes of Hp columns, or for a tail split
 * 8 * W * block_m rows of 256 fp32 partial sums (W: moe_plan_ksplit's grid,
 * one workgroup per compute unit rounded up to a multiple of 8). */
size_t moe_workspace_bytes(const moe_cfg_t* cfg, int32_t T_max);

/* Sizes in bytes of the intermediate aq / as buffers (rows = max_blocks *
 * block_m; FP8: aq u8 [rows, Ip], as f32 [rows, Ip/128]; MXFP4: aq u8
 * [rows, Ip/2], as u8 [rows, Ip/32]; FP8_UE8M0: aq u8 [rows, Ip], as u8
 * [rows, round_up(Ip/128, 4)]).  Returns MOE_ERR_* on a bad cfg. */
moe_status_t moe_intermediate_bytes(const moe_cfg_t* cfg, int32_t T, size_t* aq_bytes,
                                    size_t* as_bytes);

/* Top-k routing (FreeToken PR #270, Summary: 288-expert top-8 routing).
 * logits: f32 [T, E] row-major.  Selection is on the raw logits: descending
 * value, ties to the lower expert id (-0.0 equals +0.0); slot j holds the j-th
 * best.  weights[t, j] = exp(l_j - l_max) / sum over the k selected.
 * Outputs: ids int32 [T, top_k], weights f32 [T, top_k].  NaN logits are not
 * supported (the result is unspecified but in range). */
moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t top_k,
                            int32_t* ids, float* weights, void* stream);

/* Stable counting sort of the P = T*top_k pairs (pair f = t*top_k + j) by
 * expert ids[f].  With nb = moe_max_blocks(P, E, block_m):
 *   sorted_ids   int32 [nb*block_m]: expert e's segment starts at
 *                expert_offsets[e] and holds its pairs in increasing f, padded
 *                with the sentinel P to a multiple of block_m; every entry past
 *                the last segment is also P;
 *   block_expert int32 [nb]: expert of each block, -1 past the last segment;
 *   expert_offsets int32 [E+1]: exclusive scan of the padded segment sizes;
 *   num_post_padded int32 [1]: expert_offsets[E], left on the device.
 * Experts with no pairs get no block.  ids outside [0, E) are skipped (the
 * pair appears nowhere); a token that lists an expert twice is allowed and
 * its pairs keep f order (slower path).  E <= 1024. */
moe_status_t moe_permute_align(const int32_t* ids, int32_t T, int32_t top_k, int32_t E,
                               int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                               int32_t* expert_offsets, int32_t* num_post_padded,
                               void* stream);

/* Dynamic row quantisation (sglang PR #38546, Summary: dynamic FP8
 * activations; OCP MXFP4 1x32).  in: `rows` rows of `cols` valid elements
 * (bf16 or f32) with row stride ld_in elements; columns cols..cols_padded-1
 * are taken as zero.  cols_padded % 128 == 0.
 *   FP8:   q u8 [rows, cols_padded] e4m3; scales f32 [rows, cols_padded/128]:
 *          s = amax/448 (fp32 division), q = RNE(clamp(v/s, +-448)); amax = 0
 *          gives s = 0 and all-zero codes.
 *   MXFP4: q u8 [rows, cols_padded/2]; scales u8 [rows, cols_padded/32]:
 *          b = clamp(floor(log2 amax) - 2 + 127, 0, 254) (0 when amax = 0),
 *          codes = RNE_E2M1(clamp(v / 2^(b-127), +-6)).
 *   FP8_UE8M0: q u8 [rows, cols_padded] e4m3; scales u8 [rows, lds] with
 *          lds = round_up(cols_padded/128, 4) (rows of whole dwords; the
 *          bytes past cols_padded/128 are written 0): b as in MOE_QUANT_*,
 *          codes = RNE(v / 2^(b-127)) (exact scaling, no saturation needed).
 * Signs of zero are kept.  Results are bit-exact by definition. */
moe_status_t moe_quant_act(const void* in, int32_t in_dtype, int32_t rows, int32_t cols,
                           int64_t ld_in, int32_t cols_padded, int32_t quant_mode, void* q,
                           void* scales, void* stream);

/* Steps 1-3 of the layer in as few launches as the batch allows: top-k
 * routing, the padded permutation and the quantisation of x, with exactly
 * the results of moe_route_topk + moe_permute_align + moe_quant_act (x bf16,
 * hidden = cfg->pad.hidden valid columns, row stride ld_x, quantised to
 * cfg->pad.hidden_padded columns in cfg->quant_mode).  Up to 16 tokens it
 * is one launch (one workgroup routes and permutes while the others
 * quantise); larger batches take two (routing and quantisation side by side,
 * then the permutation).  Outputs as the three entry points (sizes from
 * moe_max_blocks, moe_quant_act); all are device buffers of the caller. */
moe_status_t moe_route_permute_quant(const moe_cfg_t* cfg, int32_t T, const float* router_logits,
                                     const void* x_bf16, int64_t ld_x, int32_t* ids, float* weights,
                                     int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                                     int32_t* num_post_padded, void* xq, void* xs, void* stream);

/* Offline weight quantisation into the CANONICAL layout.  w: f32 [E, N, K]
 * row-major (already zero-padded).
 *   FP8:   N % 128 == 0, K % 128 == 0; q u8 [E, N, K]; scales f32
 *          [E, N/128, K/128] (dequant multipliers), one per [128,128] block,
 *          same arithmetic as moe_quant_act with the block as the group.
 *   MXFP4: K % 128 == 0; q u8 [E, N, K/2]; scales u8 [E, N, K/32].
 *   FP8_UE8M0: as FP8 with scales u8 [E, N/128, K/128] (UE8M0 bytes). */
moe_status_t moe_quant_weights(int32_t quant_mode, const float* w, int32_t E, int32_t N,
                               int32_t K, void* q, void* scales, void* stream);

/* Sizes of the TILED_V2 buffers for w13 (which = 13: N = 2*Ip, K = Hp) or
 * w2 (which = 2: N = Hp, K = Ip): whole N tiles, E * ceil(N/256) * (K/128)
 * tiles of 16 (2 KB FP8 / 1 KB MXFP4 each).  Block scales of FP8 stay
 * [E, N/128, K/128] f32 (FP8_UE8M0: the bytes' exact fp32 values
 * 2^(b-127)); MXFP4 scales are E8M0 words [E][N tile][ceil(K/512)][16][64]. */
moe_status_t moe_preshuffled_bytes(const moe_cfg_t* cfg, int32_t which, size_t* w_bytes,
                                   size_t* s_bytes);

/* Rewrites CANONICAL quantised weights (moe_quant_weights' output for the
 * padded matrix of `which`) into TILED_V2, the only layout the GEMM entry
 * points read (sglang PR #38546, contract table: the runner owns its
 * preshuffle).  Ignores cfg->weight_layout.  Output sizes from
 * moe_preshuffled_bytes.  In and out must not overlap. */
moe_status_t moe_preshuffle_weights(const moe_cfg_t* cfg, int32_t which, const void* w,
                                    const void* s, void* w_out, void* s_out, void* stream);

/* Grouped gate/up GEMM + clamped SwiGLU + re-quantisation (sglang PR #38546,
 * Summary; FreeToken PR #270, Summary).  For every row r of every block b <
 * num_post_padded/block_m with pair f = sorted_ids[b*block_m + r] < T*k:
 *   h = deq(xq[f / k]) . deq(w13[block_expert[b]])^T   (fp32, N = 2Ip, K = Hp)
 *   a = silu(min(h[:Ip], L)) * clamp(h[Ip:], -L, L)
 *   aq/as row (b*block_m + r) = quantise(a) per 1x128 (FP8) or 1x32 (MXFP4)
 * Pad rows (f = T*k) get all-zero codes and zero scales.
 * xq/xs: moe_quant_act output for x (FP8: u8 [T, Hp] + f32 [T, Hp/128];
 * MXFP4: u8 [T, Hp/2] + u8 [T, Hp/32]; FP8_UE8M0: u8 [T, Hp] + u8
 * [T, round_up(Hp/128, 4)]).  w13/w13_scale: TILED_V2.
 * aq/as: sizes from moe_intermediate_bytes, indexed by sorted position, in
 * the activation format of the mode over Ip columns (FP8_UE8M0: the scale
 * bytes past Ip/128 in each row are unspecified). */
moe_status_t moe_grouped_gemm1_swiglu(const moe_cfg_t* cfg, int32_t T, const void* xq,
                                      const void* xs, const int32_t* sorted_ids,
                                      const int32_t* block_expert,
                                      const int32_t* num_post_padded, const void* w13,
                                      const void* w13_scale, void* aq, void* as, void* stream);

/* Grouped down GEMM + routing-weighted combine.  For each pair f:
 *   y_f = deq(aq row of f) . deq(w2[e])^T   (fp32, N = Hp, K = Ip)
 *   out[t, :H] = bf16_rne( sum over j = 0..k-1 in slot order of
 *                          fl32(topk_w[t, j] * y_{t*k+j}) ), fp32 accumulation.
 * out: bf16 [T, ld_out]; columns >= H are not written.  ws: at least
 * moe_workspace_bytes(cfg, T) bytes. */
moe_status_t moe_grouped_gemm2_combine(const moe_cfg_t* cfg, int32_t T, const void* aq,
                                       const void* as, const int32_t* sorted_ids,
                                       const int32_t* block_expert,
                                       const int32_t* num_post_padded, const void* w2,
                                       const void* w2_scale, const float* topk_w,
                                       void* out_bf16, int64_t ld_out, void* ws,
                                       size_t ws_bytes, void* stream);

/* K split of the grouped GEMMs (a launch choice; the pages fix none).
 * ksplit = 2, 4 or 8: with few (block, N tile) work items, each is cut into
 * ksplit pieces along K so that every compute unit streams weights:
 *   GEMM1: piece i stores fp32 partial sums h_i of its K range; a second
 *          kernel forms h = h_0 + h_1 + ... (in piece order), then the clamped
 *          SwiGLU and the re-quantisation as above;
 *   GEMM2: piece i stores its weighted rows for its K range in a plane of
 *          its own; the combine adds, plane by plane, the slots in order.
 * ksplit = -2, -4 or -8 (GEMM1 only, -8 at block_m 16 or 32 only; a "tail split"): the
 *   items that fill whole rounds of one workgroup per compute unit run
 *   unsplit with the fused epilogue, and only the remaining items are cut
 *   into -ksplit pieces and finished by the second kernel, so the last
 *   round is spread over every workgroup.
 * Results equal the unsplit ones up to fp32 summation order (and, for a
 * GEMM2 split, each plane's own storage of the weighted rows).
 * moe_plan_ksplit: the split moe_forward and moe_grouped_gemm2_combine use for
 * GEMM `which` (13: gate/up, 2: down) at T tokens on the current device
 * (1, 2, 4 or 8 when items would leave compute units idle, at most 1024
 * pairs; else for GEMM1, when the last round of items is expected to be
 * mostly idle, the tail split with the most pieces the scale layout allows,
 * at most 4 at block_m 64 and 128, where MXFP4 plans none; else 1); -1 for
 * invalid arguments.
 * moe_splitk_bytes: scratch in bytes that the explicit-split entry points need
 * for that ksplit (0 for GEMM1 without a split; 0 also if the split is not
 * usable: |ksplit| must be 1, 2, 4 or 8 and divide K/128 into pieces of at
 * least 4 K blocks, multiples of 4 for MXFP4 and FP8_UE8M0; a positive split
 * at most 1024 pairs, and for GEMM2 the y rows must fit one chunk; a tail
 * split GEMM1 only, -8 at block_m 16 or 32 only). */
int32_t moe_plan_ksplit(const moe_cfg_t* cfg, int32_t T, int32_t which);
size_t moe_splitk_bytes(const moe_cfg_t* cfg, int32_t T, int32_t which, int32_t ksplit);

/* moe_grouped_gemm1_swiglu with an explicit K split (ksplit = 1: the same
 * launch as moe_grouped_gemm1_swiglu; negative: a tail split).  ws: at least moe_splitk_bytes(cfg,
 * T, 13, ksplit) bytes of scratch (may be NULL when that is 0).  An unusable
 * ksplit returns MOE_ERR_UNSUPPORTED before anything is enqueued. */
moe_status_t moe_grouped_gemm1_swiglu_splitk(const moe_cfg_t* cfg, int32_t T, const void* xq,
                                             const void* xs, const int32_t* sorted_ids,
                                             const int32_t* block_expert,
                                             const int32_t* num_post_padded, const void* w13,
                                             const void* w13_scale, void* aq, void* as,
                                             int32_t ksplit, void* ws, size_t ws_bytes,
                                             void* stream);

/* moe_grouped_gemm2_combine with an explicit K split.  ws: at least
 * moe_splitk_bytes(cfg, T, 2, ksplit) bytes (moe_grouped_gemm2_combine uses
 * ksplit = moe_plan_ksplit(cfg, T, 2), within moe_workspace_bytes(cfg, T)). */
moe_status_t moe_grouped_gemm2_combine_splitk(const moe_cfg_t* cfg, int32_t T, const void* aq,
                                              const void* as, const int32_t* sorted_ids,
                                              const int32_t* block_expert,
                                              const int32_t* num_post_padded, const void* w2,
                                              const void* w2_scale, const float* topk_w,
                                              void* out_bf16, int64_t ld_out, int32_t ksplit,
                                              void* ws, size_t ws_bytes, void* stream);

/* Decode micro-batches (FreeToken PR #270 "glm5_next: support GLM-5.3-Flash
 * (hybrid KDA + DSA, mHC, NVFP4 expert offload)", Tuned companion: an
 * M-tiled FP8 GEMV for decode micro-batches).  For at most 16 tokens of a
 * block-FP8 layer (fp32 or UE8M0 scales) every active expert multiplies at
 * most 16 rows, so two GEMV-shaped kernels can replace the grouped GEMMs:
 * GEMM1 + clamped SwiGLU over (expert, 32 intermediate columns) items with K
 * split across the waves of a workgroup, then the re-quantisation of the
 * intermediate, GEMM2 over 16 output columns of every expert and the
 * slot-ordered combine in one kernel (no permutation, no per-pair GEMM2 rows
 * in HBM; above 4 tokens one small launch re-quantises the intermediate
 * once, first).  moe_forward does not use them: on the MI355X the K-split
 * grouped GEMMs, whose load ring runs through LDS, stream these layers'
 * weights faster at every T <= 16.
 *
 * moe_decode_supported: 1 if the decode entry points take T tokens of this
 * layer (quant mode FP8_BLOCK or FP8_UE8M0, TILED_V2, 1 <= T <= 16,
 * T*k <= 128, hidden_padded 1024, 2048 or 4096, inter_padded 128, 256, 512
 * or 1024), else 0 (also for an invalid configuration).
 *
 * moe_decode_gemm1_swiglu: for every pair f = t*k + j with topk_ids[f] in
 * [0, E): a[f, c] = silu(min(g, L)) * clamp(u, -L, L) for c < Ip, with g
 * and u the gate and up rows c and Ip + c of expert topk_ids[f] times
 * dequantised x row t (fp32 promotion per 128-wide K block; the steps of
 * moe_grouped_gemm1_swiglu before its re-quantisation).  xq, xs: quantised x
 * as moe_quant_act writes it ([T, Hp] codes; fp32 [T, Hp/128] or UE8M0
 * [T, row of whole dwords] scales); topk_ids: int32 [T, k], each token's ids
 * distinct (as routing gives them; a repeated id counts once); a: f32
 * [T*k, Ip] (rows of other pairs are not written).  xq and a 16-byte
 * aligned, xs and topk_ids 4-byte aligned, else MOE_ERR_ALIGN; a shape
 * outside moe_decode_supported: MOE_ERR_UNSUPPORTED.
 *
 * moe_decode_gemm2_combine: re-quantises each pair's row of a in 1x128 groups
 * (e4m3 codes with an fp32 scale amax/448, or a UE8M0 scale: the arithmetic
 * of moe_grouped_gemm1_swiglu's epilogue), multiplies it with w2 of the
 * pair's expert and writes out[t, :H] = sum over slots j in order of
 * topk_weights[t*k + j] * y[t*k + j] in bf16 (pairs with an id outside
 * [0, E) add nothing).  The intermediate is stored in pair order: aq u8
 * [T*k, Ip], as f32 [T*k, Ip/128] or UE8M0 bytes [T*k, row of whole dwords]
 * (aq 8-byte and as 4-byte aligned; for more than 4 tokens it is written by
 * a re-quantisation launch first and read back by GEMM2).  a 16-byte
 * aligned.  Same errors as above; ld_out < hidden: MOE_ERR_SHAPE. */
int32_t moe_decode_supported(const moe_cfg_t* cfg, int32_t T);
moe_status_t moe_decode_gemm1_swiglu(const moe_cfg_t* cfg, int32_t T, const void* xq, const void* xs,
                                     const int32_t* topk_ids, const void* w13, const void* w13_scale, float* a,
                                     void* stream);
moe_status_t moe_decode_gemm2_combine(const moe_cfg_t* cfg, int32_t T, const float* a, const int32_t* topk_ids,
                                      const float* topk_weights, const void* w2, const void* w2_scale,
                                      void* out_bf16, int64_t ld_out, void* aq, void* as, void* stream);

/* The whole layer: route, permute, quantise x, GEMM1+SwiGLU, GEMM2+combine,
 * all on `stream` with no host synchronisation.  x: bf16 [T, ld_x] (H valid
 * columns); router_logits f32 [T, E]; weights TILED_V2; out bf16 [T, ld_out].
 * ws: at least moe_workspace_bytes(cfg, T) bytes. */
moe_status_t moe_forward(const moe_cfg_t* cfg, int32_t T, const void* x_bf16, int64_t ld_x,
                         const float* router_logits, const void* w13, const void* w13_scale,
                         const void* w2, const void* w2_scale, void* out_bf16, int64_t ld_out,
                         void* ws, size_t ws_bytes, void* stream);

/* Diagnostic (not part of the layer): one 16x16 output tile C = A . B^T over
 * K = 128 from e4m3 codes, computed as one K block of the grouped GEMMs:
 * kind 0 with one FP8 MFMA (16x16x128, unit scales; GEMM2's instruction),
 * kind 1 with the operands widened exactly to f16 and four 16x16x32 f16 MFMAs
 * (GEMM1's instructions).  a, b: device u8 [16, 128] row-major e4m3 codes
 * (16-byte aligned); out: device f32 [16, 16] row-major.  Lets tests compare
 * the two matrix-core sums with an exact one. */
moe_status_t moe_diag_mfma_tile(int32_t kind, const void* a, const void* b, float* out, void* stream);

/* Diagnostic (not part of the layer): the matrix-core throughput of one
 * instruction, for pricing the GEMMs against what the part delivers beside
 * its published peak.  One launch of MOE_DIAG_MFMA_RATE_WORKGROUPS workgroups
 * of 4 waves (4 per CU on a 256-CU MI355X), each wave running `iters` rounds
 * of 8 independent accumulator chains with no memory traffic:
 *   kind 0: 16x16x32 f16 MFMA (16384 FLOP each; GEMM1's block-FP8 path),
 *   kind 1: 16x16x128 FP8 MFMA (65536 FLOP; GEMM2),
 *   kind 2: 16x16x128 FP4 MFMA (65536 FLOP; the MXFP4 GEMMs).
 * FLOPs per launch = WORKGROUPS * 4 * iters * 8 * (FLOP each); the caller
 * times the launch on `stream`.  out: device f32 [WORKGROUPS * 256], written
 * (a sink for the accumulators).  MOE_ERR_UNSUPPORTED for another kind or
 * iters < 1, MOE_ERR_NULL for out == NULL. */
#define MOE_DIAG_MFMA_RATE_WORKGROUPS 1024
moe_status_t moe_diag_mfma_rate(int32_t kind, int32_t iters, float* out, void* stream);

/* Diagnostic (not part of the layer): the HBM read rate this part reaches
 * with the GEMMs' kind of load (16-byte non-temporal loads, coalesced, four in
 * flight per lane, a contiguous share per workgroup), for pricing their weight
 * streams beside the published peak.  One launch of MOE_DIAG_STREAM_WORKGROUPS
 * workgroups of 512 threads reads `bytes` bytes of device memory at src
 * (16-byte aligned, a multiple of 16) once; the caller times it on `stream`.
 * sink: device u32 [WORKGROUPS * 512], written with a checksum of the data.
 * MOE_ERR_NULL, MOE_ERR_SHAPE (bytes < 0) and MOE_ERR_ALIGN before any
 * launch. */
#define MOE_DIAG_STREAM_WORKGROUPS 256
moe_status_t moe_diag_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Size of the scratch that moe_forward_noalloc keeps in a static device
 * array: 128 MiB, held on every GPU the library runs on until the process
 * ends.  It covers moe_workspace_bytes(cfg, T) for decode batches, e.g. up to
 * 793 tokens (block_m 16) or 731 (block_m 32) of the 288-expert top-8
 * block-FP8 layer with H = 4096, I = 1024. */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as moe_forward (the same kernels) without ws /
 * ws_bytes: the scratch is the library's static device array of
 * MOE_NOALLOC_SCRATCH_BYTES on the current device.  Returns
 * MOE_ERR_WORKSPACE (launching nothing) when moe_workspace_bytes(cfg, T)
 * exceeds it.  Allocates nothing (no hipMalloc, no allocating library
 * call); the array's device address is looked up once per device, on the
 * first call made with that device current.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (e.g. on two
 * streams) race, so serialise them.  Nothing in the array needs to start at
 * zero; it keeps the last call's contents. */
moe_status_t moe_forward_noalloc(const moe_cfg_t* cfg, int32_t T, const void* x_bf16, int64_t ld_x,
                                 const float* router_logits, const void* w13, const void* w13_scale,
                                 const void* w2, const void* w2_scale, void* out_bf16, int64_t ld_out,
                                 void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
