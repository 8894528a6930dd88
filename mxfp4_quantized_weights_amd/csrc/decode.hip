// Decode micro-batches: M-tiled GEMV kernels for T <= 16 tokens (block FP8,
// fp32 or UE8M0 scales).
//
// FreeToken PR #270 "glm5_next: support GLM-5.3-Flash (hybrid KDA + DSA,
// mHC, NVFP4 expert offload)", Tuned companion: an M-tiled FP8 GEMV for
// decode micro-batches.  sglang PR #31955 "[AMD] [GLM5] Opt-in prefill-only
// FP8 dense projection GEMM for MLA q_b/o_proj (gfx950)", Motivation: the
// small-M FP8 GEMM needs its own tuning.
//
// With at most 16 tokens, every active expert multiplies at most 16 rows
// (routing never gives a token the same expert twice), so one 16-row MFMA
// tile covers an expert's whole M: these are GEMVs over the experts' weights,
// and the layer is bound by streaming those weights once.  Two kernels:
//
//   decode_gemm1: item = (active expert, 32 intermediate columns), i.e. the
//     expert's 32 gate and 32 up rows of w13 over all of K.  The 8 waves of
//     a workgroup split K (wave w takes K blocks w, w+8, ...), load their
//     weight tiles straight from HBM into registers (the TILED_V2 tile is
//     already MFMA fragment order: each 16-byte wave load is 1 KB
//     contiguous), the next item's as each step's registers free up, and
//     multiply them with the tokens' x codes held in LDS.  The 8 partial
//     sums meet in LDS, in wave order, and the workgroup writes the clamped
//     SwiGLU output a of its 32 columns for each real pair, fp32, in pair
//     order [T*k][Ip].  No item needs another workgroup's results, so there
//     is no second pass: the 1x128 re-quantisation happens where a is read.
//   decode_gemm2: item = 16 output columns of every active expert.  Up to 4
//     tokens the workgroup re-quantises a itself (1x128 FP8 codes and
//     scales, the arithmetic of the prefill GEMM1 epilogue) into LDS; above,
//     decode_requant_kernel does it once, into aq / as, and the workgroup
//     copies those.  Its 8 waves take the active experts in turn (tiles
//     streamed into registers, one expert ahead), keep each pair's 16 output
//     values in LDS, and then add every token's k pairs in slot order,
//     weighted, into the bf16 output.  No per-pair rows go through HBM.
//
// GEMM1 widens FP8 to f16 and uses the f16 MFMA with fp32 promotion per
// 128-wide K block (exact products and fp32 sums, as the prefill GEMM1);
// GEMM2 uses the FP8 MFMA with fp32 promotion per K block (for UE8M0 the
// promotion multiplies by exact powers of two).
//
// Measured on the MI355X against the K-split grouped GEMMs of the same
// layer (288 experts, H = 4096, I = 1024), these kernels stream the weights
// more slowly at every T <= 16 (e.g. GEMM1 at T = 16: 171 against 148 us;
// the register prefetch drains at every item boundary, where the grouped
// GEMMs' LDS load ring does not), so moe_forward keeps the grouped GEMMs.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlice = 32;  // intermediate columns per decode_gemm1 item

// Active experts of the batch in increasing id (act[r] for rank r < n_act),
// per expert id the tokens that chose it (bit t of etk[e]) and per rank the
// pair of each MFMA row (rpair[16r + m]: the pair of the expert's m-th token,
// -1 past its last).  Ids outside [0, E) are ignored; a token that lists an
// expert twice counts once (its first slot).  All threads of the workgroup
// call this; ids are in LDS.
__device__ __forceinline__ int build_expert_list(const int32_t* ids, int P, int k, int E, uint32_t* emask,
                                                 int32_t* ebase, int32_t* act, uint32_t* etk, int16_t* rpair) {
  const int tid = threadIdx.x;
  if (tid < 32) emask[tid] = 0;
  for (int e = tid; e < E; e += kThreads) etk[e] = 0;
  for (int i = tid; i < kDecodeMaxPairs * 16; i += kThreads) rpair[i] = -1;
  __syncthreads();
  for (int f = tid; f < P; f += kThreads) {
    const int e = ids[f];
    if (e >= 0 && e < E) {
      atomicOr(&emask[e >> 5], 1u << (e & 31));
      atomicOr(&etk[e], 1u << (f / k));
    }
  }
  __syncthreads();
  if (tid < 64) {
    const uint32_t m = tid < 32 ? emask[tid] : 0u;
    const int c = __popc(m);
    int incl = c;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (tid >= off) incl += o;
    }
    if (tid < 32) {
      ebase[tid] = incl - c;
      int r = incl - c;
      for (uint32_t b = m; b; b &= b - 1) act[r++] = 32 * tid + __builtin_ctz(b);
    }
    if (tid == 31) ebase[32] = incl;
  }
  __syncthreads();
  for (int f = tid; f < P; f += kThreads) {
    const int e = ids[f];
    const int t = f / k, j = f - t * k;
    bool first = e >= 0 && e < E;
    for (int j2 = 0; j2 < j && first; ++j2) first = ids[t * k + j2] != e;
    if (first) {
      const int r = ebase[e >> 5] + __popc(emask[e >> 5] & ((1u << (e & 31)) - 1u));
      rpair[16 * r + __popc(etk[e] & ((1u << t) - 1u))] = (int16_t)f;
    }
  }
  __syncthreads();
  return ebase[32];
}

__device__ __forceinline__ v8i frag_from(uint4 lo, uint4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// ---------------------------------------------------------------------------
// GEMM1 + clamped SwiGLU.  KBW = K blocks per wave per item (Hp = 1024*KBW).
// ---------------------------------------------------------------------------
template <int QM, int KBW>
__global__ __launch_bounds__(kThreads) void decode_gemm1_kernel(DecodeArgs p) {
  static_assert(KBW == 1 || KBW == 2 || KBW == 4, "K blocks per wave");
  constexpr bool E8 = QM == kQuantFp8E8;
  constexpr int KB = KBW * kWaves;
  constexpr int HP = KB * 128;
  constexpr int XS_LD = E8 ? (KB + 3) / 4 * 4 : KB * 4;  // bytes per token-scale row
  __shared__ __attribute__((aligned(16))) uint8_t xq_l[kDecodeMaxT * HP];
  __shared__ __attribute__((aligned(16))) uint8_t xs_l[kDecodeMaxT * XS_LD];
  __shared__ __attribute__((aligned(16))) float red[kWaves * 16 * 64];
  __shared__ int32_t ids_l[kDecodeMaxPairs];
  __shared__ uint32_t emask[32];
  __shared__ int32_t ebase[33];
  __shared__ int32_t act[kDecodeMaxPairs];
  __shared__ uint32_t etk[1024];
  __shared__ int16_t rpair[kDecodeMaxPairs * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, k = p.k, P = T * k, Ip = p.Ip;
  const int S = Ip / kSlice;          // items per expert
  const int NG = Ip / 128;            // N tiles of w13 (128 gate + 128 up rows each)
  const int NB128 = 2 * Ip / 128;     // 128-row scale blocks of w13

  // Start-up, ordered so that no wait on one load also waits for the weight
  // stream: the routing and the quantised x are copied into LDS, the active
  // experts listed, and only then the first item's weights issued.  Every
  // pointer has a fixed address space (a generic access would make the
  // compiler's waits on the weight loads conservative).
  {
    for (int f = tid; f < P; f += kThreads) ids_l[f] = p.ids[f];
    // 8 loads in flight per lane (indices clamped into the rows, stores masked)
    const int nq = T * HP / 16;
    for (int i0 = tid; i0 < nq; i0 += 8 * kThreads) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ((const uint4*)p.xq)[min(i0 + j * kThreads, nq - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i0 + j * kThreads < nq) ((uint4*)xq_l)[i0 + j * kThreads] = v[j];
    }
    const int ns = T * XS_LD / 4;
    for (int i = tid; i < ns; i += kThreads) ((uint32_t*)xs_l)[i] = ((const uint32_t*)p.xs)[i];
    __syncthreads();
  }
  const int n_act = build_expert_list(ids_l, P, k, p.E, emask, ebase, act, etk, rpair);
  const int n_items = n_act * S;
  const int n_my = (int)blockIdx.x < n_items ? (n_items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;

  // Loads of item `it` (any index: past the last item, or with no item at
  // all, the workgroup's first item or expert 0 is loaded again and never
  // used, so every load below is unconditional and the compiler's waits
  // count exact).  The wave's weight tiles at its q-th K block kb = wave + 8q
  // are tile positions 2wn, 2wn+1 (gate) and 8+2wn, 9+2wn (up) of N tile s/4
  // (wn = s%4): two 4 KB runs.  The N tile's gate and up block scales of all
  // K blocks come as one word per lane (lane < KB: gate, K block lane; KB <=
  // lane < 2KB: up), read back with readlane.
  const uint8_t* w13 = p.w13;
  auto item_e = [&](int it, int& s) __attribute__((always_inline)) {
    const int c = it < n_items ? it : (n_items > 0 ? (int)blockIdx.x % n_items : 0);
    const int r = c / S;
    s = c - r * S;
    return n_items > 0 ? act[r] : 0;
  };
  uint4 wlo[KBW][4], whi[KBW][4];
  auto issue = [&](int e, int s, int q) __attribute__((always_inline)) {
    const int nt = s >> 2, wn = s & 3;
    const int kb = wave + kWaves * q;
    const uint8_t* b = w13 + ((((int64_t)e * NG + nt) * KB + kb) * 16) * 2048 + lane * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = (j < 2) ? 2 * wn + j : 8 + 2 * wn + (j - 2);
      wlo[q][j] = *(const uint4*)(b + pos * 2048);
      whi[q][j] = *(const uint4*)(b + pos * 2048 + 1024);
    }
  };
  auto scale_word = [&](int e, int s) __attribute__((always_inline)) {
    const int nt = s >> 2;
    const int kb = lane < KB ? lane : (lane < 2 * KB ? lane - KB : 0);
    const int blk = lane >= KB && lane < 2 * KB ? Ip / 128 + nt : nt;
    return p.s13[((int64_t)e * NB128 + blk) * KB + kb];
  };
  int s_c;
  int e_c = item_e(blockIdx.x, s_c);
  float sw_c = scale_word(e_c, s_c);
  // the scale word stays ahead of the tiles (as in the loop), so that its
  // wait at the loop head never covers the tile loads
  asm volatile("" ::: "memory");
#pragma unroll
  for (int q = 0; q < KBW; ++q) issue(e_c, s_c, q);

  const float L = p.limit;
  for (int i = 0; i < n_my; ++i) {
    const int it = (int)blockIdx.x + i * (int)gridDim.x;
    const int r = it / S, s = it - r * S;
    // this item's block scales into scalars, then the next item's scale word
    // into the same register (an in-place reload needs no copy at the loop
    // edge, which would wait for the whole prefetch), then its tiles step
    // by step as each step's registers are consumed
    float swg[KBW], swu[KBW];
#pragma unroll
    for (int q = 0; q < KBW; ++q) {
      swg[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sw_c), wave + kWaves * q));
      swu[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sw_c), KB + wave + kWaves * q));
    }
    int s_n;
    const int e_n = item_e(it + (int)gridDim.x, s_n);
    sw_c = scale_word(e_n, s_n);
    asm volatile("" ::: "memory");
    const int f_row = rpair[16 * r + (lane & 15)];
    const int tok = f_row >= 0 ? f_row / k : -1;
    v4f acc[4] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f},
                  v4f{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int q = 0; q < KBW; ++q) {
      const int kb = wave + kWaves * q;
      v8i t = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      float ts = 0.0f;
      if (tok >= 0) {
        const uint8_t* tp = xq_l + tok * HP + kb * 128 + 32 * (lane >> 4);
        t = frag_from(*(const uint4*)tp, *(const uint4*)(tp + 16));
        ts = E8 ? e8m0_value(xs_l[tok * XS_LD + kb]) : ((const float*)xs_l)[tok * KB + kb];
      }
      v8h th[4];
      widen_fp8(t, th);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v8h wh[4];
        widen_fp8(frag_from(wlo[q][j], whi[q][j]), wh);
        v4f c = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) c = mfma_f16(wh[kk], th[kk], c);
        const float sc = ts * (j < 2 ? swg[q] : swu[q]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[j][ii] = fmaf(c[ii], sc, acc[j][ii]);
      }
      issue(e_n, s_n, q);  // the next item's q-th step into the registers just used
      // keeps the loads here, in flight during the remaining steps (left to
      // itself the scheduler sinks them all past the item's last MFMA)
      asm volatile("" ::: "memory");
    }
    // K partial sums of the 8 waves, added in wave order
    float* rw = red + wave * 1024;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) rw[(j * 4 + ii) * 64 + lane] = acc[j][ii];
    __syncthreads();
    {
      // thread -> (token row m, column c of the 32): gate at tile c/16, up at
      // tile c/16 + 2; MFMA lane m + 16*((c%16)/4), element c%4
      const int c = tid & 31, m = tid >> 5;
      const int jj = c >> 4, rr = c & 15;
      const int l = m + 16 * (rr >> 2), ii = rr & 3;
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        g += red[w * 1024 + (jj * 4 + ii) * 64 + l];
        u += red[w * 1024 + ((jj + 2) * 4 + ii) * 64 + l];
      }
      const int f = rpair[16 * r + m];
      if (f >= 0) p.a[(int64_t)f * Ip + kSlice * s + c] = swiglu_clamped(g, u, L);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Re-quantisation of one unit (pair f, 128 columns gq*128 ..) of the fp32
// SwiGLU rows a: 16 lanes x 8 values (v; zero for a pair without a row),
// the arithmetic of the prefill GEMM1 epilogue (FP8: scale amax/448 and
// codes v * fl32(1/scale); UE8M0: the power-of-two scale byte).  Returns
// the packed codes of the lane and, through sv / sbyte, the scale (the exact
// fp32 value, and the UE8M0 byte).
// ---------------------------------------------------------------------------
template <int QM>
__device__ __forceinline__ uint2 requant_unit(float (&v)[8], float& sv, uint32_t& sbyte) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<16>(amax);
  uint32_t c[8];
  sbyte = 0;
  if constexpr (QM == kQuantFp8E8) {
    sbyte = ue8m0_byte(amax);
    const float inv = e8m0_inverse(sbyte);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (amax > 0.0f) ? fp8e8_quant(v[i], inv) : 0u;
    sv = e8m0_value(sbyte);
  } else {
    const float sc = amax / kE4M3Max;
    const float inv = 1.0f / sc;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (amax > 0.0f) ? fp8_quant_inv(v[i], inv) : 0u;
    sv = (amax > 0.0f) ? sc : 0.0f;
  }
  return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// Stores one unit's codes and scale into the intermediate in pair order
// (aq [P][Ip]; as fp32 [P][Ip/128] or UE8M0 bytes [P][row of whole dwords]).
template <int QM, int KB>
__device__ __forceinline__ void store_unit(const DecodeArgs& p, int f, int gq, int col, uint2 pk, float sv,
                                           uint32_t sbyte) {
  const int lane = threadIdx.x & 63;
  *(uint2*)(p.aq + (int64_t)f * KB * 128 + col) = pk;
  if ((lane & 15) == 0) {
    if constexpr (QM == kQuantFp8E8) {
      constexpr int LD = (KB + 3) / 4 * 4;
      uint8_t* srow = (uint8_t*)p.as + (int64_t)f * LD;
      srow[gq] = (uint8_t)sbyte;
      if (gq == KB - 1)
        for (int i = KB; i < LD; ++i) srow[i] = 0;
    } else {
      ((float*)p.as)[(int64_t)f * KB + gq] = sv;
    }
  }
}

// The intermediate of all pairs, once (decode batches above kDecodeSmallT):
// 32 units per workgroup.
template <int QM, int KB>
__global__ __launch_bounds__(kThreads) void decode_requant_kernel(DecodeArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = p.T * p.k, units = P * KB;
  const int u = blockIdx.x * 32 + wave * 4 + (lane >> 4);
  if (blockIdx.x * 32 + wave * 4 >= units) return;  // whole wave past the end
  const bool live = u < units;
  const int f = live ? u / KB : 0, gq = live ? u - f * KB : 0;
  const int col = gq * 128 + (lane & 15) * 8;
  const int e = p.ids[f];
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  if (live && e >= 0 && e < p.E) {
    const float* src = p.a + (int64_t)f * KB * 128 + col;
    const float4 lo = *(const float4*)src, hi = *(const float4*)(src + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  }
  float sv;
  uint32_t sbyte;
  const uint2 pk = requant_unit<QM>(v, sv, sbyte);
  if (live) store_unit<QM, KB>(p, f, gq, col, pk, sv, sbyte);
}

// ---------------------------------------------------------------------------
// Re-quantisation of a + GEMM2 + weighted combine.  Workgroup b computes
// output columns 16b .. 16b+15 of every token.  KB = Ip / 128.
// ---------------------------------------------------------------------------
template <int QM, int KB, bool REQ>
__global__ __launch_bounds__(kThreads) void decode_gemm2_kernel(DecodeArgs p) {
  static_assert(KB == 1 || KB == 2 || KB == 4 || KB == 8, "K blocks of GEMM2");
  constexpr bool E8 = QM == kQuantFp8E8;
  constexpr int IP = KB * 128;
  __shared__ __attribute__((aligned(16))) uint8_t a_l[kDecodeMaxPairs * IP];
  __shared__ __attribute__((aligned(16))) float as_l[kDecodeMaxPairs * KB];  // exact fp32 scale per (pair, K block)
  __shared__ __attribute__((aligned(16))) float y_l[kDecodeMaxPairs * 16];
  __shared__ int32_t ids_l[kDecodeMaxPairs];
  __shared__ float wts_l[kDecodeMaxPairs];
  __shared__ uint32_t emask[32];
  __shared__ int32_t ebase[33];
  __shared__ int32_t act[kDecodeMaxPairs];
  __shared__ uint32_t etk[1024];
  __shared__ int16_t rpair[kDecodeMaxPairs * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, k = p.k, P = T * k, Hp = p.Hp;
  const int NG = (Hp + 255) / 256;   // N tiles of w2
  const int sb = blockIdx.x;         // 16-row slice of w2 (output columns 16sb ..)
  const int g = sb >> 4, pos = sb & 15;

  // Start-up, ordered so that no wait on one load also waits for the weight
  // stream: the routing and the first rows of a are loaded together, the
  // active experts listed, a re-quantised into LDS, and only then the first
  // experts' weights issued.
  //
  // Re-quantisation of a (the arithmetic of the prefill GEMM1 epilogue):
  // unit = (pair, 128 columns), 16 lanes x 8 values; pass rq of a chunk
  // holds unit u0 + 32 rq + lane/16 of the lane group, every load issued
  // (clamped into the rows, masked after); pairs whose id is outside [0, E)
  // have no row of a and get zero codes.  Workgroup 0 also stores the codes
  // and scales (pair order) when asked to.
  constexpr int RQ = 8;
  const int units = P * KB;
  auto load_chunk = [&](int u0, float (&v)[RQ][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int rq = 0; rq < RQ; ++rq) {
      const int u = min(u0 + kWaves * 4 * rq + (lane >> 4), units - 1);
      const int f = u / KB, gq = u - f * KB;
      const float* src = p.a + (int64_t)f * IP + gq * 128 + (lane & 15) * 8;
      const float4 lo = *(const float4*)src, hi = *(const float4*)(src + 4);
      v[rq][0] = lo.x; v[rq][1] = lo.y; v[rq][2] = lo.z; v[rq][3] = lo.w;
      v[rq][4] = hi.x; v[rq][5] = hi.y; v[rq][6] = hi.z; v[rq][7] = hi.w;
    }
  };
  auto requant_chunk = [&](int u0, float (&v)[RQ][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int rq = 0; rq < RQ; ++rq) {
      const int ub = u0 + kWaves * 4 * rq;  // the wave's first unit of this pass
      if (ub >= units) break;
      const int u = ub + (lane >> 4);
      const bool live = u < units;
      const int f = live ? u / KB : 0, gq = live ? u - f * KB : 0;
      const int col = gq * 128 + (lane & 15) * 8;
      const bool has = live && ids_l[f] >= 0 && ids_l[f] < p.E;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (!has) v[rq][i] = 0.0f;
      float sv;
      uint32_t sbyte;
      const uint2 pk = requant_unit<QM>(v[rq], sv, sbyte);
      if (live) {
        *(uint2*)(a_l + f * IP + col) = pk;
        if ((lane & 15) == 0) as_l[f * KB + gq] = sv;
        if (blockIdx.x == 0 && p.aq) store_unit<QM, KB>(p, f, gq, col, pk, sv, sbyte);
      }
    }
  };

  int32_t my_id = 0;
  float my_w = 0.0f;
  if (tid < P) {
    my_id = p.ids[tid];
    my_w = p.topk_w[tid];
  }
  int n_act;
  if constexpr (REQ) {
    float av[RQ][8];
    load_chunk(wave * 4, av);
    for (int i = tid; i < P * 16; i += kThreads) y_l[i] = 0.0f;
    if (tid < P) {
      ids_l[tid] = my_id;
      wts_l[tid] = my_w;
    }
    __syncthreads();
    n_act = build_expert_list(ids_l, P, k, p.E, emask, ebase, act, etk, rpair);
    requant_chunk(wave * 4, av);
    for (int u0 = wave * 4 + kWaves * 4 * RQ; u0 < units; u0 += kWaves * 4 * RQ) {
      load_chunk(u0, av);
      requant_chunk(u0, av);
    }
  } else {
    // the intermediate as stored by decode_requant_kernel: codes and scales
    // copied into LDS, 8 loads in flight per lane (indices clamped, stores
    // masked)
    const int nq = P * IP / 16;
    for (int i0 = tid; i0 < nq; i0 += 8 * kThreads) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ((const uint4*)p.aq)[min(i0 + j * kThreads, nq - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (i0 + j * kThreads < nq) ((uint4*)a_l)[i0 + j * kThreads] = v[j];
    }
    for (int i = tid; i < P * KB; i += kThreads) {
      const int f = i / KB, gq = i - f * KB;
      if constexpr (E8)
        as_l[i] = e8m0_value(((const uint8_t*)p.as)[(int64_t)f * ((KB + 3) / 4 * 4) + gq]);
      else
        as_l[i] = ((const float*)p.as)[i];
    }
    for (int i = tid; i < P * 16; i += kThreads) y_l[i] = 0.0f;
    if (tid < P) {
      ids_l[tid] = my_id;
      wts_l[tid] = my_w;
    }
    __syncthreads();
    n_act = build_expert_list(ids_l, P, k, p.E, emask, ebase, act, etk, rpair);
  }

  // The wave takes ranks wave, wave + 8, ...: its i-th is rho(i), and past
  // its last it repeats the last (the repeat recomputes identical values
  // from L2-resident tiles), so loads and computes need no branches.
  const int n_mine = wave < n_act ? (n_act - 1 - wave) / kWaves + 1 : 0;
  auto rho = [&](int i) __attribute__((always_inline)) { return wave + kWaves * min(i, n_mine - 1); };
  // K block kb of row tile `pos` of N tile g (TILED_V2, tile run 4):
  // tile index (((e*NG + g)*4 + pos/4)*KB + kb)*4 + pos%4
  uint4 wlo[2][KB], whi[2][KB];
  float wsc[2][KB];
  auto issue = [&](int b, int r) __attribute__((always_inline)) {
    const int e = act[r];
    const uint8_t* t0 = p.w2 + ((((int64_t)e * NG + g) * 4 + (pos >> 2)) * KB * 4 + (pos & 3)) * 2048 + lane * 16;
    const float* sp = p.s2 + ((int64_t)e * (Hp / 128) + (sb >> 3)) * KB;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      wlo[b][kb] = *(const uint4*)(t0 + kb * 4 * 2048);
      whi[b][kb] = *(const uint4*)(t0 + kb * 4 * 2048 + 1024);
      wsc[b][kb] = sp[kb];
    }
  };
  if (n_mine > 0) {
    issue(0, rho(0));
    issue(1, rho(1));
  }
  __syncthreads();

  // GEMM2: lane l holds output rows 4(l/16) + i of the slice for MFMA row
  // (token) l%16 of the expert.  FP8 MFMA per K block, promoted by the
  // product of the two block scales (exact powers of two for UE8M0).
  auto compute = [&](int b, int r) __attribute__((always_inline)) {
    const int f = rpair[16 * r + (lane & 15)];
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      v8i t = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      float ts = 0.0f;
      if (f >= 0) {
        const uint8_t* tp = a_l + f * IP + kb * 128 + 32 * (lane >> 4);
        t = frag_from(*(const uint4*)tp, *(const uint4*)(tp + 16));
        ts = as_l[f * KB + kb];
      }
      const v4f c = mfma_fp8(frag_from(wlo[b][kb], whi[b][kb]), t, v4f{0.0f, 0.0f, 0.0f, 0.0f});
      const float sc = ts * wsc[b][kb];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) acc[ii] = fmaf(c[ii], sc, acc[ii]);
    }
    if (f >= 0) *(float4*)(y_l + f * 16 + 4 * (lane >> 4)) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  };
  for (int i = 0; i < n_mine; i += 2) {
    compute(0, rho(i));
    issue(0, rho(i + 2));
    compute(1, rho(i + 1));
    issue(1, rho(i + 3));
  }
  __syncthreads();

  // combine: token t, column 16sb + c: weighted pairs in slot order
  if (tid < T * 16) {
    const int t = tid >> 4, c = tid & 15;
    float o = 0.0f;
    for (int j = 0; j < k; ++j) o = fmaf(wts_l[t * k + j], y_l[(t * k + j) * 16 + c], o);
    const int col = 16 * sb + c;
    if (col < p.H) p.out[(int64_t)t * p.ld_out + col] = f32_to_bf16(o);
  }
}

template <int QM>
hipError_t launch_g1_q(const DecodeArgs& a, int grid, hipStream_t s) {
  switch (a.Hp / 1024) {
    case 1: hipLaunchKernelGGL((decode_gemm1_kernel<QM, 1>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_gemm1_kernel<QM, 2>), dim3(grid), dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((decode_gemm1_kernel<QM, 4>), dim3(grid), dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_ok(int mode, int T, int E, int k, int Hp, int Ip) {
  if (mode != kQuantFp8 && mode != kQuantFp8E8) return false;
  if (T < 1 || T > kDecodeMaxT || k < 1 || T * k > kDecodeMaxPairs || E < 1 || E > 1024) return false;
  if (Hp != 1024 && Hp != 2048 && Hp != 4096) return false;
  return Ip == 128 || Ip == 256 || Ip == 512 || Ip == 1024;
}

int decode_gemm1_grid() { return gemm_grid_max(); }

hipError_t launch_decode_gemm1(int mode, const DecodeArgs& a, hipStream_t s) {
  const int grid = decode_gemm1_grid();
  return mode == kQuantFp8E8 ? launch_g1_q<kQuantFp8E8>(a, grid, s) : launch_g1_q<kQuantFp8>(a, grid, s);
}

template <int QM, int KB>
static void launch_g2_kb(const DecodeArgs& a, bool req, hipStream_t s) {
  const dim3 grid((unsigned)(a.Hp / 16)), block(kThreads);
  if (req)
    hipLaunchKernelGGL((decode_gemm2_kernel<QM, KB, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_gemm2_kernel<QM, KB, false>), grid, block, 0, s, a);
}

template <int QM>
static void launch_g2_q(const DecodeArgs& a, bool req, hipStream_t s) {
  switch (a.Ip / 128) {
    case 1: launch_g2_kb<QM, 1>(a, req, s); break;
    case 2: launch_g2_kb<QM, 2>(a, req, s); break;
    case 4: launch_g2_kb<QM, 4>(a, req, s); break;
    default: launch_g2_kb<QM, 8>(a, req, s); break;
  }
}

template <int QM>
static void launch_rq_q(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.T * a.k * (a.Ip / 128) + 31) / 32)), block(kThreads);
  switch (a.Ip / 128) {
    case 1: hipLaunchKernelGGL((decode_requant_kernel<QM, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_requant_kernel<QM, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_requant_kernel<QM, 4>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((decode_requant_kernel<QM, 8>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_decode_gemm2(int mode, const DecodeArgs& a, hipStream_t s) {
  // small batches re-quantise inside GEMM2 (every workgroup, all pairs);
  // larger ones once, in a kernel of their own, into aq / as first
  const bool req = a.T <= kDecodeSmallT;
  if (!req) {
    if (mode == kQuantFp8E8)
      launch_rq_q<kQuantFp8E8>(a, s);
    else
      launch_rq_q<kQuantFp8>(a, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mode == kQuantFp8E8)
    launch_g2_q<kQuantFp8E8>(a, req, s);
  else
    launch_g2_q<kQuantFp8>(a, req, s);
  return hipGetLastError();
}

}  // namespace moe
