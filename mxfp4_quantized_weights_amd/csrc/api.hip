// C ABI of libmoe.so: argument validation (before anything is enqueued),
// workspace layout and kernel sequencing.  See include/moe.h for the contract
// of every entry point.
//
// sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark MXFP4 MoE
// on gfx950", contract table: the gate mode is explicit and only separate
// halves are accepted, the SwiGLU limit is always forwarded, the preshuffled
// layout belongs to this runner (layout tag), an unsupported configuration
// fails when it is validated rather than later, and hidden/intermediate
// padding is carried as metadata.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

constexpr int32_t kMaxExperts = 1024;
constexpr int32_t kMaxTopK = 16;
constexpr int32_t kMaxDim = 1 << 16;       // padded hidden / intermediate
constexpr int64_t kMaxPairs = 1ll << 24;   // T * top_k
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

inline moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

inline bool known_mode(int32_t m) {
  return m == MOE_QUANT_FP8_BLOCK || m == MOE_QUANT_MXFP4 || m == MOE_QUANT_FP8_UE8M0;
}
// e4m3 codes, one byte per element (block FP8 with either scale format)
inline bool fp8_codes(int32_t m) { return m != MOE_QUANT_MXFP4; }

// Bytes of one row of quantised codes and of its scales for `cols` padded
// columns: FP8 fp32 per 128, UE8M0 one byte per 128 (rows of whole dwords),
// MX one byte per 32.
inline int64_t code_row_bytes(int32_t m, int64_t cols) { return fp8_codes(m) ? cols : cols / 2; }
inline int64_t scale_row_bytes(int32_t m, int64_t cols) {
  if (m == MOE_QUANT_FP8_BLOCK) return cols / 128 * 4;
  if (m == MOE_QUANT_FP8_UE8M0) return moe::e8_scale_ld(cols);
  return cols / 32;
}
// Scale elements per row as the GEMMs index them (floats for FP8, bytes otherwise).
inline int64_t scale_row_elems(int32_t m, int64_t cols) {
  return m == MOE_QUANT_FP8_BLOCK ? cols / 128 : scale_row_bytes(m, cols);
}

moe_status_t check_cfg(const moe_cfg_t* c) {
  if (!c) return MOE_ERR_NULL;
  if (c->num_experts < 1 || c->num_experts > kMaxExperts) return MOE_ERR_SHAPE;
  if (c->top_k < 1 || c->top_k > kMaxTopK || c->top_k > c->num_experts) return MOE_ERR_SHAPE;
  if (!known_mode(c->quant_mode)) return MOE_ERR_UNSUPPORTED;
  if (c->gate_mode != MOE_GATE_SEPARATED) return MOE_ERR_UNSUPPORTED;
  if (c->block_m != 16 && c->block_m != 32 && c->block_m != 64 && c->block_m != 128) return MOE_ERR_UNSUPPORTED;
  if (!(c->swiglu_limit > 0.0f)) return MOE_ERR_UNSUPPORTED;  // rejects NaN, 0, negatives
  const moe_pad_t& p = c->pad;
  if (p.hidden < 1 || p.inter < 1 || p.hidden_padded < p.hidden || p.inter_padded < p.inter) return MOE_ERR_SHAPE;
  if (p.hidden_padded > kMaxDim || p.inter_padded > kMaxDim) return MOE_ERR_SHAPE;
  if (p.hidden_padded % 128 != 0 || p.inter_padded % 128 != 0) return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe_status_t check_tokens(const moe_cfg_t* c, int32_t T) {
  if (T < 0) return MOE_ERR_SHAPE;
  if ((int64_t)T * c->top_k > kMaxPairs) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status_t check_layout(const moe_cfg_t* c) {
  return c->weight_layout == MOE_LAYOUT_TILED_V2 ? MOE_OK : MOE_ERR_LAYOUT;
}

int32_t max_blocks(int64_t P, int32_t E, int32_t BM) {
  int64_t a = (P + (int64_t)E * (BM - 1)) / BM;
  return (int32_t)(P < a ? P : a);
}

// K blocks and N tiles per block of GEMM1 (which = 13) or GEMM2 (which = 2).
int gemm_kb(const moe_cfg_t* c, int which) {
  return (which == 13 ? c->pad.hidden_padded : c->pad.inter_padded) / 128;
}
int gemm_n_tiles(const moe_cfg_t* c, int which) {
  return which == 13 ? c->pad.inter_padded / 128 : (c->pad.hidden_padded + 255) / 256;
}

// Tail split of GEMM1 (ksplit -2, -4 or -8): only the items past the grid's
// whole rounds are cut into -ksplit pieces (the partial sums of a leftover
// item are block_m rows of 256 floats per piece); at block_m 64 and 128 at
// most 4 pieces, which bounds those partial sums.
constexpr int kTailMaxWide = 4;
bool tail_usable(const moe_cfg_t* c, int which, int ks) {
  return which == 13 && ks < -1 && (c->block_m <= 32 || -ks <= kTailMaxWide) &&
         moe::ksplit_ok(c->quant_mode, gemm_kb(c, which), -ks);
}
size_t tail_bytes(const moe_cfg_t* c, int ks) {
  return align_up((size_t)((int64_t)ks * moe::gemm_grid_max() * c->block_m * 256 * 4));
}

// A K split for GEMM `which` at T tokens is usable if the pieces align with
// the scale layout and, for GEMM2, y is not column-chunked; a tail split
// (negative) as tail_usable.
bool ksplit_usable(const moe_cfg_t* c, int32_t T, int which, int ks) {
  if (ks < 0) return tail_usable(c, which, ks);
  if (!moe::ksplit_ok(c->quant_mode, gemm_kb(c, which), ks)) return false;
  if (ks == 1) return true;
  const int64_t P = (int64_t)T * c->top_k;
  if (P > moe::kSplitMaxPairs) return false;
  return which == 13 || moe::y_chunk_cols(P, c->pad.hidden_padded) == c->pad.hidden_padded;
}

// The split the library uses: a K split of every item when workgroups would
// otherwise idle; else, for GEMM1 where the last round of items is expected
// to leave most workgroups idle, a tail split into the most pieces the scale
// layout allows (at most 4 at block_m 64 and 128, and there block FP8 only:
// on one MI355X the tensor-parallel share of the prefill layer, I = 128,
// gained 9% in GEMM1 from it, the MXFP4 share with I = 256 lost 20%).
int plan_ksplit(const moe_cfg_t* c, int32_t T, int which) {
  const int ks = moe::pick_ksplit(c->quant_mode, T, c->num_experts, c->top_k, c->block_m, gemm_kb(c, which),
                                  gemm_n_tiles(c, which));
  if (ks > 1 && ksplit_usable(c, T, which, ks)) return ks;
  if (c->block_m >= 64 && c->quant_mode == MOE_QUANT_MXFP4) return 1;
  if (which == 13 && moe::tail_split_plan_ok(T, c->num_experts, c->top_k, c->block_m, gemm_n_tiles(c, which)))
    for (int t = -moe::kSplitMax; t <= -2; t /= 2)
      if (tail_usable(c, which, t)) return t;
  return 1;
}

// Scratch of a GEMM at split ks: GEMM1 the fp32 partial sums and each pair's
// sorted row (none without a split), GEMM2 the y planes.
size_t split_bytes(const moe_cfg_t* c, int32_t T, int which, int ks) {
  if (ks < 0) return tail_bytes(c, -ks);
  const int64_t P = (int64_t)T * c->top_k;
  const int64_t Hp = c->pad.hidden_padded, Ip = c->pad.inter_padded;
  if (which == 13) return ks > 1 ? align_up((size_t)(ks * P * 2 * Ip * 4 + P * 4)) : 0;
  // unsplit: the (possibly column-chunked) y rows; split: whole planes
  const int64_t planes = ks > 1 ? ks * moe::y_plane_bytes(P, Hp) : 0, y = moe::y_reserve_bytes(P, Hp);
  return align_up((size_t)(planes > y ? planes : y));
}

// Scratch that covers every split the library can choose for any T' <= T
// (non-decreasing in T): the largest split times min(P, kSplitMaxPairs).
size_t split_reserve(const moe_cfg_t* c, int32_t T, int which) {
  const int64_t P = (int64_t)T * c->top_k;
  const int64_t Ps = P < moe::kSplitMaxPairs ? P : moe::kSplitMaxPairs;
  const int cap = moe::ksplit_cap(c->quant_mode, gemm_kb(c, which));
  const int64_t Hp = c->pad.hidden_padded, Ip = c->pad.inter_padded;
  if (which == 13) {
    const size_t full = cap > 1 ? align_up((size_t)(cap * Ps * 2 * Ip * 4 + Ps * 4)) : 0;
    const int tcap = c->block_m <= 32 || cap < kTailMaxWide ? cap : kTailMaxWide;
    const size_t tail = tail_usable(c, 13, -tcap) ? tail_bytes(c, tcap) : 0;
    return full > tail ? full : tail;
  }
  const int64_t planes = cap > 1 ? cap * moe::y_plane_bytes(Ps, Hp) : 0, y = moe::y_reserve_bytes(P, Hp);
  return align_up((size_t)(planes > y ? planes : y));
}

// Sizes of the pieces of one layer's scratch, in carve order.
struct Layout {
  size_t ids, wts, sorted, bexp, offs, npp, xq, xs, aq, as, part, y, total;
};

Layout layout_for(const moe_cfg_t* c, int32_t T) {
  Layout L{};
  const int64_t P = (int64_t)T * c->top_k;
  const int32_t nb = max_blocks(P, c->num_experts, c->block_m);
  const int64_t rows = (int64_t)nb * c->block_m;
  const int64_t Hp = c->pad.hidden_padded, Ip = c->pad.inter_padded;
  const int32_t m = c->quant_mode;
  L.ids = align_up(P * 4);
  L.wts = align_up(P * 4);
  L.sorted = align_up(rows * 4);
  L.bexp = align_up((size_t)nb * 4);
  L.offs = align_up((size_t)(c->num_experts + 1) * 4);
  L.npp = align_up(4);
  L.xq = align_up(T * code_row_bytes(m, Hp));
  L.xs = align_up(T * scale_row_bytes(m, Hp));
  L.aq = align_up(rows * code_row_bytes(m, Ip));
  L.as = align_up(rows * scale_row_bytes(m, Ip));
  L.part = split_reserve(c, T, 13);
  L.y = split_reserve(c, T, 2);
  L.total = L.ids + L.wts + L.sorted + L.bexp + L.offs + L.npp + L.xq + L.xs + L.aq + L.as + L.part + L.y;
  return L;
}

moe::GemmArgs gemm1_args(const moe_cfg_t* c, int32_t T, const void* xq, const void* xs, const int32_t* sorted,
                         const int32_t* bexp, const int32_t* npp, const void* w13, const void* s13, void* aq,
                         void* as) {
  moe::GemmArgs a{};
  const int32_t m = c->quant_mode;
  const int Hp = c->pad.hidden_padded, Ip = c->pad.inter_padded;
  a.A = (const uint8_t*)xq;
  a.As = xs;
  a.lda = code_row_bytes(m, Hp);
  a.ldas = scale_row_elems(m, Hp);
  a.sorted_ids = sorted;
  a.block_expert = bexp;
  a.npp = npp;
  a.top_k = c->top_k;
  a.num_pairs = T * c->top_k;
  a.B = (const uint8_t*)w13;
  a.Bs = s13;
  a.N = 2 * Ip;
  a.K = Hp;
  a.tile_run = moe::tile_run(c->quant_mode, 13);
  a.n_tiles = Ip / 128;
  a.aq = (uint8_t*)aq;
  a.as = as;
  a.Ip = Ip;
  a.limit = c->swiglu_limit;
  return a;
}

moe::GemmArgs gemm2_args(const moe_cfg_t* c, int32_t T, const void* aq, const void* as, const int32_t* sorted,
                         const int32_t* bexp, const int32_t* npp, const void* w2, const void* s2, uint8_t* y,
                         const float* topk_w) {
  moe::GemmArgs a{};
  const int32_t m = c->quant_mode;
  const int Hp = c->pad.hidden_padded, Ip = c->pad.inter_padded;
  a.A = (const uint8_t*)aq;
  a.As = as;
  a.lda = code_row_bytes(m, Ip);
  a.ldas = scale_row_elems(m, Ip);
  a.sorted_ids = sorted;
  a.block_expert = bexp;
  a.npp = npp;
  a.top_k = c->top_k;
  a.num_pairs = T * c->top_k;
  a.B = (const uint8_t*)w2;
  a.Bs = s2;
  a.N = Hp;
  a.K = Ip;
  a.tile_run = moe::tile_run(c->quant_mode, 2);
  a.n_tiles = (Hp + 255) / 256;
  a.Ip = Ip;
  a.limit = c->swiglu_limit;
  a.y = y;
  a.topk_w = topk_w;
  return a;
}

// Routing, permutation and quantisation of x: one launch up to 16 tokens
// (one workgroup routes and permutes, the others quantise), else two
// (routing and quantisation together, then the permutation).
hipError_t front_end(const moe_cfg_t* c, int32_t T, const float* logits, const void* x, int64_t ld_x, int32_t* ids,
                     float* wts, int32_t* sorted, int32_t* bexp, int32_t* offs, int32_t* npp, void* xq, void* xs,
                     hipStream_t s) {
  const int E = c->num_experts, k = c->top_k, BM = c->block_m;
  const int32_t nb = max_blocks((int64_t)T * k, E, BM);
  const int H = c->pad.hidden, Hp = c->pad.hidden_padded, mode = c->quant_mode;
  if (moe::front_small_ok(T, E, k))
    return moe::launch_front_small(logits, T, E, k, ids, wts, BM, nb, sorted, bexp, offs, npp, x, H, ld_x, Hp, mode,
                                   xq, xs, s);
  hipError_t e = moe::launch_route_and_quant(logits, T, E, k, ids, wts, x, H, ld_x, Hp, mode, xq, xs, s);
  if (e != hipSuccess) return e;
  return moe::launch_permute_align(ids, T, k, E, BM, nb, sorted, bexp, offs, npp, s);
}

int log2_of(int ks) { return ks >= 8 ? 3 : ks >= 4 ? 2 : ks >= 2 ? 1 : 0; }

// GEMM1, with a K split: the pieces' partial sums in `part`, then the
// SwiGLU and re-quantisation kernel.
hipError_t run_gemm1(const moe_cfg_t* c, int32_t T, moe::GemmArgs a, int32_t nb, int ks, float* part,
                     hipStream_t s) {
  if (ks < -1) {
    a.tail = 1;
    a.ks_log2 = log2_of(-ks);
    a.part = part;
    hipError_t e = moe::launch_gemm1(c->quant_mode, c->block_m, nb, a, s);
    if (e != hipSuccess) return e;
    return moe::launch_gemm1_tail_finish(c->quant_mode, -ks, c->block_m, part, a.sorted_ids, a.npp, a.n_tiles,
                                         moe::gemm_grid_max(), (int)((int64_t)T * c->top_k), a.Ip, a.limit, a.aq,
                                         a.as, s);
  }
  if (ks > 1) {
    a.ks_log2 = log2_of(ks);
    a.part = part;
  }
  hipError_t e = moe::launch_gemm1(c->quant_mode, c->block_m, nb, a, s);
  if (e != hipSuccess || ks == 1) return e;
  return moe::launch_swiglu_requant(c->quant_mode, part, ks, (int)((int64_t)T * c->top_k), a.Ip, a.limit, a.aq,
                                    a.as, s);
}

// GEMM2 and the combine, one column chunk of y at a time (see y_chunk_cols);
// with a K split, one y plane per piece (y is then never chunked).
hipError_t gemm2_and_combine(const moe_cfg_t* c, int32_t T, moe::GemmArgs a, int32_t nb, int ks, void* out_bf16,
                             int64_t ld_out, hipStream_t s) {
  const int64_t P = (int64_t)T * c->top_k;
  const int Hp = c->pad.hidden_padded, H = c->pad.hidden;
  if (ks > 1) {
    a.ks_log2 = log2_of(ks);
    a.ldy = Hp;
    a.yplane = moe::y_plane_bytes(P, Hp);
    a.yexp = moe::y_values_bytes(P, Hp);
    hipError_t e = moe::launch_gemm2(c->quant_mode, c->block_m, nb, a, s);
    if (e != hipSuccess) return e;
    return moe::launch_combine(a.y, a.yexp, T, c->top_k, 0, H, Hp, ks, a.yplane, (uint16_t*)out_bf16, ld_out, s);
  }
  const int64_t W = moe::y_chunk_cols(P, Hp);
  a.ldy = W;
  a.yexp = moe::y_values_bytes(P, W);
  for (int c0 = 0; c0 < Hp; c0 += (int)W) {
    const int wc = (int)(Hp - c0 < W ? Hp - c0 : W);
    a.nt0 = c0 / 256;
    a.n_tiles = (wc + 255) / 256;
    hipError_t e = moe::launch_gemm2(c->quant_mode, c->block_m, nb, a, s);
    if (e != hipSuccess) return e;
    const int cols = H - c0 < wc ? H - c0 : wc;
    if (cols > 0) {
      e = moe::launch_combine(a.y, a.yexp, T, c->top_k, c0, cols, W, 1, 0, (uint16_t*)out_bf16, ld_out, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Whether the decode kernels (decode.hip) take T tokens of this layer.
bool decode_takes(const moe_cfg_t* c, int32_t T) {
  return moe::decode_ok(c->quant_mode, T, c->num_experts, c->top_k, c->pad.hidden_padded, c->pad.inter_padded);
}

moe::DecodeArgs decode_args(const moe_cfg_t* c, int32_t T) {
  moe::DecodeArgs d{};
  d.T = T;
  d.E = c->num_experts;
  d.k = c->top_k;
  d.H = c->pad.hidden;
  d.Hp = c->pad.hidden_padded;
  d.Ip = c->pad.inter_padded;
  d.limit = c->swiglu_limit;
  return d;
}

// The whole layer with its scratch in ws (validated by the caller).
moe_status_t forward_impl(const moe_cfg_t* cfg, int32_t T, const void* x_bf16, int64_t ld_x,
                          const float* router_logits, const void* w13, const void* w13_scale, const void* w2,
                          const void* w2_scale, void* out_bf16, int64_t ld_out, void* ws, hipStream_t s) {
  const Layout L = layout_for(cfg, T);
  uint8_t* p = (uint8_t*)ws;
  int32_t* ids = (int32_t*)p; p += L.ids;
  float* wts = (float*)p; p += L.wts;
  int32_t* sorted = (int32_t*)p; p += L.sorted;
  int32_t* bexp = (int32_t*)p; p += L.bexp;
  int32_t* offs = (int32_t*)p; p += L.offs;
  int32_t* npp = (int32_t*)p; p += L.npp;
  void* xq = p; p += L.xq;
  void* xs = p; p += L.xs;
  void* aq = p; p += L.aq;
  void* as = p; p += L.as;
  float* part = (float*)p; p += L.part;
  uint8_t* y = p;

  const int E = cfg->num_experts, k = cfg->top_k, BM = cfg->block_m;
  const int64_t P = (int64_t)T * k;
  const int32_t nb = max_blocks(P, E, BM);
  hipError_t e;
  if ((e = front_end(cfg, T, router_logits, x_bf16, ld_x, ids, wts, sorted, bexp, offs, npp, xq, xs, s)) !=
      hipSuccess)
    return MOE_ERR_HIP;
  moe::GemmArgs a1 = gemm1_args(cfg, T, xq, xs, sorted, bexp, npp, w13, w13_scale, aq, as);
  if ((e = run_gemm1(cfg, T, a1, nb, plan_ksplit(cfg, T, 13), part, s)) != hipSuccess) return MOE_ERR_HIP;
  moe::GemmArgs a2 = gemm2_args(cfg, T, aq, as, sorted, bexp, npp, w2, w2_scale, y, wts);
  return hip_status(gemm2_and_combine(cfg, T, a2, nb, plan_ksplit(cfg, T, 2), out_bf16, ld_out, s));
}

// Arguments of moe_forward / moe_forward_noalloc other than the scratch.
moe_status_t check_forward(const moe_cfg_t* cfg, int32_t T, const void* x_bf16, int64_t ld_x,
                           const float* router_logits, const void* w13, const void* w13_scale, const void* w2,
                           const void* w2_scale, void* out_bf16, int64_t ld_out) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if ((st = check_layout(cfg)) != MOE_OK) return st;
  if (ld_x < cfg->pad.hidden || ld_out < cfg->pad.hidden) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !router_logits || !w13 || !w13_scale || !w2 || !w2_scale || !out_bf16) return MOE_ERR_NULL;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Scratch of moe_forward_noalloc: one static device array per GPU the
// library runs on, held until the process ends.  Host code never uses the
// array's name as an address (on the host it only names the symbol): the
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (resolved on the device's first call).
moe_status_t noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range or inconsistent";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a padded size is not a multiple of 128";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported quant mode, gate mode, block_m, limit or dtype";
    case MOE_ERR_LAYOUT: return "MOE_ERR_LAYOUT: weight layout tag not accepted by this call";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
  }
  return "unknown moe_status_t";
}

moe_status_t moe_validate_cfg(const moe_cfg_t* cfg) { return check_cfg(cfg); }

int32_t moe_max_blocks(int32_t num_pairs, int32_t num_experts, int32_t block_m) {
  if (num_pairs < 0 || num_experts < 1 || block_m < 1) return -1;
  return max_blocks(num_pairs, num_experts, block_m);
}

size_t moe_workspace_bytes(const moe_cfg_t* cfg, int32_t T_max) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T_max) != MOE_OK) return 0;
  return layout_for(cfg, T_max).total;
}

moe_status_t moe_intermediate_bytes(const moe_cfg_t* cfg, int32_t T, size_t* aq_bytes, size_t* as_bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if (!aq_bytes || !as_bytes) return MOE_ERR_NULL;
  const int64_t rows = (int64_t)max_blocks((int64_t)T * cfg->top_k, cfg->num_experts, cfg->block_m) * cfg->block_m;
  const int64_t Ip = cfg->pad.inter_padded;
  *aq_bytes = (size_t)(rows * code_row_bytes(cfg->quant_mode, Ip));
  *as_bytes = (size_t)(rows * scale_row_bytes(cfg->quant_mode, Ip));
  return MOE_OK;
}

moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t top_k, int32_t* ids, float* weights,
                            void* stream) {
  if (T < 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK || top_k > E) return MOE_ERR_SHAPE;
  if ((int64_t)T * top_k > kMaxPairs) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !weights) return MOE_ERR_NULL;
  return hip_status(moe::launch_route_topk(logits, T, E, top_k, ids, weights, as_stream(stream)));
}

moe_status_t moe_permute_align(const int32_t* ids, int32_t T, int32_t top_k, int32_t E, int32_t block_m,
                               int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                               int32_t* num_post_padded, void* stream) {
  if (T < 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK) return MOE_ERR_SHAPE;
  if (block_m != 16 && block_m != 32 && block_m != 64 && block_m != 128) return MOE_ERR_UNSUPPORTED;
  const int64_t P = (int64_t)T * top_k;
  if (P > kMaxPairs) return MOE_ERR_SHAPE;
  if (!expert_offsets || !num_post_padded) return MOE_ERR_NULL;
  if (P > 0 && (!ids || !sorted_ids || !block_expert)) return MOE_ERR_NULL;
  const int32_t nb = max_blocks(P, E, block_m);
  return hip_status(moe::launch_permute_align(ids, T, top_k, E, block_m, nb, sorted_ids, block_expert,
                                              expert_offsets, num_post_padded, as_stream(stream)));
}

moe_status_t moe_quant_act(const void* in, int32_t in_dtype, int32_t rows, int32_t cols, int64_t ld_in,
                           int32_t cols_padded, int32_t quant_mode, void* q, void* scales, void* stream) {
  if (in_dtype != MOE_DTYPE_BF16 && in_dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
  if (!known_mode(quant_mode)) return MOE_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 1 || cols > cols_padded || ld_in < cols) return MOE_ERR_SHAPE;
  if (cols_padded % 128 != 0) return MOE_ERR_ALIGN;
  if (rows == 0) return MOE_OK;
  if (!in || !q || !scales) return MOE_ERR_NULL;
  return hip_status(moe::launch_quant_rows(in, in_dtype == MOE_DTYPE_BF16, rows, cols, ld_in, cols_padded,
                                           quant_mode, q, scales, as_stream(stream)));
}

moe_status_t moe_route_permute_quant(const moe_cfg_t* cfg, int32_t T, const float* router_logits,
                                     const void* x_bf16, int64_t ld_x, int32_t* ids, float* weights,
                                     int32_t* sorted_ids, int32_t* block_expert, int32_t* expert_offsets,
                                     int32_t* num_post_padded, void* xq, void* xs, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if (ld_x < cfg->pad.hidden) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!router_logits || !x_bf16 || !ids || !weights || !sorted_ids || !block_expert || !expert_offsets ||
      !num_post_padded || !xq || !xs)
    return MOE_ERR_NULL;
  return hip_status(front_end(cfg, T, router_logits, x_bf16, ld_x, ids, weights, sorted_ids, block_expert,
                              expert_offsets, num_post_padded, xq, xs, as_stream(stream)));
}

moe_status_t moe_quant_weights(int32_t quant_mode, const float* w, int32_t E, int32_t N, int32_t K, void* q,
                               void* scales, void* stream) {
  if (!known_mode(quant_mode)) return MOE_ERR_UNSUPPORTED;
  if (E < 1 || N < 1 || K < 1 || N > kMaxDim * 2 || K > kMaxDim) return MOE_ERR_SHAPE;
  if (fp8_codes(quant_mode) ? (N % 128 != 0 || K % 128 != 0) : (K % 32 != 0)) return MOE_ERR_ALIGN;
  if (!w || !q || !scales) return MOE_ERR_NULL;
  hipStream_t s = as_stream(stream);
  if (fp8_codes(quant_mode))
    return hip_status(moe::launch_quant_weight_fp8(quant_mode, w, E, N, K, (uint8_t*)q, scales, s));
  // MXFP4 groups run along K: the same row quantiser as the activations
  if (K % 128 != 0) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_quant_rows(w, false, (int64_t)E * N, K, K, K, moe::kQuantMx, q, scales, s));
}

moe_status_t moe_preshuffled_bytes(const moe_cfg_t* cfg, int32_t which, size_t* w_bytes, size_t* s_bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (which != 13 && which != 2) return MOE_ERR_SHAPE;
  if (!w_bytes || !s_bytes) return MOE_ERR_NULL;
  const int64_t E = cfg->num_experts, Hp = cfg->pad.hidden_padded, Ip = cfg->pad.inter_padded;
  const int64_t N = which == 13 ? 2 * Ip : Hp, K = which == 13 ? Hp : Ip;
  // whole N tiles of 16 row tiles (a half last N tile of w2 is zero-padded)
  const int64_t NG = moe::tiled_n_groups((int)N), KB = K / 128;
  if (fp8_codes(cfg->quant_mode)) {  // UE8M0 scales are widened to fp32
    *w_bytes = (size_t)(E * NG * KB * 16 * 2048);
    *s_bytes = (size_t)(E * (N / 128) * KB * 4);
  } else {
    *w_bytes = (size_t)(E * NG * KB * 16 * 1024);
    *s_bytes = (size_t)(E * NG * ((KB + 3) / 4) * 16 * 64 * 4);
  }
  return MOE_OK;
}

moe_status_t moe_preshuffle_weights(const moe_cfg_t* cfg, int32_t which, const void* w, const void* s, void* w_out,
                                    void* s_out, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (which != 13 && which != 2) return MOE_ERR_SHAPE;
  if (!w || !s || !w_out || !s_out) return MOE_ERR_NULL;
  const int Hp = cfg->pad.hidden_padded, Ip = cfg->pad.inter_padded;
  const int N = which == 13 ? 2 * Ip : Hp, K = which == 13 ? Hp : Ip;
  const int gate_half = which == 13 ? Ip / 16 : 0;
  return hip_status(moe::launch_preshuffle(cfg->quant_mode, (const uint8_t*)w, s, cfg->num_experts, N, K, gate_half,
                                           moe::tile_run(cfg->quant_mode, which), (uint8_t*)w_out, s_out,
                                           as_stream(stream)));
}

moe_status_t moe_grouped_gemm1_swiglu(const moe_cfg_t* cfg, int32_t T, const void* xq, const void* xs,
                                      const int32_t* sorted_ids, const int32_t* block_expert,
                                      const int32_t* num_post_padded, const void* w13, const void* w13_scale, void* aq,
                                      void* as, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if ((st = check_layout(cfg)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!xq || !xs || !sorted_ids || !block_expert || !num_post_padded || !w13 || !w13_scale || !aq || !as)
    return MOE_ERR_NULL;
  const int32_t nb = max_blocks((int64_t)T * cfg->top_k, cfg->num_experts, cfg->block_m);
  const int mode = cfg->quant_mode;
  moe::GemmArgs a = gemm1_args(cfg, T, xq, xs, sorted_ids, block_expert, num_post_padded, w13, w13_scale, aq, as);
  return hip_status(moe::launch_gemm1(mode, cfg->block_m, nb, a, as_stream(stream)));
}

moe_status_t moe_grouped_gemm1_swiglu_splitk(const moe_cfg_t* cfg, int32_t T, const void* xq, const void* xs,
                                             const int32_t* sorted_ids, const int32_t* block_expert,
                                             const int32_t* num_post_padded, const void* w13, const void* w13_scale,
                                             void* aq, void* as, int32_t ksplit, void* ws, size_t ws_bytes,
                                             void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if ((st = check_layout(cfg)) != MOE_OK) return st;
  if (!ksplit_usable(cfg, T, 13, ksplit)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!xq || !xs || !sorted_ids || !block_expert || !num_post_padded || !w13 || !w13_scale || !aq || !as)
    return MOE_ERR_NULL;
  if (ksplit != 1 && !ws) return MOE_ERR_NULL;
  if (ws_bytes < split_bytes(cfg, T, 13, ksplit)) return MOE_ERR_WORKSPACE;
  const int32_t nb = max_blocks((int64_t)T * cfg->top_k, cfg->num_experts, cfg->block_m);
  moe::GemmArgs a = gemm1_args(cfg, T, xq, xs, sorted_ids, block_expert, num_post_padded, w13, w13_scale, aq, as);
  return hip_status(run_gemm1(cfg, T, a, nb, ksplit, (float*)ws, as_stream(stream)));
}

moe_status_t moe_grouped_gemm2_combine_splitk(const moe_cfg_t* cfg, int32_t T, const void* aq, const void* as,
                                              const int32_t* sorted_ids, const int32_t* block_expert,
                                              const int32_t* num_post_padded, const void* w2, const void* w2_scale,
                                              const float* topk_w, void* out_bf16, int64_t ld_out, int32_t ksplit,
                                              void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if ((st = check_layout(cfg)) != MOE_OK) return st;
  if (ld_out < cfg->pad.hidden) return MOE_ERR_SHAPE;
  if (!ksplit_usable(cfg, T, 2, ksplit)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!aq || !as || !sorted_ids || !block_expert || !num_post_padded || !w2 || !w2_scale || !topk_w || !out_bf16 ||
      !ws)
    return MOE_ERR_NULL;
  const int64_t P = (int64_t)T * cfg->top_k;
  if (ws_bytes < split_bytes(cfg, T, 2, ksplit)) return MOE_ERR_WORKSPACE;
  const int32_t nb = max_blocks(P, cfg->num_experts, cfg->block_m);
  hipStream_t s = as_stream(stream);
  uint8_t* y = (uint8_t*)ws;
  moe::GemmArgs a = gemm2_args(cfg, T, aq, as, sorted_ids, block_expert, num_post_padded, w2, w2_scale, y, topk_w);
  return hip_status(gemm2_and_combine(cfg, T, a, nb, ksplit, out_bf16, ld_out, s));
}

moe_status_t moe_grouped_gemm2_combine(const moe_cfg_t* cfg, int32_t T, const void* aq, const void* as,
                                       const int32_t* sorted_ids, const int32_t* block_expert,
                                       const int32_t* num_post_padded, const void* w2, const void* w2_scale,
                                       const float* topk_w, void* out_bf16, int64_t ld_out, void* ws,
                                       size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  return moe_grouped_gemm2_combine_splitk(cfg, T, aq, as, sorted_ids, block_expert, num_post_padded, w2, w2_scale,
                                          topk_w, out_bf16, ld_out, plan_ksplit(cfg, T, 2), ws, ws_bytes, stream);
}

int32_t moe_decode_supported(const moe_cfg_t* cfg, int32_t T) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T) != MOE_OK || check_layout(cfg) != MOE_OK) return 0;
  return decode_takes(cfg, T) ? 1 : 0;
}

moe_status_t moe_decode_gemm1_swiglu(const moe_cfg_t* cfg, int32_t T, const void* xq, const void* xs,
                                     const int32_t* topk_ids, const void* w13, const void* w13_scale, float* a,
                                     void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if ((st = check_layout(cfg)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!decode_takes(cfg, T)) return MOE_ERR_UNSUPPORTED;
  if (!xq || !xs || !topk_ids || !w13 || !w13_scale || !a) return MOE_ERR_NULL;
  if ((uintptr_t)xq % 16 || (uintptr_t)xs % 4 || (uintptr_t)topk_ids % 4 || (uintptr_t)a % 16) return MOE_ERR_ALIGN;
  moe::DecodeArgs d = decode_args(cfg, T);
  d.ids = (int32_t*)topk_ids;  // read only
  d.xq = (const uint8_t*)xq;
  d.xs = xs;
  d.w13 = (const uint8_t*)w13;
  d.s13 = (const float*)w13_scale;
  d.a = a;
  return hip_status(moe::launch_decode_gemm1(cfg->quant_mode, d, as_stream(stream)));
}

moe_status_t moe_decode_gemm2_combine(const moe_cfg_t* cfg, int32_t T, const float* a, const int32_t* topk_ids,
                                      const float* topk_weights, const void* w2, const void* w2_scale,
                                      void* out_bf16, int64_t ld_out, void* aq, void* as, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, T)) != MOE_OK) return st;
  if ((st = check_layout(cfg)) != MOE_OK) return st;
  if (ld_out < cfg->pad.hidden) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!decode_takes(cfg, T)) return MOE_ERR_UNSUPPORTED;
  if (!a || !topk_ids || !topk_weights || !w2 || !w2_scale || !out_bf16 || !aq || !as) return MOE_ERR_NULL;
  if ((uintptr_t)a % 16 || (uintptr_t)aq % 8 || (uintptr_t)as % 4 || (uintptr_t)out_bf16 % 2) return MOE_ERR_ALIGN;
  moe::DecodeArgs d = decode_args(cfg, T);
  d.ids = (int32_t*)topk_ids;  // read only
  d.topk_w = (float*)topk_weights;
  d.a = (float*)a;
  d.w2 = (const uint8_t*)w2;
  d.s2 = (const float*)w2_scale;
  d.out = (uint16_t*)out_bf16;
  d.ld_out = ld_out;
  d.aq = (uint8_t*)aq;
  d.as = as;
  return hip_status(moe::launch_decode_gemm2(cfg->quant_mode, d, as_stream(stream)));
}

int32_t moe_plan_ksplit(const moe_cfg_t* cfg, int32_t T, int32_t which) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T) != MOE_OK || (which != 13 && which != 2)) return -1;
  return plan_ksplit(cfg, T, which);
}

size_t moe_splitk_bytes(const moe_cfg_t* cfg, int32_t T, int32_t which, int32_t ksplit) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T) != MOE_OK || (which != 13 && which != 2)) return 0;
  if (!ksplit_usable(cfg, T, which, ksplit)) return 0;
  return split_bytes(cfg, T, which, ksplit);
}

moe_status_t moe_forward(const moe_cfg_t* cfg, int32_t T, const void* x_bf16, int64_t ld_x, const float* router_logits,
                         const void* w13, const void* w13_scale, const void* w2, const void* w2_scale, void* out_bf16,
                         int64_t ld_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st =
      check_forward(cfg, T, x_bf16, ld_x, router_logits, w13, w13_scale, w2, w2_scale, out_bf16, ld_out);
  if (st != MOE_OK || T == 0) return st;
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < layout_for(cfg, T).total) return MOE_ERR_WORKSPACE;
  return forward_impl(cfg, T, x_bf16, ld_x, router_logits, w13, w13_scale, w2, w2_scale, out_bf16, ld_out, ws,
                      as_stream(stream));
}

moe_status_t moe_forward_noalloc(const moe_cfg_t* cfg, int32_t T, const void* x_bf16, int64_t ld_x,
                                 const float* router_logits, const void* w13, const void* w13_scale, const void* w2,
                                 const void* w2_scale, void* out_bf16, int64_t ld_out, void* stream) {
  moe_status_t st =
      check_forward(cfg, T, x_bf16, ld_x, router_logits, w13, w13_scale, w2, w2_scale, out_bf16, ld_out);
  if (st != MOE_OK || T == 0) return st;
  if (layout_for(cfg, T).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != MOE_OK) return st;
  return forward_impl(cfg, T, x_bf16, ld_x, router_logits, w13, w13_scale, w2, w2_scale, out_bf16, ld_out, ws,
                      as_stream(stream));
}

}  // extern "C"
