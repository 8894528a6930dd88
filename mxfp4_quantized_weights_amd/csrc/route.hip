// Top-k routing and the padded stable expert permutation.
//
// Routing: FreeToken PR #270 "glm5_next: support GLM-5.3-Flash (hybrid KDA +
// DSA, mHC, NVFP4 expert offload)", Summary (288-expert top-8 routing; the
// fused router epilogue picks the same ids as a reference top-k).  Selection
// is on the raw logits, descending, ties to the lower expert id; weights are
// the softmax over the k selected logits.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_quant_rows.h"
#include "moe_route.h"

namespace moe {

// One wave per token.
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<VPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, nullptr);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  int vpl = (E + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 2)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 4)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 5)
    hipLaunchKernelGGL(route_topk_kernel<5>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (vpl <= 8)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Permute-align: stable counting sort of the pairs by expert, in one launch
// and with no scratch memory.  The tokens are cut into chunks, one per
// workgroup.  Every workgroup histograms ALL pairs, split into those before
// its chunk and those after it, so each one knows the global padded offsets
// and, per expert, how many of that expert's pairs come before its chunk:
// no workgroup waits for another.  Inside the chunk, RW ranking waves own
// consecutive token sub-ranges.  The pairs of expert e in increasing
// f = t*k + j are, when no token lists an expert twice (what top-k routing
// produces), the tokens that chose e in increasing t, so:
//   histogram: pairs outside the chunk by all waves (flat in f, coalesced),
//              the chunk's pairs per ranking wave (LDS atomics);
//   scan:      padded counts -> offsets; per-wave cursors = offset + pairs
//              before the chunk + pairs of earlier ranking waves;
//   fill:      padding sentinels, block experts and the tail past the last
//              segment, shared out over every wave of the grid;
//   rank:      each ranking wave walks its tokens 64 at a time (lane = token,
//              its k ids in registers); a 64-bit LDS mask per expert marks the
//              lanes that chose it, and a pair's position is its cursor +
//              popcount(mask & lanes below).
// If some token of a chunk lists an expert twice, that chunk's pairs are
// instead ranked with a ballot match loop over f order (same result, slower).
// The histogram of the pairs outside the chunk costs every workgroup O(P), so
// the number of chunks is capped.
// ---------------------------------------------------------------------------
constexpr int kMaxTopK = 16;
constexpr int kPermWaves = 16;      // waves per workgroup
constexpr int kPermRankWaves = 4;   // of which rank the chunk's pairs
constexpr int kPermMaxChunks = 256;

template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch /* [NW] */, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int tw = scratch[w];
    if (w < wave) base += tw;
    total += tw;
  }
  __syncthreads();
  return base + incl - v;
}

// LDS written by some lanes of a wave is read by other lanes of the same
// wave: a wave's LDS operations complete in order, so ordering the compiler's
// view is all that is needed.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The work of one workgroup: chunk `chunk` of `nchunks` (token chunks of Tc).
// `ids` may point to global memory or to LDS.  perm_smem: permute_smem_bytes.
template <int NW, int RW>
__device__ __forceinline__ void permute_align_body(const int32_t* ids, int T, int k, int E, int BM, int nb, int Tc,
                                                   int chunk, int nchunks, int32_t* __restrict__ sorted_ids,
                                                   int32_t* __restrict__ block_expert,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ npp,
                                                   unsigned char* perm_smem) {
  constexpr int NT = 64 * NW;
  static_assert(NT >= 1024, "one thread per expert in the scan");
  static_assert(RW <= NW, "ranking waves are a subset");
  int32_t* before = (int32_t*)perm_smem;          // [E] pairs before the chunk; then the expert's pair count
  int32_t* after = before + E;                    // [E] pairs after the chunk; then the segment offset
  int32_t* cur = after + E;                       // [RW][E] per-wave chunk counts; then cursors
  uint32_t* mask = (uint32_t*)(cur + RW * E);     // [RW][E][2] lane masks (lo, hi)
  int32_t* scratch = (int32_t*)(mask + RW * E * 2);  // [NW] scan partials + duplicate flag
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = T * k;
  const int tb = min(T, chunk * Tc), te = min(T, tb + Tc);
  const int fb = tb * k, fe = te * k;
  const int Tw = (Tc + RW - 1) / RW;
  const int w_begin = min(te, tb + wave * Tw), w_end = min(te, w_begin + Tw);  // used by ranking waves

  for (int i = tid; i < (2 + 3 * RW) * E; i += NT) before[i] = 0;
  if (tid == 0) scratch[NW] = 0;
  __syncthreads();

  // pairs outside the chunk, flat in f, U loads in flight per thread
  constexpr int U = 16;
  const int n_out = P - (fe - fb);
  for (int base = tid; base < n_out; base += NT * U) {
    int ev[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT;
      ev[u] = (i < n_out) ? ids[i < fb ? i : i + (fe - fb)] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = ev[u];
      if (e >= 0 && e < E) atomicAdd((base + u * NT < fb) ? &before[e] : &after[e], 1);
    }
  }
  // the chunk's pairs, per ranking wave; detect a token that lists an expert twice
  bool dup = false;
  if (wave < RW) {
    for (int t = w_begin + lane; t < w_end; t += 64) {
      int ex[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) ex[j] = (j < k) ? ids[(size_t)t * k + j] : -1;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        const int e = ex[j];
        if (j >= k || e < 0 || e >= E) continue;
        atomicAdd(&cur[wave * E + e], 1);
#pragma unroll
        for (int j2 = 0; j2 < j; ++j2) dup |= (ex[j2] == e);
      }
    }
  }
  if (dup) scratch[NW] = 1;
  __syncthreads();
  const bool any_dup = scratch[NW] != 0;

  // scan of padded counts: thread e owns expert e (E <= NT)
  const int e_own = tid;
  int cnt = 0;
  if (e_own < E) {
    cnt = before[e_own] + after[e_own];
#pragma unroll
    for (int w = 0; w < RW; ++w) cnt += cur[w * E + e_own];
  }
  const int pc = ((cnt + BM - 1) / BM) * BM;
  int total;
  const int off = block_exclusive_scan<NW>(pc, scratch, total);
  if (e_own < E) {
    int c0 = off + before[e_own];
#pragma unroll
    for (int w = 0; w < RW; ++w) {
      const int c = cur[w * E + e_own];
      cur[w * E + e_own] = c0;  // only this thread touches expert e_own
      c0 += c;
    }
    before[e_own] = cnt;
    after[e_own] = off;
    if (chunk == 0) offsets[e_own] = off;
  }
  if (chunk == 0 && tid == 0) {
    offsets[E] = total;
    *npp = total;
  }
  __syncthreads();

  // padding sentinels and block experts, one expert per wave of the grid
  const int gw = chunk * NW + wave, n_waves = nchunks * NW;
  for (int e = gw; e < E; e += n_waves) {
    const int c = before[e], o = after[e], p = ((c + BM - 1) / BM) * BM;
    for (int r = o + c + lane; r < o + p; r += 64) sorted_ids[r] = P;
    for (int b = o / BM + lane; b < (o + p) / BM; b += 64) block_expert[b] = e;
  }
  const int gt = chunk * NT + tid, n_threads = nchunks * NT;
  for (int r = total + gt; r < nb * BM; r += n_threads) sorted_ids[r] = P;
  for (int b = total / BM + gt; b < nb; b += n_threads) block_expert[b] = -1;

  if (wave >= RW) return;  // no workgroup barrier below
  int32_t* wcur = cur + wave * E;
  uint32_t* wmask = mask + wave * E * 2;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (!any_dup) {
    for (int t0 = w_begin; t0 < w_end; t0 += 64) {
      const int t = t0 + lane;
      const bool live = t < w_end;
      int ex[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        int e = (live && j < k) ? ids[(size_t)t * k + j] : -1;
        ex[j] = (e >= 0 && e < E) ? e : -1;
      }
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (ex[j] >= 0) atomicOr(&wmask[ex[j] * 2 + (lane >> 5)], 1u << (lane & 31));
      wave_lds_sync();
      uint64_t m[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        m[j] = 0;
        if (ex[j] >= 0) {
          const uint2 mm = *(const uint2*)&wmask[ex[j] * 2];
          m[j] = (uint64_t)mm.x | ((uint64_t)mm.y << 32);
          sorted_ids[wcur[ex[j]] + __popcll(m[j] & lt_mask)] = t * k + j;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (ex[j] >= 0 && (m[j] & lt_mask) == 0) {  // the expert's first lane
          wcur[ex[j]] += __popcll(m[j]);
          *(uint2*)&wmask[ex[j] * 2] = make_uint2(0u, 0u);
        }
      }
      wave_lds_sync();
    }
  } else {
    // general order: lane = pair, in f order over the wave's token range
    const int f_begin = w_begin * k, f_end = w_end * k;
    for (int f0 = f_begin; f0 < f_end; f0 += 64) {
      const int f = f0 + lane;
      const int e = (f < f_end) ? ids[f] : -1;
      const bool valid = e >= 0 && e < E;
      uint64_t active = __ballot(valid);
      int rank = 0;
      bool leader = false;
      int cnt_leader = 0;
      while (active) {
        const int ld = __ffsll((unsigned long long)active) - 1;
        const int le = __builtin_amdgcn_readlane(e, ld);
        const uint64_t mm = __ballot(valid && e == le);
        if (valid && e == le) rank = __popcll(mm & lt_mask);
        if (lane == ld) {
          leader = true;
          cnt_leader = __popcll(mm);
        }
        active &= ~mm;
      }
      if (valid) sorted_ids[wcur[e] + rank] = f;
      wave_lds_sync();
      if (leader) wcur[e] += cnt_leader;
      wave_lds_sync();
    }
  }
}

inline size_t permute_smem_bytes(int E) { return (size_t)(2 + 3 * kPermRankWaves) * E * 4 + (kPermWaves + 1) * 4; }

template <int NW, int RW>
__global__ __launch_bounds__(64 * NW) void permute_align_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                                int BM, int nb, int Tc,
                                                                int32_t* __restrict__ sorted_ids,
                                                                int32_t* __restrict__ block_expert,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ npp) {
  extern __shared__ __align__(16) unsigned char perm_smem[];
  permute_align_body<NW, RW>(ids, T, k, E, BM, nb, Tc, blockIdx.x, gridDim.x, sorted_ids, block_expert, offsets, npp,
                             perm_smem);
}

hipError_t launch_permute_align(const int32_t* ids, int T, int k, int E, int block_m, int nb, int32_t* sorted_ids,
                                int32_t* block_expert, int32_t* offsets, int32_t* npp, hipStream_t s) {
  constexpr int NW = kPermWaves, RW = kPermRankWaves;
  // one chunk per 64 tokens of each ranking wave, at most kPermMaxChunks
  int chunks = (T + RW * 64 - 1) / (RW * 64);
  chunks = chunks < 1 ? 1 : (chunks > kPermMaxChunks ? kPermMaxChunks : chunks);
  const int Tc = (T + chunks - 1) / chunks;
  const size_t smem = permute_smem_bytes(E);  // <= 57412 B for E <= 1024
  hipLaunchKernelGGL((permute_align_kernel<NW, RW>), dim3(chunks), dim3(64 * NW), smem, s, ids, T, k, E, block_m, nb,
                     Tc, sorted_ids, block_expert, offsets, npp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Front end in fewer launches than three.
//   route_quant_kernel (any batch): workgroups 0 .. nr-1 route 4 tokens each
//             (one wave per token, route_token), the others quantise the
//             rows of x; the two parts share no data.  Larger batches then
//             run permute_align_kernel.
//   front_small_kernel (T <= 16, one launch): workgroup 0 (16 waves) routes
//             every token, keeping the ids in LDS as well, then builds the
//             permutation from them (permute_small); the other workgroups
//             quantise the rows of x.  Routing runs on one CU here, one token
//             per wave; with more tokens per wave it takes longer than the
//             second launch saves, so 17 .. 64 tokens run route_quant_kernel
//             and then permute_small_kernel.
//   permute_small: routing never gives a token the same expert twice, so one
//             64-bit LDS word per expert marks the tokens that chose it
//             (T <= 64); a pair's stable rank in its expert's segment is the
//             number of marked tokens below its own, and the expert's count
//             the number of marks.  A block scan of the padded counts gives
//             the offsets; each expert's thread writes its padding sentinels
//             and block ids, then every pair its sorted position (the layout
//             of permute_align_kernel).
// ---------------------------------------------------------------------------
constexpr int kSmallT = 64;

template <int VPL, int MODE>
__global__ __launch_bounds__(256) void route_quant_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ w, int nr,
                                                          const void* __restrict__ x, int H, int64_t ld_x, int Hp,
                                                          uint8_t* __restrict__ xq, void* __restrict__ xs, int vec) {
  const int wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < nr) {
    const int t = blockIdx.x * 4 + wave;
    if (t < T) route_token<VPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, nullptr);
    return;
  }
  const int64_t gw = (int64_t)(blockIdx.x - nr) * 4 + wave, nw = (int64_t)(gridDim.x - nr) * 4;
  // two units' loads in flight per lane: large batches take two or more
  // passes of the grid
  if (vec)
    quant_rows_body<true, true, MODE, 2>(x, T, H, ld_x, Hp, xq, xs, gw, nw);
  else
    quant_rows_body<true, false, MODE>(x, T, H, ld_x, Hp, xq, xs, gw, nw);
}

// The permutation of T <= 64 tokens' pairs by one 1024-thread workgroup;
// ids may point to LDS (visible to the whole workgroup on entry).
__device__ __forceinline__ void permute_small(const int32_t* ids, int T, int k, int E, int BM, int nb,
                                              int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ npp) {
  constexpr int NW = 16;
  __shared__ uint64_t sel[1024];     // tokens that chose expert e
  __shared__ int32_t seg[1024];      // segment offset of expert e
  __shared__ int32_t scan_tmp[NW];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) sel[e] = 0;
  const int P = T * k;
  // thread f holds pair f (P <= 64 * 16)
  const int my_e = tid < P ? ids[tid] : -1;
  const int t = tid < P ? tid / k : 0;
  __syncthreads();
  if (my_e >= 0 && my_e < E) atomicOr((unsigned long long*)&sel[my_e], 1ull << t);
  __syncthreads();
  int cnt = 0;
  if (tid < E) cnt = __popcll(sel[tid]);
  const int pc = ((cnt + BM - 1) / BM) * BM;
  int total;
  const int off = block_exclusive_scan<NW>(pc, scan_tmp, total);
  if (tid < E) {
    seg[tid] = off;
    offsets[tid] = off;
    // the expert's padding sentinels and block ids, from its own count
    for (int r = off + cnt; r < off + pc; ++r) sorted_ids[r] = P;
    for (int b = off / BM; b < (off + pc) / BM; ++b) block_expert[b] = tid;
  }
  if (tid == 0) {
    offsets[E] = total;
    *npp = total;
  }
  // the tail past the last segment
  for (int r = total + tid; r < nb * BM; r += 1024) sorted_ids[r] = P;
  for (int b = total / BM + tid; b < nb; b += 1024) block_expert[b] = -1;
  __syncthreads();
  if (my_e >= 0 && my_e < E) {
    const uint64_t below = (t == 0) ? 0ull : (~0ull >> (64 - t));
    sorted_ids[seg[my_e] + __popcll(sel[my_e] & below)] = tid;
  }
}

__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                             int BM, int nb, int32_t* __restrict__ sorted_ids,
                                                             int32_t* __restrict__ block_expert,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ npp) {
  permute_small(ids, T, k, E, BM, nb, sorted_ids, block_expert, offsets, npp);
}

constexpr int kOneLaunchT = 16;

template <int VPL, int MODE>
__global__ __launch_bounds__(1024) void front_small_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                           int32_t* __restrict__ ids, float* __restrict__ w, int BM,
                                                           int nb, int32_t* __restrict__ sorted_ids,
                                                           int32_t* __restrict__ block_expert,
                                                           int32_t* __restrict__ offsets, int32_t* __restrict__ npp,
                                                           const void* __restrict__ x, int H, int64_t ld_x, int Hp,
                                                           uint8_t* __restrict__ xq, void* __restrict__ xs, int vec) {
  const int wave = threadIdx.x >> 6;
  if (blockIdx.x == 0) {
    __shared__ int32_t ids_lds[kOneLaunchT * kMaxTopK];
    for (int t = wave; t < T; t += 16)
      route_token<VPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, ids_lds + t * k);
    __syncthreads();
    permute_small(ids_lds, T, k, E, BM, nb, sorted_ids, block_expert, offsets, npp);
    return;
  }
  const int64_t gw = (int64_t)(blockIdx.x - 1) * 16 + wave, nw = (int64_t)(gridDim.x - 1) * 16;
  if (vec)
    quant_rows_body<true, true, MODE>(x, T, H, ld_x, Hp, xq, xs, gw, nw);
  else
    quant_rows_body<true, false, MODE>(x, T, H, ld_x, Hp, xq, xs, gw, nw);
}

template <int VPL>
static void launch_route_quant(int mode, dim3 grid, int nr, hipStream_t s, const float* logits, int T, int E, int k,
                               int32_t* ids, float* w, const void* x, int H, int64_t ld_x, int Hp, void* xq,
                               void* xs, int vec) {
  uint8_t* q = (uint8_t*)xq;
  if (mode == kQuantFp8)
    hipLaunchKernelGGL((route_quant_kernel<VPL, kQuantFp8>), grid, dim3(256), 0, s, logits, T, E, k, ids, w, nr, x,
                       H, ld_x, Hp, q, xs, vec);
  else if (mode == kQuantFp8E8)
    hipLaunchKernelGGL((route_quant_kernel<VPL, kQuantFp8E8>), grid, dim3(256), 0, s, logits, T, E, k, ids, w, nr, x,
                       H, ld_x, Hp, q, xs, vec);
  else
    hipLaunchKernelGGL((route_quant_kernel<VPL, kQuantMx>), grid, dim3(256), 0, s, logits, T, E, k, ids, w, nr, x, H,
                       ld_x, Hp, q, xs, vec);
}

bool front_small_ok(int T, int E, int k) { return T >= 1 && T <= kSmallT && E <= 1024 && k <= kMaxTopK; }

hipError_t launch_route_and_quant(const float* logits, int T, int E, int k, int32_t* ids, float* w, const void* x_bf16,
                                  int H, int64_t ld_x, int Hp, int mode, void* xq, void* xs, hipStream_t s) {
  const int nr = (T + 3) / 4;
  const int64_t units = (int64_t)T * (Hp / 128);
  int64_t qwg = (units + 15) / 16;  // 16 units per workgroup
  if (qwg > 4096) qwg = 4096;
  const dim3 grid((unsigned)(nr + qwg));
  const int vec = ((uintptr_t)x_bf16 % 16 == 0) && ((ld_x * 2) % 16 == 0);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)
    launch_route_quant<1>(mode, grid, nr, s, logits, T, E, k, ids, w, x_bf16, H, ld_x, Hp, xq, xs, vec);
  else if (vpl <= 5)
    launch_route_quant<5>(mode, grid, nr, s, logits, T, E, k, ids, w, x_bf16, H, ld_x, Hp, xq, xs, vec);
  else
    launch_route_quant<16>(mode, grid, nr, s, logits, T, E, k, ids, w, x_bf16, H, ld_x, Hp, xq, xs, vec);
  return hipGetLastError();
}

template <int VPL>
static void launch_front_small_vpl(int mode, dim3 grid, hipStream_t s, const float* logits, int T, int E, int k,
                                   int32_t* ids, float* w, int BM, int nb, int32_t* sorted_ids,
                                   int32_t* block_expert, int32_t* offsets, int32_t* npp, const void* x, int H,
                                   int64_t ld_x, int Hp, void* xq, void* xs, int vec) {
  uint8_t* q = (uint8_t*)xq;
  if (mode == kQuantFp8)
    hipLaunchKernelGGL((front_small_kernel<VPL, kQuantFp8>), grid, dim3(1024), 0, s, logits, T, E, k, ids, w, BM, nb,
                       sorted_ids, block_expert, offsets, npp, x, H, ld_x, Hp, q, xs, vec);
  else if (mode == kQuantFp8E8)
    hipLaunchKernelGGL((front_small_kernel<VPL, kQuantFp8E8>), grid, dim3(1024), 0, s, logits, T, E, k, ids, w, BM,
                       nb, sorted_ids, block_expert, offsets, npp, x, H, ld_x, Hp, q, xs, vec);
  else
    hipLaunchKernelGGL((front_small_kernel<VPL, kQuantMx>), grid, dim3(1024), 0, s, logits, T, E, k, ids, w, BM, nb,
                       sorted_ids, block_expert, offsets, npp, x, H, ld_x, Hp, q, xs, vec);
}

hipError_t launch_front_small(const float* logits, int T, int E, int k, int32_t* ids, float* w, int block_m, int nb,
                              int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets, int32_t* npp,
                              const void* x_bf16, int H, int64_t ld_x, int Hp, int mode, void* xq, void* xs,
                              hipStream_t s) {
  if (T > kOneLaunchT) {
    hipError_t e = launch_route_and_quant(logits, T, E, k, ids, w, x_bf16, H, ld_x, Hp, mode, xq, xs, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, s, ids, T, k, E, block_m, nb, sorted_ids,
                       block_expert, offsets, npp);
    return hipGetLastError();
  }
  // workgroup 0 routes and permutes; 1 + ceil(units / 64) workgroups in all
  // (16 waves of 4 quantisation units each)
  const int64_t units = (int64_t)T * (Hp / 128);
  const dim3 grid((unsigned)(1 + (units + 63) / 64));
  const int vec = ((uintptr_t)x_bf16 % 16 == 0) && ((ld_x * 2) % 16 == 0);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)
    launch_front_small_vpl<1>(mode, grid, s, logits, T, E, k, ids, w, block_m, nb, sorted_ids, block_expert, offsets,
                              npp, x_bf16, H, ld_x, Hp, xq, xs, vec);
  else if (vpl <= 5)
    launch_front_small_vpl<5>(mode, grid, s, logits, T, E, k, ids, w, block_m, nb, sorted_ids, block_expert, offsets,
                              npp, x_bf16, H, ld_x, Hp, xq, xs, vec);
  else
    launch_front_small_vpl<16>(mode, grid, s, logits, T, E, k, ids, w, block_m, nb, sorted_ids, block_expert,
                               offsets, npp, x_bf16, H, ld_x, Hp, xq, xs, vec);
  return hipGetLastError();
}

}  // namespace moe
