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

namespace moe {

// (value, id) is better than (ov, oid): larger value, ties to the lower id.
__device__ __forceinline__ bool better(float ov, int oid, float v, int id) {
  return ov > v || (ov == v && oid < id);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& id) {
  // lanes outside ROW_MASK keep their own value (old = src), which is a no-op
  float ov = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
  int oid = __builtin_amdgcn_update_dpp(id, id, CTRL, ROW_MASK, 0xF, false);
  if (better(ov, oid, v, id)) {
    v = ov;
    id = oid;
  }
}

// Wave-wide argmax with DPP row operations: quad swaps (xor 1, xor 2), half
// and full row mirrors make every 16-lane row uniform, row broadcasts of
// lanes 15 and 31 fold the rows into lane 63, which is read back uniformly.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  argmax_step<0xB1, 0xF>(v, id);   // quad_perm [1,0,3,2]
  argmax_step<0x4E, 0xF>(v, id);   // quad_perm [2,3,0,1]
  argmax_step<0x141, 0xF>(v, id);  // row_half_mirror
  argmax_step<0x140, 0xF>(v, id);  // row_mirror
  argmax_step<0x142, 0xA>(v, id);  // row_bcast:15 into rows 1, 3
  argmax_step<0x143, 0xC>(v, id);  // row_bcast:31 into rows 2, 3
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  id = __builtin_amdgcn_readlane(id, 63);
}

// One wave per token.  Each lane holds the logits of experts lane + 64*i;
// k rounds of a wave-wide argmax pick the experts in slot order.  NaN logits
// compare as -inf.  The softmax denominator is summed in slot order.
template <int VPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[VPL];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    float x = (e < E) ? row[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;
    if (e < E) avail |= 1u << i;
  }
  float my_v = -INFINITY;
  int my_e = 0;
  float lmax = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + 64 * i;
      if (((avail >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
    wave_argmax(bv, be);
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (j == 0) lmax = bv;
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float d = (my_v == lmax) ? 0.0f : (my_v - lmax);
  const float ex = (lane < k) ? expf(d) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = ex / sum;
  }
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

template <int NW, int RW>
__global__ __launch_bounds__(64 * NW) void permute_align_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                                int BM, int nb, int Tc,
                                                                int32_t* __restrict__ sorted_ids,
                                                                int32_t* __restrict__ block_expert,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ npp) {
  constexpr int NT = 64 * NW;
  static_assert(NT >= 1024, "one thread per expert in the scan");
  static_assert(RW <= NW, "ranking waves are a subset");
  extern __shared__ __align__(16) unsigned char perm_smem[];
  int32_t* before = (int32_t*)perm_smem;          // [E] pairs before the chunk; then the expert's pair count
  int32_t* after = before + E;                    // [E] pairs after the chunk; then the segment offset
  int32_t* cur = after + E;                       // [RW][E] per-wave chunk counts; then cursors
  uint32_t* mask = (uint32_t*)(cur + RW * E);     // [RW][E][2] lane masks (lo, hi)
  int32_t* scratch = (int32_t*)(mask + RW * E * 2);  // [NW] scan partials + duplicate flag
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = T * k;
  const int tb = min(T, (int)blockIdx.x * Tc), te = min(T, tb + Tc);
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
    if (blockIdx.x == 0) offsets[e_own] = off;
  }
  if (blockIdx.x == 0 && tid == 0) {
    offsets[E] = total;
    *npp = total;
  }
  __syncthreads();

  // padding sentinels and block experts, one expert per wave of the grid
  const int gw = blockIdx.x * NW + wave, n_waves = gridDim.x * NW;
  for (int e = gw; e < E; e += n_waves) {
    const int c = before[e], o = after[e], p = ((c + BM - 1) / BM) * BM;
    for (int r = o + c + lane; r < o + p; r += 64) sorted_ids[r] = P;
    for (int b = o / BM + lane; b < (o + p) / BM; b += 64) block_expert[b] = e;
  }
  const int gt = blockIdx.x * NT + tid, n_threads = gridDim.x * NT;
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

hipError_t launch_permute_align(const int32_t* ids, int T, int k, int E, int block_m, int nb, int32_t* sorted_ids,
                                int32_t* block_expert, int32_t* offsets, int32_t* npp, hipStream_t s) {
  constexpr int NW = kPermWaves, RW = kPermRankWaves;
  // one chunk per 64 tokens of each ranking wave, at most kPermMaxChunks
  int chunks = (T + RW * 64 - 1) / (RW * 64);
  chunks = chunks < 1 ? 1 : (chunks > kPermMaxChunks ? kPermMaxChunks : chunks);
  const int Tc = (T + chunks - 1) / chunks;
  const size_t smem = (size_t)(2 + 3 * RW) * E * 4 + (NW + 1) * 4;  // <= 57412 B for E <= 1024
  hipLaunchKernelGGL((permute_align_kernel<NW, RW>), dim3(chunks), dim3(64 * NW), smem, s, ids, T, k, E, block_m, nb,
                     Tc, sorted_ids, block_expert, offsets, npp);
  return hipGetLastError();
}

}  // namespace moe
