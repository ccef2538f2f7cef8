// Routing: top-k by logit with renormalised softmax weights, and the token-to-expert sort.
//
// Top-k follows the gate of gaudi-cookbook "fp8-moe-gather" (The fix): each token keeps its
// top_k experts; the weights are the softmax over the selected logits. Ties in the logit go
// to the lower expert id, so the result is unique and can be compared bit for bit.
//
// The sort groups pairs p = t*top_k + j by expert, ascending p within an expert (a stable
// counting sort). It is deterministic: ranks come from wave ballots, never from the order
// in which atomics land.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kMaxPerLane = MAX_EXPERTS / kWave;  // logits held per lane (E <= 1024)

// Is (la, ia) ahead of (lb, ib) in the order (descending logit, ascending id)?
__device__ __forceinline__ bool ahead(float la, int ia, float lb, int ib) {
  return la > lb || (la == lb && ia < ib);
}

// One wave per token. Each lane holds E/64 logits; k rounds of a wave-wide arg-max pick
// the experts in slot order. Lane j keeps slot j.
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights) {
  const int lane = lane_id();
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + kWave * i;
    const float l = e < E ? row[e] : 0.0f;
    // NaN is outside the contract; reading it as -inf keeps every selected id in [0, E)
    v[i] = l != l ? -__builtin_inff() : l;
  }
  uint32_t taken = 0;
  float my_l = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bl = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((taken >> i) & 1u) && ahead(v[i], e, bl, bi)) {
        bl = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ol = __shfl_xor(bl, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (ahead(ol, oi, bl, bi)) {
        bl = ol;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      my_l = bl;
      my_id = bi;
    }
  }
  // weights in double: exp(l_j - l_0) / sum over slots in slot order
  const double l0 = (double)__shfl(my_l, 0, kWave);
  const double ex = lane < k ? exp((double)my_l - l0) : 0.0;
  double tot = 0.0;
  for (int j = 0; j < k; ++j) tot += __shfl(ex, j, kWave);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    weights[(size_t)t * k + lane] = (float)(ex / tot);
  }
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Lanes of the wave whose 10-bit key equals this lane's key (E <= 1024).
__device__ __forceinline__ uint64_t match_lanes(int key, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit && valid);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// One wave: exclusive offsets over counts[0..E) into offs (LDS or global), returns total.
__device__ int wave_exclusive_offsets(const int* counts, int E, int* offs) {
  const int lane = lane_id();
  const int per = (E + kWave - 1) / kWave;
  const int lo = lane * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = lo + i;
    if (e < E) local += counts[e];
  }
  const int incl = wave_incl_scan(local);
  int run = incl - local;
  for (int i = 0; i < per; ++i) {
    const int e = lo + i;
    if (e < E) {
      offs[e] = run;
      run += counts[e];
    }
  }
  return __shfl(incl, kWave - 1, kWave);
}

// Active-expert list (ascending id), -1 past the last, per-expert tile offsets for a
// grouped GEMM with tile_m rows per tile. One wave.
__device__ void wave_active_list(const int* counts, int E, int slots, int32_t* act, int32_t* n_act,
                                 int tile_m, int32_t* tile_off) {
  const int lane = lane_id();
  const int per = (E + kWave - 1) / kWave;
  const int lo = lane * per;
  int nz = 0, tiles = 0;
  for (int i = 0; i < per; ++i) {
    const int e = lo + i;
    if (e < E) {
      nz += counts[e] > 0;
      if (tile_m > 0) tiles += (counts[e] + tile_m - 1) / tile_m;
    }
  }
  const int nz_incl = wave_incl_scan(nz);
  const int t_incl = wave_incl_scan(tiles);
  int s = nz_incl - nz, tr = t_incl - tiles;
  for (int i = 0; i < per; ++i) {
    const int e = lo + i;
    if (e < E) {
      if (counts[e] > 0) act[s++] = e;
      if (tile_m > 0) {
        tile_off[e] = tr;
        tr += (counts[e] + tile_m - 1) / tile_m;
      }
    }
  }
  const int total = __shfl(nz_incl, kWave - 1, kWave);
  const int total_tiles = __shfl(t_incl, kWave - 1, kWave);
  for (int i = total + lane; i < slots; i += kWave) act[i] = -1;
  if (lane == 0) {
    n_act[0] = total;
    if (tile_m > 0) tile_off[E] = total_tiles;
  }
}

// Whole sort in one workgroup, for small P. Counts in LDS, offsets by a wave scan, then one
// wave walks the pairs in rounds of 64 and places each by its rank among equal experts.
__global__ __launch_bounds__(1024) void sort_small_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted, int32_t* act,
                                                          int32_t* n_act, int slots, int tile_m,
                                                          int32_t* tile_off) {
  __shared__ int cnt[MAX_EXPERTS];
  __shared__ int off[MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) atomicAdd(&cnt[ids[p]], 1);
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  if (wave == 0) {
    wave_exclusive_offsets(cnt, E, off);
  } else if (wave == 1) {
    wave_active_list(cnt, E, slots, act, n_act, tile_m, tile_off);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    counts[e] = cnt[e];
    offsets[e] = off[e];
  }
  if (threadIdx.x == 0) offsets[E] = P;
  __syncthreads();
  if (wave == 0) {
    const int lane = lane_id();
    // off[] becomes the running insertion point of each expert
    for (int base = 0; base < P; base += kWave) {
      const int p = base + lane;
      const bool valid = p < P;
      const int e = valid ? ids[p] : 0;
      const uint64_t m = match_lanes(e, valid);
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      const int pos = valid ? off[e] + rank : 0;
      if (valid) sorted[pos] = p;
      // the highest lane of each group advances the insertion point
      const bool last = valid && (m >> lane) == 1ull;
      if (last) off[e] = pos + 1;
    }
  }
}

constexpr int kChunk = 256;  // pairs per workgroup in the multi-block sort

// Multi-block sort, pass 1: per-chunk expert histograms, chunk_counts[c * E + e].
__global__ __launch_bounds__(kWave) void sort_hist_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                          int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt[MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += kWave) cnt[e] = 0;
  __syncthreads();
  const int c = blockIdx.x;
  const int lo = c * kChunk, hi = min(P, lo + kChunk);
  for (int p = lo + threadIdx.x; p < hi; p += kWave) atomicAdd(&cnt[ids[p]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kWave) chunk_counts[(size_t)c * E + e] = cnt[e];
}

// Pass 2: one workgroup per expert turns its column of chunk counts into exclusive chunk
// bases (in place) and writes the expert's total.
__global__ __launch_bounds__(256) void sort_chunk_scan_kernel(int32_t* __restrict__ chunk_counts, int nchunks,
                                                              int E, int32_t* __restrict__ counts) {
  __shared__ int wsum[256 / kWave];
  const int e = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  int carry = 0;
  for (int base = 0; base < nchunks; base += blockDim.x) {
    const int c = base + threadIdx.x;
    const int v = c < nchunks ? chunk_counts[(size_t)c * E + e] : 0;
    const int incl = wave_incl_scan(v);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, tile_total = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) {
      if (w < wave) before += wsum[w];
      tile_total += wsum[w];
    }
    if (c < nchunks) chunk_counts[(size_t)c * E + e] = carry + before + incl - v;
    carry += tile_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// Pass 3: every chunk places its pairs at offsets[e] + chunk base + rank within the chunk.
// Workgroup 0 also writes offsets, the active list and the tile offsets.
__global__ __launch_bounds__(kWave) void sort_scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                             const int32_t* __restrict__ chunk_base,
                                                             const int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted, int32_t* act,
                                                             int32_t* n_act, int slots, int tile_m,
                                                             int32_t* tile_off) {
  __shared__ int cnt[MAX_EXPERTS];
  __shared__ int run[MAX_EXPERTS];
  const int lane = lane_id();
  const int c = blockIdx.x;
  for (int e = lane; e < E; e += kWave) cnt[e] = counts[e];
  __syncthreads();
  wave_exclusive_offsets(cnt, E, run);
  __syncthreads();
  if (c == 0) {
    for (int e = lane; e < E; e += kWave) offsets[e] = run[e];
    if (lane == 0) offsets[E] = P;
    wave_active_list(cnt, E, slots, act, n_act, tile_m, tile_off);
  }
  for (int e = lane; e < E; e += kWave) run[e] += chunk_base[(size_t)c * E + e];
  __syncthreads();
  const int lo = c * kChunk, hi = min(P, lo + kChunk);
  for (int base = lo; base < hi; base += kWave) {
    const int p = base + lane;
    const bool valid = p < hi;
    const int e = valid ? ids[p] : 0;
    const uint64_t m = match_lanes(e, valid);
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    const int pos = valid ? run[e] + rank : 0;
    if (valid) sorted[pos] = p;
    const bool last = valid && (m >> lane) == 1ull;
    if (last) run[e] = pos + 1;
  }
}

}  // namespace

size_t sort_scratch_bytes(int P, int E) {
  if (P <= kSmallSortPairs) return 0;
  const size_t nchunks = (size_t)(P + kChunk - 1) / kChunk;
  return nchunks * (size_t)E * sizeof(int32_t);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  const int waves_per_block = 4;
  const int blocks = (T + waves_per_block - 1) / waves_per_block;
  hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(waves_per_block * kWave), 0, s, logits, T, E, k,
                     ids, w);
  return hipGetLastError();
}

int sort_kernel_count(int P) { return P <= kSmallSortPairs ? 1 : 3; }

hipError_t launch_sort_stage(int stage, const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                             int32_t* sorted, int32_t* act, int32_t* n_act, int slots, int tile_m,
                             int32_t* tile_off, void* scratch, hipStream_t s) {
  if (P <= kSmallSortPairs) {
    hipLaunchKernelGGL(sort_small_kernel, dim3(1), dim3(1024), 0, s, ids, P, E, counts, offsets, sorted, act,
                       n_act, slots, tile_m, tile_off);
    return hipGetLastError();
  }
  const int nchunks = (P + kChunk - 1) / kChunk;
  int32_t* chunk = (int32_t*)scratch;
  switch (stage) {
    case 0:
      hipLaunchKernelGGL(sort_hist_kernel, dim3(nchunks), dim3(kWave), 0, s, ids, P, E, chunk);
      break;
    case 1:
      hipLaunchKernelGGL(sort_chunk_scan_kernel, dim3(E), dim3(256), 0, s, chunk, nchunks, E, counts);
      break;
    default:
      hipLaunchKernelGGL(sort_scatter_kernel, dim3(nchunks), dim3(kWave), 0, s, ids, P, E, chunk, counts, offsets,
                         sorted, act, n_act, slots, tile_m, tile_off);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
