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
#include "quant.hpp"
#include "topk.hpp"

namespace moe {

namespace {

// One wave per token.
template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ __align__(16) uint64_t s_cand[256 / kWave][kWave];
  const int lane = lane_id();
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
  if (t >= T) return;
  int id;
  float w;
  wave_topk<PER>(logits + (size_t)t * E, E, k, s_cand[threadIdx.x / kWave], id, w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    weights[(size_t)t * k + lane] = w;
  }
}

// The same, and the token's row of x (bf16, H columns) quantised to e4m3 with one scale
// per row, codes ostride bytes apart (the MFMA path's activations). The logits are read
// first, then the row, and the selection waits for the logits only, so the row's reads are
// in flight while the experts are chosen.
template <int PER, int IT>
__global__ __launch_bounds__(256) void route_topk_quant_kernel(const float* __restrict__ logits,
                                                               const uint16_t* __restrict__ x, int T, int E, int k,
                                                               int H, int ostride, int32_t* __restrict__ ids,
                                                               float* __restrict__ weights,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales) {
  __shared__ __align__(16) uint64_t s_cand[256 / kWave][kWave];
  const int lane = lane_id();
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
  if (t >= T) return;
  float f[PER];
  wave_topk_load<PER, false>(logits + (size_t)t * E, E, f);
  u32x4 v[IT];
  quant_row_bf16_load<IT>(x, t, H, v);
  int id;
  float l;
  wave_topk_select_lds<PER>(f, E, k, s_cand[threadIdx.x / kWave], id, l);
  const float w = wave_topk_weight(l, k);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    weights[(size_t)t * k + lane] = w;
  }
  quant_row_bf16_store<IT>(v, t, H, ostride, codes, scales);
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

// Routing and the whole sort in one workgroup, for P <= kSmallSortPairs. ROUTE: 16 waves
// route the tokens (each reading its next token's logits while it selects the current one's
// experts); otherwise the ids come from route_topk_kernel, which spreads the tokens over many
// CUs (the selection of many tokens on the one CU of this workgroup is bound by its VALU).
// Up to kWavePlacePairs pairs: counts by LDS atomics, offsets by a wave scan, and one wave
// walks the pairs in rounds of 64, placing each by its rank among equal experts. More: the
// counting sort of the multi-block kernels, in LDS: wave w takes the pairs of chunk w
// (consecutive, in rounds of 64), counts them per expert by ballots, a scan over the waves
// gives each (wave, expert) its base, a wave scan the expert offsets, and each wave places
// its pairs by their rank among equal experts. Both are stable, and no atomics decide an
// order.
constexpr int kWavePlacePairs = 512;  // up to here one wave places all pairs

template <int PER, bool ROUTE>
__global__ __launch_bounds__(1024) void route_plan_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ weights,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted, int32_t* act,
                                                          int32_t* n_act, int slots, int tile_m,
                                                          int32_t* tile_off) {
  constexpr int NW = 1024 / kWave;
  __shared__ int cnt[MAX_EXPERTS];
  __shared__ int off[MAX_EXPERTS];
  __shared__ int sid[kSmallSortPairs];
  __shared__ int wcnt[NW][MAX_EXPERTS];  // pairs of wave w's chunk per expert, then their base
  __shared__ __align__(16) uint64_t s_cand[ROUTE ? 1024 / kWave : 1][kWave];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int nwaves = blockDim.x / kWave;
  const int P = T * k;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  if constexpr (!ROUTE) {
    for (int p = threadIdx.x; p < P; p += blockDim.x) sid[p] = ids[p];
  } else {
  // a wave's tokens are t = wave, wave + nwaves, ...; the next token's logits are read while
  // the current one is selected (a wave with no token reads the last row and drops it)
  float fcur[PER], fnext[PER];
  wave_topk_load<PER>(logits + (size_t)min(wave, T - 1) * E, E, fcur);
  for (int t = wave; t < T; t += nwaves) {
    wave_topk_load<PER, false>(logits + (size_t)min(t + nwaves, T - 1) * E, E, fnext);
    int id;
    float l;
    wave_topk_select_lds<PER>(fcur, E, k, s_cand[wave], id, l);
    const float w = wave_topk_weight(l, k);
#pragma unroll
    for (int i = 0; i < PER; ++i) fcur[i] = fnext[i];
    if (lane < k) {
      sid[t * k + lane] = id;
      ids[(size_t)t * k + lane] = id;
      weights[(size_t)t * k + lane] = w;
    }
  }
  }
  if (P <= kWavePlacePairs) {
    // few pairs: counts by LDS atomics, one wave places them all in rounds of 64
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += blockDim.x) atomicAdd(&cnt[sid[p]], 1);
    __syncthreads();
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
      // off[] becomes the running insertion point of each expert
      for (int base = 0; base < P; base += kWave) {
        const int p = base + lane;
        const bool valid = p < P;
        const int e = valid ? sid[p] : 0;
        const uint64_t m = match_lanes(e, valid);
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        const int pos = valid ? off[e] + rank : 0;
        if (valid) sorted[pos] = p;
        // the highest lane of each group advances the insertion point
        const bool last = valid && (m >> lane) == 1ull;
        if (last) off[e] = pos + 1;
      }
    }
    return;
  }
  for (int i = threadIdx.x; i < NW * E; i += blockDim.x) wcnt[i / E][i % E] = 0;
  __syncthreads();
  // wave w's chunk: pairs [w * C, min(P, (w + 1) * C)), C a multiple of 64
  const int C = (P + NW * kWave - 1) / (NW * kWave) * kWave;
  const int lo = wave * C, hi = min(P, lo + C);
  for (int base = lo; base < hi; base += kWave) {
    const int p = base + lane;
    const bool valid = p < hi;
    const int e = valid ? sid[p] : 0;
    const uint64_t m = match_lanes(e, valid);
    // the highest lane of each group adds the group's size
    if (valid && (m >> lane) == 1ull) wcnt[wave][e] += __popcll(m);
  }
  __syncthreads();
  // per expert: the total, and each wave's base within the expert (exclusive over waves)
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = wcnt[w][e];
      wcnt[w][e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
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
  // wcnt[wave][] becomes this wave's running insertion point of each expert (only this wave
  // reads or writes its row from here on)
  for (int e = lane; e < E; e += kWave) wcnt[wave][e] += off[e];
  for (int base = lo; base < hi; base += kWave) {
    const int p = base + lane;
    const bool valid = p < hi;
    const int e = valid ? sid[p] : 0;
    const uint64_t m = match_lanes(e, valid);
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    const int pos = valid ? wcnt[wave][e] + rank : 0;
    if (valid) sorted[pos] = p;
    // the highest lane of each group advances the insertion point
    const bool last = valid && (m >> lane) == 1ull;
    if (last) wcnt[wave][e] = pos + 1;
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

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  const int waves_per_block = 4;
  const int blocks = (T + waves_per_block - 1) / waves_per_block;
  MOE_TOPK_DISPATCH(E, launch_kernel((route_topk_kernel<PER>), dim3(blocks), dim3(waves_per_block * kWave), 0,
                                          s, logits, T, E, k, ids, w));
  return hipGetLastError();
}

// Up to this many tokens (one per wave of the plan kernel) are routed inside it; more go to
// route_topk_kernel first.
constexpr int kPlanRouteTokens = 16;

template <int PER>
static void launch_route_topk_quant_per(int it, dim3 grid, const float* logits, const uint16_t* x, int T, int E,
                                        int k, int H, int ostride, int32_t* ids, float* w, uint8_t* codes,
                                        float* scales, hipStream_t s) {
#define MOE_RTQ(IT)                                                                                            \
  launch_kernel((route_topk_quant_kernel<PER, IT>), grid, dim3(256), 0, s, logits, x, T, E, k, H, ostride, ids, \
                w, codes, scales)
  if (it <= 1) MOE_RTQ(1);
  else if (it <= 2) MOE_RTQ(2);
  else if (it <= 4) MOE_RTQ(4);
  else if (it <= 8) MOE_RTQ(8);
  else MOE_RTQ(16);
#undef MOE_RTQ
}

bool route_topk_first(int T, int k) { return T * k > kSmallSortPairs || T > kPlanRouteTokens; }

hipError_t launch_route_topk_quant(const float* logits, const uint16_t* x, int T, int E, int k, int H, int ostride,
                                   int32_t* ids, float* w, uint8_t* codes, float* scales, hipStream_t s) {
  const int it = (H + kWave * 8 - 1) / (kWave * 8);
  if (H <= 0 || H % 8 != 0 || it > 16 || ostride < H || ostride - H >= kWave * 8 || ostride % 8 != 0)
    return hipErrorInvalidValue;
  const dim3 grid((T + 3) / 4);
  MOE_TOPK_DISPATCH(E, launch_route_topk_quant_per<PER>(it, grid, logits, x, T, E, k, H, ostride, ids, w, codes,
                                                        scales, s));
  return hipGetLastError();
}

int route_kernel_count(int T, int k) {
  const int P = T * k;
  if (P <= kSmallSortPairs) return T <= kPlanRouteTokens ? 1 : 2;
  return 4;
}

hipError_t launch_route_stage(int stage, const float* logits, int T, int E, int k, int32_t* ids, float* w,
                              int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* act, int32_t* n_act,
                              int slots, int tile_m, int32_t* tile_off, void* scratch, hipStream_t s) {
  const int P = T * k;
  if (P <= kSmallSortPairs) {
    if (T <= kPlanRouteTokens) {
      MOE_TOPK_DISPATCH(E, launch_kernel((route_plan_kernel<PER, true>), dim3(1), dim3(1024), 0, s, logits, T, E,
                                         k, ids, w, counts, offsets, sorted, act, n_act, slots, tile_m, tile_off));
      return hipGetLastError();
    }
    if (stage == 0) return launch_route_topk(logits, T, E, k, ids, w, s);
    launch_kernel((route_plan_kernel<1, false>), dim3(1), dim3(1024), 0, s, logits, T, E, k, ids, w, counts,
                  offsets, sorted, act, n_act, slots, tile_m, tile_off);
    return hipGetLastError();
  }
  const int nchunks = (P + kChunk - 1) / kChunk;
  int32_t* chunk = (int32_t*)scratch;
  switch (stage) {
    case 0:
      return launch_route_topk(logits, T, E, k, ids, w, s);
    case 1:
      launch_kernel(sort_hist_kernel, dim3(nchunks), dim3(kWave), 0, s, ids, P, E, chunk);
      break;
    case 2:
      launch_kernel(sort_chunk_scan_kernel, dim3(E), dim3(256), 0, s, chunk, nchunks, E, counts);
      break;
    default:
      launch_kernel(sort_scatter_kernel, dim3(nchunks), dim3(kWave), 0, s, ids, P, E, chunk, counts, offsets,
                         sorted, act, n_act, slots, tile_m, tile_off);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
