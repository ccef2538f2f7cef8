// One token's routing by one wave: top-k experts by logit and their renormalised softmax
// weights (gaudi-cookbook "fp8-moe-gather", The fix: each token keeps its top_k experts).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {

// The logits a lane selects from: f[i] = row[lane + 64 i] (entries past E read the last one
// and are ignored by the selection). All loads are issued together, in bounds and outside
// any branch. PIN: an empty asm then uses each value, which keeps every load where it is
// written but also waits for it there; a prefetch leaves it out so that the wait falls at
// the first use.
template <int PER, bool PIN = true>
__device__ __forceinline__ void wave_topk_load(const float* __restrict__ row, int E, float (&f)[PER]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    f[i] = row[e < E ? e : E - 1];
  }
  if constexpr (PIN) {
#pragma unroll
    for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(f[i]));
  }
}

// Selection from logits loaded by wave_topk_load: lane j < k receives slot j, the expert
// with the j-th largest logit (ties to the lower id), and that logit. PER = logits held per
// lane, E <= 64 * PER. A NaN logit reads as -inf, which keeps every id in [0, E). Call with
// all 64 lanes active.
//
// Each lane first sorts its PER keys best-first, so its current best is always its head
// (the slot of each sorted key, hence its expert lane + 64 * slot, is kept four bits each
// in one register); a round is then one wave-wide max of the heads, a ballot of the lanes
// holding that key (one lane unless logits tie exactly; the lowest id among tied heads is
// taken by a min over them), and the winning lane advancing its head with selects instead
// of a branch.
template <int PER>
__device__ __forceinline__ void wave_topk_select(const float (&f)[PER], int E, int k, int& out_id, float& out_l) {
  static_assert(PER <= 16, "slot indices are packed four bits each");
  typedef typename std::conditional<PER <= 8, uint32_t, uint64_t>::type slot_t;
  const int lane = lane_id();
  uint32_t key[PER];
  // slot i holds expert lane + 64 i; after sorting, nibble i of `slot` is the slot of the
  // i-th best key of this lane
  slot_t slot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const float v = f[i] != f[i] ? -__builtin_inff() : f[i];
    key[i] = e < E ? order_key(v) : 0u;  // every real logit has a key > 0
    slot |= (slot_t)i << (4 * i);
  }
  // insertion sort, best first: larger key, then lower id (ids rise with the slot, so a
  // strict comparison keeps equal keys in id order)
#pragma unroll
  for (int i = 1; i < PER; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = key[j] > key[j - 1];
      const uint32_t tk = sw ? key[j] : key[j - 1];
      const uint32_t bk = sw ? key[j - 1] : key[j];
      key[j - 1] = tk;
      key[j] = bk;
      const slot_t a = (slot >> (4 * (j - 1))) & 15u, b = (slot >> (4 * j)) & 15u;
      const slot_t cleared = slot & ~((slot_t)0xFF << (4 * (j - 1)));
      slot = sw ? cleared | (b << (4 * (j - 1))) | (a << (4 * j)) : slot;
    }
  int my_id = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    const uint32_t mk = wave_max_u32(key[0]);
    const uint64_t cand = __ballot(key[0] == mk);
    int win;
    if (__popcll(cand) == 1) {
      win = __builtin_ctzll(cand);
    } else {
      // tied heads: the lowest expert id among them
      const uint32_t hid = (uint32_t)(lane + kWave * (int)(slot & 15u));
      const uint32_t wid = wave_min_u32(key[0] == mk ? hid : 0xFFFFFFFFu);
      win = (int)(wid & (kWave - 1));
    }
    const int wslot = __builtin_amdgcn_readlane((int)(uint32_t)(slot & 15u), win);
    const int wid = win + kWave * wslot;
    my_id = lane == j ? wid : my_id;
    my_l = lane == j ? key_to_float(mk) : my_l;
    // the winning lane advances its head; branch-free, so no lane waits on an exec switch
    const bool adv = lane == win;
#pragma unroll
    for (int i = 0; i + 1 < PER; ++i) key[i] = adv ? key[i + 1] : key[i];
    key[PER - 1] = adv ? 0u : key[PER - 1];
    slot = adv ? slot >> 4 : slot;
  }
  out_id = my_id;
  out_l = my_l;
}

// The same selection as wave_topk_select, for k <= 8, by filtering and then ranking the few
// logits that pass. `cand` is 64 entries of LDS (16-byte aligned) that belong to this wave
// alone; their contents are overwritten.
//
// Filter: lanes 8q .. 8q+7 form group q (q < 8). The eight group maxima are eight distinct
// logits, so the smallest of them, t, is at most the k-th largest logit when k <= 8, and
// every expert to be selected has a logit >= t (about 20 of 256 logits pass for Gaussian or
// uniform logits).
// Rank: each passing expert is stored as key << 32 | ~id, which makes a larger logit, or an
// equal logit with a lower id, the larger integer; the number of larger entries is its slot.
// When more than 64 logits pass (widely tied logits), or k > 8, the round-based selection
// runs instead.
template <int PER>
__device__ __forceinline__ void wave_topk_select_lds(const float (&f)[PER], int E, int k, uint64_t* cand,
                                                     int& out_id, float& out_l) {
  if (k > 8) {
    wave_topk_select<PER>(f, E, k, out_id, out_l);
    return;
  }
  const int lane = lane_id();
  uint32_t key[PER];
  uint32_t g = 0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const float v = f[i] != f[i] ? -__builtin_inff() : f[i];
    key[i] = e < E ? order_key(v) : 0u;  // every real logit has a key > 0
    g = max(g, key[i]);
  }
  g = max(g, dpp_u32<0x111, 0xF, 0xF>(0u, g));  // row_shr:1
  g = max(g, dpp_u32<0x112, 0xF, 0xF>(0u, g));  // row_shr:2
  g = max(g, dpp_u32<0x114, 0xF, 0xF>(0u, g));  // row_shr:4; lane 8q+7 now holds group q's max
  uint32_t t = 0xFFFFFFFFu;
#pragma unroll
  for (int q = 0; q < 8; ++q) t = min(t, (uint32_t)__builtin_amdgcn_readlane((int)g, 8 * q + 7));
  t = max(t, 1u);  // with E < 64 a group may hold padding only; then every real logit passes
  uint64_t m[PER];
  int n = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    m[i] = __ballot(key[i] >= t);
    n += __popcll(m[i]);
  }
  if (n > kWave) {
    wave_topk_select<PER>(f, E, k, out_id, out_l);
    return;
  }
  // compact the candidates into cand[0, n) and zero-fill to a multiple of 8
  int base = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int below =
        (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m[i] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[i], 0u));
    if (key[i] >= t) cand[base + below] = ((uint64_t)key[i] << 32) | (uint64_t)(~(uint32_t)(lane + kWave * i));
    base += __popcll(m[i]);
  }
  const int n8 = (n + 7) & ~7;
  if (lane >= n && lane < n8) cand[lane] = 0ull;  // below every real entry
  wave_lds_sync();
  const uint64_t mine = cand[lane];  // lanes >= n hold no candidate; their rank is unused
  int rank = 0;
  for (int j = 0; j < n8; j += 8) {
    uint64_t c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) c[q] = cand[j + q];
#pragma unroll
    for (int q = 0; q < 8; ++q) rank += c[q] > mine ? 1 : 0;
  }
  wave_lds_sync();
  if (lane < n && rank < k) cand[rank] = mine;
  wave_lds_sync();
  const uint64_t r = cand[lane < k ? lane : 0];
  out_id = lane < k ? (int)~(uint32_t)r : 0;
  out_l = lane < k ? key_to_float((uint32_t)(r >> 32)) : 0.0f;
}

// Load and the filtered selection (`cand` as for wave_topk_select_lds).
template <int PER>
__device__ __forceinline__ void wave_topk_ids_lds(const float* __restrict__ row, int E, int k, uint64_t* cand,
                                                  int& out_id, float& out_l) {
  float f[PER];
  wave_topk_load<PER>(row, E, f);
  wave_topk_select_lds<PER>(f, E, k, cand, out_id, out_l);
}

// Weights of the selected slots: lane j < k gets exp(l_j - l_0) / sum_i exp(l_i - l_0),
// evaluated in double with the sum in slot order and rounded to float.
__device__ __forceinline__ float wave_topk_weight(float my_l, int k) {
  const int lane = lane_id();
  const double l0 = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const double ex = lane < k ? exp((double)my_l - l0) : 0.0;
  double tot = 0.0;
  for (int j = 0; j < k; ++j) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(ex);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b & 0xFFFFFFFFull), j);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), j);
    tot += __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  }
  return (float)(ex / tot);
}

// Both: ids and weights (`cand` as for wave_topk_select_lds).
template <int PER>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, uint64_t* cand, int& out_id,
                                          float& out_w) {
  float l;
  wave_topk_ids_lds<PER>(row, E, k, cand, out_id, l);
  out_w = wave_topk_weight(l, k);
}

// Dispatch helper: the smallest PER in {1, 2, 4, 8, 16} with 64 * PER >= E.
#define MOE_TOPK_DISPATCH(E, ...)   \
  do {                              \
    if ((E) <= 64) {                \
      constexpr int PER = 1;        \
      __VA_ARGS__;                  \
    } else if ((E) <= 128) {        \
      constexpr int PER = 2;        \
      __VA_ARGS__;                  \
    } else if ((E) <= 256) {        \
      constexpr int PER = 4;        \
      __VA_ARGS__;                  \
    } else if ((E) <= 512) {        \
      constexpr int PER = 8;        \
      __VA_ARGS__;                  \
    } else {                        \
      constexpr int PER = 16;       \
      __VA_ARGS__;                  \
    }                               \
  } while (0)

}  // namespace moe
