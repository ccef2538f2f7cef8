// One token's routing by one wave: top-k experts by logit and their renormalised softmax
// weights (gaudi-cookbook "fp8-moe-gather", The fix: each token keeps its top_k experts).
#pragma once

#include "common.hpp"

namespace moe {

// Lane j < k receives slot j: the expert with the j-th largest logit (ties to the lower
// id) and its weight exp(l_j - l_0) / sum_i exp(l_i - l_0), evaluated in double with the
// sum in slot order and rounded to float. PER = logits held per lane, E <= 64 * PER. A NaN
// logit reads as -inf, which keeps every id in [0, E). Call with all 64 lanes active.
template <int PER>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int& out_id, float& out_w) {
  const int lane = lane_id();
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    float f = e < E ? row[e] : 0.0f;
    f = f != f ? -__builtin_inff() : f;
    key[i] = e < E ? order_key(f) : 0u;  // every real logit has a key > 0
  }
  uint32_t taken = 0;
  float my_l = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t bk = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t c = ((taken >> i) & 1u) ? 0u : key[i];
      if (c > bk) {  // strict: the lowest id of a lane wins its ties
        bk = c;
        bi = lane + kWave * i;
      }
    }
    const uint32_t mk = wave_max_u32(bk);
    const uint32_t wid = wave_min_u32(bk == mk ? (uint32_t)bi : 0xFFFFFFFFu);
    if ((int)(wid & (kWave - 1)) == lane) taken |= 1u << (wid / kWave);
    if (lane == j) {
      my_id = (int)wid;
      my_l = key_to_float(mk);
    }
  }
  const double l0 = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
  const double ex = lane < k ? exp((double)my_l - l0) : 0.0;
  double tot = 0.0;
  for (int j = 0; j < k; ++j) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(ex);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b & 0xFFFFFFFFull), j);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), j);
    tot += __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  }
  out_id = my_id;
  out_w = (float)(ex / tot);
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
