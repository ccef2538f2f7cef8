// The per-row e4m3 quantiser of activation rows, shared by its own kernel and the routing
// kernel that also quantises its tokens' rows.
#pragma once

#include "common.hpp"

namespace moe {

// x / s rounded to float, for a float x and a positive float s given as rs = 1 / (double)s:
// the double product float((double)x * rs) is within 2^-52 of x / s, and x / s is never a
// float rounding midpoint (an odd 25-bit significand times s cannot fit the 24 bits of x)
// and otherwise lies at least 2^-49 from one (x - m * s is a multiple of the 49-bit product's
// ulp), so it rounds to the correctly rounded float quotient that a division gives, at the
// cost of one double multiply per value and one double division per row. Quotients small
// enough to be float subnormals round to the e4m3 zero either way.
__device__ __forceinline__ float quot(float x, double rs) { return (float)((double)x * rs); }

// Zero codes for columns cols .. ostride - 1 of a code row (ostride - cols < 512, both
// multiples of 8): the padding that makes a partial last 128-wide K block multiply zeros.
__device__ __forceinline__ void zero_tail(uint8_t* row, int cols, int ostride, int lane) {
  const int c = cols + lane * 8;
  if (c < ostride) *(uint2*)(row + c) = make_uint2(0u, 0u);
}

// One wave per row of bf16: amax, scale = amax/448 (1 if zero), codes = e4m3(x/scale).
// Lane l holds the 8-value pieces l, l + 64, ... of the row: IT of them, all read up front
// (pieces past the row end read its last piece and are ignored), so the row is read from
// memory once and every read is in flight together. Code rows are ostride bytes apart, the
// columns past cols zero. The load and the rest are split so that a caller can issue the
// reads early and do other work while they are in flight.
template <int IT>
__device__ __forceinline__ void quant_row_bf16_load(const uint16_t* __restrict__ x, int row, int cols, u32x4 (&v)[IT]) {
  const int lane = lane_id();
  const uint16_t* xr = x + (size_t)row * cols;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane * 8 + it * kWave * 8;
    v[it] = *(const u32x4*)(xr + (c < cols ? c : cols - 8));
  }
}

template <int IT>
__device__ __forceinline__ void quant_row_bf16_store(const u32x4 (&v)[IT], int row, int cols, int ostride,
                                                     uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = lane_id();
  float amax = 0.0f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const bool in = lane * 8 + it * kWave * 8 < cols;
    const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = __builtin_fmaxf(amax, in ? __builtin_fabsf(bf16_lo(w[q])) : 0.0f);
      amax = __builtin_fmaxf(amax, in ? __builtin_fabsf(bf16_hi(w[q])) : 0.0f);
    }
  }
  amax = wave_max(amax);
  const float s = amax > 0.0f ? amax / kE4M3Max : 1.0f;
  const double rs = 1.0 / (double)s;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane * 8 + it * kWave * 8;
    if (c >= cols) continue;
    const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
    uint32_t out[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t a = enc2(quot(bf16_lo(w[2 * q]), rs), quot(bf16_hi(w[2 * q]), rs));
      const uint32_t b = enc2(quot(bf16_lo(w[2 * q + 1]), rs), quot(bf16_hi(w[2 * q + 1]), rs));
      out[q] = a | (b << 16);
    }
    *(uint2*)(codes + (size_t)row * ostride + c) = make_uint2(out[0], out[1]);
  }
  zero_tail(codes + (size_t)row * ostride, cols, ostride, lane);
  if (lane == 0) scales[row] = s;
}

}  // namespace moe
