// Row-streaming GEMV helpers shared by the W8A16 kernels: 16-byte chunks of e4m3 codes
// decoded exactly in registers and dotted with bf16 or float activations.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kThreads = 256;

// sum_i dec(code_i) * x_i over the 16 codes of `c` and the 16 bf16 activations of `x0,x1`.
// Two codes at a time are widened to bf16 (exact: e4m3's 3 mantissa bits and its exponent
// range fit bf16; the unit scale leaves them unchanged) and dotted with two activations in
// float by one instruction, so each product is exact as before.
__device__ __forceinline__ float dot16_bf16(const u32x4& c, const u32x4& x0, const u32x4& x1) {
  float acc = 0.0f;
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[q], 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[q], 1.0f, true);
    acc = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2, xw[2 * q]), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, xw[2 * q + 1]), acc, false);
  }
  return acc;
}

// sum_i dec(c_i) * dec(x_i) over 16 weight codes and 16 activation codes: both are widened
// to bf16 exactly and each product of two e4m3 values (at most 8 significant bits) is exact
// in the float dot.
__device__ __forceinline__ float dot16_e4m3(const u32x4& c, const u32x4& x) {
  float acc = 0.0f;
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2 clo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[q], 1.0f, false);
    const bf16x2 chi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[q], 1.0f, true);
    const bf16x2 xlo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(xw[q], 1.0f, false);
    const bf16x2 xhi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(xw[q], 1.0f, true);
    acc = __builtin_amdgcn_fdot2_f32_bf16(clo, xlo, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(chi, xhi, acc, false);
  }
  return acc;
}

// sum_i dec(code_i) * v_i over 16 codes and 16 floats.
__device__ __forceinline__ float dot16_f32(const u32x4& c, const float* v) {
  float acc = 0.0f;
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x2 lo = dec2<false>(cw[q]);
    const f32x2 hi = dec2<true>(cw[q]);
    acc = __builtin_fmaf(lo.x, v[4 * q + 0], acc);
    acc = __builtin_fmaf(lo.y, v[4 * q + 1], acc);
    acc = __builtin_fmaf(hi.x, v[4 * q + 2], acc);
    acc = __builtin_fmaf(hi.y, v[4 * q + 3], acc);
  }
  return acc;
}

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR == kWave) {
    return wave_sum_dpp(v);
  } else {
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
  }
}


// Lane layout for rows of K bytes: LPR lanes per row, MCH 16-byte chunks per lane.

struct Layout {
  int lpr, mch;
};

inline Layout pick_layout(int K) {
  const int nc = K / 16;
  if (nc >= kWave) return Layout{kWave, (nc + kWave - 1) / kWave};
  int lpr = 8;
  while (lpr * 2 <= nc && lpr < kWave) lpr *= 2;
  return Layout{lpr, (nc + lpr - 1) / lpr};
}


}  // namespace moe
