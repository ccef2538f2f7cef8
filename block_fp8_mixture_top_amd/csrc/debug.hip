// Element-wise e4m3 conversions with the same helpers the GEMM kernels use, exported so that
// tests can check them over every code and over rounding midpoints.
#include "common.hpp"
#include "gemv.hpp"
#include "launch.hpp"

namespace moe {

namespace {

__global__ void decode_e4m3_kernel(const uint8_t* __restrict__ codes, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = dec2<false>((uint32_t)codes[i]).x;
}

// Every way the kernels turn e4m3 codes into numbers, on 16-code chunks: out[i][j][path] for
// code j of chunk i. path 0: cvt_pk_f32_fp8 (both halves of each word); 1:
// cvt_scalef32_pk_bf16_fp8 with unit scale (both halves), widened to float; 2: dot16_bf16
// against a bf16 one-hot activation (1.0 at j); 3: dot16_e4m3 against an e4m3 one-hot (code
// 0x38, 1.0, at j); 4: dot16_f32 against a float one-hot. One thread per (chunk, j).
__global__ void decode_paths_kernel(const uint8_t* __restrict__ chunks, float* __restrict__ out, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * 16) return;
  const int64_t i = t / 16;
  const int j = (int)(t % 16);
  const u32x4 c = *(const u32x4*)(chunks + i * 16);
  const uint32_t w = c[j / 4];
  const int b = j % 4;
  const f32x2 f = b < 2 ? dec2<false>(w) : dec2<true>(w);
  const bf16x2 h = b < 2 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)
                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  float* o = out + t * 5;
  o[0] = (b % 2 == 0) ? f.x : f.y;
  o[1] = (float)((b % 2 == 0) ? h.x : h.y);
  uint32_t xw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  xw[j / 2] = (j % 2 == 0) ? 0x3F80u : 0x3F800000u;  // bf16 1.0 in the low or high half
  o[2] = dot16_bf16(c, u32x4{xw[0], xw[1], xw[2], xw[3]}, u32x4{xw[4], xw[5], xw[6], xw[7]});
  uint32_t qw[4] = {0, 0, 0, 0};
  qw[j / 4] = 0x38u << (8 * (j % 4));  // e4m3 1.0 at byte j
  o[3] = dot16_e4m3(c, u32x4{qw[0], qw[1], qw[2], qw[3]});
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = q == j ? 1.0f : 0.0f;
  o[4] = dot16_f32(c, v);
}

__global__ void encode_e4m3_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  codes[i] = enc1(x[i]);
}

}  // namespace

hipError_t launch_decode_e4m3(const uint8_t* codes, float* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch_kernel(decode_e4m3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, out, n);
  return hipGetLastError();
}

hipError_t launch_decode_paths(const uint8_t* chunks, float* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch_kernel(decode_paths_kernel, dim3((unsigned)((n * 16 + 255) / 256)), dim3(256), 0, s, chunks, out, n);
  return hipGetLastError();
}

hipError_t launch_encode_e4m3(const float* x, uint8_t* codes, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch_kernel(encode_e4m3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, codes, n);
  return hipGetLastError();
}

}  // namespace moe
