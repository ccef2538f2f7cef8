// Element-wise e4m3 conversions with the same helpers the GEMM kernels use, exported so that
// tests can check them over every code and over rounding midpoints.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

__global__ void decode_e4m3_kernel(const uint8_t* __restrict__ codes, float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = dec2<false>((uint32_t)codes[i]).x;
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

hipError_t launch_encode_e4m3(const float* x, uint8_t* codes, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch_kernel(encode_e4m3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, codes, n);
  return hipGetLastError();
}

}  // namespace moe
