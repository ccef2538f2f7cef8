// W8A8 grouped GEMMs on gfx950's fp8 matrix cores, for expert batches large enough to be
// a dense contraction (prefill).
//
// Activations are quantised per row to e4m3 with a dynamic scale, as the gathered FP8 path
// of gaudi-cookbook "fp8-moe-gather" does for checkpoints with dynamic activation scales
// (section Who is affected): scale = amax/448 (1 for an all-zero row), code = e4m3(x/scale),
// rows being tokens for GEMM1 and (token, slot) pairs for GEMM2.
//
// One v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0 scales) covers exactly one 128-wide
// K block, so every MFMA result is one block's partial sum and is multiplied by that block's
// bank scale before it is accumulated (FreeToken PR #662, PR body: one scale per 128x128
// block). A and B are loaded with the same per-lane K pattern (32 contiguous bytes of a
// row per lane), so whatever order the unit walks K in, matching A and B bytes meet.
//
// GEMM1 covers all 2I features of a tile of sorted pairs, so the epilogue has the whole h
// row: silu(gate)*up, row amax, scale and e4m3 codes are produced without writing h in
// float. GEMM2 multiplies by the pair's h scale and router weight and adds into a float
// [T, H] accumulator with atomics (the scatter-add combine).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kNeutralScale = 127;  // E8M0 2^0

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, kNeutralScale, 0, kNeutralScale);
}

__device__ __forceinline__ i32x8 ld32(const uint8_t* p) {
  const u32x4 lo = *(const u32x4*)p;
  const u32x4 hi = *(const u32x4*)(p + 16);
  i32x8 r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ i32x8 zero8() {
  i32x8 r;
#pragma unroll
  for (int q = 0; q < 8; ++q) r[q] = 0;
  return r;
}

// ---------------------------------------------------------------- per-row quantisation

// One wave per row of bf16: amax, scale = amax/448 (1 if zero), codes = e4m3(x/scale).
__global__ __launch_bounds__(256) void quant_rows_bf16_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int row = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
  if (row >= rows) return;
  const int lane = lane_id();
  const uint16_t* xr = x + (size_t)row * cols;
  float amax = 0.0f;
  for (int c = lane * 8; c < cols; c += kWave * 8) {
    const u32x4 v = *(const u32x4*)(xr + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_lo(w[q])));
      amax = __builtin_fmaxf(amax, __builtin_fabsf(bf16_hi(w[q])));
    }
  }
  amax = wave_max(amax);
  const float s = amax > 0.0f ? amax / kE4M3Max : 1.0f;
  for (int c = lane * 8; c < cols; c += kWave * 8) {
    const u32x4 v = *(const u32x4*)(xr + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t a = enc2(bf16_lo(w[2 * q]) / s, bf16_hi(w[2 * q]) / s);
      const uint32_t b = enc2(bf16_lo(w[2 * q + 1]) / s, bf16_hi(w[2 * q + 1]) / s);
      out[q] = a | (b << 16);
    }
    *(uint2*)(codes + (size_t)row * cols + c) = make_uint2(out[0], out[1]);
  }
  if (lane == 0) scales[row] = s;
}

// ---------------------------------------------------------------- tile lookup

// Tile `tile` of the grouped problem -> expert and first sorted position. Tiles of one
// expert are consecutive; tile_off holds each expert's first tile (exclusive sums).
__device__ __forceinline__ int find_expert(const int32_t* tile_off, int E, int tile) {
  int lo = 0, hi = E;  // invariant: tile_off[lo] <= tile < tile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= tile) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Workgroup -> tile with the tiles of one expert kept on one XCD (workgroups are dealt to
// the 8 XCDs round-robin), so the expert's weights are fetched into one L2. nblocks is a
// multiple of 8, which makes the map a permutation of [0, nblocks).
__device__ __forceinline__ int xcd_tile(int bid, int nblocks) {
  const int per = nblocks / 8;
  const int x = bid & 7, i = bid >> 3;
  return x * per + i;
}

// ---------------------------------------------------------------- GEMM1

constexpr int kTM = kMfmaTileM;  // pairs per tile (two 16-row MFMA tiles)

// grid: one workgroup per (expert, 32-pair tile), 4 waves. Wave w owns gate features
// [w*I/4, (w+1)*I/4) and the up features I + the same range: NT 16-feature MFMA tiles each.
template <int NT>
__global__ __launch_bounds__(256) void gemm1_mfma_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                         BankArg w13, Plan plan, int E, int H, int I, int k,
                                                         int nblocks, uint8_t* __restrict__ hq,
                                                         float* __restrict__ hs) {
  __shared__ float amax_w[4][kTM];
  const int tile = xcd_tile(blockIdx.x, nblocks);
  if (tile >= plan.tile_off[E]) return;
  const int e = find_expert(plan.tile_off, E, tile);
  const int pos0 = plan.offsets[e] + (tile - plan.tile_off[e]) * kTM;
  const int pos_end = plan.offsets[e + 1];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int r16 = lane & 15, kq = lane >> 4;  // row within a 16-tile, K quarter (32 bytes)

  // B operand rows: the tokens of the two pair tiles
  const uint8_t* xrow[2];
  bool tok_ok[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int pos = pos0 + tt * 16 + r16;
    tok_ok[tt] = pos < pos_end;
    const int t = tok_ok[tt] ? plan.sorted[pos] / k : 0;
    xrow[tt] = xq + (size_t)t * H;
  }
  const int fbase = wave * (I / 4);  // first gate feature of this wave
  const uint8_t* wb = w13.codes + (size_t)e * w13.expert_stride;
  const int64_t sb = (int64_t)e * w13.sexp;

  f32x4 accg[NT][2], accu[NT][2];
#pragma unroll
  for (int f = 0; f < NT; ++f)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      accg[f][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      accu[f][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

  const int nkb = H / 128;
  for (int kb = 0; kb < nkb; ++kb) {
    const int kofs = kb * 128 + kq * 32;
    i32x8 b[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) b[tt] = tok_ok[tt] ? ld32(xrow[tt] + kofs) : zero8();
#pragma unroll
    for (int f = 0; f < NT; ++f) {
      const int rg = fbase + f * 16;  // gate rows rg..rg+15, up rows I+rg..
      const i32x8 ag = ld32(wb + (size_t)(rg + r16) * H + kofs);
      const i32x8 au = ld32(wb + (size_t)(I + rg + r16) * H + kofs);
      const float sg = load_scale(w13.scales, w13.scale_bf16, sb + (int64_t)(rg / kScaleBlock) * w13.srow + kb);
      const float su = load_scale(w13.scales, w13.scale_bf16, sb + (int64_t)((I + rg) / kScaleBlock) * w13.srow + kb);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 pg = mfma_fp8(ag, b[tt]);
        const f32x4 pu = mfma_fp8(au, b[tt]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          accg[f][tt][q] = __builtin_fmaf(sg, pg[q], accg[f][tt][q]);
          accu[f][tt][q] = __builtin_fmaf(su, pu[q], accu[f][tt][q]);
        }
      }
    }
  }

  // epilogue: D[feature 4*kq + q][token r16]; h = silu(g) * u with the x scale applied
  float xsc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int pos = pos0 + tt * 16 + r16;
    xsc[tt] = tok_ok[tt] ? xs[plan.sorted[pos] / k] : 0.0f;
  }
  float hv[NT][2][4];
  float am[2] = {0.0f, 0.0f};
#pragma unroll
  for (int f = 0; f < NT; ++f)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float g = accg[f][tt][q] * xsc[tt];
        const float u = accu[f][tt][q] * xsc[tt];
        const float v = silu(g) * u;
        hv[f][tt][q] = v;
        am[tt] = __builtin_fmaxf(am[tt], __builtin_fabsf(v));
      }
  // per-token max over the 4 K-quarter lane groups, then over the 4 waves
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    am[tt] = __builtin_fmaxf(am[tt], __shfl_xor(am[tt], 16, kWave));
    am[tt] = __builtin_fmaxf(am[tt], __shfl_xor(am[tt], 32, kWave));
    if (kq == 0) amax_w[wave][tt * 16 + r16] = am[tt];
  }
  __syncthreads();
  float sc[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int r = tt * 16 + r16;
    const float a = __builtin_fmaxf(__builtin_fmaxf(amax_w[0][r], amax_w[1][r]),
                                    __builtin_fmaxf(amax_w[2][r], amax_w[3][r]));
    sc[tt] = a > 0.0f ? a / kE4M3Max : 1.0f;
  }
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int pos = pos0 + tt * 16 + r16;
    if (!tok_ok[tt]) continue;
#pragma unroll
    for (int f = 0; f < NT; ++f) {
      const int i = fbase + f * 16 + kq * 4;
      const uint32_t lo = enc2(hv[f][tt][0] / sc[tt], hv[f][tt][1] / sc[tt]);
      const uint32_t hi = enc2(hv[f][tt][2] / sc[tt], hv[f][tt][3] / sc[tt]);
      *(uint32_t*)(hq + (size_t)pos * I + i) = lo | (hi << 16);
    }
    if (wave == 0 && kq == 0) hs[pos] = sc[tt];
  }
}

// ---------------------------------------------------------------- GEMM2

// grid.x: (expert, 32-pair tile), grid.y: H / (64*NF). A = h codes (pairs as rows), B = w2
// rows; each of the 4 waves covers NF 16-feature MFMA tiles.
// D[pair 4*kq + q][feature r16]: a wave's 16 lanes of one K quarter hold 16 consecutive
// features of one pair, so its atomics touch 64 contiguous bytes per pair row.
template <int NF>
__global__ __launch_bounds__(256) void gemm2_mfma_kernel(const uint8_t* __restrict__ hq, const float* __restrict__ hs,
                                                         BankArg w2, Plan plan, int E, int H, int I, int k,
                                                         int nblocks, float* __restrict__ acc_out) {
  constexpr int kFeat = 4 * 16 * NF;  // output features per workgroup
  const int tile = xcd_tile(blockIdx.x, nblocks);
  if (tile >= plan.tile_off[E]) return;
  const int e = find_expert(plan.tile_off, E, tile);
  const int pos0 = plan.offsets[e] + (tile - plan.tile_off[e]) * kTM;
  const int pos_end = plan.offsets[e + 1];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const int n_base = blockIdx.y * kFeat + wave * (kFeat / 4);
  const uint8_t* wb = w2.codes + (size_t)e * w2.expert_stride;
  const int64_t sb = (int64_t)e * w2.sexp;

  bool ok[2];
  const uint8_t* arow[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int pos = pos0 + tt * 16 + r16;
    ok[tt] = pos < pos_end;
    arow[tt] = hq + (size_t)(ok[tt] ? pos : pos0) * I;
  }
  f32x4 acc[2][NF];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[tt][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nkb = I / 128;
  for (int kb = 0; kb < nkb; ++kb) {
    const int kofs = kb * 128 + kq * 32;
    i32x8 a[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) a[tt] = ok[tt] ? ld32(arow[tt] + kofs) : zero8();
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = n_base + f * 16;
      const i32x8 b = ld32(wb + (size_t)(n + r16) * I + kofs);
      const float s = load_scale(w2.scales, w2.scale_bf16, sb + (int64_t)(n / kScaleBlock) * w2.srow + kb);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 p = mfma_fp8(a[tt], b);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[tt][f][q] = __builtin_fmaf(s, p[q], acc[tt][f][q]);
      }
    }
  }
  // epilogue: pair rows 4*kq + q of each 16-tile
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = pos0 + tt * 16 + kq * 4 + q;
      if (pos >= pos_end) continue;
      const int p = plan.sorted[pos];
      const int t = p / k;
      const float mult = hs[pos] * plan.w[p];
      float* orow = acc_out + (size_t)t * H;
#pragma unroll
      for (int f = 0; f < NF; ++f) unsafeAtomicAdd(orow + n_base + f * 16 + r16, acc[tt][f][q] * mult);
    }
}

__global__ void zero_f32_kernel(float* __restrict__ p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

__global__ void finalize_kernel(const float* __restrict__ acc, size_t n, void* __restrict__ out, int out_bf16) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (out_bf16) ((uint16_t*)out)[i] = f32_to_bf16(acc[i]);
  else ((float*)out)[i] = acc[i];
}

template <int NT>
hipError_t g1m(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E, int nblocks, int H,
               int I, int k, uint8_t* hq, float* hs, hipStream_t s) {
  hipLaunchKernelGGL((gemm1_mfma_kernel<NT>), dim3(nblocks), dim3(256), 0, s, xq, xs, w13, plan, E, H, I, k, nblocks,
                     hq, hs);
  return hipGetLastError();
}

}  // namespace

// Upper bound on the tiles of any routing (sum over experts of ceil(count/32) <= P/32 + E),
// rounded up to a multiple of 8 so that xcd_tile maps the grid onto [0, bound) one to one.
size_t mfma_tiles_bound(int P, int E) {
  const size_t b = (size_t)(P + kTM - 1) / kTM + (size_t)E;
  return (b + 7) / 8 * 8;
}

hipError_t launch_quant_rows_bf16(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                                  hipStream_t s) {
  const int blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(quant_rows_bf16_kernel, dim3(blocks), dim3(256), 0, s, x, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_gemm1_mfma(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E, int P,
                             int H, int I, int k, uint8_t* hq, float* hs, hipStream_t s) {
  const int nblocks = (int)mfma_tiles_bound(P, E);
  switch (I / 64) {
    case 2: return g1m<2>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
    case 4: return g1m<4>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
    case 6: return g1m<6>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
    case 8: return g1m<8>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
    default: return hipErrorInvalidValue;
  }
}

template <int NF>
static hipError_t g2m(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int nblocks,
                      int H, int I, int k, float* acc, hipStream_t s) {
  dim3 grid(nblocks, H / (64 * NF));
  hipLaunchKernelGGL((gemm2_mfma_kernel<NF>), grid, dim3(256), 0, s, hq, hs, w2, plan, E, H, I, k, nblocks, acc);
  return hipGetLastError();
}

hipError_t launch_gemm2_mfma(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int P,
                             int H, int I, int k, float* acc, hipStream_t s) {
  const int nblocks = (int)mfma_tiles_bound(P, E);
  if (H % 512 == 0) return g2m<8>(hq, hs, w2, plan, E, nblocks, H, I, k, acc, s);
  if (H % 256 == 0) return g2m<4>(hq, hs, w2, plan, E, nblocks, H, I, k, acc, s);
  return g2m<2>(hq, hs, w2, plan, E, nblocks, H, I, k, acc, s);
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* acc, size_t n, void* out, int out_bf16, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, acc, n, out, out_bf16);
  return hipGetLastError();
}

}  // namespace moe
