// Device helpers shared by the kernels: e4m3 conversion, bf16, wave64 reductions, scales.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kScaleBlock = 128;  // one scale per 128x128 block of a bank
constexpr float kE4M3Max = 448.0f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two e4m3 codes (bytes 0,1 when HI is false, bytes 2,3 when true) of a 32-bit word to
// float with gfx950's conversion instruction, which reads OCP e4m3fn (bias 7). The decode
// is exact: every e4m3 value is a float.
template <bool HI>
__device__ __forceinline__ f32x2 dec2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// Four codes of a word -> four floats.
__device__ __forceinline__ void dec4(uint32_t w, float* o) {
  f32x2 lo = dec2<false>(w);
  f32x2 hi = dec2<true>(w);
  o[0] = lo.x;
  o[1] = lo.y;
  o[2] = hi.x;
  o[3] = hi.y;
}

// Float -> e4m3 code: round to nearest even, saturate at +-448 (clamped first, so the
// instruction never sees an out-of-range value), sign of zero kept.
__device__ __forceinline__ uint8_t enc1(float v) {
  float c = __builtin_fminf(__builtin_fmaxf(v, -kE4M3Max), kE4M3Max);
  // keep -0: fmin/fmax of -0 with +-448 returns -0
  int packed = __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false);
  return (uint8_t)(packed & 0xFF);
}

// Two floats -> two codes in the low half of a word.
__device__ __forceinline__ uint32_t enc2(float a, float b) {
  float ca = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  float cb = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Low and high bf16 halves of a word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A block scale as float, from a bf16 or a float table. Written without a branch (two 16-bit
// reads: a float's high and low halves, or the bf16 value twice) so that the wait for the
// value can stay at its first use; a load inside a branch is waited for at once, together
// with every load issued before it.
struct ScaleBits {
  uint32_t hi, lo;
};

__device__ __forceinline__ ScaleBits load_scale_bits(const void* base, int is_bf16, int64_t idx) {
  const uint16_t* p = (const uint16_t*)base + (is_bf16 ? idx : 2 * idx);
  return ScaleBits{p[is_bf16 ? 0 : 1], p[0]};
}

__device__ __forceinline__ float scale_value(const ScaleBits& b, int is_bf16) {
  return __uint_as_float((b.hi << 16) | (is_bf16 ? 0u : b.lo));
}

__device__ __forceinline__ float load_scale(const void* base, int is_bf16, int64_t idx) {
  return scale_value(load_scale_bits(base, is_bf16, idx), is_bf16);
}

// Waits for a value loaded earlier at this point of the program, not sooner.
__device__ __forceinline__ void settle(ScaleBits& b) { asm volatile("" : "+v"(b.hi), "+v"(b.lo)); }

// ---- wave64 reductions on DPP (row shifts within 16-lane rows, then row broadcasts 15 and
// 31), which stay in the VALU instead of going through LDS like a shuffle. The result is
// read from lane 63 and is uniform. Call with all 64 lanes active.

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
}

// Keeps the compiler from moving one wave's LDS accesses across this point; the LDS itself
// serves a wave's accesses in the order they are issued.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xF, 0xF>(0u, v));  // row_shr:1
  v = max(v, dpp_u32<0x112, 0xF, 0xF>(0u, v));  // row_shr:2
  v = max(v, dpp_u32<0x114, 0xF, 0xF>(0u, v));  // row_shr:4
  v = max(v, dpp_u32<0x118, 0xF, 0xF>(0u, v));  // row_shr:8
  v = max(v, dpp_u32<0x142, 0xA, 0xF>(0u, v));  // row_bcast:15
  v = max(v, dpp_u32<0x143, 0xC, 0xF>(0u, v));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const uint32_t id = 0xFFFFFFFFu;
  v = min(v, dpp_u32<0x111, 0xF, 0xF>(id, v));
  v = min(v, dpp_u32<0x112, 0xF, 0xF>(id, v));
  v = min(v, dpp_u32<0x114, 0xF, 0xF>(id, v));
  v = min(v, dpp_u32<0x118, 0xF, 0xF>(id, v));
  v = min(v, dpp_u32<0x142, 0xA, 0xF>(id, v));
  v = min(v, dpp_u32<0x143, 0xC, 0xF>(id, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK, BANK_MASK>(0u, __float_as_uint(v)));  // 0u is +0.0f
}

// Sum over the 64 lanes in a fixed order (deterministic), result uniform.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0x111, 0xF, 0xF>(v);
  v += dpp_f32<0x112, 0xF, 0xF>(v);
  v += dpp_f32<0x114, 0xF, 0xF>(v);
  v += dpp_f32<0x118, 0xF, 0xF>(v);
  v += dpp_f32<0x142, 0xA, 0xF>(v);
  v += dpp_f32<0x143, 0xC, 0xF>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Float -> unsigned key whose unsigned order is the float order (NaN excluded). -0 is
// first turned into +0 (x + 0 does that and nothing else), so the two compare equal as
// floats do.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = (int)(threadIdx.x & (kWave - 1));
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// silu(g) = g / (1 + e^-g), in float.
__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// 16-byte global load kept as four words.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

// Non-temporal 16-byte load for weight bytes that are read once.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

}  // namespace moe
