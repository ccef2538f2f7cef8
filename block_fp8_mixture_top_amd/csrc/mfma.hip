// W8A8 grouped GEMMs on gfx950's fp8 matrix cores, for expert batches large enough to be
// a dense contraction (prefill).
//
// Activations are quantised to e4m3 with a dynamic scale, as the gathered FP8 path of
// gaudi-cookbook "fp8-moe-gather" does for checkpoints with dynamic activation scales
// (section Who is affected): scale = amax/448 (1 for an all-zero row), code = e4m3(x/scale),
// one scale per row (tokens for GEMM1, (token, slot) pairs for GEMM2) or, in the group
// variant, one per 128-column group of a row (the K blocks of the weight scales), h then
// being quantised inside GEMM1.
//
// One v_mfma_scale_f32_16x16x128_f8f6f4 (neutral E8M0 scales) covers exactly one 128-wide
// K block, so every MFMA result is one block's partial sum and takes that block's bank
// scale (FreeToken PR #662, PR body: one scale per 128x128 block): GEMM1 rescales its
// accumulator to the block's scale before the MFMA accumulates in place, GEMM2 scales each
// zero-start product into its accumulator. A and B are read with the same per-lane K
// pattern (chunks kq and kq + 4 of the block for lanes of K quarter kq), so whatever order
// the unit walks K in, matching A and B bytes meet.
//
// Both GEMMs work on tiles of 128 sorted (token, slot) pairs of one expert. Every operand
// goes global -> LDS with direct loads of 8 rows x 128 contiguous bytes per instruction,
// through LDS rings a few K blocks ahead of the multiply. GEMM1 (a 128-feature block of h
// per workgroup) writes h = silu(gate)*up in float; a row quantiser turns it into e4m3
// codes and one scale per (token, slot); GEMM2 copies the codes to LDS, multiplies, and
// writes each pair's y row once, in fp16 with a power-of-two exponent per 32 outputs; the
// combine kernel sums the slots of a token in slot order with the router weights.
#include "common.hpp"
#include "launch.hpp"
#include "quant.hpp"

namespace moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kNeutralScale = 127;  // E8M0 2^0

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kNeutralScale, 0, kNeutralScale);
}

// ---------------------------------------------------------------- per-row quantisation

// One wave per row of bf16 (quant_row_bf16).
template <int IT>
__global__ __launch_bounds__(256) void quant_rows_bf16_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                              int ostride, uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int row = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
  if (row >= rows) return;
  u32x4 v[IT];
  quant_row_bf16_load<IT>(x, row, cols, v);
  quant_row_bf16_store<IT>(v, row, cols, ostride, codes, scales);
}

// The same with one scale per 128-column group (cols a multiple of 128): a 512-column piece
// holds four groups, lanes 16q .. 16q+15 holding group q's 128 values, so a group's amax is
// a maximum over 16 neighbouring lanes. Codes [rows, cols], scales [rows, cols/128].
template <int IT>
__global__ __launch_bounds__(256) void quant_groups_bf16_kernel(const uint16_t* __restrict__ x, int rows, int cols,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
  const int row = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
  if (row >= rows) return;
  const int lane = lane_id();
  const uint16_t* xr = x + (size_t)row * cols;
  u32x4 v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane * 8 + it * kWave * 8;
    v[it] = *(const u32x4*)(xr + (c < cols ? c : cols - 8));
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane * 8 + it * kWave * 8;
    const bool in = c < cols;  // whole groups of 16 lanes are in or out (cols % 128 == 0)
    const uint32_t w[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = __builtin_fmaxf(amax, in ? __builtin_fabsf(bf16_lo(w[q])) : 0.0f);
      amax = __builtin_fmaxf(amax, in ? __builtin_fabsf(bf16_hi(w[q])) : 0.0f);
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, m, kWave));
    const float s = amax > 0.0f ? amax / kE4M3Max : 1.0f;
    const double rs = 1.0 / (double)s;
    if (!in) continue;
    uint32_t out[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t a = enc2(quot(bf16_lo(w[2 * q]), rs), quot(bf16_hi(w[2 * q]), rs));
      const uint32_t b = enc2(quot(bf16_lo(w[2 * q + 1]), rs), quot(bf16_hi(w[2 * q + 1]), rs));
      out[q] = a | (b << 16);
    }
    *(uint2*)(codes + (size_t)row * cols + c) = make_uint2(out[0], out[1]);
    if ((lane & 15) == 0) scales[(size_t)row * (cols / 128) + c / 128] = s;
  }
}

// The same for rows of float (h before the down GEMM, in sorted-position order), two
// 4-float reads per piece.
template <int IT>
__global__ __launch_bounds__(256) void quant_rows_f32_kernel(const float* __restrict__ x, int rows, int cols,
                                                             int ostride, uint8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
  const int row = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
  if (row >= rows) return;
  const int lane = lane_id();
  const float* xr = x + (size_t)row * cols;
  f32x4 va[IT], vb[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane * 8 + it * kWave * 8;
    const int cc = c < cols ? c : cols - 8;
    va[it] = *(const f32x4*)(xr + cc);
    vb[it] = *(const f32x4*)(xr + cc + 4);
  }
  float amax = 0.0f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const bool in = lane * 8 + it * kWave * 8 < cols;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      amax = __builtin_fmaxf(amax, in ? __builtin_fmaxf(__builtin_fabsf(va[it][q]), __builtin_fabsf(vb[it][q])) : 0.0f);
  }
  amax = wave_max(amax);
  const float s = amax > 0.0f ? amax / kE4M3Max : 1.0f;
  const double rs = 1.0 / (double)s;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = lane * 8 + it * kWave * 8;
    if (c >= cols) continue;
    const f32x4 a = va[it], b = vb[it];
    const uint32_t lo = enc2(quot(a[0], rs), quot(a[1], rs)) | (enc2(quot(a[2], rs), quot(a[3], rs)) << 16);
    const uint32_t hi = enc2(quot(b[0], rs), quot(b[1], rs)) | (enc2(quot(b[2], rs), quot(b[3], rs)) << 16);
    *(uint2*)(codes + (size_t)row * ostride + c) = make_uint2(lo, hi);
  }
  zero_tail(codes + (size_t)row * ostride, cols, ostride, lane);
  if (lane == 0) scales[row] = s;
}

// ---------------------------------------------------------------- y in fp16

// Exponent ey for a group of y values whose largest magnitude has float bits m: the values
// are stored as fp16 of v * 2^-ey, which puts the largest in [2^14, 2^15) (below the fp16
// maximum) and keeps the 11-bit significand for all values within 2^24 of it. ey is kept in
// [-60, 100], so 2^-ey and 2^ey are normal floats; a group that is all zero gets 0.
__device__ __forceinline__ int y_exponent(uint32_t m) {
  if (m == 0u) return 0;
  const int eb = (int)(m >> 23) - 127;  // floor(log2) for normal m; -127 for subnormal m
  const int ey = eb - 14;
  return ey < -60 ? -60 : (ey > 100 ? 100 : ey);
}

// out[t, n] = sum_j w[t, j] * y[t*k + j, n] * 2^e[t*k + j, n/32], slots in order; eight
// consecutive outputs (within one exponent group) per thread, read as one 16-byte load per
// slot, the slots' reads unrolled so several are in flight.
// BIAS: each pair's y also gets its expert's w2 bias (ids give the expert) before the router
// weight is applied.
// With I > 512 a pair's y comes in `parts` planes (K parts), summed first, in plane order.
template <bool BIAS>
__global__ __launch_bounds__(256) void combine_f16_kernel(const _Float16* __restrict__ y,
                                                          const int8_t* __restrict__ yexp,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ bias, int T, int H, int k,
                                                          int parts, void* __restrict__ out, int out_bf16) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const size_t idx = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (idx >= (size_t)T * H) return;
  const size_t t = idx / H, n = idx % H;
  const int EG = mfma_y_groups(H);
  const size_t yplane = (size_t)T * k * H, eplane = (size_t)T * k * EG;
  float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int j = 0; j < k; ++j) {
    const size_t p = t * k + j;
    const float wj = w[p];
    float yv[8];
    {
      const float up = __uint_as_float((uint32_t)(127 + yexp[p * EG + n / kYGroup]) << 23);  // 2^e
      const h8 v = *(const h8*)(y + p * H + n);
#pragma unroll
      for (int q = 0; q < 8; ++q) yv[q] = (float)v[q] * up;
    }
    for (int part = 1; part < parts; ++part) {
      const float up = __uint_as_float((uint32_t)(127 + yexp[part * eplane + p * EG + n / kYGroup]) << 23);
      const h8 v = *(const h8*)(y + part * yplane + p * H + n);
#pragma unroll
      for (int q = 0; q < 8; ++q) yv[q] = __builtin_fmaf((float)v[q], up, yv[q]);
    }
    if constexpr (BIAS) {
      const float* b = bias + (size_t)ids[p] * H + n;
      const f32x4 b0 = *(const f32x4*)b, b1 = *(const f32x4*)(b + 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] = __builtin_fmaf(wj, yv[q] + (q < 4 ? b0[q] : b1[q - 4]), s[q]);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] = __builtin_fmaf(wj, yv[q], s[q]);
    }
  }
  if (out_bf16) {
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (uint32_t)f32_to_bf16(s[2 * q]) | ((uint32_t)f32_to_bf16(s[2 * q + 1]) << 16);
    *(u32x4*)((uint16_t*)out + idx) = u32x4{o[0], o[1], o[2], o[3]};
  } else {
    *(f32x4*)((float*)out + idx) = f32x4{s[0], s[1], s[2], s[3]};
    *(f32x4*)((float*)out + idx + 4) = f32x4{s[4], s[5], s[6], s[7]};
  }
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

// Workgroup -> work item in [0, n), n the number of items of this routing (the grid is an
// upper bound on it). Workgroups are dealt to the 8 XCDs round-robin; XCD x gets items
// x*per .. x*per + per - 1 with per = ceil(n/8), so every XCD gets an equal share and
// consecutive items (the tiles of one expert, the blocks of one tile) stay on one XCD and
// share its L2. Returns n for a workgroup with no item; the grid must hold 8*per of them.
__device__ __forceinline__ int xcd_item(int bid, int n) {
  const int per = (n + 7) / 8;
  const int x = bid & 7, i = bid >> 3;
  const int L = x * per + i;
  return i < per && L < n ? L : n;
}


// ---------------------------------------------------------------- shared tile machinery

// silu with the hardware exp and reciprocal (about 1 ulp each). h feeds a quantiser whose
// decisions the parity check already treats as uncertain within the accumulation error of
// the matrix cores, which is orders of magnitude larger.
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

constexpr int kTM = kMfmaTileM;  // pairs per tile
constexpr int kMaxH = 8192;      // bounds the block-scale slabs staged in LDS
constexpr int kMaxI = 512;       // GEMM2 holds the h codes of up to 4 K blocks (one K part) in registers
constexpr int kMaxIParts = 4096; // I beyond 512 runs GEMM2 in K parts, one y plane each
constexpr int kStages = 3;       // depth of the LDS rings
constexpr int kRowB = 128;       // bytes of one row in one 128-wide K block

// LDS rows hold one 128-byte K block; 16-byte chunk c of row r sits at chunk position
// c ^ (r & 7). Measured on gfx950 (SQ_LDS_BANK_CONFLICT), operand reads of 16 consecutive
// rows at one chunk are conflict-free with this swizzle, while c ^ ((r ^ (r >> 3)) & 7)
// costs four conflict cycles per read and no swizzle twelve.
__device__ __forceinline__ int sw(int r) { return r & 7; }

// One direct global->LDS load: lane j copies 16 bytes from its own address g to
// lds + 16 j (lds wave-uniform). Issued as 8 rows x 128 contiguous bytes per instruction
// (lane j: row j/8, chunk position j%8), the pattern the load path serves at full rate;
// an MFMA operand read straight from global memory would touch 16 rows per instruction.
// Written as inline asm so that the compiler does not track it: its own LDS-DMA tracking
// inserts a full vmcnt(0) wait before LDS reads of other ring slots, which would undo the
// prefetch. Completion is therefore awaited explicitly (wait_vm); waits the compiler adds
// for its own loads can only be stricter. M0 (the LDS base of the DMA) is set here; these
// kernels use M0 for nothing else, and the instruction after an M0 write needs one wait state.
__device__ __forceinline__ void g2lds(const void* g, const uint8_t* lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "memory");
}

// The same with 4 bytes per lane (lane j: lds + 4 j).
__device__ __forceinline__ void g2lds4(const void* g, const uint8_t* lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(a) : "memory");
}

// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence. LDS that direct loads fill is covered by each
// wave's own wait_vm before the barrier; the empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 32 operand bytes (chunks kq and kq + 4 of K block) of row r of a swizzled LDS slab.
__device__ __forceinline__ i32x8 lds_operand(const uint8_t* slab, int r, int kq) {
  const u32x4 lo = *(const u32x4*)(slab + r * kRowB + ((kq ^ sw(r)) << 4));
  const u32x4 hi = *(const u32x4*)(slab + r * kRowB + (((kq + 4) ^ sw(r)) << 4));
  i32x8 o;
  o[0] = (int)lo.x; o[1] = (int)lo.y; o[2] = (int)lo.z; o[3] = (int)lo.w;
  o[4] = (int)hi.x; o[5] = (int)hi.y; o[6] = (int)hi.z; o[7] = (int)hi.w;
  return o;
}

// The block scales of one expert's bank as float in LDS: s[row_block * cols + col_block].
__device__ __forceinline__ void stage_scales(float* s, const BankArg& b, int64_t sb, int rows, int cols) {
  for (int q = threadIdx.x; q < rows * cols; q += 256)
    s[q] = load_scale(b.scales, b.scale_bf16, sb + (int64_t)(q / cols) * b.srow + q % cols);
}

// Block scales as accumulator rescalings. A sum over K blocks sum_kb s_kb * P_kb is kept in
// units of the latest block's scale: before block kb's products are accumulated in place by
// the MFMA, the accumulator is multiplied by s_prev / s_kb, and the final sum is the
// accumulator times the last scale. Real arithmetic gives the same value; float adds one
// rounding of the ratio per block (2^-24 relative), far below the MFMA's own accumulation
// error, and the MFMA results never wait for a VALU multiply. ratio[kb] is 0 for a zero scale
// (that block contributes nothing and is skipped), 1 where the scale does not change.
// One thread per block kb of a sequence: s_prev is the latest nonzero scale before kb, found
// by looking back (one step unless scales are zero); the thread of the final block also
// writes the last nonzero scale (0 if there is none).
__device__ __forceinline__ void scale_ratio(const float* sc, int n, int kb, float* ratio, float* last) {
  const float v = sc[kb];
  float prev = 0.0f;
  for (int j = kb - 1; j >= 0 && prev == 0.0f; --j) prev = sc[j];
  ratio[kb] = v == 0.0f ? 0.0f : (prev == 0.0f ? 1.0f : prev / v);
  if (kb == n - 1) *last = v != 0.0f ? v : prev;
}

// ---------------------------------------------------------------- GEMM1

// One workgroup per (expert, 128-pair tile, 128-feature block fb of h), 8 waves: two per
// SIMD, so that one wave's LDS reads and copies proceed under the other's MFMAs (a single
// wave serialises them). Wave w multiplies gate features fb*128 + 32(w%4) .. +32 (two 16-row
// MFMA tiles) and the matching up features by tokens 64(w/4) .. +64 of the tile. Every
// 128-wide K block is a stage of a 3-deep LDS ring, filled by direct loads shared out over
// the waves (weight rows of a feature quarter by the two waves that multiply them, the tile's
// 128 token rows by all eight); one barrier per stage. The operands of the next stage are
// read into registers while the current one is multiplied. A = weight rows (features),
// B = token rows, so lane (r16, kq) of a 16x16 result holds features 4kq..4kq+3 of token
// r16. h = silu(g)*u is written in float, [sorted pair, I]; GEMM2 quantises it per row.
//
// GROUP: x carries one scale per (token, 128-column group) xs[T, H/128], the group of each
// K block, so the scale of a block product differs per token: every MFMA starts from zero
// and its product is scaled into the accumulator by (weight block scale) x (the token's
// group scale) on the VALU. The stage's group scales of the tile's tokens travel with the
// stage in the ring (one 4-byte direct load per wave). h is then quantised in the epilogue,
// one scale per (pair, 128-feature group) = this workgroup's feature block: the group's amax
// is a maximum over the four waves holding its features (through LDS), scale = amax/448
// (float division, 1 if zero), codes = e4m3(h / scale); codes go to hq [sorted pair, I] and
// scales to hs [sorted pair, I/128]. Needs H and I multiples of 128.
template <bool GROUP>
__global__ __launch_bounds__(512, 1) void gemm1_mfma_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                            BankArg w13, Plan plan, int E, int H, int I, int k,
                                                            int nblocks, float* __restrict__ hf,
                                                            uint8_t* __restrict__ hq, float* __restrict__ hs) {
  constexpr int TM = kTM;                 // pairs per tile
  constexpr int NTT = 4;                  // token tiles per wave (64 tokens)
  constexpr int NF = 4;                   // weight tiles per wave: 2 gate + 2 up
  constexpr int QB = 64 * kRowB;          // one feature quarter's weight rows of a stage
  constexpr int XB = TM * kRowB;          // the tile's x rows of a stage
  // GROUP: the group scales of the tile's 128 token rows for the stage's K block; wave w's
  // load puts rows 16w .. 16w+15 at 256w (lane j copies row 16w + j%16 to 256w + 4j)
  constexpr int XSB = GROUP ? 8 * 256 : 0;
  constexpr int SB = 4 * QB + XB + XSB;   // one stage
  constexpr int LPW = GROUP ? 7 : 6;      // direct loads per wave per stage
  __shared__ __align__(16) uint8_t ring[kStages * SB];
  __shared__ float s_am[GROUP ? 4 * TM : 1];  // GROUP: per (feature quarter, tile row) h maxima
  // block scales, their ratios and last values of three row blocks: the gate rows' block and
  // the (up to) two blocks the up rows fall in (one unless I % 128 != 0)
  __shared__ float s_sc[3 * (kMaxH / 128)];
  __shared__ float s_rt[3 * (kMaxH / 128)];
  __shared__ float s_last[3];
  __shared__ int s_tok[TM];

  const int nfb = mfma_pad(I) / 128;
  const int nitems = plan.tile_off[E] * nfb;
  const int L = xcd_item(blockIdx.x, nitems);  // consecutive L share an expert's rows and a tile's x
  if (L >= nitems) return;
  const int tile = L / nfb, fb = L - tile * nfb;
  const int e = find_expert(plan.tile_off, E, tile);
  const int pos0 = plan.offsets[e] + (tile - plan.tile_off[e]) * TM;
  const int pos_end = plan.offsets[e + 1];
  const int nvalid = pos_end - pos0 < TM ? pos_end - pos0 : TM;
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int fq = wave & 3, th = wave >> 2;  // feature quarter, token half
  // a token half with no pair of the expert (in an expert's partial last tile) skips its
  // products; it still copies, reads and meets the barriers like the others
  const bool idle = th * 64 >= nvalid;  // wave-uniform
  const int r16 = lane & 15, kq = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;
  const uint8_t* wb = w13.codes + (size_t)e * w13.expert_stride;
  const int Hp = mfma_pad(H);  // x code rows, zero past H
  const int nkb = Hp / 128;
  // scale row blocks: the gate rows' (fb) and the up rows' first and last (rows past 2I in
  // the last feature block are clamped, so the block index is too)
  const int bu0 = (I + fb * 128) / 128;
  const int bumax = (2 * I - 1) / 128;

  // token of each tile row (rows past the expert's pairs repeat the first token; their
  // results are never stored) and the gate / up block scales of this feature block
  if (tid < TM) s_tok[tid] = plan.sorted[pos0 + (tid < nvalid ? tid : 0)] / k;
  if (tid < 3 * nkb) {
    const int sq = tid / nkb, kb = tid - sq * nkb;
    const int rb = sq == 0 ? fb : min(bu0 + sq - 1, bumax);
    s_sc[tid] = load_scale(w13.scales, w13.scale_bf16, (int64_t)e * w13.sexp + (int64_t)rb * w13.srow + kb);
  }
  __syncthreads();
  if (tid < 3 * nkb) {
    const int sq = tid / nkb;
    scale_ratio(s_sc + sq * nkb, nkb, tid - sq * nkb, s_rt + sq * nkb, s_last + sq);
  }
  __syncthreads();

  // direct-load sources. Quarter fq's 64 weight rows (0..31 gate, 32..63 up) are copied 8 rows
  // at a time: this wave takes copies 4th .. 4th+3. x copies: this wave takes tile rows
  // 16w .. 16w+15. K block kb adds kb*128 bytes.
  // rows past I (gate) or 2I (up) in the last feature block read the last valid row; their
  // results are never stored
  uint32_t wrow[4], wch[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = (th * 4 + j) * 8 + lr;
    const int row = b < 32 ? min(fb * 128 + fq * 32 + b, I - 1) : min(I + fb * 128 + fq * 32 + b - 32, 2 * I - 1);
    wrow[j] = (uint32_t)row * (uint32_t)H;
    wch[j] = (uint32_t)((lc ^ sw(b)) << 4);
  }
  // a partial last K block: chunks past the row end read the row's last chunk (finite codes,
  // multiplied by the zero x codes there)
  const uint32_t ktail = (uint32_t)(H - (nkb - 1) * 128);  // bytes of the last K block
  const uint8_t* xsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wave * 16 + j * 8 + lr;
    xsrc[j] = xq + (size_t)s_tok[r] * Hp + ((lc ^ sw(r)) << 4);
  }
  // GROUP: this lane's token row's group scales (row 16w + lane%16)
  const float* xsrow = GROUP ? xs + (size_t)s_tok[wave * 16 + r16] * nkb : xs;
  auto copy = [&](int kb, int j) {  // this wave's copy j (0 .. LPW-1) of stage kb
    uint8_t* slot = ring + (kb % kStages) * SB;
    if (j < 4) {
      const uint32_t ch = kb == nkb - 1 && wch[j] >= ktail ? ktail - 16 : wch[j];
      g2lds(wb + kb * 128 + wrow[j] + ch, slot + fq * QB + (th * 4 + j) * 1024);
    } else if (j < 6) {
      g2lds(xsrc[j - 4] + kb * 128, slot + 4 * QB + (wave * 16 + (j - 4) * 8) * kRowB);
    } else {
      g2lds4(xsrow + kb, slot + 4 * QB + XB + wave * 256);
    }
  };
  float xsc[NTT];  // x scale of token 64th + tt*16 + r16 (per-row x only)
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) xsc[tt] = GROUP ? 1.0f : xs[s_tok[th * 64 + tt * 16 + r16]];

  // Operands of one K block in registers: this wave's token rows (B) and weight rows (A),
  // and with GROUP the group scales of its tokens for that block.
  struct Ops {
    i32x8 bx[NTT];
    i32x8 wa[NF];
    float sx[GROUP ? NTT : 1];
  };
  // the group scale of tile row th*64 + t*16 + r16 in a stage slot
  auto read_sx = [&](const uint8_t* slot, int t) {
    return *(const float*)(slot + 4 * QB + XB + (th * 4 + t) * 256 + r16 * 4);
  };
  f32x4 acc[NF][NTT];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[f][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // Stage kb + 1 is read into registers while stage kb is multiplied. At step kb: this wave's
  // copies of stage kb + 1 are in, the barrier makes everyone's visible and shows every wave
  // has read stage kb into registers (its LDS reads waited for), so stage kb's slot is
  // refilled with stage kb + 3. Copies, reads and MFMAs go in two interleaved groups.
  // the scale sequence of each up tile (the gate tiles use sequence 0): rows I + fb*128 +
  // 32fq + 16(f-2) .. +15 lie in one 128-row block (I is a multiple of 16)
  int squ[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) squ[f] = 1 + min((I + fb * 128 + fq * 32 + f * 16) / 128, bumax) - bu0;
  auto step = [&](int kb, const Ops& cur, Ops& nxt) {
    // the scale ratios (GROUP: the block scales) first, so that the explicit LDS wait below
    // covers them too
    const float* sq = GROUP ? s_sc : s_rt;
    const float rs[4] = {sq[kb], sq[kb], sq[squ[0] * nkb + kb], sq[squ[1] * nkb + kb]};
    if (kb + 1 < nkb) {
      if (kb + 2 < nkb) wait_vm<LPW>();
      else wait_vm<0>();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage kb are done
      bar();
    }
    const bool refill = kb + 3 < nkb;
    // the next stage's operands; on the last step this rereads a settled slot (unused), which
    // keeps LDS reads out of branches so the compiler's waits stay exact
    const uint8_t* rslot = ring + ((kb + 1) % kStages) * SB;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (refill) {
#pragma unroll
        for (int j = 3 * g; j < 3 * g + 3; ++j) copy(kb + 3, j);
        if (GROUP && g == 1) copy(kb + 3, 6);
      }
#pragma unroll
      for (int t = 2 * g; t < 2 * g + 2; ++t) {
        nxt.bx[t] = lds_operand(rslot + 4 * QB, th * 64 + t * 16 + r16, kq);
        nxt.wa[t] = lds_operand(rslot + fq * QB, t * 16 + r16, kq);
        if constexpr (GROUP) nxt.sx[t] = read_sx(rslot, t);
      }
      // gate tiles in group 0, up tiles in group 1
      if (idle) {
      } else if constexpr (GROUP) {
        // the group's 8 products, each MFMA issued before the previous one's result is
        // scaled in (a zero block scale gives a zero factor: finite products add nothing)
        constexpr int NJ = 2 * NTT;
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 pp = mfma_fp8(cur.wa[2 * g], cur.bx[0], z);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int f = 2 * g + j / NTT, tt = j % NTT;
          f32x4 nx;
          if (j + 1 < NJ) nx = mfma_fp8(cur.wa[2 * g + (j + 1) / NTT], cur.bx[(j + 1) % NTT], z);
          const float c = rs[f] * cur.sx[tt];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[f][tt][q] = __builtin_fmaf(c, pp[q], acc[f][tt][q]);
          if (j + 1 < NJ) pp = nx;
        }
      } else {
#pragma unroll
        for (int f = 2 * g; f < 2 * g + 2; ++f) {
          const float r = rs[f];  // uniform
          if (r != 0.0f) {        // a zero block scale adds nothing
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[f][tt][q] *= r;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) acc[f][tt] = mfma_fp8(cur.wa[f], cur.bx[tt], acc[f][tt]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#pragma unroll
  for (int j = 0; j < LPW; ++j) copy(0, j);
  if (nkb > 1) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) copy(1, j);
  }
  if (nkb > 2) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) copy(2, j);
  }
  if (nkb > 2) wait_vm<2 * LPW>();
  else if (nkb > 1) wait_vm<LPW>();
  else wait_vm<0>();
  bar();
  Ops o0, o1;
  {
    const uint8_t* rslot = ring;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o0.bx[t] = lds_operand(rslot + 4 * QB, th * 64 + t * 16 + r16, kq);
      o0.wa[t] = lds_operand(rslot + fq * QB, t * 16 + r16, kq);
      if constexpr (GROUP) o0.sx[t] = read_sx(rslot, t);
    }
  }
  for (int kb = 0; kb < nkb; kb += 2) {
    step(kb, o0, o1);
    if (kb + 1 < nkb) step(kb + 1, o1, o0);
  }
  // the MLP bias of this lane's gate and up features (w13's bias: gate half, then up half);
  // without a bias the reads go to an in-bounds address and are dropped, as are those of
  // features past I (read at the last valid ones)
  const bool hb = w13.bias != nullptr;
  const float* bb = hb ? w13.bias + (size_t)e * 2 * I : (const float*)w13.codes;
  f32x4 bgv[2], buv[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int i = min(fb * 128 + fq * 32 + f * 16 + kq * 4, I - 4);
    bgv[f] = *(const f32x4*)(bb + (hb ? i : 0));
    buv[f] = *(const f32x4*)(bb + (hb ? I + i : 0));
  }
  // h of gate tile f (features fb*128 + 32fq + 16f + 4kq .. +3) for token 64th + 16tt + r16
  if constexpr (GROUP) {
    // the accumulators hold the scaled sums; h of every row (rows past the expert's pairs
    // too: every lane takes part in the maxima and the barrier; their stores are skipped)
    f32x4 hv[NTT][2];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      float m = 0.0f;
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float g = acc[f][tt][q];
          float u = acc[f + 2][tt][q];
          if (hb) {
            g += bgv[f][q];
            u += buv[f][q];
          }
          hv[tt][f][q] = silu_fast(g) * u;
          m = __builtin_fmaxf(m, __builtin_fabsf(hv[tt][f][q]));
        }
      // over the four K-quarter lanes of the token: the wave's 32 features
      m = __builtin_fmaxf(m, __shfl_xor(m, 16, kWave));
      m = __builtin_fmaxf(m, __shfl_xor(m, 32, kWave));
      if (kq == 0) s_am[fq * TM + th * 64 + tt * 16 + r16] = m;
    }
    __syncthreads();
    const int ng = I / 128;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int row = th * 64 + tt * 16 + r16;
      const int pos = pos0 + row;
      const float amax = __builtin_fmaxf(__builtin_fmaxf(s_am[row], s_am[TM + row]),
                                         __builtin_fmaxf(s_am[2 * TM + row], s_am[3 * TM + row]));
      const float sc = amax > 0.0f ? amax / kE4M3Max : 1.0f;
      const double rsc = 1.0 / (double)sc;
      if (pos >= pos_end) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int i = fb * 128 + fq * 32 + f * 16 + kq * 4;
        const f32x4 v = hv[tt][f];
        const uint32_t c4 = enc2(quot(v[0], rsc), quot(v[1], rsc)) | (enc2(quot(v[2], rsc), quot(v[3], rsc)) << 16);
        *(uint32_t*)(hq + (size_t)pos * I + i) = c4;
      }
      if (fq == 0 && kq == 0) hs[(size_t)pos * ng + fb] = sc;
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int pos = pos0 + th * 64 + tt * 16 + r16;
      if (pos >= pos_end) continue;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int i = fb * 128 + fq * 32 + f * 16 + kq * 4;  // features i .. i+3, all < I or none
        if (i >= I) continue;
        f32x4 h;
        const float gs = s_last[0] * xsc[tt], us = s_last[squ[f]] * xsc[tt];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float g = acc[f][tt][q] * gs;
          float u = acc[f + 2][tt][q] * us;
          if (hb) {
            g += bgv[f][q];
            u += buv[f][q];
          }
          h[q] = silu_fast(g) * u;
        }
        *(f32x4*)(hf + (size_t)pos * I + i) = h;
      }
    }
  }
}

// ---------------------------------------------------------------- GEMM2

// A work item is one 64-pair half of an expert's 128-pair tile, or a share of its output
// chunks when the grid has room (a tile's workgroups are consecutive items on one XCD, so
// they read the expert's w2 from L2 after the first): R = min(2, grid / (2 * tiles)) workgroups
// per half of a tile with two non-empty halves, 2R on the one half of a tile that has a
// single one, taking chunks c with c % (workgroups of the half) == their index. 4 waves, one
// per SIMD. A = w2 rows (features), B = the half's h codes (pairs as rows; e4m3 per (token,
// slot) row, scale amax/448, from the row quantiser), so lane (r16, kq) of a 16x16 result
// holds outputs 4kq..4kq+3 of pair r16: four consecutive outputs of one pair, written with
// one 8-byte store. The H outputs go in chunks of 256; wave w multiplies outputs 64w ..
// 64w+63 of each of its chunks (4 feature tiles) by the half's 64 pairs (4 pair tiles, whose
// h codes stay in registers for every K block). Each wave streams its own w2 rows, (chunk, K
// block) after (chunk, K block), through a private kRing2-deep LDS ring with kRing2 - 1
// stages in flight and no barriers. The workgroups of an expert read its w2 rows in the same
// order at about the same time, so one fetch into L2 serves all of them (measured on gfx950:
// starting each at a different chunk fetched 2.4 times the bytes from beyond L2 for no clear
// gain). Each MFMA starts from zero and its block product is scaled into the accumulator on
// the VALU while the next MFMA runs. Each pair's y row = s_h * W2 h is written once, in fp16
// with one power-of-two exponent per kYGroup (32) outputs; the combine kernel applies the
// router weights. (Measured on gfx950: 128 pairs per workgroup, a ring shared by the four
// waves, or two waves per SIMD were no faster; the w2 stream is held back by the vector
// memory path's pending-miss stalls, not by the bytes per MFMA.)
constexpr int kRing2 = 4;
constexpr int kG2PairTiles = 4;  // pair tiles per workgroup (16 pairs each)

// Wait for the copy of the stage issued `later` stages before the newest one: the loads of
// the `later` younger stages (PER each) may stay outstanding. Loads complete in issue order,
// so the count is exact for them; stores issued meanwhile (they may complete out of order)
// can only make the wait longer, never shorter.
template <int PER>  // loads per stage
__device__ __forceinline__ void wait_stage(int later) {
  if (later >= 3) wait_vm<3 * PER>();
  else if (later == 2) wait_vm<2 * PER>();
  else if (later == 1) wait_vm<PER>();
  else wait_vm<0>();
}

// GROUP: h carries one scale per (pair, 128-feature group) hs[P, I/128] (from GEMM1's
// epilogue), so the factor a block product takes is (w2 block scale) x (the pair's group
// scale for that block), per lane; the pair's y needs no final scale.
template <int KB, int NP, bool GROUP>  // K blocks of this part, pair tiles per workgroup (NP * 16 pairs)
__global__ __launch_bounds__(256, 1) void gemm2_mfma_kernel(const uint8_t* __restrict__ hq, const float* __restrict__ hs,
                                                            BankArg w2, Plan plan, int E,
                                                            int H, int I, int nblocks, int kb0, _Float16* __restrict__ y,
                                                            int8_t* __restrict__ yexp) {
  // this launch multiplies K blocks kb0 .. kb0 + KB - 1 of h and w2 (a part of K when
  // I > 512) and writes that part's y plane; y and yexp point at the plane
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  constexpr int TP = NP * 16;      // pairs per workgroup
  constexpr int PARTS = kTM / TP;  // workgroups per 128-pair tile
  constexpr int NW = 4;            // waves, one per SIMD
  constexpr int NF = 4;            // feature tiles per wave (64 outputs)
  constexpr int FW = NF * 16;      // outputs per wave and chunk
  constexpr int NCH = NW * FW;     // outputs per chunk
  constexpr int WB = FW * kRowB;   // one wave's w2 rows of a stage
  constexpr int HB = TP * kRowB;   // the workgroup's h codes of one K block
  static_assert(KB * HB <= NW * kRing2 * WB, "the h codes are staged in the ring");
  static_assert(kRing2 - 1 <= 3, "wait_stage covers up to three younger stages");
  __shared__ __align__(16) uint8_t ring[NW * kRing2 * WB];
  __shared__ float s_sc[(kMaxH / 128) * (kMaxI / 128)];
  __shared__ float s_hs[GROUP ? TP * KB : TP];  // GROUP: [pair][K block of this part]
  __shared__ int s_prow[TP];

  // Each 128-pair tile gets 2R workgroups (R = 2 where the grid, a bound on the tiles, has
  // room for it, else 1). When both 64-pair halves of the tile hold pairs, R of them take
  // each half; when only the first does (an expert's last, small tile, which is every tile
  // of a small batch), all 2R take that half. The workgroups of a half split its chunks of
  // output rows (chunk c goes to the one with c % RS == rsi), so a small batch does not
  // leave each expert's whole w2 stream to one CU.
  static_assert(PARTS == 2, "two half-tiles per tile");
  const int ntiles = plan.tile_off[E];
  const int R = max(1, min(2, (int)gridDim.x / max(2 * ntiles, 1)));
  const int nitems = ntiles * 2 * R;
  const int L = xcd_item(blockIdx.x, nitems);  // consecutive items of an expert share its w2 in L2
  if (L >= nitems) return;
  const int tile = L / (2 * R), sub = L - tile * 2 * R;
  const int e = find_expert(plan.tile_off, E, tile);
  const int t0 = plan.offsets[e] + (tile - plan.tile_off[e]) * kTM;  // the tile's first pair
  const int pos_end = plan.offsets[e + 1];
  const bool two = pos_end - t0 > TP;  // both halves hold pairs
  const int part = two ? sub / R : 0;
  const int RS = two ? R : 2 * R, rsi = two ? sub - part * R : sub;
  const int pos0 = t0 + part * TP;
  const int nvalid = pos_end - pos0 < TP ? pos_end - pos0 : TP;
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r16 = lane & 15, kq = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;
  const uint8_t* wb = w2.codes + (size_t)e * w2.expert_stride;

  const int Ip = mfma_pad(I);  // h code rows, zero past I
  stage_scales(s_sc, w2, (int64_t)e * w2.sexp + kb0, (H + 127) / 128, KB);
  if (tid < TP) {
    const bool ok = tid < nvalid;
    if constexpr (!GROUP) s_hs[tid] = hs[pos0 + (ok ? tid : 0)];
    s_prow[tid] = ok ? plan.sorted[pos0 + tid] : -1;
  }
  if constexpr (GROUP) {
    const int ng = Ip / 128;  // h groups per pair
    for (int q = tid; q < TP * KB; q += 256) {
      const int r = q / KB, kb = q - r * KB;
      s_hs[q] = hs[(size_t)(pos0 + (r < nvalid ? r : 0)) * ng + kb0 + kb];
    }
  }
  // the h codes into the ring space: (TP / 8) * KB copies of 8 rows x 128 bytes, a quarter
  // per wave (rows past the expert's pairs copy the first row; their results are never stored)
  constexpr int RG = TP / 8;  // 8-row groups
  static_assert((RG * KB) % NW == 0, "every wave copies the same number of row groups");
#pragma unroll
  for (int i = 0; i < RG * KB / NW; ++i) {
    const int q = wave + NW * i;
    const int kb = q / RG, r = (q % RG) * 8 + lr;
    const int rr = r < nvalid ? r : 0;
    g2lds(hq + (size_t)(pos0 + rr) * Ip + (kb0 + kb) * 128 + ((lc ^ sw(r)) << 4), ring + kb * HB + (q % RG) * 1024);
  }
  wait_vm<0>();  // everyone's h codes, scales and pair rows are in after the barrier
  __syncthreads();
  // pair tiles with no valid pair (in a tile's last, partial tile) are multiplied anyway
  // (rows past the expert's pairs hold the first row's codes) and their results dropped
  const int npt = min(NP, (nvalid + 15) / 16);
  i32x8 bh[KB][NP];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int pt = 0; pt < NP; ++pt) bh[kb][pt] = lds_operand(ring + kb * HB, pt * 16 + r16, kq);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's h reads are done
  __syncthreads();                     // and everyone's, before the ring is refilled

  // chunks holding outputs of this wave: those with c * NCH + FW * wave < H (the last one
  // may hold fewer than FW: H is a multiple of 16, so each feature tile is in range or out);
  // this workgroup takes c = rsi, rsi + RS, ...
  const int nch = (H - wave * FW + NCH - 1) / NCH;
  const int nchr = nch > rsi ? (nch - rsi + RS - 1) / RS : 0;
  const int nst = nchr * KB;
  // w2 copy i covers rows 8i .. 8i+7 of the wave's FW; chunk c adds c * NCH rows. Rows past H
  // read the last row and chunks past a partial last K block the row's last chunk (finite
  // codes, multiplied by the zero h codes there); neither result is stored.
  constexpr int NCP = FW / 8;  // copies per wave and stage
  uint32_t wch[NCP], woff[NCP];
#pragma unroll
  for (int i = 0; i < NCP; ++i) {
    wch[i] = (uint32_t)((lc ^ sw(i * 8 + lr)) << 4);
    woff[i] = (uint32_t)(wave * FW + i * 8 + lr) * (uint32_t)I + wch[i];
  }
  const int nkb_all = Ip / 128;
  const uint32_t ktail = (uint32_t)(I - (nkb_all - 1) * 128);  // bytes of the last K block
  uint8_t* myring = ring + wave * kRing2 * WB;
  auto issue = [&](int st) {
    const int ci = st / KB, kb = st - ci * KB;
    const int c = rsi + ci * RS;
    uint8_t* slot = myring + (st % kRing2) * WB;
    const bool ptail = kb0 + kb == nkb_all - 1 && ktail < 128;  // uniform
    if (!ptail && c * NCH + wave * FW + FW <= H) {
      const uint8_t* src = wb + (size_t)c * NCH * I + (kb0 + kb) * 128;
#pragma unroll
      for (int i = 0; i < NCP; ++i) g2lds(src + woff[i], slot + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NCP; ++i) {
        const int row = min(c * NCH + wave * FW + i * 8 + lr, H - 1);
        const uint32_t ch = ptail && wch[i] >= ktail ? ktail - 16 : wch[i];
        g2lds(wb + (size_t)row * I + (kb0 + kb) * 128 + ch, slot + i * 1024);
      }
    }
  };
#pragma unroll
  for (int st = 0; st < kRing2 - 1; ++st)
    if (st < nst) issue(st);
  f32x4 acc[NF][NP];
  // (this workgroup's chunk ci, K block kb) is stage st = ci * KB + kb; kb is unrolled so
  // that the h operands are indexed statically and stay in registers
  for (int ci = 0; ci < nchr; ++ci) {
    const int c = rsi + ci * RS;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int st = ci * KB + kb;
      // stage st has landed once at most min(kRing2 - 2, nst - 1 - st) younger stages remain
      wait_stage<NCP>(min(kRing2 - 2, nst - 1 - st));
      // the slot of stage st - 1 is refilled next, so this wave's reads of it must have
      // completed: the compiler waits for them only where their values are used, which it may
      // schedule after this refill, and nothing orders a pending LDS read before direct loads
      // into the same bytes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (st + kRing2 - 1 < nst) issue(st + kRing2 - 1);
      if (kb == 0) {
#pragma unroll
        for (int ft = 0; ft < NF; ++ft)
#pragma unroll
          for (int pt = 0; pt < NP; ++pt) acc[ft][pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      const uint8_t* slot = myring + (st % kRing2) * WB;
      i32x8 aw[NF];
#pragma unroll
      for (int ft = 0; ft < NF; ++ft) aw[ft] = lds_operand(slot, ft * 16 + r16, kq);
      const int n0 = c * NCH + wave * FW;
      // outputs n0 .. n0 + FW - 1 share one 128-row scale block
      const float sc = s_sc[(n0 / kScaleBlock) * KB + kb];  // uniform
      // the factor of each pair tile's products (GROUP: times the lane's pair's group scale)
      float cp[NP];
#pragma unroll
      for (int pt = 0; pt < NP; ++pt) cp[pt] = GROUP ? sc * s_hs[(pt * 16 + r16) * KB + kb] : sc;
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      {
        f32x4 pp = mfma_fp8(aw[0], bh[kb][0], z);
#pragma unroll
        for (int j = 0; j < NF * NP; ++j) {
          const int ft = j / NP, pt = j % NP;
          f32x4 nx;
          if (j + 1 < NF * NP) nx = mfma_fp8(aw[(j + 1) / NP], bh[kb][(j + 1) % NP], z);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[ft][pt][q] = __builtin_fmaf(cp[pt], pp[q], acc[ft][pt][q]);
          if (j + 1 < NF * NP) pp = nx;
        }
      }
      if (kb == KB - 1) {
        // y of pair 16pt + r16, outputs n0 + 16ft + 4kq .. +3, in fp16 with one exponent per
        // kYGroup outputs of the pair (GT feature tiles, held by lanes r16 + 16 kq); feature
        // tiles past H are left out of the exponent and not stored
        constexpr int GT = kYGroup / 16;
        static_assert(NF % GT == 0, "a wave's outputs are whole exponent groups");
        const int EG = mfma_y_groups(H);
#pragma unroll
        for (int pt = 0; pt < NP; ++pt) {
          if (pt < npt) {
            const int rl = pt * 16 + r16;
            const int prow = s_prow[rl];
            const float hsc = GROUP ? 1.0f : s_hs[rl];
#pragma unroll
            for (int g = 0; g < NF / GT; ++g) {
              float v[GT][4];
              uint32_t m = 0u;  // bits of the largest |v| (non-negative floats order as integers)
#pragma unroll
              for (int f = 0; f < GT; ++f) {
                const bool in = n0 + (g * GT + f) * 16 < H;  // uniform
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  v[f][q] = acc[g * GT + f][pt][q] * hsc;
                  if (in) m = max(m, __float_as_uint(__builtin_fabsf(v[f][q])));
                }
              }
              m = max(m, (uint32_t)__shfl_xor((int)m, 16, kWave));
              m = max(m, (uint32_t)__shfl_xor((int)m, 32, kWave));
              const int ey = y_exponent(m);
              const float down = __uint_as_float((uint32_t)(127 - ey) << 23);  // 2^-ey, exact
              if (prow >= 0 && n0 + g * kYGroup < H) {
#pragma unroll
                for (int f = 0; f < GT; ++f) {
                  if (n0 + (g * GT + f) * 16 >= H) continue;
                  const h4 o = {(_Float16)(v[f][0] * down), (_Float16)(v[f][1] * down),
                                (_Float16)(v[f][2] * down), (_Float16)(v[f][3] * down)};
                  *(h4*)(y + (size_t)prow * H + n0 + (g * GT + f) * 16 + kq * 4) = o;
                }
                if (kq == 0) yexp[(size_t)prow * EG + n0 / kYGroup + g] = (int8_t)ey;
              }
            }
          }
        }
      }
    }
  }
}
template <int KB, int NP, bool GROUP>
hipError_t g2m(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int nblocks, int H,
               int I, int kb0, _Float16* y, int8_t* yexp, hipStream_t s) {
  launch_kernel(gemm2_mfma_kernel<KB, NP, GROUP>, dim3(nblocks), dim3(256), 0, s, hq, hs, w2, plan, E, H, I, nblocks,
                kb0, y, yexp);
  return hipGetLastError();
}

// GEMM2 over its K parts of up to four 128-wide blocks, each into its own y plane.
template <bool GROUP>
hipError_t gemm2_parts(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int P, int H,
                       int I, _Float16* y, int8_t* yexp, hipStream_t s) {
  // two workgroups per half-tile at most; for small batches (few tiles, most of them an
  // expert's only, small one) the grid leaves room for them
  const int nb = (int)mfma_tiles_bound(P, E) * (kTM / (kG2PairTiles * 16));
  const int nblocks = nb < 1024 ? 2 * nb : nb;
  const int nkb = mfma_pad(I) / 128;
  for (int part = 0; part < mfma_k_parts(I); ++part) {
    const int kb0 = part * kMfmaPartBlocks;
    const int kbn = nkb - kb0 < kMfmaPartBlocks ? nkb - kb0 : kMfmaPartBlocks;
    _Float16* yp = y + (size_t)part * P * H;
    int8_t* ep = yexp + (size_t)part * P * mfma_y_groups(H);
    hipError_t err;
    switch (kbn) {
      case 1: err = g2m<1, kG2PairTiles, GROUP>(hq, hs, w2, plan, E, nblocks, H, I, kb0, yp, ep, s); break;
      case 2: err = g2m<2, kG2PairTiles, GROUP>(hq, hs, w2, plan, E, nblocks, H, I, kb0, yp, ep, s); break;
      case 3: err = g2m<3, kG2PairTiles, GROUP>(hq, hs, w2, plan, E, nblocks, H, I, kb0, yp, ep, s); break;
      default: err = g2m<4, kG2PairTiles, GROUP>(hq, hs, w2, plan, E, nblocks, H, I, kb0, yp, ep, s); break;
    }
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

// Upper bound on the tiles of any routing (sum over experts of ceil(count/128) <=
// P/128 + E), rounded up to a multiple of 8; a grid of bound * (items per tile) workgroups
// covers 8 * ceil(n/8) for any n items of a routing.
size_t mfma_tiles_bound(int P, int E) {
  const size_t b = (size_t)(P + kTM - 1) / kTM + (size_t)E;
  return (b + 7) / 8 * 8;
}

bool mfma_shape_ok(int H, int I) {
  return H % 16 == 0 && H > 0 && H <= kMaxH && I % 16 == 0 && I > 0 && I <= kMaxIParts;
}

bool mfma_groups_shape_ok(int H, int I) { return mfma_shape_ok(H, I) && H % 128 == 0 && I % 128 == 0; }

int mfma_k_parts(int I) { return (mfma_pad(I) / 128 + kMfmaPartBlocks - 1) / kMfmaPartBlocks; }

// Pieces of 8 values per lane, 512 columns per wave and piece; rows of up to 8192 columns.
#define MOE_QUANT_LAUNCH(KERNEL, T)                                                                          \
  static hipError_t launch_##KERNEL(const T* x, int rows, int cols, int ostride, uint8_t* codes,            \
                                    float* scales, hipStream_t s) {                                          \
    const dim3 grid((rows + 3) / 4), block(256);                                                             \
    const int it = (cols + kWave * 8 - 1) / (kWave * 8);                                                     \
    if (ostride < cols || ostride - cols >= kWave * 8 || ostride % 8 != 0) return hipErrorInvalidValue;      \
    if (it <= 1) launch_kernel(KERNEL<1>, grid, block, 0, s, x, rows, cols, ostride, codes, scales);          \
    else if (it <= 2) launch_kernel(KERNEL<2>, grid, block, 0, s, x, rows, cols, ostride, codes, scales);     \
    else if (it <= 4) launch_kernel(KERNEL<4>, grid, block, 0, s, x, rows, cols, ostride, codes, scales);     \
    else if (it <= 8) launch_kernel(KERNEL<8>, grid, block, 0, s, x, rows, cols, ostride, codes, scales);     \
    else if (it <= 16) launch_kernel(KERNEL<16>, grid, block, 0, s, x, rows, cols, ostride, codes, scales);   \
    else return hipErrorInvalidValue;                                                                        \
    return hipGetLastError();                                                                                \
  }
MOE_QUANT_LAUNCH(quant_rows_bf16_kernel, uint16_t)
MOE_QUANT_LAUNCH(quant_rows_f32_kernel, float)
#undef MOE_QUANT_LAUNCH

hipError_t launch_quant_rows_bf16(const uint16_t* x, int rows, int cols, int ostride, uint8_t* codes, float* scales,
                                  hipStream_t s) {
  return launch_quant_rows_bf16_kernel(x, rows, cols, ostride, codes, scales, s);
}

hipError_t launch_quant_rows_f32(const float* x, int rows, int cols, int ostride, uint8_t* codes, float* scales,
                                 hipStream_t s) {
  return launch_quant_rows_f32_kernel(x, rows, cols, ostride, codes, scales, s);
}

hipError_t launch_quant_groups_bf16(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                                   hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
  const int it = (cols + kWave * 8 - 1) / (kWave * 8);
  if (cols <= 0 || cols % 128 != 0) return hipErrorInvalidValue;
  if (it <= 1) launch_kernel(quant_groups_bf16_kernel<1>, grid, block, 0, s, x, rows, cols, codes, scales);
  else if (it <= 2) launch_kernel(quant_groups_bf16_kernel<2>, grid, block, 0, s, x, rows, cols, codes, scales);
  else if (it <= 4) launch_kernel(quant_groups_bf16_kernel<4>, grid, block, 0, s, x, rows, cols, codes, scales);
  else if (it <= 8) launch_kernel(quant_groups_bf16_kernel<8>, grid, block, 0, s, x, rows, cols, codes, scales);
  else if (it <= 16) launch_kernel(quant_groups_bf16_kernel<16>, grid, block, 0, s, x, rows, cols, codes, scales);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_combine_f16(const _Float16* y, const int8_t* yexp, const float* w, const int32_t* ids,
                              const float* bias, int T, int H, int k, int parts, void* out, int out_bf16,
                              hipStream_t s) {
  const size_t n = (size_t)T * H / 8;
  if (bias != nullptr)
    launch_kernel(combine_f16_kernel<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, yexp, w, ids,
                  bias, T, H, k, parts, out, out_bf16);
  else
    launch_kernel(combine_f16_kernel<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, yexp, w, ids,
                  bias, T, H, k, parts, out, out_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm1_mfma(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E, int P,
                             int H, int I, int k, float* hf, hipStream_t s) {
  if (!mfma_shape_ok(H, I)) return hipErrorInvalidValue;
  const int nblocks = (int)mfma_tiles_bound(P, E) * (mfma_pad(I) / 128);
  launch_kernel(gemm1_mfma_kernel<false>, dim3(nblocks), dim3(512), 0, s, xq, xs, w13, plan, E, H, I, k, nblocks, hf,
                nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm1_mfma_groups(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E,
                                    int P, int H, int I, int k, uint8_t* hq, float* hs, hipStream_t s) {
  if (!mfma_groups_shape_ok(H, I)) return hipErrorInvalidValue;
  const int nblocks = (int)mfma_tiles_bound(P, E) * (I / 128);
  launch_kernel(gemm1_mfma_kernel<true>, dim3(nblocks), dim3(512), 0, s, xq, xs, w13, plan, E, H, I, k, nblocks,
                nullptr, hq, hs);
  return hipGetLastError();
}

hipError_t launch_gemm2_mfma(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int P,
                             int H, int I, _Float16* y, int8_t* yexp, hipStream_t s) {
  if (!mfma_shape_ok(H, I)) return hipErrorInvalidValue;
  return gemm2_parts<false>(hq, hs, w2, plan, E, P, H, I, y, yexp, s);
}

hipError_t launch_gemm2_mfma_groups(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E,
                                    int P, int H, int I, _Float16* y, int8_t* yexp, hipStream_t s) {
  if (!mfma_groups_shape_ok(H, I)) return hipErrorInvalidValue;
  return gemm2_parts<true>(hq, hs, w2, plan, E, P, H, I, y, yexp, s);
}

}  // namespace moe
