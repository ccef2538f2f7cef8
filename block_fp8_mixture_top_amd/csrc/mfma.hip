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
// block). A and B are read with the same per-lane K pattern (chunks kq and kq + 4 of the
// block for lanes of K quarter kq), so whatever order the unit walks K in, matching A and
// B bytes meet.
//
// Both GEMMs work on tiles of 64 sorted (token, slot) pairs of one expert. Every operand
// goes global -> LDS with direct loads of 8 rows x 128 contiguous bytes per instruction,
// through LDS rings a few K blocks ahead of the multiply. GEMM1 covers all 2I features of its
// tile, so its epilogue has whole h rows: silu(gate)*up, row amax, scale and e4m3 codes are
// produced without writing h in float. GEMM2 writes each pair's y row in float once; the
// combine kernel sums the slots of a token in slot order with the router weights.
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


// ---------------------------------------------------------------- shared tile machinery

// silu with the hardware exp and reciprocal (about 1 ulp each). h feeds a quantiser whose
// decisions the parity check already treats as uncertain within the accumulation error of
// the matrix cores, which is orders of magnitude larger.
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

constexpr int kTM = kMfmaTileM;  // pairs per tile: four 16-row MFMA tiles
constexpr int kMaxH = 8192;      // bounds the block-scale slabs staged in LDS
constexpr int kMaxI = 512;       // GEMM1 keeps 64 x I h values in registers
constexpr int kStages = 3;       // depth of the LDS rings
constexpr int kRowB = 128;       // bytes of one row in one 128-wide K block

// LDS rows hold one 128-byte K block; 16-byte chunk c of row r sits at chunk position
// c ^ sw(r), so the 16 consecutive rows one operand read touches (same chunk) fall on
// distinct banks whether the LDS serves 128 or 256 bytes a clock.
__device__ __forceinline__ int sw(int r) { return (r ^ (r >> 3)) & 7; }

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

// ---------------------------------------------------------------- GEMM1

// One workgroup per (expert, 64-pair tile), 4 waves. NP = I/128 passes; in pass ps wave w
// owns gate features ps*128 + 32w .. +32 (two 16-row MFMA tiles) and the matching up
// features, for all 64 pairs. Every K block of every pass is a stage of a 3-deep LDS ring:
// each wave copies in the 64 weight rows it multiplies, and the four waves together copy
// the tile's 64 token rows of x. One barrier per stage. A = weight rows (features),
// B = token rows, so lane (r16, kq) of a 16x16 result holds features 4kq..4kq+3 of token r16.
template <int NP>
__global__ __launch_bounds__(256, 1) void gemm1_mfma_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                            BankArg w13, Plan plan, int E, int H, int I, int k,
                                                            int nblocks, uint8_t* __restrict__ hq,
                                                            float* __restrict__ hs) {
  constexpr int G = 2;                   // gate tiles per wave per pass (and as many up tiles)
  constexpr int NF = 2 * G;              // weight tiles per wave per pass
  constexpr int WB = 64 * kRowB;         // one wave's weight rows of a stage
  constexpr int XB = kTM * kRowB;        // the tile's x rows of a stage
  constexpr int SB = 4 * WB + XB;        // one stage
  constexpr int LPW = 8 + 2;             // direct loads per wave per stage
  __shared__ __align__(16) uint8_t ring[kStages * SB];
  __shared__ float s_sc[(2 * kMaxI / 128) * (kMaxH / 128)];
  __shared__ float s_amax[4][kTM];
  __shared__ int s_tok[kTM];

  const int tile = xcd_tile(blockIdx.x, nblocks);
  if (tile >= plan.tile_off[E]) return;
  const int e = find_expert(plan.tile_off, E, tile);
  const int pos0 = plan.offsets[e] + (tile - plan.tile_off[e]) * kTM;
  const int pos_end = plan.offsets[e + 1];
  const int nvalid = pos_end - pos0 < kTM ? pos_end - pos0 : kTM;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int r16 = lane & 15, kq = lane >> 4;
  const uint8_t* wb = w13.codes + (size_t)e * w13.expert_stride;
  const int nkb = H / 128;

  // token of each tile row (rows past the expert's pairs repeat the first token; their
  // results are never stored)
  if ((int)threadIdx.x < kTM)
    s_tok[threadIdx.x] = plan.sorted[pos0 + ((int)threadIdx.x < nvalid ? (int)threadIdx.x : 0)] / k;
  stage_scales(s_sc, w13, (int64_t)e * w13.sexp, 2 * I / 128, nkb);
  __syncthreads();
  float xsc[4];  // x scale of token tt*16 + r16
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) xsc[tt] = xs[s_tok[tt * 16 + r16]];

  // direct-load sources. Weight instruction i covers rows 8i .. 8i+7 of the wave's 64
  // (rows 0..31 gate, 32..63 up); pass ps adds 128 rows and K block kb adds kb*128 bytes.
  const int lr = lane >> 3, lc = lane & 7;
  uint32_t woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = i * 8 + lr;
    const int row = (b < 32 ? 0 : I - 32) + wave * 32 + b;
    woff[i] = (uint32_t)row * (uint32_t)H + (uint32_t)((lc ^ sw(b)) << 4);
  }
  // x instruction i covers tile rows 16w + 8i .. +7
  const uint8_t* xsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wave * 16 + i * 8 + lr;
    xsrc[i] = xq + (size_t)s_tok[r] * H + ((lc ^ sw(r)) << 4);
  }
  const int total = NP * nkb;
  auto issue = [&](int st) {
    const int ps = st / nkb, kb = st - ps * nkb;
    uint8_t* slot = ring + (st % kStages) * SB;
    const uint8_t* src = wb + (size_t)ps * 128 * H + kb * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) g2lds(src + woff[i], slot + wave * WB + i * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) g2lds(xsrc[i] + kb * 128, slot + 4 * WB + (wave * 16 + i * 8) * kRowB);
  };
  issue(0);
  if (total > 1) issue(1);

  float hkeep[NP][G][4][4];
  float am[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    f32x4 acc[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[f][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = 0; kb < nkb; ++kb) {
      const int st = ps * nkb + kb;
      // this wave's loads of stage st are in; after the barrier everyone's are, and every
      // wave is done with stage st - 1, whose slot the next issue refills
      if (st + 1 < total) wait_vm<LPW>();
      else wait_vm<0>();
      bar();
      if (st + 2 < total) issue(st + 2);
      const uint8_t* slot = ring + (st % kStages) * SB;
      const uint8_t* sw_ = slot + wave * WB;
      const uint8_t* sx_ = slot + 4 * WB;
      i32x8 bx[4], wa[NF];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) bx[tt] = lds_operand(sx_, tt * 16 + r16, kq);
#pragma unroll
      for (int f = 0; f < NF; ++f) wa[f] = lds_operand(sw_, f * 16 + r16, kq);
      // one scale per K block for the gate rows of this pass, one for the up rows
      const float sg = s_sc[ps * nkb + kb];
      const float su = s_sc[(ps + NP) * nkb + kb];
      // software pipelined: MFMA j + 1 is issued before the scale FMAs of MFMA j
      f32x4 pp = mfma_fp8(wa[0], bx[0]);
#pragma unroll
      for (int j = 0; j < NF * 4; ++j) {
        const int f = j / 4, tt = j % 4;
        f32x4 nx;
        if (j + 1 < NF * 4) nx = mfma_fp8(wa[(j + 1) / 4], bx[(j + 1) % 4]);
        const float sc = f < G ? sg : su;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[f][tt][q] = __builtin_fmaf(sc, pp[q], acc[f][tt][q]);
        if (j + 1 < NF * 4) pp = nx;
      }
    }
#pragma unroll
    for (int f = 0; f < G; ++f)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = acc[f][tt][q] * xsc[tt];
          const float u = acc[f + G][tt][q] * xsc[tt];
          const float v = silu_fast(g) * u;
          hkeep[ps][f][tt][q] = v;
          am[tt] = __builtin_fmaxf(am[tt], __builtin_fabsf(v));
        }
  }
  // row amax over the four K-quarter lane groups, then over the waves
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    am[tt] = __builtin_fmaxf(am[tt], __shfl_xor(am[tt], 16, kWave));
    am[tt] = __builtin_fmaxf(am[tt], __shfl_xor(am[tt], 32, kWave));
    if (kq == 0) s_amax[wave][tt * 16 + r16] = am[tt];
  }
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int r = tt * 16 + r16;
    const int pos = pos0 + r;
    if (pos >= pos_end) continue;
    const float a = __builtin_fmaxf(__builtin_fmaxf(s_amax[0][r], s_amax[1][r]),
                                    __builtin_fmaxf(s_amax[2][r], s_amax[3][r]));
    const float s = a > 0.0f ? a / kE4M3Max : 1.0f;
    const float rs = 1.0f / s;  // codes of v * (1/s): within 1 ulp of v / s
#pragma unroll
    for (int ps = 0; ps < NP; ++ps)
#pragma unroll
      for (int f = 0; f < G; ++f) {
        const int i = ps * 128 + wave * (16 * G) + f * 16 + kq * 4;
        const float* v = hkeep[ps][f][tt];
        const uint32_t lo = enc2(v[0] * rs, v[1] * rs);
        const uint32_t hi = enc2(v[2] * rs, v[3] * rs);
        *(uint32_t*)(hq + (size_t)pos * I + i) = lo | (hi << 16);
      }
    if (wave == 0 && kq == 0) hs[pos] = s;
  }
}

// ---------------------------------------------------------------- GEMM2

// One workgroup per (expert, 64-pair tile), 4 waves. The tile's h codes (64 x I) are copied
// to LDS once: A = h (pairs as rows). B = w2 rows (features). The H outputs go in chunks of
// 256; wave w owns features 64w .. 64w+64 of each chunk (FT = 4 MFMA tiles; a last chunk
// of 128 has work for waves 0 and 1 only), so lane (r16, kq) of a result holds pairs
// 4kq..4kq+3 of feature r16. Each wave streams its own w2 rows, (chunk, K block) after
// (chunk, K block), through a private 3-deep LDS ring and so never waits for the others.
// Each pair's y row = s_h * W2 h is written once, in float; the combine kernel applies the
// router weights.
template <int KB>  // I / 128
__global__ __launch_bounds__(256, 1) void gemm2_mfma_kernel(const uint8_t* __restrict__ hq, const float* __restrict__ hs,
                                                            BankArg w2, Plan plan, int E, int H, int I, int k,
                                                            int nblocks, float* __restrict__ y) {
  constexpr int FT = 4;
  constexpr int NCH = 4 * FT * 16;
  constexpr int WB = 64 * kRowB;  // one wave's w2 rows of a stage
  constexpr int HB = kTM * kRowB; // the h tile's rows of one K block
  __shared__ __align__(16) uint8_t sH[KB * HB];
  __shared__ __align__(16) uint8_t ring[4 * kStages * WB];
  __shared__ float s_sc[(kMaxH / 128) * (kMaxI / 128)];
  (void)k;

  const int tile = xcd_tile(blockIdx.x, nblocks);
  if (tile >= plan.tile_off[E]) return;
  const int e = find_expert(plan.tile_off, E, tile);
  const int pos0 = plan.offsets[e] + (tile - plan.tile_off[e]) * kTM;
  const int pos_end = plan.offsets[e + 1];
  const int nvalid = pos_end - pos0 < kTM ? pos_end - pos0 : kTM;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int r16 = lane & 15, kq = lane >> 4;
  const uint8_t* wb = w2.codes + (size_t)e * w2.expert_stride;
  const int lr = lane >> 3, lc = lane & 7;

  // h tile: 8 * KB instructions of 8 rows x 128 bytes, 2 * KB per wave (rows past the
  // expert's pairs copy the tile's first row; their results are never stored)
#pragma unroll
  for (int i = 0; i < 2 * KB; ++i) {
    const int q = wave * 2 * KB + i;
    const int kb = q >> 3, r = (q & 7) * 8 + lr;
    const int rr = r < nvalid ? r : 0;
    g2lds(hq + (size_t)(pos0 + rr) * I + kb * 128 + ((lc ^ sw(r)) << 4), sH + kb * HB + (q & 7) * 1024);
  }
  // chunks holding features of this wave: those with c * NCH + 64 * wave < H (H is a
  // multiple of 128, so a wave's 64 features are all in range or all out)
  const int nch = (H - wave * 64 + NCH - 1) / NCH;
  const int nst = nch * KB;
  // w2 instruction i covers rows 8i .. 8i+7 of the wave's 64; chunk c adds c * NCH rows
  uint32_t woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = i * 8 + lr;
    woff[i] = (uint32_t)(wave * 64 + b) * (uint32_t)I + (uint32_t)((lc ^ sw(b)) << 4);
  }
  uint8_t* myring = ring + wave * kStages * WB;
  auto issue = [&](int st) {
    const int c = st / KB, kb = st - c * KB;
    const uint8_t* src = wb + (size_t)c * NCH * I + kb * 128;
    uint8_t* slot = myring + (st % kStages) * WB;
#pragma unroll
    for (int i = 0; i < 8; ++i) g2lds(src + woff[i], slot + i * 1024);
  };
  if (nst > 0) issue(0);
  if (nst > 1) issue(1);
  stage_scales(s_sc, w2, (int64_t)e * w2.sexp, H / 128, KB);
  float hsc[4][4];
  int prow[4][4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = pos0 + pt * 16 + kq * 4 + q;
      const bool ok = pos < pos_end;
      hsc[pt][q] = ok ? hs[pos] : 0.0f;
      prow[pt][q] = ok ? plan.sorted[pos] : -1;
    }
  // everyone's h rows (and the scales) are in
  wait_vm<0>();
  __syncthreads();

  f32x4 acc[FT][4];
  for (int st = 0; st < nst; ++st) {
    const int c = st / KB, kb = st - c * KB;
    // the previous chunk's y stores are outstanding at a chunk start, and stores and
    // loads may complete out of order: drain everything there
    if (st + 1 < nst && kb != 0) wait_vm<8>();
    else wait_vm<0>();
    if (st + 2 < nst) issue(st + 2);
    if (kb == 0) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[ft][pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const uint8_t* slot = myring + (st % kStages) * WB;
    const uint8_t* hs_ = sH + kb * HB;
    i32x8 a[4], bw[FT];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) a[pt] = lds_operand(hs_, pt * 16 + r16, kq);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) bw[ft] = lds_operand(slot, ft * 16 + r16, kq);
    const int n0 = c * NCH + wave * 64;
    // features n0 .. n0 + 63 share one 128-row scale block
    const float sc = s_sc[(n0 / kScaleBlock) * KB + kb];
    f32x4 pp = mfma_fp8(a[0], bw[0]);
#pragma unroll
    for (int j = 0; j < FT * 4; ++j) {
      const int ft = j / 4, pt = j % 4;
      f32x4 nx;
      if (j + 1 < FT * 4) nx = mfma_fp8(a[(j + 1) % 4], bw[(j + 1) / 4]);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[ft][pt][q] = __builtin_fmaf(sc, pp[q], acc[ft][pt][q]);
      if (j + 1 < FT * 4) pp = nx;
    }
    if (kb == KB - 1) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (prow[pt][q] < 0) continue;
          float* yr = y + (size_t)prow[pt][q] * H + n0 + r16;
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) yr[ft * 16] = acc[ft][pt][q] * hsc[pt][q];
        }
    }
  }
}

template <int NP>
hipError_t g1m(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E, int nblocks, int H,
               int I, int k, uint8_t* hq, float* hs, hipStream_t s) {
  launch_kernel((gemm1_mfma_kernel<NP>), dim3(nblocks), dim3(256), 0, s, xq, xs, w13, plan, E, H, I, k, nblocks,
                     hq, hs);
  return hipGetLastError();
}

template <int KB>
hipError_t g2m(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int nblocks, int H,
               int I, int k, float* y, hipStream_t s) {
  launch_kernel((gemm2_mfma_kernel<KB>), dim3(nblocks), dim3(256), 0, s, hq, hs, w2, plan, E, H, I, k, nblocks,
                     y);
  return hipGetLastError();
}

}  // namespace

// Upper bound on the tiles of any routing (sum over experts of ceil(count/64) <= P/64 + E),
// rounded up to a multiple of 8 so that xcd_tile maps the grid onto [0, bound) one to one.
size_t mfma_tiles_bound(int P, int E) {
  const size_t b = (size_t)(P + kTM - 1) / kTM + (size_t)E;
  return (b + 7) / 8 * 8;
}

bool mfma_shape_ok(int H, int I) {
  return H % 128 == 0 && H > 0 && H <= kMaxH && I % 128 == 0 && I >= 128 && I <= kMaxI;
}

hipError_t launch_quant_rows_bf16(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                                  hipStream_t s) {
  const int blocks = (rows + 3) / 4;
  launch_kernel(quant_rows_bf16_kernel, dim3(blocks), dim3(256), 0, s, x, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_gemm1_mfma(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E, int P,
                             int H, int I, int k, uint8_t* hq, float* hs, hipStream_t s) {
  if (!mfma_shape_ok(H, I)) return hipErrorInvalidValue;
  const int nblocks = (int)mfma_tiles_bound(P, E);
  switch (I / 128) {
    case 1: return g1m<1>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
    case 2: return g1m<2>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
    case 3: return g1m<3>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
    default: return g1m<4>(xq, xs, w13, plan, E, nblocks, H, I, k, hq, hs, s);
  }
}

hipError_t launch_gemm2_mfma(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int P,
                             int H, int I, int k, float* y, hipStream_t s) {
  if (!mfma_shape_ok(H, I)) return hipErrorInvalidValue;
  const int nblocks = (int)mfma_tiles_bound(P, E);
  switch (I / 128) {
    case 1: return g2m<1>(hq, hs, w2, plan, E, nblocks, H, I, k, y, s);
    case 2: return g2m<2>(hq, hs, w2, plan, E, nblocks, H, I, k, y, s);
    case 3: return g2m<3>(hq, hs, w2, plan, E, nblocks, H, I, k, y, s);
    default: return g2m<4>(hq, hs, w2, plan, E, nblocks, H, I, k, y, s);
  }
}

}  // namespace moe
