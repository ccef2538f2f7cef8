// W8A16 expert GEMMs that stream the routed experts' fp8 rows from HBM.
//
// Weights are e4m3 codes, row-major [rows, K] with K contiguous and one scale per 128x128
// block (FreeToken PR #662, PR body). They are decoded exactly in registers (every e4m3
// value is a float) and multiplied with bf16 activations, which are exact in float, so each
// product is exact and only the float summation order differs from an exact evaluation.
//
// GEMM1 produces h = silu(gate) * up for every (token, slot) pair; the gate rows are
// 0..I-1 and the up rows I..2I-1 of the w13 bank (tpu-inference PR #3040, review of the w1
// weight/scale DMA), and one lane group holds gate row i and up row i together so h_i is
// formed without another pass. GEMM2 reads h back and applies the down projection; on the
// gather path it also applies the router weights and sums the slots (the combine).
//
// Lane layout: a row of K bytes is cut into 16-byte chunks; a group of LPR lanes covers a
// row, lane g of the group taking chunks g, g+LPR, ... (MCH of them). A 16-byte chunk never
// straddles a 128-wide scale block, so each chunk needs one scale.
#include "common.hpp"
#include "launch.hpp"
#include "gemv.hpp"
#include "topk.hpp"

namespace moe {

namespace {

// Routing done inside GEMM1 for small batches: one token per wave.
constexpr int kFuseTokens = kThreads / kWave;
constexpr int kFuseMaxPairs = kFuseTokens * 32;

// GEMM1 + silu*up. grid.x: tiles of row pairs, grid.y: expert slots. A lane group owns RP
// consecutive row pairs (gate i, up I+i) of the slot's expert, loads their codes once and
// applies them to every token routed to that expert.
//
// PER > 0 routes inside the kernel (wave_topk_ids_lds with PER logits per lane):
//   T == 1: every wave routes the token itself, with no barrier; the slot-th expert in
//   ascending id is the one whose id ranks `slot` among the token's top_k distinct ids.
//   2 <= T <= 4: one wave per token, an LDS bitmap of routed experts gives the slot-th one
//   and its pairs.
// Workgroup (0, 0) writes the ids and weights for the down GEMM; the weights (double exp and
// sum) are computed after the weight loads are issued, off the critical path.
// PER == 0: the slot's expert and pairs come from the sorted plan in global memory.
// XL (long rows only): x is staged per workgroup in LDS instead of being held in every
// lane's registers, which leaves room for more waves per SIMD. With fused routing (T == 1
// only) the token's x is read before routing and one barrier, after the weight reads are
// issued, publishes it; with a plan (PER == 0) each pair's x row is read, once the weight
// reads are issued, and staged between two barriers.
// A8 (PER == 0 only): the activations are e4m3 codes xq with one scale xs per (token,
// 128-column group); a 16-code chunk lies in one group, so its block product takes the
// weight block scale times the group's activation scale.
// QX (PER > 0, not XL): the same e4m3 activations, quantised here from the bf16 x in
// registers: a group's 8 chunks sit in 8 neighbouring lanes of a lane group, so its amax is
// a 3-step butterfly; scale and codes are computed as the row quantiser does.
template <int LPR, int MCH, int RP, int PER, bool XL = false, bool A8 = false, bool QX = false>
__global__ __launch_bounds__(kThreads) void gemm1_w8a16_kernel(const uint16_t* __restrict__ hidden,
                                                               const float* __restrict__ logits, int T, int E,
                                                               BankArg w13, Plan plan, int H, int I, int k,
                                                               float* __restrict__ h, int32_t* __restrict__ ids_out,
                                                               float* __restrict__ w_out,
                                                               const uint8_t* __restrict__ xq,
                                                               const float* __restrict__ xs) {
  static_assert(!A8 || (PER == 0 && !XL), "e4m3 activations come with a routing plan");
  static_assert(!QX || (PER > 0 && !XL && !A8), "in-register quantisation is for fused routing");
  constexpr int GPW = kWave / LPR;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int grp = lane / LPR, gl = lane % LPR;
  const int NC = H / 16;
  int e, cnt = 0, single = -1;  // single: the only pair (T == 1)
  const int32_t* pairs = nullptr;
  int my_id = 0;
  float my_l = 0.0f;
  bool route_wave = false;  // this wave holds a token's routing (lanes < k)
  int route_tok = 0;
  __shared__ int s_ids[PER > 0 ? kFuseMaxPairs : 1];
  __shared__ int s_pairs[PER > 0 ? kFuseMaxPairs : 1];
  __shared__ uint32_t s_bits[MAX_EXPERTS / 32];
  __shared__ __align__(16) uint64_t s_cand[PER > 0 ? kThreads / kWave : 1][kWave];  // top-k candidates
  __shared__ int s_e, s_m;
  // x of token 0, issued before routing when T == 1 (XL: 16-byte pieces q = tid + kThreads*j
  // of the row, bound for LDS)
  u32x4 x0[XL ? 1 : MCH], x1[XL || A8 ? 1 : MCH];
  float xsm[A8 || QX ? MCH : 1];  // A8, QX: the activation scale of each chunk's group
  u32x4 xq8[QX ? MCH : 1];        // QX: the chunk's e4m3 codes
  constexpr int XQ = XL ? (MCH * kWave * 2 + kThreads - 1) / kThreads : 1;
  __shared__ __align__(16) uint8_t s_x[XL ? MCH * kWave * 32 : 16];
  u32x4 xr[XQ];
  if constexpr (PER > 0) {
    if (T == 1) {
      if constexpr (XL) {
#pragma unroll
        for (int j = 0; j < XQ; ++j)
          xr[j] = ld16((const uint8_t*)hidden + (size_t)min((int)threadIdx.x + kThreads * j, 2 * NC - 1) * 16);
      } else {
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          const int c = min(gl + LPR * m, NC - 1);  // chunks past NC read the last one, unused
          x0[m] = ld16((const uint8_t*)hidden + (size_t)c * 32);
          x1[m] = ld16((const uint8_t*)hidden + (size_t)c * 32 + 16);
        }
      }
      wave_topk_ids_lds<PER>(logits, E, k, s_cand[wave], my_id, my_l);
      route_wave = wave == 0;
      int rank = 0;
      for (int j = 0; j < k; ++j) rank += __builtin_amdgcn_readlane(my_id, j) < my_id ? 1 : 0;
      const uint64_t hit = __ballot(lane < k && rank == (int)blockIdx.y);
      if (hit == 0ull) return;  // no such slot (never for T == 1: slots == top_k)
      single = __builtin_ctzll(hit);
      e = __builtin_amdgcn_readlane(my_id, single);
      cnt = 1;
    } else if constexpr (!XL) {
      const int P = T * k;
      if (threadIdx.x < MAX_EXPERTS / 32) s_bits[threadIdx.x] = 0u;
      if (wave < T) {
        wave_topk_ids_lds<PER>(logits + (size_t)wave * E, E, k, s_cand[wave], my_id, my_l);
        route_wave = true;
        route_tok = wave;
        if (lane < k) s_ids[wave * k + lane] = my_id;
      }
      __syncthreads();
      if ((int)threadIdx.x < P) atomicOr(&s_bits[s_ids[threadIdx.x] >> 5], 1u << (s_ids[threadIdx.x] & 31));
      __syncthreads();
      if (wave == 0) {
        const int slot = blockIdx.y;
        const uint32_t word = lane < MAX_EXPERTS / 32 ? s_bits[lane] : 0u;
        const int c = __popc(word);
        const int incl = wave_incl_scan(c);
        const int total = __shfl(incl, kWave - 1, kWave);
        if (slot >= total) {
          if (lane == 0) s_e = -1;
        } else if (slot >= incl - c && slot < incl) {
          uint32_t b = word;
          for (int r = slot - (incl - c); r > 0; --r) b &= b - 1u;
          s_e = lane * 32 + __builtin_ctz(b);
        }
      }
      __syncthreads();
      e = s_e;
      if (e < 0) return;
      if (wave == 0) {
        int m = 0;
        for (int base = 0; base < P; base += kWave) {
          const int p = base + lane;
          const bool hit = p < P && s_ids[p] == e;
          const uint64_t bal = __ballot(hit);
          if (hit) s_pairs[m + __popcll(bal & ((1ull << lane) - 1ull))] = p;
          m += __popcll(bal);
        }
        if (lane == 0) s_m = m;
      }
      __syncthreads();
      cnt = s_m;
      pairs = s_pairs;
    }
  } else {
    e = plan.act[blockIdx.y];
    if (e < 0) return;
    cnt = plan.counts[e];
    pairs = plan.sorted + plan.offsets[e];
  }
  if constexpr (XL && PER > 0) {
    // routing waited for the logits, read after x, so x is here: to LDS, freeing registers
#pragma unroll
    for (int j = 0; j < XQ; ++j) {
      const int q = (int)threadIdx.x + kThreads * j;
      if (q < 2 * NC) *(u32x4*)(s_x + q * 16) = xr[j];
    }
  }
  const int rows_per_block = (kThreads / kWave) * GPW * RP;
  const int i0 = blockIdx.x * rows_per_block + (wave * GPW + grp) * RP;
  const uint8_t* wb = w13.codes + (size_t)e * w13.expert_stride;
  const int64_t sb = (int64_t)e * w13.sexp;

  // The RP rows of a lane group lie in one 128-row scale block (i0 is a multiple of RP, which
  // divides 128), so a chunk's gate and up scales are shared by them. Scales are read first
  // and waited for only after every code read is issued.
  u32x4 cg[RP][MCH], cu[RP][MCH];
  // Scale blocks tile the stored [2I, H] rows, so up row I+i is in block (I+i)/128 (the same
  // as the gate blocks shifted by I/128 when 128 divides I). I is even, so the up rows of a
  // lane group, like its gate rows, share one block.
  ScaleBits bg[MCH], bu[MCH];
  const int i0c = i0 < I ? i0 : I - 1;
  const int ib = i0c / kScaleBlock, iu = (I + i0c) / kScaleBlock;
#pragma unroll
  for (int m = 0; m < MCH; ++m) {
    const int c = gl + LPR * m;
    const int cb = (c < NC ? c : NC - 1) / 8;
    bg[m] = load_scale_bits(w13.scales, w13.scale_bf16, sb + (int64_t)ib * w13.srow + cb);
    bu[m] = load_scale_bits(w13.scales, w13.scale_bf16, sb + (int64_t)iu * w13.srow + cb);
  }
  // The MLP bias of the gate and up rows (w13's bias holds the gate half, then the up half).
  // Without a bias the reads go to an in-bounds address and are dropped, so no read sits in a
  // branch.
  const bool hb = w13.bias != nullptr;
  const float* bb = hb ? w13.bias + (size_t)e * 2 * I : (const float*)w13.codes;
  float bgr[RP], bur[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int i = min(i0 + r, I - 1);
    bgr[r] = bb[hb ? i : 0];
    bur[r] = bb[hb ? I + i : 0];
  }
  // Every read is unconditional (rows past I and chunks past NC read in-bounds neighbours whose
  // results are dropped), so the compiler can count them exactly and wait only at first use.
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int i = min(i0 + r, I - 1);
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
      const int c = min(gl + LPR * m, NC - 1);
      cg[r][m] = ld16_stream(wb + (size_t)i * H + (size_t)c * 16);
      cu[r][m] = ld16_stream(wb + (size_t)(I + i) * H + (size_t)c * 16);
    }
  }
  float sg[MCH], su[MCH];
#pragma unroll
  for (int m = 0; m < MCH; ++m) {
    settle(bg[m]);
    settle(bu[m]);
    sg[m] = scale_value(bg[m], w13.scale_bf16);
    su[m] = scale_value(bu[m], w13.scale_bf16);
  }
  if constexpr (XL && PER > 0) __syncthreads();  // x in LDS (written before the weight reads were issued)
  if constexpr (PER > 0) {
    // the router weights, while the weight codes are in flight
    if (route_wave && blockIdx.x == 0 && blockIdx.y == 0) {
      const float wt = wave_topk_weight(my_l, k);
      if (lane < k) {
        ids_out[route_tok * k + lane] = my_id;
        w_out[route_tok * k + lane] = wt;
      }
    }
  }
  for (int q = 0; q < cnt; ++q) {
    const int p = single >= 0 ? single : pairs[q];
    if constexpr (XL && PER == 0) {
      // this pair's x row into LDS, once every lane is done with the previous one
      const uint8_t* xb = (const uint8_t*)(hidden + (size_t)(p / k) * H);
#pragma unroll
      for (int j = 0; j < XQ; ++j) xr[j] = ld16(xb + (size_t)min((int)threadIdx.x + kThreads * j, 2 * NC - 1) * 16);
      if (q > 0) __syncthreads();
#pragma unroll
      for (int j = 0; j < XQ; ++j) {
        const int c = (int)threadIdx.x + kThreads * j;
        if (c < 2 * NC) *(u32x4*)(s_x + c * 16) = xr[j];
      }
      __syncthreads();
    }
    if (!XL && single < 0) {
      if constexpr (A8) {
        const uint8_t* xc = xq + (size_t)(p / k) * H;
        const float* xg = xs + (size_t)(p / k) * (H / kScaleBlock);
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          const int c = min(gl + LPR * m, NC - 1);
          x0[m] = ld16(xc + (size_t)c * 16);
          xsm[m] = xg[c / 8];
        }
      } else if constexpr (!XL) {
        const uint8_t* xb = (const uint8_t*)(hidden + (size_t)(p / k) * H);
#pragma unroll
        for (int m = 0; m < MCH; ++m) {
          const int c = min(gl + LPR * m, NC - 1);
          x0[m] = ld16(xb + (size_t)c * 32);
          x1[m] = ld16(xb + (size_t)c * 32 + 16);
        }
      }
    }
    if constexpr (QX) {
      // every lane quantises its chunks (chunks past NC form whole groups of their own,
      // unused), so the butterfly runs with all lanes active
#pragma unroll
      for (int m = 0; m < MCH; ++m) {
        const uint32_t w[8] = {x0[m].x, x0[m].y, x0[m].z, x0[m].w, x1[m].x, x1[m].y, x1[m].z, x1[m].w};
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16_lo(w[q])), __builtin_fabsf(bf16_hi(w[q]))));
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off, kWave));
        const float sx = amax > 0.0f ? amax / kE4M3Max : 1.0f;
        // x / sx rounded to float, as the row quantiser divides, but by one double reciprocal
        // per group: float((double)x * (1 / (double)sx)) equals the correctly rounded float
        // quotient for bf16 x. The double product is within 2^-52 of x / sx, while x / sx is
        // never a float rounding midpoint (an odd 25-bit significand times sx cannot fit the
        // 8 bits of x) and, when not one, is at least 2^-49 away from any (x - m * sx is a
        // multiple of the 49-bit product's ulp), so both round to the same float.
        const double rx = 1.0 / (double)sx;
        auto qd = [&](float v) { return (float)((double)v * rx); };
        uint32_t cw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          cw[q] = enc2(qd(bf16_lo(w[2 * q])), qd(bf16_hi(w[2 * q]))) |
                  (enc2(qd(bf16_lo(w[2 * q + 1])), qd(bf16_hi(w[2 * q + 1]))) << 16);
        xq8[m] = u32x4{cw[0], cw[1], cw[2], cw[3]};
        xsm[m] = sx;
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int m = 0; m < MCH; ++m) {
        if (gl + LPR * m < NC) {
          u32x4 xa, xb;
          if constexpr (XL) {
            xa = *(const u32x4*)(s_x + (gl + LPR * m) * 32);
            xb = *(const u32x4*)(s_x + (gl + LPR * m) * 32 + 16);
          } else if constexpr (!A8) {
            xa = x0[m];
            xb = x1[m];
          }
          if constexpr (A8) {
            g = __builtin_fmaf(sg[m] * xsm[m], dot16_e4m3(cg[r][m], x0[m]), g);
            u = __builtin_fmaf(su[m] * xsm[m], dot16_e4m3(cu[r][m], x0[m]), u);
          } else if constexpr (QX) {
            g = __builtin_fmaf(sg[m] * xsm[m], dot16_e4m3(cg[r][m], xq8[m]), g);
            u = __builtin_fmaf(su[m] * xsm[m], dot16_e4m3(cu[r][m], xq8[m]), u);
          } else {
            g = __builtin_fmaf(sg[m], dot16_bf16(cg[r][m], xa, xb), g);
            u = __builtin_fmaf(su[m], dot16_bf16(cu[r][m], xa, xb), u);
          }
        }
      }
      g = group_sum<LPR>(g);
      u = group_sum<LPR>(u);
      if (hb) {
        g += bgr[r];
        u += bur[r];
      }
      const int i = i0 + r;
      if (gl == 0 && i < I) h[(size_t)p * I + i] = silu(g) * u;
    }
  }
}

// Token-major GEMM2 with the combine. grid.x: tiles of ROWS output rows, grid.y: tokens.
// The k*I/16 chunks of a token's (slot, chunk) space are spread over the workgroup's
// threads (MC per thread); each thread keeps its h values and its slot's router weight in
// registers and streams the matching 16 bytes of every output row. BIAS: the thread holding
// chunk 0 of a slot also adds the router weight times that expert's w2 bias to each row.
template <int MC, int ROWS, bool BIAS>
__global__ __launch_bounds__(kThreads) void gemm2_gather_kernel(const float* __restrict__ h, BankArg w2,
                                                                const int32_t* __restrict__ ids,
                                                                const float* __restrict__ wts, int H, int I,
                                                                int k, void* __restrict__ out, int out_bf16) {
  __shared__ float red[kThreads / kWave][ROWS];
  // Workgroups are dealt to the 8 XCDs round-robin in launch order. When the row tiles come
  // in multiples of 8, XCD x takes row tiles x, x + 8, ... and within one tile every token in
  // turn, so the tokens that share an expert read that tile's w2 rows through one L2 one
  // after another instead of a whole token's work apart.
  int t = (int)blockIdx.y, tile = (int)blockIdx.x;
  if (gridDim.x % 8 == 0) {
    const int L = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    const int x = L & 7, i = L >> 3, T = (int)gridDim.y;
    t = i % T;
    tile = (i / T) * 8 + x;
  }
  const int n0 = tile * ROWS;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int CPR = I / 16;
  const int F = k * CPR;
  // Thread chunk m: slot j, 16 h values c*16 .. c*16+15. Reads in dependency order, each
  // batch issued before anything waits: the slot's expert id and router weight with h (h's
  // address does not depend on the id), then the scales, then the codes; the scales are
  // waited for only after every code read is issued. Chunks past F read slot 0, chunk 0 (in
  // bounds) and are given weight 0.
  f32x4 hq[MC][4];
  int ev[MC];
  float wv[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const int f = tid + kThreads * m < F ? tid + kThreads * m : 0;
    const int j = f / CPR, c = f % CPR;
    ev[m] = ids[(size_t)t * k + j];
    wv[m] = wts[(size_t)t * k + j];
    const float* hp = h + ((size_t)t * k + j) * I + (size_t)c * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) hq[m][q] = *(const f32x4*)(hp + 4 * q);
  }
  ScaleBits sbits[MC];
  const uint8_t* wp[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const int f = tid + kThreads * m < F ? tid + kThreads * m : 0;
    const int c = f % CPR;
    sbits[m] = load_scale_bits(w2.scales, w2.scale_bf16,
                               (int64_t)ev[m] * w2.sexp + (int64_t)(n0 / kScaleBlock) * w2.srow + c / 8);
    wp[m] = w2.codes + (size_t)ev[m] * w2.expert_stride + (size_t)c * 16;
  }
  float bv[BIAS ? MC : 1][ROWS];
  if constexpr (BIAS) {
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) bv[m][r] = w2.bias[(size_t)ev[m] * H + (n0 + r < H ? n0 + r : H - 1)];
  }
  u32x4 cw[ROWS][MC];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int n = n0 + r < H ? n0 + r : H - 1;
#pragma unroll
    for (int m = 0; m < MC; ++m) cw[r][m] = ld16_stream(wp[m] + (size_t)n * I);
  }
  float hv[MC][16];
  float ws[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    settle(sbits[m]);
    const bool live = tid + kThreads * m < F;
    ws[m] = live ? wv[m] * scale_value(sbits[m], w2.scale_bf16) : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hv[m][4 * q + 0] = live ? hq[m][q].x : 0.0f;
      hv[m][4 * q + 1] = live ? hq[m][q].y : 0.0f;
      hv[m][4 * q + 2] = live ? hq[m][q].z : 0.0f;
      hv[m][4 * q + 3] = live ? hq[m][q].w : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      // a chunk past F multiplies zero codes (a NaN code times a zero weight would not vanish)
      const u32x4 code = tid + kThreads * m < F ? cw[r][m] : u32x4{0, 0, 0, 0};
      acc = __builtin_fmaf(ws[m], dot16_f32(code, hv[m]), acc);
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int m = 0; m < MC; ++m) {
        const int f = tid + kThreads * m;
        const float wb = f < F && f % CPR == 0 ? wv[m] : 0.0f;
        acc = __builtin_fmaf(wb, bv[m][r], acc);
      }
    }
    acc = wave_sum_dpp(acc);
    if (lane == 0) red[wave][r] = acc;
  }
  __syncthreads();
  if (tid < ROWS) {
    const int n = n0 + tid;
    if (n < H) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kThreads / kWave; ++w) s += red[w][tid];
      if (out_bf16) ((uint16_t*)out)[(size_t)t * H + n] = f32_to_bf16(s);
      else ((float*)out)[(size_t)t * H + n] = s;
    }
  }
}

// Expert-major GEMM2: y[p, n] for every pair p of the slot's expert. grid.x: row tiles,
// grid.y: expert slots. Same lane layout as GEMM1 with K = I and single rows.
template <int LPR, int MCH, int RP>
__global__ __launch_bounds__(kThreads) void gemm2_expert_kernel(const float* __restrict__ h, BankArg w2, Plan plan,
                                                                int H, int I, float* __restrict__ y) {
  const int e = plan.act[blockIdx.y];
  if (e < 0) return;
  constexpr int GPW = kWave / LPR;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int grp = lane / LPR, gl = lane % LPR;
  const int rows_per_block = (kThreads / kWave) * GPW * RP;
  const int n0 = blockIdx.x * rows_per_block + (wave * GPW + grp) * RP;
  const int NC = I / 16;
  const uint8_t* wb = w2.codes + (size_t)e * w2.expert_stride;
  const int64_t sb = (int64_t)e * w2.sexp;
  // The RP rows share one 128-row scale block (n0 is a multiple of RP, which divides 128).
  // Scales first, then every code read, all unconditional (out-of-range rows and chunks read
  // in-bounds neighbours whose results are dropped), so no read waits inside a branch.
  ScaleBits sbits[MCH];
  const int nb = (n0 < H ? n0 : H - 1) / kScaleBlock;
#pragma unroll
  for (int m = 0; m < MCH; ++m) {
    const int c = min(gl + LPR * m, NC - 1);
    sbits[m] = load_scale_bits(w2.scales, w2.scale_bf16, sb + (int64_t)nb * w2.srow + c / 8);
  }
  u32x4 cw[RP][MCH];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int n = min(n0 + r, H - 1);
#pragma unroll
    for (int m = 0; m < MCH; ++m) cw[r][m] = ld16_stream(wb + (size_t)n * I + (size_t)min(gl + LPR * m, NC - 1) * 16);
  }
  // the w2 bias of the RP rows, read unconditionally (dropped without a bias)
  const bool hb = w2.bias != nullptr;
  const float* bb = hb ? w2.bias + (size_t)e * H : (const float*)w2.codes;
  float brow[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) brow[r] = bb[hb ? min(n0 + r, H - 1) : 0];
  float sw[MCH];
#pragma unroll
  for (int m = 0; m < MCH; ++m) {
    settle(sbits[m]);
    sw[m] = scale_value(sbits[m], w2.scale_bf16);
  }
  const int beg = plan.offsets[e];
  const int cnt = plan.counts[e];
  for (int q = 0; q < cnt; ++q) {
    const int p = plan.sorted[beg + q];
    const float* hp = h + (size_t)p * I;
    float hv[MCH][16];
#pragma unroll
    for (int m = 0; m < MCH; ++m) {
      const int c = min(gl + LPR * m, NC - 1);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 v = *(const f32x4*)(hp + (size_t)c * 16 + 4 * qq);
        hv[m][4 * qq + 0] = v.x;
        hv[m][4 * qq + 1] = v.y;
        hv[m][4 * qq + 2] = v.z;
        hv[m][4 * qq + 3] = v.w;
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < MCH; ++m)
        if (gl + LPR * m < NC) acc = __builtin_fmaf(sw[m], dot16_f32(cw[r][m], hv[m]), acc);
      acc = group_sum<LPR>(acc);
      if (hb) acc += brow[r];
      const int n = n0 + r;
      if (gl == 0 && n < H) y[(size_t)p * H + n] = acc;
    }
  }
}

// Four consecutive outputs per thread (H is a multiple of 128), slots summed in order.
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                           int T, int H, int k, void* __restrict__ out,
                                                           int out_bf16) {
  const size_t idx = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (idx >= (size_t)T * H) return;
  const size_t t = idx / H, n = idx % H;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const f32x4 v = *(const f32x4*)(y + (t * k + j) * H + n);
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = __builtin_fmaf(wj, v[q], s[q]);
  }
  if (out_bf16) {
    const uint32_t lo = (uint32_t)f32_to_bf16(s[0]) | ((uint32_t)f32_to_bf16(s[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(s[2]) | ((uint32_t)f32_to_bf16(s[3]) << 16);
    *(uint2*)((uint16_t*)out + idx) = make_uint2(lo, hi);
  } else {
    *(f32x4*)((float*)out + idx) = s;
  }
}

template <int LPR, int MCH, int RP, int PER>
hipError_t g1(const Gemm1Args& a, hipStream_t s) {
  const int rows = (kThreads / kWave) * (kWave / LPR) * RP;
  dim3 grid((a.I + rows - 1) / rows, a.slots);
  if constexpr (PER > 0) {
    if (a.qx) {  // the caller has checked that the XL variant does not apply (gemm1_fused_qx_ok)
      launch_kernel((gemm1_w8a16_kernel<LPR, MCH, RP, PER, false, false, true>), grid, dim3(kThreads), 0, s,
                    a.hidden, a.logits, a.T, a.E, a.w13, a.plan, a.H, a.I, a.k, a.h, a.ids_out, a.w_out, a.xq,
                    a.xs);
      return hipGetLastError();
    }
  }
  if constexpr (LPR == kWave && MCH >= 4) {
    if (PER == 0 || a.T == 1) {
      launch_kernel((gemm1_w8a16_kernel<LPR, MCH, RP, PER, true>), grid, dim3(kThreads), 0, s, a.hidden, a.logits,
                    a.T, a.E, a.w13, a.plan, a.H, a.I, a.k, a.h, a.ids_out, a.w_out, a.xq, a.xs);
      return hipGetLastError();
    }
  }
  launch_kernel((gemm1_w8a16_kernel<LPR, MCH, RP, PER>), grid, dim3(kThreads), 0, s, a.hidden, a.logits, a.T,
                     a.E, a.w13, a.plan, a.H, a.I, a.k, a.h, a.ids_out, a.w_out, a.xq, a.xs);
  return hipGetLastError();
}

template <int LPR, int MCH, int RP>
hipError_t g1a8(const Gemm1Args& a, hipStream_t s) {
  const int rows = (kThreads / kWave) * (kWave / LPR) * RP;
  dim3 grid((a.I + rows - 1) / rows, a.slots);
  launch_kernel((gemm1_w8a16_kernel<LPR, MCH, RP, 0, false, true>), grid, dim3(kThreads), 0, s, a.hidden,
                a.logits, a.T, a.E, a.w13, a.plan, a.H, a.I, a.k, a.h, a.ids_out, a.w_out, a.xq, a.xs);
  return hipGetLastError();
}

template <int LPR, int MCH, int RP>
hipError_t g1r(const Gemm1Args& a, hipStream_t s) {
  if (a.xq != nullptr) return a.fused ? hipErrorInvalidValue : g1a8<LPR, MCH, RP>(a, s);
  if (!a.fused) return g1<LPR, MCH, RP, 0>(a, s);
  hipError_t err = hipErrorInvalidValue;
  MOE_TOPK_DISPATCH(a.E, err = (g1<LPR, MCH, RP, PER>(a, s)));
  return err;
}

template <int LPR, int MCH, int RP>
hipError_t g2e(const float* h, const BankArg& w, const Plan& p, int slots, int H, int I, float* y,
               hipStream_t s) {
  const int rows = (kThreads / kWave) * (kWave / LPR) * RP;
  dim3 grid((H + rows - 1) / rows, slots);
  launch_kernel((gemm2_expert_kernel<LPR, MCH, RP>), grid, dim3(kThreads), 0, s, h, w, p, H, I, y);
  return hipGetLastError();
}

}  // namespace

bool gemm1_fused_route_ok(int T, int k) { return T >= 1 && T <= kFuseTokens && T * k <= kFuseMaxPairs; }

bool gemm1_fused_qx_ok(int T, int k, int H) {
  const Layout L = pick_layout(H);
  const bool xl = T == 1 && L.lpr == kWave && L.mch >= 4;  // x staged in LDS: not with QX
  return gemm1_fused_route_ok(T, k) && !xl && H % kScaleBlock == 0;
}

hipError_t launch_gemm1_w8a16(const Gemm1Args& a, hipStream_t s) {
  const Layout L = pick_layout(a.H);
  if (L.lpr == 64) {
    switch (L.mch) {
      case 1: return g1r<64, 1, 2>(a, s);
      case 2: return g1r<64, 2, 1>(a, s);
      case 3: return g1r<64, 3, 1>(a, s);
      case 4: return g1r<64, 4, 1>(a, s);
      case 5: return g1r<64, 5, 1>(a, s);
      case 6: return g1r<64, 6, 1>(a, s);
      case 7: return g1r<64, 7, 1>(a, s);
      case 8: return g1r<64, 8, 1>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (L.lpr == 32) return L.mch == 1 ? g1r<32, 1, 2>(a, s) : g1r<32, 2, 2>(a, s);
  if (L.lpr == 16) return L.mch == 1 ? g1r<16, 1, 2>(a, s) : g1r<16, 2, 2>(a, s);
  return L.mch == 1 ? g1r<8, 1, 2>(a, s) : g1r<8, 2, 2>(a, s);
}

hipError_t launch_gemm2_expert(const float* h, const BankArg& w2, const Plan& plan, int slots, int H, int I,
                               int k, float* y, hipStream_t s) {
  (void)k;
  const Layout L = pick_layout(I);
  if (L.lpr == 64) {
    switch (L.mch) {
      case 1: return g2e<64, 1, 2>(h, w2, plan, slots, H, I, y, s);
      case 2: return g2e<64, 2, 2>(h, w2, plan, slots, H, I, y, s);
      case 3: return g2e<64, 3, 1>(h, w2, plan, slots, H, I, y, s);
      case 4: return g2e<64, 4, 1>(h, w2, plan, slots, H, I, y, s);
      case 5: return g2e<64, 5, 1>(h, w2, plan, slots, H, I, y, s);
      case 6: return g2e<64, 6, 1>(h, w2, plan, slots, H, I, y, s);
      case 7: return g2e<64, 7, 1>(h, w2, plan, slots, H, I, y, s);
      case 8: return g2e<64, 8, 1>(h, w2, plan, slots, H, I, y, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (L.lpr == 32) return L.mch == 1 ? g2e<32, 1, 2>(h, w2, plan, slots, H, I, y, s)
                                     : g2e<32, 2, 2>(h, w2, plan, slots, H, I, y, s);
  if (L.lpr == 16) return L.mch == 1 ? g2e<16, 1, 2>(h, w2, plan, slots, H, I, y, s)
                                     : g2e<16, 2, 2>(h, w2, plan, slots, H, I, y, s);
  return L.mch == 1 ? g2e<8, 1, 2>(h, w2, plan, slots, H, I, y, s) : g2e<8, 2, 2>(h, w2, plan, slots, H, I, y, s);
}

bool gemm2_gather_supported(int k, int I) {
  const int F = k * (I / 16);
  return F <= 4 * kThreads;
}

template <int MC, int ROWS>
static hipError_t g2g(const float* h, const BankArg& w2, const int32_t* ids, const float* w, int T, int H, int I,
                      int k, void* out, int out_bf16, hipStream_t s) {
  dim3 grid((H + ROWS - 1) / ROWS, T);
  if (w2.bias != nullptr)
    launch_kernel((gemm2_gather_kernel<MC, ROWS, true>), grid, dim3(kThreads), 0, s, h, w2, ids, w, H, I, k, out,
                  out_bf16);
  else
    launch_kernel((gemm2_gather_kernel<MC, ROWS, false>), grid, dim3(kThreads), 0, s, h, w2, ids, w, H, I, k, out,
                  out_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm2_gather(const float* h, const BankArg& w2, const int32_t* ids, const float* w, int T,
                               int H, int I, int k, void* out, int out_bf16, hipStream_t s) {
  const int F = k * (I / 16);
  const int mc = (F + kThreads - 1) / kThreads;
  // rows per workgroup: enough workgroups to cover the chip at small T; from a few tokens on,
  // more rows per workgroup read each token's h fewer times (16 rows measured 1.5-3% faster
  // than 8 per forward from T=4 to 64 at H=2048, I=512, top_k=8)
  const bool few = (size_t)T * H < 256 * 8 * 4;
  switch (mc) {
    case 1: return few ? g2g<1, 4>(h, w2, ids, w, T, H, I, k, out, out_bf16, s)
                       : g2g<1, 16>(h, w2, ids, w, T, H, I, k, out, out_bf16, s);
    case 2: return few ? g2g<2, 4>(h, w2, ids, w, T, H, I, k, out, out_bf16, s)
                       : g2g<2, 8>(h, w2, ids, w, T, H, I, k, out, out_bf16, s);
    case 3:
    case 4: return few ? g2g<4, 4>(h, w2, ids, w, T, H, I, k, out, out_bf16, s)
                       : g2g<4, 8>(h, w2, ids, w, T, H, I, k, out, out_bf16, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const float* y, const float* w, int T, int H, int k, void* out, int out_bf16,
                          hipStream_t s) {
  const size_t n = (size_t)T * H / 4;
  launch_kernel(combine_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, y, w,
                     T, H, k, out, out_bf16);
  return hipGetLastError();
}

}  // namespace moe
