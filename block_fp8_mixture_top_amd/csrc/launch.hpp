// Host-side launchers of the kernels (internal to the library; not part of the C ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MAX_EXPERTS 1024

namespace moe {

// Events a timed forward attaches to the next kernel it enqueues: the runtime ties them to
// that kernel's dispatch, so their elapsed time is the kernel's own execution time (no
// queue or dispatch gap). Per host thread; cleared by the launch that uses them.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
KernelEvents& kernel_events();

// Every kernel of the library is enqueued through here.
template <typename... Params, typename... Args>
inline void launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                          Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
  KernelEvents& ev = kernel_events();
  if (ev.start != nullptr) {
    const KernelEvents use = ev;
    ev = KernelEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, use.start, use.stop, 0, static_cast<Params>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, static_cast<Params>(args)...);
  }
}

// Pair counts up to this sort in one workgroup; larger ones use the three-pass sort (at
// 4096 pairs the single workgroup took about 100 us more than the three passes).
constexpr int kSmallSortPairs = 4096;  // pairs the one-workgroup sort takes

// A bank as the kernels see it.
struct BankArg {
  const uint8_t* codes;
  int64_t expert_stride;  // bytes
  const void* scales;
  int scale_bf16;
  int64_t srow;  // scale row stride, elements
  int64_t sexp;  // scale expert stride, elements
  const float* bias;  // [E, N] MLP bias in the codes' row order, or nullptr
};

// Sorted routing produced by the sort and read by the GEMMs.
struct Plan {
  const int32_t* ids;     // [P]
  const float* w;         // [P]
  const int32_t* counts;  // [E]
  const int32_t* offsets; // [E+1]
  const int32_t* sorted;  // [P]
  const int32_t* act;     // [slots], -1 past the active experts
  const int32_t* tile_off;// [E+1] or null
};

size_t sort_scratch_bytes(int P, int E);

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);

// route_topk_kernel's routing with x's rows quantised as launch_quant_rows_bf16 quantises
// them (codes[T, ostride], scales[T]), in one kernel; it stands in for stage 0 of
// launch_route_stage when route_topk_first(T, k).
bool route_topk_first(int T, int k);
hipError_t launch_route_topk_quant(const float* logits, const uint16_t* x, int T, int E, int k, int H, int ostride,
                                   int32_t* ids, float* w, uint8_t* codes, float* scales, hipStream_t s);

// Routing plus the sort: 1 kernel (route and sort in one workgroup) for P <= kSmallSortPairs,
// else 4 (top-k, then histogram, chunk scan and scatter); stage picks which.
int route_kernel_count(int T, int k);
hipError_t launch_route_stage(int stage, const float* logits, int T, int E, int k, int32_t* ids, float* w,
                              int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* act, int32_t* n_act,
                              int slots, int tile_m, int32_t* tile_off, void* scratch, hipStream_t s);

// W8A16 GEMM1 + silu(gate)*up over `slots` expert slots: h[p, I] float for every pair p.
// fused: route inside the kernel (gemm1_fused_route_ok(T, k)), writing ids_out/w_out and
// leaving the sort undone; otherwise the slot's expert and pairs come from plan.
struct Gemm1Args {
  const uint16_t* hidden;
  const float* logits;
  int T, E, H, I, k, slots;
  BankArg w13;
  Plan plan;
  float* h;
  int fused;
  int32_t* ids_out;
  float* w_out;
  // non-null: GEMM1 multiplies e4m3 activation codes [T, H] with one float scale per
  // (token, 128-column group) [T, H/128] instead of the bf16 hidden states (H % 128 == 0,
  // routing not fused)
  const uint8_t* xq = nullptr;
  const float* xs = nullptr;
  // nonzero (with fused routing): the same e4m3 activations, quantised inside GEMM1 from the
  // bf16 hidden states
  int qx = 0;
};
bool gemm1_fused_route_ok(int T, int k);
// Fused routing with the e4m3 activations quantised inside GEMM1 (not with x staged in LDS).
bool gemm1_fused_qx_ok(int T, int k, int H);
hipError_t launch_gemm1_w8a16(const Gemm1Args& a, hipStream_t s);

// Whether the token-major GEMM2 supports this (k, I) (its per-thread register budget).
bool gemm2_gather_supported(int k, int I);

// Token-major W8A16 GEMM2 with the combine fused: out[t, H].
hipError_t launch_gemm2_gather(const float* h, const BankArg& w2, const int32_t* ids, const float* w, int T,
                               int H, int I, int k, void* out, int out_bf16, hipStream_t s);

// Expert-major W8A16 GEMM2: y[p, H] float for every pair.
hipError_t launch_gemm2_expert(const float* h, const BankArg& w2, const Plan& plan, int slots, int H, int I,
                               int k, float* y, hipStream_t s);

// out[t, n] = sum_j w[t, j] * y[t*k + j, n], slots summed in order.
hipError_t launch_combine(const float* y, const float* w, int T, int H, int k, void* out, int out_bf16,
                          hipStream_t s);

// W8A8 path.
// Per-row e4m3 codes (row stride ostride bytes, columns cols .. ostride - 1 zero; ostride - cols
// < 512) and scales amax/448 of rows of bf16 x.
hipError_t launch_quant_rows_bf16(const uint16_t* x, int rows, int cols, int ostride, uint8_t* codes, float* scales,
                                  hipStream_t s);
// e4m3 codes [rows, cols] and one scale per (row, 128-column group) [rows, cols/128] of rows
// of bf16 x (cols a multiple of 128, at most 8192).
hipError_t launch_quant_groups_bf16(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                                   hipStream_t s);
constexpr int kMfmaTileM = 128;  // sorted pairs per MFMA tile
constexpr int kYGroup = 32;      // MFMA path: outputs of a pair's y that share one exponent
size_t mfma_tiles_bound(int P, int E);
// Shapes the MFMA kernels are built for: H and I multiples of 16, H up to 8192, I up to 4096.
// A last 128-wide block that is partial multiplies zero activation codes past the row end
// (the code rows of x and h are padded to mfma_pad(H), mfma_pad(I) bytes).
bool mfma_shape_ok(int H, int I);
// The group-scaled variant (x per (token, 128 columns), h per (pair, 128 features)) needs
// whole groups: H and I multiples of 128 as well.
bool mfma_groups_shape_ok(int H, int I);
__host__ __device__ inline int mfma_pad(int n) { return (n + 127) / 128 * 128; }
// exponent groups of a pair's y row
__host__ __device__ inline int mfma_y_groups(int H) { return (H + kYGroup - 1) / kYGroup; }
// GEMM2 on the matrix cores multiplies up to kMfmaPartBlocks 128-wide K blocks of h per launch;
// I beyond that runs in mfma_k_parts(I) K parts, each writing its own y plane.
constexpr int kMfmaPartBlocks = 4;
int mfma_k_parts(int I);
// hf[p, I] = silu(gate) * up in float for every sorted pair position p, from the x codes
// xq[T, mfma_pad(H)] and scales xs[T].
hipError_t launch_gemm1_mfma(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E,
                             int P, int H, int I, int k, float* hf, hipStream_t s);
// GEMM1 on x codes xq[T, H] with one scale per (token, 128-column group) xs[T, H/128]; h is
// quantised in the epilogue per (sorted pair position, 128-feature group): codes hq[P, I] and
// scales hs[P, I/128] (scale = group amax / 448, 1 for a zero group).
hipError_t launch_gemm1_mfma_groups(const uint8_t* xq, const float* xs, const BankArg& w13, const Plan& plan, int E,
                                    int P, int H, int I, int k, uint8_t* hq, float* hs, hipStream_t s);
// The same quantisation for rows of float (hf, rows in sorted-position order).
hipError_t launch_quant_rows_f32(const float* x, int rows, int cols, int ostride, uint8_t* codes, float* scales,
                                 hipStream_t s);
// y[pair, H] = s_h * W2 h for every pair from the h codes hq[P, mfma_pad(I)] and row scales
// hs, stored as fp16 of y * 2^-e with one exponent e per (pair, kYGroup outputs) in
// yexp[pair, mfma_y_groups(H)] (no atomics; the combine applies the weights).
hipError_t launch_gemm2_mfma(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E, int P,
                             int H, int I, _Float16* y, int8_t* yexp, hipStream_t s);
// The same from h codes hq[P, I] with one scale per (pair, 128-feature group) hs[P, I/128].
hipError_t launch_gemm2_mfma_groups(const uint8_t* hq, const float* hs, const BankArg& w2, const Plan& plan, int E,
                                    int P, int H, int I, _Float16* y, int8_t* yexp, hipStream_t s);
// out[t, n] = sum_j w[t, j] * (y[t*k + j, n] * 2^yexp[t*k + j, n/kYGroup] + bias[ids[t*k + j], n]),
// slots summed in order; bias may be nullptr (no w2 bias).
// parts: the number of y planes (K parts) of each pair, summed in plane order first.
hipError_t launch_combine_f16(const _Float16* y, const int8_t* yexp, const float* w, const int32_t* ids,
                              const float* bias, int T, int H, int k, int parts, void* out, int out_bf16,
                              hipStream_t s);

// Test exports.
hipError_t launch_decode_e4m3(const uint8_t* codes, float* out, int64_t n, hipStream_t s);
hipError_t launch_encode_e4m3(const float* x, uint8_t* codes, int64_t n, hipStream_t s);
hipError_t launch_decode_paths(const uint8_t* chunks, float* out, int64_t n, hipStream_t s);

}  // namespace moe
