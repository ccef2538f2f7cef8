/*
 * moe_fp8_block.h - C ABI of the block-FP8 mixture-of-experts expert library (MI355X, gfx950).
 *
 * The library computes, for T tokens, the expert part of a mixture-of-experts layer whose
 * expert weights are stored as fp8-e4m3 codes with one scale per 128x128 block:
 *
 *   route    top-k experts per token by router logit, weights = softmax over the selected
 *            logits (the full softmax renormalised over the top-k);
 *   gather   only the routed experts' weight bytes are read;
 *   GEMM1    a = W13[e] x (+ b13[e]), gate rows 0..I-1 and up rows I..2I-1,
 *            h = silu(gate) * up;
 *   GEMM2    y = W2[e] h (+ b2[e]);
 *   combine  out[t] = sum_j w[t,j] * y[t,j].
 *
 * Sources: gaudi-cookbook fixes page "fp8-moe-gather" (The fix: gather g = min(local
 * experts, tokens * top_k) routed experts while tokens * top_k <= local experts * ratio,
 * ratio 0.4; up/gate as one GEMM, down projection after it); tpu-inference PR #3040 "Add
 * another fused EP MoE kernels" (gather, GMM1, activation, GMM2 in one pass; the w1 bank
 * holds the gate half before the up half); FreeToken PR #662 "serve block-fp8 experts on
 * the cpu and hybrid backends" (bank format: e4m3 row-major [rows, K], K contiguous, one
 * scale per 128x128 block; commit "honor padded fp8 scale strides": the scale row stride
 * is passed in, never recomputed; a format/ABI probe makes a stale library fail loudly).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers unless marked "host". The caller allocates and
 *     owns every buffer; the library allocates and frees nothing and keeps no state
 *     between calls. Calls are re-entrant; concurrent calls need distinct workspaces.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is enqueued
 *     asynchronously on it; nothing is synchronised and nothing is copied to the host.
 *   - Every argument check happens before any HIP call, so a rejected call leaves the
 *     stream untouched. The return value is a moe_status; on failure
 *     moe_fp8_block_last_error() returns a message (thread-local, valid until the next
 *     call on the same thread).
 *   - Layouts are row-major and dense unless a stride is given. Sizes are elements
 *     unless they say bytes.
 */
#ifndef MOE_FP8_BLOCK_H
#define MOE_FP8_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bumped on any change of a struct, an enum or an entry point's meaning. */
#define MOE_FP8_BLOCK_ABI_VERSION 5

/* Limits checked on every call. */
#define MOE_FP8_BLOCK_MAX_EXPERTS 1024
#define MOE_FP8_BLOCK_MAX_TOPK 32

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* null pointer, non-positive size, top_k out of range, bad enum */
  MOE_ERR_UNSUPPORTED = -2, /* a valid request the library does not implement (e.g. H % 16) */
  MOE_ERR_STRIDE = -3,      /* a bank stride smaller than the unpadded extent it must hold */
  MOE_ERR_ALIGN = -4,       /* a pointer or stride that breaks the 16-byte alignment rule */
  MOE_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the size query returned */
  MOE_ERR_HIP = -6          /* a kernel launch failed; the message names it */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_PATH_AUTO = 0,   /* let the gate choose (see moe_fp8_block_select_path) */
  MOE_PATH_GATHER = 1, /* W8A16, g = min(E, T*top_k) static expert slots, combine fused into GEMM2 */
  MOE_PATH_STREAM = 2, /* W8A16, expert-major GEMM2 into a [T*top_k, H] buffer, then combine */
  MOE_PATH_MFMA = 3    /* W8A8 fp8 MFMA grouped GEMM, per-row dynamic e4m3 activation scales */
} moe_path;

/*
 * One fp8 weight bank: E experts, each an [N, K] matrix of e4m3 codes (OCP e4m3fn: bias 7,
 * largest finite 448; the codes 0x7F and 0xFF are NaN and are outside the contract).
 * Expert e row n column k is codes[e * expert_stride_bytes + n * K + k].
 * The scale of block (n / 128, k / 128) of expert e is
 *   scales[e * scale_expert_stride + (n / 128) * scale_row_stride + k / 128]
 * and multiplies the decoded code. Strides may include padding, which is never read.
 * An optional MLP bias adds bias[e * N + n] to row n of expert e's product (tpu-inference
 * PR #3040, review of the w1 bias DMA: the bias follows the weight rows, so w13's bias
 * holds the gate half 0..I-1 and then the up half I..2I-1; w2's bias is added after the
 * down projection, before the router weight is applied).
 */
typedef struct {
  const uint8_t* codes;        /* device; 16-byte aligned */
  int64_t expert_stride_bytes; /* >= N*K, multiple of 16 */
  const void* scales;          /* device; float or bf16 (uint16) per scale_dtype */
  int32_t scale_dtype;         /* moe_dtype */
  int32_t reserved;            /* must be 0 */
  int64_t scale_row_stride;    /* elements, >= ceil(K/128) */
  int64_t scale_expert_stride; /* elements, >= (ceil(N/128)-1)*scale_row_stride + ceil(K/128) */
  const float* bias;           /* device [E, N] float, 16-byte aligned, or NULL for no bias */
} moe_fp8_bank;

/*
 * Activation precision (gaudi-cookbook "fp8-moe-gather", Who is affected: dynamic activation
 * scales; The fix: up/gate as one native FP8 GEMM, the down projection in fp32).
 */
typedef enum {
  MOE_ACT_PATH = 0,      /* the path's own: bf16 activations (exact W8A16) on GATHER and
                            STREAM; e4m3 per token and per (token, slot) on MFMA */
  MOE_ACT_ROW_FP8 = 1,   /* reported only: MFMA's per-row dynamic e4m3 on both GEMMs */
  MOE_ACT_GROUP_FP8 = 2, /* dynamic e4m3 activations with one scale per 128-column group,
                            scale = group amax/448. GATHER / STREAM: GEMM1 on x quantised per
                            (token, 128 columns), GEMM2 on float h. MFMA: both GEMMs, x per
                            (token, 128 columns) and h per ((token, slot), 128 features),
                            reported as MOE_ACT_GROUP_FP8_W8A8. Needs H % 128 == 0, and on
                            MFMA also I % 128 == 0 (a gate choice of MFMA moves to STREAM
                            otherwise, a forced MFMA fails). */
  MOE_ACT_GROUP_FP8_W8A8 = 3 /* reported only: MOE_ACT_GROUP_FP8 on MFMA */
} moe_act;

/* Host-side options; NULL means the defaults below. */
typedef struct {
  float gate_ratio;                  /* gather iff T*top_k <= gate_ratio*E (default 2.0, measured) */
  int32_t force_path;                /* moe_path; anything but AUTO is taken as asked or fails */
  int32_t mfma_min_tokens_per_expert;/* grouped work uses MFMA iff T*top_k >= this*E (default 2, measured) */
  int32_t act_mode;                  /* MOE_ACT_PATH (default) or MOE_ACT_GROUP_FP8 */
  int32_t use_measured_gate;         /* 1 (default): for an (E, H, I, top_k) the library has a measured
                                        table for, the path measured fastest at this T (see
                                        moe_fp8_block_select_path); 0: the two thresholds above */
} moe_opts;

/* Filled by forward (host struct): what actually ran. */
typedef struct {
  int32_t path;     /* moe_path taken (never AUTO) */
  int32_t act_mode; /* 0: bf16 activations, exact W8A16; 1: per-row dynamic e4m3 on both GEMMs
                       (MFMA); 2: per-(token, 128-column) dynamic e4m3 on GEMM1, float GEMM2;
                       3: per-128-column-group dynamic e4m3 on both GEMMs (MFMA) */
  int32_t slots;    /* expert slots launched: min(E, T*top_k) */
  int32_t kernels;  /* kernel launches enqueued */
} moe_run_info;

/* Version of this ABI compiled into the library; a caller compares it with
 * MOE_FP8_BLOCK_ABI_VERSION and refuses a stale library (FreeToken PR #662, PR body:
 * the format probe). Never fails. */
int moe_fp8_block_abi_version(void);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* moe_fp8_block_last_error(void);

/* Writes the default options into *opts (host). Returns MOE_ERR_ARG for NULL. */
int moe_fp8_block_default_opts(moe_opts* opts);

/*
 * The gather/grouped gate, host only (gaudi-cookbook "fp8-moe-gather", The fix and the
 * VLLM_HPU_MOE_GATHER_RATIO row of its table): GATHER iff T*top_k <= gate_ratio*E,
 * else MFMA iff T*top_k >= mfma_min_tokens_per_expert*E, else STREAM. The page's ratio
 * 0.4 was chosen for another device; with use_measured_gate, a shape (E, H, I, top_k) the
 * library carries a table for takes the path measured fastest on MI355X at the nearest
 * swept T instead (the table is generated by block_fp8_mixture_top_amd/tune_gate.py from
 * the committed sweeps under profiles/; FreeToken PR #662 likewise picks its backend from
 * measured bandwidth). With act_mode MOE_ACT_GROUP_FP8 the gate uses the two thresholds
 * (the tables were measured with MOE_ACT_PATH). A forced path is reported unchanged; a gate choice the
 * shape does not support moves to STREAM, as forward does. Writes path, act_mode and slots
 * into *info; no HIP call.
 */
int moe_fp8_block_select_path(int T, int E, int H, int I, int top_k, const moe_opts* opts, moe_run_info* info);

/* Bytes of workspace moe_fp8_block_route needs for these sizes (0 if sizes are invalid). */
size_t moe_fp8_block_route_workspace_size(int T, int E, int top_k);

/*
 * Routing alone, and the token-to-expert sort.
 *   logits  [T, E] float, finite.
 *   ids     [T, top_k] int32 out: experts by descending logit, ties to the lower id.
 *   weights [T, top_k] float out: exp(l_j - l_0) / sum_i exp(l_i - l_0), evaluated in
 *           double with the sum in slot order, rounded to float.
 *   counts  [E] int32 out or NULL; offsets [E+1] int32 out (exclusive sums) or NULL;
 *   sorted_pairs [T*top_k] int32 out or NULL: pair p = t*top_k + j grouped by expert,
 *           ascending p within an expert. counts, offsets and sorted_pairs are all NULL
 *           (sort skipped) or all set.
 *   workspace: device, >= moe_fp8_block_route_workspace_size bytes (may be NULL if 0).
 * T = 0 is a no-op. E <= 1024, 1 <= top_k <= min(E, 32).
 */
int moe_fp8_block_route(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_fp8_block_forward needs for these sizes and options (0 if invalid). */
size_t moe_fp8_block_workspace_size(int T, int E, int H, int I, int top_k, const moe_opts* opts);

/*
 * The whole expert computation.
 *   hidden  [T, H] bf16 (uint16 bits), 16-byte aligned.
 *   logits  [T, E] float.
 *   w13     bank with N = 2I, K = H (gate rows 0..I-1, up rows I..2I-1). With a bias,
 *           gate = W_gate x + b13[e, 0..I-1] and up = W_up x + b13[e, I..2I-1].
 *   w2      bank with N = H, K = I. With a bias, y = W2 h + b2[e] for each (token, slot)
 *           pair before the router weight multiplies it.
 *   out     [T, H], out_dtype float or bf16 (round to nearest even from float), 16-byte
 *           aligned.
 *   ids_out [T, top_k] int32 and weights_out [T, top_k] float: the routing, or NULL.
 *   opts    host, NULL = defaults; info host, NULL = not reported.
 * H and I must be multiples of 16 (MOE_ERR_UNSUPPORTED otherwise); a last 128-wide scale
 * block may be partial. Scale blocks tile the stored rows, so w13's up row I+i takes block
 * (I+i)/128. On MFMA a partial last 128-wide K block multiplies zero activation codes past the
 * row end (the x and h code rows are padded in the workspace). Every pointer the
 * chosen path reads must be non-NULL. T = 0 is a no-op (info still filled).
 * The W8A16 paths (GATHER, STREAM) decode weights exactly and accumulate in float. MFMA
 * quantises x per token and h per (token, slot) row (with MOE_ACT_GROUP_FP8: x per (token,
 * 128 columns) and h per ((token, slot), 128 features), h inside the up/gate GEMM) to e4m3
 * with scale amax/448 (float division, 1 for a zero row or group; codes round to nearest
 * even and saturate at 448) and
 * multiplies on the fp8 matrix cores; its per-(token, slot) down-projection results reach
 * the combine in fp16 with a power-of-two exponent per 32 outputs (at most 2^-11 relative
 * rounding each). Every path writes each (token, slot) result once and sums a token's
 * slots in slot order, so all of them are deterministic.
 */
int moe_fp8_block_forward(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13,
                          const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out,
                          int out_dtype, void* workspace, size_t workspace_bytes, int32_t* ids_out,
                          float* weights_out, const moe_opts* opts, moe_run_info* info, void* stream);

/*
 * moe_fp8_block_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the workspace is a
 * static device array of the library, MOE_FP8_BLOCK_STATIC_WORKSPACE_BYTES on each GPU it
 * runs on, held until the process ends; the caller still passes inputs and outputs. A call
 * whose workspace (moe_fp8_block_workspace_size) exceeds that size fails with
 * MOE_ERR_WORKSPACE before any HIP call. The call allocates nothing. Its first call on a
 * device looks the array's address up for that device, which must be the current device
 * and the device of `stream` (MOE_ERR_ARG otherwise). Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (concurrent streams or host threads) race;
 * no kernel needs the array zeroed, and each call overwrites what it uses. Everything else
 * (arguments, errors, results) is as moe_fp8_block_forward.
 */
#define MOE_FP8_BLOCK_STATIC_WORKSPACE_BYTES (64u << 20)
int moe_fp8_block_forward_static(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13,
                                 const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out,
                                 int out_dtype, int32_t* ids_out, float* weights_out, const moe_opts* opts,
                                 moe_run_info* info, void* stream);

/* Kernel kinds named by moe_fp8_block_forward_timed. */
typedef enum {
  MOE_K_ROUTE = 1,    /* top-k and weights (on MFMA with per-row activations, when a top-k
                         kernel starts the routing, it also quantises x) */
  MOE_K_SORT = 2,     /* token-to-expert sort (one or three kernels) */
  MOE_K_QUANT = 3,    /* e4m3 activation quantisation (MFMA path, where the routing kernel
                         does not; group-fp8 on any path) */
  MOE_K_HQUANT = 4,   /* per-(token, slot) e4m3 quantisation of h before the down GEMM (MFMA path) */
  MOE_K_GEMM1 = 5,    /* gate/up GEMM with silu(gate)*up */
  MOE_K_GEMM2 = 6,    /* down GEMM (with the combine on GATHER) */
  MOE_K_COMBINE = 7   /* router-weighted sum of the slots (STREAM and MFMA paths) */
} moe_kernel;

/*
 * moe_fp8_block_forward with each kernel timed by the caller's HIP events. events: n_events
 * hipEvent_t (as void*) created by the caller with timing enabled. For every i <
 * n_events/2, kernel i is enqueued with events[2i] and events[2i+1] attached to its own
 * dispatch (hipExtLaunchKernel), so hipEventElapsedTime(events[2i], events[2i+1]) is that
 * kernel's execution time on `stream`, without queue or dispatch gaps; later kernels run
 * untimed. kinds: host array of n_events/2 int32 or NULL; receives the moe_kernel of each
 * timed kernel and 0 past the last. info->kernels counts all kernels. Everything else,
 * errors included, is as moe_fp8_block_forward; MOE_ERR_ARG if n_events < 0 or events is
 * NULL with n_events > 0.
 */
int moe_fp8_block_forward_timed(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13,
                                const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out,
                                int out_dtype, void* workspace, size_t workspace_bytes, int32_t* ids_out,
                                float* weights_out, const moe_opts* opts, moe_run_info* info, void* stream,
                                void* const* events, int n_events, int32_t* kinds);

/*
 * Test exports: the two halves of the MFMA path (route + sort first in each), so that each
 * half can be checked against a reference on its own inputs. Both take the workspace of a
 * forward forced onto MFMA (moe_fp8_block_workspace_size with force_path MOE_PATH_MFMA)
 * and need H and I multiples of 16, H up to 8192 and I up to 4096 (MOE_ERR_UNSUPPORTED
 * otherwise).
 *   mfma_up:   x quantised per token (as quantize_rows), GEMM1 on the fp8 matrix cores and
 *              h = silu(gate) * up written in float to h [T*top_k, I], row p holding the
 *              pair at sorted position p (the sorted_pairs order of moe_fp8_block_route).
 *   mfma_down: h [T*top_k, I] float in the same sorted-position order is quantised per row
 *              (scale amax/448), multiplied by w2 on the matrix cores and combined with the
 *              router weights into out [T, H] (out_dtype float or bf16), exactly as the
 *              forward's second half.
 * Pointers are device pointers, hidden/h/out 16-byte aligned. T = 0 is a no-op.
 */
int moe_fp8_block_mfma_up(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13, int T, int E, int H,
                          int I, int top_k, float* h, void* workspace, size_t workspace_bytes, void* stream);
int moe_fp8_block_mfma_down(const float* h, const float* logits, const moe_fp8_bank* w2, int T, int E, int H, int I,
                            int top_k, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * The same two halves with MOE_ACT_GROUP_FP8 (gaudi-cookbook "fp8-moe-gather", Who is
 * affected: block-quantized checkpoints with dynamic activation scales). Workspace of a
 * forward forced onto MFMA with act_mode MOE_ACT_GROUP_FP8; H and I multiples of 128, H up
 * to 8192 and I up to 4096 (MOE_ERR_UNSUPPORTED otherwise).
 *   mfma_up_groups:   x quantised per (token, 128-column group), GEMM1 on the matrix cores
 *                     and h quantised per (pair, 128-feature group): codes h_codes
 *                     [T*top_k, I] uint8 and scales h_scales [T*top_k, I/128] float (group
 *                     amax/448, 1 for a zero group), row p the pair at sorted position p.
 *   mfma_down_groups: h_codes and h_scales in that layout, multiplied by w2 on the matrix
 *                     cores and combined into out [T, H], as the forward's second half.
 * Pointers are device pointers, hidden/h_codes/out 16-byte aligned. T = 0 is a no-op.
 */
int moe_fp8_block_mfma_up_groups(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13, int T, int E,
                                 int H, int I, int top_k, uint8_t* h_codes, float* h_scales, void* workspace,
                                 size_t workspace_bytes, void* stream);
int moe_fp8_block_mfma_down_groups(const uint8_t* h_codes, const float* h_scales, const float* logits,
                                   const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out,
                                   int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The activation preparation of the MFMA path on its own: per-row dynamic e4m3.
 *   x [rows, cols] bf16; codes [rows, cols] uint8 out; scales [rows] float out, with
 *   scale = amax/448 (float division; 1 for an all-zero row) and code = e4m3 of x/scale
 *   (float division, nearest even, saturating). cols % 16 == 0 and cols <= 8192
 *   (MOE_ERR_UNSUPPORTED otherwise), 16-byte aligned x/codes.
 */
int moe_fp8_block_quantize_rows(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                                void* stream);

/*
 * The same with one scale per (row, 128-column group) (the group-fp8 activations of
 * MOE_ACT_GROUP_FP8): codes [rows, cols] uint8 out, scales [rows, cols/128] float out, each
 * group quantised as a row above. cols % 128 == 0 and cols <= 8192 (MOE_ERR_UNSUPPORTED
 * otherwise), 16-byte aligned x/codes.
 */
int moe_fp8_block_quantize_groups(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                                  void* stream);

/* Device decode of n e4m3 codes to float with the kernels' own conversion (codes and
 * out device, n >= 0). Exposed so tests can check the decode over all 256 codes. */
int moe_fp8_block_decode_e4m3(const uint8_t* codes, float* out, int64_t n, void* stream);

/* Every decode the kernels use, on n chunks of 16 codes (device, 16-byte aligned) into out
 * [n, 16, 5] float (device): for code j of chunk i, out[i][j][0] is the word conversion to
 * float (both halves of each 32-bit word), [1] the conversion to bf16 with unit scale (both
 * halves) widened to float, [2] the W8A16 dot helper (codes x bf16) against a one-hot bf16
 * activation at j, [3] the e4m3 x e4m3 dot helper against a one-hot e4m3 1.0 at j, [4] the
 * codes x float dot helper against a one-hot float at j. Each must equal the code's value.
 * Chunks must hold finite codes only (a NaN code times a zero activation is NaN). */
int moe_fp8_block_decode_e4m3_paths(const uint8_t* chunks, float* out, int64_t n, void* stream);

/* Device float -> e4m3 with the kernels' own conversion (nearest even, saturating at
 * 448, sign of zero kept). Exposed so tests can sweep rounding midpoints. */
int moe_fp8_block_encode_e4m3(const float* x, uint8_t* codes, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_BLOCK_H */
