// The C ABI: argument checks (all before any HIP call), the gather/grouped gate, workspace
// carving and kernel dispatch. Declared in include/moe_fp8_block.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/moe_fp8_block.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MOE_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_CHECK(expr, what)                   \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

moe_opts defaults() {
  moe_opts o;
  // measured crossovers on MI355X at E=256, H=2048, I=512, top_k=8 (tune_gate.py): GATHER
  // is fastest up to 2 pairs per expert, MFMA from 3; STREAM never wins there but takes the
  // grouped work of shapes the MFMA kernels do not cover
  o.gate_ratio = 2.0f;
  o.force_path = MOE_PATH_AUTO;
  o.mfma_min_tokens_per_expert = 2;
  o.act_mode = MOE_ACT_PATH;
  o.use_measured_gate = 1;
  return o;
}

// One expert shape's measured gate: path[i] is the fastest path for T <= t_max[i] (the last
// t_max is INT32_MAX). Generated from the committed sweeps by tune_gate.py.
struct GateEntry {
  int E, H, I, k, n;
  int t_max[24];
  int path[24];
};
#include "gate_table.inc"

const GateEntry* gate_entry(int E, int H, int I, int k) {
  for (const GateEntry& g : kGateTable)
    if (g.E == E && g.H == H && g.I == I && g.k == k) return &g;
  return nullptr;
}

int check_sizes(int T, int E, int top_k) {
  if (T < 0) return fail(MOE_ERR_ARG, "T must be >= 0 (got %d)", T);
  if (E < 1 || E > MOE_FP8_BLOCK_MAX_EXPERTS)
    return fail(MOE_ERR_ARG, "E must be in [1, %d] (got %d)", MOE_FP8_BLOCK_MAX_EXPERTS, E);
  if (top_k < 1 || top_k > E || top_k > MOE_FP8_BLOCK_MAX_TOPK)
    return fail(MOE_ERR_ARG, "top_k must be in [1, min(E, %d)] (got %d, E=%d)", MOE_FP8_BLOCK_MAX_TOPK, top_k, E);
  if ((int64_t)T * top_k > (int64_t)(1 << 28)) return fail(MOE_ERR_ARG, "T*top_k too large");
  return MOE_OK;
}

int check_opts(const moe_opts* o) {
  if (!(std::isfinite(o->gate_ratio) && o->gate_ratio >= 0.0f))
    return fail(MOE_ERR_ARG, "gate_ratio must be finite and >= 0");
  if (o->force_path < MOE_PATH_AUTO || o->force_path > MOE_PATH_MFMA)
    return fail(MOE_ERR_ARG, "force_path %d is not a moe_path", o->force_path);
  if (o->mfma_min_tokens_per_expert < 1) return fail(MOE_ERR_ARG, "mfma_min_tokens_per_expert must be >= 1");
  if (o->act_mode != MOE_ACT_PATH && o->act_mode != MOE_ACT_GROUP_FP8)
    return fail(MOE_ERR_ARG, "act_mode %d is not MOE_ACT_PATH or MOE_ACT_GROUP_FP8", o->act_mode);
  if (o->use_measured_gate != 0 && o->use_measured_gate != 1)
    return fail(MOE_ERR_ARG, "use_measured_gate must be 0 or 1");
  return MOE_OK;
}

// The gate (gaudi-cookbook "fp8-moe-gather", The fix): gather while T*top_k <= ratio*E, or,
// for a shape with a measured table, the path measured fastest at this T (the tables were
// measured with the paths' own activations; group-wise e4m3 takes the thresholds).
int gate(int T, int E, int H, int I, int top_k, const moe_opts& o) {
  if (o.force_path != MOE_PATH_AUTO) return o.force_path;
  if (o.use_measured_gate && o.act_mode == MOE_ACT_PATH) {
    if (const GateEntry* g = gate_entry(E, H, I, top_k)) {
      for (int i = 0; i < g->n; ++i)
        if (T <= g->t_max[i]) return g->path[i];
    }
  }
  const double P = (double)T * top_k;
  if (P <= (double)o.gate_ratio * E) return MOE_PATH_GATHER;
  if (P >= (double)o.mfma_min_tokens_per_expert * E) return MOE_PATH_MFMA;
  return MOE_PATH_STREAM;
}

// Activation precision a path runs with (moe_run_info.act_mode).
int act_of(int path, const moe_opts& o) {
  if (path == MOE_PATH_MFMA) return o.act_mode == MOE_ACT_GROUP_FP8 ? MOE_ACT_GROUP_FP8_W8A8 : MOE_ACT_ROW_FP8;
  return o.act_mode == MOE_ACT_GROUP_FP8 ? MOE_ACT_GROUP_FP8 : MOE_ACT_PATH;
}

// Path actually run: the gate's choice, moved off a path the shapes do not fit only when
// the caller left the choice to the gate.
int resolve_path(int T, int E, int H, int I, int top_k, const moe_opts& o, int* path) {
  int p = gate(T, E, H, I, top_k, o);
  const bool forced = o.force_path != MOE_PATH_AUTO;
  if (o.act_mode == MOE_ACT_GROUP_FP8) {
    if (H % 128 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "MOE_ACT_GROUP_FP8 needs H %% 128 == 0 (got H=%d)", H);
    if (p == MOE_PATH_MFMA && I % 128 != 0) {
      if (forced)
        return fail(MOE_ERR_UNSUPPORTED, "MOE_ACT_GROUP_FP8 on MFMA needs I %% 128 == 0 (got I=%d)", I);
      p = MOE_PATH_STREAM;
    }
  }
  if (p == MOE_PATH_MFMA && !moe::mfma_shape_ok(H, I)) {
    if (forced) return fail(MOE_ERR_UNSUPPORTED, "MFMA path needs H <= 8192 and I <= 4096 (got H=%d, I=%d)", H, I);
    p = MOE_PATH_STREAM;
  }
  if (p == MOE_PATH_GATHER && !moe::gemm2_gather_supported(top_k, I)) {
    if (forced) return fail(MOE_ERR_UNSUPPORTED, "GATHER path needs top_k*I <= 16384 (got %d*%d)", top_k, I);
    p = MOE_PATH_STREAM;
  }
  *path = p;
  return MOE_OK;
}

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  }
};

// Workspace layout; offsets into the caller's buffer.
struct Layout {
  size_t ids, w, counts, offsets, sorted, act, n_act, tile_off, scratch;
  size_t h, y, yexp, xq, xs, hq, hs;
  size_t total;
};

Layout layout_for(int path, int act, int T, int E, int H, int I, int top_k) {
  Layout L{};
  Carve c;
  const size_t P = (size_t)T * top_k;
  const size_t slots = P < (size_t)E ? P : (size_t)E;
  L.ids = c.take(P * 4);
  L.w = c.take(P * 4);
  L.counts = c.take((size_t)E * 4);
  L.offsets = c.take((size_t)(E + 1) * 4);
  L.sorted = c.take(P * 4);
  L.act = c.take((slots > 0 ? slots : 1) * 4);
  L.n_act = c.take(4);
  L.tile_off = c.take((size_t)(E + 1) * 4);
  L.scratch = c.take(moe::sort_scratch_bytes((int)P, E));
  // h in float, [pair or sorted position, I] (the group-scaled MFMA path writes codes only)
  if (act != MOE_ACT_GROUP_FP8_W8A8) L.h = c.take(P * (size_t)I * 4);
  if (path == MOE_PATH_STREAM) L.y = c.take(P * (size_t)H * 4);  // y in float
  if (path == MOE_PATH_MFMA) {
    // y in fp16, one exponent per (pair, kYGroup outputs), one plane per K part of GEMM2
    const size_t parts = (size_t)moe::mfma_k_parts(I);
    L.y = c.take(parts * P * (size_t)H * 2);
    L.yexp = c.take(parts * P * (size_t)moe::mfma_y_groups(H));
    if (act == MOE_ACT_GROUP_FP8_W8A8) {
      // x codes and one scale per (token, 128 columns); h codes and one scale per (sorted
      // pair, 128 features) (H and I multiples of 128)
      L.xq = c.take((size_t)T * H);
      L.xs = c.take((size_t)T * (H / 128) * 4);
      L.hq = c.take(P * (size_t)I);
      L.hs = c.take(P * (size_t)(I / 128) * 4);
    } else {
      // x and h code rows padded to whole 128-wide blocks (zero past H, I)
      L.xq = c.take((size_t)T * moe::mfma_pad(H));
      L.xs = c.take((size_t)T * 4);
      L.hq = c.take(P * (size_t)moe::mfma_pad(I));
      L.hs = c.take(P * 4);
    }
  }
  if (act == MOE_ACT_GROUP_FP8) {
    L.xq = c.take((size_t)T * H);  // x codes and one scale per (token, 128 columns)
    L.xs = c.take((size_t)T * (H / 128) * 4);
  }
  L.total = c.off;
  return L;
}

int check_bank(const moe_fp8_bank* b, const char* name, int E, int64_t N, int64_t K) {
  if (!b) return fail(MOE_ERR_ARG, "%s is NULL", name);
  if (!b->codes || !b->scales) return fail(MOE_ERR_ARG, "%s.codes/scales is NULL", name);
  if (b->scale_dtype != MOE_F32 && b->scale_dtype != MOE_BF16)
    return fail(MOE_ERR_ARG, "%s.scale_dtype %d is not MOE_F32/MOE_BF16", name, b->scale_dtype);
  if (b->reserved != 0) return fail(MOE_ERR_ARG, "%s.reserved must be 0", name);
  if (!aligned16(b->codes)) return fail(MOE_ERR_ALIGN, "%s.codes must be 16-byte aligned", name);
  if (!aligned16(b->bias)) return fail(MOE_ERR_ALIGN, "%s.bias must be 16-byte aligned", name);
  if (b->expert_stride_bytes % 16 != 0)
    return fail(MOE_ERR_ALIGN, "%s.expert_stride_bytes must be a multiple of 16 (got %lld)", name,
                (long long)b->expert_stride_bytes);
  if (b->expert_stride_bytes < N * K)
    return fail(MOE_ERR_STRIDE, "%s.expert_stride_bytes %lld < N*K = %lld", name, (long long)b->expert_stride_bytes,
                (long long)(N * K));
  const int64_t rows = cdiv(N, 128), cols = cdiv(K, 128);
  if (b->scale_row_stride < cols)
    return fail(MOE_ERR_STRIDE, "%s.scale_row_stride %lld < ceil(K/128) = %lld", name,
                (long long)b->scale_row_stride, (long long)cols);
  const int64_t need = (rows - 1) * b->scale_row_stride + cols;
  if (b->scale_expert_stride < need)
    return fail(MOE_ERR_STRIDE, "%s.scale_expert_stride %lld < %lld (the unpadded extent)", name,
                (long long)b->scale_expert_stride, (long long)need);
  (void)E;
  return MOE_OK;
}

moe::BankArg bank_arg(const moe_fp8_bank* b) {
  moe::BankArg a;
  a.codes = b->codes;
  a.expert_stride = b->expert_stride_bytes;
  a.scales = b->scales;
  a.scale_bf16 = b->scale_dtype == MOE_BF16;
  a.srow = b->scale_row_stride;
  a.sexp = b->scale_expert_stride;
  a.bias = b->bias;
  return a;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

// Enqueues the kernels of one call in order, optionally timing kernel i with the caller's
// events 2i (start) and 2i+1 (end), attached to its dispatch, and naming it in kinds[i].
struct Runner {
  hipStream_t s;
  void* const* ev;
  int nev;
  int32_t* kinds;
  int n = 0;

  template <class F>
  hipError_t run(int kind, F&& launch) {
    const bool timed = ev != nullptr && 2 * n + 1 < nev;
    if (timed) moe::kernel_events() = moe::KernelEvents{(hipEvent_t)ev[2 * n], (hipEvent_t)ev[2 * n + 1]};
    hipError_t e = launch();
    if (timed && moe::kernel_events().start != nullptr) {
      // nothing was launched (an error path): leave the events at a zero-length interval
      moe::kernel_events() = moe::KernelEvents{};
      if (e == hipSuccess) e = hipEventRecord((hipEvent_t)ev[2 * n], s);
      if (e == hipSuccess) e = hipEventRecord((hipEvent_t)ev[2 * n + 1], s);
    }
    if (kinds != nullptr && n < nev / 2) kinds[n] = kind;
    ++n;
    return e;
  }
};

#define RUN(kind, call, what) HIP_CHECK(R.run(kind, [&]() { return (call); }), what)

int forward_impl(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13, const moe_fp8_bank* w2,
                 int T, int E, int H, int I, int top_k, void* out, int out_dtype, void* workspace,
                 size_t workspace_bytes, int32_t* ids_out, float* weights_out, const moe_opts* opts,
                 moe_run_info* info, void* stream, void* const* events, int n_events, int32_t* kinds,
                 size_t* checks_only = nullptr);
int mfma_up(Runner& R, const uint16_t* hidden, const moe::BankArg& b13, const moe::Plan& plan, void* workspace,
            const Layout& L, int T, int E, int H, int I, int top_k, float* hf, bool xq_ready = false);
int mfma_down(Runner& R, const float* hf, const moe::BankArg& b2, const moe::Plan& plan, void* workspace,
              const Layout& L, int T, int E, int H, int I, int top_k, void* out, int out_bf16);
int mfma_up_groups(Runner& R, const uint16_t* hidden, const moe::BankArg& b13, const moe::Plan& plan, void* workspace,
                   const Layout& L, int T, int E, int H, int I, int top_k, uint8_t* hq, float* hs);
int mfma_down_groups(Runner& R, const uint8_t* hq, const float* hs, const moe::BankArg& b2, const moe::Plan& plan,
                     void* workspace, const Layout& L, int T, int E, int H, int I, int top_k, void* out, int out_bf16);
int mfma_half_setup(Runner& R, const float* logits, const moe_fp8_bank* bank, const char* bank_name, int64_t N,
                    int64_t K, int T, int E, int H, int I, int top_k, int act_mode, void* workspace,
                    size_t workspace_bytes, Layout* Lout, moe::Plan* plan);

}  // namespace

// The workspace of moe_fp8_block_forward_static: a device array of this library, one copy
// per GPU, held until the process ends. Host code never passes the array's name to a
// kernel (in host code it is a host-side stand-in): each device's own address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[MOE_FP8_BLOCK_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, which must be the device of
// `stream` (the symbol is looked up with that device current).
int static_workspace(void* stream, void** ws) {
  int cur = 0;
  HIP_CHECK(hipGetDevice(&cur), "hipGetDevice");
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    HIP_CHECK(hipStreamGetDevice((hipStream_t)stream, &sdev), "hipStreamGetDevice");
    if ((int)sdev != cur)
      return fail(MOE_ERR_ARG, "stream belongs to device %d but device %d is current", (int)sdev, cur);
  }
  if (cur < 0 || cur >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d past %d", cur, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[cur] == nullptr) {
    void* p = nullptr;
    HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr || ((uintptr_t)p & (kAlign - 1)) != 0) return fail(MOE_ERR_HIP, "bad static workspace address");
    g_scratch_ptr[cur] = p;
  }
  *ws = g_scratch_ptr[cur];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_fp8_block_abi_version(void) { return MOE_FP8_BLOCK_ABI_VERSION; }

const char* moe_fp8_block_last_error(void) { return g_err.c_str(); }

int moe_fp8_block_default_opts(moe_opts* opts) {
  if (!opts) return fail(MOE_ERR_ARG, "opts is NULL");
  *opts = defaults();
  return ok();
}

int moe_fp8_block_select_path(int T, int E, int H, int I, int top_k, const moe_opts* opts, moe_run_info* info) {
  if (!info) return fail(MOE_ERR_ARG, "info is NULL");
  int st = check_sizes(T, E, top_k);
  if (st) return st;
  if (H <= 0 || I <= 0) return fail(MOE_ERR_ARG, "H and I must be positive (got H=%d, I=%d)", H, I);
  const moe_opts o = opts ? *opts : defaults();
  if ((st = check_opts(&o))) return st;
  int p = 0;
  if ((st = resolve_path(T, E, H, I, top_k, o, &p))) return st;
  info->path = p;
  info->act_mode = act_of(p, o);
  const int64_t P = (int64_t)T * top_k;
  info->slots = (int)(P < E ? P : E);
  info->kernels = 0;
  return ok();
}

size_t moe_fp8_block_route_workspace_size(int T, int E, int top_k) {
  if (check_sizes(T, E, top_k)) return 0;
  const size_t P = (size_t)T * top_k;
  const size_t slots = P < (size_t)E ? P : (size_t)E;
  Carve c;
  c.take((slots > 0 ? slots : 1) * 4);
  c.take(4);
  c.take(moe::sort_scratch_bytes((int)P, E));
  return c.off;
}

int moe_fp8_block_route(const float* logits, int T, int E, int top_k, int32_t* ids, float* weights, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_pairs, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int st = check_sizes(T, E, top_k);
  if (st) return st;
  if (T == 0) return ok();
  const bool any_sort = counts || offsets || sorted_pairs;
  const bool all_sort = counts && offsets && sorted_pairs;
  if (any_sort && !all_sort) return fail(MOE_ERR_ARG, "counts, offsets and sorted_pairs must all be set or all NULL");
  if (!logits || !ids || !weights) return fail(MOE_ERR_ARG, "logits, ids and weights must be non-NULL");
  const int P = T * top_k;
  const int slots = P < E ? P : E;
  const size_t need = moe_fp8_block_route_workspace_size(T, E, top_k);
  if (all_sort && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = (hipStream_t)stream;
  if (!all_sort) {
    HIP_CHECK(moe::launch_route_topk(logits, T, E, top_k, ids, weights, s), "route_topk launch");
  } else {
    Carve c;
    const size_t o_act = c.take((size_t)slots * 4);
    const size_t o_n = c.take(4);
    const size_t o_scr = c.take(moe::sort_scratch_bytes(P, E));
    for (int st = 0; st < moe::route_kernel_count(T, top_k); ++st)
      HIP_CHECK(moe::launch_route_stage(st, logits, T, E, top_k, ids, weights, counts, offsets, sorted_pairs,
                                        at<int32_t>(workspace, o_act), at<int32_t>(workspace, o_n), slots, 0,
                                        nullptr, at<void>(workspace, o_scr), s),
                "route launch");
  }
  return ok();
}

size_t moe_fp8_block_workspace_size(int T, int E, int H, int I, int top_k, const moe_opts* opts) {
  if (check_sizes(T, E, top_k) || H <= 0 || I <= 0) return 0;
  const moe_opts o = opts ? *opts : defaults();
  if (check_opts(&o)) return 0;
  int path = 0;
  if (resolve_path(T, E, H, I, top_k, o, &path)) return 0;
  return layout_for(path, act_of(path, o), T, E, H, I, top_k).total;
}

}  // extern "C"

namespace moe {
KernelEvents& kernel_events() {
  thread_local KernelEvents ev;
  return ev;
}
}  // namespace moe

namespace {

// checks_only: run every argument check, store the workspace the call needs there and
// return without a HIP call.
int forward_impl(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13, const moe_fp8_bank* w2,
                 int T, int E, int H, int I, int top_k, void* out, int out_dtype, void* workspace,
                 size_t workspace_bytes, int32_t* ids_out, float* weights_out, const moe_opts* opts,
                 moe_run_info* info, void* stream, void* const* events, int n_events, int32_t* kinds,
                 size_t* checks_only) {
  int st = check_sizes(T, E, top_k);
  if (st) return st;
  if (H <= 0 || I <= 0) return fail(MOE_ERR_ARG, "H and I must be positive (got H=%d, I=%d)", H, I);
  // rows of 16-byte code chunks; a last 128-wide scale block may be partial on every path
  if (H % 16 != 0 || I % 16 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "H and I must be multiples of 16 (got H=%d, I=%d)", H, I);
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return fail(MOE_ERR_ARG, "out_dtype %d is not F32/BF16", out_dtype);
  const moe_opts o = opts ? *opts : defaults();
  if ((st = check_opts(&o))) return st;
  if ((st = check_bank(w13, "w13", E, 2 * (int64_t)I, H))) return st;
  if ((st = check_bank(w2, "w2", E, H, I))) return st;
  int path = 0;
  if ((st = resolve_path(T, E, H, I, top_k, o, &path))) return st;
  const int64_t P = (int64_t)T * top_k;
  if (info) {
    info->path = path;
    info->act_mode = act_of(path, o);
    info->slots = (int)(P < E ? P : E);
    info->kernels = 0;
  }
  if (T == 0) {
    if (checks_only) *checks_only = 0;
    return ok();
  }
  if (!hidden || !logits || !out) return fail(MOE_ERR_ARG, "hidden, logits and out must be non-NULL");
  if (!aligned16(hidden)) return fail(MOE_ERR_ALIGN, "hidden must be 16-byte aligned");
  if (!aligned16(out)) return fail(MOE_ERR_ALIGN, "out must be 16-byte aligned");
  const int act_mode = act_of(path, o);
  const Layout L = layout_for(path, act_mode, T, E, H, I, top_k);
  if (checks_only) {
    *checks_only = L.total;
    return ok();
  }
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  const int slots = (int)(P < E ? P : E);
  int32_t* ids = ids_out ? ids_out : at<int32_t>(workspace, L.ids);
  float* w = weights_out ? weights_out : at<float>(workspace, L.w);
  int32_t* counts = at<int32_t>(workspace, L.counts);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted = at<int32_t>(workspace, L.sorted);
  int32_t* act = at<int32_t>(workspace, L.act);
  int32_t* n_act = at<int32_t>(workspace, L.n_act);
  int32_t* tile_off = at<int32_t>(workspace, L.tile_off);
  const int out_bf16 = out_dtype == MOE_BF16;
  const moe::BankArg b13 = bank_arg(w13), b2 = bank_arg(w2);
  Runner R{s, events, n_events, kinds};

  // small gather batches route inside GEMM1; everything else routes and sorts first
  // group-fp8 activations fuse too, quantised inside GEMM1, where x is not staged in LDS
  const bool fused = path == MOE_PATH_GATHER &&
                     (act_mode == MOE_ACT_PATH ? moe::gemm1_fused_route_ok(T, top_k)
                                               : act_mode == MOE_ACT_GROUP_FP8 && moe::gemm1_fused_qx_ok(T, top_k, H));
  const int tile_m = path == MOE_PATH_MFMA ? moe::kMfmaTileM : 0;
  // per-row MFMA activations: where the routing starts with a top-k kernel of one wave per
  // token, that kernel also quantises the token's row of x
  const bool xq_route = path == MOE_PATH_MFMA && act_mode == MOE_ACT_ROW_FP8 && moe::route_topk_first(T, top_k);
  if (!fused) {
    for (int st = 0; st < moe::route_kernel_count(T, top_k); ++st) {
      if (st == 0 && xq_route) {
        RUN(MOE_K_ROUTE,
            moe::launch_route_topk_quant(logits, hidden, T, E, top_k, H, moe::mfma_pad(H), ids, w,
                                         at<uint8_t>(workspace, L.xq), at<float>(workspace, L.xs), s),
            "route launch");
        continue;
      }
      RUN(st == 0 ? MOE_K_ROUTE : MOE_K_SORT,
          moe::launch_route_stage(st, logits, T, E, top_k, ids, w, counts, offsets, sorted, act, n_act, slots,
                                  tile_m, tile_off, at<void>(workspace, L.scratch), s),
          "route launch");
    }
  }
  const moe::Plan plan{ids, w, counts, offsets, sorted, act, tile_off};

  if (path == MOE_PATH_GATHER || path == MOE_PATH_STREAM) {
    float* h = at<float>(workspace, L.h);
    moe::Gemm1Args g1{hidden, logits, T, E, H, I, top_k, slots, b13, plan, h, fused ? 1 : 0, ids, w};
    if (act_mode == MOE_ACT_GROUP_FP8 && fused) {
      g1.qx = 1;
    } else if (act_mode == MOE_ACT_GROUP_FP8) {
      // one quantisation row per (token, 128 columns)
      g1.xq = at<uint8_t>(workspace, L.xq);
      g1.xs = at<float>(workspace, L.xs);
      RUN(MOE_K_QUANT, moe::launch_quant_groups_bf16(hidden, T, H, at<uint8_t>(workspace, L.xq),
                                                     at<float>(workspace, L.xs), s),
          "quant launch");
    }
    RUN(MOE_K_GEMM1, moe::launch_gemm1_w8a16(g1, s), "gemm1 launch");
    if (path == MOE_PATH_GATHER) {
      RUN(MOE_K_GEMM2, moe::launch_gemm2_gather(h, b2, ids, w, T, H, I, top_k, out, out_bf16, s), "gemm2 launch");
    } else {
      float* y = at<float>(workspace, L.y);
      RUN(MOE_K_GEMM2, moe::launch_gemm2_expert(h, b2, plan, slots, H, I, top_k, y, s), "gemm2 launch");
      RUN(MOE_K_COMBINE, moe::launch_combine(y, w, T, H, top_k, out, out_bf16, s), "combine launch");
    }
  } else if (act_mode == MOE_ACT_GROUP_FP8_W8A8) {
    uint8_t* hq = at<uint8_t>(workspace, L.hq);
    float* hs = at<float>(workspace, L.hs);
    int st2 = mfma_up_groups(R, hidden, b13, plan, workspace, L, T, E, H, I, top_k, hq, hs);
    if (st2 == MOE_OK) st2 = mfma_down_groups(R, hq, hs, b2, plan, workspace, L, T, E, H, I, top_k, out, out_bf16);
    if (st2 != MOE_OK) return st2;
  } else {
    float* hf = at<float>(workspace, L.h);
    int st2 = mfma_up(R, hidden, b13, plan, workspace, L, T, E, H, I, top_k, hf, xq_route);
    if (st2 == MOE_OK) st2 = mfma_down(R, hf, b2, plan, workspace, L, T, E, H, I, top_k, out, out_bf16);
    if (st2 != MOE_OK) return st2;
  }
  if (info) info->kernels = R.n;
  return ok();
}

// The MFMA path's first half: x quantised per token (unless the routing kernel did it:
// xq_ready), then GEMM1 + silu*up into hf (float, [P, I] in sorted-position order).
int mfma_up(Runner& R, const uint16_t* hidden, const moe::BankArg& b13, const moe::Plan& plan, void* workspace,
            const Layout& L, int T, int E, int H, int I, int top_k, float* hf, bool xq_ready) {
  hipStream_t s = R.s;
  const int64_t P = (int64_t)T * top_k;
  uint8_t* xq = at<uint8_t>(workspace, L.xq);
  float* xs = at<float>(workspace, L.xs);
  if (!xq_ready) RUN(MOE_K_QUANT, moe::launch_quant_rows_bf16(hidden, T, H, moe::mfma_pad(H), xq, xs, s), "quant launch");
  RUN(MOE_K_GEMM1, moe::launch_gemm1_mfma(xq, xs, b13, plan, E, (int)P, H, I, top_k, hf, s), "gemm1 mfma launch");
  return MOE_OK;
}

// The second half: h quantised per (token, slot) row, the down GEMM and the combine.
int mfma_down(Runner& R, const float* hf, const moe::BankArg& b2, const moe::Plan& plan, void* workspace,
              const Layout& L, int T, int E, int H, int I, int top_k, void* out, int out_bf16) {
  hipStream_t s = R.s;
  const int64_t P = (int64_t)T * top_k;
  uint8_t* hq = at<uint8_t>(workspace, L.hq);
  float* hs = at<float>(workspace, L.hs);
  RUN(MOE_K_HQUANT, moe::launch_quant_rows_f32(hf, (int)P, I, moe::mfma_pad(I), hq, hs, s), "h quant launch");
  _Float16* y16 = at<_Float16>(workspace, L.y);
  int8_t* yexp = at<int8_t>(workspace, L.yexp);
  RUN(MOE_K_GEMM2, moe::launch_gemm2_mfma(hq, hs, b2, plan, E, (int)P, H, I, y16, yexp, s), "gemm2 mfma launch");
  RUN(MOE_K_COMBINE, moe::launch_combine_f16(y16, yexp, plan.w, plan.ids, b2.bias, T, H, top_k, moe::mfma_k_parts(I),
                                             out, out_bf16, s),
      "combine launch");
  return MOE_OK;
}

// The group-scaled variant: x quantised per (token, 128 columns), then GEMM1 with h
// quantised per (sorted pair, 128 features) in its epilogue into hq / hs.
int mfma_up_groups(Runner& R, const uint16_t* hidden, const moe::BankArg& b13, const moe::Plan& plan, void* workspace,
                   const Layout& L, int T, int E, int H, int I, int top_k, uint8_t* hq, float* hs) {
  hipStream_t s = R.s;
  const int64_t P = (int64_t)T * top_k;
  uint8_t* xq = at<uint8_t>(workspace, L.xq);
  float* xs = at<float>(workspace, L.xs);
  RUN(MOE_K_QUANT, moe::launch_quant_groups_bf16(hidden, T, H, xq, xs, s), "quant launch");
  RUN(MOE_K_GEMM1, moe::launch_gemm1_mfma_groups(xq, xs, b13, plan, E, (int)P, H, I, top_k, hq, hs, s),
      "gemm1 mfma launch");
  return MOE_OK;
}

// Its second half: the down GEMM on the group-scaled h codes, and the combine.
int mfma_down_groups(Runner& R, const uint8_t* hq, const float* hs, const moe::BankArg& b2, const moe::Plan& plan,
                     void* workspace, const Layout& L, int T, int E, int H, int I, int top_k, void* out,
                     int out_bf16) {
  hipStream_t s = R.s;
  const int64_t P = (int64_t)T * top_k;
  _Float16* y16 = at<_Float16>(workspace, L.y);
  int8_t* yexp = at<int8_t>(workspace, L.yexp);
  RUN(MOE_K_GEMM2, moe::launch_gemm2_mfma_groups(hq, hs, b2, plan, E, (int)P, H, I, y16, yexp, s),
      "gemm2 mfma launch");
  RUN(MOE_K_COMBINE, moe::launch_combine_f16(y16, yexp, plan.w, plan.ids, b2.bias, T, H, top_k, moe::mfma_k_parts(I),
                                             out, out_bf16, s),
      "combine launch");
  return MOE_OK;
}

// Checks and routing shared by the test exports of the MFMA halves: the sizes, the bank,
// the workspace of a forward forced onto MFMA with activations act_mode (MOE_ACT_ROW_FP8 or
// MOE_ACT_GROUP_FP8_W8A8), then route + sort into the workspace.
int mfma_half_setup(Runner& R, const float* logits, const moe_fp8_bank* bank, const char* bank_name, int64_t N,
                    int64_t K, int T, int E, int H, int I, int top_k, int act_mode, void* workspace,
                    size_t workspace_bytes, Layout* Lout, moe::Plan* plan) {
  int st = check_sizes(T, E, top_k);
  if (st) return st;
  if (!moe::mfma_shape_ok(H, I))
    return fail(MOE_ERR_UNSUPPORTED, "MFMA path needs H <= 8192 and I <= 4096 (got H=%d, I=%d)", H, I);
  if (act_mode == MOE_ACT_GROUP_FP8_W8A8 && !moe::mfma_groups_shape_ok(H, I))
    return fail(MOE_ERR_UNSUPPORTED, "group-scaled MFMA needs H and I multiples of 128 (got H=%d, I=%d)", H, I);
  if ((st = check_bank(bank, bank_name, E, N, K))) return st;
  if (T == 0) return ok();
  if (!logits) return fail(MOE_ERR_ARG, "logits must be non-NULL");
  const Layout L = layout_for(MOE_PATH_MFMA, act_mode, T, E, H, I, top_k);
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  const int64_t P = (int64_t)T * top_k;
  const int slots = (int)(P < E ? P : E);
  int32_t* ids = at<int32_t>(workspace, L.ids);
  float* w = at<float>(workspace, L.w);
  int32_t* counts = at<int32_t>(workspace, L.counts);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted = at<int32_t>(workspace, L.sorted);
  int32_t* act = at<int32_t>(workspace, L.act);
  int32_t* tile_off = at<int32_t>(workspace, L.tile_off);
  hipStream_t s = R.s;
  for (int stg = 0; stg < moe::route_kernel_count(T, top_k); ++stg)
    RUN(stg == 0 ? MOE_K_ROUTE : MOE_K_SORT,
        moe::launch_route_stage(stg, logits, T, E, top_k, ids, w, counts, offsets, sorted, act,
                                at<int32_t>(workspace, L.n_act), slots, moe::kMfmaTileM, tile_off,
                                at<void>(workspace, L.scratch), s),
        "route launch");
  *Lout = L;
  *plan = moe::Plan{ids, w, counts, offsets, sorted, act, tile_off};
  return MOE_OK;
}

}  // namespace

extern "C" {


int moe_fp8_block_forward(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13,
                          const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out, int out_dtype,
                          void* workspace, size_t workspace_bytes, int32_t* ids_out, float* weights_out,
                          const moe_opts* opts, moe_run_info* info, void* stream) {
  return forward_impl(hidden, logits, w13, w2, T, E, H, I, top_k, out, out_dtype, workspace, workspace_bytes, ids_out,
                      weights_out, opts, info, stream, nullptr, 0, nullptr);
}

int moe_fp8_block_forward_timed(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13,
                                const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out,
                                int out_dtype, void* workspace, size_t workspace_bytes, int32_t* ids_out,
                                float* weights_out, const moe_opts* opts, moe_run_info* info, void* stream,
                                void* const* events, int n_events, int32_t* kinds) {
  if (n_events < 0 || (n_events > 0 && events == nullptr)) return fail(MOE_ERR_ARG, "events/n_events inconsistent");
  for (int i = 0; kinds != nullptr && i < n_events / 2; ++i) kinds[i] = 0;
  return forward_impl(hidden, logits, w13, w2, T, E, H, I, top_k, out, out_dtype, workspace, workspace_bytes, ids_out,
                      weights_out, opts, info, stream, events, n_events, kinds);
}

int moe_fp8_block_mfma_up(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13, int T, int E, int H,
                          int I, int top_k, float* h, void* workspace, size_t workspace_bytes, void* stream) {
  Runner R{(hipStream_t)stream, nullptr, 0, nullptr};
  Layout L{};
  moe::Plan plan{};
  if (T > 0) {  // every check before the routing is enqueued
    if (!hidden || !h) return fail(MOE_ERR_ARG, "hidden and h must be non-NULL");
    if (!aligned16(hidden) || !aligned16(h)) return fail(MOE_ERR_ALIGN, "hidden and h must be 16-byte aligned");
  }
  int st = mfma_half_setup(R, logits, w13, "w13", 2 * (int64_t)I, H, T, E, H, I, top_k, MOE_ACT_ROW_FP8, workspace,
                           workspace_bytes, &L, &plan);
  if (st != MOE_OK || T == 0) return st;
  st = mfma_up(R, hidden, bank_arg(w13), plan, workspace, L, T, E, H, I, top_k, h);
  return st != MOE_OK ? st : ok();
}

int moe_fp8_block_mfma_down(const float* h, const float* logits, const moe_fp8_bank* w2, int T, int E, int H, int I,
                            int top_k, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  Runner R{(hipStream_t)stream, nullptr, 0, nullptr};
  Layout L{};
  moe::Plan plan{};
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return fail(MOE_ERR_ARG, "out_dtype %d is not F32/BF16", out_dtype);
  if (T > 0) {
    if (!h || !out) return fail(MOE_ERR_ARG, "h and out must be non-NULL");
    if (!aligned16(h) || !aligned16(out)) return fail(MOE_ERR_ALIGN, "h and out must be 16-byte aligned");
  }
  int st = mfma_half_setup(R, logits, w2, "w2", H, I, T, E, H, I, top_k, MOE_ACT_ROW_FP8, workspace, workspace_bytes,
                           &L, &plan);
  if (st != MOE_OK || T == 0) return st;
  st = mfma_down(R, h, bank_arg(w2), plan, workspace, L, T, E, H, I, top_k, out, out_dtype == MOE_BF16);
  return st != MOE_OK ? st : ok();
}

int moe_fp8_block_mfma_up_groups(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13, int T, int E,
                                 int H, int I, int top_k, uint8_t* h_codes, float* h_scales, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  Runner R{(hipStream_t)stream, nullptr, 0, nullptr};
  Layout L{};
  moe::Plan plan{};
  if (T > 0) {
    if (!hidden || !h_codes || !h_scales) return fail(MOE_ERR_ARG, "hidden, h_codes and h_scales must be non-NULL");
    if (!aligned16(hidden) || !aligned16(h_codes))
      return fail(MOE_ERR_ALIGN, "hidden and h_codes must be 16-byte aligned");
  }
  int st = mfma_half_setup(R, logits, w13, "w13", 2 * (int64_t)I, H, T, E, H, I, top_k, MOE_ACT_GROUP_FP8_W8A8,
                           workspace, workspace_bytes, &L, &plan);
  if (st != MOE_OK || T == 0) return st;
  st = mfma_up_groups(R, hidden, bank_arg(w13), plan, workspace, L, T, E, H, I, top_k, h_codes, h_scales);
  return st != MOE_OK ? st : ok();
}

int moe_fp8_block_mfma_down_groups(const uint8_t* h_codes, const float* h_scales, const float* logits,
                                   const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out,
                                   int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  Runner R{(hipStream_t)stream, nullptr, 0, nullptr};
  Layout L{};
  moe::Plan plan{};
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return fail(MOE_ERR_ARG, "out_dtype %d is not F32/BF16", out_dtype);
  if (T > 0) {
    if (!h_codes || !h_scales || !out) return fail(MOE_ERR_ARG, "h_codes, h_scales and out must be non-NULL");
    if (!aligned16(h_codes) || !aligned16(out)) return fail(MOE_ERR_ALIGN, "h_codes and out must be 16-byte aligned");
  }
  int st = mfma_half_setup(R, logits, w2, "w2", H, I, T, E, H, I, top_k, MOE_ACT_GROUP_FP8_W8A8, workspace,
                           workspace_bytes, &L, &plan);
  if (st != MOE_OK || T == 0) return st;
  st = mfma_down_groups(R, h_codes, h_scales, bank_arg(w2), plan, workspace, L, T, E, H, I, top_k, out,
                        out_dtype == MOE_BF16);
  return st != MOE_OK ? st : ok();
}

int moe_fp8_block_forward_static(const uint16_t* hidden, const float* logits, const moe_fp8_bank* w13,
                                 const moe_fp8_bank* w2, int T, int E, int H, int I, int top_k, void* out,
                                 int out_dtype, int32_t* ids_out, float* weights_out, const moe_opts* opts,
                                 moe_run_info* info, void* stream) {
  size_t need = 0;
  int st = forward_impl(hidden, logits, w13, w2, T, E, H, I, top_k, out, out_dtype, nullptr, 0, ids_out, weights_out,
                        opts, info, stream, nullptr, 0, nullptr, &need);
  if (st != MOE_OK) return st;
  if (need > (size_t)MOE_FP8_BLOCK_STATIC_WORKSPACE_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this call needs %zu bytes of workspace; the static workspace holds %zu (use moe_fp8_block_forward "
                "with a caller workspace)",
                need, (size_t)MOE_FP8_BLOCK_STATIC_WORKSPACE_BYTES);
  if (T == 0) return ok();
  void* ws = nullptr;
  if ((st = static_workspace(stream, &ws)) != MOE_OK) return st;
  return forward_impl(hidden, logits, w13, w2, T, E, H, I, top_k, out, out_dtype, ws,
                      (size_t)MOE_FP8_BLOCK_STATIC_WORKSPACE_BYTES, ids_out, weights_out, opts, info, stream, nullptr,
                      0, nullptr);
}

int moe_fp8_block_quantize_rows(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales, void* stream) {
  if (rows < 0 || cols <= 0) return fail(MOE_ERR_ARG, "rows must be >= 0 and cols > 0");
  if (cols % 16 != 0 || cols > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "cols must be a multiple of 16 and at most 8192 (got %d)", cols);
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(MOE_ERR_ARG, "x, codes and scales must be non-NULL");
  if (!aligned16(x) || !aligned16(codes)) return fail(MOE_ERR_ALIGN, "x and codes must be 16-byte aligned");
  HIP_CHECK(moe::launch_quant_rows_bf16(x, rows, cols, cols, codes, scales, (hipStream_t)stream), "quant launch");
  return ok();
}

int moe_fp8_block_quantize_groups(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                                  void* stream) {
  if (rows < 0 || cols <= 0) return fail(MOE_ERR_ARG, "rows must be >= 0 and cols > 0");
  if (cols % 128 != 0 || cols > 8192)
    return fail(MOE_ERR_UNSUPPORTED, "cols must be a multiple of 128 and at most 8192 (got %d)", cols);
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(MOE_ERR_ARG, "x, codes and scales must be non-NULL");
  if (!aligned16(x) || !aligned16(codes)) return fail(MOE_ERR_ALIGN, "x and codes must be 16-byte aligned");
  HIP_CHECK(moe::launch_quant_groups_bf16(x, rows, cols, codes, scales, (hipStream_t)stream), "quant launch");
  return ok();
}

int moe_fp8_block_decode_e4m3(const uint8_t* codes, float* out, int64_t n, void* stream) {
  if (n < 0) return fail(MOE_ERR_ARG, "n must be >= 0");
  if (n == 0) return ok();
  if (!codes || !out) return fail(MOE_ERR_ARG, "codes and out must be non-NULL");
  HIP_CHECK(moe::launch_decode_e4m3(codes, out, n, (hipStream_t)stream), "decode launch");
  return ok();
}

int moe_fp8_block_decode_e4m3_paths(const uint8_t* chunks, float* out, int64_t n, void* stream) {
  if (n < 0) return fail(MOE_ERR_ARG, "n must be >= 0");
  if (n == 0) return ok();
  if (!chunks || !out) return fail(MOE_ERR_ARG, "chunks and out must be non-NULL");
  if (!aligned16(chunks)) return fail(MOE_ERR_ALIGN, "chunks must be 16-byte aligned");
  HIP_CHECK(moe::launch_decode_paths(chunks, out, n, (hipStream_t)stream), "decode paths launch");
  return ok();
}

int moe_fp8_block_encode_e4m3(const float* x, uint8_t* codes, int64_t n, void* stream) {
  if (n < 0) return fail(MOE_ERR_ARG, "n must be >= 0");
  if (n == 0) return ok();
  if (!x || !codes) return fail(MOE_ERR_ARG, "x and codes must be non-NULL");
  HIP_CHECK(moe::launch_encode_e4m3(x, codes, n, (hipStream_t)stream), "encode launch");
  return ok();
}

}  // extern "C"
