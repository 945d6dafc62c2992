// Host side of the C ABI: validation, workspace layout and the launch
// sequence of the layer forward.  No allocation, no host copy, no
// synchronisation: every call only enqueues kernels on the caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe_ffn.h"
#include "kernels.hpp"

using namespace moe;

namespace {

thread_local std::string g_last_error;

// measurement hook (moe_profile_stage)
struct ProfileHook {
  int stage = -1;
  void *const *start = nullptr;
  void *const *stop = nullptr;
  int n = 0;
  long calls = 0;
};
thread_local ProfileHook g_profile;

thread_local LaunchEvents g_launch_events;

// Stages whose work is a single kernel: their events ride on that kernel's
// launch (recorded by the GPU at the kernel's own start and end).  The router
// stages (no kernel, one or two) are bracketed by event records instead.
bool single_kernel_stage(int stage) {
  return stage >= MOE_STAGE_PERMUTE && stage <= MOE_STAGE_COMBINE;
}

// Arms (begin = true) or closes the hook's events around `stage`.
hipError_t profile_mark(int stage, bool begin, hipStream_t st) {
  if (g_profile.stage != stage || g_profile.n <= 0) return hipSuccess;
  const int i = (int)(g_profile.calls % g_profile.n);
  hipEvent_t start = static_cast<hipEvent_t>(g_profile.start[i]);
  hipEvent_t stop = static_cast<hipEvent_t>(g_profile.stop[i]);
  if (single_kernel_stage(stage)) {
    if (begin) {
      g_launch_events = LaunchEvents{start, stop};
      return hipSuccess;
    }
    if (!g_launch_events.start) return hipSuccess;  // the kernel took them
    g_launch_events = LaunchEvents{};               // no kernel ran: an empty interval
    hipError_t e = hipEventRecord(start, st);
    return e != hipSuccess ? e : hipEventRecord(stop, st);
  }
  return hipEventRecord(begin ? start : stop, st);
}

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() { return MOE_OK; }

// Token counts from which the expert GEMMs use the LDS-tiled kernels (routed
// experts, shared expert); below them the weight-streaming kernels.
constexpr int kTiledMinTokens = 512;
constexpr int kTiledMinTokensShared = 256;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t act_bytes(const moe_config &c) { return c.act_dtype == MOE_DTYPE_F32 ? 4 : 2; }

bool has_shared(const moe_config &c) { return c.shared_I > 0; }
bool has_shared_gate(const moe_config &c) { return c.shared_I > 0 && c.shared_gated; }
int logits_ld(const moe_config &c) { return c.E + (has_shared_gate(c) ? 1 : 0); }

// Which kernels run the routed expert GEMMs, and the rows per chunk of the
// expert-sorted rows that the permutation cuts for them.
//   streaming: experts hold a few rows; the GEMMs read each weight once
//   tiled:     from kTiledMinTokens tokens; still bound by weight reads
//   big tile:  experts hold >= kBigTileRows rows on average; matrix-core
//              bound.  Runs gate_up; the down projection (which also
//              multiplies the low halves of h) stays on the tiled kernel.
// Measured on the weight-bound sizes (DeepSeek-V4-style layer, T=4096,
// 92 rows per expert at the median): gate_up on the big tile with 128- or
// 256-row tiles, with or without loading only the token fragments that hold
// rows, and on its register-staged form, was no faster than the tiled kernel.
struct GemmPlan {
  bool tiled, big;        // routed experts
  bool tiled_shared, big_shared;
  bool mx_scaled;         // MXFP4 routed gate_up on the block-scaled matrix cores
  int chunk_rows;         // streaming kernel chunks, or the big-tile kernel's row tile
};

constexpr long kBigTileRows = 256;
constexpr int kQueuedLaunches = 6;  // tiled routed/shared gate_up and down, big-tile routed/shared gate_up

// 32-bit offsets of the big-tile kernel: activations, h and one expert's
// weights below 4 GiB
bool big_fits(const moe_config &c, long rows) {
  const double lim = 4294967296.0 - 65536.0;
  const double act = (double)rows * std::max(c.H, std::max(c.I, c.shared_I)) * 2.0;
  const double w = 2.0 * std::max(c.I, c.shared_I) * (double)c.H * 2.0;
  return act < lim && w < lim;
}

GemmPlan gemm_plan(const moe_config &c) {
  GemmPlan p{};
  const bool mfma = c.w_dtype != MOE_DTYPE_F32;
  const long slots = (long)c.T * c.K;
  const long active = std::max(1L, std::min<long>(c.E, slots));
  p.tiled = mfma && c.T >= kTiledMinTokens;
  p.big = p.tiled && slots / active >= kBigTileRows && big_fits(c, slots);
  p.tiled_shared = c.act_dtype != MOE_DTYPE_F32 && c.T >= kTiledMinTokensShared;
  p.big_shared = p.tiled_shared && c.T >= kBigTileRows && big_fits(c, c.T);
  p.mx_scaled = p.big && c.w_dtype == MOE_DTYPE_MXFP4 && c.mx_gemm == MOE_MX_BLOCK_SCALED && c.H % 64 == 0 &&
                c.H <= 4096;
  p.chunk_rows = p.big ? bigtile_rows() : p.tiled ? tiled_tile_rows() : stream_chunk_rows(slots, c.E);
  return p;
}

// Workspace carve-up; every buffer starts on a 256-byte boundary.
struct Layout {
  size_t logits, gamma, scores, indices, weights, counts, offsets, active_all, n_active_all,
      mtile_prefix, mtile_prefix2, chunks, n_chunks, perm, inv;
  size_t h, y, sh_h, sh_y, mxq, mxs, tile_queue, total;
};

Layout make_layout(const moe_config &c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t T = c.T, K = c.K, E = c.E, H = c.H, I = c.I, Is = c.shared_I;
  int mt, n_split, per;
  router_logits_plan(c.T, c.H, logits_ld(c), c.act_dtype == MOE_DTYPE_BF16, &mt, &n_split, &per);
  L.logits = take((size_t)n_split * T * logits_ld(c) * 8);
  L.gamma = take(T * 4);
  L.scores = take(T * E * 4);
  L.indices = take(T * K * 4);
  L.weights = take(T * K * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.active_all = take(E * 4);
  L.n_active_all = take(4);
  L.mtile_prefix = take((E + 1) * 4);
  L.mtile_prefix2 = take((E + 1) * 4);
  L.chunks = take((T * K + E) * 16);
  L.n_chunks = take(4);
  L.perm = take(T * K * 4);
  L.inv = take(T * K * 4);
  // bf16 activations keep h as a bf16 (hi, lo) pair: h = hi + lo to ~16 bits
  const size_t hparts = c.act_dtype == MOE_DTYPE_BF16 ? 2 : 1;
  L.h = take(hparts * T * K * I * act_bytes(c));
  L.y = take(T * K * H * 4);
  L.sh_h = take(hparts * T * Is * act_bytes(c));
  L.sh_y = take(Is ? T * H * 4 : 0);
  // the activations as two MXFP8 terms for the block-scaled gate_up
  const bool mxs = gemm_plan(c).mx_scaled;
  L.mxq = take(mxs ? T * H * 2 : 0);
  L.mxs = take(mxs ? T * (H / 32) * 2 : 0);
  // tile counters of the tiled and big-tile launches
  L.tile_queue = take(kQueuedLaunches * kTiledQueueInts * 4);
  L.total = off;
  return L;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

int check_workspace(const moe_config &c, void *ws, size_t ws_bytes) {
  const size_t need = make_layout(c).total;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return MOE_OK;
}

#define REQUIRE_PTR(p, name)                                                          \
  do {                                                                                \
    if (!(p)) return fail(MOE_ERR_INVALID, "%s is NULL", name);                       \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID, "%s is not 16-byte aligned", name); \
  } while (0)

#define OPTIONAL_PTR(p, name)                                                        \
  do {                                                                               \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_INVALID, "%s is not 16-byte aligned", name); \
  } while (0)

int hip_fail(hipError_t e, const char *what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                         \
  do {                                              \
    hipError_t e_ = (expr);                         \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

struct RouteBuffers {
  float *scores;
  int32_t *indices;
  float *weights;
};

// Router + permutation; shared by both entry points.
int enqueue_route(const moe_config &c, const void *x, const void *gate_w, const void *sh_gate,
                  const float *router_bias, const float *expert_bias, const RouteBuffers &rb,
                  int32_t *user_counts, char *ws, const Layout &L, bool need_permute,
                  hipStream_t st) {
  LogitsArgs la{};
  la.x = x;
  la.gate = gate_w;
  la.sh_gate = has_shared_gate(c) ? sh_gate : nullptr;
  la.partial = reinterpret_cast<double *>(ws + L.logits);
  la.T = c.T;
  la.H = c.H;
  la.E = c.E;
  la.ldl = logits_ld(c);
  int mt;
  router_logits_plan(c.T, c.H, la.ldl, c.act_dtype == MOE_DTYPE_BF16, &mt, &la.n_split,
                     &la.blocks_per_split);
  // few columns and tokens: the select kernel computes the logits itself
  const bool fused = router_fused_applies(c.T, c.H, c.E, la.sh_gate != nullptr);
  HIP_TRY(profile_mark(MOE_STAGE_ROUTER_LOGITS, true, st), "profile event");
  if (!fused) HIP_TRY(launch_router_logits(la, c.act_dtype == MOE_DTYPE_BF16, st), "router logits launch");
  HIP_TRY(profile_mark(MOE_STAGE_ROUTER_LOGITS, false, st), "profile event");

  SelectArgs sa{};
  sa.partial = la.partial;
  sa.n_split = la.n_split;
  sa.router_bias = router_bias;
  sa.expert_bias = expert_bias;
  sa.scores = rb.scores;
  sa.indices = rb.indices;
  sa.weights = rb.weights;
  sa.gamma = reinterpret_cast<float *>(ws + L.gamma);
  sa.T = c.T;
  sa.E = c.E;
  sa.K = c.K;
  sa.ldl = la.ldl;
  sa.score_fn = c.score_fn;
  sa.n_group = c.n_group;
  sa.topk_group = c.topk_group;
  sa.norm = c.norm_topk_prob;
  sa.route_scale = c.route_scale;
  sa.has_shared_gate = la.sh_gate != nullptr;
  if (fused) {
    sa.x = x;
    sa.gate = gate_w;
    sa.sh_gate = la.sh_gate;
    sa.H = c.H;
    sa.x_bf16 = c.act_dtype == MOE_DTYPE_BF16;
  }
  HIP_TRY(profile_mark(MOE_STAGE_ROUTER_SELECT, true, st), "profile event");
  HIP_TRY(launch_router_select(sa, st), "router select launch");
  HIP_TRY(profile_mark(MOE_STAGE_ROUTER_SELECT, false, st), "profile event");

  if (need_permute || user_counts) {
    PermuteArgs pa{};
    pa.indices = rb.indices;
    pa.counts = reinterpret_cast<int32_t *>(ws + L.counts);
    pa.user_counts = user_counts;
    pa.offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    pa.active_all = reinterpret_cast<int32_t *>(ws + L.active_all);
    pa.n_active_all = reinterpret_cast<int32_t *>(ws + L.n_active_all);
    pa.mtile_prefix = reinterpret_cast<int32_t *>(ws + L.mtile_prefix);
    pa.chunks = reinterpret_cast<int4 *>(ws + L.chunks);
    pa.n_chunks = reinterpret_cast<int32_t *>(ws + L.n_chunks);
    pa.chunk_rows = gemm_plan(c).chunk_rows;
    pa.tile_rows = pa.chunk_rows;
    pa.mtile_prefix2 = reinterpret_cast<int32_t *>(ws + L.mtile_prefix2);
    pa.tile_rows2 = tiled_tile_rows();
    pa.perm = reinterpret_cast<int32_t *>(ws + L.perm);
    pa.inv = reinterpret_cast<int32_t *>(ws + L.inv);
    pa.n_slots = c.T * c.K;
    pa.E = c.E;
    HIP_TRY(profile_mark(MOE_STAGE_PERMUTE, true, st), "profile event");
    HIP_TRY(launch_permute(pa, st), "permute launch");
    HIP_TRY(profile_mark(MOE_STAGE_PERMUTE, false, st), "profile event");
  }
  return MOE_OK;
}

}  // namespace

namespace moe {
LaunchEvents &pending_launch_events() { return g_launch_events; }
}  // namespace moe

extern "C" {

MOE_API int moe_abi_version(void) { return MOE_FFN_ABI_VERSION; }

MOE_API int moe_profile_stage(int stage, void *const *start_events, void *const *stop_events,
                              int n_events) {
  if (stage >= MOE_NUM_STAGES) return fail(MOE_ERR_INVALID, "stage %d >= %d", stage, MOE_NUM_STAGES);
  if (stage < 0) {
    g_profile = ProfileHook{};
    return MOE_OK;
  }
  if (!start_events || !stop_events || n_events <= 0)
    return fail(MOE_ERR_INVALID, "profile events missing");
  g_profile = ProfileHook{stage, start_events, stop_events, n_events, 0};
  return MOE_OK;
}

MOE_API const char *moe_last_error(void) { return g_last_error.c_str(); }

MOE_API const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

MOE_API int moe_validate(const moe_config *cfg) {
  if (!cfg) return fail(MOE_ERR_INVALID, "config is NULL");
  const moe_config &c = *cfg;
  if (c.T < 0) return fail(MOE_ERR_INVALID, "T = %d < 0", c.T);
  if (c.H <= 0 || c.E <= 0 || c.I <= 0 || c.K <= 0)
    return fail(MOE_ERR_INVALID, "H, E, I, K must be positive (got %d, %d, %d, %d)", c.H, c.E, c.I, c.K);
  if (c.K > c.E) return fail(MOE_ERR_INVALID, "K = %d > E = %d", c.K, c.E);
  if (c.act_dtype != MOE_DTYPE_F32 && c.act_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID, "act_dtype %d is not f32 or bf16", c.act_dtype);
  if (c.w_dtype != MOE_DTYPE_F32 && c.w_dtype != MOE_DTYPE_BF16 && c.w_dtype != MOE_DTYPE_MXFP4)
    return fail(MOE_ERR_INVALID, "w_dtype %d is unknown", c.w_dtype);
  if (c.score_fn < MOE_SCORE_SOFTMAX || c.score_fn > MOE_SCORE_SQRTSOFTPLUS)
    return fail(MOE_ERR_INVALID, "score_fn %d is unknown", c.score_fn);
  if (c.n_group < 1) return fail(MOE_ERR_INVALID, "n_group = %d < 1", c.n_group);
  if (c.E % c.n_group) return fail(MOE_ERR_INVALID, "E = %d is not a multiple of n_group = %d", c.E, c.n_group);
  if (c.topk_group < 1 || c.topk_group > c.n_group)
    return fail(MOE_ERR_INVALID, "topk_group = %d outside [1, n_group = %d]", c.topk_group, c.n_group);
  if (c.n_group > 1 && c.E / c.n_group < 2)
    return fail(MOE_ERR_INVALID, "group-limited selection needs at least 2 experts per group");
  if (c.n_group > 1 && c.K > c.topk_group * (c.E / c.n_group))
    return fail(MOE_ERR_INVALID, "K = %d exceeds the %d experts of the kept groups", c.K,
                c.topk_group * (c.E / c.n_group));
  if (c.norm_topk_prob != 0 && c.norm_topk_prob != 1)
    return fail(MOE_ERR_INVALID, "norm_topk_prob must be 0 or 1");
  if (!std::isfinite(c.route_scale)) return fail(MOE_ERR_INVALID, "route_scale is not finite");
  if (std::isnan(c.swiglu_limit) || c.swiglu_limit < 0)
    return fail(MOE_ERR_INVALID, "swiglu_limit must be >= 0 or +inf");
  if (c.shared_I < 0) return fail(MOE_ERR_INVALID, "shared_I = %d < 0", c.shared_I);
  if (c.shared_gated != 0 && c.shared_gated != 1) return fail(MOE_ERR_INVALID, "shared_gated must be 0 or 1");
  if (c.activation != MOE_ACT_SWIGLU && c.activation != MOE_ACT_SWIGLU_OAI)
    return fail(MOE_ERR_INVALID, "activation %d is unknown", c.activation);
  if (c.mx_gemm != MOE_MX_DECODE && c.mx_gemm != MOE_MX_BLOCK_SCALED)
    return fail(MOE_ERR_INVALID, "mx_gemm %d is unknown", c.mx_gemm);

  if (c.E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E = %d > %d", c.E, MOE_MAX_EXPERTS);
  if (c.K > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "K = %d > %d", c.K, MOE_MAX_TOPK);
  if (c.n_group > MOE_MAX_GROUPS)
    return fail(MOE_ERR_UNSUPPORTED, "n_group = %d > %d", c.n_group, MOE_MAX_GROUPS);
  if (c.H % 32 || c.I % 32 || c.shared_I % 32)
    return fail(MOE_ERR_UNSUPPORTED, "H, I and shared_I must be multiples of 32 (got %d, %d, %d)", c.H,
                c.I, c.shared_I);
  const bool pair_ok = (c.act_dtype == MOE_DTYPE_F32 && c.w_dtype == MOE_DTYPE_F32) ||
                       (c.act_dtype == MOE_DTYPE_BF16 && c.w_dtype == MOE_DTYPE_BF16) ||
                       (c.act_dtype == MOE_DTYPE_BF16 && c.w_dtype == MOE_DTYPE_MXFP4);
  if (!pair_ok)
    return fail(MOE_ERR_UNSUPPORTED, "activation/weight formats %d/%d are not implemented", c.act_dtype,
                c.w_dtype);
  const double slots = (double)c.T * c.K;
  if (slots * c.H * 4 > 1.0e12 || (double)c.T * c.E > 2.0e9)
    return fail(MOE_ERR_UNSUPPORTED, "T = %d is too large for 32-bit row indexing", c.T);
  return ok();
}

MOE_API int moe_workspace_bytes(const moe_config *cfg, size_t *bytes) {
  const int v = moe_validate(cfg);
  if (v != MOE_OK) return v;
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
  *bytes = make_layout(*cfg).total;
  return MOE_OK;
}

MOE_API int moe_route(const moe_config *cfg, const void *x, const void *gate_w,
                      const float *router_bias, const float *expert_bias, float *scores,
                      int32_t *indices, float *weights, int32_t *counts, void *workspace,
                      size_t workspace_bytes, void *stream) {
  const int v = moe_validate(cfg);
  if (v != MOE_OK) return v;
  const moe_config &c = *cfg;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  OPTIONAL_PTR(counts, "counts");
  if (c.T == 0) {
    if (counts) HIP_TRY(launch_fill_i32(counts, 0, c.E, st), "fill launch");
    return MOE_OK;
  }
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(gate_w, "gate_w");
  REQUIRE_PTR(scores, "scores");
  REQUIRE_PTR(indices, "indices");
  REQUIRE_PTR(weights, "weights");
  OPTIONAL_PTR(router_bias, "router_bias");
  OPTIONAL_PTR(expert_bias, "expert_bias");
  const int w = check_workspace(c, workspace, workspace_bytes);
  if (w != MOE_OK) return w;
  moe_config rc = c;
  rc.shared_gated = 0;  // the router call has no shared-expert gate column
  const Layout L = make_layout(c);
  return enqueue_route(rc, x, gate_w, nullptr, router_bias, expert_bias,
                       RouteBuffers{scores, indices, weights}, counts,
                       static_cast<char *>(workspace), L, false, st);
}

}  // extern "C"

namespace {

// The layer forward of moe_ffn_forward after validation of cfg, on the given
// workspace (checked here against the layout's size and alignment).
int forward_impl(const moe_config &c, const void *x, const moe_weights *wt, void *out, float *scores,
                 int32_t *indices, float *weights, int32_t *counts, void *workspace, size_t workspace_bytes,
                 hipStream_t st) {
  OPTIONAL_PTR(counts, "counts");
  if (c.T == 0) {
    if (counts) HIP_TRY(launch_fill_i32(counts, 0, c.E, st), "fill launch");
    return MOE_OK;
  }
  if (!wt) return fail(MOE_ERR_INVALID, "weights struct is NULL");
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(out, "out");
  REQUIRE_PTR(wt->gate_w, "gate_w");
  REQUIRE_PTR(wt->w_gate_up, "w_gate_up");
  REQUIRE_PTR(wt->w_down, "w_down");
  OPTIONAL_PTR(wt->router_bias, "router_bias");
  OPTIONAL_PTR(wt->expert_bias, "expert_bias");
  OPTIONAL_PTR(wt->b_gate_up, "b_gate_up");
  OPTIONAL_PTR(wt->b_down, "b_down");
  OPTIONAL_PTR(scores, "scores");
  OPTIONAL_PTR(indices, "indices");
  OPTIONAL_PTR(weights, "weights");
  if (c.w_dtype == MOE_DTYPE_MXFP4) {
    if (!wt->w_gate_up_scale || !wt->w_down_scale)
      return fail(MOE_ERR_INVALID, "MXFP4 experts need w_gate_up_scale and w_down_scale");
  }
  if (has_shared(c)) {
    REQUIRE_PTR(wt->sh_gate_up, "sh_gate_up");
    REQUIRE_PTR(wt->sh_down, "sh_down");
    if (c.shared_gated) REQUIRE_PTR(wt->sh_gate, "sh_gate");
  }
  const size_t io_bytes = (size_t)c.T * c.H * act_bytes(c);
  if (overlaps(x, io_bytes, out, io_bytes))
    return fail(MOE_ERR_INVALID, "out overlaps x (the shared expert reads the unmodified input)");
  const int w = check_workspace(c, workspace, workspace_bytes);
  if (w != MOE_OK) return w;

  char *ws = static_cast<char *>(workspace);
  const Layout L = make_layout(c);
  RouteBuffers rb{scores ? scores : reinterpret_cast<float *>(ws + L.scores),
                  indices ? indices : reinterpret_cast<int32_t *>(ws + L.indices),
                  weights ? weights : reinterpret_cast<float *>(ws + L.weights)};
  int r = enqueue_route(c, x, wt->gate_w, wt->sh_gate, wt->router_bias, wt->expert_bias, rb, counts, ws,
                        L, true, st);
  if (r != MOE_OK) return r;

  const WFormat wf = c.w_dtype == MOE_DTYPE_F32 ? W_F32 : (c.w_dtype == MOE_DTYPE_BF16 ? W_BF16 : W_MXFP4);
  const WFormat af = c.act_dtype == MOE_DTYPE_F32 ? W_F32 : W_BF16;
  const GemmPlan plan = gemm_plan(c);
  const int32_t *counts_ws = reinterpret_cast<int32_t *>(ws + L.counts);
  const int32_t *offsets_ws = reinterpret_cast<int32_t *>(ws + L.offsets);
  const int32_t *active_all_ws = reinterpret_cast<int32_t *>(ws + L.active_all);
  const int32_t *n_active_all_ws = reinterpret_cast<int32_t *>(ws + L.n_active_all);
  const int32_t *mtile_prefix_ws = reinterpret_cast<int32_t *>(ws + L.mtile_prefix);
  const int32_t *mtile_prefix2_ws = reinterpret_cast<int32_t *>(ws + L.mtile_prefix2);
  const int4 *chunks_ws = reinterpret_cast<const int4 *>(ws + L.chunks);
  const int32_t *n_chunks_ws = reinterpret_cast<int32_t *>(ws + L.n_chunks);
  const int32_t *perm_ws = reinterpret_cast<int32_t *>(ws + L.perm);
  const long slots = (long)c.T * c.K;
  const int max_groups = (int)std::min<long>(c.E, slots);
  const long max_chunks = std::min(slots, slots / plan.chunk_rows + max_groups);
  const size_t H = c.H, I = c.I, Is = c.shared_I;
  const bool hilo = c.act_dtype == MOE_DTYPE_BF16;
  char *h_lo = ws + L.h + (size_t)c.T * c.K * c.I * 2;
  char *sh_h_lo = ws + L.sh_h + (size_t)c.T * c.shared_I * 2;
  // shared expert: one group of T rows, cut into chunks on the fly (narrow
  // chunks at small T, so that enough work items stream its weights)
  const int sh_chunk_rows = c.T <= 128 ? 16 : 32;
  const long sh_chunks = ((long)c.T + sh_chunk_rows - 1) / sh_chunk_rows;
  // the tiled and big-tile launches' tile counters start at zero (one fill
  // for all of them)
  int32_t *queue = reinterpret_cast<int32_t *>(ws + L.tile_queue);
  auto tile_queue = [&](int launch) { return queue + launch * kTiledQueueInts; };
  if (plan.tiled || plan.tiled_shared)
    HIP_TRY(launch_fill_i32(queue, 0, kQueuedLaunches * kTiledQueueInts, st), "fill launch");
  // where routed and shared experts both run on the streaming kernels with
  // bf16 operands, the shared expert's gate_up items ride in the routed
  // gate_up launch.  Measured at T=72 (DeepSeek-V4-style / qwen3_5_moe
  // layers): gate_up 924 -> 914 and 615 -> 608 us against two launches.  Its
  // down items are not carried: each holds 16 rows of h (hi and lo) where a
  // routed item holds two or three, and carried they cost more than their own
  // launch (down 465 -> 471 and 327 -> 358 us).
  const bool fold = has_shared(c) && !plan.tiled && !plan.tiled_shared && wf == W_BF16 && af == W_BF16;

  // routed gate_up + SwiGLU over x rows gathered by slot
  ExpertGemmArgs g1{};
  g1.A = x;
  g1.perm = perm_ws;
  g1.topk = c.K;
  g1.chunks = chunks_ws;
  g1.n_chunks = n_chunks_ws;
  g1.chunk_rows = plan.chunk_rows;
  g1.counts = counts_ws;
  g1.offsets = offsets_ws;
  g1.active = active_all_ws;
  g1.n_active = n_active_all_ws;
  g1.W = wt->w_gate_up;
  g1.Wscale = wt->w_gate_up_scale;
  g1.w_stride = wf == W_MXFP4 ? 2 * I * H / 2 : 2 * I * H;
  g1.s_stride = 2 * I * H / 32;
  g1.Kdim = c.H;
  g1.N = c.I;
  g1.n_tiles = c.I / 16;
  g1.bias = wt->b_gate_up;
  g1.bias_stride = 2 * I;
  g1.out = ws + L.h;
  if (hilo) g1.out_lo = h_lo;
  g1.limit = c.swiglu_limit;
  g1.act = c.activation;
  if (fold) {
    g1.rows2 = c.T;
    g1.A2 = x;
    g1.W2 = wt->sh_gate_up;
    g1.Kdim2 = c.H;
    g1.N2 = c.shared_I;
    g1.out2 = ws + L.sh_h;
    if (hilo) g1.out2_lo = sh_h_lo;
  }
  HIP_TRY(profile_mark(MOE_STAGE_GATE_UP, true, st), "profile event");
  if (wf == W_F32) {
    HIP_TRY(launch_gate_up_f32(g1, max_groups, st), "routed gate_up launch");
  } else if (plan.tiled) {
    TiledGemmArgs t1{g1, active_all_ws, n_active_all_ws, mtile_prefix_ws};
    if (plan.mx_scaled && bigtile_mx_scaled_applies(t1)) {
      const MxActs xa{reinterpret_cast<uint8_t *>(ws + L.mxq), reinterpret_cast<uint16_t *>(ws + L.mxs)};
      HIP_TRY(launch_mxfp8_split(static_cast<const uint16_t *>(x), c.T, c.H, xa, st), "activation split launch");
      HIP_TRY(launch_bigtile_mx_scaled(t1, xa, slots, max_groups, st), "routed gate_up launch");
    } else if (plan.big) {
      HIP_TRY(launch_bigtile(t1, true, wf, slots, max_groups, tile_queue(4), st), "routed gate_up launch");
    }
    else HIP_TRY(launch_tiled(t1, true, wf, slots, max_groups, tile_queue(0), st), "routed gate_up launch");
  } else {
    HIP_TRY(launch_stream(g1, true, wf, max_chunks, st), "routed gate_up launch");
  }
  HIP_TRY(profile_mark(MOE_STAGE_GATE_UP, false, st), "profile event");

  if (has_shared(c)) {
    ExpertGemmArgs s1{};
    s1.A = x;
    s1.single_rows = c.T;
    s1.chunk_rows = sh_chunk_rows;
    s1.W = wt->sh_gate_up;
    s1.Kdim = c.H;
    s1.N = c.shared_I;
    s1.n_tiles = c.shared_I / 16;
    s1.out = ws + L.sh_h;
    if (hilo) s1.out_lo = sh_h_lo;
    s1.limit = c.swiglu_limit;
    s1.act = c.activation;
    HIP_TRY(profile_mark(MOE_STAGE_SHARED_GATE_UP, true, st), "profile event");
    if (fold) {
      // ran in the routed launch
    } else if (af == W_F32) {
      HIP_TRY(launch_gate_up_f32(s1, 1, st), "shared gate_up launch");
    } else if (plan.tiled_shared) {
      TiledGemmArgs ts{s1, nullptr, nullptr, nullptr};
      if (plan.big_shared) HIP_TRY(launch_bigtile(ts, true, af, c.T, 1, tile_queue(5), st), "shared gate_up launch");
      else HIP_TRY(launch_tiled(ts, true, af, c.T, 1, tile_queue(1), st), "shared gate_up launch");
    } else {
      HIP_TRY(launch_stream(s1, true, af, sh_chunks, st), "shared gate_up launch");
    }
    HIP_TRY(profile_mark(MOE_STAGE_SHARED_GATE_UP, false, st), "profile event");
  }

  // routed down
  ExpertGemmArgs g2{};
  g2.A = ws + L.h;
  if (hilo) g2.A_lo = h_lo;
  g2.chunks = chunks_ws;
  g2.n_chunks = n_chunks_ws;
  g2.chunk_rows = plan.chunk_rows;
  g2.counts = counts_ws;
  g2.offsets = offsets_ws;
  g2.active = active_all_ws;
  g2.n_active = n_active_all_ws;
  g2.W = wt->w_down;
  g2.Wscale = wt->w_down_scale;
  g2.w_stride = wf == W_MXFP4 ? H * I / 2 : H * I;
  g2.s_stride = H * I / 32;
  g2.Kdim = c.I;
  g2.N = c.H;
  g2.n_tiles = c.H / 32;
  g2.bias = wt->b_down;
  g2.bias_stride = H;
  g2.out = ws + L.y;
  // one expert per token and no shared expert: the down epilogue writes the
  // weighted output row itself and no combine pass is needed
  const bool direct = c.K == 1 && !has_shared(c) && wf != W_F32;
  if (direct) {
    g2.direct_out = out;
    g2.perm = perm_ws;
    g2.weights = rb.weights;
  }

  HIP_TRY(profile_mark(MOE_STAGE_DOWN, true, st), "profile event");
  if (wf == W_F32) {
    HIP_TRY(launch_down_f32(g2, max_groups, st), "routed down launch");
  } else if (plan.tiled) {
    TiledGemmArgs t2{g2, active_all_ws, n_active_all_ws, plan.big ? mtile_prefix2_ws : mtile_prefix_ws};
    HIP_TRY(launch_tiled(t2, false, wf, slots, max_groups, tile_queue(2), st), "routed down launch");
  } else {
    HIP_TRY(launch_stream(g2, false, wf, max_chunks, st), "routed down launch");
  }
  HIP_TRY(profile_mark(MOE_STAGE_DOWN, false, st), "profile event");

  if (has_shared(c)) {
    ExpertGemmArgs s2{};
    s2.A = ws + L.sh_h;
    if (hilo) s2.A_lo = sh_h_lo;
    s2.single_rows = c.T;
    s2.chunk_rows = sh_chunk_rows;
    s2.W = wt->sh_down;
    s2.Kdim = c.shared_I;
    s2.N = c.H;
    s2.n_tiles = c.H / 32;
    s2.out = ws + L.sh_y;
    HIP_TRY(profile_mark(MOE_STAGE_SHARED_DOWN, true, st), "profile event");
    if (af == W_F32) {
      HIP_TRY(launch_down_f32(s2, 1, st), "shared down launch");
    } else if (plan.tiled_shared) {
      TiledGemmArgs ts{s2, nullptr, nullptr, nullptr};
      HIP_TRY(launch_tiled(ts, false, af, c.T, 1, tile_queue(3), st), "shared down launch");
    } else {
      HIP_TRY(launch_stream(s2, false, af, sh_chunks, st), "shared down launch");
    }
    HIP_TRY(profile_mark(MOE_STAGE_SHARED_DOWN, false, st), "profile event");
  }

  if (direct) {
    ++g_profile.calls;
    return MOE_OK;
  }

  CombineArgs ca{};
  ca.y = reinterpret_cast<const float *>(ws + L.y);
  ca.inv = reinterpret_cast<const int32_t *>(ws + L.inv);
  ca.weights = rb.weights;
  ca.ysh = has_shared(c) ? reinterpret_cast<const float *>(ws + L.sh_y) : nullptr;
  ca.gamma = has_shared_gate(c) ? reinterpret_cast<const float *>(ws + L.gamma) : nullptr;
  ca.out = out;
  ca.T = c.T;
  ca.H = c.H;
  ca.K = c.K;
  HIP_TRY(profile_mark(MOE_STAGE_COMBINE, true, st), "profile event");
  HIP_TRY(launch_combine(ca, c.act_dtype == MOE_DTYPE_BF16, st), "combine launch");
  HIP_TRY(profile_mark(MOE_STAGE_COMBINE, false, st), "profile event");
  ++g_profile.calls;
  return MOE_OK;
}

}  // namespace

extern "C" {

MOE_API int moe_ffn_forward(const moe_config *cfg, const void *x, const moe_weights *wt, void *out,
                            float *scores, int32_t *indices, float *weights, int32_t *counts,
                            void *workspace, size_t workspace_bytes, void *stream) {
  const int v = moe_validate(cfg);
  if (v != MOE_OK) return v;
  return forward_impl(*cfg, x, wt, out, scores, indices, weights, counts, workspace, workspace_bytes,
                      reinterpret_cast<hipStream_t>(stream));
}

MOE_API int moe_backward_workspace_bytes(const moe_config *cfg, size_t *bytes) {
  const int v = moe_validate(cfg);
  if (v != MOE_OK) return v;
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
  const moe_config &c = *cfg;
  *bytes = backward_layout(c.T, c.K, c.E, c.H, c.I, c.shared_I, nullptr, nullptr);
  return ok();
}

MOE_API int moe_ffn_backward(const moe_config *cfg, const void *x, const moe_weights *wt, const void *dout,
                             const float *scores, const int32_t *indices, const moe_grads *g, void *workspace,
                             size_t workspace_bytes, void *stream) {
  const int v = moe_validate(cfg);
  if (v != MOE_OK) return v;
  const moe_config &c = *cfg;
  if (c.w_dtype == MOE_DTYPE_MXFP4) return fail(MOE_ERR_UNSUPPORTED, "the backward takes f32 or bf16 experts");
  if (!wt) return fail(MOE_ERR_INVALID, "weights is NULL");
  if (!g) return fail(MOE_ERR_INVALID, "grads is NULL");
  REQUIRE_PTR(g->dgate, "dgate");
  REQUIRE_PTR(g->dw_gate_up, "dw_gate_up");
  REQUIRE_PTR(g->dw_down, "dw_down");
  if (!wt->router_bias != !g->drouter_bias)
    return fail(MOE_ERR_INVALID, "drouter_bias is required exactly when router_bias is given");
  if (!wt->b_gate_up != !g->db_gate_up)
    return fail(MOE_ERR_INVALID, "db_gate_up is required exactly when b_gate_up is given");
  if (!wt->b_down != !g->db_down) return fail(MOE_ERR_INVALID, "db_down is required exactly when b_down is given");
  OPTIONAL_PTR(g->drouter_bias, "drouter_bias");
  OPTIONAL_PTR(g->db_gate_up, "db_gate_up");
  OPTIONAL_PTR(g->db_down, "db_down");
  if (has_shared(c)) {
    REQUIRE_PTR(wt->sh_gate_up, "sh_gate_up");
    REQUIRE_PTR(wt->sh_down, "sh_down");
    REQUIRE_PTR(g->dsh_gate_up, "dsh_gate_up");
    REQUIRE_PTR(g->dsh_down, "dsh_down");
    if (c.shared_gated) {
      REQUIRE_PTR(wt->sh_gate, "sh_gate");
      REQUIRE_PTR(g->dsh_gate, "dsh_gate");
    }
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t E = c.E, H = c.H, I = c.I, Is = c.shared_I;
  if (c.T == 0) {  // no tokens: every gradient is zero
    auto zero = [&](float *p, size_t n) { return p ? launch_fill_i32(reinterpret_cast<int32_t *>(p), 0, n, st) : hipSuccess; };
    HIP_TRY(zero(g->dgate, E * H), "fill launch");
    HIP_TRY(zero(g->dw_gate_up, E * 2 * I * H), "fill launch");
    HIP_TRY(zero(g->dw_down, E * H * I), "fill launch");
    HIP_TRY(zero(g->drouter_bias, E), "fill launch");
    HIP_TRY(zero(g->db_gate_up, E * 2 * I), "fill launch");
    HIP_TRY(zero(g->db_down, E * H), "fill launch");
    if (has_shared(c)) {
      HIP_TRY(zero(g->dsh_gate_up, 2 * Is * H), "fill launch");
      HIP_TRY(zero(g->dsh_down, H * Is), "fill launch");
      HIP_TRY(zero(c.shared_gated ? g->dsh_gate : nullptr, H), "fill launch");
    }
    return ok();
  }
  REQUIRE_PTR(g->dx, "dx");  // [T, H]: only with tokens
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(dout, "dout");
  REQUIRE_PTR(scores, "scores");
  REQUIRE_PTR(indices, "indices");
  REQUIRE_PTR(wt->gate_w, "gate_w");
  REQUIRE_PTR(wt->w_gate_up, "w_gate_up");
  REQUIRE_PTR(wt->w_down, "w_down");
  OPTIONAL_PTR(wt->b_gate_up, "b_gate_up");
  OPTIONAL_PTR(wt->b_down, "b_down");
  const size_t need = backward_layout(c.T, c.K, c.E, c.H, c.I, c.shared_I, nullptr, nullptr);
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  BackwardArgs a{};
  a.T = c.T; a.K = c.K; a.E = c.E; a.H = c.H; a.I = c.I; a.Is = c.shared_I;
  a.act_bf16 = c.act_dtype == MOE_DTYPE_BF16;
  a.w_bf16 = c.w_dtype == MOE_DTYPE_BF16;
  a.norm = c.norm_topk_prob;
  a.score_fn = c.score_fn;
  a.limit = c.swiglu_limit;
  a.act = c.activation;
  a.route_scale = c.route_scale;
  a.x = x; a.dout = dout; a.gate_w = wt->gate_w; a.w_gate_up = wt->w_gate_up; a.w_down = wt->w_down;
  a.b_gate_up = wt->b_gate_up; a.b_down = wt->b_down;
  if (has_shared(c)) {
    a.sh_gate_up = wt->sh_gate_up;
    a.sh_down = wt->sh_down;
    a.sh_gate = c.shared_gated ? wt->sh_gate : nullptr;
  }
  a.scores = scores;
  a.indices = indices;
  a.g = GradPtrs{g->dx, g->dgate, g->drouter_bias, g->dw_gate_up, g->dw_down, g->db_gate_up, g->db_down,
                 g->dsh_gate_up, g->dsh_down, g->dsh_gate};
  backward_layout(c.T, c.K, c.E, c.H, c.I, c.shared_I, &a, static_cast<char *>(workspace));
  HIP_TRY(launch_backward(a, st), "backward launch");
  return ok();
}

MOE_API int moe_balance_count(const int32_t *indices, const uint8_t *token_mask, int32_t T, int32_t K,
                              int32_t E, int64_t *tokens_per_expert, void *stream) {
  if (T < 0) return fail(MOE_ERR_INVALID, "T = %d < 0", T);
  if (K <= 0 || E <= 0) return fail(MOE_ERR_INVALID, "K = %d and E = %d must be positive", K, E);
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E = %d > %d", E, MOE_MAX_EXPERTS);
  if ((double)T * K > 2.0e9) return fail(MOE_ERR_UNSUPPORTED, "T * K = %.0f slots is too many", (double)T * K);
  if (!tokens_per_expert) return fail(MOE_ERR_INVALID, "tokens_per_expert is NULL");
  if (reinterpret_cast<uintptr_t>(tokens_per_expert) & 7)
    return fail(MOE_ERR_INVALID, "tokens_per_expert is not 8-byte aligned");
  if (T == 0) return MOE_OK;
  if (!indices) return fail(MOE_ERR_INVALID, "indices is NULL");
  if (reinterpret_cast<uintptr_t>(indices) & 3) return fail(MOE_ERR_INVALID, "indices is not 4-byte aligned");
  BalanceCountArgs a{indices, token_mask, tokens_per_expert, T, K, E};
  HIP_TRY(launch_balance_count(a, reinterpret_cast<hipStream_t>(stream)), "balance count launch");
  return MOE_OK;
}

MOE_API int moe_balance_update(int64_t *tokens_per_expert, float *expert_bias, int32_t E,
                               float bias_update_rate, float *step_balance, void *stream) {
  if (E <= 0) return fail(MOE_ERR_INVALID, "E = %d must be positive", E);
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E = %d > %d", E, MOE_MAX_EXPERTS);
  if (!std::isfinite(bias_update_rate)) return fail(MOE_ERR_INVALID, "bias_update_rate is not finite");
  if (!tokens_per_expert) return fail(MOE_ERR_INVALID, "tokens_per_expert is NULL");
  if (reinterpret_cast<uintptr_t>(tokens_per_expert) & 7)
    return fail(MOE_ERR_INVALID, "tokens_per_expert is not 8-byte aligned");
  if (bias_update_rate != 0.f && !expert_bias)
    return fail(MOE_ERR_INVALID, "expert_bias is NULL with a non-zero bias_update_rate");
  if (expert_bias && (reinterpret_cast<uintptr_t>(expert_bias) & 3))
    return fail(MOE_ERR_INVALID, "expert_bias is not 4-byte aligned");
  if (step_balance && (reinterpret_cast<uintptr_t>(step_balance) & 3))
    return fail(MOE_ERR_INVALID, "step_balance is not 4-byte aligned");
  BalanceUpdateArgs a{tokens_per_expert, expert_bias, step_balance, bias_update_rate, E};
  HIP_TRY(launch_balance_update(a, reinterpret_cast<hipStream_t>(stream)), "balance update launch");
  return MOE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Forward without allocation: moe_ffn_forward on a scratch array that the
// library holds in device memory, one per GPU, for callers that cannot
// allocate a workspace.
// ---------------------------------------------------------------------------

// In host code `scratch` names a host-side stand-in, not device memory: host
// code uses only the device address that hipGetSymbolAddress returns for it
// (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
int scratch_ptr(void **out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255) != 0)
      return fail(MOE_ERR_HIP, "scratch array has no 256-byte aligned device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

MOE_API int moe_ffn_forward_noalloc(const moe_config *cfg, const void *x, const moe_weights *wt, void *out,
                                    float *scores, int32_t *indices, float *weights, int32_t *counts,
                                    void *stream) {
  const int v = moe_validate(cfg);
  if (v != MOE_OK) return v;
  const size_t need = make_layout(*cfg).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this configuration needs %zu bytes of scratch; the no-allocation forward holds %zu "
                "(use moe_ffn_forward with a workspace)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (cfg->T > 0) {
    const int r = scratch_ptr(&ws);
    if (r != MOE_OK) return r;
  }
  return forward_impl(*cfg, x, wt, out, scores, indices, weights, counts, ws, MOE_NOALLOC_SCRATCH_BYTES,
                      reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
