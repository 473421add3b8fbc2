// Host front end of the C ABI declared in include/gdn_beam.h: argument checks,
// the per-context state machine (init -> step(t) -> select(t) -> step(t+1) ...),
// the workspace carve-up, and the hand-off to the kernel launchers.  Every check
// runs before any launch, so a rejected call leaves the context unchanged.
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "gdn_layout.h"

using namespace gdn;

struct gdn_beam_ctx {
  gdn_beam_config cfg;
  Layout L;
  void* ws;
  size_t ws_bytes;
  int t;          // step expected next
  int stepped;    // step(t) issued, select(t) not yet
  int W_cur;      // beams alive at step t
  int mode;       // steps of this decode: 0 none yet, 1 transition records, 2 full states
  const void* states;   // state buffer of a full-state decode
};

namespace {

thread_local std::string g_last_error;

// Step-launch timing, process-wide (a decode makes a new context per init): the next
// `cap` step launches stamp their start and end on event pairs 2i, 2i + 1.
struct StepTimer {
  std::mutex m;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;
  // the pair for a launch about to be issued, or none past the capacity
  bool take(hipEvent_t& e0, hipEvent_t& e1) {
    std::lock_guard<std::mutex> g(m);
    if (n >= cap) return false;
    e0 = ev[2 * n];
    e1 = ev[2 * n + 1];
    ++n;
    return true;
  }
  // a launch that took a pair and failed gives it back (it recorded nothing)
  void give_back(bool taken) {
    if (!taken) return;
    std::lock_guard<std::mutex> g(m);
    if (n > 0) --n;
  }
} g_timer;

// Projection-phase stamps: the next step launch of the process writes them, once armed.
struct StampArm {
  std::mutex m;
  uint32_t* buf = nullptr;
  size_t records = 0;
  bool take(uint32_t*& b, size_t& n) {
    std::lock_guard<std::mutex> g(m);
    if (!buf) return false;
    b = buf;
    n = records;
    buf = nullptr;
    records = 0;
    return true;
  }
} g_stamp;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gdn_status hip_fail(int err, const char* where) {
  g_last_error = std::string(where) + ": " + hip_error_string(err);
  return GDN_ERR_HIP;
}

bool dims_supported(int d_k, int d_v) {
  return (d_k == 16 && d_v == 16) || (d_k == 128 && d_v == 128) || (d_k == 128 && d_v == 256) ||
         (d_k == 128 && d_v == 512) || (d_k == 256 && d_v == 256) || (d_k == 256 && d_v == 512);
}

gdn_status check_config(const gdn_beam_config* c) {
  if (!c) return GDN_ERR_INVALID_ARG;
  if (c->R < 1 || c->H < 1 || c->T_max < 1 || c->W_max < 1 || c->V_max < 1)
    return GDN_ERR_INVALID_ARG;
  if ((c->io_dtype != GDN_F32 && c->io_dtype != GDN_BF16) ||
      (c->wout_dtype != GDN_F32 && c->wout_dtype != GDN_BF16))
    return GDN_ERR_INVALID_ARG;
  if (c->H_K < 0 || (c->H_K > 0 && c->H % c->H_K != 0)) return GDN_ERR_INVALID_ARG;
  if (!dims_supported(c->d_k, c->d_v)) return GDN_ERR_UNSUPPORTED;
  // d_k = 256 with fp32 q, k, v would stage 200 KB per workgroup: bf16 io only
  if (c->d_k == 256 && c->io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  // an fp32 codebook keeps z in registers as fp32: d_v <= 256 with it
  if (c->d_v > 256 && c->wout_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (c->T_max > kMaxT || c->W_max > kMaxW || c->V_max > kMaxV) return GDN_ERR_CAPACITY;
  // flat candidate index b*V + c and per-request scratch sizes must fit in 31 bits
  if (int64_t(c->W_max) * c->V_max >= (int64_t(1) << 31)) return GDN_ERR_CAPACITY;
  if (int64_t(c->R) * c->H * c->T_max * c->W_max >= (int64_t(1) << 31)) return GDN_ERR_CAPACITY;
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_beam_status_str(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_BAD_STATE: return "call out of order";
    case GDN_ERR_CAPACITY: return "capacity exceeded";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_UNSUPPORTED: return "unsupported head dims or dtype";
    case GDN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* gdn_beam_last_error(void) { return g_last_error.c_str(); }

gdn_status gdn_beam_workspace_bytes(const gdn_beam_config* cfg, size_t* bytes) {
  gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!bytes) return GDN_ERR_INVALID_ARG;
  *bytes = make_layout(*cfg).total;
  return GDN_OK;
}

gdn_status gdn_beam_init(const gdn_beam_config* cfg, const float* S_ctx, int32_t W0,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         gdn_beam_ctx** out) {
  gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  if (!S_ctx || !workspace || !out) return GDN_ERR_INVALID_ARG;
  if (!aligned16(S_ctx) || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return GDN_ERR_INVALID_ARG;
  if (W0 < 1) return GDN_ERR_INVALID_ARG;
  if (W0 > cfg->W_max) return GDN_ERR_CAPACITY;
  Layout L = make_layout(*cfg);
  if (workspace_bytes < L.total) return GDN_ERR_WORKSPACE;

  gdn_beam_ctx* ctx = new (std::nothrow) gdn_beam_ctx;
  if (!ctx) return GDN_ERR_INVALID_ARG;
  ctx->cfg = *cfg;
  ctx->L = L;
  ctx->ws = workspace;
  ctx->ws_bytes = workspace_bytes;
  ctx->t = 0;
  ctx->stepped = 0;
  ctx->W_cur = W0;
  ctx->mode = 0;
  ctx->states = nullptr;

  InitArgs a{cfg->R, cfg->H, cfg->d_k, cfg->d_v, cfg->W_max, cfg->T_max, cfg->io_dtype,
             S_ctx, workspace, L};
  int err = launch_init(a, stream);
  if (err) {
    delete ctx;
    return hip_fail(err, "gdn_beam_init");
  }
  *out = ctx;
  return GDN_OK;
}

gdn_status gdn_beam_step(gdn_beam_ctx* ctx, int32_t t, const void* q, const void* k,
                         const void* v, const float* alpha, const float* beta, float* o,
                         hipStream_t stream) {
  if (!ctx) return GDN_ERR_INVALID_ARG;
  if (!q || !k || !v || !alpha || !beta || !o) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(alpha) ||
      !aligned16(beta) || !aligned16(o))
    return GDN_ERR_INVALID_ARG;
  const gdn_beam_config& c = ctx->cfg;
  if (t < 0) return GDN_ERR_INVALID_ARG;
  if (t >= c.T_max) return GDN_ERR_CAPACITY;
  if (t != ctx->t || ctx->mode == 2) return GDN_ERR_BAD_STATE;
  StepArgs a{c.R, c.H, key_heads(c), c.d_k, c.d_v, c.W_max, c.T_max, t, ctx->W_cur, c.io_dtype,
             q, k, v, alpha, beta, o, ctx->ws, ctx->L, nullptr, nullptr, nullptr, 0};
  g_stamp.take(a.stamps, a.stamp_records);
  const bool timed = g_timer.take(a.ev0, a.ev1);
  int err = launch_step(a, stream);
  if (err) {
    g_timer.give_back(timed);
    return hip_fail(err, "gdn_beam_step");
  }
  ctx->stepped = 1;
  ctx->mode = 1;
  return GDN_OK;
}

gdn_status gdn_fullstate_bytes(const gdn_beam_config* cfg, size_t* bytes) {
  if (!bytes) return GDN_ERR_INVALID_ARG;
  const gdn_status st = check_config(cfg);
  if (st != GDN_OK) return st;
  *bytes = 2 * fullstate_half_bytes(*cfg);
  return GDN_OK;
}

gdn_status gdn_fullstate_step(gdn_beam_ctx* ctx, int32_t t, const float* S_ctx, const void* q,
                              const void* k, const void* v, const float* alpha,
                              const float* beta, float* o, void* states, size_t states_bytes,
                              hipStream_t stream) {
  if (!ctx) return GDN_ERR_INVALID_ARG;
  if (!q || !k || !v || !alpha || !beta || !o || !states) return GDN_ERR_INVALID_ARG;
  if (t == 0 && !S_ctx) return GDN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(alpha) ||
      !aligned16(beta) || !aligned16(o) || !aligned16(states) || (S_ctx && !aligned16(S_ctx)))
    return GDN_ERR_INVALID_ARG;
  const gdn_beam_config& c = ctx->cfg;
  if (t < 0) return GDN_ERR_INVALID_ARG;
  if (t >= c.T_max) return GDN_ERR_CAPACITY;
  const size_t half = fullstate_half_bytes(c);
  if (states_bytes < 2 * half) return GDN_ERR_WORKSPACE;
  if (t != ctx->t || ctx->mode == 1) return GDN_ERR_BAD_STATE;
  if (t > 0 && states != ctx->states) return GDN_ERR_BAD_STATE;   // parents live in it
  FullStepArgs a{c.R, c.H, key_heads(c), c.d_k, c.d_v, c.W_max, c.T_max, t, ctx->W_cur, c.io_dtype, S_ctx,
                 q, k, v, alpha, beta, o, states, half,
                 reinterpret_cast<const int32_t*>(static_cast<char*>(ctx->ws) + ctx->L.anc[t & 1]),
                 nullptr, nullptr};
  const bool timed = g_timer.take(a.ev0, a.ev1);
  int err = launch_fullstate(a, stream);
  if (err) {
    g_timer.give_back(timed);
    return hip_fail(err, "gdn_fullstate_step");
  }
  ctx->stepped = 1;
  ctx->mode = 2;
  ctx->states = states;
  return GDN_OK;
}

}  // extern "C"

namespace {

// The checks of a select call, in order; GDN_OK when it may launch.
gdn_status check_select(const gdn_beam_ctx* ctx, int32_t t, const float* o, const void* Wout,
                        int32_t V, int32_t W_next, const int32_t* forced_parent,
                        const int32_t* forced_token, const int32_t* parent, const int32_t* token,
                        const float* score) {
  if (!ctx) return GDN_ERR_INVALID_ARG;
  if (!o || !Wout || !parent || !token || !score) return GDN_ERR_INVALID_ARG;
  if ((forced_parent == nullptr) != (forced_token == nullptr)) return GDN_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(Wout) || !aligned16(parent) || !aligned16(token) ||
      !aligned16(score))
    return GDN_ERR_INVALID_ARG;
  if (forced_parent && (!aligned16(forced_parent) || !aligned16(forced_token)))
    return GDN_ERR_INVALID_ARG;
  const gdn_beam_config& c = ctx->cfg;
  if (t < 0 || V < 1 || W_next < 1) return GDN_ERR_INVALID_ARG;
  if (t >= c.T_max) return GDN_ERR_CAPACITY;
  if (t != ctx->t || !ctx->stepped) return GDN_ERR_BAD_STATE;
  if (V > c.V_max || W_next > c.W_max) return GDN_ERR_CAPACITY;
  if (int64_t(W_next) > int64_t(ctx->W_cur) * V) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_beam_select(gdn_beam_ctx* ctx, int32_t t, const float* o, const void* Wout,
                           int32_t V, int32_t W_next, const int32_t* forced_parent,
                           const int32_t* forced_token, int32_t* parent, int32_t* token,
                           float* score, hipStream_t stream) {
  const gdn_status st = check_select(ctx, t, o, Wout, V, W_next, forced_parent, forced_token,
                                     parent, token, score);
  if (st != GDN_OK) return st;
  const gdn_beam_config& c = ctx->cfg;
  SelectArgs a{c.R, c.H, c.d_v, c.W_max, c.V_max, c.T_max, t, ctx->W_cur, V, W_next, c.wout_dtype,
               o, Wout, forced_parent, forced_token, parent, token, score, ctx->ws, ctx->L,
               static_cast<char*>(ctx->ws), ctx->L.S};
  int err = launch_select(a, stream);
  if (err) return hip_fail(err, "gdn_beam_select");
  ctx->t = t + 1;
  ctx->stepped = 0;
  ctx->W_cur = W_next;
  return GDN_OK;
}

gdn_status gdn_beam_select_static(gdn_beam_ctx* ctx, int32_t t, const float* o, const void* Wout,
                                  int32_t V, int32_t W_next, const int32_t* forced_parent,
                                  const int32_t* forced_token, int32_t* parent, int32_t* token,
                                  float* score, hipStream_t stream) {
  if (ctx) {
    // the configuration's selection scratch, laid out from the start of the array
    const SelScratch S = make_sel_scratch(ctx->cfg, 0);
    if (S.end > kStaticScratchBytes) {
      g_last_error = "gdn_beam_select_static: the configuration needs " + std::to_string(S.end) +
                     " bytes of selection scratch; the static array holds " +
                     std::to_string(kStaticScratchBytes);
      return GDN_ERR_CAPACITY;
    }
  }
  const gdn_status st = check_select(ctx, t, o, Wout, V, W_next, forced_parent, forced_token,
                                     parent, token, score);
  if (st != GDN_OK) return st;
  char* base = nullptr;
  int err = static_scratch(&base);
  if (err) return hip_fail(err, "gdn_beam_select_static");
  const gdn_beam_config& c = ctx->cfg;
  SelectArgs a{c.R, c.H, c.d_v, c.W_max, c.V_max, c.T_max, t, ctx->W_cur, V, W_next, c.wout_dtype,
               o, Wout, forced_parent, forced_token, parent, token, score, ctx->ws, ctx->L,
               base, make_sel_scratch(c, 0)};
  err = launch_select(a, stream);
  if (err) return hip_fail(err, "gdn_beam_select_static");
  ctx->t = t + 1;
  ctx->stepped = 0;
  ctx->W_cur = W_next;
  return GDN_OK;
}

gdn_status gdn_beam_export_bytes(const gdn_beam_ctx* ctx, int32_t what, size_t* bytes) {
  if (!ctx || !bytes) return GDN_ERR_INVALID_ARG;
  const gdn_beam_config& c = ctx->cfg;
  const size_t R = c.R, H = c.H, T = c.T_max, W = c.W_max;
  switch (what) {
    case GDN_EXPORT_ANCESTRY:
    case GDN_EXPORT_TOKENS: *bytes = R * W * T * 4; break;
    case GDN_EXPORT_CUM: *bytes = R * W * 4; break;
    case GDN_EXPORT_GTR_ALPHA: *bytes = R * H * T * W * 4; break;
    case GDN_EXPORT_GTR_DELTA: *bytes = R * H * T * W * size_t(c.d_v) * 4; break;
    case GDN_EXPORT_GTR_KEY: *bytes = R * size_t(key_heads(c)) * T * W * size_t(c.d_k) * io_bytes(c.io_dtype); break;
    case GDN_EXPORT_STATUS: *bytes = 4; break;
    default: return GDN_ERR_INVALID_ARG;
  }
  return GDN_OK;
}

gdn_status gdn_beam_export(const gdn_beam_ctx* ctx, int32_t what, void* dst, size_t dst_bytes,
                           hipStream_t stream) {
  size_t n = 0;
  gdn_status st = gdn_beam_export_bytes(ctx, what, &n);
  if (st != GDN_OK) return st;
  if (!dst || !aligned16(dst)) return GDN_ERR_INVALID_ARG;
  if (dst_bytes < n) return GDN_ERR_CAPACITY;
  const Layout& L = ctx->L;
  size_t off = 0;
  const int par = ctx->t & 1;   // buffers of the coming step
  switch (what) {
    case GDN_EXPORT_ANCESTRY: off = L.anc[par]; break;
    case GDN_EXPORT_TOKENS: off = L.tok[par]; break;
    case GDN_EXPORT_CUM: off = L.cum[par]; break;
    case GDN_EXPORT_GTR_ALPHA: off = L.gtr_alpha; break;
    case GDN_EXPORT_GTR_DELTA: off = L.gtr_delta; break;
    case GDN_EXPORT_GTR_KEY: off = L.gtr_key; break;
    case GDN_EXPORT_STATUS: off = L.status; break;
  }
  int err = copy_d2d(dst, static_cast<const char*>(ctx->ws) + off, n, stream);
  if (err) return hip_fail(err, "gdn_beam_export");
  return GDN_OK;
}

gdn_status gdn_beam_query(const gdn_beam_ctx* ctx, int32_t* t_next, int32_t* W_cur) {
  if (!ctx || !t_next || !W_cur) return GDN_ERR_INVALID_ARG;
  *t_next = ctx->t;
  *W_cur = ctx->W_cur;
  return GDN_OK;
}

void gdn_beam_destroy(gdn_beam_ctx* ctx) { delete ctx; }

gdn_status gdn_beam_time_steps(int32_t capacity) {
  if (capacity < 0 || capacity > 65536) return GDN_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_timer.m);
  for (hipEvent_t e : g_timer.ev) (void)hipEventDestroy(e);
  g_timer.ev.clear();
  g_timer.cap = g_timer.n = 0;
  std::vector<hipEvent_t> ev(2 * size_t(capacity), nullptr);
  for (size_t i = 0; i < ev.size(); ++i) {
    const hipError_t e = hipEventCreate(&ev[i]);
    if (e != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      return hip_fail(int(e), "gdn_beam_time_steps");
    }
  }
  g_timer.ev.swap(ev);
  g_timer.cap = capacity;
  return GDN_OK;
}

gdn_status gdn_beam_stamp_projection(void* buf, size_t bytes) {
  if (buf && (!aligned16(buf) || bytes < size_t(kStampWords) * 4)) return GDN_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_stamp.m);
  g_stamp.buf = static_cast<uint32_t*>(buf);
  g_stamp.records = buf ? bytes / (size_t(kStampWords) * 4) : 0;
  return GDN_OK;
}

gdn_status gdn_beam_stream_probe(void* dst, const void* src, size_t bytes, int32_t mode,
                                 hipStream_t stream) {
  if (!dst || !aligned16(dst) || bytes % 16 != 0 || mode < 0 || mode > 2) return GDN_ERR_INVALID_ARG;
  if (mode != 2 && (!src || !aligned16(src))) return GDN_ERR_INVALID_ARG;
  if (bytes == 0) return GDN_OK;
  const int err = launch_stream_probe(dst, src, bytes, mode, stream);
  return err ? hip_fail(err, "gdn_beam_stream_probe") : GDN_OK;
}

gdn_status gdn_beam_step_times(float* ms, int32_t cap, int32_t* n) {
  if (!n || cap < 0 || (cap > 0 && !ms)) return GDN_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_timer.m);
  const int m = g_timer.n < cap ? g_timer.n : cap;
  for (int i = 0; i < m; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], g_timer.ev[2 * i], g_timer.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(int(e), "gdn_beam_step_times");
  }
  *n = g_timer.n;
  g_timer.n = 0;
  return GDN_OK;
}

size_t gdn_beam_prefill_workspace_bytes(int32_t H, int32_t d_k, int32_t d_v, int64_t N) {
  if (H < 1 || N < 0 || !dims_supported(d_k, d_v)) return 0;
  return prefill_workspace_bytes(H, d_k, N);
}

gdn_status gdn_beam_prefill(int32_t R, int32_t H, int32_t H_K, int32_t d_k, int32_t d_v, int64_t N,
                            const float* k, const float* v, const float* alpha,
                            const float* beta, const int32_t* offsets, float* S_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (R < 1 || H < 1 || N < 0 || H_K < 0) return GDN_ERR_INVALID_ARG;
  if (H_K == 0) H_K = H;
  if (H % H_K != 0) return GDN_ERR_INVALID_ARG;
  if (!dims_supported(d_k, d_v)) return GDN_ERR_UNSUPPORTED;
  if (!offsets || !S_out) return GDN_ERR_INVALID_ARG;
  if (N > 0 && (!k || !v || !alpha || !beta)) return GDN_ERR_INVALID_ARG;
  if (!aligned16(offsets) || !aligned16(S_out)) return GDN_ERR_INVALID_ARG;
  if (N > 0 && (!aligned16(k) || !aligned16(v) || !aligned16(alpha) || !aligned16(beta)))
    return GDN_ERR_INVALID_ARG;
  if (N >= (int64_t(1) << 31)) return GDN_ERR_CAPACITY;
  float* ws = nullptr;
  if (workspace && prefill_chunked(d_k)) {
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return GDN_ERR_INVALID_ARG;
    if (workspace_bytes < prefill_workspace_bytes(H, d_k, N)) return GDN_ERR_WORKSPACE;
    ws = static_cast<float*>(workspace);
  }
  PrefillArgs a{R, H, H_K, d_k, d_v, N, k, v, alpha, beta, offsets, S_out, ws};
  int err = launch_prefill(a, stream);
  if (err) return hip_fail(err, "gdn_beam_prefill");
  return GDN_OK;
}

}  // extern "C"
