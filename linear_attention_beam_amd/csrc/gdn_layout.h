// Internal: workspace layout and launch arguments shared by the host front end
// (gdn_beam_api.cpp) and the kernels (gdn_step.hip, gdn_select.hip).  Not installed.
#pragma once
#include <cstddef>
#include <cstdint>
#include "../../include/gdn_beam.h"

#if defined(__HIPCC__)
#define GDN_HD __host__ __device__
#else
#define GDN_HD
#endif

namespace gdn {

constexpr int kMaxT = 8;          // SID steps
constexpr int kMaxW = 1024;       // beams per step (one sorting workgroup holds them)
constexpr int kMaxV = 65536;      // codebook
constexpr int kHistBins = 2048;   // radix digits per selection pass (11 bits)
// Static selection scratch of gdn_beam_select_static, per GPU (GDN_STATIC_SCRATCH_BYTES).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kStaticScratchDevices = 64;

// Per-request selection results handed from the tile choice to the refinement.
struct SelState {
  uint32_t n_tiles;     // tiles chosen for refinement
  uint32_t n_groups;    // refinement groups (code tile x up to 32 beams)
  uint32_t theta;       // key of the K-th chosen tile (0: fewer than K tiles exist)
  uint32_t pad;
};

// Byte offsets of the per-call scratch of one selection (256-aligned): nothing in these
// regions outlives a gdn_beam_select call.  Inside the workspace they follow the beam
// state; a selection may also take them from another buffer laid out the same way.
struct SelScratch {
  size_t z;           // [R,W_max,d_v] f32  head-summed outputs (fp32 codebook)
  size_t zf;          // [R,n_chunks(W_max),d_v/16,3,64] u32x4: z as bf16 hi/mid/lo MFMA operand
  size_t woutT;       // [V_max,d_v] wout dtype, codebook transposed
  size_t tmax;        // [R, n_tiles(V_max)*W_max] f32, per request [n_tiles(V)][W_t] ([W_t][n_tiles(V)]
                      // where the selection is bounded)
  size_t lse_part;    // [R,W_max,n_vgroups(V_max)] float4 (max, sum of exp, min tile max, 0)
  size_t lse;         // [R,W_max] f32
  size_t sel;         // [R] SelState
  size_t cand;        // [R, n_tiles(V_max)*W_max] u32 flat tiles inside the boundary digit
  size_t tiles;       // [R,W_max] u32 chosen flat tiles, grouped by code tile
  size_t groups;      // [R,max_groups] u32 refinement groups
  size_t gtiles;      // [R,max_groups,32] u32 the tiles of each group
  size_t rkeys;       // [R,W_max,kTile] u32 keys of the chosen tiles' candidates
  size_t flog;        // [R,W_max] f32 logits of the forced candidates
  size_t f16flag;     // u32: a code tile of the bf16 codebook does not fit fp16 (zero
                      // between selections)
  size_t tscale;      // [n_tiles(V_max)] i32: exponent s_j of code tile j's fp16 scale 2^s_j
  size_t woutT16;     // [V_max,d_v] fp16: the bf16 codebook transposed, tile j scaled by 2^s_j
  size_t zscale;      // [R,W_max] f32: 2^-t_b, undoes beam b's scale of z
  size_t end;         // first byte past the regions (256-aligned)
};

// Byte offsets of every region inside the caller's workspace (256-aligned).
struct Layout {
  size_t s_frag;      // [R,H] S_ctx in MFMA fragment order, 4*d_vp*d_k bytes each
  size_t gtr_alpha;   // [R,H,T_max,W_max] f32
  size_t gtr_delta;   // [R,H,T_max,W_max,d_v] f32
  size_t gtr_key;     // [R,H,T_max,W_max,d_k] io dtype
  size_t anc[2];      // [R,W_max,T_max] i32, ping-pong by step parity
  size_t tok[2];      // [R,W_max,T_max] i32
  size_t cum[2];      // [R,W_max] f32
  size_t order[2];    // [R,W_max] i32 beam processing order of a step (siblings adjacent)
  size_t opos[2];     // [R,W_max] i32 position of each beam in that order
  SelScratch S;       // the selection's per-call scratch
  size_t status;      // [64] i32
  size_t total;
};

GDN_HD inline int dvp_of(int d_v) { return d_v < 32 ? 32 : d_v; }   // rows padded to one MFMA block
GDN_HD inline int io_bytes(gdn_dtype d) { return d == GDN_BF16 ? 2 : 4; }

// Codes per tile: one 32-row MFMA block.  The selection keeps one maximum per
// (beam, tile) and refines at most W_next tiles.
constexpr int kTile = 32;
GDN_HD inline int n_tiles(int V) { return (V + kTile - 1) / kTile; }
GDN_HD inline int n_chunks(int W) { return (W + 31) / 32; }   // 32-beam MFMA columns
// refinement groups: sum over code tiles of ceil(beams / 32) <= ceil(K/32) + min(Vt, K)
GDN_HD inline int max_groups(int W_max, int Vt_max) {
  return n_chunks(W_max) + 1 + (Vt_max < W_max ? Vt_max : W_max);
}
// First-pass work unit: 32 beams x (128 .. 1024) codes; log-sum-exp parts per unit.
constexpr int kCodesPerWave = 128;
GDN_HD inline int n_vgroups(int V) { return (V + kCodesPerWave - 1) / kCodesPerWave; }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int key_heads(const gdn_beam_config& c) { return c.H_K > 0 ? c.H_K : c.H; }

// The selection's scratch regions of a configuration, laid out from byte `off`.
inline SelScratch make_sel_scratch(const gdn_beam_config& c, size_t off) {
  SelScratch S{};
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t R = c.R, W = c.W_max, V = c.V_max;
  const size_t dv = c.d_v, ew = io_bytes(c.wout_dtype);
  const size_t Vt = size_t(n_tiles(c.V_max));
  S.z = take(R * W * dv * 4);
  S.zf = take(R * size_t(n_chunks(c.W_max)) * 32 * dv * 6);
  S.woutT = take(V * dv * ew);
  S.tmax = take(R * Vt * W * 4);
  S.lse_part = take(R * W * size_t(n_vgroups(c.V_max)) * 16);
  S.lse = take(R * W * 4);
  S.sel = take(R * sizeof(SelState));
  S.cand = take(R * Vt * W * 4);
  S.tiles = take(R * W * 4);
  S.groups = take(R * size_t(max_groups(c.W_max, n_tiles(c.V_max))) * 4);
  S.gtiles = take(R * size_t(max_groups(c.W_max, n_tiles(c.V_max))) * 32 * 4);
  S.rkeys = take(R * W * kTile * 4);
  S.flog = take(R * W * 4);
  S.f16flag = take(128);
  S.tscale = take(Vt * 4);
  S.woutT16 = take(V * dv * 2);
  S.zscale = take(R * W * 4);
  S.end = off;
  return S;
}

inline Layout make_layout(const gdn_beam_config& c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t R = c.R, H = c.H, T = c.T_max, W = c.W_max;
  const size_t dk = c.d_k, dv = c.d_v, e = io_bytes(c.io_dtype);
  L.s_frag = take(R * H * 4 * size_t(dvp_of(c.d_v)) * dk);
  L.gtr_alpha = take(R * H * T * W * 4);
  L.gtr_delta = take(R * H * T * W * dv * 4);
  L.gtr_key = take(R * size_t(key_heads(c)) * T * W * dk * e);
  for (int i = 0; i < 2; ++i) L.anc[i] = take(R * W * T * 4);
  for (int i = 0; i < 2; ++i) L.tok[i] = take(R * W * T * 4);
  for (int i = 0; i < 2; ++i) L.cum[i] = take(R * W * 4);
  for (int i = 0; i < 2; ++i) L.order[i] = take(R * W * 4);
  for (int i = 0; i < 2; ++i) L.opos[i] = take(R * W * 4);
  L.S = make_sel_scratch(c, off);
  off = L.S.end;
  L.status = take(64 * 4);
  L.total = off;
  return L;
}

// ---- launch arguments (host -> kernel TU) ----
struct InitArgs {
  int R, H, d_k, d_v, W_max, T_max;
  gdn_dtype io;
  const float* S_ctx;
  void* ws;
  Layout L;
};

struct StepArgs {
  int R, H, HK, d_k, d_v, W_max, T_max, t, W;
  gdn_dtype io;
  const void *q, *k, *v;
  const float *alpha, *beta;
  float* o;
  void* ws;
  Layout L;
  hipEvent_t ev0, ev1;    // non-null: the launch records its own start and end on them
  uint32_t* stamps;       // non-null: projection-phase stamps (kStampWords per record)
  size_t stamp_records;   // records the buffer holds
};

// Projection-phase stamp of one (workgroup, wave, chunk) of a step launch, as uint32
// words: shader-clock cycle before the first projection MFMA (lo, hi), after the last
// result is read (lo, hi), HW_ID, XCC_ID, MFMA flops of the phase, and the bits of the
// value that read the results.  Record ((wid * NW) + wave) * chunks + chunk, wid the
// launch's work item (request-head, then row block), NW waves per workgroup.
constexpr int kStampWords = 8;

struct SelectArgs {
  int R, H, d_v, W_max, V_max, T_max, t, W, V, W_next;
  gdn_dtype wout_dtype;
  const float* o;
  const void* Wout;
  const int32_t *forced_parent, *forced_token;
  int32_t *parent, *token;
  float* score;
  void* ws;               // workspace: beam state, ancestry, status
  Layout L;
  char* scr;              // base of the selection scratch regions S (offsets from scr)
  SelScratch S;
};

// Chunked prefill: 32-token chunks; per (chunk, head) the preparation kernel stores the
// 32 x 32 chunk matrix and two 32-entry decay products.
constexpr int kChunk = 32;
constexpr int kPrepFloats = kChunk * kChunk + 2 * kChunk;

struct PrefillArgs {
  int R, H, HK, d_k, d_v;
  int64_t N;
  const float *k, *v, *alpha, *beta;
  const int32_t* offsets;
  float* S_out;
  float* ws;            // chunked form's workspace, or null for the token-sequential form
};

struct FullStepArgs {
  int R, H, HK, d_k, d_v, W_max, T_max, t, W;
  gdn_dtype io;
  const float* S_ctx;
  const void *q, *k, *v;
  const float *alpha, *beta;
  float* o;
  void* states;           // two generations of R*H*W_max*d_v*d_k fp32 states
  size_t half_bytes;      // bytes of one generation
  const int32_t* anc;     // ancestry of step t in the workspace
  hipEvent_t ev0, ev1;    // non-null: the launch records its own start and end on them
};

inline size_t fullstate_half_bytes(const gdn_beam_config& c) {
  return size_t(c.R) * c.H * c.W_max * size_t(c.d_v) * c.d_k * 4;
}

// Kernel launchers (gdn_step.hip, gdn_select.hip, gdn_fullstate.hip).  Return a
// hipError_t value.
int launch_init(const InitArgs& a, hipStream_t s);
int launch_step(const StepArgs& a, hipStream_t s);
int launch_select(const SelectArgs& a, hipStream_t s);
// Device address of the current device's static selection scratch (kStaticScratchBytes,
// 256-aligned); looked up once per device.  Returns a hipError_t value.
int static_scratch(char** ptr);
int launch_prefill(const PrefillArgs& a, hipStream_t s);
bool prefill_chunked(int d_k);
size_t prefill_workspace_bytes(int H, int d_k, int64_t N);
int launch_fullstate(const FullStepArgs& a, hipStream_t s);
// Streaming probe (gdn_probe.hip): mode 0 copies bytes / 16 16-byte units, mode 1 reads them.
int launch_stream_probe(void* dst, const void* src, size_t bytes, int mode, hipStream_t s);
int copy_d2d(void* dst, const void* src, size_t bytes, hipStream_t s);
const char* hip_error_string(int err);

}  // namespace gdn
