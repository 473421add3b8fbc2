// Step-side HIP kernels for large-beam Gated DeltaNet decoding on gfx950 (CDNA4).
//
// OneLA reading note (paper-archivist.com), sections 2.1-2.5: one shared state
// S_ctx per (request, head), append-only transition records (alpha, delta, k) in
// fixed slots, an ancestry index, and a fused shared-context step.
//
// Kernels
//   init_kernel      S_ctx -> MFMA fragment order in the workspace; clear beam state.
//   step_kernel      fused step: S_ctx [q|k] on MFMA (eqs. 6-7 initial terms), replay
//                    along the ancestor records (eqs. 6-7), eq. (8), record append.
#include <hip/hip_ext.h>

#include <type_traits>

#include "gdn_device.h"

namespace gdn {

// ---------------------------------------------------------------- init

// S_frag per (r,h): bf16 io: blocks (rb, kk, part) of 64 lanes x 8 bf16,
//   lane l -> S[32 rb + frag_row(l%32)][d_k/2*(l/32) + 8 kk + i], part 0 = hi, 1 = lo.
// f32 io: blocks (rb, kk4) of 64 lanes x 4 f32, lane l -> S[..][d_k/2*(l/32) + 4 kk4 + i].
// One thread per 16-byte fragment position: it loads the 8 (bf16 io) or 4 (f32 io)
// source values once and writes every part, so all loads of the grid are independent.
__global__ void __launch_bounds__(256) init_kernel(InitArgs a) {
  const int dk = a.d_k, dv = a.d_v, dvp = dvp_of(dv), nrb = dvp / 32;
  const bool bf = a.io == GDN_BF16;
  const int nkk = bf ? dk / 16 : dk / 8;           // fragment columns per 32-row block
  const int per_rh = nrb * nkk * 64;
  const size_t n = size_t(a.R) * a.H * per_rh;
  char* ws = static_cast<char*>(a.ws);
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t g = size_t(blockIdx.x) * blockDim.x + threadIdx.x; g < n; g += stride) {
    const size_t rh = g / per_rh;
    const int c = int(g % per_rh);
    const int lane = c & 63, blk = c >> 6;           // blk = rb * nkk + kk
    const int kk = blk % nkk, rb = blk / nkk;
    const int row = 32 * rb + frag_row(lane & 31);
    const float* S = a.S_ctx + rh * dv * dk;
    u32x4* dst = reinterpret_cast<u32x4*>(ws + a.L.s_frag + rh * 4 * dvp * dk);
    if (bf) {
      const int k0 = (dk / 2) * (lane >> 5) + 8 * kk;
      f32x4 x0 = {}, x1 = {};
      if (row < dv) {
        x0 = *reinterpret_cast<const f32x4*>(S + size_t(row) * dk + k0);
        x1 = *reinterpret_cast<const f32x4*>(S + size_t(row) * dk + k0 + 4);
      }
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = i < 4 ? x0[i] : x1[i - 4];
        hi[i] = f2bf(x);
        lo[i] = f2bf(x - bf2f(hi[i]));
      }
      dst[(2 * blk) * 64 + lane] = pack8(hi);
      dst[(2 * blk + 1) * 64 + lane] = pack8(lo);
    } else {
      const int k0 = (dk / 2) * (lane >> 5) + 4 * kk;
      f32x4 f = {};
      if (row < dv) f = *reinterpret_cast<const f32x4*>(S + size_t(row) * dk + k0);
      reinterpret_cast<f32x4*>(dst)[c] = f;
    }
  }
  // beam state: cumulative scores 0, empty ancestry and SID prefixes, clear status
  const size_t nb = size_t(a.R) * a.W_max * a.T_max;
  float* cum = reinterpret_cast<float*>(ws + a.L.cum[0]);
  int32_t* anc = reinterpret_cast<int32_t*>(ws + a.L.anc[0]);
  int32_t* tok = reinterpret_cast<int32_t*>(ws + a.L.tok[0]);
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nb; i += stride) {
    anc[i] = tok[i] = 0;
    if (i < size_t(a.R) * a.W_max) cum[i] = 0.0f;
  }
  if (blockIdx.x == 0 && threadIdx.x < 64)
    reinterpret_cast<int32_t*>(ws + a.L.status)[threadIdx.x] = 0;
  // the selection's flag for code tiles that do not fit fp16 starts clear (each selection
  // clears it after use)
  if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<uint32_t*>(ws + a.L.S.f16flag) = 0u;
}

// ---------------------------------------------------------------- step

struct StepK {
  int H, HK, W, W_max, T_max, t, nrh;
  const void *q, *k, *v;
  const float *alpha, *beta;
  float* o;
  const char* s_frag;
  float* gtr_alpha;
  float* gtr_delta;
  void* gtr_key;
  const int32_t* anc;
  const int32_t* order;    // [R,W_max] processing order of the beams (steps t >= 1)
  uint32_t* stamps;        // projection-phase stamps (measurement), or null
  uint32_t stamp_records;
};

// Sizes of the fused step for head dims (DK, DV) and io dtype.
template <int DK, int DV, bool BF16, int TT = 0>
struct StepCfg {
  static constexpr int DVP = DV < 32 ? 32 : DV;
  // rows of d_v per workgroup.  d_k = 256 from t = 1 on: 128 rows (four waves, each with
  // the full register file: its S_ctx fragments alone take 128 registers), so that the
  // ancestor records' keys and delta rows stay in registers too; t = 0 replays nothing
  // and keeps 256 rows with two waves per SIMD
  static constexpr bool WIDE = DK > 128 && TT > 0;
  static constexpr int DVMAX = WIDE ? 128 : 256;
  static constexpr int DVB = DVP > DVMAX ? DVMAX : DVP;
  static constexpr int MINB = WIDE ? 1 : 2;            // workgroups per CU the registers allow
  static constexpr int NRB = DVP / DVB;          // workgroups per (request, head)
  static constexpr int NW = DVB / 32;            // one wave per 32-row block of d_v
  static constexpr int NT = NW * 64;
  static constexpr int E = BF16 ? 2 : 4;         // bytes per io element
  static constexpr int QB = DK * E;              // bytes of one q / k row
  static constexpr int VB = (DV < DVB ? DV : DVB) * E;   // bytes of a workgroup's v rows
  static constexpr int QROW = QB + 16;           // padded LDS rows (bank spread)
  static constexpr int VROW = VB + 16;
  static constexpr int QU = 32 * QB / 16 / NT;   // 16-byte staging units per thread
  static constexpr int VU = 32 * VB / 16 / NT;
  static constexpr int TPB = NT / 32;            // threads per beam in the dot phase
  static constexpr int SEGB = QB / TPB;          // bytes of q / k each of them takes
  static constexpr int SLOT = 32 * (2 * QROW + VROW) + 2 * 32 * 4 + 32 * kMaxT * 4;
  static_assert(QU >= 1 && VU >= 1 && SEGB >= 16 && SEGB % 16 == 0, "unsupported shape");
};

template <bool BF16>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float s) {
  if constexpr (BF16) {
    // (bit-cast whole vectors, never single elements of one: hipcc lowers a bit-cast
    // of an ext-vector element to element 0)
    const bf16x8 x = __builtin_bit_cast(bf16x8, a);
    const bf16x8 y = __builtin_bit_cast(bf16x8, b);
    s = __builtin_amdgcn_fdot2_f32_bf16(x.s01, y.s01, s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(x.s23, y.s23, s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(x.s45, y.s45, s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(x.s67, y.s67, s, false);
  } else {
    const f32x4 x = __builtin_bit_cast(f32x4, a);
    const f32x4 y = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(x[i], y[i], s);
  }
  return s;
}

// Fused SID step (OneLA reading note, sections 2.3-2.5).  One workgroup per
// (request, head); wave w owns rows [32 w, 32 w + 32) of d_v and keeps that block of
// S_ctx (bf16 hi/lo, or fp32) as MFMA A fragments in registers for every beam.  Beams
// go through in chunks of 32: a chunk's q, k, v, gates and ancestry indices are
// loaded with contiguous reads into registers while the previous chunk computes, then
// written to a double-buffered LDS slot.  Per chunk:
//   issue    the ancestor records' keys (for the dots) and delta rows (for the
//            replay), then the next chunk's inputs;
//   dots     threads cooperate per beam on k_t.q_t and, for each ancestor record j,
//            k_j.q_t and k_j.k_t (contiguous reads of the records' keys);
//   per wave U = S_block [q|k] on MFMA (B fragments from LDS), then eqs. (6)-(7) on
//            the accumulators and eq. (8); delta_t and o_t stored;
//   append   k_t rows copied from LDS to slot (t, b) of the record pool, alpha_t.
// From t = 1 on, chunks take the beams in the order the selection left (children of
// one parent adjacent, subtrees contiguous), so the records that siblings and cousins
// share are gathered back to back, from cache.
template <int DK, int DV, bool BF16, int TT>
__global__ void __launch_bounds__((StepCfg<DK, DV, BF16, TT>::NT), (StepCfg<DK, DV, BF16, TT>::MINB)) step_kernel(StepK a) {
  using C = StepCfg<DK, DV, BF16, TT>;
  constexpr int NT = C::NT, QROW = C::QROW, VROW = C::VROW, TPB = C::TPB;
  constexpr int UPQ = C::QB / 16, UPV = C::VB / 16;      // 16-byte units per row
  constexpr int NJ = TT;                                 // ancestor records replayed
  constexpr int NJ1 = NJ > 0 ? NJ : 1;
  constexpr int HK = DK / 2;
  constexpr int SCN = 1 + 3 * NJ;                        // kq, alpha_j, cq_j, ck_j
  __shared__ __align__(16) unsigned char lds[2 * C::SLOT + 32 * SCN * 4];
  __shared__ int ord[NJ > 0 ? kMaxW : 1];
  // per wave: its 32 x 32 block of delta_t (then o_t) as [beam][row], rows padded to 36
  // (where the LDS allows; else each lane stores its own 16 rows)
  constexpr int XT = 36;
  constexpr bool TURN = 2 * C::SLOT + 32 * (1 + 3 * 7) * 4 + 4 * kMaxW + C::NW * 32 * XT * 4 <= 160 * 1024;
  __shared__ __align__(16) float xt[TURN ? C::NW * 32 * XT : 1];
  float* sc = reinterpret_cast<float*>(lds + 2 * C::SLOT);

  const int wid = xcd_work_id();
  if (wid >= a.nrh * C::NRB) return;                      // whole block, before any barrier
  // d_v rows beyond 256 go to further workgroups of the same (request, head): rows of
  // the state evolve independently; the per-beam dot products are redone by each
  const int rh = wid / C::NRB, rb = wid % C::NRB, row_base = rb * C::DVB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = lane & 31, hf = lane >> 5;
  const int W = a.W, r = rh / a.H;
  // grouped value heads: q, k and the records' keys belong to key head h / (H / HK)
  const int grp = a.H / a.HK, hv = rh % a.H;
  const int rk = r * a.HK + hv / grp;
  const bool key_writer = hv % grp == 0;
  const int nch = (W + 31) >> 5;
  const size_t slot_t = size_t(rh) * a.T_max + TT;       // (r,h,t) row of the record pool
  const size_t kslot_t = size_t(rk) * a.T_max + TT;      // (r,h_k,t) row of the key pool
  const unsigned char* qg = static_cast<const unsigned char*>(a.q);
  const unsigned char* kg = static_cast<const unsigned char*>(a.k);
  const unsigned char* vg = static_cast<const unsigned char*>(a.v);
  unsigned char* keyg = static_cast<unsigned char*>(a.gtr_key);

  if constexpr (NJ > 0) {
    for (int i = tid; i < W; i += NT) {
      const int x = a.order[size_t(r) * a.W_max + i];
      ord[i] = x < 0 ? 0 : (x >= W ? W - 1 : x);
    }
  }
  auto beam_of = [&](int x) { return NJ > 0 ? ord[x] : x; };

  // this wave's block of S_ctx as A fragments (layout written by init_kernel)
  constexpr int NA = BF16 ? 2 * (DK / 16) : DK / 8;
  u32x4 afr[NA];
  {
    const u32x4* fr = reinterpret_cast<const u32x4*>(a.s_frag + size_t(rh) * 4 * C::DVP * DK);
#pragma unroll
    for (int i = 0; i < NA; ++i) afr[i] = fr[((rb * C::NW + w) * NA + i) * 64 + lane];
  }

  // ---- staging of one chunk: registers <- global (contiguous), LDS <- registers
  u32x4 sq[C::QU], sk[C::QU], sv[C::VU];
  float sab = 0.0f;
  constexpr int NAI = (32 * NJ1 + NT - 1) / NT;
  int sanc[NAI];
  auto stage_load = [&](int c) {
    const int c0 = c * 32, nb = min(32, W - c0);
    const size_t base = size_t(rh) * W, kbase = size_t(rk) * W;
#pragma unroll
    for (int i = 0; i < C::QU; ++i) {
      const int u = tid + i * NT;
      if (u / UPQ < nb) {
        const size_t row = kbase + beam_of(c0 + u / UPQ);
        sq[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qg + row * C::QB + size_t(u % UPQ) * 16));
        sk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kg + row * C::QB + size_t(u % UPQ) * 16));
      }
    }
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
      const int u = tid + i * NT;
      if (u / UPV < nb)
        sv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vg + ((base + beam_of(c0 + u / UPV)) * DV + row_base) * C::E +
                                                size_t(u % UPV) * 16));
    }
    if (tid < 64 && (tid & 31) < nb) {
      const size_t bi = base + beam_of(c0 + (tid & 31));
      sab = tid < 32 ? a.alpha[bi] : a.beta[bi];
    }
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      const int e = tid + i * NT, bb = e / NJ1, j = e % NJ1;
      if (NJ > 0 && e < 32 * NJ && bb < nb)
        sanc[i] = a.anc[(size_t(r) * a.W_max + beam_of(c0 + bb)) * a.T_max + j];
    }
  };
  auto stage_store = [&](int slot) {
    unsigned char* L = lds + slot * C::SLOT;
#pragma unroll
    for (int i = 0; i < C::QU; ++i) {
      const int u = tid + i * NT, bb = u / UPQ, o = (u % UPQ) * 16;
      *reinterpret_cast<u32x4*>(L + bb * QROW + o) = sq[i];
      *reinterpret_cast<u32x4*>(L + 32 * QROW + bb * QROW + o) = sk[i];
    }
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
      const int u = tid + i * NT, bb = u / UPV, o = (u % UPV) * 16;
      *reinterpret_cast<u32x4*>(L + 64 * QROW + bb * VROW + o) = sv[i];
    }
    float* ab = reinterpret_cast<float*>(L + 64 * QROW + 32 * VROW);
    if (tid < 64) ab[tid] = sab;
    int* an = reinterpret_cast<int*>(L + 64 * QROW + 32 * VROW + 256);
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      const int e = tid + i * NT, bb = e / NJ1, j = e % NJ1;
      if (NJ > 0 && e < 32 * NJ) {
        const int s = sanc[i];
        an[bb * kMaxT + j] = s < 0 ? 0 : (s >= a.W_max ? a.W_max - 1 : s);
      }
    }
  };

  if constexpr (NJ > 0) __syncthreads();                  // ord complete
  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int c0 = c * 32, nb = min(32, W - c0);
    const unsigned char* L = lds + (c & 1) * C::SLOT;
    const unsigned char* Lq = L;
    const unsigned char* Lk = L + 32 * QROW;
    const unsigned char* Lv = L + 64 * QROW;
    const float* Lab = reinterpret_cast<const float*>(L + 64 * QROW + 32 * VROW);
    const int* Lan = reinterpret_cast<const int*>(L + 64 * QROW + 32 * VROW + 256);

    // Issue order for the chunk (loads complete in issue order): the ancestor keys for
    // the dot products, the ancestors' delta rows for this wave's replay, the next
    // chunk's inputs.  The dots wait only for the keys.
    // dot-phase role: TPB threads per beam; thread sg takes the 16-byte pieces sg,
    // sg + TPB, ... of a row, so TPB neighbours read 16 TPB contiguous bytes at a time
    const int bm = tid / TPB, sg = tid % TPB;
    constexpr int SV = C::SEGB / 16;
    auto piece = [&](int i) { return 16 * sg + 16 * TPB * i; };
    u32x4 kj[NJ1][SV];
    float aj[NJ1];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int sl = bm < nb ? Lan[bm * kMaxT + j] : 0;
      const size_t rec = (size_t(rh) * a.T_max + j) * a.W_max + sl;
      const size_t krec = (size_t(rk) * a.T_max + j) * a.W_max + sl;
      aj[j] = a.gtr_alpha[rec];
#pragma unroll
      for (int i = 0; i < SV; ++i)
        kj[j][i] = *reinterpret_cast<const u32x4*>(keyg + krec * C::QB + piece(i));
    }
    const bool valid = m < nb;
    const int b = valid ? beam_of(c0 + m) : 0;
    const int row0 = 32 * w + 16 * hf;                   // first row of this lane half (local)
    const int grow0 = row_base + row0;                   // ... of the state
    // turned layout of the epilogue (where the wave's LDS block exists): lane l holds
    // rows sr .. sr + 3 of this wave's 32 rows for beams 8 q + sb (q < 4), so that eight
    // lanes cover one beam's 128 contiguous bytes of a record, of delta_t and of o_t
    const int sb = lane >> 3, sr = 4 * (lane & 7);
    f32x4 dj[NJ1][4];
    if constexpr (TURN) {
      const int rt = min(row_base + 32 * w + sr, DV - 4);    // in range (rows >= DV unused)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int bb = 8 * q + sb;
          const size_t rec = (size_t(rh) * a.T_max + j) * a.W_max + (bb < nb ? Lan[bb * kMaxT + j] : 0);
          dj[j][q] = *reinterpret_cast<const f32x4*>(a.gtr_delta + rec * DV + rt);
        }
    } else {
      const int rowl = min(grow0, DV - 16);                // in range (rows >= DV unused)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const size_t rec = (size_t(rh) * a.T_max + j) * a.W_max + (valid ? Lan[m * kMaxT + j] : 0);
        const f32x4* dp = reinterpret_cast<const f32x4*>(a.gtr_delta + rec * DV + rowl);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) dj[j][q4] = dp[q4];
      }
    }
    if (c + 1 < nch) stage_load(c + 1);                  // in flight until the end of the chunk

    // ---- dots: TPB threads per beam, SEGB bytes of d_k each; then a barrier (the
    // epilogue reads them per beam)
    auto dots = [&]() {
      {
        u32x4 xq[SV], xk[SV];
#pragma unroll
        for (int i = 0; i < SV; ++i) {
          xq[i] = *reinterpret_cast<const u32x4*>(Lq + bm * QROW + piece(i));
          xk[i] = *reinterpret_cast<const u32x4*>(Lk + bm * QROW + piece(i));
        }
        float kq = 0.0f;
#pragma unroll
        for (int i = 0; i < SV; ++i) kq = dot16<BF16>(xk[i], xq[i], kq);
        float cq[NJ1], ck[NJ1];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          cq[j] = 0.0f;
          ck[j] = 0.0f;
#pragma unroll
          for (int i = 0; i < SV; ++i) {
            cq[j] = dot16<BF16>(kj[j][i], xq[i], cq[j]);
            ck[j] = dot16<BF16>(kj[j][i], xk[i], ck[j]);
          }
        }
#pragma unroll
        for (int off = 1; off < TPB; off <<= 1) {
          kq += __shfl_xor(kq, off);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            cq[j] += __shfl_xor(cq[j], off);
            ck[j] += __shfl_xor(ck[j], off);
          }
        }
        if (sg == 0) {
          sc[bm * SCN] = kq;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            sc[bm * SCN + 1 + j] = aj[j];
            sc[bm * SCN + 1 + NJ + j] = cq[j];
            sc[bm * SCN + 1 + 2 * NJ + j] = ck[j];
          }
        }
      }
      __syncthreads();
    };

    // ---- this wave's row block for the chunk's 32 beams (lane: beam m, rows half hf)
    f32x16 accq = {}, acck = {};
    auto project = [&]() {
      if constexpr (BF16) {
#pragma unroll
        for (int kk = 0; kk < DK / 16; ++kk) {
          const int off = m * QROW + (HK * hf + 8 * kk) * 2;
          const bf16x8 bq = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Lq + off));
          const bf16x8 bk = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Lk + off));
          const bf16x8 ahi = __builtin_bit_cast(bf16x8, afr[2 * kk]);
          const bf16x8 alo = __builtin_bit_cast(bf16x8, afr[2 * kk + 1]);
          accq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bq, accq, 0, 0, 0);
          acck = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bk, acck, 0, 0, 0);
          accq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bq, accq, 0, 0, 0);
          acck = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bk, acck, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kk4 = 0; kk4 < DK / 8; ++kk4) {
          const int off = m * QROW + (HK * hf + 4 * kk4) * 4;
          const f32x4 bq = *reinterpret_cast<const f32x4*>(Lq + off);
          const f32x4 bk = *reinterpret_cast<const f32x4*>(Lk + off);
          const f32x4 af = __builtin_bit_cast(f32x4, afr[kk4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            accq = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bq[i], accq, 0, 0, 0);
            acck = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bk[i], acck, 0, 0, 0);
          }
        }
      }
    };
    // projection-phase stamps (a measurement; the launch's results are the same): the
    // shader clock before the first projection MFMA and after a VALU operation has read
    // the last results, which waits for them.  With stamps on, the dot products of the
    // chunk start only after that wait.
    const bool stamping = a.stamps != nullptr;             // launch-uniform
    uint64_t ts0 = 0;
    auto stamp_begin = [&]() {
      if (stamping) {
        __builtin_amdgcn_sched_barrier(0);
        ts0 = __builtin_amdgcn_s_memtime();
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto stamp_end = [&]() {
      if (stamping) {
        __builtin_amdgcn_sched_barrier(0);
        const float probe = accq[15] + acck[15];          // waits for both accumulators
        __builtin_amdgcn_sched_barrier(0);
        const uint64_t ts1 = __builtin_amdgcn_s_memtime();
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t rec = uint32_t((wid * C::NW + w) * nch + c);
        if (lane == 0 && rec < a.stamp_records) {
          constexpr uint32_t flops = BF16 ? uint32_t(DK / 16) * 4u * 32768u : uint32_t(DK / 8) * 8u * 4096u;
          const uint32_t hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));   // HW_ID
          const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)); // XCC_ID
          u32x4* dst = reinterpret_cast<u32x4*>(a.stamps + size_t(rec) * kStampWords);
          dst[0] = u32x4{uint32_t(ts0), uint32_t(ts0 >> 32), uint32_t(ts1), uint32_t(ts1 >> 32)};
          dst[1] = u32x4{hw, xcc, flops, __float_as_uint(probe)};
        }
      }
    };
    // with at most two records to replay (d_k <= 128) the projection goes first, on the
    // matrix cores while the records' keys are still on their way; deeper replays and
    // wider keys keep the order that fits their registers
    if constexpr (NJ <= 2 && DK <= 128) {
      stamp_begin();
      project();
      stamp_end();
      dots();
    } else {
      dots();
      stamp_begin();
      project();
      stamp_end();
    }

    {
      float* dbase = a.gtr_delta + slot_t * a.W_max * DV;
      float* obase = a.o + size_t(rh) * W * DV;
      if constexpr (TURN) {
        // the accumulators turn through the wave's LDS block (the wave alone uses it;
        // its LDS operations complete in order), then eqs. (6)-(8) run per beam of the
        // turned layout and delta_t, o_t go straight out
        float* tw = xt + w * (32 * XT);
        const int rl = 32 * w + sr;                          // row among this workgroup's rows
        const int gr = row_base + rl;                        // row of the state
        constexpr int RV = (DV < C::DVB ? DV : C::DVB) - 4;  // last row group staged in Lv
        f32x4 uq[4], uk[4];
        auto turn = [&](const f32x16& x, f32x4* y) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4*>(tw + m * XT + 16 * hf + 4 * q4) =
                f32x4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] = *reinterpret_cast<const f32x4*>(tw + (8 * q + sb) * XT + sr);
          asm volatile("" ::: "memory");                     // the block's reads before its reuse
        };
        turn(accq, uq);
        turn(acck, uk);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int bb = 8 * q + sb;                         // beam slot of the chunk
          const float* sp = sc + bb * SCN;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const float ajj = sp[1 + j], cqj = sp[1 + NJ + j], ckj = sp[1 + 2 * NJ + j];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uq[q][i] = fmaf(dj[j][q][i], cqj, ajj * uq[q][i]);   // eq. (6)
              uk[q][i] = fmaf(dj[j][q][i], ckj, ajj * uk[q][i]);   // eq. (7)
            }
          }
          const float kq = sp[0], al = Lab[bb], be = Lab[32 + bb];
          float vv[4];
          const int rv = rl < RV ? rl : RV;
          if constexpr (BF16) {
            const uint32_t* vp = reinterpret_cast<const uint32_t*>(Lv + bb * VROW + rv * 2);
            const uint32_t v01 = vp[0], v23 = vp[1];
            vv[0] = bf2f(v01 & 0xFFFFu); vv[1] = bf2f(v01 >> 16);
            vv[2] = bf2f(v23 & 0xFFFFu); vv[3] = bf2f(v23 >> 16);
          } else {
            const f32x4 x = *reinterpret_cast<const f32x4*>(Lv + bb * VROW + rv * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[i] = x[i];
          }
          f32x4 dt, ot;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dt[i] = be * (vv[i] - al * uk[q][i]);            // eq. (8) delta_t
            ot[i] = fmaf(dt[i], kq, al * uq[q][i]);          // eq. (8) o_t
          }
          if (bb < nb && gr < DV) {
            const size_t bo = size_t(beam_of(c0 + bb)) * DV + gr;
            *reinterpret_cast<f32x4*>(dbase + bo) = dt;
            *reinterpret_cast<f32x4*>(obase + bo) = ot;
          }
        }
      } else if (grow0 < DV && valid) {
        // accumulator register i of this lane = physical row row0 + i of beam b
        const float* s = sc + m * SCN;
        const float kq = s[0];
        const float al = Lab[m], be = Lab[32 + m];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float ajj = s[1 + j], cqj = s[1 + NJ + j], ckj = s[1 + 2 * NJ + j];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              accq[4 * q4 + i] = fmaf(dj[j][q4][i], cqj, ajj * accq[4 * q4 + i]);   // eq. (6)
              acck[4 * q4 + i] = fmaf(dj[j][q4][i], ckj, ajj * acck[4 * q4 + i]);   // eq. (7)
            }
          }
        }
        float vin[16];
        if constexpr (BF16) {
          const u32x4* vp = reinterpret_cast<const u32x4*>(Lv + m * VROW + row0 * 2);
          unpack8(vp[0], vin);
          unpack8(vp[1], vin + 8);
        } else {
          const f32x4* vp = reinterpret_cast<const f32x4*>(Lv + m * VROW + row0 * 4);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            for (int i = 0; i < 4; ++i) vin[4 * q4 + i] = vp[q4][i];
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 dt, ot;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * q4 + i;
            dt[i] = be * (vin[e] - al * acck[e]);              // eq. (8) delta_t
            ot[i] = fmaf(dt[i], kq, al * accq[e]);             // eq. (8) o_t
          }
          reinterpret_cast<f32x4*>(dbase + size_t(b) * DV + grow0)[q4] = dt;
          reinterpret_cast<f32x4*>(obase + size_t(b) * DV + grow0)[q4] = ot;
        }
      }
    }

    // ---- append: k_t rows to slots (t, b) of the chunk's beams (once per key head),
    // and alpha_t
    {
      if (key_writer && rb == 0)
        for (int u = tid; u < nb * UPQ; u += NT)
          *reinterpret_cast<u32x4*>(keyg + (kslot_t * a.W_max + beam_of(c0 + u / UPQ)) * C::QB + (u % UPQ) * 16) =
              *reinterpret_cast<const u32x4*>(Lk + (u / UPQ) * QROW + (u % UPQ) * 16);
      if (rb == 0 && tid < nb) a.gtr_alpha[slot_t * a.W_max + beam_of(c0 + tid)] = Lab[tid];
    }
    if (c + 1 < nch) stage_store((c + 1) & 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launchers

int launch_init(const InitArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  const int nkk = a.io == GDN_BF16 ? a.d_k / 16 : a.d_k / 8;
  const size_t n = size_t(a.R) * a.H * (dvp_of(a.d_v) / 32) * nkk * 64;
  size_t blocks = (n + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 16384 ? 16384 : blocks);
  hipLaunchKernelGGL(init_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a);
  return last_launch_error();
}

template <int DK, int DV, bool BF16>
static int launch_step_t(const StepArgs& a, hipStream_t s) {
  const int nrh = a.R * a.H;
  char* ws = static_cast<char*>(a.ws);
  StepK k{a.H, a.HK, a.W, a.W_max, a.T_max, a.t, nrh, a.q, a.k, a.v, a.alpha, a.beta, a.o,
          ws + a.L.s_frag, reinterpret_cast<float*>(ws + a.L.gtr_alpha),
          reinterpret_cast<float*>(ws + a.L.gtr_delta), ws + a.L.gtr_key,
          reinterpret_cast<const int32_t*>(ws + a.L.anc[a.t & 1]),
          reinterpret_cast<const int32_t*>(ws + a.L.order[a.t & 1]),
          a.stamps, uint32_t(a.stamp_records < 0xFFFFFFFFu ? a.stamp_records : 0xFFFFFFFFu)};
  // one workgroup per (request, head, block of d_v rows): S_ctx is read once and kept
  // in registers.  With timing events, the dispatch itself stamps its start and end
  // (nothing more is put on the stream)
  auto go = [&](auto tt) {
    constexpr int TT = decltype(tt)::value;
    using C = StepCfg<DK, DV, BF16, TT>;
    const long grid = (long(nrh) * C::NRB + 7) / 8 * 8;
    auto kern = step_kernel<DK, DV, BF16, TT>;
    if (a.ev0) hipExtLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), 0, s, a.ev0, a.ev1, 0, k);
    else hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), 0, s, k);
  };
  switch (a.t) {
    case 0: go(std::integral_constant<int, 0>{}); break;
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    default: go(std::integral_constant<int, 7>{}); break;
  }
  return last_launch_error();
}

int launch_step(const StepArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  const bool bf = a.io == GDN_BF16;
  if (a.d_k == 16 && a.d_v == 16) return bf ? launch_step_t<16, 16, true>(a, s) : launch_step_t<16, 16, false>(a, s);
  if (a.d_k == 128 && a.d_v == 128) return bf ? launch_step_t<128, 128, true>(a, s) : launch_step_t<128, 128, false>(a, s);
  if (a.d_k == 128 && a.d_v == 256) return bf ? launch_step_t<128, 256, true>(a, s) : launch_step_t<128, 256, false>(a, s);
  if (a.d_k == 256 && a.d_v == 256 && bf) return launch_step_t<256, 256, true>(a, s);
  if (a.d_k == 128 && a.d_v == 512) return bf ? launch_step_t<128, 512, true>(a, s) : launch_step_t<128, 512, false>(a, s);
  if (a.d_k == 256 && a.d_v == 512 && bf) return launch_step_t<256, 512, true>(a, s);
  return int(hipErrorInvalidValue);
}

}  // namespace gdn
