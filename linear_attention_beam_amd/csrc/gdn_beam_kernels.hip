// HIP kernels for large-beam Gated DeltaNet decoding on gfx950 (CDNA4).
//
// OneLA reading note (paper-archivist.com), sections 2.1-2.5: one shared state
// S_ctx per (request, head), append-only transition records (alpha, delta, k) in
// fixed slots, an ancestry index, and a fused shared-context step.  RecoGEM
// (conceptio mirror) section 4.3: exact top-K over a request's W x C candidates.
//
// Kernels
//   init_kernel      S_ctx -> MFMA fragment order in the workspace; clear beam state.
//   step_kernel      fused step: S_ctx [q|k] on MFMA (eqs. 6-7 initial terms), replay
//                    along the ancestor records (eqs. 6-7), eq. (8), record append.
//   zsum_kernel      z_b = sum_h o_b; resets the per-request selection state.
//   wout_t_kernel    codebook transpose Wout[d_v,V] -> [V,d_v] (MFMA operand order).
//   logits_kernel    logits = z Wout on MFMA, stored [V][W_t]; online log-sum-exp parts.
//   lse_kernel       combines the parts into logsumexp per beam.
//   hist_kernel      first radix pass over every candidate key, 2048 digits spread over
//                    the request's exact key range (one histogram per block).
//   digit_kernel     sums a request's histograms and picks the boundary digit.
//   compact_kernel   keys above the boundary digit -> winners; keys inside it -> kept.
//   finalize_kernel  finishes the radix select on the kept keys, breaks ties by flat
//                    index, sorts the winners, writes the top-W, and remaps ancestry,
//                    SID prefixes and scores (eq. 9).
//   prefill_kernel   eq. (3) over each request's prompt (the state S_ctx).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "gdn_layout.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t f2bf(float x) {       // round to nearest even
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// 8 consecutive bf16 held in a u32x4 -> 8 floats
__device__ __forceinline__ void unpack8(const u32x4& p, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(p[i] << 16);
    f[2 * i + 1] = __uint_as_float(p[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ u32x4 pack8(const uint32_t* b) {
  u32x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = b[2 * i] | (b[2 * i + 1] << 16);
  return p;
}

// order-preserving key: larger float -> larger key; -0 is folded into +0 first
__device__ __forceinline__ uint32_t f2key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// the candidate score, evaluated identically wherever it is needed
__device__ __forceinline__ float cand_score(float cum, float logit, float lse) {
  return cum + (logit - lse);
}

__device__ __forceinline__ int xcd_work_id() {
  // consecutive blocks are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of work so the workgroups of one (request, head) share an L2
  const int n = gridDim.x;          // launched as a multiple of 8
  const int b = blockIdx.x;
  return (b & 7) * (n >> 3) + (b >> 3);
}

// MFMA row m of a 32-row block holds physical row 16*((m/4)%2) + 4*(m/8) + m%4, so
// that in the 32x32 accumulator lane half hf owns rows [16 hf, 16 hf + 16) in order.
__device__ __forceinline__ int frag_row(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// ---------------------------------------------------------------- init

// S_frag per (r,h): bf16 io: blocks (rb, kk, part) of 64 lanes x 8 bf16,
//   lane l -> S[32 rb + frag_row(l%32)][d_k/2*(l/32) + 8 kk + i], part 0 = hi, 1 = lo.
// f32 io: blocks (rb, kk4) of 64 lanes x 4 f32, lane l -> S[..][d_k/2*(l/32) + 4 kk4 + i].
__global__ void init_kernel(InitArgs a) {
  const int rh = blockIdx.x;
  const int r = rh / a.H, h = rh % a.H;
  const int dk = a.d_k, dv = a.d_v, dvp = dvp_of(dv), nrb = dvp / 32;
  char* ws = static_cast<char*>(a.ws);
  const float* S = a.S_ctx + size_t(rh) * dv * dk;
  u32x4* dst = reinterpret_cast<u32x4*>(ws + a.L.s_frag + size_t(rh) * 4 * dvp * dk);
  if (a.io == GDN_BF16) {
    const int nkk = dk / 16;
    const int nchunk = nrb * nkk * 2 * 64;
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
      const int lane = c & 63, blk = c >> 6;
      const int part = blk & 1, kk = (blk >> 1) % nkk, rb = (blk >> 1) / nkk;
      const int row = 32 * rb + frag_row(lane & 31);
      const int k0 = (dk / 2) * (lane >> 5) + 8 * kk;
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = row < dv ? S[size_t(row) * dk + k0 + i] : 0.0f;
        const uint32_t hi = f2bf(x);
        b[i] = part == 0 ? hi : f2bf(x - bf2f(hi));
      }
      dst[c] = pack8(b);
    }
  } else {
    const int nkk4 = dk / 8;
    const int nchunk = nrb * nkk4 * 64;
    for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
      const int lane = c & 63, blk = c >> 6;
      const int kk4 = blk % nkk4, rb = blk / nkk4;
      const int row = 32 * rb + frag_row(lane & 31);
      const int k0 = (dk / 2) * (lane >> 5) + 4 * kk4;
      f32x4 f;
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = row < dv ? S[size_t(row) * dk + k0 + i] : 0.0f;
      reinterpret_cast<f32x4*>(dst)[c] = f;
    }
  }
  if (h == 0) {  // beam state of request r: cumulative scores 0, empty ancestry
    float* cum = reinterpret_cast<float*>(ws + a.L.cum[0]) + size_t(r) * a.W_max;
    int32_t* anc = reinterpret_cast<int32_t*>(ws + a.L.anc[0]) + size_t(r) * a.W_max * a.T_max;
    int32_t* tok = reinterpret_cast<int32_t*>(ws + a.L.tok[0]) + size_t(r) * a.W_max * a.T_max;
    for (int i = threadIdx.x; i < a.W_max; i += blockDim.x) cum[i] = 0.0f;
    for (int i = threadIdx.x; i < a.W_max * a.T_max; i += blockDim.x) anc[i] = tok[i] = 0;
  }
  if (rh == 0 && threadIdx.x < 64)
    reinterpret_cast<int32_t*>(ws + a.L.status)[threadIdx.x] = 0;
}

// ---------------------------------------------------------------- step

struct StepK {
  int H, W, W_max, T_max, t, nrh;
  const void *q, *k, *v;
  const float *alpha, *beta;
  float* o;
  const char* s_frag;
  float* gtr_alpha;
  float* gtr_delta;
  void* gtr_key;
  const int32_t* anc;
};

// Sizes of the fused step for head dims (DK, DV) and io dtype.
template <int DK, int DV, bool BF16>
struct StepCfg {
  static constexpr int DVP = DV < 32 ? 32 : DV;
  static constexpr int NW = DVP / 32;            // one wave per 32-row block of d_v
  static constexpr int NT = NW * 64;
  static constexpr int E = BF16 ? 2 : 4;         // bytes per io element
  static constexpr int QB = DK * E;              // bytes of one q / k row
  static constexpr int VB = DV * E;              // bytes of one v row
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
template <int DK, int DV, bool BF16, int TT>
__global__ void __launch_bounds__((StepCfg<DK, DV, BF16>::NT), 2) step_kernel(StepK a) {
  using C = StepCfg<DK, DV, BF16>;
  constexpr int NT = C::NT, QROW = C::QROW, VROW = C::VROW, TPB = C::TPB;
  constexpr int UPQ = C::QB / 16, UPV = C::VB / 16;      // 16-byte units per row
  constexpr int NJ = TT;                                 // ancestor records replayed
  constexpr int NJ1 = NJ > 0 ? NJ : 1;
  constexpr int HK = DK / 2;
  constexpr int SCN = 1 + 3 * NJ;                        // kq, alpha_j, cq_j, ck_j
  __shared__ __align__(16) unsigned char lds[2 * C::SLOT + 32 * SCN * 4];
  float* sc = reinterpret_cast<float*>(lds + 2 * C::SLOT);

  const int rh = xcd_work_id();
  if (rh >= a.nrh) return;                                // whole block, before any barrier
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = lane & 31, hf = lane >> 5;
  const int W = a.W, r = rh / a.H;
  const int nch = (W + 31) >> 5;
  const size_t slot_t = size_t(rh) * a.T_max + TT;       // (r,h,t) row of the record pool
  const unsigned char* qg = static_cast<const unsigned char*>(a.q);
  const unsigned char* kg = static_cast<const unsigned char*>(a.k);
  const unsigned char* vg = static_cast<const unsigned char*>(a.v);
  unsigned char* keyg = static_cast<unsigned char*>(a.gtr_key);

  // this wave's block of S_ctx as A fragments (layout written by init_kernel)
  constexpr int NA = BF16 ? 2 * (DK / 16) : DK / 8;
  u32x4 afr[NA];
  {
    const u32x4* fr = reinterpret_cast<const u32x4*>(a.s_frag + size_t(rh) * 4 * C::DVP * DK);
#pragma unroll
    for (int i = 0; i < NA; ++i) afr[i] = fr[(w * NA + i) * 64 + lane];
  }

  // ---- staging of one chunk: registers <- global (contiguous), LDS <- registers
  u32x4 sq[C::QU], sk[C::QU], sv[C::VU];
  float sab = 0.0f;
  constexpr int NAI = (32 * NJ1 + NT - 1) / NT;
  int sanc[NAI];
  auto stage_load = [&](int c) {
    const int c0 = c * 32, nb = min(32, W - c0);
    const size_t base = size_t(rh) * W + c0;
#pragma unroll
    for (int i = 0; i < C::QU; ++i) {
      const int u = tid + i * NT;
      if (u / UPQ < nb) {
        sq[i] = *reinterpret_cast<const u32x4*>(qg + base * C::QB + size_t(u) * 16);
        sk[i] = *reinterpret_cast<const u32x4*>(kg + base * C::QB + size_t(u) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
      const int u = tid + i * NT;
      if (u / UPV < nb) sv[i] = *reinterpret_cast<const u32x4*>(vg + base * C::VB + size_t(u) * 16);
    }
    if (tid < 64 && (tid & 31) < nb) sab = tid < 32 ? a.alpha[base + tid] : a.beta[base + tid - 32];
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      const int e = tid + i * NT, bb = e / NJ1, j = e % NJ1;
      if (NJ > 0 && e < 32 * NJ && bb < nb) sanc[i] = a.anc[(size_t(r) * a.W_max + c0 + bb) * a.T_max + j];
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
    const int bm = tid / TPB, sg = tid % TPB;             // dot-phase role
    constexpr int SV = C::SEGB / 16;
    u32x4 kj[NJ1][SV];
    float aj[NJ1];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const size_t rec = (size_t(rh) * a.T_max + j) * a.W_max + (bm < nb ? Lan[bm * kMaxT + j] : 0);
      aj[j] = a.gtr_alpha[rec];
#pragma unroll
      for (int i = 0; i < SV; ++i)
        kj[j][i] = *reinterpret_cast<const u32x4*>(keyg + rec * C::QB + sg * C::SEGB + 16 * i);
    }
    const bool valid = m < nb;
    const int b = c0 + m;
    const int row0 = 32 * w + 16 * hf;
    const int rowl = min(row0, DV - 16);                 // in range (rows >= DV unused)
    f32x4 dj[NJ1][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const size_t rec = (size_t(rh) * a.T_max + j) * a.W_max + (valid ? Lan[m * kMaxT + j] : 0);
      const f32x4* dp = reinterpret_cast<const f32x4*>(a.gtr_delta + rec * DV + rowl);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) dj[j][q4] = dp[q4];
    }
    if (c + 1 < nch) stage_load(c + 1);                  // in flight until the end of the chunk

    // ---- dots: TPB threads per beam, SEGB bytes of d_k each
    {
      u32x4 xq[SV], xk[SV];
#pragma unroll
      for (int i = 0; i < SV; ++i) {
        xq[i] = *reinterpret_cast<const u32x4*>(Lq + bm * QROW + sg * C::SEGB + 16 * i);
        xk[i] = *reinterpret_cast<const u32x4*>(Lk + bm * QROW + sg * C::SEGB + 16 * i);
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

    // ---- this wave's row block for the chunk's 32 beams (lane: beam m, rows half hf)
    f32x16 accq = {}, acck = {};
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

    {
      // accumulator register i of this lane = physical row row0 + i of beam b
      if (row0 < DV && valid) {
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
        f32x4* dout = reinterpret_cast<f32x4*>(a.gtr_delta + (slot_t * a.W_max + b) * DV + row0);
        f32x4* oout = reinterpret_cast<f32x4*>(a.o + (size_t(rh) * W + b) * DV + row0);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 dt, ot;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * q4 + i;
            dt[i] = be * (vin[e] - al * acck[e]);              // eq. (8) delta_t
            ot[i] = fmaf(dt[i], kq, al * accq[e]);             // eq. (8) o_t
          }
          dout[q4] = dt;
          oout[q4] = ot;
        }
      }
    }

    // ---- append: k_t rows (contiguous slots c0..c0+nb-1) and alpha_t
    {
      unsigned char* dst = keyg + (slot_t * a.W_max + c0) * C::QB;
      for (int u = tid; u < nb * UPQ; u += NT)
        *reinterpret_cast<u32x4*>(dst + size_t(u) * 16) =
            *reinterpret_cast<const u32x4*>(Lk + (u / UPQ) * QROW + (u % UPQ) * 16);
      if (tid < nb) a.gtr_alpha[slot_t * a.W_max + c0 + tid] = Lab[tid];
    }
    if (c + 1 < nch) stage_store((c + 1) & 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- select: z, Wout^T

// z[r,b,:] = sum_h o[r,h,b,:]; thread 0.. also reset the selection state of the request.
__global__ void zsum_kernel(const float* __restrict__ o, float* __restrict__ z, int H, int W,
                           int W_max, int d_v, int K, uint32_t* hist, SelState* sel, int R) {
  const int r = blockIdx.y;
  const int n4 = W * d_v / 4;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
    f32x4 s = {};
    for (int h = 0; h < H; ++h)
      s += reinterpret_cast<const f32x4*>(o + (size_t(r) * H + h) * W * d_v)[i];
    const int b = (4 * i) / d_v, c = (4 * i) % d_v;
    *reinterpret_cast<f32x4*>(z + (size_t(r) * W_max + b) * d_v + c) = s;
  }
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) {
      SelState st{};
      st.kmax = 0u;
      st.kmin = 0xFFFFFFFFu;
      st.need = uint32_t(K);
      sel[r] = st;
    }
  }
}

template <typename WT>
__global__ void wout_t_kernel(const WT* __restrict__ w, WT* __restrict__ wt, int d_v, int V) {
  __shared__ WT tile[32][33];
  const int c0 = blockIdx.x * 32, i0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 256 threads: 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int i = i0 + y, c = c0 + tx;
    tile[y][tx] = (i < d_v && c < V) ? w[size_t(i) * V + c] : WT{};
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, i = i0 + tx;
    if (c < V && i < d_v) wt[size_t(c) * d_v + i] = tile[tx][y];
  }
}

// ---------------------------------------------------------------- select: logits

struct LogitsK {
  int W, W_max, V, nchunk, nvg;
  const float* z;       // [R,W_max,DV]
  const void* woutT;    // [V,DV]
  float* logits;        // per request [V][W]
  float4* lse_part;     // [R,W_max,nvg]: max, sum of exp(x - max), min
  size_t logits_stride; // elements per request
};

// One wave: 32 beams x kCodesPerWave codes.  A = Wout^T rows (codes), B = z columns
// (beams), so lane l keeps beam l%32 and can fold its 16 codes per tile into a running
// log-sum-exp without cross-lane traffic.  bf16 codebook: z is split into three bf16
// terms (hi, mid, lo), exact products against the bf16 codebook, fp32 accumulation.
template <int DV, bool WBF16>
__global__ void __launch_bounds__(256) logits_kernel(LogitsK a) {
  constexpr int HV = DV / 2;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int per_req = a.nchunk * a.nvg;
  const int r = blockIdx.y;
  if (gw >= per_req) return;
  const int chunk = gw / a.nvg, vg = gw % a.nvg;
  const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
  const int b = chunk * 32 + m;
  const bool bvalid = b < a.W;
  const float* zr = a.z + (size_t(r) * a.W_max + (bvalid ? b : 0)) * DV + HV * hf;
  float* lg = a.logits + size_t(r) * a.logits_stride;

  float mrun = -INFINITY, srun = 0.0f, nrun = INFINITY;
  const int code_lo = vg * kCodesPerWave;
  const int code_hi = min(a.V, code_lo + kCodesPerWave);

  if constexpr (WBF16) {
    constexpr int KS = DV / 16;
    u32x4 zh[KS], zm[KS], zl[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint32_t bh[8], bm[8], bl[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = bvalid ? zr[8 * kk + i] : 0.0f;
        bh[i] = f2bf(x);
        const float r1 = x - bf2f(bh[i]);
        bm[i] = f2bf(r1);
        bl[i] = f2bf(r1 - bf2f(bm[i]));
      }
      zh[kk] = pack8(bh); zm[kk] = pack8(bm); zl[kk] = pack8(bl);
    }
    const u32x4* wt = static_cast<const u32x4*>(a.woutT);
    for (int c0 = code_lo; c0 < code_hi; c0 += 32) {
      const int code = c0 + m;
      const bool cv = code < a.V;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 w = __builtin_bit_cast(bf16x8, cv ? wt[(size_t(code) * DV + HV * hf) / 8 + kk] : u32x4{});
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, __builtin_bit_cast(bf16x8, zl[kk]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, __builtin_bit_cast(bf16x8, zm[kk]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, __builtin_bit_cast(bf16x8, zh[kk]), acc, 0, 0, 0);
      }
      // acc[i]: code c0 + 8*(i/4) + 4*hf + i%4, beam b
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cc = c0 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (cc < a.V) {
          tmax = fmaxf(tmax, acc[i]);
          nrun = fminf(nrun, acc[i]);
          if (bvalid) lg[size_t(cc) * a.W + b] = acc[i];
        }
      }
      if (tmax > mrun) { srun = (mrun == -INFINITY) ? 0.0f : srun * expf(mrun - tmax); mrun = tmax; }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cc = c0 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (cc < a.V) srun += expf(acc[i] - mrun);
      }
    }
  } else {
    const float* wt = static_cast<const float*>(a.woutT);
    float zf[HV];
#pragma unroll
    for (int i = 0; i < HV; ++i) zf[i] = bvalid ? zr[i] : 0.0f;
    for (int c0 = code_lo; c0 < code_hi; c0 += 32) {
      const int code = c0 + m;
      const bool cv = code < a.V;
      const float* wr = wt + size_t(cv ? code : 0) * DV + HV * hf;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < HV; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(cv ? wr[kk] : 0.0f, zf[kk], acc, 0, 0, 0);
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cc = c0 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (cc < a.V) {
          tmax = fmaxf(tmax, acc[i]);
          nrun = fminf(nrun, acc[i]);
          if (bvalid) lg[size_t(cc) * a.W + b] = acc[i];
        }
      }
      if (tmax > mrun) { srun = (mrun == -INFINITY) ? 0.0f : srun * expf(mrun - tmax); mrun = tmax; }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cc = c0 + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (cc < a.V) srun += expf(acc[i] - mrun);
      }
    }
  }
  // merge the two lane halves of beam b
  const float mo = __shfl_xor(mrun, 32), so = __shfl_xor(srun, 32);
  const float mm = fmaxf(mrun, mo);
  float ss = 0.0f;
  if (mrun != -INFINITY) ss += srun * expf(mrun - mm);
  if (mo != -INFINITY) ss += so * expf(mo - mm);
  const float nn = fminf(nrun, __shfl_xor(nrun, 32));
  if (hf == 0 && bvalid) a.lse_part[(size_t(r) * a.W_max + b) * a.nvg + vg] = make_float4(mm, ss, nn, 0.0f);
}

// logsumexp per beam, and the request's exact key range: the score is monotone in
// the logit, so the row's largest / smallest logits give its largest / smallest keys.
__global__ void lse_kernel(const float4* __restrict__ part, float* __restrict__ lse,
                           const float* __restrict__ cum, SelState* sel, int W, int W_max,
                           int nvg, int R) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= R * W) return;
  const int r = i / W, b = i % W;
  const float4* p = part + (size_t(r) * W_max + b) * nvg;
  float mm = -INFINITY, mn = INFINITY;
  for (int g = 0; g < nvg; ++g) {
    mm = fmaxf(mm, p[g].x);
    mn = fminf(mn, p[g].z);
  }
  float s = 0.0f;
  for (int g = 0; g < nvg; ++g)
    if (p[g].x != -INFINITY) s += p[g].y * expf(p[g].x - mm);
  const float l = mm + logf(s);
  lse[size_t(r) * W_max + b] = l;
  const float c = cum[size_t(r) * W_max + b];
  atomicMax(&sel[r].kmax, f2key(cand_score(c, mm, l)));
  atomicMin(&sel[r].kmin, f2key(cand_score(c, mn, l)));
}

// ---------------------------------------------------------------- select: radix passes

struct SelK {
  int W, W_max, V, K, nblk, T_max, t;
  size_t logits_stride;
  const float* logits;   // per request [V][W]
  const float* lse;      // [R,W_max]
  const float* cum;      // [R,W_max] of step t
  uint32_t* hist;        // [R,kSelBlocksMax,kHistBins], one histogram per block
  SelState* sel;
  uint64_t* winners;     // [R,W_max]: key << 32 | flat, keys above the boundary digit
  uint32_t* cand;        // [R,logits_stride]: flat indices inside the boundary digit
};

__device__ __forceinline__ uint32_t cand_key(const float* lg, const float* lse, const float* cum,
                                             int W, int b, int c) {
  return f2key(cand_score(cum[b], lg[size_t(c) * W + b], lse[b]));
}

// Candidates of one request are its [V][W] logits; block `blk` covers codes [c0, c1).
// With W >= 256 a thread owns beams tid + 256 i for every code; with W < 256 it owns
// beam tid % W for every (256 / W)-th code.  Loads are issued eight at a time.
template <typename F>
__device__ __forceinline__ void for_each_candidate(const SelK& a, int r, int blk, F&& f) {
  constexpr int U = 8;
  const int tid = threadIdx.x;
  const int W = a.W;
  const int cpb = (a.V + a.nblk - 1) / a.nblk;
  const int c0 = blk * cpb, c1 = min(a.V, c0 + cpb);
  const float* lg = a.logits + size_t(r) * a.logits_stride;
  const float* lse = a.lse + size_t(r) * a.W_max;
  const float* cum = a.cum + size_t(r) * a.W_max;
  int b0, bstep, cs, cstep;
  if (W >= 256) {
    b0 = tid; bstep = 256; cs = c0; cstep = 1;
  } else {
    const int G = 256 / W;
    if (tid >= G * W) return;
    b0 = tid % W; bstep = W; cs = c0 + tid / W; cstep = G;
  }
  for (int b = b0; b < W; b += bstep) {
    const float cb = cum[b], lb = lse[b];
    int c = cs;
    for (; c + (U - 1) * cstep < c1; c += U * cstep) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = lg[size_t(c + u * cstep) * W + b];
#pragma unroll
      for (int u = 0; u < U; ++u) f(f2key(cand_score(cb, x[u], lb)), b, c + u * cstep);
    }
    for (; c < c1; c += cstep) f(f2key(cand_score(cb, lg[size_t(c) * W + b], lb)), b, c);
  }
}

// First radix pass over all candidates of a request.  The range [kmin, kmax] (exact
// key bounds) is split into 2048 digits of width 2^shift; each block stores its own
// histogram (plain stores: the next kernel reads them, so no fence is needed).
__device__ __forceinline__ int first_shift(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  const int bits = span ? 32 - __clz(span) : 0;
  return bits > 11 ? bits - 11 : 0;
}

__global__ void __launch_bounds__(256) hist_kernel(SelK a) {
  __shared__ uint32_t h[kHistBins];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const SelState* st = a.sel + r;
  const uint32_t lo = st->kmin, hi = st->kmax;
  const int shift = first_shift(lo, hi);
  for (int i = tid; i < kHistBins; i += 256) h[i] = 0;
  __syncthreads();
  for_each_candidate(a, r, blockIdx.x, [&](uint32_t key, int, int) {
    if (key >= lo && key <= hi) atomicAdd(&h[(key - lo) >> shift], 1u);
  });
  __syncthreads();
  uint32_t* gh = a.hist + (size_t(r) * kSelBlocksMax + blockIdx.x) * kHistBins;
  for (int i = tid; i < kHistBins; i += 256) gh[i] = h[i];
}

// One block per request: sum the block histograms and pick the digit d holding the
// K-th largest key: keys above d are winners, keys inside d go on to the finish.
__global__ void __launch_bounds__(1024) digit_kernel(SelK a) {
  __shared__ uint32_t h[kHistBins];
  __shared__ uint32_t scan[256];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  SelState* st = a.sel + r;
  const uint32_t lo = st->kmin, hi = st->kmax;
  const int shift = first_shift(lo, hi);
  const uint32_t* rh = a.hist + size_t(r) * kSelBlocksMax * kHistBins;
  for (int d = tid; d < kHistBins; d += 1024) {
    uint32_t c = 0;
#pragma unroll 8
    for (int bk = 0; bk < a.nblk; ++bk) c += rh[size_t(bk) * kHistBins + d];
    h[d] = c;
  }
  __syncthreads();
  // digit scan on the first 256 threads (all threads take part in the barriers)
  constexpr int PER = kHistBins / 256;
  const uint32_t need = uint32_t(a.K);
  const bool act = tid < 256;
  uint32_t cnt[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {          // thread tid owns digits from the top down
    cnt[i] = act ? h[kHistBins - 1 - (tid * PER + i)] : 0u;
    tot += cnt[i];
  }
  if (act) scan[tid] = tot;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t x = (act && tid >= off) ? scan[tid - off] : 0u;
    __syncthreads();
    if (act) scan[tid] += x;
    __syncthreads();
  }
  if (!act) return;
  uint32_t above = scan[tid] - tot;
  if (above < need && need <= above + tot) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (above < need && need <= above + cnt[i]) {
        const uint32_t d = uint32_t(kHistBins - 1 - (tid * PER + i));
        const uint32_t nlo = lo + (d << shift);
        const uint64_t top = uint64_t(nlo) + (uint64_t(1) << shift) - 1;
        st->lo = nlo;
        st->hi = top < hi ? uint32_t(top) : hi;
        st->need = need - above;
        st->shift = shift == 0 ? -1 : (shift > 11 ? shift - 11 : 0);
      }
      above += cnt[i];
    }
  }
}

// Split the candidates by the boundary digit [lo, hi]: keys above it are winners,
// keys inside it are kept (flat index) for the finish kernel.
__global__ void __launch_bounds__(256) compact_kernel(SelK a) {
  const int r = blockIdx.y;
  SelState* st = a.sel + r;
  const uint32_t lo = st->lo, hi = st->hi;
  const size_t cap = size_t(a.V) * a.W;
  for_each_candidate(a, r, blockIdx.x, [&](uint32_t key, int b, int c) {
    if (key >= lo) {
      const uint32_t flat = uint32_t(b) * uint32_t(a.V) + uint32_t(c);
      if (key > hi) {
        const uint32_t i = atomicAdd(&st->n_win, 1u);
        if (i < uint32_t(a.W_max)) a.winners[size_t(r) * a.W_max + i] = (uint64_t(key) << 32) | flat;
      } else {
        const uint32_t i = atomicAdd(&st->n_cand, 1u);
        if (i < cap) a.cand[size_t(r) * a.logits_stride + i] = flat;
      }
    }
  });
}

struct FinK {
  int W, W_max, V, K, T_max, t;
  size_t logits_stride;
  const float* logits;
  const float* lse;
  const float* cum;        // step t
  float* cum_next;
  const int32_t* anc;      // step t
  int32_t* anc_next;
  const int32_t* tok;
  int32_t* tok_next;
  const SelState* sel;
  const uint64_t* winners;
  const uint32_t* cand;
  const int32_t *forced_parent, *forced_token;
  int32_t *parent, *token;
  float* score;
  int32_t* status;
};

// One 1024-thread block per request: finish the radix select inside the boundary
// digit (at most two more 11-bit passes over its candidates), keep the `need`
// smallest flat indices among keys equal to the threshold, sort the K winners by
// score descending then flat index ascending, write the top-W, and remap ancestry,
// SID prefixes and cumulative scores by eq. (9).
__global__ void __launch_bounds__(1024) finalize_kernel(FinK a) {
  __shared__ uint64_t s[kMaxW];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scan[1024];
  __shared__ uint32_t cnt, sh_lo, sh_hi, sh_need;
  __shared__ int sh_shift;
  const int r = blockIdx.x, tid = threadIdx.x;
  const SelState st = a.sel[r];
  const float* lg = a.logits + size_t(r) * a.logits_stride;
  const float* lse = a.lse + size_t(r) * a.W_max;
  const float* cum = a.cum + size_t(r) * a.W_max;
  const uint32_t* cand = a.cand + size_t(r) * a.logits_stride;
  const uint32_t n_cand = min(st.n_cand, uint32_t(a.V) * uint32_t(a.W));
  const uint32_t n_win = min(st.n_win, uint32_t(a.K));
  const uint32_t V = uint32_t(a.V);
  auto key_of = [&](uint32_t flat) {
    return cand_key(lg, lse, cum, a.W, int(flat / V), int(flat % V));
  };

  // radix passes inside [lo, hi] until a single key remains (theta = lo = hi)
  uint32_t lo = st.lo, hi = st.hi, need = st.need;
  int shift = st.shift;
  while (shift >= 0) {
    for (int i = tid; i < kHistBins; i += 1024) hist[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < n_cand; i += 1024) {
      const uint32_t key = key_of(cand[i]);
      if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
    }
    __syncthreads();
    const uint32_t c0 = hist[kHistBins - 1 - 2 * tid], c1 = hist[kHistBins - 2 - 2 * tid];
    scan[tid] = c0 + c1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const uint32_t x = tid >= off ? scan[tid - off] : 0u;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    uint32_t above = scan[tid] - (c0 + c1);
    for (int i = 0; i < 2; ++i) {
      const uint32_t ci = i ? c1 : c0;
      if (above < need && need <= above + ci) {
        const uint32_t d = uint32_t(kHistBins - 1 - (2 * tid + i));
        const uint32_t nlo = lo + (d << shift);
        const uint64_t top = uint64_t(nlo) + (uint64_t(1) << shift) - 1;
        sh_lo = nlo;
        sh_hi = top < hi ? uint32_t(top) : hi;
        sh_need = need - above;
        sh_shift = shift == 0 ? -1 : (shift > 11 ? shift - 11 : 0);
      }
      above += ci;
    }
    __syncthreads();
    lo = sh_lo; hi = sh_hi; need = sh_need; shift = sh_shift;
    __syncthreads();
  }
  const uint32_t theta = lo;

  // ties at theta: keep the `need` smallest flat indices (radix over the flat index)
  if (tid == 0) cnt = 0;
  __syncthreads();
  for (uint32_t i = tid; i < n_cand; i += 1024)
    if (key_of(cand[i]) == theta) atomicAdd(&cnt, 1u);
  __syncthreads();
  const uint32_t n_eq = cnt;
  uint32_t phi = 0xFFFFFFFFu;
  if (need < n_eq) {
    uint32_t pre = 0, nd = need;
    for (int sh = 24; sh >= 0; sh -= 8) {
      for (int i = tid; i < 256; i += 1024) hist[i] = 0;
      __syncthreads();
      const uint32_t himask = sh == 24 ? 0u : (0xFFFFFFFFu << (sh + 8));
      for (uint32_t i = tid; i < n_cand; i += 1024) {
        const uint32_t f = cand[i];
        if ((f & himask) == (pre & himask) && key_of(f) == theta) atomicAdd(&hist[(f >> sh) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t below = 0;
        for (int d = 0; d < 256; ++d) {
          if (below < nd && nd <= below + hist[d]) {
            pre |= uint32_t(d) << sh;
            nd -= below;
            break;
          }
          below += hist[d];
        }
        sh_lo = pre;
        sh_need = nd;
      }
      __syncthreads();
      pre = sh_lo;
      nd = sh_need;
      __syncthreads();
    }
    phi = pre;
  }

  // gather the K winners
  if (tid == 0) cnt = 0;
  __syncthreads();
  for (uint32_t i = tid; i < n_win; i += 1024) {
    const uint32_t j = atomicAdd(&cnt, 1u);
    if (j < uint32_t(kMaxW)) s[j] = a.winners[size_t(r) * a.W_max + i];
  }
  for (uint32_t i = tid; i < n_cand; i += 1024) {
    const uint32_t f = cand[i];
    const uint32_t key = key_of(f);
    if (key > theta || (key == theta && f <= phi)) {
      const uint32_t j = atomicAdd(&cnt, 1u);
      if (j < uint32_t(kMaxW)) s[j] = (uint64_t(key) << 32) | f;
    }
  }
  __syncthreads();
  const uint32_t got = cnt;
  if (tid == 0 && got != uint32_t(a.K)) atomicOr(a.status, 2);
  // pad to a power of two with the smallest entry, then sort descending by
  // (key, ~flat): score descending, flat index ascending
  int n = 1;
  while (n < a.K) n <<= 1;
  for (int i = tid; i < n; i += 1024) {
    if (uint32_t(i) >= got) s[i] = 0;
    else s[i] = (s[i] & 0xFFFFFFFF00000000ull) | uint64_t(0xFFFFFFFFu - uint32_t(s[i]));
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n; i += 1024) {
        const int p = i ^ j;
        if (p > i) {
          const bool desc = (i & k) == 0;
          const uint64_t x = s[i], y = s[p];
          if (desc ? (x < y) : (x > y)) { s[i] = y; s[p] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < a.K; i += 1024) {
    const uint64_t e = s[i];
    const uint32_t flat = 0xFFFFFFFFu - uint32_t(e);
    int p = int(flat / V), c = int(flat % V);
    if (uint32_t(i) >= got || p >= a.W) {   // only if fewer than K were gathered (flagged)
      p = 0;
      c = 0;
    }
    const float sc = key2f(uint32_t(e >> 32));
    const size_t o = size_t(r) * a.K + i;
    a.parent[o] = p;
    a.token[o] = c;
    a.score[o] = sc;
    int fp = p, fc = c;
    float fs = sc;
    if (a.forced_parent) {
      fp = a.forced_parent[o];
      fc = a.forced_token[o];
      if (fp < 0 || fp >= a.W || fc < 0 || fc >= a.V) {
        atomicOr(a.status, 1);
        fp = fp < 0 ? 0 : (fp >= a.W ? a.W - 1 : fp);
        fc = fc < 0 ? 0 : (fc >= a.V ? a.V - 1 : fc);
      }
      fs = cand_score(cum[fp], lg[size_t(fc) * a.W + fp], lse[fp]) + 0.0f;
    }
    // eq. (9): the child copies its parent's ancestry and appends the parent's slot
    const int32_t* ap = a.anc + (size_t(r) * a.W_max + fp) * a.T_max;
    const int32_t* tp = a.tok + (size_t(r) * a.W_max + fp) * a.T_max;
    int32_t* an = a.anc_next + (size_t(r) * a.W_max + i) * a.T_max;
    int32_t* tn = a.tok_next + (size_t(r) * a.W_max + i) * a.T_max;
    for (int j = 0; j < a.T_max; ++j) {
      an[j] = j < a.t ? ap[j] : (j == a.t ? fp : 0);
      tn[j] = j < a.t ? tp[j] : (j == a.t ? fc : 0);
    }
    a.cum_next[size_t(r) * a.W_max + i] = fs;
  }
}

// ---------------------------------------------------------------- prefill (eq. 3)

// One workgroup per (request, head); thread (row, half) holds S[row][half*DK/2 ..] in
// registers.  Each token: u = S k (row dot, reduced over the row's lanes),
// S <- alpha S + beta (v - alpha u) k^T.
template <int DK, int DV>
__global__ void __launch_bounds__(DV < 32 ? 256 : 2 * DV) prefill_kernel(PrefillArgs a) {
  constexpr int TPR = DV < 32 ? 256 / DV : 2;        // lanes per row
  constexpr int COLS = DK / TPR;
  const int rh = blockIdx.x, r = rh / a.H, h = rh % a.H;
  const int row = threadIdx.x / TPR, cp = threadIdx.x % TPR;
  int beg = a.offsets[r], end = a.offsets[r + 1];
  beg = beg < 0 ? 0 : (beg > a.N ? int(a.N) : beg);
  end = end < beg ? beg : (end > a.N ? int(a.N) : end);
  float S[COLS];
#pragma unroll
  for (int c = 0; c < COLS; ++c) S[c] = 0.0f;
  float kc[COLS];
  float vn = 0.0f, an = 0.0f, bn = 0.0f;
  auto load = [&](int i, float* kk, float& vv, float& aa, float& bb) {
    const float* kp = a.k + (size_t(i) * a.H + h) * DK + cp * COLS;
#pragma unroll
    for (int c = 0; c < COLS; ++c) kk[c] = kp[c];
    vv = a.v[(size_t(i) * a.H + h) * DV + row];
    aa = a.alpha[size_t(i) * a.H + h];
    bb = a.beta[size_t(i) * a.H + h];
  };
  if (beg < end) load(beg, kc, vn, an, bn);
  for (int i = beg; i < end; ++i) {
    float kcur[COLS];
#pragma unroll
    for (int c = 0; c < COLS; ++c) kcur[c] = kc[c];
    const float vv = vn, aa = an, bb = bn;
    if (i + 1 < end) load(i + 1, kc, vn, an, bn);
    float u = 0.0f;
#pragma unroll
    for (int c = 0; c < COLS; ++c) u = fmaf(S[c], kcur[c], u);
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) u += __shfl_xor(u, off);
    const float d = bb * (vv - aa * u);
#pragma unroll
    for (int c = 0; c < COLS; ++c) S[c] = fmaf(d, kcur[c], aa * S[c]);
  }
  float* out = a.S_out + ((size_t(rh) * DV + row) * DK) + cp * COLS;
#pragma unroll
  for (int c = 0; c < COLS; ++c) out[c] = S[c];
}

// ---------------------------------------------------------------- launchers

static int last_launch_error() { return int(hipGetLastError()); }

int launch_init(const InitArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(init_kernel, dim3(a.R * a.H), dim3(256), 0, s, a);
  return last_launch_error();
}

template <int DK, int DV, bool BF16>
static int launch_step_t(const StepArgs& a, hipStream_t s) {
  constexpr int NT = StepCfg<DK, DV, BF16>::NT;
  const int nrh = a.R * a.H;
  // one workgroup per (request, head): S_ctx is read once and kept in registers
  const long grid = (long(nrh) + 7) / 8 * 8;
  char* ws = static_cast<char*>(a.ws);
  StepK k{a.H, a.W, a.W_max, a.T_max, a.t, nrh, a.q, a.k, a.v, a.alpha, a.beta, a.o,
          ws + a.L.s_frag, reinterpret_cast<float*>(ws + a.L.gtr_alpha),
          reinterpret_cast<float*>(ws + a.L.gtr_delta), ws + a.L.gtr_key,
          reinterpret_cast<const int32_t*>(ws + a.L.anc[a.t & 1])};
  switch (a.t) {
    case 0: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 0>), dim3(grid), dim3(NT), 0, s, k); break;
    case 1: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 1>), dim3(grid), dim3(NT), 0, s, k); break;
    case 2: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 2>), dim3(grid), dim3(NT), 0, s, k); break;
    case 3: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 3>), dim3(grid), dim3(NT), 0, s, k); break;
    case 4: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 4>), dim3(grid), dim3(NT), 0, s, k); break;
    case 5: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 5>), dim3(grid), dim3(NT), 0, s, k); break;
    case 6: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 6>), dim3(grid), dim3(NT), 0, s, k); break;
    default: hipLaunchKernelGGL((step_kernel<DK, DV, BF16, 7>), dim3(grid), dim3(NT), 0, s, k); break;
  }
  return last_launch_error();
}

int launch_step(const StepArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  const bool bf = a.io == GDN_BF16;
  if (a.d_k == 16 && a.d_v == 16) return bf ? launch_step_t<16, 16, true>(a, s) : launch_step_t<16, 16, false>(a, s);
  if (a.d_k == 128 && a.d_v == 128) return bf ? launch_step_t<128, 128, true>(a, s) : launch_step_t<128, 128, false>(a, s);
  if (a.d_k == 128 && a.d_v == 256) return bf ? launch_step_t<128, 256, true>(a, s) : launch_step_t<128, 256, false>(a, s);
  return int(hipErrorInvalidValue);
}

template <int DV>
static int launch_logits_t(const SelectArgs& a, const LogitsK& k, hipStream_t s) {
  const int per_req = k.nchunk * k.nvg;
  dim3 grid((per_req + 3) / 4, a.R);
  if (a.wout_dtype == GDN_BF16)
    hipLaunchKernelGGL((logits_kernel<DV, true>), grid, dim3(256), 0, s, k);
  else
    hipLaunchKernelGGL((logits_kernel<DV, false>), grid, dim3(256), 0, s, k);
  return last_launch_error();
}

int launch_select(const SelectArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  char* ws = static_cast<char*>(a.ws);
  const Layout& L = a.L;
  const size_t stride = size_t(a.W_max) * size_t(a.V_max);   // per-request candidates
  const int par = a.t & 1;
  float* z = reinterpret_cast<float*>(ws + L.z);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.hist);
  SelState* sel = reinterpret_cast<SelState*>(ws + L.sel);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  float4* lse_part = reinterpret_cast<float4*>(ws + L.lse_part);
  float* lse = reinterpret_cast<float*>(ws + L.lse);
  uint64_t* winners = reinterpret_cast<uint64_t*>(ws + L.winners);
  uint32_t* cand = reinterpret_cast<uint32_t*>(ws + L.cand);
  float* cum = reinterpret_cast<float*>(ws + L.cum[par]);
  float* cum_next = reinterpret_cast<float*>(ws + L.cum[par ^ 1]);
  int32_t* anc = reinterpret_cast<int32_t*>(ws + L.anc[par]);
  int32_t* anc_next = reinterpret_cast<int32_t*>(ws + L.anc[par ^ 1]);
  int32_t* tok = reinterpret_cast<int32_t*>(ws + L.tok[par]);
  int32_t* tok_next = reinterpret_cast<int32_t*>(ws + L.tok[par ^ 1]);
  int32_t* status = reinterpret_cast<int32_t*>(ws + L.status);
  int err;

  {  // head sum, selection-state reset
    const int n4 = a.W * a.d_v / 4;
    int gx = (n4 + 255) / 256;
    gx = gx < 1 ? 1 : (gx > 1024 ? 1024 : gx);
    hipLaunchKernelGGL(zsum_kernel, dim3(gx, a.R), dim3(256), 0, s, a.o, z, a.H, a.W, a.W_max,
                       a.d_v, a.W_next, hist, sel, a.R);
    if ((err = last_launch_error())) return err;
  }
  {  // codebook transpose
    dim3 grid((a.V + 31) / 32, (a.d_v + 31) / 32);
    if (a.wout_dtype == GDN_BF16)
      hipLaunchKernelGGL((wout_t_kernel<uint16_t>), grid, dim3(256), 0, s,
                         static_cast<const uint16_t*>(a.Wout), reinterpret_cast<uint16_t*>(ws + L.woutT), a.d_v, a.V);
    else
      hipLaunchKernelGGL((wout_t_kernel<float>), grid, dim3(256), 0, s,
                         static_cast<const float*>(a.Wout), reinterpret_cast<float*>(ws + L.woutT), a.d_v, a.V);
    if ((err = last_launch_error())) return err;
  }
  const int nvg = n_vgroups(a.V);
  {  // logits and log-sum-exp parts
    LogitsK k{a.W, a.W_max, a.V, (a.W + 31) / 32, nvg, z, ws + L.woutT, logits, lse_part, stride};
    if (a.d_v == 16) err = launch_logits_t<16>(a, k, s);
    else if (a.d_v == 128) err = launch_logits_t<128>(a, k, s);
    else if (a.d_v == 256) err = launch_logits_t<256>(a, k, s);
    else return int(hipErrorInvalidValue);
    if (err) return err;
  }
  {
    const int n = a.R * a.W;
    hipLaunchKernelGGL(lse_kernel, dim3((n + 255) / 256), dim3(256), 0, s, lse_part, lse, cum,
                       sel, a.W, a.W_max, nvg, a.R);
    if ((err = last_launch_error())) return err;
  }
  {  // exact top-W_next: three radix passes, then gather
    const size_t N = size_t(a.V) * a.W;
    long nblk = long((N + kSelPerBlock - 1) / kSelPerBlock);
    nblk = nblk < 1 ? 1 : (nblk > kSelBlocksMax ? kSelBlocksMax : nblk);
    nblk = nblk > a.V ? a.V : nblk;                      // every block owns >= 1 code
    SelK k{a.W, a.W_max, a.V, a.W_next, int(nblk), a.T_max, a.t, stride, logits, lse, cum,
           hist, sel, winners, cand};
    dim3 grid(nblk, a.R);
    hipLaunchKernelGGL(hist_kernel, grid, dim3(256), 0, s, k);
    hipLaunchKernelGGL(digit_kernel, dim3(a.R), dim3(1024), 0, s, k);
    hipLaunchKernelGGL(compact_kernel, grid, dim3(256), 0, s, k);
    if ((err = last_launch_error())) return err;
  }
  {  // order, write the top-W, remap ancestry (eq. 9)
    FinK k{a.W, a.W_max, a.V, a.W_next, a.T_max, a.t, stride, logits, lse, cum, cum_next,
           anc, anc_next, tok, tok_next, sel, winners, cand, a.forced_parent, a.forced_token,
           a.parent, a.token, a.score, status};
    hipLaunchKernelGGL(finalize_kernel, dim3(a.R), dim3(1024), 0, s, k);
    if ((err = last_launch_error())) return err;
  }
  return 0;
}

template <int DK, int DV>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  constexpr int threads = DV < 32 ? 256 : 2 * DV;
  hipLaunchKernelGGL((prefill_kernel<DK, DV>), dim3(a.R * a.H), dim3(threads), 0, s, a);
  return last_launch_error();
}

int launch_prefill(const PrefillArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  if (a.d_k == 16 && a.d_v == 16) return launch_prefill_t<16, 16>(a, s);
  if (a.d_k == 128 && a.d_v == 128) return launch_prefill_t<128, 128>(a, s);
  if (a.d_k == 128 && a.d_v == 256) return launch_prefill_t<128, 256>(a, s);
  return int(hipErrorInvalidValue);
}

int copy_d2d(void* dst, const void* src, size_t bytes, hipStream_t s) {
  return int(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
}

const char* hip_error_string(int err) { return hipGetErrorString(hipError_t(err)); }

}  // namespace gdn
