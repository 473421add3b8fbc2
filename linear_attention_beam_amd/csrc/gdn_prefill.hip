// Prefill: the shared state S_ctx of every (request, head) from its prompt by the Gated
// DeltaNet recurrence, eq. (3) of the OneLA reading note (paper-archivist.com), section 1.2.
//
// Two forms of the same recurrence:
//  * token-sequential (no workspace): one thread group per (request, head, row block)
//    applies eq. (3) token by token in fp32;
//  * chunked (with a workspace): the prompt is cut into 32-token chunks and each chunk is
//    applied at once.  With S_0 the state entering a chunk of tokens t = 0..n-1 and
//    g_t = a_0 ... a_t, unrolling eq. (3) gives the update vectors
//      d_t = b_t (v_t - g_t S_0 k_t - sum_{i<t} (g_t / g_i) (k_i . k_t) d_i)
//    i.e. (I + diag(b) A) D = diag(b) (V - diag(g) K S_0^T), A_{t,i} = (g_t/g_i) k_t.k_i
//    for i < t, and the state leaving the chunk S_n = g_{n-1} S_0 + D^T diag(g_{n-1}/g) K.
//    A preparation kernel, parallel over all chunks, forms X = (I + diag(b) A)^-1 diag(b)
//    by forward substitution together with the in-chunk decays; the chunk kernel then runs
//    per (request, head) over its chunks in order with three matrix products per chunk
//      E = V - diag(g) K S_0^T,   D = X E,   S_n = g_{n-1} S_0 + D^T diag(g_{n-1}/g) K
//    on MFMA, every operand split into bf16 hi + lo parts and multiplied as
//    hi*hi + hi*lo + lo*hi with fp32 accumulation; the state stays in fp32 accumulators.
//
// Chunks are aligned to 32-token blocks of the stacked prompt array, not to request starts:
// a block holding the end of one prompt and the start of the next has two segments, and
// every in-chunk product (decays, A, X) stays inside one segment, so block b serves each
// request it overlaps with that request's tokens only.
#include <type_traits>

#include "gdn_device.h"

namespace gdn {

// ---------------------------------------------------------------- token-sequential form

// One workgroup per (request, head, block of up to 128 rows): rows of S evolve
// independently given the token.  Thread (row, part) holds S[row][part*COLS ..] in
// registers.  Each token: u = S k (row dot, reduced over the row's lanes),
// S <- alpha S + beta (v - alpha u) k^T.
template <int DK, int DV>
struct PrefillCfg {
  static constexpr int RB = DV < 128 ? DV : 128;                         // rows per block
  static constexpr int TPR = DV < 32 ? 256 / DV : (DK > 128 ? 4 : 2);    // lanes per row
  static constexpr int NT = RB * TPR;
};

__device__ __forceinline__ void request_span(const PrefillArgs& a, int r, int& beg, int& end) {
  beg = a.offsets[r];
  end = a.offsets[r + 1];
  beg = beg < 0 ? 0 : (beg > a.N ? int(a.N) : beg);
  end = end < beg ? beg : (end > a.N ? int(a.N) : end);
}

template <int DK, int DV>
__global__ void __launch_bounds__((PrefillCfg<DK, DV>::NT)) prefill_kernel(PrefillArgs a) {
  constexpr int TPR = PrefillCfg<DK, DV>::TPR;
  constexpr int COLS = DK / TPR;
  const int rh = blockIdx.x, r = rh / a.H, h = rh % a.H;
  const int hk = h / (a.H / a.HK);                        // key head of value head h
  const int row = blockIdx.y * PrefillCfg<DK, DV>::RB + threadIdx.x / TPR, cp = threadIdx.x % TPR;
  int beg, end;
  request_span(a, r, beg, end);
  float S[COLS];
#pragma unroll
  for (int c = 0; c < COLS; ++c) S[c] = 0.0f;
  float kc[COLS];
  float vn = 0.0f, an = 0.0f, bn = 0.0f;
  auto load = [&](int i, float* kk, float& vv, float& aa, float& bb) {
    const float* kp = a.k + (size_t(i) * a.HK + hk) * DK + cp * COLS;
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

// ---------------------------------------------------------------- chunked form: shared parts

// bf16 hi + lo parts of 8 floats: hi = bf16(x) (nearest even), lo = bf16(x - hi).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const __bf16 h = static_cast<__bf16>(x[s]);
    hi[s] = h;
    lo[s] = static_cast<__bf16>(x[s] - static_cast<float>(h));
  }
}

// Position of index j (0..31) of a K = 32 contraction inside the two bf16 32x32x16 MFMA
// operands that cover it: block u = j / 16, lane half hf = (j / 4) % 2, slot s in 0..7.
// The slots follow the rows a 32x32 fp32 accumulator holds in registers 8u .. 8u+7
// (row 8 (i/4) + 4 hf + i % 4 in register i), so an accumulator is used directly as the
// B operand of the next product, with the A operand stored in the same order.
__device__ __forceinline__ int k32_unit(int j) { return ((j >> 4) << 1) | ((j >> 2) & 1); }
__device__ __forceinline__ int k32_slot(int j) { return (((j >> 3) & 1) << 2) | (j & 3); }

// ---------------------------------------------------------------- chunked form: preparation

// One wave per (32-token block b, value head h).  Writes, at ws + (b H + h) kPrepFloats:
//   X[t][j]  (32 x 32)  the chunk matrix (I + diag(b) A)^-1 diag(b) of the block's segments
//   g[t]     (32)       a-product over the segment's tokens up to and including t
//   sfx[t]   (32)       a-product over the segment's tokens after t
// A token that no request owns is a segment of its own.  X is block diagonal over
// segments: entries across segments are exactly 0.
template <int DK>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) chunk_prep_kernel(PrefillArgs a) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int hk = h / (a.H / a.HK);
  const int l = threadIdx.x, tl = l & 31, hf = l >> 5;
  const int64_t p0 = int64_t(b) * kChunk;
  __shared__ float s_alpha[kChunk], s_beta[kChunk];
  // column i of L: s_lt[i][t % 2][t / 2] = L[t][i], so a lane half reads its rows at once
  __shared__ __align__(16) float s_lt[kChunk][2][kChunk / 2 + 4];

  // segment id of token p0 + tl: its request, or -1 - tl when no request owns it
  const int64_t p = p0 + tl;
  int sid = -1 - tl;
  if (p < a.N) {
    int lo = 0, hi = a.R - 1;                   // largest r with clamp(offsets[r]) <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      int o = a.offsets[mid];
      o = o < 0 ? 0 : (o > a.N ? int(a.N) : o);
      if (o <= p) lo = mid; else hi = mid - 1;
    }
    int beg, end;
    request_span(a, lo, beg, end);
    if (p >= beg && p < end) sid = lo;
  }
  const bool own = sid >= 0;
  // segments are runs of equal ids: bit t of `starts` marks a segment starting at token t;
  // token c's segment is [seg_lo(c), seg_hi(c))
  const int sid_prev = __shfl(sid, (tl + 63) & 63);
  const uint32_t starts = uint32_t(__ballot(tl == 0 || sid != sid_prev)) | 1u;
  auto seg_hi = [&](int c) {
    const uint32_t m = c == 31 ? 0u : (starts & (0xFFFFFFFFu << (c + 1)));
    return m ? __builtin_ctz(m) : kChunk;
  };
  auto seg_lo = [&](int c) { return 31 - __builtin_clz(starts & (0xFFFFFFFFu >> (31 - c))); };
  if (hf == 0) {
    const size_t pa = size_t(own ? p : 0) * a.H + h;
    const float al = a.alpha[pa], be = a.beta[pa];
    s_alpha[tl] = own ? al : 1.0f;
    s_beta[tl] = own ? be : 0.0f;
  }

  // G = K K^T over the block (rows of tokens no request owns are zero), bf16 hi+lo split:
  // lane (t, hf) holds k_t[16 kb + 8 hf .. +8], which is both its A and its B fragment.
  f32x16 G;
#pragma unroll
  for (int i = 0; i < 16; ++i) G[i] = 0.0f;
  const float* kp = a.k + (size_t(own ? p : 0) * a.HK + hk) * DK + 8 * hf;
#pragma unroll
  for (int kb = 0; kb < DK / 16; ++kb) {
    float x[8];
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 u0 = own ? *reinterpret_cast<const f32x4*>(kp + 16 * kb) : zero;
    const f32x4 u1 = own ? *reinterpret_cast<const f32x4*>(kp + 16 * kb + 4) : zero;
#pragma unroll
    for (int s = 0; s < 4; ++s) { x[s] = u0[s]; x[4 + s] = u1[s]; }
    bf16x8 xh, xl;
    split8(x, xh, xl);
    G = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, xh, G, 0, 0, 0);
    G = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, xl, G, 0, 0, 0);
    G = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, xh, G, 0, 0, 0);
  }
  __syncthreads();

  // L[t][c] = b_t (a_{c+1} ... a_t) G[t][c] for c < t in c's segment, else 0.  Lane
  // (c, hf) holds column c and rows t = 8 (i/4) + 4 hf + i%4; the a-products run along t.
  {
    const int c = tl, chi = seg_hi(c);
    float run = 1.0f;
    float gam[16];
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
      run *= t > c ? s_alpha[t] : 1.0f;
      if (((t >> 2) & 1) == 0) gam[4 * (t >> 3) + (t & 3)] = hf ? gam[4 * (t >> 3) + (t & 3)] : run;
      else gam[4 * (t >> 3) + (t & 3)] = hf ? run : gam[4 * (t >> 3) + (t & 3)];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = 8 * (i >> 2) + 4 * hf + (i & 3);
      const bool in = t > c && t < chi;
      s_lt[c][t & 1][t >> 1] = in ? s_beta[t] * gam[i] * G[i] : 0.0f;
    }
  }
  __syncthreads();

  // Column j of X solves (I + L) x = b_j e_j by forward substitution.  Lane (j, hf) owns
  // rows 2q + hf of column j; once x_t is fixed (by the half owning row t, then shared
  // with the other half), each half adds L[row][t] x_t to the sums of its rows below t.
  // L is zero on and above the diagonal, so the rows at or above t may take the update.
  const int j = tl, jhi = seg_hi(j);
  float x[kChunk / 2], acc[kChunk / 2];
#pragma unroll
  for (int q = 0; q < kChunk / 2; ++q) acc[q] = 0.0f;
#pragma unroll
  for (int t = 0; t < kChunk; ++t) {
    const float bt = s_beta[t];
    const float own_x = t == j ? bt : ((t > j && t < jhi) ? -acc[t >> 1] : 0.0f);
    const float other = __shfl_xor(own_x, 32);
    const float xt = hf == (t & 1) ? own_x : other;
    x[t >> 1] = hf == (t & 1) ? xt : x[t >> 1];
    if (t + 1 < kChunk) {
      const float* lr = s_lt[t][hf];
#pragma unroll
      for (int q = (t >> 1) & ~3; q < kChunk / 2; q += 4) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(lr + q);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q + e] = fmaf(lv[e], xt, acc[q + e]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);       // keep the L loads of each step with it
  }
  float* w = a.ws + (size_t(b) * a.H + h) * kPrepFloats;
#pragma unroll
  for (int q = 0; q < kChunk / 2; ++q) w[(2 * q + hf) * kChunk + j] = x[q];

  // in-segment a-products up to and including, and after, each token (ascending order)
  if (hf == 0) {
    const int lo = seg_lo(tl), hi = seg_hi(tl);
    float g = 1.0f, f = 1.0f;
#pragma unroll
    for (int q = 0; q < kChunk; ++q) {
      const float aq = s_alpha[q];
      g *= (q >= lo && q <= tl) ? aq : 1.0f;
      f *= (q > tl && q < hi) ? aq : 1.0f;
    }
    w[kChunk * kChunk + tl] = g;
    w[kChunk * kChunk + kChunk + tl] = f;
  }
}

// ---------------------------------------------------------------- chunked form: chunk kernel

// One workgroup per (request, head, block of RB rows): NW waves, each owning 32 rows of
// S^T (d x rows) as DK/32 fp32 32x32 accumulators.  Chunk operands go through LDS in bf16
// hi/lo MFMA fragment order, double buffered: while chunk n is computed, chunk n+1 is
// already in the other buffer and chunk n+2 is in flight from HBM into registers.
template <int DK, int DV>
struct ChunkCfg {
  static constexpr int NW = DV / 32 < 8 ? DV / 32 : 8;
  static constexpr int NT = 64 * NW;
  static constexpr int RB = 32 * NW;
  static constexpr int NB = DV / RB;              // workgroups per (request, head)
  static constexpr int NTD = DK / 32;
  // LDS buffer: KA (32 rows t x DK, A of E), KD (DK rows d x 32, A of the state update),
  // XA (32 x 32, A of D), each as bf16 hi then lo.  The chunk decays g_{n-1} stay in
  // registers.
  static constexpr int KA = 0;
  static constexpr int KA_HALF = 32 * DK * 2;
  static constexpr int KD = KA + 2 * KA_HALF;
  static constexpr int KD_HALF = DK * 64;
  static constexpr int XA = KD + 2 * KD_HALF;
  static constexpr int XA_HALF = 32 * 64;
  // With d_k = 128 and 8 waves, V of the chunk also goes through LDS (16-byte loads
  // instead of one 4-byte load per token and lane): rows of 32 tokens as token pairs,
  // [pair][row][2], pair rows padded so that tokens t and t + 4 (the two lane halves of an
  // accumulator) fall on different LDS banks.
  static constexpr bool VL = DK == 128 && NW == 8;
  static constexpr int VPS = 2 * RB + 16;         // floats per token pair
  static constexpr int VS = XA + 2 * XA_HALF;
  static constexpr int BUF = VS + (VL ? 16 * VPS * 4 : 0);
  static constexpr int KITEMS = 16 * (DK / 4);    // 2 tokens x 4 columns of K each
  static constexpr int XITEMS = 32 * 16;          // 2 columns of one X row each
  static constexpr int VITEMS = 16 * (RB / 4);    // 2 tokens x 4 rows of V each
  static constexpr int KPT = KITEMS / NT;
  static constexpr int XPT = XITEMS / NT;
  static constexpr int VPT = VL ? VITEMS / NT : 1;
  static_assert(KITEMS % NT == 0 && XITEMS % NT == 0 && VITEMS % NT == 0,
                "items split evenly over threads");
};

// byte offset of 16-byte unit q of row t of KA (swizzled over 16 rows)
template <int DK>
__device__ __forceinline__ int ka_off(int t, int q) { return t * (DK * 2) + ((q ^ (t & 15)) << 4); }
// byte offset of 16-byte unit q (0..3) of row m of a 32-column fragment array (KD, XA)
__device__ __forceinline__ int k32_off(int m, int q) { return (m << 6) + ((q ^ ((m >> 2) & 3)) << 4); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// bf16 hi + lo parts of a pair, packed: hi = bf16(x) (nearest even), lo = bf16(x - hi).
// The hi values are read back from the packed word, one rounding per pair.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hp, uint32_t& lp) {
  hp = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x0, x1}), bf16x2));
  const f32x2 r = {x0 - __uint_as_float(hp << 16), x1 - __uint_as_float(hp & 0xFFFF0000u)};
  lp = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}
__device__ __forceinline__ void split8p(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t hq, lq;
    split2(x[2 * q], x[2 * q + 1], hq, lq);
    h[q] = hq;
    l[q] = lq;
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

template <int DK, int DV>
__global__ void __launch_bounds__((ChunkCfg<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(2))) chunk_kernel(PrefillArgs a) {
  using C = ChunkCfg<DK, DV>;
  extern __shared__ __align__(16) unsigned char lds[];
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int rb = w % C::NB, rh = w / C::NB, r = rh / a.H, h = rh % a.H;
  const int hk = h / (a.H / a.HK);
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, ln = l & 31, hf = l >> 5;
  const int row = rb * C::RB + 32 * wave + ln;        // this lane's state row (column n)
  int beg, end;
  request_span(a, r, beg, end);
  const int b0 = beg / kChunk, b1 = end > beg ? (end - 1) / kChunk + 1 : b0;
  const size_t kstride = size_t(a.HK) * DK, vstride = size_t(a.H) * DV;   // floats per token

  // Loads use a per-chunk base (uniform) plus offsets fixed per thread; only the array's
  // last block, which may reach past N, clamps its rows (to row 0 of the block).  Rows of
  // other requests are loaded and then replaced by zeros where a block is shared.  The
  // lambdas that touch these arrays are forced inline: one call left out of line (past the
  // inliner's cost limit) passes them by address and puts them in scratch memory.
  f32x4 kreg[C::KPT][2], vreg[C::VPT][2];
  f32x2 kgs[C::KPT][2];                  // g and sfx of the item's two tokens
  f32x2 xreg[C::XPT];
  float gcl = 1.0f;
  // byte offsets (fixed per thread) of the K rows, X pairs and V rows this thread loads
  uint32_t koff[C::KPT][2], voff[16], vloff[C::VPT][2];
#pragma unroll
  for (int m = 0; m < C::KPT; ++m) {
    const int it = tid + m * C::NT, t2 = it / (DK / 4), d4 = it % (DK / 4);
#pragma unroll
    for (int e = 0; e < 2; ++e) koff[m][e] = uint32_t(((2 * t2 + e) * kstride + 4 * d4) * 4);
  }
#pragma unroll
  for (int m = 0; m < C::VPT; ++m) {
    const int it = tid + m * C::NT, tp = it / (C::RB / 4), g = it % (C::RB / 4);
#pragma unroll
    for (int e = 0; e < 2; ++e) vloff[m][e] = uint32_t(((2 * tp + e) * vstride + 4 * g) * 4);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
    voff[i] = uint32_t(((8 * (i >> 2) + 4 * hf + (i & 3)) * vstride + row) * 4);
  // clamp: the array's last block, which may reach past N (rows past N read row 0)
  auto fetch = [&](int b, auto clamp) __attribute__((always_inline)) {
    const char* kb = reinterpret_cast<const char*>(a.k + size_t(b) * kChunk * kstride + size_t(hk) * DK);
    const float* pw = a.ws + (size_t(b) * a.H + h) * kPrepFloats;
    const int nrow = int(a.N - int64_t(b) * kChunk);
#pragma unroll
    for (int m = 0; m < C::KPT; ++m) {
      const int it = tid + m * C::NT, t2 = it / (DK / 4);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t o = koff[m][e];
        if constexpr (decltype(clamp)::value)
          o = 2 * t2 + e < nrow ? o : o - uint32_t((2 * t2 + e) * kstride * 4);
        kreg[m][e] = *reinterpret_cast<const f32x4*>(kb + o);
      }
      kgs[m][0] = *reinterpret_cast<const f32x2*>(pw + kChunk * kChunk + 2 * t2);
      kgs[m][1] = *reinterpret_cast<const f32x2*>(pw + kChunk * kChunk + kChunk + 2 * t2);
    }
    if constexpr (C::VL) {
      const char* vb = reinterpret_cast<const char*>(a.v + size_t(b) * kChunk * vstride +
                                                     size_t(h) * DV + size_t(rb) * C::RB);
#pragma unroll
      for (int m = 0; m < C::VPT; ++m) {
        const int it = tid + m * C::NT, tp = it / (C::RB / 4);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint32_t o = vloff[m][e];
          if constexpr (decltype(clamp)::value)
            o = 2 * tp + e < nrow ? o : o - uint32_t((2 * tp + e) * vstride * 4);
          vreg[m][e] = *reinterpret_cast<const f32x4*>(vb + o);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < C::XPT; ++m) {
      const int it = tid + m * C::NT, tr = it >> 4, q2 = it & 15;
      xreg[m] = *reinterpret_cast<const f32x2*>(pw + tr * kChunk + 2 * q2);
    }
    // g of the request's last token in the block (the chunk's decay of the state)
    int tlast = end - b * kChunk;
    tlast = (tlast > kChunk ? kChunk : tlast) - 1;
    gcl = pw[kChunk * kChunk + tlast];
  };
  auto shared_block = [&](int b) { return b * kChunk < beg || (b + 1) * kChunk > end; };
  auto valid = [&](int b, int t) { const int p = b * kChunk + t; return p >= beg && p < end; };
  // registers of block b -> LDS buffer (bf16 hi/lo fragments)
  // MASK: a block shared with another request (its rows are replaced by zeros)
  auto stage = [&](int b, unsigned char* buf, auto mask) __attribute__((always_inline)) {
    constexpr bool part = decltype(mask)::value;
#pragma unroll
    for (int m = 0; m < C::KPT; ++m) {
      const int it = tid + m * C::NT, t2 = it / (DK / 4), d4 = it % (DK / 4);
      f32x4 kv[2];
      float gv[2], sv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        kv[e] = kreg[m][e];
        gv[e] = kgs[m][0][e];
        sv[e] = kgs[m][1][e];
      }
      if constexpr (part) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bool ok = valid(b, 2 * t2 + e);
          kv[e] = ok ? kv[e] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          gv[e] = ok ? gv[e] : 0.0f;
          sv[e] = ok ? sv[e] : 0.0f;
        }
      }
      const int d = 4 * d4;
      // KA rows t: -g_t k_t[d .. d+4], one 8-byte piece each (hi, lo)
      const int q = ((d >> 5) << 2) | k32_unit(d & 31);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int off = ka_off<DK>(2 * t2 + e, q) + (k32_slot(d & 31) << 1);
        uint2 hv, lv;
        split2(-gv[e] * kv[e][0], -gv[e] * kv[e][1], hv.x, lv.x);
        split2(-gv[e] * kv[e][2], -gv[e] * kv[e][3], hv.y, lv.y);
        *reinterpret_cast<uint2*>(buf + C::KA + off) = hv;
        *reinterpret_cast<uint2*>(buf + C::KA + C::KA_HALF + off) = lv;
      }
      // KD rows d + s: sfx_t k_t[d + s] for the token pair, one 4-byte piece each
      const int t = 2 * t2;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int off = k32_off(d + s2, k32_unit(t)) + (k32_slot(t) << 1);
        uint32_t hv, lv;
        split2(sv[0] * kv[0][s2], sv[1] * kv[1][s2], hv, lv);
        *reinterpret_cast<uint32_t*>(buf + C::KD + off) = hv;
        *reinterpret_cast<uint32_t*>(buf + C::KD + C::KD_HALF + off) = lv;
      }
    }
#pragma unroll
    for (int m = 0; m < C::XPT; ++m) {
      const int it = tid + m * C::NT, tr = it >> 4, t = 2 * (it & 15);
      f32x2 xv = xreg[m];
      if constexpr (part) xv = valid(b, tr) ? xv : f32x2{0.0f, 0.0f};
      const int off = k32_off(tr, k32_unit(t)) + (k32_slot(t) << 1);
      uint32_t hv, lv;
      split2(xv[0], xv[1], hv, lv);
      *reinterpret_cast<uint32_t*>(buf + C::XA + off) = hv;
      *reinterpret_cast<uint32_t*>(buf + C::XA + C::XA_HALF + off) = lv;
    }
    if constexpr (C::VL) {
#pragma unroll
      for (int m = 0; m < C::VPT; ++m) {
        const int it = tid + m * C::NT, tp = it / (C::RB / 4), g = it % (C::RB / 4);
        f32x4 v0 = vreg[m][0], v1 = vreg[m][1];
        if constexpr (part) {
          v0 = valid(b, 2 * tp) ? v0 : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          v1 = valid(b, 2 * tp + 1) ? v1 : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float* vp = reinterpret_cast<float*>(buf + C::VS) + tp * C::VPS + 8 * g;
        *reinterpret_cast<f32x4*>(vp) = f32x4{v0[0], v1[0], v0[1], v1[1]};
        *reinterpret_cast<f32x4*>(vp + 4) = f32x4{v0[2], v1[2], v0[3], v1[3]};
      }
    }
  };
  auto stage_any = [&](int b, unsigned char* buf) __attribute__((always_inline)) {
    if (shared_block(b)) stage(b, buf, std::true_type{});
    else stage(b, buf, std::false_type{});
  };
  // V rows of the chunk in accumulator order: register i holds token 8 (i/4) + 4 hf + i%4
  auto fetch_v = [&](int b, f32x16& vv, auto clamp) __attribute__((always_inline)) {
    const char* vb = reinterpret_cast<const char*>(a.v + size_t(b) * kChunk * vstride + size_t(h) * DV);
    const int nrow = int(a.N - int64_t(b) * kChunk);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t o = voff[i];
      if constexpr (decltype(clamp)::value)
        o = 8 * (i >> 2) + 4 * hf + (i & 3) < nrow ? o : uint32_t(row * 4);
      vv[i] = *reinterpret_cast<const float*>(vb + o);
    }
  };
  auto mask_v = [&](int b, f32x16& vv) __attribute__((always_inline)) {
    if (shared_block(b)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = 8 * (i >> 2) + 4 * hf + (i & 3);
        vv[i] = valid(b, t) ? vv[i] : 0.0f;
      }
    }
  };

  f32x16 S[C::NTD];
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) S[nt][i] = 0.0f;

  // one chunk from LDS buffer cur: E = V - diag(g) K S^T, D = X E,
  // S^T <- g_{n-1} S^T + (diag(sfx) K)^T D
  auto compute = [&](int b, const unsigned char* cur, f32x16 E, float gc, auto mask)
      __attribute__((always_inline)) {
    if constexpr (C::VL) {        // V rows of tokens 8 (i/4) + 4 hf + i%4, i = 2q, 2q + 1
      const float* vp = reinterpret_cast<const float*>(cur + C::VS) + 2 * (32 * wave + ln);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int t = 8 * (q >> 1) + 4 * hf + 2 * (q & 1);
        const f32x2 x = *reinterpret_cast<const f32x2*>(vp + (t >> 1) * C::VPS);
        E[2 * q] = x[0];
        E[2 * q + 1] = x[1];
      }
    } else if constexpr (decltype(mask)::value) {
      mask_v(b, E);
    }
    // KA holds -g_t k_t
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float sv[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) sv[s2] = S[nt][8 * u + s2];
        bf16x8 bh, bl;
        split8p(sv, bh, bl);
        const int off = ka_off<DK>(ln, (nt << 2) | (u << 1) | hf);
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(cur + C::KA + off);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(cur + C::KA + C::KA_HALF + off);
        E = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, E, 0, 0, 0);
        E = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, E, 0, 0, 0);
        E = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, E, 0, 0, 0);
      }
    }
    f32x16 D;
#pragma unroll
    for (int i = 0; i < 16; ++i) D[i] = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float ev[8];
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) ev[s2] = E[8 * u + s2];
      bf16x8 bh, bl;
      split8p(ev, bh, bl);
      const int off = k32_off(ln, (u << 1) | hf);
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(cur + C::XA + off);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(cur + C::XA + C::XA_HALF + off);
      D = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, D, 0, 0, 0);
      D = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, D, 0, 0, 0);
      D = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, D, 0, 0, 0);
    }
    bf16x8 dh[2], dl[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float dv[8];
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) dv[s2] = D[8 * u + s2];
      split8p(dv, dh[u], dl[u]);
    }
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) S[nt][i] *= gc;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int off = k32_off(32 * nt + ln, (u << 1) | hf);
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(cur + C::KD + off);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(cur + C::KD + C::KD_HALF + off);
        S[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, dh[u], S[nt], 0, 0, 0);
        S[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, dl[u], S[nt], 0, 0, 0);
        S[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, dh[u], S[nt], 0, 0, 0);
      }
    }
  };

  // Blocks [b0, bin) lie inside the array and run pipelined with straight-line loads; a
  // request that holds the array's last, partial block finishes with it unpipelined.
  // Only a request's first and last blocks can be shared with another request: the first
  // is staged before the loop, the last in the loop's last-but-one pass, so the body of
  // the main loop is one straight run of code (no masks, no branches) in which the
  // compiler can place the next chunk's staging among the current chunk's MFMAs.
  const int bin = b1 < int(a.N / kChunk) ? b1 : int(a.N / kChunk);
  const std::false_type inside, whole;
  const std::true_type masked;
  f32x16 vcur, vnext;
  float g0 = 1.0f, g1 = 1.0f;                       // chunk decays of blocks b, b + 1
  if (b0 < bin) {
    fetch(b0, inside);
    g0 = gcl;
    if constexpr (!C::VL) {
      fetch_v(b0, vcur, inside);
      mask_v(b0, vcur);
    }
    stage_any(b0, lds);
    fetch(b0 + 1 < bin ? b0 + 1 : b0, inside);
    g1 = gcl;
  }
  __syncthreads();
  int b = b0;
  for (; b + 2 < bin; ++b) {                        // stages b + 1 <= bin - 2: whole blocks
    unsigned char* cur = lds + ((b - b0) & 1) * C::BUF;
    unsigned char* nxt = lds + (((b - b0) & 1) ^ 1) * C::BUF;
    if constexpr (!C::VL) fetch_v(b + 1, vnext, inside);
    // the products read cur first; the staging of block b + 1 (register arithmetic, then
    // LDS writes to nxt) follows them in program order, so that its arithmetic can move
    // in among the MFMAs; block b + 2's loads go out last and land during the next pass
    compute(b, cur, vcur, g0, whole);
    stage(b + 1, nxt, whole);
    fetch(b + 2, inside);
    g0 = g1;
    g1 = gcl;
    vcur = vnext;
    __syncthreads();
  }
  if (b + 1 < bin) {                                // stages the last block of the array part
    unsigned char* cur = lds + ((b - b0) & 1) * C::BUF;
    unsigned char* nxt = lds + (((b - b0) & 1) ^ 1) * C::BUF;
    stage_any(b + 1, nxt);
    if constexpr (!C::VL) fetch_v(b + 1, vnext, inside);
    compute(b, cur, vcur, g0, masked);
    g0 = g1;
    vcur = vnext;
    __syncthreads();
    ++b;
  }
  if (b < bin) compute(b, lds + ((b - b0) & 1) * C::BUF, vcur, g0, masked);
  if (bin < b1) {
    const int bt = b1 - 1;
    __syncthreads();
    fetch(bt, std::true_type{});
    if constexpr (!C::VL) fetch_v(bt, vcur, std::true_type{});
    stage(bt, lds, masked);
    __syncthreads();
    compute(bt, lds, vcur, gcl, masked);
  }

  // S_out[r][h][row][d]: register i of tile nt holds d = 32 nt + 8 (i/4) + 4 hf + i%4
  float* out = a.S_out + (size_t(rh) * DV + row) * DK;
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4*>(out + 32 * nt + 8 * g + 4 * hf) =
          f32x4{S[nt][4 * g], S[nt][4 * g + 1], S[nt][4 * g + 2], S[nt][4 * g + 3]};
}

// ---------------------------------------------------------------- launchers

template <int DK, int DV>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  using C = PrefillCfg<DK, DV>;
  hipLaunchKernelGGL((prefill_kernel<DK, DV>), dim3(a.R * a.H, DV / C::RB), dim3(C::NT), 0, s, a);
  return last_launch_error();
}

template <int DK, int DV>
static int launch_chunked_t(const PrefillArgs& a, hipStream_t s) {
  using C = ChunkCfg<DK, DV>;
  const int nb = int((a.N + kChunk - 1) / kChunk);
  if (nb > 0) {
    hipLaunchKernelGGL((chunk_prep_kernel<DK>), dim3(nb, a.H), dim3(64), 0, s, a);
    if (int e = last_launch_error()) return e;
  }
  // dynamic LDS above 64 KiB (set on every launch: the attribute is per device)
  if (int e = int(hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_kernel<DK, DV>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, 2 * C::BUF)))
    return e;
  hipLaunchKernelGGL((chunk_kernel<DK, DV>), dim3(a.R * a.H * C::NB), dim3(C::NT), 2 * C::BUF, s, a);
  return last_launch_error();
}

bool prefill_chunked(int d_k) { return d_k >= 128; }

size_t prefill_workspace_bytes(int H, int d_k, int64_t N) {
  if (!prefill_chunked(d_k)) return 0;
  return size_t((N + kChunk - 1) / kChunk) * size_t(H) * kPrepFloats * sizeof(float);
}

int launch_prefill(const PrefillArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  if (a.ws) {
    if (a.d_k == 128 && a.d_v == 128) return launch_chunked_t<128, 128>(a, s);
    if (a.d_k == 128 && a.d_v == 256) return launch_chunked_t<128, 256>(a, s);
    if (a.d_k == 256 && a.d_v == 256) return launch_chunked_t<256, 256>(a, s);
    if (a.d_k == 128 && a.d_v == 512) return launch_chunked_t<128, 512>(a, s);
    if (a.d_k == 256 && a.d_v == 512) return launch_chunked_t<256, 512>(a, s);
    return int(hipErrorInvalidValue);
  }
  if (a.d_k == 16 && a.d_v == 16) return launch_prefill_t<16, 16>(a, s);
  if (a.d_k == 128 && a.d_v == 128) return launch_prefill_t<128, 128>(a, s);
  if (a.d_k == 128 && a.d_v == 256) return launch_prefill_t<128, 256>(a, s);
  if (a.d_k == 256 && a.d_v == 256) return launch_prefill_t<256, 256>(a, s);
  if (a.d_k == 128 && a.d_v == 512) return launch_prefill_t<128, 512>(a, s);
  if (a.d_k == 256 && a.d_v == 512) return launch_prefill_t<256, 512>(a, s);
  return int(hipErrorInvalidValue);
}

}  // namespace gdn
