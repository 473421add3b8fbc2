// Selection-side HIP kernels for large-beam Gated DeltaNet decoding on gfx950.
//
// Scoring follows the beam-search objective of OneLA (paper-archivist.com) section 1.1,
// eq. (1) and large-beam decoding's global top-k; the exact request-level top-K with a
// per-row precut follows RecoGEM
// (conceptio mirror) section 4.3; the ancestry remap is OneLA eq. (9).
//
// No score matrix is materialised.  Codes are cut into tiles of 32 (one MFMA block of
// rows).  The first pass keeps, per (beam, tile), the largest logit, and per beam the
// log-sum-exp.  The exact top-K of the tiles, ranked by the score of their largest
// logit, must contain every tile that holds one of the top-K candidates: each chosen
// tile owns a candidate that ranks at or above its tile-mates, so any candidate of an
// unchosen tile has K distinct candidates ahead of it.  Only the chosen tiles are
// recomputed, with the same MFMA sequence (bit-identical logits), and the exact top-K
// is taken over their 32 K candidates.
//
// Kernels
//   wprep_kernel     large selections: the codebook transposed to [V,d_v] and rescaled
//                    into fp16 tile by tile (exponent per 32-code tile).
//   zsum_kernel      z_b = sum_h o_b, stored as the MFMA operand: two fp16 terms and the
//                    beam's scale where wprep_kernel ran and every tile fits fp16, else
//                    bf16 hi/mid/lo (bf16 codebook), or fp32 (fp32 codebook); its last
//                    grid row transposes the codebook Wout[d_v,V] -> [V,d_v] where
//                    wprep_kernel did not run.
//   logits_kernel    first pass on MFMA: per (beam, tile) largest logit, online
//                    log-sum-exp parts per code group.
//   tile_select_kernel  one block per request: log-sum-exp per beam, then the exact
//                    top-K tiles by radix passes over the tile maxima (or, for requests
//                    with many tiles, over the few that reach a lower bound taken from the
//                    code groups' maxima) and a finish inside the boundary digit; groups
//                    the chosen tiles by code tile.
//   refine_kernel    recomputes the chosen tiles' logits (one MFMA block per group) and
//                    writes their 32 candidate keys each.
//   final_kernel     exact top-K over the refined keys in LDS, ties by flat index,
//                    sort, the top-W outputs, and the remap of ancestry, SID prefixes
//                    and cumulative scores (eq. 9).
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "gdn_device.h"

namespace gdn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- z and its operand

// zf per request: [chunk][kk][term][lane] u32x4, chunk = b / 32, kk < d_v / 16, term
// 0/1/2 = hi/mid/lo bf16 parts of z, lane l -> beam 32 chunk + l % 32 and elements
// d = d_v / 2 * (l / 32) + 8 kk + i (i < 8): the B operand of the logits MFMA.
__device__ __forceinline__ size_t zf_lane_base(int r, int nch_max, int d_v, int b, int hf) {
  return (size_t(r) * nch_max + (b >> 5)) * size_t(d_v / 16) * 3 * 64 + (b & 31) + 32 * hf;
}

__device__ __forceinline__ uint32_t f2h_bits(float x) {
  return uint32_t(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}
__device__ __forceinline__ float h2f(uint32_t b) {
  return float(__builtin_bit_cast(_Float16, uint16_t(b)));
}

// ---- two-term fp16 operands (bf16 codebook)
//
// The logits take z in two fp16 terms, h = fp16(z 2^t) and l = fp16(z 2^t - h), against
// the bf16 codebook rescaled into fp16 tile by tile (code tile j times 2^s_j): fp16 holds
// 11 significant bits, so |z 2^t - h - l| <= 2^-24 |z 2^t|, the precision of fp32 itself,
// and the products are exact in the fp32 accumulator.  A tile fits when its entries' 8
// significant bits stay on fp16's grid after its scale, which holds when its nonzero
// entries' exponents span at most 32 binades (and none is subnormal, infinite or NaN).
// If any tile does not fit, z goes in three bf16 terms (hi, mid, lo) against the
// codebook as it is: 24 significant bits, one more MFMA per k-step.  t is chosen per
// beam so that its largest |z| lands in [2^14, 2^15); s_j so that the tile's largest
// entry stays below 2^15.

struct WprepK {
  int d_v, V, split;
  const void* wout;     // [d_v,V]
  void* woutT;          // [V,d_v]
  uint16_t* woutT16;    // [V,d_v] fp16, tile j scaled by 2^s_j
  int32_t* tscale;      // [n_tiles(V)] s_j
  uint32_t* f16flag;    // set if a tile does not fit fp16
};

// Codebook transpose Wout[d_v,V] -> Wout^T[V,d_v], the first launch of a selection; for a
// bf16 codebook also each code tile's fp16 form.  Block j: the 32 codes of tile j, one per
// lane of each half-wave, and d_v / 8 rows per half-wave: every load of a thread is issued
// at once (a half-wave reads 32 consecutive codes of a row), the tile's exponent range is
// reduced over the block, and each thread writes its rows of the tile's 32 transposed
// rows in both forms.  The flag is touched only by a tile that does not fit.
template <int DV>
__global__ void __launch_bounds__(256) wprep_kernel(WprepK a) {
  constexpr int RPT = DV / 8;                       // rows per thread
  const int j = blockIdx.x;
  const int ci = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int c = 32 * j + ci, r0 = rg * RPT;
  const bool live = c < a.V;
  if (!a.split) {                                   // launch-uniform
    const float* w = static_cast<const float*>(a.wout);
    float x[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) x[i] = live ? w[size_t(r0 + i) * a.V + c] : 0.0f;
    if (live) {
      float* dst = static_cast<float*>(a.woutT) + size_t(c) * DV + r0;
#pragma unroll
      for (int i = 0; i < RPT; ++i) dst[i] = x[i];
    }
    return;
  }
  const uint16_t* w = static_cast<const uint16_t*>(a.wout);
  uint32_t x[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) x[i] = live ? uint32_t(w[size_t(r0 + i) * a.V + c]) : 0u;
  uint32_t emax = 0u, nemin = 0u, bad = 0u;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const uint32_t e = (x[i] >> 7) & 0xFFu;
    if (x[i] & 0x7FFFu) {
      emax = max(emax, e);
      nemin = max(nemin, 255u - e);
      bad |= (e == 0u || e == 255u) ? 1u : 0u;
    }
  }
  __shared__ uint32_t part[3][4];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    emax = max(emax, uint32_t(__shfl_xor(int(emax), off)));
    nemin = max(nemin, uint32_t(__shfl_xor(int(nemin), off)));
    bad |= uint32_t(__shfl_xor(int(bad), off));
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    part[0][wv] = emax;
    part[1][wv] = nemin;
    part[2][wv] = bad;
  }
  __syncthreads();
  emax = max(max(part[0][0], part[0][1]), max(part[0][2], part[0][3]));
  nemin = max(max(part[1][0], part[1][1]), max(part[1][2], part[1][3]));
  bad = part[2][0] | part[2][1] | part[2][2] | part[2][3];
  const uint32_t emin = 255u - nemin;
  const bool fits = bad == 0u && (emax == 0u || emax - emin <= 31u);
  // |W| < 2^(emax - 126): scaled by 2^(141 - emax) the tile's largest entry is below 2^15
  const int sj = emax ? 141 - int(emax) : 0;
  if (threadIdx.x == 0) {
    a.tscale[j] = sj;
    if (!fits) atomicOr(a.f16flag, 1u);
  }
  if (live) {
    uint16_t* d16 = static_cast<uint16_t*>(a.woutT) + size_t(c) * DV + r0;
    uint16_t* h16 = a.woutT16 + size_t(c) * DV + r0;
    if constexpr (RPT >= 8) {
#pragma unroll
      for (int q = 0; q < RPT / 8; ++q) {
        uint32_t hb[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) hb[k] = f2h_bits(ldexpf(bf2f(x[8 * q + k]), sj));
        reinterpret_cast<u32x4*>(d16)[q] = pack8(x + 8 * q);
        reinterpret_cast<u32x4*>(h16)[q] = pack8(hb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        d16[i] = uint16_t(x[i]);
        h16[i] = uint16_t(f2h_bits(ldexpf(bf2f(x[i]), sj)));
      }
    }
  }
}

struct ZsumK {
  int R, H, W, W_max, d_v, V, nch_max;
  int zblocks;          // blocks of the head sum; blocks after them transpose the codebook
  int split;            // bf16 codebook: write zf; fp32 codebook: write z
  int f16_on;           // the two-term fp16 form may be used (its codebook prepared)
  const float* o;       // [R,H,W,d_v]
  float* z;             // [R,W_max,d_v]
  u32x4* zf;
  float* zscale;        // [R,W_max] 2^-t_b (two-term fp16 form)
  const uint32_t* f16flag;
  const void* wout;     // [d_v,V] (transpose blocks)
  void* woutT;          // [V,d_v]
};

// 32 x 32 tiles of Wout[d_v,V] -> Wout^T[V,d_v] through LDS, tiles t0, t0 + nb, ...
template <typename WT>
__device__ void transpose_codebook(const WT* __restrict__ w, WT* __restrict__ wt, int d_v, int V,
                                   int t0, int nb) {
  __shared__ WT tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 256 threads: 32 x 8
  const int ntc = (V + 31) / 32, nt = ntc * ((d_v + 31) / 32);
  for (int t = t0; t < nt; t += nb) {
    const int c0 = (t % ntc) * 32, i0 = (t / ntc) * 32;
    for (int y = ty; y < 32; y += 8) {
      const int i = i0 + y, c = c0 + tx;
      tile[y][tx] = (i < d_v && c < V) ? w[size_t(i) * V + c] : WT{};
    }
    __syncthreads();
    for (int y = ty; y < 32; y += 8) {
      const int c = c0 + y, i = i0 + tx;
      if (c < V && i < d_v) wt[size_t(c) * d_v + i] = tile[tx][y];
    }
    __syncthreads();
  }
}


// Blocks [0, zblocks): one thread per 8 consecutive elements of one beam of one request
// (beams padded to a multiple of 32 with zeros); all heads' loads are in flight at once
// (up to 16), the sum runs in head order.  For a bf16 codebook z is written as the MFMA
// operand: two fp16 terms and the beam's scale where that form is on and every code tile
// fits fp16, else three bf16 terms.  Later blocks (when the codebook was not prepared by
// wprep_kernel): the codebook transpose.  STREAM: o is far larger than the last-level
// cache, and its loads are non-temporal (streamed past that cache rather than evicting
// the step's records).
template <bool STREAM>
__global__ void __launch_bounds__(256) zsum_kernel(ZsumK a) {
  if (int(blockIdx.x) >= a.zblocks) {
    const int t0 = blockIdx.x - a.zblocks, nb = gridDim.x - a.zblocks;
    if (a.split)
      transpose_codebook(static_cast<const uint16_t*>(a.wout), static_cast<uint16_t*>(a.woutT), a.d_v, a.V, t0, nb);
    else
      transpose_codebook(static_cast<const float*>(a.wout), static_cast<float*>(a.woutT), a.d_v, a.V, t0, nb);
    return;
  }
  const bool f16 = a.split && a.f16_on && *a.f16flag == 0u;   // launch-uniform
  const int g8 = a.d_v / 8, HV = a.d_v / 2;
  const int per_req = ((a.W + 31) & ~31) * g8;
  const int n = a.R * per_req;
  // a beam's g8 threads are consecutive lanes of one wave (per_req is a multiple of
  // 32 g8 and the stride of 64): the loop runs the same count on every lane
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += a.zblocks * blockDim.x) {
    const int r = i / per_req, e = i % per_req;
    const int b = e / g8, d0 = 8 * (e % g8);
    f32x4 s0 = {}, s1 = {};
    if (b < a.W) {
      const float* p0 = a.o + (size_t(r) * a.H * a.W + b) * a.d_v + d0;
      const size_t hstride = size_t(a.W) * a.d_v;
      for (int h0 = 0; h0 < a.H; h0 += 16) {
        f32x4 x0[16], x1[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float* p = p0 + size_t(h0 + u < a.H ? h0 + u : h0) * hstride;
          if constexpr (STREAM) {
            x0[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
            x1[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
          } else {
            x0[u] = *reinterpret_cast<const f32x4*>(p);
            x1[u] = *reinterpret_cast<const f32x4*>(p + 4);
          }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (h0 + u < a.H) { s0 += x0[u]; s1 += x1[u]; }
      }
    }
    if (a.split) {
      const int hf = d0 / HV, kk = (d0 % HV) / 8;
      u32x4* dst = a.zf + zf_lane_base(r, a.nch_max, a.d_v, b, hf) + size_t(kk) * 3 * 64;
      if (f16) {
        // the beam's largest |z| over its g8 threads, then the scale 2^t that puts it in
        // [2^14, 2^15)
        float mx = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) mx = fmaxf(mx, fmaxf(fabsf(s0[k]), fabsf(s1[k])));
        for (int off = 1; off < g8; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        int ex = 0;
        (void)frexpf(mx, &ex);                                // mx < 2^ex
        int tb = (mx > 0.0f && __builtin_isfinite(mx)) ? 15 - ex : 0;
        tb = tb < -100 ? -100 : (tb > 100 ? 100 : tb);
        uint32_t hh[8], hl[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float x = ldexpf(k < 4 ? s0[k] : s1[k - 4], tb);
          hh[k] = f2h_bits(x);
          hl[k] = f2h_bits(x - h2f(hh[k]));
        }
        dst[0] = pack8(hh);
        dst[64] = pack8(hl);
        if (d0 == 0 && b < a.W) a.zscale[size_t(r) * a.W_max + b] = ldexpf(1.0f, -tb);
      } else {
        uint32_t bh[8], bm[8], bl[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float x = k < 4 ? s0[k] : s1[k - 4];
          bh[k] = f2bf(x);
          const float r1 = x - bf2f(bh[k]);
          bm[k] = f2bf(r1);
          bl[k] = f2bf(r1 - bf2f(bm[k]));
        }
        dst[0] = pack8(bh);
        dst[64] = pack8(bm);
        dst[128] = pack8(bl);
      }
    } else if (b < a.W) {
      float* dst = a.z + (size_t(r) * a.W_max + b) * a.d_v + d0;
      *reinterpret_cast<f32x4*>(dst) = s0;
      *reinterpret_cast<f32x4*>(dst + 4) = s1;
    }
  }
}

// ---------------------------------------------------------------- one 32 x 32 logits block

// A = codebook rows (codes c0 + lane % 32), B = z columns (32 beams); lane half hf
// holds elements d_v/2 * hf + ...  acc[i] -> code c0 + 8 (i / 4) + 4 hf + i % 4,
// beam = column lane % 32.  Both passes call exactly these, so a candidate's logit has
// the same bits in both.  Rows past the codebook load code 0 and columns past the
// beams load beam 0 of the chunk: MFMA rows and columns are independent, and those
// results are never used.
template <int DV>
__device__ __forceinline__ void load_codes_bf16(const u32x4* wt, int code, int V, int hf, u32x4* w) {
  constexpr int KS = DV / 16, HV = DV / 2;
  const size_t row = size_t(code < V ? code : 0) * DV + HV * hf;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) w[kk] = wt[row / 8 + kk];
}

template <int KS>
__device__ __forceinline__ f32x16 block_mfma_bf16(const u32x4* w, const u32x4* zh, const u32x4* zm,
                                                  const u32x4* zl, f32x16 acc = {}) {
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, w[kk]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, __builtin_bit_cast(bf16x8, zl[kk]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, __builtin_bit_cast(bf16x8, zm[kk]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, __builtin_bit_cast(bf16x8, zh[kk]), acc, 0, 0, 0);
  }
  return acc;
}

// The same block with z in two fp16 terms (h, l) against the rescaled fp16 codebook.
template <int KS>
__device__ __forceinline__ f32x16 block_mfma_f16(const u32x4* w, const u32x4* zh, const u32x4* zl,
                                                 f32x16 acc = {}) {
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const f16x8 x = __builtin_bit_cast(f16x8, w[kk]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, __builtin_bit_cast(f16x8, zl[kk]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, __builtin_bit_cast(f16x8, zh[kk]), acc, 0, 0, 0);
  }
  return acc;
}

// Either form of the bf16-codebook block: two fp16 terms (F16) or three bf16 terms.
template <bool F16, int KS>
__device__ __forceinline__ f32x16 block_mfma_split(const u32x4* w, const u32x4* zh, const u32x4* zm,
                                                   const u32x4* zl, f32x16 acc = {}) {
  if constexpr (F16) return block_mfma_f16<KS>(w, zh, zm, acc);
  else return block_mfma_bf16<KS>(w, zh, zm, zl, acc);
}

template <int DV>
__device__ __forceinline__ f32x16 block_mfma_f32(const float* wt, int code, int V, int hf,
                                                 const float* zv) {
  constexpr int HV = DV / 2;
  const float* wr = wt + size_t(code < V ? code : 0) * DV + HV * hf;
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < HV; ++kk)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wr[kk], zv[kk], acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------- first pass

struct LogitsK {
  int R, W, W_max, V, nchunk, nvg, cpw, nch_max;
  int beam_major;        // tile maxima per request [W][n_tiles(V)] (else [n_tiles(V)][W])
  const float* z;        // [R,W_max,DV]      fp32 codebook
  const u32x4* zf;       // operand fragments bf16 codebook
  const void* woutT;     // [V,DV]
  const void* woutT16;   // [V,DV] fp16, tile j scaled by 2^s_j (two-term form)
  const float* zscale;   // [R,W_max] 2^-t_b (two-term form)
  const int32_t* tscale; // [n_tiles(V)] s_j
  const uint32_t* f16flag; // set: the three-term form
  int f16_on;            // the two-term form may be used
  float* tmax;           // per request: largest logit of each (beam, tile)
  size_t tmax_stride;    // elements per request
  float4* lse_part;      // [R,W_max,nvg]: max, sum of exp(x - max), min tile max
  int gpb = 1;           // code groups per block (consecutive; one z operand load)
  int cpw_shift = 0;     // log2 cpw
};

// Beam chunks (waves) per first-pass block; the block shares one code group.
constexpr int kLogitsWaves = 8;
// Codes per group are at most 1024 (the launcher's choice): 32 tiles.
constexpr int kMaxGroupTiles = 32;
// Code groups one block may take in turn (the launcher's choice, d_v <= 256 with a bf16
// codebook), and the blocks below which it stops merging them: one per CU.
constexpr int kMaxGroupsPerBlock = 8;
constexpr int kLogitsMinBlocks = 256;
// LDS row of the staged tile maxima: one tile for the block's 256 beams, padded so
// that a beam-major read of 32 tiles of one beam spreads over the banks.
constexpr int kTmRow = kLogitsWaves * 32 + 1;
// Tiles the selection keeps in LDS between its bound and the exact K-th key, the
// (beam, code group) pairs whose tiles it reads to find them, and the code groups per
// beam its masks cover.
constexpr int kSelList = 8192;
constexpr int kSelPairs = 4096;
constexpr int kMaxGroupsMask = 128;

// Block: kLogitsWaves chunks of 32 beams x gpb consecutive groups of cpw codes, taken
// in turn.  Chunks are numbered over all requests, request-major, so that every wave
// has one wherever a request has fewer chunks than a block has waves (the codebook is
// the same for all requests).  Each 32-code tile of the codebook is staged once per
// block in LDS (double-buffered; one barrier per stage of two tiles for d_v <= 128, of
// one tile above) and read by every wave as its A operand.  Lane l keeps beam l % 32
// and folds its 16 codes of every tile into the tile maximum (with its partner half)
// and a running log-sum-exp; at the end of each code group both go out and the running
// state starts again.  Waves past the last chunk follow the barriers and store nothing.
template <int DV, bool WBF16>
__global__ void __launch_bounds__(64 * kLogitsWaves) logits_kernel(LogitsK a) {
  constexpr int HV = DV / 2;
  const int wave = threadIdx.x >> 6;
  // 1-D grid over (chunk group, run of gpb code groups), code groups fastest; the blocks
  // of one chunk group (which read the same z operand) share an XCD
  const int nbg = (a.nvg + a.gpb - 1) / a.gpb;
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int vg0 = (wid % nbg) * a.gpb, cg = wid / nbg;
  const int gc = cg * kLogitsWaves + wave;          // chunk over all requests
  const bool wvalid = gc < a.R * a.nchunk;
  const int r = wvalid ? gc / a.nchunk : 0, chunk = wvalid ? gc % a.nchunk : 0;
  const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
  const int b = chunk * 32 + m;
  const bool bvalid = wvalid && b < a.W;
  float* tm_r = a.tmax + size_t(r) * a.tmax_stride;
  const int code_lo = vg0 * a.cpw;
  const int code_hi = min(a.V, code_lo + a.gpb * a.cpw);

  float mrun = -INFINITY, srun = 0.0f, nrun = INFINITY;
  // tile maxima of the block, staged in LDS on the bf16 paths with z in registers (the
  // folds of the pair loop below then hold no branch) and written out, coalesced in
  // either layout, once their code group is done; two buffers, for code groups of even
  // and odd index
  constexpr bool STAGE_TM = WBF16 && DV <= 256;
  const int vt = (a.V + 31) >> 5;
  __shared__ float tms[STAGE_TM ? 2 * kMaxGroupTiles * kTmRow : 1];
  // request and first beam of each wave's chunk (request -1: no chunk), for the flush
  __shared__ int slot_r[STAGE_TM ? kLogitsWaves : 1], slot_b[STAGE_TM ? kLogitsWaves : 1];
  if constexpr (STAGE_TM) {
    if (lane == 0) {
      slot_r[wave] = wvalid ? r : -1;
      slot_b[wave] = chunk * 32;
    }
  }
  auto put_tm = [&](float tm, int c0) {
    if constexpr (STAGE_TM) {
      const int rel = c0 - code_lo;
      tms[((((rel >> a.cpw_shift) & 1) * kMaxGroupTiles) + ((rel & (a.cpw - 1)) >> 5)) * kTmRow + wave * 32 + m] = tm;
    } else if (hf == 0 && bvalid) {
      tm_r[a.beam_major ? size_t(b) * vt + (c0 >> 5) : size_t(c0 >> 5) * a.W + b] = tm;
    }
  };
  // fold of a tile whose 32 codes all exist: the same arithmetic as fold below, as
  // straight-line code (selects in place of its branches)
  // exp(x - m) as exp2(fma(x, log2 e, -m log2 e)): one rounding of the exact x log2 e -
  // round(m log2 e), an error of about |m| 2^-24 in the exponent, below 1e-7 relative for
  // |m| < 2 (and |m| 2^-24 absolute in the log-sum-exp, the size of the rounding of the
  // score itself)
  // fb: the logits are acc x fb (1 but for the two-term fp16 form, whose accumulators
  // carry the scale 2^(s + t_b)); lb = log2 e x fb
  auto fold_full = [&](const f32x16& acc, int c0, float fb, float lb) {
    float tm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tm = fmaxf(tm, acc[i]);
    tm = fmaxf(tm, __shfl_xor(tm, 32)) * fb;
    put_tm(tm, c0);
    nrun = fminf(nrun, tm);
    const bool up = tm > mrun;
    const float sc = mrun == -INFINITY ? 0.0f : srun * __builtin_amdgcn_exp2f((mrun - tm) * kLog2e);
    srun = up ? sc : srun;
    mrun = up ? tm : mrun;
    const float nml = -mrun * kLog2e;
#pragma unroll
    for (int i = 0; i < 16; ++i) srun += __builtin_amdgcn_exp2f(fmaf(acc[i], lb, nml));
  };
  auto fold = [&](const f32x16& acc, int c0, float fb, float lb) {
    const bool full = c0 + 32 <= a.V;              // block-uniform
    float tm = -INFINITY;
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) tm = fmaxf(tm, acc[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (c0 + 8 * (i >> 2) + 4 * hf + (i & 3) < a.V) tm = fmaxf(tm, acc[i]);
    }
    tm = fmaxf(tm, __shfl_xor(tm, 32)) * fb;       // code c0 is valid: tm is finite
    put_tm(tm, c0);
    nrun = fminf(nrun, tm);
    if (tm > mrun) {
      srun = mrun == -INFINITY ? 0.0f : srun * __builtin_amdgcn_exp2f((mrun - tm) * kLog2e);
      mrun = tm;
    }
    const float nml = -mrun * kLog2e;
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) srun += __builtin_amdgcn_exp2f(fmaf(acc[i], lb, nml));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (c0 + 8 * (i >> 2) + 4 * hf + (i & 3) < a.V)
          srun += __builtin_amdgcn_exp2f(fmaf(acc[i], lb, nml));
    }
  };

  // Code group g done: its tile maxima from LDS to tmax (all threads, after a barrier
  // that follows the group's last fold) ...
  auto flush_tm = [&](int g) {
    if constexpr (STAGE_TM) {
      const int glo = g * a.cpw, nt = (min(a.V, glo + a.cpw) - glo + 31) >> 5;
      const float* tb = tms + ((g - vg0) & 1) * kMaxGroupTiles * kTmRow;
      if (a.beam_major) {
        // 32 lanes per beam: one contiguous row of the group's tiles, 32 at a time
        const int t0 = threadIdx.x & 31;
        for (int bb = threadIdx.x >> 5; bb < kLogitsWaves * 32; bb += 2 * kLogitsWaves) {
          const int rs = slot_r[bb >> 5], bs = slot_b[bb >> 5] + (bb & 31);
          if (rs >= 0 && bs < a.W)
            for (int ti = t0; ti < nt; ti += 32)
              a.tmax[size_t(rs) * a.tmax_stride + size_t(bs) * vt + (glo >> 5) + ti] = tb[ti * kTmRow + bb];
        }
      } else {
        for (int e = threadIdx.x; e < nt * kLogitsWaves * 32; e += 64 * kLogitsWaves) {
          const int bb = e % (kLogitsWaves * 32), ti = e / (kLogitsWaves * 32);
          const int rs = slot_r[bb >> 5], bs = slot_b[bb >> 5] + (bb & 31);
          if (rs >= 0 && bs < a.W)
            a.tmax[size_t(rs) * a.tmax_stride + size_t((glo >> 5) + ti) * a.W + bs] = tb[ti * kTmRow + bb];
        }
      }
    }
  };
  // ... and its log-sum-exp part (the two lane halves of beam b merged), after which the
  // running state starts again for the next group
  auto flush_lse = [&](int g) {
    const float mo = __shfl_xor(mrun, 32), so = __shfl_xor(srun, 32);
    const float mm = fmaxf(mrun, mo);
    float ss = 0.0f;
    if (mrun != -INFINITY) ss += srun * __builtin_amdgcn_exp2f((mrun - mm) * kLog2e);
    if (mo != -INFINITY) ss += so * __builtin_amdgcn_exp2f((mo - mm) * kLog2e);
    if (hf == 0 && bvalid) a.lse_part[(size_t(r) * a.W_max + b) * a.nvg + g] = make_float4(mm, ss, nrun, 0.0f);
    mrun = -INFINITY;
    srun = 0.0f;
    nrun = INFINITY;
  };
  int tm_next = vg0;                                 // first group whose maxima are still in LDS

  // the bf16 codebook's two forms: z in two fp16 terms against the rescaled codebook
  // (F16), or in three bf16 terms; one instantiation runs, chosen per launch
  auto bf16_body = [&](auto f16c) {
    constexpr bool F16 = decltype(f16c)::value;
    constexpr int KS = DV / 16;
    constexpr int NTERM = F16 ? 2 : 3;             // MFMAs per k-step
    constexpr int RS = DV / 8 + 1;                 // LDS row stride in u32x4 (16 B pad)
    // the logits of tile j are acc x 2^-(t_b + s_j): the beam's factor, the tile's
    // exponents (staged in LDS with the first codebook tile)
    const float zsb = F16 ? (bvalid ? a.zscale[size_t(r) * a.W_max + b] : 1.0f) : 1.0f;
    __shared__ float tsf[F16 ? kMaxGroupTiles * kMaxGroupsPerBlock : 1];   // 2^-s_j of the block's tiles
    if constexpr (F16) {
      if (threadIdx.x < kMaxGroupTiles * kMaxGroupsPerBlock && code_lo + 32 * int(threadIdx.x) < code_hi)
        tsf[threadIdx.x] = ldexpf(1.0f, -a.tscale[(code_lo >> 5) + threadIdx.x]);
    }
    auto tfac = [&](int c0) { return F16 ? zsb * tsf[(c0 - code_lo) >> 5] : 1.0f; };
    // codebook tiles staged per barrier: two where the z operand leaves the registers
    constexpr int TPS = KS <= 8 ? 2 : 1;
    constexpr int NE = TPS * 32 * DV / 8;          // u32x4 per stage
    constexpr int PT = (NE + 64 * kLogitsWaves - 1) / (64 * kLogitsWaves);
    __shared__ u32x4 tile[2][TPS * 32 * RS];
    const u32x4* wt = static_cast<const u32x4*>(F16 ? a.woutT16 : a.woutT);
    // thread e-th entry of a tile: row e / (DV / 8), column e % (DV / 8); rows past the
    // codebook load code 0 (never used)
    // two register sets for tiles in flight (the pipelined path fetches two stages ahead)
    u32x4 stg[PT], stg2[PT];
    // (every thread has PT entries where NE is a multiple of the block: the loads are
    // then unconditional, and the compiler counts them exactly)
    constexpr bool ALL_E = NE % (64 * kLogitsWaves) == 0;
    auto fetch = [&](int c0, u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int e = threadIdx.x + u * 64 * kLogitsWaves;
        if (ALL_E || e < NE) {
          const int row = c0 + e / (DV / 8);
          dst[u] = wt[size_t(row < a.V ? row : 0) * (DV / 8) + e % (DV / 8)];
        }
      }
    };
    auto put = [&](int buf, const u32x4* src) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int e = threadIdx.x + u * 64 * kLogitsWaves;
        if (ALL_E || e < NE) tile[buf][(e / (DV / 8)) * RS + e % (DV / 8)] = src[u];
      }
    };
    const u32x4* zb = a.zf + zf_lane_base(r, a.nch_max, DV, chunk * 32, hf) + m;
    if constexpr (KS <= 16) {
      // the first tile's loads go out before the z operand's (loads complete in order,
      // so staging the tile then waits for those alone)
      fetch(code_lo, stg);
      u32x4 zh[KS], zm[KS], zl[F16 ? 1 : KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        zh[kk] = zb[(3 * kk) * 64];
        zm[kk] = zb[(3 * kk + 1) * 64];
        if constexpr (!F16) zl[kk] = zb[(3 * kk + 2) * 64];
      }
      put(0, stg);
      // wait for the whole z operand here, so that inside the loop only the prefetched
      // tile is waited for
      if constexpr (F16) asm volatile("" ::"v"(zm[KS - 1][0]));
      else asm volatile("" ::"v"(zl[KS - 1][0]));
      __syncthreads();
      if (code_lo + 32 * TPS < code_hi) fetch(code_lo + 32 * TPS, stg);
      // A fragments of tile `sub` of LDS buffer `buf`
      auto frags = [&](u32x4* w, int buf, int sub) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) w[kk] = tile[buf][(32 * sub + m) * RS + (HV / 8) * hf + kk];
      };
      auto mfma_tile = [&](int buf, int sub) {
        u32x4 w[KS];
        frags(w, buf, sub);
        return block_mfma_split<F16, KS>(w, zh, zm, zl);
      };
      // software pipeline over stages of two tiles (64 codes, one barrier): the MFMAs of
      // stage i + 1 are issued before the epilogue of stage i, so the matrix cores and
      // the VALU work at the same time.  Stage i + 1 is staged into the buffer stage
      // i - 1 used (every wave finished with it before the previous barrier).  A group
      // with an odd number of tiles computes one unused tile at its end.
      // (d_v = 256 holds twice the z operand: there the tiles go one after the other)
      if constexpr (KS <= 8) {
        f32x16 a0 = mfma_tile(0, 0), a1 = mfma_tile(0, 1);
        int buf = 0, c0 = code_lo;
        // the tiles of stage 1 are in flight in stg; those of stage 2 go into stg2: a
        // stage's tiles are fetched two passes before they are staged
        fetch(code_lo + 128, stg2);
        // stages with a successor: both of their tiles are whole, and the body is one
        // basic block in which the MFMAs of the next stage interleave with the folds of
        // this one (fetches are issued unconditionally on clamped rows; past the block's
        // codes they are never staged).  `slot` holds the next stage's tiles and then
        // takes those of the stage after the following one; the loop alternates stg and
        // stg2.
        auto stage = [&](u32x4* slot) __attribute__((always_inline)) {
          put(buf ^ 1, slot);
          __syncthreads();
          if (c0 != code_lo && (c0 & (a.cpw - 1)) == 0) {    // block-uniform: c0 opens a group
            flush_lse((c0 >> a.cpw_shift) - 1);
            flush_tm((c0 >> a.cpw_shift) - 1);
            tm_next = c0 >> a.cpw_shift;
            // the flush's stores complete here (vmcnt 0): with stores in flight the
            // compiler waits for every load before staging a tile, and the tiles of two
            // stages ahead are in flight here
            __builtin_amdgcn_s_waitcnt(0x0F70);
          }
          fetch(c0 + 192, slot);
          const float f0 = tfac(c0), f1 = tfac(c0 + 32);
          f32x16 n0, n1;
          if constexpr (F16) {
            // two fp16 terms: two MFMAs per A fragment.  Left to itself the compiler
            // reads each fragment into one register set and waits for it before its two
            // MFMAs, and the folds follow all of them.  So each tile's eight fragments
            // are read first, behind a scheduling barrier (the MFMAs then wait for them
            // in order), and its 16 MFMAs go out among the fold of one tile of the
            // stage before, four vector instructions after each (five or six: 2-5%
            // slower on stress; three: 1% slower).
            u32x4 w[KS];
            frags(w, buf ^ 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            n0 = block_mfma_split<F16, KS>(w, zh, zm, zl);
            fold_full(a0, c0, f0, kLog2e * f0);
#pragma unroll
            for (int i = 0; i < NTERM * KS; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
            }
            __builtin_amdgcn_sched_barrier(0);
            frags(w, buf ^ 1, 1);
            __builtin_amdgcn_sched_barrier(0);
            n1 = block_mfma_split<F16, KS>(w, zh, zm, zl);
            fold_full(a1, c0 + 32, f1, kLog2e * f1);
#pragma unroll
            for (int i = 0; i < NTERM * KS; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          } else {
            n0 = mfma_tile(buf ^ 1, 0);
            n1 = mfma_tile(buf ^ 1, 1);
            fold_full(a0, c0, f0, kLog2e * f0);
            fold_full(a1, c0 + 32, f1, kLog2e * f1);
#pragma unroll
            for (int i = 0; i < 2 * NTERM * KS; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three VALU
            }
          }
          a0 = n0;
          a1 = n1;
          buf ^= 1;
          c0 += 64;
        };
        // n stages with a successor, in pairs (one back edge: every load the loop
        // leaves in flight is then one the compiler can count), an odd one last
        const int n = (code_hi - code_lo + 63) / 64 - 1;
        for (int k = 0; k < (n >> 1); ++k) {
          stage(stg);
          stage(stg2);
        }
        if (n & 1) stage(stg);
        // the last stage may open a group: the previous group's maxima go out at the end
        if (c0 != code_lo && (c0 & (a.cpw - 1)) == 0) flush_lse((c0 >> a.cpw_shift) - 1);
        const float f0 = tfac(c0);
        fold(a0, c0, f0, kLog2e * f0);
        if (c0 + 32 < code_hi) {
          const float f1 = tfac(c0 + 32);
          fold(a1, c0 + 32, f1, kLog2e * f1);
        }
      } else if constexpr (F16) {
        // d_v = 256, two fp16 terms (z takes 128 registers): one tile per stage,
        // pipelined as above.  A tile's 16 fragments are read in two halves of eight
        // (the MFMAs keep their order, kk ascending); the first half's 16 MFMAs go out
        // among the fold of the tile before.  Tiles are fetched two stages ahead.
        static_assert(KS == 16, "d_v = 256");
        f32x16 a0 = mfma_tile(0, 0);
        int buf = 0, c0 = code_lo;
        fetch(code_lo + 64, stg2);
        auto stage = [&](u32x4* slot) __attribute__((always_inline)) {
          put(buf ^ 1, slot);
          __syncthreads();
          if (c0 != code_lo && (c0 & (a.cpw - 1)) == 0) {    // block-uniform: c0 opens a group
            flush_lse((c0 >> a.cpw_shift) - 1);
            flush_tm((c0 >> a.cpw_shift) - 1);
            tm_next = c0 >> a.cpw_shift;
            __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0): the flush's stores
          }
          fetch(c0 + 96, slot);
          const float f0 = tfac(c0);
          u32x4 w[8];
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) w[kk] = tile[buf ^ 1][m * RS + (HV / 8) * hf + kk];
          __builtin_amdgcn_sched_barrier(0);
          f32x16 n0 = block_mfma_split<F16, 8>(w, zh, zm, zl);
          fold_full(a0, c0, f0, kLog2e * f0);
#pragma unroll
          for (int i = 0; i < NTERM * 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) w[kk] = tile[buf ^ 1][m * RS + (HV / 8) * hf + 8 + kk];
          __builtin_amdgcn_sched_barrier(0);
          n0 = block_mfma_split<F16, 8>(w, zh + 8, zm + 8, zl, n0);
          __builtin_amdgcn_sched_barrier(0);
          a0 = n0;
          buf ^= 1;
          c0 += 32;
        };
        const int n = (code_hi - code_lo + 31) / 32 - 1;       // tiles with a successor
        for (int k = 0; k < (n >> 1); ++k) {
          stage(stg);
          stage(stg2);
        }
        if (n & 1) stage(stg);
        // the last tile may open a group: the previous group's maxima go out at the end
        if (c0 != code_lo && (c0 & (a.cpw - 1)) == 0) flush_lse((c0 >> a.cpw_shift) - 1);
        const float f0 = tfac(c0);
        fold(a0, c0, f0, kLog2e * f0);
      } else {
        int buf = 0;
        for (int c0 = code_lo; c0 < code_hi; c0 += 32) {
          const bool more = c0 + 32 < code_hi;       // block-uniform
          if (c0 != code_lo && (c0 & (a.cpw - 1)) == 0) {    // block-uniform: c0 opens a group
            flush_lse((c0 >> a.cpw_shift) - 1);
            flush_tm((c0 >> a.cpw_shift) - 1);
            tm_next = c0 >> a.cpw_shift;
            __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0): the flush's stores
          }
          const float f0 = tfac(c0);
          fold(mfma_tile(buf, 0), c0, f0, kLog2e * f0);
          if (more) {
            put(buf ^ 1, stg);
            __syncthreads();
            if (c0 + 64 < code_hi) fetch(c0 + 64, stg);
          }
          buf ^= 1;
        }
      }
    } else {
      // d_v > 256: the z operand does not fit in registers; each tile re-reads it in
      // chunks of eight k-steps (same MFMA order, kk ascending)
      constexpr int KZ = 8;
      fetch(code_lo, stg);
      put(0, stg);
      __syncthreads();
      int buf = 0;
      for (int c0 = code_lo; c0 < code_hi; c0 += 32) {
        const bool more = c0 + 32 < code_hi;         // block-uniform
        if (more) fetch(c0 + 32, stg);
        f32x16 acc = {};
#pragma unroll 1
        for (int k0 = 0; k0 < KS; k0 += KZ) {
          u32x4 zh[KZ], zm[KZ], zl[KZ], w[KZ];
#pragma unroll
          for (int kk = 0; kk < KZ; ++kk) {
            zh[kk] = zb[(3 * (k0 + kk)) * 64];
            zm[kk] = zb[(3 * (k0 + kk) + 1) * 64];
            zl[kk] = F16 ? zm[kk] : zb[(3 * (k0 + kk) + 2) * 64];
            w[kk] = tile[buf][m * RS + (HV / 8) * hf + k0 + kk];
          }
          acc = block_mfma_split<F16, KZ>(w, zh, zm, zl, acc);
        }
        const float f0 = tfac(c0);
        fold(acc, c0, f0, kLog2e * f0);
        if (more) put(buf ^ 1, stg);
        __syncthreads();
        buf ^= 1;
      }
    }
  };
  if constexpr (WBF16) {
    if (a.f16_on && *a.f16flag == 0u) bf16_body(std::true_type{});   // launch-uniform
    else bf16_body(std::false_type{});
  } else {
    const float* zr = a.z + (size_t(r) * a.W_max + (bvalid ? b : 0)) * DV + HV * hf;
    float zv[HV];
#pragma unroll
    for (int i = 0; i < HV; ++i) zv[i] = bvalid ? zr[i] : 0.0f;
    const float* wt = static_cast<const float*>(a.woutT);
    for (int c0 = code_lo; c0 < code_hi; c0 += 32)
      fold(block_mfma_f32<DV>(wt, c0 + m, a.V, hf, zv), c0, 1.0f, kLog2e);
  }
  // the block's last group (and a group the last stage closed)
  const int g_last = (code_hi - 1) >> a.cpw_shift;
  if constexpr (STAGE_TM) {
    __syncthreads();
    for (int g = tm_next; g <= g_last; ++g) flush_tm(g);
  }
  flush_lse(g_last);
}

// ---------------------------------------------------------------- block-wide radix and sort helpers

// The range [lo, hi] is split into 2048 digits of width 2^shift.
__device__ __forceinline__ int first_shift(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  const int bits = span ? 32 - __clz(span) : 0;
  return bits > 11 ? bits - 11 : 0;
}

// Shared scalars of the 1024-thread select blocks.
struct RadixSh {
  uint32_t lo, hi, need, cnt;
  int shift;
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = uint32_t(__shfl_up(int(x), off));
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive prefix sum of v over a 1024-thread block in thread order; `total` gets
// the block sum.  Two barriers; wsum[16] is scratch.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  const uint32_t wx = wave_incl_scan(lane < 16 ? wsum[lane] : 0u);
  const uint32_t before = uint32_t(__shfl(int(wx), (wv + 63) & 63));
  total = uint32_t(__shfl(int(wx), 15));
  __syncthreads();
  return x - v + (wv ? before : 0u);
}

// Block of 1024 threads, hist[2048] complete: find the digit of [lo, lo + 2048 << shift)
// that holds the need-th largest key and leave in sh its range, the count still to take
// inside it and the next digit width (-1 once the digit is a single value).  Thread t
// owns digits 2047 - 2t and 2046 - 2t: the keys above them are a prefix sum.  If the
// histogram holds fewer than `need` keys (inconsistent input, e.g. NaN scores), sh ends
// the search (shift -1, nothing more to take): every caller's loop terminates and the
// shortfall shows up as fewer winners than asked for.
__device__ void pick_digit(const uint32_t* hist, uint32_t* wsum, uint32_t lo, uint32_t hi, int shift,
                           uint32_t need, RadixSh& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sh.lo = lo;
    sh.hi = lo;
    sh.need = 0u;
    sh.shift = -1;
  }
  const uint32_t c0 = hist[kHistBins - 1 - 2 * tid], c1 = hist[kHistBins - 2 - 2 * tid];
  uint32_t total;
  uint32_t above = block_excl_scan(c0 + c1, wsum, total);
  for (int i = 0; i < 2; ++i) {
    const uint32_t ci = i ? c1 : c0;
    if (above < need && need <= above + ci) {
      const uint32_t d = uint32_t(kHistBins - 1 - (2 * tid + i));
      const uint32_t nlo = lo + (d << shift);
      const uint64_t top = uint64_t(nlo) + (uint64_t(1) << shift) - 1;
      sh.lo = nlo;
      sh.hi = top < hi ? uint32_t(top) : hi;
      sh.need = need - above;
      sh.shift = shift == 0 ? -1 : (shift > 11 ? shift - 11 : 0);
    }
    above += ci;
  }
  __syncthreads();
}

// Radix passes inside [lo, hi] over n keys (key_at(i)) until one key value remains:
// returns theta, the value of the need-th largest key; `need` becomes the number of
// keys equal to theta still to take.  Every thread of the 1024-thread block calls it.
template <typename KeyAt>
__device__ uint32_t radix_finish(KeyAt key_at, uint32_t n, uint32_t lo, uint32_t hi, uint32_t& need,
                                 int shift, uint32_t* hist, uint32_t* wsum, RadixSh& sh) {
  const int tid = threadIdx.x;
  while (shift >= 0) {
    for (int i = tid; i < kHistBins; i += 1024) hist[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += 1024) {
      const uint32_t key = key_at(i);
      if (key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
    }
    __syncthreads();
    pick_digit(hist, wsum, lo, hi, shift, need, sh);
    lo = sh.lo; hi = sh.hi; need = sh.need; shift = sh.shift;
    __syncthreads();
  }
  return lo;
}

// Among the keys equal to theta, the need-th smallest flat index (radix over the flat
// index, 8 bits a pass); all of them when need covers every tie (returns ~0).
template <typename KeyAt, typename FlatAt>
__device__ uint32_t tie_cut(KeyAt key_at, FlatAt flat_at, uint32_t n, uint32_t theta, uint32_t need,
                            uint32_t* hist, RadixSh& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.cnt = 0;
  __syncthreads();
  uint32_t mine = 0;
  for (uint32_t i = tid; i < n; i += 1024) mine += key_at(i) == theta;
  if (mine) atomicAdd(&sh.cnt, mine);
  __syncthreads();
  const uint32_t n_eq = sh.cnt;
  __syncthreads();
  if (need >= n_eq) return 0xFFFFFFFFu;
  uint32_t pre = 0, nd = need;
  for (int s = 24; s >= 0; s -= 8) {
    for (int i = tid; i < 256; i += 1024) hist[i] = 0;
    __syncthreads();
    const uint32_t himask = s == 24 ? 0u : (0xFFFFFFFFu << (s + 8));
    for (uint32_t i = tid; i < n; i += 1024) {
      if (key_at(i) != theta) continue;
      const uint32_t f = flat_at(i);
      if ((f & himask) == (pre & himask)) atomicAdd(&hist[(f >> s) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // the digit holding the nd-th entry: lane l sums digits 4l .. 4l + 3, an inclusive
      // scan over the lanes, and the lane whose range holds nd resolves its four
      const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2],
                     h3 = hist[4 * tid + 3];
      const uint32_t own = h0 + h1 + h2 + h3;
      uint32_t incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = uint32_t(__shfl_up(int(incl), off));
        if (tid >= off) incl += y;
      }
      const uint32_t excl = incl - own;
      const uint64_t hit = __ballot(excl < nd && nd <= incl);
      if (tid == 0 && !hit) { sh.lo = pre; sh.need = nd; }     // no digit: nothing changes
      if (hit && tid == __ffsll((long long)hit) - 1) {
        uint32_t below = excl, d = 4 * tid;
        if (nd > below + h0) {
          below += h0; ++d;
          if (nd > below + h1) {
            below += h1; ++d;
            if (nd > below + h2) { below += h2; ++d; }
          }
        }
        sh.lo = pre | (d << s);
        sh.need = nd - below;
      }
    }
    __syncthreads();
    pre = sh.lo;
    nd = sh.need;
    __syncthreads();
  }
  return pre;
}

template <int J>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v) {
  return (uint64_t(lane_xor<J>(uint32_t(v >> 32))) << 32) | lane_xor<J>(uint32_t(v));
}

// One compare-exchange of a bitonic network inside a wave: partner lane ^ J; this
// lane keeps the larger entry iff desc == ((lane & J) == 0).
template <int J>
__device__ __forceinline__ uint64_t bitonic_cx(uint64_t v, bool desc) {
  const uint64_t o = lane_xor64<J>(v);
  const bool lower = (threadIdx.x & J) == 0;
  return (desc == lower) ? (v > o ? v : o) : (v < o ? v : o);
}

// Merge of bitonic runs of k = 2^LK lanes: runs with (lane & k) == 0 end descending.
template <int LK>
__device__ __forceinline__ uint64_t wave_merge(uint64_t v) {
  constexpr int k = 1 << LK;
  const bool desc = LK == 6 || (threadIdx.x & k) == 0;
  if constexpr (LK >= 6) v = bitonic_cx<32>(v, desc);
  if constexpr (LK >= 5) v = bitonic_cx<16>(v, desc);
  if constexpr (LK >= 4) v = bitonic_cx<8>(v, desc);
  if constexpr (LK >= 3) v = bitonic_cx<4>(v, desc);
  if constexpr (LK >= 2) v = bitonic_cx<2>(v, desc);
  return bitonic_cx<1>(v, desc);
}

// The first np (a power of two <= 64) lanes of the wave sorted descending (lane 0
// the largest); lanes past np sort their own entries among themselves.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v, int np) {
  if (np >= 2) v = wave_merge<1>(v);
  if (np >= 4) v = wave_merge<2>(v);
  if (np >= 8) v = wave_merge<3>(v);
  if (np >= 16) v = wave_merge<4>(v);
  if (np >= 32) v = wave_merge<5>(v);
  if (np >= 64) v = wave_merge<6>(v);
  return v;
}

// Number of entries above v in the NW sorted runs of 64 other than run w: a binary
// search in every run at once (run w is searched too and ignored), so that the NW
// reads of a step issue together.
template <int NW>
__device__ __forceinline__ uint32_t count_above(uint64_t v, const uint64_t* runs, int w) {
  uint32_t c[NW];
#pragma unroll
  for (int u = 0; u < NW; ++u) c[u] = 0u;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    uint64_t x[NW];
#pragma unroll
    for (int u = 0; u < NW; ++u) x[u] = runs[u * 64 + c[u] + s - 1];
#pragma unroll
    for (int u = 0; u < NW; ++u) c[u] += x[u] > v ? uint32_t(s) : 0u;
  }
  uint64_t y[NW];
#pragma unroll
  for (int u = 0; u < NW; ++u) y[u] = runs[u * 64 + 63];
  uint32_t above = 0u;
#pragma unroll
  for (int u = 0; u < NW; ++u)
    if (u != w) above += c[u] + (c[u] == 63u && y[u] > v);   // the search caps at 63
  return above;
}

// Block-wide descending sort of n <= 1024 distinct nonzero entries, entry i held by
// thread i < n (other threads hold anything).  Each wave holding entries sorts them in
// its lanes and lays the run out in `runs`; an entry's rank is its place in its own
// run plus the entries above it in every other run.  Returns entry i in thread i < n,
// 0 past n.  `runs` and `out` may be arrays the entries were read from before the call.
__device__ __forceinline__ uint64_t rank_sort_desc(uint64_t v, int n, uint64_t* runs, uint64_t* out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = (n + 63) >> 6;
  if (tid >= n) v = 0ull;                                 // padding sorts last in every run
  if (nw <= 1) {                                          // one run: sorted in place
    int np = 1;
    while (np < n) np <<= 1;
    return w == 0 ? wave_sort_desc(v, np) : 0ull;
  }
  if (w < nw) v = wave_sort_desc(v, 64);
  __syncthreads();
  if (w < nw) runs[tid] = v;
  __syncthreads();
  if (w < nw) {
    uint32_t above = 0u;
    switch (nw) {
      case 2: above = count_above<2>(v, runs, w); break;
      case 3: above = count_above<3>(v, runs, w); break;
      case 4: above = count_above<4>(v, runs, w); break;
      case 5: above = count_above<5>(v, runs, w); break;
      case 6: above = count_above<6>(v, runs, w); break;
      case 7: above = count_above<7>(v, runs, w); break;
      case 8: above = count_above<8>(v, runs, w); break;
      case 9: above = count_above<9>(v, runs, w); break;
      case 10: above = count_above<10>(v, runs, w); break;
      case 11: above = count_above<11>(v, runs, w); break;
      case 12: above = count_above<12>(v, runs, w); break;
      case 13: above = count_above<13>(v, runs, w); break;
      case 14: above = count_above<14>(v, runs, w); break;
      case 15: above = count_above<15>(v, runs, w); break;
      default: above = count_above<16>(v, runs, w); break;
    }
    if (v != 0ull) out[lane + above] = v;                 // lane + above < 64 nw <= 1024
  }
  __syncthreads();
  return tid < n ? out[tid] : 0ull;
}

// ---------------------------------------------------------------- tile select

struct TileSelK {
  int W, W_max, Vt, K, K_full, G_max, nvg;
  int tg_shift;            // log2 of the tiles in one code group of the first pass
  size_t stride;           // tile maxima / kept tiles per request (n_tiles(V_max) * W_max)
  const float* tmax;       // per request [Vt][W], beam-major [W][Vt] when bounded
  const float4* lse_part;  // [R,W_max,nvg]
  const float* cum;        // [R,W_max] of step t
  float* lse;              // [R,W_max] out
  SelState* sel;           // n_tiles, n_groups out
  uint32_t* cand;          // [R,stride] tiles inside the boundary digit
  uint32_t* tiles;         // [R,W_max] chosen flat tiles b * Vt + j, grouped by j
  uint32_t* groups;        // [R,G_max] start | count << 10 | j << 16
  uint32_t* gtiles;        // [R,G_max,32] the tiles of each group (refinement operands)
  int32_t* status;
};

// One 1024-thread block per request.
//  1. log-sum-exp of every beam from its parts; the request's tile-key range (the
//     score is monotone in the logit: the largest logit and the smallest tile maximum
//     of each row bound its tile keys).
//  2. A lower bound theta0 on the K-th largest tile key: each code group's largest
//     logit is one of its tile maxima, so the W * nvg group keys are keys of distinct
//     tiles, and the low edge of the histogram digit holding the K-th largest of them
//     has at least K tile keys at or above it.  Per beam, the smallest tile-maximum key
//     whose tile key reaches theta0 (the key is monotone in the logit).
//  3. One pass over all tile maxima: those at or above their beam's threshold (a few
//     more than K) go to an LDS list with their keys; when the list overflows, the
//     passes below read every tile instead.
//  4. Over the list: 2048-digit histogram, the digit holding the K-th largest key;
//     keys above the digit are chosen, keys inside it are kept.
//  5. The rest of the K inside the digit, ties by flat tile index: one sort of the kept
//     tiles when at most 1024 (the usual case: a handful), else a radix finish.
//  6. Counting sort of the K chosen tiles by code tile j, cut into groups of at most
//     32 beams: one MFMA block of the refinement each.
template <bool BOUNDED>
__global__ void __launch_bounds__(1024) tile_select_kernel(TileSelK a) {
  __shared__ float lse_s[kMaxW], cum_s[kMaxW];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t fill[kHistBins];
  __shared__ uint32_t jstart[kHistBins];
  __shared__ uint32_t chosen[kMaxW];
  __shared__ uint64_t cs[kMaxW], xs[kMaxW];                // kept tiles as (key, ~flat); sorted
  __shared__ uint32_t wsum[16];
  __shared__ RadixSh sh;
  __shared__ uint32_t kmin_sh, kmax_sh, nwin_sh, ncand_sh, theta_sh, nlist_sh;
  __shared__ uint32_t kthr_s[BOUNDED ? kMaxW : 1];         // per beam: least passing tile-max key
  __shared__ uint64_t list[BOUNDED ? kSelList : 1];        // (key, ~flat) at or above theta0
  __shared__ uint32_t pairs[BOUNDED ? kSelPairs : 1];      // (beam << 16 | group) that can pass
  const int r = blockIdx.x, tid = threadIdx.x;
  const int W = a.W;
  const uint32_t Vt = uint32_t(a.Vt), K = uint32_t(a.K);
  const float* tm = a.tmax + size_t(r) * a.stride;
  uint32_t* cand = a.cand + size_t(r) * a.stride;
  const size_t cap = size_t(Vt) * W;

  // Bounded (the launcher's choice where a request's tiles outnumber the list): the
  // tile maxima are beam-major, and the bounded pass below reads only the code groups
  // that can hold a tile above the bound; else they are tile-major and read twice, by
  // the passes over every tile.
  constexpr bool bounded = BOUNDED;
  auto tm_at = [&](int bb, int jj) { return bounded ? size_t(bb) * Vt + jj : size_t(jj) * W + bb; };
  // thread -> one beam b and every G-th tile from jg; its first U tiles are loaded now,
  // under the log-sum-exp phase, and kept for the passes (not in the bounded mode)
  constexpr int U = 16;
  const int G = 1024 / W;
  const bool act = tid < G * W;
  const int b = act ? tid % W : 0, jg = act ? tid / W : 0;
  float x0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int jj = jg + u * G;
    x0[u] = !bounded && act && jj < a.Vt ? tm[tm_at(b, jj)] : 0.0f;
  }
  // the first eight log-sum-exp parts and the cumulative score of beam tid are loaded
  // before the first barrier too (a barrier waits for every load in flight)
  const float4* lp = a.lse_part + (size_t(r) * a.W_max + (tid < W ? tid : 0)) * a.nvg;
  float4 q[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    q[u] = tid < W && u < a.nvg ? lp[u] : make_float4(-INFINITY, 0.0f, INFINITY, 0.0f);
  const float c = tid < W ? a.cum[size_t(r) * a.W_max + tid] : 0.0f;
  if (tid == 0) { kmin_sh = 0xFFFFFFFFu; kmax_sh = 0u; nwin_sh = 0u; ncand_sh = 0u; nlist_sh = 0u; }
  for (int i = tid; i < kHistBins; i += 1024) hist[i] = 0;
  __syncthreads();
  float lt = 0.0f;                                        // log-sum-exp of beam tid
  {
    uint32_t kmx = 0u, kmn = 0xFFFFFFFFu;
    if (tid < W) {
      float mm = -INFINITY, mn = INFINITY, s = 0.0f;
      for (int g0 = 0; g0 < a.nvg; g0 += 8) {
        if (g0 > 0) {
#pragma unroll
          for (int u = 0; u < 8; ++u)
            q[u] = g0 + u < a.nvg ? lp[g0 + u] : make_float4(-INFINITY, 0.0f, INFINITY, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          mn = fminf(mn, q[u].z);
          if (q[u].x > mm) {
            s = mm == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f((mm - q[u].x) * kLog2e);
            mm = q[u].x;
          }
          if (q[u].x != -INFINITY) s += q[u].y * __builtin_amdgcn_exp2f((q[u].x - mm) * kLog2e);
        }
      }
      const float l = mm + logf(s);
      lt = l;
      lse_s[tid] = l;
      cum_s[tid] = c;
      a.lse[size_t(r) * a.W_max + tid] = l;
      kmx = f2key(cand_score(c, mm, l));
      kmn = f2key(cand_score(c, mn, l));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      kmx = max(kmx, uint32_t(__shfl_xor(int(kmx), off)));
      kmn = min(kmn, uint32_t(__shfl_xor(int(kmn), off)));
    }
    if ((tid & 63) == 0) { atomicMax(&kmax_sh, kmx); atomicMin(&kmin_sh, kmn); }
  }
  __syncthreads();
  const uint32_t kmin = kmin_sh, kmax = kmax_sh;
  const int shift0 = first_shift(kmin, kmax);

  // ---- bounded mode: theta0 from the code groups' largest and smallest tile maxima (hist
  // is clear), then each beam's threshold on its tile maxima.  A group of n tiles has one
  // tile at its largest tile maximum and n - 1 others at or above its smallest, so the
  // multiset {max key once, min key n - 1 times} over all groups is dominated tile by tile
  // by the true tile keys, and its K-th largest key is a lower bound on theirs (where the
  // top-K concentrates in a few beams, counting one tile per group would be far looser)
  uint32_t theta0 = kmin;
  if constexpr (bounded) {
    if (tid < W) {
      const float c = cum_s[tid];
      const int tpg = 1 << a.tg_shift;
      auto add = [&](int u, float gx, float gn) {
        const int n = min(tpg, a.Vt - u * tpg);
        const uint32_t kx = f2key(cand_score(c, gx, lt)), kn = f2key(cand_score(c, gn, lt));
        if (kx >= kmin && kx <= kmax) atomicAdd(&hist[(kx - kmin) >> shift0], 1u);
        if (n > 1 && kn >= kmin && kn <= kmax) atomicAdd(&hist[(kn - kmin) >> shift0], uint32_t(n - 1));
      };
      if (a.nvg <= 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (u < a.nvg) add(u, q[u].x, q[u].z);
      } else {
        for (int u = 0; u < a.nvg; ++u) {
          const float4 p = lp[u];
          add(u, p.x, p.z);
        }
      }
    }
    __syncthreads();
    pick_digit(hist, wsum, kmin, kmax, shift0, K, sh);
    theta0 = sh.lo;                                       // kmin when the counts fall short
    for (int i = tid; i < kHistBins; i += 1024) hist[i] = 0;
    if (tid < W) {
      // the least tile-maximum key x whose tile key reaches theta0, by bisection over
      // the keys of -inf .. +inf (tile maxima are never NaN); 0 (every tile tested by
      // its key) for a beam whose cumulative score or log-sum-exp is not finite
      const float c = cum_s[tid];
      uint32_t kt = 0u;
      if (theta0 > kmin && __builtin_isfinite(c) && __builtin_isfinite(lt)) {
        auto reach = [&](uint32_t kx) { return f2key(cand_score(c, key2f(kx), lt)) >= theta0; };
        uint32_t lo = 0x007FFFFFu, hi = 0xFF800000u;      // keys of -inf and +inf
        if (!reach(lo)) {
          if (!reach(hi)) {
            kt = 0xFFFFFFFFu;
          } else {
            while (hi - lo > 1u) {
              const uint32_t mid = lo + ((hi - lo) >> 1);
              if (reach(mid)) hi = mid;
              else lo = mid;
            }
            kt = hi;
          }
        }
      }
      kthr_s[tid] = kt;
    }
    __syncthreads();
  }

  const float cb = cum_s[b], lb = lse_s[b];
  // every tile of this thread's beam b: f(key, j)
  auto stream = [&](auto&& f) {
    if (!act) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = jg + u * G;
      if (jj < a.Vt) f(f2key(cand_score(cb, bounded ? tm[tm_at(b, jj)] : x0[u], lb)), jj);
    }
    // the rest in batches of UB loads in flight (large codebooks: up to 256 per thread)
    constexpr int UB = 32;
    for (int j = jg + U * G; j < a.Vt; j += UB * G) {
      float x[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int jj = j + u * G;
        x[u] = jj < a.Vt ? tm[tm_at(b, jj)] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int jj = j + u * G;
        if (jj < a.Vt) f(f2key(cand_score(cb, x[u], lb)), jj);
      }
    }
  };
  // the split of one key: above the boundary digit chosen, inside it kept
  uint32_t lo, hi, need;
  int shift1;
  auto split = [&](uint32_t key, uint32_t flat) {
    if (key < lo) return;
    if (key > hi) {
      const uint32_t p = atomicAdd(&nwin_sh, 1u);
      if (p < uint32_t(kMaxW)) chosen[p] = flat;
    } else {
      const uint32_t p = atomicAdd(&ncand_sh, 1u);
      if (p < cap) cand[p] = flat;
      if (p < uint32_t(kMaxW)) cs[p] = (uint64_t(key) << 32) | uint64_t(0xFFFFFFFFu - flat);
    }
  };
  bool use_list = false;
  if constexpr (bounded) {
    // ---- the list: the (beam, group) pairs whose group maximum reaches the beam's
    // threshold, compacted by one block scan; then the tiles of those group rows
    // (consecutive lanes on consecutive tiles of a row) whose tile-maximum key
    // reaches the threshold and whose key reaches theta0.  Too many pairs (ties):
    // every tile of every beam is tested.
    uint32_t npairs;
    {
      uint32_t gw[kMaxGroupsMask / 32] = {};
      uint32_t cnt = 0u;
      if (tid < W) {
        const uint32_t kt = kthr_s[tid];
        auto mark = [&](int u, float gx) {
          if (f2key(gx) >= kt) { gw[u >> 5] |= 1u << (u & 31); ++cnt; }
        };
        if (a.nvg <= 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (u < a.nvg) mark(u, q[u].x);
        } else if (a.nvg <= kMaxGroupsMask) {
          for (int u = 0; u < a.nvg; ++u) mark(u, lp[u].x);
        } else {
          cnt = uint32_t(kSelPairs) + 1u;                 // no mask: every tile
        }
      }
      uint32_t off = block_excl_scan(cnt, wsum, npairs);
      if (npairs <= uint32_t(kSelPairs) && tid < W) {
        for (int u = 0; u < a.nvg; ++u)
          if ((gw[u >> 5] >> (u & 31)) & 1u) pairs[off++] = (uint32_t(tid) << 16) | uint32_t(u);
      }
      __syncthreads();
    }
    auto test = [&](float x, int bb, int jj) {
      if (f2key(x) < kthr_s[bb]) return;
      const uint32_t key = f2key(cand_score(cum_s[bb], x, lse_s[bb]));
      if (key < theta0) return;
      const uint32_t p = atomicAdd(&nlist_sh, 1u);
      if (p < uint32_t(kSelList))
        list[p] = (uint64_t(key) << 32) | uint64_t(0xFFFFFFFFu - (uint32_t(bb) * Vt + uint32_t(jj)));
    };
    if (npairs <= uint32_t(kSelPairs)) {
      const int ts = a.tg_shift, tpg = 1 << ts;
      const int nitem = int(npairs) << ts;
      constexpr int UB = 16;
      for (int i0 = 0; i0 < nitem; i0 += UB * 1024) {
        float x[UB];
        int ib[UB], ij[UB];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int it = i0 + u * 1024 + tid;
          const uint32_t pr = pairs[it < nitem ? it >> ts : 0];
          ib[u] = int(pr >> 16);
          ij[u] = (int(pr & 0xFFFFu) << ts) + (it & (tpg - 1));
          const bool live = it < nitem && ij[u] < a.Vt;
          x[u] = tm[live ? tm_at(ib[u], ij[u]) : 0];
          ib[u] = live ? ib[u] : -1;
        }
#pragma unroll
        for (int u = 0; u < UB; ++u)
          if (ib[u] >= 0) test(x[u], ib[u], ij[u]);
      }
    } else if (act) {
      // every tile of this thread's beam
      for (int j0 = jg; j0 < a.Vt; j0 += 32 * G) {
        float x[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int jj = j0 + u * G;
          x[u] = jj < a.Vt ? tm[tm_at(b, jj)] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int jj = j0 + u * G;
          if (jj < a.Vt) test(x[u], b, jj);
        }
      }
    }
    __syncthreads();
    const uint32_t nlist = nlist_sh;
    use_list = nlist <= uint32_t(kSelList);               // block-uniform
    if (use_list) {
      const int sh0 = first_shift(theta0, kmax);
      for (uint32_t p = tid; p < nlist; p += 1024) {
        const uint32_t key = uint32_t(list[p] >> 32);
        if (key <= kmax) atomicAdd(&hist[(key - theta0) >> sh0], 1u);
      }
      __syncthreads();
      pick_digit(hist, wsum, theta0, kmax, sh0, K, sh);
      lo = sh.lo; hi = sh.hi; need = sh.need; shift1 = sh.shift;
      __syncthreads();
      for (uint32_t p = tid; p < nlist; p += 1024) {
        const uint64_t e = list[p];
        split(uint32_t(e >> 32), 0xFFFFFFFFu - uint32_t(e));
      }
    }
  }
  if (!use_list) {
    // ---- every tile: 2048-digit histogram over the key range, then the split
    stream([&](uint32_t key, int) {
      if (key >= kmin && key <= kmax) atomicAdd(&hist[(key - kmin) >> shift0], 1u);
    });
    __syncthreads();
    pick_digit(hist, wsum, kmin, kmax, shift0, K, sh);
    lo = sh.lo; hi = sh.hi; need = sh.need; shift1 = sh.shift;
    __syncthreads();
    stream([&](uint32_t key, int j) { split(key, uint32_t(b) * Vt + uint32_t(j)); });
  }
  __syncthreads();
  const uint32_t n_cand = min(ncand_sh, uint32_t(cap));
  uint32_t theta, nwin;
  if (n_cand <= uint32_t(kMaxW)) {
    // sorted as (key, ~flat) descending, the first `need` kept tiles complete the K
    const uint32_t above = nwin_sh;
    const uint64_t v = rank_sort_desc(uint32_t(tid) < n_cand ? cs[tid] : 0ull, int(n_cand), cs, xs);
    const uint32_t take = min(need, n_cand);
    if (uint32_t(tid) < take && above + tid < uint32_t(kMaxW)) chosen[above + tid] = 0xFFFFFFFFu - uint32_t(v);
    if (uint32_t(tid) + 1 == take) theta_sh = uint32_t(v >> 32);
    __syncthreads();
    theta = take ? theta_sh : lo;
    nwin = above + take;
  } else {
    auto key_at = [&](uint32_t i) {
      const uint32_t f = cand[i];
      const uint32_t bb = f / Vt;
      return f2key(cand_score(cum_s[bb], tm[tm_at(int(bb), int(f % Vt))], lse_s[bb]));
    };
    auto flat_at = [&](uint32_t i) { return cand[i]; };
    theta = radix_finish(key_at, n_cand, lo, hi, need, shift1, hist, wsum, sh);
    const uint32_t phi = tie_cut(key_at, flat_at, n_cand, theta, need, hist, sh);
    for (uint32_t i = tid; i < n_cand; i += 1024) {
      const uint32_t f = cand[i];
      const uint32_t key = key_at(i);
      if (key > theta || (key == theta && f <= phi)) {
        const uint32_t p = atomicAdd(&nwin_sh, 1u);
        if (p < uint32_t(kMaxW)) chosen[p] = f;
      }
    }
    __syncthreads();
    nwin = nwin_sh;
  }
  // the K-th tile key bounds the K-th candidate key from below when K tiles are chosen
  if (tid == 0) a.sel[r].theta = a.K == a.K_full ? theta : 0u;
  for (int j = tid; j < kHistBins; j += 1024) hist[j] = 0;
  __syncthreads();
  const uint32_t got = min(nwin, K);
  if (tid == 0 && nwin != K) atomicOr(a.status, 2);
  for (uint32_t p = tid; p < got; p += 1024) atomicAdd(&hist[chosen[p] % Vt], 1u);
  __syncthreads();
  // exclusive scans over j of the counts (low 16 bits) and the group counts (high 16)
  const uint32_t n0 = hist[2 * tid], n1 = hist[2 * tid + 1];
  const uint32_t g0 = (n0 + 31) / 32, g1 = (n1 + 31) / 32;
  const uint32_t v = (n0 + n1) | ((g0 + g1) << 16);
  uint32_t total;
  const uint32_t ex = block_excl_scan(v, wsum, total);
  const uint32_t s0 = ex & 0xFFFFu, gs0 = ex >> 16;
  const uint32_t s1 = s0 + n0, gs1 = gs0 + g0;
  if (tid == 0) {
    a.sel[r].n_groups = total >> 16;
    a.sel[r].n_tiles = got;
  }
  fill[2 * tid] = s0;
  fill[2 * tid + 1] = s1;
  jstart[2 * tid] = s0;
  jstart[2 * tid + 1] = s1;
  hist[2 * tid] = gs0;                          // first group of code tile j
  hist[2 * tid + 1] = gs1;
  uint32_t* grp = a.groups + size_t(r) * a.G_max;
  for (uint32_t q = 0; q < g0; ++q)
    grp[gs0 + q] = (s0 + 32 * q) | (min(32u, n0 - 32 * q) << 10) | (uint32_t(2 * tid) << 16);
  for (uint32_t q = 0; q < g1; ++q)
    grp[gs1 + q] = (s1 + 32 * q) | (min(32u, n1 - 32 * q) << 10) | (uint32_t(2 * tid + 1) << 16);
  __syncthreads();
  uint32_t* tl = a.tiles + size_t(r) * a.W_max;
  uint32_t* gt = a.gtiles + size_t(r) * a.G_max * 32;
  for (uint32_t p = tid; p < got; p += 1024) {
    const uint32_t f = chosen[p], j = f % Vt;
    const uint32_t q = atomicAdd(&fill[j], 1u), off = q - jstart[j];
    tl[q] = f;
    gt[(hist[j] + off / 32) * 32 + off % 32] = f;
  }
}

// ---------------------------------------------------------------- refinement

struct RefineK {
  int W, W_max, V, Vt, G_max, nch_max;
  const float* z;
  const u32x4* zf;
  const void* woutT;
  const float* lse;
  const float* cum;
  const SelState* sel;
  const uint32_t* groups;
  const uint32_t* gtiles;
  uint32_t* rkeys;       // [R,W_max,32]: keys of the chosen tiles' candidates (0: no code)
  const void* woutT16;   // [V,DV] fp16, tile j scaled by 2^s_j (two-term form)
  const float* zscale;   // [R,W_max] 2^-t_b (two-term form)
  const int32_t* tscale; // [n_tiles(V)] s_j
  const uint32_t* f16flag; // set: the three-term form
  int f16_on;            // the two-term form may be used
  int forced_blocks;     // first blocks: the forced candidates' logits (32 per block)
  int K;                 // forced candidates per request (W_next)
  const int32_t *forced_parent, *forced_token;   // [R,K] (or null)
  float* flog;           // [R,W_max] logits of the forced candidates
  int32_t* status;
};

// Logit of forced candidate i of request r (forced_parent[r, i], forced_token[r, i]) into
// flog[r, i]: an fp32 dot product of z (rebuilt exactly from its three bf16 parts for a
// bf16 codebook) and the code's row.  Eight lanes take one candidate, each a strided set
// of 8-element units of d_v read as 16-byte pieces, and add their partial sums; every
// load of a wave is issued at once.  Out-of-range entries are clamped and flagged
// (status bit 0).
template <int DV, bool WBF16>
__device__ __forceinline__ void forced_logit8(const RefineK& a, int r, int i) {
  constexpr int NU = DV / 8;                               // 8-element units of d_v
  constexpr int UPL = (NU + 7) / 8;                        // units per lane
  constexpr int HV = DV / 2;
  const int j = threadIdx.x & 7;
  const bool live = i < a.K;
  const size_t o = size_t(r) * a.K + (live ? i : 0);
  int b = a.forced_parent[o], c = a.forced_token[o];
  if (b < 0 || b >= a.W || c < 0 || c >= a.V) {
    if (live && j == 0) atomicOr(a.status, 1);
    b = b < 0 ? 0 : (b >= a.W ? a.W - 1 : b);
    c = c < 0 ? 0 : (c >= a.V ? a.V - 1 : c);
  }
  float zd[UPL][8], wd[UPL][8];
  // z from its operand terms: (h + l) 2^-t (exact: h + l has 22 significant bits) for the
  // two-term fp16 form, (hi + mid) + lo for the three bf16 terms
  const bool f16 = WBF16 && a.f16_on && *a.f16flag == 0u;
  const float zs = f16 ? a.zscale[size_t(r) * a.W_max + b] : 1.0f;
#pragma unroll
  for (int q = 0; q < UPL; ++q) {
    const int u = j + 8 * q;
    const int d0 = 8 * (u < NU ? u : 0);                   // elements d0 .. d0 + 7
    if constexpr (WBF16) {
      const int hf = d0 / HV, kk = (d0 % HV) / 8;
      const u32x4* p = a.zf + zf_lane_base(r, a.nch_max, DV, b, hf) + size_t(kk) * 3 * 64;
      const u32x4 p0 = p[0], p1 = p[64], p2 = f16 ? p1 : p[128];
      unpack8(static_cast<const u32x4*>(a.woutT)[(size_t(c) * DV + d0) / 8], wd[q]);
      if (f16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t hb = (e & 1) ? (p0[e / 2] >> 16) : (p0[e / 2] & 0xFFFFu);
          const uint32_t lb = (e & 1) ? (p1[e / 2] >> 16) : (p1[e / 2] & 0xFFFFu);
          zd[q][e] = u < NU ? (h2f(hb) + h2f(lb)) * zs : 0.0f;
        }
      } else {
        float zh[8], zm[8], zl[8];
        unpack8(p0, zh);
        unpack8(p1, zm);
        unpack8(p2, zl);
#pragma unroll
        for (int e = 0; e < 8; ++e) zd[q][e] = u < NU ? (zh[e] + zm[e]) + zl[e] : 0.0f;
      }
    } else {
      const f32x4* zp = reinterpret_cast<const f32x4*>(a.z + (size_t(r) * a.W_max + b) * DV + d0);
      const f32x4* wp = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.woutT) + size_t(c) * DV + d0);
      const f32x4 z0 = zp[0], z1 = zp[1], w0 = wp[0], w1 = wp[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        zd[q][e] = u < NU ? z0[e] : 0.0f;
        zd[q][4 + e] = u < NU ? z1[e] : 0.0f;
        wd[q][e] = w0[e];
        wd[q][4 + e] = w1[e];
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < UPL; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(zd[q][e], wd[q][e], s);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (live && j == 0) a.flog[size_t(r) * a.W_max + i] = s;
}

// Blocks [0, forced_blocks) (forced parent maps only): the forced candidates' logits, 32
// per block, first in the grid so that they run beside the refinement.  Later blocks: one
// wave per group: code tile j against up to 32 beams that chose it.  Columns are
// independent in the MFMA, so every logit equals the first pass's bit for bit.
template <int DV, bool WBF16>
__global__ void __launch_bounds__(256, 3) refine_kernel(RefineK a) {
  constexpr int HV = DV / 2;
  const int r = blockIdx.y;
  if (int(blockIdx.x) < a.forced_blocks) {               // block-uniform
    forced_logit8<DV, WBF16>(a, r, int(blockIdx.x) * 32 + int(threadIdx.x >> 3));
    return;
  }
  const int rb = int(blockIdx.x) - a.forced_blocks;        // block of the refinement
  const int g = rb * 4 + (threadIdx.x >> 6);              // < G_max by the launch
  const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
  // the group count and the group's descriptor and tiles are loaded together; a wave
  // past the last group leaves once they are in (the operand loads below need them)
  const uint32_t ng = a.sel[r].n_groups;
  const uint32_t desc = a.groups[size_t(r) * a.G_max + g];
  const uint32_t f = a.gtiles[(size_t(r) * a.G_max + g) * 32 + m];
  if (g >= int(ng)) return;                                 // wave-uniform, no barrier follows
  const int start = int(desc & 1023u), cnt = int((desc >> 10) & 63u), j = int(desc >> 16);
  const bool valid = m < cnt;
  const int b = valid ? int(f / uint32_t(a.Vt)) : 0;
  const int c0 = 32 * j;
  // the beam's cumulative score and log-sum-exp go out with the operands
  const float cb = a.cum[size_t(r) * a.W_max + b], lb = a.lse[size_t(r) * a.W_max + b];
  f32x16 acc;
  float fb = 1.0f;                                          // logits = acc x fb
  if constexpr (WBF16) {
    // the same MFMA sequence as the first pass (kk ascending), in the same form, with
    // operands held for at most eight kk at a time
    constexpr int KS = DV / 16, KP = KS > 8 ? 8 : KS;
    const u32x4* zb = a.zf + zf_lane_base(r, a.nch_max, DV, b, hf);
    const int code = c0 + m;
    const size_t row = size_t(code < a.V ? code : 0) * DV + HV * hf;
    auto run = [&](auto f16c) {
      constexpr bool F16 = decltype(f16c)::value;
      const u32x4* wt = static_cast<const u32x4*>(F16 ? a.woutT16 : a.woutT);
      acc = f32x16{};
#pragma unroll 1
      for (int k0 = 0; k0 < KS; k0 += KP) {
        u32x4 zh[KP], zm[KP], zl[KP], w[KP];
#pragma unroll
        for (int kk = 0; kk < KP; ++kk) {
          zh[kk] = zb[(3 * (k0 + kk)) * 64];
          zm[kk] = zb[(3 * (k0 + kk) + 1) * 64];
          zl[kk] = F16 ? zm[kk] : zb[(3 * (k0 + kk) + 2) * 64];
          w[kk] = wt[row / 8 + k0 + kk];
        }
        __builtin_amdgcn_sched_barrier(0);        // every operand load issued before the MFMAs
        acc = block_mfma_split<F16, KP>(w, zh, zm, zl, acc);
      }
    };
    if (a.f16_on && *a.f16flag == 0u) {                     // launch-uniform
      fb = ldexpf(a.zscale[size_t(r) * a.W_max + b], -a.tscale[j]);
      run(std::true_type{});
    } else {
      run(std::false_type{});
    }
  } else {
    const float* zr = a.z + (size_t(r) * a.W_max + b) * DV + HV * hf;
    float zv[HV];
#pragma unroll
    for (int i = 0; i < HV; ++i) zv[i] = zr[i];
    acc = block_mfma_f32<DV>(static_cast<const float*>(a.woutT), c0 + m, a.V, hf, zv);
  }
  if (valid) {
    // lane half hf holds codes 8 q + 4 hf + (0..3): four 16-byte runs of the row
    u32x4* out = reinterpret_cast<u32x4*>(a.rkeys + (size_t(r) * a.W_max + start + m) * kTile);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 kq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = f2key(cand_score(cb, acc[4 * q + e] * fb, lb));
        kq[e] = c0 + 8 * q + 4 * hf + e < a.V ? key : 0u;
      }
      out[2 * q + hf] = kq;
    }
  }
}

// ---------------------------------------------------------------- final select

struct FinK {
  int W, W_max, V, Vt, K, Kt, T_max, t, d_v, nch_max, split;
  const SelState* sel;
  const uint32_t* rkeys;
  const uint32_t* tiles;
  const float* lse;
  const float* cum;        // step t
  float* cum_next;
  const int32_t* anc;      // step t
  int32_t* anc_next;
  const int32_t* tok;
  int32_t* tok_next;
  const int32_t* opos;     // [R,W_max] position of each beam in step t's processing order
  int32_t* order_next;     // [R,W_max] processing order of step t + 1
  int32_t* opos_next;
  const float* flog;       // [R,W_max] logits of the forced candidates
  const int32_t *forced_parent, *forced_token;
  int32_t *parent, *token;
  float* score;
  int32_t* status;
  uint32_t* f16flag;
  int f16_on;
};

// Refined keys kept in LDS by the final select; more than this many keys at or above
// the tile threshold (massive ties) are read from global memory instead.
constexpr int kFinCap = 8192;
// Ancestry and SID prefix entries (live beams x past steps) the final select stages in
// LDS at its start; beyond this they are read from global memory where needed.
constexpr int kAncCap = 4096;
static_assert(kAncCap % 1024 == 0 && kMaxW <= 1024, "final select: one block of 1024 threads");

// One 1024-thread block per request.  Only refined keys at or above the K-th tile key
// can be among the top K (when K tiles were chosen: their maxima are K candidates);
// they are compacted into LDS.  Then the exact top-K (score descending, flat index
// b * V + c ascending): when at most 1024 keys were kept, one sort of all of them;
// otherwise a radix select of the K winners and a sort of those (one entry per thread:
// runs of 64 sorted inside the waves, ranks by binary search across runs).  Last,
// the top-W outputs and the eq. (9) remap of ancestry, SID prefixes and cumulative
// scores, from the parents' rows staged in LDS at the start.
__global__ void __launch_bounds__(1024) final_kernel(FinK a) {
  __shared__ uint32_t ck[kFinCap], ce[kFinCap];
  __shared__ uint32_t tl[kMaxW];
  __shared__ union {
    uint32_t hist[kHistBins];
    uint64_t s[kMaxW];
  } u;
  __shared__ uint32_t wsum[16];
  __shared__ RadixSh sh;
  __shared__ uint32_t kmax_sh, m_sh;
  __shared__ int32_t pa[kAncCap], pt[kAncCap];           // [b][j < t] of the live beams
  __shared__ float cum_s[kMaxW];
  __shared__ int32_t opos_s[kMaxW];
  __shared__ uint64_t runs[kMaxW];                         // sorted runs of the rank sort
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const uint32_t n = uint32_t(a.Kt) * kTile;
  const uint32_t V = uint32_t(a.V), Vt = uint32_t(a.Vt);
  const uint32_t lo = max(a.sel[r].theta, 1u);            // key 0 marks a padding code
  const uint32_t* rk = a.rkeys + size_t(r) * a.W_max * kTile;
  if (tid == 0) { kmax_sh = 0u; m_sh = 0u; }
  {
    // every global load of the prologue is issued before the first is used: the tile
    // list (Kt <= 1024), the live beams' cumulative scores and order positions, their
    // ancestry and SID prefix rows (up to 4 x 1024 entries each) and the refined keys
    const size_t rw = size_t(r) * a.W_max;
    const uint32_t tlv = tid < a.Kt ? a.tiles[rw + tid] : 0u;
    const float cumv = tid < a.W ? a.cum[rw + tid] : 0.0f;
    const int32_t oposv = tid < a.W && a.t > 0 ? a.opos[rw + tid] : tid;
    const int nanc = a.W * a.t <= kAncCap ? a.W * a.t : 0;
    int32_t pav[kAncCap / 1024], ptv[kAncCap / 1024];
#pragma unroll
    for (int q = 0; q < kAncCap / 1024; ++q) {
      const int e = q * 1024 + tid;
      const size_t g = e < nanc ? (rw + e / a.t) * a.T_max + e % a.t : 0;
      pav[q] = e < nanc ? a.anc[g] : 0;
      ptv[q] = e < nanc ? a.tok[g] : 0;
    }
    constexpr int IT = kMaxW * kTile / 4 / 1024;         // u32x4 loads per thread
    const u32x4* src = reinterpret_cast<const u32x4*>(rk);
    u32x4 kv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t q = uint32_t(it) * 1024 + tid;
      kv[it] = q < n / 4 ? src[q] : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < a.Kt) tl[tid] = tlv;
    if (tid < a.W) { cum_s[tid] = cumv; opos_s[tid] = oposv; }
#pragma unroll
    for (int q = 0; q < kAncCap / 1024; ++q)
      if (q * 1024 + tid < nanc) { pa[q * 1024 + tid] = pav[q]; pt[q * 1024 + tid] = ptv[q]; }
    // compaction of the keys at or above lo in one block scan of the per-thread counts
    // (its barriers also publish the tile list)
    uint32_t lmax = 0u, cnt = 0u;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kv[it][e];
        cnt += key >= lo;
        lmax = key >= lo ? max(lmax, key) : lmax;
      }
    uint32_t total;
    uint32_t p = block_excl_scan(cnt, wsum, total);
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kv[it][e];
        if (key >= lo) {
          if (p < uint32_t(kFinCap)) { ck[p] = key; ce[p] = 4 * (uint32_t(it) * 1024 + tid) + e; }
          ++p;
        }
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, uint32_t(__shfl_xor(int(lmax), off)));
    if (lane == 0) atomicMax(&kmax_sh, lmax);
    if (tid == 0) m_sh = total;
  }
  __syncthreads();
  const uint32_t m = m_sh, hi = kmax_sh;
  const bool inl = m <= uint32_t(kFinCap);
  const uint32_t ns = inl ? m : n;
  auto key_at = [&](uint32_t i) { return inl ? ck[i] : rk[i]; };
  auto flat_at = [&](uint32_t i) {
    const uint32_t e = inl ? ce[i] : i;
    const uint32_t f = tl[e >> 5];
    return (f / Vt) * V + (f % Vt) * kTile + (e & 31u);
  };
  uint64_t v;
  uint32_t got, nsort;
  if (inl && m <= uint32_t(kMaxW)) {
    // few keys at or above the tile threshold (the usual case: a little over K):
    // sorting all of them as (key, ~flat) ranks the top K directly
    v = uint32_t(tid) < m ? (uint64_t(ck[tid]) << 32) | uint64_t(0xFFFFFFFFu - flat_at(tid)) : 0ull;
    got = min(m, uint32_t(a.K));
    if (tid == 0 && m < uint32_t(a.K)) atomicOr(a.status, 2);
    nsort = m;
  } else {
    uint32_t need = uint32_t(a.K);
    const uint32_t theta = radix_finish(key_at, ns, lo, hi, need, first_shift(lo, hi), u.hist, wsum, sh);
    const uint32_t phi = tie_cut(key_at, flat_at, ns, theta, need, u.hist, sh);
    // gather the K winners as (key, ~flat): sorting these descending ranks by score
    // descending, then flat index ascending
    if (tid == 0) sh.cnt = 0;
    __syncthreads();
    for (uint32_t i0 = 0; i0 < ns; i0 += 1024) {
      const uint32_t i = i0 + tid;
      bool win = false;
      uint64_t ent = 0;
      if (i < ns) {
        const uint32_t key = key_at(i);
        if (key >= theta) {
          const uint32_t f = flat_at(i);
          win = key > theta || f <= phi;
          ent = (uint64_t(key) << 32) | uint64_t(0xFFFFFFFFu - f);
        }
      }
      const uint64_t mask = __ballot(win);
      if (mask) {
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&sh.cnt, uint32_t(__popcll(mask)));
        base = uint32_t(__shfl(int(base), 0));
        if (win) {
          const uint32_t p = base + uint32_t(__popcll(mask & ((1ull << lane) - 1ull)));
          if (p < uint32_t(kMaxW)) u.s[p] = ent;
        }
      }
    }
    __syncthreads();
    got = min(sh.cnt, uint32_t(kMaxW));
    if (tid == 0 && sh.cnt != uint32_t(a.K)) atomicOr(a.status, 2);
    v = uint32_t(tid) < got ? u.s[tid] : 0ull;
    nsort = got;
  }
  v = rank_sort_desc(v, int(nsort), runs, u.s);
  // thread i holds rank i
  const float* lse = a.lse + size_t(r) * a.W_max;
  int okey = 0;                                           // parent's position (order below)
  if (tid < a.K) {
    const int i = tid;
    const uint32_t flat = 0xFFFFFFFFu - uint32_t(v);
    int p = int(flat / V), c = int(flat % V);
    if (uint32_t(i) >= got || p >= a.W) {   // only if fewer than K were gathered (flagged)
      p = 0;
      c = 0;
    }
    const float sc = key2f(uint32_t(v >> 32));
    const size_t o = size_t(r) * a.K + i;
    a.parent[o] = p;
    a.token[o] = c;
    a.score[o] = sc;
    int fp = p, fc = c;
    float fs = sc;
    if (a.forced_parent) {
      // the refinement flagged entries out of range; they are clamped the same way
      fp = a.forced_parent[o];
      fc = a.forced_token[o];
      fp = fp < 0 ? 0 : (fp >= a.W ? a.W - 1 : fp);
      fc = fc < 0 ? 0 : (fc >= a.V ? a.V - 1 : fc);
      fs = cand_score(cum_s[fp], a.flog[size_t(r) * a.W_max + i], lse[fp]) + 0.0f;
    }
    // eq. (9): the child copies its parent's ancestry and appends the parent's slot
    const bool lds = a.W * a.t <= kAncCap;                 // block-uniform
    const int32_t* ap = lds ? pa + fp * a.t : a.anc + (size_t(r) * a.W_max + fp) * a.T_max;
    const int32_t* tp = lds ? pt + fp * a.t : a.tok + (size_t(r) * a.W_max + fp) * a.T_max;
    int32_t* an = a.anc_next + (size_t(r) * a.W_max + i) * a.T_max;
    int32_t* tn = a.tok_next + (size_t(r) * a.W_max + i) * a.T_max;
    for (int j = 0; j < a.T_max; ++j) {
      an[j] = j < a.t ? ap[j] : (j == a.t ? fp : 0);
      tn[j] = j < a.t ? tp[j] : (j == a.t ? fc : 0);
    }
    a.cum_next[size_t(r) * a.W_max + i] = fs;
    okey = opos_s[fp];
  }
  // processing order of step t + 1: a counting sort of the beams by their parent's
  // position in step t's order, so children of one parent are adjacent and subtrees
  // stay contiguous (any order is correct; this one makes shared records cache hits)
  __syncthreads();
  u.hist[tid] = 0u;
  __syncthreads();
  if (tid < a.K) atomicAdd(&u.hist[okey], 1u);
  __syncthreads();
  uint32_t total;
  const uint32_t start = block_excl_scan(u.hist[tid], wsum, total);
  u.hist[tid] = start;
  __syncthreads();
  if (tid < a.K) {
    const uint32_t p = atomicAdd(&u.hist[okey], 1u);
    a.order_next[size_t(r) * a.W_max + p] = tid;
    a.opos_next[size_t(r) * a.W_max + tid] = int32_t(p);
  }
  // every kernel that reads the fp16 flag has run: report the three-term form (status
  // bit 2), then clear the flag for the next selection
  if (r == 0 && tid == 0) {
    if (a.split && a.f16_on && *a.f16flag != 0u) atomicOr(a.status, 4);
    *a.f16flag = 0u;
  }
}

// ---------------------------------------------------------------- launchers

template <int DV>
static int launch_dv(const SelectArgs& a, const LogitsK& lk, const RefineK& rk, int groups,
                     hipStream_t s, bool refine) {
  const bool bf = a.wout_dtype == GDN_BF16;
  if (!refine) {
    dim3 grid(((a.R * lk.nchunk + kLogitsWaves - 1) / kLogitsWaves) * ((lk.nvg + lk.gpb - 1) / lk.gpb));
    if (bf) hipLaunchKernelGGL((logits_kernel<DV, true>), grid, dim3(64 * kLogitsWaves), 0, s, lk);
    else hipLaunchKernelGGL((logits_kernel<DV, false>), grid, dim3(64 * kLogitsWaves), 0, s, lk);
  } else {
    dim3 grid(groups, a.R);                       // groups: blocks, set by the caller
    if (bf) hipLaunchKernelGGL((refine_kernel<DV, true>), grid, dim3(256), 0, s, rk);
    else hipLaunchKernelGGL((refine_kernel<DV, false>), grid, dim3(256), 0, s, rk);
  }
  return last_launch_error();
}

static int launch_by_dv(const SelectArgs& a, const LogitsK& lk, const RefineK& rk, int groups,
                        hipStream_t s, bool refine) {
  if (a.d_v == 16) return launch_dv<16>(a, lk, rk, groups, s, refine);
  if (a.d_v == 128) return launch_dv<128>(a, lk, rk, groups, s, refine);
  if (a.d_v == 256) return launch_dv<256>(a, lk, rk, groups, s, refine);
  if (a.d_v == 512) return launch_dv<512>(a, lk, rk, groups, s, refine);
  return int(hipErrorInvalidValue);
}

int launch_select(const SelectArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  char* ws = static_cast<char*>(a.ws);
  const Layout& L = a.L;
  const int par = a.t & 1;
  const int Vt = n_tiles(a.V);
  const int nch = n_chunks(a.W), nch_max = n_chunks(a.W_max);
  const int Kt = int(a.W_next < int64_t(a.W) * Vt ? a.W_next : int64_t(a.W) * Vt);
  const size_t tstride = size_t(n_tiles(a.V_max)) * a.W_max;
  const int G_max = max_groups(a.W_max, n_tiles(a.V_max));
  const int split = a.wout_dtype == GDN_BF16;
  char* scr = a.scr;
  const SelScratch& S = a.S;
  float* z = reinterpret_cast<float*>(scr + S.z);
  u32x4* zf = reinterpret_cast<u32x4*>(scr + S.zf);
  void* woutT = scr + S.woutT;
  float* tmax = reinterpret_cast<float*>(scr + S.tmax);
  float4* lse_part = reinterpret_cast<float4*>(scr + S.lse_part);
  float* lse = reinterpret_cast<float*>(scr + S.lse);
  SelState* sel = reinterpret_cast<SelState*>(scr + S.sel);
  uint32_t* cand = reinterpret_cast<uint32_t*>(scr + S.cand);
  uint32_t* tiles = reinterpret_cast<uint32_t*>(scr + S.tiles);
  uint32_t* groups = reinterpret_cast<uint32_t*>(scr + S.groups);
  uint32_t* gtiles = reinterpret_cast<uint32_t*>(scr + S.gtiles);
  uint32_t* rkeys = reinterpret_cast<uint32_t*>(scr + S.rkeys);
  float* cum = reinterpret_cast<float*>(ws + L.cum[par]);
  float* cum_next = reinterpret_cast<float*>(ws + L.cum[par ^ 1]);
  int32_t* anc = reinterpret_cast<int32_t*>(ws + L.anc[par]);
  int32_t* anc_next = reinterpret_cast<int32_t*>(ws + L.anc[par ^ 1]);
  int32_t* tok = reinterpret_cast<int32_t*>(ws + L.tok[par]);
  int32_t* tok_next = reinterpret_cast<int32_t*>(ws + L.tok[par ^ 1]);
  int32_t* status = reinterpret_cast<int32_t*>(ws + L.status);
  const int32_t* opos = reinterpret_cast<const int32_t*>(ws + L.opos[par]);
  int32_t* order_next = reinterpret_cast<int32_t*>(ws + L.order[par ^ 1]);
  int32_t* opos_next = reinterpret_cast<int32_t*>(ws + L.opos[par ^ 1]);
  int err;

  float* flog = reinterpret_cast<float*>(scr + S.flog);
  uint32_t* f16flag = reinterpret_cast<uint32_t*>(scr + S.f16flag);
  int32_t* tscale = reinterpret_cast<int32_t*>(scr + S.tscale);
  void* woutT16 = scr + S.woutT16;
  float* zscale = reinterpret_cast<float*>(scr + S.zscale);
  // The two-term fp16 form saves a third of the logits' MFMA work but needs the codebook
  // prepared by a launch of its own (~11 us); it pays where the selection's MFMA work is
  // large (R W V d_v >= 2^33 multiply-adds: the stress and growing decodes), and small
  // selections keep three bf16 terms with the transpose inside the head-sum launch.
  // GDN_BEAM_F16_MIN_MACS overrides the threshold (0: wherever the codebook fits)
  double min_macs = 8589934592.0;
  if (const char* e = getenv("GDN_BEAM_F16_MIN_MACS")) {
    if (*e) min_macs = atof(e);
  }
  const int f16_on = split && double(a.R) * a.W * a.V * a.d_v >= min_macs;
  if (f16_on) {  // codebook transpose and each code tile's fp16 form
    WprepK k{a.d_v, a.V, split, a.Wout, woutT, static_cast<uint16_t*>(woutT16), tscale, f16flag};
    const dim3 g = dim3(unsigned(Vt)), b = dim3(256);
    if (a.d_v == 16) hipLaunchKernelGGL(wprep_kernel<16>, g, b, 0, s, k);
    else if (a.d_v == 128) hipLaunchKernelGGL(wprep_kernel<128>, g, b, 0, s, k);
    else if (a.d_v == 256) hipLaunchKernelGGL(wprep_kernel<256>, g, b, 0, s, k);
    else hipLaunchKernelGGL(wprep_kernel<512>, g, b, 0, s, k);
    if ((err = last_launch_error())) return err;
  }
  {  // head sum into the MFMA operand; the codebook transpose in the last blocks unless
     // wprep_kernel did it
    const long n = long(a.R) * nch * 32 * (a.d_v / 8);
    long zb = (n + 255) / 256;
    zb = zb < 1 ? 1 : (zb > 65536 ? 65536 : zb);
    const int ntr = ((a.V + 31) / 32) * ((a.d_v + 31) / 32);
    const int tb = f16_on ? 0 : (ntr < 256 ? ntr : 256);
    ZsumK k{a.R, a.H, a.W, a.W_max, a.d_v, a.V, nch_max, int(zb), split, f16_on, a.o, z, zf, zscale,
            f16flag, a.Wout, woutT};
    // o above half of the 256 MiB last-level cache: streamed (512 MiB of o: 144 -> 120
    // us per launch; 64 MiB of o is still in that cache, and plain loads hit it)
    const bool stream = size_t(a.R) * a.H * a.W * a.d_v * 4 > (size_t(128) << 20);
    if (stream) hipLaunchKernelGGL(zsum_kernel<true>, dim3(unsigned(zb + tb)), dim3(256), 0, s, k);
    else hipLaunchKernelGGL(zsum_kernel<false>, dim3(unsigned(zb + tb)), dim3(256), 0, s, k);
    if ((err = last_launch_error())) return err;
  }
  // codes per wave: 128 .. 1024, larger while the grid keeps >= 8192 waves, so that
  // the z operand is reloaded fewer times on large codebooks (at 4096 codes and
  // 256-512 beams of d_v = 256, 8192 rather than 16384 took 30 us off a 0.44 ms
  // selection; 32768 cost 150 us on 1024 beams of 8192 codes)
  int cpw = 128;
  while (cpw < 1024 && cpw < a.V && int64_t(a.R) * nch * ((a.V + 2 * cpw - 1) / (2 * cpw)) >= 8192) cpw *= 2;
  const int nvg = (a.V + cpw - 1) / cpw;
  // the bounded tile selection where a request's tiles outnumber its list (and the code
  // groups' maxima number at least K); it reads the tile maxima beam-major
  const bool bounded = int64_t(a.W) * Vt > kSelList && int64_t(a.W) * nvg >= Kt;
  LogitsK lk{a.R, a.W, a.W_max, a.V, nch, nvg, cpw, nch_max, bounded ? 1 : 0, z, zf, woutT, woutT16,
             zscale, tscale, f16flag, f16_on, tmax, tstride, lse_part};
  while ((1 << lk.cpw_shift) < cpw) ++lk.cpw_shift;         // cpw is a power of two
  // d_v <= 256 with a bf16 codebook (z in registers, tile maxima staged): a block takes
  // up to eight code groups in turn while the grid keeps a block per CU, so that fewer
  // blocks start and end one after the other on a CU (each group's tile maxima and
  // log-sum-exp part are those of a block of its own).  GDN_BEAM_LOGITS_GPB sets it
  // (tests).
  if (a.d_v <= 256 && split) {
    const int64_t nchg = (int64_t(a.R) * nch + kLogitsWaves - 1) / kLogitsWaves;
    int cap = kMaxGroupsPerBlock;
    bool forced_gpb = false;
    if (const char* e = getenv("GDN_BEAM_LOGITS_GPB")) {
      const int v = atoi(e);
      if (v >= 1) { cap = v < kMaxGroupsPerBlock ? v : kMaxGroupsPerBlock; forced_gpb = true; }
    }
    while (lk.gpb * 2 <= cap && lk.gpb * 2 <= nvg &&
           (forced_gpb || nchg * ((nvg + 2 * lk.gpb - 1) / (2 * lk.gpb)) >= kLogitsMinBlocks))
      lk.gpb *= 2;
  }
  RefineK rk{a.W, a.W_max, a.V, Vt, G_max, nch_max, z, zf, woutT, lse, cum, sel, groups, gtiles, rkeys,
             woutT16, zscale, tscale, f16flag, f16_on, 0, a.W_next, a.forced_parent, a.forced_token, flog,
             status};
  if ((err = launch_by_dv(a, lk, rk, 0, s, false))) return err;
  {
    int tg_shift = 0;
    while ((kTile << (tg_shift + 1)) <= cpw) ++tg_shift;    // cpw / 32 tiles, a power of two
    TileSelK k{a.W, a.W_max, Vt, Kt, a.W_next, G_max, nvg, tg_shift, tstride, tmax, lse_part, cum, lse,
               sel, cand, tiles, groups, gtiles, status};
    if (bounded) hipLaunchKernelGGL(tile_select_kernel<true>, dim3(a.R), dim3(1024), 0, s, k);
    else hipLaunchKernelGGL(tile_select_kernel<false>, dim3(a.R), dim3(1024), 0, s, k);
    if ((err = last_launch_error())) return err;
  }
  {  // groups <= ceil(Kt / 32) + min(Vt, Kt) <= G_max; the forced candidates' logits in
     // blocks after the refinement's (32 per block)
    const int gmax = (Kt + 31) / 32 + (Vt < Kt ? Vt : Kt);
    rk.forced_blocks = a.forced_parent ? (a.W_next + 31) / 32 : 0;
    if ((err = launch_by_dv(a, lk, rk, rk.forced_blocks + (gmax + 3) / 4, s, true))) return err;
  }
  {
    FinK k{a.W, a.W_max, a.V, Vt, a.W_next, Kt, a.T_max, a.t, a.d_v, nch_max, split, sel, rkeys, tiles,
           lse, cum, cum_next, anc, anc_next, tok, tok_next, opos, order_next, opos_next, flog,
           a.forced_parent, a.forced_token, a.parent, a.token, a.score, status, f16flag, f16_on};
    hipLaunchKernelGGL(final_kernel, dim3(a.R), dim3(1024), 0, s, k);
    if ((err = last_launch_error())) return err;
  }
  return 0;
}

// ---------------------------------------------------------------- static scratch

// The selection scratch of gdn_beam_select_static, for callers that cannot allocate:
// one array per GPU, which that GPU holds from the library's first use on it until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the host it
// names a stand-in, not device memory): it uses the device address static_scratch()
// looked up for the current device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

int static_scratch(char** ptr) {
  static std::mutex m;
  static char* addr[kStaticScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= kStaticScratchDevices) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> g(m);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));    // with device `dev` current
    if (e != hipSuccess) return int(e);
    addr[dev] = static_cast<char*>(p);
  }
  *ptr = addr[dev];
  return 0;
}

int copy_d2d(void* dst, const void* src, size_t bytes, hipStream_t s) {
  return int(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
}

const char* hip_error_string(int err) { return hipGetErrorString(hipError_t(err)); }

}  // namespace gdn
