// Selection-side HIP kernels for large-beam Gated DeltaNet decoding on gfx950.
//
// Scoring follows the beam-search objective of OneLA (paper-archivist.com) section 2.1
// and eq. (1); the request-level exact top-K follows RecoGEM (conceptio mirror)
// section 4.3; the ancestry remap is OneLA eq. (9).
//
// Kernels
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
#include "gdn_device.h"

namespace gdn {

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
    // codebook fragments of the current tile; the next tile's are loaded during its MFMAs
    auto load_w = [&](int c0, u32x4* wf) {
      const int code = c0 + m;
      const size_t row = size_t(code < a.V ? code : 0) * DV + HV * hf;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) wf[kk] = code < a.V ? wt[row / 8 + kk] : u32x4{};
    };
    u32x4 wcur[KS], wnext[KS];
    load_w(code_lo, wcur);
    for (int c0 = code_lo; c0 < code_hi; c0 += 32) {
      if (c0 + 32 < code_hi) load_w(c0 + 32, wnext);
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 w = __builtin_bit_cast(bf16x8, wcur[kk]);
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
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) wcur[kk] = wnext[kk];
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
__global__ void __launch_bounds__(256) lse_kernel(const float4* __restrict__ part,
                                                  float* __restrict__ lse,
                                                  const float* __restrict__ cum, SelState* sel,
                                                  int W, int W_max, int nvg) {
  const int r = blockIdx.y;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  if (b < W) {
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
    kmax = f2key(cand_score(c, mm, l));
    kmin = f2key(cand_score(c, mn, l));
  }
  // one atomic per wave (all lanes of a block belong to request r)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmax = max(kmax, uint32_t(__shfl_xor(int(kmax), off)));
    kmin = min(kmin, uint32_t(__shfl_xor(int(kmin), off)));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&sel[r].kmax, kmax);
    atomicMin(&sel[r].kmin, kmin);
  }
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

// ---------------------------------------------------------------- launchers

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
    hipLaunchKernelGGL(lse_kernel, dim3((a.W + 255) / 256, a.R), dim3(256), 0, s, lse_part, lse,
                       cum, sel, a.W, a.W_max, nvg);
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

int copy_d2d(void* dst, const void* src, size_t bytes, hipStream_t s) {
  return int(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
}

const char* hip_error_string(int err) { return hipGetErrorString(hipError_t(err)); }

}  // namespace gdn
