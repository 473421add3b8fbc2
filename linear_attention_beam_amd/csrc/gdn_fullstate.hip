// FullState step for large-beam Gated DeltaNet decoding on gfx950: the baseline the
// OneLA reading note measures against (section 1.3, Fig. 2: every beam carries its own
// d_v x d_k state, copied on reorder; section 2.2 eq. (4) for the update).
//
//   fullstate_kernel  one workgroup per (request, head, beam): reads the parent's
//                     state (S_ctx at t = 0), computes P k and P q, then
//                     delta = beta (v - alpha P k), S = alpha P + delta k^T (written
//                     whole) and o = S q = alpha P q + delta (k . q).
#include <hip/hip_ext.h>

#include "gdn_device.h"

namespace gdn {

struct FullK {
  int H, HK, W, W_max, T_max, t;
  const float* S_ctx;          // [R,H,DV,DK] fp32
  const void *q, *k, *v;       // [R,H,W,DK|DV] io dtype
  const float *alpha, *beta;   // [R,H,W]
  float* o;                    // [R,H,W,DV]
  const float* prev;           // [R,H,W_max,DV,DK] states of step t-1 (t >= 1)
  float* next;                 // [R,H,W_max,DV,DK] states of step t
  const int32_t* anc;          // ancestry of step t [R,W_max,T_max]
};

template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, size_t i) {   // elements i .. i+3
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t i) {
  if constexpr (BF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[i]) << 16);
  else return static_cast<const float*>(base)[i];
}

// Sum over the L consecutive lanes that share a state row (L a power of two <= 32).
template <int L>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (L >= 2) x += __uint_as_float(lane_xor<1>(__float_as_uint(x)));
  if constexpr (L >= 4) x += __uint_as_float(lane_xor<2>(__float_as_uint(x)));
  if constexpr (L >= 8) x += __uint_as_float(lane_xor<4>(__float_as_uint(x)));
  if constexpr (L >= 16) x += __uint_as_float(lane_xor<8>(__float_as_uint(x)));
  if constexpr (L >= 32) x += __uint_as_float(lane_xor<16>(__float_as_uint(x)));
  if constexpr (L >= 64) x += __uint_as_float(lane_xor<32>(__float_as_uint(x)));
  return x;
}

// Lanes: DK / 4 per state row (one 16-byte column slice each), 256 / (DK / 4) rows
// at a time; the parent state's rows are loaded up to CH row batches at once (all of
// them in flight), then computed and streamed out.
template <int DK, int DV, bool BF16>
__global__ void __launch_bounds__(256) fullstate_kernel(FullK a) {
  constexpr int LPR = DK / 4;
  constexpr int RPI = 256 / LPR;
  constexpr int NB = (DV + RPI - 1) / RPI;       // row batches
  constexpr int CH = NB > 16 ? 16 : NB;          // batches held in registers at once
  const size_t bid = blockIdx.x;                 // ((r * H + h) * W + b)
  const int b = int(bid % a.W);
  const size_t rh = bid / a.W;
  const int r = int(rh / a.H);
  const int tid = threadIdx.x, lr = tid % LPR, row0 = tid / LPR;

  const float* P;
  if (a.t == 0) {
    P = a.S_ctx + rh * DV * DK;
  } else {
    int p = a.anc[(size_t(r) * a.W_max + b) * a.T_max + a.t - 1];
    p = p < 0 ? 0 : (p >= a.W_max ? a.W_max - 1 : p);
    P = a.prev + (rh * a.W_max + p) * DV * DK;
  }
  float* S = a.next + (rh * a.W_max + b) * DV * DK;
  const size_t beam = rh * a.W + b;
  const size_t kbeam = (size_t(r) * a.HK + int(rh % a.H) / (a.H / a.HK)) * a.W + b;   // key head
  const f32x4 k4 = load4<BF16>(a.k, kbeam * DK + 4 * lr);
  const f32x4 q4 = load4<BF16>(a.q, kbeam * DK + 4 * lr);
  const float al = a.alpha[beam], be = a.beta[beam];
  const float kq = row_sum<LPR>(k4[0] * q4[0] + k4[1] * q4[1] + k4[2] * q4[2] + k4[3] * q4[3]);
#pragma unroll 1
  for (int b0 = 0; b0 < NB; b0 += CH) {
  f32x4 pr[CH];
  float vr[CH];
#pragma unroll
  for (int it = 0; it < CH; ++it) {
    const int row = row0 + (b0 + it) * RPI;
    pr[it] = row < DV ? *reinterpret_cast<const f32x4*>(P + size_t(row) * DK + 4 * lr) : f32x4{};
    vr[it] = row < DV ? load1<BF16>(a.v, beam * DV + row) : 0.0f;
  }
#pragma unroll
  for (int it = 0; it < CH; ++it) {
    const int row = row0 + (b0 + it) * RPI;
    const f32x4 x = pr[it];
    const float uk = row_sum<LPR>(x[0] * k4[0] + x[1] * k4[1] + x[2] * k4[2] + x[3] * k4[3]);
    const float uq = row_sum<LPR>(x[0] * q4[0] + x[1] * q4[1] + x[2] * q4[2] + x[3] * q4[3]);
    const float dl = be * (vr[it] - al * uk);                // eq. (4): delta
    if (row < DV) {
      f32x4 s;
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = fmaf(dl, k4[e], al * x[e]);   // alpha P + delta k^T
      *reinterpret_cast<f32x4*>(S + size_t(row) * DK + 4 * lr) = s;
      if (lr == 0) a.o[beam * DV + row] = fmaf(dl, kq, al * uq);      // S q
    }
  }
  }
}

template <int DK, int DV, bool BF16>
static int launch_full_t(const FullStepArgs& s, hipStream_t st) {
  const float* prev = reinterpret_cast<const float*>(static_cast<const char*>(s.states) +
                                                     ((s.t + 1) & 1) * s.half_bytes);
  float* next = reinterpret_cast<float*>(static_cast<char*>(s.states) + (s.t & 1) * s.half_bytes);
  FullK k{s.H, s.HK, s.W, s.W_max, s.T_max, s.t, s.S_ctx, s.q, s.k, s.v, s.alpha, s.beta, s.o, prev,
          next, s.anc};
  const size_t blocks = size_t(s.R) * s.H * s.W;
  if (s.ev0)   // the dispatch itself stamps its start and end
    hipExtLaunchKernelGGL((fullstate_kernel<DK, DV, BF16>), dim3(unsigned(blocks)), dim3(256), 0, st, s.ev0,
                          s.ev1, 0, k);
  else
    hipLaunchKernelGGL((fullstate_kernel<DK, DV, BF16>), dim3(unsigned(blocks)), dim3(256), 0, st, k);
  return last_launch_error();
}

int launch_fullstate(const FullStepArgs& s, hipStream_t st) {
  (void)hipGetLastError();
  const bool bf = s.io == GDN_BF16;
  if (s.d_k == 16 && s.d_v == 16) return bf ? launch_full_t<16, 16, true>(s, st) : launch_full_t<16, 16, false>(s, st);
  if (s.d_k == 128 && s.d_v == 128) return bf ? launch_full_t<128, 128, true>(s, st) : launch_full_t<128, 128, false>(s, st);
  if (s.d_k == 128 && s.d_v == 256) return bf ? launch_full_t<128, 256, true>(s, st) : launch_full_t<128, 256, false>(s, st);
  if (s.d_k == 256 && s.d_v == 256 && bf) return launch_full_t<256, 256, true>(s, st);
  if (s.d_k == 128 && s.d_v == 512) return bf ? launch_full_t<128, 512, true>(s, st) : launch_full_t<128, 512, false>(s, st);
  if (s.d_k == 256 && s.d_v == 512 && bf) return launch_full_t<256, 512, true>(s, st);
  return int(hipErrorInvalidValue);
}

}  // namespace gdn
