// Prefill: the shared state S_ctx of every (request, head) from its prompt by the Gated
// DeltaNet recurrence, eq. (3) of the OneLA reading note (paper-archivist.com), section 1.2.
#include "gdn_device.h"

namespace gdn {

// ---------------------------------------------------------------- prefill (eq. 3)

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

template <int DK, int DV>
__global__ void __launch_bounds__((PrefillCfg<DK, DV>::NT)) prefill_kernel(PrefillArgs a) {
  constexpr int TPR = PrefillCfg<DK, DV>::TPR;
  constexpr int COLS = DK / TPR;
  const int rh = blockIdx.x, r = rh / a.H, h = rh % a.H;
  const int hk = h / (a.H / a.HK);                        // key head of value head h
  const int row = blockIdx.y * PrefillCfg<DK, DV>::RB + threadIdx.x / TPR, cp = threadIdx.x % TPR;
  int beg = a.offsets[r], end = a.offsets[r + 1];
  beg = beg < 0 ? 0 : (beg > a.N ? int(a.N) : beg);
  end = end < beg ? beg : (end > a.N ? int(a.N) : end);
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

// ---------------------------------------------------------------- launcher

template <int DK, int DV>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  using C = PrefillCfg<DK, DV>;
  hipLaunchKernelGGL((prefill_kernel<DK, DV>), dim3(a.R * a.H, DV / C::RB), dim3(C::NT), 0, s, a);
  return last_launch_error();
}

int launch_prefill(const PrefillArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  if (a.d_k == 16 && a.d_v == 16) return launch_prefill_t<16, 16>(a, s);
  if (a.d_k == 128 && a.d_v == 128) return launch_prefill_t<128, 128>(a, s);
  if (a.d_k == 128 && a.d_v == 256) return launch_prefill_t<128, 256>(a, s);
  if (a.d_k == 256 && a.d_v == 256) return launch_prefill_t<256, 256>(a, s);
  if (a.d_k == 128 && a.d_v == 512) return launch_prefill_t<128, 512>(a, s);
  if (a.d_k == 256 && a.d_v == 512) return launch_prefill_t<256, 512>(a, s);
  return int(hipErrorInvalidValue);
}

}  // namespace gdn
