// Device helpers shared by the decoding kernels: operand types, bf16 rounding,
// order-preserving score keys, the XCD-aware block order and the MFMA row order.
#pragma once
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

// order-preserving key: larger float -> larger key; -0 is folded into +0 first.  Every
// NaN maps to key 1, below -inf (key 0x007FFFFF) and above 0, the key of a padding code:
// a NaN score ranks below every number, as a full sort that puts NaN last does.
__device__ __forceinline__ uint32_t f2key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return s != s ? 1u : k;
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// the candidate score, evaluated identically wherever it is needed
__device__ __forceinline__ float cand_score(float cum, float logit, float lse) {
  return cum + (logit - lse);
}

// Work item of block b of an n-block 1-D grid: blocks are dealt round-robin to the 8
// XCDs, so XCD x runs blocks x, x + 8, ...; it is given the contiguous work range
// [x q + min(x, n % 8), ...) with q = n / 8 (a bijection for any n), so work items
// next to each other share one XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, q = n >> 3, rr = n & 7;
  return x * q + (x < rr ? x : rr) + (b >> 3);
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

// Value of lane (lane ^ J) of the wave.  J = 1, 2: DPP quad permutes; 4: DPP row
// shifts by 4 either way; 8: DPP row rotate by 8; 16: swizzle (xor mode); 32: LDS
// permute.  The DPP forms are plain VALU moves.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, false));
  else if constexpr (J == 2) return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xF, 0xF, false));
  else if constexpr (J == 4) {
    const uint32_t up = uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x104, 0xF, 0xF, false));
    const uint32_t dn = uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x114, 0xF, 0xF, false));
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (J == 8) return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x128, 0xF, 0xF, false));
  else if constexpr (J == 16) return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), (16 << 10) | 0x1F));
  else return uint32_t(__shfl_xor(int(v), 32));
}

inline int last_launch_error() { return int(hipGetLastError()); }

}  // namespace gdn
