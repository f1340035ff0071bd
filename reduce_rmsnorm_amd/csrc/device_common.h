// Device helpers shared by the fused kernel and the unfused comparator
// kernels (gfx950): 16-byte vector <-> float conversion, the TwoSum and
// round-to-odd steps of the compensated sum, and the wave64 sum.
#pragma once

#include <hip/hip_runtime.h>

namespace tw {
namespace dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));


template <bool BF16> struct Elem { static constexpr int kPerVec = BF16 ? 8 : 4; };

__device__ __forceinline__ float as_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned as_u(float f) { return __builtin_bit_cast(unsigned, f); }

// 16 bytes -> floats.  bf16 is the upper half of a float32.
template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4& v, float* f) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = as_f(v[k] << 16);
      f[2 * k + 1] = as_f(v[k] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = as_f(v[k]);
  }
}

// floats -> 16 bytes.  bf16 uses the hardware round-to-nearest-even pack.
template <bool BF16>
__device__ __forceinline__ u32x4 pack(const float* f) {
  u32x4 v;
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f32x2 p = {f[2 * k], f[2 * k + 1]};
      v[k] = __builtin_bit_cast(unsigned, __builtin_convertvector(p, bf16x2));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = as_u(f[k]);
  }
  return v;
}

// Store of one 16-byte vector, vector index `vec` of a row that starts at
// `row` and holds `row_bytes` bytes, as a buffer store with the streaming bit
// (nt) and the device-scope coherence bit (sc1): the line is written through
// the XCD's L2 instead of staying there dirty until it is evicted, which
// streams the outputs faster alongside the reads.  Every caller's offset lies
// inside the row.
constexpr int kRawBufferFlags = 0x00020000;   // word 3 of a raw buffer resource on gfx9
constexpr int kStoreSc1Nt = 16 | 2;           // cache-policy bits: sc1, nt
__device__ __forceinline__ void store_stream(const u32x4& v, u32x4* row, int vec, int row_bytes) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, row_bytes, kRawBufferFlags);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, vec * 16, 0, kStoreSc1Nt);
}

// s + b = t + e exactly (Knuth's TwoSum); the error e is added to c.
__device__ __forceinline__ void two_sum_into(float& s, float& c, float b) {
  const float t = s + b;
  const float bv = t - s;
  const float av = t - bv;
  c += (s - av) + (b - bv);
  s = t;
}

// Round s + c to float32 with round-to-odd: the nearest value x, moved one
// unit toward the exact sum when x is inexact and even.
__device__ __forceinline__ float round_to_odd(float s, float c, float x) {
  const float bv = x - s;
  const float av = x - bv;
  const float r = (s - av) + (c - bv);          // s + c - x, exactly
  unsigned xb = as_u(x);
  const bool bump = (r != 0.0f) & ((xb & 1u) == 0u);
  const bool away = ((as_u(r) ^ xb) & 0x80000000u) == 0u;   // r has x's sign
  xb += bump ? (away ? 1u : 0xFFFFFFFFu) : 0u;
  return as_f(xb);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return as_f(__builtin_amdgcn_update_dpp(0, (int)as_u(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; the result is uniform (scalar).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: quads
  v += dpp<0x141>(v);   // row_half_mirror: 8 lanes
  v += dpp<0x140>(v);   // row_mirror: 16 lanes
  v += as_f((unsigned)__builtin_amdgcn_ds_swizzle((int)as_u(v), 0x401F));   // swap 16
  const float lo = as_f((unsigned)__builtin_amdgcn_readlane((int)as_u(v), 0));
  const float hi = as_f((unsigned)__builtin_amdgcn_readlane((int)as_u(v), 32));
  return lo + hi;
}

}  // namespace dev
}  // namespace tw
