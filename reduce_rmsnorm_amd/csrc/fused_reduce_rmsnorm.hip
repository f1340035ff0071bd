// Fused reduce + residual-add + RMSNorm for CDNA4 (gfx950).
//
// What is computed (per token row, float32 arithmetic) follows the per-CTA
// kernel sketch in the blog post "TokenWeave: Why Hiding Tensor-Parallel
// Communication Needs Wave Arithmetic, Not Finer Tiles", section "Fix two:
// RMSNorm was never insignificant", and the RMSNorm equation in "TokenWeave
// Guide: Compute-Communication Overlap for LLMs", section "Fused
// AllReduce-RMSNorm: Bypassing Global Memory":
//
//   x   = P_0 + ... + P_{N-1} + R          reduce the partials, add residual
//   rs  = rsqrt(sum(x*x) / h + eps)        sum of squares on the registers
//   out = (x * rs) * w ,  residual_out = x
//
// Design for gfx950 (the pages' kernel ran on 2-8 SMs next to an NVSwitch
// that did the reduction; here the N partials sit in this GPU's HBM and the
// kernel is bound by HBM bandwidth, so it spreads over all 256 CUs):
//
//  * One workgroup per token row.  Each thread owns VPT 16-byte vectors of the
//    row (vector v = tid + j*BLOCK), so every load and store instruction of a
//    wave covers 1 KiB of contiguous memory.
//  * All (N+1)*VPT loads of a thread are issued before the first use; out of
//    range vectors (h not a multiple of BLOCK*VPT*elems) load a clamped,
//    valid address and contribute zero, so no branch splits the load batch.
//  * The partials and the residual are summed with an error-free
//    transformation (TwoSum) into a float32 pair (s, c); x = s + c.  For bf16
//    the stored residual is rounded to odd in float32 first and then to bf16
//    with round-to-nearest-even, which gives the correctly rounded bf16 of
//    s + c (float32 carries 16 more bits than bf16).
//  * The sum of squares is reduced within a wave64 with DPP (quad_perm,
//    row_half_mirror, row_mirror), ds_swizzle (swap 16) and two readlanes,
//    then across waves through LDS in wave order.  The order depends only on
//    the kernel geometry, which depends only on h and the element size, so a
//    row gives the same bits whichever launch (full, shard, split) runs it.
//  * Partials and residual are streamed with non-temporal loads, the outputs
//    with non-temporal stores; the weight row (read by every workgroup) uses
//    ordinary loads so it stays in L2.

#include <hip/hip_runtime.h>

#include <array>
#include <cstdio>
#include <utility>

#include "launch.h"

namespace tw {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct KArgs {
  const u32x4* partials[kMaxPartials];
  const u32x4* residual;
  const u32x4* weight;
  u32x4* out;
  u32x4* residual_out;
  int64_t row_begin;
  int32_t nvec;      // 16-byte vectors per row
  float hidden;      // h as float32 (exact: h <= 2^24)
  float eps;
};

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

template <int N, int BLOCK, int VPT, bool BF16>
__global__ __launch_bounds__(BLOCK) void fused_reduce_rmsnorm_kernel(KArgs a) {
  constexpr int E = Elem<BF16>::kPerVec;
  constexpr int NW = BLOCK / 64;
  __shared__ float wave_part[NW];

  const int tid = threadIdx.x;
  const int64_t row = a.row_begin + blockIdx.x;
  const int64_t base = row * (int64_t)a.nvec;
  const int nvec = a.nvec;

  int vi[VPT];
  bool valid[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + j * BLOCK;
    valid[j] = v < nvec;
    vi[j] = valid[j] ? v : nvec - 1;
  }

  // Issue every load of the row before the first use.
  u32x4 raw[N + 1][VPT];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      raw[i][j] = __builtin_nontemporal_load(a.partials[i] + base + vi[j]);
#pragma unroll
  for (int j = 0; j < VPT; ++j)
    raw[N][j] = __builtin_nontemporal_load(a.residual + base + vi[j]);
  u32x4 wraw[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) wraw[j] = a.weight[vi[j]];

  // Compensated float32 sum: partials in order, then the residual.
  float x[VPT][E];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    float s[E], c[E], t[E];
    unpack<BF16>(raw[0][j], s);
#pragma unroll
    for (int e = 0; e < E; ++e) c[e] = 0.0f;
#pragma unroll
    for (int i = 1; i <= N; ++i) {
      unpack<BF16>(raw[i][j], t);
#pragma unroll
      for (int e = 0; e < E; ++e) two_sum_into(s[e], c[e], t[e]);
    }
    float keep[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float xe = s[e] + c[e];
      x[j][e] = valid[j] ? xe : 0.0f;
      keep[e] = BF16 ? round_to_odd(s[e], c[e], xe) : xe;
    }
    if (valid[j])
      __builtin_nontemporal_store(pack<BF16>(keep), a.residual_out + base + vi[j]);
#pragma unroll
    for (int e = 0; e < E; ++e) ss = __builtin_fmaf(x[j][e], x[j][e], ss);
  }

  // Row sum of squares: wave, then waves in order through LDS.
  const float wsum = wave_sum(ss);
  if ((tid & 63) == 0) wave_part[tid >> 6] = wsum;
  __syncthreads();
  float total = wave_part[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) total += wave_part[w];
  const float rs = __builtin_amdgcn_rsqf(total / a.hidden + a.eps);

#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    float w[E], y[E];
    unpack<BF16>(wraw[j], w);
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = (x[j][e] * rs) * w[e];
    if (valid[j]) __builtin_nontemporal_store(pack<BF16>(y), a.out + base + vi[j]);
  }
}

using KernelFn = void (*)(KArgs);

struct Geometry { int block, vpt; };

// (threads per workgroup, vectors per thread) by 16-byte vectors per row: the
// first entry whose capacity covers the row.  Measured on MI355X at 184 MB
// per launch: for h = 8192 bf16 (1024 vectors) 512 x 2 beat 256 x 4 and
// 1024 x 1, for h = 4096 512 x 1, for h = 16384 1024 x 2.  Two vectors per
// thread keep 18 loads in flight per thread at N = 8 with about 120 VGPRs,
// so two 512-thread workgroups fit on a CU.
constexpr Geometry kGeometry[] = {
    {64, 1}, {128, 1}, {256, 1}, {512, 1}, {512, 2}, {1024, 2}, {1024, 4}, {1024, 8}};
constexpr int kNumGeometries = sizeof(kGeometry) / sizeof(kGeometry[0]);
constexpr int kMaxVectors = 8192;

int geometry_index(int64_t nvec) {
  for (int g = 0; g < kNumGeometries; ++g)
    if (nvec <= (int64_t)kGeometry[g].block * kGeometry[g].vpt) return g;
  return -1;
}

template <bool BF16, int G, int... Ns>
constexpr std::array<KernelFn, sizeof...(Ns)> row_of(std::integer_sequence<int, Ns...>) {
  return {&fused_reduce_rmsnorm_kernel<Ns + 1, kGeometry[G].block, kGeometry[G].vpt, BF16>...};
}

template <bool BF16, int... Gs>
constexpr std::array<std::array<KernelFn, kMaxPartials>, sizeof...(Gs)> table_of(
    std::integer_sequence<int, Gs...>) {
  return {row_of<BF16, Gs>(std::make_integer_sequence<int, kMaxPartials>{})...};
}

const auto kTableF32 = table_of<false>(std::make_integer_sequence<int, kNumGeometries>{});
const auto kTableBF16 = table_of<true>(std::make_integer_sequence<int, kNumGeometries>{});

}  // namespace

void kernel_geometry(int64_t hidden, int32_t elem_bytes, int* block, int* vecs_per_thread) {
  const int64_t nvec = hidden * elem_bytes / 16;
  const int g = geometry_index(nvec);
  *block = g < 0 ? 0 : kGeometry[g].block;
  *vecs_per_thread = g < 0 ? 0 : kGeometry[g].vpt;
}

int launch_fused(const FusedLaunch& L, char* err, size_t errlen) {
  const bool bf16 = L.dtype == 1;
  const int elem_bytes = bf16 ? 2 : 4;
  const int64_t nvec = L.hidden * elem_bytes / 16;
  const int g = geometry_index(nvec);
  if (g < 0 || nvec > kMaxVectors || L.num_partials < 1 || L.num_partials > kMaxPartials ||
      L.num_rows <= 0 || L.num_rows > 0x7FFFFFFF) {
    std::snprintf(err, errlen, "internal: launch shape outside the compiled kernels");
    return (int)hipErrorInvalidValue;
  }
  KArgs k{};
  for (int i = 0; i < L.num_partials; ++i) k.partials[i] = static_cast<const u32x4*>(L.partials[i]);
  k.residual = static_cast<const u32x4*>(L.residual);
  k.weight = static_cast<const u32x4*>(L.weight);
  k.out = static_cast<u32x4*>(L.out);
  k.residual_out = static_cast<u32x4*>(L.residual_out);
  k.row_begin = L.row_begin;
  k.nvec = (int32_t)nvec;
  k.hidden = (float)L.hidden;
  k.eps = L.eps;

  const KernelFn fn = bf16 ? kTableBF16[g][L.num_partials - 1] : kTableF32[g][L.num_partials - 1];
  void* args[] = {&k};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn),
                                       dim3((unsigned)L.num_rows), dim3(kGeometry[g].block), args, 0,
                                       static_cast<hipStream_t>(L.stream));
  if (e != hipSuccess) {
    std::snprintf(err, errlen, "hipLaunchKernel: %s", hipGetErrorString(e));
    return (int)e;
  }
  return 0;
}

}  // namespace tw
