// Unfused comparator for gfx950: the reduce-then-normalize sequence that the
// fused kernel replaces.  The blog post "TokenWeave: Why Hiding
// Tensor-Parallel Communication Needs Wave Arithmetic, Not Finer Tiles"
// measures its fused kernel against a standalone AllReduce followed by a
// standalone RMSNorm (section "What it buys"), and describes the standard
// RMSNorm as reading the tensor twice, once for the variance and once to
// scale, and writing it once (section "Fix two: RMSNorm was never
// insignificant").  On one GPU those two steps are:
//
//  reduce_kernel       reduced = round(P_0 + ... + P_{N-1})       N reads, 1 write
//  add_rmsnorm_kernel  pass 1: x = reduced + R, residual_out = round(x),
//                              sum of squares of x                 2 reads, 1 write
//                      pass 2: re-read residual_out, out = (x' * rs) * w
//                                                                  1 read,  1 write
//
// so (N+3) reads and 3 writes against the fused kernel's (N+1) and 2.  The
// arithmetic is the fused kernel's kind (compensated float32 sums, correctly
// rounded stores, a wave/LDS sum of squares in a fixed order); what differs is
// the rounding of the intermediate tensors, which the unfused flow stores and
// reads back.  The reduce step streams with the fused kernel's geometry and
// load orders; the add + RMSNorm step uses the plain row table.

#include <hip/hip_runtime.h>

#include <array>
#include <cstdio>
#include <utility>

#include "device_common.h"
#include "geometry.h"
#include "launch.h"

namespace tw {
namespace {

using namespace dev;

struct ReduceArgs {
  const u32x4* partials[kMaxPartials];
  u32x4* reduced;
  int32_t nvec;
};

struct AddNormArgs {
  const u32x4* input;
  const u32x4* residual;
  const u32x4* weight;
  u32x4* out;
  u32x4* residual_out;
  int32_t nvec;
  float hidden;
  float eps;
};

// The reduce step uses the fused kernel's row geometry, load orders and
// pacing (all loads of CHUNK slots at once, or the partials in summation order
// with SEQ in flight and a PACE pause between them), so that the comparator
// streams as well as the fused kernel does.
// Like the fused kernel it takes partial 0's address and the row length as
// leading scalar arguments (k_first, k_nvec: copies of a.partials[0] and
// a.nvec) that this file's build preloads into SGPRs, so a wave's first load
// does not wait for the argument block.  No value is shared between threads,
// so the geometry never changes a bit.
template <int N, int BLOCK, int VPT, bool BF16, int WPE, int CHUNK, int SEQ, int PACE>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(WPE)))
void reduce_kernel(const u32x4* k_first, int32_t k_nvec, ReduceArgs a) {
  constexpr int E = Elem<BF16>::kPerVec;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * k_nvec;
  const int nvec = k_nvec;
  const u32x4* tp[N];
  int vi[VPT];
  bool valid[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + j * BLOCK;
    valid[j] = v < nvec;
    vi[j] = valid[j] ? v : nvec - 1;
  }
#pragma unroll
  for (int j0 = 0; j0 < VPT; j0 += CHUNK) {
    u32x4 raw[N][CHUNK];
    float s[CHUNK][E], c[CHUNK][E];
    if constexpr (SEQ > 0) {
#pragma unroll
      for (int i = 0; i < SEQ && i < N; ++i)
#pragma unroll
        for (int jj = 0; jj < CHUNK; ++jj)
          raw[i][jj] = __builtin_nontemporal_load((i == 0 ? k_first : a.partials[i]) + base +
                                                  vi[j0 + jj]);
      // The other partials' addresses arrive while the first loads are in
      // flight.
      __builtin_amdgcn_sched_barrier(0);
      if (j0 == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) tp[i] = i == 0 ? k_first : a.partials[i];
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i)
#pragma unroll
        for (int jj = 0; jj < CHUNK; ++jj)
          raw[i][jj] = __builtin_nontemporal_load((i == 0 ? k_first : a.partials[i]) + base +
                                                  vi[j0 + jj]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (SEQ > 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < CHUNK; ++jj) {
        if (i == 0) {
          unpack<BF16>(raw[0][jj], s[jj]);
#pragma unroll
          for (int e = 0; e < E; ++e) c[jj][e] = 0.0f;
        } else {
          float t[E];
          unpack<BF16>(raw[i][jj], t);
#pragma unroll
          for (int e = 0; e < E; ++e) two_sum_into(s[jj][e], c[jj][e], t[e]);
        }
      }
      if constexpr (SEQ > 0) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PACE > 0) __builtin_amdgcn_s_sleep(PACE);
        if (i + SEQ < N) {
#pragma unroll
          for (int jj = 0; jj < CHUNK; ++jj)
            raw[i + SEQ < N ? i + SEQ : N - 1][jj] = __builtin_nontemporal_load(
                tp[i + SEQ < N ? i + SEQ : N - 1] + base + vi[j0 + jj]);
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < CHUNK; ++jj) {
      float keep[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xe = s[jj][e] + c[jj][e];
        keep[e] = BF16 ? round_to_odd(s[jj][e], c[jj][e], xe) : xe;
      }
      if (valid[j0 + jj]) store_stream(pack<BF16>(keep), a.reduced + base, vi[j0 + jj], nvec * 16);
    }
  }
}

template <int BLOCK, int VPT, bool BF16>
__global__ __launch_bounds__(BLOCK) void add_rmsnorm_kernel(AddNormArgs a) {
  constexpr int E = Elem<BF16>::kPerVec;
  constexpr int NW = BLOCK / 64;
  __shared__ float wave_part[NW];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * a.nvec;
  const int nvec = a.nvec;
  int vi[VPT];
  bool valid[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + j * BLOCK;
    valid[j] = v < nvec;
    vi[j] = valid[j] ? v : nvec - 1;
  }
  // Pass 1: x = input + residual, store it, sum of squares of x.
  u32x4 rin[VPT], rres[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    rin[j] = a.input[base + vi[j]];
    rres[j] = a.residual[base + vi[j]];
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    float s[E], c[E], t[E], keep[E];
    unpack<BF16>(rin[j], s);
    unpack<BF16>(rres[j], t);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      c[e] = 0.0f;
      two_sum_into(s[e], c[e], t[e]);
      const float xe = s[e] + c[e];
      keep[e] = BF16 ? round_to_odd(s[e], c[e], xe) : xe;
      if (valid[j]) ss = __builtin_fmaf(xe, xe, ss);
    }
    if (valid[j]) a.residual_out[base + vi[j]] = pack<BF16>(keep);
  }
  const float wsum = wave_sum(ss);
  if ((tid & 63) == 0) wave_part[tid >> 6] = wsum;
  __syncthreads();
  float total = wave_part[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) total += wave_part[w];
  const float rs = __builtin_amdgcn_rsqf(total / a.hidden + a.eps);
  // Pass 2: read the stored tensor again and scale it.  Each thread re-reads
  // only the elements it stored itself; the barrier above (a workgroup-scope
  // fence) keeps the compiler from forwarding the stored values, so these are
  // real loads, and a wave's accesses to one address stay in program order.
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const u32x4 xr = a.residual_out[base + vi[j]];
    const u32x4 wr = a.weight[vi[j]];
    float x[E], w[E], y[E];
    unpack<BF16>(xr, x);
    unpack<BF16>(wr, w);
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = (x[e] * rs) * w[e];
    if (valid[j]) store_stream(pack<BF16>(y), a.out + base, vi[j], nvec * 16);
  }
}

using ReduceFn = void (*)(const u32x4*, int32_t, ReduceArgs);
using AddNormFn = void (*)(AddNormArgs);

constexpr int reduce_order(int g, int n, bool seq_order) {
  return seq_order ? fused_geometry(g, n).seq : 0;
}
constexpr int reduce_pace(int g, int n, bool seq_order) {
  return reduce_order(g, n, seq_order) > 0 ? fused_pace(g, n) : 0;
}
// Occupancy cap of the reduce step: the fused geometry's, except above ten
// partials, where the cap would make the compiler spill the loaded values.
constexpr int reduce_waves(int g, int n) { return n <= 10 ? fused_geometry(g, n).waves_per_eu : 1; }
template <bool BF16, bool SEQ_ORDER, int G, int... Ns>
constexpr std::array<ReduceFn, sizeof...(Ns)> reduce_row(std::integer_sequence<int, Ns...>) {
  return {&reduce_kernel<Ns + 1, fused_geometry(G, Ns + 1).block, fused_geometry(G, Ns + 1).vpt,
                         BF16, reduce_waves(G, Ns + 1),
                         fused_geometry(G, Ns + 1).chunk, reduce_order(G, Ns + 1, SEQ_ORDER),
                         reduce_pace(G, Ns + 1, SEQ_ORDER)>...};
}
template <bool BF16, bool SEQ_ORDER, int... Gs>
constexpr std::array<std::array<ReduceFn, kMaxPartials>, sizeof...(Gs)> reduce_table(
    std::integer_sequence<int, Gs...>) {
  return {reduce_row<BF16, SEQ_ORDER, Gs>(std::make_integer_sequence<int, kMaxPartials>{})...};
}
template <bool BF16, int... Gs>
constexpr std::array<AddNormFn, sizeof...(Gs)> addnorm_table(std::integer_sequence<int, Gs...>) {
  return {&add_rmsnorm_kernel<kGeometry[Gs].block, kGeometry[Gs].vpt, BF16>...};
}

using Geoms = std::make_integer_sequence<int, kNumGeometries>;
// [bf16][sequenced order][row class][N - 1]
const std::array<std::array<std::array<std::array<ReduceFn, kMaxPartials>, kNumGeometries>, 2>, 2>
    kReduce = {{{reduce_table<false, false>(Geoms{}), reduce_table<false, true>(Geoms{})},
                {reduce_table<true, false>(Geoms{}), reduce_table<true, true>(Geoms{})}}};
const auto kAddNormF32 = addnorm_table<false>(std::make_integer_sequence<int, kNumGeometries>{});
const auto kAddNormBF16 = addnorm_table<true>(std::make_integer_sequence<int, kNumGeometries>{});

int shape_error(int64_t nvec, int64_t rows, int g, char* err, size_t errlen) {
  if (g < 0 || nvec > kMaxVectors || rows <= 0 || rows > 0x7FFFFFFF) {
    std::snprintf(err, errlen, "internal: launch shape outside the compiled kernels");
    return (int)hipErrorInvalidValue;
  }
  return 0;
}

}  // namespace

int launch_reduce(const ReduceLaunch& L, char* err, size_t errlen) {
  const bool bf16 = L.dtype == 1;
  const int64_t nvec = L.hidden * (bf16 ? 2 : 4) / 16;
  const int g = geometry_index(nvec);
  if (const int e = shape_error(nvec, L.num_rows, g, err, errlen)) return e;
  if (L.num_partials < 1 || L.num_partials > kMaxPartials || L.num_cus < 1) {
    std::snprintf(err, errlen, "internal: partial count outside the compiled kernels");
    return (int)hipErrorInvalidValue;
  }
  ReduceArgs k{};
  for (int i = 0; i < L.num_partials; ++i) k.partials[i] = static_cast<const u32x4*>(L.partials[i]);
  k.reduced = static_cast<u32x4*>(L.reduced);
  k.nvec = (int32_t)nvec;
  const Geometry geo = fused_geometry(g, L.num_partials);
  // The fused kernel's rule for the load order, for a chain of N tensors
  // (the reduce reads no residual).
  const bool seq = use_sequenced_order(L.num_rows, round_rows(geo.block, L.num_cus),
                                       L.num_partials - 1, geo.seq);
  const ReduceFn fn = kReduce[bf16][seq][g][L.num_partials - 1];
  // Row ranges of at most max_rows_per_dispatch rows, each its own dispatch
  // with the tensors' base pointers advanced to the range's first row.
  const int64_t chunk = max_rows_per_dispatch(geo.block);
  hipError_t e = hipSuccess;
  for (int64_t r0 = 0; r0 < L.num_rows && e == hipSuccess; r0 += chunk) {
    const int64_t n = L.num_rows - r0 < chunk ? L.num_rows - r0 : chunk;
    ReduceArgs kc = k;
    for (int i = 0; i < L.num_partials; ++i) kc.partials[i] = k.partials[i] + r0 * nvec;
    kc.reduced = k.reduced + r0 * nvec;
    const u32x4* first = kc.partials[0];
    int32_t nvec32 = kc.nvec;
    void* args[] = {&first, &nvec32, &kc};
    e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)n),
                        dim3(geo.block), args, 0, static_cast<hipStream_t>(L.stream));
  }
  if (e != hipSuccess) {
    std::snprintf(err, errlen, "hipLaunchKernel: %s", hipGetErrorString(e));
    return (int)e;
  }
  return 0;
}

int launch_add_rmsnorm(const AddNormLaunch& L, char* err, size_t errlen) {
  const bool bf16 = L.dtype == 1;
  const int64_t nvec = L.hidden * (bf16 ? 2 : 4) / 16;
  const int g = geometry_index(nvec);
  if (const int e = shape_error(nvec, L.num_rows, g, err, errlen)) return e;
  AddNormArgs k{};
  k.input = static_cast<const u32x4*>(L.input);
  k.residual = static_cast<const u32x4*>(L.residual);
  k.weight = static_cast<const u32x4*>(L.weight);
  k.out = static_cast<u32x4*>(L.out);
  k.residual_out = static_cast<u32x4*>(L.residual_out);
  k.nvec = (int32_t)nvec;
  k.hidden = (float)L.hidden;
  k.eps = L.eps;
  const AddNormFn fn = bf16 ? kAddNormBF16[g] : kAddNormF32[g];
  const int64_t chunk = max_rows_per_dispatch(kGeometry[g].block);
  hipError_t e = hipSuccess;
  for (int64_t r0 = 0; r0 < L.num_rows && e == hipSuccess; r0 += chunk) {
    const int64_t n = L.num_rows - r0 < chunk ? L.num_rows - r0 : chunk;
    AddNormArgs kc = k;
    kc.input = k.input + r0 * nvec;
    kc.residual = k.residual + r0 * nvec;
    kc.out = k.out + r0 * nvec;
    kc.residual_out = k.residual_out + r0 * nvec;
    void* args[] = {&kc};
    e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)n),
                        dim3(kGeometry[g].block), args, 0, static_cast<hipStream_t>(L.stream));
  }
  if (e != hipSuccess) {
    std::snprintf(err, errlen, "hipLaunchKernel: %s", hipGetErrorString(e));
    return (int)e;
  }
  return 0;
}

}  // namespace tw
