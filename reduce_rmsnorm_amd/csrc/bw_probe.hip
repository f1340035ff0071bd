// Bandwidth probes for MI355X (gfx950): measurement only, not on the fused
// path.  They move exactly the bytes they are told to, so they serve two
// purposes in the benchmark:
//   * the achievable-bandwidth envelope for the fused kernel's traffic mix
//     (nsrc streamed reads and ndst streamed writes of equal-size tensors);
//   * calibration of the FETCH_SIZE / WRITE_SIZE hardware counters: a probe
//     that reads (writes) a known number of bytes gives the factor between the
//     counter and bytes.
//
// Every probe walks 16-byte vectors [0, nvec) of each tensor with a grid-stride
// loop; loads and stores are non-temporal, like the fused kernel's streams.
//
// A third kind of probe records where each workgroup ran (XCC and compute unit
// as the hardware reports them), which shows how a stream's CU mask maps onto
// the eight XCDs.  A fourth does nothing at all: back-to-back launches of it
// measure the fixed cost of a dependent launch of a given grid.
//
// The schedule twins bound the fused kernel's own schedule rather than a flat
// stream: one workgroup per row of the fused kernel's geometry (geometry.h),
// its load order (the N+1 tensors in summation order, one in flight per
// thread, with the same pause between tensors, or all at once), its stores of
// both outputs (the same write-through streaming buffer stores) and its one
// LDS barrier per row, with the arithmetic replaced by an xor.  What a twin gains over the fused kernel
// is what the arithmetic costs; what it lacks against the peak is the
// schedule's own bound.

#include <hip/hip_runtime.h>

#include <array>
#include <chrono>
#include <cstdint>
#include <utility>

#include "device_common.h"
#include "geometry.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxStreams = 17;
constexpr int kBlock = 256;
constexpr int kUnroll = 4;

struct ProbeArgs {
  const u32x4* src[kMaxStreams];
  u32x4* dst[kMaxStreams];
  int32_t nsrc, ndst;
  int64_t nvec;
};

// NSRC reads and ndst writes per vector index, kUnroll indices per thread in
// flight (NSRC is a template argument so that every load is issued up front).
template <int NSRC>
__global__ __launch_bounds__(kBlock) void probe_read_write(ProbeArgs a) {
  const int64_t stride = (int64_t)gridDim.x * kBlock * kUnroll;
  for (int64_t i0 = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x; i0 < a.nvec; i0 += stride) {
    u32x4 acc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kBlock;
      const int64_t ii = i < a.nvec ? i : a.nvec - 1;
      u32x4 t = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < NSRC; ++k) t ^= __builtin_nontemporal_load(a.src[k] + ii);
      acc[u] = t;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kBlock;
      if (i < a.nvec)
        for (int k = 0; k < a.ndst; ++k) __builtin_nontemporal_store(acc[u] + (unsigned)k, a.dst[k] + i);
    }
  }
}

// Reads only.  The xor of everything read is stored only if it equals an
// unlikely pattern, which keeps the loads alive without writing.
template <int NSRC>
__global__ __launch_bounds__(kBlock) void probe_read(ProbeArgs a) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  u32x4 t = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < a.nvec; i += stride)
#pragma unroll
    for (int k = 0; k < NSRC; ++k) t ^= __builtin_nontemporal_load(a.src[k] + i);
  const int64_t me = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t.x == 0x7F7F1234u && t.y == 0x00001234u && a.ndst > 0 && me < a.nvec) a.dst[0][me] = t;
}

// Writes only.
__global__ __launch_bounds__(kBlock) void probe_write(ProbeArgs a) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < a.nvec; i += stride) {
    const u32x4 t = {(unsigned)i, 1u, 2u, 3u};
    for (int k = 0; k < a.ndst; ++k) __builtin_nontemporal_store(t, a.dst[k] + i);
  }
}

// Hardware register reads (s_getreg immediates: size-1 in [15:11], bit offset in
// [10:6], register id in [5:0]).  HW_ID (id 4) packs wave, SIMD, pipe, CU,
// shader-array and shader-engine ids; XCC_ID (id 20) holds the XCD's index in
// its low four bits.
constexpr int kHwIdAll = (31 << 11) | 4;
constexpr int kXccId = (3 << 11) | 20;
constexpr int kPlacementBlock = 64;

// One wave per workgroup.  Each workgroup stays resident for a short, fixed
// time (so that the dispatcher spreads the grid over every CU it may use), then
// lane 0 stores {HW_ID, XCC_ID, workgroup index, 1} at dst[0][workgroup].
__global__ __launch_bounds__(kPlacementBlock) void probe_placement(ProbeArgs a) {
  const unsigned hw = __builtin_amdgcn_s_getreg(kHwIdAll);
  const unsigned xcc = __builtin_amdgcn_s_getreg(kXccId);
  for (int k = 0; k < 32; ++k) __builtin_amdgcn_s_sleep(8);
  if (threadIdx.x == 0 && (int64_t)blockIdx.x < a.nvec) {
    const u32x4 rec = {hw, xcc, (unsigned)blockIdx.x, 1u};
    a.dst[0][blockIdx.x] = rec;
  }
}

// Schedule twin of the fused kernel for rows of BLOCK * VPT vectors and NSRC
// = N + 1 tensors: vector slot j of a thread is tid + j * BLOCK, the slots are
// taken one at a time, and each slot's tensors are loaded in order with one
// in flight (SEQ) and a pause of PACE * 64 clocks after each, or all at once
// (!SEQ).  WRITES: both outputs are stored (residual_out per slot, out after
// the barrier) with the fused kernel's store (store_stream); otherwise the
// loads are kept alive by a store that never happens for real data.
template <int NSRC, int BLOCK, int VPT, bool SEQ, int PACE, bool WRITES>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(8)))
void probe_row_twin(ProbeArgs a) {
  constexpr int NW = BLOCK / 64;
  __shared__ unsigned part[NW];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * (BLOCK * VPT);
  u32x4 acc[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int64_t v = base + tid + j * BLOCK;
    if constexpr (SEQ) {
      u32x4 raw = __builtin_nontemporal_load(a.src[0] + v);
#pragma unroll
      for (int i = 0; i < NSRC; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        acc[j] = i == 0 ? raw : acc[j] ^ raw;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PACE > 0) __builtin_amdgcn_s_sleep(PACE);
        if (i + 1 < NSRC) raw = __builtin_nontemporal_load(a.src[i + 1 < NSRC ? i + 1 : 0] + v);
      }
    } else {
      u32x4 raw[NSRC];
#pragma unroll
      for (int i = 0; i < NSRC; ++i) raw[i] = __builtin_nontemporal_load(a.src[i] + v);
      acc[j] = raw[0];
#pragma unroll
      for (int i = 1; i < NSRC; ++i) acc[j] ^= raw[i];
    }
    if constexpr (WRITES)
      tw::dev::store_stream(acc[j], a.dst[1] + base, tid + j * BLOCK, BLOCK * VPT * 16);
  }
  unsigned x = 0;
#pragma unroll
  for (int j = 0; j < VPT; ++j) x ^= acc[j].x;
  if ((tid & 63) == 0) part[tid >> 6] = x;
  __syncthreads();
  unsigned tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += part[w];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int64_t v = base + tid + j * BLOCK;
    const u32x4 o = acc[j] + tot;
    if constexpr (WRITES) tw::dev::store_stream(o, a.dst[0] + base, tid + j * BLOCK, BLOCK * VPT * 16);
    else if (o.x == 0x7F7F1234u && o.y == 0x00001234u && o.z == 0x5A5A5A5Au) a.dst[0][v] = o;
  }
}

using ProbeFn = void (*)(ProbeArgs);

// Twins for the fused kernel's sequenced row classes, by N: 1024 x 1 (rows
// of 1024 vectors, h = 8192 bf16), 512 x 1 (512 vectors, h = 4096) and 1024 x
// 2 (2048 vectors, h = 16384), each with the pace the fused kernel uses for
// that class and N, and all-at-once forms for launches under one round.
constexpr int kTwinClass[3] = {1024, 512, 2048};    // vectors per row
constexpr int twin_pace(int c, int n) {
  return tw::fused_pace(tw::geometry_index(kTwinClass[c]), n);
}
template <int C> struct TwinShape;
template <> struct TwinShape<0> { static constexpr int block = 1024, vpt = 1; };
template <> struct TwinShape<1> { static constexpr int block = 512, vpt = 1; };
template <> struct TwinShape<2> { static constexpr int block = 1024, vpt = 2; };
template <int C, bool SEQ, bool WRITES, int... Ns>
constexpr std::array<ProbeFn, sizeof...(Ns)> twin_row(std::integer_sequence<int, Ns...>) {
  return {&probe_row_twin<Ns + 2, TwinShape<C>::block, TwinShape<C>::vpt, SEQ,
                          SEQ ? twin_pace(C, Ns + 1) : 0, WRITES>...};
}
template <bool SEQ, bool WRITES>
constexpr std::array<std::array<ProbeFn, 16>, 3> twin_table() {
  return {twin_row<0, SEQ, WRITES>(std::make_integer_sequence<int, 16>{}),
          twin_row<1, SEQ, WRITES>(std::make_integer_sequence<int, 16>{}),
          twin_row<2, SEQ, WRITES>(std::make_integer_sequence<int, 16>{})};
}
// [sequenced][writes][class][N - 1]
const std::array<std::array<std::array<std::array<ProbeFn, 16>, 3>, 2>, 2> kTwin = {
    {{twin_table<false, false>(), twin_table<false, true>()},
     {twin_table<true, false>(), twin_table<true, true>()}}};

template <int... Ks>
constexpr std::array<ProbeFn, sizeof...(Ks)> rw_table(std::integer_sequence<int, Ks...>) {
  return {&probe_read_write<Ks + 1>...};
}
template <int... Ks>
constexpr std::array<ProbeFn, sizeof...(Ks)> r_table(std::integer_sequence<int, Ks...>) {
  return {&probe_read<Ks + 1>...};
}
const auto kReadWrite = rw_table(std::make_integer_sequence<int, kMaxStreams>{});
const auto kRead = r_table(std::make_integer_sequence<int, kMaxStreams>{});

// No memory access and no work: 1024 threads per workgroup, as the fused
// kernel's widest rows use.
constexpr int kEmptyBlock = 1024;
__global__ __launch_bounds__(kEmptyBlock) void probe_empty(ProbeArgs) {}

}  // namespace

// kind 0: read+write, 1: read only, 2: write only, 3: placement (one 16-byte
// record per workgroup into dst[0], which must hold at least grid vectors),
// 4: empty (grid workgroups of 1024 threads; no tensor is touched),
// 5: schedule twin reading nsrc tensors and writing dst[0] (out) and dst[1]
// (residual_out), 6: the same twin without the writes (dst[0] must still be
// given).  The twins take grid rows of nvec / grid vectors each, which must be
// 1024, 512 or 2048; `sequenced` selects the fused kernel's sequenced load
// order (else all loads at once).
// Returns 0 or a HIP error code; -1 for arguments out of range.  nvec counts
// 16-byte vectors per tensor.
extern "C" int tw_probe_twin_launch(int kind, int sequenced, const void* const* src, int nsrc,
                                    void* const* dst, int64_t nvec, int grid, void* stream) {
  if ((kind != 5 && kind != 6) || nsrc < 2 || nsrc > kMaxStreams || grid < 1 || nvec < 1 ||
      nvec % grid != 0 || dst == nullptr || dst[0] == nullptr || (kind == 5 && dst[1] == nullptr))
    return -1;
  const int64_t row = nvec / grid;
  int c = -1;
  for (int k = 0; k < 3; ++k)
    if (row == kTwinClass[k]) c = k;
  if (c < 0) return -1;
  ProbeArgs a{};
  for (int k = 0; k < nsrc; ++k) {
    if (src[k] == nullptr) return -1;
    a.src[k] = static_cast<const u32x4*>(src[k]);
  }
  a.dst[0] = static_cast<u32x4*>(dst[0]);
  a.dst[1] = kind == 5 ? static_cast<u32x4*>(dst[1]) : nullptr;
  a.nsrc = nsrc;
  a.ndst = kind == 5 ? 2 : 1;
  a.nvec = nvec;
  void* args[] = {&a};
  const ProbeFn fn = kTwin[sequenced != 0][kind == 5][c][nsrc - 2];
  const int block = c == 1 ? 512 : 1024;
  return (int)hipLaunchKernel((const void*)fn, dim3(grid), dim3(block), args, 0,
                              static_cast<hipStream_t>(stream));
}

// Host time of one launch of the empty kernel through a launch API: api 0
// hipLaunchKernel, 1 hipModuleLaunchKernel on a function handle fetched once,
// 2 hipExtLaunchKernel.  `launches` back-to-back launches of `grid`
// workgroups on `stream`, timed on the host with no synchronization inside the
// loop, best of five; *us_per_launch receives the time per launch.  The caller
// keeps `launches` small enough for the GPU to keep up (an empty launch takes
// under 2 us).  Returns 0 or a HIP error code; -1 for arguments out of range.
extern "C" int tw_probe_launch_cost(int api, int grid, int launches, void* stream,
                                    double* us_per_launch) {
  if (api < 0 || api > 2 || grid < 1 || grid > 65536 || launches < 1 || launches > 100000 ||
      us_per_launch == nullptr)
    return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  ProbeArgs e{};
  void* args[] = {&e};
  hipFunction_t f = nullptr;
  if (api == 1) {
    const hipError_t r = hipGetFuncBySymbol(&f, (const void*)&probe_empty);
    if (r != hipSuccess) return (int)r;
  }
  auto one = [&]() -> hipError_t {
    if (api == 0)
      return hipLaunchKernel((const void*)&probe_empty, dim3(grid), dim3(kEmptyBlock), args, 0, s);
    if (api == 1) return hipModuleLaunchKernel(f, grid, 1, 1, kEmptyBlock, 1, 1, 0, s, args, nullptr);
    return hipExtLaunchKernel((const void*)&probe_empty, dim3(grid), dim3(kEmptyBlock), args, 0, s,
                              nullptr, nullptr, 0);
  };
  double best = 1e30;
  for (int rep = 0; rep < 6; ++rep) {
    hipError_t r = hipStreamSynchronize(s);
    if (r != hipSuccess) return (int)r;
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < launches; ++i)
      if ((r = one()) != hipSuccess) return (int)r;
    const auto t1 = std::chrono::steady_clock::now();
    const double us = std::chrono::duration<double, std::micro>(t1 - t0).count() / launches;
    if (rep > 0 && us < best) best = us;     // the first pass warms up
  }
  const hipError_t r = hipStreamSynchronize(s);
  if (r != hipSuccess) return (int)r;
  *us_per_launch = best;
  return 0;
}

extern "C" int tw_probe_launch(int kind, const void* const* src, int nsrc, void* const* dst,
                               int ndst, int64_t nvec, int grid, void* stream) {
  if (kind < 0 || kind > 4 || nsrc < 0 || nsrc > kMaxStreams || ndst < 0 || ndst > kMaxStreams ||
      nvec < 1 || grid < 1 || grid > 65536)
    return -1;
  if (kind == 4) {
    ProbeArgs e{};
    void* eargs[] = {&e};
    return (int)hipLaunchKernel((const void*)&probe_empty, dim3(grid), dim3(kEmptyBlock), eargs,
                                0, static_cast<hipStream_t>(stream));
  }
  if (kind == 3) {
    if (ndst != 1 || dst[0] == nullptr || nvec < grid) return -1;
    ProbeArgs p{};
    p.dst[0] = static_cast<u32x4*>(dst[0]);
    p.ndst = 1;
    p.nvec = nvec;
    void* pargs[] = {&p};
    return (int)hipLaunchKernel((const void*)&probe_placement, dim3(grid), dim3(kPlacementBlock),
                                pargs, 0, static_cast<hipStream_t>(stream));
  }
  if ((kind != 2 && nsrc < 1) || (kind != 1 && ndst < 1)) return -1;
  ProbeArgs a{};
  for (int k = 0; k < nsrc; ++k) {
    if (src[k] == nullptr) return -1;
    a.src[k] = static_cast<const u32x4*>(src[k]);
  }
  for (int k = 0; k < ndst; ++k) {
    if (dst[k] == nullptr) return -1;
    a.dst[k] = static_cast<u32x4*>(dst[k]);
  }
  a.nsrc = nsrc;
  a.ndst = ndst;
  a.nvec = nvec;
  const void* fn = kind == 0 ? (const void*)kReadWrite[nsrc - 1]
                 : kind == 1 ? (const void*)kRead[nsrc - 1] : (const void*)&probe_write;
  void* args[] = {&a};
  return (int)hipLaunchKernel(fn, dim3(grid), dim3(kBlock), args, 0, static_cast<hipStream_t>(stream));
}
