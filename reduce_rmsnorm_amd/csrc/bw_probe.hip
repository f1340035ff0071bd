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

#include <hip/hip_runtime.h>

#include <array>
#include <cstdint>
#include <utility>

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

using ProbeFn = void (*)(ProbeArgs);

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
// 4: empty (grid workgroups of 1024 threads; no tensor is touched).
// Returns 0 or a HIP error code; -1 for arguments out of range.  nvec counts
// 16-byte vectors per tensor.
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
