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
//  * Two load orders with the same arithmetic.  Either all (N+1)*VPT loads
//    of a thread are issued before the first use (wide rows issue them a few
//    vector slots at a time), or the tensors are loaded in summation order
//    with one or two in flight per thread, so that fewer DRAM regions are
//    open across the chip at a time and the stream is faster.  The geometry
//    table (geometry.h) says which row classes and partial counts use the
//    sequenced order; a launch too small to fill the CUs issues all loads at
//    once regardless, since it would otherwise wait out one latency per
//    tensor, and so does a launch just past one round of workgroups with many
//    tensors per row, whose extra rows would run almost alone.  A launch
//    whose last round is at most half full runs the strided kernel below
//    instead of one workgroup per row.  In the sequenced order a wave pauses briefly (s_sleep, a pace
//    set per row class and N in geometry.h) after adding each tensor, before
//    requesting the next: with many tensors per row, fewer requests in flight
//    stream faster.  Out of range vectors (h not a multiple of
//    BLOCK*VPT*elems) load a clamped, valid address and contribute zero, so no
//    branch splits a load batch.
//  * The partials and the residual are summed with an error-free
//    transformation (TwoSum) into a float32 pair (s, c); x = s + c.  For bf16
//    the stored residual is rounded to odd in float32 first and then to bf16
//    with round-to-nearest-even, which gives the correctly rounded bf16 of
//    s + c (float32 carries 16 more bits than bf16).
//  * The sum of squares is reduced within a wave64 with DPP (quad_perm,
//    row_half_mirror, row_mirror), ds_swizzle (swap 16) and two readlanes,
//    then across waves through LDS in wave order.  The order depends only on
//    the kernel geometry, which depends only on h, the element size and N (not
//    on the launch or its load order), so a row gives the same bits whichever
//    launch (full, shard, split, grid) runs it.
//  * Partials and residual are streamed with non-temporal loads, the outputs
//    with non-temporal stores that write through the L2 (store_stream); the
//    weight row (read by every workgroup) uses ordinary loads so it stays in
//    L2.
//  * The one-row-per-workgroup kernel takes the first tensor's address, the
//    first row and the row length as leading scalar arguments, which this
//    file's build preloads into SGPRs at wave launch (kernel-argument
//    preloading, -mllvm -amdgpu-kernarg-preload-count=3).  A wave issues its
//    row's first load at once; the rest of the argument block (the other
//    tensors' addresses, the weight) arrives from memory while that load is in
//    flight.

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


struct KArgs {
  const u32x4* partials[kMaxPartials];
  const u32x4* residual;
  const u32x4* weight;
  u32x4* out;
  u32x4* residual_out;
  int64_t row_begin;
  int64_t row_end;   // one past the launch's last row (read by the strided kernel)
  int32_t nvec;      // 16-byte vectors per row
  float hidden;      // h as float32 (exact: h <= 2^24)
  float eps;
};

// Tensor I of the summation: partial I for I < N, the residual for I == N.
// Partial 0 is k_first, the kernel's own (preloaded) copy of its address.
#define TW_TENSOR(I) ((I) == 0 ? k_first : (I) < N ? a.partials[(I) < N ? (I) : 0] : a.residual)

// Store of an output vector VEC of the row at `base`: written through the L2
// (store_stream) where the kernel's constant WT says so, else a plain
// non-temporal store (the strided kernel's many-partial forms, where the
// buffer store's offset register would spill at the occupancy cap, and the
// consecutive-rows kernel on fewer workgroups than CUs).
#define TW_STORE(V, TENSOR, VEC)                                                       \
  {                                                                                    \
    if constexpr (WT) store_stream((V), (TENSOR) + base, (VEC), nvec * 16);           \
    else __builtin_nontemporal_store((V), (TENSOR) + base + (VEC));                    \
  }

// Finishing one vector slot J from its compensated pair (S, C): x, the stored
// residual (correctly rounded for bf16) and the slot's share of the sum of
// squares, added in slot order.
#define TW_FINISH_SLOT(J, S, C)                                                        \
  {                                                                                    \
    float keep[E];                                                                     \
_Pragma("unroll")                                                                      \
    for (int e = 0; e < E; ++e) {                                                      \
      const float xe = (S)[e] + (C)[e];                                                \
      x[J][e] = valid[J] ? xe : 0.0f;                                                  \
      keep[e] = BF16 ? round_to_odd((S)[e], (C)[e], xe) : xe;                          \
    }                                                                                  \
    if (valid[J]) TW_STORE(pack<BF16>(keep), a.residual_out, vi[J])                    \
_Pragma("unroll")                                                                      \
    for (int e = 0; e < E; ++e) ss = __builtin_fmaf(x[J][e], x[J][e], ss);             \
  }

// The sequenced summation of CHUNK vector slots starting at slot J0 of the
// row at `base`: tensor i is added into (s, c) once it has arrived, then,
// after a pause of PACE * 64 clocks, tensor i + SEQ is requested.  Tensors
// 0 .. SEQ-1 must already be in flight in raw[], and tp[] must hold the
// tensors' addresses.
#define TW_SEQ_ADD(J0)                                                                 \
_Pragma("unroll")                                                                      \
  for (int i = 0; i <= N; ++i) {                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                 \
_Pragma("unroll")                                                                      \
    for (int jj = 0; jj < CHUNK; ++jj) {                                               \
      if (i == 0) {                                                                    \
        unpack<BF16>(raw[0][jj], s[jj]);                                               \
_Pragma("unroll")                                                                      \
        for (int e = 0; e < E; ++e) c[jj][e] = 0.0f;                                   \
      } else {                                                                         \
        float t[E];                                                                    \
        unpack<BF16>(raw[i][jj], t);                                                   \
_Pragma("unroll")                                                                      \
        for (int e = 0; e < E; ++e) two_sum_into(s[jj][e], c[jj][e], t[e]);            \
      }                                                                                \
    }                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                 \
    if constexpr (PACE > 0) __builtin_amdgcn_s_sleep(PACE);                            \
    if (i + SEQ <= N) {                                                                \
_Pragma("unroll")                                                                      \
      for (int jj = 0; jj < CHUNK; ++jj)                                               \
        raw[i + SEQ <= N ? i + SEQ : N][jj] =                                          \
            __builtin_nontemporal_load(tp[i + SEQ <= N ? i + SEQ : N] + base +          \
                                       vi[(J0) + jj]);                                 \
    }                                                                                  \
  }

// The end of a row: the row's sum of squares (wave, then the waves in order
// through the LDS array PART[BLOCK / 64]), rs, and the `out` stores.
#define TW_NORMALIZE(PART)                                                             \
  /* Row sum of squares: wave, then waves in order through LDS. */                     \
  const float wsum = wave_sum(ss);                                                     \
  if ((tid & 63) == 0) (PART)[tid >> 6] = wsum;                                        \
  __syncthreads();                                                                     \
  float total = (PART)[0];                                                             \
_Pragma("unroll")                                                                      \
  for (int w = 1; w < NW; ++w) total += (PART)[w];                                     \
  const float rs = __builtin_amdgcn_rsqf(total / a.hidden + a.eps);                    \
                                                                                       \
_Pragma("unroll")                                                                      \
  for (int j = 0; j < VPT; ++j) {                                                      \
    float w[E], y[E];                                                                  \
    unpack<BF16>(wraw[j], w);                                                          \
_Pragma("unroll")                                                                      \
    for (int e = 0; e < E; ++e) y[e] = (x[j][e] * rs) * w[e];                          \
    if (valid[j]) TW_STORE(pack<BF16>(y), a.out, vi[j])                                \
  }

// The per-row body of both fused kernels: everything the fused step does to
// the row ROW_EXPR, by one workgroup, with the wave partial sums in the LDS
// array wave_part[BLOCK / 64], E, NW, k_first (partial 0) and k_nvec (16-byte
// vectors per row) in scope.  Written once and expanded
// into each kernel, so that both compile it in a kernel's own context (an
// inlined device function allocated registers differently and spilled).
//
// Two load orders, chosen by the geometry and giving the same arithmetic:
//  * SEQ == 0: the N+1 loads of CHUNK vector slots are issued together.  With
//    CHUNK == VPT every load of the row is in flight before the first use;
//    wide rows take CHUNK slots at a time so their values fit in registers.
//  * SEQ == D > 0: the tensors are loaded in summation order, D of them in
//    flight: tensor i + D is requested once tensor i has been added (and,
//    with PACE > 0, after a pause of PACE * 64 clocks).  Fewer DRAM regions
//    are open at a time across the chip, which streams faster when there are
//    many partials.  The first loads go out before anything
//    else; the other tensors' addresses and the weight row are fetched while
//    they are in flight (scheduling barriers keep that order).
#define TW_FUSED_ROW_BODY(ROW_EXPR)                                                    \
  const int tid = threadIdx.x;                                                         \
  const int64_t row = (ROW_EXPR);                                                      \
  const int64_t base = row * (int64_t)k_nvec;                                          \
  const int nvec = k_nvec;                                                             \
                                                                                       \
  int vi[VPT];                                                                         \
  bool valid[VPT];                                                                     \
_Pragma("unroll")                                                                      \
  for (int j = 0; j < VPT; ++j) {                                                      \
    const int v = tid + j * BLOCK;                                                     \
    valid[j] = v < nvec;                                                               \
    vi[j] = valid[j] ? v : nvec - 1;                                                   \
  }                                                                                    \
                                                                                       \
  u32x4 wraw[VPT];                                                                     \
  if constexpr (CHUNK == VPT && SEQ == 0) {                                            \
_Pragma("unroll")                                                                      \
    for (int j = 0; j < VPT; ++j) wraw[j] = a.weight[vi[j]];                           \
  }                                                                                    \
                                                                                       \
  /* Compensated float32 sum: partials in order, then the residual. */                 \
  float x[VPT][E];                                                                     \
  float ss = 0.0f;                                                                     \
  if constexpr (SEQ > 0) {                                                             \
    const u32x4* tp[N + 1];                                                            \
_Pragma("unroll")                                                                      \
    for (int j0 = 0; j0 < VPT; j0 += CHUNK) {                                          \
      u32x4 raw[N + 1][CHUNK];                                                         \
      float s[CHUNK][E], c[CHUNK][E];                                                  \
_Pragma("unroll")                                                                      \
      for (int i = 0; i < SEQ && i <= N; ++i)                                          \
_Pragma("unroll")                                                                      \
        for (int jj = 0; jj < CHUNK; ++jj)                                             \
          raw[i][jj] = __builtin_nontemporal_load(TW_TENSOR(i) + base + vi[j0 + jj]);  \
      __builtin_amdgcn_sched_barrier(0);                                               \
      if (j0 == 0) {                                                                   \
_Pragma("unroll")                                                                      \
        for (int i = 0; i <= N; ++i) tp[i] = TW_TENSOR(i);                             \
        if (CHUNK == VPT) {                                                            \
_Pragma("unroll")                                                                      \
          for (int j = 0; j < VPT; ++j) wraw[j] = a.weight[vi[j]];                     \
        }                                                                              \
      }                                                                                \
      __builtin_amdgcn_sched_barrier(0);                                               \
      TW_SEQ_ADD(j0)                                                                   \
_Pragma("unroll")                                                                      \
      for (int jj = 0; jj < CHUNK; ++jj) TW_FINISH_SLOT(j0 + jj, s[jj], c[jj])         \
    }                                                                                  \
  } else {                                                                             \
_Pragma("unroll")                                                                      \
    for (int j0 = 0; j0 < VPT; j0 += CHUNK) {                                          \
      u32x4 raw[N + 1][CHUNK];                                                         \
_Pragma("unroll")                                                                      \
      for (int i = 0; i < N; ++i)                                                      \
_Pragma("unroll")                                                                      \
        for (int jj = 0; jj < CHUNK; ++jj)                                             \
          raw[i][jj] = __builtin_nontemporal_load(TW_TENSOR(i) + base + vi[j0 + jj]);  \
_Pragma("unroll")                                                                      \
      for (int jj = 0; jj < CHUNK; ++jj)                                               \
        raw[N][jj] = __builtin_nontemporal_load(a.residual + base + vi[j0 + jj]);      \
_Pragma("unroll")                                                                      \
      for (int jj = 0; jj < CHUNK; ++jj) {                                             \
        const int j = j0 + jj;                                                         \
        float s[E], c[E], t[E];                                                        \
        unpack<BF16>(raw[0][jj], s);                                                   \
_Pragma("unroll")                                                                      \
        for (int e = 0; e < E; ++e) c[e] = 0.0f;                                       \
_Pragma("unroll")                                                                      \
        for (int i = 1; i <= N; ++i) {                                                 \
          unpack<BF16>(raw[i][jj], t);                                                 \
_Pragma("unroll")                                                                      \
          for (int e = 0; e < E; ++e) two_sum_into(s[e], c[e], t[e]);                  \
        }                                                                              \
        TW_FINISH_SLOT(j, s, c)                                                        \
      }                                                                                \
      if constexpr (CHUNK < VPT) __builtin_amdgcn_sched_barrier(0);                    \
    }                                                                                  \
  }                                                                                    \
  if constexpr (CHUNK < VPT) {                                                         \
_Pragma("unroll")                                                                      \
    for (int j = 0; j < VPT; ++j) wraw[j] = a.weight[vi[j]];                           \
  }                                                                                    \
                                                                                       \
  TW_NORMALIZE(wave_part)

// One workgroup per row: the launch grid is the row count.  k_first,
// k_row_begin and k_nvec repeat a.partials[0], a.row_begin and a.nvec as
// preloaded scalar arguments.
template <int N, int BLOCK, int VPT, bool BF16, int WPE, int CHUNK, int SEQ, int PACE>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(WPE)))
void fused_reduce_rmsnorm_kernel(const u32x4* k_first, int64_t k_row_begin, int32_t k_nvec,
                                 KArgs a) {
  constexpr int E = Elem<BF16>::kPerVec;
  constexpr int NW = BLOCK / 64;
  constexpr bool WT = true;
  __shared__ float wave_part[NW];
  TW_FUSED_ROW_BODY(k_row_begin + blockIdx.x)
}

// One resident round of workgroups over a launch of one to four rounds of
// rows: workgroup b takes rows b, b + G, b + 2G, ... (G, the grid, is one
// round), in the sequenced load order.  Before a row's sum of squares is
// reduced, the workgroup requests the first tensors of its next row, so the
// barrier and the `out` stores overlap that row's first loads.  With one
// workgroup per row, the rows past the last full round start on whichever
// CUs free up first; here the workgroups that carry them were placed with
// the first round.  That is faster when the last round is at most half full
// (the launch rule is use_strided_grid in geometry.h).  The per-row
// arithmetic is the one-row kernel's (the same macros), so a row gives the
// same bits in either kernel.  Two LDS buffers for the wave sums, used alternately,
// make one barrier per row enough: a wave can only write a buffer again after
// passing the next row's barrier, which every wave reaches after reading it.
template <int N, int BLOCK, int VPT, bool BF16, int WPE, int CHUNK, int SEQ, int PACE>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(WPE)))
void fused_reduce_rmsnorm_strided_kernel(const u32x4* k_first, int64_t k_row_begin,
                                         int32_t k_nvec, KArgs a) {
  static_assert(SEQ > 0 && CHUNK == VPT, "the strided kernel loads all slots in one sequence");
  constexpr int E = Elem<BF16>::kPerVec;
  constexpr int NW = BLOCK / 64;
  constexpr bool WT = N <= 9;
  __shared__ float wave_part[2][NW];
  const int tid = threadIdx.x;
  const int nvec = k_nvec;
  int vi[VPT];
  bool valid[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + j * BLOCK;
    valid[j] = v < nvec;
    vi[j] = valid[j] ? v : nvec - 1;
  }
  int64_t row = k_row_begin + blockIdx.x;
  u32x4 raw[N + 1][CHUNK];
#pragma unroll
  for (int i = 0; i < SEQ && i <= N; ++i)
#pragma unroll
    for (int jj = 0; jj < CHUNK; ++jj)
      raw[i][jj] = __builtin_nontemporal_load(TW_TENSOR(i) + row * (int64_t)nvec + vi[jj]);
  __builtin_amdgcn_sched_barrier(0);
  const u32x4* tp[N + 1];
#pragma unroll
  for (int i = 0; i <= N; ++i) tp[i] = TW_TENSOR(i);
  u32x4 wraw[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) wraw[j] = a.weight[vi[j]];
  __builtin_amdgcn_sched_barrier(0);
  for (int parity = 0;; parity ^= 1) {
    // Recomputed from the row each time: carried across iterations, the
    // compiler keeps it in vector registers and spills.
    const int64_t base = row * (int64_t)nvec;
    float x[VPT][E];
    float ss = 0.0f;
    float s[CHUNK][E], c[CHUNK][E];
    TW_SEQ_ADD(0)
#pragma unroll
    for (int jj = 0; jj < CHUNK; ++jj) TW_FINISH_SLOT(jj, s[jj], c[jj])
    const int64_t next = row + gridDim.x;
    const bool more = next < a.row_end;           // the same for the whole workgroup
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
#pragma unroll
      for (int i = 0; i < SEQ && i <= N; ++i)
#pragma unroll
        for (int jj = 0; jj < CHUNK; ++jj)
          raw[i][jj] = __builtin_nontemporal_load(tp[i] + next * (int64_t)nvec + vi[jj]);
    }
    __builtin_amdgcn_sched_barrier(0);
    TW_NORMALIZE(wave_part[parity])
    if (!more) break;
    row = next;
  }
}

// A fixed number of workgroups: workgroup b takes the consecutive rows
// [b*rows_per_wg, min((b+1)*rows_per_wg, row_end)), as the blog's kernel
// sketch partitions tokens over its CTAs (tokens per CTA = ceil(T / grid)).
// A barrier between rows keeps a row's wave partial sums from overwriting the
// previous row's while a slower wave still reads them.  Few workgroups are
// launched by design, so no occupancy cap is requested.  WT picks the store
// form by the grid (rows_form below): with fewer workgroups than CUs the plain
// non-temporal stores are the faster, from one workgroup per CU on the
// write-through ones (profiles: "Store form of the consecutive-rows kernel").
template <int N, int BLOCK, int VPT, bool BF16, int CHUNK, int SEQ, int PACE, bool WT>
__global__ __launch_bounds__(BLOCK) void fused_reduce_rmsnorm_rows_kernel(KArgs a,
                                                                          int64_t rows_per_wg,
                                                                          int64_t row_end) {
  constexpr int E = Elem<BF16>::kPerVec;
  constexpr int NW = BLOCK / 64;
  __shared__ float wave_part[NW];
  const u32x4* const k_first = a.partials[0];
  const int32_t k_nvec = a.nvec;
  const int64_t first = a.row_begin + (int64_t)blockIdx.x * rows_per_wg;
  const int64_t last = first + rows_per_wg < row_end ? first + rows_per_wg : row_end;
  for (int64_t r = first; r < last; ++r) {
    if (r != first) __syncthreads();
    TW_FUSED_ROW_BODY(r)
  }
}

using KernelFn = void (*)(const u32x4*, int64_t, int32_t, KArgs);
using RowsKernelFn = void (*)(KArgs, int64_t, int64_t);

// Kernel tables by [row class][N - 1].  SEQ_ORDER selects the geometry's own
// load order; without it every entry takes the short form (all tensors at
// once, or a few in flight for 512 x 3; the same arithmetic, for launches too
// small to fill the CUs).
constexpr int load_order(int g, int n, bool seq_order) {
  return seq_order ? fused_geometry(g, n).seq : short_form_depth(fused_geometry(g, n));
}
constexpr int load_pace(int g, int n, bool seq_order) {
  return seq_order && load_order(g, n, seq_order) > 0 ? fused_pace(g, n) : 0;
}
constexpr int load_waves_per_eu(int g, int n, bool seq_order) {
  return seq_order ? fused_geometry(g, n).waves_per_eu : short_form_waves_per_eu(g, n);
}
template <bool BF16, bool SEQ_ORDER, int G, int... Ns>
constexpr std::array<KernelFn, sizeof...(Ns)> row_of(std::integer_sequence<int, Ns...>) {
  return {&fused_reduce_rmsnorm_kernel<Ns + 1, fused_geometry(G, Ns + 1).block,
                                       fused_geometry(G, Ns + 1).vpt, BF16,
                                       load_waves_per_eu(G, Ns + 1, SEQ_ORDER),
                                       fused_geometry(G, Ns + 1).chunk,
                                       load_order(G, Ns + 1, SEQ_ORDER),
                                       load_pace(G, Ns + 1, SEQ_ORDER)>...};
}
// The strided kernel exists for the sequenced geometries that load all of a
// thread's vector slots in one sequence (1024 x 1 and 512 x 1; the 1024 x 2
// class, one slot at a time, would spill).
template <bool BF16, int G, int NN>
constexpr KernelFn strided_fn() {
  if constexpr (fused_geometry(G, NN).seq > 0 &&
                fused_geometry(G, NN).chunk == fused_geometry(G, NN).vpt)
    return &fused_reduce_rmsnorm_strided_kernel<
        NN, fused_geometry(G, NN).block, fused_geometry(G, NN).vpt, BF16,
        fused_geometry(G, NN).waves_per_eu, fused_geometry(G, NN).chunk,
        fused_geometry(G, NN).seq, fused_pace(G, NN)>;
  else
    return nullptr;
}
template <bool BF16, int G, int... Ns>
constexpr std::array<KernelFn, sizeof...(Ns)> strided_row_of(std::integer_sequence<int, Ns...>) {
  return {strided_fn<BF16, G, Ns + 1>()...};
}
template <bool BF16, int... Gs>
constexpr std::array<std::array<KernelFn, kMaxPartials>, sizeof...(Gs)> strided_table_of(
    std::integer_sequence<int, Gs...>) {
  return {strided_row_of<BF16, Gs>(std::make_integer_sequence<int, kMaxPartials>{})...};
}
// Both vector slots of a 1024 x 2 row loaded at once, no occupancy cap (the
// use_both_slots rule); the same thread mapping and arithmetic as the
// geometry's other forms.
template <bool BF16, int G, int NN>
constexpr KernelFn both_slots_fn() {
  if constexpr (fused_geometry(G, NN).block == 1024 && fused_geometry(G, NN).vpt == 2 && NN <= 11)
    return &fused_reduce_rmsnorm_kernel<NN, 1024, 2, BF16, 1, 2, 0, 0>;
  else
    return nullptr;
}
template <bool BF16, int G, int... Ns>
constexpr std::array<KernelFn, sizeof...(Ns)> both_slots_row_of(std::integer_sequence<int, Ns...>) {
  return {both_slots_fn<BF16, G, Ns + 1>()...};
}
template <bool BF16, int... Gs>
constexpr std::array<std::array<KernelFn, kMaxPartials>, sizeof...(Gs)> both_slots_table_of(
    std::integer_sequence<int, Gs...>) {
  return {both_slots_row_of<BF16, Gs>(std::make_integer_sequence<int, kMaxPartials>{})...};
}
// Forms of the consecutive-rows kernel, picked by the launched grid:
//   0  fewer workgroups than CUs: all loads at once, plain non-temporal stores;
//   1  a workgroup on every CU, less than a round: all at once, write-through;
//   2  a round or more: the sequenced order, write-through.
constexpr int kRowsForms = 3;
constexpr int rows_form(int64_t grid, int64_t round, int num_cus) {
  return grid >= round ? 2 : grid >= num_cus ? 1 : 0;
}
template <bool BF16, int FORM, int G, int... Ns>
constexpr std::array<RowsKernelFn, sizeof...(Ns)> rows_row_of(std::integer_sequence<int, Ns...>) {
  return {&fused_reduce_rmsnorm_rows_kernel<Ns + 1, fused_geometry(G, Ns + 1).block,
                                            fused_geometry(G, Ns + 1).vpt, BF16,
                                            fused_geometry(G, Ns + 1).chunk,
                                            load_order(G, Ns + 1, FORM == 2),
                                            load_pace(G, Ns + 1, FORM == 2), FORM != 0>...};
}

template <bool BF16, bool SEQ_ORDER, int... Gs>
constexpr std::array<std::array<KernelFn, kMaxPartials>, sizeof...(Gs)> table_of(
    std::integer_sequence<int, Gs...>) {
  return {row_of<BF16, SEQ_ORDER, Gs>(std::make_integer_sequence<int, kMaxPartials>{})...};
}
template <bool BF16, int FORM, int... Gs>
constexpr std::array<std::array<RowsKernelFn, kMaxPartials>, sizeof...(Gs)> rows_table_of(
    std::integer_sequence<int, Gs...>) {
  return {rows_row_of<BF16, FORM, Gs>(std::make_integer_sequence<int, kMaxPartials>{})...};
}

using Geoms = std::make_integer_sequence<int, kNumGeometries>;
// [bf16][sequenced order]
const std::array<std::array<std::array<std::array<KernelFn, kMaxPartials>, kNumGeometries>, 2>, 2>
    kTable = {{{table_of<false, false>(Geoms{}), table_of<false, true>(Geoms{})},
               {table_of<true, false>(Geoms{}), table_of<true, true>(Geoms{})}}};
// [bf16]
const std::array<std::array<std::array<KernelFn, kMaxPartials>, kNumGeometries>, 2> kStridedTable = {
    {strided_table_of<false>(Geoms{}), strided_table_of<true>(Geoms{})}};
// [bf16]
const std::array<std::array<std::array<KernelFn, kMaxPartials>, kNumGeometries>, 2> kBothSlotsTable = {
    {both_slots_table_of<false>(Geoms{}), both_slots_table_of<true>(Geoms{})}};
// [bf16][rows_form]
const std::array<
    std::array<std::array<std::array<RowsKernelFn, kMaxPartials>, kNumGeometries>, kRowsForms>, 2>
    kRowsTable = {{{rows_table_of<false, 0>(Geoms{}), rows_table_of<false, 1>(Geoms{}),
                    rows_table_of<false, 2>(Geoms{})},
                   {rows_table_of<true, 0>(Geoms{}), rows_table_of<true, 1>(Geoms{}),
                    rows_table_of<true, 2>(Geoms{})}}};

}  // namespace

void kernel_geometry(int64_t hidden, int32_t elem_bytes, int32_t num_partials, int* block,
                     int* vecs_per_thread) {
  const int64_t nvec = hidden * elem_bytes / 16;
  const int g = geometry_index(nvec);
  *block = g < 0 ? 0 : fused_geometry(g, num_partials).block;
  *vecs_per_thread = g < 0 ? 0 : fused_geometry(g, num_partials).vpt;
}

int launch_fused(const FusedLaunch& L, char* err, size_t errlen) {
  const bool bf16 = L.dtype == 1;
  const int elem_bytes = bf16 ? 2 : 4;
  const int64_t nvec = L.hidden * elem_bytes / 16;
  const FusedPlan plan = plan_fused(nvec, L.num_partials, L.num_rows, L.num_cus);
  const int g = plan.geometry;
  if (g < 0 || L.num_partials < 1 || L.num_partials > kMaxPartials || L.num_rows <= 0 ||
      L.num_rows > 0x7FFFFFFF || L.num_cus < 1) {
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

  const int block = plan.geo.block;
  hipError_t e;
  if (L.max_workgroups <= 0 || L.max_workgroups >= L.num_rows) {
    const int64_t round = plan.round;
    // Dispatches over consecutive row ranges of about equal size, each within
    // the byte and work-item limits; the per-row code is the same in each.
    const int64_t chunk = plan.rows_per_dispatch;
    e = hipSuccess;
    for (int64_t r0 = 0; r0 < L.num_rows && e == hipSuccess; r0 += chunk) {
      const int64_t n = L.num_rows - r0 < chunk ? L.num_rows - r0 : chunk;
      k.row_begin = L.row_begin + r0;
      k.row_end = k.row_begin + n;
      // Each dispatch takes its own kernel for its row count (geometry.h).
      const RowKernel rk = fused_row_kernel(g, L.num_partials, n, L.num_cus);
      const KernelFn fn =
          rk == RowKernel::kStrided     ? kStridedTable[bf16][g][L.num_partials - 1]
          : rk == RowKernel::kBothSlots ? kBothSlotsTable[bf16][g][L.num_partials - 1]
                                        : kTable[bf16][rk == RowKernel::kSequenced][g][L.num_partials - 1];
      if (fn == nullptr) {
        std::snprintf(err, errlen, "internal: no kernel of the chosen form for this row class");
        return (int)hipErrorInvalidValue;
      }
      const int64_t grid = rk == RowKernel::kStrided ? round : n;
      const u32x4* first = k.partials[0];
      int64_t row_begin = k.row_begin;
      int32_t nvec32 = k.nvec;
      void* args[] = {&first, &row_begin, &nvec32, &k};
      e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)grid), dim3(block),
                          args, 0, static_cast<hipStream_t>(L.stream));
    }
  } else {
    const int64_t cap = max_rows_per_dispatch(block);
    const int64_t wgs = L.max_workgroups < cap ? L.max_workgroups : cap;
    int64_t rows_per_wg = (L.num_rows + wgs - 1) / wgs;
    int64_t row_end = L.row_begin + L.num_rows;
    const unsigned grid = (unsigned)((L.num_rows + rows_per_wg - 1) / rows_per_wg);
    const int form = rows_form(grid, round_rows(block, L.num_cus), L.num_cus);
    const RowsKernelFn fn = kRowsTable[bf16][form][g][L.num_partials - 1];
    void* args[] = {&k, &rows_per_wg, &row_end};
    e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(block), args, 0,
                        static_cast<hipStream_t>(L.stream));
  }
  if (e != hipSuccess) {
    std::snprintf(err, errlen, "hipLaunchKernel: %s", hipGetErrorString(e));
    return (int)e;
  }
  return 0;
}

}  // namespace tw
