// Row geometry of the row-per-workgroup kernels: threads per workgroup and
// 16-byte vectors per thread, chosen from the row width (and, through
// fused_geometry, the partial count) alone.  Every kernel
// that normalizes rows uses this table, so the per-row arithmetic (and its
// reduction order) never depends on the launch.
#pragma once

#include <cstdint>

namespace tw {

struct Geometry {
  int block;          // threads per workgroup
  int vpt;            // 16-byte vectors per thread
  int waves_per_eu;   // occupancy the compiler must allow (1: no constraint)
  int chunk;          // vector slots whose loads are issued together (divides vpt)
  int seq;            // 0: all N+1 tensors of a chunk loaded at once; D > 0: the
                      // tensors are loaded in summation order, D in flight
};

// (threads per workgroup, vectors per thread) by 16-byte vectors per row: the
// first entry whose capacity covers the row.  Measured on MI355X at 184-738 MB
// per launch, N = 8 bf16, all loads of a row issued at once:
//  * h = 8192 (1024 vectors): 512 x 2 at 6 waves per SIMD (at most 80 VGPRs,
//    three workgroups per CU) 31.5 us; uncapped 32.7 us; 1024 x 1 33.4 us;
//    256 x 4 36.0-36.5 us.  (With five or more partials fused_geometry below
//    replaces this entry.)
//  * h = 4096 (512 vectors): 512 x 1 at 8 waves per SIMD 122.9-123.2 us
//    (T = 8192); 256 x 2 128.9 us.
//  * h = 16384 (2048 vectors): 512 x 4 at 4 waves per SIMD, loads two slots
//    at a time, 123.9 us (T = 2048); 1024 x 2 133.4 us; 256 x 8 132.1 us.
// The occupancy cap applies up to N = 8 partials, where it costs no scratch;
// with more partials the compiler's own allocation is kept.
// Row widths between the powers of two get workgroups that fit them, one
// vector per thread, so that no wave of a workgroup is empty and more of the
// waves a CU holds carry data: 320 threads for up to 320 vectors (h = 2560
// bf16; six workgroups per CU), 384 for up to 384 (h = 3072; five), 640 for up
// to 640 (h = 5120; three, where two 1024-thread workgroups held six empty
// waves each).  Measured at T = 1024, N = 8, us, the next larger class's
// workgroup / the fitted one: h = 2560 12.97 / 11.24 (N = 2: 6.87 / 6.28,
// N = 16: 22.03 / 17.58), h = 3072 14.22 / 13.04, h = 5120 23.32 / 20.75
// (N = 16: 41.03 / 34.41; T = 4096, with the 1024 x 1 pause, 86.64 / 83.48;
// unpaced, as fused_pace now has it, 80.16).  Below 7 partials the
// 640-thread form is slower (h = 5120, N = 2: 11.60 / 12.31, N = 4: 15.55 /
// 15.87, N = 5: 16.23 / 16.88), so those take the 512 x 2 class's geometry.
// Likewise 1025-1536 vectors (h = 9216-12288 bf16) run 512 x 3 from N = 6 on,
// one vector slot at a time in sequence, four workgroups per CU, where 1024 x
// 2 left half its threads without a second vector: N = 8, T = 1024, us, 1024
// x 2 / 512 x 3: h = 12288 51.26 / 47.58 (N = 16: 87.18 / 76.29; T = 4096:
// 200.06 / 190.11), h = 10240 47.94 / 41.74, h = 9216 46.87 / 39.92; N = 6
// 41.12 / 41.02; below N = 6 it was slower (N = 2: 23.71 / 24.08, N = 4: 32.14
// / 33.00) and 1024 x 2 is kept.
constexpr Geometry kGeometry[] = {
    {64, 1, 1, 1, 0},  {128, 1, 1, 1, 0}, {256, 1, 1, 1, 0},  {320, 1, 8, 1, 0},
    {384, 1, 8, 1, 0}, {512, 1, 8, 1, 0}, {640, 1, 8, 1, 0},  {512, 2, 6, 2, 0},
    {512, 3, 4, 1, 0}, {512, 4, 4, 2, 0}, {1024, 4, 1, 1, 0}, {1024, 8, 1, 1, 0}};
constexpr int kMaxCappedPartials = 8;

// The geometry the fused kernels use for row class g and N partials.
//
// Loading the tensors in summation order, with only D of them in flight per
// thread (over CHUNK vector slots at a time), keeps fewer DRAM regions open
// at once than issuing all N+1 loads together, and beats it once there are
// enough partials.  Measured on MI355X
// (bf16, inputs and outputs rotated past the MALL):
//  * 512 x 2 class (h = 8192): 1024 x 1 with D = 1, T = 1024: N = 7 28.3 us
//    against 29.2; N = 8 30.8 against 31.7; N = 12 40.5 against 44.0; N = 16
//    50.3 against 55.3 (T = 4096, N = 8: 117.5 against 123.2).  N = 5, 6 do
//    best with D = 2 (23.2 against 23.9 us, 25.9 against 26.9); for N <= 4
//    loading everything at once stays best (N = 2: 16.0 against 16.6 us).
//    Re-measured with the preloaded kernel arguments, D = 1 still wins from
//    N = 7 on: N = 8 30.72 against 31.27 us (T = 4096: 117.8 against 124.8),
//    N = 16 50.5 against 52.9.
//  * 512 x 1 class (h = 4096, T = 8192): D = 1, N = 8 120.2 against 124.5 us;
//    N = 2 53.3 against 54.0.  Two in flight is slower at every N tried (N = 8:
//    124.2 against 118.6 us; N = 16 at T = 4096: 111.0 against 104.1).
//  * 512 x 4 class (h = 16384, T = 2048): 1024 x 2 loading one vector slot
//    at a time, each in sequence with one tensor in flight (46 VGPRs, 8 waves
//    per SIMD): N = 2 56.8 against 59.5 us, N = 4 77.8 against 79.7, N = 8
//    120.7 against 124.6.  Sequencing all four slots of 512 x 4 at once
//    spills or loses occupancy instead.
// Otherwise, up to kMaxCappedPartials the table entry applies with its
// occupancy cap; above it the cap is dropped (it would force spills).
constexpr Geometry fused_geometry(int g, int n) {
  const Geometry k = kGeometry[g];
  if (k.block == 640 && k.vpt == 1)                     // below N = 7: the 512 x 2 class's choice
    return n >= 7 ? Geometry{640, 1, 8, 1, 1} : n >= 5 ? Geometry{1024, 1, 8, 1, 2}
                                                       : Geometry{512, 2, 6, 2, 0};
  if ((k.block == 320 || k.block == 384) && k.vpt == 1 && n >= 2)
    return Geometry{k.block, 1, 8, 1, 1};
  if (k.block == 512 && k.vpt == 3)                     // below N = 6: the 512 x 4 class's choice
    return n >= 6 ? Geometry{512, 3, 8, 1, 1} : n >= 2 ? Geometry{1024, 2, 8, 1, 1}
                                                       : Geometry{512, 4, 4, 2, 0};
  if (k.block == 512 && k.vpt == 2 && n >= 5) return Geometry{1024, 1, 8, 1, n >= 7 ? 1 : 2};
  if (k.block == 512 && k.vpt == 1 && n >= 2) return Geometry{512, 1, 8, 1, 1};
  if (k.block == 512 && k.vpt == 4 && n >= 2) return Geometry{1024, 2, 8, 1, 1};
  if (n <= kMaxCappedPartials) return k;
  return Geometry{k.block, k.vpt, 1, k.chunk, k.seq};
}
// The sequenced load order wins only once a launch fills every CU with
// resident workgroups: with fewer rows each workgroup waits out its tensors
// one latency at a time, and issuing all loads at once is faster (T = 128,
// N = 8, h = 8192: 7.05 us against 9.34; h = 4096 at T = 512: 9.99 against
// 11.05).  The crossover is one full round of workgroups: 256 CUs times the
// workgroups that fit on a CU at 8 waves per SIMD (512 rows for 1024 x 1,
// 1024 for 512 x 1); just past it, long chains of tensors still issue all
// loads at once (use_sequenced_order below).  Both orders do the same
// arithmetic, so the choice never changes a bit of the result.
constexpr int kNumCUs = 256;
constexpr int64_t seq_min_workgroups(int block) { return (int64_t)kNumCUs * (8 * 4 * 64 / block); }

// A sequenced launch whose rows are not a whole number of rounds leaves its
// last round partly empty.  With one workgroup per row those last rows land
// on whichever CUs free up first; launching one round of workgroups that each
// take every round-th row (the strided kernel) places the workgroups that
// carry them with the first round instead, and overlaps each workgroup's row
// boundary with its next row's first loads.  It wins while the last round is at most half full and
// the launch is under four rounds; with fuller last rounds, and on whole or
// longer launches, the hardware's own dispatch of one-row workgroups
// balances better.  Measured on MI355X (N = 8 bf16, rotated past the MALL,
// one-row kernel against strided, us per launch; at N = 8, launches below one
// and a half rounds issue all loads at once instead, see use_sequenced_order):
//  * h = 8192, round 512: T = 520 22.47 / 22.10, 576 22.87 / 22.40, 640
//    22.87 / 22.26, 768 25.29 / 24.41 (N = 16: 43.18 / 41.78), 1152
//    36.91 / 36.16, 1280 38.96 / 38.06, 1792 52.77 / 52.02; not taken:
//    896 28.09 / 28.25, 960 29.33 / 29.46, 1024 30.65 / 30.63, 1536
//    44.91 / 45.36, 2048 59.04 / 59.55, 4096 117.1 / 120.6.
//  * h = 4096, round 1024: T = 1280 23.31 / 22.71, 1536 25.28 / 24.99, 2560
//    39.01 / 38.87; not taken: 1792 27.98 / 28.07, 3072 44.85 / 45.29, 4096
//    59.32 / 60.09, 8192 116.6 / 121.6.
// Both kernels do the same per-row arithmetic: the choice never changes a bit.
constexpr bool use_strided_grid(int64_t rows, int64_t round) {
  const int64_t tail = rows % round;
  return rows > round && rows < 4 * round && tail > 0 && 2 * tail <= round;
}

// Whether a launch of `rows` rows loads in the geometry's sequenced order
// (which loads the N+1 tensors `seq` at a time, so a thread waits out
// ceil((N+1)/seq) latencies in a row).  Below one round it does not (above).
// Just past one round the rows beyond it run almost alone, each waiting out
// its whole chain of latencies: with a chain of 8 or more, issuing all loads
// at once is faster until the launch reaches one and a half rounds, from
// where the sequenced order (one-row or strided kernel) catches up.  At
// exactly one round the sequenced order still wins.  Measured on MI355X
// (bf16, rotated past the MALL, us per launch, sequenced / all at once):
//  * h = 8192, round 512, N = 8: T = 512 16.43 / 17.17; 520 22.06 / 19.92,
//    544 22.28 / 20.27, 576 22.39 / 20.42, 600 22.16 / 20.47, 640 22.28 /
//    20.61, 700 23.14 / 22.08, 736 23.91 / 23.52; 768 24.37 / 24.37, 800
//    26.42 / 26.39.  N = 12, T = 600: 30.83 / 27.04; N = 16, T = 544: 39.47 /
//    33.14, 700 40.38 / 37.63.  Chains of 3-3.5: N = 5, T = 544 15.29 /
//    15.51; N = 6, T = 600 16.81 / 17.11.
//  * h = 4096, round 1024, N = 8: T = 1024 16.12 / 17.21; 1040 22.17 /
//    18.74, 1088 22.29 / 18.50, 1280 22.73 / 20.29, 1400 23.97 / 22.25; 1536
//    25.05 / 25.04.  N = 2, T = 1300: 11.36 / 11.60.
//  * h = 16384, round 512, N = 8: T = 512 31.08 / 33.88; 576 45.87 / 40.30,
//    640 46.37 / 41.77; 768 50.73 / 50.71.
// Between two and four rounds the two orders stay within 2% of each other
// either way (the strided kernel runs there), so the sequenced one is kept.
// Those are launches alone, back to back.  With a GEMM writing one partial
// before each fused launch, as in a layer, all at once saves 1.1-2.0 us at
// 576-704 x 8192, 4.1 at 1100 x 4096 and 5.9 at 576 x 16384 (N = 8); right
// after another fused launch the 640- and 704-row launches lose about 1.3 us
// instead.  The rule follows the layer's case.
constexpr bool use_sequenced_order(int64_t rows, int64_t round, int num_partials, int seq) {
  if (seq <= 0 || rows < round) return false;
  const int chain = (num_partials + 1 + seq - 1) / seq;
  return !(chain >= 8 && rows > round && 2 * rows < 3 * round);
}

// The kernel one dispatch of `rows` rows of row class g with n partials
// runs: one workgroup per row with all loads at once, one workgroup per row
// in the sequenced order, or the strided kernel (which exists for the
// sequenced geometries that load all vector slots in one sequence).
enum class RowKernel { kAllAtOnce, kSequenced, kStrided };
constexpr RowKernel fused_row_kernel(int g, int n, int64_t rows) {
  const Geometry geo = fused_geometry(g, n);
  const int64_t round = seq_min_workgroups(geo.block);
  if (!use_sequenced_order(rows, round, n, geo.seq)) return RowKernel::kAllAtOnce;
  if (geo.chunk == geo.vpt && use_strided_grid(rows, round)) return RowKernel::kStrided;
  return RowKernel::kSequenced;
}

// The depth of the short form of a geometry's load order, the one launches
// too small for the sequenced order take: 0 issues all N+1 loads of a chunk at
// once.  512 x 3 keeps three tensors in flight per vector slot instead, since
// all of them would not fit in registers beside the three slots' sums (that
// form spilled and took 11.72 against 10.45 us at 128 rows x 12288, N = 8;
// three in flight took 10.73, and 13.99 against 14.47 at 256 rows).
constexpr int short_form_depth(const Geometry& geo) {
  return geo.block == 512 && geo.vpt == 3 ? 3 : 0;
}

// Pacing of the sequenced load order: after adding a tensor, a wave pauses
// for PACE * 64 clocks (s_sleep) before it requests the next one.  Fewer
// requests in flight across the chip let HBM work more efficiently, and the
// more tensors a row has, the more that pays.  Measured on MI355X (bf16,
// rotated past the MALL, times per launch; PACE 0 / best):
//  * 1024 x 1 class (h = 8192, T = 1024): N = 5, 6 best unpaced; N = 8 30.83
//    against 30.73 us (PACE 4), N = 12 40.60 against 40.18 (8), N = 16 50.81
//    against 49.56 (10).
//  * 512 x 1 class (h = 4096, T = 4096): N <= 6 best unpaced (N = 2: 28.27
//    against 28.35 at PACE 2); N = 8 60.26 against 59.56 (8), N = 12 82.93
//    against 78.42 (10), N = 16 106.10 against 96.67 (12).
//  * 1024 x 2 class (h = 16384, T = 1024): N <= 4 best unpaced; N = 8 61.23
//    against 60.04 (10), N = 16 103.48 against 97.44 (12).
// Partial counts between the measured ones take the nearer measured pace.
// The fitted classes hold more workgroups per CU, and the pause that suits
// the power-of-two classes slows them (T = 4096, us, unpaced / half the
// 512 x 1 or 1024 x 1 pause / the full one): 640 threads (h = 5120), N = 7
// 72.99 / 74.26 / 75.96, N = 12 108.13 / 112.30 / 118.50, N = 16 135.13 /
// 144.02 / 156.58; 320 threads (h = 2560), N = 8 39.71 / 40.91 / 42.91, N = 16
// 65.57 / 69.64 / 77.10; 384 threads (h = 3072), N = 8 46.69 / 46.93 / 47.38,
// N = 12 63.29 / 62.98 / 63.95, N = 16 79.79 / 78.54 / 81.64.  So 320 and 640
// run unpaced and 384 takes half of 512 x 1's pause.  512 x 3 keeps 1024 x 2's
// (h = 12288, N = 8, T = 1024: 49.58 / 48.89 / 47.54; N = 16 82.10 / 79.67 /
// 76.14).
constexpr int fused_pace(int g, int n) {
  const Geometry k = kGeometry[g];
  if (k.block == 512 && k.vpt == 2 && n >= 7)           // 1024 x 1, sequenced
    return n <= 8 ? 4 : n <= 10 ? 5 : n <= 12 ? 8 : 10;
  if (k.block == 512 && k.vpt == 1 && n >= 8)           // 512 x 1, sequenced
    return n <= 8 ? 8 : n <= 12 ? 10 : 12;
  if (k.block == 384 && k.vpt == 1 && n >= 8)           // half of 512 x 1's
    return n <= 8 ? 4 : n <= 12 ? 5 : 6;
  if (k.block == 512 && k.vpt == 3 && n >= 6)           // as 1024 x 2
    return n <= 6 ? 4 : n <= 12 ? 10 : 12;
  if (k.block == 512 && k.vpt == 4 && n >= 6)           // 1024 x 2, sequenced
    return n <= 6 ? 4 : n <= 12 ? 10 : 12;
  return 0;
}

constexpr int kNumGeometries = sizeof(kGeometry) / sizeof(kGeometry[0]);
constexpr int kMaxVectors = 8192;

inline int geometry_index(int64_t nvec) {
  for (int g = 0; g < kNumGeometries; ++g)
    if (nvec <= (int64_t)kGeometry[g].block * kGeometry[g].vpt) return g;
  return -1;
}

}  // namespace tw
