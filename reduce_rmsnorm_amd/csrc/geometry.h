// Row geometry and launch rules of the row-per-workgroup kernels.
//
// The geometry (threads per workgroup, 16-byte vectors per thread) depends on
// the row width, the element size and the partial count N alone, and every
// kernel that normalizes rows uses it, so the per-row arithmetic and its
// reduction order never depend on the launch.  The launch rules (which load
// order and which kernel a dispatch runs) depend on the row count and on the
// number of CUs the launch may use; they change no result bit.
//
// Every rule below was chosen by measurement on MI355X; the figures are in
// profiles/launch_rules_mi355x.md, under the name of the function or table.
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

// Row classes by 16-byte vectors per row: the first entry whose capacity
// covers the row (profiles: "Row classes").  320, 384 and 640 threads fit the
// widths between the powers of two (h = 2560, 3072, 5120 bf16) so that no
// wave is empty; 512 x 3 covers 1025-1536 vectors.
constexpr Geometry kGeometry[] = {
    {64, 1, 1, 1, 0},  {128, 1, 1, 1, 0}, {256, 1, 1, 1, 0},  {320, 1, 8, 1, 0},
    {384, 1, 8, 1, 0}, {512, 1, 8, 1, 0}, {640, 1, 8, 1, 0},  {512, 2, 6, 2, 0},
    {512, 3, 4, 1, 0}, {512, 4, 4, 2, 0}, {1024, 4, 1, 1, 0}, {1024, 8, 1, 1, 0}};
// Occupancy caps hold up to this many partials; above, they would force spills.
constexpr int kMaxCappedPartials = 8;

// The geometry the fused kernels use for row class g and N partials: where
// enough partials make it pay, the tensors are loaded in summation order with
// one or two in flight per thread, which keeps fewer DRAM regions open across
// the chip (profiles: "Sequenced load order").
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

// Occupancy of the short form (all loads at once, the form of launches too
// small for the sequenced order): the geometry's cap up to kMaxCappedPartials,
// none above, where holding every tensor of a slot at once would spill under
// the cap.  1024 x 2 (two slots' sums beside one slot's nine tensors) already
// needs a few registers more than the cap leaves at kMaxCappedPartials.
constexpr int short_form_waves_per_eu(int g, int n) {
  const Geometry geo = fused_geometry(g, n);
  const bool wide = geo.block == 1024 && geo.vpt == 2;
  return n < kMaxCappedPartials || (n == kMaxCappedPartials && !wide) ? geo.waves_per_eu : 1;
}

// The sequenced geometries run at 8 waves per SIMD, 4 SIMDs per CU.
constexpr int kWavesPerCU = 8 * 4;

// One round: the workgroups of `block` threads resident at once on num_cus CUs.
constexpr int64_t round_rows(int block, int num_cus) {
  return (int64_t)num_cus * (kWavesPerCU * 64 / block);
}

// A sequenced launch of one to four rounds whose last round is at most half
// full runs one round of workgroups, each taking every round-th row: its rows
// past the full rounds then start with the first round (profiles: "Strided
// kernel").  Fuller or longer launches balance better with one row per
// workgroup.
constexpr bool use_strided_grid(int64_t rows, int64_t round) {
  const int64_t tail = rows % round;
  return rows > round && rows < 4 * round && tail > 0 && 2 * tail <= round;
}

// Whether a launch loads in the geometry's sequenced order (each thread then
// waits out ceil((N+1)/seq) latencies in a row).  Below one round it does not:
// too few rows to hide the chain.  Just past one round, with chains of 8 or
// more, the rows beyond the first round run almost alone, and all loads at
// once win until one and a half rounds (profiles: "One round").
constexpr bool use_sequenced_order(int64_t rows, int64_t round, int num_partials, int seq) {
  if (seq <= 0 || rows < round) return false;
  const int chain = (num_partials + 1 + seq - 1) / seq;
  return !(chain >= 8 && rows > round && 2 * rows < 3 * round);
}

// A 1024 x 2 launch that puts one workgroup on nearly every CU (more than
// seven eighths of them, none with two) issues both vector slots' loads at
// once with no occupancy cap, where the short form takes one slot at a time:
// each CU then has one row to stream and nothing to share its registers
// with.  Up to 11 partials; with more, and on fewer or more rows, it was
// slower (profiles: "Both slots at once").
constexpr bool use_both_slots(const Geometry& geo, int n, int64_t rows, int num_cus) {
  return geo.block == 1024 && geo.vpt == 2 && n <= 11 && 8 * rows > 7 * (int64_t)num_cus &&
         rows <= num_cus;
}

// The kernel one dispatch of `rows` rows of row class g with n partials runs
// on num_cus CUs: one workgroup per row with all loads at once (of one chunk
// of vector slots at a time, or of both slots of 1024 x 2), one workgroup per
// row in the sequenced order, or the strided kernel (which exists for the
// sequenced geometries that load all vector slots in one sequence).
enum class RowKernel { kAllAtOnce, kSequenced, kStrided, kBothSlots };
constexpr RowKernel fused_row_kernel(int g, int n, int64_t rows, int num_cus) {
  const Geometry geo = fused_geometry(g, n);
  const int64_t round = round_rows(geo.block, num_cus);
  if (!use_sequenced_order(rows, round, n, geo.seq))
    return use_both_slots(geo, n, rows, num_cus) ? RowKernel::kBothSlots : RowKernel::kAllAtOnce;
  if (geo.chunk == geo.vpt && use_strided_grid(rows, round)) return RowKernel::kStrided;
  return RowKernel::kSequenced;
}

// Depth of the short form of a geometry's load order: 0 issues all N+1 loads
// of a chunk at once.  512 x 3 keeps three tensors in flight per slot, since
// all of them would spill beside the three slots' sums (profiles: "Short form
// of 512 x 3").
constexpr int short_form_depth(const Geometry& geo) {
  return geo.block == 512 && geo.vpt == 3 ? 3 : 0;
}

// Pacing of the sequenced order: after adding a tensor a wave pauses for
// PACE * 64 clocks (s_sleep) before it requests the next; with many tensors
// per row, fewer requests in flight stream faster (profiles: "Pacing").  The
// fitted classes hold more workgroups per CU and run unpaced (320, 640) or at
// half the pause of their power-of-two neighbour (384); 512 x 3 borrows
// 1024 x 2's.  Counts between the measured ones take the nearer pace.
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

constexpr int geometry_index(int64_t nvec) {
  for (int g = 0; g < kNumGeometries; ++g)
    if (nvec <= (int64_t)kGeometry[g].block * kGeometry[g].vpt) return g;
  return -1;
}

}  // namespace tw
