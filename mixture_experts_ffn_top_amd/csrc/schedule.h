// Tile list of the grouped expert GEMMs: which (K-split, expert, M-tile,
// N-tile) each schedule entry computes. Plain arithmetic over the expert table
// the plan kernel builds (gemm.hip), usable on the host as well, so that the
// mapping can be checked exhaustively on a CPU.
//
// The list. Per K-split, experts in id order; inside an expert, groups of up
// to kGroupM M-tiles, and inside a group runs of N-tiles wide enough that one
// run covers about kRunTiles tiles (4 M-tiles x 2 N-tiles, 8 x 1, 1 x 8 ...),
// N first inside a run. Consecutive entries thus share weight tiles and
// activation tiles, and a run never mixes two experts' weights.
//
// Slices. Entry b belongs to XCD b % kXcds (the hardware deals workgroups to
// the XCDs round-robin, and the persistent kernel's workgroup b only takes
// entries b + i * grid, with grid a multiple of kXcds), slot b / kXcds, and
// XCD x computes the list positions [x * chunk, (x + 1) * chunk) in slot
// order, chunk = ceil(entries / kXcds). (Cutting the slices at equal
// estimated cost instead, with an expert's short last M-tile counted cheaper,
// measured no faster on the Mixtral-shaped GEMM and slower where the weight
// stream sets the time: there every tile streams the same weight bytes.)
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define MOE_SCHED_FN __host__ __device__ __forceinline__
#else
#define MOE_SCHED_FN inline
#endif

namespace moe {
namespace sched {

constexpr int kXcds = 8;
constexpr int kRunTiles = 8;  // tiles per run of the list order
constexpr int kGroupM = 8;    // M-tiles per group of the list order

MOE_SCHED_FN int imin(int a, int b) { return a < b ? a : b; }
MOE_SCHED_FN int imax(int a, int b) { return a > b ? a : b; }

// The expert table: first[e] = M-tiles before expert e (first[E] = all of
// them), rows lo[e] .. hi[e] - 1.
struct Table {
  const int* first;
  const int* lo;
  const int* hi;
  int E, bm, n_tiles_n, k_splits;
  int per_split;  // entries of one K-split's list
  int n_real;     // per_split * k_splits
};

// The expert holding split-local entry idx: the last e with
// first[e] * n_tiles_n <= idx.
MOE_SCHED_FN int expert_of(const Table& t, int idx) {
  int lo_e = 0, hi_e = t.E - 1;
  while (lo_e < hi_e) {
    const int mid = (lo_e + hi_e + 1) / 2;
    if (t.first[mid] * t.n_tiles_n <= idx) lo_e = mid;
    else hi_e = mid - 1;
  }
  return lo_e;
}

// M-tile and N-tile of entry j of an expert with me M-tiles.
MOE_SCHED_FN void local_tile(int me, int n_tiles_n, int j, int* m, int* n) {
  const int mg = imin(me, kGroupM);
  const int ng = imax(1, kRunTiles / mg);
  const int mgi = j / (mg * n_tiles_n);
  const int mgw = imin(mg, me - mgi * mg);
  const int jj = j - mgi * mg * n_tiles_n;
  const int ngi = jj / (mgw * ng);
  const int w = imin(ng, n_tiles_n - ngi * ng);
  const int r = jj - ngi * mgw * ng;
  *m = mgi * mg + r / w;
  *n = ngi * ng + r % w;
}

// Entry of the list at position L: expert, K-split, first row and N-tile.
struct Entry {
  int ex, ks, row0, row_end, n_t;
};

MOE_SCHED_FN Entry entry_at(const Table& t, int L) {
  Entry e;
  e.ks = L / t.per_split;
  const int idx = L - e.ks * t.per_split;
  e.ex = expert_of(t, idx);
  const int me = t.first[e.ex + 1] - t.first[e.ex];
  int m, n;
  local_tile(me, t.n_tiles_n, idx - t.first[e.ex] * t.n_tiles_n, &m, &n);
  e.row0 = t.lo[e.ex] + m * t.bm;
  e.row_end = t.hi[e.ex];
  e.n_t = n;
  return e;
}

// List range [*begin, *end) of XCD x.
MOE_SCHED_FN void xcd_range(const Table& t, int x, int* begin, int* end) {
  const int chunk = (t.n_real + kXcds - 1) / kXcds;
  *begin = imin(x * chunk, t.n_real);
  *end = imin((x + 1) * chunk, t.n_real);
}

}  // namespace sched
}  // namespace moe
