// Tile list of the grouped expert GEMMs: which (expert, M-tile, N-tile, and
// K-range) each schedule entry computes. Plain arithmetic over the expert
// table the plan kernel builds (gemm.hip), usable on the host as well, so
// that the mapping can be checked exhaustively on a CPU.
//
// The list. Experts in id order; inside an expert, groups of up to kGroupM
// M-tiles, and inside a group runs of N-tiles wide enough that one run covers
// about kRunTiles tiles (4 M-tiles x 2 N-tiles, 8 x 1, 1 x 8 ...), N first
// inside a run. Consecutive entries thus share weight tiles and activation
// tiles, and a run never mixes two experts' weights.
//
// Slots. Slot b belongs to XCD b % kXcds (the hardware deals workgroups to
// the XCDs round-robin, and the persistent kernel's workgroup v takes the
// slots v + i * W, W workgroups, a multiple of kXcds) and is that XCD's slot
// j = b / kXcds. XCD x computes the list positions [cut(x), cut(x + 1)) in
// slot order. The cuts split the list into eighths of equal count, or (the
// gate/up GEMM on the 256-row tile) of equal estimated cost: an
// M-tile whose rows fill at most half of it has one wavefront with rows per
// SIMD and costs about 0.78 of a full one (per-tile timestamps of the
// many-expert GEMMs: 0.74-0.80 for up to 128 rows, 1.0 beyond), and inside
// an expert the cost is spread evenly over its positions. On the many-expert
// shape the experts with one short M-tile come last in id order; counted
// equal they filled the last XCD's slice while the first workgroups of every
// other XCD ran one full tile more than the rest. (Counted equal, the tiles
// of the weight-streaming 128-row tile each stream the same weight bytes;
// cost cuts measured no faster on the Mixtral-shaped GEMM, whose short last
// M-tiles interleave with full ones.)
//
// The last round. When K may be split (the down GEMM), T tiles on W
// workgroups make q = T / W full rounds and a last round of r = T % W tiles
// that would leave W - r workgroups idle for a whole tile's time. Those r
// tiles are instead split s = min(cap, W / r) ways along K: the last round
// has r * s entries of 1/s of a tile each (K-range ks of tile u, ordered
// K-range first, so that entries reading the same weight K-range are
// neighbours), their fp32 partial sums are added afterwards, and every other
// tile computes all of K and stores its output directly. Each XCD then takes
// q full rounds' positions [x * q * W/8, (x + 1) * q * W/8) and the
// last-round entries [x * W/8, (x + 1) * W/8).
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
  const int* cfirst;  // estimated cost before expert e (cfirst[E]: all); null: slices of equal count
  int E, bm, n_tiles_n;
  int tiles;  // entries of the list: min(first[E], the host's M-tile bound) * n_tiles_n
};

// Estimated cost of an expert's tiles: kCostFull a tile, kCostShort for
// those of an M-tile at most half full.
constexpr int kCostFull = 100;
constexpr int kCostShort = 78;

MOE_SCHED_FN int expert_cost(int rows, int bm, int n_tiles_n) {
  if (rows <= 0) return 0;
  const int me = (rows + bm - 1) / bm;
  const int last = rows - (me - 1) * bm;
  return n_tiles_n * ((me - 1) * kCostFull + (2 * last <= bm ? kCostShort : kCostFull));
}

// The expert holding list position idx: the last e with
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

// A schedule entry: expert, first row and end row of the expert, N-tile;
// K-range ks of s (s = 1: all of K) and, when split, the tile's index u
// among the last round's tiles.
struct Entry {
  int ex, row0, row_end, n_t, ks, s, u;
};

// Entry of the list at position L (all of K).
MOE_SCHED_FN Entry entry_at(const Table& t, int L) {
  Entry e;
  e.ex = expert_of(t, L);
  const int me = t.first[e.ex + 1] - t.first[e.ex];
  int m, n;
  local_tile(me, t.n_tiles_n, L - t.first[e.ex] * t.n_tiles_n, &m, &n);
  e.row0 = t.lo[e.ex] + m * t.bm;
  e.row_end = t.hi[e.ex];
  e.n_t = n;
  e.ks = 0;
  e.s = 1;
  e.u = 0;
  return e;
}

// First list position of XCD x's slice (x = kXcds: the list's end).
MOE_SCHED_FN int xcd_cut(const Table& t, int x) {
  if (x >= kXcds) return t.tiles;
  if (t.cfirst == nullptr) return imin(x * ((t.tiles + kXcds - 1) / kXcds), t.tiles);
  // the expert holding cost x / kXcds of the total, and the position inside
  // it in proportion
  const int th = (int)(((long long)t.cfirst[t.E] * x + kXcds - 1) / kXcds);
  int lo_e = 0, hi_e = t.E - 1;
  while (lo_e < hi_e) {
    const int mid = (lo_e + hi_e + 1) / 2;
    if (t.cfirst[mid] <= th) lo_e = mid;
    else hi_e = mid - 1;
  }
  const int ce = t.cfirst[lo_e + 1] - t.cfirst[lo_e];
  const int te = (t.first[lo_e + 1] - t.first[lo_e]) * t.n_tiles_n;
  const int in = ce > 0 ? (int)(((long long)(th - t.cfirst[lo_e]) * te + ce - 1) / ce) : 0;
  return imin(t.first[lo_e] * t.n_tiles_n + imin(in, te), t.tiles);
}

// List range [*begin, *end) of XCD x when the last round is not split.
MOE_SCHED_FN void xcd_range(const Table& t, int x, int* begin, int* end) {
  *begin = xcd_cut(t, x);
  *end = xcd_cut(t, x + 1);
}

// Rounds of a schedule on W workgroups: q full rounds, r tiles left, split s
// ways (s = 1: the last round is not split). cap = 1: K is never split.
struct Rounds {
  int W, q, r, s;
};

MOE_SCHED_FN Rounds rounds_of(const Table& t, int W, int cap) {
  Rounds d;
  d.W = W;
  d.q = t.tiles / W;
  d.r = t.tiles - d.q * W;
  d.s = d.r > 0 && cap > 1 ? imax(1, imin(cap, W / d.r)) : 1;
  return d;
}

// Entry of slot b; false if the slot holds none. Each XCD's entries fill a
// prefix of its slots, so a workgroup stops at its first empty slot.
MOE_SCHED_FN bool slot_entry(const Table& t, const Rounds& d, int b, Entry* en) {
  const int x = b % kXcds, j = b / kXcds;
  if (d.s == 1) {
    int begin, end;
    xcd_range(t, x, &begin, &end);
    if (begin + j >= end) return false;
    *en = entry_at(t, begin + j);
    return true;
  }
  const int w8 = d.W / kXcds;
  const int full = d.q * w8;  // full-round slots of each XCD
  if (j < full) {
    *en = entry_at(t, x * full + j);
    return true;
  }
  const int v = x * w8 + (j - full);  // last-round entry
  if (j - full >= w8 || v >= d.r * d.s) return false;
  const int u = v % d.r;
  *en = entry_at(t, d.q * d.W + u);
  en->ks = v / d.r;
  en->s = d.s;
  en->u = u;
  return true;
}

// Slots that can hold an entry for T tiles on W workgroups: a cost slice
// holds at most kCostFull / kCostShort (< 4/3) of an eighth of the tiles and
// one more (or q full rounds and a split last one: at most T + W).
MOE_SCHED_FN int slots_bound(int T, int W) { return ((4 * T + 2) / 3 + 3 * kXcds - 1) / kXcds * kXcds + W; }

// K-range [*k0, *k1) of range ks of s over K elements in steps of bk: whole
// steps, ceil(steps / s) per range.
MOE_SCHED_FN void k_range(int K, int bk, int ks, int s, int* k0, int* k1) {
  const int steps = (K + bk - 1) / bk;
  const int per = (steps + s - 1) / s * bk;
  *k0 = ks * per;
  *k1 = imin(K, *k0 + per);
}

}  // namespace sched
}  // namespace moe
