// Exhaustive check of the grouped-GEMM schedule (schedule.h) on the host:
// for many seeded expert-size patterns, workgroup counts and K-split caps,
// the slots 0 .. grid-1 that the plan kernel fills must hold every (expert,
// M-tile, N-tile) exactly once, or, for a tile of a split last round, each of
// its K-ranges exactly once; each XCD's entries must be a prefix of its slots
// (the persistent workgroups stop at the first empty one); the XCD slices,
// of equal count or of equal estimated cost, must tile the list in order;
// the split round must fit on the workgroups, and the K-ranges must
// partition K. Prints "ok <cases> <split cases> <cost-sliced cases>" or the
// first failure.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <map>
#include <random>
#include <tuple>
#include <vector>

#include "schedule.h"

using namespace moe::sched;

static int fail(const char* what, int c) {
  std::printf("FAIL case %d: %s\n", c, what);
  return 1;
}

int main() {
  std::mt19937_64 rng(20251202);
  int cases = 0, split_cases = 0, cost_cases = 0;
  // K-ranges: whole 64-element steps, ceil(steps / s) a range, covering [0, K)
  for (int K = 1; K <= 4096; K += 37)
    for (int sp = 1; sp <= 8; ++sp) {
      int at = 0;
      for (int ks = 0; ks < sp; ++ks) {
        int k0, k1;
        k_range(K, 64, ks, sp, &k0, &k1);
        if (k0 % 64) return fail("K-range not on a step", K);
        if (k0 < K && k0 != at) return fail("K-ranges not contiguous", K);
        if (k0 < K) at = k1;
      }
      if (at != K) return fail("K-ranges do not cover K", K);
    }
  for (int c = 0; c < 600; ++c) {
    const int bm_choices[3] = {256, 128, 64};
    const int bm = bm_choices[rng() % 3];
    const int E = 1 + (int)(rng() % (c % 10 == 0 ? 1024 : 64));
    const int n_tiles_n = 1 + (int)(rng() % 120);
    const int cap_choices[4] = {1, 2, 3, 8};
    const int cap = cap_choices[rng() % 4];
    // expert sizes: uniform around a mean, Zipf-like, one hot expert, mostly empty, or near multiples of bm
    std::vector<int> cnt(E, 0);
    const int mode = (int)(rng() % 5);
    for (int e = 0; e < E; ++e) {
      switch (mode) {
        case 0: cnt[e] = (int)(rng() % (3 * bm)); break;
        case 1: cnt[e] = (int)(4000.0 / (e + 1)) + (int)(rng() % 3); break;
        case 2: cnt[e] = e == 0 ? (int)(rng() % 20000) : (int)(rng() % 3); break;
        case 3: cnt[e] = rng() % 4 == 0 ? (int)(rng() % 700) : 0; break;
        default: cnt[e] = 4 * bm + (int)(rng() % 64) - 32; break;
      }
    }
    std::vector<int> offsets(E + 1, 0);
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + cnt[e];
    const int rows = offsets[E];
    const int max_tiles = (rows + bm - 1) / bm + std::min(E, rows);
    const int64_t tiles64 = ((int64_t)max_tiles * n_tiles_n + kXcds - 1) / kXcds * kXcds;
    if (tiles64 > 400000 || tiles64 == 0) continue;  // no rows: the GEMM is not launched
    // workgroups as the host picks them: up to 256 (a multiple of 8), fewer
    // when the schedule has fewer entries
    const int64_t want = cap > 1 ? tiles64 * cap : tiles64;
    const int W = (int)std::min<int64_t>(want, 8 * (1 + (int)(rng() % 32)));
    const bool costed = rng() % 3 != 0;  // slices of equal estimated cost (without a split)
    const int grid = slots_bound((int)tiles64, W);
    // the expert table, as the plan kernel builds it
    std::vector<int> first(E + 1, 0), cfirst(E + 1, 0), lo(E), hi(E);
    for (int e = 0; e < E; ++e) {
      lo[e] = offsets[e];
      hi[e] = offsets[e + 1];
      first[e + 1] = first[e] + (hi[e] > lo[e] ? (hi[e] - lo[e] + bm - 1) / bm : 0);
      cfirst[e + 1] = cfirst[e] + expert_cost(hi[e] - lo[e], bm, n_tiles_n);
    }
    Table t;
    t.first = first.data();
    t.lo = lo.data();
    t.hi = hi.data();
    t.cfirst = nullptr;
    t.E = E;
    t.bm = bm;
    t.n_tiles_n = n_tiles_n;
    t.tiles = std::min(first[E], max_tiles) * n_tiles_n;
    if (first[E] > max_tiles) return fail("M-tile bound", c);
    const Rounds d = rounds_of(t, W, cap);
    if (costed && d.s == 1) t.cfirst = cfirst.data();
    if (d.s < 1 || d.s > cap) return fail("split count out of range", c);
    if (d.s > 1 && (d.r * d.s > W || d.r == 0)) return fail("split round does not fit the workgroups", c);
    for (int b = grid; b < grid + W; ++b) {  // nothing past the grid
      Entry en;
      if (slot_entry(t, d, b, &en)) return fail("entry past the grid", c);
    }
    if (d.s == 1) {  // the slices tile the list in order
      int covered = 0;
      for (int x = 0; x < kXcds; ++x) {
        int begin, end;
        xcd_range(t, x, &begin, &end);
        if (begin != covered || end < begin) return fail("slices not contiguous", c);
        covered = end;
      }
      if (covered != t.tiles) return fail("slices do not cover the list", c);
    }
    // every slot, as the plan kernel fills them
    std::map<std::tuple<int, int, int>, std::vector<int>> seen;  // tile -> K-ranges seen
    std::map<std::tuple<int, int, int>, int> split_u;
    std::vector<int> used(kXcds, 0), last_valid(kXcds, -1);
    for (int b = 0; b < grid; ++b) {
      Entry en;
      const int x = b % kXcds, j = b / kXcds;
      if (!slot_entry(t, d, b, &en)) continue;
      if (j != last_valid[x] + 1) return fail("entries not a prefix of the XCD's slots", c);
      last_valid[x] = j;
      if (en.ex < 0 || en.ex >= E) return fail("entry out of range", c);
      if (en.row0 < lo[en.ex] || en.row0 >= hi[en.ex] || (en.row0 - lo[en.ex]) % bm) return fail("bad row", c);
      if (en.row_end != hi[en.ex]) return fail("bad end row", c);
      if (en.n_t < 0 || en.n_t >= n_tiles_n) return fail("bad N-tile", c);
      if (en.s != 1 && en.s != d.s) return fail("bad split count", c);
      if (en.ks < 0 || en.ks >= en.s) return fail("bad K-range", c);
      const auto key = std::make_tuple(en.ex, en.row0, en.n_t);
      auto& ks = seen[key];
      if (!ks.empty() && ((int)ks.size() >= en.s || std::count(ks.begin(), ks.end(), en.ks)))
        return fail("tile or K-range scheduled twice", c);
      if (!ks.empty() && en.s == 1) return fail("tile both whole and split", c);
      ks.push_back(en.ks);
      if (en.s > 1) {
        if (en.u < 0 || en.u >= d.r) return fail("bad split index", c);
        auto it = split_u.find(key);
        if (it == split_u.end()) split_u[key] = en.u;
        else if (it->second != en.u) return fail("split index differs between K-ranges", c);
        const Entry ref = entry_at(t, d.q * d.W + en.u);
        if (ref.ex != en.ex || ref.row0 != en.row0 || ref.n_t != en.n_t) return fail("split table mismatch", c);
      }
    }
    int64_t expect = 0;
    for (int e = 0; e < E; ++e) expect += (int64_t)(first[e + 1] - first[e]) * n_tiles_n;
    if ((int64_t)seen.size() != expect) return fail("tile missing", c);
    int n_split = 0;
    for (const auto& kv : seen) {
      const int want_s = split_u.count(kv.first) ? d.s : 1;
      if ((int)kv.second.size() != want_s) return fail("K-ranges missing", c);
      n_split += want_s > 1;
    }
    if (d.s > 1 && n_split != d.r) return fail("split tile count", c);
    std::vector<int> us;
    for (const auto& kv : split_u) us.push_back(kv.second);
    std::sort(us.begin(), us.end());
    if (std::unique(us.begin(), us.end()) != us.end()) return fail("split index shared", c);
    // the last round adds at most one short round: workgroup v's slots are
    // v + i W; count whole tiles and split entries
    int worst_whole = 0, worst_split = 0;
    for (int v = 0; v < W; ++v) {
      int whole = 0, split = 0;
      for (int b = v; b < grid; b += W) {
        Entry en;
        if (!slot_entry(t, d, b, &en)) break;
        (en.s > 1 ? split : whole)++;
      }
      worst_whole = std::max(worst_whole, whole);
      worst_split = std::max(worst_split, split);
    }
    if (d.s > 1 && (worst_whole > d.q || worst_split > 1)) return fail("split round not balanced", c);
    split_cases += d.s > 1;
    cost_cases += t.cfirst != nullptr;
    ++cases;
  }
  if (split_cases < 50) return fail("too few split cases", split_cases);
  if (cost_cases < 50) return fail("too few cost-sliced cases", cost_cases);
  std::printf("ok %d %d %d\n", cases, split_cases, cost_cases);
  return 0;
}
