// Exhaustive check of the grouped-GEMM tile list (schedule.h) on the host:
// for many seeded expert-size patterns, the entries 0 .. grid-1 that the plan
// kernel fills must hold every (K-split, expert, M-tile, N-tile) exactly once,
// and each XCD's entries must be a prefix of its slots (the persistent
// workgroups stop at the first empty entry). Prints "ok <cases>" or the first
// failure.
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
  int cases = 0;
  for (int c = 0; c < 500; ++c) {
    const int bm_choices[3] = {256, 128, 64};
    const int bm = bm_choices[rng() % 3];
    const int E = 1 + (int)(rng() % (c % 10 == 0 ? 1024 : 64));
    const int n_tiles_n = 1 + (int)(rng() % 120);
    const int splits_choices[4] = {1, 2, 3, 8};
    const int k_splits = splits_choices[rng() % 4];
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
    const int64_t grid64 = ((int64_t)max_tiles * n_tiles_n * k_splits + kXcds - 1) / kXcds * kXcds;
    if (grid64 > 400000) continue;
    const int grid = (int)grid64;
    // the expert table, as the plan kernel builds it
    std::vector<int> first(E + 1, 0), lo(E), hi(E);
    for (int e = 0; e < E; ++e) {
      lo[e] = offsets[e];
      hi[e] = offsets[e + 1];
      first[e + 1] = first[e] + (hi[e] > lo[e] ? (hi[e] - lo[e] + bm - 1) / bm : 0);
    }
    Table t;
    t.first = first.data();
    t.lo = lo.data();
    t.hi = hi.data();
    t.E = E;
    t.bm = bm;
    t.n_tiles_n = n_tiles_n;
    t.k_splits = k_splits;
    t.per_split = std::min(first[E], max_tiles) * n_tiles_n;
    t.n_real = t.per_split * k_splits;
    if (first[E] > max_tiles) return fail("M-tile bound", c);
    // every entry of the grid, as the plan kernel fills them
    std::map<std::tuple<int, int, int, int>, int> seen;
    const int slots = grid / kXcds;
    for (int b = 0; b < grid; ++b) {
      int begin, end;
      xcd_range(t, b % kXcds, &begin, &end);
      const int L = begin + b / kXcds;
      if (L >= end) continue;
      const Entry en = entry_at(t, L);
      if (en.ex < 0 || en.ex >= E || en.ks < 0 || en.ks >= k_splits) return fail("entry out of range", c);
      if (en.row0 < lo[en.ex] || en.row0 >= hi[en.ex] || (en.row0 - lo[en.ex]) % bm) return fail("bad row", c);
      if (en.n_t < 0 || en.n_t >= n_tiles_n) return fail("bad N-tile", c);
      if (++seen[std::make_tuple(en.ks, en.ex, en.row0, en.n_t)] > 1) return fail("tile scheduled twice", c);
    }
    int64_t expect = 0;
    for (int e = 0; e < E; ++e) expect += (int64_t)(first[e + 1] - first[e]) * n_tiles_n * k_splits;
    if ((int64_t)seen.size() != expect) return fail("tile missing", c);
    // each XCD's tiles are a prefix of its slots, and the slices tile the list
    int covered = 0;
    for (int x = 0; x < kXcds; ++x) {
      int begin, end;
      xcd_range(t, x, &begin, &end);
      if (end - begin > slots) return fail("slice exceeds the XCD's slots", c);
      if (begin != covered && end > begin) return fail("slices not contiguous", c);
      covered = std::max(covered, end);
    }
    if (covered != t.n_real) return fail("slices do not cover the list", c);
    ++cases;
  }
  std::printf("ok %d\n", cases);
  return 0;
}
