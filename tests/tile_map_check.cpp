// Host-side property check of the grouped GEMMs' workgroup -> tile map
// (xcd_tile_at in the library's internal header, compiled here for the host).
//
// For each case (large m-tiles, total m-tiles, n-tiles, reserve) it walks every
// position q of each of the 8 XCD sequences and checks:
//   1. every (m-tile, n-tile) pair is produced exactly once over all XCDs;
//   2. each XCD's valid positions form a prefix (a workgroup that loops over
//      q, q + G, ... may stop at the first invalid one);
//   3. no XCD gets more than ceil(total / 8) m-tiles, so the grid
//      8 * ceil(bound / 8) * n_tiles covers every sequence for any bound >= total;
//   4. an m-tile's n-tiles sit at consecutive positions, in n-tile order;
//   5. each XCD's large m-tiles are one contiguous, increasing range;
//   6. an XCD's last min(reserve, small) positions hold its highest-numbered
//      (smallest) small m-tiles, in increasing order.
// And the compact tiles' row split between the two wave rows (compact_f0 /
// compact_f1 in the same header), for every row count 1..160 and both forms:
//   7. the split of a tile's row count equals the split of its class bound (the
//      K loop is chosen by class, the epilogue by row count);
//   8. the two bands cover every row: 32 * (f0 + f1) >= rows;
//   9. they stay within the compact stage's rows, 32 * (f0 + f1) <= class bound,
//      and within a wave's 4 accumulator blocks; wave row 0 holds at least one.
// Prints one line per failing case and exits non-zero if any failed.
//
//   check [seed] [random_cases]
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "moe_internal.h"

namespace {

int fails = 0;

void fail(const char* what, int large, int total, int nt, int reserve, int x, int q) {
  if (++fails <= 20)
    std::printf("FAIL %s: large=%d total=%d n_tiles=%d reserve=%d xcd=%d q=%d\n", what, large,
                total, nt, reserve, x, q);
}

void check_case(int large, int total, int n_tiles, int reserve) {
  moe::MTileMap tm{};
  tm.large = large;
  tm.total = total;
  std::vector<int> seen((size_t)total * n_tiles, 0);
  const int cap = (total + 7) / 8;
  for (int x = 0; x < 8; ++x) {
    std::vector<int> seq;  // m-tile at each m-position of this XCD
    bool ended = false;
    // walk well past the grid the host would launch
    const int qmax = (cap + 3) * n_tiles;
    for (int q = 0; q < qmax; ++q) {
      int mt = -1, nt = -1;
      const bool ok = moe::xcd_tile_at(tm, n_tiles, x, q, reserve, &mt, &nt);
      if (!ok) {
        ended = true;
        continue;
      }
      if (ended) fail("valid position after an invalid one", large, total, n_tiles, reserve, x, q);
      if (mt < 0 || mt >= total || nt < 0 || nt >= n_tiles) {
        fail("tile out of range", large, total, n_tiles, reserve, x, q);
        continue;
      }
      if (nt != q % n_tiles) fail("n-tile not in position order", large, total, n_tiles, reserve, x, q);
      if (q % n_tiles == 0) {
        seq.push_back(mt);
      } else if (seq.empty() || seq.back() != mt) {
        fail("m-tile's n-tiles not consecutive", large, total, n_tiles, reserve, x, q);
      }
      seen[(size_t)mt * n_tiles + nt] += 1;
    }
    if ((int)seq.size() > cap) fail("more than ceil(total/8) m-tiles", large, total, n_tiles, reserve, x, -1);
    // large m-tiles: one contiguous increasing range
    std::vector<int> lg, sm;
    for (int mt : seq) (mt < large ? lg : sm).push_back(mt);
    for (size_t i = 1; i < lg.size(); ++i)
      if (lg[i] != lg[i - 1] + 1) fail("large m-tiles not contiguous", large, total, n_tiles, reserve, x, (int)i);
    // the reserve: the last R positions hold the XCD's R highest small m-tiles, ascending
    const int R = reserve < (int)sm.size() ? reserve : (int)sm.size();
    std::vector<int> sorted_sm = sm;
    std::sort(sorted_sm.begin(), sorted_sm.end());
    for (int i = 0; i < R; ++i) {
      const int pos = (int)seq.size() - R + i;
      const int want = sorted_sm[sorted_sm.size() - R + i];
      if (pos < 0 || seq[pos] != want) fail("reserve not the XCD's smallest tiles last", large, total, n_tiles, reserve, x, pos);
    }
  }
  for (size_t i = 0; i < seen.size(); ++i)
    if (seen[i] != 1) {
      fail(seen[i] ? "tile produced more than once" : "tile never produced", large, total, n_tiles,
           reserve, -1, (int)i);
      break;
    }
}

void check_compact_split() {
  for (int spread = 0; spread < 2; ++spread)
    for (int rows = 1; rows <= 160; ++rows) {
      const int cls = rows <= 32 ? 32 : rows <= 64 ? 64 : rows <= 128 ? 128 : 160;
      const int f0 = moe::compact_f0(rows, spread), f1 = moe::compact_f1(rows, spread);
      const bool ok = f0 == moe::compact_f0(cls, spread) && f1 == moe::compact_f1(cls, spread) &&
                      32 * (f0 + f1) >= rows && 32 * (f0 + f1) <= cls && f0 >= 1 && f0 <= 4 &&
                      f1 >= 0 && f1 <= 4;
      if (!ok && ++fails <= 20)
        std::printf("FAIL compact split: rows=%d spread=%d f0=%d f1=%d\n", rows, spread, f0, f1);
    }
}

}  // namespace

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? (unsigned)std::atoi(argv[1]) : 2024u;
  const int n_random = argc > 2 ? std::atoi(argv[2]) : 3000;
  const int n_tiles_set[] = {1, 2, 8, 16, 28, 56};
  int cases = 0;
  // edge cases: nothing, all large, all small, fewer tiles than XCDs
  const int edge[][2] = {{0, 0}, {0, 1}, {1, 1}, {0, 7}, {7, 7}, {3, 9}, {8, 8}, {0, 8},
                         {9, 9}, {0, 256}, {256, 256}, {17, 300}, {64, 65}};
  for (const auto& lt : edge)
    for (int nt : n_tiles_set)
      for (int rsv : {0, (32 + nt - 1) / nt, 1000}) {
        check_case(lt[0], lt[1], nt, rsv);
        ++cases;
      }
  std::mt19937 rng(seed);
  for (int i = 0; i < n_random; ++i) {
    const int nt = n_tiles_set[rng() % 6];
    int total;
    switch (rng() % 4) {
      case 0: total = (int)(rng() % 16); break;
      case 1: total = (int)(rng() % 300); break;
      case 2: total = (int)(rng() % 5000); break;
      default: total = (int)(rng() % 2000) + 1; break;
    }
    const int large = total ? (int)(rng() % (total + 1)) : 0;
    const int rsv = (rng() % 3 == 0) ? 0 : (32 + nt - 1) / nt;
    check_case(large, total, nt, rsv);
    ++cases;
  }
  // products past 32 bits (C1 >= 65536): large launches, one n-tile
  for (int total : {70000, 600000}) {
    check_case(total / 3, total, 1, 32);
    check_case(total, total, 1, 32);
    check_case(0, total, 1, 32);
    cases += 3;
  }
  check_compact_split();
  cases += 320;
  std::printf("%d cases, %d failures\n", cases, fails);
  return fails ? 1 : 0;
}
