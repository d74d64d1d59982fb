// Host-side check of the grouped GEMMs' work lists (built with hipcc, run on
// the CPU).  It applies the rules of worklist.h exactly as the device builder
// does (tile counts, the tail decision, the item order, the XCD order, the K
// split of the last round) to many random expert-count vectors and checks:
//   - xcd_order is a bijection of [0, F) for both orders;
//   - the items (full ones and the split tiles) cover every (sorted row,
//     column tile) pair of every expert exactly once, each tile within its
//     expert's segment, with at most bm rows (bm + xr for a flagged tail tile,
//     which must be the expert's last tile);
//   - the K parts of a split tile cover [0, nk) exactly once for several nk;
//   - the item count stays within the grid bound the host sizes launches by.
// Usage: worklist_check [cases] [seed].  Prints "worklist ok <cases>" or the
// first failure (exit status 1).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "worklist.h"

using namespace moe;

namespace {

int fail(const char* what, int c, long a = 0, long b = 0) {
  std::printf("worklist FAIL case %d: %s (%ld, %ld)\n", c, what, a, b);
  return 1;
}

int exclusive_scan(std::vector<int>& v) {
  int s = 0;
  for (int& x : v) {
    const int y = x;
    x = s;
    s += y;
  }
  return s;
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 2000;
  const unsigned seed = argc > 2 ? (unsigned)std::atoi(argv[2]) : 1u;
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };

  // xcd_order alone: a bijection for every total up to a few rounds
  for (int total = 0; total <= 1300; ++total)
    for (int win = 0; win < 2; ++win) {
      std::vector<char> seen(total, 0);
      for (int b = 0; b < total; ++b) {
        const int L = xcd_order(b, total, win != 0);
        if (L < 0 || L >= total || seen[L]) return fail("xcd_order not a bijection", -1, total, b);
        seen[L] = 1;
      }
    }

  const int bms[3] = {32, 128, 256};
  for (int c = 0; c < cases; ++c) {
    const int E = uni(0, 3) == 0 ? uni(1, 8) : uni(1, 256);
    const int bm = bms[uni(0, 2)];
    const int xr = bm == 256 && uni(0, 3) ? kTailRows : 0;
    const int ntn = uni(1, 3) == 0 ? uni(1, 4) : uni(1, 120);
    const int ncu_opts[5] = {0, 256, 304, 80, uni(1, 300)};
    const int ncu = ncu_opts[uni(0, 4)];
    const int split_ncu = uni(0, 1) ? ncu : 0;
    const bool windows = uni(0, 1) != 0;
    // counts: empty experts, tiny ones, near multiples of bm, skewed loads
    std::vector<int> cnt(E);
    const int style = uni(0, 3);
    for (int e = 0; e < E; ++e) {
      int v;
      switch (style) {
        case 0: v = uni(0, 3 * bm); break;
        case 1: v = uni(0, 4) == 0 ? 0 : bm * uni(0, 9) + uni(-2, 40); break;
        case 2: v = (int)(20000.0 / (e + 1)) + uni(0, 50); break;
        default: v = uni(0, 1) ? 0 : uni(1, 33); break;
      }
      cnt[e] = v < 0 ? 0 : v;
    }
    std::vector<int> offs(E + 1);
    for (int e = 0; e < E; ++e) offs[e + 1] = offs[e] + cnt[e];
    const int M = offs[E];

    // the device builder's steps
    bool tails = false;
    if (xr > 0 && ncu > 0) {
      std::vector<int> t0(E), t1(E);
      for (int e = 0; e < E; ++e) t0[e] = row_tiles(cnt[e], bm, 0), t1[e] = row_tiles(cnt[e], bm, xr);
      const int plain = exclusive_scan(t0) * ntn, fused = exclusive_scan(t1) * ntn;
      tails = est_rounds(fused, ncu, split_ncu) < est_rounds(plain, ncu, split_ncu);
    }
    const int xuse = tails ? xr : 0;
    std::vector<int> tst(E + 1);
    for (int e = 0; e < E; ++e) tst[e] = row_tiles(cnt[e], bm, xuse);
    tst.resize(E);
    const int tiles = exclusive_scan(tst);
    tst.push_back(tiles);
    const int total = tiles * ntn;
    int R, P;
    split_plan(total, split_ncu, &R, &P);
    const int F = total - R;
    const int n_items = F + R * P;
    // grid bound of the host plan: (ceil(M / bm) + E) column-tile rows, plus
    // one round of split parts
    const long bound = ((long)(M + bm - 1) / bm + E) * ntn + (split_ncu > 0 ? 256 : 0);
    if (n_items > bound && split_ncu <= 256) return fail("more items than the grid bound", c, n_items, bound);
    if (R > 0 && (P < 2 || P > kMaxSplitParts || R * P > split_ncu)) return fail("bad split plan", c, R, P);

    std::vector<int2> work(n_items), split_tiles(R);
    for (int j = 0; j < R; ++j) split_tiles[j] = work_item(F + j, tst.data(), offs.data(), E, ntn, bm);
    for (int b = 0; b < n_items; ++b)
      work[b] = b < F ? work_item(xcd_order(b, F, windows), tst.data(), offs.data(), E, ntn, bm)
                      : make_int2(kSplitItem | (b - F), 0);

    // coverage of (row, column tile) pairs
    std::vector<unsigned char> cover((size_t)M * ntn, 0);
    auto mark = [&](int2 wk) -> int {
      const int e = item_expert(wk), n = item_col_tile(wk), r0 = item_first_row(wk);
      if (e < 0 || e >= E) return fail("expert out of range", c, e);
      if (n < 0 || n >= ntn) return fail("column tile out of range", c, n, ntn);
      if (r0 < offs[e] || r0 >= offs[e + 1]) return fail("first row outside the segment", c, r0, e);
      if ((r0 - offs[e]) % bm) return fail("tile does not start on a bm boundary", c, r0 - offs[e], bm);
      const bool tail = item_is_tail(wk);
      if (tail && !xuse) return fail("tail flag without tail rows", c, e);
      const int rem = offs[e + 1] - r0;
      if (tail && rem > bm + xuse) return fail("tail tile misses rows", c, rem, bm + xuse);
      if (!tail && rem > bm && rem - bm <= xuse) return fail("last rows left to an unflagged tile", c, rem);
      const int rows = item_rows(rem, tail, bm, xuse);
      if (rows < 1) return fail("empty tile", c, e);
      for (int r = r0; r < r0 + rows; ++r) {
        unsigned char& v = cover[(size_t)r * ntn + n];
        if (v) return fail("row covered twice", c, r, n);
        v = 1;
      }
      return 0;
    };
    std::vector<int> parts_seen(R, 0);
    for (int b = 0; b < n_items; ++b) {
      const int2 wk = work[b];
      if (item_is_split(wk)) {
        if (b < F) return fail("split part among the full items", c, b);
        int j, p;
        split_part(wk, P, &j, &p);
        if (j < 0 || j >= R || p < 0 || p >= P) return fail("split part out of range", c, j, p);
        if (parts_seen[j] & (1 << p)) return fail("split part listed twice", c, j, p);
        parts_seen[j] |= 1 << p;
      } else {
        if (b >= F) return fail("full item among the split parts", c, b);
        if (mark(wk)) return 1;
      }
    }
    for (int j = 0; j < R; ++j) {
      if (parts_seen[j] != (1 << P) - 1) return fail("split tile misses parts", c, j, parts_seen[j]);
      if (mark(split_tiles[j])) return 1;
    }
    for (size_t i = 0; i < cover.size(); ++i)
      if (!cover[i]) return fail("row never covered", c, (long)(i / ntn), (long)(i % ntn));
    // K ranges of the parts
    const int nks[6] = {1, 2, 7, 12, 64, 224};
    for (int nk : nks) {
      int next = 0;
      for (int p = 0; p < P; ++p) {
        int kb0, ke0;
        split_k_range(p, P, nk, &kb0, &ke0);
        if (kb0 != next || ke0 < kb0 || kb0 > nk - 1) return fail("K parts not contiguous", c, nk, p);
        next = ke0;
      }
      if (next != nk) return fail("K parts do not end at nk", c, nk, next);
    }
  }
  std::printf("worklist ok %d\n", cases);
  return 0;
}
