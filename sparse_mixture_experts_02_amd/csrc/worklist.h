// Work lists of the grouped expert GEMMs: which (expert, row tile, column
// tile) items exist, in which order the XCDs take them, which of them are cut
// along K, and how a kernel decodes an item.
//
// The rows of a grouped GEMM are the assignments in expert-sorted order (the
// Dew "Mixture of experts" page, section "Expert computation and placement":
// tokens sorted into expert order, the experts run as one grouped product).
// Every function here is host-and-device code: the device builder in
// dispatch.hip and the GEMM kernels use them, and a host program in the tests
// re-runs the same rules over many expert-count vectors and checks that the
// items cover every sorted row and column tile exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kColGroup = 4;       // column tiles per ordering group
constexpr int kMaxSplitParts = 8;  // K parts per split item at most (4 measured 0.5-4% slower with the 16-block fix-up)
constexpr int32_t kSplitItem = (int32_t)0x80000000;
// A work item {expert | column_tile << 8, first_row | kTailTile} is the last
// row tile of its expert and holds all of the expert's remaining rows (at most
// BM + kTailRows; 256-row bf16 tiles only).
constexpr int kTailRows = 32;
constexpr int32_t kTailTile = (int32_t)0x80000000;

__host__ __device__ inline int wl_min(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int wl_max(int a, int b) { return a > b ? a : b; }

// Row tiles of an expert with c rows: bm rows each, except that the last one
// may take up to xr more (xr = 0: plain tiles).  An empty expert has none.
__host__ __device__ inline int row_tiles(int c, int bm, int xr) {
  return c == 0 ? 0 : wl_max(1, (c - xr + bm - 1) / bm);
}

// Split of a GEMM's last partial round along K: with `split_ncu` compute
// units and `total` items, the R = total % split_ncu items past the last full
// round are each cut into P = min(kMaxSplitParts, split_ncu / R) K ranges when
// P >= 2 (R = 0, P = 1 otherwise: no split).
__host__ __device__ inline void split_plan(int total, int split_ncu, int* R, int* P) {
  int r = 0, p = 1;
  if (split_ncu > 0 && total > 0) {
    r = total % split_ncu;
    p = r > 0 ? wl_min(kMaxSplitParts, split_ncu / r) : 1;
    if (p < 2) r = 0, p = 1;
  }
  *R = r;
  *P = p;
}

// Estimated makespan in rounds of `ncu` blocks: the full rounds plus the last
// partial one, which costs a K-split part's share when it is split, else a
// whole tile.
__host__ __device__ inline float est_rounds(int total, int ncu, int split_ncu) {
  const int R = total % ncu;
  int P = 1;
  if (split_ncu > 0 && R > 0) P = wl_min(kMaxSplitParts, split_ncu / R);
  return (float)(total / ncu) + (R == 0 ? 0.f : (P >= 2 ? 1.f / P : 1.f));
}

// Position of work item b in the operand-sharing order.  Blocks are handed
// to the 8 XCDs round-robin (b % 8).  Contiguous: XCD x receives one
// contiguous range of the order.  Windows: an XCD's 32 CUs run its blocks in
// rounds of 32, so the order is dealt out in windows of 32 items, XCD x
// taking windows x, x + 8, x + 16, ...; its 32 concurrently running tiles are
// then one window of the order (with 8 row tiles per expert, exactly one
// group of 4 column tiles x 8 row tiles) and share 4 weight column tiles and
// 8 row tiles of activations in its L2, where contiguous ranges straddle the
// groups (prefill layer -2..-3.4%; the decode weight stream is 3% slower
// with windows).  Items past the last whole 256-item round go to the XCDs
// in contiguous ranges.  A bijection of [0, total).
__host__ __device__ inline int xcd_order(int b, int total, bool windows) {
  const int full = windows ? (total / 256) * 256 : 0;
  if (b < full) {
    const int i = b / 8, x = b % 8;
    return 256 * (i / 32) + 32 * x + i % 32;
  }
  b -= full;
  total -= full;
  const int q = total / 8, r = total % 8, x = b % 8, i = b / 8;
  return full + (x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i);
}

// The item at position L of the order: experts ascending; inside an expert,
// groups of kColGroup column tiles; inside a group, column tile slowest and
// row tile fastest.  `tst` (E+1) is the exclusive scan of the experts' row
// tiles (tst[E] = all row tiles), `offs` (E+1) the segment offsets, `ntn` the
// column tiles, `bm` the rows per tile.  Returns {expert | column_tile << 8,
// first sorted row | kTailTile when the tile holds more than bm rows}.
__host__ __device__ inline int2 work_item(int L, const int* tst, const int* offs, int E, int ntn, int bm) {
  // expert: the last x with tst[x] * ntn <= L (empty experts have
  // tst[x] == tst[x + 1] and are skipped)
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tst[mid] * ntn <= L) lo = mid; else hi = mid;
  }
  const int x = lo;
  const int mt = tst[x + 1] - tst[x];
  const int q = L - tst[x] * ntn;
  const int full = (ntn / kColGroup) * kColGroup * mt;
  // all operands are non-negative: unsigned division is the shorter sequence
  int m, n;
  if (q < full) {
    const unsigned gsz = (unsigned)(kColGroup * mt);
    const unsigned grp = (unsigned)q / gsz, r = (unsigned)q - grp * gsz;
    n = (int)(grp * kColGroup + r / (unsigned)mt);
    m = (int)(r % (unsigned)mt);
  } else {
    const unsigned r = (unsigned)(q - full);
    n = (ntn / kColGroup) * kColGroup + (int)(r / (unsigned)mt);
    m = (int)(r % (unsigned)mt);
  }
  // the last tile of an expert with more than bm remaining rows holds them all
  const bool tail = m == mt - 1 && offs[x + 1] - (offs[x] + m * bm) > bm;
  return make_int2(x | (n << 8), (offs[x] + m * bm) | (tail ? kTailTile : 0));
}

// Decoding of a (non-split) item.
__host__ __device__ inline int item_expert(int2 wk) { return wk.x & 0xff; }
__host__ __device__ inline int item_col_tile(int2 wk) { return wk.x >> 8; }
__host__ __device__ inline int item_first_row(int2 wk) { return wk.y & 0x7fffffff; }
__host__ __device__ inline bool item_is_tail(int2 wk) { return (wk.y & kTailTile) != 0; }
__host__ __device__ inline bool item_is_split(int2 wk) { return wk.x < 0; }
// Rows of a tile whose expert has `rem` rows from its first row on: bm, or
// all of them (at most bm + xr) for a tail tile.
__host__ __device__ inline int item_rows(int rem, bool tail, int bm, int xr) {
  return wl_min(rem, tail ? bm + xr : bm);
}
// A split item {kSplitItem | q, 0} is part p of split tile j (q = j*P + p);
// the part covers K steps [p*nk/P, (p+1)*nk/P) of nk.
__host__ __device__ inline void split_part(int2 wk, int P, int* j, int* p) {
  const int q = wk.x & 0x7fffffff;
  *j = q / P;
  *p = q - *j * P;
}
__host__ __device__ inline void split_k_range(int p, int P, int nk, int* kb0, int* ke0) {
  *kb0 = p * nk / P;
  *ke0 = (p + 1) * nk / P;
}

}  // namespace moe
