// Sort of the T*K (token, expert) assignments into expert-contiguous order
// (the Dew "Mixture of experts" page, section "Expert computation and
// placement": tokens are sorted into expert order so the experts run as one
// grouped product).  A stable counting sort in three launches:
//
//   count   one block per chunk of 1024 assignments: LDS histogram per expert
//   scan    one block: per-expert totals, the exclusive scan into segment
//           offsets, each chunk's starting row inside every segment, and the
//           work lists of the grouped GEMMs (empty experts get no item, so
//           they launch no MFMA work; whether an expert's last row tile
//           takes its tail rows is decided here, see build_work_lists)
//   scatter one block per chunk: the chunk is walked in order; inside a wave
//           equal experts are found with nine ballots (expert id bits plus a
//           validity bit) and ranked by popcount, and waves are ordered
//           through per-wave counts in LDS.  Row order inside a segment is
//           therefore increasing (t, k).
//
// Decode-sized calls (T*K <= 1024) run the three steps in one block of one
// launch.  Assignments whose expert is the sentinel E (dropped by the
// dynamic threshold or the capacity) take no row.
//
// The host never reads the counts: the GEMM grids are sized by the bound
// (ceil(T*K / bm) + E) * column tiles on the number of items and surplus
// blocks exit.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void count_kernel(DispatchArgs a) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int64_t beg = (int64_t)blockIdx.x * kDispatchChunk;
  const int64_t end = min(a.M, beg + kDispatchChunk);
  for (int64_t i = beg + tid; i < end; i += kThreads) {
    const int e = a.sel32[i];
    if (e < a.E) atomicAdd(&hist[e], 1);  // e == E: a dropped assignment
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += kThreads) a.chunk_counts[(int64_t)blockIdx.x * a.E + e] = hist[e];
}

// Exclusive scan of v[0..n) (n <= kScanThreads) in LDS; returns the total.
// Called by all kScanThreads threads; thread i reads and writes only v[i].
// Each wave scans its 64 values with shuffles, wave 0 scans the wave totals,
// and each value adds its wave's offset: three barriers whatever n is.
__device__ int block_exclusive_scan(int* v, int* tmp, int n) {
  constexpr int NWV = kScanThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int x = tid < n ? v[tid] : 0;
  int s = x;  // inclusive scan inside the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(s, off);
    if (lane >= off) s += y;
  }
  if (lane == 63) tmp[wv] = s;
  __syncthreads();
  if (wv == 0) {
    const int t = lane < NWV ? tmp[lane] : 0;
    int u = t;
#pragma unroll
    for (int off = 1; off < NWV; off <<= 1) {
      const int y = __shfl_up(u, off);
      if (lane >= off) u += y;
    }
    if (lane < NWV) tmp[NWV + lane] = u - t;  // exclusive offset of wave `lane`
  }
  __syncthreads();
  const int excl = s - x + tmp[NWV + wv];
  if (tid < n) v[tid] = excl;
  if (tid == n - 1) tmp[2 * NWV] = excl + x;
  __syncthreads();
  return n > 0 ? tmp[2 * NWV] : 0;
}

// Work lists of the grouped GEMMs from the per-expert counts `cnts` and
// segment offsets `offs` (both in LDS), by the rules of worklist.h (tile
// counts, the tail decision, the item order, the XCD order, the K split).
// Empty experts contribute no item.  Called by all kScanThreads threads of
// one block; `tst` (E+1) and `tmp` (kScanThreads) are LDS scratch.
__device__ void build_work_lists(const DispatchArgs& a, const int* cnts, const int* offs, int* tst, int* tmp) {
  const int tid = threadIdx.x;
  const int E = a.E;
  for (int g = 0; g < a.nspec; ++g) {
    const WorkSpec& sp = a.spec[g];
    __syncthreads();
    // Row tiles per expert: bm rows each; with tail rows (xr) the last one
    // takes up to xr more.  Tail rows make the last tile of an expert dearer
    // (one more 32-row strip), so they are used only when they lower the
    // estimated makespan: full rounds on ncu CUs plus the last partial round
    // (a K-split part's share when that round is split, else a whole tile).
    bool tails = false;
    if (sp.xr > 0 && sp.ncu > 0) {
      if (tid < E) tst[tid] = row_tiles(cnts[tid], sp.bm, 0);
      __syncthreads();
      const int plain = block_exclusive_scan(tst, tmp, E) * sp.ntn;
      if (tid < E) tst[tid] = row_tiles(cnts[tid], sp.bm, sp.xr);
      __syncthreads();
      const int fused = block_exclusive_scan(tst, tmp, E) * sp.ntn;
      tails = est_rounds(fused, sp.ncu, sp.split_ncu) < est_rounds(plain, sp.ncu, sp.split_ncu);
    }
    if (tid < E) tst[tid] = row_tiles(cnts[tid], sp.bm, tails ? sp.xr : 0);
    __syncthreads();
    const int tiles = block_exclusive_scan(tst, tmp, E);
    if (tid == 0) tst[E] = tiles;
    __syncthreads();
    const int ntn = sp.ntn;
    const int total = tiles * ntn;
    // Items past the last full round of split_ncu blocks are cut along K.
    int R, P;
    split_plan(total, sp.split_ncu, &R, &P);
    const int F = total - R;
    const int n_items = F + R * P;
    if (tid == 0) {
      sp.num_work[0] = n_items;
      if (sp.split_info) {
        sp.split_info[0] = R;
        sp.split_info[1] = P;
      }
    }
    for (int j = tid; j < R; j += kScanThreads) sp.split_tiles[j] = work_item(F + j, tst, offs, E, ntn, sp.bm);
    // Blocks [0, F) take the full items in the XCD order; blocks [F, F+R*P)
    // the split parts, which blocks b % 8 spread evenly over the XCDs and
    // which dispatch last.
    for (int b = tid; b < n_items && b < sp.max_work; b += kScanThreads)
      sp.work[b] = b < F ? work_item(xcd_order(b, F, sp.windows != 0), tst, offs, E, ntn, sp.bm)
                         : make_int2(kSplitItem | (b - F), 0);
  }
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(DispatchArgs a) {
  __shared__ int part[kScanThreads];   // [J][E] partial chunk sums, then their prefixes
  __shared__ int tmp[kScanThreads];
  __shared__ int offs[kMaxExperts + 1];
  __shared__ int tst[kMaxExperts + 1];
  __shared__ int cnts[kMaxExperts];
  const int tid = threadIdx.x;
  const int E = a.E;
  const int nch = a.nchunks;
  // chunk-range lanes per expert (no more than there are chunks)
  const int J = max(1, min(kScanThreads / E, nch));
  const int e = tid % E, j = tid / E;
  const bool worker = j < J;
  const int cb = worker ? (int)((int64_t)j * nch / J) : 0;
  const int ce = worker ? (int)((int64_t)(j + 1) * nch / J) : 0;

  // A worker's chunk counts (2 to kScanBatch of them) are loaded in one
  // batch (addresses clamped into its range, the extra lanes masked) and
  // kept for the bases below; single chunks and longer ranges loop.
  constexpr int kScanBatch = 16;
  const int per = ce - cb;
  const bool batched = per > 1 && per <= kScanBatch;
  int cc[kScanBatch];
  int s = 0;
  if (batched) {
#pragma unroll
    for (int q = 0; q < kScanBatch; ++q) {
      const int b = min(cb + q, max(ce - 1, 0));
      const int v = a.chunk_counts[(int64_t)b * E + e];
      cc[q] = q < per ? v : 0;
    }
#pragma unroll
    for (int q = 0; q < kScanBatch; ++q) s += cc[q];
  } else {
    for (int b = cb; b < ce; ++b) s += a.chunk_counts[(int64_t)b * E + e];
  }
  // Exclusive scan over j of part[j*E + e] for every expert at once: a
  // Hillis-Steele scan whose strides are multiples of E.
  const int n = J * E;
  tmp[tid] = worker ? s : 0;
  __syncthreads();
  for (int off = E; off < n; off <<= 1) {
    const int y = (tid >= off && worker) ? tmp[tid - off] : 0;
    __syncthreads();
    if (worker) tmp[tid] += y;
    __syncthreads();
  }
  if (worker) part[tid] = tmp[tid] - s;
  __syncthreads();
  if (tid < E) {
    const int run = tmp[(J - 1) * E + tid];  // the expert's count
    offs[tid] = run;  // count, scanned below
    cnts[tid] = run;
    a.counts[tid] = run;
    if (a.counts_out) a.counts_out[tid] = run;
  }
  __syncthreads();
  const int M = block_exclusive_scan(offs, tmp, E);
  // Thread E writes the end offset from its own copy of the total: offs[E]
  // is written by thread 0, which for E >= 64 sits in another wave, and is
  // read by other threads only after the next barrier.
  if (tid == 0) offs[E] = M;
  if (tid <= E) {
    const int o = tid == E ? M : offs[tid];
    a.offsets[tid] = o;
    if (a.offsets_out) a.offsets_out[tid] = o;
  }
  if (worker) {
    int base = offs[e] + part[j * E + e];
    if (batched) {
#pragma unroll
      for (int q = 0; q < kScanBatch; ++q)
        if (q < per) {
          a.chunk_base[(int64_t)(cb + q) * E + e] = base;
          base += cc[q];
        }
    } else {
      for (int b = cb; b < ce; ++b) {
        const int64_t idx = (int64_t)b * E + e;
        const int c = a.chunk_counts[idx];
        a.chunk_base[idx] = base;
        base += c;
      }
    }
  }

  build_work_lists(a, cnts, offs, tst, tmp);
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(DispatchArgs a) {
  __shared__ int running[kMaxExperts];
  __shared__ int wcount[kThreads / 64][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = a.E;
  for (int e = tid; e < E; e += kThreads) {
    running[e] = a.chunk_base[(int64_t)blockIdx.x * E + e];
#pragma unroll
    for (int q = 0; q < kThreads / 64; ++q) wcount[q][e] = 0;
  }
  __syncthreads();
  const int64_t beg = (int64_t)blockIdx.x * kDispatchChunk;
  const int64_t end = min(a.M, beg + kDispatchChunk);
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t base = beg; base < end; base += kThreads) {
    const int64_t i = base + tid;
    const int ei = i < end ? a.sel32[i] : E;
    const bool valid = ei < E;                        // E: past the end, or a dropped assignment
    const int e = valid ? ei : kMaxExperts;           // the sentinel only matches itself
    uint64_t same = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      const int on = (e >> bit) & 1;
      const uint64_t b = __ballot(on);
      same &= on ? b : ~b;
    }
    const int rank = __popcll(same & below);
    if (valid && rank == 0) wcount[w][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int pos = running[e] + rank;
      for (int q = 0; q < w; ++q) pos += wcount[q][e];
      a.sorted_tok[pos] = (int32_t)(i / a.K);
      a.sorted_slot[pos] = (int32_t)i;
      if (a.sorted_w) a.sorted_w[pos] = a.weights[i];
    }
    __syncthreads();
    for (int x = tid; x < E; x += kThreads) {
      int add = 0;
#pragma unroll
      for (int q = 0; q < kThreads / 64; ++q) {
        add += wcount[q][x];
        wcount[q][x] = 0;
      }
      running[x] += add;
    }
    __syncthreads();
  }
}

// The whole sort for T*K <= kScanThreads assignments (decode-sized calls) in
// one block of kScanThreads threads: thread i owns assignment i.  Counts,
// offsets and work lists as in scan_kernel; the stable rank of assignment i
// inside its expert is its rank among equal experts of its wave (nine
// ballots) plus the counts of the earlier waves, so the order inside a
// segment is increasing (t, k) as in scatter_kernel.
__global__ __launch_bounds__(kScanThreads) void dispatch_small_kernel(DispatchArgs a) {
  constexpr int W = kScanThreads / 64;
  __shared__ int tmp[kScanThreads];
  __shared__ int offs[kMaxExperts + 1];
  __shared__ int tst[kMaxExperts + 1];
  __shared__ int cnts[kMaxExperts];
  __shared__ int wcount[W][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = a.E;
  for (int x = tid; x < E; x += kScanThreads) {
    cnts[x] = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) wcount[q][x] = 0;
  }
  __syncthreads();
  const int ei = tid < a.M ? a.sel32[tid] : E;
  const bool valid = ei < E;                 // E: past the end, or a dropped assignment
  const int e = valid ? ei : kMaxExperts;    // the sentinel only matches itself
  uint64_t same = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const int on = (e >> bit) & 1;
    const uint64_t b = __ballot(on);
    same &= on ? b : ~b;
  }
  const int rank = __popcll(same & ((1ull << lane) - 1ull));
  if (valid && rank == 0) wcount[w][e] = __popcll(same);
  __syncthreads();
  if (tid < E) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) c += wcount[q][tid];
    cnts[tid] = c;
    offs[tid] = c;
    a.counts[tid] = c;
    if (a.counts_out) a.counts_out[tid] = c;
  }
  __syncthreads();
  const int M = block_exclusive_scan(offs, tmp, E);
  if (tid == 0) offs[E] = M;  // read by other threads after the barrier below
  if (tid <= E) {
    const int o = tid == E ? M : offs[tid];
    a.offsets[tid] = o;
    if (a.offsets_out) a.offsets_out[tid] = o;
  }
  __syncthreads();
  if (valid) {
    int pos = offs[e] + rank;
    for (int q = 0; q < w; ++q) pos += wcount[q][e];
    a.sorted_tok[pos] = (int32_t)(tid / a.K);
    a.sorted_slot[pos] = (int32_t)tid;
    if (a.sorted_w) a.sorted_w[pos] = a.weights[tid];
  }
  build_work_lists(a, cnts, offs, tst, tmp);
}

// Capacity (the Dew "Mixture of experts" page, section "Expert computation
// and placement", capacity_factor): each sequence keeps at most `slots`
// assignments per expert, the first in token order.  In the stable sorted
// order an expert's rows from one sequence are contiguous and in (t, k)
// order, so a row's rank among them is its distance to the first row of the
// segment whose token is in the same sequence (a binary search).
__global__ __launch_bounds__(kThreads) void capacity_kernel(CapacityArgs a) {
  __shared__ int offs[kMaxExperts + 1];
  const int E = a.E;
  for (int e = threadIdx.x; e <= E; e += kThreads) offs[e] = a.offsets[e];
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r >= offs[E]) return;
  // expert: the last e with offs[e] <= r
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offs[mid] <= r) lo = mid; else hi = mid;
  }
  const int64_t t = a.sorted_tok[r];
  const int64_t s0 = t - t % a.seq_len;
  int64_t b = offs[lo], c = r;  // first row in [b, r] whose token is >= s0
  while (b < c) {
    const int64_t mid = (b + c) >> 1;
    if (a.sorted_tok[mid] < s0) b = mid + 1; else c = mid;
  }
  if (r - b >= a.slots) {
    const int32_t slot = a.sorted_slot[r];
    a.sel32[slot] = E;
    if (a.kept) a.kept[slot] = 0;
  }
}

}  // namespace

hipError_t launch_capacity(const CapacityArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((a.M + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(capacity_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.M <= kScanThreads) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(count_kernel, dim3(a.nchunks), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
  hipLaunchKernelGGL(scatter_kernel, dim3(a.nchunks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
