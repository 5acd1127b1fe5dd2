// Segmented stable counting sort of bucket ranks.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: rows are sorted by LSH bucket.)
// Ties keep their original order.  Ranks have at most 16 bits; one pass
// sorts one 8-bit digit (least significant first), so r <= 8 takes one
// pass and r <= 16 two.
//
// A pass over a segment cut into tiles of kTile elements:
//   1. hist:    each tile counts its digits in LDS -> counts[seg][digit][tile]
//   2. scatter: each tile sums the counts of the segment into its first
//               output slot per digit, then each wave ranks its elements
//               among equal digits of the lower lanes (ballot per digit
//               bit), chunk by chunk in order, and writes the row index.
// A segment of one tile takes a single fused kernel.
//
// HBM traffic per pass: 2 bytes of rank read twice (hist + scatter) or
// 4 bytes of input permutation + 2 of rank per element, 4 bytes written.
#include "ha_kernels.h"

namespace ha {

constexpr int kTile = 4096;
constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kWaveSpan = kTile / kSortWaves;   // elements per wave per tile

struct SortPass {
  const uint16_t* rank;     // [heads][n]
  int n;
  int len, first, stride, pieces;
  const int32_t* perm_in;   // [segs][len] or null (identity over the segment)
  int shift, bits;
  int32_t* perm_out;        // [segs][len]
  int tiles;
  int32_t* counts;          // [segs][256][tiles]
};

// Row (within the head) of element e of segment `seg`, and its digit.
__device__ __forceinline__ void sort_elem(const SortPass& p, int64_t seg, int e, int32_t* row,
                                          uint32_t* digit) {
  const int64_t hd = seg / p.pieces;
  const int piece = static_cast<int>(seg % p.pieces);
  int32_t r = p.perm_in ? p.perm_in[seg * p.len + e] : p.first + piece * p.stride + e;
  *row = r;
  *digit = (static_cast<uint32_t>(p.rank[hd * p.n + r]) >> p.shift) & ((1u << p.bits) - 1u);
}

__global__ __launch_bounds__(kSortThreads) void sort_hist_kernel(SortPass p) {
  __shared__ int hist[256];
  const int tile = blockIdx.x;
  const int64_t seg = blockIdx.y;
  const int nb = 1 << p.bits;
  for (int b = threadIdx.x; b < nb; b += kSortThreads) hist[b] = 0;
  __syncthreads();
  const int e0 = tile * kTile;
  const int e1 = min(p.len, e0 + kTile);
  for (int e = e0 + threadIdx.x; e < e1; e += kSortThreads) {
    int32_t row;
    uint32_t dg;
    sort_elem(p, seg, e, &row, &dg);
    atomicAdd(&hist[dg], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += kSortThreads)
    p.counts[(seg * 256 + b) * p.tiles + tile] = hist[b];
}

// Rank the wave's 64 elements among equal digits: the mask of lanes with the
// same digit, the number of them below this lane, and their count.
__device__ __forceinline__ uint64_t wave_peers(bool valid, uint32_t dg, int bits, int lane,
                                               int* below, int* count) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < bits; ++b) {
    const bool set = (dg >> b) & 1u;
    const uint64_t m = __ballot(valid && set);
    peers &= set ? m : ~m;
  }
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  *below = __popcll(peers & lower);
  *count = __popcll(peers);
  return peers;
}

// One tile [e0, e1) of a segment: each wave holds kWaveSpan consecutive
// elements (kChunks chunks of 64) in registers.  base[d] is the tile's first
// output slot for digit d.  Per-wave digit counts give each wave its own
// slots (stable across waves); inside a wave the chunks take their slots in
// order through LDS fetch-and-add by the first lane of each digit group
// (LDS operations of one wave complete in issue order, so the chunks stay
// ordered while their ranking overlaps).
constexpr int kChunks = kWaveSpan / 64;
__device__ __forceinline__ void scatter_tile(const SortPass& p, int64_t seg, int e0, int e1,
                                             const int* base, int (*wh)[256]) {
  const int nb = 1 << p.bits;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ws = e0 + w * kWaveSpan;
  int32_t row[kChunks];
  uint32_t dg[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int e = ws + 64 * c + lane;
    row[c] = 0;
    dg[c] = 0;
    if (e < e1) sort_elem(p, seg, e, &row[c], &dg[c]);
  }
  for (int i = threadIdx.x; i < kSortWaves * 256; i += kSortThreads) (&wh[0][0])[i] = 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    if (ws + 64 * c + lane < e1) atomicAdd(&wh[w][dg[c]], 1);
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += kSortThreads) {
    int run = base[b];
    for (int v = 0; v < kSortWaves; ++v) {
      const int x = wh[v][b];
      wh[v][b] = run;
      run += x;
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (ws + 64 * c >= e1) break;                 // wave-uniform
    const bool valid = ws + 64 * c + lane < e1;
    int below, cnt;
    const uint64_t peers = wave_peers(valid, dg[c], p.bits, lane, &below, &cnt);
    int slot = 0;
    if (valid && below == 0) slot = atomicAdd(&wh[w][dg[c]], cnt);
    const int leader = valid ? static_cast<int>(__builtin_ctzll(peers)) : lane;
    slot = __shfl(slot, leader);
    if (valid) p.perm_out[seg * p.len + slot + below] = row[c];
  }
}

// Tile t of a segment: its first slot per digit is the number of elements
// with a smaller digit in the segment plus those with the same digit in the
// tiles before it (read from the per-tile counts of the histogram pass).
__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(SortPass p) {
  __shared__ int wh[kSortWaves][256];
  __shared__ int base[256];
  __shared__ int tot[256];
  const int tile = blockIdx.x;
  const int64_t seg = blockIdx.y;
  const int nb = 1 << p.bits;
  const int e0 = tile * kTile;
  const int e1 = min(p.len, e0 + kTile);
  for (int b = threadIdx.x; b < 256; b += kSortThreads) {
    int before = 0, all = 0;
    if (b < nb) {
      const int32_t* c = p.counts + (seg * 256 + b) * p.tiles;
      for (int t = 0; t < p.tiles; ++t) {
        const int x = c[t];
        before += t < tile ? x : 0;
        all += x;
      }
    }
    base[b] = before;
    tot[b] = all;
  }
  __syncthreads();
  if (threadIdx.x < 64) {                         // exclusive scan of the 256 digit totals
    const int lane = threadIdx.x;
    int v[4];
    int sum = 0;
    for (int i = 0; i < 4; ++i) {
      v[i] = tot[lane * 4 + i];
      sum += v[i];
    }
    int incl = sum;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int run = incl - sum;
    for (int i = 0; i < 4; ++i) {
      base[lane * 4 + i] += run;
      run += v[i];
    }
  }
  __syncthreads();
  scatter_tile(p, seg, e0, e1, base, wh);
}

// Whole segment in one tile: histogram, scan and scatter in one block.
__global__ __launch_bounds__(kSortThreads) void sort_single_tile_kernel(SortPass p) {
  __shared__ int wh[kSortWaves][256];
  __shared__ int base[256];
  const int64_t seg = blockIdx.x;
  const int nb = 1 << p.bits;
  for (int b = threadIdx.x; b < 256; b += kSortThreads) base[b] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < p.len; e += kSortThreads) {
    int32_t row;
    uint32_t dg;
    sort_elem(p, seg, e, &row, &dg);
    atomicAdd(&base[dg], 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {                         // exclusive scan of the 256 digit totals
    const int lane = threadIdx.x;
    int v[4];
    int sum = 0;
    for (int i = 0; i < 4; ++i) {
      v[i] = base[lane * 4 + i];
      sum += v[i];
    }
    int incl = sum;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int run = incl - sum;
    for (int i = 0; i < 4; ++i) {
      base[lane * 4 + i] = run;
      run += v[i];
    }
  }
  __syncthreads();
  (void)nb;
  scatter_tile(p, seg, 0, p.len, base, wh);
}

size_t sort_ws_bytes(int64_t heads, int len, int pieces, int r) {
  const int64_t segs = heads * pieces;
  const int64_t tiles = (static_cast<int64_t>(len) + kTile - 1) / kTile;
  size_t bytes = align_up(static_cast<size_t>(segs) * 256 * (tiles < 1 ? 1 : tiles) * 4, 256);
  if (r > 8) bytes += align_up(static_cast<size_t>(segs) * len * 4, 256);
  return bytes;
}

static int run_pass(SortPass p, int64_t segs, hipStream_t s) {
  if (p.tiles == 1) {
    hipLaunchKernelGGL(sort_single_tile_kernel, dim3(static_cast<unsigned>(segs)),
                       dim3(kSortThreads), 0, s, p);
    return after_launch("sort (single tile)", s);
  }
  dim3 g(p.tiles, static_cast<unsigned>(segs));
  hipLaunchKernelGGL(sort_hist_kernel, g, dim3(kSortThreads), 0, s, p);
  HA_TRY(after_launch("sort hist", s));
  hipLaunchKernelGGL(sort_scatter_kernel, g, dim3(kSortThreads), 0, s, p);
  return after_launch("sort scatter", s);
}

int launch_sort(const uint16_t* rank, int64_t heads, int n, int len, int first, int stride,
                int pieces, int r, int32_t* perm, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t segs = heads * pieces;
  if (segs == 0 || len == 0) return HA_OK;
  if (ws_bytes < sort_ws_bytes(heads, len, pieces, r)) {
    set_error("sort: workspace %zu < %zu bytes", ws_bytes, sort_ws_bytes(heads, len, pieces, r));
    return HA_EWORKSPACE;
  }
  const int tiles = (len + kTile - 1) / kTile;
  Carve cv(ws, ws_bytes);
  int32_t* counts = cv.take<int32_t>(static_cast<size_t>(segs) * 256 * tiles);
  int32_t* tmp = r > 8 ? cv.take<int32_t>(static_cast<size_t>(segs) * len) : nullptr;

  SortPass p;
  p.rank = rank;
  p.n = n;
  p.len = len;
  p.first = first;
  p.stride = stride;
  p.pieces = pieces;
  p.tiles = tiles;
  p.counts = counts;
  timing_begin(HA_K_SORT, s);
  int st;
  if (r <= 8) {
    p.perm_in = nullptr;
    p.shift = 0;
    p.bits = r;
    p.perm_out = perm;
    st = run_pass(p, segs, s);
  } else {
    p.perm_in = nullptr;
    p.shift = 0;
    p.bits = 8;
    p.perm_out = tmp;
    st = run_pass(p, segs, s);
    if (st == HA_OK) {
      p.perm_in = tmp;
      p.shift = 8;
      p.bits = r - 8;
      p.perm_out = perm;
      st = run_pass(p, segs, s);
    }
  }
  timing_end(HA_K_SORT, s);
  return st;
}

}  // namespace ha
