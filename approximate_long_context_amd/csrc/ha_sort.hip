// Segmented stable counting sort of bucket ranks.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: rows are sorted by LSH bucket.)
// Ties keep their original order.  Ranks have at most 16 bits; one pass
// sorts one 8-bit digit (least significant first), so r <= 8 takes one
// pass and r <= 16 two.
//
// One launch sorts a batch of jobs (for example Q and K of a problem, or
// every level of the causal recursion); each job is a set of equal-length
// segments of one rank array.  A pass over the batch cuts every segment
// into tiles of kTile elements:
//   1. hist:    each tile counts its digits in LDS -> counts[seg][tile][digit]
//   2. scatter: each tile sums the counts of the segment into its first
//               output slot per digit, then each wave ranks its elements
//               among equal digits of the lower lanes (ballot per digit
//               bit), chunk by chunk in order, and writes the row index.
// The workgroups of all jobs form one flat grid; a workgroup finds its job
// by scanning the (few) job start offsets.
//
// HBM traffic per pass: 2 bytes of rank read twice (hist + scatter) or
// 4 bytes of input permutation + 2 of rank per element, 4 bytes written.
#include "ha_device.h"
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
  int32_t* perm_out;        // [segs][len]
  int tiles;
  int32_t* counts;          // [segs][tiles][256]
  uint32_t block0;          // first workgroup of this job in the flat grid
};

struct SortBatch {
  SortPass job[kSortMaxJobs];
  int njobs;
  int shift, bits;
};

// The job, segment and tile of workgroup `b` of the flat grid.  Callers
// pass the XCD-remapped id, so consecutive tiles of a segment run on one
// XCD: the scatter's short digit runs of neighbouring tiles share cache
// lines, which then fill in one L2 and are written back once.
__device__ __forceinline__ const SortPass& find_job(const SortBatch& B, uint32_t b, int64_t* seg, int* tile) {
  int j = 0;
  for (int i = 1; i < B.njobs; ++i) j = b >= B.job[i].block0 ? i : j;
  const SortPass& p = B.job[j];
  const uint32_t local = b - p.block0;
  *seg = local / static_cast<uint32_t>(p.tiles);
  *tile = static_cast<int>(local % static_cast<uint32_t>(p.tiles));
  return p;
}

// Row (within the head) of element e of segment `seg`, and its digit.
__device__ __forceinline__ void sort_elem(const SortPass& p, int shift, int bits, int64_t seg, int e,
                                          int32_t* row, uint32_t* digit) {
  const int64_t hd = seg / p.pieces;
  const int piece = static_cast<int>(seg % p.pieces);
  int32_t r = p.perm_in ? p.perm_in[seg * p.len + e] : p.first + piece * p.stride + e;
  *row = r;
  *digit = (static_cast<uint32_t>(p.rank[hd * p.n + r]) >> shift) & ((1u << bits) - 1u);
}

__global__ __launch_bounds__(kSortThreads) void sort_hist_kernel(SortBatch B) {
  __shared__ int hist[256];
  int64_t seg;
  int tile;
  const SortPass& p = find_job(B, static_cast<uint32_t>(xcd_remap(blockIdx.x, gridDim.x)), &seg, &tile);
  for (int b = threadIdx.x; b < 256; b += kSortThreads) hist[b] = 0;
  __syncthreads();
  const int e0 = tile * kTile;
  const int e1 = min(p.len, e0 + kTile);
  for (int e = e0 + threadIdx.x; e < e1; e += kSortThreads) {
    int32_t row;
    uint32_t dg;
    sort_elem(p, B.shift, B.bits, seg, e, &row, &dg);
    atomicAdd(&hist[dg], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < 256; b += kSortThreads)
    p.counts[(seg * p.tiles + tile) * 256 + b] = hist[b];
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
__device__ __forceinline__ void scatter_tile(const SortPass& p, int shift, int bits, int64_t seg, int e0,
                                             int e1, const int* base, int (*wh)[256]) {
  const int nb = 1 << bits;
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
    if (e < e1) sort_elem(p, shift, bits, seg, e, &row[c], &dg[c]);
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
    const uint64_t peers = wave_peers(valid, dg[c], bits, lane, &below, &cnt);
    int slot = 0;
    if (valid && below == 0) slot = atomicAdd(&wh[w][dg[c]], cnt);
    const int leader = valid ? static_cast<int>(__builtin_ctzll(peers)) : lane;
    slot = __shfl(slot, leader);
    if (valid) p.perm_out[seg * p.len + slot + below] = row[c];
  }
}

// Tile t of a segment: its first slot per digit is the number of elements
// with a smaller digit in the segment plus those with the same digit in the
// tiles before it (read from the per-tile counts of the histogram pass;
// thread b reads digit b of every tile, so each tile's row is one
// coalesced 1 KiB read).
__global__ __launch_bounds__(kSortThreads) void sort_scatter_kernel(SortBatch B) {
  __shared__ int wh[kSortWaves][256];
  __shared__ int base[256];
  __shared__ int tot[256];
  int64_t seg;
  int tile;
  const SortPass& p = find_job(B, static_cast<uint32_t>(xcd_remap(blockIdx.x, gridDim.x)), &seg, &tile);
  const int e0 = tile * kTile;
  const int e1 = min(p.len, e0 + kTile);
  {
    const int b = threadIdx.x;                    // kSortThreads == 256 digits
    const int32_t* c = p.counts + seg * p.tiles * 256 + b;
    int before = 0, all = 0;
    int t = 0;
    for (; t + 4 <= p.tiles; t += 4) {
      const int x0 = c[(t + 0) * 256], x1 = c[(t + 1) * 256], x2 = c[(t + 2) * 256], x3 = c[(t + 3) * 256];
      before += (t + 0 < tile ? x0 : 0) + (t + 1 < tile ? x1 : 0) + (t + 2 < tile ? x2 : 0) +
                (t + 3 < tile ? x3 : 0);
      all += x0 + x1 + x2 + x3;
    }
    for (; t < p.tiles; ++t) {
      const int x = c[t * 256];
      before += t < tile ? x : 0;
      all += x;
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
  scatter_tile(p, B.shift, B.bits, seg, e0, e1, base, wh);
}

static size_t job_ws_bytes(int64_t segs, int len, int r) {
  const int64_t tiles = (static_cast<int64_t>(len) + kTile - 1) / kTile;
  size_t bytes = align_up(static_cast<size_t>(segs) * 256 * (tiles < 1 ? 1 : tiles) * 4, 256);
  if (r > 8) bytes += align_up(static_cast<size_t>(segs) * len * 4, 256);
  return bytes;
}

size_t sort_ws_bytes(int64_t heads, int len, int pieces, int r) { return job_ws_bytes(heads * pieces, len, r); }

size_t sort_batch_ws_bytes(const SortJobDesc* jobs, int njobs, int r) {
  size_t bytes = 0;
  for (int j = 0; j < njobs; ++j) bytes += job_ws_bytes(jobs[j].heads * jobs[j].pieces, jobs[j].len, r);
  return bytes;
}

int launch_sort_batch(const SortJobDesc* jobs, int njobs, int r, void* ws, size_t ws_bytes, hipStream_t s) {
  if (njobs < 0 || njobs > kSortMaxJobs) {
    set_error("sort: %d jobs in one batch (at most %d)", njobs, kSortMaxJobs);
    return HA_EINVAL;
  }
  if (ws_bytes < sort_batch_ws_bytes(jobs, njobs, r)) {
    set_error("sort: workspace %zu < %zu bytes", ws_bytes, sort_batch_ws_bytes(jobs, njobs, r));
    return HA_EWORKSPACE;
  }
  Carve cv(ws, ws_bytes);
  SortBatch B{};
  int32_t* tmp[kSortMaxJobs] = {};
  int32_t* out[kSortMaxJobs] = {};
  uint64_t blocks = 0;
  for (int j = 0; j < njobs; ++j) {
    const SortJobDesc& d = jobs[j];
    const int64_t segs = d.heads * d.pieces;
    if (segs == 0 || d.len == 0) continue;
    const int tiles = (d.len + kTile - 1) / kTile;
    SortPass& p = B.job[B.njobs++];
    p.rank = d.rank;
    p.n = d.n;
    p.len = d.len;
    p.first = d.first;
    p.stride = d.stride;
    p.pieces = d.pieces;
    p.tiles = tiles;
    p.counts = cv.take<int32_t>(static_cast<size_t>(segs) * 256 * tiles);
    p.perm_in = nullptr;
    out[B.njobs - 1] = d.perm;
    tmp[B.njobs - 1] = r > 8 ? cv.take<int32_t>(static_cast<size_t>(segs) * d.len) : nullptr;
    p.block0 = static_cast<uint32_t>(blocks);
    blocks += static_cast<uint64_t>(segs) * tiles;
  }
  if (B.njobs == 0) return HA_OK;
  if (blocks >= (uint64_t(1) << 31)) {
    set_error("sort: %llu tiles in one batch", static_cast<unsigned long long>(blocks));
    return HA_EUNSUPPORTED;
  }
  const dim3 grid(static_cast<unsigned>(blocks));
  HA_TRY(launch_gate(HA_K_SORT));
  timing_begin(HA_K_SORT, s);
  int st = HA_OK;
  for (int pass = 0; pass < (r > 8 ? 2 : 1) && st == HA_OK; ++pass) {
    const bool two = r > 8;
    B.shift = pass == 0 ? 0 : 8;
    B.bits = two ? (pass == 0 ? 8 : r - 8) : r;
    for (int j = 0; j < B.njobs; ++j) {
      B.job[j].perm_in = pass == 0 ? nullptr : tmp[j];
      B.job[j].perm_out = (two && pass == 0) ? tmp[j] : out[j];
    }
    hipLaunchKernelGGL(sort_hist_kernel, grid, dim3(kSortThreads), 0, s, B);
    st = after_launch("sort hist", s);
    if (st != HA_OK) break;
    hipLaunchKernelGGL(sort_scatter_kernel, grid, dim3(kSortThreads), 0, s, B);
    st = after_launch("sort scatter", s);
  }
  timing_end(HA_K_SORT, s);
  return st;
}

int launch_sort(const uint16_t* rank, int64_t heads, int n, int len, int first, int stride,
                int pieces, int r, int32_t* perm, void* ws, size_t ws_bytes, hipStream_t s) {
  SortJobDesc d{rank, heads, n, len, first, stride, pieces, perm};
  return launch_sort_batch(&d, 1, r, ws, ws_bytes, s);
}

}  // namespace ha
