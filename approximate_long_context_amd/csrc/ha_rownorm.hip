// Row-norm-sampling variant of the product with V (non-causal problems).
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: the product with V is
// approximated by row-norm sampling; "Builds on": approximate matrix
// multiplication via row norm sampling.)
//
// The normaliser keeps its exact block row sums plus uniform samples; the
// numerator's residual (keys outside the row's block) is estimated from m
// key positions drawn with probability proportional to the squared norm of
// the value row, each kept draw weighted 1 / (m p).  Probabilities are exact
// integers so that draws are reproducible bit for bit:
//   w_t = ||v_t||^2 in fp32 (squares rounded, groups of 8 consecutive
//         squares summed by halving, group sums by halving);
//   n_t = floor(w_t 2^(40 - e)) with max w = f 2^e, f in [0.5, 1);
//   c_t = n_0 + ... + n_t over the sorted key positions, T = c_last;
//   draw i: word x of Philox counter (i / 4, node, head, 2 batch + 2),
//   r = floor(x T / 2^32), position = smallest t with c_t > r;
//   weight T / (m n_t), folded into a per-head copy of the drawn V rows.
// Kernels here: squared norms, the per-problem integer CDF (max, chunk
// scans, chunk offsets), the draws (binary search) and the copy of the drawn
// K / weighted V rows.  The result
//   out = (N_blk + N_rn) / (D_blk + D_unif),  lse = ln(D_blk + D_unif)
// takes two attention passes: the first, in the lse-only mode (no V rows,
// no P V products), stores the plain estimator's lse; the second attends
// to the block keys plus the drawn rows (unit weight in its own normaliser D2 = D_blk + sum of their
// exponentials) and scales its output by D2 / (D_blk + D_unif) =
// exp(own lse - stored lse), which turns (N_blk + N_rn) / D2 into the result.
#include <cmath>

#include "ha_device.h"
#include "ha_kernels.h"
#include "ha_rng.h"

namespace ha {

constexpr int kRnQBits = 40;

// ---- squared row norms: 8 lanes per row (64 columns) or 16 (128); squares
// and sums rounded separately (no multiply-add contraction) -----------------

#pragma clang fp contract(off)
template <typename T, int D>
__global__ __launch_bounds__(256) void rownorm_sqnorm_kernel(const T* __restrict__ v, int64_t rows,
                                                             float* __restrict__ w) {
  constexpr int LPR = D / 8;                       // lanes per row, one group of 8 each
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  for (int64_t r0 = wave * RPW; r0 < rows; r0 += nwaves * RPW) {
    const int64_t row = r0 + lane / LPR;
    const int64_t rs = row < rows ? row : rows - 1;
    const T* src = v + rs * D + 8 * (lane % LPR);
    float sq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = static_cast<float>(src[i]);
      sq[i] = x * x;
    }
    // halving within the group: pairs 4 apart, 2 apart, 1 apart
#pragma unroll
    for (int i = 0; i < 4; ++i) sq[i] = sq[i] + sq[i + 4];
    sq[0] = sq[0] + sq[2];
    sq[1] = sq[1] + sq[3];
    float g = sq[0] + sq[1];
    // halving over the groups (xor partners: lane i < h pairs with i + h)
#pragma unroll
    for (int h = LPR / 2; h >= 1; h >>= 1) g = g + __shfl_xor(g, h);
    if (row < rows && lane % LPR == 0) w[row] = g;
  }
}

// ---- integer CDF: per-problem max, chunk scans, chunk offsets -----------------
// (1) rownorm_max_kernel: one workgroup per 2048 rows of a KV problem, the
//     largest w among them (row order: the maximum does not depend on it);
// (2) rownorm_chunk_kernel: one workgroup per 2048 sorted positions: the
//     problem's largest w from the chunk maxima (exact, any order), then the
//     quantised weights n_t (gathered through the permutation) and their
//     inclusive scan within the chunk, plus the chunk's total;
// (3) rownorm_offset_kernel: each chunk adds the totals of the chunks before
//     it (exact int64 sums, so the order of additions does not matter).

constexpr int kRnThreads = 256;
constexpr int kRnChunk = 2048;                      // 8 positions per thread

__global__ __launch_bounds__(kRnThreads) void rownorm_max_kernel(const float* __restrict__ w, RnGeom g, int nchunk,
                                                                  float* __restrict__ cmax) {
  __shared__ float red[kRnThreads / 64];
  const int64_t prob = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const int n = g.seg;
  const int64_t bkv = prob / g.pieces;
  const float* wp = w + bkv * g.n_head + g.k_first + (prob - bkv * g.pieces) * g.stride;
  float mx = 0.f;
  for (int t = chunk * kRnChunk + threadIdx.x; t < min((chunk + 1) * kRnChunk, n); t += kRnThreads)
    mx = fmaxf(mx, wp[t]);
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) mx = fmaxf(mx, __shfl_xor(mx, h));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) cmax[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(kRnThreads) void rownorm_chunk_kernel(const float* __restrict__ w,
                                                                    const int32_t* __restrict__ perm_k, RnGeom g,
                                                                    int nchunk, const float* __restrict__ cmax,
                                                                    int64_t* __restrict__ cum,
                                                                    int64_t* __restrict__ chunk_sum) {
  __shared__ int64_t ssum[kRnThreads];
  __shared__ int sh_s;
  const int64_t prob = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  if (threadIdx.x < 64) {                           // the problem's largest weight, its shift 40 - e
    float mx = 0.f;
    for (int c = threadIdx.x; c < nchunk; c += 64) mx = fmaxf(mx, cmax[prob * nchunk + c]);
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) mx = fmaxf(mx, __shfl_xor(mx, h));
    if (threadIdx.x == 0) {
      int e = 0;
      if (mx > 0.f) frexp(static_cast<double>(mx), &e);
      sh_s = mx > 0.f ? kRnQBits - e : -100000;     // no positive weight: every n_t = 0
    }
  }
  __syncthreads();
  const int sh = sh_s;
  const int n = g.seg;
  const float* wp = w + (prob / g.pieces) * g.n_head;   // perm_k holds rows of the head
  const int32_t* pk = perm_k + prob * n;
  int64_t* cp = cum + prob * n;
  constexpr int PER = kRnChunk / kRnThreads;
  const int t0 = chunk * kRnChunk + threadIdx.x * PER;
  int64_t v[PER];
  int64_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int t = t0 + i;
    const int ts = t < n ? t : n - 1;
    const double x = ldexp(static_cast<double>(wp[pk[ts]]), sh);
    v[i] = (t < n && sh > -100000) ? static_cast<int64_t>(floor(x)) : 0;
    local += v[i];
  }
  ssum[threadIdx.x] = local;
  __syncthreads();
  for (int off = 1; off < kRnThreads; off <<= 1) {
    const int64_t add = threadIdx.x >= off ? ssum[threadIdx.x - off] : 0;
    __syncthreads();
    ssum[threadIdx.x] += add;
    __syncthreads();
  }
  int64_t run = ssum[threadIdx.x] - local;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    run += v[i];
    if (t0 + i < n) cp[t0 + i] = run;
  }
  if (threadIdx.x == kRnThreads - 1) chunk_sum[blockIdx.x] = ssum[kRnThreads - 1];
}

__global__ __launch_bounds__(kRnThreads) void rownorm_offset_kernel(int n, int nchunk,
                                                                     const int64_t* __restrict__ chunk_sum,
                                                                     int64_t* __restrict__ cum) {
  const int64_t prob = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  if (chunk == 0) return;
  int64_t off = 0;
  for (int c = 0; c < chunk; ++c) off += chunk_sum[prob * nchunk + c];
  int64_t* cp = cum + prob * n;
  for (int t = chunk * kRnChunk + threadIdx.x; t < min((chunk + 1) * kRnChunk, n); t += kRnThreads) cp[t] += off;
}

// ---- draws ---------------------------------------------------------------------

__global__ void rownorm_sample_kernel(const int64_t* __restrict__ cum, int n, int pieces, int node_first,
                                      uint64_t seed, int heads, int kv_heads, int m, int64_t total_ctr,
                                      int32_t* __restrict__ out) {
  const int nctr = (m + 3) / 4;
  const int G = heads / kv_heads;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total_ctr;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t bhp = t / nctr;                   // (query head) * pieces + piece
    const int j = static_cast<int>(t % nctr);
    const int64_t bh = bhp / pieces;
    const int piece = static_cast<int>(bhp - bh * pieces);
    const int h = static_cast<int>(bh % heads);
    const int b = static_cast<int>(bh / heads);
    const int64_t* cp = cum + ((static_cast<int64_t>(b) * kv_heads + h / G) * pieces + piece) * n;
    const uint64_t T = static_cast<uint64_t>(cp[n - 1]);
    U32x4 c = {static_cast<uint32_t>(j), static_cast<uint32_t>(node_first + piece), static_cast<uint32_t>(h),
               static_cast<uint32_t>(2 * b + 2)};
    U32x4 r = philox4x32_10(c, seed);
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      const int i = 4 * j + wi;
      if (i >= m) break;
      const uint64_t x = philox_word(r, wi);
      // floor(x T / 2^32) exactly: T = Th 2^32 + Tl
      const uint64_t rr = x * (T >> 32) + ((x * (T & 0xFFFFFFFFull)) >> 32);
      int lo = 0, hi = n - 1;                       // smallest t with c_t > rr
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (static_cast<uint64_t>(cp[mid]) > rr) hi = mid;
        else lo = mid + 1;
      }
      out[bhp * m + i] = T > 0 ? lo : 0;
    }
  }
}

// ---- the sampled rows: K as is, V scaled by T / (m n_t) ----------------------------
// One copy per query head in sample order ([BH][m][d]), read by the second
// attention pass in place of the rows the sample positions name.

template <typename T>
__global__ void rownorm_sample_gather_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                             const int32_t* __restrict__ perm_k, const int64_t* __restrict__ cum,
                                             const int32_t* __restrict__ sidx, RnGeom g, int d, int m, int heads,
                                             int kv_heads, int64_t total, T* __restrict__ kc, T* __restrict__ vc) {
  const int G = heads / kv_heads;
  const int n = g.seg;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t sj = e / d;                       // ((query head) * pieces + piece) * m + sample
    const int c = static_cast<int>(e % d);
    const int64_t bhp = sj / m;
    const int64_t bh = bhp / g.pieces;
    const int piece = static_cast<int>(bhp - bh * g.pieces);
    const int h = static_cast<int>(bh % heads);
    const int64_t bkv = (bh / heads) * kv_heads + h / G;
    const int64_t prob = bkv * g.pieces + piece;
    const int t = sidx[sj];                         // sorted key position
    const int64_t* cp = cum + prob * n;
    const int64_t nt = cp[t] - (t > 0 ? cp[t - 1] : 0);
    const double scale = nt > 0 ? static_cast<double>(cp[n - 1]) / (static_cast<double>(m) * nt) : 0.0;
    const int64_t src = (bkv * g.n_head + perm_k[prob * n + t]) * d + c;
    kc[e] = k[src];
    vc[e] = static_cast<T>(static_cast<float>(v[src]) * static_cast<float>(scale));
  }
}

// ---- launches ------------------------------------------------------------------------

static unsigned grid_for(int64_t work, int per_block) {
  int64_t blocks = (work + per_block - 1) / per_block;
  if (blocks > 65536) blocks = 65536;
  return static_cast<unsigned>(blocks < 1 ? 1 : blocks);
}

int launch_rownorm_sqnorm(const void* v, int dtype, int64_t rows, int d, float* w, hipStream_t s) {
  if (rows == 0) return HA_OK;
  const int rpw = 64 / (d / 8);
  const unsigned g = grid_for(rows, 4 * rpw);
  if (dtype == HA_BF16) {
    if (d == 64) hipLaunchKernelGGL((rownorm_sqnorm_kernel<bf16, 64>), dim3(g), dim3(256), 0, s, static_cast<const bf16*>(v), rows, w);
    else hipLaunchKernelGGL((rownorm_sqnorm_kernel<bf16, 128>), dim3(g), dim3(256), 0, s, static_cast<const bf16*>(v), rows, w);
  } else {
    if (d == 64) hipLaunchKernelGGL((rownorm_sqnorm_kernel<float, 64>), dim3(g), dim3(256), 0, s, static_cast<const float*>(v), rows, w);
    else hipLaunchKernelGGL((rownorm_sqnorm_kernel<float, 128>), dim3(g), dim3(256), 0, s, static_cast<const float*>(v), rows, w);
  }
  return after_launch("row-norm squared norms", s);
}

size_t rownorm_cdf_ws_bytes(int64_t problems, int n) {
  const int64_t nchunk = (n + kRnChunk - 1) / kRnChunk;
  return static_cast<size_t>(problems) * nchunk * (sizeof(int64_t) + sizeof(float)) + 64;
}

int launch_rownorm_cdf(const float* w, const int32_t* perm_k, int64_t kv_problems, const RnGeom& g, int64_t* cum,
                       void* ws, hipStream_t s) {
  const int64_t problems = kv_problems * g.pieces;
  if (problems == 0 || g.seg == 0) return HA_OK;
  const int nchunk = (g.seg + kRnChunk - 1) / kRnChunk;
  int64_t* chunk_sum = static_cast<int64_t*>(ws);
  float* cmax = reinterpret_cast<float*>(chunk_sum + problems * nchunk);
  const unsigned grid = static_cast<unsigned>(problems * nchunk);
  hipLaunchKernelGGL(rownorm_max_kernel, dim3(grid), dim3(kRnThreads), 0, s, w, g, nchunk, cmax);
  hipLaunchKernelGGL(rownorm_chunk_kernel, dim3(grid), dim3(kRnThreads), 0, s, w, perm_k, g, nchunk, cmax, cum,
                     chunk_sum);
  hipLaunchKernelGGL(rownorm_offset_kernel, dim3(grid), dim3(kRnThreads), 0, s, g.seg, nchunk, chunk_sum, cum);
  return after_launch("row-norm cdf", s);
}

int launch_rownorm_samples(const int64_t* cum, const RnGeom& g, int node_first, uint64_t seed, int batch,
                           int heads, int kv_heads, int m, int32_t* out, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(batch) * heads * g.pieces * ((m + 3) / 4);
  if (total == 0 || g.seg == 0) return HA_OK;
  hipLaunchKernelGGL(rownorm_sample_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, cum, g.seg, g.pieces,
                     node_first, seed, heads, kv_heads, m, total, out);
  return after_launch("row-norm samples", s);
}

int launch_rownorm_sample_gather(const void* k, const void* v, int dtype, const int32_t* perm_k,
                                 const int64_t* cum, const int32_t* sidx, const RnGeom& g, int batch, int heads,
                                 int kv_heads, int d, int m, void* kc, void* vc, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(batch) * heads * g.pieces * m * d;
  if (total == 0 || g.seg == 0) return HA_OK;
  const unsigned grid = grid_for(total, 256);
  if (dtype == HA_BF16)
    hipLaunchKernelGGL(rownorm_sample_gather_kernel<bf16>, dim3(grid), dim3(256), 0, s, static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), perm_k, cum, sidx, g, d, m, heads, kv_heads, total,
                       static_cast<bf16*>(kc), static_cast<bf16*>(vc));
  else
    hipLaunchKernelGGL(rownorm_sample_gather_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(k),
                       static_cast<const float*>(v), perm_k, cum, sidx, g, d, m, heads, kv_heads, total,
                       static_cast<float*>(kc), static_cast<float*>(vc));
  return after_launch("row-norm sampled rows", s);
}

}  // namespace ha
