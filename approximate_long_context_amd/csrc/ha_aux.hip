// Auxiliary kernels of the HyperAttention forward: sample positions,
// permutation gather, and the log-sum-exp merge with unsort.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: uniform column sampling for the
// normaliser; queries and keys re-ordered by bucket.)
#include <cmath>

#include "ha_kernels.h"
#include "ha_rng.h"

namespace ha {

// ---- sample positions ---------------------------------------------------------

__global__ void sample_idx_kernel(uint64_t seed, int heads, int node_first, int node_count,
                                  uint32_t ns, int m, int64_t total_ctr, int32_t* __restrict__ out) {
  const int nctr = (m + 3) / 4;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total_ctr;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t prob = t / nctr;
    const int j = static_cast<int>(t % nctr);
    const int node = node_first + static_cast<int>(prob % node_count);
    const int h = static_cast<int>((prob / node_count) % heads);
    const int b = static_cast<int>(prob / (static_cast<int64_t>(node_count) * heads));
    U32x4 c = {static_cast<uint32_t>(j), static_cast<uint32_t>(node), static_cast<uint32_t>(h),
               static_cast<uint32_t>(2 * b + 1)};
    U32x4 r = philox4x32_10(c, seed);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = 4 * j + w;
      if (i < m) out[prob * m + i] = sample_position(philox_word(r, w), ns);
    }
  }
}

int launch_sample_indices(uint64_t seed, int batch, int heads, int node_first, int node_count,
                          int ns, int m, int32_t* out, hipStream_t s) {
  if (m == 0 || batch == 0 || heads == 0 || node_count == 0) return HA_OK;
  const int64_t total = static_cast<int64_t>(batch) * heads * node_count * ((m + 3) / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  HA_TRY(launch_gate(HA_K_SAMPLES));
  timing_begin(HA_K_SAMPLES, s);
  hipLaunchKernelGGL(sample_idx_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, seed,
                     heads, node_first, node_count, static_cast<uint32_t>(ns), m, total, out);
  timing_end(HA_K_SAMPLES, s);
  return after_launch("sample indices", s);
}

// ---- permutation gather -----------------------------------------------------

__global__ void gather_kernel(const uint4v* __restrict__ src, int n, int cpr, const int32_t* __restrict__ perm,
                              int rows_per_head, int64_t total, uint4v* __restrict__ dst) {
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t rowg = t / cpr;          // destination row (head-major)
    const int c = static_cast<int>(t % cpr);
    const int64_t hd = rowg / rows_per_head;
    const int32_t srow = perm[rowg];
    dst[t] = src[(hd * n + srow) * cpr + c];
  }
}

int launch_gather(const void* src, int dtype, int64_t heads, int n, int d, const int32_t* perm,
                  int rows_per_head, void* dst, hipStream_t s) {
  const int cpr = d * (dtype == HA_BF16 ? 2 : 4) / 16;
  const int64_t total = heads * rows_per_head * cpr;
  if (total == 0) return HA_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  HA_TRY(launch_gate(HA_K_GATHER));
  timing_begin(HA_K_GATHER, s);
  hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint4v*>(src), n, cpr, perm, rows_per_head, total,
                     static_cast<uint4v*>(dst));
  timing_end(HA_K_GATHER, s);
  return after_launch("gather", s);
}

// ---- strided row copy (debug dumps of permutations and sample positions) -----

__global__ void copy_rows_i32_kernel(const int32_t* __restrict__ src, int64_t spitch, int32_t* __restrict__ dst,
                                     int64_t dpitch, int width, int64_t total) {
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = t / width;
    const int c = static_cast<int>(t % width);
    dst[r * dpitch + c] = src[r * spitch + c];
  }
}

int launch_copy_rows_i32(const int32_t* src, int64_t spitch, int32_t* dst, int64_t dpitch, int width, int64_t rows,
                         hipStream_t s) {
  const int64_t total = rows * width;
  if (total == 0) return HA_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_rows_i32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src, spitch, dst,
                     dpitch, width, total);
  return after_launch("row copy", s);
}

// ---- log-sum-exp merge + unsort ---------------------------------------------

template <typename T>
__global__ void merge_unsort_kernel(const float* __restrict__ o1, const float* __restrict__ l1,
                                    const float* __restrict__ o2, const float* __restrict__ l2,
                                    const int32_t* __restrict__ perm, int n, int d, int64_t total,
                                    T* __restrict__ out, float* __restrict__ lse) {
  const int cpr = d / 4;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t rp = t / cpr;            // head * n + sorted position
    const int c = static_cast<int>(t % cpr);
    const int64_t hd = rp / n;
    const float a = l1[rp], bb = l2[rp];
    const float mm = fmaxf(a, bb);
    float L, wa, wb;
    if (mm == -INFINITY) {
      L = -INFINITY;
      wa = 0.f;
      wb = 0.f;
    } else {
      L = mm + logf(expf(a - mm) + expf(bb - mm));
      wa = expf(a - L);
      wb = expf(bb - L);
    }
    const floatx4 x = reinterpret_cast<const floatx4*>(o1)[t];
    const floatx4 y = reinterpret_cast<const floatx4*>(o2)[t];
    const int64_t orow = hd * n + perm[rp];
    T* dst = out + orow * d + 4 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = static_cast<T>(x[i] * wa + y[i] * wb);
    if (c == 0 && lse) lse[orow] = L;
  }
}

int launch_merge_unsort(const float* o1, const float* l1, const float* o2, const float* l2,
                        const int32_t* perm, int64_t heads, int n, int d, int dtype, void* out,
                        float* lse, hipStream_t s) {
  const int64_t total = heads * n * (d / 4);
  if (total == 0) return HA_OK;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  HA_TRY(launch_gate(HA_K_MERGE));
  timing_begin(HA_K_MERGE, s);
  if (dtype == HA_BF16)
    hipLaunchKernelGGL(merge_unsort_kernel<bf16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       o1, l1, o2, l2, perm, n, d, total, static_cast<bf16*>(out), lse);
  else
    hipLaunchKernelGGL(merge_unsort_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       o1, l1, o2, l2, perm, n, d, total, static_cast<float*>(out), lse);
  timing_end(HA_K_MERGE, s);
  return after_launch("merge+unsort", s);
}

}  // namespace ha
