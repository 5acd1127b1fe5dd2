// Projection matrix and sortLSH hash kernels.
//
// Hash ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: Hamming-sorted LSH finds the
// large entries).  Each row x gets the code sum_p [<x, R_p> > 0] 2^p and
// the rank = position of that code in the reflected-binary Gray sequence,
// so that consecutive buckets differ in one hash bit.
//
// The fp32 dot products follow one fixed order so that ranks are exact
// and reproducible: the d products are cut into groups of 8 consecutive
// elements, each group is summed by halving (pairs 4, 2, 1 apart), and the
// d/8 group sums are combined by halving as well (pairs d/16, ..., 1
// apart).  No multiply-add contraction.
//
// HBM traffic: each input row is read once (d * elem bytes) and 2 bytes
// of rank are written.
#include "ha_kernels.h"
#include "ha_rng.h"

namespace ha {

__global__ void proj_kernel(uint64_t seed, int total, float* __restrict__ R) {
  const int pairs = (total + 1) / 2;
  for (int pi = blockIdx.x * blockDim.x + threadIdx.x; pi < pairs; pi += gridDim.x * blockDim.x) {
    float z0, z1;
    gauss_pair(seed, static_cast<uint32_t>(pi), &z0, &z1);
    R[2 * pi] = z0;
    if (2 * pi + 1 < total) R[2 * pi + 1] = z1;
  }
}

int launch_projections(uint64_t seed, int d, int r, float* R, hipStream_t s) {
  const int total = d * r;
  const int blocks = (total / 2 + 255) / 256;
  timing_begin(HA_K_PROJ, s);
  hipLaunchKernelGGL(proj_kernel, dim3(blocks < 1 ? 1 : blocks), dim3(256), 0, s, seed, total, R);
  timing_end(HA_K_PROJ, s);
  return after_launch("projections", s);
}

__device__ __forceinline__ uint32_t gray_inverse(uint32_t x) {
  x ^= x >> 1;
  x ^= x >> 2;
  x ^= x >> 4;
  x ^= x >> 8;
  return x;
}

// Halving sum of v[0 .. N): pairs N/2 apart, then N/4 apart, ... (the fixed
// order of the group sums).
template <int N>
__device__ __forceinline__ float halving_sum(const float* v) {
#pragma clang fp contract(off)
  if constexpr (N == 1) {
    return v[0];
  } else {
    float h[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) h[i] = v[i] + v[i + N / 2];
    return halving_sum<N / 2>(h);
  }
}

// One row per lane.  A workgroup of 4 waves takes 256 consecutive rows per
// step: the rows are read with coalesced 16-byte loads into LDS (padded
// rows, conflict-free), then each lane walks its own row group by group.
// The projection values are uniform across lanes and come from scalar
// loads.  Per row: d r products and the adds of the two halving levels.
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void hash_kernel(const T* __restrict__ x, int64_t rows,
                                                   const float* __restrict__ Rm,
                                                   uint16_t* __restrict__ rank) {
#pragma clang fp contract(off)
  constexpr int G = D / 8;                          // groups of 8 elements
  constexpr int ROWB = D * static_cast<int>(sizeof(T));
  constexpr int CH = ROWB / 16;                     // 16-byte chunks per row
  constexpr int STR = ROWB + 16;                    // LDS row stride (bytes)
  constexpr int TR = 256;                           // rows per workgroup step
  __shared__ __attribute__((aligned(16))) char stage[TR * STR];
  const int tid = threadIdx.x;
  const char* xb = reinterpret_cast<const char*>(x);

  for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * TR; r0 < rows; r0 += static_cast<int64_t>(gridDim.x) * TR) {
    const int nr = rows - r0 < TR ? static_cast<int>(rows - r0) : TR;
    // coalesced staging: chunk q of the step = row q / CH, chunk q % CH
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int q = c * TR + tid;
      const int rr = q / CH, cc = q % CH;
      uint4v w = {0u, 0u, 0u, 0u};
      if (rr < nr) w = *reinterpret_cast<const uint4v*>(xb + (r0 + rr) * ROWB + 16 * cc);
      *reinterpret_cast<uint4v*>(stage + rr * STR + 16 * cc) = w;
    }
    __syncthreads();

    const char* row = stage + tid * STR;
    float xv[D];                                     // this lane's row in fp32
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (sizeof(T) == 2) {
        const uint4v w = *reinterpret_cast<const uint4v*>(row + 16 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[8 * g + 2 * i] = __uint_as_float(w[i] << 16);
          xv[8 * g + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
      } else {
        const floatx4 a = *reinterpret_cast<const floatx4*>(row + 32 * g);
        const floatx4 b = *reinterpret_cast<const floatx4*>(row + 32 * g + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[8 * g + i] = a[i];
          xv[8 * g + 4 + i] = b[i];
        }
      }
    }
    // one projection at a time (its d values sit in scalar registers)
    uint32_t code = 0;
#pragma unroll 1
    for (int p = 0; p < R; ++p) {
      const float* rp = Rm + p * D;
      float gsum[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = xv[8 * g + i] * rp[8 * g + i];
        gsum[g] = halving_sum<8>(pr);
      }
      code |= (halving_sum<G>(gsum) > 0.f ? 1u : 0u) << p;
    }
    if (tid < nr) rank[r0 + tid] = static_cast<uint16_t>(gray_inverse(code));
    __syncthreads();
  }
}

template <typename T, int D>
static int launch_hash_d(const T* x, int64_t rows, int r, const float* R, uint16_t* rank,
                         hipStream_t s) {
  int64_t blocks = (rows + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  dim3 g(static_cast<unsigned>(blocks)), b(256);
  switch (r) {
#define HA_HASH_CASE(RR) \
    case RR: hipLaunchKernelGGL((hash_kernel<T, D, RR>), g, b, 0, s, x, rows, R, rank); break;
    HA_HASH_CASE(1) HA_HASH_CASE(2) HA_HASH_CASE(3) HA_HASH_CASE(4)
    HA_HASH_CASE(5) HA_HASH_CASE(6) HA_HASH_CASE(7) HA_HASH_CASE(8)
    HA_HASH_CASE(9) HA_HASH_CASE(10) HA_HASH_CASE(11) HA_HASH_CASE(12)
    HA_HASH_CASE(13) HA_HASH_CASE(14) HA_HASH_CASE(15) HA_HASH_CASE(16)
#undef HA_HASH_CASE
    default:
      set_error("hash: proj_bits %d outside [1, 16]", r);
      return HA_EINVAL;
  }
  return HA_OK;
}

int launch_hash(const void* x, int dtype, int64_t rows, int d, int r, const float* R,
                uint16_t* rank, hipStream_t s) {
  if (rows == 0) return HA_OK;
  int st;
  timing_begin(HA_K_HASH, s);
  if (dtype == HA_BF16) {
    st = d == 64 ? launch_hash_d<bf16, 64>(static_cast<const bf16*>(x), rows, r, R, rank, s)
                 : launch_hash_d<bf16, 128>(static_cast<const bf16*>(x), rows, r, R, rank, s);
  } else {
    st = d == 64 ? launch_hash_d<float, 64>(static_cast<const float*>(x), rows, r, R, rank, s)
                 : launch_hash_d<float, 128>(static_cast<const float*>(x), rows, r, R, rank, s);
  }
  timing_end(HA_K_HASH, s);
  if (st != HA_OK) return st;
  return after_launch("hash", s);
}

}  // namespace ha
