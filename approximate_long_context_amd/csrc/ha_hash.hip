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
// elements; a lane owns one group (one 16-byte load of bf16), sums it by
// halving (pairs 4, 2, 1 apart), and the group sums are combined by an
// xor butterfly across the d/8 lanes of the row, which is the same
// halving order over the groups (fp32 addition is commutative).  No
// multiply-add contraction.
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

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x);

template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float* x) {
  uint4v w = *reinterpret_cast<const uint4v*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* x) {
  floatx4 a = *reinterpret_cast<const floatx4*>(p);
  floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

template <typename T, int D, int R>
__global__ __launch_bounds__(256) void hash_kernel(const T* __restrict__ x, int64_t rows,
                                                   const float* __restrict__ Rm,
                                                   uint16_t* __restrict__ rank) {
#pragma clang fp contract(off)
  constexpr int LPR = D / 8;      // lanes per row
  constexpr int RPW = 64 / LPR;   // rows per wave
  const int lane = threadIdx.x & 63;
  const int grp = lane % LPR;
  const int sub = lane / LPR;
  float rr[R][8];
#pragma unroll
  for (int p = 0; p < R; ++p)
#pragma unroll
    for (int i = 0; i < 8; ++i) rr[p][i] = Rm[p * D + 8 * grp + i];

  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  for (int64_t rb = wave * RPW; rb < rows; rb += nwaves * RPW) {
    const int64_t row = rb + sub;
    const bool valid = row < rows;
    float xv[8];
    if (valid) {
      load8<T>(x + row * D + 8 * grp, xv);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = 0.f;
    }
    uint32_t code = 0;
#pragma unroll
    for (int p = 0; p < R; ++p) {
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = xv[i] * rr[p][i];
      float s4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[i] = pr[i] + pr[i + 4];
      float s2a = s4[0] + s4[2];
      float s2b = s4[1] + s4[3];
      float t = s2a + s2b;
#pragma unroll
      for (int o = LPR / 2; o >= 1; o >>= 1) t = t + __shfl_xor(t, o);
      code |= (t > 0.f ? 1u : 0u) << p;
    }
    if (valid && grp == 0) rank[row] = static_cast<uint16_t>(gray_inverse(code));
  }
}

template <typename T, int D>
static int launch_hash_d(const T* x, int64_t rows, int r, const float* R, uint16_t* rank,
                         hipStream_t s) {
  constexpr int RPW = 64 / (D / 8);
  int64_t waves = (rows + RPW - 1) / RPW;
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 65536) blocks = 65536;
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
