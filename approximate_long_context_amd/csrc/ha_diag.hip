// The method's fine-grained parameters as diagnostics.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary: sections Approach and Limitations -- alpha, the
// largest squared column norm of the softmax matrix D^-1 A, and the ratio
// of row norms of A after the large entries are removed; section
// Surprising findings -- alpha taken without the first 32 columns for
// chatglm2.)
//
//   colmass_kernel:  c_j = sum_i P_ij^2 = sum_i exp(2 (q_i . k_j - lse_i))
//                    for every key column of every query head (exact lse
//                    of the full softmax given; causal: i >= j), key-owned
//                    like the dK/dV pass: a lane owns one key column,
//                    query tiles stream through LDS, S = Q K^T by MFMA;
//   alpha_kernel:    alpha = max_{j >= skip} c_j per query head;
//   kappa_kernel:    r_i = exp(lse_exact_i) (1 - exp(lse_block_i -
//                    lse_exact_i)), the row sum of A outside the row's
//                    block, and kappa = max_i r_i / min_i r_i per head (fp64).
#include <cmath>

#include "ha_device.h"
#include "ha_kernels.h"

namespace ha {

constexpr int kDgT = 64;         // query rows per LDS tile
constexpr int kDgW = 8;          // waves per workgroup (32 keys each)
constexpr int kDgNT = 64 * kDgW;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDgNT, 4) void colmass_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                           const float* __restrict__ lse, int n, int H, int Hkv,
                                                           float* __restrict__ colmass) {
  constexpr int STR = D + 8;                       // LDS row stride (bf16)
  constexpr int NQF = D / 16;
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int CPT = kDgT * CPR / kDgNT;          // chunks per thread per tile
  constexpr int JSTEP = kDgNT / CPR;
  constexpr int TB = kDgT * STR * 2 + kDgT * 4;    // Q tile + lse log2 e
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h2 = lane >> 5;
  const int col = lane & 31;

  const int KT = (n + 32 * kDgW - 1) / (32 * kDgW);
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / KT;
  const int k0 = (lid % KT) * 32 * kDgW;
  const int bkv = (bh / H) * Hkv + (bh % H) / (H / Hkv);
  const bf16* qb = q + static_cast<int64_t>(bh) * n * D;
  const bf16* kb = k + static_cast<int64_t>(bkv) * n * D;
  const float* lb = lse + static_cast<int64_t>(bh) * n;

  const int kj = k0 + wave * 32 + col;
  const int kjs = kj < n ? kj : n - 1;
  bf16x8 kf[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c)
    kf[c] = __builtin_bit_cast(bf16x8, ld16(kb, static_cast<uint32_t>(kjs * D + 16 * c + 8 * h2) * 2));

  const int qa0 = CAUSAL ? k0 : 0;
  const int ntiles = (n - qa0 + kDgT - 1) / kDgT;
  const int c_in_row = tid % CPR;
  const int j_first = tid / CPR;
  uint4v qreg[CPT];
  float lreg = 0.f;
  auto load_tile = [&](int it) {
    const int tq0 = qa0 + it * kDgT;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int row = min(tq0 + j_first + c * JSTEP, n - 1);
      qreg[c] = ld16(qb, static_cast<uint32_t>(row * D + 8 * c_in_row) * 2);
    }
    lreg = lb[min(tq0 + (tid & (kDgT - 1)), n - 1)];
  };
  auto store_tile = [&](int buf, int it) {
    bf16* qs = reinterpret_cast<bf16*>(smem + buf * TB);
    float* ls = reinterpret_cast<float*>(smem + buf * TB + kDgT * STR * 2);
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      *reinterpret_cast<uint4v*>(&qs[(j_first + c * JSTEP) * STR + 8 * c_in_row]) = qreg[c];
    if (tid < kDgT) ls[tid] = qa0 + it * kDgT + tid < n ? lreg * (2.f * kLog2e) : INFINITY;
  };

  float acc = 0.f;
  if (ntiles > 0) load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    store_tile(buf, it);
    __syncthreads();
    if (it + 1 < ntiles) load_tile(it + 1);
    const int tq0 = qa0 + it * kDgT;
    const bf16* qs = reinterpret_cast<const bf16*>(smem + buf * TB);
    const float* ls = reinterpret_cast<const float*>(smem + buf * TB + kDgT * STR * 2);
    const int lim = kj - tq0;                      // causal: query j of the tile counts iff j >= lim
#pragma unroll
    for (int qt = 0; qt < kDgT / 32; ++qt) {
      floatx16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int c = 0; c < NQF; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&qs[(32 * qt + col) * STR + 16 * c + 8 * h2]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[c], s, 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = 32 * qt + 8 * g + 4 * h2;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(ls + j0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = fmaf(s[4 * g + i], 2.f * kLog2e, -l4[i]);
          if constexpr (CAUSAL) x = j0 + i >= lim ? x : -INFINITY;
          acc += fast_exp2(x);
        }
      }
    }
  }
  acc += __shfl_xor(acc, 32);
  if (h2 == 0 && kj < n) colmass[static_cast<int64_t>(bh) * n + kj] = acc;
}

__global__ __launch_bounds__(256) void alpha_kernel(const float* __restrict__ colmass, int n, int skip,
                                                    float* __restrict__ alpha) {
  __shared__ float red[4];
  const float* c = colmass + static_cast<int64_t>(blockIdx.x) * n;
  float mx = -INFINITY;
  for (int j = skip + static_cast<int>(threadIdx.x); j < n; j += 256) mx = fmaxf(mx, c[j]);
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) mx = fmaxf(mx, __shfl_xor(mx, h));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) alpha[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void kappa_kernel(const float* __restrict__ lse_exact,
                                                    const float* __restrict__ lse_block,
                                                    const int32_t* __restrict__ perm_q, int n,
                                                    float* __restrict__ kappa) {
  __shared__ double rmax[4], rmin[4];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * n;
  double mx = 0.0, mn = INFINITY;
  for (int t = threadIdx.x; t < n; t += 256) {
    const double le = lse_exact[base + perm_q[base + t]];
    const double lbk = lse_block[base + t];
    const double r = exp(le) * -expm1(lbk - le);   // exact row sum minus the block's
    mx = fmax(mx, r);
    mn = fmin(mn, r);
  }
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    mx = fmax(mx, __shfl_xor(mx, h));
    mn = fmin(mn, __shfl_xor(mn, h));
  }
  if ((threadIdx.x & 63) == 0) {
    rmax[threadIdx.x >> 6] = mx;
    rmin[threadIdx.x >> 6] = mn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double a = fmax(fmax(rmax[0], rmax[1]), fmax(rmax[2], rmax[3]));
    const double b = fmin(fmin(rmin[0], rmin[1]), fmin(rmin[2], rmin[3]));
    kappa[blockIdx.x] = b > 0.0 ? static_cast<float>(a / b) : INFINITY;
  }
}

int launch_colmass(const void* q, const void* k, const float* lse, int batch, int n, int d, int heads,
                   int kv_heads, int causal, int skip, float* colmass, float* alpha, hipStream_t s) {
  const int64_t BH = static_cast<int64_t>(batch) * heads;
  if (BH == 0 || n == 0) return HA_OK;
  const int KT = (n + 32 * kDgW - 1) / (32 * kDgW);
  const dim3 grid(static_cast<unsigned>(BH * KT));
  const size_t lds = 2 * static_cast<size_t>(kDgT * (d + 8) * 2 + kDgT * 4);
  const bf16* qq = static_cast<const bf16*>(q);
  const bf16* kk = static_cast<const bf16*>(k);
  if (d == 64) {
    if (causal) hipLaunchKernelGGL((colmass_kernel<64, true>), grid, dim3(kDgNT), lds, s, qq, kk, lse, n, heads, kv_heads, colmass);
    else hipLaunchKernelGGL((colmass_kernel<64, false>), grid, dim3(kDgNT), lds, s, qq, kk, lse, n, heads, kv_heads, colmass);
  } else {
    if (causal) hipLaunchKernelGGL((colmass_kernel<128, true>), grid, dim3(kDgNT), lds, s, qq, kk, lse, n, heads, kv_heads, colmass);
    else hipLaunchKernelGGL((colmass_kernel<128, false>), grid, dim3(kDgNT), lds, s, qq, kk, lse, n, heads, kv_heads, colmass);
  }
  HA_TRY(after_launch("column squared mass", s));
  if (alpha) {
    hipLaunchKernelGGL(alpha_kernel, dim3(static_cast<unsigned>(BH)), dim3(256), 0, s, colmass, n, skip, alpha);
    return after_launch("alpha", s);
  }
  return HA_OK;
}

int launch_kappa(const float* lse_exact, const float* lse_block, const int32_t* perm_q, int64_t problems, int n,
                 float* kappa, hipStream_t s) {
  if (problems == 0 || n == 0) return HA_OK;
  hipLaunchKernelGGL(kappa_kernel, dim3(static_cast<unsigned>(problems)), dim3(256), 0, s, lse_exact, lse_block,
                     perm_q, n, kappa);
  return after_launch("residual row-sum ratio", s);
}

}  // namespace ha
