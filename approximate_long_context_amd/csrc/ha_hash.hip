// Projection matrix and sortLSH hash kernels.
//
// Hash ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: Hamming-sorted LSH finds the
// large entries).  Each row x gets the code sum_p [<x, R_p> > 0] 2^p and
// the rank = position of that code in the reflected-binary Gray sequence,
// so that consecutive buckets differ in one hash bit.
//
// Bit p is the sign of the exact real dot product <x, R_p> (an exact zero,
// or a non-finite value in x or R_p, gives 0), so ranks do not depend on an
// evaluation order.  A lane computes t = sum_k x_k R_pk in fp32 with fused
// multiply-adds (four interleaved chains); its distance from the exact sum
// is at most gamma_{d+4} sum_k |x_k R_pk| + d 2^-150 (each step rounds once;
// the second term covers subnormal partial sums), and the sum of magnitudes
// is at most max_k |x_k| * sum_k |R_pk|.  When t is finite and |t| exceeds
// that bound (with margin) its sign is the exact sign.  Otherwise (a fraction of a percent of
// random rows) an fp64 pass with exact products decides unless |t| is below
// 2 d 2^-53 sum |x_k R_pk|, and what remains (exact cancellation) goes to an
// exact integer accumulator.
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
  HA_TRY(launch_gate(HA_K_PROJ));
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

// The exact sign bit of <x, R_p> for a row that the fp32 bound left open:
// fp64 with exact products first, then, for sums that cancel below the
// fp64 bound, exact integer arithmetic.  `row` is the row (d elements of
// T, in LDS or global memory), `rp` projection p.  Rare: its digit array
// lives in private memory and its loops stay rolled, so it costs the
// common path no registers.
template <typename T, int D>
__device__ __forceinline__ uint32_t exact_sign_bit(const T* row, const float* rp) {
  auto elem = [&](int k) -> float {
    if constexpr (sizeof(T) == 2) {
      return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, row[k])) << 16);
    } else {
      return row[k];
    }
  };
  double t = 0.0, s = 0.0;
#pragma unroll 1
  for (int k = 0; k < D; ++k) {
    const double pr = static_cast<double>(elem(k)) * static_cast<double>(rp[k]);   // exact
    t += pr;
    s += fabs(pr);
  }
  if (!(s <= 1e300)) return 0u;                  // a non-finite operand (products stay below 2^257)
  if (fabs(t) > 2.0 * D * 0x1p-53 * s) return t > 0.0 ? 1u : 0u;
  if (s == 0.0) return 0u;
  // exact: sum of m 2^e with m = mx mr < 2^48 and e >= -298, as signed
  // 32-bit digits (digit i weighs 2^(32 i - 298)) accumulated in int64
  constexpr int kLimbs = 19;
  int64_t limb[kLimbs];
#pragma unroll 1
  for (int i = 0; i < kLimbs; ++i) limb[i] = 0;
#pragma unroll 1
  for (int k = 0; k < D; ++k) {
    const uint32_t xb = __float_as_uint(elem(k)), rb = __float_as_uint(rp[k]);
    uint32_t ex = (xb >> 23) & 255u, er = (rb >> 23) & 255u;
    uint64_t mx = xb & 0x7FFFFFu, mr = rb & 0x7FFFFFu;
    if (ex) mx |= 0x800000u; else ex = 1;       // value = m 2^(e - 150)
    if (er) mr |= 0x800000u; else er = 1;
    const uint64_t m = mx * mr;
    if (m == 0) continue;
    const int sh = static_cast<int>(ex + er) - 300 + 298;
    const int q = sh >> 5, r = sh & 31;
    const uint64_t lo = (m & 0xFFFFFFFFull) << r, hi = (m >> 32) << r;
    int64_t d0 = static_cast<int64_t>(lo & 0xFFFFFFFFull);
    int64_t d1 = static_cast<int64_t>((lo >> 32) + (hi & 0xFFFFFFFFull));
    int64_t d2 = static_cast<int64_t>(hi >> 32);
    if ((xb ^ rb) >> 31) {
      d0 = -d0;
      d1 = -d1;
      d2 = -d2;
    }
    limb[q] += d0;
    limb[q + 1] += d1;
    limb[q + 2] += d2;
  }
  int64_t carry = 0;
  bool nonzero = false;
#pragma unroll 1
  for (int i = 0; i < kLimbs; ++i) {
    const int64_t v = limb[i] + carry;
    const int64_t low = v & 0xFFFFFFFFll;         // in [0, 2^32)
    carry = (v - low) >> 32;                       // exact: v - low is a multiple of 2^32
    nonzero |= low != 0;
  }
  return (carry > 0 || (carry == 0 && nonzero)) ? 1u : 0u;
}

// A workgroup takes 64 consecutive rows per step, one row per lane, with
// one wave per 128 bytes of row (NW = d * elem / 128 waves: 1 for bf16 at
// d = 64).  The rows are read with coalesced 16-byte loads into LDS (padded
// rows, conflict-free; a full step's chunk c of thread t is the 16 bytes at
// step base + 16 (c NT + t), so one uniform base serves every load); the
// next step's chunks are loaded into registers while this step computes.
// Wave w walks its 128-byte column slice of its lane's row one 16-byte
// chunk at a time (a rolled loop: few values live at once, so four waves
// fit per SIMD): the chunk's values in fp32, their largest magnitude, and
// for every projection fused multiply-adds into four chains (projection
// values are uniform and come from scalar loads).  Wave 0 adds the partials
// of the other waves (through LDS), tests the bounds, and only for the rare
// rows some bound leaves open runs the exact decision, in one rolled loop.
constexpr int kHashRows = 64;

template <typename T, int D, int R>
__global__ __launch_bounds__(D * sizeof(T) / 2) void hash_kernel(const T* __restrict__ x, int64_t rows,
                                                   const float* __restrict__ Rm,
                                                   uint16_t* __restrict__ rank) {
  constexpr int ROWB = D * static_cast<int>(sizeof(T));
  constexpr int NW = ROWB / 128;                    // waves per workgroup
  constexpr int NT = 64 * NW;
  constexpr int DW = D / NW;                        // elements per wave
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
  constexpr int CH = ROWB / 16;                     // 16-byte chunks per row
  constexpr int CPT = kHashRows * CH / NT;          // chunks per thread and step (8)
  constexpr int STR = ROWB + 16;                    // LDS row stride (bytes)
  constexpr int TR = kHashRows;
  static_assert(NW >= 1 && DW % EPC == 0 && CPT * NT == TR * CH && NT % CH == 0, "hash split");
  // |t - <x, R_p>| <= gamma_{D+4} max|x| sum|R_p| + D 2^-150 (see above);
  // the factor 1.0001 covers the rounding of the bound itself, and the
  // absolute term D 2^-148 also covers a bound that falls in the subnormals
  constexpr float kGam = 1.0001f * (D + 4) * 0x1p-24f / (1.f - (D + 4) * 0x1p-24f);
  constexpr float kAbs = D * 0x1p-148f;
  __shared__ __attribute__((aligned(16))) char stage[TR * STR];
  __shared__ float part[NW > 1 ? NW : 1][R + 1][64];   // per wave: partial sums and max|x| (NW > 1)
  __shared__ float rn1[R];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const char* xb = reinterpret_cast<const char*>(x);

  // sum_k |R_pk| per projection (lanes split k, a butterfly sums; wave 0
  // publishes it, read back after the first step's barrier)
  if (wave == 0) {
#pragma unroll
    for (int p = 0; p < R; ++p) {
      float a = 0.f;
#pragma unroll
      for (int k = lane; k < D; k += 64) a += fabsf(Rm[p * D + k]);
#pragma unroll
      for (int h = 32; h >= 1; h >>= 1) a += __shfl_xor(a, h);
      if (lane == 0) rn1[p] = a;
    }
  }

  // coalesced staging: chunk q = c NT + tid of a step is chunk q % CH of
  // row q / CH (NT is a multiple of CH, so the LDS slot of chunk c is
  // this thread's first slot + c (NT / CH) rows)
  const int64_t rstep = static_cast<int64_t>(gridDim.x) * TR;
  uint4v pre[CPT];
  auto load_step = [&](int64_t r0) {
    if (r0 + TR <= rows) {
      const char* base = xb + r0 * ROWB + 16 * tid;
#pragma unroll
      for (int c = 0; c < CPT; ++c) pre[c] = *reinterpret_cast<const uint4v*>(base + 16 * NT * c);
    } else {                                        // the last, partial step: rows past the end repeat the last row
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int q = c * NT + tid;
        const int64_t rr = min(r0 + q / CH, rows - 1);
        pre[c] = *reinterpret_cast<const uint4v*>(xb + rr * ROWB + 16 * (q % CH));
      }
    }
  };
  char* wslot = stage + (tid / CH) * STR + 16 * (tid % CH);
  if (static_cast<int64_t>(blockIdx.x) * TR < rows) load_step(static_cast<int64_t>(blockIdx.x) * TR);
  for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * TR; r0 < rows; r0 += rstep) {
    const int nr = rows - r0 < TR ? static_cast<int>(rows - r0) : TR;
#pragma unroll
    for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint4v*>(wslot + c * (NT / CH) * STR) = pre[c];
    __syncthreads();
    if (r0 + rstep < rows) load_step(r0 + rstep);

    const char* row = stage + lane * STR;
    const char* slice = row + wave * 128;
    float acc[R][4];
#pragma unroll
    for (int p = 0; p < R; ++p) acc[p][0] = acc[p][1] = acc[p][2] = acc[p][3] = 0.f;
    float xinf = 0.f;                                // max |x_k| (a NaN is skipped; t is then NaN)
#pragma unroll 1
    for (int g = 0; g < DW / EPC; ++g) {
      const uint4v w = *reinterpret_cast<const uint4v*>(slice + 16 * g);
      float xv[EPC];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(T) == 2) {
          xv[2 * i] = __uint_as_float(w[i] << 16);
          xv[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        } else {
          xv[i] = __uint_as_float(w[i]);
        }
      }
#pragma unroll
      for (int k = 0; k < EPC; ++k) xinf = fmaxf(xinf, fabsf(xv[k]));
#pragma unroll
      for (int p = 0; p < R; ++p) {
        const float* rp = Rm + p * D + wave * DW + EPC * g;
#pragma unroll
        for (int k = 0; k < EPC; ++k) acc[p][k & 3] = fmaf(xv[k], rp[k], acc[p][k & 3]);
      }
    }
    // bits from the full sums (wave 0): settled ones directly, the open
    // ones (rare) by the exact decision
    auto decide_all = [&](const float* t) -> uint32_t {
      uint32_t code = 0, open = 0;
#pragma unroll
      for (int p = 0; p < R; ++p) {
        const float bound = fmaf(xinf * rn1[p], kGam, kAbs);
        // settled: beyond the bound and finite (a partial sum that overflowed
        // leaves t infinite or NaN)
        const float at = fabsf(t[p]);
        if (at > bound && at <= 0x1.fffffep127f) code |= (t[p] > 0.f ? 1u : 0u) << p;
        else open |= 1u << p;
      }
      if (open) {
#pragma unroll 1
        for (int p = 0; p < R; ++p)
          if ((open >> p) & 1u) code |= exact_sign_bit<T, D>(reinterpret_cast<const T*>(row), Rm + p * D) << p;
      }
      return code;
    };
    float t[R];
#pragma unroll
    for (int p = 0; p < R; ++p) t[p] = (acc[p][0] + acc[p][1]) + (acc[p][2] + acc[p][3]);
    uint32_t code = 0;
    if constexpr (NW == 1) {
      code = decide_all(t);
    } else {
#pragma unroll
      for (int p = 0; p < R; ++p) part[wave][p][lane] = t[p];
      part[wave][R][lane] = xinf;
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int w = 1; w < NW; ++w) xinf = fmaxf(xinf, part[w][R][lane]);
#pragma unroll
        for (int p = 0; p < R; ++p) {
#pragma unroll
          for (int w = 1; w < NW; ++w) t[p] += part[w][p][lane];
        }
        code = decide_all(t);
      }
    }
    if (wave == 0) {
      if (lane < nr) rank[r0 + lane] = static_cast<uint16_t>(gray_inverse(code));
    }
    __syncthreads();
  }
}

template <typename T, int D>
static int launch_hash_d(const T* x, int64_t rows, int r, const float* R, uint16_t* rank,
                         hipStream_t s) {
  constexpr int NT = 64 * (D * static_cast<int>(sizeof(T)) / 128);
  int64_t blocks = (rows + kHashRows - 1) / kHashRows;
  const int64_t cap = 256 * 4096 / NT;               // 64 waves per CU, then a grid-stride loop
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  dim3 g(static_cast<unsigned>(blocks)), b(NT);
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
  HA_TRY(launch_gate(HA_K_HASH));
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
