// Random draws of the method, identical on host and device.
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds of
//   (c0,c1,c2,c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
// with the key advanced by the Weyl constants between rounds.
//
// The sortLSH hash ("HyperAttention: Long-context Attention in Near-Linear
// Time", research-map summary, section Approach: Hamming-sorted LSH) is
// read here as random-hyperplane hashing with Gaussian directions.  The
// Gaussians come from Box-Muller on Philox words, with every
// transcendental step written as a fixed sequence of IEEE fp64 add, mul
// and div (contraction off) plus exact frexp/ldexp scaling, so that the
// device kernel and the host export produce the same fp32 matrix bit for
// bit:
//   ln f     : 2 s (1 + s^2/3 + ... + s^20/21),  s = (f-1)/(f+1),
//              f in (sqrt2/2, sqrt2] by exact power-of-two reduction;
//   sin, cos : Taylor to a^19 / a^20 on a in [-pi/4, pi/4] after an exact
//              quarter-turn reduction of the 33-bit odd numerator;
//   sqrt     : six Newton steps from 0.41731 + 0.59016 f, f in [1/4, 1).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace ha {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct U32x4 {
  uint32_t x, y, z, w;
};

__host__ __device__ inline U32x4 philox4x32_10(U32x4 c, uint64_t seed) {
  uint32_t k0 = static_cast<uint32_t>(seed);
  uint32_t k1 = static_cast<uint32_t>(seed >> 32);
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    uint64_t p0 = static_cast<uint64_t>(kPhiloxM0) * c.x;
    uint64_t p1 = static_cast<uint64_t>(kPhiloxM1) * c.z;
    U32x4 n;
    n.x = static_cast<uint32_t>(p1 >> 32) ^ c.y ^ k0;
    n.y = static_cast<uint32_t>(p1);
    n.z = static_cast<uint32_t>(p0 >> 32) ^ c.w ^ k1;
    n.w = static_cast<uint32_t>(p0);
    c = n;
  }
  return c;
}

__host__ __device__ inline uint32_t philox_word(const U32x4& r, int i) {
  return i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w;
}

__host__ __device__ inline int bit_length_u64(uint64_t y) {
#if defined(__HIP_DEVICE_COMPILE__)
  return 64 - __clzll(static_cast<long long>(y));
#else
  return 64 - __builtin_clzll(y);
#endif
}

// -2 ln u, u = (x + 1/2) / 2^32.
__host__ __device__ inline double gauss_neg2_log_u(uint32_t x) {
#pragma clang fp contract(off)
  const double kLn2 = 0.6931471805599453;
  const double kSqrt2 = 1.4142135623730951;
  uint64_t y = 2ull * x + 1ull;                  // u = y / 2^33
  int e = bit_length_u64(y) - 1;
  double f = ldexp(static_cast<double>(y), -e);  // [1, 2), exact
  if (f > kSqrt2) {
    f = f * 0.5;
    e = e + 1;
  }
  double s = (f - 1.0) / (f + 1.0);
  double z = s * s;
  double acc = 1.0 / 21.0;
  acc = acc * z + 1.0 / 19.0;
  acc = acc * z + 1.0 / 17.0;
  acc = acc * z + 1.0 / 15.0;
  acc = acc * z + 1.0 / 13.0;
  acc = acc * z + 1.0 / 11.0;
  acc = acc * z + 1.0 / 9.0;
  acc = acc * z + 1.0 / 7.0;
  acc = acc * z + 1.0 / 5.0;
  acc = acc * z + 1.0 / 3.0;
  acc = acc * z + 1.0;
  double ln_f = 2.0 * (s * acc);
  double ln_u = ln_f + static_cast<double>(e - 33) * kLn2;
  return -2.0 * ln_u;
}

// (cos, sin) of 2 pi u, u = (x + 1/2) / 2^32.
__host__ __device__ inline void gauss_sincos_2pi(uint32_t x, double* c_out, double* s_out) {
#pragma clang fp contract(off)
  const double kHalfPi = 1.5707963267948966;
  int64_t y = 2ll * x + 1ll;                     // 4u = y / 2^31
  int q = static_cast<int>(y >> 31);
  int64_t rem = y & ((1ll << 31) - 1);
  if (rem >= (1ll << 30)) {
    rem = rem - (1ll << 31);
    q = q + 1;
  }
  double w = ldexp(static_cast<double>(rem), -31);   // [-1/2, 1/2), exact
  double a = w * kHalfPi;
  double a2 = a * a;
  double sacc = -1.0 / 121645100408832000.0;         // -1/19!
  sacc = sacc * a2 + 1.0 / 355687428096000.0;        // 1/17!
  sacc = sacc * a2 + -1.0 / 1307674368000.0;         // -1/15!
  sacc = sacc * a2 + 1.0 / 6227020800.0;             // 1/13!
  sacc = sacc * a2 + -1.0 / 39916800.0;              // -1/11!
  sacc = sacc * a2 + 1.0 / 362880.0;                 // 1/9!
  sacc = sacc * a2 + -1.0 / 5040.0;                  // -1/7!
  sacc = sacc * a2 + 1.0 / 120.0;                    // 1/5!
  sacc = sacc * a2 + -1.0 / 6.0;                     // -1/3!
  sacc = sacc * a2 + 1.0;
  double sin_a = a * sacc;
  double cacc = 1.0 / 2432902008176640000.0;         // 1/20!
  cacc = cacc * a2 + -1.0 / 6402373705728000.0;      // -1/18!
  cacc = cacc * a2 + 1.0 / 20922789888000.0;         // 1/16!
  cacc = cacc * a2 + -1.0 / 87178291200.0;           // -1/14!
  cacc = cacc * a2 + 1.0 / 479001600.0;              // 1/12!
  cacc = cacc * a2 + -1.0 / 3628800.0;               // -1/10!
  cacc = cacc * a2 + 1.0 / 40320.0;                  // 1/8!
  cacc = cacc * a2 + -1.0 / 720.0;                   // -1/6!
  cacc = cacc * a2 + 1.0 / 24.0;                     // 1/4!
  cacc = cacc * a2 + -1.0 / 2.0;                     // -1/2!
  cacc = cacc * a2 + 1.0;
  double cos_a = cacc;
  switch (q & 3) {
    case 0: *c_out = cos_a;  *s_out = sin_a;  break;
    case 1: *c_out = -sin_a; *s_out = cos_a;  break;
    case 2: *c_out = -cos_a; *s_out = -sin_a; break;
    default: *c_out = sin_a; *s_out = -cos_a; break;
  }
}

__host__ __device__ inline double gauss_sqrt(double v) {
#pragma clang fp contract(off)
  int e;
  double f = frexp(v, &e);
  if (e & 1) {
    f = f * 0.5;
    e = e + 1;
  }
  double y = 0.41731 + 0.59016 * f;
  for (int i = 0; i < 6; ++i) y = 0.5 * (y + f / y);
  return ldexp(y, e / 2);
}

// Element e of the projection matrix (e = p*d + k): counter (e/4, 0, 0, 0);
// words (w0, w1) feed elements 4j, 4j+1 and (w2, w3) feed 4j+2, 4j+3.
__host__ __device__ inline void gauss_pair(uint64_t seed, uint32_t pair, float* z0, float* z1) {
#pragma clang fp contract(off)
  U32x4 c = {pair >> 1, 0u, 0u, 0u};
  U32x4 r = philox4x32_10(c, seed);
  uint32_t wa = (pair & 1) ? r.z : r.x;
  uint32_t wb = (pair & 1) ? r.w : r.y;
  double rho = gauss_sqrt(gauss_neg2_log_u(wa));
  double cs, sn;
  gauss_sincos_2pi(wb, &cs, &sn);
  *z0 = static_cast<float>(rho * cs);
  *z1 = static_cast<float>(rho * sn);
}

// Sample position i of problem (batch b, query head h, recursion node):
// word i of counters (i/4, node, h, 2b+1), mapped to floor(w * ns / 2^32).
__host__ __device__ inline int32_t sample_position(uint32_t word, uint32_t ns) {
  return static_cast<int32_t>((static_cast<uint64_t>(word) * ns) >> 32);
}

}  // namespace ha
