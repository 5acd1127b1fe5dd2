// Backward of the HyperAttention forward for fp32 inputs, on gfx950.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Key results: the method is timed forward
// and backward; section Approach for the forward it differentiates.)
//
// The same weighted-softmax backward as the bf16 kernels -- for fixed ranks
// and samples, with P = W o exp(S - lse), D = rowsum(dO o O) and
// dS = P o (dO V^T - D):  dQ = dS K,  dK = dS^T Q,  dV = P^T dO  -- in fp32
// throughout, with vector arithmetic: a wave handles one (row, key) pair at
// a time, its lanes splitting the head dimension (d / 64 elements each), and
// the two dot products of the pair (S and dP) are wave sums.  This serves the
// fp32 workloads (one head at n = 1024 and small problems); the bf16 kernels
// are the fast path.  Every output element has one writer and a fixed order
// of summation, so results are bitwise deterministic:
//   * bwd32_qstat_kernel: per row (lse log2 e, D);
//   * bwd32_dq_kernel: one wave per query row -- its block keys, then its
//     kept samples (weight seg / m each, duplicates counted), or for an exact
//     causal leaf the keys up to the row;
//   * bwd32_dkv_kernel: one wave per key -- the queries of its block, every
//     query head of the KV group, or for a leaf the queries from the key on;
//   * bwd32_dkv_sample_kernel: one wave per (sample slot, query chunk) --
//     the chunk's partial [dK | dV] row of the slot's key, summed over the
//     chunks and added to the key rows by the deterministic sample reduction
//     of the bf16 path.
#include <cmath>

#include "ha_device.h"
#include "ha_kernels.h"

namespace ha {

namespace {

// sum over the 64 lanes, taken from lane 0 so every lane holds the same value
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return __shfl(x, 0);
}

template <int E>
__device__ __forceinline__ void load_slice(const float* row, int lane, float (&x)[E]) {
#pragma unroll
  for (int i = 0; i < E; ++i) x[i] = row[E * lane + i];
}

// one (query, key) pair: P and dS from the query's statistics, the key's
// log2 weight lw (0 inside the block, log2(seg / m) for a sample)
struct Pair {
  float pe, ds;
};

template <int E>
__device__ __forceinline__ Pair pair_terms(const float (&q)[E], const float (&g)[E], const float (&k)[E],
                                              const float (&v)[E], float l2, float drow, float lw) {
  float s = 0.f, dp = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    s = fmaf(q[i], k[i], s);
    dp = fmaf(g[i], v[i], dp);
  }
  s = wave_sum(s);
  dp = wave_sum(dp);
  const float pe = exp2f(fmaf(s, kLog2e, lw - l2));
  return {pe, pe * (dp - drow)};
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void bwd32_qstat_kernel(BwdParams p) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rows = static_cast<int64_t>(p.BH) * p.n;
  const int64_t nw = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  for (int64_t r = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6; r < rows; r += nw) {
    float o[E], g[E];
    load_slice(static_cast<const float*>(p.out) + r * D, lane, o);
    load_slice(static_cast<const float*>(p.dout) + r * D, lane, g);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) acc = fmaf(o[i], g[i], acc);
    acc = wave_sum(acc);
    if (lane == 0) {
      floatx2 st;
      st[0] = p.lse[r] * kLog2e;
      st[1] = acc;
      *reinterpret_cast<floatx2*>(p.qstat + 2 * r) = st;
    }
  }
}

template <int D, bool LEAF>
__global__ __launch_bounds__(256) void bwd32_dq_kernel(BwdParams p) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (w >= static_cast<int64_t>(p.BH) * p.pieces * p.seg) return;
  const int64_t prob = w / p.seg;                   // bh * pieces + piece
  const int pos = static_cast<int>(w - prob * p.seg);
  const int bh = static_cast<int>(prob / p.pieces);
  const int piece = static_cast<int>(prob - static_cast<int64_t>(bh) * p.pieces);
  const int bkv = (bh / p.H) * p.Hkv + (bh % p.H) / (p.H / p.Hkv);
  const int qrow = LEAF ? p.q_first + piece * p.stride + pos : p.perm_q[prob * p.seg + pos];
  const int64_t qr = static_cast<int64_t>(bh) * p.n + qrow;
  const float* kb = static_cast<const float*>(p.k) + static_cast<int64_t>(bkv) * p.n_k * D;
  const float* vb = static_cast<const float*>(p.v) + static_cast<int64_t>(bkv) * p.n_k * D;
  float q[E], g[E], acc[E];
  load_slice(static_cast<const float*>(p.q) + qr * D, lane, q);
  load_slice(static_cast<const float*>(p.dout) + qr * D, lane, g);
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.f;
  const floatx2 st = *reinterpret_cast<const floatx2*>(p.qstat + 2 * qr);
  auto add_key = [&](int krow, float lw) {
    float k[E], v[E];
    load_slice(kb + static_cast<int64_t>(krow) * D, lane, k);
    load_slice(vb + static_cast<int64_t>(krow) * D, lane, v);
    const Pair t = pair_terms<E>(q, g, k, v, st[0], st[1], lw);
#pragma unroll
    for (int i = 0; i < E; ++i) acc[i] = fmaf(t.ds, k[i], acc[i]);
  };
  if constexpr (LEAF) {
    const int k0 = p.k_first + piece * p.stride;
    for (int j = 0; j <= pos; ++j) add_key(k0 + j, 0.f);
  } else {
    const int32_t* pk = p.perm_k + (static_cast<int64_t>(bkv) * p.pieces + piece) * p.seg_k;
    const int t = pos / p.b_eff;
    const int blo = min(t * p.b_k, p.seg_k), bhi = min(blo + p.b_k, p.seg_k);
    for (int j = blo; j < bhi; ++j) add_key(pk[j], 0.f);
    const int32_t* si = p.sidx + prob * p.m;
    for (int i = 0; i < p.m; ++i) {
      const int sp = si[i];
      if (sp / p.b_k == t) continue;                // inside the row's block: excluded
      add_key(pk[sp], p.log2w);
    }
  }
  float* dst = p.dq + qr * D + E * lane;
#pragma unroll
  for (int i = 0; i < E; ++i) dst[i] = p.accumulate ? dst[i] + acc[i] : acc[i];
}

template <int D, bool LEAF>
__global__ __launch_bounds__(256) void bwd32_dkv_kernel(BwdParams p) {
  constexpr int E = D / 64;
  const int G = p.H / p.Hkv;
  const int lane = threadIdx.x & 63;
  const int64_t w = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (w >= static_cast<int64_t>(p.BH / G) * p.pieces * p.seg_k) return;
  const int64_t kprob = w / p.seg_k;                // bkv * pieces + piece
  const int kpos = static_cast<int>(w - kprob * p.seg_k);
  const int bkv = static_cast<int>(kprob / p.pieces);
  const int piece = static_cast<int>(kprob - static_cast<int64_t>(bkv) * p.pieces);
  const int b = bkv / p.Hkv, gk = bkv - b * p.Hkv;
  const int krow = LEAF ? p.k_first + piece * p.stride + kpos : p.perm_k[kprob * p.seg_k + kpos];
  const int64_t kr = static_cast<int64_t>(bkv) * p.n_k + krow;
  float k[E], v[E], ak[E], av[E];
  load_slice(static_cast<const float*>(p.k) + kr * D, lane, k);
  load_slice(static_cast<const float*>(p.v) + kr * D, lane, v);
#pragma unroll
  for (int i = 0; i < E; ++i) ak[i] = av[i] = 0.f;
  // queries of this key: a leaf's from the key on; else the query block that
  // pairs with the key's block
  int p0, p1;
  if constexpr (LEAF) {
    p0 = kpos;
    p1 = p.seg;
  } else {
    const int t = kpos / p.b_k;
    p0 = min(t * p.b_eff, p.seg);
    p1 = min(p0 + p.b_eff, p.seg);
  }
  for (int gi = 0; gi < G; ++gi) {
    const int bh = b * p.H + gk * G + gi;
    const int64_t prob = static_cast<int64_t>(bh) * p.pieces + piece;
    for (int pos = p0; pos < p1; ++pos) {
      const int qrow = LEAF ? p.q_first + piece * p.stride + pos : p.perm_q[prob * p.seg + pos];
      const int64_t qr = static_cast<int64_t>(bh) * p.n + qrow;
      float q[E], g[E];
      load_slice(static_cast<const float*>(p.q) + qr * D, lane, q);
      load_slice(static_cast<const float*>(p.dout) + qr * D, lane, g);
      const floatx2 st = *reinterpret_cast<const floatx2*>(p.qstat + 2 * qr);
      const Pair t = pair_terms<E>(q, g, k, v, st[0], st[1], 0.f);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        av[i] = fmaf(t.pe, g[i], av[i]);
        ak[i] = fmaf(t.ds, q[i], ak[i]);
      }
    }
  }
  float* dk = p.dk + kr * D + E * lane;
  float* dv = p.dv + kr * D + E * lane;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    dk[i] = p.accumulate ? dk[i] + ak[i] : ak[i];
    dv[i] = p.accumulate ? dv[i] + av[i] : av[i];
  }
}

// partial [dK | dV] row of sample slot `slot` ((bh * pieces + piece) * m + i)
// over the queries of chunk `ch` that keep the sample, weight seg_k / m
template <int D>
__global__ __launch_bounds__(256) void bwd32_dkv_sample_kernel(BwdParams p, int nchunk) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rows = static_cast<int64_t>(p.BH) * p.pieces * p.m;
  const int64_t w = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (w >= rows * nchunk) return;
  const int ch = static_cast<int>(w / rows);
  const int64_t slot = w - static_cast<int64_t>(ch) * rows;
  const int64_t prob = slot / p.m;
  const int bh = static_cast<int>(prob / p.pieces);
  const int piece = static_cast<int>(prob - static_cast<int64_t>(bh) * p.pieces);
  const int bkv = (bh / p.H) * p.Hkv + (bh % p.H) / (p.H / p.Hkv);
  const int kpos = p.sidx[slot];
  const int krow = p.perm_k[(static_cast<int64_t>(bkv) * p.pieces + piece) * p.seg_k + kpos];
  const int64_t kr = static_cast<int64_t>(bkv) * p.n_k + krow;
  float k[E], v[E], ak[E], av[E];
  load_slice(static_cast<const float*>(p.k) + kr * D, lane, k);
  load_slice(static_cast<const float*>(p.v) + kr * D, lane, v);
#pragma unroll
  for (int i = 0; i < E; ++i) ak[i] = av[i] = 0.f;
  const int kt = kpos / p.b_k;
  const int q1 = min((ch + 1) * p.qchunk, p.seg);
  for (int pos = ch * p.qchunk; pos < q1; ++pos) {
    if (pos / p.b_eff == kt) continue;              // the sample lies in this row's block
    const int qrow = p.perm_q[prob * p.seg + pos];
    const int64_t qr = static_cast<int64_t>(bh) * p.n + qrow;
    float q[E], g[E];
    load_slice(static_cast<const float*>(p.q) + qr * D, lane, q);
    load_slice(static_cast<const float*>(p.dout) + qr * D, lane, g);
    const floatx2 st = *reinterpret_cast<const floatx2*>(p.qstat + 2 * qr);
    const Pair t = pair_terms<E>(q, g, k, v, st[0], st[1], p.log2w);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      av[i] = fmaf(t.pe, g[i], av[i]);
      ak[i] = fmaf(t.ds, q[i], ak[i]);
    }
  }
  float* dst = p.part + (static_cast<int64_t>(ch) * rows + slot) * (2 * D) + E * lane;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    dst[i] = ak[i];
    dst[D + i] = av[i];
  }
}

// ---- launches (called by the bf16 launchers for fp32 problems) -----------------------

static unsigned wave_blocks(int64_t waves) { return static_cast<unsigned>((waves + 3) / 4); }

int launch_bwd32_qstat(const BwdParams& p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.BH) * p.n;
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (p.d == 64) hipLaunchKernelGGL(bwd32_qstat_kernel<64>, dim3(blocks), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(bwd32_qstat_kernel<128>, dim3(blocks), dim3(256), 0, s, p);
  return HA_OK;
}

int launch_bwd32_dq(const BwdParams& p, hipStream_t s) {
  const int64_t waves = static_cast<int64_t>(p.BH) * p.pieces * p.seg;
  const dim3 g(wave_blocks(waves)), b(256);
  const bool leaf = p.perm_q == nullptr;
  if (p.d == 64) {
    if (leaf) hipLaunchKernelGGL((bwd32_dq_kernel<64, true>), g, b, 0, s, p);
    else hipLaunchKernelGGL((bwd32_dq_kernel<64, false>), g, b, 0, s, p);
  } else {
    if (leaf) hipLaunchKernelGGL((bwd32_dq_kernel<128, true>), g, b, 0, s, p);
    else hipLaunchKernelGGL((bwd32_dq_kernel<128, false>), g, b, 0, s, p);
  }
  return HA_OK;
}

int launch_bwd32_dkv(const BwdParams& p, bool samples, hipStream_t s) {
  const int G = p.H / p.Hkv;
  if (!samples) {
    const bool leaf = p.perm_q == nullptr;
    if (leaf && p.diag == 1) return HA_OK;          // the leaf's keys are complete after its one pass
    const int64_t waves = static_cast<int64_t>(p.BH / G) * p.pieces * p.seg_k;
    const dim3 g(wave_blocks(waves)), b(256);
    if (p.d == 64) {
      if (leaf) hipLaunchKernelGGL((bwd32_dkv_kernel<64, true>), g, b, 0, s, p);
      else hipLaunchKernelGGL((bwd32_dkv_kernel<64, false>), g, b, 0, s, p);
    } else {
      if (leaf) hipLaunchKernelGGL((bwd32_dkv_kernel<128, true>), g, b, 0, s, p);
      else hipLaunchKernelGGL((bwd32_dkv_kernel<128, false>), g, b, 0, s, p);
    }
    return HA_OK;
  }
  const int nchunk = (p.seg + p.qchunk - 1) / p.qchunk;
  const int64_t waves = static_cast<int64_t>(p.BH) * p.pieces * p.m * nchunk;
  const dim3 g(wave_blocks(waves)), b(256);
  if (p.d == 64) hipLaunchKernelGGL(bwd32_dkv_sample_kernel<64>, g, b, 0, s, p, nchunk);
  else hipLaunchKernelGGL(bwd32_dkv_sample_kernel<128>, g, b, 0, s, p, nchunk);
  return launch_bwd_sample_reduce(p, nchunk, s);
}

}  // namespace ha
