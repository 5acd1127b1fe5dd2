// Attention kernels of the HyperAttention forward on gfx950.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: exact masked row sums inside
// the diagonal blocks of the sorted matrix plus uniform column sampling
// for the rest of the normaliser; section Limitations and the summary:
// recursive causal masking.)
//
// One kernel template serves every attention step:
//   * a problem of `seg` sorted queries and `seg` sorted keys (a whole head
//     when non-causal, one off-diagonal quadrant of a causal level):
//     sorted query p attends the keys of its block [t b, (t+1) b), t = p/b,
//     and the m sampled key positions outside its block, each with weight
//     seg/m, in one online softmax (the log-sum-exp merge of the two parts
//     is exactly this shared softmax);
//   * an exact causal leaf: row i of the leaf attends leaf keys 0..i.
// Rows are loaded through the sort permutations (no gathered copies) and
// written back to their original rows (the unsort).
//
// Work split: a workgroup of 4 waves owns 128 consecutive sorted queries
// (32 per wave).  Keys stream through LDS in tiles of 64.  Per wave and
// tile, S^T = K Q^T (keys x queries) is built with MFMA, so each lane owns
// one query column: lanes l and l+32 share query l%32 and hold different
// keys.  The softmax runs on those registers, P^T is converted in place
// into the B operand of O^T = V^T P^T, and O^T (d x queries) stays in
// registers.  bf16 uses v_mfma_f32_32x32x16_bf16 (V is stored transposed in
// LDS, keys permuted within 16-key chunks so one 16-byte LDS read yields
// an operand), fp32 uses v_mfma_f32_32x32x2_f32.  Accumulation and softmax
// are fp32.  The running maximum is only raised when a tile exceeds it by
// more than 2^8 (then the accumulators are rescaled once).
#include <cmath>
#include <type_traits>

#include "ha_kernels.h"
#include "ha_rng.h"

namespace ha {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = 4;
constexpr int kTQ = 32 * kAttnWaves;   // queries per workgroup
constexpr int kKT = 64;                // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.f;        // log2 slack before rescaling

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  // Dispatch places workgroup i on XCD i % 8; give each XCD a contiguous
  // range of logical tiles so tiles sharing keys share an L2.
  const int full = nblocks / 8 * 8;
  if (bid >= full) return bid;
  const int per = nblocks / 8;
  return (bid % 8) * per + bid / 8;
}

__device__ __forceinline__ int vt_pos(int j) {
  // swap bits 2 and 3 of the key index inside its 16-key chunk
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

template <typename T>
struct Tr;

template <>
struct Tr<bf16> {
  static constexpr int KC = 16;        // k per MFMA
};
template <>
struct Tr<float> {
  static constexpr int KC = 2;
};

template <typename T, int D>
struct Smem {
  static constexpr int KSTR = (sizeof(T) == 2) ? D + 8 : D + 1;     // K row stride (elements)
  static constexpr int VSTR = (sizeof(T) == 2) ? kKT + 8 : D + 1;   // V^T row / V row stride
  static constexpr int VROWS = (sizeof(T) == 2) ? D : kKT;
  alignas(16) T k[kKT * KSTR];
  alignas(16) T v[VROWS * VSTR];
  int slist[kMaxSamples];
  int nvalid;
};

template <typename T, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams p) {
  constexpr int KC = Tr<T>::KC;
  constexpr int NQF = D / KC;          // Q fragments per lane
  constexpr int NDT = D / 32;          // O^T tiles
  typedef Smem<T, D> SM;
  __shared__ SM sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h2 = lane >> 5;            // half-wave
  const int col = lane & 31;           // query column of this lane

  const int QT = (p.seg + kTQ - 1) / kTQ;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % QT;
  const int rest = lid / QT;
  const int piece = rest % p.pieces;
  const int bh = rest / p.pieces;
  const int b = bh / p.H;
  const int hq = bh % p.H;
  const int bkv = b * p.Hkv + hq / (p.H / p.Hkv);

  const int q0 = qt * kTQ;
  const int qend = min(q0 + kTQ, p.seg);
  const int64_t qpiece = static_cast<int64_t>(bh) * p.pieces + piece;    // [BH][pieces]
  const int64_t kpiece = static_cast<int64_t>(bkv) * p.pieces + piece;   // [BHkv][pieces]

  const T* qbase = static_cast<const T*>(p.q) + static_cast<int64_t>(bh) * p.n * D;
  const T* kbase = static_cast<const T*>(p.k) + static_cast<int64_t>(bkv) * p.n * D;
  const T* vbase = static_cast<const T*>(p.v) + static_cast<int64_t>(bkv) * p.n * D;
  const bool mat = p.qs != nullptr;   // materialised sorted copies
  const T* qsb = mat ? static_cast<const T*>(p.qs) + qpiece * p.seg * D : nullptr;
  const T* ksb = mat ? static_cast<const T*>(p.ks) + kpiece * p.seg * D : nullptr;
  const T* vsb = mat ? static_cast<const T*>(p.vs) + kpiece * p.seg * D : nullptr;
  const int32_t* pq = p.perm_q ? p.perm_q + qpiece * p.seg : nullptr;
  const int32_t* pk = p.perm_k ? p.perm_k + kpiece * p.seg : nullptr;
  const int qrow0 = p.q_first + piece * p.stride;
  const int krow0 = p.k_first + piece * p.stride;

  // ---- key ranges ---------------------------------------------------------
  const bool leaf = p.kind == kKindLeaf;
  int ka0 = 0, ka1 = 0;
  bool multi_block = false;
  if (p.use_block) {
    if (leaf) {
      ka0 = 0;
      ka1 = qend;
    } else {
      const int t0 = q0 / p.b_eff;
      const int t1 = (qend - 1) / p.b_eff;
      multi_block = t0 != t1;
      ka0 = t0 * p.b_eff;
      ka1 = (t1 + 1) * p.b_eff;
    }
  }
  const bool samp = p.use_samples && p.m > 0 && !leaf;
  const bool samp_multi = samp && ((q0 / p.b_eff) != ((qend - 1) / p.b_eff));

  // ---- sample list (compacted when all rows share one block) --------------
  if (samp) {
    const int32_t* si = p.sidx + qpiece * p.m;
    if (!samp_multi) {
      if (wave == 0) {
        const int tq = q0 / p.b_eff;
        int run = 0;
        for (int c = 0; c < p.m; c += 64) {
          const int i = c + lane;
          int s = i < p.m ? si[i] : 0;
          const bool keep = i < p.m && (s / p.b_eff) != tq;
          const uint64_t bal = __ballot(keep);
          const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
          if (keep) sm.slist[run + __popcll(bal & lower)] = s;
          run += __popcll(bal);
        }
        if (lane == 0) sm.nvalid = run;
      }
    } else {
      for (int i = threadIdx.x; i < p.m; i += kAttnThreads) sm.slist[i] = si[i];
      if (threadIdx.x == 0) sm.nvalid = p.m;
    }
  }
  __syncthreads();
  const int nsamp = samp ? sm.nvalid : 0;

  // ---- query fragments ------------------------------------------------------
  const int ql = q0 + wave * 32 + col;          // this lane's query (sorted/local pos)
  const bool qvalid = ql < qend;
  const int qls = qvalid ? ql : q0;             // clamp for loads
  const T* qrow;
  if (mat) qrow = qsb + static_cast<int64_t>(qls) * D;
  else qrow = qbase + static_cast<int64_t>(pq ? pq[qls] : qrow0 + qls) * D;

  typedef typename std::conditional<sizeof(T) == 2, bf16x8, float>::type QF;
  QF qf[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) {
    if constexpr (sizeof(T) == 2) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * h2);
    else qf[c] = qrow[2 * c + h2];
  }

  floatx16 o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float mrun = -INFINITY;   // running max, log2 units (incl. sample bias)
  float lsum = 0.f;         // this lane's share of the row sum

  const int nA = ka1 > ka0 ? (ka1 - ka0 + kKT - 1) / kKT : 0;
  const int nB = (nsamp + kKT - 1) / kKT;
  const int ntiles = nA + nB;
  const int row_blk = ql / p.b_eff;

  for (int it = 0; it < ntiles; ++it) {
    const bool isB = it >= nA;
    const int kb = isB ? (it - nA) * kKT : ka0 + it * kKT;
    const int kcnt = isB ? min(kKT, nsamp - kb) : min(kKT, ka1 - kb);

    // ---- stage K and V rows of this tile in LDS ---------------------------
    if constexpr (sizeof(T) == 2) {
      constexpr int CPR = D / 8;   // 16-byte chunks per row
      for (int ch = threadIdx.x; ch < kKT * CPR; ch += kAttnThreads) {
        const int j = ch / CPR;
        const int c8 = ch % CPR;
        uint4v kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
        if (j < kcnt) {
          const int kp = isB ? sm.slist[kb + j] : kb + j;
          const T *kr, *vr;
          if (mat && !leaf) {
            kr = ksb + static_cast<int64_t>(kp) * D;
            vr = vsb + static_cast<int64_t>(kp) * D;
          } else {
            const int64_t row = (pk && !leaf) ? pk[kp] : krow0 + kp;
            kr = kbase + row * D;
            vr = vbase + row * D;
          }
          kw = *reinterpret_cast<const uint4v*>(kr + 8 * c8);
          vw = *reinterpret_cast<const uint4v*>(vr + 8 * c8);
        }
        *reinterpret_cast<uint4v*>(&sm.k[j * SM::KSTR + 8 * c8]) = kw;
        unsigned short* vt = reinterpret_cast<unsigned short*>(sm.v);
        const int pj = vt_pos(j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vt[(8 * c8 + 2 * i) * SM::VSTR + pj] = static_cast<unsigned short>(vw[i] & 0xFFFFu);
          vt[(8 * c8 + 2 * i + 1) * SM::VSTR + pj] = static_cast<unsigned short>(vw[i] >> 16);
        }
      }
    } else {
      constexpr int CPR = D / 4;
      for (int ch = threadIdx.x; ch < kKT * CPR; ch += kAttnThreads) {
        const int j = ch / CPR;
        const int c4 = ch % CPR;
        floatx4 kw = {0.f, 0.f, 0.f, 0.f}, vw = {0.f, 0.f, 0.f, 0.f};
        if (j < kcnt) {
          const int kp = isB ? sm.slist[kb + j] : kb + j;
          const T *kr, *vr;
          if (mat && !leaf) {
            kr = ksb + static_cast<int64_t>(kp) * D;
            vr = vsb + static_cast<int64_t>(kp) * D;
          } else {
            const int64_t row = (pk && !leaf) ? pk[kp] : krow0 + kp;
            kr = kbase + row * D;
            vr = vbase + row * D;
          }
          kw = *reinterpret_cast<const floatx4*>(kr + 4 * c4);
          vw = *reinterpret_cast<const floatx4*>(vr + 4 * c4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm.k[j * SM::KSTR + 4 * c4 + i] = kw[i];
          sm.v[j * SM::VSTR + 4 * c4 + i] = vw[i];
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for 64 keys x 32 queries -----------------------------
    floatx16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
      for (int c = 0; c < NQF; ++c) {
        if constexpr (sizeof(T) == 2) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sm.k[(32 * kt + col) * SM::KSTR + 16 * c + 8 * h2]);
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], s[kt], 0, 0, 0);
        } else {
          const float ka = sm.k[(32 * kt + col) * SM::KSTR + 2 * c + h2];
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, qf[c], s[kt], 0, 0, 0);
        }
      }
    }

    // ---- masks ----------------------------------------------------------------
    const bool diag = leaf && (kb + kKT - 1 > q0 + wave * 32);
    const bool need_mask = kcnt < kKT || (isB ? samp_multi : (multi_block || diag));
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
          bool ok = j < kcnt;
          if (isB) {
            if (samp_multi) ok = ok && (sm.slist[kb + min(j, kcnt - 1)] / p.b_eff) != row_blk;
          } else if (leaf) {
            ok = ok && (kb + j <= ql);
          } else if (multi_block) {
            ok = ok && ((kb + j) / p.b_eff) == row_blk;
          }
          if (!ok) s[kt][r] = -INFINITY;
        }
    }

    // ---- online softmax -------------------------------------------------------
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float bias = isB ? p.log2w : 0.f;
    const float tmax = mx * kLog2e + bias;
    const bool raise = tmax > mrun + kRescale;
    if (__any(raise)) {
      const float mnew = raise ? fmaxf(mrun, tmax) : mrun;
      const float alpha = (mnew == mrun) ? 1.f : exp2f(mrun - mnew);
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      lsum *= alpha;
      mrun = mnew;
    }
    const float off = bias - (mrun == -INFINITY ? 0.f : mrun);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(fmaf(s[kt][r], kLog2e, off));
        s[kt][r] = e;
        lsum += e;
      }

    // ---- O^T += V^T P^T -------------------------------------------------------
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c16 = 0; c16 < 4; ++c16) {
        const int kt = c16 >> 1;
        const int hi = c16 & 1;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const bf16x2 two = __builtin_convertvector(
              (float __attribute__((ext_vector_type(2)))){s[kt][8 * hi + i], s[kt][8 * hi + i + 1]},
              bf16x2);
          pb[i] = two[0];
          pb[i + 1] = two[1];
        }
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(&sm.v[(32 * t + col) * SM::VSTR + 16 * c16 + 8 * h2]);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[t], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
          const int key = 32 * kt + 8 * (jr >> 2) + 4 * h2 + (jr & 3);
#pragma unroll
          for (int t = 0; t < NDT; ++t) {
            const float va = sm.v[key * SM::VSTR + 32 * t + col];
            o[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[kt][jr], o[t], 0, 0, 0);
          }
        }
    }
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const bool any = ltot > 0.f;
  const float inv = any ? 1.f / ltot : 0.f;
  const float lse2 = any ? (mrun + log2f(ltot)) * kLn2 : -INFINITY;
  if (!qvalid) return;

  // (row, destination) of this query
  int64_t orow;
  if (leaf || !pq) orow = qrow0 + ql;
  else orow = pq[ql];
  const int64_t ridx = static_cast<int64_t>(bh) * p.n + orow;

  int mode = p.out_mode;
  float w_new = 1.f, w_old = 0.f, lse_out = lse2;
  const float* acc_row = nullptr;
  if (mode == kOutMerge) {
    const float l1 = p.acc_lse[ridx];
    const float mm = fmaxf(l1, lse2);
    if (mm == -INFINITY) {
      lse_out = -INFINITY;
      w_old = 0.f;
      w_new = 0.f;
    } else {
      const float e1 = expf(l1 - mm), e2 = expf(lse2 - mm);
      lse_out = mm + logf(e1 + e2);
      w_old = expf(l1 - lse_out);
      w_new = expf(lse2 - lse_out);
    }
    acc_row = p.acc_o + ridx * D;
  }
  const bool to_final = mode == kOutFinal || ((mode == kOutLeaf || mode == kOutMerge) && piece == 0);
  const bool to_acc = ((mode == kOutLeaf || mode == kOutMerge) && piece != 0) || mode == kOutAcc;

#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dc = 32 * t + 8 * g + 4 * h2;   // 4 consecutive columns
      floatx4 val;
#pragma unroll
      for (int i = 0; i < 4; ++i) val[i] = o[t][4 * g + i] * inv;
      if (mode == kOutMerge) {
        const floatx4 old = *reinterpret_cast<const floatx4*>(acc_row + dc);
#pragma unroll
        for (int i = 0; i < 4; ++i) val[i] = old[i] * w_old + val[i] * w_new;
      }
      if (mode == kOutPartial) {
        *reinterpret_cast<floatx4*>(p.part_o + (qpiece * p.seg + ql) * D + dc) = val;
      } else if (to_acc) {
        *reinterpret_cast<floatx4*>(p.acc_o + ridx * D + dc) = val;
      } else if (to_final) {
        if constexpr (sizeof(T) == 2) {
          bf16x4 ob;
#pragma unroll
          for (int i = 0; i < 4; ++i) ob[i] = static_cast<bf16>(val[i]);
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.out) + ridx * D + dc) = ob;
        } else {
          *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + ridx * D + dc) = val;
        }
      }
    }
  if (h2 == 0) {
    if (mode == kOutPartial) p.part_lse[qpiece * p.seg + ql] = lse2;
    else if (to_acc) p.acc_lse[ridx] = lse_out;
    else if (to_final && p.lse) p.lse[ridx] = lse_out;
  }
}

template <typename T, int D>
static void launch_attn_t(const AttnParams& p, unsigned blocks, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<T, D>), dim3(blocks), dim3(kAttnThreads), 0, s, p);
}

int launch_attention(const AttnParams& p, int timing_kind, hipStream_t s) {
  if (p.seg == 0 || p.BH == 0 || p.pieces == 0) return HA_OK;
  if (p.m > kMaxSamples) {
    set_error("attention: samples %d > %d", p.m, kMaxSamples);
    return HA_EUNSUPPORTED;
  }
  const int64_t QT = (p.seg + kTQ - 1) / kTQ;
  const int64_t blocks = static_cast<int64_t>(p.BH) * p.pieces * QT;
  if (blocks > 0x7FFFFFFF) {
    set_error("attention: grid of %lld workgroups too large", static_cast<long long>(blocks));
    return HA_EUNSUPPORTED;
  }
  timing_begin(timing_kind, s);
  if (p.dtype == HA_BF16) {
    if (p.d == 64) launch_attn_t<bf16, 64>(p, static_cast<unsigned>(blocks), s);
    else launch_attn_t<bf16, 128>(p, static_cast<unsigned>(blocks), s);
  } else {
    if (p.d == 64) launch_attn_t<float, 64>(p, static_cast<unsigned>(blocks), s);
    else launch_attn_t<float, 128>(p, static_cast<unsigned>(blocks), s);
  }
  timing_end(timing_kind, s);
  return after_launch("attention", s);
}

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
  timing_begin(HA_K_GATHER, s);
  hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint4v*>(src), n, cpr, perm, rows_per_head, total,
                     static_cast<uint4v*>(dst));
  timing_end(HA_K_GATHER, s);
  return after_launch("gather", s);
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
