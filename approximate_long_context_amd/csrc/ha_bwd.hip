// Backward of the HyperAttention forward on gfx950 (non-causal problems).
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary: section Approach for the forward; section Key
// results times the method forward and backward.)
//
// For fixed ranks and samples the forward is a softmax over key rows with
// fixed multiplicities W (1 inside the query's block of the sorted matrix,
// seg / m per kept sample), so with P = W o exp(S - lse) rebuilt from the
// forward's lse, D = rowsum(dO o O) and dS = P o (dO V^T - D):
//     dQ = dS K,   dK = dS^T Q,   dV = P^T dO.
// The kernels keep the forward's conventions (bf16 operands, fp32
// accumulation, v_mfma_f32_32x32x16_bf16 with each lane owning one column
// of a 32-wide result, 64-row tiles double-buffered through LDS):
//   * bwd_qstat_kernel: per query, in sorted order, lse in log2 units and
//     D, so later passes read both contiguously;
//   * bwd_dq_kernel: query-owned like the forward -- a workgroup of 4 waves
//     owns 128 consecutive sorted queries, block and sample key tiles
//     stream through LDS; per 32-key half S^T = K Q^T and dP^T = V dO^T,
//     dS is packed to bf16 and dQ^T += K^T dS^T reads K transposed;
// Both attention passes build P without branches (a masked logit becomes
// -inf, whose exp2 is 0) in a masked and an unmasked instance of the tile
// body, chosen per tile and wave; tile loads are unconditional (clamped
// rows get P = dS = 0).
//   * bwd_dkv_kernel: key-owned -- a workgroup owns 128 sorted keys (block
//     part, every query head of the group) or 128 sample slots of one query
//     head and a chunk of its queries (sample part); per 32-query half
//     S = Q K^T and dP = dO V^T with a lane owning a key column, then
//     dV^T += dO^T P and dK^T += Q^T dS read Q and dO transposed.  Block
//     keys are stored (each key's block is owned by one workgroup); sample
//     slots store their chunk's partial rows, and bwd_dkv_reduce_kernel
//     sums them over the chunks and adds them to the key rows.
#include <cmath>

#include "ha_device.h"
#include "ha_kernels.h"

namespace ha {

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

constexpr int kBT = 64;      // rows per LDS tile
constexpr int kBW = 4;       // waves per workgroup
constexpr int kBNT = 64 * kBW;
constexpr int kBTQ = 32 * kBW;   // rows owned by a workgroup

// Waves per SIMD the register budget is set for.  d = 64: two (at most 256
// VGPRs; two 4-wave workgroups per CU, whose tile phases drift apart).
// d = 128: one -- a wave then holds up to 512 registers (the accumulators
// in AGPRs), where at two waves per SIMD the operands and accumulators
// spilled to scratch memory (measured 3.7x slower).
template <int D>
constexpr int bwd_min_waves() { return D == 64 ? 2 : 1; }

template <int D>
struct BGeo {
  static constexpr int STR = D + 8;               // LDS row stride (bf16 elements)
  static constexpr int TB = kBT * STR * 2;        // bytes of one tile
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int CPT = kBT * CPR / kBNT;    // chunks per thread per tile
  static constexpr int NQF = D / 16;              // k-chunks of one MFMA operand row
  static constexpr int NDT = D / 32;              // 32-column result tiles over d
  static_assert((kBT * CPR) % kBNT == 0, "tile split");
};

// ---- per-row statistics: (lse log2 e, D = rowsum(dO o O)) in row order ------------------

template <int D>
__global__ __launch_bounds__(256) void bwd_qstat_kernel(BwdParams p) {
  constexpr int LPR = D / 8;                      // lanes per row, 8 elements each
  constexpr int RPW = 64 / LPR;
  const bf16* o = static_cast<const bf16*>(p.out);
  const bf16* dout = static_cast<const bf16*>(p.dout);
  const int64_t rows = static_cast<int64_t>(p.BH) * p.n;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  for (int64_t r0 = wave * RPW; r0 < rows; r0 += nwaves * RPW) {
    const int64_t t = r0 + lane / LPR;
    const int64_t row = t < rows ? t : rows - 1;
    const int64_t off = row * D + 8 * (lane % LPR);
    const uint4v a = *reinterpret_cast<const uint4v*>(o + off);
    const uint4v g = *reinterpret_cast<const uint4v*>(dout + off);
    const float l = p.lse[row];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += __uint_as_float(a[i] << 16) * __uint_as_float(g[i] << 16);
      acc += __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(g[i] & 0xFFFF0000u);
    }
#pragma unroll
    for (int sh = LPR / 2; sh >= 1; sh >>= 1) acc += __shfl_xor(acc, sh);
    if (t < rows && lane % LPR == 0) {
      floatx2 st;
      st[0] = l * kLog2e;
      st[1] = acc;
      *reinterpret_cast<floatx2*>(p.qstat + 2 * t) = st;
    }
  }
}

int launch_bwd_qstat(const BwdParams& p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.BH) * p.n;
  if (rows == 0) return HA_OK;
  const int rpw = 64 / (p.d / 8);
  int64_t blocks = (rows + 4 * rpw - 1) / (4 * rpw);
  if (blocks > 16384) blocks = 16384;
  if (p.dtype == HA_F32) HA_TRY(launch_bwd32_qstat(p, s));
  else if (p.d == 64) hipLaunchKernelGGL(bwd_qstat_kernel<64>, dim3(blocks), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(bwd_qstat_kernel<128>, dim3(blocks), dim3(256), 0, s, p);
  return after_launch("backward row statistics", s);
}

// ---- dQ (query-owned) -----------------------------------------------------------------

// LDS after the two K/V tile buffers: brow[bcap], srow[m], sblk[m], rrow[m],
// one count per 64 samples.
static int dq_list_bytes(int bcap, int m) { return 4 * (bcap + 3 * m + (m + 63) / 64); }

// IDENT: the problem's rows are in row order (exact causal leaves); the
// permutations are not read.
template <int D, bool IDENT>
__global__ __launch_bounds__(kBNT, bwd_min_waves<D>()) void bwd_dq_kernel(BwdParams p) {
  typedef BGeo<D> G;
  constexpr int NQF = G::NQF, NDT = G::NDT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h2 = lane >> 5;
  const int col = lane & 31;

  const int QT = (p.seg + kBTQ - 1) / kBTQ;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = lid % QT;
  const int prob = lid / QT;                      // bh * pieces + piece
  const int bh = prob / p.pieces;
  const int piece = prob - bh * p.pieces;
  const int b = bh / p.H;
  const int bkv = b * p.Hkv + (bh % p.H) / (p.H / p.Hkv);
  const int q0 = qt * kBTQ;
  const int qend = min(q0 + kBTQ, p.seg);
  const int b_eff = p.b_eff;

  const bf16* qb = static_cast<const bf16*>(p.q) + static_cast<int64_t>(bh) * p.n * D;
  const bf16* gb = static_cast<const bf16*>(p.dout) + static_cast<int64_t>(bh) * p.n * D;
  const bf16* kbase = static_cast<const bf16*>(p.k) + static_cast<int64_t>(bkv) * p.n_k * D;
  const bf16* vbase = static_cast<const bf16*>(p.v) + static_cast<int64_t>(bkv) * p.n_k * D;
  const int32_t* pq = IDENT ? nullptr : p.perm_q + static_cast<int64_t>(prob) * p.seg;
  const int32_t* pk = IDENT ? nullptr : p.perm_k + (static_cast<int64_t>(bkv) * p.pieces + piece) * p.seg_k;
  const int qrow0 = piece * p.stride + p.q_first;
  const int krow0 = piece * p.stride + p.k_first;
  const int b_k = p.b_k;
  auto krow_of = [&](int t) { return IDENT ? krow0 + t : pk[t]; };

  // query block t pairs with key block t
  int ka1 = min(((qend - 1) / b_eff + 1) * b_k, p.seg_k);
  const int ka0 = min((q0 / b_eff) * b_k, ka1);
  if (p.causal) ka1 = min(ka1, qend);             // keys after the last query carry no weight
  const bool multi_block = (q0 / b_eff) != ((qend - 1) / b_eff);
  const bool samp = p.m > 0;
  const bool samp_multi = samp && multi_block;
  const int nbl = ka1 - ka0;

  // ---- key row lists (as the forward): block rows, compacted sample rows
  int* brow = reinterpret_cast<int*>(smem + 4 * G::TB);
  int* srow = brow + p.bcap;
  int* sblk = srow + p.m;                         // block of each sample's sorted position
  int* rrow = sblk + p.m;
  int* ccount = rrow + p.m;
  const bool blist = !IDENT && p.bcap > 0;
  int nsamp = 0;
  if (blist)
    for (int j = tid; j < nbl; j += kBNT) brow[j] = krow_of(ka0 + j);
  if (samp) {
    const int32_t* si = p.sidx + static_cast<int64_t>(prob) * p.m;
    const int tq = q0 / b_eff;
    int* raw = samp_multi ? srow : rrow;
    for (int c = 64 * wave; c < p.m; c += kBNT) {
      const int i = c + lane;
      const int sp = i < p.m ? si[i] : 0;
      if (i < p.m) {
        sblk[i] = sp / b_k;
        raw[i] = krow_of(sp);
      }
      const uint64_t keep = __ballot(i < p.m && (samp_multi || (sp / b_k) != tq));
      if (lane == 0) ccount[c / 64] = __popcll(keep);
    }
    __syncthreads();
    for (int k = 0; k < (p.m + 63) / 64; ++k) nsamp += ccount[k];
    if (!samp_multi) {
      for (int c = 64 * wave; c < p.m; c += kBNT) {
        int base = 0;
        for (int k = 0; k < c / 64; ++k) base += ccount[k];
        const int i = c + lane;
        const bool keep = i < p.m && sblk[i] != tq;
        const uint64_t bal = __ballot(keep);
        const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        if (keep) srow[base + __popcll(bal & lower)] = rrow[i];
      }
    }
  }
  __syncthreads();

  // ---- this lane's query: operands, lse and D
  const int ql = q0 + wave * 32 + col;
  const int qls = ql < qend ? ql : q0;
  const int orow = IDENT ? qrow0 + qls : pq[qls];
  const int64_t ridx = static_cast<int64_t>(bh) * p.n + orow;
  const floatx2 qst = *reinterpret_cast<const floatx2*>(p.qstat + 2 * ridx);
  const float lse2 = qst[0];
  const float dl = qst[1];
  bf16x8 qf[NQF], gf[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) {
    const uint32_t off = static_cast<uint32_t>(orow * D + 16 * c + 8 * h2) * 2;
    qf[c] = __builtin_bit_cast(bf16x8, ld16(qb, off));
    gf[c] = __builtin_bit_cast(bf16x8, ld16(gb, off));
  }
  floatx16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

  const int nA = nbl > 0 ? (nbl + kBT - 1) / kBT : 0;
  const int nB = (nsamp + kBT - 1) / kBT;
  const int ntiles = nA + nB;

  // ---- tile staging
  const int c_in_row = tid % G::CPR;
  const int j_first = tid / G::CPR;
  constexpr int JSTEP = kBNT / G::CPR;
  uint4v kreg[G::CPT], vreg[G::CPT];
  auto load_tile = [&](int it) {
    const bool isB = it >= nA;
    const int kb = isB ? (it - nA) * kBT : ka0 + it * kBT;
    const int kcnt = isB ? min(kBT, nsamp - kb) : min(kBT, ka1 - kb);
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const int j = min(j_first + c * JSTEP, kcnt - 1);
      const int row = isB ? srow[kb + j] : (blist ? brow[kb - ka0 + j] : krow_of(kb + j));
      const uint32_t off = static_cast<uint32_t>(row * D + 8 * c_in_row) * 2;
      kreg[c] = ld16(kbase, off);
      vreg[c] = ld16(vbase, off);
    }
  };
  auto store_tile = [&](int buf) {
    bf16* ks = reinterpret_cast<bf16*>(smem + (2 * buf) * G::TB);
    bf16* vs = reinterpret_cast<bf16*>(smem + (2 * buf + 1) * G::TB);
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const int j = j_first + c * JSTEP;
      *reinterpret_cast<uint4v*>(&ks[j * G::STR + 8 * c_in_row]) = kreg[c];
      *reinterpret_cast<uint4v*>(&vs[j * G::STR + 8 * c_in_row]) = vreg[c];
    }
  };

  const int row_blk = ql / b_eff;
  if (ntiles > 0) load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    store_tile(buf);
    __syncthreads();
    if (it + 1 < ntiles) load_tile(it + 1);
    const bool isB = it >= nA;
    const int kb = isB ? (it - nA) * kBT : ka0 + it * kBT;
    const int kcnt = isB ? min(kBT, nsamp - kb) : min(kBT, ka1 - kb);
    if (p.causal && kb > q0 + 32 * wave + 31) continue;   // every key of the tile after this wave's queries
    const bf16* ks = reinterpret_cast<const bf16*>(smem + (2 * buf) * G::TB);
    const bf16* vs = reinterpret_cast<const bf16*>(smem + (2 * buf + 1) * G::TB);
    const float off = (isB ? p.log2w : 0.f) - lse2;
    // key j of a block tile lies in the query's key block iff (unsigned)(j - lo) < b_k
    const int lo = row_blk * b_k - kb;
    const bool blk_test = !isB && multi_block;
    const bool smp_test = isB && samp_multi;
    const bool cau_test = p.causal && kb + kBT - 1 > q0;   // some key of the tile after some query
    auto tile = [&](auto mflag) {
      constexpr bool M = decltype(mflag)::value;
#pragma unroll
      for (int kt = 0; kt < kBT / 32; ++kt) {
        bf16x8 ka[NQF], va[NQF];
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
          const int e = (32 * kt + col) * G::STR + 16 * c + 8 * h2;
          ka[c] = *reinterpret_cast<const bf16x8*>(&ks[e]);
          va[c] = *reinterpret_cast<const bf16x8*>(&vs[e]);
        }
        floatx16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qf[c], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c], gf[c], dp, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 kto[NDT][2];
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          kto[t][0] = lds_tr_operand(ks, G::STR, 2 * kt, t, lane);
          kto[t][1] = lds_tr_operand(ks, G::STR, 2 * kt + 1, t, lane);
        }
        bf16x8 da, db;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = fmaf(s[r], kLog2e, off);
          if constexpr (M) {
            const int j = 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
            bool ok = j < kcnt;
            if (blk_test) ok &= static_cast<unsigned>(j - lo) < static_cast<unsigned>(b_k);
            if (smp_test) ok &= sblk[kb + min(j, kcnt - 1)] != row_blk;
            if (cau_test) ok &= kb + j <= ql;
            x = ok ? x : -INFINITY;
          }
          const float pr = fast_exp2(x);
          const bf16 dsv = static_cast<bf16>(pr * (dp[r] - dl));
          if (r < 8) da[r] = dsv;
          else db[r - 8] = dsv;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kto[t][0], da, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kto[t][1], db, acc[t], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (kcnt < kBT || blk_test || smp_test || cau_test) tile(Flag<true>());
    else tile(Flag<false>());
  }

  // ---- dQ rows (fp32): register r of tile t holds column 32 t + 8 (r / 4) + 4 h2 + r % 4
  if (ql < qend) {
    float* dst = p.dq + ridx * D;
    floatx4 old[NDT][4];
    if (p.accumulate) {
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) old[t][g] = *reinterpret_cast<const floatx4*>(dst + 32 * t + 8 * g + 4 * h2);
    }
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        floatx4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = acc[t][4 * g + i];
        if (p.accumulate) v4 += old[t][g];
        *reinterpret_cast<floatx4*>(dst + 32 * t + 8 * g + 4 * h2) = v4;
      }
  }
}

// ---- dK, dV (key-owned) ---------------------------------------------------------------

// LDS per buffer: Q tile, dO tile (64 rows each), lse log2 e [64], D[64].
template <int D>
constexpr int dkv_buf_bytes() { return 2 * BGeo<D>::TB + 2 * kBT * 4; }

// MASK 0: every query tile lies wholly inside or wholly outside a key's
// block (block sizes that are multiples of the 64-row tile), so the block
// mask is a per-lane, per-tile bias (0 or -inf) folded into the exponent.
// MASK 1: per-element block masks (other block sizes).  MASK 2: per-element
// causal mask (exact causal problems, the keys' own query square).  Ragged
// query rows always carry lse = +inf; lanes past the last key need no mask,
// their column is never stored.
template <int D, bool SAMPLE, int MASK, bool IDENT>
__global__ __launch_bounds__(kBNT, bwd_min_waves<D>()) void bwd_dkv_kernel(BwdParams p) {
  typedef BGeo<D> G;
  constexpr int NQF = G::NQF, NDT = G::NDT;
  constexpr int BUF = dkv_buf_bytes<D>();
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h2 = lane >> 5;
  const int col = lane & 31;
  const int b_eff = p.b_eff;
  const int G_ = p.H / p.Hkv;

  // ---- work item: key problem (KV head, piece), its keys [k0, kend), the
  // query problems qprob0 + hh * pieces (hh < nheads) and their queries [qa0, qa1)
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  int bkv, piece, qprob0, nheads, k0, kend, qa0, qa1, chunk = 0, sprob = 0;
  if constexpr (!SAMPLE) {
    const int KT = (p.seg_k + kBTQ - 1) / kBTQ;
    const int kprob = lid / KT;
    bkv = kprob / p.pieces;
    piece = kprob - bkv * p.pieces;
    k0 = (lid % KT) * kBTQ;
    kend = min(k0 + kBTQ, p.seg_k);
    const int b = bkv / p.Hkv;
    qprob0 = (b * p.H + (bkv % p.Hkv) * G_) * p.pieces + piece;
    nheads = G_;
    // key block t pairs with query block t
    qa1 = min(((kend - 1) / p.b_k + 1) * b_eff, p.seg);
    qa0 = min((k0 / p.b_k) * b_eff, qa1);
    if (p.diag == 2) {
      qa0 = k0;
      qa1 = min(qa1, k0 + kBTQ);
    } else if (p.diag == 1) {
      qa0 = k0 + kBTQ;
    }
  } else {
    const int NC = (p.seg + p.qchunk - 1) / p.qchunk;
    const int SG = (p.m + kBTQ - 1) / kBTQ;
    chunk = lid % NC;
    const int rest = lid / NC;
    k0 = (rest % SG) * kBTQ;
    kend = min(k0 + kBTQ, p.m);
    sprob = rest / SG;                            // bh * pieces + piece
    const int bh = sprob / p.pieces;
    piece = sprob - bh * p.pieces;
    bkv = (bh / p.H) * p.Hkv + (bh % p.H) / G_;
    qprob0 = sprob;
    nheads = 1;
    qa0 = chunk * p.qchunk;
    qa1 = min(qa0 + p.qchunk, p.seg);
  }
  const bf16* kbase = static_cast<const bf16*>(p.k) + static_cast<int64_t>(bkv) * p.n_k * D;
  const bf16* vbase = static_cast<const bf16*>(p.v) + static_cast<int64_t>(bkv) * p.n_k * D;
  const int32_t* pk = IDENT ? nullptr : p.perm_k + (static_cast<int64_t>(bkv) * p.pieces + piece) * p.seg_k;
  const int qrow0 = piece * p.stride + p.q_first;

  // ---- this lane's key: operands and block
  const int kj = k0 + wave * 32 + col;           // key position (block) or sample slot (sample)
  const bool kvalid = kj < kend;
  const int kjs = kvalid ? kj : k0;
  int kpos;                                      // sorted key position
  if constexpr (SAMPLE) kpos = p.sidx[static_cast<int64_t>(sprob) * p.m + kjs];
  else kpos = kjs;
  const int krow = IDENT ? piece * p.stride + p.k_first + kpos : pk[kpos];
  const int kblk = kpos / p.b_k;                 // pairs with query block kblk
  bf16x8 kf[NQF], vf[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) {
    const uint32_t off = static_cast<uint32_t>(krow * D + 16 * c + 8 * h2) * 2;
    kf[c] = __builtin_bit_cast(bf16x8, ld16(kbase, off));
    vf[c] = __builtin_bit_cast(bf16x8, ld16(vbase, off));
  }
  floatx16 dk[NDT], dv[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[t][r] = dv[t][r] = 0.f;

  const int qtiles = qa1 > qa0 ? (qa1 - qa0 + kBT - 1) / kBT : 0;
  const int ntiles = qtiles * nheads;
  const float wbias = SAMPLE ? p.log2w : 0.f;

  // ---- tile staging: query rows of Q and dO and their statistics.  The
  // permutation entries of a tile are fetched one tile ahead of its rows,
  // so no row load waits on a load issued in the same iteration.
  const int c_in_row = tid % G::CPR;
  const int j_first = tid / G::CPR;
  constexpr int JSTEP = kBNT / G::CPR;
  uint4v qreg[G::CPT], greg[G::CPT];
  int prow[G::CPT];
  floatx2 sreg[G::CPT];
  bool sval[G::CPT];
  auto tile_rows = [&](int it, int& tq0, int& qcnt, int& qprob) {
    tq0 = qa0 + (it % qtiles) * kBT;
    qcnt = min(kBT, qa1 - tq0);
    qprob = qprob0 + (it / qtiles) * p.pieces;
  };
  auto fetch_perm = [&](int it) {
    int tq0, qcnt, qprob;
    tile_rows(it, tq0, qcnt, qprob);
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const int t = tq0 + min(j_first + c * JSTEP, qcnt - 1);
      prow[c] = IDENT ? qrow0 + t : p.perm_q[static_cast<int64_t>(qprob) * p.seg + t];
    }
  };
  // rows of Q and dO and the rows' statistics (every thread loads its row's;
  // rows past the tile carry lse = +inf: P = 0).  No load is conditional, so
  // none forces a wait where control flow joins.
  auto load_tile = [&](int it) {
    int tq0, qcnt, qprob;
    tile_rows(it, tq0, qcnt, qprob);
    const int bh = qprob / p.pieces;
    const bf16* qb = static_cast<const bf16*>(p.q) + static_cast<int64_t>(bh) * p.n * D;
    const bf16* gb = static_cast<const bf16*>(p.dout) + static_cast<int64_t>(bh) * p.n * D;
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const uint32_t off = static_cast<uint32_t>(prow[c] * D + 8 * c_in_row) * 2;
      qreg[c] = ld16(qb, off);
      greg[c] = ld16(gb, off);
      sreg[c] = *reinterpret_cast<const floatx2*>(p.qstat + 2 * (static_cast<int64_t>(bh) * p.n + prow[c]));
      sval[c] = j_first + c * JSTEP < qcnt;     // applied at the store, not here: no wait on the load
    }
  };
  auto store_tile = [&](int buf) {
    char* base = smem + buf * BUF;
    bf16* qs = reinterpret_cast<bf16*>(base);
    bf16* gs = reinterpret_cast<bf16*>(base + G::TB);
    float* ls = reinterpret_cast<float*>(base + 2 * G::TB);
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const int j = j_first + c * JSTEP;
      *reinterpret_cast<uint4v*>(&qs[j * G::STR + 8 * c_in_row]) = qreg[c];
      *reinterpret_cast<uint4v*>(&gs[j * G::STR + 8 * c_in_row]) = greg[c];
      if (c_in_row == 0) {                      // accumulator starts: -lse (natural log units), -D
        ls[j] = sval[c] ? -sreg[c][0] * kLn2 : -INFINITY;
        ls[kBT + j] = -sreg[c][1];
      }
    }
  };

  if (ntiles > 0) {
    fetch_perm(0);
    load_tile(0);
    if (ntiles > 1) fetch_perm(1);
  }
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    store_tile(buf);
    __syncthreads();
    if (it + 1 < ntiles) {
      load_tile(it + 1);
      if (it + 2 < ntiles) fetch_perm(it + 2);
    }
    int tq0, qcnt, qprob_unused;
    tile_rows(it, tq0, qcnt, qprob_unused);
    const char* base = smem + buf * BUF;
    const bf16* qs = reinterpret_cast<const bf16*>(base);
    const bf16* gs = reinterpret_cast<const bf16*>(base + G::TB);
    const float* ls = reinterpret_cast<const float*>(base + 2 * G::TB);
    // query j of the tile lies in this lane's key block iff (unsigned)(j - lo) < b_eff
    const int lo = kblk * b_eff - tq0;
    float bias = wbias;
    if constexpr (MASK == 0) {
      const bool tin = static_cast<unsigned>(-lo) < static_cast<unsigned>(b_eff);
      if (SAMPLE ? tin : !tin) bias = -INFINITY;
    }
    {
#pragma unroll
      for (int qt = 0; qt < kBT / 32; ++qt) {
        bf16x8 qa[NQF], ga[NQF];
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
          const int e = (32 * qt + col) * G::STR + 16 * c + 8 * h2;
          qa[c] = *reinterpret_cast<const bf16x8*>(&qs[e]);
          ga[c] = *reinterpret_cast<const bf16x8*>(&gs[e]);
        }
        // S and dP accumulate onto the rows' statistics, so they end as
        // S - lse and dP - D (register r holds query 32 qt + 8 (r / 4) + 4 h2 + r % 4)
        floatx16 s, dp;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j0 = 32 * qt + 8 * g + 4 * h2;
          const floatx4 a4 = *reinterpret_cast<const floatx4*>(ls + j0);
          const floatx4 b4 = *reinterpret_cast<const floatx4*>(ls + kBT + j0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[4 * g + i] = a4[i];
            dp[4 * g + i] = b4[i];
          }
        }
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[c], kf[c], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[c], vf[c], dp, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 gto[NDT][2], qto[NDT][2];
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          gto[t][0] = lds_tr_operand(gs, G::STR, 2 * qt, t, lane);
          gto[t][1] = lds_tr_operand(gs, G::STR, 2 * qt + 1, t, lane);
          qto[t][0] = lds_tr_operand(qs, G::STR, 2 * qt, t, lane);
          qto[t][1] = lds_tr_operand(qs, G::STR, 2 * qt + 1, t, lane);
        }
        bf16x8 pa, pb, da, db;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j0 = 32 * qt + 8 * g + 4 * h2;      // 4 consecutive queries of the tile
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            float x = fmaf(s[r], kLog2e, bias);
            if constexpr (MASK == 1) {
              const bool in_blk = static_cast<unsigned>(j0 + i - lo) < static_cast<unsigned>(b_eff);
              x = (SAMPLE ? !in_blk : in_blk) ? x : -INFINITY;
            } else if constexpr (MASK == 2) {
              x = j0 + i >= kpos - tq0 ? x : -INFINITY;   // query position >= key position
            }
            const float pr = fast_exp2(x);
            const bf16 pv = static_cast<bf16>(pr);
            const bf16 dsv = static_cast<bf16>(pr * dp[r]);
            if (r < 8) {
              pa[r] = pv;
              da[r] = dsv;
            } else {
              pb[r - 8] = pv;
              db[r - 8] = dsv;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gto[t][0], pa, dv[t], 0, 0, 0);
          dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gto[t][1], pb, dv[t], 0, 0, 0);
          dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qto[t][0], da, dk[t], 0, 0, 0);
          dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qto[t][1], db, dk[t], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- dK, dV rows (fp32): register r of tile t holds column 32 t + 8 (r / 4) + 4 h2 + r % 4.
  // Block keys: the final rows.  Sample slots: this chunk's partial row
  // [dK | dV] of the slot, summed over the chunks by bwd_dkv_reduce_kernel.
  if (kvalid) {
    float* dkr;
    float* dvr;
    bool add = false;
    if constexpr (SAMPLE) {
      dkr = p.part + ((static_cast<int64_t>(chunk) * p.BH * p.pieces + sprob) * p.m + kj) * (2 * D);
      dvr = dkr + D;
    } else {
      dkr = p.dk + (static_cast<int64_t>(bkv) * p.n_k + krow) * D;
      dvr = p.dv + (static_cast<int64_t>(bkv) * p.n_k + krow) * D;
      add = p.accumulate;
    }
    floatx4 ok_[NDT][4], ov_[NDT][4];
    if (add) {
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          ok_[t][g] = *reinterpret_cast<const floatx4*>(dkr + 32 * t + 8 * g + 4 * h2);
          ov_[t][g] = *reinterpret_cast<const floatx4*>(dvr + 32 * t + 8 * g + 4 * h2);
        }
    }
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * t + 8 * g + 4 * h2;
        floatx4 a, c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = dk[t][4 * g + i];
          c[i] = dv[t][4 * g + i];
        }
        if (add) {
          a += ok_[t][g];
          c += ov_[t][g];
        }
        *reinterpret_cast<floatx4*>(dkr + c0) = a;
        *reinterpret_cast<floatx4*>(dvr + c0) = c;
      }
  }
}

// Sum of the sample slots' partial [dK | dV] rows, in a fixed order.  Several
// slots can name one key row (duplicate draws, and the query heads of a KV
// group draw on the same keys), so per problem (KV head, piece) the G m slots
// of its query heads are first sorted by (key position, head, draw) -- a
// bitonic sort in LDS writing the sorted keys to the workspace -- and then one
// wave per run of equal key positions sums the run's partial rows over the
// query chunks, slot by slot in that order, and adds the total to the key's
// dK and dV rows as their only writer: bitwise deterministic results.
constexpr int kRedCap = kBwdMaxGroupSamples;   // slots per problem (G m) the sort holds in LDS

__global__ __launch_bounds__(1024) void bwd_red_sort_kernel(BwdParams p) {
  __shared__ uint64_t key[kRedCap];
  const int G = p.H / p.Hkv;
  const int S = G * p.m;
  int P = 1;
  while (P < S) P <<= 1;
  const int prob = blockIdx.x;                      // (batch * Hkv + g) * pieces + piece
  const int bkv = prob / p.pieces, piece = prob - bkv * p.pieces;
  const int b = bkv / p.Hkv, g = bkv - b * p.Hkv;
  for (int e = threadIdx.x; e < P; e += 1024) {
    uint64_t kk = ~0ull;
    if (e < S) {
      const int gi = e / p.m, i = e - gi * p.m;
      const int64_t bh = static_cast<int64_t>(b) * p.H + g * G + gi;
      const uint32_t kpos = static_cast<uint32_t>(p.sidx[(bh * p.pieces + piece) * p.m + i]);
      kk = (static_cast<uint64_t>(kpos) << 32) | static_cast<uint32_t>(e);
    }
    key[e] = kk;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int e = threadIdx.x; e < P; e += 1024) {
        const int x = e ^ j;
        if (x > e) {
          const uint64_t a = key[e], c = key[x];
          if ((a > c) == ((e & k) == 0)) {
            key[e] = c;
            key[x] = a;
          }
        }
      }
      __syncthreads();
    }
  uint64_t* out = p.red_keys + static_cast<int64_t>(prob) * S;
  for (int e = threadIdx.x; e < S; e += 1024) out[e] = key[e];
}

template <int D>
__global__ __launch_bounds__(256) void bwd_red_sum_kernel(BwdParams p, int nchunk) {
  constexpr int PL = 2 * D / 64;                    // [dK | dV] columns per lane
  const int G = p.H / p.Hkv;
  const int S = G * p.m;
  const int64_t w = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t nprob = static_cast<int64_t>(p.BH / G) * p.pieces;
  if (w >= nprob * S) return;
  const int prob = static_cast<int>(w / S);
  const int e = static_cast<int>(w - static_cast<int64_t>(prob) * S);
  const uint64_t* sk = p.red_keys + static_cast<int64_t>(prob) * S;
  const uint32_t kpos = static_cast<uint32_t>(sk[e] >> 32);
  if (e > 0 && static_cast<uint32_t>(sk[e - 1] >> 32) == kpos) return;   // not the first slot of its run
  const int bkv = prob / p.pieces, piece = prob - bkv * p.pieces;
  const int b = bkv / p.Hkv, g = bkv - b * p.Hkv;
  const int64_t cstride = static_cast<int64_t>(p.BH) * p.pieces * p.m * (2 * D);
  float acc[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) acc[i] = 0.f;
  for (int x = e; x < S && static_cast<uint32_t>(sk[x] >> 32) == kpos; ++x) {
    const int loc = static_cast<int>(sk[x] & 0xFFFFFFFFull);
    const int gi = loc / p.m, i = loc - gi * p.m;
    const int64_t bh = static_cast<int64_t>(b) * p.H + g * G + gi;
    const float* src = p.part + ((bh * p.pieces + piece) * p.m + i) * (2 * D) + PL * lane;
    for (int ch = 0; ch < nchunk; ++ch) {
      const float* r = src + ch * cstride;
#pragma unroll
      for (int c = 0; c < PL; ++c) acc[c] += r[c];
    }
  }
  const int krow = p.perm_k[static_cast<int64_t>(prob) * p.seg_k + kpos];
  const int col = PL * lane;                         // column of [dK | dV]
  float* dst = (col < D ? p.dk : p.dv) + (static_cast<int64_t>(bkv) * p.n_k + krow) * D + (col < D ? col : col - D);
#pragma unroll
  for (int c = 0; c < PL; ++c) dst[c] += acc[c];
}

// The deterministic sum of the sample partials (both dtypes).
int launch_bwd_sample_reduce(const BwdParams& p, int nchunk, hipStream_t s) {
  const int64_t nprob = static_cast<int64_t>(p.BH / (p.H / p.Hkv)) * p.pieces;
  hipLaunchKernelGGL(bwd_red_sort_kernel, dim3(static_cast<unsigned>(nprob)), dim3(1024), 0, s, p);
  const int64_t threads = nprob * (p.H / p.Hkv) * p.m * 64;   // one wave per sorted slot
  const dim3 g(static_cast<unsigned>((threads + 255) / 256)), b(256);
  if (p.d == 64) hipLaunchKernelGGL((bwd_red_sum_kernel<64>), g, b, 0, s, p, nchunk);
  else hipLaunchKernelGGL((bwd_red_sum_kernel<128>), g, b, 0, s, p, nchunk);
  return HA_OK;
}

// ---- launches ---------------------------------------------------------------------------

// n_k = 0, seg_k = 0 and b_k = 0 mean a square problem (n_k = n, seg_k = seg,
// b_k = b_eff).
static BwdParams bwd_normalized(const BwdParams& p) {
  BwdParams q = p;
  if (q.n_k == 0) q.n_k = q.n;
  if (q.seg_k == 0) q.seg_k = q.seg;
  if (q.b_k == 0) q.b_k = q.b_eff;
  return q;
}

template <int D, bool IDENT>
static int launch_dq_d(const BwdParams& p, hipStream_t s) {
  BwdParams q = p;
  q.bcap = 0;
  const int64_t span = static_cast<int64_t>((kBTQ - 1) / p.b_eff + 2) * p.b_k;
  const int64_t cap = span < p.seg_k ? span : p.seg_k;
  if (cap <= kBlockListCap) q.bcap = static_cast<int>(cap);
  const size_t lds = 4 * BGeo<D>::TB + dq_list_bytes(q.bcap, p.m);
  const int64_t blocks = static_cast<int64_t>(p.BH) * p.pieces * ((p.seg + kBTQ - 1) / kBTQ);
  auto fn = bwd_dq_kernel<D, IDENT>;
  // once per instantiation (thread-safe static initialisation)
  static const hipError_t attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  HA_CHECK_HIP(attr_err);
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(kBNT), lds, s, q);
  return HA_OK;
}

int launch_bwd_dq(const BwdParams& p0, hipStream_t s) {
  const BwdParams p = bwd_normalized(p0);
  if (p.seg == 0 || p.BH == 0) return HA_OK;
  if (p.seg_k < 1 || p.b_k < 1 || (p.causal && (p.seg_k != p.seg || p.b_k != p.b_eff))) {
    set_error("backward dq: a problem needs keys; causal problems are square");
    return HA_EINVAL;
  }
  if (p.m > kMaxSamples) {
    set_error("backward: samples %d > %d", p.m, kMaxSamples);
    return HA_EUNSUPPORTED;
  }
  HA_TRY(launch_gate(HA_K_BWD_DQ));
  timing_begin(HA_K_BWD_DQ, s);
  if (!p.perm_q != !p.perm_k || (!p.perm_q && p.m > 0)) {
    set_error("backward dq: both permutations or neither; samples need them");
    return HA_EINVAL;
  }
  int st;
  if (p.dtype == HA_F32) st = launch_bwd32_dq(p, s);
  else if (p.perm_q) st = p.d == 64 ? launch_dq_d<64, false>(p, s) : launch_dq_d<128, false>(p, s);
  else st = p.d == 64 ? launch_dq_d<64, true>(p, s) : launch_dq_d<128, true>(p, s);
  timing_end(HA_K_BWD_DQ, s);
  if (st != HA_OK) return st;
  return after_launch("backward dq", s);
}

template <int D, bool SAMPLE, int MASK, bool IDENT>
static int launch_dkv_d2(const BwdParams& p, hipStream_t s) {
  int64_t blocks;
  const int nchunk = (p.seg + p.qchunk - 1) / p.qchunk;
  if constexpr (SAMPLE) {
    blocks = static_cast<int64_t>(p.BH) * p.pieces * ((p.m + kBTQ - 1) / kBTQ) * nchunk;
  } else {
    blocks = static_cast<int64_t>(p.BH / (p.H / p.Hkv)) * p.pieces * ((p.seg_k + kBTQ - 1) / kBTQ);
  }
  if (blocks == 0) return HA_OK;
  const size_t lds = 2 * dkv_buf_bytes<D>();
  hipLaunchKernelGGL((bwd_dkv_kernel<D, SAMPLE, MASK, IDENT>), dim3(static_cast<unsigned>(blocks)), dim3(kBNT), lds,
                     s, p);
  if constexpr (SAMPLE) return launch_bwd_sample_reduce(p, nchunk, s);
  return HA_OK;
}

template <int D, bool SAMPLE>
static int launch_dkv_d(const BwdParams& p, hipStream_t s) {
  if constexpr (SAMPLE) {
    if (p.b_eff % kBT) return launch_dkv_d2<D, true, 1, false>(p, s);
    return launch_dkv_d2<D, true, 0, false>(p, s);
  } else {
    if (!p.perm_q) {                               // exact causal leaves
      if (p.diag == 2) return launch_dkv_d2<D, false, 2, true>(p, s);
      if (p.b_eff % kBT) return launch_dkv_d2<D, false, 1, true>(p, s);
      return launch_dkv_d2<D, false, 0, true>(p, s);
    }
    if (p.b_eff % kBT) return launch_dkv_d2<D, false, 1, false>(p, s);
    return launch_dkv_d2<D, false, 0, false>(p, s);
  }
}

int launch_bwd_dkv(const BwdParams& p0, bool samples, hipStream_t s) {
  const BwdParams p = bwd_normalized(p0);
  if (p.seg == 0 || p.BH == 0 || (samples && p.m == 0)) return HA_OK;
  if (p.seg_k < 1 || p.b_k < 1 || (p.causal && (p.seg_k != p.seg || p.b_k != p.b_eff))) {
    set_error("backward dk/dv: a problem needs keys; causal problems are square");
    return HA_EINVAL;
  }
  if (samples && (!p.part || !p.red_keys || !p.perm_k || p.qchunk < kBT || p.qchunk % kBT)) {
    set_error("backward dk/dv: bad sample partial buffer, sort buffer, permutation or query chunk");
    return HA_EINVAL;
  }
  if (samples && static_cast<int64_t>(p.H / p.Hkv) * p.m > kRedCap) {
    set_error("backward dk/dv: (heads / kv_heads) * samples = %lld exceeds %d",
              static_cast<long long>(p.H / p.Hkv) * p.m, kRedCap);
    return HA_EUNSUPPORTED;
  }
  if (p.causal && (samples || (p.diag != 1 && p.diag != 2))) {
    set_error("backward dk/dv: causal problems take no samples and need a diagonal part");
    return HA_EINVAL;
  }
  if (!p.perm_q != !p.perm_k || (!p.perm_q && !p.causal) || (p.perm_q && p.causal)) {
    set_error("backward dk/dv: row-order problems are exactly the causal leaves");
    return HA_EINVAL;
  }
  HA_TRY(launch_gate(HA_K_BWD_DKV));
  timing_begin(HA_K_BWD_DKV, s);
  int st;
  if (p.dtype == HA_F32) st = launch_bwd32_dkv(p, samples, s);
  else if (p.d == 64) st = samples ? launch_dkv_d<64, true>(p, s) : launch_dkv_d<64, false>(p, s);
  else st = samples ? launch_dkv_d<128, true>(p, s) : launch_dkv_d<128, false>(p, s);
  timing_end(HA_K_BWD_DKV, s);
  if (st != HA_OK) return st;
  return after_launch(samples ? "backward dk/dv samples" : "backward dk/dv block", s);
}

}  // namespace ha
