// Attention kernel of the HyperAttention forward on gfx950.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary, section Approach: exact masked row sums inside
// the diagonal blocks of the sorted matrix plus uniform column sampling
// for the rest of the normaliser; section Limitations and the summary:
// recursive causal masking.)
//
// One kernel template serves every attention step:
//   * kKindSorted: a problem of `seg` sorted queries and `seg` sorted keys
//     (a whole head when non-causal, one off-diagonal quadrant of a causal
//     level): sorted query p attends the keys of its block [t b, (t+1) b),
//     t = p / b, and the m sampled key positions outside its block with
//     weight seg / m each, in one online softmax -- the log-sum-exp merge
//     of the two parts is exactly this shared softmax;
//   * kKindLeaf: exact causal attention inside a leaf (row i attends leaf
//     keys 0..i).
// Rows are loaded through the sort permutations (no gathered copies) and
// results go back to their original rows (the unsort).
//
// Work split: a workgroup of NW waves owns 32*NW consecutive sorted queries
// (32 per wave).  Keys stream through LDS in tiles of 64, double buffered:
// the next tile's rows are loaded into registers while the current one is
// computed, then written to the other buffer; one barrier per tile.  The
// key rows of a sorted problem (block keys and the samples that count) are
// listed in LDS once per workgroup, so a tile load is one global access per
// row.  Per wave and tile, S^T = K Q^T (64 keys x 32 queries) is built with
// MFMA, so each lane owns one query column (lanes l and l+32 share query
// l%32 and hold different keys).  The softmax runs on those registers, P^T
// is packed into the B operand of O^T = V^T P^T, and O^T (d x 32) stays in
// registers.  bf16 uses v_mfma_f32_32x32x16_bf16 with V row-major in LDS,
// read as the A operand with the transposing LDS read (ds_read_b64_tr_b16;
// keys permuted inside 16-key chunks to match P), and row sums taken from
// the packed bf16 P with v_dot2_f32_bf16; fp32 uses
// v_mfma_f32_32x32x2_f32.  Accumulation and softmax are fp32.
//
// Per query and key the kernel does 4 d MFMA flops (Q K^T and P V) and
// reads each of its K/V rows once per workgroup; Q rows are read once.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "ha_device.h"
#include "ha_kernels.h"

namespace ha {

constexpr int kKT = 64;                // keys per LDS tile
constexpr float kRescale = 8.f;        // log2 slack before rescaling

constexpr int align16(int x) { return (x + 15) / 16 * 16; }

template <typename T, int D, int NW, int QPW>
struct Geo {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int NT = 64 * NW;            // threads
  static constexpr int NQT = QPW / 32;          // 32-query MFMA tiles per wave
  static constexpr int TQ = QPW * NW;           // queries per workgroup
  // K rows: stride with 16-byte slots that differ mod 256 B for 16
  // consecutive rows (conflict-free 128-bit operand reads).  bf16 V rows:
  // stride = 64 B mod 256 B so the 8 rows x 64 B of one transposing read
  // fill the banks exactly twice.
  static constexpr int KSTR = BF ? D + 8 : D + 1;
  static constexpr int VSTR = BF ? D + 32 : D + 1;
  static constexpr int KBYTES = align16(kKT * KSTR * static_cast<int>(sizeof(T)));
  static constexpr int VBYTES = align16(kKT * VSTR * static_cast<int>(sizeof(T)));
  static constexpr int BUF = KBYTES + VBYTES;   // one K/V buffer
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                             // chunks per row
  static constexpr int CPT = kKT * CPR / NT;                      // chunks per thread per tensor
  static_assert(NT % CPR == 0 && (kKT * CPR) % NT == 0, "tile split");
  static_assert(QPW == 32, "one 32-query MFMA tile per wave");
};

// LDS bytes after the two K/V buffers (sorted problems): brow[bcap],
// srow[m], spos[m], rrow[m] and one count per 64 samples.
__host__ __device__ constexpr int list_bytes(int bcap, int m) { return 4 * (bcap + 3 * m + (m + 63) / 64); }

// Minimum waves per SIMD the register allocation must allow: 4 (<= 128
// VGPRs) for the bf16 d = 64 shapes of 8 waves x 32 queries, where it fits
// without spilling and measurably pays; 2 otherwise.
template <typename T, int D, int KIND, int NW, int QPW>
constexpr int min_waves() {
  return (sizeof(T) == 2 && D == 64 && NW == 8 && QPW == 32) ? 4 : 2;
}

template <typename T, int D, int KIND, int OUT, int NW, int QPW>
__global__ __launch_bounds__(64 * NW, (min_waves<T, D, KIND, NW, QPW>())) void attn_kernel(AttnParams p) {
  typedef Geo<T, D, NW, QPW> G;
  constexpr bool BF = G::BF;
  constexpr int NQT = G::NQT;
  constexpr int KC = BF ? 16 : 2;       // k per MFMA
  constexpr int NQF = D / KC;           // Q fragments per lane and query tile
  constexpr int NDT = D / 32;           // O^T tiles per query tile
  constexpr bool LEAF = KIND == kKindLeaf;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps wave-level bounds scalar
  const int h2 = lane >> 5;             // half-wave
  const int col = lane & 31;            // query column of this lane in a 32-query tile

  const int QT = (p.seg + G::TQ - 1) / G::TQ;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  int qt = lid % QT;
  if (LEAF) qt = QT - 1 - qt;           // longest causal tiles first
  const int rest = lid / QT;
  const int piece = rest % p.pieces;
  const int bh = rest / p.pieces;
  const int b = bh / p.H;
  const int hq = bh % p.H;
  const int bkv = b * p.Hkv + hq / (p.H / p.Hkv);

  const int q0 = qt * G::TQ;
  const int qend = min(q0 + G::TQ, p.seg);
  const int wq0 = q0 + wave * QPW;              // first query of this wave
  const int wq_max = wq0 + QPW - 1;             // last query of this wave
  const int64_t qpiece = static_cast<int64_t>(bh) * p.pieces + piece;    // [BH][pieces]
  const int64_t kpiece = static_cast<int64_t>(bkv) * p.pieces + piece;   // [BHkv][pieces]

  const T* qbase = static_cast<const T*>(p.q) + static_cast<int64_t>(bh) * p.n * D;
  const T* kbase = static_cast<const T*>(p.k) + static_cast<int64_t>(bkv) * p.n_k * D;
  const T* vbase = static_cast<const T*>(p.v) + static_cast<int64_t>(bkv) * p.n_k * D;
  const bool mat = !LEAF && p.qs != nullptr;   // materialised sorted copies
  const T* ksb = mat ? static_cast<const T*>(p.ks) + kpiece * p.seg_k * D : nullptr;
  const T* vsb = mat ? static_cast<const T*>(p.vs) + kpiece * p.seg_k * D : nullptr;
  // kOutRescale(Merge): sample rows come from the compact per-head copies, row = sample index
  constexpr bool RS = OUT == kOutRescale || OUT == kOutRescaleMerge;
  constexpr bool MERGE = OUT == kOutMerge || OUT == kOutRescaleMerge;
  // kOutLse: the normaliser alone (no V rows, no P V products)
  constexpr bool LO = OUT == kOutLse;
  const T* kcb = RS ? static_cast<const T*>(p.smp_k) + qpiece * p.m * D : nullptr;
  const T* vcb = RS ? static_cast<const T*>(p.smp_v) + qpiece * p.m * D : nullptr;
  const int32_t* pq = (!LEAF && p.perm_q) ? p.perm_q + qpiece * p.seg : nullptr;
  const int32_t* pk = (!LEAF && p.perm_k) ? p.perm_k + kpiece * p.seg_k : nullptr;
  const int qrow0 = p.q_first + piece * p.stride;
  const int krow0 = p.k_first + piece * p.stride;

  // ---- key ranges -------------------------------------------------------------
  int ka0 = 0, ka1 = 0;
  const bool multi_block = !LEAF && (q0 / p.b_eff) != ((qend - 1) / p.b_eff);
  if (p.use_block) {
    if (LEAF) {
      ka1 = qend;
    } else {
      // query block t pairs with key block t (key blocks of b_k; the last
      // block may be short, and a rectangular problem's may be empty)
      ka1 = min(((qend - 1) / p.b_eff + 1) * p.b_k, p.seg_k);
      ka0 = min((q0 / p.b_eff) * p.b_k, ka1);
    }
  }
  const bool samp = !LEAF && p.use_samples && p.m > 0;
  const bool samp_multi = samp && multi_block;

  // row of k/v (or of the sorted copies) holding sorted key position kp
  auto key_row = [&](int kp) -> int { return mat ? kp : (pk ? pk[kp] : krow0 + kp); };

  // ---- key row lists (sorted problems) -------------------------------------------
  // Staged in LDS once per workgroup so that loading a tile costs one global
  // access per row: brow = rows of the block keys [ka0, ka1) (when bcap > 0)
  // and srow = rows of the samples that count for the workgroup's rows.
  // When all rows share one block, the samples inside it are dropped from
  // the list (compacted in sample order); otherwise every sample is kept
  // and spos (sorted positions) serves the per-row mask.
  int* brow = reinterpret_cast<int*>(smem + 2 * G::BUF);
  int* srow = brow + p.bcap;
  int* spos = srow + p.m;
  int* rrow = spos + p.m;                 // rows before compaction
  int* ccount = rrow + p.m;               // kept samples per 64
  const bool blist = !LEAF && p.bcap > 0;
  const int nbl = ka1 - ka0;
  const int nA = ka1 > ka0 ? (nbl + kKT - 1) / kKT : 0;

  // ---- tile staging: global -> registers -> LDS ------------------------------
  const int c_in_row = tid % G::CPR;            // chunk column, fixed per thread
  const int j_first = tid / G::CPR;             // first key row of this thread
  constexpr int JSTEP = G::NT / G::CPR;
  uint4v kreg[G::CPT], vreg[G::CPT];

  // ---- prologue loads ------------------------------------------------------------
  // Issued in dependency levels so that their latencies overlap: first the
  // permutation entries (query rows, the rows of the first block tile, the
  // first list entries, sample positions), then what they address (query
  // fragments, the first tile's K/V rows, sample rows), then the LDS lists.
  // Common case (permuted rows, block list, samples): every load of a level
  // is unconditional (indices clamped into range) so the levels overlap.
  const int32_t* si = samp ? p.sidx + qpiece * p.m : nullptr;
  const bool fast = !LEAF && !mat && pq != nullptr && pk != nullptr && blist && samp && nbl > 0;
  const bool early0 = !LEAF && nA > 0;          // first tile is a block tile: load it now
  int ql[NQT], orow[NQT];   // query (sorted / local position) and its original row
  int t0row[G::CPT];
  int bl = 0, sp = 0, sr = 0;
  typedef typename std::conditional<BF, bf16x8, float>::type QF;
  QF qf[NQT][NQF];
  auto load_q = [&]() {
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
      const int qls = ql[u] < qend ? ql[u] : q0;
      const T* qb = mat ? static_cast<const T*>(p.qs) + qpiece * p.seg * D : qbase;
      const uint32_t qoff = static_cast<uint32_t>(mat ? qls : orow[u]) * (D * sizeof(T));
#pragma unroll
      for (int c = 0; c < NQF; ++c) {
        if constexpr (BF) qf[u][c] = __builtin_bit_cast(bf16x8, ld16(qb, qoff + (16 * c + 8 * h2) * 2));
        else qf[u][c] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(qb) + qoff + (2 * c + h2) * 4);
      }
    }
  };
  auto load_t0 = [&]() {
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const uint32_t off = static_cast<uint32_t>(t0row[c] * D + G::EPC * c_in_row) * sizeof(T);
      kreg[c] = ld16(mat ? ksb : kbase, off);
      if constexpr (!LO) vreg[c] = ld16(mat ? vsb : vbase, off);
    }
  };
#pragma unroll
  for (int u = 0; u < NQT; ++u) ql[u] = wq0 + 32 * u + col;
  if (fast) {
    const int kc0 = min(kKT, nbl);
#pragma unroll
    for (int u = 0; u < NQT; ++u) orow[u] = pq[ql[u] < qend ? ql[u] : q0];
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) t0row[c] = pk[ka0 + min(j_first + c * JSTEP, kc0 - 1)];
    bl = pk[ka0 + min(tid, nbl - 1)];
    sp = si[min(tid, p.m - 1)];
    load_q();
    load_t0();                                  // rows past kc0 repeat a valid row; masked
    sr = RS ? tid : pk[sp];
  } else {
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
      const int qls = ql[u] < qend ? ql[u] : q0;
      orow[u] = pq ? pq[qls] : qrow0 + qls;
    }
    if (early0) {
#pragma unroll
      for (int c = 0; c < G::CPT; ++c) t0row[c] = key_row(ka0 + min(j_first + c * JSTEP, min(kKT, nbl) - 1));
    }
    if (blist && tid < nbl) bl = key_row(ka0 + tid);
    if (samp && tid < p.m) sp = si[tid];
    load_q();
    if (early0) load_t0();
    if (samp && tid < p.m) sr = RS ? tid : key_row(sp);
  }

  int nsamp = 0;
  if (!LEAF) {
    if (blist) {
      if (tid < nbl) brow[tid] = bl;
      for (int j = tid + G::NT; j < nbl; j += G::NT) brow[j] = key_row(ka0 + j);
    }
    if (samp) {
      const int tblo = (q0 / p.b_eff) * p.b_k;   // the workgroup's key block (when it has one)
      int* raw = samp_multi ? srow : rrow;
      for (int c = 64 * wave; c < p.m; c += G::NT) {
        const int i = c + lane;
        const bool first = c == 64 * wave;     // i == tid: loaded above
        const int spi = first ? sp : (i < p.m ? si[i] : 0);
        if (i < p.m) {
          spos[i] = spi;
          raw[i] = first ? sr : (RS ? i : key_row(spi));
        }
        const uint64_t keep =
            __ballot((i < p.m) & (samp_multi | (static_cast<unsigned>(spi - tblo) >= static_cast<unsigned>(p.b_k))));
        if (lane == 0) ccount[c / 64] = __popcll(keep);
      }
      __syncthreads();
      const int nchunk = (p.m + 63) / 64;
      for (int k = 0; k < nchunk; ++k) nsamp += ccount[k];
      if (!samp_multi) {
        for (int c = 64 * wave; c < p.m; c += G::NT) {
          int base = 0;
          for (int k = 0; k < c / 64; ++k) base += ccount[k];
          const int i = c + lane;
          const bool keep = (i < p.m) && (static_cast<unsigned>(spos[i] - tblo) >= static_cast<unsigned>(p.b_k));
          const uint64_t bal = __ballot(keep);
          const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
          if (keep) srow[base + __popcll(bal & lower)] = rrow[i];
        }
      }
    }
    if (blist || samp) __syncthreads();
  }

  floatx16 o[NQT][NDT];
#pragma unroll
  for (int u = 0; u < NQT; ++u)
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[u][t][r] = 0.f;
  float mrun[NQT], lsum[NQT];   // running max (log2 units, incl. sample weight); lane's row-sum share
#pragma unroll
  for (int u = 0; u < NQT; ++u) {
    mrun[u] = -INFINITY;
    lsum[u] = 0.f;
  }
  // kept in step with mrun[0] by the one-tile bf16 body: -mrun[0], or 0
  // while the lane has no reference
  float nref = 0.f;

  const int nB = (nsamp + kKT - 1) / kKT;
  const int ntiles = nA + nB;

  // leaf rows are contiguous: per-thread base + a uniform step per tile
  const uint32_t leaf_off = static_cast<uint32_t>((krow0 + j_first) * D + G::EPC * c_in_row) * sizeof(T);
  auto load_tile = [&](int it) {
    const bool isB = it >= nA;
    const int kb = isB ? (it - nA) * kKT : ka0 + it * kKT;
    const int kcnt = isB ? min(kKT, nsamp - kb) : min(kKT, ka1 - kb);
    if constexpr (LEAF) {
      // rows past the leaf's last key repeat that key (finite values, masked)
#pragma unroll
      for (int c = 0; c < G::CPT; ++c) {
        uint32_t off;
        if (kcnt == kKT) {
          off = leaf_off + static_cast<uint32_t>((kb + c * JSTEP) * D) * sizeof(T);
        } else {
          const int j = min(j_first + c * JSTEP, kcnt - 1);
          off = static_cast<uint32_t>((krow0 + kb + j) * D + G::EPC * c_in_row) * sizeof(T);
        }
        kreg[c] = ld16(kbase, off);
        vreg[c] = ld16(vbase, off);
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const int j = j_first + c * JSTEP;
      uint4v kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (j < kcnt) {
        const int row = isB ? srow[kb + j] : (blist ? brow[kb - ka0 + j] : key_row(kb + j));
        const uint32_t off = static_cast<uint32_t>(row * D + G::EPC * c_in_row) * sizeof(T);
        kw = ld16((RS && isB) ? kcb : (mat ? ksb : kbase), off);
        if constexpr (!LO) vw = ld16((RS && isB) ? vcb : (mat ? vsb : vbase), off);
      }
      kreg[c] = kw;
      vreg[c] = vw;
    }
  };

  auto store_tile = [&](int buf) {
    T* ks = reinterpret_cast<T*>(smem + buf * G::BUF);
    T* vs = reinterpret_cast<T*>(smem + buf * G::BUF + G::KBYTES);
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
      const int j = j_first + c * JSTEP;
      if constexpr (BF) {
        *reinterpret_cast<uint4v*>(&ks[j * G::KSTR + 8 * c_in_row]) = kreg[c];
        if constexpr (!LO) *reinterpret_cast<uint4v*>(&vs[j * G::VSTR + 8 * c_in_row]) = vreg[c];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ks[j * G::KSTR + 4 * c_in_row + i] = __uint_as_float(kreg[c][i]);
          if constexpr (!LO) vs[j * G::VSTR + 4 * c_in_row + i] = __uint_as_float(vreg[c][i]);
        }
      }
    }
  };

  // transposing-read address pieces (bf16): provider lane j16 of its 16-lane
  // group supplies key offset j16 >> 2 and column offset 4 (j16 & 3)
  const int tr_key = 4 * h2 + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  if (ntiles > 0 && !early0) load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    store_tile(buf);
    __syncthreads();
    if (it + 1 < ntiles) load_tile(it + 1);

    const bool isB = it >= nA;
    const int kb = isB ? (it - nA) * kKT : ka0 + it * kKT;
    const int kcnt = isB ? min(kKT, nsamp - kb) : min(kKT, ka1 - kb);
    if (LEAF && kb > wq_max) continue;         // every key of the tile is after this wave's queries
    const T* ks = reinterpret_cast<const T*>(smem + buf * G::BUF);
    const T* vs = reinterpret_cast<const T*>(smem + buf * G::BUF + G::KBYTES);

    if constexpr (BF) {
      // ---- bf16: half-tile pipeline ------------------------------------------------
      // Keys [0, 32) and [32, 64) of the tile are two halves.  The S^T MFMAs
      // of the second half do not depend on the softmax of the first, nor
      // the P V MFMAs of the first half on the softmax of the second, so
      // each pair is issued alternately (on gfx950 this hides only part of
      // the matrix time: the two units largely take turns within a SIMD).
      // Weights are taken against the running reference mrun
      // as it stands; a half is redone after raising mrun only when some
      // lane's weights of that half sum above 2^15 (or no reference exists
      // yet), which bounds every weight while keeping the result exact.
      const bf16x2 ones = {static_cast<bf16>(1.f), static_cast<bf16>(1.f)};
      const float bias = isB ? p.log2w : 0.f;
      const bool diag = LEAF && (kb + kKT - 1 > wq0);
      const bool need_mask = kcnt < kKT || (isB ? samp_multi : (multi_block || diag));
      // a leaf half needs its mask only when it is short or reaches past the
      // wave's first query
      auto need_half = [&](int kt) {
        if constexpr (LEAF) return kcnt < 32 * (kt + 1) || kb + 32 * kt + 31 > wq0;
        return need_mask;
      };
      const int blo = LEAF ? 0 : (ql[0] / p.b_eff) * p.b_k;   // the query's key block [blo, blo + b_k)

      auto k_read = [&](int kt, int c) {
        return *reinterpret_cast<const bf16x8*>(&ks[(32 * kt + col) * G::KSTR + 16 * c + 8 * h2]);
      };
      auto v_read = [&](int c16, int t) {
        const T* vp = vs + (16 * c16 + tr_key) * G::VSTR + 32 * t + tr_col;
        const short4v lo = lds_read_tr16(vp);
        const short4v hv = lds_read_tr16(vp + 8 * G::VSTR);
        const short __attribute__((ext_vector_type(8))) va8 = {lo[0], lo[1], lo[2], lo[3], hv[0], hv[1], hv[2], hv[3]};
        return __builtin_bit_cast(bf16x8, va8);
      };
      auto mask_half = [&](int kt, floatx16& sv) {
        if constexpr (LEAF) {
          // keys j < jhi of the tile count: the tile's fill and the causal limit
          const int jhi = min(kcnt, ql[0] - kb + 1);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (!(j < jhi)) sv[r] = -INFINITY;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
            bool ok = j < kcnt;
            if (isB) {
              if (samp_multi) ok = ok && (static_cast<unsigned>(spos[kb + min(j, kcnt - 1)] - blo) >= static_cast<unsigned>(p.b_k));
            } else if (multi_block) {
              ok = ok && (static_cast<unsigned>(kb + j - blo) < static_cast<unsigned>(p.b_k));
            }
            if (!ok) sv[r] = -INFINITY;
          }
        }
      };
      auto offset = [&]() { return LEAF ? nref : bias + nref; };   // leaves carry no sample weight
      // weights of S elements i, i+1 into the B operands of the half's two
      // 16-key chunks (elements 0..7 -> pa, 8..15 -> pb), summed into l
      auto p_pair = [&](const floatx16& sv, int i, float off, bf16x8& pa, bf16x8& pb, float& l) {
        const float e0 = fast_exp2(fmaf(sv[i], kLog2e, off));
        const float e1 = fast_exp2(fmaf(sv[i + 1], kLog2e, off));
        const bf16x2 two = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){e0, e1}, bf16x2);
        l = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l, false);
        if (i < 8) {
          pa[i] = two[0];
          pa[i + 1] = two[1];
        } else {
          pb[i - 8] = two[0];
          pb[i - 7] = two[1];
        }
      };
      auto raise_half = [&](const floatx16& sv) {
        float mx = fmaxf(sv[0], sv[1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sv[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float tmax = mx * kLog2e + bias;
        const bool raise = tmax > mrun[0] + kRescale;
        if (__any(raise)) {
          const float mnew = raise ? fmaxf(mrun[0], tmax) : mrun[0];
          const float alpha = (mnew == mrun[0]) ? 1.f : fast_exp2(mrun[0] - mnew);
          if constexpr (!LO) {
#pragma unroll
            for (int t = 0; t < NDT; ++t)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[0][t][r] *= alpha;
          }
          lsum[0] *= alpha;
          mrun[0] = mnew;
          nref = mnew == -INFINITY ? 0.f : -mnew;
        }
      };
      // rare path: some lane's weights of the half outgrew the reference
      auto settle = [&](const floatx16& sv, bf16x8& pa, bf16x8& pb, float& l) {
        if (__any(!(l <= 32768.f) || mrun[0] == -INFINITY)) {
          raise_half(sv);
          const float off = offset();
          l = 0.f;
#pragma unroll
          for (int i = 0; i < 16; i += 2) p_pair(sv, i, off, pa, pb, l);
        }
        lsum[0] += l;
      };

      // phase 1: S^T of keys [0, 32)
      floatx16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
      for (int c = 0; c < NQF; ++c) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_read(0, c), qf[0][c], s0, 0, 0, 0);
      if (need_half(0)) mask_half(0, s0);

      // phase 2: S^T of keys [32, 64), each MFMA followed by a share of the
      // weights of keys [0, 32).  Written out in issue order; the
      // scheduling fences keep the compiler from regrouping it.
      bf16x8 pa, pb;
      float l0 = 0.f;
      if (it == 0) raise_half(s0);        // first tile: take the reference before any weight
      {
        const float off = offset();
        constexpr int kPer = 16 / NQF;
        bf16x8 ka = k_read(1, 0);
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
          bf16x8 kn = ka;
          if (c + 1 < NQF) kn = k_read(1, c + 1);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[0][c], s1, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = kPer * c; i < kPer * (c + 1); i += 2) p_pair(s0, i, off, pa, pb, l0);
          __builtin_amdgcn_sched_barrier(0);
          ka = kn;
        }
      }
      settle(s0, pa, pb, l0);
      if (need_half(1)) mask_half(1, s1);

      // phase 3: P V of keys [0, 32), each MFMA followed by a share of the
      // weights of keys [32, 64)
      bf16x8 pc, pd;
      float l1 = 0.f;
      {
        const float off = offset();
        constexpr int kSteps = 2 * NDT;
        constexpr int kPer = 16 / kSteps;
        if constexpr (LO) {
#pragma unroll
          for (int i = 0; i < 16; i += 2) p_pair(s1, i, off, pc, pd, l1);
        } else {
          bf16x8 va = v_read(0, 0);
#pragma unroll
          for (int st = 0; st < kSteps; ++st) {
            const int c16 = st / NDT, t = st % NDT;
            bf16x8 vn = va;
            if (st + 1 < kSteps) vn = v_read((st + 1) / NDT, (st + 1) % NDT);
            o[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, c16 == 0 ? pa : pb, o[0][t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = kPer * st; i < kPer * (st + 1); i += 2) p_pair(s1, i, off, pc, pd, l1);
            __builtin_amdgcn_sched_barrier(0);
            va = vn;
          }
        }
      }
      settle(s1, pc, pd, l1);

      // phase 4: P V of keys [32, 64)
      if constexpr (!LO) {
#pragma unroll
        for (int st = 0; st < 2 * NDT; ++st) {
          const int c16 = 2 + st / NDT, t = st % NDT;
          o[0][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_read(c16, t), c16 == 2 ? pc : pd, o[0][t], 0, 0, 0);
        }
      }
    } else {
      // ---- fp32: S^T = K Q^T for 64 keys x 32 queries ---------------------------
      floatx16 s[2][NQT];
  #pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
  #pragma unroll
        for (int u = 0; u < NQT; ++u)
  #pragma unroll
          for (int r = 0; r < 16; ++r) s[kt][u][r] = 0.f;
  #pragma unroll
        for (int c = 0; c < NQF; ++c) {
          const float ka = ks[(32 * kt + col) * G::KSTR + 2 * c + h2];
  #pragma unroll
          for (int u = 0; u < NQT; ++u)
            s[kt][u] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, qf[u][c], s[kt][u], 0, 0, 0);
        }
      }

      // ---- masks -------------------------------------------------------------------
      const bool diag = LEAF && (kb + kKT - 1 > wq0);
      const bool need_mask = kcnt < kKT || (isB ? samp_multi : (multi_block || diag));
      if (need_mask) {
  #pragma unroll
        for (int u = 0; u < NQT; ++u) {
          const int row_blk = ql[u] / p.b_eff;
  #pragma unroll
          for (int kt = 0; kt < 2; ++kt)
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
              bool ok = j < kcnt;
              if (isB) {
                if (samp_multi) ok = ok && (spos[kb + min(j, kcnt - 1)] / p.b_k) != row_blk;
              } else if (LEAF) {
                ok = ok && (kb + j <= ql[u]);
              } else if (multi_block) {
                ok = ok && ((kb + j) / p.b_k) == row_blk;
              }
              if (!ok) s[kt][u][r] = -INFINITY;
            }
        }
      }

      // ---- online softmax ------------------------------------------------------------
      // All weights of a row are taken relative to one running reference
      // mrun (log2 units, sample weight included), raised when a tile's
      // maximum exceeds it by more than 2^8.  For the causal leaves the tile
      // maximum is only computed when no reference exists yet or when a
      // tile's fresh weights sum above 2^15 on some lane; otherwise the
      // weights are used as they are (exact either way, and bounded).
      const float bias = isB ? p.log2w : 0.f;
      auto tile_max_raise = [&](int u) {
        float mx0 = fmaxf(s[0][u][0], s[0][u][1]), mx1 = fmaxf(s[1][u][0], s[1][u][1]);
  #pragma unroll
        for (int r = 2; r < 16; ++r) {
          mx0 = fmaxf(mx0, s[0][u][r]);
          mx1 = fmaxf(mx1, s[1][u][r]);
        }
        float mx = fmaxf(mx0, mx1);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float tmax = mx * kLog2e + bias;
        const bool raise = tmax > mrun[u] + kRescale;
        if (__any(raise)) {
          const float mnew = raise ? fmaxf(mrun[u], tmax) : mrun[u];
          const float alpha = (mnew == mrun[u]) ? 1.f : fast_exp2(mrun[u] - mnew);
          if constexpr (!LO) {
  #pragma unroll
            for (int t = 0; t < NDT; ++t)
  #pragma unroll
              for (int r = 0; r < 16; ++r) o[u][t][r] *= alpha;
          }
          lsum[u] *= alpha;
          mrun[u] = mnew;
        }
      };

      // ---- P, row sums and O^T += V^T P^T -----------------------------------------
      {
        tile_max_raise(0);
        const float off = bias - (mrun[0] == -INFINITY ? 0.f : mrun[0]);
  #pragma unroll
        for (int kt = 0; kt < 2; ++kt)
  #pragma unroll
          for (int jr = 0; jr < 16; ++jr) {
            const float e = fast_exp2(fmaf(s[kt][0][jr], kLog2e, off));
            lsum[0] += e;
            const int key = 32 * kt + 8 * (jr >> 2) + 4 * h2 + (jr & 3);
            if constexpr (!LO) {
  #pragma unroll
              for (int t = 0; t < NDT; ++t) {
                const float va = vs[key * G::VSTR + 32 * t + col];
                o[0][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, e, o[0][t], 0, 0, 0);
              }
            }
          }
      }
    }
  }

  // ---- epilogue -------------------------------------------------------------------
  // The result leaves through LDS so that rows are read and written in
  // 128-byte slices (8 lanes x 16 bytes per row) rather than as 16-byte
  // pieces of 32 rows per instruction: per wave and 32-dim slice t, the
  // normalised O^T (32 queries x 32 dims, fp32) is staged in the K/V
  // buffers, then lane L merges and stores dims 4 (L & 7) .. +3 of staged
  // query (L >> 3) + 8 k.
  if constexpr (LO) {
    // the lse of each query at its original row (lanes 0-31 hold the queries)
#pragma unroll
    for (int u = 0; u < NQT; ++u) {
      const float ltot = lsum[u] + __shfl_xor(lsum[u], 32);
      const bool any = ltot > 0.f;
      const float lse2 = any ? (mrun[u] + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
      if (h2 == 0 && ql[u] < qend) p.lse[static_cast<int64_t>(bh) * p.n + orow[u]] = lse2;
    }
    return;
  }
  const bool to_final = OUT == kOutFinal || OUT == kOutRescale || ((OUT == kOutLeaf || MERGE) && piece == p.final_piece);
  const bool to_acc = ((OUT == kOutLeaf || MERGE) && piece != p.final_piece) || OUT == kOutAcc;
  constexpr int SST = 36;                         // staged row stride (floats)
  constexpr int STG = 32 * SST + 64;              // floats per wave: slice, lse, rows
  static_assert(NW * STG * 4 <= 2 * G::BUF, "epilogue staging fits the K/V buffers");
  float* stg = reinterpret_cast<float*>(smem) + wave * STG;
  float* stg_lse = stg + 32 * SST;
  int* stg_row = reinterpret_cast<int*>(stg_lse + 32);
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };
  __syncthreads();                                // every wave is done with the K/V tiles
  const int c = lane & 7;                         // this lane's 4-column chunk of a slice
#pragma unroll
  for (int u = 0; u < NQT; ++u) {
    // ltot >= 1 when any key counted (the weights are relative to a running
    // reference that some counted key reached), so the hardware reciprocal
    // and base-2 logarithm (1 ulp) serve
    const float ltot = lsum[u] + __shfl_xor(lsum[u], 32);
    const bool any = ltot > 0.f;
    const float inv = any ? __builtin_amdgcn_rcpf(ltot) : 0.f;
    const float lse2 = any ? (mrun[u] + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
    // rows of the staged queries (clamped into range; `valid` marks the real ones)
    const uint64_t valid = __ballot(ql[u] < qend);
    if (h2 == 0) {
      const int qls = ql[u] < qend ? ql[u] : q0;
      stg_lse[col] = lse2;
      stg_row[col] = OUT == kOutPartial ? qls : (LEAF ? qrow0 + qls : orow[u]);
    }
    wave_sync();
    int rowk[4];
    float lqk[4];
    bool vk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int qi = (lane >> 3) + 8 * k;
      rowk[k] = stg_row[qi];
      lqk[k] = stg_lse[qi];
      vk[k] = (valid >> qi) & 1ull;
    }
    // merge: all accumulator loads of this lane are issued before any is used
    floatx4 oldv[NDT][4];
    float w_old[4], w_new[4], lse_out[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w_old[k] = 0.f;
      w_new[k] = 1.f;
      lse_out[k] = lqk[k];
    }
    float w_rs[4];
    if constexpr (RS) {
      // rescale to the normaliser stored at the row: exp(own lse - stored lse);
      // the rescaled result carries the stored lse
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lref = p.lse_ref[static_cast<int64_t>(bh) * p.n + rowk[k]];
        const bool none = lqk[k] == -INFINITY || lref == -INFINITY;
        w_rs[k] = none ? 0.f : fast_exp2((lqk[k] - lref) * kLog2e);
        if constexpr (OUT == kOutRescale) w_new[k] = w_rs[k];
        else lqk[k] = lref;
      }
    }
    if constexpr (MERGE) {
      float l1[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t ridx = static_cast<int64_t>(bh) * p.n + rowk[k];
        l1[k] = p.acc_lse[ridx];
#pragma unroll
        for (int t = 0; t < NDT; ++t) oldv[t][k] = *reinterpret_cast<const floatx4*>(p.acc_o + ridx * D + 32 * t + 4 * c);
      }
      // lse = m + ln(e^(l1 - m) + e^(l2 - m)), m = max(l1, l2): the sum lies
      // in [1, 2], so hardware exp2 / log2 / reciprocal (1 ulp) serve
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float mm = fmaxf(l1[k], lqk[k]);
        const bool none = mm == -INFINITY;
        const float ms = none ? 0.f : mm;
        const float ea = fast_exp2((l1[k] - ms) * kLog2e);
        const float eb = fast_exp2((lqk[k] - ms) * kLog2e);
        const float sum = ea + eb;
        const float r = __builtin_amdgcn_rcpf(sum);
        w_old[k] = none ? 0.f : ea * r;
        w_new[k] = none ? 0.f : eb * r;
        if constexpr (RS) w_new[k] *= w_rs[k];
        lse_out[k] = none ? -INFINITY : ms + __builtin_amdgcn_logf(sum) * kLn2;
      }
    }
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        floatx4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = o[u][t][4 * g + i] * inv;
        *reinterpret_cast<floatx4*>(stg + col * SST + 8 * g + 4 * h2) = v;
      }
      wave_sync();
      const int dc = 32 * t + 4 * c;              // 4 consecutive columns
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int qi = (lane >> 3) + 8 * k;
        floatx4 val = *reinterpret_cast<const floatx4*>(stg + qi * SST + 4 * c);
        if (!vk[k]) continue;
        // one lane per row writes the lse, on the last slice
        const bool head = t == NDT - 1 && c == 0;
        if constexpr (OUT == kOutPartial) {
          // sorted position rowk of piece `piece` at row q_first + piece stride + rowk
          const int64_t pr = static_cast<int64_t>(bh) * p.n + qrow0 + rowk[k];
          *reinterpret_cast<floatx4*>(p.part_o + pr * D + dc) = val;
          if (head) p.part_lse[pr] = lqk[k];
        } else {
          const int64_t ridx = static_cast<int64_t>(bh) * p.n + rowk[k];
          if constexpr (MERGE) {
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] = oldv[t][k][i] * w_old[k] + val[i] * w_new[k];
          }
          if constexpr (OUT == kOutRescale) {
#pragma unroll
            for (int i = 0; i < 4; ++i) val[i] *= w_new[k];
          }
          if (to_acc) {
            *reinterpret_cast<floatx4*>(p.acc_o + ridx * D + dc) = val;
            if (head) p.acc_lse[ridx] = lse_out[k];
          } else if (to_final) {
            if constexpr (BF) {
              bf16x4 ob;
#pragma unroll
              for (int i = 0; i < 4; ++i) ob[i] = static_cast<bf16>(val[i]);
              *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.out) + ridx * D + dc) = ob;
            } else {
              *reinterpret_cast<floatx4*>(static_cast<float*>(p.out) + ridx * D + dc) = val;
            }
            if (OUT != kOutRescale && head && p.lse) p.lse[ridx] = lse_out[k];
          }
        }
      }
      wave_sync();                                // before the next slice is staged
    }
  }
}

// ---- launch -----------------------------------------------------------------------

template <typename T, int D, int KIND, int OUT, int NW, int QPW>
static int launch_attn_t(const AttnParams& p, hipStream_t s) {
  typedef Geo<T, D, NW, QPW> G;
  const int64_t QT = (p.seg + G::TQ - 1) / G::TQ;
  const int64_t blocks = static_cast<int64_t>(p.BH) * p.pieces * QT;
  if (blocks > 0x7FFFFFFF) {
    set_error("attention: grid of %lld workgroups too large", static_cast<long long>(blocks));
    return HA_EUNSUPPORTED;
  }
  AttnParams q = p;
  q.bcap = 0;
  size_t lds = 2 * G::BUF;
  if (KIND == kKindSorted) {
    if (p.use_block) {
      // a workgroup's queries span at most (TQ - 1) / b_eff + 2 blocks
      const int64_t span = static_cast<int64_t>((G::TQ - 1) / p.b_eff + 2) * p.b_k;
      const int64_t cap = span < p.seg_k ? span : p.seg_k;
      if (cap <= kBlockListCap) q.bcap = static_cast<int>(cap);
    }
    lds += list_bytes(q.bcap, p.m);
  }
  if (lds > kLdsBytes) {
    set_error("attention: %zu bytes of LDS needed (%d samples, d = %d), limit %zu", lds, p.m, D, kLdsBytes);
    return HA_EUNSUPPORTED;
  }
  auto fn = attn_kernel<T, D, KIND, OUT, NW, QPW>;
  // once per instantiation (thread-safe static initialisation)
  static const hipError_t attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  HA_CHECK_HIP(attr_err);
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(G::NT), lds, s, q);
  return HA_OK;
}

size_t attention_lds_bound(int dtype, int d, int m) {
  // K/V buffers do not depend on the workgroup shape; the block key list
  // is staged only up to kBlockListCap rows
  size_t buf;
  if (dtype == HA_BF16) buf = d == 64 ? 2 * Geo<bf16, 64, 8, 32>::BUF : 2 * Geo<bf16, 128, 8, 32>::BUF;
  else buf = d == 64 ? 2 * Geo<float, 64, 8, 32>::BUF : 2 * Geo<float, 128, 8, 32>::BUF;
  return buf + static_cast<size_t>(list_bytes(kBlockListCap, m));
}

// Workgroup shape: waves x queries per wave.  HYPERATTN_SHAPE_LEAF /
// HYPERATTN_SHAPE_SORTED ("4x32", "8x32") override the default for tuning.
static int shape_override(int kind) {
  auto parse = [](const char* name) {
    const char* s = std::getenv(name);
    if (!s) return 0;
    if (!std::strcmp(s, "4x32")) return 1;
    if (!std::strcmp(s, "8x32")) return 2;
    return 0;
  };
  // read once (thread-safe static initialisation)
  static const int leaf = parse("HYPERATTN_SHAPE_LEAF"), sorted = parse("HYPERATTN_SHAPE_SORTED");
  return kind == kKindLeaf ? leaf : sorted;
}

template <typename T, int D, int KIND, int OUT>
static int launch_attn_shape(const AttnParams& p, hipStream_t s) {
  // Default (measured on MI355X): bf16 causal leaves of >= 256 rows 8
  // waves x 32 queries (d = 64: 128 VGPRs, 4 waves per SIMD; d = 128: 2
  // waves per SIMD, each K/V tile shared by twice the queries of a 4-wave
  // workgroup, which pays on long leaves); sorted problems 8 waves x 32
  // queries when the block holds >= 256 rows (all of a block's queries
  // share each K/V tile), else 4 waves x 32.
  int shape = shape_override(KIND);
  if (shape == 0) {
    if (KIND == kKindLeaf) shape = (sizeof(T) == 2 && p.seg >= 256) ? 2 : 1;
    else shape = (p.seg >= 256 && p.b_eff >= 256) ? 2 : 1;
  }
  if (shape == 2) return launch_attn_t<T, D, KIND, OUT, 8, 32>(p, s);
  return launch_attn_t<T, D, KIND, OUT, 4, 32>(p, s);
}

template <typename T, int D>
static int launch_attn_d(const AttnParams& p, hipStream_t s) {
  if (p.kind == kKindLeaf) {
    if (p.out_mode == kOutLeaf) return launch_attn_shape<T, D, kKindLeaf, kOutLeaf>(p, s);
    if (p.out_mode == kOutAcc) return launch_attn_shape<T, D, kKindLeaf, kOutAcc>(p, s);
  } else {
    if (p.out_mode == kOutFinal) return launch_attn_shape<T, D, kKindSorted, kOutFinal>(p, s);
    if (p.out_mode == kOutPartial) return launch_attn_shape<T, D, kKindSorted, kOutPartial>(p, s);
    if (p.out_mode == kOutMerge) return launch_attn_shape<T, D, kKindSorted, kOutMerge>(p, s);
    if (p.out_mode == kOutRescale) return launch_attn_shape<T, D, kKindSorted, kOutRescale>(p, s);
    if (p.out_mode == kOutRescaleMerge) return launch_attn_shape<T, D, kKindSorted, kOutRescaleMerge>(p, s);
    if (p.out_mode == kOutLse) return launch_attn_shape<T, D, kKindSorted, kOutLse>(p, s);
  }
  set_error("attention: unsupported kind %d / output mode %d", p.kind, p.out_mode);
  return HA_EINVAL;
}

int launch_attention(const AttnParams& p_in, int timing_kind, hipStream_t s) {
  AttnParams p = p_in;                       // key geometry defaults to the query side's
  if (p.n_k == 0) p.n_k = p.n;
  if (p.seg_k == 0) p.seg_k = p.seg;
  if (p.b_k == 0) p.b_k = p.b_eff;
  if (p.seg == 0 || p.BH == 0 || p.pieces == 0) return HA_OK;
  if (p.seg_k == 0 || p.b_k < 1 || (p.kind == kKindLeaf && (p.seg_k != p.seg || p.b_k != p.b_eff))) {
    set_error("attention: bad key geometry (seg_k %d, b_k %d)", p.seg_k, p.b_k);
    return HA_EINVAL;
  }
  if (p.m > kMaxSamples) {
    set_error("attention: samples %d > %d", p.m, kMaxSamples);
    return HA_EUNSUPPORTED;
  }
  if (p.out_mode == kOutLse && (!p.lse || p.qs)) {
    set_error("attention: the lse-only mode needs lse and reads rows through the permutations");
    return HA_EINVAL;
  }
  if ((p.out_mode == kOutRescale || p.out_mode == kOutRescaleMerge) &&
      (!p.lse_ref || (p.m > 0 && (!p.smp_k || !p.smp_v || !p.sidx)))) {
    set_error("attention: rescaling needs lse_ref and the sampled rows");
    return HA_EINVAL;
  }
  const int64_t head_bytes = static_cast<int64_t>(p.n > p.n_k ? p.n : p.n_k) * p.d * (p.dtype == HA_BF16 ? 2 : 4);
  if (head_bytes >= (int64_t(1) << 32)) {
    set_error("attention: one head of q/k/v spans %lld bytes (limit 4 GiB)", static_cast<long long>(head_bytes));
    return HA_EUNSUPPORTED;
  }
  HA_TRY(launch_gate(timing_kind));
  timing_begin(timing_kind, s);
  int st;
  if (p.dtype == HA_BF16) st = p.d == 64 ? launch_attn_d<bf16, 64>(p, s) : launch_attn_d<bf16, 128>(p, s);
  else st = p.d == 64 ? launch_attn_d<float, 64>(p, s) : launch_attn_d<float, 128>(p, s);
  timing_end(timing_kind, s);
  if (st != HA_OK) return st;
  return after_launch("attention", s);
}

}  // namespace ha
