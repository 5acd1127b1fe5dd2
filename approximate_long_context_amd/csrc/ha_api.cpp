// Host driver and C ABI of the HyperAttention forward.
//
// ("HyperAttention: Long-context Attention in Near-Linear Time",
// research-map summary: sections Approach and Limitations, and the summary
// line on the recursive causal-masking extension.)
//
// Non-causal forward, all on the caller's stream:
//   projections -> hash Q, hash K -> sort Q, sort K (one segment per head)
//   -> sample positions (node 1) -> fused block + sample attention with
//   the merge and the unsort in its epilogue.
// Causal forward: projections and hashes once; the exact causal leaves of
// length n / 2^L write the first leaf's rows to the output and the others
// to an fp32 accumulator; then for level l = L .. 1 (deepest first) the
// 2^(l-1) off-diagonal quadrants of that level (queries = odd halves,
// keys = even halves, each n / 2^l long) are sorted, sampled and attended
// in one batched launch each, merged into the accumulator; the rows of
// the leftmost quadrant of a level are final and go to the output.  No
// host synchronisation inside.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ha_kernels.h"
#include "ha_rng.h"

namespace ha {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

int hip_status(hipError_t e, const char* what) {
  set_error("%s failed: %s", what, hipGetErrorString(e));
  return HA_EHIP;
}

static bool sync_mode() {
  static int mode = [] {
    const char* s = std::getenv("HYPERATTN_SYNC");
    return (s && s[0] == '1') ? 1 : 0;
  }();
  return mode != 0;
}

int after_launch(const char* stage, hipStream_t stream) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("launch of %s failed: %s", stage, hipGetErrorString(e));
    return HA_EHIP;
  }
  if (sync_mode()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
      set_error("%s failed while running: %s", stage, hipGetErrorString(e));
      return HA_EHIP;
    }
  }
  return HA_OK;
}

// ---- injected failures (HYPERATTN_FAIL_AT) -----------------------------------

static const char* const kStageNames[HA_K_COUNT] = {"proj", "hash", "sort", "samples", "gather", "attend",
                                                    "merge", "leaf", "quadrant", "bwd_dq", "bwd_dkv"};

int launch_gate(int kind) {
  const char* s = std::getenv("HYPERATTN_FAIL_AT");   // read per launch: tests change it between calls
  if (s && kind >= 0 && kind < HA_K_COUNT && !std::strcmp(s, kStageNames[kind])) {
    set_error("injected failure before the %s launch (HYPERATTN_FAIL_AT)", kStageNames[kind]);
    return HA_EHIP;
  }
  return HA_OK;
}

// ---- timing hooks -----------------------------------------------------------

struct TimingRec {
  int kind;
  hipEvent_t start, stop;
};

static std::mutex g_tmu;
static bool g_timing = false;
static std::vector<TimingRec> g_recs;
static std::vector<hipEvent_t> g_event_pool;
static std::vector<size_t> g_open;   // indices of records awaiting timing_end

static hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void timing_begin(int kind, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing) return;
  TimingRec r{kind, pool_event(), pool_event()};
  if (!r.start || !r.stop) return;
  (void)hipEventRecord(r.start, s);
  g_recs.push_back(r);
  g_open.push_back(g_recs.size() - 1);
}

void timing_end(int kind, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing || g_open.empty()) return;
  size_t i = g_open.back();
  g_open.pop_back();
  if (g_recs[i].kind != kind) return;
  (void)hipEventRecord(g_recs[i].stop, s);
}

// ---- validation and planning ------------------------------------------------

struct Shape {
  int batch, n, d, heads, kv_heads, block, samples, r, causal, s, dtype, flags;
  int levels = 0;    // causal levels (every split even)
  int leaf = 0;      // causal leaf length (every split even)
  bool odd = false;  // causal: some span splits unevenly (node-by-node driver)
  int nlev = 0;      // causal: depth of the recursion (levels of quadrants)
};

static int validate(Shape& sh) {
  if (sh.dtype != HA_BF16 && sh.dtype != HA_F32) {
    set_error("dtype %d is neither HA_BF16 nor HA_F32", sh.dtype);
    return HA_EINVAL;
  }
  if (sh.batch < 0 || sh.n < 0 || sh.heads < 0 || sh.kv_heads < 0) {
    set_error("negative size");
    return HA_EINVAL;
  }
  if (sh.kv_heads == 0 || sh.heads % sh.kv_heads != 0) {
    if (!(sh.heads == 0 && sh.kv_heads == 0)) {
      set_error("heads (%d) must be a positive multiple of kv_heads (%d)", sh.heads, sh.kv_heads);
      return HA_EINVAL;
    }
  }
  if (sh.block < 1 || sh.samples < 0) {
    set_error("block must be >= 1 and samples >= 0 (block %d, samples %d)", sh.block, sh.samples);
    return HA_EINVAL;
  }
  if (sh.r < 1 || sh.r > 16) {
    set_error("proj_bits %d outside [1, 16]", sh.r);
    return HA_EINVAL;
  }
  if (sh.causal && sh.s < 1) {
    set_error("causal needs min_seq_len >= 1 (got %d)", sh.s);
    return HA_EINVAL;
  }
  if (sh.d != 64 && sh.d != 128) {
    set_error("head dim %d not built (64 or 128)", sh.d);
    return HA_EUNSUPPORTED;
  }
  if (sh.flags & ~(HA_FLAG_MATERIALIZE | HA_FLAG_UNFUSED | HA_FLAG_ROWNORM)) {
    set_error("unknown flags 0x%x", sh.flags);
    return HA_EINVAL;
  }
  if (sh.causal && (sh.flags & ~HA_FLAG_ROWNORM)) {
    set_error("flags other than HA_FLAG_ROWNORM apply to the non-causal forward only");
    return HA_EUNSUPPORTED;
  }
  if ((sh.flags & HA_FLAG_ROWNORM) && sh.flags != HA_FLAG_ROWNORM) {
    set_error("the row-norm variant takes no other flag");
    return HA_EINVAL;
  }
  if (sh.samples > kMaxSamples) {
    set_error("samples %d > %d", sh.samples, kMaxSamples);
    return HA_EUNSUPPORTED;
  }
  if (attention_lds_bound(sh.dtype, sh.d, sh.samples) > kLdsBytes) {
    set_error("%d samples need %zu bytes of LDS at this dtype and d = %d (limit %zu)", sh.samples,
              attention_lds_bound(sh.dtype, sh.d, sh.samples), sh.d, kLdsBytes);
    return HA_EUNSUPPORTED;
  }
  if (sh.n == 0) return HA_OK;
  if (!sh.causal) return HA_OK;
  // even splits all the way down: one launch per level; otherwise (an odd
  // span, split with the extra row on the right) one launch per node
  int ns = sh.n, L = 0;
  sh.odd = false;
  while (ns > sh.s) {
    if (ns % 2) sh.odd = true;
    ns = ns - ns / 2;
    ++L;
  }
  sh.levels = sh.odd ? 0 : L;
  sh.leaf = sh.odd ? 0 : ns;
  sh.nlev = L;
  return HA_OK;
}

struct Plan {
  float* R;
  uint16_t* rank_q;
  uint16_t* rank_k;
  int32_t* perm_q;
  int32_t* perm_k;
  int32_t* sidx;
  void* sort_ws;
  size_t sort_ws_bytes;
  float* acc_o;
  float* acc_lse;
  void* qs;
  void* ks;
  void* vs;
  float* part_o[3];
  float* part_lse[3];
  float* rn_w;                 // row-norm variant: squared norms of V rows [BHkv][n]
  int64_t* rn_cum;             // integer CDF per (KV head, piece)
  int32_t* rn_sidx;            // draws per (query head, piece)
  void* rn_ws;                 // CDF scratch: chunk maxima and chunk totals
  void* rn_kc;                 // drawn K rows per (query head, piece) [BH][pieces][m][d]
  void* rn_vc;                 // drawn V rows, weighted [BH][pieces][m][d]
  float* rn_lse;               // non-causal: lse when the caller passes none; causal:
                               // the plain estimator's lse at each quadrant row [BH][n]
  size_t total;
};

static bool causal_rownorm(const Shape& sh) {
  return sh.causal && (sh.flags & HA_FLAG_ROWNORM) && sh.samples > 0;
}

static Plan make_plan(const Shape& sh, void* ws, size_t cap) {
  Plan pl{};
  Carve cv(ws, cap);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  const size_t esz = sh.dtype == HA_BF16 ? 2 : 4;
  // row-norm buffers: `pieces` problems of at most `seg` keys per head
  auto take_rn = [&](int64_t pieces, int64_t seg, size_t cdf_ws) {
    pl.rn_w = cv.take<float>(BK * sh.n);
    pl.rn_cum = cv.take<int64_t>(BK * pieces * seg);
    pl.rn_sidx = cv.take<int32_t>(BH * pieces * sh.samples);
    pl.rn_ws = cv.take<char>(cdf_ws);
    pl.rn_kc = cv.take<char>(BH * pieces * sh.samples * sh.d * esz);
    pl.rn_vc = cv.take<char>(BH * pieces * sh.samples * sh.d * esz);
    pl.rn_lse = cv.take<float>(BH * sh.n);
  };
  pl.R = cv.take<float>(static_cast<size_t>(sh.r) * sh.d);
  pl.rank_q = cv.take<uint16_t>(BH * sh.n);
  pl.rank_k = cv.take<uint16_t>(BK * sh.n);
  if (!sh.causal) {
    pl.perm_q = cv.take<int32_t>(BH * sh.n);
    pl.perm_k = cv.take<int32_t>(BK * sh.n);
    pl.sidx = cv.take<int32_t>(BH * (sh.samples > 0 ? sh.samples : 1));
    pl.sort_ws_bytes = sort_ws_bytes(BH, sh.n, 1, sh.r) + sort_ws_bytes(BK, sh.n, 1, sh.r);
    pl.sort_ws = cv.take<char>(pl.sort_ws_bytes);
    const bool rn = sh.flags & HA_FLAG_ROWNORM;
    if ((sh.flags & HA_FLAG_MATERIALIZE) && !rn) {
      pl.qs = cv.take<char>(BH * sh.n * sh.d * esz);
      pl.ks = cv.take<char>(BK * sh.n * sh.d * esz);
      pl.vs = cv.take<char>(BK * sh.n * sh.d * esz);
    }
    if ((sh.flags & HA_FLAG_UNFUSED) && !rn) {
      for (int i = 0; i < 2; ++i) {
        pl.part_o[i] = cv.take<float>(BH * sh.n * sh.d);
        pl.part_lse[i] = cv.take<float>(BH * sh.n);
      }
    }
    if (rn) take_rn(1, sh.n, rownorm_cdf_ws_bytes(BK, sh.n));
  } else if (sh.odd) {
    const int half = sh.n - sh.n / 2;         // the longest quadrant side
    pl.acc_o = cv.take<float>(BH * sh.n * sh.d);
    pl.acc_lse = cv.take<float>(BH * sh.n);
    pl.perm_q = cv.take<int32_t>(BH * half);
    pl.perm_k = cv.take<int32_t>(BK * half);
    pl.sidx = cv.take<int32_t>(BH * (sh.samples > 0 ? sh.samples : 1));
    pl.sort_ws_bytes = sort_ws_bytes(BH, half, 1, sh.r) + sort_ws_bytes(BK, half, 1, sh.r);
    pl.sort_ws = cv.take<char>(pl.sort_ws_bytes);
    if (causal_rownorm(sh)) take_rn(1, half, rownorm_cdf_ws_bytes(BK, half));
  } else {
    if (sh.levels > 0) {
      pl.acc_o = cv.take<float>(BH * sh.n * sh.d);
      pl.acc_lse = cv.take<float>(BH * sh.n);
      pl.perm_q = cv.take<int32_t>(BH * (sh.n / 2));
      pl.perm_k = cv.take<int32_t>(BK * (sh.n / 2));
      const int64_t maxp = int64_t(1) << (sh.levels - 1);
      pl.sidx = cv.take<int32_t>(BH * maxp * (sh.samples > 0 ? sh.samples : 1));
      size_t mx = 0;
      for (int l = 1; l <= sh.levels; ++l) {
        const int seg = sh.n >> l;
        const int pieces = 1 << (l - 1);
        const size_t b = sort_ws_bytes(BH, seg, pieces, sh.r) + sort_ws_bytes(BK, seg, pieces, sh.r);
        if (b > mx) mx = b;
      }
      pl.sort_ws_bytes = mx;
      pl.sort_ws = cv.take<char>(mx);
      if (causal_rownorm(sh)) {
        size_t cdf = 0;
        for (int l = 1; l <= sh.levels; ++l) {
          const size_t b = rownorm_cdf_ws_bytes(BK << (l - 1), sh.n >> l);
          if (b > cdf) cdf = b;
        }
        take_rn(maxp, sh.n / 2 / maxp, cdf);
      }
    }
  }
  pl.total = align_up(cv.used, 256) + 256;
  return pl;
}

// Causal recursion node by node (some span has odd length): the exact
// leaves first, then every node's quadrant (queries [mid, hi), keys
// [lo, mid), rectangular when the span is odd) deepest first, merged into the
// accumulator.  Rows become final in the first leaf and in the quadrants of
// the nodes on the leftmost path (no shallower node holds them in its right
// half), which write the output directly.
struct CausalNode {
  int lo, mid, hi, id, depth;
  bool leftmost;                  // no shallower node holds its rows in its right half
};

// The recursion tree of a causal problem of n rows: spans of at most s rows
// are leaves; a longer span [lo, hi) splits at mid = lo + floor((hi - lo) / 2)
// (node ids: root 1, children 2 id and 2 id + 1).  Quadrants deepest first.
static void causal_nodes(int n, int s, std::vector<CausalNode>& leaves, std::vector<CausalNode>& quads) {
  std::vector<CausalNode> todo{{0, 0, n, 1, 0, true}};
  while (!todo.empty()) {
    CausalNode nd = todo.back();
    todo.pop_back();
    const int ns = nd.hi - nd.lo;
    if (ns <= s) {
      leaves.push_back(nd);
      continue;
    }
    nd.mid = nd.lo + ns / 2;
    quads.push_back(nd);
    todo.push_back({nd.lo, 0, nd.mid, 2 * nd.id, nd.depth + 1, nd.leftmost});
    todo.push_back({nd.mid, 0, nd.hi, 2 * nd.id + 1, nd.depth + 1, false});
  }
  std::stable_sort(quads.begin(), quads.end(),
                   [](const CausalNode& a, const CausalNode& b) { return a.depth > b.depth; });
}

// ---- intermediates for hyperattn_forward_debug ----------------------------------
// After the sort and sample kernels of the sorted problems of one launch
// (every piece of one level, or one node): copy their permutations and
// samples into the dump at level `lvl` (queries of piece i at row q_first +
// i * stride of the head, keys at k_first + i * stride, samples of piece i
// at node slot slot0 + i), then run the same attention kernel once with the
// block keys alone and once with the samples alone, writing the parts
// (kOutPartial) at the same rows.
static int debug_sorted(const ha_debug_dump& dd, const AttnParams& qp, const Shape& sh, int lvl, int slot0,
                        hipStream_t s) {
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  const int64_t n = sh.n;
  const int64_t P = sh.causal ? (int64_t(1) << (sh.nlev - 1)) : 1;
  const int seg_k = qp.seg_k ? qp.seg_k : qp.seg;
  // one copy row per (head, piece): pieces > 1 tile the head (pieces * stride == n)
  const int64_t pitch = qp.pieces > 1 ? qp.stride : n;
  if (qp.pieces > 1 && static_cast<int64_t>(qp.pieces) * qp.stride != n) {
    set_error("forward_debug: pieces do not tile the head");
    return HA_EINVAL;
  }
  if (dd.perm_q)
    HA_TRY(launch_copy_rows_i32(qp.perm_q, qp.seg, dd.perm_q + lvl * BH * n + qp.q_first, pitch, qp.seg,
                                BH * qp.pieces, s));
  if (dd.perm_k)
    HA_TRY(launch_copy_rows_i32(qp.perm_k, seg_k, dd.perm_k + lvl * BK * n + qp.k_first, pitch, seg_k,
                                BK * qp.pieces, s));
  if (dd.idx && sh.samples > 0)
    HA_TRY(launch_copy_rows_i32(qp.sidx, static_cast<int64_t>(qp.pieces) * sh.samples,
                                dd.idx + (lvl * BH * P + slot0) * sh.samples, P * sh.samples,
                                qp.pieces * sh.samples, BH, s));
  AttnParams pp = qp;
  pp.out_mode = kOutPartial;
  if (dd.o_blk) {
    pp.use_block = 1;
    pp.use_samples = 0;
    pp.part_o = dd.o_blk + lvl * BH * n * sh.d;
    pp.part_lse = dd.lse_blk + lvl * BH * n;
    HA_TRY(launch_attention(pp, HA_K_ATTEND, s));
  }
  if (dd.o_smp) {
    pp.use_block = 0;
    pp.use_samples = 1;
    pp.part_o = dd.o_smp + lvl * BH * n * sh.d;
    pp.part_lse = dd.lse_smp + lvl * BH * n;
    HA_TRY(launch_attention(pp, HA_K_ATTEND, s));
  }
  return HA_OK;
}

// The exact-leaf kernel once more, into the dump's o_leaf / lse_leaf.
static int debug_leaf(const ha_debug_dump& dd, const AttnParams& lp, hipStream_t s) {
  if (!dd.o_leaf) return HA_OK;
  AttnParams dp = lp;
  dp.out_mode = kOutAcc;
  dp.acc_o = dd.o_leaf;
  dp.acc_lse = dd.lse_leaf;
  return launch_attention(dp, HA_K_LEAF, s);
}

// Row-norm variant of one launch of sorted quadrant problems (every piece
// of one level, or one node; queries at q_first + i * stride, keys at
// k_first + i * stride): the plain estimator (block keys + uniform samples)
// stores its lse, ln(D_blk + D_unif), at the query rows (the lse-only
// mode: no V rows, no P V products); the pieces' draws
// (node ids node_first + i) and their K / weighted V rows are made; the
// second pass attends to the block keys plus the draws, rescales to the
// stored lse and merges into the accumulator like the plain quadrant.
static int quadrant_rownorm(AttnParams qp, const Shape& sh, const Plan& pl, int node_first, uint64_t seed,
                            hipStream_t s) {
  AttnParams p1 = qp;
  p1.out_mode = kOutLse;
  p1.lse = pl.rn_lse;
  HA_TRY(launch_attention(p1, HA_K_QUADRANT, s));
  RnGeom g;
  g.seg = qp.seg_k ? qp.seg_k : qp.seg;
  g.pieces = qp.pieces;
  g.n_head = sh.n;
  g.k_first = qp.k_first;
  g.stride = qp.stride;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  HA_TRY(launch_rownorm_cdf(pl.rn_w, qp.perm_k, BK, g, pl.rn_cum, pl.rn_ws, s));
  HA_TRY(launch_rownorm_samples(pl.rn_cum, g, node_first, seed, sh.batch, sh.heads, sh.kv_heads, sh.samples,
                                pl.rn_sidx, s));
  HA_TRY(launch_rownorm_sample_gather(qp.k, qp.v, sh.dtype, qp.perm_k, pl.rn_cum, pl.rn_sidx, g, sh.batch,
                                      sh.heads, sh.kv_heads, sh.d, sh.samples, pl.rn_kc, pl.rn_vc, s));
  qp.out_mode = kOutRescaleMerge;
  qp.sidx = pl.rn_sidx;
  qp.smp_k = pl.rn_kc;
  qp.smp_v = pl.rn_vc;
  qp.lse_ref = pl.rn_lse;
  qp.log2w = 0.f;
  return launch_attention(qp, HA_K_QUADRANT, s);
}

static int forward_causal_nodes(const AttnParams& ap, const Shape& sh, const Plan& pl, uint64_t seed,
                                hipStream_t s, const ha_debug_dump* dbg) {
  typedef CausalNode Node;
  std::vector<Node> leaves, quads;
  causal_nodes(sh.n, sh.s, leaves, quads);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  if (causal_rownorm(sh) && !quads.empty())
    HA_TRY(launch_rownorm_sqnorm(ap.v, sh.dtype, BK * sh.n, sh.d, pl.rn_w, s));
  for (const Node& nd : leaves) {
    AttnParams lp = ap;
    lp.kind = kKindLeaf;
    lp.pieces = 1;
    lp.seg = nd.hi - nd.lo;
    lp.stride = 0;
    lp.q_first = nd.lo;
    lp.k_first = nd.lo;
    lp.b_eff = lp.seg;
    lp.use_block = 1;
    lp.use_samples = 0;
    lp.out_mode = kOutLeaf;
    lp.final_piece = nd.leftmost ? 0 : -1;
    lp.acc_o = pl.acc_o;
    lp.acc_lse = pl.acc_lse;
    HA_TRY(launch_attention(lp, HA_K_LEAF, s));
    if (dbg) HA_TRY(debug_leaf(*dbg, lp, s));
  }
  for (const Node& nd : quads) {
    const int nq = nd.hi - nd.mid, nk = nd.mid - nd.lo;
    const SortJobDesc jobs[2] = {{pl.rank_q, BH, sh.n, nq, nd.mid, nq, 1, pl.perm_q},
                                 {pl.rank_k, BK, sh.n, nk, nd.lo, nk, 1, pl.perm_k}};
    HA_TRY(launch_sort_batch(jobs, 2, sh.r, pl.sort_ws, pl.sort_ws_bytes, s));
    HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, nd.id, 1, nk, sh.samples, pl.sidx, s));
    AttnParams qp = ap;
    qp.kind = kKindSorted;
    qp.pieces = 1;
    qp.seg = nq;
    qp.seg_k = nk;
    qp.q_first = nd.mid;
    qp.k_first = nd.lo;
    qp.stride = 0;
    qp.perm_q = pl.perm_q;
    qp.perm_k = pl.perm_k;
    qp.b_eff = sh.block < nq ? sh.block : nq;
    qp.b_k = static_cast<int>((static_cast<int64_t>(qp.b_eff) * nk + nq - 1) / nq);
    qp.use_block = 1;
    qp.use_samples = sh.samples > 0;
    qp.sidx = pl.sidx;
    qp.m = sh.samples;
    qp.log2w = sh.samples > 0 ? static_cast<float>(std::log2(static_cast<double>(nk) / sh.samples)) : 0.f;
    qp.out_mode = kOutMerge;
    qp.final_piece = nd.leftmost ? 0 : -1;
    qp.acc_o = pl.acc_o;
    qp.acc_lse = pl.acc_lse;
    if (dbg) HA_TRY(debug_sorted(*dbg, qp, sh, nd.depth, nd.id - (1 << nd.depth), s));
    if (causal_rownorm(sh)) HA_TRY(quadrant_rownorm(qp, sh, pl, nd.id, seed, s));
    else HA_TRY(launch_attention(qp, HA_K_QUADRANT, s));
  }
  return HA_OK;
}

// The segments of causal level l (queries [mid, hi) and keys [lo, mid) of
// every node at that depth) in one batched sort.
static int sort_causal_level(const uint16_t* rank_q, const uint16_t* rank_k, int64_t BH, int64_t BK, int n,
                             int l, int r, int32_t* perm_q, int32_t* perm_k, void* ws, size_t ws_bytes,
                             hipStream_t s) {
  const int seg = n >> l;
  const int pieces = 1 << (l - 1);
  const SortJobDesc jobs[2] = {{rank_q, BH, n, seg, seg, 2 * seg, pieces, perm_q},
                               {rank_k, BK, n, seg, 0, 2 * seg, pieces, perm_k}};
  return launch_sort_batch(jobs, 2, r, ws, ws_bytes, s);
}

static int forward_impl(const void* q, const void* k, const void* v, Shape sh, uint64_t seed,
                        void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t s,
                        const ha_debug_dump* dbg = nullptr) {
  HA_TRY(validate(sh));
  if (sh.n == 0 || sh.batch == 0 || sh.heads == 0) return HA_OK;
  if (!q || !k || !v || !out) {
    set_error("null q, k, v or out");
    return HA_EINVAL;
  }
  const Plan need = make_plan(sh, nullptr, 0);
  if (!ws || ws_bytes < need.total) {
    set_error("workspace of %zu bytes < %zu required", ws_bytes, need.total);
    return HA_EWORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256) {
    set_error("workspace must be 256-byte aligned");
    return HA_EINVAL;
  }
  const Plan pl = make_plan(sh, ws, ws_bytes);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;

  HA_TRY(launch_projections(seed, sh.d, sh.r, pl.R, s));
  HA_TRY(launch_hash(q, sh.dtype, BH * sh.n, sh.d, sh.r, pl.R, pl.rank_q, s));
  HA_TRY(launch_hash(k, sh.dtype, BK * sh.n, sh.d, sh.r, pl.R, pl.rank_k, s));

  AttnParams ap;
  ap.q = q;
  ap.k = k;
  ap.v = v;
  ap.dtype = sh.dtype;
  ap.d = sh.d;
  ap.n = sh.n;
  ap.H = sh.heads;
  ap.Hkv = sh.kv_heads;
  ap.BH = static_cast<int>(BH);
  ap.out = out;
  ap.lse = lse;

  if (!sh.causal) {
    const SortJobDesc jobs[2] = {{pl.rank_q, BH, sh.n, sh.n, 0, sh.n, 1, pl.perm_q},
                                 {pl.rank_k, BK, sh.n, sh.n, 0, sh.n, 1, pl.perm_k}};
    HA_TRY(launch_sort_batch(jobs, 2, sh.r, pl.sort_ws, pl.sort_ws_bytes, s));
    HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, 1, 1, sh.n, sh.samples, pl.sidx, s));
    ap.kind = kKindSorted;
    ap.pieces = 1;
    ap.seg = sh.n;
    ap.stride = sh.n;
    ap.perm_q = pl.perm_q;
    ap.perm_k = pl.perm_k;
    ap.b_eff = sh.block < sh.n ? sh.block : sh.n;
    ap.sidx = pl.sidx;
    ap.m = sh.samples;
    ap.log2w = sh.samples > 0 ? static_cast<float>(std::log2(static_cast<double>(sh.n) / sh.samples)) : 0.f;
    if (sh.flags & HA_FLAG_ROWNORM) {
      // pass 1 (lse only: no V rows, no P V products): the plain estimator
      // (block + uniform samples) stores lse = ln(D_blk + D_unif); pass 2: block keys + row-norm draws (K and
      // weighted V rows copied per head) rescaled to that normaliser
      float* lse1 = lse ? lse : pl.rn_lse;
      ap.lse = lse1;
      if (sh.samples == 0) {                    // no draws: the numerator is the block part alone
        ap.out_mode = kOutFinal;
        return launch_attention(ap, HA_K_ATTEND, s);
      }
      ap.out_mode = kOutLse;
      HA_TRY(launch_attention(ap, HA_K_ATTEND, s));
      HA_TRY(launch_rownorm_sqnorm(v, sh.dtype, BK * sh.n, sh.d, pl.rn_w, s));
      RnGeom g;
      g.seg = sh.n;
      g.n_head = sh.n;
      HA_TRY(launch_rownorm_cdf(pl.rn_w, pl.perm_k, BK, g, pl.rn_cum, pl.rn_ws, s));
      HA_TRY(launch_rownorm_samples(pl.rn_cum, g, 1, seed, sh.batch, sh.heads, sh.kv_heads, sh.samples,
                                    pl.rn_sidx, s));
      HA_TRY(launch_rownorm_sample_gather(k, v, sh.dtype, pl.perm_k, pl.rn_cum, pl.rn_sidx, g, sh.batch, sh.heads,
                                          sh.kv_heads, sh.d, sh.samples, pl.rn_kc, pl.rn_vc, s));
      ap.out_mode = kOutRescale;
      ap.lse_ref = lse1;
      ap.sidx = pl.rn_sidx;
      ap.smp_k = pl.rn_kc;
      ap.smp_v = pl.rn_vc;
      ap.log2w = 0.f;
      return launch_attention(ap, HA_K_ATTEND, s);
    }
    if (sh.flags & HA_FLAG_MATERIALIZE) {
      HA_TRY(launch_gather(q, sh.dtype, BH, sh.n, sh.d, pl.perm_q, sh.n, pl.qs, s));
      HA_TRY(launch_gather(k, sh.dtype, BK, sh.n, sh.d, pl.perm_k, sh.n, pl.ks, s));
      HA_TRY(launch_gather(v, sh.dtype, BK, sh.n, sh.d, pl.perm_k, sh.n, pl.vs, s));
      ap.qs = pl.qs;
      ap.ks = pl.ks;
      ap.vs = pl.vs;
    }
    if (sh.flags & HA_FLAG_UNFUSED) {
      ap.out_mode = kOutPartial;
      ap.use_block = 1;
      ap.use_samples = 0;
      ap.part_o = pl.part_o[0];
      ap.part_lse = pl.part_lse[0];
      HA_TRY(launch_attention(ap, HA_K_ATTEND, s));
      ap.use_block = 0;
      ap.use_samples = 1;
      ap.part_o = pl.part_o[1];
      ap.part_lse = pl.part_lse[1];
      HA_TRY(launch_attention(ap, HA_K_ATTEND, s));
      return launch_merge_unsort(pl.part_o[0], pl.part_lse[0], pl.part_o[1], pl.part_lse[1],
                                 pl.perm_q, BH, sh.n, sh.d, sh.dtype, out, lse, s);
    }
    ap.out_mode = kOutFinal;
    ap.use_block = 1;
    ap.use_samples = sh.samples > 0;
    if (dbg) HA_TRY(debug_sorted(*dbg, ap, sh, 0, 0, s));
    return launch_attention(ap, HA_K_ATTEND, s);
  }

  // ---- causal ----
  if (sh.odd) return forward_causal_nodes(ap, sh, pl, seed, s, dbg);
  AttnParams lp = ap;
  lp.kind = kKindLeaf;
  lp.pieces = sh.n / sh.leaf;
  lp.seg = sh.leaf;
  lp.stride = sh.leaf;
  lp.b_eff = sh.leaf;
  lp.use_block = 1;
  lp.use_samples = 0;
  lp.out_mode = kOutLeaf;
  lp.acc_o = pl.acc_o;
  lp.acc_lse = pl.acc_lse;
  HA_TRY(launch_attention(lp, HA_K_LEAF, s));
  if (dbg) HA_TRY(debug_leaf(*dbg, lp, s));
  if (causal_rownorm(sh) && sh.levels > 0)
    HA_TRY(launch_rownorm_sqnorm(v, sh.dtype, BK * sh.n, sh.d, pl.rn_w, s));

  for (int l = sh.levels; l >= 1; --l) {
    const int seg = sh.n >> l;
    const int pieces = 1 << (l - 1);
    HA_TRY(sort_causal_level(pl.rank_q, pl.rank_k, BH, BK, sh.n, l, sh.r, pl.perm_q, pl.perm_k, pl.sort_ws,
                             pl.sort_ws_bytes, s));
    HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, pieces, pieces, seg, sh.samples,
                                 pl.sidx, s));
    AttnParams qp = ap;
    qp.kind = kKindSorted;
    qp.pieces = pieces;
    qp.seg = seg;
    qp.q_first = seg;
    qp.k_first = 0;
    qp.stride = 2 * seg;
    qp.perm_q = pl.perm_q;
    qp.perm_k = pl.perm_k;
    qp.b_eff = sh.block < seg ? sh.block : seg;
    qp.use_block = 1;
    qp.use_samples = sh.samples > 0;
    qp.sidx = pl.sidx;
    qp.m = sh.samples;
    qp.log2w = sh.samples > 0 ? static_cast<float>(std::log2(static_cast<double>(seg) / sh.samples)) : 0.f;
    qp.out_mode = kOutMerge;
    qp.acc_o = pl.acc_o;
    qp.acc_lse = pl.acc_lse;
    if (dbg) HA_TRY(debug_sorted(*dbg, qp, sh, l - 1, 0, s));
    if (causal_rownorm(sh)) HA_TRY(quadrant_rownorm(qp, sh, pl, pieces, seed, s));
    else HA_TRY(launch_attention(qp, HA_K_QUADRANT, s));
  }
  return HA_OK;
}


// ---- rectangular non-causal problems ----------------------------------------------
// n_q queries and n_k keys per head: query blocks of b_eff = min(block, n_q)
// sorted positions, key blocks of b_k = ceil(b_eff n_k / n_q), query block t
// paired with key block t; samples uniform over the n_k keys, weight n_k / m.

struct RectPlan {
  float* R;
  uint16_t* rank_q;
  uint16_t* rank_k;
  int32_t* perm_q;
  int32_t* perm_k;
  int32_t* sidx;
  void* sort_ws;
  size_t sort_ws_bytes;
  size_t total;
};

static RectPlan rect_plan(const Shape& sh, int n_k, void* ws, size_t cap) {
  RectPlan pl{};
  Carve cv(ws, cap);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  pl.R = cv.take<float>(static_cast<size_t>(sh.r) * sh.d);
  pl.rank_q = cv.take<uint16_t>(BH * sh.n);
  pl.rank_k = cv.take<uint16_t>(BK * n_k);
  pl.perm_q = cv.take<int32_t>(BH * sh.n);
  pl.perm_k = cv.take<int32_t>(BK * n_k);
  pl.sidx = cv.take<int32_t>(BH * (sh.samples > 0 ? sh.samples : 1));
  pl.sort_ws_bytes = sort_ws_bytes(BH, sh.n, 1, sh.r) + sort_ws_bytes(BK, n_k, 1, sh.r);
  pl.sort_ws = cv.take<char>(pl.sort_ws_bytes);
  pl.total = align_up(cv.used, 256) + 256;
  return pl;
}

static int rect_validate(Shape& sh, int n_k) {
  HA_TRY(validate(sh));
  if (n_k < 0 || (sh.n > 0 && n_k == 0)) {
    set_error("rectangular problem: n_k = %d (queries need keys)", n_k);
    return HA_EINVAL;
  }
  if (static_cast<int64_t>(n_k) * sh.d * 4 >= (int64_t(1) << 32) ||
      static_cast<int64_t>(sh.n) * sh.d * 4 >= (int64_t(1) << 32)) {
    set_error("rectangular problem: one head spans 4 GiB or more");
    return HA_EUNSUPPORTED;
  }
  return HA_OK;
}

static int forward_rect_impl(const void* q, const void* k, const void* v, Shape sh, int n_k, uint64_t seed,
                             void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t s) {
  HA_TRY(rect_validate(sh, n_k));
  if (sh.n == 0 || sh.batch == 0 || sh.heads == 0) return HA_OK;
  if (!q || !k || !v || !out) {
    set_error("null q, k, v or out");
    return HA_EINVAL;
  }
  const size_t need = rect_plan(sh, n_k, nullptr, 0).total;
  if (!ws || ws_bytes < need) {
    set_error("workspace of %zu bytes < %zu required", ws_bytes, need);
    return HA_EWORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256) {
    set_error("workspace must be 256-byte aligned");
    return HA_EINVAL;
  }
  const RectPlan pl = rect_plan(sh, n_k, ws, ws_bytes);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  HA_TRY(launch_projections(seed, sh.d, sh.r, pl.R, s));
  HA_TRY(launch_hash(q, sh.dtype, BH * sh.n, sh.d, sh.r, pl.R, pl.rank_q, s));
  HA_TRY(launch_hash(k, sh.dtype, BK * n_k, sh.d, sh.r, pl.R, pl.rank_k, s));
  const SortJobDesc jobs[2] = {{pl.rank_q, BH, sh.n, sh.n, 0, sh.n, 1, pl.perm_q},
                               {pl.rank_k, BK, n_k, n_k, 0, n_k, 1, pl.perm_k}};
  HA_TRY(launch_sort_batch(jobs, 2, sh.r, pl.sort_ws, pl.sort_ws_bytes, s));
  HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, 1, 1, n_k, sh.samples, pl.sidx, s));
  AttnParams ap;
  ap.q = q;
  ap.k = k;
  ap.v = v;
  ap.dtype = sh.dtype;
  ap.d = sh.d;
  ap.n = sh.n;
  ap.n_k = n_k;
  ap.H = sh.heads;
  ap.Hkv = sh.kv_heads;
  ap.BH = static_cast<int>(BH);
  ap.kind = kKindSorted;
  ap.pieces = 1;
  ap.seg = sh.n;
  ap.seg_k = n_k;
  ap.stride = sh.n;
  ap.perm_q = pl.perm_q;
  ap.perm_k = pl.perm_k;
  ap.b_eff = sh.block < sh.n ? sh.block : sh.n;
  ap.b_k = static_cast<int>((static_cast<int64_t>(ap.b_eff) * n_k + sh.n - 1) / sh.n);
  ap.sidx = pl.sidx;
  ap.m = sh.samples;
  ap.log2w = sh.samples > 0 ? static_cast<float>(std::log2(static_cast<double>(n_k) / sh.samples)) : 0.f;
  ap.out_mode = kOutFinal;
  ap.out = out;
  ap.lse = lse;
  ap.use_block = 1;
  ap.use_samples = sh.samples > 0;
  return launch_attention(ap, HA_K_ATTEND, s);
}

// ---- backward -------------------------------------------------------------------
// Same projections, hashes, sorts and samples as the forward (recomputed
// from the seed), then the per-row statistics (lse, D = rowsum(dO * O)) and,
// for every problem the forward solved, dQ, the block part of dK / dV and
// the sample part of dK / dV.  Non-causal: one problem per head (dQ and the
// block part stored, the sample part added).  Causal: the exact leaves first
// (dQ stored; dK / dV of each key's own 256-query square stored, the later
// queries added), then every level's quadrant problems, all added.

struct BwdPlan {
  float* R;
  uint16_t* rank_q;
  uint16_t* rank_k;
  int32_t* perm_q;
  int32_t* perm_k;
  int32_t* sidx;
  void* sort_ws;
  size_t sort_ws_bytes;
  float* qstat;
  float* part;
  uint64_t* red_keys;
  size_t total;
};

static int64_t bwd_part_floats(int64_t BH, int seg, int pieces, int m, int d) {
  const int qc = bwd_query_chunk(seg);
  return static_cast<int64_t>((seg + qc - 1) / qc) * BH * pieces * m * 2 * d;
}

static BwdPlan backward_plan(const Shape& sh, void* ws, size_t cap) {
  BwdPlan pl{};
  Carve cv(ws, cap);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  const int m1 = sh.samples > 0 ? sh.samples : 1;
  pl.R = cv.take<float>(static_cast<size_t>(sh.r) * sh.d);
  pl.rank_q = cv.take<uint16_t>(BH * sh.n);
  pl.rank_k = cv.take<uint16_t>(BK * sh.n);
  pl.qstat = cv.take<float>(2 * BH * sh.n);
  if (!sh.causal) {
    pl.perm_q = cv.take<int32_t>(BH * sh.n);
    pl.perm_k = cv.take<int32_t>(BK * sh.n);
    pl.sidx = cv.take<int32_t>(BH * m1);
    pl.sort_ws_bytes = sort_ws_bytes(BH, sh.n, 1, sh.r) + sort_ws_bytes(BK, sh.n, 1, sh.r);
    pl.sort_ws = cv.take<char>(pl.sort_ws_bytes);
    pl.part = cv.take<float>(bwd_part_floats(BH, sh.n, 1, sh.samples, sh.d));
    pl.red_keys = cv.take<uint64_t>(BH * m1);
  } else if (sh.levels > 0) {
    pl.perm_q = cv.take<int32_t>(BH * (sh.n / 2));
    pl.perm_k = cv.take<int32_t>(BK * (sh.n / 2));
    pl.sidx = cv.take<int32_t>(BH * (int64_t(1) << (sh.levels - 1)) * m1);
    size_t mx = 0;
    int64_t part = 0;
    for (int l = 1; l <= sh.levels; ++l) {
      const int seg = sh.n >> l;
      const int pieces = 1 << (l - 1);
      const size_t b = sort_ws_bytes(BH, seg, pieces, sh.r) + sort_ws_bytes(BK, seg, pieces, sh.r);
      if (b > mx) mx = b;
      const int64_t f = bwd_part_floats(BH, seg, pieces, sh.samples, sh.d);
      if (f > part) part = f;
    }
    pl.sort_ws_bytes = mx;
    pl.sort_ws = cv.take<char>(mx);
    pl.part = cv.take<float>(part);
    pl.red_keys = cv.take<uint64_t>(BH * (int64_t(1) << (sh.levels - 1)) * m1);
  } else if (sh.odd) {
    const int half = sh.n - sh.n / 2;           // the longest quadrant side
    pl.perm_q = cv.take<int32_t>(BH * half);
    pl.perm_k = cv.take<int32_t>(BK * half);
    pl.sidx = cv.take<int32_t>(BH * m1);
    pl.sort_ws_bytes = sort_ws_bytes(BH, half, 1, sh.r) + sort_ws_bytes(BK, half, 1, sh.r);
    pl.sort_ws = cv.take<char>(pl.sort_ws_bytes);
    pl.part = cv.take<float>(bwd_part_floats(BH, half, 1, sh.samples, sh.d));
    pl.red_keys = cv.take<uint64_t>(BH * m1);
  }
  pl.total = align_up(cv.used, 256) + 256;
  return pl;
}

static int backward_impl(const void* q, const void* k, const void* v, const void* out, const float* lse,
                         const void* dout, Shape sh, uint64_t seed, float* dq, float* dk, float* dv, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  HA_TRY(validate(sh));
  if (sh.flags) {
    set_error("backward takes no flags");
    return HA_EINVAL;
  }
  if (sh.kv_heads > 0 && static_cast<int64_t>(sh.heads / sh.kv_heads) * sh.samples > kBwdMaxGroupSamples) {
    set_error("backward: (heads / kv_heads) * samples = %lld exceeds %d",
              static_cast<long long>(sh.heads / sh.kv_heads) * sh.samples, kBwdMaxGroupSamples);
    return HA_EUNSUPPORTED;
  }
  if (sh.n == 0 || sh.batch == 0 || sh.heads == 0) return HA_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) {
    set_error("null pointer argument");
    return HA_EINVAL;
  }
  const size_t need = backward_plan(sh, nullptr, 0).total;
  if (!ws || ws_bytes < need) {
    set_error("workspace of %zu bytes < %zu required", ws_bytes, need);
    return HA_EWORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256) {
    set_error("workspace must be 256-byte aligned");
    return HA_EINVAL;
  }
  if (static_cast<int64_t>(sh.n) * sh.d * (sh.dtype == HA_BF16 ? 2 : 4) >= (int64_t(1) << 32)) {
    set_error("backward: one head of q/k/v spans 4 GiB or more");
    return HA_EUNSUPPORTED;
  }
  const BwdPlan pl = backward_plan(sh, ws, ws_bytes);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  HA_TRY(launch_projections(seed, sh.d, sh.r, pl.R, s));
  HA_TRY(launch_hash(q, sh.dtype, BH * sh.n, sh.d, sh.r, pl.R, pl.rank_q, s));
  HA_TRY(launch_hash(k, sh.dtype, BK * sh.n, sh.d, sh.r, pl.R, pl.rank_k, s));

  BwdParams bp;
  bp.dtype = sh.dtype;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.out = out;
  bp.dout = dout;
  bp.lse = lse;
  bp.qstat = pl.qstat;
  bp.d = sh.d;
  bp.n = sh.n;
  bp.H = sh.heads;
  bp.Hkv = sh.kv_heads;
  bp.BH = static_cast<int>(BH);
  bp.part = pl.part;
  bp.red_keys = pl.red_keys;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  HA_TRY(launch_bwd_qstat(bp, s));

  // one sorted problem per piece: queries [p stride + q_first, + seg), keys
  // [p stride + k_first, + seg_k); query blocks of b_eff = min(block, seg) pair
  // with key blocks of ceil(b_eff seg_k / seg), samples weigh seg_k / m
  auto sorted_problems = [&](int seg, int pieces, int q_first, int k_first, int stride, int accumulate,
                             const int32_t* perm_q, const int32_t* perm_k, int seg_k) -> int {
    BwdParams qp = bp;
    qp.pieces = pieces;
    qp.seg = seg;
    qp.seg_k = seg_k;
    qp.stride = stride;
    qp.q_first = q_first;
    qp.k_first = k_first;
    qp.perm_q = perm_q;
    qp.perm_k = perm_k;
    qp.sidx = pl.sidx;
    qp.m = sh.samples;
    qp.log2w = sh.samples > 0 ? static_cast<float>(std::log2(static_cast<double>(seg_k) / sh.samples)) : 0.f;
    qp.b_eff = sh.block < seg ? sh.block : seg;
    qp.b_k = static_cast<int>((static_cast<int64_t>(qp.b_eff) * seg_k + seg - 1) / seg);
    qp.qchunk = bwd_query_chunk(seg);
    qp.accumulate = accumulate;
    HA_TRY(launch_bwd_dq(qp, s));
    HA_TRY(launch_bwd_dkv(qp, false, s));
    return launch_bwd_dkv(qp, true, s);
  };

  if (!sh.causal) {
    const SortJobDesc jobs[2] = {{pl.rank_q, BH, sh.n, sh.n, 0, sh.n, 1, pl.perm_q},
                                 {pl.rank_k, BK, sh.n, sh.n, 0, sh.n, 1, pl.perm_k}};
    HA_TRY(launch_sort_batch(jobs, 2, sh.r, pl.sort_ws, pl.sort_ws_bytes, s));
    HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, 1, 1, sh.n, sh.samples, pl.sidx, s));
    return sorted_problems(sh.n, 1, 0, 0, sh.n, 0, pl.perm_q, pl.perm_k, sh.n);
  }

  if (sh.odd) {
    // node by node: the exact leaves (each row in one leaf, so they store),
    // then every quadrant (rectangular when its span is odd), accumulated
    std::vector<CausalNode> leaves, quads;
    causal_nodes(sh.n, sh.s, leaves, quads);
    for (const CausalNode& nd : leaves) {
      BwdParams lp = bp;
      lp.pieces = 1;
      lp.seg = nd.hi - nd.lo;
      lp.stride = 0;
      lp.q_first = nd.lo;
      lp.k_first = nd.lo;
      lp.b_eff = lp.seg;
      lp.causal = 1;
      HA_TRY(launch_bwd_dq(lp, s));
      lp.diag = 2;
      HA_TRY(launch_bwd_dkv(lp, false, s));
      lp.diag = 1;
      lp.accumulate = 1;
      HA_TRY(launch_bwd_dkv(lp, false, s));
    }
    for (const CausalNode& nd : quads) {
      const int nq = nd.hi - nd.mid, nk = nd.mid - nd.lo;
      const SortJobDesc jobs[2] = {{pl.rank_q, BH, sh.n, nq, nd.mid, nq, 1, pl.perm_q},
                                   {pl.rank_k, BK, sh.n, nk, nd.lo, nk, 1, pl.perm_k}};
      HA_TRY(launch_sort_batch(jobs, 2, sh.r, pl.sort_ws, pl.sort_ws_bytes, s));
      HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, nd.id, 1, nk, sh.samples, pl.sidx, s));
      HA_TRY(sorted_problems(nq, 1, nd.mid, nd.lo, 0, 1, pl.perm_q, pl.perm_k, nk));
    }
    return HA_OK;
  }

  // exact causal leaves, rows in their own order
  BwdParams lp = bp;
  lp.pieces = sh.n / sh.leaf;
  lp.seg = sh.leaf;
  lp.stride = sh.leaf;
  lp.b_eff = sh.leaf;
  lp.causal = 1;
  HA_TRY(launch_bwd_dq(lp, s));
  lp.diag = 2;
  HA_TRY(launch_bwd_dkv(lp, false, s));
  lp.diag = 1;
  lp.accumulate = 1;
  HA_TRY(launch_bwd_dkv(lp, false, s));

  // quadrant problems of every level: queries [mid, hi), keys [lo, mid) of each node
  for (int l = sh.levels; l >= 1; --l) {
    const int seg = sh.n >> l;
    const int pieces = 1 << (l - 1);
    HA_TRY(sort_causal_level(pl.rank_q, pl.rank_k, BH, BK, sh.n, l, sh.r, pl.perm_q, pl.perm_k, pl.sort_ws,
                             pl.sort_ws_bytes, s));
    HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, pieces, pieces, seg, sh.samples, pl.sidx, s));
    HA_TRY(sorted_problems(seg, pieces, seg, 0, 2 * seg, 1, pl.perm_q, pl.perm_k, seg));
  }
  return HA_OK;
}

// ---- backward of a rectangular non-causal problem -----------------------------------
// n_q queries, n_k keys per head; the forward's geometry (query blocks of
// b_eff = min(block, n_q), key blocks of ceil(b_eff n_k / n_q), samples over
// the n_k keys with weight n_k / m).

static BwdPlan backward_rect_plan(const Shape& sh, int n_k, void* ws, size_t cap) {
  BwdPlan pl{};
  Carve cv(ws, cap);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  const int m1 = sh.samples > 0 ? sh.samples : 1;
  pl.R = cv.take<float>(static_cast<size_t>(sh.r) * sh.d);
  pl.rank_q = cv.take<uint16_t>(BH * sh.n);
  pl.rank_k = cv.take<uint16_t>(BK * n_k);
  pl.qstat = cv.take<float>(2 * BH * sh.n);
  pl.perm_q = cv.take<int32_t>(BH * sh.n);
  pl.perm_k = cv.take<int32_t>(BK * n_k);
  pl.sidx = cv.take<int32_t>(BH * m1);
  pl.sort_ws_bytes = sort_ws_bytes(BH, sh.n, 1, sh.r) + sort_ws_bytes(BK, n_k, 1, sh.r);
  pl.sort_ws = cv.take<char>(pl.sort_ws_bytes);
  pl.part = cv.take<float>(bwd_part_floats(BH, sh.n, 1, sh.samples, sh.d));
  pl.red_keys = cv.take<uint64_t>(BH * m1);
  pl.total = align_up(cv.used, 256) + 256;
  return pl;
}

static int backward_rect_impl(const void* q, const void* k, const void* v, const void* out, const float* lse,
                              const void* dout, Shape sh, int n_k, uint64_t seed, float* dq, float* dk, float* dv,
                              void* ws, size_t ws_bytes, hipStream_t s) {
  HA_TRY(rect_validate(sh, n_k));
  if (sh.kv_heads > 0 && static_cast<int64_t>(sh.heads / sh.kv_heads) * sh.samples > kBwdMaxGroupSamples) {
    set_error("backward: (heads / kv_heads) * samples = %lld exceeds %d",
              static_cast<long long>(sh.heads / sh.kv_heads) * sh.samples, kBwdMaxGroupSamples);
    return HA_EUNSUPPORTED;
  }
  if (sh.n == 0 || sh.batch == 0 || sh.heads == 0) return HA_OK;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) {
    set_error("null pointer argument");
    return HA_EINVAL;
  }
  const size_t need = backward_rect_plan(sh, n_k, nullptr, 0).total;
  if (!ws || ws_bytes < need) {
    set_error("workspace of %zu bytes < %zu required", ws_bytes, need);
    return HA_EWORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256) {
    set_error("workspace must be 256-byte aligned");
    return HA_EINVAL;
  }
  const BwdPlan pl = backward_rect_plan(sh, n_k, ws, ws_bytes);
  const int64_t BH = static_cast<int64_t>(sh.batch) * sh.heads;
  const int64_t BK = static_cast<int64_t>(sh.batch) * sh.kv_heads;
  HA_TRY(launch_projections(seed, sh.d, sh.r, pl.R, s));
  HA_TRY(launch_hash(q, sh.dtype, BH * sh.n, sh.d, sh.r, pl.R, pl.rank_q, s));
  HA_TRY(launch_hash(k, sh.dtype, BK * n_k, sh.d, sh.r, pl.R, pl.rank_k, s));
  const SortJobDesc jobs[2] = {{pl.rank_q, BH, sh.n, sh.n, 0, sh.n, 1, pl.perm_q},
                               {pl.rank_k, BK, n_k, n_k, 0, n_k, 1, pl.perm_k}};
  HA_TRY(launch_sort_batch(jobs, 2, sh.r, pl.sort_ws, pl.sort_ws_bytes, s));
  HA_TRY(launch_sample_indices(seed, sh.batch, sh.heads, 1, 1, n_k, sh.samples, pl.sidx, s));

  BwdParams bp;
  bp.dtype = sh.dtype;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.out = out;
  bp.dout = dout;
  bp.lse = lse;
  bp.qstat = pl.qstat;
  bp.d = sh.d;
  bp.n = sh.n;
  bp.n_k = n_k;
  bp.H = sh.heads;
  bp.Hkv = sh.kv_heads;
  bp.BH = static_cast<int>(BH);
  bp.part = pl.part;
  bp.red_keys = pl.red_keys;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  HA_TRY(launch_bwd_qstat(bp, s));
  bp.pieces = 1;
  bp.seg = sh.n;
  bp.seg_k = n_k;
  bp.stride = 0;
  bp.perm_q = pl.perm_q;
  bp.perm_k = pl.perm_k;
  bp.sidx = pl.sidx;
  bp.m = sh.samples;
  bp.log2w = sh.samples > 0 ? static_cast<float>(std::log2(static_cast<double>(n_k) / sh.samples)) : 0.f;
  bp.b_eff = sh.block < sh.n ? sh.block : sh.n;
  bp.b_k = static_cast<int>((static_cast<int64_t>(bp.b_eff) * n_k + sh.n - 1) / sh.n);
  bp.qchunk = bwd_query_chunk(sh.n);
  bp.accumulate = 0;
  HA_TRY(launch_bwd_dq(bp, s));
  HA_TRY(launch_bwd_dkv(bp, false, s));
  return launch_bwd_dkv(bp, true, s);
}

// ---- allocation-free forward ----------------------------------------------------
// The workspace of hyperattn_forward_noalloc is a device array of the library
// itself: one copy per GPU, created by the loader with the code object and
// held until the process ends.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept per device.  No kernel of the
// forward needs the array zeroed (every workspace buffer is written before
// it is read within a call), so nothing is cleared between calls.

}  // namespace ha

static __device__ __align__(256) char scratch[HA_NOALLOC_SCRATCH_BYTES];

namespace ha {

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];

static int scratch_address(void** out) {
  int dev = -1;
  HA_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("forward_noalloc: device %d outside the %d the library tracks", dev, kMaxDevices);
    return HA_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256) {
      set_error("forward_noalloc: scratch array at %p is not 256-byte aligned", ptr);
      return HA_EHIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return HA_OK;
}

static int forward_noalloc_impl(const void* q, const void* k, const void* v, Shape sh, uint64_t seed, void* out,
                                float* lse, hipStream_t s) {
  HA_TRY(validate(sh));
  if (sh.n == 0 || sh.batch == 0 || sh.heads == 0) return HA_OK;
  if (!q || !k || !v || !out) {
    set_error("null q, k, v or out");
    return HA_EINVAL;
  }
  const size_t need = make_plan(sh, nullptr, 0).total;
  if (need > HA_NOALLOC_SCRATCH_BYTES) {
    set_error("forward_noalloc: these sizes need %zu bytes of workspace, more than the %zu-byte scratch array",
              need, static_cast<size_t>(HA_NOALLOC_SCRATCH_BYTES));
    return HA_EWORKSPACE;
  }
  void* ws = nullptr;
  HA_TRY(scratch_address(&ws));
  return forward_impl(q, k, v, sh, seed, out, lse, ws, HA_NOALLOC_SCRATCH_BYTES, s);
}

}  // namespace ha

using namespace ha;

extern "C" {

const char* hyperattn_last_error(void) { return g_last_error.c_str(); }

const char* hyperattn_version(void) { return "hyperattn-gfx950 0.1"; }

size_t hyperattn_workspace_bytes(int batch, int n, int d, int heads, int kv_heads, int block,
                                 int samples, int proj_bits, int causal, int min_seq_len,
                                 int dtype, int flags) {
  Shape sh{batch, n, d, heads, kv_heads, block, samples, proj_bits, causal, min_seq_len, dtype, flags};
  if (validate(sh) != HA_OK) return 0;
  return make_plan(sh, nullptr, 0).total;
}

int hyperattn_forward_ex(const void* q, const void* k, const void* v, int dtype, int batch, int n,
                         int d, int heads, int kv_heads, int block, int samples, int proj_bits,
                         int causal, int min_seq_len, uint64_t seed, int flags, void* out,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Shape sh{batch, n, d, heads, kv_heads, block, samples, proj_bits, causal, min_seq_len, dtype, flags};
  return forward_impl(q, k, v, sh, seed, out, lse, workspace, workspace_bytes,
                      static_cast<hipStream_t>(stream));
}

int hyperattn_forward(const void* q, const void* k, const void* v, int dtype, int batch, int n,
                      int d, int heads, int kv_heads, int block, int samples, int proj_bits,
                      int causal, int min_seq_len, uint64_t seed, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return hyperattn_forward_ex(q, k, v, dtype, batch, n, d, heads, kv_heads, block, samples,
                              proj_bits, causal, min_seq_len, seed, 0, out, lse, workspace,
                              workspace_bytes, stream);
}

int hyperattn_debug_levels(int n, int causal, int min_seq_len) {
  if (n < 0 || (causal && min_seq_len < 1)) return -1;
  if (!causal) return 1;
  int L = 0;
  for (int64_t ns = n; ns > min_seq_len; ns -= ns / 2) ++L;
  return L;
}

int hyperattn_forward_debug(const void* q, const void* k, const void* v, int dtype, int batch, int n, int d,
                            int heads, int kv_heads, int block, int samples, int proj_bits, int causal,
                            int min_seq_len, uint64_t seed, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream, const ha_debug_dump* dump) {
  g_last_error.clear();
  if (!dump) {
    set_error("forward_debug: null dump");
    return HA_EINVAL;
  }
  if (!dump->o_blk != !dump->lse_blk || !dump->o_smp != !dump->lse_smp || !dump->o_leaf != !dump->lse_leaf) {
    set_error("forward_debug: an o_* / lse_* pair has one pointer missing");
    return HA_EINVAL;
  }
  Shape sh{batch, n, d, heads, kv_heads, block, samples, proj_bits, causal, min_seq_len, dtype, 0};
  return forward_impl(q, k, v, sh, seed, out, lse, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                      dump);
}

int hyperattn_forward_noalloc(const void* q, const void* k, const void* v, int dtype, int batch, int n, int d,
                              int heads, int kv_heads, int block, int samples, int proj_bits, int causal,
                              int min_seq_len, uint64_t seed, void* out, float* lse, void* stream) {
  g_last_error.clear();
  Shape sh{batch, n, d, heads, kv_heads, block, samples, proj_bits, causal, min_seq_len, dtype, 0};
  return forward_noalloc_impl(q, k, v, sh, seed, out, lse, static_cast<hipStream_t>(stream));
}

size_t hyperattn_rect_workspace_bytes(int batch, int n_q, int n_k, int d, int heads, int kv_heads, int block,
                                      int samples, int proj_bits, int dtype) {
  Shape sh{batch, n_q, d, heads, kv_heads, block, samples, proj_bits, 0, 0, dtype, 0};
  if (rect_validate(sh, n_k) != HA_OK) return 0;
  return rect_plan(sh, n_k, nullptr, 0).total;
}

int hyperattn_forward_rect(const void* q, const void* k, const void* v, int dtype, int batch, int n_q, int n_k,
                           int d, int heads, int kv_heads, int block, int samples, int proj_bits, uint64_t seed,
                           void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Shape sh{batch, n_q, d, heads, kv_heads, block, samples, proj_bits, 0, 0, dtype, 0};
  return forward_rect_impl(q, k, v, sh, n_k, seed, out, lse, workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream));
}

size_t hyperattn_backward_workspace_bytes(int batch, int n, int d, int heads, int kv_heads, int block,
                                          int samples, int proj_bits, int causal, int min_seq_len,
                                          int dtype) {
  Shape sh{batch, n, d, heads, kv_heads, block, samples, proj_bits, causal, min_seq_len, dtype, 0};
  if (validate(sh) != HA_OK) return 0;
  return backward_plan(sh, nullptr, 0).total;
}

int hyperattn_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, int dtype, int batch, int n, int d, int heads, int kv_heads,
                       int block, int samples, int proj_bits, int causal, int min_seq_len, uint64_t seed,
                       float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  Shape sh{batch, n, d, heads, kv_heads, block, samples, proj_bits, causal, min_seq_len, dtype, 0};
  return backward_impl(q, k, v, out, lse, dout, sh, seed, dq, dk, dv, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream));
}

size_t hyperattn_backward_rect_workspace_bytes(int batch, int n_q, int n_k, int d, int heads, int kv_heads,
                                               int block, int samples, int proj_bits, int dtype) {
  Shape sh{batch, n_q, d, heads, kv_heads, block, samples, proj_bits, 0, 0, dtype, 0};
  if (rect_validate(sh, n_k) != HA_OK) return 0;
  return backward_rect_plan(sh, n_k, nullptr, 0).total;
}

int hyperattn_backward_rect(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, int dtype, int batch, int n_q, int n_k, int d, int heads,
                            int kv_heads, int block, int samples, int proj_bits, uint64_t seed, float* dq,
                            float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Shape sh{batch, n_q, d, heads, kv_heads, block, samples, proj_bits, 0, 0, dtype, 0};
  return backward_rect_impl(q, k, v, out, lse, dout, sh, n_k, seed, dq, dk, dv, workspace, workspace_bytes,
                            static_cast<hipStream_t>(stream));
}

int hyperattn_row_sqnorms(const void* x, int dtype, int64_t rows, int d, float* w, void* stream) {
  g_last_error.clear();
  if (rows < 0 || (rows > 0 && (!x || !w))) {
    set_error("row_sqnorms: bad arguments");
    return HA_EINVAL;
  }
  if ((dtype != HA_BF16 && dtype != HA_F32) || (d != 64 && d != 128)) {
    set_error("row_sqnorms: dtype %d / d %d not built", dtype, d);
    return HA_EUNSUPPORTED;
  }
  return launch_rownorm_sqnorm(x, dtype, rows, d, w, static_cast<hipStream_t>(stream));
}

size_t hyperattn_rownorm_samples_workspace_bytes(int batch, int kv_heads, int n) {
  if (batch < 0 || kv_heads < 1 || n < 0) return 0;
  return rownorm_cdf_ws_bytes(static_cast<int64_t>(batch) * kv_heads, n);
}

int hyperattn_rownorm_samples(const float* w, const int32_t* perm_k, int batch, int heads, int kv_heads, int n,
                              int samples, uint64_t seed, int64_t* cum, int32_t* sidx, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads || n < 0 || samples < 0 ||
      (n > 0 && batch > 0 && (!w || !perm_k || !cum || (samples > 0 && !sidx)))) {
    set_error("rownorm_samples: bad arguments");
    return HA_EINVAL;
  }
  const int64_t problems = static_cast<int64_t>(batch) * kv_heads;
  if (n > 0 && batch > 0 && (!workspace || workspace_bytes < rownorm_cdf_ws_bytes(problems, n))) {
    set_error("rownorm_samples: workspace of %zu bytes, %zu needed", workspace_bytes,
              rownorm_cdf_ws_bytes(problems, n));
    return HA_EWORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  RnGeom g;
  g.seg = n;
  g.n_head = n;
  HA_TRY(launch_rownorm_cdf(w, perm_k, problems, g, cum, workspace, s));
  return launch_rownorm_samples(cum, g, 1, seed, batch, heads, kv_heads, samples, sidx, s);
}

int hyperattn_column_sqmass(const void* q, const void* k, const float* lse, int dtype, int batch, int n, int d,
                            int heads, int kv_heads, int causal, int skip, float* colmass, float* alpha,
                            void* stream) {
  g_last_error.clear();
  if (batch < 0 || n < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads || skip < 0 ||
      (batch > 0 && n > 0 && (!q || !k || !lse || !colmass))) {
    set_error("column_sqmass: bad arguments");
    return HA_EINVAL;
  }
  if (dtype != HA_BF16 || (d != 64 && d != 128)) {
    set_error("column_sqmass: bf16 with d 64 or 128 only");
    return HA_EUNSUPPORTED;
  }
  if (static_cast<int64_t>(n) * d * 2 >= (int64_t(1) << 32)) {
    set_error("column_sqmass: one head spans 4 GiB or more");
    return HA_EUNSUPPORTED;
  }
  return launch_colmass(q, k, lse, batch, n, d, heads, kv_heads, causal, skip, colmass, alpha,
                        static_cast<hipStream_t>(stream));
}

int hyperattn_residual_ratio(const float* lse_exact, const float* lse_block, const int32_t* perm_q,
                             int64_t problems, int n, float* kappa, void* stream) {
  g_last_error.clear();
  if (problems < 0 || n < 0 || (problems > 0 && n > 0 && (!lse_exact || !lse_block || !perm_q || !kappa))) {
    set_error("residual_ratio: bad arguments");
    return HA_EINVAL;
  }
  return launch_kappa(lse_exact, lse_block, perm_q, problems, n, kappa, static_cast<hipStream_t>(stream));
}

int hyperattn_projections_host(uint64_t seed, int d, int proj_bits, float* host_out) {
  g_last_error.clear();
  if (!host_out || d < 1 || proj_bits < 1 || proj_bits > 16) {
    set_error("projections: bad arguments");
    return HA_EINVAL;
  }
  const int total = d * proj_bits;
  for (int pi = 0; pi < (total + 1) / 2; ++pi) {
    float z0, z1;
    gauss_pair(seed, static_cast<uint32_t>(pi), &z0, &z1);
    host_out[2 * pi] = z0;
    if (2 * pi + 1 < total) host_out[2 * pi + 1] = z1;
  }
  return HA_OK;
}

int hyperattn_projections(uint64_t seed, int d, int proj_bits, float* dev_out, void* stream) {
  g_last_error.clear();
  if (!dev_out || d < 1 || proj_bits < 1 || proj_bits > 16) {
    set_error("projections: bad arguments");
    return HA_EINVAL;
  }
  return launch_projections(seed, d, proj_bits, dev_out, static_cast<hipStream_t>(stream));
}

int hyperattn_hash(const void* x, int dtype, int64_t rows, int d, int proj_bits,
                   const float* proj_dev, uint16_t* rank_out, void* stream) {
  g_last_error.clear();
  if (rows < 0 || (rows > 0 && (!x || !proj_dev || !rank_out)) ||
      (dtype != HA_BF16 && dtype != HA_F32) || proj_bits < 1 || proj_bits > 16) {
    set_error("hash: bad arguments");
    return HA_EINVAL;
  }
  if (d != 64 && d != 128) {
    set_error("hash: head dim %d not built", d);
    return HA_EUNSUPPORTED;
  }
  return launch_hash(x, dtype, rows, d, proj_bits, proj_dev, rank_out,
                     static_cast<hipStream_t>(stream));
}

size_t hyperattn_sort_workspace_bytes(int64_t heads, int len, int pieces, int proj_bits) {
  if (heads < 0 || len < 0 || pieces < 0 || proj_bits < 1 || proj_bits > 16) return 0;
  return sort_ws_bytes(heads, len, pieces, proj_bits);
}

int hyperattn_sort(const uint16_t* rank, int64_t heads, int n, int len, int first, int stride,
                   int pieces, int proj_bits, int32_t* perm_out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (heads < 0 || n < 0 || len < 0 || first < 0 || stride < 0 || pieces < 0 || proj_bits < 1 ||
      proj_bits > 16) {
    set_error("sort: bad arguments");
    return HA_EINVAL;
  }
  if (heads == 0 || len == 0 || pieces == 0) return HA_OK;
  if (static_cast<int64_t>(first) + static_cast<int64_t>(pieces - 1) * stride + len > n) {
    set_error("sort: segments run past n");
    return HA_EINVAL;
  }
  if (!rank || !perm_out) {
    set_error("sort: null pointer");
    return HA_EINVAL;
  }
  return launch_sort(rank, heads, n, len, first, stride, pieces, proj_bits, perm_out, workspace,
                     workspace_bytes, static_cast<hipStream_t>(stream));
}

int hyperattn_sample_indices(uint64_t seed, int batch, int heads, int node_first, int node_count,
                             int ns, int samples, int32_t* idx_out, void* stream) {
  g_last_error.clear();
  if (batch < 0 || heads < 0 || node_first < 0 || node_count < 0 || ns < 1 || samples < 0 ||
      (samples > 0 && batch > 0 && heads > 0 && node_count > 0 && !idx_out)) {
    set_error("sample_indices: bad arguments");
    return HA_EINVAL;
  }
  return launch_sample_indices(seed, batch, heads, node_first, node_count, ns, samples, idx_out,
                               static_cast<hipStream_t>(stream));
}

int hyperattn_gather(const void* src, int dtype, int64_t heads, int n, int d, const int32_t* perm,
                     int rows_per_head, void* dst, void* stream) {
  g_last_error.clear();
  if (heads < 0 || n < 0 || rows_per_head < 0 || (dtype != HA_BF16 && dtype != HA_F32) ||
      d < 8 || d % 8 || (heads * rows_per_head > 0 && (!src || !perm || !dst))) {
    set_error("gather: bad arguments");
    return HA_EINVAL;
  }
  return launch_gather(src, dtype, heads, n, d, perm, rows_per_head, dst,
                       static_cast<hipStream_t>(stream));
}

int hyperattn_attend(const void* q, const void* k, const void* v, int dtype, int batch, int n,
                     int d, int heads, int kv_heads, int block, int samples,
                     const int32_t* perm_q, const int32_t* perm_k, const int32_t* idx, int parts,
                     float* o_out, float* lse_out, void* stream) {
  g_last_error.clear();
  Shape sh{batch, n, d, heads, kv_heads, block, samples, 7, 0, 0, dtype, 0};
  HA_TRY(validate(sh));
  if (parts < 1 || parts > 3) {
    set_error("attend: parts %d outside 1..3", parts);
    return HA_EINVAL;
  }
  if (n == 0 || batch == 0 || heads == 0) return HA_OK;
  if (!q || !k || !v || !perm_q || !perm_k || !o_out || !lse_out || ((parts & 2) && samples > 0 && !idx)) {
    set_error("attend: null pointer");
    return HA_EINVAL;
  }
  AttnParams ap;
  ap.q = q;
  ap.k = k;
  ap.v = v;
  ap.dtype = dtype;
  ap.d = d;
  ap.n = n;
  ap.H = heads;
  ap.Hkv = kv_heads;
  ap.BH = batch * heads;
  ap.kind = kKindSorted;
  ap.pieces = 1;
  ap.seg = n;
  ap.stride = n;
  ap.perm_q = perm_q;
  ap.perm_k = perm_k;
  ap.b_eff = block < n ? block : n;
  ap.use_block = (parts & 1) ? 1 : 0;
  ap.use_samples = (parts & 2) ? 1 : 0;
  ap.sidx = idx;
  ap.m = samples;
  ap.log2w = samples > 0 ? static_cast<float>(std::log2(static_cast<double>(n) / samples)) : 0.f;
  ap.out_mode = kOutPartial;
  ap.part_o = o_out;
  ap.part_lse = lse_out;
  return launch_attention(ap, HA_K_ATTEND, static_cast<hipStream_t>(stream));
}

int hyperattn_merge_unsort(const float* o1, const float* lse1, const float* o2, const float* lse2,
                           const int32_t* perm_q, int64_t heads, int n, int d, int dtype,
                           void* out, float* lse_out, void* stream) {
  g_last_error.clear();
  if (heads < 0 || n < 0 || d < 4 || d % 4 || (dtype != HA_BF16 && dtype != HA_F32) ||
      (heads * n > 0 && (!o1 || !lse1 || !o2 || !lse2 || !perm_q || !out))) {
    set_error("merge_unsort: bad arguments");
    return HA_EINVAL;
  }
  return launch_merge_unsort(o1, lse1, o2, lse2, perm_q, heads, n, d, dtype, out, lse_out,
                             static_cast<hipStream_t>(stream));
}

int hyperattn_causal_leaves(const void* q, const void* k, const void* v, int dtype, int batch,
                            int n, int d, int heads, int kv_heads, int leaf_len, float* o_out,
                            float* lse_out, void* stream) {
  g_last_error.clear();
  Shape sh{batch, n, d, heads, kv_heads, 1, 0, 7, 0, 0, dtype, 0};
  HA_TRY(validate(sh));
  if (leaf_len < 1) {
    set_error("causal_leaves: leaf_len %d < 1", leaf_len);
    return HA_EINVAL;
  }
  if (n % leaf_len) {
    set_error("causal_leaves: n %d not a multiple of leaf_len %d", n, leaf_len);
    return HA_ESHAPE;
  }
  if (n == 0 || batch == 0 || heads == 0) return HA_OK;
  if (!q || !k || !v || !o_out || !lse_out) {
    set_error("causal_leaves: null pointer");
    return HA_EINVAL;
  }
  AttnParams lp;
  lp.q = q;
  lp.k = k;
  lp.v = v;
  lp.dtype = dtype;
  lp.d = d;
  lp.n = n;
  lp.H = heads;
  lp.Hkv = kv_heads;
  lp.BH = batch * heads;
  lp.kind = kKindLeaf;
  lp.pieces = n / leaf_len;
  lp.seg = leaf_len;
  lp.stride = leaf_len;
  lp.b_eff = leaf_len;
  lp.use_block = 1;
  lp.use_samples = 0;
  lp.out_mode = kOutAcc;
  lp.acc_o = o_out;
  lp.acc_lse = lse_out;
  HA_TRY(launch_attention(lp, HA_K_LEAF, static_cast<hipStream_t>(stream)));
  return HA_OK;
}

int hyperattn_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_recs.clear();
  g_open.clear();
  g_timing = enable != 0;
  return HA_OK;
}

int hyperattn_timing_read(double* ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_tmu);
  double acc[HA_K_COUNT] = {0};
  int64_t cnt[HA_K_COUNT] = {0};
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) {
      set_error("timing: event synchronisation failed");
      return HA_EHIP;
    }
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.start, r.stop) == hipSuccess) {
      acc[r.kind] += t;
      cnt[r.kind] += 1;
    }
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_recs.clear();
  g_open.clear();
  for (int i = 0; i < HA_K_COUNT; ++i) {
    if (ms) ms[i] = acc[i];
    if (launches) launches[i] = cnt[i];
  }
  return HA_OK;
}

}  // extern "C"
