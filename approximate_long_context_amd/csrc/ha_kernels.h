// Internal launch interface between the host driver and the HIP kernels.
#pragma once

#include "ha_common.h"

namespace ha {

// ---- timing hooks (ha_api.cpp) -------------------------------------------
// HA_EHIP, with a message, when HYPERATTN_FAIL_AT names the stage of kernel
// class `kind`; launchers call it before enqueuing anything.
int launch_gate(int kind);
void timing_begin(int kind, hipStream_t s);
void timing_end(int kind, hipStream_t s);

// ---- projections + hash (ha_hash.hip) ------------------------------------
int launch_projections(uint64_t seed, int d, int r, float* R, hipStream_t s);
int launch_hash(const void* x, int dtype, int64_t rows, int d, int r, const float* R,
                uint16_t* rank, hipStream_t s);

// ---- segmented stable counting sort (ha_sort.hip) ------------------------
size_t sort_ws_bytes(int64_t heads, int len, int pieces, int r);
// One job of a batched sort: segment p (< pieces) of head h holds rows
// first + p * stride + [0, len) of rank[h * n ...]; perm [heads][pieces][len].
struct SortJobDesc {
  const uint16_t* rank;
  int64_t heads;
  int n, len, first, stride, pieces;
  int32_t* perm;
};
constexpr int kSortMaxJobs = 16;
size_t sort_batch_ws_bytes(const SortJobDesc* jobs, int njobs, int r);
int launch_sort_batch(const SortJobDesc* jobs, int njobs, int r, void* ws, size_t ws_bytes, hipStream_t s);
int launch_sort(const uint16_t* rank, int64_t heads, int n, int len, int first, int stride,
                int pieces, int r, int32_t* perm, void* ws, size_t ws_bytes, hipStream_t s);

// ---- samples, gather, merge (ha_attn.hip) --------------------------------
int launch_sample_indices(uint64_t seed, int batch, int heads, int node_first, int node_count,
                          int ns, int m, int32_t* out, hipStream_t s);
int launch_gather(const void* src, int dtype, int64_t heads, int n, int d, const int32_t* perm,
                  int rows_per_head, void* dst, hipStream_t s);
// dst[r * dpitch + c] = src[r * spitch + c] for r < rows, c < width (int32)
int launch_copy_rows_i32(const int32_t* src, int64_t spitch, int32_t* dst, int64_t dpitch, int width, int64_t rows,
                         hipStream_t s);
int launch_merge_unsort(const float* o1, const float* l1, const float* o2, const float* l2,
                        const int32_t* perm, int64_t heads, int n, int d, int dtype, void* out,
                        float* lse, hipStream_t s);

// ---- attention kernel (ha_attn.hip) --------------------------------------
enum AttnKind { kKindSorted = 0, kKindLeaf = 1 };
enum AttnOut {
  kOutFinal = 0,      // out/lse at the original row (perm_q or identity)
  kOutPartial = 1,    // fp32 part_o/part_lse at the sorted position (offset by the problem's first row)
  kOutLeaf = 2,       // piece 0 -> out/lse, other pieces -> acc (no read)
  kOutMerge = 3,      // merge with acc at the row; piece 0 -> out/lse, else -> acc
  kOutAcc = 4,        // every piece -> acc at the row (no read)
  kOutRescale = 5,    // out at the original row, scaled by exp(own lse - lse_ref there); lse kept
  kOutRescaleMerge = 6, // as kOutRescale, the result (lse = lse_ref) then merged like kOutMerge
  kOutLse = 7           // lse alone at the original row (no V, no P V products)
};

constexpr int kMaxSamples = 4096;   // sample list staged in LDS
constexpr int kBlockListCap = 2048; // largest block key list staged in LDS
constexpr size_t kLdsBytes = 160 * 1024;   // LDS of one gfx950 workgroup
// The largest LDS a sorted-problem attention launch with m samples needs
// for this dtype and head dim (block key list at its cap).
size_t attention_lds_bound(int dtype, int d, int m);

struct AttnParams {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  int dtype = HA_BF16;
  int d = 64;
  int n = 0;             // rows per head in q (and in k, v unless n_k is set)
  int n_k = 0;           // rows per head in k, v (launch_attention: 0 -> n)
  int H = 1, Hkv = 1;    // query / kv heads per batch entry
  int BH = 0;            // batch * H
  // problems: `pieces` per head, each of `seg` queries and `seg` keys.
  // Piece i reads query rows q_first + i*stride + [0, seg) and key rows
  // k_first + i*stride + [0, seg) (through the permutations when given).
  int pieces = 1;
  int seg = 0;
  int seg_k = 0;         // keys per problem (0 -> seg; rectangular problems)
  int q_first = 0, k_first = 0, stride = 0;
  const int32_t* perm_q = nullptr;   // [BH][pieces][seg]  sorted pos -> row
  const int32_t* perm_k = nullptr;   // [BHkv][pieces][seg]
  // materialised sorted copies ([BH or BHkv][pieces*seg][d]); when set,
  // rows are read at their sorted position and perm_q is used for stores.
  const void* qs = nullptr;
  const void* ks = nullptr;
  const void* vs = nullptr;
  int kind = kKindSorted;
  int b_eff = 1;         // query block size
  int b_k = 0;           // key block size (0 -> b_eff; rectangular problems)
  int bcap = 0;          // LDS block key list capacity (set by the launcher)
  int use_block = 1;
  int use_samples = 1;
  const int32_t* sidx = nullptr;     // [BH][pieces][m] sorted key positions
  int m = 0;
  // kOutRescale / kOutRescaleMerge: the sampled keys' K and V rows
  // ([BH][pieces][m][d] dtype, sample order), read in place of the rows
  // sidx names, and the normaliser the result is rescaled to ([BH][n],
  // natural log, at the original row)
  const void* smp_k = nullptr;
  const void* smp_v = nullptr;
  const float* lse_ref = nullptr;
  float log2w = 0.f;                 // log2(seg / m)
  int out_mode = kOutFinal;
  int final_piece = 0;               // kOutLeaf / kOutMerge: the piece whose rows are final (-1: none)
  void* out = nullptr;               // [BH][n][d] dtype
  float* lse = nullptr;              // [BH][n] (may be null for kOutFinal)
  float* acc_o = nullptr;            // [BH][n][d]
  float* acc_lse = nullptr;          // [BH][n]
  // kOutPartial: [BH][n][d] / [BH][n]; the result of sorted position t of
  // piece i goes to row q_first + i * stride + t of its head (so one problem
  // per head with q_first 0 fills [BH][n] in sorted order)
  float* part_o = nullptr;
  float* part_lse = nullptr;
};

int launch_attention(const AttnParams& p, int timing_kind, hipStream_t s);

// ---- backward (ha_bwd.hip) ------------------------------------------------
struct BwdParams {
  int dtype = HA_BF16;               // of q, k, v, out, dout (HA_F32: the fp32 kernels)
  const void* q = nullptr;           // [BH][n][d]
  const void* k = nullptr;           // [BHkv][n][d]
  const void* v = nullptr;
  const void* out = nullptr;         // forward output [BH][n][d]
  const void* dout = nullptr;        // upstream gradient [BH][n][d]
  const float* lse = nullptr;        // forward lse [BH][n] (natural log)
  float* qstat = nullptr;            // per row: (lse log2 e, rowsum(dout * out)) [BH][n][2]
  int d = 64;
  int n = 0;                         // rows per query head (q, out, dout, dq, lse)
  int n_k = 0;                       // rows per KV head (k, v, dk, dv); 0: n
  int H = 1, Hkv = 1;
  int BH = 0;
  // Problems: piece p of every head has queries at rows p * stride + q_first + t
  // and keys at rows p * stride + k_first + t (t < seg), in sorted order
  // through perm_q / perm_k ([heads][pieces][seg], rows within the head) or in
  // row order when a permutation is null.
  int pieces = 1;
  int seg = 0;
  int seg_k = 0;                     // keys per problem (0: seg); rectangular when they differ
  int stride = 0;
  int q_first = 0, k_first = 0;
  const int32_t* perm_q = nullptr;   // [BH][pieces][seg]
  const int32_t* perm_k = nullptr;   // [BHkv][pieces][seg_k]
  const int32_t* sidx = nullptr;     // [BH][pieces][m] sorted key positions (< seg_k)
  int m = 0;
  float log2w = 0.f;                 // log2(seg_k / m)
  int b_eff = 1;                     // query block
  int b_k = 0;                       // key block (0: b_eff); query block t pairs with key block t
  int causal = 0;                    // exact causal problem: key position <= query position
  int diag = 0;                      // causal dK/dV: 2 = the keys' own 256-query square, 1 = the queries after it
  int accumulate = 0;                // add to dq / dk / dv instead of storing
  int bcap = 0;                      // LDS block key list capacity (launcher)
  int qchunk = 2048;                 // queries per sample-key workgroup (bwd_query_chunk)
  float* part = nullptr;             // sample-key partials [ceil(seg / qchunk)][BH][pieces][m][2 d] fp32
  uint64_t* red_keys = nullptr;      // sorted (key position, slot) per (KV head, piece): [BHkv][pieces][G m]
  float* dq = nullptr;               // [BH][n][d] fp32
  float* dk = nullptr;               // [BHkv][n][d] fp32
  float* dv = nullptr;
};

// Largest (heads / kv_heads) * samples of a backward (the sample reduction
// sorts that many slots per problem in LDS).
constexpr int kBwdMaxGroupSamples = 8192;

// Queries per sample-key workgroup of the dK/dV pass: at least 2048, and
// at most 64 chunks per problem (bounds the partial buffer).
inline int bwd_query_chunk(int seg) {
  const int per64 = ((seg + 63) / 64 + 63) / 64 * 64;
  return per64 > 2048 ? per64 : 2048;
}

// Row-norm variant (ha_rownorm.hip).  Problems are (KV head, piece): piece
// i of a head has `seg` sorted key positions (perm_k [heads][pieces][seg],
// rows within the head of n_head rows) over the rows k_first + i * stride +
// [0, seg) of the head.  One whole head per problem: pieces 1, seg = n_head,
// k_first = stride = 0.
struct RnGeom {
  int seg = 0;
  int pieces = 1;
  int n_head = 0;
  int k_first = 0;
  int stride = 0;
};
int launch_rownorm_sqnorm(const void* v, int dtype, int64_t rows, int d, float* w, hipStream_t s);
size_t rownorm_cdf_ws_bytes(int64_t problems, int n);
// integer CDF per problem: cum [kv_problems][pieces][seg]
int launch_rownorm_cdf(const float* w, const int32_t* perm_k, int64_t kv_problems, const RnGeom& g, int64_t* cum,
                       void* ws, hipStream_t s);
// draws [batch][heads][pieces][m]; piece i uses node id node_first + i
int launch_rownorm_samples(const int64_t* cum, const RnGeom& g, int node_first, uint64_t seed, int batch,
                           int heads, int kv_heads, int m, int32_t* out, hipStream_t s);
// drawn K rows and weighted V rows [batch][heads][pieces][m][d]
int launch_rownorm_sample_gather(const void* k, const void* v, int dtype, const int32_t* perm_k,
                                 const int64_t* cum, const int32_t* sidx, const RnGeom& g, int batch, int heads,
                                 int kv_heads, int d, int m, void* kc, void* vc, hipStream_t s);

// Diagnostics (ha_diag.hip).
int launch_colmass(const void* q, const void* k, const float* lse, int batch, int n, int d, int heads,
                   int kv_heads, int causal, int skip, float* colmass, float* alpha, hipStream_t s);
int launch_kappa(const float* lse_exact, const float* lse_block, const int32_t* perm_q, int64_t problems, int n,
                 float* kappa, hipStream_t s);

int launch_bwd_qstat(const BwdParams& p, hipStream_t s);
int launch_bwd_dq(const BwdParams& p, hipStream_t s);
int launch_bwd_dkv(const BwdParams& p, bool samples, hipStream_t s);
// deterministic sum of the sample partials into dk / dv (ha_bwd.hip)
int launch_bwd_sample_reduce(const BwdParams& p, int nchunk, hipStream_t s);
// fp32 kernels (ha_bwd32.hip), reached through the launchers above
int launch_bwd32_qstat(const BwdParams& p, hipStream_t s);
int launch_bwd32_dq(const BwdParams& p, hipStream_t s);
int launch_bwd32_dkv(const BwdParams& p, bool samples, hipStream_t s);

}  // namespace ha
