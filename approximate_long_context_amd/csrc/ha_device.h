// Small device helpers shared by the forward and backward attention kernels.
#pragma once

#include "ha_common.h"

namespace ha {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  // Dispatch places workgroup i on XCD i % 8; give each XCD a contiguous
  // range of logical tiles so tiles that share keys share an L2.
  const int full = nblocks / 8 * 8;
  if (bid >= full) return bid;
  const int per = nblocks / 8;
  return (bid % 8) * per + bid / 8;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load from a workgroup-uniform base plus a per-lane byte offset
// below 2^32 (one head's rows; the host checks n * d * element < 2^32), so
// the base stays in scalar registers and the lane carries 32 bits.
__device__ __forceinline__ uint4v ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint4v*>(static_cast<const char*>(base) + off);
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// 4 bf16 of a transposing LDS read (gfx950 ds_read_b64_tr_b16): inside each
// group of 16 lanes, lane i receives element (i & 3) of the 8-byte rows
// addressed by lanes 4v + (i >> 2), v = 0..3.
__device__ __forceinline__ short4v lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(const_cast<void*>(p)));
}

// The A operand (8 bf16) of v_mfma_f32_32x32x16_bf16 for the transposed
// tile X^T, X row-major in LDS at `rows` (row stride `stride` elements):
// rows 16 c16 + ... of the chunk, columns 32 t + ...; the rows inside the
// 16-row chunk come in the order that matches a B operand packed from the
// MFMA result registers (D register r of lane l: row 8 (r / 4) + 4 (l / 32)
// + r % 4).
__device__ __forceinline__ bf16x8 lds_tr_operand(const bf16* rows, int stride, int c16, int t, int lane) {
  const int h2 = lane >> 5;
  const int tr_key = 4 * h2 + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const bf16* vp = rows + (16 * c16 + tr_key) * stride + 32 * t + tr_col;
  const short4v lo = lds_read_tr16(vp);
  const short4v hv = lds_read_tr16(vp + 8 * stride);
  const short __attribute__((ext_vector_type(8))) v8 = {lo[0], lo[1], lo[2], lo[3], hv[0], hv[1], hv[2], hv[3]};
  return __builtin_bit_cast(bf16x8, v8);
}

}  // namespace ha
