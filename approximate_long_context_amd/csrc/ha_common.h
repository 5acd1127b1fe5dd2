// Shared definitions of the HyperAttention HIP library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "hyperattn.h"

namespace ha {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int uint4v __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Status propagation inside the library: every internal call returns an
// int status (HA_OK or a negative HA_E* code) and records a message.
void set_error(const char* fmt, ...);
int hip_status(hipError_t e, const char* what);

#define HA_CHECK_HIP(call)                                   \
  do {                                                       \
    hipError_t _e = (call);                                  \
    if (_e != hipSuccess) return ::ha::hip_status(_e, #call); \
  } while (0)

#define HA_TRY(call)              \
  do {                            \
    int _s = (call);              \
    if (_s != HA_OK) return _s;   \
  } while (0)

// After a launch: report launch errors and, when HYPERATTN_SYNC=1, wait
// and report execution errors of that stage.
int after_launch(const char* stage, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// A bump allocator over the caller's workspace (no device allocation).
struct Carve {
  char* base;
  size_t cap;
  size_t used = 0;
  Carve(void* b, size_t c) : base(static_cast<char*>(b)), cap(c) {}
  template <typename T>
  T* take(size_t count) {
    used = align_up(used, 256);
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return static_cast<float>(x); }

}  // namespace ha
