// Shared device/host helpers of libmao (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/mao.h"

namespace mao {

typedef uint16_t bf16_t;  // raw bf16 bits

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest even, NaN kept NaN: the gfx950 conversion
// instruction (v_cvt_pk_bf16_f32), which agrees bit for bit with the
// round-half-even bit arithmetic on every non-NaN fp32 input (all 2^32
// patterns checked on the GPU).
typedef __attribute__((ext_vector_type(2))) float f32x2_cvt_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_cvt_t;

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Two values packed into one 32-bit word (lo in the low half), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_cvt_t));
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void store_f32(T* p, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// Sum over a 64-wide wavefront (result valid in every lane).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024); every thread gets
// the total. `scratch` holds >= 16 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += scratch[i];
  return t;
}

__device__ __forceinline__ double block_sum_d(double v, double* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum_d(v);
  __syncthreads();
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < nw; ++i) t += scratch[i];
  return t;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Thread-local last-error text.
void set_error(const char* fmt, ...);

#define MAO_HIP_CHECK(expr)                                                   \
  do {                                                                        \
    hipError_t _e = (expr);                                                   \
    if (_e != hipSuccess) {                                                   \
      ::mao::set_error("%s failed: %s", #expr, hipGetErrorString(_e));        \
      return MAO_E_HIP;                                                       \
    }                                                                         \
  } while (0)

#define MAO_LAUNCH_CHECK()                                                    \
  do {                                                                        \
    hipError_t _e = hipGetLastError();                                        \
    if (_e != hipSuccess) {                                                   \
      ::mao::set_error("kernel launch failed: %s", hipGetErrorString(_e));    \
      return MAO_E_HIP;                                                       \
    }                                                                         \
  } while (0)

#define MAO_TRY(expr)                                                         \
  do {                                                                        \
    mao_status _s = (expr);                                                   \
    if (_s != MAO_OK) return _s;                                              \
  } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Leading dimension (elements) of a workspace matrix whose rows hold n
// elements: a multiple of 64 plus 64 more, so that consecutive rows never sit
// a multiple of 4 KiB apart (row strides that are large powers of two send the
// same K-slice of many rows to the same memory channel).
inline int64_t ws_ld(int64_t n) { return round_up(n, 64) + 64; }
inline int64_t ceil_div(int64_t x, int64_t a) { return (x + a - 1) / a; }

// Bump allocator over the caller's workspace (or a size-only dry run when
// base == nullptr).
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T> T* take(size_t count) {
    used = align_up(used, 256);
    T* p = base ? (T*)(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

}  // namespace mao
