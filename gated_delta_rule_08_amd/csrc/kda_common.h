// kda_common.h -- internal helpers shared by the gfx950 kernels of libkda.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kda.h"

namespace kda {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> fp32
// bf16 is carried as raw uint16 bits.  bf16 -> fp32 is exact; fp32 -> bf16
// rounds to nearest even (NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// gfx950 converts with v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// I/O element types: float for fp32, uint16_t (bf16 bits) for bf16.
template <typename IO> struct io_traits;
template <> struct io_traits<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct io_traits<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// Input preparation from raw projections (heqinghuang "From GPT2 to Kimi3,
// Explained", section 09: SiLU then unit length for queries and keys, sigmoid
// write strength; engineermaxxing ch. 06b: the per-channel gate is a sigmoid).
// Hardware reciprocal, exponential and logarithm (about 1 ulp): their error is
// far below the bf16 rounding of the prepared operands.
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + fast_exp(-x));
}
__device__ __forceinline__ float silu(float x) { return x * sigmoid(x); }
// log(sigmoid(x)) = min(x, 0) - log(1 + e^-|x|), finite for every finite x
__device__ __forceinline__ float log_sigmoid(float x) {
  return fminf(x, 0.f) - __logf(1.f + fast_exp(-fabsf(x)));
}
// reciprocal of the normaliser max(norm, 1e-12) applied to a row
__device__ __forceinline__ float inv_norm(float sumsq) { return rsqrtf(fmaxf(sumsq, 1e-24f)); }

// Sanitised sequence bounds, shared by every prefill kernel: offsets are
// clamped to [0, T] and made nondecreasing so that no access leaves [0, T).
__device__ __forceinline__ int clamp_tok(int x, int T) { return x < 0 ? 0 : (x > T ? T : x); }

// ---------------------------------------------------------------- host-side status
void set_error(const char* fmt, ...);
kda_status_t hip_status(hipError_t e, const char* what);
kda_status_t check_launch(const char* what);

// Raises a kernel's dynamic LDS limit to `bytes` before its first launch on the
// current device.  `done` holds one bit per device (devices 64 and up set the
// attribute on every call); the attribute call is idempotent, so two threads
// racing on a first launch both set it, which is harmless, and the bit is
// published with release order.  Safe to call from several host threads.
kda_status_t allow_dynamic_lds(const void* fn, size_t bytes, std::atomic<uint64_t>& done,
                               const char* what);

}  // namespace kda
