// Internal helpers shared by the libmoe sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------ types

typedef uint16_t bf16_t;   // bf16 storage (upper half of an fp32)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float round_bf16(float v) { return bf16_bits_to_f32(f32_to_bf16_bits(v)); }
// pack two fp32 into two bf16 (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Storage traits: bf16 (uint16 storage) or fp32.
template <typename T> struct Store;
template <> struct Store<bf16_t> {
  static constexpr int kDtype = MOE_BF16;
  __device__ __forceinline__ static float load(const bf16_t *p) { return bf16_bits_to_f32(*p); }
  __device__ __forceinline__ static float round(float v) { return round_bf16(v); }
};
template <> struct Store<float> {
  static constexpr int kDtype = MOE_F32;
  __device__ __forceinline__ static float load(const float *p) { return *p; }
  __device__ __forceinline__ static float round(float v) { return v; }
};

// ------------------------------------------------------------------ host side

// thread-local message of the last failure
void set_error(const char *fmt, ...);
void clear_error();

// Launch bookkeeping for the optional per-kernel timing.
struct TimedLaunch {
  TimedLaunch(const char *name, hipStream_t s);
  ~TimedLaunch();
  const char *name_;
  hipStream_t stream_;
  int slot_;
};

// Check the last launch; returns MOE_OK or MOE_ERR_HIP with a message.
int check_launch(const char *what);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MOE_REQUIRE(cond, code, ...)   \
  do {                                 \
    if (!(cond)) {                     \
      ::moe::set_error(__VA_ARGS__);   \
      return (code);                   \
    }                                  \
  } while (0)

#define MOE_LAUNCH(name, stream, ...)                               \
  do {                                                              \
    ::moe::TimedLaunch _tl(name, stream);                           \
    __VA_ARGS__;                                                    \
  } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

}  // namespace moe
