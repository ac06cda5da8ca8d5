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

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (lo in bits 0..15) with gfx950's packed conversion
// (one v_cvt_pk_bf16_f32): round to nearest, ties to even -- measured on MI355X it
// equals the bit arithmetic u + 0x7fff + ((u >> 16) & 1) >> 16 on every
// non-NaN fp32 pattern, denormals included; a NaN stays a quiet NaN (sign and
// leading payload bits kept).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2v_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float v) { return pack_bf16x2(v, 0.0f) & 0xffffu; }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float round_bf16(float v) { return bf16_bits_to_f32(f32_to_bf16_bits(v)); }

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

// S[slot_to_row[t*k+j]] = store(w[that row] * dY[t]) for T tokens (w NULL:
// a copy), the weight-gradient operand of the gathered backward; launched on
// stream s, named "row_scale" for timing (csrc/permute.hip).
int launch_row_scale_scatter(const bf16_t *dy, const int32_t *slot_to_row, const float *w,
                             int64_t T, int d, int k, bf16_t *s_rows, hipStream_t s);

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
