// Internal helpers shared by the library's translation units: element types,
// bf16 rounding, error reporting, launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <cstdio>
#include <string>

#include "rp.h"

namespace rp {

// bf16 storage type (bit pattern of the upper half of an IEEE fp32).
struct alignas(2) bf16 {
  uint16_t u;
};

__host__ __device__ inline float to_f(float x) { return x; }
__host__ __device__ inline float to_f(bf16 x) {
  union { uint32_t u; float f; } c;
  c.u = uint32_t(x.u) << 16;
  return c.f;
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN. On the device the hardware
// conversion (v_cvt_pk_bf16_f32 on gfx950) does it in one instruction; the
// host spells out the same rounding.
__host__ __device__ inline bf16 to_bf16(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return bf16{__builtin_bit_cast(uint16_t, (__bf16)f)};
#else
  union { uint32_t u; float f; } c;
  c.f = f;
  uint32_t u = c.u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{uint16_t((u >> 16) | 0x40u)};
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16{uint16_t(u >> 16)};
#endif
}

template <class T> __host__ __device__ inline T from_f(float f);
template <> __host__ __device__ inline float from_f<float>(float f) { return f; }
template <> __host__ __device__ inline bf16 from_f<bf16>(float f) { return to_bf16(f); }

template <class T> struct DT;
template <> struct DT<float> { static constexpr int id = RP_DTYPE_F32; };
template <> struct DT<bf16> { static constexpr int id = RP_DTYPE_BF16; };

inline size_t dtype_size(int dt) { return dt == RP_DTYPE_BF16 ? 2 : 4; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Wave-level sums (wave64) in a fixed butterfly order: deterministic.
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// error reporting (thread-local last error)
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
const char* last_error();

}  // namespace rp

// Return RP_ERR_HIP (with the HIP error text) from the enclosing function.
#define RP_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) {                                                           \
      ::rp::set_error("%s:%d: %s failed: %s", __FILE__, __LINE__, #call,              \
                      hipGetErrorString(e_));                                         \
      return RP_ERR_HIP;                                                              \
    }                                                                                 \
  } while (0)

// Return a status from the enclosing function when a sub-call fails.
#define RP_TRY(call)                 \
  do {                               \
    rp_status s_ = (call);           \
    if (s_ != RP_OK) return s_;      \
  } while (0)

#define RP_CHECK(cond, code, ...)         \
  do {                                    \
    if (!(cond)) {                        \
      ::rp::set_error(__VA_ARGS__);       \
      return (code);                      \
    }                                     \
  } while (0)

// Kernel launch + immediate launch-error check.
#define RP_LAUNCH(kernel, grid, block, lds, stream, ...)                               \
  do {                                                                                 \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                 \
    RP_HIP(hipGetLastError());                                                         \
  } while (0)
