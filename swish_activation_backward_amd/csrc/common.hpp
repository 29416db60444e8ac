// Device-side helpers shared by the gfx950 kernels: storage types, 16-byte vectors,
// fp32 <-> storage conversion (round-to-nearest-even) and the Swish-gradient factor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swg {

typedef __bf16 bf16;
typedef _Float16 fp16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 fp16x8 __attribute__((ext_vector_type(8)));

// 16 bytes of storage viewed as VEC elements, widened to / narrowed from fp32.
// VEC = 8 for 16-bit types, 4 for fp32.  Narrowing rounds to nearest even
// (gfx950 v_cvt_pk_bf16_f32 / v_cvt_f16_f32).
template <typename T> struct Vec16;

template <> struct Vec16<bf16> {
  static constexpr int VEC = 8;
  __device__ static inline void widen(const u32x4& raw, float* f) {
    // bf16 -> fp32 is exact: the 16 payload bits become the high half of the word.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(raw[i] << 16);
      f[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
  }
  __device__ static inline u32x4 narrow(const float* f) {
    f32x8 v = {f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
    bf16x8 h = __builtin_convertvector(v, bf16x8);
    return __builtin_bit_cast(u32x4, h);
  }
};

template <> struct Vec16<fp16> {
  static constexpr int VEC = 8;
  __device__ static inline void widen(const u32x4& raw, float* f) {
    fp16x8 h = __builtin_bit_cast(fp16x8, raw);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  }
  __device__ static inline u32x4 narrow(const float* f) {
    fp16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (fp16)f[i];
    return __builtin_bit_cast(u32x4, h);
  }
};

template <> struct Vec16<float> {
  static constexpr int VEC = 4;
  __device__ static inline void widen(const u32x4& raw, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(raw[i]);
  }
  __device__ static inline u32x4 narrow(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
  }
};

template <typename T> __device__ inline float to_f32(T v) { return (float)v; }
template <typename T> __device__ inline T from_f32(float v) { return (T)v; }

// Streaming 16-byte global accesses.  Non-temporal: the data is touched once.
__device__ inline u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ inline void st16_stream(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Sigmoid pieces without overflow and without cancellation in 1 - s:
//   a = exp(-|t|) in (0, 1],  r = 1 / (1 + a)
//   t >= 0:  s = r,      1 - s = a r
//   t <  0:  s = a r,    1 - s = r
// so s (1 - s) = a r^2 for either sign.  exp uses the hardware base-2 exponential
// (v_exp_f32) and the reciprocal v_rcp_f32.
struct SigmoidParts {
  float s;       // sigma(t)
  float s1ms;    // sigma(t) * (1 - sigma(t))
};

__device__ inline SigmoidParts sigmoid_parts(float t) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float a = __builtin_amdgcn_exp2f(-__builtin_fabsf(t) * kLog2e);
  const float r = __builtin_amdgcn_rcpf(1.0f + a);
  const float ar = a * r;
  SigmoidParts p;
  p.s = t >= 0.0f ? r : ar;
  p.s1ms = ar * r;
  return p;
}

// sigma(t) alone (the forward's SiLU): 1 / (1 + 2^(-t log2 e)).  Correct for every finite
// t without the sign split above: for t below about -88 the exponential overflows to
// +inf and the reciprocal gives 0, the limit of sigma.
__device__ inline float sigmoid_only(float t) {
  constexpr float kLog2e = 1.4426950408889634f;
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t * kLog2e));
}

// s'(t) = sigma(t) (1 + t (1 - sigma(t))) = sigma(t) + t sigma(t)(1 - sigma(t)).
__device__ inline float swish_factor(float t) {
  const SigmoidParts p = sigmoid_parts(t);
  return __builtin_fmaf(t, p.s1ms, p.s);
}

}  // namespace swg
