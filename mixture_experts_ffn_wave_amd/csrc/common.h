// Device-side helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;

// ---- scalar conversions (round to nearest even on the way down) ----------
template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

// ---- 16-byte vector memory helpers ----------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Element access inside a 16-byte chunk holding 16/sizeof(T) elements.
template <typename T> struct Chunk {
  static constexpr int N = 16 / sizeof(T);
  union { u32x4 raw; T e[N]; };
};

// 4 consecutive elements of T packed for one store (8 bytes for 16-bit T, 16 for f32).
template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  union { u32x2 raw; T e[4]; } u;
  u.e[0] = from_f32<T>(a); u.e[1] = from_f32<T>(b); u.e[2] = from_f32<T>(c); u.e[3] = from_f32<T>(d);
  st8(p, u.raw);
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}
template <typename T> __device__ __forceinline__ void load4(const T* p, float* out) {
  union { u32x2 raw; T e[4]; } u;
  u.raw = ld8(p);
  for (int i = 0; i < 4; ++i) out[i] = to_f32<T>(u.e[i]);
}
template <> __device__ __forceinline__ void load4<float>(const float* p, float* out) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}

// 8 consecutive elements of T: one 16-byte access for 16-bit T, two for f32.
template <typename T> __device__ __forceinline__ void store8(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    union { u32x4 raw; T e[8]; } u;
#pragma unroll
    for (int i = 0; i < 8; ++i) u.e[i] = from_f32<T>(v[i]);
    st16(p, u.raw);
  } else {
    store4<float>(p, v[0], v[1], v[2], v[3]);
    store4<float>(p + 4, v[4], v[5], v[6], v[7]);
  }
}
template <typename T> __device__ __forceinline__ void unpack8(u32x4 raw, float* out) {
  static_assert(sizeof(T) == 2, "8 elements per 16 bytes");
  union { u32x4 raw; T e[8]; } u;
  u.raw = raw;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = to_f32<T>(u.e[i]);
}
// RUN (4 or 8) consecutive elements
template <typename T, int RUN> __device__ __forceinline__ void store_run(T* p, const float* v) {
  if constexpr (RUN == 8) store8<T>(p, v);
  else store4<T>(p, v[0], v[1], v[2], v[3]);
}
template <typename T, int RUN> __device__ __forceinline__ void load_run(const T* p, float* out) {
  if constexpr (RUN == 8) unpack8<T>(ld16(p), out);
  else load4<T>(p, out);
}

// ---- MFMA 32x32 step over 16 values of k -------------------------------
// Lane l supplies operand row (l % 32) and the 8 consecutive k values starting
// at 8 * (l / 32); `a` and `b` each hold those 8 values as raw 16-byte chunks
// (one chunk for 16-bit types, two for f32).  The 32x32 f32 accumulator holds,
// in register r of lane l, element [row 8*(r/4) + 4*(l/32) + r%4][col l%32]
// where rows come from `a` and columns from `b`.
template <typename T> struct Mma32;

template <> struct Mma32<__bf16> {
  static constexpr int kChunks = 1;
  __device__ __forceinline__ static void run(f32x16& c, const u32x4* a, const u32x4* b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  }
};
template <> struct Mma32<_Float16> {
  static constexpr int kChunks = 1;
  __device__ __forceinline__ static void run(f32x16& c, const u32x4* a, const u32x4* b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[0]),
                                               __builtin_bit_cast(f16x8, b[0]), c, 0, 0, 0);
  }
};
// f32: eight 32x32x2 steps.  Step i contracts k = i (lanes 0-31) with k = 8 + i
// (lanes 32-63); the eight steps together cover all 16 k values, so the sum is
// the same contraction in a different order.
template <> struct Mma32<float> {
  static constexpr int kChunks = 2;
  __device__ __forceinline__ static void run(f32x16& c, const u32x4* a, const u32x4* b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // read the element into a scalar first: a bit_cast applied directly to a
      // vector-element expression drops the element index in this compiler
      const uint32_t ua = a[i >> 2][i & 3];
      const uint32_t ub = b[i >> 2][i & 3];
      const float av = __uint_as_float(ua);
      const float bv = __uint_as_float(ub);
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, c, 0, 0, 0);
    }
  }
};

// ---- wave reductions ------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// sigmoid and silu with the hardware reciprocal (v_rcp_f32, about 1 ulp)
// instead of a correctly rounded division: their results are rounded to the
// activation dtype next.  exp(-g) = inf gives rcp = 0, the correct limit.
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
