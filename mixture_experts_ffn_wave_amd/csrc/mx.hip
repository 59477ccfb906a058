// MX-fp8 quantisation of the expert GEMM operands (gfx950).
//
// MX-fp8 as used for the experts in the KohakUwULLM README ("Key features"):
// e4m3 element values with one UE8M0 (power-of-two) scale per block of 32
// values.  The block scale is the smallest power of two 2^x with every
// |v| / 2^x within the e4m3 range (amax <= 448 * 2^x), so nothing saturates;
// x is clamped to [-127, 127] and an all-zero block gets x = -127.  Elements
// are then rounded to nearest e4m3 (ties to even), subnormals k * 2^-9.
//
// Blocks always run along the reduction axis of the GEMM that consumes the
// operand: along rows for row operands (activations [tokens][K], weights
// [N][K]), and along tokens for the weight gradients, which the transposing
// quantiser lays out K-contiguous with every expert segment restarting its
// blocks and padded with zeros to a multiple of 128 tokens.

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int NT = 256;

// smallest x with amax <= 448 * 2^x, clamped to [-127, 127]
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  const float m = frexpf(amax, &e);          // amax = (2m) 2^(e-1), 2m in [1, 2); 448 = 1.75 * 2^8
  const int x = (2.0f * m <= 1.75f) ? (e - 1) - 8 : (e - 1) - 7;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// e4m3 bits of q (|q| <= 448, so no saturation is needed)
__device__ __forceinline__ uint32_t e4m3_bits(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);   // k 2^-9; k = 8 is 2^-6 (0x08)
  int e;
  frexpf(a, &e);                              // a in [2^(e-1), 2^e)
  float mq = rintf(ldexpf(a, 4 - e));         // 3 mantissa bits: a / 2^(e-4) in [8, 16]
  int E = e - 1;
  if (mq >= 16.0f) { mq = 8.0f; ++E; }
  return sign | (uint32_t)((E + 7) << 3) | ((uint32_t)mq - 8u);
}

// quantise 32 values: 32 payload bytes + the scale byte
__device__ __forceinline__ uint8_t mx_block(const float (&v)[32], u32x4 (&out)[2]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int x = mx_scale_exp(amax);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= e4m3_bits(ldexpf(v[4 * w + b], -x)) << (8 * b);
    out[w >> 2][w & 3] = word;
  }
  return (uint8_t)(x + 127);
}

template <typename T>
__global__ void __launch_bounds__(NT) mx_quant_rows_kernel(MxRowsArgs a) {
  const int kb_per_row = a.K / 32;
  const int64_t nb = a.R * kb_per_row;
  const T* in = static_cast<const T*>(a.in);
  for (int64_t b = (int64_t)blockIdx.x * NT + threadIdx.x; b < nb; b += (int64_t)gridDim.x * NT) {
    const int64_t r = b / kb_per_row;
    const int kb = (int)(b - r * kb_per_row), k0 = kb * 32;
    const T* src = in + (int64_t)(k0 / a.sub) * a.block_stride + r * a.ld_in + (k0 % a.sub);
    float v[32];
#pragma unroll
    for (int c = 0; c < 32 * (int)sizeof(T) / 16; ++c) {
      Chunk<T> ch;
      ch.raw = ld16(src + c * Chunk<T>::N);
#pragma unroll
      for (int i = 0; i < Chunk<T>::N; ++i) v[c * Chunk<T>::N + i] = to_f32<T>(ch.e[i]);
    }
    u32x4 o[2];
    const uint8_t sc = mx_block(v, o);
    uint8_t* dst = a.out + r * a.K + k0;
    st16(dst, o[0]);
    st16(dst + 16, o[1]);
    a.scales[r * kb_per_row + kb] = sc;
  }
}

// grid: x = padded 32-block, y = column tile of NT columns
template <typename T>
__global__ void __launch_bounds__(NT) mx_quant_cols_kernel(MxColsArgs a) {
  const int64_t p = (int64_t)blockIdx.x * 32;           // padded K position of this block
  int g;
  int64_t pstart;
  if (a.pad) {
    if (p >= a.pad[a.G]) return;
    int lo = 0, hi = a.G - 1;                             // last g with pad[g] <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.pad[mid] <= p) lo = mid; else hi = mid - 1;
    }
    g = lo;
    pstart = a.pad[g];
  } else {
    g = (int)(p / a.seg_len);
    if (g >= a.G) return;
    pstart = (int64_t)g * a.seg_len;
  }
  const int c = blockIdx.y * NT + threadIdx.x;
  if (c >= a.C) return;
  const int64_t tstart = a.seg ? a.seg[g] : (int64_t)g * a.seg_len;
  const int64_t n = a.seg ? (int64_t)(a.seg[g + 1] - a.seg[g]) : a.seg_len;
  const int64_t t0 = p - pstart;
  const T* in = static_cast<const T*>(a.in) + tstart * a.ld_in + c;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = (t0 + i < n) ? to_f32<T>(in[(t0 + i) * a.ld_in]) : 0.0f;
  u32x4 o[2];
  const uint8_t sc = mx_block(v, o);
  const int64_t row = a.row0 + c, k = a.k0 + p;
  uint8_t* dst = a.out + row * a.Kpad + k;
  st16(dst, o[0]);
  st16(dst + 16, o[1]);
  a.scales[row * (a.Kpad / 32) + k / 32] = sc;
}

__global__ void mx_pad_offsets_kernel(const int32_t* offsets, int32_t* pad, int G, int align) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int32_t acc = 0;
  pad[0] = 0;
  for (int g = 0; g < G; ++g) {
    const int32_t n = offsets[g + 1] - offsets[g];
    acc += (n + align - 1) / align * align;
    pad[g + 1] = acc;
  }
}

__global__ void mx_single_segment_kernel(int32_t* seg_pad, int64_t T, int align) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  seg_pad[0] = 0;
  seg_pad[1] = (int32_t)T;
  seg_pad[2] = 0;
  seg_pad[3] = (int32_t)((T + align - 1) / align * align);
}

}  // namespace

hipError_t launch_mx_single_segment(int32_t* seg_pad, int64_t T, int align, hipStream_t s) {
  hipLaunchKernelGGL(mx_single_segment_kernel, dim3(1), dim3(64), 0, s, seg_pad, T, align);
  return hipGetLastError();
}

hipError_t launch_mx_quant_rows(int dt, const MxRowsArgs& a, hipStream_t s) {
  if (a.K % 32 || a.sub % 32 || a.sub <= 0) return hipErrorInvalidValue;
  const int64_t nb = a.R * (a.K / 32);
  if (nb == 0) return hipSuccess;
  int64_t grid = (nb + NT - 1) / NT;
  if (grid > 65536) grid = 65536;
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL(mx_quant_rows_kernel<__bf16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL(mx_quant_rows_kernel<_Float16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(int dt, const MxColsArgs& a, hipStream_t s) {
  if (a.Kpad % 128 || a.k0 % 32 || a.C <= 0) return hipErrorInvalidValue;
  if (!a.pad && (a.seg_len % 32)) return hipErrorInvalidValue;
  if (a.nblk <= 0) return hipSuccess;
  if (a.nblk > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.nblk, (unsigned)((a.C + NT - 1) / NT));
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL(mx_quant_cols_kernel<__bf16>, grid, dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL(mx_quant_cols_kernel<_Float16>, grid, dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mx_pad_offsets(const int32_t* offsets, int32_t* pad, int G, int align, hipStream_t s) {
  hipLaunchKernelGGL(mx_pad_offsets_kernel, dim3(1), dim3(64), 0, s, offsets, pad, G, align);
  return hipGetLastError();
}

}  // namespace moe
