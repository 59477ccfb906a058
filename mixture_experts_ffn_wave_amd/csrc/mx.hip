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
#include "mx_codec.h"

namespace moe {
namespace {

constexpr int NT = 256;

// Row operands: four lanes per 32-value block, eight values (one 16-byte
// load) per lane, so a wave reads 1 KB and writes 512 bytes contiguously.
template <typename T>
__global__ void __launch_bounds__(NT) mx_quant_rows_kernel(MxRowsArgs a) {
  static_assert(sizeof(T) == 2, "16-bit inputs");
  const int kq = a.K / 8;                                   // 8-value pieces per row
  const int64_t nq = a.R * kq;                              // a multiple of 4: quads stay whole
  const T* in = static_cast<const T*>(a.in);
  const int lane = threadIdx.x & 63;
  for (int64_t q = (int64_t)blockIdx.x * NT + threadIdx.x; q < nq; q += (int64_t)gridDim.x * NT) {
    const int64_t r = q / kq;
    const int k0 = (int)(q - r * kq) * 8;
    const T* src = in + (int64_t)(k0 / a.sub) * a.block_stride + r * a.ld_in + (k0 % a.sub);
    float v[8];
    unpack8<T>(ld16(src), v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int x = mx_scale_exp(amax);
    const float sc = ldexpf(1.0f, -x);
    const u32x2 o = {e4m3x4(v[0], v[1], v[2], v[3], sc), e4m3x4(v[4], v[5], v[6], v[7], sc)};
    st8(a.out + r * a.K + k0, o);
    if ((lane & 3) == 0) a.scales[r * (a.K / 32) + k0 / 32] = (uint8_t)(x + 127);
  }
}

// Transposing quantiser.  One workgroup per 128 padded K positions x TC
// columns (TC = 64, or 128 when the row-wise blocks are wanted too): the 128
// token rows x TC columns are read with 16-byte row loads into LDS, then wave
// j quantises the 32-token block j of the tile for its lane's TC / 64
// columns, reading them back from LDS (64 lanes = one 128-byte row: no bank
// conflicts).  The quantised bytes go back through LDS (over the input tile,
// which is dead by then) so that each output row's 128-byte span (four
// blocks) leaves as eight consecutive 16-byte stores and its four scale
// bytes as one 4-byte store.  Tiles never straddle a segment: segment starts
// (pad) and seg_len are multiples of 128.  With rq set, the same tile also
// gives the row-wise codes (blocks of 32 along the columns), as the row
// quantiser lays them out: four consecutive lanes per block, eight values
// each (a wave reads four whole tile rows from LDS, without bank conflicts),
// before the tile is overwritten.
constexpr int kColsTileK = 128;
constexpr int kColsOutRow = kColsTileK + 16;                // staged output row (padded: no bank conflicts)

template <typename T, int TC>
__global__ void __launch_bounds__(NT) mx_quant_cols_kernel(MxColsArgs a) {
  static_assert(sizeof(T) == 2, "16-bit inputs");
  static_assert(TC == 64 || TC == 128, "tile width");
  static_assert(TC * kColsOutRow <= kColsTileK * TC * (int)sizeof(T), "output staging fits");
  __shared__ __attribute__((aligned(16))) T tile[kColsTileK][TC];
  __shared__ __attribute__((aligned(16))) uint8_t qsc[TC][kColsTileK / 32];
  uint8_t* qout = reinterpret_cast<uint8_t*>(&tile[0][0]);  // [TC][kColsOutRow], after the quantise reads
  const int64_t p0 = (int64_t)blockIdx.x * kColsTileK;     // padded K position of this tile
  int g;
  int64_t pstart;
  if (a.pad) {
    if (p0 >= a.pad[a.G]) return;
    int lo = 0, hi = a.G - 1;                               // last g with pad[g] <= p0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.pad[mid] <= p0) lo = mid; else hi = mid - 1;
    }
    g = lo;
    pstart = a.pad[g];
  } else {
    g = (int)(p0 / a.seg_len);
    if (g >= a.G) return;
    pstart = (int64_t)g * a.seg_len;
  }
  const int c0 = blockIdx.y * TC;
  const int64_t tstart = a.seg ? a.seg[g] : (int64_t)g * a.seg_len;
  const int64_t n = a.seg ? (int64_t)(a.seg[g + 1] - a.seg[g]) : a.seg_len;
  const int64_t tt0 = p0 - pstart;                          // first token of the tile within the segment
  const T* in = static_cast<const T*>(a.in) + (a.gather ? 0 : tstart * a.ld_in);
  // ---- load: 128 rows x 16 pieces of 16 bytes; rows past the segment and
  // columns past C read as zero
  constexpr int VP = 16 / (int)sizeof(T);                   // values per piece
  constexpr int PIECES = TC / VP;                   // pieces per tile row
#pragma unroll
  for (int i = 0; i < kColsTileK * PIECES / NT; ++i) {
    const int q = threadIdx.x + NT * i, r = q / PIECES, pc = q % PIECES;
    const int col = c0 + pc * VP;
    const int64_t t = tt0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t < n && col < a.C) {
      v = ld16(in + (a.gather ? (int64_t)a.gather[tstart + t] : t) * a.ld_in + col);
      if (a.wrow) {                                         // w x, rounded as the stored rows would be
        const float w = a.wrow[tstart + t];
        Chunk<T> ch;
        ch.raw = v;
#pragma unroll
        for (int u = 0; u < VP; ++u) ch.e[u] = from_f32<T>(w * to_f32<T>(ch.e[u]));
        v = ch.raw;
      }
    }
    *reinterpret_cast<u32x4*>(&tile[r][pc * VP]) = v;
  }
  __syncthreads();
  // ---- row-wise blocks (optional): 128 rows x TC / 32 blocks, in order
  if (a.rq) {
    constexpr int PPR = TC / 8;                             // 8-value pieces per tile row
#pragma unroll
    for (int i = 0; i < kColsTileK * PPR / NT; ++i) {
      const int q = threadIdx.x + NT * i, r = q / PPR, pc = q % PPR;
      const int col = c0 + 8 * pc;
      const int64_t t = tt0 + r;
      float v[8];
      unpack8<T>(*reinterpret_cast<const u32x4*>(&tile[r][8 * pc]), v);
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));        // the block's four lanes
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int x = mx_scale_exp(amax);
      const float sc = ldexpf(1.0f, -x);
      const u32x2 o = {e4m3x4(v[0], v[1], v[2], v[3], sc), e4m3x4(v[4], v[5], v[6], v[7], sc)};
      if (t < n && col < a.C) {
        const int64_t row = tstart + t;
        st8(a.rq + row * a.rld + col, o);
        if ((pc & 3) == 0) a.rqs[row * a.rlds + col / 32] = (uint8_t)(x + 127);
      }
    }
  }
  // ---- token blocks: wave j, block j of the tile, columns lane (+ 64)
  constexpr int NCC = TC / 64;
  const int j = threadIdx.x >> 6, cl = threadIdx.x & 63;
  u32x4 o[NCC][2];
  int xs[NCC];
#pragma unroll
  for (int cc = 0; cc < NCC; ++cc) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = to_f32<T>(tile[32 * j + i][cl + 64 * cc]);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int x = mx_scale_exp(amax);
    const float sc = ldexpf(1.0f, -x);
#pragma unroll
    for (int w = 0; w < 8; ++w) o[cc][w >> 2][w & 3] = e4m3x4(v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3], sc);
    xs[cc] = x;
  }
  __syncthreads();                                          // input tile dead: reused for the output rows
#pragma unroll
  for (int cc = 0; cc < NCC; ++cc) {
    const int r = cl + 64 * cc;
    *reinterpret_cast<u32x4*>(qout + r * kColsOutRow + 32 * j) = o[cc][0];
    *reinterpret_cast<u32x4*>(qout + r * kColsOutRow + 32 * j + 16) = o[cc][1];
    qsc[r][j] = (uint8_t)(xs[cc] + 127);
  }
  __syncthreads();
  // ---- store: output row c0 + r gets 128 bytes at K position k0 + p0 (eight
  // lanes per row) and four scale bytes
  const int64_t k = a.k0 + p0;
#pragma unroll
  for (int i = 0; i < TC * 8 / NT; ++i) {
    const int q = threadIdx.x + NT * i, r = q >> 3, pc = q & 7;
    if (c0 + r < a.C)
      st16(a.out + (a.row0 + c0 + r) * a.Kpad + k + pc * 16, *reinterpret_cast<const u32x4*>(qout + r * kColsOutRow + pc * 16));
  }
  if (threadIdx.x < TC && c0 + (int)threadIdx.x < a.C) {
    const int r = threadIdx.x;
    *reinterpret_cast<uint32_t*>(a.scales + (a.row0 + c0 + r) * (a.Kpad / 32) + k / 32) =
        *reinterpret_cast<const uint32_t*>(&qsc[r][0]);
  }
}

// pad[0] = 0, pad[g + 1] = sum over g' <= g of len(g') rounded up to align:
// thread g rounds its segment's length, then a scan over the segments
// (waves in order).  G <= NT.
__global__ void __launch_bounds__(NT) mx_pad_offsets_kernel(const int32_t* offsets, int32_t* pad, int G, int align) {
  __shared__ int32_t s_w[NT / 64];
  const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
  int32_t v = 0;
  if (g < G) {
    const int32_t n = offsets[g + 1] - offsets[g];
    v = (n + align - 1) / align * align;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) s_w[wave] = v;
  __syncthreads();
  for (int w = 0; w < wave; ++w) v += s_w[w];
  if (g == 0) pad[0] = 0;
  if (g < G) pad[g + 1] = v;
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
  const int64_t nq = a.R * (a.K / 8);
  if (nq == 0) return hipSuccess;
  int64_t grid = (nq + NT - 1) / NT;
  if (grid > 65536) grid = 65536;
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL(mx_quant_rows_kernel<__bf16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL(mx_quant_rows_kernel<_Float16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(int dt, const MxColsArgs& a, hipStream_t s) {
  if (a.Kpad % kColsTileK || a.k0 % kColsTileK || a.C <= 0 || a.C % 8 || a.ld_in % 8) return hipErrorInvalidValue;
  if (!a.pad && (a.seg_len % kColsTileK)) return hipErrorInvalidValue;
  if (a.nblk <= 0) return hipSuccess;
  const int64_t tiles = (a.nblk * 32 + kColsTileK - 1) / kColsTileK;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  if (a.rq && (!a.rqs || a.gather || a.C % 32)) return hipErrorInvalidValue;
  if (a.wrow && !a.gather) return hipErrorInvalidValue;
  // 64-column tiles measured faster than 128 for the token-axis codes alone;
  // with the row-wise codes too, 128 (whole 128-byte row pieces)
  if (a.rq) {
    const dim3 grid((unsigned)tiles, (unsigned)((a.C + 127) / 128));
    switch (dt) {
      case DT_BF16: hipLaunchKernelGGL((mx_quant_cols_kernel<__bf16, 128>), grid, dim3(NT), 0, s, a); break;
      case DT_F16: hipLaunchKernelGGL((mx_quant_cols_kernel<_Float16, 128>), grid, dim3(NT), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  constexpr int tc = 64;
  const dim3 grid((unsigned)tiles, (unsigned)((a.C + tc - 1) / tc));
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL((mx_quant_cols_kernel<__bf16, tc>), grid, dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL((mx_quant_cols_kernel<_Float16, tc>), grid, dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mx_pad_offsets(const int32_t* offsets, int32_t* pad, int G, int align, hipStream_t s) {
  if (G < 1 || G > NT) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_pad_offsets_kernel, dim3(1), dim3(NT), 0, s, offsets, pad, G, align);
  return hipGetLastError();
}

}  // namespace moe
