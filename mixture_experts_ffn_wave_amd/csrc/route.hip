// Router: logits on the matrix cores, f32 softmax, top-k and renormalisation.
//
// spark-gpt README, feature list (Qwen3-MoE layers): softmax taken in fp32,
// top-k over the experts, the chosen probabilities optionally rescaled to sum
// to one (KochiLLM v1.0 model card, "Architecture").
//
// A workgroup owns 32 tokens.  The expert weights (rows of W_r, padded to a
// multiple of 32) are the MFMA "A" operand and the token rows the "B"
// operand, so the logits of a token end up in the accumulator layout: lane l
// holds token l % 32 for half of the experts (e = 32 s + 8 (r/4) + 4 (l/32) +
// r%4), the other half sits in lane l ^ 32.  Softmax and top-k then need only
// one cross-lane exchange per reduction.  Top-k is k rounds of "largest
// remaining logit, lower expert index on ties", which also fixes the slot
// order.  Up to 64 experts the four waves of a workgroup split the K range;
// above, they split the experts (both kernels below).

#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KB = 128;
constexpr int LROW = KB + 16;

// The logit bias and the selection bias (zeros without them) staged in LDS
// at kernel start by threads 0 .. 32 NSUB - 1, so that the epilogue reads
// them without global round trips.
template <int NSUB>
__device__ __forceinline__ void stage_bias(float* s_bias, float* s_sel, const RouteArgs& a) {
  const int i = threadIdx.x;
  if (i < 32 * NSUB) {
    s_bias[i] = (a.bias && i < a.E) ? a.bias[i] : 0.0f;
    s_sel[i] = (a.sel_bias && i < a.E) ? a.sel_bias[i] : 0.0f;
  }
}

// Softmax, probabilities, top-k and weights of the 32 tokens tb.. tb+31 whose
// logits sit in acc (lane l: token tb + l % 32, experts 32 s + 8 (r/4) +
// 4 (l/32) + r%4 in register r of acc[s]); s_bias / s_sel as staged by
// stage_bias.  s_wts: kWtsLds floats of LDS owned by this wave, where the
// chosen probabilities wait for their sum when they are renormalised.
// With a selection bias (aux-loss-free balancing, KohakUwULLM README, "Key
// features") the experts are ranked on probability + bias instead of on the
// logits; the weights are the unbiased probabilities either way.
constexpr int kWtsStride = 65;                 // 64 slots per token, odd stride: no bank conflicts
constexpr int kWtsLds = 32 * kWtsStride;
template <int NSUB>
__device__ __forceinline__ void route_epilogue(const f32x16 (&acc)[NSUB], int64_t tb, int lane, const RouteArgs& a,
                                               const float* s_bias, const float* s_sel, float* s_wts) {
  const int h = lane >> 5;
  const int64_t t = tb + (lane & 31);
  const bool tv = t < a.T;
  const int E = a.E;

  // logits (+ constant bias); padded experts never take part
  float z[NSUB][16];
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = s * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      z[s][r] = (e < E) ? acc[s][r] + s_bias[e] : -INFINITY;
      m = fmaxf(m, z[s][r]);
    }
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  float sum = 0.0f;
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = s * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (e < E) sum += expf(z[s][r] - m);
    }
  sum += __shfl_xor(sum, 32, 64);
  const bool sel = a.sel_bias != nullptr;
  if (sel) {
    // z now holds the probabilities (padded experts stay -inf)
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = s * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (e < E) z[s][r] = expf(z[s][r] - m) / sum;
      }
  }

  if (tv) {
    float* prow = a.probs + t * E;
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e0 = s * 32 + 8 * q + 4 * h;
        if (e0 >= E) continue;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = sel ? z[s][4 * q + i] : expf(z[s][4 * q + i] - m) / sum;
        if ((E & 3) == 0) {
          *reinterpret_cast<f32x4*>(prow + e0) = (f32x4){p[0], p[1], p[2], p[3]};
        } else {
          for (int i = 0; i < 4; ++i)
            if (e0 + i < E) prow[e0 + i] = p[i];
        }
      }
  }

  // top-k: k rounds of (largest remaining logit, lower index on ties).  The
  // ranking values and the candidates are fixed before the rounds, and each
  // round's scan is made of selects, not branches.
  float rk[NSUB][16];
  uint32_t avail[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    avail[s] = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = s * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      rk[s][r] = sel ? z[s][r] + s_sel[e] : z[s][r];
      if (e < E) avail[s] |= 1u << r;
    }
  }
  float psum = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY, bp = 0.0f;               // best ranking value, and its probability (sel)
    int be = -1;
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = s * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool better = ((avail[s] >> r) & 1u) && (be < 0 || rk[s][r] > bv);
        bv = better ? rk[s][r] : bv;
        bp = better ? z[s][r] : bp;
        be = better ? e : be;
      }
    const float pv = __shfl_xor(bv, 32, 64);
    const float pp = __shfl_xor(bp, 32, 64);
    const int pe = __shfl_xor(be, 32, 64);
    const bool partner = (be < 0) || (pe >= 0 && (pv > bv || (pv == bv && pe < be)));
    const float wv = partner ? pv : bv;
    const float wp = partner ? pp : bp;
    const int we = partner ? pe : be;
    if (!partner) {
      const int s = we >> 5, w5 = we & 31;
      const int r = ((w5 >> 3) << 2) | (w5 & 3);
#pragma unroll
      for (int ss = 0; ss < NSUB; ++ss)
        if (ss == s) avail[ss] &= ~(1u << r);
    }
    const float pj = sel ? wp : expf(wv - m) / sum;
    psum += pj;
    if (tv && h == 0) {
      a.idx[t * a.k + j] = we;
      if (a.renorm) s_wts[(lane & 31) * kWtsStride + j] = pj;
      else a.wts[t * a.k + j] = pj;
    }
  }
  if (a.renorm && tv && h == 0) {
    for (int j = 0; j < a.k; ++j) a.wts[t * a.k + j] = s_wts[(lane & 31) * kWtsStride + j] / psum;
  }
}

// Exchange with the partner lane of butterfly stage S inside each group of
// eight lanes, as a DPP move (a VALU operand modifier, no LDS round trip):
// stage 0 pairs lanes i, i ^ 1 and stage 1 lanes i, i ^ 2 (quad permutes),
// stage 2 lane i with lane 7 - i of its half-row (half mirror).  After the
// three stages every lane of the group has combined all eight values, in the
// same pairs as an xor-1, 2, 4 butterfly (after stage 1 each quad holds one
// value), so maxima, sums and the ranking below come out identical.
template <int S>
__device__ __forceinline__ int x8(int v) {
  static_assert(S >= 0 && S < 3, "three stages");
  constexpr int CTRL = S == 0 ? 0xB1 : (S == 1 ? 0x4E : 0x141);   // quad_perm [1,0,3,2], [2,3,0,1]; row_half_mirror
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int S>
__device__ __forceinline__ float x8f(float v) { return __int_as_float(x8<S>(__float_as_int(v))); }

// One stage of the top-k round's merge: keep the partner's candidate when it
// ranks higher (larger value, lower expert index on equal values; -1 = none).
template <int S>
__device__ __forceinline__ void topk_merge(float& bv, float& bp, float& bz, int& be) {
  const float ov = x8f<S>(bv), op = x8f<S>(bp), oz = x8f<S>(bz);
  const int oe = x8<S>(be);
  const bool take = (be < 0) || (oe >= 0 && (ov > bv || (ov == bv && oe < be)));
  if (take) {
    bv = ov;
    bp = op;
    bz = oz;
    be = oe;
  }
}

// The same epilogue with all four waves of a workgroup: the 32 tokens'
// logits sit in LDS in the accumulator layout ([subtile][register][lane],
// see route_epilogue); wave w takes tokens 8w .. 8w+7, eight lanes per token,
// lane g of a token owning experts EPL g .. EPL g + EPL - 1.  Maxima, sums and
// the k rounds of the top-k are butterflies over the token's eight lanes
// (ties to the lower expert index, as before).  s_wts: kWtsLds floats of LDS
// apart from the logits, rows indexed by token.
template <int NSUB>
__device__ __forceinline__ void route_epilogue_wide(const float* red, int64_t tb, int wave, int lane,
                                                    const RouteArgs& a, const float* s_bias, const float* s_sel,
                                                    float* s_wts) {
  constexpr int EPL = 4 * NSUB;                   // experts per lane (32 NSUB over 8 lanes)
  static_assert(EPL <= 32, "taken mask");
  const int tl = wave * 8 + (lane >> 3), g = lane & 7;
  const int64_t t = tb + tl;
  const bool tv = t < a.T;
  const int E = a.E;
  const bool sel = a.sel_bias != nullptr;
  // gather this lane's logits (+ constant bias) from the accumulator layout
  float z[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = g * EPL + i, sub = e >> 5, w = e & 31;
    const int r = 4 * (w >> 3) + (w & 3), hh = (w >> 2) & 1;
    const float v = red[((sub * 16) + r) * 64 + tl + 32 * hh];
    z[i] = (e < E) ? v + s_bias[e] : -INFINITY;
    m = fmaxf(m, z[i]);
  }
  m = fmaxf(m, x8f<0>(m));
  m = fmaxf(m, x8f<1>(m));
  m = fmaxf(m, x8f<2>(m));
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (g * EPL + i < E) sum += expf(z[i] - m);
  sum += x8f<0>(sum);
  sum += x8f<1>(sum);
  sum += x8f<2>(sum);
  // probabilities (kept in z when a selection bias ranks on them); the ReLU
  // router stores its gates max(z, 0) in their place
  const bool relu = a.relu != 0;
  float p[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    p[i] = (g * EPL + i < E) ? (relu ? fmaxf(z[i], 0.0f) : expf(z[i] - m) / sum) : 0.0f;
  if (tv) {
    float* prow = a.probs + t * E + g * EPL;
    if ((E & 3) == 0) {
#pragma unroll
      for (int q = 0; q < EPL / 4; ++q)
        if (g * EPL + 4 * q < E)
          *reinterpret_cast<f32x4*>(prow + 4 * q) = (f32x4){p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]};
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (g * EPL + i < E) prow[i] = p[i];
    }
  }
  // top-k: k rounds of (largest remaining ranking value, lower index on ties);
  // the ReLU router only takes positive logits, a round without one leaves
  // the slot empty (index -1, weight 0).  The ranking values and the
  // candidates are fixed before the rounds, and each round's scan over the
  // lane's experts is made of selects, not branches.
  float rk[EPL];
  uint32_t avail = 0u;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = g * EPL + i;
    rk[i] = sel ? p[i] + s_sel[e < E ? e : 0] : z[i];
    if (e < E && (!relu || z[i] > 0.0f)) avail |= 1u << i;
  }
  float psum = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY, bp = 0.0f, bz = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const bool better = ((avail >> i) & 1u) && (bi < 0 || rk[i] > bv);
      bv = better ? rk[i] : bv;
      bp = better ? p[i] : bp;
      bz = better ? z[i] : bz;
      bi = better ? i : bi;
    }
    int be = bi < 0 ? -1 : g * EPL + bi;
    topk_merge<0>(bv, bp, bz, be);
    topk_merge<1>(bv, bp, bz, be);
    topk_merge<2>(bv, bp, bz, be);
    if (be >= 0 && be / EPL == g) avail &= ~(1u << (be - g * EPL));
    // (the chosen probability is the p of the stored row: the same expression)
    const float pj = be < 0 ? 0.0f : (relu ? bz : bp);
    psum += pj;
    if (tv && g == 0) {
      a.idx[t * a.k + j] = be;
      if (a.renorm) s_wts[tl * kWtsStride + j] = pj;
      else a.wts[t * a.k + j] = pj;
    }
  }
  if (a.renorm && tv && g == 0) {
    for (int j = 0; j < a.k; ++j) a.wts[t * a.k + j] = s_wts[tl * kWtsStride + j] / psum;
  }
}

// Few experts (E <= 64): 32 tokens per workgroup of KW waves that split the K
// range.  Wave w multiplies chunks w, w + KW, ... into accumulators of its
// own, staged through LDS tiles of its own (no workgroup barrier inside the
// loop); the partial logits are then added in wave order through LDS and
// wave 0 finishes the tokens.  Four times the waves of one-wave workgroups
// over the same tokens, so each wave's serial chain of loads and MFMAs is a
// quarter as long.
template <typename T, int NSUB, int KW>
__global__ void __launch_bounds__(KW * 64) route_ksplit_kernel(RouteArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int BK = KB / ES;
  constexpr int EP = 32 * NSUB;
  constexpr int XPL = 32 * 8 / 64;        // 16-byte chunks of the x tile per lane
  constexpr int WPL = EP * 8 / 64;        // 16-byte chunks of the W tile per lane
  constexpr int WREG = (32 + EP) * LROW;  // one wave's tiles
  constexpr int RED = (KW - 1) * NSUB * 16 * 64 * 4;
  static_assert(RED <= KW * WREG && (NSUB * 16 * 64 + kWtsLds) * 4 <= KW * WREG,
                "partial logits, logits and weights scratch fit in the tiles' LDS");
  __shared__ __attribute__((aligned(16))) char lds[KW * WREG];
  __shared__ float s_bias[EP], s_sel[EP];
  static_assert(EP <= KW * 64, "bias staged by one thread per expert");
  stage_bias<NSUB>(s_bias, s_sel, a);

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char* lx = lds + wave * WREG;
  char* lw = lx + 32 * LROW;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const char* xb = static_cast<const char*>(a.x);
  const char* wb = static_cast<const char*>(a.w);

  auto load = [&](int kc, u32x4* rx, u32x4* rw) {
#pragma unroll
    for (int s = 0; s < XPL; ++s) {
      const int c = lane + 64 * s, r = c >> 3, cc = c & 7;
      rx[s] = (t0 + r < a.T) ? ld16(xb + ((t0 + r) * a.d + kc) * ES + cc * 16) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < WPL; ++s) {
      const int c = lane + 64 * s, r = c >> 3, cc = c & 7;
      rw[s] = (r < a.E) ? ld16(wb + ((int64_t)r * a.d + kc) * ES + cc * 16) : (u32x4){0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = 0.0f;

  constexpr int CH = Mma32<T>::kChunks;
  constexpr int PF = 2;
  const int nk = a.d / BK;
  const int nmine = wave < nk ? (nk - wave + KW - 1) / KW : 0;   // chunks wave, wave + KW, ...
  u32x4 rx[PF][XPL], rw[PF][WPL];
#pragma unroll
  for (int q = 0; q < PF; ++q)
    if (q < nmine) load((wave + KW * q) * BK, rx[q], rw[q]);
  for (int i0 = 0; i0 < nmine; i0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int i = i0 + q;
      if (i < nmine) {
        // LDS accesses of one wave execute in order: the tiles written here
        // are read below, and the reads of the previous chunk came first
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s = 0; s < XPL; ++s) {
          const int c = lane + 64 * s;
          st16(lx + (c >> 3) * LROW + (c & 7) * 16, rx[q][s]);
        }
#pragma unroll
        for (int s = 0; s < WPL; ++s) {
          const int c = lane + 64 * s;
          st16(lw + (c >> 3) * LROW + (c & 7) * 16, rw[q][s]);
        }
        asm volatile("" ::: "memory");
        if (i + PF < nmine) load((wave + KW * (i + PF)) * BK, rx[q], rw[q]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          const int kb = ks * 16 * ES + (lane >> 5) * 8 * ES;
          u32x4 fb[CH];
          const char* xrow = lx + (lane & 31) * LROW + kb;
#pragma unroll
          for (int ch = 0; ch < CH; ++ch) fb[ch] = ld16(xrow + ch * 16);
#pragma unroll
          for (int s = 0; s < NSUB; ++s) {
            u32x4 fa[CH];
            const char* wrow = lw + (s * 32 + (lane & 31)) * LROW + kb;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) fa[ch] = ld16(wrow + ch * 16);
            Mma32<T>::run(acc[s], fa, fb);
          }
        }
        asm volatile("" ::: "memory");
      }
    }
  }

  // partial logits of waves 1.. KW-1 -> LDS; wave 0 adds them in wave order
  float* red = reinterpret_cast<float*>(lds);
  __syncthreads();
  if (wave > 0) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[(((wave - 1) * NSUB + s) * 16 + r) * 64 + lane] = acc[s][r];
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < KW; ++w)
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[s][r] += red[(((w - 1) * NSUB + s) * 16 + r) * 64 + lane];
  }
  __syncthreads();                                 // every wave has read the partials
  float* logits = red;                             // [NSUB][16][64], then the weights scratch
  if (wave == 0) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) logits[((s * 16) + r) * 64 + lane] = acc[s][r];
  }
  __syncthreads();
  route_epilogue_wide<NSUB>(logits, t0, wave, lane, a, s_bias, s_sel, logits + NSUB * 16 * 64);
}

// Many experts (64 < E <= 256): 32 tokens per workgroup of four waves that
// split the experts.  The x tile and the whole W tile of a K chunk are
// staged once in LDS; wave w multiplies expert subtiles w, w + 4, ... (NSUB/4
// of them) for the 32 tokens over the full K range.  The logits then meet in
// LDS in the accumulator layout and wave 0 finishes the tokens.  Eight waves
// per CU instead of two for the same tokens.
template <typename T, int NSUB>
__global__ void __launch_bounds__(256) route_esplit_kernel(RouteArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int BK = KB / ES;
  constexpr int EP = 32 * NSUB;
  constexpr int NW = 4, SPW = NSUB / NW;           // expert subtiles per wave
  constexpr int NTH = 64 * NW;
  constexpr int XPT = 32 * 8 / NTH;                // 16-byte chunks of the x tile per thread (1)
  constexpr int WPT = EP * 8 / NTH;                // 16-byte chunks of the W tile per thread
  constexpr int TILES = (32 + EP) * LROW;
  static_assert(NSUB % NW == 0 && XPT == 1 && WPT >= 1, "tile split");
  static_assert(NSUB * 16 * 64 * 4 <= TILES, "logits fit in the tiles' LDS");
  __shared__ __attribute__((aligned(16))) char lds[TILES];
  __shared__ float s_bias[EP], s_sel[EP];
  __shared__ float s_wts[kWtsLds];
  stage_bias<NSUB>(s_bias, s_sel, a);              // visible after the K loop's first barrier
  char* lx = lds;
  char* lw = lds + 32 * LROW;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const char* xb = static_cast<const char*>(a.x);
  const char* wb = static_cast<const char*>(a.w);
  auto load = [&](int kc, u32x4& rx, u32x4* rw) {
    {
      const int r = tid >> 3, cc = tid & 7;
      rx = (t0 + r < a.T) ? ld16(xb + ((t0 + r) * a.d + kc) * ES + cc * 16) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < WPT; ++s) {
      const int c = tid + NTH * s, r = c >> 3, cc = c & 7;
      rw[s] = (r < a.E) ? ld16(wb + ((int64_t)r * a.d + kc) * ES + cc * 16) : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&](const u32x4& rx, const u32x4* rw) {
    st16(lx + (tid >> 3) * LROW + (tid & 7) * 16, rx);
#pragma unroll
    for (int s = 0; s < WPT; ++s) {
      const int c = tid + NTH * s;
      st16(lw + (c >> 3) * LROW + (c & 7) * 16, rw[s]);
    }
  };

  f32x16 acc[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = 0.0f;

  constexpr int CH = Mma32<T>::kChunks;
  constexpr int PF = 2;
  const int nk = a.d / BK;
  u32x4 rx[PF], rw[PF][WPT];
#pragma unroll
  for (int q = 0; q < PF; ++q)
    if (q < nk) load(q * BK, rx[q], rw[q]);
  for (int kc0 = 0; kc0 < nk; kc0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int kc = kc0 + q;
      if (kc < nk) {
        stage(rx[q], rw[q]);
        __syncthreads();
        if (kc + PF < nk) load((kc + PF) * BK, rx[q], rw[q]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          const int kb = ks * 16 * ES + (lane >> 5) * 8 * ES;
          u32x4 fb[CH];
          const char* xrow = lx + (lane & 31) * LROW + kb;
#pragma unroll
          for (int ch = 0; ch < CH; ++ch) fb[ch] = ld16(xrow + ch * 16);
#pragma unroll
          for (int s = 0; s < SPW; ++s) {
            u32x4 fa[CH];
            const char* wrow = lw + ((wave + NW * s) * 32 + (lane & 31)) * LROW + kb;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) fa[ch] = ld16(wrow + ch * 16);
            Mma32<T>::run(acc[s], fa, fb);
          }
        }
        __syncthreads();
      }
    }
  }

  // every wave's subtiles -> LDS in the accumulator layout [subtile][r][lane]
  float* red = reinterpret_cast<float*>(lds);
  __syncthreads();                                 // (also covers an empty K loop)
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(((wave + NW * s) * 16) + r) * 64 + lane] = acc[s][r];
  __syncthreads();
  route_epilogue_wide<NSUB>(red, t0, wave, lane, a, s_bias, s_sel, s_wts);
}

// Many experts, more tokens per workgroup: 64 tokens and eight waves (two
// token halves by four expert quarters).  Each K chunk of W_r staged in LDS
// then serves 64 tokens instead of 32: x still streams once from HBM, and
// W_r (re-read from L2 by every workgroup, four times the bytes of x's rows
// at 128 experts with 32 tokens) is read half as often.  One workgroup per
// CU at 16384 tokens.  The two halves finish their tokens as above, four
// waves each.
template <typename T, int NSUB>
__global__ void __launch_bounds__(512) route_esplit64_kernel(RouteArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int BK = KB / ES;
  constexpr int EP = 32 * NSUB;
  constexpr int NW = 8, SPW = NSUB / 4;            // expert subtiles per wave
  constexpr int NTH = 64 * NW;
  constexpr int WPT = EP * 8 / NTH;                // 16-byte chunks of the W tile per thread
  constexpr int TILES = (64 + EP) * LROW;
  constexpr int RED = 2 * NSUB * 16 * 64 * 4;      // logits of both halves
  constexpr int LDSB = TILES > RED ? TILES : RED;
  static_assert(NSUB % 4 == 0 && 64 * 8 == NTH && WPT >= 1 && WPT * NTH == EP * 8, "tile split");
  __shared__ __attribute__((aligned(16))) char lds[LDSB];
  __shared__ float s_bias[EP], s_sel[EP];
  __shared__ float s_wts[2 * kWtsLds];
  stage_bias<NSUB>(s_bias, s_sel, a);              // visible after the K loop's first barrier
  char* lx = lds;
  char* lw = lds + 64 * LROW;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int th = wave & 1, eg = wave >> 1;         // token half, expert quarter
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const char* xb = static_cast<const char*>(a.x);
  const char* wb = static_cast<const char*>(a.w);
  auto load = [&](int kc, u32x4& rx, u32x4* rw) {
    {
      const int r = tid >> 3, cc = tid & 7;
      rx = (t0 + r < a.T) ? ld16(xb + ((t0 + r) * a.d + kc) * ES + cc * 16) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < WPT; ++s) {
      const int c = tid + NTH * s, r = c >> 3, cc = c & 7;
      rw[s] = (r < a.E) ? ld16(wb + ((int64_t)r * a.d + kc) * ES + cc * 16) : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&](const u32x4& rx, const u32x4* rw) {
    st16(lx + (tid >> 3) * LROW + (tid & 7) * 16, rx);
#pragma unroll
    for (int s = 0; s < WPT; ++s) {
      const int c = tid + NTH * s;
      st16(lw + (c >> 3) * LROW + (c & 7) * 16, rw[s]);
    }
  };

  f32x16 acc[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = 0.0f;

  constexpr int CH = Mma32<T>::kChunks;
  constexpr int PF = 3;
  const int nk = a.d / BK;
  u32x4 rx[PF], rw[PF][WPT];
#pragma unroll
  for (int q = 0; q < PF; ++q)
    if (q < nk) load(q * BK, rx[q], rw[q]);
  for (int kc0 = 0; kc0 < nk; kc0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int kc = kc0 + q;
      if (kc < nk) {
        stage(rx[q], rw[q]);
        __syncthreads();
        if (kc + PF < nk) load((kc + PF) * BK, rx[q], rw[q]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          const int kb = ks * 16 * ES + (lane >> 5) * 8 * ES;
          u32x4 fb[CH];
          const char* xrow = lx + (th * 32 + (lane & 31)) * LROW + kb;
#pragma unroll
          for (int ch = 0; ch < CH; ++ch) fb[ch] = ld16(xrow + ch * 16);
#pragma unroll
          for (int s = 0; s < SPW; ++s) {
            u32x4 fa[CH];
            const char* wrow = lw + ((eg + 4 * s) * 32 + (lane & 31)) * LROW + kb;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) fa[ch] = ld16(wrow + ch * 16);
            Mma32<T>::run(acc[s], fa, fb);
          }
        }
        __syncthreads();
      }
    }
  }

  // logits -> LDS: [token half][subtile][r][lane] (the accumulator layout)
  float* red = reinterpret_cast<float*>(lds);
  __syncthreads();                                 // (also covers an empty K loop)
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((th * NSUB + eg + 4 * s) * 16 + r) * 64 + lane] = acc[s][r];
  __syncthreads();
  const int half = wave >> 2;                      // waves 0-3 finish tokens 0-31, waves 4-7 tokens 32-63
  route_epilogue_wide<NSUB>(red + half * NSUB * 16 * 64, t0 + 32 * half, wave & 3, lane, a, s_bias, s_sel,
                            s_wts + half * kWtsLds);
}

template <typename T, int NSUB>
hipError_t launch_route_esplit64(const RouteArgs& a, hipStream_t s) {
  const int64_t grid = (a.T + 63) / 64;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((route_esplit64_kernel<T, NSUB>), dim3((unsigned)grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <typename T, int NSUB>
hipError_t launch_route_esplit(const RouteArgs& a, hipStream_t s) {
  const int64_t grid = (a.T + 31) / 32;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((route_esplit_kernel<T, NSUB>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int NSUB, int KW>
hipError_t launch_route_ksplit(const RouteArgs& a, hipStream_t s) {
  const int64_t grid = (a.T + 31) / 32;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((route_ksplit_kernel<T, NSUB, KW>), dim3((unsigned)grid), dim3(KW * 64), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_route_dt(const RouteArgs& a, hipStream_t s) {
  const int nsub = (a.E + 31) / 32;
  if (nsub <= 1) return launch_route_ksplit<T, 1, 4>(a, s);
  if (nsub <= 2) return launch_route_ksplit<T, 2, 4>(a, s);
  if (nsub <= 4) return launch_route_esplit64<T, 4>(a, s);
  return launch_route_esplit<T, 8>(a, s);
}

// Aux-loss-free balancing update, one thread per expert: the sign of
// (mean load - load) decided exactly in integers, then one f32 addition.
__global__ void __launch_bounds__(256) balance_update_kernel(const int32_t* counts, float* sel_bias, int64_t T,
                                                             int E, int k, float gamma) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int64_t diff = T * k - (int64_t)E * counts[e];
  const float sgn = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
  sel_bias[e] = sel_bias[e] + gamma * sgn;
}

// ---- Sinkhorn router (KohakUwULLM README, "Key features": Sinkhorn routers
// beside the default; the published Sinkhorn-Knopp balancing of the batch's
// probability matrix).  The probabilities come from the plain router pass.
constexpr int SKT = kSinkhornTokens;
constexpr int SK_EMAX = 256;

// One block of 32 tokens of one round: a_t = (1/T) / sum_e p_te b_e (b = 1
// in the first round; eight lanes per token, each summing every eighth
// expert, then a fixed butterfly), and the block's column partials
// sum_t p_te a_t over its tokens in order.
__global__ void __launch_bounds__(256) sinkhorn_rows_kernel(SinkhornArgs a, int first) {
  __shared__ float s_p[SKT * (SK_EMAX + 1)];
  __shared__ float s_b[SK_EMAX], s_a[SKT];
  const int tid = threadIdx.x, E = a.E, ld = E + 1;
  const int64_t t0 = (int64_t)blockIdx.x * SKT;
  const int nt = (a.T - t0) < SKT ? (int)(a.T - t0) : SKT;
  for (int e = tid; e < E; e += 256) s_b[e] = first ? 1.0f : a.b[e];
  for (int i = tid; i < nt * E; i += 256) {
    const int t = i / E, e = i - t * E;
    s_p[t * ld + e] = a.probs[(t0 + t) * E + e];
  }
  __syncthreads();
  {
    const int t = tid >> 3, g = tid & 7;
    float sum = 0.0f;
    if (t < nt)
      for (int e = g; e < E; e += 8) sum = fmaf(s_p[t * ld + e], s_b[e], sum);
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    sum += __shfl_xor(sum, 4, 64);
    if (g == 0 && t < nt) s_a[t] = 1.0f / ((float)a.T * sum);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float c = 0.0f;
    for (int t = 0; t < nt; ++t) c = fmaf(s_p[t * ld + e], s_a[t], c);
    a.part[(int64_t)blockIdx.x * E + e] = c;
  }
}

// b_e = (1/E) / (sum over blocks of the column partials, in block order).
__global__ void __launch_bounds__(256) sinkhorn_cols_kernel(SinkhornArgs a) {
  const int64_t nblk = (a.T + SKT - 1) / SKT;
  for (int e = threadIdx.x; e < a.E; e += 256) {
    float c = 0.0f;
    for (int64_t b = 0; b < nblk; ++b) c += a.part[b * a.E + e];
    a.b[e] = 1.0f / ((float)a.E * c);
  }
}

// Top-k of p_te b_e per token (k rounds: largest remaining score, lower
// expert index on ties, slots in that order); weights = the chosen p_te,
// divided by their sum (in slot order) when renormalising.  Eight lanes per
// token, lane g owning experts g, g + 8, ...; rounds are butterflies over
// the eight lanes.
__global__ void __launch_bounds__(256) sinkhorn_select_kernel(SinkhornArgs a) {
  constexpr int EPL = SK_EMAX / 8;
  __shared__ float s_b[SK_EMAX];
  const int tid = threadIdx.x, E = a.E;
  for (int e = tid; e < E; e += 256) s_b[e] = a.b[e];
  __syncthreads();
  const int t_l = tid >> 3, g = tid & 7;
  const int64_t t = (int64_t)blockIdx.x * SKT + t_l;
  const bool tv = t < a.T;
  float p[EPL], v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = g + 8 * i;
    const bool ok = tv && e < E;
    p[i] = ok ? a.probs[t * E + e] : 0.0f;
    v[i] = ok ? p[i] * s_b[e] : -INFINITY;
  }
  uint32_t taken = 0u;
  float psum = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY, bp = 0.0f;
    int be = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = g + 8 * i;
      if (e < E && !((taken >> i) & 1u) && (be < 0 || v[i] > bv)) {
        bv = v[i];
        bp = p[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64), op = __shfl_xor(bp, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (be < 0 || (oe >= 0 && (ov > bv || (ov == bv && oe < be)))) {
        bv = ov;
        bp = op;
        be = oe;
      }
    }
    if (be >= 0 && (be & 7) == g) taken |= 1u << (be >> 3);
    psum += bp;
    if (tv && g == 0) {
      a.idx[t * a.k + j] = be;
      a.wts[t * a.k + j] = bp;                     // divided by the sum below when renormalising
    }
  }
  if (a.renorm && tv && g == 0)
    for (int j = 0; j < a.k; ++j) a.wts[t * a.k + j] = a.wts[t * a.k + j] / psum;
}

// ---- Expert-choice router (KohakUwULLM README, "Key features": expert-choice
// routers beside the default; the published method: every expert takes its C
// tokens of largest probability).
constexpr int EC_T = 64;                           // tokens per transpose tile

// probs [T, E] -> pT [E, T] through LDS (reads and writes along rows).
__global__ void __launch_bounds__(256) ec_transpose_kernel(ExpertChoiceArgs a) {
  __shared__ float tile[EC_T][65];
  const int E = a.E;
  const int64_t t0 = (int64_t)blockIdx.x * EC_T;
  const int nt = (a.T - t0) < EC_T ? (int)(a.T - t0) : EC_T;
  for (int i = threadIdx.x; i < nt * E; i += 256) {
    const int t = i / E, e = i - t * E;
    tile[t][e] = a.probs[(t0 + t) * E + e];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * E; i += 256) {
    const int e = i / nt, t = i - e * nt;
    a.pT[(int64_t)e * a.T + t0 + t] = tile[t][e];
  }
}

// One workgroup per expert.  Probabilities are non-negative, so their f32
// bit patterns order as unsigned integers: four 8-bit radix passes find the
// pattern K of the C-th largest value and how many tokens equal to K are
// taken (the rest of the C are above K); a last pass in token order takes the
// tokens above K and the first of those equal to K (a block prefix count).
__global__ void __launch_bounds__(256) expert_choice_kernel(ExpertChoiceArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_key, s_wave[4];
  __shared__ long long s_need;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x, E = a.E;
  const float* col = a.pT + (int64_t)e * a.T;
  uint32_t prefix = 0u, mask = 0u;
  long long need = a.C;                            // tokens still to take at or below the prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    for (int64_t t = tid; t < a.T; t += 256) {
      const uint32_t key = __float_as_uint(col[t]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      long long above = 0;
      int dsel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (above + (long long)hist[dg] >= need) { dsel = dg; break; }
        above += hist[dg];
      }
      s_key = prefix | ((uint32_t)dsel << shift);
      s_need = need - above;
    }
    __syncthreads();
    prefix = s_key;
    need = s_need;
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  // prefix = K; take key > K, and the first `need` tokens with key == K
  long long base = 0;                              // tokens equal to K before this chunk
  for (int64_t c0 = 0; c0 < a.T; c0 += 256) {
    const int64_t t = c0 + tid;
    const bool tv = t < a.T;
    const float pv = tv ? col[t] : 0.0f;
    const uint32_t key = __float_as_uint(pv);
    const bool eq = tv && key == prefix;
    // exclusive prefix count of eq over the chunk: within the wave, then waves in order
    const unsigned long long bal = __ballot(eq);
    const uint32_t below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    uint32_t before = 0u, total = 0u;
    for (int w = 0; w < 4; ++w) {
      before += (w < wave) ? s_wave[w] : 0u;
      total += s_wave[w];
    }
    const long long rank = base + before + below;
    const bool take = tv && (key > prefix || (eq && rank < need));
    if (tv) {
      a.idx[t * E + e] = take ? e : -1;
      a.wts[t * E + e] = take ? pv : 0.0f;
    }
    base += total;
    __syncthreads();                               // s_wave reused by the next chunk
  }
}

}  // namespace

hipError_t launch_balance_update(const int32_t* counts, float* sel_bias, int64_t T, int E, int k, float gamma,
                                 hipStream_t s) {
  if (E < 1 || E > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(balance_update_kernel, dim3(1), dim3(256), 0, s, counts, sel_bias, T, E, k, gamma);
  return hipGetLastError();
}

hipError_t launch_sinkhorn_rows(const SinkhornArgs& a, bool first, hipStream_t s) {
  const int64_t grid = (a.T + SKT - 1) / SKT;
  if (grid == 0) return hipSuccess;
  if (a.E < 1 || a.E > SK_EMAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sinkhorn_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, a, first ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_sinkhorn_cols(const SinkhornArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.E < 1 || a.E > SK_EMAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sinkhorn_cols_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sinkhorn_select(const SinkhornArgs& a, hipStream_t s) {
  const int64_t grid = (a.T + SKT - 1) / SKT;
  if (grid == 0) return hipSuccess;
  if (a.E < 1 || a.E > SK_EMAX || a.k < 1 || a.k > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sinkhorn_select_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_expert_choice(const ExpertChoiceArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.E < 1 || a.E > 64 || a.C < 0 || a.C > a.T) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ec_transpose_kernel, dim3((unsigned)((a.T + EC_T - 1) / EC_T)), dim3(256), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(expert_choice_kernel, dim3((unsigned)a.E), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route(int dt, const RouteArgs& a, hipStream_t s) {
  switch (dt) {
    case DT_BF16: return launch_route_dt<__bf16>(a, s);
    case DT_F16: return launch_route_dt<_Float16>(a, s);
    case DT_F32: return launch_route_dt<float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
