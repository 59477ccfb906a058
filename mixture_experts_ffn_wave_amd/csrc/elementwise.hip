// Bandwidth-bound kernels of the layer: weighted combine and its backward,
// the router backward (softmax Jacobian, renormalisation, balancing term),
// the reduction of the router weight gradient, and the balancing statistic.
// Every reduction runs in a fixed order; there are no float atomics.

#include <math.h>

#include "common.h"
#include "kernels.h"
#include "mx_codec.h"

namespace moe {
namespace {

constexpr int NT = 256;

// y[t] = sum_j w[t,j] * y_perm[inv[t,j]] (+ y_shared[t]); one wave per token,
// 16-byte vectors along the row (y_perm rows are f32), f32 accumulation in
// slot order.  Slots go in batches of KG whose row loads are all issued
// before the first is used (a load under a per-slot branch would wait for
// each row in turn).
template <typename T, int KG, typename YT>
__global__ void __launch_bounds__(NT) combine_kernel(CombineArgs a) {
  constexpr int VR = 16 / sizeof(T);   // output elements per 16-byte chunk
  constexpr int YC = VR * sizeof(YT) / 16;   // 16-byte chunks of y_perm per output chunk
  const YT* yperm = static_cast<const YT*>(a.y_perm);
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (NT / 64);
  const int64_t rowbytes = (int64_t)a.d * sizeof(T);
  const int nch = (int)(rowbytes / 16);
  const char* ys = static_cast<const char*>(a.y_shared);
  char* yo = static_cast<char*>(a.y);
  for (int64_t t = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6); t < a.T; t += waves) {
    int r_l = 0;
    float w_l = 0.0f;
    if (lane < a.k) {
      r_l = a.inv[t * a.k + lane];
      w_l = a.wts[t * a.k + lane];
    }
    for (int c0 = 0; c0 < nch; c0 += 64) {
      const int c = c0 + lane;
      const bool ok = c < nch;
      float acc[VR];
#pragma unroll
      for (int i = 0; i < VR; ++i) acc[i] = 0.0f;
      for (int j0 = 0; j0 < a.k; j0 += KG) {
        u32x4 v[KG][YC];
        int r[KG];
#pragma unroll
        for (int u = 0; u < KG; ++u) {
          r[u] = __shfl(r_l, (j0 + u) & 63, 64);
          const bool use = ok && j0 + u < a.k && r[u] >= 0;
          const u32x4* src = reinterpret_cast<const u32x4*>(yperm + (int64_t)r[u] * a.d + (int64_t)c * VR);
#pragma unroll
          for (int q = 0; q < YC; ++q) v[u][q] = use ? src[q] : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < KG; ++u) {
          const float w = __shfl(w_l, (j0 + u) & 63, 64);
          if (j0 + u < a.k && r[u] >= 0) {                  // wave-uniform
#pragma unroll
            for (int q = 0; q < YC; ++q) {
              Chunk<YT> yc;
              yc.raw = v[u][q];
#pragma unroll
              for (int i = 0; i < Chunk<YT>::N; ++i)
                acc[Chunk<YT>::N * q + i] = fmaf(w, to_f32<YT>(yc.e[i]), acc[Chunk<YT>::N * q + i]);
            }
          }
        }
      }
      if (ok) {
        if (ys) {
          Chunk<T> ch;
          ch.raw = ld16(ys + t * rowbytes + (int64_t)c * 16);
#pragma unroll
          for (int i = 0; i < VR; ++i) acc[i] += to_f32<T>(ch.e[i]);
        }
        Chunk<T> o;
#pragma unroll
        for (int i = 0; i < VR; ++i) o.e[i] = from_f32<T>(acc[i]);
        st16(yo + t * rowbytes + (int64_t)c * 16, o.raw);
      }
    }
  }
}

// dY_perm[inv[t,j]] = w[t,j] * dy[t];  g[t,j] = <dy[t], y_perm[inv[t,j]]>.
// Slots in batches of KG: the batch's y_perm rows and the dy row are loaded
// together; each slot's dot product keeps its own order (row position, then
// the butterfly).
// MX-fp8 row-wise codes of one 16-byte chunk c (8 values) of a row: the four
// lanes holding chunks 4b .. 4b+3 (consecutive lanes) form a 32-value block,
// whose maximum they exchange; the lane of chunk 4b writes the scale byte.
// Every lane of the wave calls this (the exchange is a shuffle).
template <typename T>
__device__ __forceinline__ void mx_row_codes(u32x4 raw, bool ok, uint8_t* q, uint8_t* qs, int c) {
  float v[8];
  unpack8<T>(raw, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int x = mx_scale_exp(amax);
  const float sc = ldexpf(1.0f, -x);
  const u32x2 o = {e4m3x4(v[0], v[1], v[2], v[3], sc), e4m3x4(v[4], v[5], v[6], v[7], sc)};
  if (ok) {
    st8(q, o);
    if ((c & 3) == 0) *qs = (uint8_t)(x + 127);
  }
}

template <typename T, int KG, bool MXQ, bool GD>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) combine_bwd_kernel(CombineBwdArgs a) {
  constexpr int VR = 16 / sizeof(T);
  const T* yperm = static_cast<const T*>(a.y_perm);   // (GD) in the activation dtype
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (NT / 64);
  const int64_t rowbytes = (int64_t)a.d * sizeof(T);
  const int nch = (int)(rowbytes / 16);
  const char* dyb = static_cast<const char*>(a.dy);
  char* dyp = static_cast<char*>(a.dy_perm);
  for (int64_t t = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6); t < a.T; t += waves) {
    int r_l = 0;
    float w_l = 0.0f;
    if (lane < a.k) {
      r_l = a.inv[t * a.k + lane];
      w_l = a.wts[t * a.k + lane];
    }
    for (int j0 = 0; j0 < a.k; j0 += KG) {
      int r[KG];
      float w[KG], dot[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        r[u] = __shfl(r_l, (j0 + u) & 63, 64);
        w[u] = __shfl(w_l, (j0 + u) & 63, 64);
        dot[u] = 0.0f;
      }
      for (int c0 = 0; c0 < nch; c0 += 64) {
        const int c = c0 + lane;
        const bool ok = c < nch;
        Chunk<T> dv;
        dv.raw = ok ? ld16(dyb + t * rowbytes + (int64_t)c * 16) : (u32x4){0u, 0u, 0u, 0u};
        if constexpr (MXQ && sizeof(T) == 2) {
          if (a.dq && j0 == 0) mx_row_codes<T>(dv.raw, ok, a.dq + t * a.d + (int64_t)c * 8, a.dqs + t * (a.d / 32) + c / 4, c);
        }
        Chunk<T> yv[KG];
#pragma unroll
        for (int u = 0; u < KG; ++u) {
          const bool use = GD && ok && j0 + u < a.k && r[u] >= 0;
          yv[u].raw = use ? ld16(yperm + (int64_t)r[u] * a.d + (int64_t)c * VR) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < KG; ++u) {
          if (j0 + u < a.k && r[u] >= 0) {                  // wave-uniform
            Chunk<T> o;
#pragma unroll
            for (int i = 0; i < VR; ++i) {
              const float dd = to_f32<T>(dv.e[i]);
              if constexpr (GD) dot[u] = fmaf(dd, to_f32<T>(yv[u].e[i]), dot[u]);
              o.e[i] = a.copy ? dv.e[i] : from_f32<T>(w[u] * dd);
            }
            if (ok && !a.no_rows) st16(dyp + (int64_t)r[u] * rowbytes + (int64_t)c * 16, o.raw);
            if constexpr (MXQ && sizeof(T) == 2) {
              // MX-fp8 experts: the row-wise codes of the stored values; the
              // four lanes of chunks 4b .. 4b+3 hold one 32-value block
              if (a.q)
                mx_row_codes<T>(o.raw, ok, a.q + (int64_t)r[u] * a.d + (int64_t)c * 8,
                                a.qs + (int64_t)r[u] * (a.d / 32) + c / 4, c);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        if (j0 + u < a.k) {
          if constexpr (GD) {
            const float ds = wave_sum(dot[u]);
            if (lane == 0) a.g[t * a.k + j0 + u] = ds;
            if (a.wsorted && lane == 0 && r[u] >= 0) a.wsorted[r[u]] = w[u];
          } else {
            if (lane == 0 && r[u] >= 0) a.wsorted[r[u]] = w[u];
          }
        }
      }
    }
  }
}

// Routing-weight gradient of assignment (t, j) = flat index tj: g[tj], or
// the sum of the expert-sorted row's partials in index order.
__device__ __forceinline__ float slot_g(const float* g, const float* gpart, const int32_t* inv, int gparts,
                                        int64_t tj) {
  if (!gpart) return g[tj];
  const int r = inv[tj];
  if (r < 0) return 0.0f;                         // an empty slot (no expert)
  const float* p = gpart + (int64_t)r * gparts;
  float s = 0.0f;
  if ((gparts & 3) == 0) {
    // 16-byte loads (a row then starts 16-byte aligned), added in the same
    // order; all of a row's loads can be in flight before the first add
#pragma unroll 4
    for (int i = 0; i < gparts; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
      s += v[0];
      s += v[1];
      s += v[2];
      s += v[3];
    }
  } else {
    for (int i = 0; i < gparts; ++i) s += p[i];
  }
  return s;
}

// Balancing-term scale aux_coef * E / (T^2 k) (times count_e gives
// aux_coef * E * f_e / T): over all tokens, or over the real ones (T and the
// counts those of the real tokens; no real token, no term).
__device__ __forceinline__ float aux_grad_scale(float aux_coef, int E, int64_t T, int k, const int32_t* mask,
                                                const int32_t* rcounts) {
  const float Tn = mask ? (float)rcounts[E] : (float)T;
  return Tn > 0.0f ? aux_coef * (float)E / (Tn * Tn * (float)k) : 0.0f;
}

// Router backward for one token per wave.
//   dp_e  = (selected e = e_j) ? (renorm ? (g_j - sum_i w_i g_i) / S : g_j) : 0
//   dp_e += aux_coef * E * f_e / T,   f_e = count_e / (T k)
//           (with a real-token mask: real tokens only, T and counts theirs)
//   dz_e  = p_e * (dp_e - sum_e' p_e' dp_e')
// dz is written as a hi/lo pair in the activation dtype (hi = round(dz),
// lo = round(dz - hi)) so the matrix-core products that consume it keep
// nearly f32 accuracy.  Per-block column sums of dz feed dbias.
template <typename T>
__global__ void __launch_bounds__(NT) router_dz_kernel(RouterDzArgs a) {
  // one wave per token; lane l holds experts l, l+64, l+128, l+192
  __shared__ float s_bias[NT / 64][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float aux_scale = aux_grad_scale(a.aux_coef, a.E, a.T, a.k, a.mask, a.rcounts);
  const int32_t* cnt = a.mask ? a.rcounts : a.counts;
  float dp_aux[4], bias_acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    dp_aux[q] = (e < a.E) ? aux_scale * (float)cnt[e] : 0.0f;
    bias_acc[q] = 0.0f;
  }
  T* dz = static_cast<T*>(a.dz_hl);
  const int64_t ld = 2 * (int64_t)a.Ep;
  const int64_t nwaves = (int64_t)gridDim.x * (NT / 64);
  for (int64_t t = (int64_t)blockIdx.x * (NT / 64) + wave; t < a.T; t += nwaves) {
    float p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      p[q] = (e < a.E) ? a.probs[t * a.E + e] : 0.0f;
    }
    float gj = 0.0f, wj = 0.0f;
    int ej = -1;
    if (lane < a.k) {
      ej = a.idx[t * a.k + lane];
      if ((unsigned)ej >= (unsigned)a.E) ej = -1;
      if (ej >= 0) {                                   // an empty slot carries nothing
        gj = slot_g(a.g, a.gpart, a.inv, a.gparts, t * a.k + lane);
        wj = a.wts[t * a.k + lane];
      }
    }
    // p of this slot's expert, from the lane that holds it
    float pj = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (64 * q < a.E) {
        const float v = __shfl(p[q], ej & 63, 64);
        if (ej >= 0 && (ej >> 6) == q) pj = v;
      }
    }
    const float S = wave_sum(pj);
    const float wg = wave_sum(wj * gj);
    const float dps = a.renorm ? (gj - wg) / S : gj;
    const bool real = !a.mask || a.mask[t] != 0;       // fillers get no balancing term
    float dp[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) dp[q] = real ? dp_aux[q] : 0.0f;
    // scatter the k slot gradients to the lanes that hold their experts
    for (int j = 0; j < a.k; ++j) {
      const int eb = __shfl(ej, j, 64);
      const float db = __shfl(dps, j, 64);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q == eb) dp[q] += db;
    }
    float dot = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) dot = fmaf(p[q], dp[q], dot);
    dot = wave_sum(dot);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      // softmax Jacobian, or (ReLU gates) the gate's derivative 1[gate > 0]
      const float v = (e < a.E) ? (a.relu ? (p[q] > 0.0f ? dp[q] : 0.0f) : p[q] * (dp[q] - dot)) : 0.0f;
      if (e < a.Ep) {
        const T hi = from_f32<T>(v);
        const T lo = from_f32<T>(v - to_f32<T>(hi));
        dz[t * ld + e] = hi;
        dz[t * ld + a.Ep + e] = lo;
      }
      bias_acc[q] += v;
    }
  }
  // per-block column sums of dz, waves combined in index order
#pragma unroll
  for (int q = 0; q < 4; ++q) s_bias[wave][lane + 64 * q] = bias_acc[q];
  __syncthreads();
  if (tid < a.E)
    a.dbias_part[(int64_t)blockIdx.x * a.E + tid] = ((s_bias[0][tid] + s_bias[1][tid]) + s_bias[2][tid]) + s_bias[3][tid];
}

// Router backward for few experts, one block of kRouterSmallTokens tokens per
// workgroup: the dz of router_dz_kernel (one thread per token), then the
// block's partial dW_r[e][c] = sum_t dz[t][e] x[t][c] in f32 (threads over
// 8-column pieces of x, in G token groups whose sums are added in group order
// through LDS) and its partial dbias.  Reading x here replaces the matrix-core
// product dz^T x and its padded [2 Ep, d] f32 partials.
template <typename T, int EM>
__global__ void __launch_bounds__(NT) router_bwd_small_kernel(RouterBwdSmallArgs a) {
  constexpr int TB = kRouterSmallTokens;
  __shared__ float s_dz[TB][EM];
  extern __shared__ float s_red[];                // [E][d] when G > 1
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int E = a.E;
  // ---- dz, one thread per token
  if (tid < TB) {
    const int64_t t = t0 + tid;
    float dzv[EM];
#pragma unroll
    for (int e = 0; e < EM; ++e) dzv[e] = 0.0f;
    if (t < a.T) {
      float p[EM], dp[EM];
      const bool real = !a.mask || a.mask[t] != 0;     // fillers get no balancing term
      const float aux_scale = real ? aux_grad_scale(a.aux_coef, E, a.T, a.k, a.mask, a.rcounts) : 0.0f;
      const int32_t* cnt = a.mask ? a.rcounts : a.counts;
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        p[e] = (e < E) ? a.probs[t * E + e] : 0.0f;
        dp[e] = (e < E) ? aux_scale * (float)cnt[e] : 0.0f;
      }
      // slot gradients; with renormalisation w = p_sel / S
      float S = 0.0f, wg = 0.0f;
      for (int j = 0; j < a.k; ++j) {
        const int ej = a.idx[t * a.k + j];
        if (ej < 0) continue;                          // an empty slot carries nothing
        float pj = 0.0f;
#pragma unroll
        for (int e = 0; e < EM; ++e) pj = (e == ej) ? p[e] : pj;
        S += pj;
        wg = fmaf(a.wts[t * a.k + j], slot_g(a.g, a.gpart, a.inv, a.gparts, t * a.k + j), wg);
      }
      for (int j = 0; j < a.k; ++j) {
        const int ej = a.idx[t * a.k + j];
        if (ej < 0) continue;
        const float gj = slot_g(a.g, a.gpart, a.inv, a.gparts, t * a.k + j);
        const float dps = a.renorm ? (gj - wg) / S : gj;
#pragma unroll
        for (int e = 0; e < EM; ++e) dp[e] += (e == ej) ? dps : 0.0f;
      }
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < EM; ++e) dot = fmaf(p[e], dp[e], dot);
      T* dz = static_cast<T*>(a.dz_hl) + t * 2 * (int64_t)a.Ep;
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        if (e < E) {
          const float v = a.relu ? (p[e] > 0.0f ? dp[e] : 0.0f) : p[e] * (dp[e] - dot);
          dzv[e] = v;
          const T hi = from_f32<T>(v);
          dz[e] = hi;
          dz[a.Ep + e] = from_f32<T>(v - to_f32<T>(hi));
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EM; ++e) s_dz[tid][e] = dzv[e];
  }
  __syncthreads();
  // ---- partial dbias: column sums over the block's tokens, in token order
  if (tid < E) {
    float sacc = 0.0f;
    for (int i = 0; i < TB; ++i) sacc += s_dz[i][tid];
    a.dbias_part[(int64_t)blockIdx.x * E + tid] = sacc;
  }
  // ---- partial dW_r
  const int nch = a.d / 8;                        // 8-column pieces of a row (<= NT)
  const int G = NT / nch;                         // token groups
  const int c = tid % nch, grp = tid / nch;
  float acc[EM][8];
#pragma unroll
  for (int e = 0; e < EM; ++e)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[e][i] = 0.0f;
  if (grp < G) {
    // tokens grp, grp + G, ... in batches of 8 whose loads are all issued
    // before any is used (rows past T read as zero, and their dz is zero)
    constexpr int NB = 8, VPR = 8 * sizeof(T) / 16;       // 16-byte vectors per 8 values
    const T* xb = static_cast<const T*>(a.x) + (int64_t)c * 8;
    for (int i0 = grp; i0 < TB; i0 += NB * G) {
      u32x4 raw[NB][VPR];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = i0 + u * G;
        const bool ok = i < TB && t0 + i < a.T;
#pragma unroll
        for (int v = 0; v < VPR; ++v)
          raw[u][v] = ok ? ld16(xb + (t0 + i) * a.d + v * (16 / sizeof(T))) : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int i = i0 + u * G;
        if (i >= TB) break;
        float xv[8];
        if constexpr (sizeof(T) == 2) {
          unpack8<T>(raw[u][0], xv);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) xv[q] = __uint_as_float(raw[u][q >> 2][q & 3]);
        }
#pragma unroll
        for (int e = 0; e < EM; ++e) {
          const float z = s_dz[i][e];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[e][q] = fmaf(z, xv[q], acc[e][q]);
        }
      }
    }
  }
  // groups added in order: group 0 stores, groups 1.. G-1 add in turn
  for (int gi = 0; gi < G; ++gi) {
    if (G > 1) __syncthreads();
    if (grp == gi) {
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        if (e < E) {
          float* r = s_red + (int64_t)e * a.d + c * 8;
#pragma unroll
          for (int q = 0; q < 8; ++q) r[q] = (gi == 0 ? 0.0f : r[q]) + acc[e][q];
        }
      }
    }
  }
  if (G > 1) __syncthreads();
  float* out = a.dw_part + (int64_t)blockIdx.x * E * a.d;
  if (G > 1) {
    for (int i = tid; i < E * nch; i += NT) {
      const float* r = s_red + (int64_t)i * 8;
      store4<float>(out + (int64_t)i * 8, r[0], r[1], r[2], r[3]);
      store4<float>(out + (int64_t)i * 8 + 4, r[4], r[5], r[6], r[7]);
    }
  } else if (grp == 0) {
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) {
        store4<float>(out + (int64_t)e * a.d + c * 8, acc[e][0], acc[e][1], acc[e][2], acc[e][3]);
        store4<float>(out + (int64_t)e * a.d + c * 8 + 4, acc[e][4], acc[e][5], acc[e][6], acc[e][7]);
      }
  }
}

// w2 rows [0, E) and [Ep, Ep + E) = W_r, every other row zero.
template <typename T>
__global__ void __launch_bounds__(NT) stack2_kernel(Stack2Args a) {
  const int64_t n = 2 * (int64_t)a.Ep * a.d;
  const T* w = static_cast<const T*>(a.w);
  T* w2 = static_cast<T*>(a.w2);
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const int64_t row = i / a.d, col = i - row * a.d;
    const int64_t src = row % a.Ep;
    w2[i] = (src < a.E) ? w[src * a.d + col] : from_f32<T>(0.0f);
  }
}

// Blocks [0, nbw): block b reduces columns 64 VEC (b % (d / (64 VEC))) ..
// + 64 VEC - 1 of row e = b / (d / (64 VEC)), VEC consecutive columns per
// lane: dW_r[e][n] = sum_s part[s][e][n] (+ sum_s part[s][lo_row + e][n]).
// Its 16 waves each sum every 16th split (hi and lo apart), then the wave
// partials are added in index order.  Blocks [nbw, nbw + E): dbias[e] = sum
// over router_dz blocks of their partial.
constexpr int kReduceThreads = 1024;
template <typename T, int VEC>
__global__ void __launch_bounds__(kReduceThreads) router_reduce_kernel(RouterReduceArgs a, int nbw) {
  constexpr int NWV = kReduceThreads / 64;
  __shared__ float sh[2][NWV][64 * VEC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if ((int)blockIdx.x >= nbw) {
    const int e = blockIdx.x - nbw;
    float v = 0.0f;
    for (int b = tid; b < a.nb; b += kReduceThreads) v += a.dbias_part[(int64_t)b * a.E + e];
    v = wave_sum(v);
    if (lane == 0) sh[0][wave][0] = v;
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
      for (int w = 0; w < NWV; ++w) s += sh[0][w][0];
      a.dbias[e] = s;
    }
    return;
  }
  typedef __attribute__((__vector_size__(VEC * sizeof(float)))) float VT;   // VEC floats, one load
  const int groups = a.d / (64 * VEC);
  const int e = blockIdx.x / groups;
  const int col = (blockIdx.x - e * groups) * 64 * VEC + lane * VEC;
  const int64_t sstride = (int64_t)a.rows * a.d;
  const float* ph = a.part + (int64_t)e * a.d + col;
  const float* pl = a.part + (int64_t)(a.lo_row + e) * a.d + col;
  float hi[VEC], lo[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) hi[c] = lo[c] = 0.0f;
  if (a.lo_row >= 0) {
#pragma unroll 4
    for (int s = wave; s < a.splits; s += NWV) {
      const VT h = *reinterpret_cast<const VT*>(ph + s * sstride), l = *reinterpret_cast<const VT*>(pl + s * sstride);
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        hi[c] += h[c];
        lo[c] += l[c];
      }
    }
  } else {
#pragma unroll 4
    for (int s = wave; s < a.splits; s += NWV) {
      const VT h = *reinterpret_cast<const VT*>(ph + s * sstride);
#pragma unroll
      for (int c = 0; c < VEC; ++c) hi[c] += h[c];
    }
  }
#pragma unroll
  for (int c = 0; c < VEC; ++c) {
    sh[0][wave][lane * VEC + c] = hi[c];
    sh[1][wave][lane * VEC + c] = lo[c];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      float h = 0.0f, l = 0.0f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        h += sh[0][w][lane * VEC + c];
        l += sh[1][w][lane * VEC + c];
      }
      static_cast<T*>(a.dw)[(int64_t)e * a.d + col + c] = from_f32<T>(h + l);
    }
  }
}

// out[i] = sum_s part[s][i] over the splits in order; 4 elements per thread.
template <typename T>
__global__ void __launch_bounds__(NT) split_reduce_kernel(SplitReduceArgs a) {
  const int64_t n4 = a.n / 4;
  T* out = static_cast<T*>(a.out);
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * NT) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(a.part + 4 * i);
    for (int s = 1; s < a.splits; ++s) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.part + (int64_t)s * a.n + 4 * i);
      acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
    }
    store4<T>(out + 4 * i, acc[0], acc[1], acc[2], acc[3]);
  }
}

// dx[t] = sum_j dX_perm[inv[t, j]] (+ dx_shared[t]) + router part, where the
// router part is either sum_e dz[t, e] W_r[e] computed here (few experts) or
// the f32 rows of a matrix-core product (dxr).  16-byte vectors along the row,
// fixed summation order.  A wave takes TW tokens per pass (TW = 2 when a row
// is at most 64 vectors and k <= 32): token u's slot indices and router
// gradients sit in lanes 32 u + j, all TW tokens' row gathers issue together
// and the router weight vectors are loaded once for both.
template <typename T, int KG, int TW, typename PT>
__global__ void __launch_bounds__(NT) unpermute_kernel(UnpermuteArgs a) {
  constexpr int VR = 16 / sizeof(T);
  constexpr int PC = VR * (int)sizeof(PT) / 16;           // 16-byte pieces of dX_perm per output chunk
  constexpr int PV = 16 / (int)sizeof(PT);                 // dX_perm values per piece
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (NT / 64);
  const int64_t rowbytes = (int64_t)a.d * sizeof(T);
  const int64_t prowbytes = (int64_t)a.d * sizeof(PT);    // rows of dX_perm and dx_shared
  const int nch = (int)(rowbytes / 16);
  const char* gp = static_cast<const char*>(a.dx_perm);
  const char* sp = static_cast<const char*>(a.dx_shared);
  const T* dz = static_cast<const T*>(a.dz_hl);
  const char* wr = static_cast<const char*>(a.w_router);
  char* out = static_cast<char*>(a.dx);
  const int sub = TW > 1 ? lane >> 5 : 0, sl = TW > 1 ? lane & 31 : lane;   // token of this lane's slot / expert
  for (int64_t tb = ((int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6)) * TW; tb < a.T; tb += waves * TW) {
    int64_t t[TW];
    bool tv[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      t[u] = tb + u;
      tv[u] = t[u] < a.T;                                 // wave-uniform
    }
    const int64_t tm = tb + sub;
    int r_l = -1;
    if (sl < a.k && tm < a.T) r_l = a.inv[tm * a.k + sl];
    // router part inline (few experts): lane 32 u + e holds dz[t_u][e] = hi + lo
    float z_l = 0.0f;
    if (!a.dxr && sl < a.E && tm < a.T)
      z_l = to_f32<T>(dz[tm * 2 * a.Ep + sl]) + to_f32<T>(dz[tm * 2 * a.Ep + a.Ep + sl]);
    for (int c0 = 0; c0 < nch; c0 += 64) {
      const int c = c0 + lane;
      const bool ok = c < nch;
      float acc[TW][VR];
#pragma unroll
      for (int u = 0; u < TW; ++u)
#pragma unroll
        for (int i = 0; i < VR; ++i) acc[u][i] = 0.0f;
      // slots in batches of KG (per token) whose row loads are issued together
      for (int j0 = 0; j0 < a.k; j0 += KG) {
        Chunk<PT> gv[TW][KG][PC];
        int r[TW][KG];
#pragma unroll
        for (int u = 0; u < TW; ++u)
#pragma unroll
          for (int q = 0; q < KG; ++q) {
            r[u][q] = __shfl(r_l, (32 * u + j0 + q) & 63, 64);
            const bool use = ok && tv[u] && j0 + q < a.k && r[u][q] >= 0;
#pragma unroll
            for (int pc = 0; pc < PC; ++pc)
              gv[u][q][pc].raw = use ? ld16(gp + (int64_t)r[u][q] * prowbytes + ((int64_t)c * PC + pc) * 16)
                                     : (u32x4){0u, 0u, 0u, 0u};
          }
#pragma unroll
        for (int u = 0; u < TW; ++u)
#pragma unroll
          for (int q = 0; q < KG; ++q) {
            if (j0 + q < a.k && r[u][q] >= 0) {            // wave-uniform
#pragma unroll
              for (int i = 0; i < VR; ++i) acc[u][i] += to_f32<PT>(gv[u][q][i / PV].e[i % PV]);
            }
          }
      }
      // (every lane stays in the loop: the router part below shuffles)
#pragma unroll
      for (int u = 0; u < TW; ++u) {
        if (sp && ok && tv[u]) {
          Chunk<PT> ch[PC];
#pragma unroll
          for (int pc = 0; pc < PC; ++pc) ch[pc].raw = ld16(sp + t[u] * prowbytes + ((int64_t)c * PC + pc) * 16);
#pragma unroll
          for (int i = 0; i < VR; ++i) acc[u][i] += to_f32<PT>(ch[i / PV].e[i % PV]);
        }
        if (a.dxr && ok && tv[u]) {
          const f32x4* src = reinterpret_cast<const f32x4*>(a.dxr + t[u] * a.d + (int64_t)c * VR);
#pragma unroll
          for (int q = 0; q < VR / 4; ++q) {
            const f32x4 v = src[q];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[u][4 * q + i] += v[i];
          }
        }
      }
      if (!a.dxr) {
        float rz[TW][VR];
#pragma unroll
        for (int u = 0; u < TW; ++u)
#pragma unroll
          for (int i = 0; i < VR; ++i) rz[u][i] = 0.0f;
        // experts in groups of 8 whose weight loads are issued together
        for (int e0 = 0; e0 < a.E; e0 += 8) {
          Chunk<T> w[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (ok && e0 + q < a.E) w[q].raw = ld16(wr + (int64_t)(e0 + q) * rowbytes + (int64_t)c * 16);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
#pragma unroll
            for (int u = 0; u < TW; ++u) {
              const float z = __shfl(z_l, (32 * u + e0 + q) & 63, 64);
              if (e0 + q < a.E) {
#pragma unroll
                for (int i = 0; i < VR; ++i) rz[u][i] = fmaf(z, to_f32<T>(w[q].e[i]), rz[u][i]);
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < TW; ++u)
#pragma unroll
          for (int i = 0; i < VR; ++i) acc[u][i] += rz[u][i];
      }
#pragma unroll
      for (int u = 0; u < TW; ++u) {
        if (ok && tv[u]) {
          Chunk<T> o;
#pragma unroll
          for (int i = 0; i < VR; ++i) o.e[i] = from_f32<T>(acc[u][i]);
          st16(out + t[u] * rowbytes + (int64_t)c * 16, o.raw);
        }
      }
    }
  }
}

// ---- balancing statistic -----------------------------------------------------
// Threads form a (token lane) x (expert) grid: EP2 = E rounded up to a power of
// two experts per row of threads, NT / EP2 token lanes.
constexpr int kAuxTokens = 64;

__device__ __forceinline__ int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

__global__ void __launch_bounds__(NT) aux_partials_kernel(AuxArgs a) {
  __shared__ float sp[NT], se[NT];
  __shared__ int sc[NT], sr[NT];
  const int EP2 = pow2_at_least(a.E);
  const int TL = NT / EP2;
  const int e = threadIdx.x % EP2, tl = threadIdx.x / EP2;
  const int64_t t0 = (int64_t)blockIdx.x * kAuxTokens;
  int64_t t1 = t0 + kAuxTokens;
  if (t1 > a.T) t1 = a.T;
  float ps = 0.0f, ent = 0.0f;
  int cnt = 0, nreal = 0;                            // (real-token mask only)
  if (e < a.E) {
    // four tokens' loads issued together, then added in token order
    for (int64_t tb = t0 + tl; tb < t1; tb += 4 * TL) {
      float p[4];
      bool use[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t t = tb + u * TL;
        use[u] = t < t1 && (!a.mask || a.mask[t] != 0);
        p[u] = use[u] ? a.probs[t * a.E + e] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (use[u]) {
          ps += p[u];
          if (p[u] > 0.0f) ent -= p[u] * logf(p[u]);
          if (a.mask) {
            const int64_t t = tb + u * TL;
            for (int j = 0; j < a.k; ++j) cnt += a.idx[t * a.k + j] == e ? 1 : 0;
            nreal += 1;
          }
        }
      }
    }
  }
  sp[threadIdx.x] = ps;
  se[threadIdx.x] = ent;
  sc[threadIdx.x] = cnt;
  sr[threadIdx.x] = nreal;
  __syncthreads();
  if (tl == 0 && e < a.E) {
    float s1 = 0.0f, s2 = 0.0f;
    int c = 0, r = 0;
    for (int l = 0; l < TL; ++l) {
      s1 += sp[l * EP2 + e];
      s2 += se[l * EP2 + e];
      c += sc[l * EP2 + e];
      r += sr[l * EP2 + e];
    }
    a.part[((int64_t)blockIdx.x * 2 + 0) * a.E + e] = s1;
    a.part[((int64_t)blockIdx.x * 2 + 1) * a.E + e] = s2;
    if (a.mask) {
      a.cpart[(int64_t)blockIdx.x * (a.E + 1) + e] = c;
      if (e == 0) a.cpart[(int64_t)blockIdx.x * (a.E + 1) + a.E] = r;   // real tokens of the block
    }
  }
}

// Sums (fixed order: butterfly within waves, then waves in index order) of K
// values at once; every thread gets the results.
template <int K>
__device__ __forceinline__ void block_sum_d(double (&v)[K], double (*sh)[NT / 64]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < K; ++i)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v[i] += __shfl_xor(v[i], o, 64);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < K; ++i) sh[i][wave] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < K; ++i) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += sh[i][w];
    v[i] = s;
  }
}

__global__ void __launch_bounds__(NT) aux_finalize_kernel(AuxArgs a, int nblk) {
  __shared__ double sh[6][NT / 64];
  __shared__ float cp[NT], ce[NT];
  __shared__ float colp[256], cole[256];
  const int EP2 = pow2_at_least(a.E);
  const int TL = NT / EP2;
  {
    const int e = threadIdx.x % EP2, tl = threadIdx.x / EP2;
    float s1 = 0.0f, s2 = 0.0f;
    if (e < a.E) {
      // blocks tl, tl + TL, ... in that order; eight blocks' loads issued
      // together (a chain of single loads left this one block waiting on
      // memory for most of its time)
      for (int b0 = tl; b0 < nblk; b0 += 8 * TL) {
        float v1[8], v2[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int b = b0 + u * TL;
          v1[u] = b < nblk ? a.part[((int64_t)b * 2 + 0) * a.E + e] : 0.0f;
          v2[u] = b < nblk ? a.part[((int64_t)b * 2 + 1) * a.E + e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (b0 + u * TL < nblk) {
            s1 += v1[u];
            s2 += v2[u];
          }
        }
      }
    }
    cp[threadIdx.x] = s1;
    ce[threadIdx.x] = s2;
    __syncthreads();
    if (tl == 0 && e < a.E) {
      float t1 = 0.0f, t2 = 0.0f;
      for (int l = 0; l < TL; ++l) {
        t1 += cp[l * EP2 + e];
        t2 += ce[l * EP2 + e];
      }
      colp[e] = t1;
      cole[e] = t2;
    }
    __syncthreads();
  }
  // real-token mask: the real tokens' counts and their number, summed over
  // the blocks' integer partials (exact), and written out for the backward
  __shared__ int s_real;
  if (a.mask) {
    const int e = threadIdx.x;
    if (e < a.E) {
      int c = 0;
      for (int b = 0; b < nblk; ++b) c += a.cpart[(int64_t)b * (a.E + 1) + e];
      a.rcounts[e] = c;
    }
    if (threadIdx.x < 64) {
      int r = 0;
      for (int b = threadIdx.x; b < nblk; b += 64) r += a.cpart[(int64_t)b * (a.E + 1) + a.E];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) r += __shfl_xor(r, o, 64);
      if (threadIdx.x == 0) {
        s_real = r;
        a.rcounts[a.E] = r;
      }
    }
    __syncthreads();
  }
  const int e = threadIdx.x;
  const bool valid = e < a.E;
  const float ps = valid ? colp[e] : 0.0f, ent = valid ? cole[e] : 0.0f;
  const double T = a.mask ? (double)s_real : (double)a.T;
  const double cnt = valid ? (double)(a.mask ? a.rcounts[e] : a.counts[e]) : 0.0;
  const double f = (T > 0) ? cnt / (T * (a.kf ? a.kf : a.k)) : 0.0;
  const double P = (T > 0) ? (double)ps / T : 0.0;
  if (valid) {
    a.f[e] = (float)f;
    a.p_mean[e] = (float)P;
  }
  // pass 1: sum f P, entropy, counts, unused; min and max of the counts
  double v1[4] = {valid ? f * P : 0.0, valid ? (double)ent : 0.0, cnt, (valid && cnt == 0.0) ? 1.0 : 0.0};
  double mn = valid ? cnt : 1e300, mx = valid ? cnt : -1.0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, o, 64));
    mx = fmax(mx, __shfl_xor(mx, o, 64));
  }
  __shared__ double smn[NT / 64], smx[NT / 64];
  const int lane = e & 63, wave = e >> 6;
  if (lane == 0) { smn[wave] = mn; smx[wave] = mx; }
  block_sum_d<4>(v1, sh);          // its barriers also publish smn / smx
  const double mean = v1[2] / a.E;
  // pass 2: population variance of the counts about their mean
  double v2[1] = {valid ? (cnt - mean) * (cnt - mean) : 0.0};
  block_sum_d<1>(v2, sh + 4);
  if (e == 0) {
    for (int w = 0; w < NT / 64; ++w) { mn = fmin(mn, smn[w]); mx = fmax(mx, smx[w]); }
    const double var = v2[0] / a.E;
    moe_aux_out* o = static_cast<moe_aux_out*>(a.out);
    o->aux = (float)(a.E * v1[0]);
    o->aux_raw = (float)v1[0];
    o->entropy_mean = (T > 0) ? (float)(v1[1] / T) : 0.0f;
    o->count_cv = mean > 0 ? (float)(sqrt(var) / mean) : 0.0f;
    o->count_min = (int32_t)mn;
    o->count_max = (int32_t)mx;
    o->n_unused = (int32_t)v1[3];
    o->reserved = 0;
  }
}

}  // namespace

// Slots per batch of the gathering kernels: all k when k <= 4, else 8.
inline int slot_batch(int k) { return k <= 2 ? 2 : (k <= 4 ? 4 : 8); }
#define MOE_LAUNCH_SLOT_BATCH(KERN, TY, ...)                                                         \
  do {                                                                                               \
    const int kg = slot_batch(a.k);                                                                  \
    if (kg == 2) hipLaunchKernelGGL((KERN<TY, 2 __VA_OPT__(, ) __VA_ARGS__>), dim3((unsigned)grid), dim3(NT), 0, s, a); \
    else if (kg == 4) hipLaunchKernelGGL((KERN<TY, 4 __VA_OPT__(, ) __VA_ARGS__>), dim3((unsigned)grid), dim3(NT), 0, s, a); \
    else hipLaunchKernelGGL((KERN<TY, 8 __VA_OPT__(, ) __VA_ARGS__>), dim3((unsigned)grid), dim3(NT), 0, s, a); \
  } while (0)

hipError_t launch_combine(int dt, const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  int64_t grid = (a.T + 3) / 4;
  if (grid > 8192) grid = 8192;
  switch (dt) {
    case DT_BF16:
      if (a.y_f32) MOE_LAUNCH_SLOT_BATCH(combine_kernel, __bf16, float);
      else MOE_LAUNCH_SLOT_BATCH(combine_kernel, __bf16, __bf16);
      break;
    case DT_F16:
      if (a.y_f32) MOE_LAUNCH_SLOT_BATCH(combine_kernel, _Float16, float);
      else MOE_LAUNCH_SLOT_BATCH(combine_kernel, _Float16, _Float16);
      break;
    case DT_F32: MOE_LAUNCH_SLOT_BATCH(combine_kernel, float, float); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int dt, const CombineBwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  int64_t grid = (a.T + 3) / 4;
  if (grid > 8192) grid = 8192;
  switch (dt) {
    // g from y_perm (MX-fp8 experts; y_perm in the activation dtype) or the
    // per-row weights (the down dgrad then forms g); the MX row-code writes
    // are a separate instantiation, so the plain kernel carries none of their
    // code.  A bf16 layer with bf16 experts keeps Y_perm in f32: no g here.
    case DT_BF16:
      // (the MX instantiation in batches of at most four slots: within four
      // waves per SIMD's registers; the slots' results do not depend on it)
      if (a.q || a.dq) {
        if (a.k <= 2)
          hipLaunchKernelGGL((combine_bwd_kernel<__bf16, 2, true, true>), dim3((unsigned)grid), dim3(NT), 0, s, a);
        else
          hipLaunchKernelGGL((combine_bwd_kernel<__bf16, 4, true, true>), dim3((unsigned)grid), dim3(NT), 0, s, a);
      }
      else if (a.g) return hipErrorInvalidValue;
      else MOE_LAUNCH_SLOT_BATCH(combine_bwd_kernel, __bf16, false, false);
      break;
    case DT_F16:
      if (a.g) MOE_LAUNCH_SLOT_BATCH(combine_bwd_kernel, _Float16, false, true);
      else MOE_LAUNCH_SLOT_BATCH(combine_bwd_kernel, _Float16, false, false);
      break;
    case DT_F32:
      if (a.g) MOE_LAUNCH_SLOT_BATCH(combine_bwd_kernel, float, false, true);
      else MOE_LAUNCH_SLOT_BATCH(combine_bwd_kernel, float, false, false);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int router_dz_blocks(int64_t T) {
  int64_t g = (T + 3) / 4;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return (int)g;
}

hipError_t launch_router_dz(int dt, const RouterDzArgs& a, hipStream_t s) {
  const int grid = router_dz_blocks(a.T);
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL(router_dz_kernel<__bf16>, dim3(grid), dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL(router_dz_kernel<_Float16>, dim3(grid), dim3(NT), 0, s, a); break;
    case DT_F32: hipLaunchKernelGGL(router_dz_kernel<float>, dim3(grid), dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int router_small_blocks(int64_t T) {
  const int64_t g = (T + kRouterSmallTokens - 1) / kRouterSmallTokens;
  return (int)(g < 1 ? 1 : g);
}

template <typename T>
hipError_t launch_router_bwd_small_t(const RouterBwdSmallArgs& a, hipStream_t s) {
  const int grid = router_small_blocks(a.T);
  const int nch = a.d / 8, G = NT / nch;
  const size_t shm = G > 1 ? (size_t)a.E * a.d * sizeof(float) : 0;
  // (EM = E rounded up: every dW_r product runs EM wide)
  if (a.E <= 4) hipLaunchKernelGGL((router_bwd_small_kernel<T, 4>), dim3(grid), dim3(NT), shm, s, a);
  else if (a.E <= 8) hipLaunchKernelGGL((router_bwd_small_kernel<T, 8>), dim3(grid), dim3(NT), shm, s, a);
  else hipLaunchKernelGGL((router_bwd_small_kernel<T, 16>), dim3(grid), dim3(NT), shm, s, a);
  return hipGetLastError();
}

hipError_t launch_router_bwd_small(int dt, const RouterBwdSmallArgs& a, hipStream_t s) {
  if (a.E < 1 || a.E > kRouterSmallMaxE || a.d % 8 || a.d > kRouterSmallMaxD || a.T <= 0) return hipErrorInvalidValue;
  switch (dt) {
    case DT_BF16: return launch_router_bwd_small_t<__bf16>(a, s);
    case DT_F16: return launch_router_bwd_small_t<_Float16>(a, s);
    case DT_F32: return launch_router_bwd_small_t<float>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stack2(int dt, const Stack2Args& a, hipStream_t s) {
  const int64_t n = 2 * (int64_t)a.Ep * a.d;
  int64_t grid = (n + NT - 1) / NT;
  if (grid > 2048) grid = 2048;
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL(stack2_kernel<__bf16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL(stack2_kernel<_Float16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F32: hipLaunchKernelGGL(stack2_kernel<float>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_router_reduce(int dt, const RouterReduceArgs& a, hipStream_t s) {
  if (a.d % 64) return hipErrorInvalidValue;
  // the widest loads (4 or 2 columns per lane) that still give every CU a
  // block; with few rows, blocks of 64 single columns (many splits then
  // spread over more blocks)
  int vec = 1;
  for (int v = 4; v > 1; v /= 2)
    if (a.d % (64 * v) == 0 && (int64_t)a.E * (a.d / (64 * v)) >= 256) { vec = v; break; }
  const int64_t nbw = (int64_t)a.E * (a.d / (64 * vec));
  const int64_t grid = nbw + (a.dbias ? a.E : 0);
  if (grid == 0) return hipSuccess;
#define MOE_LAUNCH_RR(TY)                                                                                        \
  do {                                                                                                           \
    if (vec == 4) hipLaunchKernelGGL((router_reduce_kernel<TY, 4>), dim3((unsigned)grid), dim3(kReduceThreads), 0, s, a, (int)nbw); \
    else if (vec == 2) hipLaunchKernelGGL((router_reduce_kernel<TY, 2>), dim3((unsigned)grid), dim3(kReduceThreads), 0, s, a, (int)nbw); \
    else hipLaunchKernelGGL((router_reduce_kernel<TY, 1>), dim3((unsigned)grid), dim3(kReduceThreads), 0, s, a, (int)nbw); \
  } while (0)
  switch (dt) {
    case DT_BF16: MOE_LAUNCH_RR(__bf16); break;
    case DT_F16: MOE_LAUNCH_RR(_Float16); break;
    case DT_F32: MOE_LAUNCH_RR(float); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_LAUNCH_RR
  return hipGetLastError();
}

hipError_t launch_split_reduce(int dt, const SplitReduceArgs& a, hipStream_t s) {
  if (a.n % 4) return hipErrorInvalidValue;
  const int64_t n4 = a.n / 4;
  if (n4 == 0) return hipSuccess;
  int64_t grid = (n4 + NT - 1) / NT;
  if (grid > 8192) grid = 8192;
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL(split_reduce_kernel<__bf16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL(split_reduce_kernel<_Float16>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F32: hipLaunchKernelGGL(split_reduce_kernel<float>, dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int TW>
hipError_t launch_unpermute_tw(int dt, const UnpermuteArgs& a, hipStream_t s) {
  int64_t grid = (a.T + 4 * TW - 1) / (4 * TW);
  if (grid > 8192) grid = 8192;
  switch (dt) {
    case DT_BF16:
      if (a.src_f32) MOE_LAUNCH_SLOT_BATCH(unpermute_kernel, __bf16, TW, float);
      else MOE_LAUNCH_SLOT_BATCH(unpermute_kernel, __bf16, TW, __bf16);
      break;
    case DT_F16: MOE_LAUNCH_SLOT_BATCH(unpermute_kernel, _Float16, TW, _Float16); break;
    case DT_F32: MOE_LAUNCH_SLOT_BATCH(unpermute_kernel, float, TW, float); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_unpermute(int dt, const UnpermuteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  // two tokens per wave pass when a row is one pass of the wave and the slot
  // indices / router gradients of a token fit in half a wave
  const bool pair = (int64_t)a.d * dtype_bytes(dt) <= 64 * 16 && a.k <= 32 && (a.dxr || a.E <= 32);
  return pair ? launch_unpermute_tw<2>(dt, a, s) : launch_unpermute_tw<1>(dt, a, s);
}

int aux_blocks(int64_t T) { return (int)((T + kAuxTokens - 1) / kAuxTokens); }

hipError_t launch_aux(const AuxArgs& a, hipStream_t s) {
  const int nblk = aux_blocks(a.T);
  if (nblk > 0) {
    hipLaunchKernelGGL(aux_partials_kernel, dim3(nblk), dim3(NT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(aux_finalize_kernel, dim3(1), dim3(NT), 0, s, a, nblk);
  return hipGetLastError();
}

}  // namespace moe
