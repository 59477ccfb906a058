// Grouped GEMMs of the MoE layer on gfx950 matrix cores (MFMA 32x32x16 for
// bf16/f16, 32x32x2 for f32), LDS-staged 128x128 tiles, four waves per
// workgroup, each wave a 64x64 quadrant (2x2 MFMA tiles).
//
// Two kernel families:
//   row_gemm    -- output rows are token rows.  Rows come in segments (one per
//                  expert, read from the device offsets array, so the host
//                  never learns the per-expert sizes) or as one dense segment.
//                  Used for gate/up (+SwiGLU epilogue), down, the two dgrad
//                  GEMMs (+SwiGLU backward / unpermute epilogues) and the
//                  router's input gradient.
//   wgrad_gemm  -- the contraction runs over a segment's tokens (weight
//                  gradients); both operands are read token-major and
//                  transposed while being staged into LDS.
//
// Every workgroup works out its own tile from the offsets array (a prefix sum
// over at most 256 segments), so no schedule buffer and no host sync is
// needed.  Workgroup ids are remapped so that each of the 8 XCDs (which own
// separate L2 caches; hardware hands out ids round-robin over them) receives a
// contiguous run of tiles: neighbouring n-tiles of one m-tile share the token
// rows, neighbouring m-tiles of one expert share its weights.
//
// MFMA operand roles: the weight-side tile feeds the MFMA "A" operand and the
// token-side tile the "B" operand, so each lane ends up holding 4 consecutive
// output columns of one token row -- an 8-byte (16-bit types) or 16-byte
// (f32) store.

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128;          // token rows (row_gemm) / output rows (wgrad) per tile
constexpr int BN = 128;          // output columns per tile
constexpr int KB = 128;          // bytes of k staged per LDS chunk
constexpr int LROW = KB + 16;    // LDS row stride: 16 bytes of padding keeps ds_read_b128 conflict-free
constexpr int NT = 256;          // threads per workgroup

// Maps the hardware workgroup id onto a logical tile index in [0, R) so that
// XCD x (= id % 8) gets logical tiles [x*Q, (x+1)*Q).  Returns -1 for ids
// beyond the work.
__device__ __forceinline__ int xcd_logical(int hw, int R) {
  const int q = (R + 7) >> 3;
  const int y = hw >> 3;
  if (y >= q) return -1;
  const int l = (hw & 7) * q + y;
  return l < R ? l : -1;
}

// Stage 4 rows x 16 bytes of a token-major source into LDS rows of k:
// chunk i holds source row k = 4*kg + i, columns cg*VR .. cg*VR+VR-1; element
// v of every chunk goes to LDS row cg*VR + v at k offset 4*kg.
template <typename T>
__device__ __forceinline__ void store_transposed(char* lds, const u32x4* c, int kg, int cg) {
  constexpr int ES = sizeof(T);
  constexpr int VR = 16 / ES;
  if constexpr (ES == 2) {
#pragma unroll
    for (int v = 0; v < VR; ++v) {
      const int w = v >> 1, sh = (v & 1) * 16;
      uint32_t e0 = (c[0][w] >> sh) & 0xffffu, e1 = (c[1][w] >> sh) & 0xffffu;
      uint32_t e2 = (c[2][w] >> sh) & 0xffffu, e3 = (c[3][w] >> sh) & 0xffffu;
      u32x2 o = {e0 | (e1 << 16), e2 | (e3 << 16)};
      st8(lds + (cg * VR + v) * LROW + (4 * kg) * ES, o);
    }
  } else {
#pragma unroll
    for (int v = 0; v < VR; ++v) {
      u32x4 o = {c[0][v], c[1][v], c[2][v], c[3][v]};
      st16(lds + (cg * VR + v) * LROW + (4 * kg) * ES, o);
    }
  }
}

__device__ __forceinline__ void store_normal(char* lds, const u32x4* r, int tid) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = tid + NT * s;
    st16(lds + (c >> 3) * LROW + (c & 7) * 16, r[s]);
  }
}

// One LDS chunk of MFMA work: KB bytes of k for the wave's 2x2 tiles.
// qrow[ns] / prow[ms] are the LDS rows (lane 0's) of the wave's operand tiles.
template <typename T>
__device__ __forceinline__ void mfma_chunk(f32x16 (&acc)[2][2], const char* lq, const char* lp,
                                           const int (&qrow)[2], const int (&prow)[2], int lane) {
  constexpr int ES = sizeof(T);
  constexpr int KSTEPS = KB / ES / 16;
  constexpr int CH = Mma32<T>::kChunks;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int kb = ks * 16 * ES + (lane >> 5) * 8 * ES;
    u32x4 fa[2][CH], fb[2][CH];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
      const char* base = lq + (qrow[ns] + (lane & 31)) * LROW + kb;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) fa[ns][ch] = ld16(base + ch * 16);
    }
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const char* base = lp + (prow[ms] + (lane & 31)) * LROW + kb;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) fb[ms][ch] = ld16(base + ch * 16);
    }
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) Mma32<T>::run(acc[ns][ms], fa[ns], fb[ms]);
  }
}

// ------------------------------------------------------------ row GEMM ----
template <typename T, int OP, int EPI>
__global__ void __launch_bounds__(NT) row_gemm(RowGemmArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int BK = KB / ES;
  constexpr int VR = 16 / ES;
  constexpr int NCG = BN / VR;
  constexpr bool QT = (OP == OP_DOWN_DGRAD || OP == OP_GU_DGRAD || OP == OP_ROUTER_DX);
  constexpr int TILE_N = (OP == OP_GU_FWD) ? BN / 2 : BN;   // output (H) columns per tile

  __shared__ __attribute__((aligned(16))) char lp[BM * LROW];
  __shared__ __attribute__((aligned(16))) char lq[BN * LROW];
  __shared__ int s_scan[NT / 64];
  __shared__ int s_loc[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_ntiles = a.N / TILE_N;

  // ---- which (segment, m-tile, n-tile) this workgroup computes
  int my_nt = 0;
  if (tid < a.G) {
    const int64_t len = a.offsets ? (int64_t)(a.offsets[tid + 1] - a.offsets[tid]) : a.M;
    my_nt = (int)((len + BM - 1) / BM);
  }
  int incl = my_nt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_scan[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int sw = s_scan[w];
    before += (w < wave) ? sw : 0;
    total += sw;
  }
  const int start = before + incl - my_nt;
  const int logical = xcd_logical(blockIdx.x, total * n_ntiles);
  if (logical < 0) return;                       // uniform across the workgroup
  const int mt = logical / n_ntiles, ntile = logical - mt * n_ntiles;
  if (tid < a.G && mt >= start && mt < start + my_nt) { s_loc[0] = tid; s_loc[1] = mt - start; }
  __syncthreads();
  const int g = s_loc[0];
  const int64_t seg0 = a.offsets ? a.offsets[g] : 0;
  const int64_t seg1 = a.offsets ? a.offsets[g + 1] : a.M;
  const int64_t row0 = seg0 + (int64_t)s_loc[1] * BM;
  const int rows = (int)((seg1 - row0) < BM ? (seg1 - row0) : BM);
  const int n0 = ntile * TILE_N;

  const char* Pb = static_cast<const char*>(a.P);
  const char* Qb = static_cast<const char*>(a.Q) + (int64_t)g * a.q_group_stride * ES;

  // ---- global -> register loaders for one K chunk starting at element kc
  auto load_p = [&](int kc, u32x4* r) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = tid + NT * s, rr = c >> 3, cc = c & 7;
      if (rr < rows) r[s] = ld16(Pb + ((row0 + rr) * a.ldp + kc) * ES + cc * 16);
      else r[s] = (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto load_q = [&](int kc, u32x4* r) {
    if constexpr (!QT) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = tid + NT * s, q = c >> 3, cc = c & 7;
        int64_t off;
        if constexpr (OP == OP_GU_FWD) {
          // tile = 64 gate rows then the 64 matching up rows of one expert block
          const int blk = n0 / a.sub, r0 = n0 - blk * a.sub;
          const int wrow = blk * 2 * a.sub + (q < 64 ? r0 + q : a.sub + r0 + (q - 64));
          off = (int64_t)wrow * a.ldq + kc;
        } else {
          // OP_DOWN_FWD: Q[n][c] = W[c / sub][n][c % sub]
          const int blk = kc / a.sub, kk = kc - blk * a.sub;
          off = ((int64_t)blk * a.N + (n0 + q)) * a.sub + kk;
        }
        r[s] = ld16(Qb + off * ES + cc * 16);
      }
    } else {
      const int kg = tid / NCG, cg = tid % NCG;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kc + 4 * kg + i;
        int64_t off;
        if constexpr (OP == OP_DOWN_DGRAD) {
          // Q[c][k] = W[c / sub][k][c % sub]; a tile never straddles two blocks
          const int blk = n0 / a.sub, c0 = n0 - blk * a.sub;
          off = ((int64_t)blk * a.K + k) * a.sub + c0 + cg * VR;
        } else {
          off = (int64_t)k * a.ldq + n0 + cg * VR;
        }
        r[i] = ld16(Qb + off * ES);
      }
    }
  };
  auto stage = [&](const u32x4* rp, const u32x4* rq) {
    store_normal(lp, rp, tid);
    if constexpr (!QT) store_normal(lq, rq, tid);
    else store_transposed<T>(lq, rq, tid / NCG, tid % NCG);
  };

  const int wm = wave & 1, wn = wave >> 1;
  const int qrow[2] = {(OP == OP_GU_FWD) ? wn * 32 : wn * 64, (OP == OP_GU_FWD) ? 64 + wn * 32 : wn * 64 + 32};
  const int prow[2] = {wm * 64, wm * 64 + 32};
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = a.K / BK;
  u32x4 rp[4], rq[4];
  load_p(0, rp);
  load_q(0, rq);
  stage(rp, rq);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const bool more = kc + 1 < nk;
    if (more) {
      load_p((kc + 1) * BK, rp);
      load_q((kc + 1) * BK, rq);
    }
    mfma_chunk<T>(acc, lq, lp, qrow, prow, lane);
    __syncthreads();
    if (more) stage(rp, rq);
    __syncthreads();
  }

  // ---- epilogue: lane holds columns qrow[ns] + 8*rq + 4*(lane/32) + 0..3 of row prow[ms] + lane%32
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int ml = prow[ms] + (lane & 31);
    if (ml >= rows) continue;
    const int64_t row = row0 + ml;
#pragma unroll
    for (int rq4 = 0; rq4 < 4; ++rq4) {
      const int nl = 8 * rq4 + 4 * (lane >> 5);
      if constexpr (EPI == EPI_SWIGLU_FWD) {
        const int hc = n0 + wn * 32 + nl;
        const int blk = hc / a.sub;
        const int gcol = blk * 2 * a.sub + (hc - blk * a.sub);
        float gv[4], uv[4], hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[i] = acc[0][ms][4 * rq4 + i];
          uv[i] = acc[1][ms][4 * rq4 + i];
          hv[i] = silu_f(gv[i]) * uv[i];
        }
        T* gu = static_cast<T*>(a.C) + row * a.ldc;
        store4<T>(gu + gcol, gv[0], gv[1], gv[2], gv[3]);
        store4<T>(gu + gcol + a.sub, uv[0], uv[1], uv[2], uv[3]);
        store4<T>(static_cast<T*>(a.C2) + row * a.ldc2 + hc, hv[0], hv[1], hv[2], hv[3]);
      } else {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
          const int n = n0 + qrow[ns] + nl;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[ns][ms][4 * rq4 + i];
          if constexpr (EPI == EPI_STORE) {
            store4<T>(static_cast<T*>(a.C) + row * a.ldc + n, v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_STORE_F32) {
            store4<float>(static_cast<float*>(a.C) + row * a.ldc + n, v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            // v = dH for H column n; G, U saved in the packed [G | U] layout
            const int blk = n / a.sub;
            const int gcol = blk * 2 * a.sub + (n - blk * a.sub);
            const T* gu = static_cast<const T*>(a.aux) + row * a.ldaux;
            float G[4], U[4], dG[4], dU[4];
            load4<T>(gu + gcol, G);
            load4<T>(gu + gcol + a.sub, U);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sg = sigmoid_f(G[i]);
              dG[i] = v[i] * U[i] * sg * (1.0f + G[i] * (1.0f - sg));
              dU[i] = v[i] * G[i] * sg;
            }
            T* dgu = static_cast<T*>(a.C) + row * a.ldc;
            store4<T>(dgu + gcol, dG[0], dG[1], dG[2], dG[3]);
            store4<T>(dgu + gcol + a.sub, dU[0], dU[1], dU[2], dU[3]);
          } else if constexpr (EPI == EPI_UNPERMUTE) {
            // dx[t] = this product + sum_j dX_perm[inv[t, j]] (+ f32 addend)
            for (int j = 0; j < a.topk; ++j) {
              const int64_t r = a.inv[row * a.topk + j];
              if (r < 0) continue;                 // only for an out-of-range routing index
              float t4[4];
              load4<T>(static_cast<const T*>(a.gath) + r * a.ldg + n, t4);
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] += t4[i];
            }
            if (a.aux) {
              float t4[4];
              load4<float>(static_cast<const float*>(a.aux) + row * a.ldaux + n, t4);
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] += t4[i];
            }
            store4<T>(static_cast<T*>(a.C) + row * a.ldc + n, v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------- wgrad GEMM ----
template <typename T, int OUT_F32>
__global__ void __launch_bounds__(NT) wgrad_gemm(WgradArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int BK = KB / ES;
  constexpr int VR = 16 / ES;
  constexpr int NCG = BN / VR;

  __shared__ __attribute__((aligned(16))) char lp[BM * LROW];
  __shared__ __attribute__((aligned(16))) char lq[BN * LROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_mt = a.M / BM, n_nt = a.N / BN;
  const int logical = xcd_logical(blockIdx.x, a.G * a.splits * n_mt * n_nt);
  if (logical < 0) return;
  int rest = logical;
  const int nt = rest % n_nt; rest /= n_nt;
  const int mt = rest % n_mt; rest /= n_mt;
  const int sp = rest % a.splits;
  const int g = rest / a.splits;

  const int64_t s0 = a.offsets ? a.offsets[g] : 0;
  const int64_t s1 = a.offsets ? a.offsets[g + 1] : a.Mtok;
  const int64_t nchunk = (s1 - s0 + BK - 1) / BK;
  const int64_t per = (nchunk + a.splits - 1) / a.splits;
  const int64_t kbeg = s0 + sp * per * BK;
  int64_t kend = kbeg + per * BK;
  if (kend > s1) kend = s1;
  const int nk = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;
  const int m0 = mt * BM, n0 = nt * BN;

  const char* Pb = static_cast<const char*>(a.P);
  const char* Qb = static_cast<const char*>(a.Q);
  const int kg = tid / NCG, cg = tid % NCG;
  auto load = [&](int64_t kc, u32x4* rp, u32x4* rq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = kc + 4 * kg + i;
      if (t < kend) {
        rp[i] = ld16(Pb + (t * a.ldp + m0 + cg * VR) * ES);
        rq[i] = ld16(Qb + (t * a.ldq + n0 + cg * VR) * ES);
      } else {
        rp[i] = (u32x4){0u, 0u, 0u, 0u};
        rq[i] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };

  const int wm = wave & 1, wn = wave >> 1;
  const int qrow[2] = {wn * 64, wn * 64 + 32};
  const int prow[2] = {wm * 64, wm * 64 + 32};
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nk > 0) {
    u32x4 rp[4], rq[4];
    load(kbeg, rp, rq);
    store_transposed<T>(lp, rp, kg, cg);
    store_transposed<T>(lq, rq, kg, cg);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
      const bool more = kc + 1 < nk;
      if (more) load(kbeg + (int64_t)(kc + 1) * BK, rp, rq);
      mfma_chunk<T>(acc, lq, lp, qrow, prow, lane);
      __syncthreads();
      if (more) {
        store_transposed<T>(lp, rp, kg, cg);
        store_transposed<T>(lq, rq, kg, cg);
      }
      __syncthreads();
    }
  }

  // out[m][n] at C + g*cgs + sp*css + (n/sub)*(M*sub) + m*sub + n%sub
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int64_t m = m0 + prow[ms] + (lane & 31);
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
#pragma unroll
      for (int rq4 = 0; rq4 < 4; ++rq4) {
        const int n = n0 + qrow[ns] + 8 * rq4 + 4 * (lane >> 5);
        const int blk = n / a.sub;
        const int64_t off = (int64_t)g * a.c_group_stride + (int64_t)sp * a.c_split_stride +
                            ((int64_t)blk * a.M + m) * a.sub + (n - blk * a.sub);
        const float v0 = acc[ns][ms][4 * rq4 + 0], v1 = acc[ns][ms][4 * rq4 + 1];
        const float v2 = acc[ns][ms][4 * rq4 + 2], v3 = acc[ns][ms][4 * rq4 + 3];
        if constexpr (OUT_F32) store4<float>(static_cast<float*>(a.C) + off, v0, v1, v2, v3);
        else store4<T>(static_cast<T*>(a.C) + off, v0, v1, v2, v3);
      }
    }
  }
}

template <typename T, int OP, int EPI>
hipError_t launch_row_t(const RowGemmArgs& a, hipStream_t s) {
  const int tile_n = (OP == OP_GU_FWD) ? BN / 2 : BN;
  const int64_t n_ntiles = a.N / tile_n;
  int64_t mtiles;
  if (a.offsets) mtiles = (a.M + (int64_t)a.G * (BM - 1)) / BM;   // >= sum_g ceil(len_g / BM)
  else mtiles = (a.M + BM - 1) / BM;
  int64_t grid = mtiles * n_ntiles;
  grid = (grid + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((row_gemm<T, OP, EPI>), dim3((unsigned)grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_row_dt(int op, int epi, const RowGemmArgs& a, hipStream_t s) {
  switch (op) {
    case OP_GU_FWD: return launch_row_t<T, OP_GU_FWD, EPI_SWIGLU_FWD>(a, s);
    case OP_DOWN_FWD:
      if (epi == EPI_STORE_F32) return launch_row_t<T, OP_DOWN_FWD, EPI_STORE_F32>(a, s);
      return launch_row_t<T, OP_DOWN_FWD, EPI_STORE>(a, s);
    case OP_DOWN_DGRAD: return launch_row_t<T, OP_DOWN_DGRAD, EPI_SWIGLU_BWD>(a, s);
    case OP_GU_DGRAD:
      if (epi == EPI_UNPERMUTE) return launch_row_t<T, OP_GU_DGRAD, EPI_UNPERMUTE>(a, s);
      return launch_row_t<T, OP_GU_DGRAD, EPI_STORE>(a, s);
    case OP_ROUTER_DX:
      if (epi == EPI_UNPERMUTE) return launch_row_t<T, OP_ROUTER_DX, EPI_UNPERMUTE>(a, s);
      return launch_row_t<T, OP_ROUTER_DX, EPI_STORE_F32>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_wgrad_dt(const WgradArgs& a, hipStream_t s) {
  int64_t grid = (int64_t)a.G * a.splits * (a.M / BM) * (a.N / BN);
  grid = (grid + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (a.out_f32) hipLaunchKernelGGL((wgrad_gemm<T, 1>), dim3((unsigned)grid), dim3(NT), 0, s, a);
  else hipLaunchKernelGGL((wgrad_gemm<T, 0>), dim3((unsigned)grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_row_gemm(int dt, int op, int epi, const RowGemmArgs& a, hipStream_t s) {
  switch (dt) {
    case DT_BF16: return launch_row_dt<__bf16>(op, epi, a, s);
    case DT_F16: return launch_row_dt<_Float16>(op, epi, a, s);
    case DT_F32: return launch_row_dt<float>(op, epi, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_wgrad(int dt, const WgradArgs& a, hipStream_t s) {
  switch (dt) {
    case DT_BF16: return launch_wgrad_dt<__bf16>(a, s);
    case DT_F16: return launch_wgrad_dt<_Float16>(a, s);
    case DT_F32: return launch_wgrad_dt<float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
