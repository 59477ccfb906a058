// Expert histogram, prefix scan and the stable token permutation.
//
// The assignments (t, j) are ordered by (expert ascending, token ascending),
// deterministically and without atomics on global memory:
//   1. permute_hist: each block of kHistTokens tokens builds, in LDS, one bit per
//      token for every expert (bit set <=> the token chose that expert).  The
//      popcount of the bits below a token is the token's rank among the
//      block's tokens of that expert; the full popcount is the block's count.
//      Ranks go to inv_perm (scratch until step 3), counts to the workspace.
//   2. permute_scan: one workgroup turns the [blocks x E] counts into
//      counts[E], offsets[E+1] and the first output row of every
//      (block, expert) pair (expert totals first, so every block's row is
//      written once; several threads per expert share its blocks).
//   3. permute_scatter: a wave takes one token (or two, for rows of at most
//      1 KB) per pass, computes its k destination rows, writes inv_perm /
//      perm_token, reads the token's row of x once and writes it k times
//      (every access a full 16-byte vector, rows contiguous).

#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Scratch of moe_permute_noalloc: the [blocks x E] counts and first rows that
// moe_permute keeps in the caller's workspace, in a fixed device array (each
// GPU the library runs on holds its own copy until the process ends).  Host
// code reaches it only through the address hipGetSymbolAddress returns for
// the current device (permute_scratch below), never through its name.
static __device__ __align__(256) uint8_t scratch[kPermuteScratchBytes];

constexpr int NT = 256;
constexpr int WORDS = kHistTokens / 32;   // 32-bit mask words per expert per block

__global__ void __launch_bounds__(NT) permute_hist(PermuteArgs a) {
  extern __shared__ uint32_t sm[];
  uint32_t* mask = sm;                     // [E][WORDS]
  uint32_t* pre = sm + a.E * WORDS;        // [E][WORDS] popcount of the words before
  const int tid = threadIdx.x;
  const int64_t tb = (int64_t)blockIdx.x * kHistTokens;
  for (int i = tid; i < a.E * WORDS; i += NT) mask[i] = 0u;
  __syncthreads();
  for (int s = 0; s < kHistTokens / NT; ++s) {
    const int tl = tid + NT * s;
    const int64_t t = tb + tl;
    if (t < a.T) {
      for (int j = 0; j < a.k; ++j) {
        const int e = a.idx[t * a.k + j];
        if ((unsigned)e < (unsigned)a.E) atomicOr(&mask[e * WORDS + (tl >> 5)], 1u << (tl & 31));
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += NT) {
    uint32_t run = 0;
    for (int w = 0; w < WORDS; ++w) {
      pre[e * WORDS + w] = run;
      run += __popc(mask[e * WORDS + w]);
    }
    a.block_counts[(int64_t)blockIdx.x * a.E + e] = (int32_t)run;
  }
  __syncthreads();
  for (int s = 0; s < kHistTokens / NT; ++s) {
    const int tl = tid + NT * s;
    const int64_t t = tb + tl;
    if (t < a.T) {
      for (int j = 0; j < a.k; ++j) {
        const int e = a.idx[t * a.k + j];
        int rank = 0;
        if ((unsigned)e < (unsigned)a.E) {
          const int w = tl >> 5, b = tl & 31;
          rank = (int)(pre[e * WORDS + w] + __popc(mask[e * WORDS + w] & ((1u << b) - 1u)));
        }
        a.inv[t * a.k + j] = rank;
      }
    }
  }
}

__global__ void __launch_bounds__(NT) permute_scan(PermuteArgs a, int nblk) {
  // P threads per expert (P a power of two, P E <= NT, so one expert's
  // threads share a wave): thread p of expert e owns a contiguous range of
  // blocks.  Range sums, a scan over the P threads, an exclusive scan over
  // the experts, then every thread writes its blocks' first output rows.
  __shared__ int32_t s_tot[NT], s_w[NT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int P = 1;
  while (2 * P * a.E <= NT && 2 * P <= 64) P *= 2;
  const int e = tid / P, p = tid - e * P;
  const bool ve = e < a.E;
  const int per = (nblk + P - 1) / P;
  const int b0 = p * per < nblk ? p * per : nblk;
  const int b1 = b0 + per < nblk ? b0 + per : nblk;
  int part = 0;
  if (ve) {
#pragma unroll 4
    for (int b = b0; b < b1; ++b) part += a.block_counts[(int64_t)b * a.E + e];
  }
  int incl = part;                                  // inclusive over the expert's threads
  for (int o = 1; o < P; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (p >= o) incl += t;
  }
  if (ve && p == P - 1) s_tot[e] = incl;
  __syncthreads();
  // exclusive scan of the expert totals: thread x < E owns expert x
  const int cnt = tid < a.E ? s_tot[tid] : 0;
  int ex = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(ex, o, 64);
    if (lane >= o) ex += t;
  }
  if (lane == 63) s_w[wave] = ex;
  __syncthreads();
  for (int w = 0; w < wave; ++w) ex += s_w[w];
  if (tid < a.E) {
    a.counts[tid] = cnt;
    a.offsets[tid] = ex - cnt;
    if (tid == a.E - 1) a.offsets[a.E] = ex;
  }
  __syncthreads();                                  // s_tot reused: expert offsets
  if (tid < a.E) s_tot[tid] = ex - cnt;
  __syncthreads();
  if (ve) {
    int run = s_tot[e] + incl - part;
#pragma unroll 4
    for (int b = b0; b < b1; ++b) {
      const int c = a.block_counts[(int64_t)b * a.E + e];
      a.block_base[(int64_t)b * a.E + e] = run;
      run += c;
    }
  }
}

// TW tokens per wave pass (TW = 2 when a row is at most 64 vectors and
// k <= 32): token u's slots sit in lanes 32 u + j, and all TW rows are loaded
// before any is stored.
template <typename T, int TW>
__global__ void __launch_bounds__(NT) permute_scatter(PermuteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (NT / 64);
  const int64_t rowbytes = (int64_t)a.d * sizeof(T);
  const int nch = (int)(rowbytes / 16);
  const char* xb = static_cast<const char*>(a.x);
  char* xp = static_cast<char*>(a.x_perm);
  const int sub = TW > 1 ? lane >> 5 : 0, sl = TW > 1 ? lane & 31 : lane;
  for (int64_t tb = ((int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6)) * TW; tb < a.T; tb += waves * TW) {
    const int64_t tm = tb + sub;
    int r_mine = -1;
    if (sl < a.k && tm < a.T) {
      const int e = a.idx[tm * a.k + sl];
      if ((unsigned)e < (unsigned)a.E) {
        const int rank = a.inv[tm * a.k + sl];
        r_mine = a.block_base[(tm / kHistTokens) * a.E + e] + rank;
        a.perm_token[r_mine] = (int32_t)tm;
      }
      a.inv[tm * a.k + sl] = r_mine;
    }
    if (!xp) continue;                                    // indices only (no row gather)
    // every lane runs the same number of iterations so the shuffles stay convergent
    for (int c0 = 0; c0 < nch; c0 += 64) {
      const int c = c0 + lane;
      const bool ok = c < nch;
      u32x4 v[TW];
#pragma unroll
      for (int u = 0; u < TW; ++u)
        v[u] = ok && tb + u < a.T ? ld16(xb + (tb + u) * rowbytes + (int64_t)c * 16) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < TW; ++u)
        for (int j = 0; j < a.k; ++j) {
          const int r = __shfl(r_mine, (32 * u + j) & 63, 64);
          if (ok && r >= 0) st16(xp + (int64_t)r * rowbytes + (int64_t)c * 16, v[u]);
        }
    }
  }
}

}  // namespace

hipError_t launch_permute_hist(const PermuteArgs& a, hipStream_t s) {
  const int64_t nblk = (a.T + kHistTokens - 1) / kHistTokens;
  if (nblk == 0) return hipSuccess;
  const size_t shm = (size_t)a.E * WORDS * 2 * sizeof(uint32_t);
  hipLaunchKernelGGL(permute_hist, dim3((unsigned)nblk), dim3(NT), shm, s, a);
  return hipGetLastError();
}

hipError_t launch_permute_scan(const PermuteArgs& a, hipStream_t s) {
  const int nblk = (int)((a.T + kHistTokens - 1) / kHistTokens);
  hipLaunchKernelGGL(permute_scan, dim3(1), dim3(NT), 0, s, a, nblk);
  return hipGetLastError();
}

template <int TW>
hipError_t launch_permute_scatter_tw(int dt, const PermuteArgs& a, hipStream_t s) {
  int64_t grid = (a.T + 4 * TW - 1) / (4 * TW);
  if (grid > 4096) grid = 4096;
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL((permute_scatter<__bf16, TW>), dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F16: hipLaunchKernelGGL((permute_scatter<_Float16, TW>), dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    case DT_F32: hipLaunchKernelGGL((permute_scatter<float, TW>), dim3((unsigned)grid), dim3(NT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t permute_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));    // the array's address on the current device
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_permute_scatter(int dt, const PermuteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const bool pair = (int64_t)a.d * dtype_bytes(dt) <= 64 * 16 && a.k <= 32;
  return pair ? launch_permute_scatter_tw<2>(dt, a, s) : launch_permute_scatter_tw<1>(dt, a, s);
}

}  // namespace moe
