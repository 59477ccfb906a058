// Internal interface between the host API (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

inline int dtype_bytes(int dt) { return dt == DT_F32 ? 4 : 2; }

// ---------------------------------------------------------------- router --
struct RouteArgs {
  const void* x;        // [T, d]
  const void* w;        // [E, d]
  const float* bias;    // [E] or nullptr
  float* probs;         // [T, E]
  int32_t* idx;         // [T, k]
  float* wts;           // [T, k]
  int64_t T;
  int d, E, k, renorm;
};
hipError_t launch_route(int dt, const RouteArgs& a, hipStream_t s);

// ------------------------------------------------------------- permute --
constexpr int kHistTokens = 1024;   // tokens per histogram block
struct PermuteArgs {
  const int32_t* idx;   // [T, k]
  const void* x;        // [T, d]
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  int32_t* perm_token;  // [T*k]
  int32_t* inv;         // [T, k]  (holds block-local ranks between the kernels)
  void* x_perm;         // [T*k, d]
  int32_t* block_counts;// ws [nblk, E]
  int32_t* block_base;  // ws [nblk, E]
  int64_t T;
  int d, E, k;
};
hipError_t launch_permute_hist(const PermuteArgs& a, hipStream_t s);
hipError_t launch_permute_scan(const PermuteArgs& a, hipStream_t s);
hipError_t launch_permute_scatter(int dt, const PermuteArgs& a, hipStream_t s);

// ----------------------------------------------------- grouped GEMMs --
// Row-grouped GEMM: output rows are token rows grouped in segments (one per
// expert, from `offsets`), or one dense segment of M rows.
enum RowOp { OP_GU_FWD = 0, OP_DOWN_FWD = 1, OP_DOWN_DGRAD = 2, OP_GU_DGRAD = 3, OP_ROUTER_DX = 4 };
enum RowEpi { EPI_SWIGLU_FWD = 0, EPI_STORE = 1, EPI_SWIGLU_BWD = 2, EPI_STORE_F32 = 4 };

struct RowGemmArgs {
  const void* P; int64_t ldp;      // token-side operand [rows, K], elements
  const void* Q; int64_t ldq;      // weight-side source (layout depends on the op)
  int64_t q_group_stride;          // elements between consecutive experts' weights
  const int32_t* offsets;          // [G+1] row segments, or nullptr for one segment of M rows
  int G;                           // number of segments
  int64_t M;                       // rows (dense) / total rows (grouped, for the grid bound)
  int N;                           // output columns (H columns for OP_GU_FWD)
  int K;                           // contraction length
  int sub;                         // width of one shared expert (= I for routed experts)
  void* C; int64_t ldc;            // main output
  void* C2; int64_t ldc2;          // second output (H for OP_GU_FWD)
  const void* aux; int64_t ldaux;  // saved GU (SwiGLU backward epilogue)
};
// tile: 256 (16-bit types only) or 128; the plan chooses it once per GEMM.
hipError_t launch_row_gemm(int dt, int op, int epi, int tile, const RowGemmArgs& a, hipStream_t s);

// Weight-gradient GEMM: out[m][n] = sum over the segment's tokens t of P[t][m] * Q[t][n].
struct WgradArgs {
  const void* P; int64_t ldp;      // [tokens, M]
  const void* Q; int64_t ldq;      // [tokens, N]
  const int32_t* offsets;          // [G+1] token segments, or nullptr for [0, Mtok)
  int G;
  int64_t Mtok;
  int M, N;
  int splits;                      // split of each segment's tokens (partials summed later)
  void* C;                         // out[m][n] at C + g*cgs + split*css + (n/sub)*(M*sub) + m*sub + n%sub
  int64_t c_group_stride, c_split_stride;
  int sub;
  int out_f32;                     // 1: write f32 partials, 0: write act dtype
};
// One kernel symbol per weight gradient (same tile engine) so profiles tell them apart.
enum WgradOp { WG_DOWN = 0, WG_GATE_UP = 1, WG_ROUTER = 2 };
hipError_t launch_wgrad(int dt, int op, int tile, const WgradArgs& a, hipStream_t s);

// ------------------------------------------------------ element-wise --
struct CombineArgs {
  const float* y_perm; const int32_t* inv; const float* wts; const void* y_shared; void* y;
  int64_t T; int d, k;
};
hipError_t launch_combine(int dt, const CombineArgs& a, hipStream_t s);

struct CombineBwdArgs {
  const void* dy; const float* y_perm; const int32_t* inv; const float* wts;
  void* dy_perm;  // [T*k, d]
  float* g;       // [T, k]
  int64_t T; int d, k;
};
hipError_t launch_combine_bwd(int dt, const CombineBwdArgs& a, hipStream_t s);

struct RouterDzArgs {
  const float* g; const float* wts; const int32_t* idx; const float* probs; const int32_t* counts;
  void* dz_hl;          // [T, 2*Ep] act: hi part then lo part
  float* dbias_part;    // [gridDim, E]
  int64_t T; int E, Ep, k, renorm; float aux_coef;
};
int router_dz_blocks(int64_t T);
hipError_t launch_router_dz(int dt, const RouterDzArgs& a, hipStream_t s);

struct Stack2Args {    // w2 = [W_r; W_r] padded to Ep rows each, zeros elsewhere
  const void* w; void* w2; int E, Ep, d;
};
hipError_t launch_stack2(int dt, const Stack2Args& a, hipStream_t s);

struct RouterReduceArgs {
  const float* part;     // [splits, 2*Ep, d]
  int splits; int E, Ep, d;
  void* dw;              // [E, d] act
  const float* dbias_part; int nb; float* dbias;  // optional
};
hipError_t launch_router_reduce(int dt, const RouterReduceArgs& a, hipStream_t s);

// Deterministic sum of split-K partials: out[i] = sum_s part[s * n + i] (s in
// order), rounded once to the output dtype.
struct SplitReduceArgs {
  const float* part;     // [splits, n]
  int64_t n; int splits;
  void* out;             // [n] act
};
hipError_t launch_split_reduce(int dt, const SplitReduceArgs& a, hipStream_t s);

// dx = gathered dX_perm rows (+ dx_shared) + router input gradient
struct UnpermuteArgs {
  const void* dx_perm;     // [T*k, d]
  const int32_t* inv;      // [T, k]
  const void* dx_shared;   // [T, d] or nullptr
  const float* dxr;        // [T, d] f32 router part, or nullptr: computed from dz_hl and w_router
  const void* dz_hl;       // [T, 2*Ep]
  const void* w_router;    // [E, d]
  void* dx;                // [T, d]
  int64_t T; int d, k, E, Ep;
};
hipError_t launch_unpermute(int dt, const UnpermuteArgs& a, hipStream_t s);
constexpr int kRouterDxVectorMaxE = 32;   // up to this many experts the router part of dx is computed inline

// Mirror of moe_aux_scalars (include/moe.h); the host checks the layouts match.
struct moe_aux_out {
  float aux, aux_raw, entropy_mean, count_cv;
  int32_t count_min, count_max, n_unused, reserved;
};

struct AuxArgs {
  const float* probs; const int32_t* counts; float* f; float* p_mean; void* out;
  float* part;           // ws [nblk, 2, E]
  int64_t T; int E, k;
};
int aux_blocks(int64_t T);
hipError_t launch_aux(const AuxArgs& a, hipStream_t s);

}  // namespace moe
