// Internal interface between the host API (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// DT_MXFP8: GEMM operands are MX-fp8 (e4m3 payload bytes plus one UE8M0 scale
// byte per 32 values along K); GEMM outputs are bf16 (or f32 where stated).
enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_MXFP8 = 3 };

inline int dtype_bytes(int dt) { return dt == DT_F32 ? 4 : (dt == DT_MXFP8 ? 1 : 2); }

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
  const float* sel_bias = nullptr;  // [E] or nullptr: experts chosen on probs + sel_bias (weights unbiased)
  int relu = 0;                      // 1: ReLU router (gates max(z, 0) in probs, positive logits only)
};
hipError_t launch_route(int dt, const RouteArgs& a, hipStream_t s);

// Sinkhorn router over the saved probabilities [T, E] (E <= 256): rounds of
// a_t = (1/T) / sum_e p_te b_e and b_e = (1/E) / sum_t p_te a_t (column sums
// from per-block partials in block order), then top-k of p_te b_e per token.
constexpr int kSinkhornTokens = 32;   // tokens per workgroup
struct SinkhornArgs {
  const float* probs;   // [T, E]
  float* b;             // [E] column scales (out; read by later rounds)
  float* part;          // [ceil(T / kSinkhornTokens), E] column partials (workspace)
  int32_t* idx;         // [T, k] out (select)
  float* wts;           // [T, k] out (select)
  int64_t T;
  int E, k, renorm;
};
hipError_t launch_sinkhorn_rows(const SinkhornArgs& a, bool first, hipStream_t s);
hipError_t launch_sinkhorn_cols(const SinkhornArgs& a, hipStream_t s);
hipError_t launch_sinkhorn_select(const SinkhornArgs& a, hipStream_t s);

// Expert-choice router over the saved probabilities [T, E] (E <= 64): every
// expert takes the C tokens with the largest probs[t, e] (lower token index
// first on ties), found by a radix select on the f32 bit patterns of its
// column; written as [T, E] slots (idx[t, e] = e or -1, wts = the taken
// probabilities or 0).  pT: [E, T] f32 workspace (the transposed probabilities).
struct ExpertChoiceArgs {
  const float* probs; float* pT; int32_t* idx; float* wts;
  int64_t T; int E; int64_t C;
};
hipError_t launch_expert_choice(const ExpertChoiceArgs& a, hipStream_t s);
// sel_bias[e] += gamma * sign(T k - E counts[e]) (aux-loss-free balancing update), E <= 256
hipError_t launch_balance_update(const int32_t* counts, float* sel_bias, int64_t T, int E, int k, float gamma,
                                 hipStream_t s);

// ------------------------------------------------------------- permute --
constexpr int kHistTokens = 256;    // tokens per histogram block
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
// Fixed device scratch of the allocation-free permute (moe_permute_noalloc):
// its size, and its address on the current device (looked up once per device).
constexpr size_t kPermuteScratchBytes = (size_t)1 << 20;
constexpr int kMaxDevices = 64;
hipError_t permute_scratch(void** ptr);
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
  void* C2; int64_t ldc2;          // second output: H (SwiGLU forward); for the SwiGLU backward of
                                   // routed experts, optional wrow[r] H[r] rounded once (the down
                                   // weight gradient's operand), H in f32 from the saved G, U
  const void* aux; int64_t ldaux;  // saved GU (SwiGLU backward epilogue)
  // DT_MXFP8 only: scale bytes of P ([rows][K/32], row stride ldp/32) and of
  // Q ([rows][K/32], row stride ldq/32, group stride q_group_stride/32)
  const uint8_t* Ps; const uint8_t* Qs;
  // DT_MXFP8 with a SwiGLU epilogue, quantised along the rows (blocks of 32
  // columns) for the next GEMM; nullptr skips it.  Forward: H into Hq
  // [rows][ldc2], Hs [rows][ldc2/32].  Backward: [dG | dU] into Hq
  // [rows][ldc], Hs [rows][ldc/32].
  uint8_t* Hq; uint8_t* Hs;
  // Optional: token-side row r is row gather[r] of P (and of Ps for MX), P
  // holding p_rows rows (p_rows * ldp * element bytes < 2^31); nullptr reads
  // row r itself
  const int32_t* gather; int64_t p_rows;
  // EPI_SWIGLU_BWD of the routed experts of a 16-bit or f32 layer (nullptr
  // otherwise): wrow [rows] f32 routing weight of each row, dH = wrow[r] *
  // (P Q)[r]; gpart [rows][gparts] f32, the partial row sums of
  // (P Q)[r][n] * H[r][n] (H = silu(G) U from the saved G, U, in f32) over
  // each wave's BN / WN columns, written at index n0 / (BN / WN) + wave column
  const float* wrow; float* gpart; int gparts;
  // EPI_SWIGLU_BWD, 16-bit layers, optional: the rounding remainders
  // v - round(v) of [dG | dU] (C_lo, layout of C) and of the C2 values
  // (C2_lo, layout of C2), rounded to the layer's dtype; the weight
  // gradients add their products to those of the rounded values
  void* C_lo = nullptr; void* C2_lo = nullptr;
  // DT_MXFP8 with EPI_SWIGLU_BWD, optional: [dG | dU] also quantised along the
  // tokens (blocks of 32 rows from each segment's start) for the gate/up
  // weight gradient: column j of [dG | dU] is row j of Tq [2 sub-blocks][ldt]
  // (scales Ts [..][ldt/32]), segment g's rows at K positions tpad[g] ..
  // (tpad: [G+1] padded offsets, multiples of 128; nullptr = position = row).
  // DT_MXFP8 with EPI_SWIGLU_FWD, optional: H so, for the down weight
  // gradient (column j of H is row j of Tq).
  uint8_t* Tq = nullptr; uint8_t* Ts = nullptr; const int32_t* tpad = nullptr; int64_t ldt = 0;
};
// Intermediates a bf16 layer with bf16 experts keeps in f32 (the saved gate/up
// pre-activations [G | U], the expert output rows Y_perm and the input-gradient
// rows dX_perm and dx_shared): rounded to bf16 they alone move y, dx and the
// router gradient by up to 2-3 % of their RMS.  MX-fp8 experts keep [G | U]
// and dX_perm in bf16 and Y_perm in f32; f16 and f32 layers keep all of them
// in their own dtype.
inline bool f32_intermediates(int dt, bool mx) { return dt == DT_BF16 && !mx; }
// Output tile shapes (rows x columns): TILE_128 = 128 x 128 (every dtype),
// TILE_256 = 256 x 256, TILE_128x256 = 128 x 256 and TILE_256PP = 256 x 256
// with the ping-pong main loop (16-bit types; the last two for the row GEMMs
// only).  The plan chooses one per GEMM.
enum TileShape { TILE_128 = 128, TILE_256 = 256, TILE_128x256 = 384, TILE_256PP = 512 };
inline int tile_rows(int t) { return (t == TILE_256 || t == TILE_256PP) ? 256 : 128; }
inline int tile_cols(int t) { return t == TILE_128 ? 128 : 256; }
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
  // DT_MXFP8 only: P is [M][Kpad] and Q is [N][Kpad] (token axis contiguous,
  // segments at the padded offsets `offsets`, each a multiple of 128 tokens),
  // with scale bytes Ps [M][Kpad/32], Qs [N][Kpad/32].
  const uint8_t* Ps; const uint8_t* Qs;
};
// One kernel symbol per weight gradient (same tile engine) so profiles tell them apart.
enum WgradOp { WG_DOWN = 0, WG_GATE_UP = 1, WG_ROUTER = 2 };
hipError_t launch_wgrad(int dt, int op, int tile, const WgradArgs& a, hipStream_t s);

// ------------------------------------------------- MX-fp8 quantisation --
// e4m3 payload plus one UE8M0 scale byte (exponent + 127) per block of 32
// values along K; the scale is the smallest power of two 2^x with
// amax <= 448 * 2^x (x clamped to [-127, 127], -127 for an all-zero block).

// Row operands: element (r, k) at in + (k / sub) * block_stride + r * ld_in + k % sub
// (sub = K: plain rows; sub < K: K concatenates blocks of width sub).
struct MxRowsArgs {
  const void* in; int64_t ld_in; int64_t block_stride; int sub;
  int64_t R; int K;
  uint8_t* out;        // [R][K]
  uint8_t* scales;     // [R][K/32]
};
hipError_t launch_mx_quant_rows(int dt, const MxRowsArgs& a, hipStream_t s);

// Transposing quantiser: the token axis of in ([tokens][C], row stride ld_in)
// becomes K.  Tokens come in G segments (seg = bounds, or fixed segments of
// seg_len); segment g occupies K positions k0 + [pad[g], pad[g+1]) (pad =
// padded bounds, multiples of 32, or g * seg_len); 32-blocks restart at each
// segment start and positions past its tokens hold zeros.  Column c becomes
// output row row0 + c.
struct MxColsArgs {
  const void* in; int64_t ld_in; int C;
  const int32_t* seg; const int32_t* pad; int G; int seg_len;
  int64_t nblk;        // grid bound: number of 32-blocks to cover (>= pad[G] / 32)
  int64_t k0, Kpad, row0;
  uint8_t* out;        // [rows][Kpad]
  uint8_t* scales;     // [rows][Kpad/32]
  // optional: token t of a segment is row gather[seg start + t] of in
  // (rows of x picked by perm_token instead of the rows of x_perm)
  const int32_t* gather = nullptr;
  // optional, from the same read: the row-wise codes too (blocks of 32 along
  // C), input row i (= seg start + t) to rq + i * rld + col, its scale bytes
  // to rqs + i * rlds + col / 32; C a multiple of 32, no gather
  uint8_t* rq = nullptr; uint8_t* rqs = nullptr;
  int64_t rld = 0, rlds = 0;
  // optional, with gather: input row i scaled by wrow[seg start + t] and
  // rounded to the input dtype first (the w dy rows of dY_perm, formed as the
  // combine backward forms them)
  const float* wrow = nullptr;
};
hipError_t launch_mx_quant_cols(int dt, const MxColsArgs& a, hipStream_t s);

// pad[g+1] = pad[g] + ceil((offsets[g+1] - offsets[g]) / align) * align, pad[0] = 0
hipError_t launch_mx_pad_offsets(const int32_t* offsets, int32_t* pad, int G, int align, hipStream_t s);
// one segment of T tokens: seg_pad = {0, T, 0, ceil(T / align) * align}
hipError_t launch_mx_single_segment(int32_t* seg_pad, int64_t T, int align, hipStream_t s);

// ------------------------------------------------------ element-wise --
struct CombineArgs {
  const void* y_perm;   // [T*k, d]: f32 when y_f32, else the activation dtype
  const int32_t* inv; const float* wts; const void* y_shared; void* y;
  int64_t T; int d, k;
  int y_f32;
};
hipError_t launch_combine(int dt, const CombineArgs& a, hipStream_t s);

struct CombineBwdArgs {
  const void* dy; const void* y_perm; const int32_t* inv; const float* wts;
  void* dy_perm;  // [T*k, d]: row inv[t, j] = wts[t, j] dy[t], or dy[t] itself when `copy`
  float* g;       // [T, k]: g = <dy, y_perm row> (y_perm in the act dtype: MX-fp8 experts), or nullptr
  int64_t T; int d, k;
  // without g: the routing weight of each expert-sorted row, wsorted[inv[t, j]] = wts[t, j]
  float* wsorted = nullptr;
  // MX-fp8 experts (16-bit layer): dY_perm also quantised along its rows
  // (blocks of 32) into q [T*k, d] and qs [T*k, d/32]; nullptr skips it
  uint8_t* q = nullptr; uint8_t* qs = nullptr;
  // and dY itself (the shared experts' output gradient) into dq [T, d], dqs [T, d/32]
  uint8_t* dq = nullptr; uint8_t* dqs = nullptr;
  int copy = 0;   // 1: dy_perm rows are plain copies of dy rows (no routing weight)
  int no_rows = 0;  // 1 (MX, with q): the dy_perm rows themselves are not stored, only their codes
};
hipError_t launch_combine_bwd(int dt, const CombineBwdArgs& a, hipStream_t s);

struct RouterDzArgs {
  const float* g; const float* wts; const int32_t* idx; const float* probs; const int32_t* counts;
  void* dz_hl;          // [T, 2*Ep] act: hi part then lo part
  float* dbias_part;    // [gridDim, E]
  int64_t T; int E, Ep, k, renorm; float aux_coef;
  // balancing statistic over real tokens: mask [T] (0 = filler) and the real
  // tokens' counts [E] plus their number at [E]; nullptr = every token
  const int32_t* mask = nullptr; const int32_t* rcounts = nullptr;
  // g from partial sums instead of g [T, k]: g[t, j] = sum over p < gparts of
  // gpart[inv[t, j] * gparts + p], in that order
  const float* gpart = nullptr; const int32_t* inv = nullptr; int gparts = 0;
  int relu = 0;         // 1: probs hold ReLU gates; dz = dp where the gate is positive, else 0
};
int router_dz_blocks(int64_t T);
hipError_t launch_router_dz(int dt, const RouterDzArgs& a, hipStream_t s);

struct Stack2Args {    // w2 = [W_r; W_r] padded to Ep rows each, zeros elsewhere
  const void* w; void* w2; int E, Ep, d;
};
hipError_t launch_stack2(int dt, const Stack2Args& a, hipStream_t s);

// Few experts (E <= kRouterSmallMaxE, d <= kRouterSmallMaxD): one kernel takes
// dz for a block of tokens (written as the hi/lo pair of RouterDzArgs, experts
// e < E only), the block's partial dW_r = dz^T x in f32 and its partial dbias.
constexpr int kRouterSmallMaxE = 16, kRouterSmallMaxD = 2048, kRouterSmallTokens = 64;
struct RouterBwdSmallArgs {
  const float* g; const float* wts; const int32_t* idx; const float* probs; const int32_t* counts;
  const void* x;          // [T, d] act
  void* dz_hl;            // [T, 2*Ep] act (entries e < E and Ep + e, e < E)
  float* dw_part;         // [nblk, E, d]
  float* dbias_part;      // [nblk, E]
  int64_t T; int E, Ep, d, k, renorm; float aux_coef;
  const int32_t* mask = nullptr; const int32_t* rcounts = nullptr;   // as in RouterDzArgs
  const float* gpart = nullptr; const int32_t* inv = nullptr; int gparts = 0;  // as in RouterDzArgs
  int relu = 0;                                                                 // as in RouterDzArgs
};
int router_small_blocks(int64_t T);
hipError_t launch_router_bwd_small(int dt, const RouterBwdSmallArgs& a, hipStream_t s);

struct RouterReduceArgs {
  const float* part;     // [splits, rows, d]: row e (+ row lo_row + e when lo_row >= 0) of each split
  int splits; int E, rows, lo_row, d;
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
  int src_f32 = 0;         // dx_perm and dx_shared rows are f32 (else the activation dtype)
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
  int64_t T; int E, k;    // k: routing slots per token (idx [T, k])
  int kf = 0;             // k of f_e = count_e / (T kf); 0: kf = k (expert choice: the capacity factor)
  // statistic over real tokens only (mask [T], 0 = filler): counts are then
  // taken from idx [T, k] under the mask into rcounts [E + 1] (number of real
  // tokens at [E]), with per-block integer partials in cpart [nblk, E + 1]
  const int32_t* mask = nullptr; const int32_t* idx = nullptr;
  int32_t* rcounts = nullptr; int32_t* cpart = nullptr;
};
int aux_blocks(int64_t T);
hipError_t launch_aux(const AuxArgs& a, hipStream_t s);

}  // namespace moe
