// Host side of the C ABI: plan creation and validation, workspace layout,
// and the launch sequence of each call.  Nothing here touches device data;
// every size the device produces (counts, offsets) stays on the device.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "moe.h"

using namespace moe;

static_assert(sizeof(moe_aux_scalars) == sizeof(moe::moe_aux_out), "aux struct layout");

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

const char* kKernelNames =
    "route,permute_hist,permute_scan,permute_scatter,gemm_gate_up_swiglu,gemm_down,"
    "gemm_gate_up_swiglu_shared,gemm_down_shared,combine,combine_bwd,router_dz,"
    "gemm_down_dgrad_swiglu,gemm_wgrad_down,gemm_gate_up_dgrad,gemm_wgrad_gate_up,"
    "gemm_down_dgrad_swiglu_shared,gemm_wgrad_down_shared,gemm_wgrad_gate_up_shared,"
    "gemm_gate_up_dgrad_shared,stack_router,gemm_router_dx,unpermute,gemm_wgrad_router,router_reduce,aux,"
    "wgrad_reduce,mx_quantize,router_bwd_small,balance_update,sinkhorn_rows,sinkhorn_cols,sinkhorn_select,"
    "expert_choice";

}  // namespace

struct moe_plan_s {
  moe_config cfg;
  int dt;
  int64_t T, A;
  int d, E, k, I, Ns, Is, Ep;
  int kf;                  // top_k: T kf routed rows (at most) and the f_e denominator
  int nblk_hist, nblk_dz, nblk_aux, router_splits;
  // GEMM tile per call site, chosen once at plan time
  int t_gu, t_down, t_gu_s, t_down_s, t_down_dgrad, t_gu_dgrad, t_down_dgrad_s, t_gu_dgrad_s, t_router_dx;
  int t_wg_down, t_wg_gu, t_wg_down_s, t_wg_gu_s, t_wg_router;
  // split-K factor of each weight-gradient GEMM (1 = no split, no partials)
  int sp_wg_down, sp_wg_gu, sp_wg_down_s, sp_wg_gu_s;
  // workspace regions (byte offsets)
  size_t o_block_counts, o_block_base, o_dy_perm, o_g, o_dzhl, o_w2, o_dgu, o_dx_perm, o_dgu_s,
      o_dxs, o_dxr, o_dwr_part, o_dbias_part, o_aux_part, o_wg_part, o_wsorted, o_gpart, o_wh, o_dgu_lo,
      o_wh_lo, o_sk_part, o_ec_pt, ws_total;
  // bf16 experts seeing few tokens each: the expert weight gradients add the
  // products of the rounding remainders of [dG | dU] and of w H (see run_wgrad)
  bool comp = false;
  // partial sums of the routing-weight gradient per expert-sorted row (the
  // down dgrad's waves along its columns), 16-bit and f32 expert plans
  int gparts = 0;
  bool router_dx_gemm;     // many experts: the router part of dx goes through the matrix cores
  bool router_small;       // few experts: dz, dW_r and dbias partials in one kernel (no dz^T x GEMM)
  int nblk_small;          // its token blocks
  // MX-fp8 experts: every expert GEMM operand is quantised into the workspace
  // (payload at .pay, scale bytes at .sc) right before the GEMM that reads it
  bool mx = false;
  struct MxBuf { size_t pay = 0, sc = 0; };
  MxBuf mx_xq, mx_hq, mx_wgu, mx_wd, mx_sxq, mx_shq, mx_swgu, mx_swd;                 // forward
  MxBuf mx_dyq, mx_wdt, mx_dguq, mx_wgut, mx_dyt, mx_ht, mx_dgut, mx_xt;              // backward, routed
  MxBuf mx_sdyq, mx_swdt, mx_sdguq, mx_swgut, mx_sdyt, mx_sht, mx_sdgut, mx_sxt;      // backward, shared
  size_t o_mx_pad = 0, o_mx_seg1 = 0;  // padded expert offsets [E+1]; single-segment bounds [2] + pad [2]
  bool keep_inter = false;             // MX: also store [dG | dU] and dY_perm rows (moe_keep_intermediates)
  bool fused = false;                  // MX: the fused path only (moe_config.mx_fused): fewer regions
  // the optional saved-codes buffer (offsets into it): the weights along the
  // backward's reduction axes and H along the tokens, routed and shared
  MxBuf sv_wdt, sv_wgut, sv_ht, sv_swdt, sv_swgut, sv_sht;
  size_t sv_total = 0;
  int64_t Apad = 0, Tpad = 0;          // padded token axes of the transposed operands
  // timing probe
  std::string probe_name;
  std::vector<hipEvent_t> ev0, ev1;
  int probe_n = 0;

  ~moe_plan_s() { release_events(); }
  void release_events() {
    for (auto e : ev0) (void)hipEventDestroy(e);
    for (auto e : ev1) (void)hipEventDestroy(e);
    ev0.clear();
    ev1.clear();
    probe_n = 0;
  }
};

// bf16 and f32 experts: the down dgrad writes w H rows (the routing weight
// times H in f32, rounded once) for the down weight gradient, and dY_perm
// holds plain copies of dy's rows; f16 experts keep dY_perm = w dy and read H
static bool wh_rows(const moe_plan_s* p) { return !p->mx && p->dt != DT_F16; }

namespace {

// Records a hipEvent pair around one launch when the probe targets `name`.
struct Probe {
  moe_plan p;
  hipStream_t s;
  bool on;
  Probe(moe_plan p_, const char* name, hipStream_t s_) : p(p_), s(s_) {
    on = !p->probe_name.empty() && p->probe_name == name && p->probe_n < (int)p->ev0.size();
    if (on) (void)hipEventRecord(p->ev0[p->probe_n], s);
  }
  ~Probe() {
    if (on) {
      (void)hipEventRecord(p->ev1[p->probe_n], s);
      ++p->probe_n;
    }
  }
};

char* wsp(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                        \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

moe_status check_ws(moe_plan p, void* ws, size_t ws_bytes) {
  if (p->ws_total == 0) return MOE_OK;
  if (!ws) return MOE_ERR_WORKSPACE;
  if (ws_bytes < p->ws_total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

constexpr int kCUs = 256;
// mean rows per expert below which a bf16 plan adds the remainder terms to
// the expert weight gradients (moe_plan_s::comp)
constexpr int kCompTokens = 128;
// largest number of Sinkhorn rounds one moe_route_sinkhorn call accepts
constexpr int kSinkhornMaxIters = 1000;

// Tile override for tuning and tests: MOE_ROW_TILE = 128, 256, 128x256 or
// 256pp, MOE_WGRAD_TILE = 128, 256 or 256pp, read once per plan; any other
// value, or a shape the tile does not divide, keeps the default choice.
int env_tile(const char* name, bool wide) {
  const char* v = std::getenv(name);
  if (!v) return 0;
  if (wide && std::strcmp(v, "128x256") == 0) return TILE_128x256;
  if (std::strcmp(v, "256pp") == 0) return TILE_256PP;
  const int t = std::atoi(v);
  return (t == 128 || t == 256) ? t : 0;
}

// Row GEMMs: 256 x 256 ping-pong tiles (8 waves, one workgroup per CU) where
// they divide the shape and the GEMM has at least kPPTileMin of them (whole
// rounds over the 256 CUs, so the last round is a small share), or at least
// kPPTileMinLongK of them with a contraction of kPPLongK or more (each tile
// then runs long enough that its prologue and epilogue are a small share:
// the shared expert's down and gate/up dgrad of the large-expert workload,
// 768 tiles with K = 3072 and 6144, ran 30 % faster than on 128 x 128
// tiles; with K = 512 or 768 the 128 x 128 tiles stay faster); otherwise
// 128 x 256 tiles (4 waves, two workgroups per CU) with at least four rounds
// of them (2048 tiles): they move a quarter less operand data per FLOP than
// 128 x 128, but a short grid of fewer, longer tiles ends unevenly, so
// smaller GEMMs keep 128 x 128 (three workgroups per CU).  `tiles256` = the
// GEMM's 128 x 256 tile count (an upper bound for grouped GEMMs).  The
// 8-wave 256 x 256 tile without ping-pong only on request.
constexpr int64_t kWideTileMin = 2048;
constexpr int64_t kPPTileMin = 1024, kPPTileMinLongK = 512;
constexpr int kPPLongK = 1024;
int choose_row_tile(int dt, int ncols, int block_align, int64_t tiles256, int K, int override_tile) {
  if (dt == DT_F32) return TILE_128;
  if (ncols % 256 || block_align % 256) return TILE_128;
  if (override_tile) return override_tile;
  if (tiles256 / 2 >= kPPTileMin || (tiles256 / 2 >= kPPTileMinLongK && K >= kPPLongK)) return TILE_256PP;
  return tiles256 >= kWideTileMin ? TILE_128x256 : TILE_128;
}
// Weight-gradient GEMMs: W = G (M/bt)(N/bt) output tiles of bt x bt (bt =
// 128 or 256) over `ktok` tokens per group, optionally split s ways over the
// tokens into f32 partials that one extra pass sums in order; every split
// keeps at least 512 tokens per group.
//   128 x 128 tiles (several workgroups per CU): fewer than 384 tiles leave
//   CUs with one workgroup or none, so the token range is split until about
//   512 workgroups run (at most 4 ways);
//   256 x 256 tiles (one workgroup per CU): the split s (up to 8) minimises
//   the estimated time below.
// Estimated time = rounds of W s workgroups over the CUs x the time of one
// tile / s, plus the partials' traffic (s W bt^2 f32 written and read back at
// ~5 TB/s); a 256 x 256 tile taken at ~6.5 TFLOP/s per CU, the 128 x 128 one
// at 0.55 of that.  The tile with the smaller estimate (each at its split)
// runs; 256 x 256 uses the ping-pong main loop (measured 6-15 % faster than
// the 8-wave lockstep loop at the large-expert and skewed workloads), the
// lockstep one only on request.  MOE_WGRAD_SPLITS (1..8) forces a split.
double wgrad_seconds(int bt, int64_t W, double ktok, int s) {
  const double tile_s = 2.0 * bt * bt * ktok / (bt == 256 ? 6.5e12 : 6.5e12 * 0.55);
  const double rounds = (double)((W * s + kCUs - 1) / kCUs);
  return rounds * tile_s / s + (s > 1 ? 2.0 * s * (double)W * bt * bt * 4 / 5e12 : 0.0);
}
int best_wgrad_splits(int bt, int64_t W, double tokens_per_group) {
  if (W <= 0) return 1;
  if (bt == 128) {
    if (W >= 384) return 1;
    int s = (int)(512 / W);
    if (s > 4) s = 4;
    while (s > 1 && tokens_per_group / s < 512) --s;
    return s < 1 ? 1 : s;
  }
  int best = 1;
  double best_t = 1e30;
  for (int s = 1; s <= 8; ++s) {
    if (s > 1 && tokens_per_group / s < 512) break;
    const double t = wgrad_seconds(bt, W, tokens_per_group, s);
    if (t < best_t) { best_t = t; best = s; }
  }
  return best;
}
int choose_wgrad_tile(int dt, double segs, int M, int N, double ktok, int override_tile) {
  if (dt == DT_F32) return 128;
  if (M % 256 || N % 256) return 128;
  if (override_tile) return override_tile;
  const int64_t w256 = (int64_t)segs * (M / 256) * (N / 256), w128 = (int64_t)segs * (M / 128) * (N / 128);
  const double t256 = wgrad_seconds(256, w256, ktok, best_wgrad_splits(256, w256, ktok));
  const double t128 = wgrad_seconds(128, w128, ktok, best_wgrad_splits(128, w128, ktok));
  return t256 <= t128 ? TILE_256PP : 128;
}
int choose_wgrad_splits(int tile, int G, int M, int N, double tokens_per_group) {
  const char* v = std::getenv("MOE_WGRAD_SPLITS");
  if (v) {
    const int s = std::atoi(v);
    if (s >= 1 && s <= 8) return s;
  }
  const int bt = tile_rows(tile);
  return best_wgrad_splits(bt, (int64_t)G * (M / bt) * (N / bt), tokens_per_group);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_INVALID: return "a size or flag is out of range";
    case MOE_ERR_UNSUPPORTED: return "valid but unsupported configuration (dtype or alignment)";
    case MOE_ERR_WORKSPACE: return "workspace missing or smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "the HIP runtime reported an error";
    case MOE_ERR_SCRATCH: return "the call needs more scratch than the fixed device array of an allocation-free call";
  }
  return "unknown status";
}

const char* moe_version(void) { return "moe-ffn-mi355x 0.1 gfx950"; }

const char* moe_kernel_names(void) { return kKernelNames; }

moe_status moe_workspace_region(moe_plan p, const char* name, size_t* offset, size_t* bytes) {
  if (!p || !name || !offset || !bytes) return MOE_ERR_NULL;
  const size_t es = dtype_bytes(p->dt);
  const std::string n(name);
  size_t o = 0, b = 0;
  // a fused MX plan has no act-dtype dY_perm / [dG | dU] rows
  if (p->fused && (n == "dy_perm" || n == "dgu" || n == "dgu_shared")) return MOE_ERR_INVALID;
  if (n == "dy_perm") {
    o = p->o_dy_perm; b = (size_t)p->A * p->d * es;
  } else if (n == "dgu") {
    o = p->o_dgu; b = (size_t)p->A * 2 * p->I * es;
  } else if (n == "wh" && wh_rows(p)) {
    o = p->o_wh; b = (size_t)p->A * p->I * es;
  } else if (n == "dgu_lo" && p->comp) {
    o = p->o_dgu_lo; b = (size_t)p->A * 2 * p->I * es;
  } else if (n == "wh_lo" && p->comp) {
    o = p->o_wh_lo; b = (size_t)p->A * p->I * es;
  } else if (n == "dx_perm") {
    o = p->o_dx_perm; b = (size_t)p->A * p->d * (f32_intermediates(p->dt, p->mx) ? 4 : es);
  } else if (n == "dgu_shared" && p->Ns > 0) {
    o = p->o_dgu_s; b = (size_t)p->T * 2 * p->Ns * p->Is * es;
  } else if (n == "dx_shared" && p->Ns > 0) {
    o = p->o_dxs; b = (size_t)p->T * p->d * (f32_intermediates(p->dt, p->mx) ? 4 : es);
  } else if (p->mx && n == "mx_pad") {
    o = p->o_mx_pad; b = (size_t)(p->E + 1) * 4;
  } else if (p->mx && n.rfind("mx_", 0) == 0) {
    // MX operand codes: "<buffer>" is the e4m3 payload, "<buffer>.scales" its scale bytes
    const bool sc = n.size() > 7 && n.compare(n.size() - 7, 7, ".scales") == 0;
    const std::string base = sc ? n.substr(0, n.size() - 7) : n;
    const int64_t A = p->A, T = p->T, d = p->d, I = p->I, E = p->E, NI = (int64_t)p->Ns * p->Is;
    struct Entry { const char* name; const moe_plan_s::MxBuf* buf; int64_t rows, K; bool shared; };
    // (a fused plan: x's codes for its T rows only, and none of the backward's
    // own weight and H codes, which the saved-codes buffer holds)
    const Entry tab[] = {
        {"mx_xq", &p->mx_xq, p->fused ? T : A, d, false}, {"mx_hq", &p->mx_hq, A, I, false},
        {"mx_wgu", &p->mx_wgu, E * 2 * I, d, false}, {"mx_wd", &p->mx_wd, E * d, I, false},
        {"mx_dyq", &p->mx_dyq, A, d, false},     {"mx_wdt", &p->mx_wdt, I, E * d, false},
        {"mx_dguq", &p->mx_dguq, A, 2 * I, false}, {"mx_wgut", &p->mx_wgut, d, E * 2 * I, false},
        {"mx_dyt", &p->mx_dyt, d, p->Apad, false}, {"mx_ht", &p->mx_ht, I, p->Apad, false},
        {"mx_dgut", &p->mx_dgut, 2 * I, p->Apad, false}, {"mx_xt", &p->mx_xt, d, p->Apad, false},
        {"mx_sxq", &p->mx_sxq, T, d, true},      {"mx_shq", &p->mx_shq, T, NI, true},
        {"mx_swgu", &p->mx_swgu, 2 * NI, d, true}, {"mx_swd", &p->mx_swd, d, NI, true},
        {"mx_sdyq", &p->mx_sdyq, T, d, true},    {"mx_swdt", &p->mx_swdt, NI, d, true},
        {"mx_sdguq", &p->mx_sdguq, T, 2 * NI, true}, {"mx_swgut", &p->mx_swgut, d, 2 * NI, true},
        {"mx_sdyt", &p->mx_sdyt, d, p->Tpad, true}, {"mx_sht", &p->mx_sht, NI, p->Tpad, true},
        {"mx_sdgut", &p->mx_sdgut, 2 * NI, p->Tpad, true}, {"mx_sxt", &p->mx_sxt, d, p->Tpad, true},
    };
    const Entry* hit = nullptr;
    for (const Entry& t : tab)
      if (base == t.name) hit = &t;
    if (!hit || (hit->shared && p->Ns == 0)) return MOE_ERR_INVALID;
    if (p->fused) {
      for (const char* own : {"mx_wdt", "mx_wgut", "mx_ht", "mx_swdt", "mx_swgut", "mx_sht"})
        if (base == own) return MOE_ERR_INVALID;
    }
    o = sc ? hit->buf->sc : hit->buf->pay;
    b = (size_t)hit->rows * (sc ? hit->K / 32 : hit->K);
  } else {
    return MOE_ERR_INVALID;
  }
  *offset = o;
  *bytes = b;
  return MOE_OK;
}

moe_status moe_plan_create(const moe_config* cfg, moe_plan* out) {
  if (!out) return MOE_ERR_NULL;
  *out = nullptr;
  if (!cfg) return MOE_ERR_NULL;
  const moe_config& c = *cfg;
  if (c.T < 0 || c.T > (int64_t)1 << 30) return MOE_ERR_INVALID;
  if (c.d_model <= 0 || c.d_ff <= 0) return MOE_ERR_INVALID;
  if (c.n_experts < 1 || c.n_experts > 256) return MOE_ERR_INVALID;
  if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > 64) return MOE_ERR_INVALID;
  if (c.n_shared < 0 || c.n_shared > 8) return MOE_ERR_INVALID;
  if (c.n_shared > 0 && c.d_ff_shared <= 0) return MOE_ERR_INVALID;
  if (c.renorm != 0 && c.renorm != 1) return MOE_ERR_INVALID;
  if (c.has_router_bias != 0 && c.has_router_bias != 1) return MOE_ERR_INVALID;
  if (c.act_dtype < MOE_F32 || c.act_dtype > MOE_MXFP8_E4M3) return MOE_ERR_INVALID;
  if (c.expert_dtype < MOE_F32 || c.expert_dtype > MOE_MXFP8_E4M3) return MOE_ERR_INVALID;
  if (!(c.aux_coef == c.aux_coef)) return MOE_ERR_INVALID;  // NaN
  if (c.router != MOE_ROUTER_SOFTMAX && c.router != MOE_ROUTER_RELU && c.router != MOE_ROUTER_EXPERT_CHOICE)
    return MOE_ERR_INVALID;
  // ReLU gates and expert-choice probabilities are the weights themselves
  if (c.router != MOE_ROUTER_SOFTMAX && c.renorm) return MOE_ERR_INVALID;
  // expert choice: one routing slot per expert, E <= 64 slots
  if (c.router == MOE_ROUTER_EXPERT_CHOICE && c.n_experts > 64) return MOE_ERR_UNSUPPORTED;
  if (c.act_dtype == MOE_MXFP8_E4M3) return MOE_ERR_UNSUPPORTED;
  const bool mx = c.expert_dtype == MOE_MXFP8_E4M3;
  if (mx && c.act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;   // MX GEMMs write bf16
  if (!mx && c.expert_dtype != c.act_dtype) return MOE_ERR_UNSUPPORTED;
  if (c.mx_fused != 0 && c.mx_fused != 1) return MOE_ERR_INVALID;
  if (c.mx_fused && !mx) return MOE_ERR_INVALID;
  if (c.mx_fused && c.T * c.d_model >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;   // the x-row gather
  if (c.d_model % 128 || c.d_ff % 128) return MOE_ERR_UNSUPPORTED;
  if (c.n_shared > 0 && c.d_ff_shared % 128) return MOE_ERR_UNSUPPORTED;
  const int64_t A = c.T * c.top_k;
  if (A >= ((int64_t)1 << 31)) return MOE_ERR_INVALID;
  // the down dgrad of 16-bit / f32 experts gathers dy's rows with 32-bit byte offsets
  if (!mx && c.T * c.d_model * (c.act_dtype == MOE_F32 ? 4 : 2) >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  const int64_t A_ = A;

  moe_plan p = new (std::nothrow) moe_plan_s();
  if (!p) return MOE_ERR_INVALID;
  p->cfg = c;
  p->dt = c.act_dtype == MOE_F32 ? DT_F32 : (c.act_dtype == MOE_F16 ? DT_F16 : DT_BF16);
  p->mx = mx;
  p->fused = mx && c.mx_fused;
  p->T = c.T;
  p->A = A;
  p->d = c.d_model;
  p->E = c.n_experts;
  // routing slots per token: top_k, or every expert's slot for expert choice
  p->k = c.router == MOE_ROUTER_EXPERT_CHOICE ? c.n_experts : c.top_k;
  p->kf = c.top_k;
  p->I = c.d_ff;
  p->Ns = c.n_shared;
  p->Is = c.n_shared > 0 ? c.d_ff_shared : 0;
  p->Ep = (c.n_experts + 63) / 64 * 64;
  p->nblk_hist = (int)((c.T + kHistTokens - 1) / kHistTokens);
  p->nblk_dz = router_dz_blocks(c.T);
  p->nblk_aux = aux_blocks(c.T);
  {
    // split the router weight-gradient contraction over tokens so that about
    // 512 workgroups run, each with at least 256 tokens
    const int tiles = (2 * p->Ep / 128) * (p->d / 128);
    int s = (512 + tiles - 1) / tiles;
    const int by_tokens = (int)(c.T / 256);
    if (s > by_tokens) s = by_tokens;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    p->router_splits = s;
  }
  p->router_dx_gemm = p->E > kRouterDxVectorMaxE;
  p->router_small = p->E <= kRouterSmallMaxE && p->d <= kRouterSmallMaxD;
  p->nblk_small = router_small_blocks(c.T);
  {
    const double E = p->E, A = (double)A_, T = (double)c.T;
    const double rps = E > 0 ? A / E : 0;               // rows per expert if balanced
    const int rt = env_tile("MOE_ROW_TILE", true), wt = env_tile("MOE_WGRAD_TILE", false);
    const int d = p->d, I = p->I, NI = p->Ns * p->Is;
    // gate/up: output columns are 2I packed, tile columns pair gate/up halves (needs I % (tile/2))
    const int64_t mt = (A_ + (int64_t)p->E * 127) / 128, mts = (c.T + 127) / 128;   // row tiles (bounds)
    p->t_gu = choose_row_tile(p->dt, 2 * I, 2 * I, mt * (I / 128), d, rt);
    p->t_down = choose_row_tile(p->dt, d, 256, mt * (d / 256), I, rt);
    p->t_down_dgrad = choose_row_tile(p->dt, I, I, mt * (I / 256), d, rt);
    p->t_gu_dgrad = choose_row_tile(p->dt, d, 256, mt * (d / 256), 2 * I, rt);
    p->t_router_dx = 128;                                 // K = 2 Ep is tiny
    p->t_wg_down = choose_wgrad_tile(p->dt, E, d, I, rps, wt);
    p->t_wg_gu = choose_wgrad_tile(p->dt, E, 2 * I, d, rps, wt);
    p->t_wg_router = 128;
    // MX-fp8 experts: 256 x 256 tiles (8 waves, the plain ring) where the
    // 16-bit layer would take its 256 x 256 (ping-pong) tiles, for the forward
    // GEMMs, the gate/up dgrad and the weight gradients; the down dgrad, whose
    // epilogue writes the token-axis codes of 128-row tiles, keeps 128 x 128
    auto mx_row = [](int t) { return (t == TILE_256PP || t == TILE_256) ? TILE_256 : TILE_128; };
    if (p->mx) {
      p->t_gu = mx_row(p->t_gu);
      p->t_down = mx_row(p->t_down);
      p->t_gu_dgrad = mx_row(p->t_gu_dgrad);
      p->t_wg_down = mx_row(p->t_wg_down);
      p->t_wg_gu = mx_row(p->t_wg_gu);
      p->t_down_dgrad = 128;
    }
    p->sp_wg_down = choose_wgrad_splits(p->t_wg_down, E, d, I, rps);
    p->sp_wg_gu = choose_wgrad_splits(p->t_wg_gu, E, 2 * I, d, rps);
    if (p->Ns > 0) {
      p->t_gu_s = choose_row_tile(p->dt, 2 * NI, 2 * p->Is, mts * (NI / 128), d, rt);
      p->t_down_s = choose_row_tile(p->dt, d, 256, mts * (d / 256), NI, rt);
      p->t_down_dgrad_s = choose_row_tile(p->dt, NI, p->Is, mts * (NI / 256), d, rt);
      p->t_gu_dgrad_s = choose_row_tile(p->dt, d, 256, mts * (d / 256), 2 * NI, rt);
      p->t_wg_down_s = (p->Is % 256 == 0) ? choose_wgrad_tile(p->dt, 1, d, NI, T, wt) : 128;
      p->t_wg_gu_s = choose_wgrad_tile(p->dt, 1, 2 * NI, d, T, wt);
      if (p->mx) {
        p->t_gu_s = mx_row(p->t_gu_s);
        p->t_down_s = mx_row(p->t_down_s);
        p->t_gu_dgrad_s = mx_row(p->t_gu_dgrad_s);
        p->t_wg_down_s = mx_row(p->t_wg_down_s);
        p->t_wg_gu_s = mx_row(p->t_wg_gu_s);
        p->t_down_dgrad_s = 128;
      }
      p->sp_wg_down_s = choose_wgrad_splits(p->t_wg_down_s, 1, d, NI, T);
      p->sp_wg_gu_s = choose_wgrad_splits(p->t_wg_gu_s, 1, 2 * NI, d, T);
    } else {
      p->t_gu_s = p->t_down_s = p->t_down_dgrad_s = p->t_gu_dgrad_s = p->t_wg_down_s = p->t_wg_gu_s = 128;
      p->sp_wg_down_s = p->sp_wg_gu_s = 1;
    }
  }
  const size_t es = dtype_bytes(p->dt);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  p->o_block_counts = take((size_t)p->nblk_hist * p->E * 4);
  p->o_block_base = take((size_t)p->nblk_hist * p->E * 4);
  p->o_dy_perm = take(p->fused ? 0 : (size_t)A * p->d * es);
  p->o_g = take(p->mx ? (size_t)A * 4 : 0);
  if (!p->mx) {
    // waves along the columns of the down dgrad's tile: BN / WN columns each
    const int wcols = p->t_down_dgrad == TILE_128x256 ? 128 : 64;   // 128 x 128, 256 x 256, 256 x 256 pp: 64
    p->gparts = p->I / wcols;
  }
  p->o_wsorted = take((size_t)A * 4);
  p->o_gpart = take(p->mx ? 0 : (size_t)A * p->gparts * 4);
  p->o_dzhl = take((size_t)p->T * 2 * p->Ep * es);
  p->o_w2 = take(p->router_dx_gemm ? (size_t)2 * p->Ep * p->d * es : 0);
  p->o_dgu = take(p->fused ? 0 : (size_t)A * 2 * p->I * es);
  // w H rows, the down weight gradient's operand (bf16 and f32 experts)
  p->o_wh = take(wh_rows(p) ? (size_t)A * p->I * es : 0);
  {
    // fewer than kCompTokens rows per expert on average (bf16): a weight
    // gradient element then sums a handful of products, and one bf16
    // rounding of an operand shows in it undamped
    p->comp = p->dt == DT_BF16 && !p->mx && A > 0 && A < (int64_t)kCompTokens * p->E;
    const char* v = std::getenv("MOE_WGRAD_COMP");
    if (v && p->dt == DT_BF16 && !p->mx) p->comp = std::atoi(v) != 0;
  }
  p->o_dgu_lo = take(p->comp ? (size_t)A * 2 * p->I * es : 0);
  // Sinkhorn router: column partials of its token blocks
  p->o_sk_part = take((size_t)((p->T + kSinkhornTokens - 1) / kSinkhornTokens) * p->E * 4);
  // expert choice: the transposed probabilities
  p->o_ec_pt = take(c.router == MOE_ROUTER_EXPERT_CHOICE ? (size_t)p->T * p->E * 4 : 0);
  p->o_wh_lo = take(p->comp ? (size_t)A * p->I * es : 0);
  // input-gradient rows of the experts, f32 in a bf16 layer (f32_intermediates)
  const size_t xs = f32_intermediates(p->dt, p->mx) ? 4 : es;
  p->o_dx_perm = take((size_t)A * p->d * xs);
  p->o_dgu_s = take(p->fused ? 0 : (size_t)p->T * 2 * p->Ns * p->Is * es);
  p->o_dxs = take(p->Ns > 0 ? (size_t)p->T * p->d * xs : 0);
  p->o_dxr = take(p->router_dx_gemm ? (size_t)p->T * p->d * 4 : 0);
  p->o_dwr_part = take(p->router_small ? (size_t)p->nblk_small * p->E * p->d * 4
                                        : (size_t)p->router_splits * 2 * p->Ep * p->d * 4);
  p->o_dbias_part = take((size_t)(p->router_small ? p->nblk_small : p->nblk_dz) * p->E * 4);
  // f32 [nblk, 2, E] partials, then (real-token mask) int32 [nblk, E + 1]
  p->o_aux_part = take((size_t)(p->nblk_aux > 0 ? p->nblk_aux : 1) * (3 * p->E + 1) * 4);
  {
    // one f32 partial buffer, reused by every split weight-gradient GEMM in turn
    size_t part = 0;
    auto need = [&](int sp, int64_t elems) {
      if (sp > 1 && (size_t)sp * elems * 4 > part) part = (size_t)sp * elems * 4;
    };
    const int cf = p->comp ? 2 : 1;                   // rounded values' and remainders' partials
    need(cf * p->sp_wg_down, (int64_t)p->E * p->d * p->I);
    need(cf * p->sp_wg_gu, (int64_t)p->E * 2 * p->I * p->d);
    need(p->sp_wg_down_s, (int64_t)p->d * p->Ns * p->Is);
    need(p->sp_wg_gu_s, (int64_t)2 * p->Ns * p->Is * p->d);
    p->o_wg_part = take(part);
  }
  if (p->mx) {
    // MX operands: payload bytes + one scale byte per 32 (both 256-byte aligned)
    auto mxb = [&](int64_t rows, int64_t K) {
      moe_plan_s::MxBuf b;
      b.pay = take((size_t)rows * K);
      b.sc = take((size_t)rows * (K / 32));
      return b;
    };
    const int64_t A = p->A, T = p->T, d = p->d, I = p->I, E = p->E, NI = (int64_t)p->Ns * p->Is;
    p->Apad = (A + 128 * E + 127) / 128 * 128;     // >= sum over experts of their counts rounded up to 128
    p->Tpad = (T + 127) / 128 * 128;
    p->mx_xq = mxb(p->fused ? T : A, d);             // (fused: x's T rows, gathered on load)
    p->mx_hq = mxb(A, I);
    p->mx_wgu = mxb(E * 2 * I, d);
    p->mx_wd = mxb(E * d, I);
    p->mx_dyq = mxb(A, d);
    const bool own = !p->fused;                      // the backward's own weight and H codes
    p->mx_wdt = mxb(own ? I : 0, E * d);
    p->mx_dguq = mxb(A, 2 * I);
    p->mx_wgut = mxb(own ? d : 0, E * 2 * I);
    p->mx_dyt = mxb(d, p->Apad);
    p->mx_ht = mxb(own ? I : 0, p->Apad);
    p->mx_dgut = mxb(2 * I, p->Apad);
    p->mx_xt = mxb(d, p->Apad);
    p->o_mx_pad = take((size_t)(E + 1) * 4);
    p->o_mx_seg1 = take(4 * 4);
    {
      size_t so = 0;
      auto sb = [&](int64_t rows, int64_t K) {
        moe_plan_s::MxBuf b;
        b.pay = so; so += ((size_t)rows * K + 255) / 256 * 256;
        b.sc = so; so += ((size_t)rows * (K / 32) + 255) / 256 * 256;
        return b;
      };
      p->sv_wdt = sb(I, E * d);
      p->sv_wgut = sb(d, E * 2 * I);
      p->sv_ht = sb(I, p->Apad);
      if (NI > 0) {
        p->sv_swdt = sb(NI, d);
        p->sv_swgut = sb(d, 2 * NI);
        p->sv_sht = sb(NI, p->Tpad);
      }
      p->sv_total = so;
    }
    if (NI > 0) {
      p->mx_sxq = mxb(T, d);
      p->mx_shq = mxb(T, NI);
      p->mx_swgu = mxb(2 * NI, d);
      p->mx_swd = mxb(d, NI);
      p->mx_sdyq = mxb(T, d);
      p->mx_swdt = mxb(own ? NI : 0, d);
      p->mx_sdguq = mxb(T, 2 * NI);
      p->mx_swgut = mxb(own ? d : 0, 2 * NI);
      p->mx_sdyt = mxb(d, p->Tpad);
      p->mx_sht = mxb(own ? NI : 0, p->Tpad);
      p->mx_sdgut = mxb(2 * NI, p->Tpad);
      p->mx_sxt = mxb(d, p->Tpad);
    }
  }
  p->ws_total = off;
  *out = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan plan) { delete plan; }

size_t moe_workspace_bytes(moe_plan plan) { return plan ? plan->ws_total : 0; }
size_t moe_mx_saved_bytes(moe_plan plan) { return (plan && plan->mx) ? plan->sv_total : 0; }

// Weight-gradient GEMM into `out` ([G][group_elems], act dtype), split over
// tokens `splits` ways through f32 partials when splits > 1.
// lo_p / lo_q (optional, one of them): the rounding remainders of P or Q in
// the same layout.  The GEMM then runs twice, on (P, Q) and on (lo_p, Q) or
// (P, lo_q), into consecutive f32 partial slots, and the reduce adds all
// slots in order: the weight gradient of operands carrying about twice the
// dtype's mantissa bits.
moe_status run_wgrad(moe_plan p, int op, int tile, int splits, WgradArgs a, void* out, int64_t group_elems,
                     void* ws, const char* name, hipStream_t s, int gdt = -1, const void* lo_p = nullptr,
                     const void* lo_q = nullptr) {
  if (gdt < 0) gdt = p->dt;
  a.splits = splits;
  a.c_group_stride = group_elems;
  if (lo_p || lo_q) {
    float* part = reinterpret_cast<float*>(wsp(ws, p->o_wg_part));
    const int64_t slot = (int64_t)a.G * group_elems;
    a.C = part; a.c_split_stride = slot; a.out_f32 = 1;
    {
      Probe pr(p, name, s);
      MOE_TRY(launch_wgrad(gdt, op, tile, a, s));
    }
    WgradArgs b = a;
    if (lo_p) b.P = lo_p;
    else b.Q = lo_q;
    b.C = part + splits * slot;
    {
      Probe pr(p, name, s);
      MOE_TRY(launch_wgrad(gdt, op, tile, b, s));
    }
    SplitReduceArgs r{part, slot, 2 * splits, out};
    Probe pr(p, "wgrad_reduce", s);
    MOE_TRY(launch_split_reduce(p->dt, r, s));
    return MOE_OK;
  }
  if (splits <= 1) {
    a.C = out; a.c_split_stride = 0; a.out_f32 = 0;
    Probe pr(p, name, s);
    MOE_TRY(launch_wgrad(gdt, op, tile, a, s));
    return MOE_OK;
  }
  float* part = reinterpret_cast<float*>(wsp(ws, p->o_wg_part));
  a.C = part; a.c_split_stride = (int64_t)a.G * group_elems; a.out_f32 = 1;
  {
    Probe pr(p, name, s);
    MOE_TRY(launch_wgrad(gdt, op, tile, a, s));
  }
  SplitReduceArgs r{part, (int64_t)a.G * group_elems, splits, out};
  Probe pr(p, "wgrad_reduce", s);
  MOE_TRY(launch_split_reduce(p->dt, r, s));
  return MOE_OK;
}

#define MOE_TRY_STATUS(expr)            \
  do {                                  \
    moe_status st_ = (expr);            \
    if (st_ != MOE_OK) return st_;      \
  } while (0)

// ---- MX-fp8 operand helpers
struct MxOp { uint8_t* pay; uint8_t* sc; };
MxOp mxop(void* ws, const moe_plan_s::MxBuf& b) {
  return {reinterpret_cast<uint8_t*>(wsp(ws, b.pay)), reinterpret_cast<uint8_t*>(wsp(ws, b.sc))};
}
// a region of the saved-codes buffer (moe_ffn_args / moe_saved .mx_saved)
MxOp svop(const void* saved, const moe_plan_s::MxBuf& b) {
  uint8_t* base = static_cast<uint8_t*>(const_cast<void*>(saved));
  return {base + b.pay, base + b.sc};
}
// rows operand: element (r, k) at in + (k / sub) * block_stride + r * ld_in + k % sub
moe_status mx_rows(moe_plan p, hipStream_t s, const void* in, int64_t ld_in, int64_t block_stride, int sub,
                   int64_t R, int K, MxOp o) {
  MxRowsArgs a{in, ld_in, block_stride, sub, R, K, o.pay, o.sc};
  Probe pr(p, "mx_quantize", s);
  MOE_TRY(launch_mx_quant_rows(p->dt, a, s));
  return MOE_OK;
}
// transposed operand: the token axis of in [tokens][C] becomes K
// rq (optional): the row-wise codes of the same input too, row i at
// rq.pay + i * rld (scales rq.sc + i * rld / 32)
moe_status mx_cols(moe_plan p, hipStream_t s, const void* in, int64_t ld_in, int C, const int32_t* seg,
                   const int32_t* pad, int G, int seg_len, int64_t nblk, int64_t k0, int64_t Kpad, int64_t row0,
                   MxOp o, const int32_t* gather = nullptr, MxOp rq = {nullptr, nullptr}, int64_t rld = 0,
                   const float* wrow = nullptr) {
  MxColsArgs a{in, ld_in, C, seg, pad, G, seg_len, nblk, k0, Kpad, row0, o.pay, o.sc, gather};
  a.rq = rq.pay; a.rqs = rq.sc; a.rld = rld; a.rlds = rld / 32; a.wrow = wrow;
  Probe pr(p, "mx_quantize", s);
  MOE_TRY(launch_mx_quant_cols(p->dt, a, s));
  return MOE_OK;
}
// MX row GEMM operands
void mx_pq(RowGemmArgs& a, MxOp P, int64_t ldp, MxOp Q, int64_t ldq, int64_t q_group_stride) {
  a.P = P.pay; a.Ps = P.sc; a.ldp = ldp;
  a.Q = Q.pay; a.Qs = Q.sc; a.ldq = ldq; a.q_group_stride = q_group_stride;
}

// ------------------------------------------------------------------ route --
moe_status moe_route(moe_plan p, const void* x, const void* w_router, const float* bias, float* probs,
                     int32_t* topk_idx, float* topk_w, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (p->T == 0) return MOE_OK;
  if (!x || !w_router || !probs || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (p->cfg.has_router_bias && !bias) return MOE_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->cfg.router == MOE_ROUTER_EXPERT_CHOICE) return MOE_ERR_INVALID;   // moe_route_expert_choice
  RouteArgs a{x, w_router, p->cfg.has_router_bias ? bias : nullptr, probs, topk_idx, topk_w,
              p->T, p->d, p->E, p->k, p->cfg.renorm};
  a.relu = p->cfg.router == MOE_ROUTER_RELU;
  Probe pr(p, "route", s);
  return hip_status(launch_route(p->dt, a, s));
}

moe_status moe_route_expert_choice(moe_plan p, const void* x, const void* w_router, const float* bias,
                                   float* probs, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (p->cfg.router != MOE_ROUTER_EXPERT_CHOICE) return MOE_ERR_INVALID;
  if (p->T == 0) return MOE_OK;
  if (!x || !w_router || !probs || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (p->cfg.has_router_bias && !bias) return MOE_ERR_NULL;
  moe_status st = check_ws(p, ws, ws_bytes);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    // the probabilities (the plain top-1 this writes into the slots is
    // overwritten by the experts' choice)
    RouteArgs a{x, w_router, p->cfg.has_router_bias ? bias : nullptr, probs, topk_idx, topk_w,
                p->T, p->d, p->E, 1, 0};
    Probe pr(p, "route", s);
    MOE_TRY(launch_route(p->dt, a, s));
  }
  ExpertChoiceArgs b{probs, reinterpret_cast<float*>(wsp(ws, p->o_ec_pt)), topk_idx, topk_w, p->T, p->E,
                     p->T * p->kf / p->E};
  Probe pr(p, "expert_choice", s);
  return hip_status(launch_expert_choice(b, s));
}

moe_status moe_route_balanced(moe_plan p, const void* x, const void* w_router, const float* bias,
                              const float* sel_bias, float* probs, int32_t* topk_idx, float* topk_w, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (p->cfg.router != MOE_ROUTER_SOFTMAX) return MOE_ERR_INVALID;   // ranks on probabilities (top-k)
  if (p->T == 0) return MOE_OK;
  if (!x || !w_router || !sel_bias || !probs || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (p->cfg.has_router_bias && !bias) return MOE_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RouteArgs a{x, w_router, p->cfg.has_router_bias ? bias : nullptr, probs, topk_idx, topk_w,
              p->T, p->d, p->E, p->k, p->cfg.renorm, sel_bias};
  Probe pr(p, "route", s);
  return hip_status(launch_route(p->dt, a, s));
}

moe_status moe_route_sinkhorn(moe_plan p, const void* x, const void* w_router, const float* bias, int32_t n_iter,
                              float* probs, int32_t* topk_idx, float* topk_w, float* col_scale, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (n_iter < 1 || n_iter > kSinkhornMaxIters) return MOE_ERR_INVALID;
  if (p->cfg.router != MOE_ROUTER_SOFTMAX) return MOE_ERR_INVALID;   // balances probabilities
  if (p->T == 0) return MOE_OK;
  if (!x || !w_router || !probs || !topk_idx || !topk_w || !col_scale) return MOE_ERR_NULL;
  if (p->cfg.has_router_bias && !bias) return MOE_ERR_NULL;
  moe_status st = check_ws(p, ws, ws_bytes);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    // the probabilities (the plain router's choice is overwritten below)
    RouteArgs a{x, w_router, p->cfg.has_router_bias ? bias : nullptr, probs, topk_idx, topk_w,
                p->T, p->d, p->E, p->k, p->cfg.renorm};
    Probe pr(p, "route", s);
    MOE_TRY(launch_route(p->dt, a, s));
  }
  SinkhornArgs a{probs, col_scale, reinterpret_cast<float*>(wsp(ws, p->o_sk_part)), topk_idx, topk_w,
                 p->T, p->E, p->k, p->cfg.renorm};
  for (int it = 0; it < n_iter; ++it) {
    {
      Probe pr(p, "sinkhorn_rows", s);
      MOE_TRY(launch_sinkhorn_rows(a, it == 0, s));
    }
    Probe pr(p, "sinkhorn_cols", s);
    MOE_TRY(launch_sinkhorn_cols(a, s));
  }
  Probe pr(p, "sinkhorn_select", s);
  return hip_status(launch_sinkhorn_select(a, s));
}

moe_status moe_balance_update(moe_plan p, const int32_t* counts, float* sel_bias, float gamma, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (p->cfg.router != MOE_ROUTER_SOFTMAX) return MOE_ERR_INVALID;  // the balanced top-k router's update
  if (!counts || !sel_bias) return MOE_ERR_NULL;
  if (!(gamma >= 0.0f) || !(gamma < INFINITY)) return MOE_ERR_INVALID;   // also rejects NaN
  hipStream_t s = static_cast<hipStream_t>(stream);
  Probe pr(p, "balance_update", s);
  return hip_status(launch_balance_update(counts, sel_bias, p->T, p->E, p->k, gamma, s));
}

// ---------------------------------------------------------------- permute --
moe_status moe_permute(moe_plan p, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* inv_perm, void* x_perm, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (p->T > 0 && (!topk_idx || !perm_token || !inv_perm || (x_perm && !x))) return MOE_ERR_NULL;
  moe_status st = check_ws(p, ws, ws_bytes);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PermuteArgs a{topk_idx, x, counts, offsets, perm_token, inv_perm, x_perm,
                reinterpret_cast<int32_t*>(wsp(ws, p->o_block_counts)),
                reinterpret_cast<int32_t*>(wsp(ws, p->o_block_base)), p->T, p->d, p->E, p->k};
  {
    Probe pr(p, "permute_hist", s);
    MOE_TRY(launch_permute_hist(a, s));
  }
  {
    Probe pr(p, "permute_scan", s);
    MOE_TRY(launch_permute_scan(a, s));
  }
  {
    Probe pr(p, "permute_scatter", s);
    MOE_TRY(launch_permute_scatter(p->dt, a, s));
  }
  return MOE_OK;
}

// Scratch bytes moe_permute needs: [blocks x E] counts, then [blocks x E] first rows.
static size_t permute_scratch_bytes(moe_plan p) { return 2 * align_up((size_t)p->nblk_hist * p->E * 4); }

moe_status moe_permute_noalloc(moe_plan p, const int32_t* topk_idx, const void* x, int32_t* counts, int32_t* offsets,
                               int32_t* perm_token, int32_t* inv_perm, void* x_perm, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (p->T > 0 && (!topk_idx || !perm_token || !inv_perm || (x_perm && !x))) return MOE_ERR_NULL;
  if (permute_scratch_bytes(p) > kPermuteScratchBytes) return MOE_ERR_SCRATCH;
  void* scr = nullptr;
  MOE_TRY(permute_scratch(&scr));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* bc = static_cast<int32_t*>(scr);
  int32_t* bb = reinterpret_cast<int32_t*>(static_cast<char*>(scr) + permute_scratch_bytes(p) / 2);
  PermuteArgs a{topk_idx, x, counts, offsets, perm_token, inv_perm, x_perm, bc, bb, p->T, p->d, p->E, p->k};
  {
    Probe pr(p, "permute_hist", s);
    MOE_TRY(launch_permute_hist(a, s));
  }
  {
    Probe pr(p, "permute_scan", s);
    MOE_TRY(launch_permute_scan(a, s));
  }
  {
    Probe pr(p, "permute_scatter", s);
    MOE_TRY(launch_permute_scatter(p->dt, a, s));
  }
  return MOE_OK;
}

// ------------------------------------------------------------- expert FFN --
moe_status mx_expert_ffn(moe_plan p, const moe_ffn_args* f, void* ws, hipStream_t s);

moe_status moe_expert_ffn(moe_plan p, const moe_ffn_args* f, void* ws, size_t ws_bytes, void* stream) {
  if (!p || !f) return MOE_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->T == 0) return MOE_OK;
  const bool gather = p->mx && f->perm_token;       // MX: token rows gathered from x on load
  // (H may be NULL for MX experts given a saved-codes buffer: it then exists only as its codes)
  const bool h_opt = p->mx && f->mx_saved;
  if (p->fused && (!f->perm_token || !f->mx_saved)) return MOE_ERR_NULL;   // the fused path only
  if ((!gather && !f->x_perm) || !f->offsets || !f->w_gate_up || !f->w_down || !f->gu || (!f->h && !h_opt) ||
      !f->y_perm)
    return MOE_ERR_NULL;
  if (gather && !f->x) return MOE_ERR_NULL;
  if (gather && p->T * p->d >= (int64_t)1 << 31) return MOE_ERR_INVALID;   // 32-bit gather offsets
  if (p->Ns > 0 && (!f->x || !f->ws_gate_up || !f->ws_down || !f->gu_shared || (!f->h_shared && !h_opt) ||
                    !f->y_shared))
    return MOE_ERR_NULL;
  if (p->mx) {
    moe_status st = check_ws(p, ws, ws_bytes);
    if (st != MOE_OK) return st;
    return mx_expert_ffn(p, f, ws, s);
  }
  const int d = p->d, I = p->I;
  {
    RowGemmArgs a{};
    a.P = f->x_perm; a.ldp = d;
    a.Q = f->w_gate_up; a.ldq = d; a.q_group_stride = (int64_t)2 * I * d;
    a.offsets = f->offsets; a.G = p->E; a.M = p->A; a.N = I; a.K = d; a.sub = I;
    a.C = f->gu; a.ldc = 2 * I; a.C2 = f->h; a.ldc2 = I;
    Probe pr(p, "gemm_gate_up_swiglu", s);
    MOE_TRY(launch_row_gemm(p->dt, OP_GU_FWD, EPI_SWIGLU_FWD, p->t_gu, a, s));
  }
  {
    RowGemmArgs a{};
    a.P = f->h; a.ldp = I;
    a.Q = f->w_down; a.ldq = I; a.q_group_stride = (int64_t)d * I;
    a.offsets = f->offsets; a.G = p->E; a.M = p->A; a.N = d; a.K = I; a.sub = I;
    a.C = f->y_perm; a.ldc = d;                       // Y_perm: f32 in a bf16 layer, else the activation dtype
    Probe pr(p, "gemm_down", s);
    MOE_TRY(launch_row_gemm(p->dt, OP_DOWN_FWD, f32_intermediates(p->dt, p->mx) ? EPI_STORE_F32 : EPI_STORE,
                            p->t_down, a, s));
  }
  if (p->Ns > 0) {
    const int Is = p->Is, NI = p->Ns * p->Is;
    {
      RowGemmArgs a{};
      a.P = f->x; a.ldp = d;
      a.Q = f->ws_gate_up; a.ldq = d; a.q_group_stride = 0;
      a.offsets = nullptr; a.G = 1; a.M = p->T; a.N = NI; a.K = d; a.sub = Is;
      a.C = f->gu_shared; a.ldc = 2 * NI; a.C2 = f->h_shared; a.ldc2 = NI;
      Probe pr(p, "gemm_gate_up_swiglu_shared", s);
      MOE_TRY(launch_row_gemm(p->dt, OP_GU_FWD, EPI_SWIGLU_FWD, p->t_gu_s, a, s));
    }
    {
      RowGemmArgs a{};
      a.P = f->h_shared; a.ldp = NI;
      a.Q = f->ws_down; a.ldq = Is; a.q_group_stride = 0;
      a.offsets = nullptr; a.G = 1; a.M = p->T; a.N = d; a.K = NI; a.sub = Is;
      a.C = f->y_shared; a.ldc = d;
      Probe pr(p, "gemm_down_shared", s);
      MOE_TRY(launch_row_gemm(p->dt, OP_DOWN_FWD, EPI_STORE, p->t_down_s, a, s));
    }
  }
  return MOE_OK;
}

// MX-fp8 forward of the experts: each GEMM operand quantised along that GEMM's
// reduction axis just before the GEMM (KohakUwULLM README, "Key features").
moe_status mx_expert_ffn(moe_plan p, const moe_ffn_args* f, void* ws, hipStream_t s) {
  const int64_t d = p->d, I = p->I, E = p->E, A = p->A;
  const MxOp xq = mxop(ws, p->mx_xq), hq = mxop(ws, p->mx_hq), wgu = mxop(ws, p->mx_wgu), wd = mxop(ws, p->mx_wd);
  // token rows: x quantised once per token and gathered by perm_token on load
  // (into the shared experts' buffer when there are shared experts, which
  // read the same codes), else the T*k rows of x_perm
  const bool gather = f->perm_token != nullptr;
  const MxOp xrows = (gather && p->Ns > 0) ? mxop(ws, p->mx_sxq) : xq;
  if (gather) MOE_TRY_STATUS(mx_rows(p, s, f->x, d, 0, (int)d, p->T, (int)d, xrows));
  else MOE_TRY_STATUS(mx_rows(p, s, f->x_perm, d, 0, (int)d, A, (int)d, xq));
  // with a saved-codes buffer: the weights' backward codes from the pass that
  // makes their row-wise ones, and H's token-axis codes from the epilogue
  const void* sv = f->mx_saved;
  int32_t* pad = reinterpret_cast<int32_t*>(wsp(ws, p->o_mx_pad));
  if (sv) {
    Probe pr(p, "mx_quantize", s);
    MOE_TRY(launch_mx_pad_offsets(f->offsets, pad, (int)E, 128, s));
  }
  if (sv)   // W_gu [E][2I][d]: along d (forward) and along each expert's 2I (dX = [dG | dU] W_gu)
    MOE_TRY_STATUS(mx_cols(p, s, f->w_gate_up, d, (int)d, nullptr, nullptr, (int)E, (int)(2 * I), E * 2 * I / 32, 0,
                           E * 2 * I, 0, svop(sv, p->sv_wgut), nullptr, wgu, d));
  else
    MOE_TRY_STATUS(mx_rows(p, s, f->w_gate_up, d, 0, (int)d, E * 2 * I, (int)d, wgu));
  {
    RowGemmArgs a{};
    mx_pq(a, xrows, d, wgu, d, 2 * I * d);
    if (gather) { a.gather = f->perm_token; a.p_rows = p->T; }
    a.offsets = f->offsets; a.G = (int)E; a.M = A; a.N = (int)I; a.K = (int)d; a.sub = (int)I;
    a.C = f->gu; a.ldc = 2 * I; a.C2 = f->h; a.ldc2 = I;
    a.Hq = hq.pay; a.Hs = hq.sc;                     // the epilogue also quantises H row-wise
    if (sv) {                                        // and along the tokens, for dW_d
      const MxOp ht = svop(sv, p->sv_ht);
      a.Tq = ht.pay; a.Ts = ht.sc; a.tpad = pad; a.ldt = p->Apad;
    }
    Probe pr(p, "gemm_gate_up_swiglu", s);
    MOE_TRY(launch_row_gemm(DT_MXFP8, OP_GU_FWD, EPI_SWIGLU_FWD, p->t_gu, a, s));
  }
  if (sv)   // W_d [E][d][I]: along I (forward) and along each expert's d (dH = dY W_d)
    MOE_TRY_STATUS(mx_cols(p, s, f->w_down, I, (int)I, nullptr, nullptr, (int)E, (int)d, E * d / 32, 0, E * d, 0,
                           svop(sv, p->sv_wdt), nullptr, wd, I));
  else
    MOE_TRY_STATUS(mx_rows(p, s, f->w_down, I, 0, (int)I, E * d, (int)I, wd));
  {
    RowGemmArgs a{};
    mx_pq(a, hq, I, wd, I, d * I);
    a.offsets = f->offsets; a.G = (int)E; a.M = A; a.N = (int)d; a.K = (int)I; a.sub = (int)I;
    a.C = f->y_perm; a.ldc = d;                      // Y_perm in bf16 (the MX layer's error dwarfs its rounding)
    Probe pr(p, "gemm_down", s);
    MOE_TRY(launch_row_gemm(DT_MXFP8, OP_DOWN_FWD, EPI_STORE, p->t_down, a, s));
  }
  if (p->Ns > 0) {
    const int64_t Is = p->Is, NI = p->Ns * p->Is, T = p->T;
    const MxOp sxq = mxop(ws, p->mx_sxq), shq = mxop(ws, p->mx_shq), swgu = mxop(ws, p->mx_swgu),
               swd = mxop(ws, p->mx_swd);
    if (!gather) MOE_TRY_STATUS(mx_rows(p, s, f->x, d, 0, (int)d, T, (int)d, sxq));
    if (sv) {   // W_sgu[s] [2Is][d]: rows s 2Is.. of [2 NI][d], and K positions s 2Is.. of [d][2 NI]
      for (int sh = 0; sh < p->Ns; ++sh)
        MOE_TRY_STATUS(mx_cols(p, s, static_cast<const char*>(f->ws_gate_up) + (int64_t)sh * 2 * Is * d * 2, d,
                               (int)d, nullptr, nullptr, 1, (int)(2 * Is), 2 * Is / 32, sh * 2 * Is, 2 * NI, 0,
                               svop(sv, p->sv_swgut), nullptr,
                               {swgu.pay + sh * 2 * Is * d, swgu.sc + sh * 2 * Is * (d / 32)}, d));
    } else {
      MOE_TRY_STATUS(mx_rows(p, s, f->ws_gate_up, d, 0, (int)d, 2 * NI, (int)d, swgu));
    }
    {
      RowGemmArgs a{};
      mx_pq(a, sxq, d, swgu, d, 0);
      a.offsets = nullptr; a.G = 1; a.M = T; a.N = (int)NI; a.K = (int)d; a.sub = (int)Is;
      a.C = f->gu_shared; a.ldc = 2 * NI; a.C2 = f->h_shared; a.ldc2 = NI;
      a.Hq = shq.pay; a.Hs = shq.sc;                 // the epilogue also quantises H row-wise
      if (sv) {                                      // and along the T tokens, for dWs_d
        const MxOp sht = svop(sv, p->sv_sht);
        a.Tq = sht.pay; a.Ts = sht.sc; a.ldt = p->Tpad;
      }
      Probe pr(p, "gemm_gate_up_swiglu_shared", s);
      MOE_TRY(launch_row_gemm(DT_MXFP8, OP_GU_FWD, EPI_SWIGLU_FWD, p->t_gu_s, a, s));
    }
    // shared down weights [Ns][d][Is] concatenated along K into [d][NI]
    if (sv) {   // W_sd[s] [d][Is]: columns s Is.. of [d][NI], and rows s Is.. of [NI][d]
      for (int sh = 0; sh < p->Ns; ++sh)
        MOE_TRY_STATUS(mx_cols(p, s, static_cast<const char*>(f->ws_down) + (int64_t)sh * d * Is * 2, Is, (int)Is,
                               nullptr, nullptr, 1, (int)d, d / 32, 0, d, sh * Is, svop(sv, p->sv_swdt), nullptr,
                               {swd.pay + sh * Is, swd.sc + sh * Is / 32}, NI));
    } else {
      MOE_TRY_STATUS(mx_rows(p, s, f->ws_down, Is, d * Is, (int)Is, d, (int)NI, swd));
    }
    {
      RowGemmArgs a{};
      mx_pq(a, shq, NI, swd, NI, 0);
      a.offsets = nullptr; a.G = 1; a.M = T; a.N = (int)d; a.K = (int)NI; a.sub = (int)Is;
      a.C = f->y_shared; a.ldc = d;
      Probe pr(p, "gemm_down_shared", s);
      MOE_TRY(launch_row_gemm(DT_MXFP8, OP_DOWN_FWD, EPI_STORE, p->t_down_s, a, s));
    }
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- combine --
moe_status moe_combine(moe_plan p, const void* y_perm, const int32_t* inv_perm, const float* topk_w,
                       const void* y_shared, void* y, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (p->T == 0) return MOE_OK;
  if (!y_perm || !inv_perm || !topk_w || !y) return MOE_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  CombineArgs a{y_perm, inv_perm, topk_w, y_shared, y, p->T, p->d, p->k,
                p->dt == DT_F32 || f32_intermediates(p->dt, p->mx)};
  Probe pr(p, "combine", s);
  return hip_status(launch_combine(p->dt, a, s));
}

// --------------------------------------------------------------- backward --
// MX-fp8 backward of the experts (routed and shared): both dgrad GEMMs, both
// weight gradients, each operand quantised along its GEMM's reduction axis --
// the weight gradients' along the tokens of each expert segment.
moe_status mx_backward_experts(moe_plan p, const moe_saved* sv, const void* dy, const moe_grads* gr, void* ws,
                               hipStream_t s, void* dy_perm, void* dgu, void* dx_perm, void* dgu_s, void* dxs) {
  const int64_t d = p->d, I = p->I, E = p->E, A = p->A, T = p->T, Apad = p->Apad;
  int32_t* pad = reinterpret_cast<int32_t*>(wsp(ws, p->o_mx_pad));
  // the weights' and H's codes from the forward's saved-codes buffer, if given
  const void* svb = sv->mx_saved;
  const MxOp dyq = mxop(ws, p->mx_dyq), dguq = mxop(ws, p->mx_dguq), dyt = mxop(ws, p->mx_dyt),
             dgut = mxop(ws, p->mx_dgut), xt = mxop(ws, p->mx_xt),
             wdt = svb ? svop(svb, p->sv_wdt) : mxop(ws, p->mx_wdt),
             wgut = svb ? svop(svb, p->sv_wgut) : mxop(ws, p->mx_wgut),
             ht = svb ? svop(svb, p->sv_ht) : mxop(ws, p->mx_ht);
  {
    Probe pr(p, "mx_quantize", s);
    MOE_TRY(launch_mx_pad_offsets(sv->offsets, pad, (int)E, 128, s));
  }
  if (T > 0) {
    // dH = dY_perm W_d (reduction over d): W_d [E][d][I] transposed to [I][E d]
    // dY_perm: its row-wise codes came from the combine backward; token blocks for dW_d,
    // from dy's rows gathered by perm_token and scaled by their routing weights
    // (the combine backward wrote those, not the rows), else from the stored rows
    if (sv->perm_token)
      MOE_TRY_STATUS(mx_cols(p, s, dy, d, (int)d, sv->offsets, pad, (int)E, 0, Apad / 32, 0, Apad, 0, dyt,
                             sv->perm_token, {nullptr, nullptr}, 0,
                             reinterpret_cast<const float*>(wsp(ws, p->o_wsorted))));
    else
      MOE_TRY_STATUS(mx_cols(p, s, dy_perm, d, (int)d, sv->offsets, pad, (int)E, 0, Apad / 32, 0, Apad, 0, dyt));
    if (!svb)
      MOE_TRY_STATUS(mx_cols(p, s, sv->w_down, I, (int)I, nullptr, nullptr, (int)E, (int)d, E * d / 32, 0, E * d, 0,
                             wdt));
    RowGemmArgs a{};
    mx_pq(a, dyq, d, wdt, E * d, d);
    a.offsets = sv->offsets; a.G = (int)E; a.M = A; a.N = (int)I; a.K = (int)d; a.sub = (int)I;
    a.C = p->keep_inter ? dgu : nullptr; a.ldc = 2 * I; a.aux = sv->gu; a.ldaux = 2 * I;
    a.Hq = dguq.pay; a.Hs = dguq.sc;                 // the epilogue writes [dG | dU] row-wise
    a.Tq = dgut.pay; a.Ts = dgut.sc; a.tpad = pad; a.ldt = Apad;   // and along the tokens, for dW_gu
    Probe pr(p, "gemm_down_dgrad_swiglu", s);
    MOE_TRY(launch_row_gemm(DT_MXFP8, OP_DOWN_DGRAD, EPI_SWIGLU_BWD, 128, a, s));
  }
  {
    // dW_d[e] = dY_perm[seg]^T H[seg]: token axis blocked per segment (dY_perm's done above)
    if (!svb) MOE_TRY_STATUS(mx_cols(p, s, sv->h, I, (int)I, sv->offsets, pad, (int)E, 0, Apad / 32, 0, Apad, 0, ht));
    WgradArgs a{};
    a.P = dyt.pay; a.Ps = dyt.sc; a.ldp = Apad; a.Q = ht.pay; a.Qs = ht.sc; a.ldq = Apad;
    a.offsets = pad; a.G = (int)E; a.Mtok = Apad; a.M = (int)d; a.N = (int)I; a.sub = (int)I;
    MOE_TRY_STATUS(run_wgrad(p, WG_DOWN, p->t_wg_down, p->sp_wg_down, a, gr->dw_down, d * I, ws, "gemm_wgrad_down", s,
                             DT_MXFP8));
  }
  if (T > 0) {
    // dX_perm = [dG | dU] W_gu (reduction over 2I): W_gu [E][2I][d] transposed to [d][E 2I]
    // [dG | dU]: row-wise and token-axis codes from the SwiGLU-backward epilogue
    if (!svb)
      MOE_TRY_STATUS(mx_cols(p, s, sv->w_gate_up, d, (int)d, nullptr, nullptr, (int)E, (int)(2 * I), E * 2 * I / 32,
                             0, E * 2 * I, 0, wgut));
    RowGemmArgs a{};
    mx_pq(a, dguq, 2 * I, wgut, E * 2 * I, 2 * I);
    a.offsets = sv->offsets; a.G = (int)E; a.M = A; a.N = (int)d; a.K = (int)(2 * I); a.sub = (int)I;
    a.C = dx_perm; a.ldc = d;
    Probe pr(p, "gemm_gate_up_dgrad", s);
    MOE_TRY(launch_row_gemm(DT_MXFP8, OP_GU_DGRAD, EPI_STORE, p->t_gu_dgrad, a, s));
  }
  {
    if (sv->perm_token)                        // x's rows gathered by perm_token (x_perm not read)
      MOE_TRY_STATUS(mx_cols(p, s, sv->x, d, (int)d, sv->offsets, pad, (int)E, 0, Apad / 32, 0, Apad, 0, xt,
                             sv->perm_token));
    else
      MOE_TRY_STATUS(mx_cols(p, s, sv->x_perm, d, (int)d, sv->offsets, pad, (int)E, 0, Apad / 32, 0, Apad, 0, xt));
    WgradArgs a{};
    a.P = dgut.pay; a.Ps = dgut.sc; a.ldp = Apad; a.Q = xt.pay; a.Qs = xt.sc; a.ldq = Apad;
    a.offsets = pad; a.G = (int)E; a.Mtok = Apad; a.M = (int)(2 * I); a.N = (int)d; a.sub = (int)d;
    MOE_TRY_STATUS(run_wgrad(p, WG_GATE_UP, p->t_wg_gu, p->sp_wg_gu, a, gr->dw_gate_up, 2 * I * d, ws,
                             "gemm_wgrad_gate_up", s, DT_MXFP8));
  }
  if (p->Ns > 0) {
    const int64_t Is = p->Is, NI = p->Ns * p->Is, Tpad = p->Tpad;
    int32_t* seg_pad = reinterpret_cast<int32_t*>(wsp(ws, p->o_mx_seg1));   // {0, T} then {0, Tpad}
    const MxOp sdyq = mxop(ws, p->mx_sdyq), sdguq = mxop(ws, p->mx_sdguq), sdyt = mxop(ws, p->mx_sdyt),
               sdgut = mxop(ws, p->mx_sdgut), sxt = mxop(ws, p->mx_sxt),
               swdt = svb ? svop(svb, p->sv_swdt) : mxop(ws, p->mx_swdt),
               swgut = svb ? svop(svb, p->sv_swgut) : mxop(ws, p->mx_swgut),
               sht = svb ? svop(svb, p->sv_sht) : mxop(ws, p->mx_sht);
    {
      Probe pr(p, "mx_quantize", s);
      MOE_TRY(launch_mx_single_segment(seg_pad, T, 128, s));
    }
    if (T > 0) {
      // dY's row-wise codes (sdyq) came from the combine backward
      for (int sh = 0; sh < p->Ns && !svb; ++sh)   // W_sd[s] [d][Is] -> rows s Is.. of [NI][d]
        MOE_TRY_STATUS(mx_cols(p, s, static_cast<const char*>(sv->ws_down) + (int64_t)sh * d * Is * 2, Is, (int)Is,
                               nullptr, nullptr, 1, (int)d, d / 32, 0, d, sh * Is, swdt));
      RowGemmArgs a{};
      mx_pq(a, sdyq, d, swdt, d, 0);
      a.offsets = nullptr; a.G = 1; a.M = T; a.N = (int)NI; a.K = (int)d; a.sub = (int)Is;
      a.C = p->keep_inter ? dgu_s : nullptr; a.ldc = 2 * NI; a.aux = sv->gu_shared; a.ldaux = 2 * NI;
      a.Hq = sdguq.pay; a.Hs = sdguq.sc;             // the epilogue writes [dG | dU] row-wise
      a.Tq = sdgut.pay; a.Ts = sdgut.sc; a.ldt = Tpad;   // and along the tokens (one segment), for dWs_gu
      Probe pr(p, "gemm_down_dgrad_swiglu_shared", s);
      MOE_TRY(launch_row_gemm(DT_MXFP8, OP_DOWN_DGRAD, EPI_SWIGLU_BWD, 128, a, s));
    }
    {
      MOE_TRY_STATUS(mx_cols(p, s, dy, d, (int)d, seg_pad, seg_pad + 2, 1, 0, Tpad / 32, 0, Tpad, 0, sdyt));
      if (!svb)
        MOE_TRY_STATUS(mx_cols(p, s, sv->h_shared, NI, (int)NI, seg_pad, seg_pad + 2, 1, 0, Tpad / 32, 0, Tpad, 0,
                               sht));
      WgradArgs a{};
      a.P = sdyt.pay; a.Ps = sdyt.sc; a.ldp = Tpad; a.Q = sht.pay; a.Qs = sht.sc; a.ldq = Tpad;
      a.offsets = seg_pad + 2; a.G = 1; a.Mtok = Tpad; a.M = (int)d; a.N = (int)NI; a.sub = (int)Is;
      MOE_TRY_STATUS(run_wgrad(p, WG_DOWN, p->t_wg_down_s, p->sp_wg_down_s, a, gr->dws_down, d * NI, ws,
                               "gemm_wgrad_down_shared", s, DT_MXFP8));
    }
    {
      MOE_TRY_STATUS(mx_cols(p, s, sv->x, d, (int)d, seg_pad, seg_pad + 2, 1, 0, Tpad / 32, 0, Tpad, 0, sxt));
      WgradArgs a{};
      a.P = sdgut.pay; a.Ps = sdgut.sc; a.ldp = Tpad; a.Q = sxt.pay; a.Qs = sxt.sc; a.ldq = Tpad;
      a.offsets = seg_pad + 2; a.G = 1; a.Mtok = Tpad; a.M = (int)(2 * NI); a.N = (int)d; a.sub = (int)d;
      MOE_TRY_STATUS(run_wgrad(p, WG_GATE_UP, p->t_wg_gu_s, p->sp_wg_gu_s, a, gr->dws_gate_up, 2 * NI * d, ws,
                               "gemm_wgrad_gate_up_shared", s, DT_MXFP8));
    }
    if (T > 0) {
      for (int sh = 0; sh < p->Ns && !svb; ++sh)   // W_sgu[s] [2Is][d] -> K positions s 2Is.. of [d][2 NI]
        MOE_TRY_STATUS(mx_cols(p, s, static_cast<const char*>(sv->ws_gate_up) + (int64_t)sh * 2 * Is * d * 2, d,
                               (int)d, nullptr, nullptr, 1, (int)(2 * Is), 2 * Is / 32, sh * 2 * Is, 2 * NI, 0, swgut));
      RowGemmArgs a{};
      mx_pq(a, sdguq, 2 * NI, swgut, 2 * NI, 0);
      a.offsets = nullptr; a.G = 1; a.M = T; a.N = (int)d; a.K = (int)(2 * NI); a.sub = (int)d;
      a.C = dxs; a.ldc = d;
      Probe pr(p, "gemm_gate_up_dgrad_shared", s);
      MOE_TRY(launch_row_gemm(DT_MXFP8, OP_GU_DGRAD, EPI_STORE, p->t_gu_dgrad_s, a, s));
    }
  }
  return MOE_OK;
}

moe_status moe_backward(moe_plan p, const moe_saved* sv, const void* dy, const moe_grads* gr, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!p || !sv || !gr) return MOE_ERR_NULL;
  if (!gr->dw_router || !gr->dw_gate_up || !gr->dw_down) return MOE_ERR_NULL;
  if (!sv->offsets) return MOE_ERR_NULL;
  if (p->Ns > 0 && (!gr->dws_gate_up || !gr->dws_down)) return MOE_ERR_NULL;
  if (p->T > 0) {
    if (!dy || !gr->dx || !sv->x || !sv->w_router || !sv->probs || !sv->topk_idx || !sv->topk_w ||
        !sv->counts || !sv->inv_perm || (!sv->x_perm && !(p->mx && sv->perm_token)) || !sv->gu ||
        (!sv->h && !(p->mx && sv->mx_saved)) ||
        (!p->mx && !sv->perm_token) ||
        !sv->y_perm ||
        !sv->w_gate_up || !sv->w_down)
      return MOE_ERR_NULL;
    if (p->Ns > 0 &&
        (!sv->ws_gate_up || !sv->ws_down || !sv->gu_shared || (!sv->h_shared && !(p->mx && sv->mx_saved))))
      return MOE_ERR_NULL;
    if (sv->real_mask && !sv->real_counts) return MOE_ERR_NULL;
    if (p->fused && (!sv->perm_token || !sv->mx_saved)) return MOE_ERR_NULL;   // the fused path only
  } else if (!sv->w_router || !sv->w_gate_up || !sv->w_down) {
    return MOE_ERR_NULL;
  }
  moe_status st = check_ws(p, ws, ws_bytes);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = p->d, I = p->I, E = p->E, k = p->k, Ep = p->Ep;
  void* dy_perm = wsp(ws, p->o_dy_perm);
  float* g = reinterpret_cast<float*>(wsp(ws, p->o_g));
  void* dzhl = wsp(ws, p->o_dzhl);
  void* w2 = wsp(ws, p->o_w2);
  void* dgu = wsp(ws, p->o_dgu);
  void* dx_perm = wsp(ws, p->o_dx_perm);
  void* dgu_s = wsp(ws, p->o_dgu_s);
  void* dxs = wsp(ws, p->o_dxs);
  float* dxr = reinterpret_cast<float*>(wsp(ws, p->o_dxr));
  float* dwr_part = reinterpret_cast<float*>(wsp(ws, p->o_dwr_part));
  float* dbias_part = reinterpret_cast<float*>(wsp(ws, p->o_dbias_part));

  float* wsorted = reinterpret_cast<float*>(wsp(ws, p->o_wsorted));
  float* gpart = reinterpret_cast<float*>(wsp(ws, p->o_gpart));
  void* wh = wsp(ws, p->o_wh);
  void* dgu_lo = wsp(ws, p->o_dgu_lo);
  void* wh_lo = wsp(ws, p->o_wh_lo);
  if (p->T > 0) {
    {
      // dY_perm = w dy at each assignment's row; MX-fp8 experts also take the
      // routing-weight gradient g = <dy, Y_perm> here (their Y_perm is the
      // quantised forward's), the others the per-row weights (the down
      // dgrad forms g from dy W_d and the saved G, U)
      CombineBwdArgs a{dy, sv->y_perm, sv->inv_perm, sv->topk_w, dy_perm,
                       p->mx ? g : nullptr, p->T, d, k};
      if (!p->mx) a.wsorted = wsorted;
      if (p->mx && sv->perm_token) {                 // MX: dY_perm's token-axis codes gather dy (see there)
        a.wsorted = wsorted;
        a.no_rows = p->keep_inter ? 0 : 1;
      }
      if (wh_rows(p)) a.copy = 1;                    // the routing weight goes on the H side
      if (p->mx) {                                   // MX experts: dY_perm's row-wise codes too
        const MxOp dyq = mxop(ws, p->mx_dyq);
        a.q = dyq.pay;
        a.qs = dyq.sc;
        if (p->Ns > 0) {                             // and dY's, for the shared experts
          const MxOp sdyq = mxop(ws, p->mx_sdyq);
          a.dq = sdyq.pay;
          a.dqs = sdyq.sc;
        }
      }
      Probe pr(p, "combine_bwd", s);
      MOE_TRY(launch_combine_bwd(p->dt, a, s));
    }
    if (!p->mx) {
      // dH = w (dy W_d) on dy's rows gathered by perm_token, the SwiGLU
      // backward, and the partial row sums of (dy W_d) * H for g
      RowGemmArgs a{};
      a.P = dy; a.ldp = d; a.gather = sv->perm_token; a.p_rows = p->T;
      a.Q = sv->w_down; a.ldq = I; a.q_group_stride = (int64_t)d * I;
      a.offsets = sv->offsets; a.G = E; a.M = p->A; a.N = I; a.K = d; a.sub = I;
      a.C = dgu; a.ldc = 2 * I; a.aux = sv->gu; a.ldaux = 2 * I;
      a.wrow = wsorted; a.gpart = gpart; a.gparts = p->gparts;
      if (wh_rows(p)) { a.C2 = wh; a.ldc2 = I; }      // w H, the down weight gradient's operand
      if (p->comp) { a.C_lo = dgu_lo; a.C2_lo = wh_lo; }
      Probe pr(p, "gemm_down_dgrad_swiglu", s);
      MOE_TRY(launch_row_gemm(p->dt, OP_DOWN_DGRAD, EPI_SWIGLU_BWD, p->t_down_dgrad, a, s));
    }
    const float* gp = p->mx ? nullptr : gpart;
    if (p->router_small) {
      RouterBwdSmallArgs a{g, sv->topk_w, sv->topk_idx, sv->probs, sv->counts, sv->x, dzhl, dwr_part, dbias_part,
                           p->T, E, Ep, d, k, p->cfg.renorm, p->cfg.aux_coef, sv->real_mask, sv->real_counts};
      a.gpart = gp; a.inv = sv->inv_perm; a.gparts = p->gparts; a.relu = p->cfg.router == MOE_ROUTER_RELU;
      Probe pr(p, "router_bwd_small", s);
      MOE_TRY(launch_router_bwd_small(p->dt, a, s));
    } else {
      RouterDzArgs a{g, sv->topk_w, sv->topk_idx, sv->probs, sv->counts, dzhl, dbias_part,
                     p->T, E, Ep, k, p->cfg.renorm, p->cfg.aux_coef, sv->real_mask, sv->real_counts};
      a.gpart = gp; a.inv = sv->inv_perm; a.gparts = p->gparts; a.relu = p->cfg.router == MOE_ROUTER_RELU;
      Probe pr(p, "router_dz", s);
      MOE_TRY(launch_router_dz(p->dt, a, s));
    }
  }
  if (!p->mx) {
    // dW_d[e] = sum over the expert's rows of dy[t] (w H)[r]: dy is the
    // caller's own values, w H is rounded once (f16: (w dy)[r] H[r])
    WgradArgs a{};
    a.P = dy_perm; a.ldp = d; a.Q = wh_rows(p) ? wh : sv->h; a.ldq = I;
    a.offsets = sv->offsets; a.G = E; a.Mtok = p->A; a.M = d; a.N = I; a.sub = I;
    MOE_TRY_STATUS(run_wgrad(p, WG_DOWN, p->t_wg_down, p->sp_wg_down, a, gr->dw_down, (int64_t)d * I, ws,
                             "gemm_wgrad_down", s, -1, nullptr, p->comp ? wh_lo : nullptr));
  }
  if (p->T > 0 && !p->mx) {
    RowGemmArgs a{};
    a.P = dgu; a.ldp = 2 * I;
    a.Q = sv->w_gate_up; a.ldq = d; a.q_group_stride = (int64_t)2 * I * d;
    a.offsets = sv->offsets; a.G = E; a.M = p->A; a.N = d; a.K = 2 * I; a.sub = I;
    a.C = dx_perm; a.ldc = d;                         // f32 rows in a bf16 layer
    Probe pr(p, "gemm_gate_up_dgrad", s);
    MOE_TRY(launch_row_gemm(p->dt, OP_GU_DGRAD, f32_intermediates(p->dt, p->mx) ? EPI_STORE_F32 : EPI_STORE,
                            p->t_gu_dgrad, a, s));
  }
  if (!p->mx) {
    WgradArgs a{};
    a.P = dgu; a.ldp = 2 * I; a.Q = sv->x_perm; a.ldq = d;
    a.offsets = sv->offsets; a.G = E; a.Mtok = p->A; a.M = 2 * I; a.N = d; a.sub = d;
    MOE_TRY_STATUS(run_wgrad(p, WG_GATE_UP, p->t_wg_gu, p->sp_wg_gu, a, gr->dw_gate_up, (int64_t)2 * I * d, ws,
                             "gemm_wgrad_gate_up", s, -1, p->comp ? dgu_lo : nullptr));
  }
  if (p->Ns > 0 && !p->mx) {
    const int Is = p->Is, NI = p->Ns * p->Is;
    if (p->T > 0) {
      RowGemmArgs a{};
      a.P = dy; a.ldp = d;
      a.Q = sv->ws_down; a.ldq = Is; a.q_group_stride = 0;
      a.offsets = nullptr; a.G = 1; a.M = p->T; a.N = NI; a.K = d; a.sub = Is;
      a.C = dgu_s; a.ldc = 2 * NI; a.aux = sv->gu_shared; a.ldaux = 2 * NI;
      Probe pr(p, "gemm_down_dgrad_swiglu_shared", s);
      MOE_TRY(launch_row_gemm(p->dt, OP_DOWN_DGRAD, EPI_SWIGLU_BWD, p->t_down_dgrad_s, a, s));
    }
    {
      WgradArgs a{};
      a.P = dy; a.ldp = d; a.Q = sv->h_shared; a.ldq = NI;
      a.offsets = nullptr; a.G = 1; a.Mtok = p->T; a.M = d; a.N = NI; a.sub = Is;
      MOE_TRY_STATUS(run_wgrad(p, WG_DOWN, p->t_wg_down_s, p->sp_wg_down_s, a, gr->dws_down, (int64_t)d * NI, ws,
                               "gemm_wgrad_down_shared", s));
    }
    {
      WgradArgs a{};
      a.P = dgu_s; a.ldp = 2 * NI; a.Q = sv->x; a.ldq = d;
      a.offsets = nullptr; a.G = 1; a.Mtok = p->T; a.M = 2 * NI; a.N = d; a.sub = d;
      MOE_TRY_STATUS(run_wgrad(p, WG_GATE_UP, p->t_wg_gu_s, p->sp_wg_gu_s, a, gr->dws_gate_up, (int64_t)2 * NI * d,
                               ws, "gemm_wgrad_gate_up_shared", s));
    }
  }
  if (p->mx) MOE_TRY_STATUS(mx_backward_experts(p, sv, dy, gr, ws, s, dy_perm, dgu, dx_perm, dgu_s, dxs));
  if (p->Ns > 0 && p->T > 0 && !p->mx) {
    const int NI = p->Ns * p->Is;
    RowGemmArgs b{};
    b.P = dgu_s; b.ldp = 2 * NI;
    b.Q = sv->ws_gate_up; b.ldq = d; b.q_group_stride = 0;
    b.offsets = nullptr; b.G = 1; b.M = p->T; b.N = d; b.K = 2 * NI; b.sub = d;
    b.C = dxs; b.ldc = d;                             // f32 rows in a bf16 layer
    Probe pr(p, "gemm_gate_up_dgrad_shared", s);
    MOE_TRY(launch_row_gemm(p->dt, OP_GU_DGRAD, f32_intermediates(p->dt, p->mx) ? EPI_STORE_F32 : EPI_STORE,
                            p->t_gu_dgrad_s, b, s));
  }
  if (p->router_dx_gemm && p->T > 0) {
    {
      Stack2Args a{sv->w_router, w2, E, Ep, d};
      Probe pr(p, "stack_router", s);
      MOE_TRY(launch_stack2(p->dt, a, s));
    }
    RowGemmArgs a{};
    a.P = dzhl; a.ldp = 2 * Ep;
    a.Q = w2; a.ldq = d; a.q_group_stride = 0;
    a.offsets = nullptr; a.G = 1; a.M = p->T; a.N = d; a.K = 2 * Ep; a.sub = d;
    a.C = dxr; a.ldc = d;
    Probe pr(p, "gemm_router_dx", s);
    MOE_TRY(launch_row_gemm(p->dt, OP_ROUTER_DX, EPI_STORE_F32, p->t_router_dx, a, s));
  }
  if (p->T > 0) {
    UnpermuteArgs a{dx_perm, sv->inv_perm, p->Ns > 0 ? dxs : nullptr, p->router_dx_gemm ? dxr : nullptr,
                    dzhl, sv->w_router, gr->dx, p->T, d, k, E, Ep};
    a.src_f32 = f32_intermediates(p->dt, p->mx) ? 1 : 0;
    Probe pr(p, "unpermute", s);
    MOE_TRY(launch_unpermute(p->dt, a, s));
  }
  if (!p->router_small) {
    WgradArgs a{};
    a.P = dzhl; a.ldp = 2 * Ep; a.Q = sv->x; a.ldq = d;
    a.offsets = nullptr; a.G = 1; a.Mtok = p->T; a.M = 2 * Ep; a.N = d; a.splits = p->router_splits;
    a.C = dwr_part; a.c_group_stride = 0; a.c_split_stride = (int64_t)2 * Ep * d; a.sub = d; a.out_f32 = 1;
    Probe pr(p, "gemm_wgrad_router", s);
    MOE_TRY(launch_wgrad(p->dt, WG_ROUTER, p->t_wg_router, a, s));
  }
  {
    const int nsm = p->T > 0 ? p->nblk_small : 0;
    RouterReduceArgs a = p->router_small
        ? RouterReduceArgs{dwr_part, nsm, E, E, -1, d, gr->dw_router, dbias_part, nsm, gr->dbias}
        : RouterReduceArgs{dwr_part, p->router_splits, E, 2 * Ep, Ep, d, gr->dw_router,
                           dbias_part, p->T > 0 ? p->nblk_dz : 0, gr->dbias};
    Probe pr(p, "router_reduce", s);
    MOE_TRY(launch_router_reduce(p->dt, a, s));
  }
  return MOE_OK;
}

// -------------------------------------------------------------- aux stats --
moe_status moe_aux_stats(moe_plan p, const float* probs, const int32_t* counts, float* f, float* p_mean,
                         moe_aux_scalars* out, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (!counts || !f || !p_mean || !out) return MOE_ERR_NULL;
  if (p->T > 0 && !probs) return MOE_ERR_NULL;
  moe_status st = check_ws(p, ws, ws_bytes);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  AuxArgs a{probs, counts, f, p_mean, out, reinterpret_cast<float*>(wsp(ws, p->o_aux_part)), p->T, p->E, p->k};
  a.kf = p->kf;
  Probe pr(p, "aux", s);
  return hip_status(launch_aux(a, s));
}

moe_status moe_aux_stats_masked(moe_plan p, const float* probs, const int32_t* topk_idx, const int32_t* real_mask,
                                float* f, float* p_mean, int32_t* real_counts, moe_aux_scalars* out, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!p) return MOE_ERR_NULL;
  if (!f || !p_mean || !real_counts || !out) return MOE_ERR_NULL;
  if (p->T > 0 && (!probs || !topk_idx || !real_mask)) return MOE_ERR_NULL;
  moe_status st = check_ws(p, ws, ws_bytes);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = reinterpret_cast<float*>(wsp(ws, p->o_aux_part));
  const int nb = p->nblk_aux > 0 ? p->nblk_aux : 1;
  AuxArgs a{probs, nullptr, f, p_mean, out, part, p->T, p->E, p->k};
  a.kf = p->kf;
  a.mask = real_mask;
  a.idx = topk_idx;
  a.rcounts = real_counts;
  a.cpart = reinterpret_cast<int32_t*>(part + (size_t)nb * 2 * p->E);
  Probe pr(p, "aux", s);
  return hip_status(launch_aux(a, s));
}

// ------------------------------------------------------------------ probe --
moe_status moe_mx_quantize_rows(const void* in, int32_t act_dtype, int64_t rows, int32_t K, uint8_t* payload,
                                uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID;
  if (act_dtype != MOE_BF16 && act_dtype != MOE_F16) return MOE_ERR_INVALID;
  if (rows == 0) return MOE_OK;
  if (!in || !payload || !scales) return MOE_ERR_NULL;
  MxRowsArgs a{in, K, 0, K, rows, K, payload, scales};
  return hip_status(launch_mx_quant_rows(act_dtype == MOE_F16 ? DT_F16 : DT_BF16, a, static_cast<hipStream_t>(stream)));
}

moe_status moe_probe_enable(moe_plan p, const char* kernel, int max_launches) {
  if (!p) return MOE_ERR_NULL;
  p->release_events();
  p->probe_name.clear();
  if (max_launches <= 0) return MOE_OK;
  if (!kernel) return MOE_ERR_NULL;
  const std::string name(kernel);
  // accept only names from the list
  const std::string all = std::string(",") + kKernelNames + ",";
  if (all.find("," + name + ",") == std::string::npos) return MOE_ERR_INVALID;
  if (max_launches > 100000) return MOE_ERR_INVALID;
  p->ev0.resize(max_launches);
  p->ev1.resize(max_launches);
  for (int i = 0; i < max_launches; ++i) {
    if (hipEventCreate(&p->ev0[i]) != hipSuccess || hipEventCreate(&p->ev1[i]) != hipSuccess) {
      p->ev0.resize(i);
      p->ev1.resize(i);
      p->release_events();
      return MOE_ERR_HIP;
    }
  }
  p->probe_name = name;
  p->probe_n = 0;
  return MOE_OK;
}

moe_status moe_mx_saved_region(moe_plan p, const char* name, size_t* offset, size_t* bytes) {
  if (!p || !name || !offset || !bytes) return MOE_ERR_NULL;
  if (!p->mx) return MOE_ERR_INVALID;
  const std::string n(name);
  const bool sc = n.size() > 7 && n.compare(n.size() - 7, 7, ".scales") == 0;
  const std::string base = sc ? n.substr(0, n.size() - 7) : n;
  const int64_t d = p->d, I = p->I, E = p->E, NI = (int64_t)p->Ns * p->Is;
  struct Entry { const char* name; const moe_plan_s::MxBuf* buf; int64_t rows, K; bool shared; };
  const Entry tab[] = {
      {"mx_wdt", &p->sv_wdt, I, E * d, false},      {"mx_wgut", &p->sv_wgut, d, E * 2 * I, false},
      {"mx_ht", &p->sv_ht, I, p->Apad, false},      {"mx_swdt", &p->sv_swdt, NI, d, true},
      {"mx_swgut", &p->sv_swgut, d, 2 * NI, true}, {"mx_sht", &p->sv_sht, NI, p->Tpad, true},
  };
  for (const Entry& t : tab) {
    if (base != t.name) continue;
    if (t.shared && p->Ns == 0) return MOE_ERR_INVALID;
    *offset = sc ? t.buf->sc : t.buf->pay;
    *bytes = (size_t)t.rows * (sc ? t.K / 32 : t.K);
    return MOE_OK;
  }
  return MOE_ERR_INVALID;
}

moe_status moe_keep_intermediates(moe_plan p, int keep) {
  if (!p) return MOE_ERR_NULL;
  if (p->fused && keep) return MOE_ERR_UNSUPPORTED;        // no room for the rows in its workspace
  p->keep_inter = keep != 0;
  return MOE_OK;
}

moe_status moe_probe_read(moe_plan p, float* total_ms, int* launches) {
  if (!p || !total_ms || !launches) return MOE_ERR_NULL;
  float tot = 0.0f;
  for (int i = 0; i < p->probe_n; ++i) {
    if (hipEventSynchronize(p->ev1[i]) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, p->ev0[i], p->ev1[i]) != hipSuccess) return MOE_ERR_HIP;
    tot += ms;
  }
  *total_ms = tot;
  *launches = p->probe_n;
  p->probe_n = 0;
  return MOE_OK;
}

}  // extern "C"
