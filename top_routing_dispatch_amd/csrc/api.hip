// C ABI of the MoE layer library: argument validation, workspace carving and
// the launch sequence of each entry point.  Declarations and the contract of
// every function are in include/moe.h.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "common.h"
#include "moe.h"

using namespace moe;

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char* where, hipError_t e) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
}

moe_status hip_status(const char* where, hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  set_error(where, e);
  (void)hipGetLastError();   // clear the sticky launch error
  return MOE_ERR_HIP;
}

bool debug_on() { return tuning().debug > 0; }

#define MOE_TRY_HIP(where, expr)                        \
  do {                                                  \
    const moe_status _st = hip_status(where, (expr));   \
    if (_st != MOE_OK) return _st;                      \
  } while (0)
#define MOE_TRY(expr)                                   \
  do {                                                  \
    const moe_status _st = (expr);                      \
    if (_st != MOE_OK) return _st;                      \
  } while (0)

// MOE_DEBUG=1: device tables copied to the host and checked before going on.
template <typename T>
moe_status to_host(const T* dev, size_t n, std::vector<T>* out, hipStream_t s) {
  out->assign(n, T());
  if (n == 0) return MOE_OK;
  MOE_TRY_HIP("debug copy", hipMemcpyAsync(out->data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, s));
  MOE_TRY_HIP("debug copy", hipStreamSynchronize(s));
  return MOE_OK;
}

moe_status debug_fail(const char* where, const char* msg) {
  debug_message(where, msg);
  return MOE_ERR_DEBUG_CHECK;
}

moe_status debug_check_dispatch(const char* where, const moe_config* c, int capacity, int rows_cap,
                                const int32_t* idx, const int32_t* counts, const int32_t* offsets,
                                const int32_t* row_of, const int32_t* tor, hipStream_t s) {
  const int T = c->num_tokens, k = c->top_k, E = c->num_experts;
  std::vector<int32_t> hi, hc, ho, hr, ht;
  MOE_TRY(to_host(idx, (size_t)T * k, &hi, s));
  MOE_TRY(to_host(counts, (size_t)E, &hc, s));
  MOE_TRY(to_host(offsets, (size_t)E + 1, &ho, s));
  MOE_TRY(to_host(row_of, (size_t)T * k, &hr, s));
  MOE_TRY(to_host(tor, (size_t)rows_cap, &ht, s));
  char msg[200];
  if (!check_dispatch(hi.data(), hc.data(), ho.data(), hr.data(), ht.data(), T, k, E, capacity, rows_cap, msg,
                      sizeof(msg)))
    return debug_fail(where, msg);
  return MOE_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool opt_aligned(const void* p) { return p == nullptr || aligned16(p); }
inline size_t esize(int dt) { return dt == BF16 ? 2 : 4; }
inline size_t carve(size_t bytes) { return round_up(bytes, 256); }

struct Derived {
  int capacity;     // INT32_MAX when dropless
  int rows_cap;     // A_cap
  int group_rows;   // bound on one expert's rows: a token gives an expert at most one row
};

moe_status derive(const moe_config* c, Derived* d) {
  const long long A = (long long)c->num_tokens * c->top_k;
  if (c->capacity_factor > 0.0f) {
    const double C = ceil((double)c->capacity_factor * (double)A / (double)c->num_experts);
    d->capacity = C >= 2147483647.0 ? INT32_MAX : (int)C;
    const long long ec = (long long)c->num_experts * d->capacity;
    d->rows_cap = (int)(A < ec ? A : ec);
  } else {
    d->capacity = INT32_MAX;
    d->rows_cap = (int)A;
  }
  d->group_rows = c->num_tokens < d->capacity ? c->num_tokens : d->capacity;
  return MOE_OK;
}

// The kernels address their matrix operands with 32-bit byte offsets from one
// buffer descriptor per operand.  Every operand such a descriptor covers must
// span at most kMaxOperandBytes (4 GiB minus the 2 MiB the weight-streaming
// kernel keeps above its range for rows that return zeros); larger shapes are
// rejected before anything is launched instead of wrapping.
constexpr long long kMaxOperandBytes = 0xffe00000LL;
inline bool span_ok(long long rows, long long cols, long long elem) {
  return rows * cols * elem <= kMaxOperandBytes;
}

moe_status validate_spans(const moe_config* c) {
  const long long es = c->act_dtype == BF16 ? 2 : 4;
  const long long T = c->num_tokens, D = c->d_model, E = c->num_experts, k = c->top_k, F = c->d_ff;
  const long long nF = (c->activation == SWIGLU ? 2 : 1) * F;
  const long long SF = (long long)c->num_shared * c->d_ff_shared;
  long long A = T * k;                                   // rows of the permuted operands (upper bound)
  if (c->capacity_factor > 0.0f) {
    const double cap = ceil((double)c->capacity_factor * (double)A / (double)E);
    if (cap * (double)E < (double)A) A = (long long)cap * E;
  }
  const bool ok = span_ok(T, D, es) &&                  // x (router, gate/up, shared)
                  span_ok(A, D, es) && span_ok(A, F, es) &&   // x_perm / y_perm, H
                  span_ok(nF, D, es) && span_ok(D, F, es) &&  // one expert's weights
                  span_ok(E, 3 * D, 4) &&                      // router weight (float32, or its bf16 planes)
                  span_ok(T, SF, es) && span_ok(2 * SF, D, es) && span_ok(D, SF, es);   // shared experts
  return ok ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

moe_status validate_config(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_tokens < 0 || c->d_model <= 0 || c->num_experts <= 0 || c->top_k <= 0 || c->d_ff <= 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->top_k > c->num_experts) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_shared < 0 || (c->num_shared > 0 && c->d_ff_shared <= 0)) return MOE_ERR_INVALID_ARGUMENT;
  if (c->scoring < 0 || c->scoring > 2) return MOE_ERR_INVALID_ARGUMENT;
  if (c->activation < 0 || c->activation > 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->act_dtype < 0 || c->act_dtype > 1 || c->router_dtype < 0 || c->router_dtype > 1)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!(c->capacity_factor == c->capacity_factor)) return MOE_ERR_INVALID_ARGUMENT;   // NaN
  if (c->num_experts > kMaxExperts || c->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == F32 && c->router_dtype == BF16) return MOE_ERR_UNSUPPORTED;
  const int vec = c->act_dtype == BF16 ? 8 : 4;
  if (c->d_model % vec || c->d_ff % vec) return MOE_ERR_UNSUPPORTED;
  if (c->num_shared > 0 && (((long long)c->num_shared * c->d_ff_shared) % vec)) return MOE_ERR_UNSUPPORTED;
  const long long T = c->num_tokens;
  if (T * c->num_experts > INT32_MAX / 2 || T * c->top_k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if ((long long)c->num_shared * c->d_ff_shared > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  return validate_spans(c);
}

// Workspace pieces ---------------------------------------------------------
size_t router_split_bytes(const moe_config* c);
// route workspace: logits [T, E] f32 | refinement flags [T] | router weight planes
size_t ws_route(const moe_config* c) {
  return carve((size_t)c->num_tokens * c->num_experts * 4) + carve((size_t)c->num_tokens * 4) +
         router_split_bytes(c);
}
size_t ws_permute(const moe_config* c) {
  return carve((size_t)ceil_div(c->num_tokens, kPermuteTile) * c->num_experts * 4);
}
size_t ffn_partial_bytes_any(int act, int D, int F, int max_rows, int G);
// expert FFN workspace: h [max_rows, F] | 4 tile prefixes of G+1 | float32
// partial sums of contraction splits
size_t ws_ffn(const moe_config* c, int G, int F, int max_rows, int act) {
  return carve((size_t)max_rows * F * esize(act)) + 4 * carve((size_t)(G + 1) * 4) +
         carve(ffn_partial_bytes_any(act, c->d_model, F, max_rows, G));
}
size_t ws_stats(const moe_config* c) {
  return carve((size_t)ceil_div(c->num_tokens, kStatsChunk) * c->num_experts * 4);
}

size_t ffn_partial_bytes(int act, int activation, int D, int F, int max_rows, int G, bool grouped,
                         int group_rows = INT_MAX);

struct Layout {
  size_t logits, flags, wsplit, probs, idx, w, tile_counts, counts, offsets, tile_prefix, tile_prefix2, row_of, tor, h,
      h_shared, yperm, partial, kpart, kpart_shared, total;
};

Layout layer_layout(const moe_config* c, const Derived& d) {
  Layout L{};
  const size_t T = c->num_tokens, E = c->num_experts, k = c->top_k;
  const size_t es = esize(c->act_dtype);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += carve(bytes); return at; };
  L.logits = take(T * E * 4);
  L.flags = take(T * 4);
  L.wsplit = take(router_split_bytes(c));
  L.probs = take(T * E * 4);
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.tile_counts = take((size_t)ceil_div(c->num_tokens, kPermuteTile) * E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.tile_prefix = take((E + 1) * 4);
  L.tile_prefix2 = take(3 * (E + 1) * 4);
  L.row_of = take(T * k * 4);
  L.tor = take((size_t)d.rows_cap * 4);
  // the shared experts run beside the routed ones: separate activations
  L.h = take((size_t)d.rows_cap * c->d_ff * es);
  L.h_shared = take((size_t)T * c->num_shared * c->d_ff_shared * es);
  L.yperm = take((size_t)d.rows_cap * c->d_model * es);
  L.partial = take((size_t)ceil_div(c->num_tokens, kStatsChunk) * E * 4);
  // float32 partial sums of contraction splits: routed and shared experts
  // run on different streams, each with its own
  L.kpart = take(ffn_partial_bytes(c->act_dtype, c->activation, c->d_model, c->d_ff, d.rows_cap, c->num_experts, true,
                                   d.group_rows));
  L.kpart_shared = take(c->num_shared > 0 ? ffn_partial_bytes(c->act_dtype, SWIGLU, c->d_model,
                                                              c->num_shared * c->d_ff_shared, c->num_tokens, 1, false)
                                          : 0);
  L.total = o;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(ws) + off); }

// Launch helpers -----------------------------------------------------------
// bf16 tokens with a float32 router weight run on the matrix cores: the weight
// is split exactly into three bf16 planes and the GEMM runs over K = 3D with
// the token columns wrapping (x . w = x . hi + x . mid + x . lo).
inline bool router_split(const moe_config* c) {
  return c->router_dtype == F32 && c->act_dtype == BF16 && c->d_model % 64 == 0;
}
size_t router_split_bytes(const moe_config* c) {
  return router_split(c) ? carve((size_t)c->num_experts * 3 * c->d_model * 2) : 0;
}

// MOE_ROUTER_KERNEL=0 keeps the router on the general GEMM (tuning aid).
bool router_kernel_enabled() {
  const int v = tuning().router_kernel;
  return v == kUnset || v != 0;
}

moe_status run_router_logits(const moe_config* c, const void* x, const void* w_router, float* logits,
                             void* split_ws, hipStream_t s) {
  GroupedGemm g{};
  g.A = x; g.a_rows = nullptr; g.lda = c->d_model;
  g.B = w_router; g.b_group_stride = 0;
  g.C = logits; g.ldc = c->num_experts;
  g.M_max = c->num_tokens; g.N = c->num_experts; g.K = c->d_model;
  g.G = 1; g.offsets = nullptr; g.tile_prefix = nullptr;
  g.epilogue = EPI_STORE_F32;
  g.a_kwrap = 0;
  const int planes = c->router_dtype == BF16 ? 1 : 3;
  if (c->act_dtype == BF16 && (planes == 1 || router_split(c)) &&
      router_kernel_fits(c->num_tokens, c->num_experts, c->d_model, planes) && router_kernel_enabled()) {
    const bf16_t* wp = static_cast<const bf16_t*>(w_router);
    if (planes == 3) {
      bf16_t* sp = static_cast<bf16_t*>(split_ws);
      MOE_TRY_HIP("router weight split", launch_split_bf16x3(static_cast<const float*>(w_router), c->num_experts,
                                                             c->d_model, sp, s));
      wp = sp;
    }
    MOE_TRY_HIP("router logits", launch_router_logits(static_cast<const bf16_t*>(x), wp, planes, logits,
                                                      c->num_tokens, c->num_experts, c->d_model, s));
  } else if (c->router_dtype == BF16) {
    MOE_TRY_HIP("router logits (bf16)", launch_gemm_bf16(g, s));
  } else if (router_split(c)) {
    bf16_t* planes = static_cast<bf16_t*>(split_ws);
    MOE_TRY_HIP("router weight split", launch_split_bf16x3(static_cast<const float*>(w_router), c->num_experts,
                                                           c->d_model, planes, s));
    g.B = planes;
    g.K = 3 * c->d_model;
    g.a_kwrap = c->d_model;
    MOE_TRY_HIP("router logits (bf16 x3)", launch_gemm_bf16(g, s));
  } else {
    MOE_TRY_HIP("router logits (f32)", launch_gemm_f32(g, c->act_dtype, F32, s));
  }
  return MOE_OK;
}

moe_status run_select(const moe_config* c, const float* logits, const void* x, const void* w_router,
                      const float* sel_bias, int32_t* idx, float* w, float* probs, int32_t* flags,
                      hipStream_t s) {
  RouteArgs a{};
  a.logits = logits; a.x = x; a.w_router = w_router;
  a.sel_bias = c->scoring == SIGMOID_BIAS ? sel_bias : nullptr;
  a.topk_idx = idx; a.topk_w = w; a.probs = probs;
  a.T = c->num_tokens; a.D = c->d_model; a.E = c->num_experts; a.k = c->top_k;
  a.scoring = c->scoring; a.renormalize = c->renormalize;
  a.act_dtype = c->act_dtype; a.router_dtype = c->router_dtype;
  MOE_TRY_HIP("route select", launch_route_select(a, flags, s));
  return MOE_OK;
}

// Records stage event `which` (0 = start, 1 = stop) when timing is requested.
moe_status mark(void* const* ev, int stage, int which, hipStream_t s) {
  if (ev == nullptr || ev[2 * stage + which] == nullptr) return MOE_OK;
  MOE_TRY_HIP("stage event", hipEventRecord(static_cast<hipEvent_t>(ev[2 * stage + which]), s));
  return MOE_OK;
}

// Kernel choice for one projection: -1 = the general kernels (any K), else a
// tile configuration of the pipelined bf16 kernel (K a multiple of 64).  The
// tile height follows the average rows per group; MOE_GEMM_CFG=<n> overrides
// the choice (tuning aid; -1 forces the general kernels), MOE_GEMM_CFG_DOWN
// that of the down projection alone.
constexpr int kDeepCfg = 13;   // 256x256 tiles, 8 waves, register-staged slices

int pick_cfg(int act, int K, int max_rows, int G, bool down) {
  if (act != BF16 || K % 64 != 0) return -1;
  const Tuning t = tuning();
  const int forced = down && t.gemm_cfg_down != kUnset ? t.gemm_cfg_down : t.gemm_cfg;
  if (forced != kUnset) return (forced >= -1 && forced < kGemmConfigs) ? forced : -1;
  // measured on MI355X at the Switch / Mixtral / DeepSeekMoE / DeepSeek-V3
  // shapes: 256x256 tiles on 8 waves (64-deep slices staged in registers and
  // written to two LDS stages, interleaved schedule; 1-5% faster per layer
  // than the DMA rings of configuration 0, bit-identical results) once groups
  // are a few hundred rows deep; for shallow groups the persistent
  // weight-streaming kernel with 128x128 tiles and waves side by side over
  // the columns (gate/up: two workgroups per CU, so that one's activation
  // epilogue overlaps the other's weight stream; down: one workgroup per CU,
  // four slices deep)
  const int avg = G > 0 ? max_rows / G : max_rows;
  if (avg >= 160) return kDeepCfg;
  return kGemmV3Configs + (down ? 5 : 6);
}

int cfg_bm(int act, int cfg) {
  if (act != BF16) return kF32GemmBM;
  if (cfg < 0) {
    GroupedGemm dummy{};
    return gemm_bf16_bm(dummy);
  }
  if (cfg < kGemmV3Configs) return gemm_v3_bm(cfg);
  return gemm_ws_bm(cfg - kGemmV3Configs);
}

struct FfnPlan {
  int cfg_up, cfg_dn, bm_up, bm_dn;
  // split: groups of at most sh_rows rows go to the persistent weight-streaming
  // configuration cfg_sh (m-tiles of sh_bm rows), deeper groups to cfg_up / cfg_dn
  bool split;
  int cfg_sh, sh_rows, sh_bm;
  // contraction splits (1 = none) of the four launches: gate/up, down, and
  // the gate/up and down of the shallow groups of a split
  int ks_up, ks_dn, ks_sh_up, ks_sh_dn;
};

// Contraction split of a weight-streaming launch whose tiles do not spread
// evenly over the CUs (decode-sized batches: a few rows per expert, and the
// down projection has only D / 128 column tiles per expert): units of K / KS
// for KS in {1, 2, 4, 8}, with K / 64 divisible by KS and at least 4 slices
// of 64 per unit; a launch of U units takes about ceil(U / 256) / KS tile
// times on 256 CUs (the persistent grid deals units round-robin), and the
// smallest KS within 10% of the best estimate is taken (the partial sums
// cost an extra pass; at most 256 MB of them).  The tile count is bounded on
// the host from the row and group counts (the routing is known on the device
// only); the bound is loose when there are many groups, so launches bounded
// at 512 tiles or more are not split (measured: the Switch-shaped down
// projection, bound 1,152 tiles for 768 real ones, ran 132 -> 176 us split
// in two).  MOE_GEMM_KSPLIT=<n> forces n where it divides the contraction
// (tuning aid and test hook).
constexpr int kSplitUnits = 256;
constexpr long long kMaxPartialBytes = 256LL << 20;
int pick_ksplit(int act, int cfg, int epi, int N, int K, int G, int max_rows, bool grouped) {
  if (act != BF16 || cfg < kGemmV3Configs || K % 64 != 0 || max_rows <= 0) return 1;
  const int nk = K / 64;
  const int f = tuning().gemm_ksplit;
  if (f != kUnset && (f == 1 || ((f == 2 || f == 4 || f == 8) && nk % f == 0))) return f;
  const int c = cfg - kGemmV3Configs;
  const int cols = epi == EPI_SWIGLU ? gemm_ws_bn(c) / 2 : gemm_ws_bn(c);
  const int bm = gemm_ws_bm(c);
  const long long m_tiles = grouped ? max_rows / bm + (G < max_rows ? G : max_rows) : ceil_div(max_rows, bm);
  const long long tiles = m_tiles * ceil_div(N, cols);
  if (tiles >= 2 * kSplitUnits) return 1;
  const long long row_bytes = (long long)(epi == EPI_SWIGLU ? 2 : 1) * N * 4;
  double est[4];
  double best = 1e300;
  for (int i = 0, ks = 1; i < 4; ++i, ks *= 2) {
    const bool ok = ks == 1 || (nk % ks == 0 && nk / ks >= 4 && ks * max_rows * row_bytes <= kMaxPartialBytes);
    est[i] = ok ? (double)((tiles * ks + kSplitUnits - 1) / kSplitUnits) / ks : 1e300;
    best = est[i] < best ? est[i] : best;
  }
  for (int i = 0, ks = 1; i < 4; ++i, ks *= 2)
    if (est[i] <= 1.1 * best) return ks;
  return 1;
}

// Shallow groups are split off when both contractions are long (the
// weight stream of a tile then dwarfs its start-up) and groups are shallow on
// average.  MOE_GEMM_SPLIT=0 / 1 overrides the choice (tuning aid).  When
// every group is shallow (at most sh_rows rows in all: a decode-sized
// batch) both projections run on the shallow-group configuration alone.
constexpr int kShallowRows = 64;

// group_rows bounds the rows of any one group (the layer knows one: a token
// gives an expert at most one row); with every group shallow the
// weight-streaming configuration takes both projections on all CUs.
FfnPlan plan_ffn(int act, int activation, int D, int F, int max_rows, int G, bool grouped,
                 int group_rows = INT_MAX) {
  FfnPlan pl;
  const int grp = max_rows < group_rows ? max_rows : group_rows;   // rows of the largest group
  pl.cfg_up = pick_cfg(act, D, max_rows, G, false);
  pl.cfg_dn = pick_cfg(act, F, max_rows, G, true);
  // shallow groups: the persistent weight-streaming kernel with 64x128 tiles
  // and a 5-deep ring (measured ~1% per DeepSeek-V3-shaped layer ahead of the
  // 64x256 persistent configuration of the deep-tile kernel)
  pl.cfg_sh = kGemmV3Configs + 3;
  const Tuning t = tuning();
  if (t.gemm_shcfg != kUnset && t.gemm_shcfg >= 0 && t.gemm_shcfg < kGemmConfigs)
    pl.cfg_sh = t.gemm_shcfg;       // tuning aid: a configuration index >= 0
  // groups of at most sh_rows rows are shallow (64 by default; the tiles of
  // the weight-streaming configuration may be shorter, a group then takes
  // several of them)
  pl.sh_bm = cfg_bm(act, pl.cfg_sh);
  pl.sh_rows = pl.sh_bm > kShallowRows ? pl.sh_bm : kShallowRows;
  if (t.shallow_rows != kUnset && t.shallow_rows >= pl.sh_bm && t.shallow_rows <= 4096) pl.sh_rows = t.shallow_rows;
  const bool forced = t.gemm_cfg != kUnset;
  if (!forced && pl.cfg_up >= 0 && pl.cfg_dn >= 0 && D % 64 == 0 && F % 64 == 0 && grp <= pl.sh_rows) {
    pl.cfg_up = pl.cfg_sh;
    pl.cfg_dn = pl.cfg_sh;
  }
  pl.bm_up = cfg_bm(act, pl.cfg_up);
  pl.bm_dn = cfg_bm(act, pl.cfg_dn);
  const bool able = grouped && pl.cfg_up >= 0 && pl.cfg_dn >= 0 && D % 64 == 0 && F % 64 == 0;
  const int avg = G > 0 ? max_rows / G : max_rows;
  pl.split = able && D >= 1024 && F >= 1024 && avg < 320 && grp > pl.sh_rows;
  if (able && t.gemm_split != kUnset) pl.split = t.gemm_split != 0;
  const int epi_up = activation == SWIGLU ? EPI_SWIGLU : EPI_GELU;
  pl.ks_up = pick_ksplit(act, pl.cfg_up, epi_up, F, D, G, max_rows, grouped);
  pl.ks_dn = pick_ksplit(act, pl.cfg_dn, EPI_STORE_ACT, D, F, G, max_rows, grouped);
  pl.ks_sh_up = pl.split ? pick_ksplit(act, pl.cfg_sh, epi_up, F, D, G, max_rows, grouped) : 1;
  pl.ks_sh_dn = pl.split ? pick_ksplit(act, pl.cfg_sh, EPI_STORE_ACT, D, F, G, max_rows, grouped) : 1;
  return pl;
}

// Bytes of float32 partial sums that the contraction splits of one expert FFN
// need (the launches run one after another and share them).
size_t ffn_ksplit_bytes(int act, int activation, int D, int F, int max_rows, int G, bool grouped,
                        int group_rows = INT_MAX) {
  const FfnPlan pl = plan_ffn(act, activation, D, F, max_rows, G, grouped, group_rows);
  const size_t ldp_up = (size_t)(activation == SWIGLU ? 2 : 1) * F;
  const int ks_up = pl.ks_up > pl.ks_sh_up ? pl.ks_up : pl.ks_sh_up;
  const int ks_dn = pl.ks_dn > pl.ks_sh_dn ? pl.ks_dn : pl.ks_sh_dn;
  size_t b = 0;
  if (ks_up > 1) b = (size_t)ks_up * max_rows * ldp_up * 4;
  if (ks_dn > 1) b = b > (size_t)ks_dn * max_rows * D * 4 ? b : (size_t)ks_dn * max_rows * D * 4;
  return b;
}
size_t ffn_tail_bytes(int act, int activation, int D, int F, int max_rows, int G, bool grouped,
                      int group_rows = INT_MAX);
// The contraction splits' partial sums, then (from a 256-byte boundary) the
// unit blocks of the down projection's split tail.
size_t ffn_partial_bytes(int act, int activation, int D, int F, int max_rows, int G, bool grouped,
                         int group_rows) {
  return round_up(ffn_ksplit_bytes(act, activation, D, F, max_rows, G, grouped, group_rows), 256) +
         ffn_tail_bytes(act, activation, D, F, max_rows, G, grouped, group_rows);
}
// ... for either activation, grouped or not (moe_expert_ffn's workspace)
size_t ffn_partial_bytes_any(int act, int D, int F, int max_rows, int G) {
  size_t b = 0;
  for (int a : {SWIGLU, GELU})
    for (bool gr : {false, true}) {
      const size_t v = ffn_partial_bytes(act, a, D, F, max_rows, G, gr);
      b = v > b ? v : b;
    }
  return b;
}

// The last round of a 256x256-tile launch with a long contraction (a round
// takes long there): when the tiles do not fill a whole number of rounds (one
// workgroup per CU), the full rounds run as they are and each remaining tile
// runs as S units over a part of the contraction each (S from tail_units:
// S times the remaining tiles fill at most one round), whose float32 sums a
// second kernel adds in a fixed order.  Measured on MI355X (Mixtral-shaped
// down projection, K = 14336, 64 tiles left after two rounds, S = 4):
// 1123 us without a split, 947-958 us with the remaining tiles as four
// 128x128 quarters each (the form this replaces), 854-859 us split; no gain
// at K = 1408 or 2048, where it is not used.  MOE_GEMM_TAIL=0 turns it off
// (tuning aid).
bool tail_split_enabled() {
  const int v = tuning().gemm_tail;
  return v == kUnset || v != 0;
}
// parents: the 256x256-tile configurations with one workgroup per CU (DMA
// rings, or register-staged slices on 8 waves)
constexpr int kTailParentCfg = 0, kTailParentStagedCfg = kDeepCfg;
constexpr int kTailBlock = 256 * 256;   // floats per unit block of the split tail

size_t ffn_tail_bytes(int act, int activation, int D, int F, int max_rows, int G, bool grouped, int group_rows) {
  if (act != BF16 || !grouped || F < 4096 || F % 64 != 0 || !tail_split_enabled()) return 0;
  const FfnPlan pl = plan_ffn(act, activation, D, F, max_rows, G, grouped, group_rows);
  if (pl.cfg_dn != kTailParentCfg && pl.cfg_dn != kTailParentStagedCfg) return 0;
  return (size_t)num_cus() * kTailBlock * 4;
}

hipError_t launch_gemm(int act, int cfg, const GroupedGemm& g, hipStream_t s);

hipError_t launch_gemm_tail_split(int act, int cfg, const GroupedGemm& g, hipStream_t s) {
  const bool parent = cfg == kTailParentCfg || cfg == kTailParentStagedCfg;
  const int round = num_cus();
  // (the unit blocks are in the workspace whenever this split applies:
  // ffn_tail_bytes follows the same conditions)
  if (act != BF16 || !parent || g.offsets == nullptr || g.K < 4096 || !tail_split_enabled() ||
      g.epilogue != EPI_STORE_ACT || g.tail_part == nullptr || g.tail_cap < round)
    return launch_gemm(act, cfg, g, s);
  GroupedGemm full = g, tail = g;
  full.tail_mode = 1;
  full.round = round;
  hipError_t e = launch_gemm(act, cfg, full, s);
  if (e != hipSuccess) return e;
  tail.tail_mode = 2;
  tail.round = round;
  tail.epilogue = EPI_TAIL_PART;
  e = launch_gemm(act, cfg, tail, s);
  if (e != hipSuccess) return e;
  return launch_tail_reduce(tail, s);
}

hipError_t launch_gemm(int act, int cfg, const GroupedGemm& g, hipStream_t s) {
  if (g.ksplit > 1 && (act != BF16 || cfg < kGemmV3Configs)) return hipErrorInvalidValue;
  if (act != BF16) return launch_gemm_f32(g, F32, F32, s);
  if (cfg >= kGemmV3Configs) return launch_gemm_ws(g, cfg - kGemmV3Configs, s);
  if (cfg >= 0) return launch_gemm_v3(g, cfg, s);
  return launch_gemm_bf16(g, s);
}

// gate/up (+activation) then down projection for G groups.  prefix_up holds
// the m-tile prefix for the plan's bm_up over all groups (computed by the
// caller when offsets are given); prefix_ws has room for three more prefixes
// of G+1 entries (the down projection's when it tiles differently, or the
// class prefixes of a split).
// A second stream for the shallow groups of a split: their persistent
// weight-streaming launches take `cus` CUs (their HBM stream needs few) while
// the deep-tile launches, which are bound by the matrix cores, run on the
// caller's stream on the remaining CUs, and on all of them once the shallow
// groups are done.
struct SideStream {
  hipStream_t s;
  hipEvent_t fork, join;
  int cus;
};

// CUs of the concurrent shallow-group launch (MOE_SHALLOW_CUS overrides;
// 0 runs the shallow groups in line after the deep ones), from the average
// rows per group: where it is well above the shallow threshold the deep
// groups carry most of the work and the shallow ones' weight stream needs
// few CUs; near or below it most groups are shallow and their stream needs
// most of the chip.  Measured on MI355X, routed FFN, DeepSeek-V3 shape
// (8192 tokens, 256 rows per expert on average): in line 7.01 ms; beside the
// deep tiles on 64 CUs 6.71, 96 6.85, 128 6.96, 160 6.95.  Its first 256
// tokens (8 rows on average), whole layer: 64 CUs 3.23 ms, 128 2.00, 192
// 1.71, 224 1.69, all 256 1.69, in line 1.76.
int shallow_cus(int max_rows, int G, int sh_rows) {
  const int v = tuning().shallow_cus;
  if (v != kUnset) return v < 0 ? 0 : v;
  const long long avg = G > 0 ? max_rows / G : max_rows;
  const int n = num_cus();                       // 256 on MI355X: 64, or all
  return avg >= 2LL * sh_rows ? (n + 3) / 4 : n;
}

moe_status run_ffn(int act, int activation, int G, int D, int F, int max_rows, const void* x_in,
                   const int32_t* gather, const int32_t* offsets, const int32_t* prefix_up,
                   int32_t* prefix_ws, const void* w13, const void* w2, void* h, void* y_out, float* part,
                   hipStream_t s, void* const* ev = nullptr, int stage_up = 0, int stage_down = 0,
                   const SideStream* side = nullptr, int group_rows = INT_MAX) {
  const FfnPlan pl = plan_ffn(act, activation, D, F, max_rows, G, offsets != nullptr, group_rows);
  const int n_mat = activation == SWIGLU ? 2 : 1;
  GroupedGemm g1{};
  g1.A = x_in; g1.a_rows = gather; g1.lda = D;
  g1.B = w13; g1.b_group_stride = (long long)n_mat * F * D;
  g1.C = h; g1.ldc = F;
  g1.M_max = max_rows; g1.N = F; g1.K = D;
  g1.G = G; g1.offsets = offsets; g1.tile_prefix = prefix_up;
  g1.epilogue = activation == SWIGLU ? EPI_SWIGLU : EPI_GELU;
  GroupedGemm g2{};
  g2.A = h; g2.a_rows = nullptr; g2.lda = F;
  g2.B = w2; g2.b_group_stride = (long long)D * F;
  g2.C = y_out; g2.ldc = D;
  g2.M_max = max_rows; g2.N = D; g2.K = F;
  g2.G = G; g2.offsets = offsets; g2.tile_prefix = prefix_up;
  g2.epilogue = EPI_STORE_ACT;
  g1.partial = part; g1.ldp = n_mat * F; g1.ksplit = pl.ks_up;
  g2.partial = part; g2.ldp = D; g2.ksplit = pl.ks_dn;
  {
    const int gm = tuning().tile_gm;
    g1.tile_gm = g2.tile_gm = (gm != kUnset && gm > 0 && gm <= 64) ? gm : 0;
  }
  GroupedGemm g1s = g1, g2s = g2;       // shallow groups of a split
  g1s.ksplit = pl.ks_sh_up;
  g2s.ksplit = pl.ks_sh_dn;
  // the split tail's unit blocks follow the contraction splits' sums (their
  // own region: the shallow launches may use those on another stream)
  if (part != nullptr && ffn_tail_bytes(act, activation, D, F, max_rows, G, offsets != nullptr, group_rows) > 0) {
    g2.tail_part = part + round_up(ffn_ksplit_bytes(act, activation, D, F, max_rows, G, offsets != nullptr,
                                                    group_rows), 256) / 4;
    g2.tail_cap = num_cus();
  }
  if (pl.split) {
    int32_t* deep_up = prefix_ws;
    int32_t* deep_dn = pl.bm_dn != pl.bm_up ? prefix_ws + (G + 1) : deep_up;
    int32_t* shallow = prefix_ws + 2 * (G + 1);
    const TilePrefixReq r0{deep_up, pl.bm_up, pl.sh_rows, INT_MAX};
    const TilePrefixReq r1{deep_dn != deep_up ? deep_dn : nullptr, pl.bm_dn, pl.sh_rows, INT_MAX};
    const TilePrefixReq r2{shallow, pl.sh_bm, 0, pl.sh_rows};
    MOE_TRY_HIP("tile prefix", launch_tile_prefix_classes(offsets, G, r0, r1, r2, s));
    g1.tile_prefix = deep_up;
    g2.tile_prefix = deep_dn;
    g1s.tile_prefix = shallow;
    g2s.tile_prefix = shallow;
  } else if (offsets != nullptr && pl.bm_dn != pl.bm_up) {
    MOE_TRY_HIP("tile prefix", launch_tile_prefix(offsets, G, pl.bm_dn, prefix_ws, s));
    g2.tile_prefix = prefix_ws;
  }
  // Concurrent shallow groups: both of their projections on the side stream
  // (the gate/up of a group before its down, in stream order), issued before
  // the deep launches so that they hold their CUs from the start; the two
  // classes write disjoint rows of h and y_out.  The stage events then span
  // the deep launches (gate/up) and the rest up to the join (down).
  // (only the shallow launches may use the contraction split's partial sums,
  // which the two launches of the side stream use one after the other)
  const bool concurrent = pl.split && side != nullptr && side->cus > 0 &&
                          pl.cfg_sh >= kGemmV3Configs && pl.ks_up <= 1 && pl.ks_dn <= 1;
  MOE_TRY(mark(ev, stage_up, 0, s));
  if (concurrent) {
    g1s.cus = side->cus;
    g2s.cus = side->cus;
    MOE_TRY_HIP("fork", hipEventRecord(side->fork, s));
    MOE_TRY_HIP("fork", hipStreamWaitEvent(side->s, side->fork, 0));
    MOE_TRY_HIP("expert gate/up (shallow groups)", launch_gemm(act, pl.cfg_sh, g1s, side->s));
    MOE_TRY_HIP("expert down (shallow groups)", launch_gemm(act, pl.cfg_sh, g2s, side->s));
    MOE_TRY_HIP("join", hipEventRecord(side->join, side->s));
  }
  MOE_TRY_HIP("expert gate/up", launch_gemm(act, pl.cfg_up, g1, s));
  if (pl.split && !concurrent) MOE_TRY_HIP("expert gate/up (shallow groups)", launch_gemm(act, pl.cfg_sh, g1s, s));
  MOE_TRY(mark(ev, stage_up, 1, s));
  MOE_TRY(mark(ev, stage_down, 0, s));
  MOE_TRY_HIP("expert down", launch_gemm_tail_split(act, pl.cfg_dn, g2, s));
  if (pl.split && !concurrent) MOE_TRY_HIP("expert down (shallow groups)", launch_gemm(act, pl.cfg_sh, g2s, s));
  if (concurrent) MOE_TRY_HIP("join", hipStreamWaitEvent(s, side->join, 0));
  MOE_TRY(mark(ev, stage_down, 1, s));
  return MOE_OK;
}

// One projection of an ungrouped (shared-expert) FFN over `rows` rows:
// gate/up with SwiGLU into h (up == true), or down from h into y_out.
moe_status run_ffn_part(int act, int activation, int G, int D, int F, int rows, const void* x_in, const void* w13,
                        const void* w2, void* h, void* y_out, float* part, hipStream_t s, void* const* ev, int stage,
                        bool up) {
  const FfnPlan pl = plan_ffn(act, activation, D, F, rows, G, false);
  GroupedGemm g{};
  g.partial = part;
  g.ldp = up ? (activation == SWIGLU ? 2 : 1) * F : D;
  g.ksplit = up ? pl.ks_up : pl.ks_dn;
  if (up) {
    g.A = x_in; g.lda = D; g.B = w13; g.b_group_stride = (long long)(activation == SWIGLU ? 2 : 1) * F * D;
    g.C = h; g.ldc = F; g.N = F; g.K = D;
    g.epilogue = activation == SWIGLU ? EPI_SWIGLU : EPI_GELU;
  } else {
    g.A = h; g.lda = F; g.B = w2; g.b_group_stride = (long long)D * F;
    g.C = y_out; g.ldc = D; g.N = D; g.K = F;
    g.epilogue = EPI_STORE_ACT;
  }
  g.a_rows = nullptr; g.M_max = rows; g.G = G; g.offsets = nullptr; g.tile_prefix = nullptr;
  MOE_TRY(mark(ev, stage, 0, s));
  MOE_TRY_HIP(up ? "shared gate/up" : "shared down", launch_gemm(act, up ? pl.cfg_up : pl.cfg_dn, g, s));
  MOE_TRY(mark(ev, stage, 1, s));
  return MOE_OK;
}

// How the shared experts run beside the routed path: 0 = after the routed
// experts on the caller's stream; 1 = gate/up on the auxiliary stream during
// routing, joined before the routed experts; 2 = both projections on the
// auxiliary stream from the start, joined before the combine; 3 = both on
// the auxiliary stream from the end of the permutation (beside the routed
// experts, leaving the routing kernels the whole chip), joined before the
// combine.  MOE_SHARED_OVERLAP overrides (tuning aid).
int shared_overlap() {
  const int v = tuning().shared_overlap;
  return (v != kUnset && v >= 0 && v <= 3) ? v : 2;
}

// A library-owned stream per device for the layer's work that does not depend
// on the routing (the shared experts' gate/up projection), forked from and
// joined back to the caller's stream with events.  Default priority.  The
// mutex keeps the fork / join sequences of concurrent host threads from
// interleaving.
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t stats_fork = nullptr, stats_join = nullptr;   // load statistics beside the experts
  hipStream_t s2 = nullptr;                                 // shallow expert groups beside the deep ones
  hipEvent_t side_fork = nullptr, side_join = nullptr;
};
constexpr int kMaxDevices = 64;
AuxStream g_aux[kMaxDevices];
std::mutex g_aux_mu;

moe_status aux_stream(AuxStream** out) {
  int dev = 0;
  MOE_TRY_HIP("hipGetDevice", hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  AuxStream& a = g_aux[dev];
  if (a.s == nullptr) {
    MOE_TRY_HIP("auxiliary stream", hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking));
    MOE_TRY_HIP("fork event", hipEventCreateWithFlags(&a.fork, hipEventDisableTiming));
    MOE_TRY_HIP("join event", hipEventCreateWithFlags(&a.join, hipEventDisableTiming));
    MOE_TRY_HIP("fork event", hipEventCreateWithFlags(&a.stats_fork, hipEventDisableTiming));
    MOE_TRY_HIP("join event", hipEventCreateWithFlags(&a.stats_join, hipEventDisableTiming));
    MOE_TRY_HIP("side stream", hipStreamCreateWithFlags(&a.s2, hipStreamNonBlocking));
    MOE_TRY_HIP("fork event", hipEventCreateWithFlags(&a.side_fork, hipEventDisableTiming));
    MOE_TRY_HIP("join event", hipEventCreateWithFlags(&a.side_join, hipEventDisableTiming));
  }
  *out = &a;
  return MOE_OK;
}

// Backward -----------------------------------------------------------------
// The backward's extra operands: the gate/up products and their gradients
// [A, n_mat F] of the routed and [T, 2 S F_s] of the shared experts, and the
// transposed expert weights [D, n_mat F].
moe_status validate_backward_spans(const moe_config* c) {
  Derived d;
  derive(c, &d);
  const long long nF = (c->activation == SWIGLU ? 2LL : 1LL) * c->d_ff;
  const long long SF = (long long)c->num_shared * c->d_ff_shared;
  if (!span_ok(d.rows_cap, nF, 2) || !span_ok(c->num_tokens, 2 * SF, 2) || !span_ok(c->d_model, nF, 2))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct BwLayout {
  size_t fwd, y, dyp, gu, dh, dgu, dxp, w13t, w2t, ones, dw, dlogits, dxr, rpart, pre, gus, dhs, dgus, dxs, ws13t,
      ws2t, rplanes, rplanes_t, raux, total;
};

BwLayout bw_layout(const moe_config* c, const Derived& d) {
  BwLayout B{};
  const size_t T = c->num_tokens, E = c->num_experts, k = c->top_k, D = c->d_model, F = c->d_ff;
  const size_t A = d.rows_cap, nF = (c->activation == SWIGLU ? 2 : 1) * F;
  const size_t SF = (size_t)c->num_shared * c->d_ff_shared;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += carve(bytes); return at; };
  B.fwd = take(layer_layout(c, d).total);
  B.y = take(T * D * 2);
  B.dyp = take(A * D * 2);
  B.gu = take(A * nF * 2);
  B.dh = take(A * F * 2);
  B.dgu = take(A * nF * 2);
  B.dxp = take(A * D * 2);
  B.w13t = take(E * D * nF * 2);
  B.w2t = take(E * F * D * 2);
  B.ones = take(T * k * 4);
  B.dw = take(T * k * 4);
  B.dlogits = take(T * E * 4);
  B.dxr = take(T * D * 4);
  B.rpart = take((size_t)std::max(kF32MaxSplit, 3 * kRouterMfmaSplit) * E * D * 4);
  B.pre = take(2 * (E + 1) * 4);
  B.gus = take(T * 2 * SF * 2);
  B.dhs = take(T * SF * 2);
  B.dgus = take(T * 2 * SF * 2);
  B.dxs = take(T * D * 2);
  B.ws13t = take(2 * SF * D * 2);
  B.ws2t = take(SF * D * 2);
  B.rplanes = take(T * 3 * E * 2);
  B.rplanes_t = take(T * 3 * E * 2);
  B.raux = take((kRouterMfmaSplit + 1 + 3 * E) * 4);
  B.total = o;
  return B;
}

// One bf16 product C [rows, N] = A [rows, K] B_g^T for groups given by
// offsets (or one group of `rows` rows), store epilogue, on the kernel the
// forward would pick for this contraction.
moe_status bw_gemm(const char* what, const void* A, const int32_t* a_rows, int lda, const void* B, long long bstride,
                   void* C, int ldc, int rows, int N, int K, int G, const int32_t* offsets, int32_t* prefix,
                   hipStream_t s) {
  const int cfg = pick_cfg(BF16, K, rows, G, false);
  GroupedGemm g{};
  g.A = A; g.a_rows = a_rows; g.lda = lda;
  g.B = B; g.b_group_stride = bstride;
  g.C = C; g.ldc = ldc;
  g.M_max = rows; g.N = N; g.K = K;
  g.G = G; g.offsets = offsets; g.tile_prefix = nullptr;
  g.epilogue = EPI_STORE_ACT;
  if (offsets != nullptr) {
    MOE_TRY_HIP("tile prefix", launch_tile_prefix(offsets, G, cfg_bm(BF16, cfg), prefix, s));
    g.tile_prefix = prefix;
  }
  MOE_TRY_HIP(what, launch_gemm(BF16, cfg, g, s));
  return MOE_OK;
}

// Expert choice --------------------------------------------------------------
int ec_capacity(const moe_config* c) {
  if (c->num_tokens <= 0) return 0;
  const double cf = c->capacity_factor > 0.0f ? (double)c->capacity_factor : 1.0;
  const double v = ceil(cf * (double)c->num_tokens * (double)c->top_k / (double)c->num_experts);
  return v >= (double)c->num_tokens ? c->num_tokens : (int)v;
}

struct EcLayout {
  size_t logits, wsplit, pT, tor, roww, offsets, prefixes, selbits, selpre, h, yperm, h_shared, kpart, kpart_shared,
      total;
};

EcLayout ec_layout(const moe_config* c) {
  EcLayout L{};
  const size_t T = c->num_tokens, E = c->num_experts, C = ec_capacity(c);
  const size_t es = esize(c->act_dtype);
  const size_t W = (T + 31) / 32;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += carve(bytes); return at; };
  L.logits = take(T * E * 4);
  L.wsplit = take(router_split_bytes(c));
  L.pT = take(T * E * 4);
  L.tor = take(E * C * 4);
  L.roww = take(E * C * 4);
  L.offsets = take((E + 1) * 4);
  L.prefixes = take(4 * (E + 1) * 4);
  L.selbits = take(E * W * 4);
  L.selpre = take(E * W * 4);
  L.h = take(E * C * c->d_ff * es);
  L.yperm = take(E * C * c->d_model * es);
  L.h_shared = take(T * c->num_shared * c->d_ff_shared * es);
  L.kpart = take(ffn_partial_bytes(c->act_dtype, c->activation, c->d_model, c->d_ff, (int)(E * C), (int)E, true,
                                   (int)C));
  L.kpart_shared = take(c->num_shared > 0 ? ffn_partial_bytes(c->act_dtype, SWIGLU, c->d_model,
                                                              c->num_shared * c->d_ff_shared, (int)T, 1, false)
                                          : 0);
  L.total = o;
  return L;
}

moe_status validate_ec(const moe_config* c) {
  MOE_TRY(validate_config(c));
  if (c->num_experts > kEcMaxExperts || c->num_tokens > kEcMaxTokens) return MOE_ERR_UNSUPPORTED;
  if ((long long)c->num_experts * ec_capacity(c) > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const long long rows = (long long)c->num_experts * ec_capacity(c);
  if (!span_ok(rows, c->d_model, esize(c->act_dtype)) || !span_ok(rows, c->d_ff, esize(c->act_dtype)))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

namespace moe {
void debug_message(const char* where, const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, msg);
}
}  // namespace moe

extern "C" {

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEBUG_CHECK: return "MOE_ERR_DEBUG_CHECK";
  }
  return "unknown moe_status";
}

const char* moe_last_error(void) { return g_last_error; }

moe_status moe_capacity(const moe_config* cfg, int32_t* capacity, int32_t* rows_cap) {
  MOE_TRY(validate_config(cfg));
  Derived d;
  derive(cfg, &d);
  if (capacity) *capacity = d.capacity;
  if (rows_cap) *rows_cap = d.rows_cap;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, int32_t op, size_t* bytes) {
  MOE_TRY(validate_config(cfg));
  if (bytes == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  Derived d;
  derive(cfg, &d);
  switch (op) {
    case MOE_OP_ROUTE: *bytes = ws_route(cfg); break;
    case MOE_OP_PERMUTE: *bytes = ws_permute(cfg); break;
    case MOE_OP_EXPERT_FFN:
      *bytes = ws_ffn(cfg, cfg->num_experts, cfg->d_ff, d.rows_cap, cfg->act_dtype);
      break;
    case MOE_OP_SHARED_FFN:
      *bytes = ws_ffn(cfg, 1, cfg->num_shared * cfg->d_ff_shared, cfg->num_tokens, cfg->act_dtype);
      break;
    case MOE_OP_LOAD_STATS: *bytes = ws_stats(cfg); break;
    case MOE_OP_LAYER: *bytes = layer_layout(cfg, d).total; break;
    case MOE_OP_EXPERT_CHOICE:
      MOE_TRY(validate_ec(cfg));
      *bytes = ec_layout(cfg).total;
      break;
    case MOE_OP_LAYER_BACKWARD:
      MOE_TRY(validate_backward_spans(cfg));
      *bytes = bw_layout(cfg, d).total;
      break;
    default: return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* sel_bias, int32_t* topk_idx, float* topk_w, float* probs,
                     void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (cfg->num_tokens > 0 && (x == nullptr || topk_idx == nullptr || topk_w == nullptr || ws == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (w_router == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (!opt_aligned(x) || !aligned16(w_router) || !opt_aligned(sel_bias) || !opt_aligned(topk_idx) ||
      !opt_aligned(topk_w) || !opt_aligned(probs) || !opt_aligned(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ws_route(cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (cfg->num_tokens == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = static_cast<float*>(ws);
  const size_t lb = carve((size_t)cfg->num_tokens * cfg->num_experts * 4);
  int32_t* flags = at<int32_t>(ws, lb);
  MOE_TRY(run_router_logits(cfg, x, w_router, logits, at<void>(ws, lb + carve((size_t)cfg->num_tokens * 4)), s));
  return run_select(cfg, logits, x, w_router, sel_bias, topk_idx, topk_w, probs, flags, s);
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* token_of_row,
                       void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_config(cfg));
  Derived d;
  derive(cfg, &d);
  const bool any = cfg->num_tokens > 0;
  if (counts == nullptr || offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (any && (topk_idx == nullptr || row_of == nullptr || ws == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (d.rows_cap > 0 && token_of_row == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!opt_aligned(topk_idx) || !opt_aligned(x) || !aligned16(counts) || !aligned16(offsets) ||
      !opt_aligned(row_of) || !opt_aligned(token_of_row) || !opt_aligned(x_perm) || !opt_aligned(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ws_permute(cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PermuteArgs a{};
  a.topk_idx = topk_idx; a.T = cfg->num_tokens; a.k = cfg->top_k; a.E = cfg->num_experts;
  a.capacity = d.capacity; a.rows_cap = d.rows_cap;
  a.tile_counts = static_cast<int32_t*>(ws);
  a.counts = counts; a.offsets = offsets; a.row_of = row_of; a.token_of_row = token_of_row;
  a.tile_prefix = nullptr; a.bm = 1;
  MOE_TRY_HIP("permute", launch_permute(a, s));
  if (debug_on() && any)
    MOE_TRY(debug_check_dispatch("moe_permute", cfg, d.capacity, d.rows_cap, topk_idx, counts, offsets, row_of,
                                 token_of_row, s));
  if (x != nullptr)
    MOE_TRY_HIP("gather rows", launch_gather_rows(x, token_of_row, offsets, cfg->num_experts, d.rows_cap,
                                                  cfg->d_model, (int)esize(cfg->act_dtype), x_perm, s));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, int32_t num_groups, int32_t d_ff, int32_t activation,
                          int32_t max_rows, const void* x_in, const int32_t* gather_rows,
                          const int32_t* offsets, const void* w13, const void* w2, void* y_out,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (num_groups <= 0 || d_ff <= 0 || max_rows < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (activation != SWIGLU && activation != GELU) return MOE_ERR_INVALID_ARGUMENT;
  if (num_groups > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  const int vec = cfg->act_dtype == BF16 ? 8 : 4;
  if (d_ff % vec) return MOE_ERR_UNSUPPORTED;
  {
    const long long es = esize(cfg->act_dtype), nF = (activation == SWIGLU ? 2LL : 1LL) * d_ff;
    // x_in rows (without a gather map; with one, the caller keeps the rows it
    // names within the same bound), H, y_out and one group's weights
    if (!span_ok(max_rows, cfg->d_model, es) || !span_ok(max_rows, d_ff, es) || !span_ok(nF, cfg->d_model, es) ||
        !span_ok(cfg->d_model, d_ff, es))
      return MOE_ERR_UNSUPPORTED;
  }
  if (max_rows > 0 && (x_in == nullptr || w13 == nullptr || w2 == nullptr || y_out == nullptr || ws == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!opt_aligned(x_in) || !opt_aligned(gather_rows) || !opt_aligned(offsets) || !opt_aligned(w13) ||
      !opt_aligned(w2) || !opt_aligned(y_out) || !opt_aligned(ws))
    return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ws_ffn(cfg, num_groups, d_ff, max_rows, cfg->act_dtype)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (max_rows == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on()) {
    int rows = max_rows;
    char msg[200];
    if (offsets != nullptr) {
      std::vector<int32_t> ho;
      MOE_TRY(to_host(offsets, (size_t)num_groups + 1, &ho, s));
      if (!check_group_offsets(ho.data(), num_groups, max_rows, msg, sizeof(msg)))
        return debug_fail("moe_expert_ffn", msg);
      rows = ho[num_groups];
    }
    if (gather_rows != nullptr) {
      std::vector<int32_t> hg;
      MOE_TRY(to_host(gather_rows, (size_t)rows, &hg, s));
      if (!check_gather_rows(hg.data(), rows, msg, sizeof(msg))) return debug_fail("moe_expert_ffn", msg);
    }
  }
  void* h = ws;
  int32_t* prefix_up = nullptr;
  int32_t* prefix_dn = nullptr;
  const size_t hb = carve((size_t)max_rows * d_ff * esize(cfg->act_dtype));
  float* part = at<float>(ws, hb + 4 * carve((size_t)(num_groups + 1) * 4));
  if (offsets != nullptr) {
    prefix_up = at<int32_t>(ws, hb);
    prefix_dn = at<int32_t>(ws, hb + carve((size_t)(num_groups + 1) * 4));
    const FfnPlan pl = plan_ffn(cfg->act_dtype, activation, cfg->d_model, d_ff, max_rows, num_groups, true);
    if (!pl.split) MOE_TRY_HIP("tile prefix", launch_tile_prefix(offsets, num_groups, pl.bm_up, prefix_up, s));
  }
  return run_ffn(cfg->act_dtype, activation, num_groups, cfg->d_model, d_ff, max_rows, x_in, gather_rows,
                 offsets, prefix_up, prefix_dn, w13, w2, h, y_out, part, s);
}

moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of,
                       const float* topk_w, const void* y_shared, void* y, void* stream) {
  MOE_TRY(validate_config(cfg));
  Derived d;
  derive(cfg, &d);
  if (cfg->num_tokens > 0 && (row_of == nullptr || topk_w == nullptr || y == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (d.rows_cap > 0 && cfg->num_tokens > 0 && y_perm == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  if (!opt_aligned(y_perm) || !opt_aligned(row_of) || !opt_aligned(topk_w) || !opt_aligned(y_shared) ||
      !opt_aligned(y))
    return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_on() && cfg->num_tokens > 0) {
    std::vector<int32_t> hr;
    MOE_TRY(to_host(row_of, (size_t)cfg->num_tokens * cfg->top_k, &hr, s));
    char msg[200];
    if (!check_row_map(hr.data(), cfg->num_tokens, cfg->top_k, d.rows_cap, msg, sizeof(msg)))
      return debug_fail("moe_combine", msg);
  }
  MOE_TRY_HIP("combine", launch_combine(y_perm, row_of, topk_w, y_shared, y, cfg->num_tokens, cfg->top_k,
                                        cfg->d_model, cfg->act_dtype, s));
  return MOE_OK;
}

moe_status moe_load_stats(const moe_config* cfg, const int32_t* counts, const float* probs, float alpha,
                          float* f, float* P, float* aux_loss, float* imbalance, int32_t* dropped,
                          void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_config(cfg));
  Derived d;
  derive(cfg, &d);
  if (counts == nullptr || (cfg->num_tokens > 0 && (probs == nullptr || ws == nullptr)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(counts) || !opt_aligned(probs) || !opt_aligned(ws)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ws_stats(cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  StatsArgs a{};
  a.counts = counts; a.probs = probs; a.partial = static_cast<float*>(ws);
  a.T = cfg->num_tokens; a.E = cfg->num_experts; a.k = cfg->top_k; a.capacity = d.capacity;
  a.alpha = alpha; a.f = f; a.P = P; a.aux_loss = aux_loss; a.imbalance = imbalance; a.dropped = dropped;
  MOE_TRY_HIP("load stats", launch_load_stats(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* wt, const void* x, void* y,
                             int32_t* topk_idx, float* topk_w, int32_t* counts, float alpha, float* stats,
                             int32_t* dropped, void* ws, size_t ws_bytes, void* stream) {
  return moe_layer_forward_timed(cfg, wt, x, y, topk_idx, topk_w, counts, alpha, stats, dropped, ws, ws_bytes,
                                 stream, nullptr);
}

// Small batches run the whole layer in one launch (one workgroup per token):
// at a few dozen tokens the staged path is nine launches of almost no work
// each.  Every workgroup routes the whole batch and runs one token through
// its experts, so the choice is made on that per-workgroup work: the
// float64 logits of the batch and the token's expert and shared products.
// Measured on MI355X, the staged path takes 65-75 us at these sizes and the
// fused one 16 us plus about 50 ns per thousand expert multiply-adds.
// MOE_FUSED=1 takes every batch that fits, 0 none.
constexpr double kFusedAutoRouteMacs = 262144.0;
constexpr double kFusedAutoFfnMacs = 1048576.0;

static bool layer_runs_fused(const moe_config* c) {
  const int SF = c->num_shared * c->d_ff_shared;
  if (c->num_tokens <= 0 || !fused_layer_fits(c->act_dtype, c->num_tokens, c->d_model, c->num_experts, c->top_k,
                                              c->d_ff, SF))
    return false;
  const int mode = tuning().fused;
  if (mode != kUnset) return mode != 0;
  const double D = c->d_model, nm = c->activation == SWIGLU ? 2.0 : 1.0;
  const double route = (double)c->num_tokens * c->num_experts * D;
  const double ffn = (double)c->top_k * c->d_ff * D * (nm + 1.0) + 3.0 * SF * D;
  return route <= kFusedAutoRouteMacs && ffn <= kFusedAutoFfnMacs;
}

// The layer forward; routing_only: stop after the permutation (routing,
// selection and dispatch tables in the workspace, no expert or shared work:
// the backward runs the expert products itself); single_stream: every kernel
// on the caller's stream (no auxiliary stream, so nothing is created on first
// use).
static moe_status layer_forward_impl(const moe_config* cfg, const moe_weights* wt, const void* x, void* y,
                                     int32_t* topk_idx, float* topk_w, int32_t* counts, float alpha, float* stats,
                                     int32_t* dropped, void* ws, size_t ws_bytes, void* stream, void* const* ev,
                                     bool routing_only, bool single_stream = false) {
  MOE_TRY(validate_config(cfg));
  if (wt == nullptr || wt->w_router == nullptr || wt->w13 == nullptr || wt->w2 == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_shared > 0 && (wt->ws13 == nullptr || wt->ws2 == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  const bool any = cfg->num_tokens > 0;
  if (any && (x == nullptr || y == nullptr || ws == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!opt_aligned(x) || !opt_aligned(y) || !opt_aligned(topk_idx) || !opt_aligned(topk_w) ||
      !opt_aligned(counts) || !opt_aligned(stats) || !opt_aligned(dropped) || !opt_aligned(ws) ||
      !aligned16(wt->w_router) || !opt_aligned(wt->sel_bias) || !aligned16(wt->w13) || !aligned16(wt->w2) ||
      !opt_aligned(wt->ws13) || !opt_aligned(wt->ws2))
    return MOE_ERR_INVALID_ARGUMENT;
  Derived d;
  derive(cfg, &d);
  const Layout L = layer_layout(cfg, d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = cfg->num_tokens, E = cfg->num_experts, D = cfg->d_model;
  const bool want_stats = stats != nullptr || dropped != nullptr;

  if (!routing_only && layer_runs_fused(cfg)) {
    FusedArgs fa{};
    fa.x = x; fa.w_router = wt->w_router; fa.sel_bias = wt->sel_bias; fa.w13 = wt->w13; fa.w2 = wt->w2;
    fa.ws13 = cfg->num_shared > 0 ? wt->ws13 : nullptr;
    fa.ws2 = cfg->num_shared > 0 ? wt->ws2 : nullptr;
    fa.y = y; fa.topk_idx = topk_idx; fa.topk_w = topk_w; fa.counts = counts; fa.stats = stats;
    fa.dropped = dropped;
    fa.T = T; fa.D = D; fa.E = E; fa.k = cfg->top_k; fa.F = cfg->d_ff;
    fa.SF = cfg->num_shared * cfg->d_ff_shared;
    fa.scoring = cfg->scoring; fa.renormalize = cfg->renormalize; fa.activation = cfg->activation;
    fa.capacity = d.capacity; fa.alpha = alpha;
    MOE_TRY(mark(ev, MOE_STAGE_FUSED_LAYER, 0, s));
    MOE_TRY_HIP("fused layer", launch_fused_layer(fa, cfg->act_dtype, cfg->router_dtype, s));
    MOE_TRY(mark(ev, MOE_STAGE_FUSED_LAYER, 1, s));
    return MOE_OK;
  }

  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float* w = topk_w ? topk_w : at<float>(ws, L.w);
  int32_t* cnt = counts ? counts : at<int32_t>(ws, L.counts);
  int32_t* off = at<int32_t>(ws, L.offsets);
  int32_t* tp = at<int32_t>(ws, L.tile_prefix);
  int32_t* row_of = at<int32_t>(ws, L.row_of);
  int32_t* tor = at<int32_t>(ws, L.tor);
  float* probs = want_stats ? at<float>(ws, L.probs) : nullptr;

  // The shared experts' gate/up projection needs only x: it runs on the
  // auxiliary stream while routing and permutation (short, latency-bound
  // kernels that leave most of the chip idle) run here, and is joined before
  // the routed experts, which need the whole chip.
  const bool shared = !routing_only && any && cfg->num_shared > 0;
  const int SF = cfg->num_shared * cfg->d_ff_shared;
  const int overlap = shared && !single_stream ? shared_overlap() : 0;
  // The load statistics need only the probabilities and the counts: they run
  // on the auxiliary stream beside the expert GEMMs, joined at the end.
  const bool stats_aside = any && want_stats && !single_stream;
  // The shallow expert groups (when the plan splits them off) run on a second
  // auxiliary stream beside the deep ones.
  const FfnPlan ffn_plan = plan_ffn(cfg->act_dtype, cfg->activation, D, cfg->d_ff, d.rows_cap, E, true, d.group_rows);
  const int side_cus = shallow_cus(d.rows_cap, E, ffn_plan.sh_rows);
  const bool side_ffn = !routing_only && any && d.rows_cap > 0 && !single_stream && side_cus > 0 && ffn_plan.split;
  std::unique_lock<std::mutex> aux_lock(g_aux_mu, std::defer_lock);
  AuxStream* aux = nullptr;
  if (overlap > 0 || stats_aside || side_ffn) {
    aux_lock.lock();
    MOE_TRY(aux_stream(&aux));
  }
  auto fork_shared = [&]() -> moe_status {
    MOE_TRY_HIP("fork", hipEventRecord(aux->fork, s));
    MOE_TRY_HIP("fork", hipStreamWaitEvent(aux->s, aux->fork, 0));
    MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                         at<float>(ws, L.kpart_shared), aux->s, ev, MOE_STAGE_SHARED_GATE_UP, true));
    MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                         at<float>(ws, L.kpart_shared), aux->s, ev, MOE_STAGE_SHARED_DOWN, false));
    MOE_TRY_HIP("join", hipEventRecord(aux->join, aux->s));
    return MOE_OK;
  };
  if (overlap == 1 || overlap == 2) {
    MOE_TRY_HIP("fork", hipEventRecord(aux->fork, s));
    MOE_TRY_HIP("fork", hipStreamWaitEvent(aux->s, aux->fork, 0));
    MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                         at<float>(ws, L.kpart_shared), aux->s, ev, MOE_STAGE_SHARED_GATE_UP, true));
    if (overlap == 2)
      MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                           at<float>(ws, L.kpart_shared), aux->s, ev, MOE_STAGE_SHARED_DOWN, false));
    MOE_TRY_HIP("join", hipEventRecord(aux->join, aux->s));
  }

  if (any) {
    float* logits = at<float>(ws, L.logits);
    MOE_TRY(mark(ev, MOE_STAGE_ROUTER_LOGITS, 0, s));
    MOE_TRY(run_router_logits(cfg, x, wt->w_router, logits, at<void>(ws, L.wsplit), s));
    MOE_TRY(mark(ev, MOE_STAGE_ROUTER_LOGITS, 1, s));
    MOE_TRY(mark(ev, MOE_STAGE_ROUTE_SELECT, 0, s));
    MOE_TRY(run_select(cfg, logits, x, wt->w_router, wt->sel_bias, idx, w, probs, at<int32_t>(ws, L.flags), s));
    MOE_TRY(mark(ev, MOE_STAGE_ROUTE_SELECT, 1, s));
  }

  PermuteArgs pa{};
  pa.topk_idx = idx; pa.T = T; pa.k = cfg->top_k; pa.E = E;
  pa.capacity = d.capacity; pa.rows_cap = d.rows_cap;
  pa.tile_counts = at<int32_t>(ws, L.tile_counts);
  pa.counts = cnt; pa.offsets = off; pa.row_of = row_of; pa.token_of_row = tor;
  pa.tile_prefix = tp;
  pa.bm = ffn_plan.bm_up;
  MOE_TRY(mark(ev, MOE_STAGE_PERMUTE, 0, s));
  MOE_TRY_HIP("permute", launch_permute(pa, s));
  MOE_TRY(mark(ev, MOE_STAGE_PERMUTE, 1, s));
  if (debug_on() && any)
    MOE_TRY(debug_check_dispatch("moe_layer_forward", cfg, d.capacity, d.rows_cap, idx, cnt, off, row_of, tor, s));
  if (routing_only) return MOE_OK;

  StatsArgs sa{};
  if (want_stats) {
    sa.counts = cnt; sa.probs = probs; sa.partial = at<float>(ws, L.partial);
    sa.T = T; sa.E = E; sa.k = cfg->top_k; sa.capacity = d.capacity; sa.alpha = alpha;
    if (stats) { sa.f = stats; sa.P = stats + E; sa.aux_loss = stats + 2 * E; sa.imbalance = stats + 2 * E + 1; }
    sa.dropped = dropped;
  }
  if (stats_aside) {
    MOE_TRY_HIP("fork", hipEventRecord(aux->stats_fork, s));
    MOE_TRY_HIP("fork", hipStreamWaitEvent(aux->s, aux->stats_fork, 0));
    MOE_TRY(mark(ev, MOE_STAGE_LOAD_STATS, 0, aux->s));
    MOE_TRY_HIP("load stats", launch_load_stats(sa, aux->s));
    MOE_TRY(mark(ev, MOE_STAGE_LOAD_STATS, 1, aux->s));
    MOE_TRY_HIP("join", hipEventRecord(aux->stats_join, aux->s));
  }

  if (overlap == 1) MOE_TRY_HIP("join", hipStreamWaitEvent(s, aux->join, 0));
  if (overlap == 3) MOE_TRY(fork_shared());

  if (any) {
    void* h = at<void>(ws, L.h);
    void* yperm = at<void>(ws, L.yperm);
    SideStream side{};
    if (side_ffn) side = SideStream{aux->s2, aux->side_fork, aux->side_join, side_cus};
    if (d.rows_cap > 0)
      MOE_TRY(run_ffn(cfg->act_dtype, cfg->activation, E, D, cfg->d_ff, d.rows_cap, x, tor, off, tp,
                      at<int32_t>(ws, L.tile_prefix2), wt->w13, wt->w2, h, yperm, at<float>(ws, L.kpart), s, ev,
                      MOE_STAGE_EXPERT_GATE_UP, MOE_STAGE_EXPERT_DOWN, side_ffn ? &side : nullptr, d.group_rows));
    if (shared && overlap == 0)
      MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                           at<float>(ws, L.kpart_shared), s, ev, MOE_STAGE_SHARED_GATE_UP, true));
    if (shared && overlap < 2)
      MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                           at<float>(ws, L.kpart_shared), s, ev, MOE_STAGE_SHARED_DOWN, false));
    if (overlap >= 2) MOE_TRY_HIP("join", hipStreamWaitEvent(s, aux->join, 0));
    const void* y_shared = shared ? y : nullptr;
    MOE_TRY(mark(ev, MOE_STAGE_COMBINE, 0, s));
    MOE_TRY_HIP("combine", launch_combine(yperm, row_of, w, y_shared, y, T, cfg->top_k, D, cfg->act_dtype, s));
    MOE_TRY(mark(ev, MOE_STAGE_COMBINE, 1, s));
  }

  if (stats_aside) {
    MOE_TRY_HIP("join", hipStreamWaitEvent(s, aux->stats_join, 0));
  } else if (want_stats) {
    MOE_TRY(mark(ev, MOE_STAGE_LOAD_STATS, 0, s));
    MOE_TRY_HIP("load stats", launch_load_stats(sa, s));
    MOE_TRY(mark(ev, MOE_STAGE_LOAD_STATS, 1, s));
  }
  return MOE_OK;
}


moe_status moe_layer_stages(const moe_config* cfg, int32_t* runs) {
  MOE_TRY(validate_config(cfg));
  if (runs == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < MOE_NUM_STAGES; ++i) runs[i] = 0;
  if (cfg->num_tokens == 0) {
    runs[MOE_STAGE_PERMUTE] = runs[MOE_STAGE_LOAD_STATS] = 1;
    return MOE_OK;
  }
  if (layer_runs_fused(cfg)) {
    runs[MOE_STAGE_FUSED_LAYER] = 1;
    return MOE_OK;
  }
  for (int i = 0; i < MOE_NUM_STAGES; ++i) runs[i] = 1;
  runs[MOE_STAGE_FUSED_LAYER] = 0;
  if (cfg->num_shared == 0) runs[MOE_STAGE_SHARED_GATE_UP] = runs[MOE_STAGE_SHARED_DOWN] = 0;
  return MOE_OK;
}

moe_status moe_layer_forward_timed(const moe_config* cfg, const moe_weights* wt, const void* x, void* y,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts, float alpha, float* stats,
                                   int32_t* dropped, void* ws, size_t ws_bytes, void* stream,
                                   void* const* ev) {
  return layer_forward_impl(cfg, wt, x, y, topk_idx, topk_w, counts, alpha, stats, dropped, ws, ws_bytes, stream,
                            ev, false);
}

}  // extern "C"

// Scratch of the allocation-free layer forward: one array per GPU, in the
// library's device code, alive until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); it uses the device address hipGetSymbolAddress returns, looked
// up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

moe_status static_scratch(void** out) {
  int dev = 0;
  MOE_TRY_HIP("hipGetDevice", hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      MOE_TRY_HIP("scratch address", hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) {
        snprintf(g_last_error, sizeof(g_last_error), "static scratch: unusable device address");
        return MOE_ERR_HIP;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_layer_forward_static(const moe_config* cfg, const moe_weights* wt, const void* x, void* y,
                                    int32_t* topk_idx, float* topk_w, int32_t* counts, float alpha, float* stats,
                                    int32_t* dropped, void* stream) {
  MOE_TRY(validate_config(cfg));
  Derived d;
  derive(cfg, &d);
  const size_t need = layer_layout(cfg, d).total;
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES) {
    snprintf(g_last_error, sizeof(g_last_error),
             "moe_layer_forward_static: this configuration needs %zu bytes of scratch, the static scratch holds %zu",
             need, (size_t)MOE_STATIC_SCRATCH_BYTES);
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  void* ws = nullptr;
  MOE_TRY(static_scratch(&ws));
  return layer_forward_impl(cfg, wt, x, y, topk_idx, topk_w, counts, alpha, stats, dropped, ws,
                            (size_t)MOE_STATIC_SCRATCH_BYTES, stream, nullptr, false, true);
}

moe_status moe_layer_backward(const moe_config* cfg, const moe_weights* wt, const void* x, const void* dy,
                              float alpha, void* dx, float* dw_router, float* dw13, float* dw2, float* dws13,
                              float* dws2, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_config(cfg));
  if (cfg->act_dtype != BF16) return MOE_ERR_UNSUPPORTED;
  if (wt == nullptr || wt->w_router == nullptr || wt->w13 == nullptr || wt->w2 == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  const bool shared = cfg->num_shared > 0;
  if (shared && (wt->ws13 == nullptr || wt->ws2 == nullptr || dws13 == nullptr || dws2 == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (dw_router == nullptr || dw13 == nullptr || dw2 == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  const bool any = cfg->num_tokens > 0;
  if (any && (x == nullptr || dy == nullptr || dx == nullptr || ws == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!opt_aligned(x) || !opt_aligned(dy) || !opt_aligned(dx) || !aligned16(dw_router) || !aligned16(dw13) ||
      !aligned16(dw2) || !opt_aligned(dws13) || !opt_aligned(dws2) || !opt_aligned(ws) ||
      !aligned16(wt->w_router) || !aligned16(wt->w13) || !aligned16(wt->w2) || !opt_aligned(wt->ws13) ||
      !opt_aligned(wt->ws2))
    return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(validate_backward_spans(cfg));
  Derived d;
  derive(cfg, &d);
  const BwLayout B = bw_layout(cfg, d);
  if (ws_bytes < B.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = cfg->num_tokens, E = cfg->num_experts, k = cfg->top_k, D = cfg->d_model, F = cfg->d_ff;
  const int A = d.rows_cap;
  const bool swiglu = cfg->activation == SWIGLU;
  const int nF = (swiglu ? 2 : 1) * F;
  const int SF = cfg->num_shared * cfg->d_ff_shared;
  if (!any) {
    // no tokens: every gradient is zero
    MOE_TRY_HIP("zero", launch_fill_f32(dw_router, 0.0f, (long long)E * D, s));
    MOE_TRY_HIP("zero", launch_fill_f32(dw13, 0.0f, (long long)E * nF * D, s));
    MOE_TRY_HIP("zero", launch_fill_f32(dw2, 0.0f, (long long)E * D * F, s));
    if (shared) {
      MOE_TRY_HIP("zero", launch_fill_f32(dws13, 0.0f, 2LL * SF * D, s));
      MOE_TRY_HIP("zero", launch_fill_f32(dws2, 0.0f, (long long)D * SF, s));
    }
    return MOE_OK;
  }
  // forward recomputation: routing and permutation, then the expert products
  // below (the gate/up product is stored before the activation, which the
  // backward needs, and the activation is applied to it elementwise)
  void* fws = at<void>(ws, B.fwd);
  const Layout L = layer_layout(cfg, d);
  MOE_TRY(layer_forward_impl(cfg, wt, x, at<void>(ws, B.y), nullptr, nullptr, nullptr, alpha, nullptr, nullptr, fws,
                             L.total, stream, nullptr, true));
  const int32_t* idx = at<int32_t>(fws, L.idx);
  const float* tw = at<float>(fws, L.w);
  const int32_t* counts = at<int32_t>(fws, L.counts);
  const int32_t* off = at<int32_t>(fws, L.offsets);
  const int32_t* row_of = at<int32_t>(fws, L.row_of);
  const int32_t* tor = at<int32_t>(fws, L.tor);
  bf16_t* h = at<bf16_t>(fws, L.h);
  bf16_t* yperm = at<bf16_t>(fws, L.yperm);
  const float* logits = at<float>(fws, L.logits);
  bf16_t* dyp = at<bf16_t>(ws, B.dyp);
  bf16_t* gu = at<bf16_t>(ws, B.gu);
  bf16_t* dh = at<bf16_t>(ws, B.dh);
  bf16_t* dgu = at<bf16_t>(ws, B.dgu);
  bf16_t* dxp = at<bf16_t>(ws, B.dxp);
  bf16_t* w13t = at<bf16_t>(ws, B.w13t);
  bf16_t* w2t = at<bf16_t>(ws, B.w2t);
  float* dwt = at<float>(ws, B.dw);
  float* dlog = at<float>(ws, B.dlogits);
  int32_t* pre = at<int32_t>(ws, B.pre);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* dyb = static_cast<const bf16_t*>(dy);

  if (A > 0) {
    MOE_TRY(bw_gemm("expert gate/up (recomputed)", x, tor, D, wt->w13, (long long)nF * D, gu, nF, A, nF, D, E, off,
                    pre, s));
    MOE_TRY_HIP("expert activation (recomputed)", launch_act_fwd(gu, h, off + E, A, F, swiglu, s));
    MOE_TRY(bw_gemm("expert down (recomputed)", h, nullptr, F, wt->w2, (long long)D * F, yperm, D, A, D, F, E, off,
                    pre, s));
  }
  // combine: dw[t, j] = <dy[t], y_perm[row]>, dy_perm[row] = w[t, j] dy[t]
  MOE_TRY_HIP("combine backward", launch_bw_combine(dyb, yperm, row_of, tw, T, k, D, dwt, dyp, s));
  // routed experts: weights transposed for the data-gradient products
  MOE_TRY_HIP("transpose w2", launch_transpose_bf16(static_cast<const bf16_t*>(wt->w2), w2t, E, D, F, off, s));
  MOE_TRY_HIP("transpose w13", launch_transpose_bf16(static_cast<const bf16_t*>(wt->w13), w13t, E, nF, D, off, s));
  if (A > 0) {
    MOE_TRY(bw_gemm("expert dH", dyp, nullptr, D, w2t, (long long)F * D, dh, F, A, F, D, E, off, pre, s));
    MOE_TRY_HIP("activation backward", launch_bw_act(gu, dh, dgu, off + E, A, F, swiglu, s));
    MOE_TRY(bw_gemm("expert dX", dgu, nullptr, nF, w13t, (long long)D * nF, dxp, D, A, D, nF, E, off, pre + (E + 1),
                    s));
  }
  MOE_TRY_HIP("expert dW2", launch_wgrad(dyp, D, h, F, nullptr, off, E, A, D, F, dw2, s));
  MOE_TRY_HIP("expert dW13", launch_wgrad(dgu, nF, xb, D, tor, off, E, A, nF, D, dw13, s));
  // shared experts (weight 1, every token)
  bf16_t* dxs = nullptr;
  if (shared) {
    bf16_t* gus = at<bf16_t>(ws, B.gus);
    bf16_t* dhs = at<bf16_t>(ws, B.dhs);
    bf16_t* dgus = at<bf16_t>(ws, B.dgus);
    bf16_t* ws13t = at<bf16_t>(ws, B.ws13t);
    bf16_t* ws2t = at<bf16_t>(ws, B.ws2t);
    dxs = at<bf16_t>(ws, B.dxs);
    bf16_t* hs = at<bf16_t>(fws, L.h_shared);
    MOE_TRY_HIP("transpose ws2", launch_transpose_bf16(static_cast<const bf16_t*>(wt->ws2), ws2t, 1, D, SF, nullptr, s));
    MOE_TRY_HIP("transpose ws13", launch_transpose_bf16(static_cast<const bf16_t*>(wt->ws13), ws13t, 1, 2 * SF, D, nullptr, s));
    MOE_TRY(bw_gemm("shared gate/up (recomputed)", x, nullptr, D, wt->ws13, 0, gus, 2 * SF, T, 2 * SF, D, 1, nullptr,
                    nullptr, s));
    MOE_TRY_HIP("shared activation (recomputed)", launch_act_fwd(gus, hs, nullptr, T, SF, true, s));
    MOE_TRY(bw_gemm("shared dH", dy, nullptr, D, ws2t, 0, dhs, SF, T, SF, D, 1, nullptr, nullptr, s));
    MOE_TRY_HIP("shared activation backward", launch_bw_act(gus, dhs, dgus, nullptr, T, SF, true, s));
    MOE_TRY(bw_gemm("shared dX", dgus, nullptr, 2 * SF, ws13t, 0, dxs, D, T, D, 2 * SF, 1, nullptr, nullptr, s));
    MOE_TRY_HIP("shared dW2", launch_wgrad(dyb, D, hs, SF, nullptr, nullptr, 1, T, D, SF, dws2, s));
    MOE_TRY_HIP("shared dW13", launch_wgrad(dgus, 2 * SF, xb, D, nullptr, nullptr, 1, T, 2 * SF, D, dws13, s));
  }
  // router: d loss / d logits, then its weight and input gradients
  MOE_TRY_HIP("router backward", launch_router_grad(logits, idx, tw, dwt, counts, T, E, k, cfg->scoring,
                                                    cfg->renormalize, alpha, dlog, s));
  // on the matrix cores where the shapes allow (the exact three-plane split
  // of the logit gradients keeps every product exact), else float32 FMA
  float* dxr = at<float>(ws, B.dxr);
  const bool mfma_dw = E % 4 == 0 && D % 4 == 0;
  const bool mfma_dx = mfma_dw && T % 4 == 0 && cfg->router_dtype == BF16;
  if (mfma_dw) {
    MOE_TRY_HIP("router gradients", launch_router_grad_mfma(dlog, xb, static_cast<const bf16_t*>(wt->w_router), T, E,
                                                            D, dw_router, mfma_dx ? dxr : nullptr,
                                                            at<bf16_t>(ws, B.rplanes), at<bf16_t>(ws, B.rplanes_t),
                                                            at<int32_t>(ws, B.raux), at<float>(ws, B.rpart), s));
  } else {
    MOE_TRY_HIP("router dW", launch_gemm_f32_strided(dlog, 1, E, x, true, D, 1, E, D, T, dw_router,
                                                     at<float>(ws, B.rpart), s));
  }
  if (!mfma_dx)
    MOE_TRY_HIP("router dx", launch_gemm_f32_strided(dlog, E, 1, wt->w_router, cfg->router_dtype == BF16, D, 1, T,
                                                     D, E, dxr, nullptr, s));
  // dx = sum of the token's expert rows (weight 1) + shared + router
  float* ones = at<float>(ws, B.ones);
  MOE_TRY_HIP("ones", launch_fill_f32(ones, 1.0f, (long long)T * k, s));
  MOE_TRY_HIP("dx rows", launch_combine(dxp, row_of, ones, dxs, dx, T, k, D, BF16, s));
  MOE_TRY_HIP("dx router", launch_add_f32_to_bf16(static_cast<bf16_t*>(dx), dxr, (long long)T * D, s));
  return MOE_OK;
}

moe_status moe_expert_choice_capacity(const moe_config* cfg, int32_t* capacity) {
  MOE_TRY(validate_ec(cfg));
  if (capacity == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  *capacity = ec_capacity(cfg);
  return MOE_OK;
}

moe_status moe_expert_choice_forward(const moe_config* cfg, const moe_weights* wt, const void* x, void* y,
                                     int32_t* token_of_row, float* row_w, int32_t* unselected,
                                     void* ws, size_t ws_bytes, void* stream, void* const* ev) {
  MOE_TRY(validate_ec(cfg));
  if (wt == nullptr || wt->w_router == nullptr || wt->w13 == nullptr || wt->w2 == nullptr)
    return MOE_ERR_INVALID_ARGUMENT;
  if (cfg->num_shared > 0 && (wt->ws13 == nullptr || wt->ws2 == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  const bool any = cfg->num_tokens > 0;
  if (any && (x == nullptr || y == nullptr || ws == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!opt_aligned(x) || !opt_aligned(y) || !opt_aligned(token_of_row) || !opt_aligned(row_w) ||
      !opt_aligned(unselected) || !opt_aligned(ws) || !aligned16(wt->w_router) || !aligned16(wt->w13) ||
      !aligned16(wt->w2) || !opt_aligned(wt->ws13) || !opt_aligned(wt->ws2))
    return MOE_ERR_INVALID_ARGUMENT;
  const EcLayout L = ec_layout(cfg);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!any) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = cfg->num_tokens, E = cfg->num_experts, D = cfg->d_model, F = cfg->d_ff;
  const int C = ec_capacity(cfg);
  const int SF = cfg->num_shared * cfg->d_ff_shared;
  int32_t* tor = token_of_row ? token_of_row : at<int32_t>(ws, L.tor);
  float* roww = row_w ? row_w : at<float>(ws, L.roww);
  int32_t* off = at<int32_t>(ws, L.offsets);
  int32_t* prefix_up = at<int32_t>(ws, L.prefixes);
  float* pT = at<float>(ws, L.pT);
  uint32_t* selbits = at<uint32_t>(ws, L.selbits);
  int32_t* selpre = at<int32_t>(ws, L.selpre);
  float* logits = at<float>(ws, L.logits);

  MOE_TRY(mark(ev, MOE_STAGE_ROUTER_LOGITS, 0, s));
  MOE_TRY(run_router_logits(cfg, x, wt->w_router, logits, at<void>(ws, L.wsplit), s));
  MOE_TRY(mark(ev, MOE_STAGE_ROUTER_LOGITS, 1, s));
  MOE_TRY(mark(ev, MOE_STAGE_ROUTE_SELECT, 0, s));
  MOE_TRY_HIP("expert-choice route", launch_ec_route(logits, T, E, C, pT, off, tor, roww, selbits, selpre,
                                                     unselected, s));
  MOE_TRY(mark(ev, MOE_STAGE_ROUTE_SELECT, 1, s));
  // every expert takes exactly C rows
  const FfnPlan pl = plan_ffn(cfg->act_dtype, cfg->activation, D, F, E * C, E, true, C);
  if (!pl.split) MOE_TRY_HIP("tile prefix", launch_tile_prefix(off, E, pl.bm_up, prefix_up, s));
  MOE_TRY(run_ffn(cfg->act_dtype, cfg->activation, E, D, F, E * C, x, tor, off, prefix_up, prefix_up + (E + 1),
                  wt->w13, wt->w2, at<void>(ws, L.h), at<void>(ws, L.yperm), at<float>(ws, L.kpart), s, ev,
                  MOE_STAGE_EXPERT_GATE_UP, MOE_STAGE_EXPERT_DOWN, nullptr, C));
  if (cfg->num_shared > 0) {
    MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                         at<float>(ws, L.kpart_shared), s, ev, MOE_STAGE_SHARED_GATE_UP, true));
    MOE_TRY(run_ffn_part(cfg->act_dtype, SWIGLU, 1, D, SF, T, x, wt->ws13, wt->ws2, at<void>(ws, L.h_shared), y,
                         at<float>(ws, L.kpart_shared), s, ev, MOE_STAGE_SHARED_DOWN, false));
  }
  MOE_TRY(mark(ev, MOE_STAGE_COMBINE, 0, s));
  MOE_TRY_HIP("expert-choice combine", launch_ec_combine(at<void>(ws, L.yperm), pT, selbits, selpre,
                                                         cfg->num_shared > 0 ? y : nullptr, y, T, E, C, D,
                                                         cfg->act_dtype, unselected, s));
  MOE_TRY(mark(ev, MOE_STAGE_COMBINE, 1, s));
  return MOE_OK;
}

moe_status moe_ep_send_layout(int32_t num_experts, int32_t num_ranks, const int32_t* offsets,
                              int32_t* send_counts, int32_t* send_offsets, void* stream) {
  if (num_experts <= 0 || num_ranks <= 0 || num_ranks > num_experts || num_experts % num_ranks != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (num_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (offsets == nullptr || send_counts == nullptr || send_offsets == nullptr) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY_HIP("ep send layout", launch_ep_send_layout(offsets, num_experts, num_ranks, send_counts, send_offsets,
                                                      static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_ep_recv_layout(int32_t num_ranks, int32_t local_experts, const int32_t* recv_counts,
                              int32_t rows_cap, int32_t* local_offsets, int32_t* gather, void* stream) {
  if (num_ranks <= 0 || local_experts <= 0 || rows_cap < 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((long long)num_ranks * local_experts > 65536 || local_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (recv_counts == nullptr || local_offsets == nullptr || (rows_cap > 0 && gather == nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY_HIP("ep receive layout", launch_ep_recv_layout(recv_counts, num_ranks, local_experts, rows_cap,
                                                         local_offsets, gather, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

}  // extern "C"
