// Internal helpers shared by the HIP sources of the MoE layer library.
// Not part of the C ABI (see include/moe.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <atomic>

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kNumXcd = 8;         // MI355X: 8 accelerator complex dies, one L2 each

enum Dtype { F32 = 0, BF16 = 1 };
enum Scoring { SOFTMAX_TOPK = 0, TOPK_SOFTMAX = 1, SIGMOID_BIAS = 2 };
enum Activation { SWIGLU = 0, GELU = 1 };

typedef uint16_t bf16_t;   // bfloat16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Workgroups are dealt to the XCDs round-robin (workgroup i runs on XCD i % 8).
// Renumber them so that each XCD works on one contiguous range of logical
// tiles, which then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % kNumXcd;
  const int local = bid / kNumXcd;
  const int per = nblocks / kNumXcd;
  const int rem = nblocks % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Compute units of the current device (cached after the first call).
// Tuning aids (MOE_* environment variables forcing a kernel choice), read
// once per process; kUnset where a variable is not set.  Launch paths take a
// copy from tuning() and never call getenv.
constexpr int kUnset = -2147483647 - 1;
struct Tuning {
  int router_kernel = kUnset;    // MOE_ROUTER_KERNEL: 0 keeps the router on the general GEMM
  int router_path = kUnset;      // MOE_ROUTER_PATH: tiled (0) / split (1) / gemv (2)
  int gemm_cfg = kUnset;         // MOE_GEMM_CFG: tile configuration of the grouped GEMMs
  int gemm_cfg_down = kUnset;    // MOE_GEMM_CFG_DOWN: ... of the down projection alone
  int gemm_ksplit = kUnset;      // MOE_GEMM_KSPLIT: contraction split of weight-streaming launches
  int gemm_shcfg = kUnset;       // MOE_GEMM_SHCFG: configuration of the shallow groups
  int gemm_split = kUnset;       // MOE_GEMM_SPLIT: 0 / 1 shallow-group split off / on
  int gemm_tail = kUnset;        // MOE_GEMM_TAIL: 0 turns the last-round split off
  int shared_overlap = kUnset;   // MOE_SHARED_OVERLAP: 0 / 1 / 2
  int shallow_cus = kUnset;      // MOE_SHALLOW_CUS: CUs of the concurrent shallow-group launch (0 = in line)
  int tile_gm = kUnset;          // MOE_TILE_GM: m-tiles per run of the grouped GEMMs' tile order
  int wgrad_tile = kUnset;       // MOE_WGRAD_TILE: 128 / 256
  int wgrad_swz = kUnset;        // MOE_WGRAD_SWZ: 0 / 1 / 2
  int fused = kUnset;            // MOE_FUSED: 1 / 0 one-workgroup layer for every / no batch that fits
  int debug = kUnset;            // MOE_DEBUG: 1 checks the dispatch tables on the host (synchronises)
  int shallow_rows = kUnset;     // MOE_SHALLOW_ROWS: groups of at most this many rows count as shallow
};
Tuning tuning();

inline int num_cus() {
  static std::atomic<int> cached{0};     // host threads may race to fill it: same value
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

// gelu(z) = z * Phi(z) = z/2 * erfc(-z/sqrt(2)) for outputs rounded to bf16.
// erfc(a), a >= 0, from Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7):
// erfc(a) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-a^2), t = 1 / (1 + p a).
// For z < 0 the result is z/2 * erfc(|x|) directly, so small values keep
// their relative accuracy instead of coming out of 1 - erf.  Evaluated on
// y = x * sqrt(log2 e), so that exp(-x^2) = 2^(-y^2) is one hardware exp2 and
// p a = (p / sqrt(log2 e)) |y|.
__device__ __forceinline__ float gelu_bf16out(float z) {
  const float y = z * 0.84932180028801907f;               // z / sqrt(2) * sqrt(log2 e)
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.27273748087922250f * fabsf(y));
  const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float c = poly * __builtin_amdgcn_exp2f(-y * y);  // erfc(|z| / sqrt(2))
  return 0.5f * z * (y >= 0.0f ? 2.0f - c : c);
}

// float32 -> bfloat16 bit pattern by the hardware conversion (round to
// nearest even), for kernel outputs.
__device__ __forceinline__ bf16_t f32_to_bf16_rn(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

// silu(z) = z * sigmoid(z); the reciprocal is the hardware one (1 ulp), which
// keeps the result within a few ulp of the float32 quotient.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float gelu_erf_f32(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// ---------------------------------------------------------------------------
// Launchers implemented in the .hip files (all enqueue on `stream`).
// ---------------------------------------------------------------------------

// Epilogue kinds of the grouped GEMM C[r, n] = sum_k A[r, k] * B_g[n, k].
enum Epilogue {
  EPI_STORE_F32 = 0,   // C float32
  EPI_STORE_ACT = 1,   // C in the activation type
  EPI_SWIGLU = 2,      // B rows n and F+n are gate and up: H = silu(g) * u
  EPI_GELU = 3,        // H = gelu(C)
  EPI_TAIL_PART = 4,   // float32 sums of one unit of the split tail (tail_mode 2)
};

struct GroupedGemm {
  const void* A;              // rows of K elements (act type)
  const int32_t* a_rows;      // [M_max] gather map or nullptr
  int lda;
  const void* B;              // [G][rows_b][K]
  long long b_group_stride;   // elements
  void* C;                    // [M_max][ldc]
  int ldc;
  int M_max, N, K;            // N = output columns (SwiGLU: F)
  int G;
  const int32_t* offsets;     // [G+1] or nullptr (one group of M_max rows)
  const int32_t* tile_prefix; // [G+1] m-tile prefix for the kernel's BM (grouped case)
  int epilogue;
  int a_kwrap;                // 0, or: A column k is read at k % a_kwrap (a multiple of 64)
  // Last-round split of a tiled launch (non-persistent kernels, map_tile):
  // 0: every tile;
  // 1: only the tiles of the full rounds, the first (total / round) * round
  //    tiles of the order (round = workgroups that run at once);
  // 2: the remaining tiles, each as S units over consecutive K / S slices
  //    (S from tail_units, so that S times the remaining tiles fill at most
  //    one round): unit b writes its float32 sums as block b of BM x BN floats
  //    at `tail_part` (epilogue EPI_TAIL_PART; the buffer holds `tail_cap`
  //    blocks), and tail_reduce adds each tile's S blocks in order into C
  //    (with S = 1 the units store their tiles into C themselves).
  int tail_mode;
  int round;
  // Persistent launches: CUs the grid may occupy (0 = all of them), so that
  // a launch can run beside another one on the remaining CUs.
  int cus;
  // m-tiles per run of the tile order that sweeps a group's n-tiles (0 = 8)
  int tile_gm;
  // Split of the contraction (weight-streaming kernel only): with ksplit > 1
  // every tile runs as ksplit units over consecutive K / ksplit slices; each
  // unit writes its float32 sums to partial[(ks * M_max + row) * ldp + col]
  // (SwiGLU: gate column h at col h, up column h at col N + h; ldp >= 2N,
  // else ldp >= N), and a second kernel adds the ksplit parts in a fixed
  // order and applies the epilogue.  0 or 1: no split.
  int ksplit;
  float* partial;
  int ldp;
  float* tail_part;   // tail_mode 2: float32 unit blocks (tail_cap of BM x BN)
  int tail_cap;
};

// Exact split of a float32 matrix into three bfloat16 planes, hi + mid + lo = w:
// out[e][j][d] = plane j of w[e][d], out has [E][3][D] layout.
hipError_t launch_split_bf16x3(const float* w, int E, int D, bf16_t* out, hipStream_t s);

// Tile order of the grouped GEMMs.  The tiles that exist (known on the device
// only) are numbered group by group; inside a group, runs of up to 8 m-tiles
// sweep all n-tiles, so the blocks that run together share both the group's
// weight tiles and its activation rows in L2.  decode_tile maps logical tile L
// (below tile_count) to group g, first row of the tile, rows in the tile and
// n-tile.
template <int BM>
__device__ __forceinline__ int tile_count(const GroupedGemm& p, int n_tiles) {
  return (p.offsets == nullptr ? ceil_div(p.M_max, BM) : p.tile_prefix[p.G]) * n_tiles;
}

//
// SCALAR: the tables are read through the constant address space, so that
// (uniform) reads become scalar loads, which a kernel with vector loads in
// flight can wait for without waiting for those.
typedef const __attribute__((address_space(4))) int32_t const_i32;
#ifndef MOE_TILE_GM
#define MOE_TILE_GM 8          // m-tiles per run that sweeps the n-tiles
#endif
template <bool SCALAR>
__device__ __forceinline__ int ld_table(const int32_t* t, int i) {
  if constexpr (SCALAR) return ((const_i32*)t)[i];
  else return t[i];
}

template <int BM, bool SCALAR = false>
__device__ __forceinline__ void decode_tile(const GroupedGemm& p, int n_tiles, int L, int& g, int& row0, int& rows,
                                            int& nt) {
  const int GM = p.tile_gm > 0 ? p.tile_gm : MOE_TILE_GM;
  if (p.offsets == nullptr) {
    const int mt_all = ceil_div(p.M_max, BM);
    const int sub = L / (GM * n_tiles);
    const int first = sub * GM;
    const int gm = min(mt_all - first, GM);
    const int loc = L - sub * GM * n_tiles;
    const int mt = first + loc % gm;
    nt = loc / gm;
    g = 0;
    row0 = mt * BM;
    rows = min(BM, p.M_max - row0);
    return;
  }
  const int* tp = p.tile_prefix;
  const int mtile = L / n_tiles;          // tiles of group g are [tp[g] n, tp[g+1] n)
  int lo = 0, hi = p.G;                   // tp[lo] <= mtile < tp[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_table<SCALAR>(tp, mid) <= mtile) lo = mid; else hi = mid;
  }
  g = lo;                                 // last group starting at or before: non-empty
  const int tg = ld_table<SCALAR>(tp, g);
  const int mg = ld_table<SCALAR>(tp, g + 1) - tg;
  const int local = L - tg * n_tiles;
  const int sub = local / (GM * n_tiles);
  const int first = sub * GM;
  const int gm = min(mg - first, GM);
  const int loc = local - sub * GM * n_tiles;
  const int m = first + loc % gm;
  nt = loc / gm;
  row0 = ld_table<SCALAR>(p.offsets, g) + m * BM;
  rows = min(BM, ld_table<SCALAR>(p.offsets, g + 1) - row0);
}

// Tile of this workgroup in a grid sized for the upper bound of tiles:
// workgroup ids are dealt so that every XCD gets one contiguous, equally long
// stretch of the tile order.  Returns false for workgroups beyond the last
// tile.
template <int BM>
__device__ __forceinline__ bool map_tile(const GroupedGemm& p, int n_tiles, int& g, int& row0, int& rows,
                                         int& nt) {
  const int bid = blockIdx.x;
  int total = tile_count<BM>(p, n_tiles);
  if (p.tail_mode == 1) total = total / p.round * p.round;
  if (bid >= total) return false;
  decode_tile<BM>(p, n_tiles, xcd_remap(bid, total), g, row0, rows, nt);
  return true;
}

// m-tile prefix for grouped GEMMs: prefix[g] = sum_{h<g} ceil((off[h+1]-off[h]) / bm).
hipError_t launch_tile_prefix(const int32_t* offsets, int G, int bm, int32_t* prefix, hipStream_t s);
// m-tile prefixes restricted to a class of groups: group h counts
// ceil(n_h / bm) m-tiles when lo < n_h <= hi and none otherwise.  Up to three
// prefixes in one launch (unused ones: out == nullptr).
struct TilePrefixReq {
  int32_t* out;
  int bm, lo, hi;
};
hipError_t launch_tile_prefix_classes(const int32_t* offsets, int G, TilePrefixReq r0, TilePrefixReq r1,
                                      TilePrefixReq r2, hipStream_t s);

// Units of the split tail (tail_mode 2): of `total` tiles, the first `main`
// fill whole rounds; each of the r left over runs as S units, S the largest
// power of two up to 8 with S * r <= round that divides the nk slices and
// leaves at least four per unit (1 if none does).
__host__ __device__ inline void tail_units(int total, int round, int nk, int& main, int& r, int& S) {
  main = total / round * round;
  r = total - main;
  S = 1;
  while (S < 8 && 2 * S * r <= round && nk % (2 * S) == 0 && nk / (2 * S) >= 4) S *= 2;
}
// The split tail's sum of units and store (tail_mode 2), after its GEMM launch.
hipError_t launch_tail_reduce(const GroupedGemm& g, hipStream_t s);

// bf16 MFMA grouped GEMM; returns the BM its tiles use via bm_out when non-null.
hipError_t launch_gemm_bf16(const GroupedGemm& g, hipStream_t s);
int gemm_bf16_bm(const GroupedGemm& g);
// bf16 grouped GEMM for deep groups (K % 64 == 0, or % 32 for the 32-deep
// configurations): tile configurations 0 .. kGemmV3Configs-1.
constexpr int kGemmV3Configs = 14;
hipError_t launch_gemm_v3(const GroupedGemm& g, int cfg, hipStream_t s);
int gemm_v3_bm(int cfg);
// Persistent weight-streaming bf16 grouped GEMM for shallow groups (K % 64 ==
// 0); its tile configurations follow in the same numbering: kGemmV3Configs +
// cfg.
constexpr int kGemmWsConfigs = 8;
hipError_t launch_gemm_ws(const GroupedGemm& g, int cfg, hipStream_t s);
int gemm_ws_bm(int cfg);
int gemm_ws_bn(int cfg);
constexpr int kGemmConfigs = kGemmV3Configs + kGemmWsConfigs;
// float32 SIMT grouped GEMM.  a_dtype / b_dtype select float32 or bf16 operands.
hipError_t launch_gemm_f32(const GroupedGemm& g, int a_dtype, int b_dtype, hipStream_t s);
constexpr int kF32GemmBM = 64;

// Router logits for bf16 tokens and bf16 weights [E, planes, D] (planes = 1,
// or 3 for the exact plane split of float32 weights): logits [T, E] float32.
// router_kernel_fits tells whether the shape is one it handles (D % 64 == 0,
// E <= 256 for one plane, <= 128 for three).
bool router_kernel_fits(int T, int E, int D, int planes);
hipError_t launch_router_logits(const bf16_t* x, const bf16_t* w, int planes, float* logits, int T, int E, int D,
                                hipStream_t s);

struct RouteArgs {
  const float* logits;        // [T, E]
  const void* x;              // [T, D] act type (near-tie refinement)
  const void* w_router;       // [E, D] router type
  const float* sel_bias;      // [E] or nullptr
  int32_t* topk_idx;          // [T, k]
  float* topk_w;              // [T, k]
  float* probs;               // [T, E] or nullptr
  int T, D, E, k;
  int scoring, renormalize, act_dtype, router_dtype;
};
// flags: [T] int32 scratch (tokens that need the float64 refinement pass).
hipError_t launch_route_select(const RouteArgs& a, int32_t* flags, hipStream_t s);

struct PermuteArgs {
  const int32_t* topk_idx;    // [T, k]
  int T, k, E;
  int capacity;               // INT32_MAX when dropless
  int rows_cap;               // A_cap
  int32_t* tile_counts;       // ws [ntiles][E]
  int32_t* counts;            // [E]
  int32_t* offsets;           // [E+1]
  int32_t* row_of;            // [T, k]
  int32_t* token_of_row;      // [A_cap]
  int32_t* tile_prefix;       // [E+1] m-tile prefix for bm (or nullptr)
  int bm;
};
constexpr int kPermuteTile = 256;   // tokens per histogram / scatter block
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// Expert-choice routing and combine (expert_choice.hip): E <= 256 experts,
// T <= 8192 tokens (the sort keys of one expert's column sit in LDS).
constexpr int kEcMaxExperts = 256;
constexpr int kEcMaxTokens = 8192;
hipError_t launch_ec_route(const float* logits, int T, int E, int C, float* pT, int32_t* offsets,
                           int32_t* token_of_row, float* row_w, uint32_t* selbits, int32_t* selpre,
                           int32_t* unselected, hipStream_t s);
hipError_t launch_ec_combine(const void* y_perm, const float* pT, const uint32_t* selbits, const int32_t* selpre,
                             const void* y_shared, void* y, int T, int E, int C, int D, int act_dtype,
                             int32_t* unselected, hipStream_t s);
// Backward pass kernels (backward.hip).
hipError_t launch_transpose_bf16(const bf16_t* in, bf16_t* out, int G, int R, int C, const int32_t* offsets,
                                 hipStream_t s);
hipError_t launch_bw_combine(const bf16_t* dy, const bf16_t* yp, const int32_t* row_of, const float* tw, int T, int k,
                             int D, float* dw, bf16_t* dyp, hipStream_t s);
hipError_t launch_act_fwd(const bf16_t* gu, bf16_t* h, const int32_t* rows_valid, int rows_max, int F, bool swiglu,
                          hipStream_t s);
hipError_t launch_bw_act(const bf16_t* gu, const bf16_t* dh, bf16_t* dgu, const int32_t* rows_valid, int rows_max,
                         int F, bool swiglu, hipStream_t s);
hipError_t launch_wgrad(const bf16_t* A, int lda, const bf16_t* B, int ldb, const int32_t* b_rows,
                        const int32_t* offsets, int G, int rows_max, int M, int N, float* C, hipStream_t s);
hipError_t launch_router_grad(const float* logits, const int32_t* idx, const float* tw, const float* dw,
                              const int32_t* counts, int T, int E, int k, int scoring, int renormalize, float alpha,
                              float* dlogits, hipStream_t s);
// partial: NULL, or room for kF32MaxSplit * M * N floats (the contraction is
// then split over up to that many parts when the output tiles are few).
constexpr int kF32MaxSplit = 32;
hipError_t launch_gemm_f32_strided(const float* A, long long am, long long ak, const void* B, bool b_bf16,
                                   long long bk, long long bn, int M, int N, int K, float* C, float* partial,
                                   hipStream_t s);
// Router gradients on the matrix cores: dlogits [T, E] (float32) split
// exactly into three bf16 planes; dW_router [E, D] = dlogits^T x over up to
// kRouterMfmaSplit token chunks (partial: room for 3 kRouterMfmaSplit E D
// floats), and, when dx_router is given (T % 4 == 0, bf16 w_router [E, D]),
// dx_router [T, D] = dlogits w_router.  planes [T][3E], planes_t [3E][T],
// aux: kRouterMfmaSplit + 1 + 3E ints.  E % 4 == 0 and D % 4 == 0.
constexpr int kRouterMfmaSplit = 10;
hipError_t launch_router_grad_mfma(const float* dlog, const bf16_t* x, const bf16_t* w_router, int T, int E, int D,
                                   float* dw_router, float* dx_router, bf16_t* planes, bf16_t* planes_t,
                                   int32_t* aux, float* partial, hipStream_t s);
hipError_t launch_add_f32_to_bf16(bf16_t* y, const float* add, long long n, hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, long long n, hipStream_t s);
// Expert-parallel send / receive layouts (ep.hip).
hipError_t launch_ep_send_layout(const int32_t* offsets, int E, int R, int32_t* send_counts, int32_t* send_offsets,
                                 hipStream_t s);
hipError_t launch_ep_recv_layout(const int32_t* recv_counts, int R, int El, int rows_cap, int32_t* local_offsets,
                                 int32_t* gather, hipStream_t s);
hipError_t launch_gather_rows(const void* x, const int32_t* token_of_row, const int32_t* offsets,
                              int E, int rows_cap, int D, int elem_bytes, void* x_perm,
                              hipStream_t s);

hipError_t launch_combine(const void* y_perm, const int32_t* row_of, const float* topk_w,
                          const void* y_shared, void* y, int T, int k, int D, int act_dtype,
                          hipStream_t s);

struct StatsArgs {
  const int32_t* counts;      // [E]
  const float* probs;         // [T, E]
  float* partial;             // ws [nchunks][E]
  int T, E, k, capacity;
  float alpha;
  float* f; float* P; float* aux_loss; float* imbalance; int32_t* dropped;
};
constexpr int kStatsChunk = 64;     // tokens per partial-sum block (multiple of 4)
hipError_t launch_load_stats(const StatsArgs& a, hipStream_t s);

// Whole layer forward in one workgroup for small batches (fused.hip).
struct FusedArgs {
  const void* x;              // [T, D] act dtype
  const void* w_router;       // [E, D] router dtype
  const float* sel_bias;      // [E] or nullptr
  const void* w13;            // [E, 2F or F, D]
  const void* w2;             // [E, D, F]
  const void* ws13;           // [2 SF, D] or nullptr
  const void* ws2;            // [D, SF]
  void* y;                    // [T, D] act dtype out
  int32_t* topk_idx;          // [T, k] or nullptr
  float* topk_w;              // [T, k] or nullptr
  int32_t* counts;            // [E] or nullptr
  float* stats;               // [2E + 2] or nullptr
  int32_t* dropped;           // [1] or nullptr
  int T, D, E, k, F, SF;      // SF = S * F_s (0 = no shared experts)
  int scoring, renormalize, activation, capacity;
  float alpha;
};
constexpr int kFusedMaxTokens = 256;

// Host-side checks of dispatch tables in host memory (checks.hip); false
// with a message in msg when a table breaks its definition.
bool check_group_offsets(const int32_t* off, int G, int max_rows, char* msg, size_t n);
bool check_gather_rows(const int32_t* rows, int n_rows, char* msg, size_t n);
bool check_row_map(const int32_t* row_of, int T, int k, int rows_cap, char* msg, size_t n);
bool check_dispatch(const int32_t* idx, const int32_t* counts, const int32_t* offsets, const int32_t* row_of,
                    const int32_t* tor, int T, int k, int E, int capacity, int rows_cap, char* msg, size_t n);
// Sets the library's last error message (api.hip).
void debug_message(const char* where, const char* msg);
bool fused_layer_fits(int act_dtype, int T, int D, int E, int k, int F, int SF);
hipError_t launch_fused_layer(const FusedArgs& a, int act_dtype, int router_dtype, hipStream_t s);

}  // namespace moe
