// Router logits s[t, e] = sum_d x[t, d] w[e, d] for bf16 tokens and bf16
// weights given as NP planes (NP = 1: the weights; NP = 3: the exact split of
// float32 weights into hi + mid + lo made by launch_split_bf16x3), for
// E <= 256 and D a multiple of 64 ("Top-k 路由" page, step 1 of the gate: one
// bias-free linear layer).
//
// 65 <= E <= 256 and many tokens: one workgroup owns a block of BM tokens and
// BN experts (router_shape picks the block that moves the fewest bytes per
// CU; every token fragment feeds NP MFMAs).  Operands stream through an LDS
// ring (up to 4 deep) of 64-deep K slices (buffer loads with the LDS bit).
// At most 16 tokens (rows fitting in LDS): one wave per expert
// (router_gemv_kernel below).
// E <= 64, or few tokens: one workgroup owns 16 tokens and up to 64 experts
// (every expert when E <= 64; blocks of 16 experts side by side in the grid
// when the tokens are few and the experts many); its eight waves split the
// contraction (wave w takes the 32-deep steps w, w + 8, ...), load their
// operands straight into registers for 16x16x32 MFMAs, and add their partial
// sums in LDS at the end in a fixed order.
// Either way the MFMA sums of at most 64 products per plane are added into
// float64 accumulators, which keeps the logits within a small multiple of
// float32 rounding of the exact sum, as the selection's near-tie refinement
// requires.
#include "common.h"

#include <algorithm>
#include <cstdlib>
#include <cstring>

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void lds_void_r;

__device__ __forceinline__ void dma16_r(__amdgpu_buffer_rsrc_t r, unsigned voff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_r*)lds, 16, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm_r() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 128-byte rows (64 bf16), chunk c of row r in slot c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz_r(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// A workgroup owns BM tokens and BN experts (the grid's y dimension runs over
// blocks of BN experts); its four waves are laid out WGM x WGN over them, each
// owning 32 tokens and BN / WGN experts.
template <int BM, int BN, int NP>
struct RCfg {
  static constexpr int WGM = BM / 32, WGN = 4 / WGM;  // wave layout
  static constexpr int XB = BM * 128, WB = NP * BN * 128;  // bytes per slice
  static constexpr int STAGE = XB + WB;
  static constexpr int NST = (160 * 1024) / STAGE < 4 ? (160 * 1024) / STAGE : 4;
  static constexpr int X_INS = XB / 1024 / 4, W_INS = WB / 1024 / 4;   // per wave per slice
  static constexpr int INS = X_INS + W_INS;
  static constexpr int WN = BN / WGN;                 // experts per wave
  static constexpr int TN = WN / 32;                  // 32-column blocks per wave
  static_assert(WGM >= 1 && WGM * WGN == 4 && BM == 32 * WGM, "wave layout");
  static_assert(XB % 4096 == 0 && WB % 4096 == 0, "load split");
  static_assert(TN >= 1 && WN % 32 == 0, "wave tile");
  static_assert(NST >= 2 && STAGE * NST <= 160 * 1024, "LDS");
  static_assert(INS * (NST - 2) <= 63, "vmcnt range");
};

template <int BM, int BN, int NP>
__global__ __launch_bounds__(256) void router_logits_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                            float* __restrict__ logits, int T, int E, int D) {
  using C = RCfg<BM, BN, NP>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int row0 = blockIdx.x * BM;
  const int rows = min(BM, T - row0);
  const int e0 = blockIdx.y * BN;
  const int nk = D / 64;

  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(x), 0, (int)0xffffffffu, 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(w), 0, (int)((unsigned)E * NP * (unsigned)D * 2u), 0x00020000);
  // byte offsets of this wave's loads at slice 0 (rows past the end clamped);
  // the weight slice holds plane p of BN rows at LDS rows p*BN ..
  unsigned x_off[C::X_INS], w_off[C::W_INS];
#pragma unroll
  for (int q = 0; q < C::X_INS; ++q) {
    const int r = (wave * C::X_INS + q) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    x_off[q] = ((unsigned)(row0 + min(r, rows - 1)) * (unsigned)D + c * 8) * 2u;
  }
#pragma unroll
  for (int q = 0; q < C::W_INS; ++q) {
    const int r = (wave * C::W_INS + q) * 8 + (lane >> 3);     // LDS row: plane r / BN, expert r % BN
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const unsigned e = (unsigned)min(e0 + r % BN, E - 1), pl = (unsigned)(r / BN);
    w_off[q] = ((e * NP + pl) * (unsigned)D + c * 8) * 2u;
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    char* st = smem + (kt % C::NST) * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::X_INS; ++q) dma16_r(x_rsrc, x_off[q] + kt * 128u, st + (wave * C::X_INS + q) * 1024);
#pragma unroll
    for (int q = 0; q < C::W_INS; ++q)
      dma16_r(w_rsrc, w_off[q] + kt * 128u, st + C::XB + (wave * C::W_INS + q) * 1024);
  };

  floatx16_t acc[C::TN];
  double dacc[C::TN][16];
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc[j][r] = 0.0f; dacc[j][r] = 0.0; }

  for (int s = 0; s < C::NST - 1 && s < nk; ++s) issue(s);
  const int fr = lane & 31, fh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    // slice kt has landed: while the refills so far all existed, exactly the
    // NST-2 younger slices' loads are outstanding
    if (kt + C::NST - 2 < nk) wait_vm_r<C::INS * (C::NST - 2)>();
    else wait_vm_r<0>();
    __builtin_amdgcn_s_barrier();            // ... for every wave; slot kt-1 is free
    if (kt + C::NST - 1 < nk) issue(kt + C::NST - 1);
    const char* sx = smem + (kt % C::NST) * C::STAGE;
    const char* sw = sx + C::XB;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sx + swz_r(wm * 32 + fr, kk * 2 + fh));
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int r = wn * C::WN + j * 32 + fr;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(sw + swz_r(p * BN + r, kk * 2 + fh));
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) { dacc[j][r] += (double)acc[j][r]; acc[j][r] = 0.0f; }
  }

  // lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + (r%4)
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int e = e0 + wn * C::WN + j * 32 + fr;
    if (e >= E) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
      if (rl < rows) logits[(long long)(row0 + rl) * E + e] = (float)dacc[j][r];
    }
  }
}

template <int BM, int BN, int NP>
hipError_t launch_router_cfg(const bf16_t* x, const bf16_t* w, float* logits, int T, int E, int D, hipStream_t s) {
  using C = RCfg<BM, BN, NP>;
  static std::atomic<bool> allowed[64];   // per device: attribute set (host threads may race)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !allowed[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_logits_kernel<BM, BN, NP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::STAGE * C::NST);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) allowed[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((router_logits_kernel<BM, BN, NP>), dim3(ceil_div(T, BM), ceil_div(E, BN)), dim3(256),
                     C::STAGE * C::NST, s, x, w, logits, T, E, D);
  return hipGetLastError();
}

// Block shape of the tiled router kernel.  Every workgroup streams its BM
// token rows and its BN experts' weight rows (NP planes) through LDS once.
// A shape whose LDS ring leaves room for a second workgroup on the CU runs
// two at a time, one's float64 additions and waits beside the other's
// MFMAs, so the time goes with the rounds of workgroups per CU slot times
// the bytes one workgroup moves (ties: more workgroups).  Measured on
// MI355X at the DeepSeek-V3 shape (8192 tokens, 256 experts, D = 7168):
// 64 x 64 blocks, two per CU, 58-62 us; 64 x 128 and 128 x 64, one per CU,
// 74-82 us; 32 x 256 (every workgroup re-reading all of W_g) 80-116 us.
struct RouterShape { int bm, bn; };
RouterShape router_shape(int T, int E, int NP) {
  static const RouterShape cand1[] = {{32, 256}, {32, 128}, {64, 128}, {64, 64}, {128, 64}};
  static const RouterShape cand3[] = {{32, 128}, {64, 64}};
  const RouterShape* c = NP == 1 ? cand1 : cand3;
  const int n = NP == 1 ? 5 : 2;
  const int cus = num_cus();
  RouterShape best{0, 0};
  long long best_cost = 0, best_wgs = 0;
  for (int i = 0; i < n; ++i) {
    if (NP == 1 && c[i].bn > 128 && E <= 128) continue;      // blocks wider than the experts
    const int stage = (c[i].bm + NP * c[i].bn) * 128;        // the ring of RCfg
    const int nst = std::min(4, (160 * 1024) / stage);
    const int slots = std::min(2, (160 * 1024) / (stage * nst));
    const long long wgs = (long long)ceil_div(T, c[i].bm) * ceil_div(E, c[i].bn);
    const long long cost = ((wgs + (long long)cus * slots - 1) / ((long long)cus * slots)) *
                           (c[i].bm + (long long)NP * c[i].bn);
    if (best.bm == 0 || cost < best_cost || (cost == best_cost && wgs > best_wgs)) {
      best = c[i];
      best_cost = cost;
      best_wgs = wgs;
    }
  }
  return best;
}

template <int NP>
hipError_t launch_router_tiled(const bf16_t* x, const bf16_t* w, float* logits, int T, int E, int D, hipStream_t s) {
  const RouterShape sh = router_shape(T, E, NP);
  if constexpr (NP == 1) {
    if (sh.bm == 32 && sh.bn == 256) return launch_router_cfg<32, 256, 1>(x, w, logits, T, E, D, s);
    if (sh.bm == 32 && sh.bn == 128) return launch_router_cfg<32, 128, 1>(x, w, logits, T, E, D, s);
    if (sh.bm == 64 && sh.bn == 128) return launch_router_cfg<64, 128, 1>(x, w, logits, T, E, D, s);
    if (sh.bm == 64 && sh.bn == 64) return launch_router_cfg<64, 64, 1>(x, w, logits, T, E, D, s);
    return launch_router_cfg<128, 64, 1>(x, w, logits, T, E, D, s);
  } else {
    if (sh.bm == 32) return launch_router_cfg<32, 128, 3>(x, w, logits, T, E, D, s);
    return launch_router_cfg<64, 64, 3>(x, w, logits, T, E, D, s);
  }
}

template <int NB, int NP, int U>
__global__ __launch_bounds__(512) void router_small_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                           float* __restrict__ logits, int T, int E, int D) {
  constexpr int NW = 8;                             // waves
  __shared__ double part[NW / 2][16][NB * 16 + 1];  // [wave % 4][token][expert] partial sums
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = blockIdx.x * 16;
  const int e0 = blockIdx.y * (NB * 16);            // this workgroup's experts e0 .. e0 + 16 NB - 1
  const int tok = min(row0 + (lane & 15), T - 1);   // rows past the end read the last row
  const int kg = (lane >> 4) * 8;                   // this lane's 8 of a 32-deep step
  const bf16_t* xr = x + (long long)tok * D + kg;
  const bf16_t* wr[NB][NP];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int p = 0; p < NP; ++p)
      wr[b][p] = w + ((long long)min(e0 + b * 16 + (lane & 15), E - 1) * NP + p) * D + kg;

  floatx4_t acc[NB];
  double dacc[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[b][r] = 0.0f; dacc[b][r] = 0.0; }
  // U steps of this wave per iteration, their loads issued together; each
  // step's MFMA sums (32 products per plane) go to float64 at once
  const int nsteps = D / 32;
  for (int s0 = wave; s0 < nsteps; s0 += NW * U) {
    bf16x8_t a[U], bv[U][NB][NP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = min(s0 + NW * u, nsteps - 1);  // steps past the end are loaded but not used
      a[u] = *reinterpret_cast<const bf16x8_t*>(xr + st * 32);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int p = 0; p < NP; ++p) bv[u][b][p] = *reinterpret_cast<const bf16x8_t*>(wr[b][p] + st * 32);
    }
    // Every load of the batch is issued before the first product: with a
    // branch per step the compiler moved each step's loads down to its MFMA
    // and waited for them one step at a time.  A step past the end multiplies
    // a token fragment with its bits cleared (zeros: the sums do not change).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const unsigned keep = (s0 + NW * u < nsteps) ? 0xffffffffu : 0u;
      const bf16x8_t au = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, a[u]) & keep);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int p = 0; p < NP; ++p) acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, bv[u][b][p], acc[b], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) { dacc[b][r] += (double)acc[b][r]; acc[b][r] = 0.0f; }
      }
    }
  }
  // lane holds expert column (lane & 15) of block b and token rows 4 (lane >> 4) + r;
  // waves 4..7 hand their sums to waves 0..3, which then write theirs
  const int w4 = wave & 3;
  if (wave >= 4) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[w4][4 * (lane >> 4) + r][b * 16 + (lane & 15)] = dacc[b][r];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        double& slot = part[w4][4 * (lane >> 4) + r][b * 16 + (lane & 15)];
        slot = dacc[b][r] + slot;
      }
  }
  __syncthreads();
  const int ne = min(NB * 16, E - e0);
  for (int i = threadIdx.x; i < 16 * ne; i += 512) {
    const int tr = i / ne, e = i % ne;
    if (row0 + tr < T)
      logits[(long long)(row0 + tr) * E + e0 + e] =
          (float)(((part[0][tr][e] + part[1][tr][e]) + part[2][tr][e]) + part[3][tr][e]);
  }
}

// Grid: 16-token blocks x blocks of 16 NB experts (one expert block when
// E <= 16 NB).
template <int NB, int NP>
hipError_t launch_router_small(const bf16_t* x, const bf16_t* w, float* logits, int T, int E, int D, hipStream_t s) {
  constexpr int U = NP == 1 ? (NB <= 2 ? 8 : 4) : 2;
  hipLaunchKernelGGL((router_small_kernel<NB, NP, U>), dim3(ceil_div(T, 16), ceil_div(E, NB * 16)), dim3(512), 0, s,
                     x, w, logits, T, E, D);
  return hipGetLastError();
}

// A handful of tokens (decode-sized batches): one wave per expert.  The
// token rows are staged in LDS; the wave streams its expert's weight row (NP
// planes) into registers with the loads of up to 16 steps of 512 columns in
// flight at once, and each lane adds the 8 (x NP) products of a step in
// float32 (every bf16 x bf16 product is exact in float32) before adding that
// into a float64 accumulator per token; the lanes' sums are then added in a
// fixed butterfly order.
constexpr int kGemvMaxTokens = 16;
constexpr int kGemvLds = 128 * 1024;

__device__ __forceinline__ double wave_sum_f64_r(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float dot8_bf16(const uint4 a, const uint4 b, float s) {
  const unsigned av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), s);
    s = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(bv[i] & 0xffff0000u), s);
  }
  return s;
}

template <int NP>
__global__ __launch_bounds__(256) void router_gemv_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w,
                                                          float* __restrict__ logits, int T, int E, int D) {
  extern __shared__ __attribute__((aligned(16))) char smem[];   // x [T][D]
  constexpr int U = 16 / NP;                                    // steps per batch of loads
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n16 = T * D / 8;                                    // 16-byte chunks of x
  // staged 8 chunks per thread at a time, with no branch between the 8 loads
  // so that they are in flight together: indexes past the end are clamped to
  // the last chunk (which is then written again with its own value)
  for (int i0 = threadIdx.x; i0 < n16; i0 += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = reinterpret_cast<const uint4*>(x)[min(i0 + 256 * u, n16 - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) reinterpret_cast<uint4*>(smem)[min(i0 + 256 * u, n16 - 1)] = v[u];
  }
  __syncthreads();
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  const bf16_t* wr = w + (long long)e * NP * D;
  double acc[kGemvMaxTokens];
#pragma unroll
  for (int t = 0; t < kGemvMaxTokens; ++t) acc[t] = 0.0;
  for (int k0 = 0; k0 < D; k0 += 512 * U) {
    // the batch's weight loads, all in flight together (columns past the row
    // end re-read its last 8 and add nothing)
    uint4 wv[U][NP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(k0 + u * 512 + lane * 8, D - 8);
#pragma unroll
      for (int p = 0; p < NP; ++p) wv[u][p] = *reinterpret_cast<const uint4*>(wr + (long long)p * D + k);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kGemvMaxTokens; ++t) {
      if (t < T) {                                              // uniform
        uint4 xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = min(k0 + u * 512 + lane * 8, D - 8);
          xv[u] = *reinterpret_cast<const uint4*>(smem + ((size_t)t * D + k) * 2);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float s = 0.0f;
#pragma unroll
          for (int p = 0; p < NP; ++p) s = dot8_bf16(xv[u], wv[u][p], s);
          acc[t] += (k0 + u * 512 + lane * 8 < D) ? (double)s : 0.0;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kGemvMaxTokens; ++t) {
    if (t < T) {
      const double v = wave_sum_f64_r(acc[t]);
      if (lane == 0) logits[(long long)t * E + e] = (float)v;
    }
  }
}

template <int NP>
hipError_t launch_router_gemv(const bf16_t* x, const bf16_t* w, float* logits, int T, int E, int D, hipStream_t s) {
  const int lds = T * D * 2;
  static std::atomic<bool> allowed[64];   // per device: attribute set (host threads may race)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !allowed[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_gemv_kernel<NP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kGemvLds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) allowed[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((router_gemv_kernel<NP>), dim3(ceil_div(E, 4)), dim3(256), lds, s, x, w, logits, T, E, D);
  static_assert(kGemvLds <= 160 * 1024, "LDS");
  return hipGetLastError();
}

// Which router kernel: 2 = one wave per expert (a handful of tokens whose
// rows fit in LDS); 1 = the small-E kernel, with the experts split over
// workgroups when E > 64 (few tokens: the tiled kernel would run ceil(T / 32)
// workgroups, each reading every expert's weights; measured on MI355X at
// E = 256, D = 7168: 79 us for one token on the tiled kernel); 0 = the tiled
// kernel.  MOE_ROUTER_PATH=gemv / split / tiled forces a kernel where it
// applies (tuning aid and test hook).
int router_path(int T, int E, int D) {
  // with few experts the one-wave-per-expert kernel has few waves: measured
  // on MI355X at E = 8, D = 4096: 8.6 us for one token (small-E kernel 13),
  // 17 us for eight (small-E kernel 14)
  const bool gemv = T <= (E > 64 ? kGemvMaxTokens : 2) && (long long)T * D * 2 <= kGemvLds;
  const int forced = tuning().router_path;
  if (forced == 2 && T <= kGemvMaxTokens && (long long)T * D * 2 <= kGemvLds) return 2;
  if (forced == 1) return 1;
  if (forced == 0) return E <= 64 ? 1 : 0;
  if (gemv) return 2;
  return (E <= 64 || T <= 512) ? 1 : 0;
}

}  // namespace

bool router_kernel_fits(int T, int E, int D, int planes) {
  return T > 0 && E > 0 && D > 0 && D % 64 == 0 && (planes == 1 ? E <= 256 : planes == 3 && E <= 128);
}

hipError_t launch_router_logits(const bf16_t* x, const bf16_t* w, int planes, float* logits, int T, int E, int D,
                                hipStream_t s) {
  if (!router_kernel_fits(T, E, D, planes)) return hipErrorInvalidValue;
  const int path = router_path(T, E, D);
  if (path == 2) {
    if (planes == 3) return launch_router_gemv<3>(x, w, logits, T, E, D, s);
    return launch_router_gemv<1>(x, w, logits, T, E, D, s);
  }
  if (E <= 64) {
    if (planes == 3) {
      if (E <= 16) return launch_router_small<1, 3>(x, w, logits, T, E, D, s);
      if (E <= 32) return launch_router_small<2, 3>(x, w, logits, T, E, D, s);
      return launch_router_small<4, 3>(x, w, logits, T, E, D, s);
    }
    if (E <= 16) return launch_router_small<1, 1>(x, w, logits, T, E, D, s);
    if (E <= 32) return launch_router_small<2, 1>(x, w, logits, T, E, D, s);
    return launch_router_small<4, 1>(x, w, logits, T, E, D, s);
  }
  if (path == 1) {
    if (planes == 3) return launch_router_small<1, 3>(x, w, logits, T, E, D, s);
    return launch_router_small<1, 1>(x, w, logits, T, E, D, s);
  }
  if (planes == 3) return launch_router_tiled<3>(x, w, logits, T, E, D, s);
  return launch_router_tiled<1>(x, w, logits, T, E, D, s);
}

}  // namespace moe
