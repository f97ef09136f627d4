// Grouped GEMMs of the MoE layer: C[r, n] = sum_k A[r, k] * B_g[n, k] for the
// rows r of group g, with optional row gather on A and fused activation
// epilogues.  Both operands are K-contiguous (nn.Linear weight layout), so the
// same kernel serves the router (A = tokens, B = router weight), the gate/up
// projection (A = tokens gathered through the permutation, B = gate/up rows,
// SwiGLU or GELU epilogue) and the down projection (A = hidden rows).
//
// The grouped form is the "grouped GEMM" execution the "别只比较 Top-k" page
// names in its Execute step; per-group row ranges come from the dispatch
// offsets on the device, so no host synchronisation is needed.
#include "common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// m-tile prefix over groups
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ off, int G,
                                                           int bm, int32_t* __restrict__ prefix) {
  __shared__ int s[kMaxExperts];
  const int g = threadIdx.x;
  s[g] = (g < G) ? ceil_div(off[g + 1] - off[g], bm) : 0;
  __syncthreads();
  for (int d = 1; d < kMaxExperts; d <<= 1) {
    const int v = (g >= d) ? s[g - d] : 0;
    __syncthreads();
    s[g] += v;
    __syncthreads();
  }
  if (g < G) prefix[g + 1] = s[g];
  if (g == 0) prefix[0] = 0;
}

// Class-restricted prefixes (see launch_tile_prefix_classes): one inclusive
// scan over the groups per requested prefix.
__global__ __launch_bounds__(1024) void tile_prefix_classes_kernel(const int32_t* __restrict__ off, int G,
                                                                   TilePrefixReq r0, TilePrefixReq r1,
                                                                   TilePrefixReq r2) {
  __shared__ int s[kMaxExperts];
  const int g = threadIdx.x;
  const int n = (g < G) ? off[g + 1] - off[g] : 0;
  for (int q = 0; q < 3; ++q) {
    const TilePrefixReq r = q == 0 ? r0 : (q == 1 ? r1 : r2);
    if (r.out == nullptr) continue;     // uniform: the same request for every thread
    s[g] = (n > r.lo && n <= r.hi) ? ceil_div(n, r.bm) : 0;
    __syncthreads();
    for (int d = 1; d < kMaxExperts; d <<= 1) {
      const int v = (g >= d) ? s[g - d] : 0;
      __syncthreads();
      s[g] += v;
      __syncthreads();
    }
    if (g < G) r.out[g + 1] = s[g];
    if (g == 0) r.out[0] = 0;
    __syncthreads();                    // s is rewritten by the next request
  }
}

// Number of m-tiles that can exist: sum_g ceil(n_g / BM) <= floor(M / BM) + #non-empty groups.
inline int m_tiles_bound(const GroupedGemm& p, int bm) {
  if (p.offsets == nullptr) return ceil_div(p.M_max, bm);
  return p.M_max / bm + (p.G < p.M_max ? p.G : p.M_max);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  256 threads = 4 waves in a 2 x 2 arrangement; each wave
// owns a (BM/2) x (BN/2) sub-tile built from 32x32x16 MFMA blocks.  Operand
// tiles are staged through LDS with a register prefetch of the next K slice
// (double-buffered LDS, one barrier per K step).
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int LDS = BK + 8;       // padded LDS row, elements (breaks bank aliasing)
  static constexpr int CPR = BK / 8;       // 16-byte chunks per row
  static constexpr int RPP = 256 / CPR;    // rows per load pass
  static constexpr int A_PASSES = BM / RPP;
  static constexpr int B_PASSES = BN / RPP;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile/load mismatch");
};

// PRECISE: every BK-deep slice is summed by the MFMAs in float32 and then
// added into float64 accumulators, so rounding error does not grow with K
// (used for the router logits, which decide the expert selection).
// NPF: K slices held in registers ahead of the one being multiplied (the
// loads of NPF slices are in flight while the LDS copy of the next one is
// written).
template <int BM, int BN, int BK, int EPI, typename OutT, bool PRECISE = false, int NPF = 1>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const GroupedGemm p, int n_tiles) {
  using C = Tile<BM, BN, BK>;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * C::LDS];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int g, row0, rows, nt;
  if (!map_tile<BM>(p, n_tiles, g, row0, rows, nt)) return;

  const int K = p.K;
  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(p.B) + (long long)g * p.b_group_stride;
  const int kc = (tid % C::CPR) * 8;

  const bf16_t* a_ptr[C::A_PASSES];
#pragma unroll
  for (int i = 0; i < C::A_PASSES; ++i) {
    const int r = tid / C::CPR + i * C::RPP;
    a_ptr[i] = nullptr;
    if (r < rows) {
      const long long src = p.a_rows ? (long long)p.a_rows[row0 + r] : (long long)(row0 + r);
      a_ptr[i] = A + src * p.lda + kc;
    }
  }
  const bf16_t* b_ptr[C::B_PASSES];
#pragma unroll
  for (int i = 0; i < C::B_PASSES; ++i) {
    const int r = tid / C::CPR + i * C::RPP;
    int brow;
    bool ok;
    if constexpr (EPI == EPI_SWIGLU) {
      // 32-row sub-tiles alternate gate / up for the same 32 hidden columns, so
      // one wave holds matching gate and up accumulators.
      const int s = r >> 5, wc = s / C::TN, ls = s % C::TN;
      const int h = nt * (BN / 2) + (wc * (C::TN / 2) + (ls >> 1)) * 32 + (r & 31);
      ok = h < p.N;
      brow = (ls & 1) ? p.N + h : h;
    } else {
      const int n = nt * BN + r;
      ok = n < p.N;
      brow = n;
    }
    b_ptr[i] = ok ? B + (long long)brow * K + kc : nullptr;
  }

  u32x4_t ra[NPF][C::A_PASSES], rb[NPF][C::B_PASSES];
  auto gload = [&](int slot, int k0) __attribute__((always_inline)) {
    const bool kin = (k0 + kc) < K;
    const int ka = p.a_kwrap ? k0 % p.a_kwrap : k0;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < C::A_PASSES; ++i)
      ra[slot][i] = (a_ptr[i] && kin) ? *reinterpret_cast<const u32x4_t*>(a_ptr[i] + ka) : zero;
#pragma unroll
    for (int i = 0; i < C::B_PASSES; ++i)
      rb[slot][i] = (b_ptr[i] && kin) ? *reinterpret_cast<const u32x4_t*>(b_ptr[i] + k0) : zero;
  };
  auto sstore = [&](int slot, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::A_PASSES; ++i) {
      const int r = tid / C::CPR + i * C::RPP;
      *reinterpret_cast<u32x4_t*>(&sA[buf][r * C::LDS + kc]) = ra[slot][i];
    }
#pragma unroll
    for (int i = 0; i < C::B_PASSES; ++i) {
      const int r = tid / C::CPR + i * C::RPP;
      *reinterpret_cast<u32x4_t*>(&sB[buf][r * C::LDS + kc]) = rb[slot][i];
    }
  };

  floatx16_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  constexpr int DM = PRECISE ? C::TM : 1, DN = PRECISE ? C::TN : 1, DR = PRECISE ? 16 : 1;
  double dacc[DM][DN][DR];
  if constexpr (PRECISE) {
#pragma unroll
    for (int i = 0; i < DM; ++i)
#pragma unroll
      for (int j = 0; j < DN; ++j)
#pragma unroll
        for (int r = 0; r < DR; ++r) dacc[i][j][r] = 0.0;
  }

  const int nk = ceil_div(K, BK);
  // slice j lives in register slot j % NPF until it is copied to LDS
#pragma unroll
  for (int u = 0; u < NPF; ++u)
    if (u < nk) gload(u, u * BK);
  sstore(0, 0);
  __syncthreads();
  const int frag_k = (lane >> 5) * 8;
  for (int kb = 0; kb < nk; kb += NPF) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int kt = kb + u;
      if (kt >= nk) break;
      const int buf = kt & 1;
      // slot u is free (slice kt is in LDS): fetch slice kt + NPF into it
      if (kt + NPF < nk) gload(u, (kt + NPF) * BK);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8_t af[C::TM], bfv[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
          const int row = wm * C::WM + i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][row * C::LDS + kk * 16 + frag_k]);
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const int row = wn * C::WN + j * 32 + (lane & 31);
          bfv[j] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][row * C::LDS + kk * 16 + frag_k]);
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
      }
      if constexpr (PRECISE) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              dacc[i][j][r] += (double)acc[i][j][r];
              acc[i][j][r] = 0.0f;
            }
      }
      if (kt + 1 < nk) sstore((u + 1) % NPF, buf ^ 1);
      __syncthreads();
    }
  }

  // Epilogue.  MFMA 32x32 output: lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + (r%4) for accumulator element r.
  OutT* __restrict__ Cout = static_cast<OutT*>(p.C);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * C::WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (rl >= rows) continue;
      OutT* crow = Cout + (long long)(row0 + rl) * p.ldc;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int q = 0; q < C::TN / 2; ++q) {
          const int h = nt * (BN / 2) + (wn * (C::TN / 2) + q) * 32 + (lane & 31);
          if (h < p.N) crow[h] = from_f32<OutT>(silu_f32(acc[i][2 * q][r]) * acc[i][2 * q + 1][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const int n = nt * BN + wn * C::WN + j * 32 + (lane & 31);
          if (n < p.N) {
            float v;
            if constexpr (PRECISE) v = (float)dacc[i][j][r];
            else v = acc[i][j][r];
            if constexpr (EPI == EPI_GELU) v = gelu_erf_f32(v);
            crow[n] = from_f32<OutT>(v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 SIMT kernel (float32 activations, float32 router weight).  64 x 64
// tiles, 16-deep K slices staged transposed in LDS, 4 x 4 outputs per thread.
// ---------------------------------------------------------------------------
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float v[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
};
template <> struct Vec4<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float v[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
};

template <typename TA, typename TB, int EPI, typename OutT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GroupedGemm p, int n_tiles) {
  constexpr int BM = kF32GemmBM, BN = 64, BK = 16;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  int g, row0, rows, nt;
  if (!map_tile<BM>(p, n_tiles, g, row0, rows, nt)) return;

  const int K = p.K;
  const TA* __restrict__ A = static_cast<const TA*>(p.A);
  const TB* __restrict__ B = static_cast<const TB*>(p.B) + (long long)g * p.b_group_stride;
  const int lr = tid >> 2, lk = (tid & 3) * 4;

  const TA* a_ptr = nullptr;
  if (lr < rows) {
    const long long src = p.a_rows ? (long long)p.a_rows[row0 + lr] : (long long)(row0 + lr);
    a_ptr = A + src * p.lda + lk;
  }
  const TB* b_ptr = nullptr;
  {
    int brow;
    bool ok;
    if constexpr (EPI == EPI_SWIGLU) {
      const int h = nt * (BN / 2) + (lr & 31);
      ok = h < p.N;
      brow = (lr >= 32) ? p.N + h : h;
    } else {
      const int n = nt * BN + lr;
      ok = n < p.N;
      brow = n;
    }
    if (ok) b_ptr = B + (long long)brow * K + lk;
  }

  // Each 16-deep slice is accumulated in float32, then added in float64.
  float acc[4][4] = {};
  double dacc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    float va[4] = {0, 0, 0, 0}, vb[4] = {0, 0, 0, 0};
    if (a_ptr && k0 + lk < K) Vec4<TA>::load(a_ptr + k0, va);
    if (b_ptr && k0 + lk < K) Vec4<TB>::load(b_ptr + k0, vb);
#pragma unroll
    for (int q = 0; q < 4; ++q) { sA[lk + q][lr] = va[q]; sB[lk + q][lr] = vb[q]; }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dacc[i][j] += (double)acc[i][j];
        acc[i][j] = 0.0f;
      }
    __syncthreads();
  }

  OutT* __restrict__ Cout = static_cast<OutT*>(p.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = ty + 16 * i;
    if (rl >= rows) continue;
    OutT* crow = Cout + (long long)(row0 + rl) * p.ldc;
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int h = nt * (BN / 2) + tx + 16 * j;
        if (h < p.N) crow[h] = from_f32<OutT>(silu_f32((float)dacc[i][j]) * (float)dacc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nt * BN + tx + 16 * j;
        if (n < p.N) {
          float v = (float)dacc[i][j];
          if constexpr (EPI == EPI_GELU) v = gelu_erf_f32(v);
          crow[n] = from_f32<OutT>(v);
        }
      }
    }
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 64;

template <int EPI, typename OutT, int BM = kBM, int BN = kBN, bool PRECISE = false, int NPF = 1>
hipError_t launch_bf16_epi(const GroupedGemm& p, hipStream_t s) {
  const int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int n_tiles = ceil_div(p.N, cols);
  const int m_tiles = m_tiles_bound(p, BM);
  if (m_tiles == 0 || n_tiles == 0) return hipSuccess;
  const long long blocks = (long long)m_tiles * n_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, kBK, EPI, OutT, PRECISE, NPF>), dim3((unsigned)blocks), dim3(256),
                     0, s, p, n_tiles);
  return hipGetLastError();
}

template <typename TA, typename TB, int EPI, typename OutT>
hipError_t launch_f32_epi(const GroupedGemm& p, hipStream_t s) {
  const int cols = (EPI == EPI_SWIGLU) ? 32 : 64;
  const int n_tiles = ceil_div(p.N, cols);
  const int m_tiles = m_tiles_bound(p, kF32GemmBM);
  if (m_tiles == 0 || n_tiles == 0) return hipSuccess;
  const long long blocks = (long long)m_tiles * n_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, EPI, OutT>), dim3((unsigned)blocks), dim3(256), 0, s,
                     p, n_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_prefix(const int32_t* offsets, int G, int bm, int32_t* prefix, hipStream_t s) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(kMaxExperts), 0, s, offsets, G, bm, prefix);
  return hipGetLastError();
}

hipError_t launch_tile_prefix_classes(const int32_t* offsets, int G, TilePrefixReq r0, TilePrefixReq r1,
                                      TilePrefixReq r2, hipStream_t s) {
  if (G > kMaxExperts) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_prefix_classes_kernel, dim3(1), dim3(kMaxExperts), 0, s, offsets, G, r0, r1, r2);
  return hipGetLastError();
}

int gemm_bf16_bm(const GroupedGemm&) { return kBM; }

hipError_t launch_gemm_bf16(const GroupedGemm& p, hipStream_t s) {
  switch (p.epilogue) {
    // float32 output is the router logits: small tiles, float64 slice accumulation
    case EPI_STORE_F32: return launch_bf16_epi<EPI_STORE_F32, float, 64, 64, true, 4>(p, s);
    case EPI_STORE_ACT: return launch_bf16_epi<EPI_STORE_ACT, bf16_t>(p, s);
    case EPI_SWIGLU: return launch_bf16_epi<EPI_SWIGLU, bf16_t>(p, s);
    case EPI_GELU: return launch_bf16_epi<EPI_GELU, bf16_t>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(const GroupedGemm& p, int a_dtype, int b_dtype, hipStream_t s) {
  if (b_dtype != F32) return hipErrorInvalidValue;
  if (a_dtype == BF16) {
    if (p.epilogue != EPI_STORE_F32) return hipErrorInvalidValue;
    return launch_f32_epi<bf16_t, float, EPI_STORE_F32, float>(p, s);
  }
  switch (p.epilogue) {
    case EPI_STORE_F32:
    case EPI_STORE_ACT: return launch_f32_epi<float, float, EPI_STORE_F32, float>(p, s);
    case EPI_SWIGLU: return launch_f32_epi<float, float, EPI_SWIGLU, float>(p, s);
    case EPI_GELU: return launch_f32_epi<float, float, EPI_GELU, float>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
