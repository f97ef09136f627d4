// Pipelined bf16 grouped GEMM for K a multiple of 64 (the expert FFN shapes).
//
// C[r, n] = sum_k A[r, k] * B_g[n, k] for the rows r of group g, as in
// gemm.hip, with the same tile scheduler and epilogues, restructured for the
// matrix cores:
//   * operand tiles move global -> LDS by buffer loads with the LDS bit
//     (buffer_load_dwordx4 ... lds: no VGPR staging) into an NST-deep ring of
//     LDS slots, so NST-1 K-slices (64 deep) are in flight while the matrix
//     cores work on the current one;
//   * MFMA fragments are double-buffered: the LDS reads of the next 16-deep
//     step are issued before the MFMAs of the current one;
//   * LDS rows are 128 B (64 bf16) with the 16-byte chunk c of row r stored in
//     slot c ^ ((r >> 1) & 7): a 16-lane pass of a fragment read (16
//     consecutive rows, same chunk) touches every bank once.  A load
//     instruction writes lane i to byte 16 i of an 8-row group, so lane i
//     fetches the chunk that belongs in its slot.
// Per slice: s_waitcnt vmcnt(loads of the younger slices) completes this
// wave's loads of the slice; the workgroup barrier makes every wave's loads
// visible and guarantees that the slot refilled next is no longer read.
#include "common.h"

namespace moe {
namespace {

template <int BM, int BN, int WGM, int WGN, int NST>
struct Cfg2 {
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int NWAVES = WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;     // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;       // 32x32 MFMA blocks per wave
  static constexpr int ROWB = 128;                       // bytes per LDS row (64 bf16)
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_INS = BM / 8 / NWAVES;          // 1 KB load instructions per wave per slice
  static constexpr int B_INS = BN / 8 / NWAVES;
  static constexpr int INS = A_INS + B_INS;
  static_assert(BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0, "load split");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(STAGE * NST <= 160 * 1024, "LDS");
  static_assert(INS * (NST - 2) <= 63, "vmcnt range");
};

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer descriptor over `bytes` bytes from `base` (loads past the end
// return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane, buffer -> LDS: lane i lands at lds + 16 * i.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned voff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int BM, int BN, int WGM, int WGN, int NST, int EPI, typename OutT>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_v2_kernel(const GroupedGemm p, int n_tiles) {
  using C = Cfg2<BM, BN, WGM, WGN, NST>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  int g, row0, rows, nt;
  if (!map_tile<BM>(p, n_tiles, g, row0, rows, nt)) return;

  const int K = p.K;
  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(p.B) + (long long)g * p.b_group_stride;

  // Byte offsets of this wave's load instructions (rows past the tile end
  // clamped to a valid row: their outputs are never stored).
  const int lrow = lane >> 3;                           // row inside an 8-row group
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A, 0xffffffffu);
  const int b_rows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B, (unsigned)b_rows * (unsigned)K * 2u);
  unsigned a_off[C::A_INS], b_off[C::B_INS];
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int r = (wave * C::A_INS + q) * 8 + lrow;
    const int rr = r < rows ? r : rows - 1;
    const unsigned src = p.a_rows ? (unsigned)p.a_rows[row0 + rr] : (unsigned)(row0 + rr);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    a_off[q] = (src * (unsigned)p.lda + c * 8) * 2u;
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int r = (wave * C::B_INS + q) * 8 + lrow;
    int brow;
    if constexpr (EPI == EPI_SWIGLU) {
      // 32-row sub-tiles alternate gate / up rows of the same hidden columns
      const int s = r >> 5, wc = s / C::TN, ls = s % C::TN;
      int h = nt * (BN / 2) + (wc * (C::TN / 2) + (ls >> 1)) * 32 + (r & 31);
      h = h < p.N ? h : p.N - 1;
      brow = (ls & 1) ? p.N + h : h;
    } else {
      const int n = nt * BN + r;
      brow = n < p.N ? n : p.N - 1;
    }
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    b_off[q] = ((unsigned)brow * (unsigned)K + c * 8) * 2u;
  }

  auto issue = [&](int kt) __attribute__((always_inline)) {
    char* st = smem + (kt % NST) * C::STAGE;
    const unsigned kb = kt * 128u;
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q) dma16(a_rsrc, a_off[q] + kb, st + (wave * C::A_INS + q) * 1024);
#pragma unroll
    for (int q = 0; q < C::B_INS; ++q)
      dma16(b_rsrc, b_off[q] + kb, st + C::A_BYTES + (wave * C::B_INS + q) * 1024);
  };

  floatx16_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = K / 64;
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nk) issue(st);

  const int fr = lane & 31;              // fragment row inside a 32-row block
  const int fc = lane >> 5;              // which 8-wide half of a 16-deep step
  // fragments of 16-deep step kk of the slice held in LDS slot `slot`
  bf16x8_t af[2][C::TM], bfv[2][C::TN];
  auto load_frags = [&](int buf, int slot, int kk) __attribute__((always_inline)) {
    const char* sa = smem + slot * C::STAGE;
    const char* sb = sa + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      af[buf][i] = *reinterpret_cast<const bf16x8_t*>(sa + swz(wm * C::WM + i * 32 + fr, kk * 2 + fc));
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      bfv[buf][j] = *reinterpret_cast<const bf16x8_t*>(sb + swz(wn * C::WN + j * 32 + fr, kk * 2 + fc));
  };
  // A burst of MFMAs runs at raised wave priority so that a co-resident wave's
  // memory instructions are issued around it rather than into it.
  auto mfmas = [&](int buf) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfv[buf][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Slice kt has landed for every wave.  Younger slices issued so far:
  // min(NST - 2, nk - 1 - kt).
  auto slice_ready = [&](int kt) __attribute__((always_inline)) {
    if (kt + NST - 2 < nk) wait_vmcnt<C::INS * (NST - 2)>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };

  slice_ready(0);
  load_frags(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt % NST;
    // refill the slot of slice kt-1: every wave finished reading it before the
    // barrier that published slice kt
    if (kt + NST - 1 < nk) issue(kt + NST - 1);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      load_frags((kk + 1) & 1, slot, kk + 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(kk & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kt + 1 < nk) {
      // the step-3 fragments are in registers before the slot is handed back;
      // the next slice's first fragments are fetched while this slice's last
      // MFMAs run
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      slice_ready(kt + 1);
      load_frags(0, (kt + 1) % NST, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
  }

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
            float v = acc[i][j][r];
            if constexpr (EPI == EPI_GELU) v = gelu_erf_f32(v);
            crow[n] = from_f32<OutT>(v);
          }
        }
      }
    }
  }
}

inline int m_bound(const GroupedGemm& p, int bm) {
  if (p.offsets == nullptr) return ceil_div(p.M_max, bm);
  return p.M_max / bm + (p.G < p.M_max ? p.G : p.M_max);
}

template <int BM, int BN, int WGM, int WGN, int NST, int EPI>
hipError_t launch_cfg(const GroupedGemm& p, hipStream_t s) {
  using C = Cfg2<BM, BN, WGM, WGN, NST>;
  const int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int n_tiles = ceil_div(p.N, cols);
  const int m_tiles = m_bound(p, BM);
  if (m_tiles == 0 || n_tiles == 0) return hipSuccess;
  const long long blocks = (long long)m_tiles * n_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  // dynamic LDS above 64 KB has to be allowed explicitly, once per device
  static std::atomic<bool> allowed[64];   // per device: attribute set (host threads may race)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !allowed[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_v2_kernel<BM, BN, WGM, WGN, NST, EPI, bf16_t>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::STAGE * NST);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) allowed[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((gemm_v2_kernel<BM, BN, WGM, WGN, NST, EPI, bf16_t>), dim3((unsigned)blocks),
                     dim3(C::THREADS), C::STAGE * NST, s, p, n_tiles);
  return hipGetLastError();
}

}  // namespace

// Tile configurations, selected by v2_config.
template <int EPI>
static hipError_t launch_v2_epi(const GroupedGemm& p, int cfg, hipStream_t s) {
  switch (cfg) {
    case 0: return launch_cfg<256, 128, 2, 2, 3, EPI>(p, s);
    case 1: return launch_cfg<128, 128, 2, 2, 4, EPI>(p, s);
    case 2: return launch_cfg<256, 256, 2, 2, 2, EPI>(p, s);
    case 3: return launch_cfg<128, 256, 2, 2, 3, EPI>(p, s);
    case 4: return launch_cfg<256, 256, 2, 4, 2, EPI>(p, s);
    case 5: return launch_cfg<64, 256, 1, 4, 3, EPI>(p, s);
    // two workgroups per CU (<= 80 KB of LDS each)
    case 6: return launch_cfg<64, 256, 1, 4, 2, EPI>(p, s);
    case 7: return launch_cfg<128, 128, 2, 2, 2, EPI>(p, s);
    case 8: return launch_cfg<64, 128, 1, 2, 3, EPI>(p, s);
    case 9: return launch_cfg<128, 256, 2, 4, 2, EPI>(p, s);
  }
  return hipErrorInvalidValue;
}

int gemm_v2_bm(int cfg) {
  static const int bm[] = {256, 128, 256, 128, 256, 64, 64, 128, 64, 128};
  return (cfg >= 0 && cfg < kGemmV2Configs) ? bm[cfg] : 0;
}

hipError_t launch_gemm_v2(const GroupedGemm& p, int cfg, hipStream_t s) {
  switch (p.epilogue) {
    case EPI_STORE_ACT: return launch_v2_epi<EPI_STORE_ACT>(p, cfg, s);
    case EPI_SWIGLU: return launch_v2_epi<EPI_SWIGLU>(p, cfg, s);
    case EPI_GELU: return launch_v2_epi<EPI_GELU>(p, cfg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
