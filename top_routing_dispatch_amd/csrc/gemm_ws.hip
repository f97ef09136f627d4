// bf16 grouped GEMM for shallow groups, where each group's weights are the
// bulk of the traffic and the kernel runs at the speed of the weight stream.
//
// C[r, n] = sum_k A[r, k] * B_g[n, k] with the tile order, tile prefix and
// epilogues of the other grouped GEMM kernels.  What is particular here:
//   * a persistent grid of one (or two) workgroups per CU walks its tiles
//     (every gridDim.x-th tile of the order), and the LDS ring of K slices
//     runs across tile boundaries: while the last slices of one tile are
//     multiplied and its outputs written, the first slices of the next tile
//     are already on their way, so the weight stream of a CU does not stop
//     between tiles;
//   * loads and stores are issued by different wavefronts: NLW loader waves
//     issue the ring's loads and wait for them with exact vmcnt counts, the
//     compute waves multiply and write the outputs, so output stores never
//     sit in a loader's vmcnt (which counts stores too) and never delay the
//     stream; one barrier per slice hands slices from the loaders to the
//     compute waves and free slots back;
//   * the output block of a compute wave is staged in an LDS area of its own
//     (16 rows at a time), apart from the ring, for 16-byte row stores;
//   * the workgroups of one XCD take consecutive tiles of the order, so the
//     n-tiles of a group (which share its activation rows) run in one L2;
//   * when the tiles are too few to keep every CU streaming (a handful of
//     token rows, as in decoding), the contraction of each tile can be split
//     into ksplit units of K / ksplit: the units write float32 partial sums,
//     and splitk_reduce_kernel adds them in a fixed order and applies the
//     epilogue.
// LDS rows are BK*2 bytes; the 16-byte chunk c of row r sits in slot
// c ^ ((r / (16 / CPR)) % CPR) (CPR chunks per row), so that the 16 rows read
// by one pass of a fragment load cover all 64 banks once.
#include "common.h"

#include <algorithm>
#include <type_traits>

namespace moe {
namespace {

template <int BM, int BN, int WGM, int WGN, int BK, int NST>
struct CfgW {
  static constexpr int NWAVES = WGM * WGN;               // compute waves
  static constexpr int NLW = 4;                          // loader waves
  static constexpr int THREADS = 64 * (NWAVES + NLW);
  static constexpr int WM = BM / WGM, WN = BN / WGN;     // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;       // 32x32 MFMA blocks per wave
  static constexpr int RB = BK * 2;                      // bytes per LDS row
  static constexpr int CPR = BK / 8;                     // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;                  // rows per 1 KB load instruction
  static constexpr int KK = BK / 16;                     // MFMA k-steps per slice
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int RING = NST * STAGE;
  static constexpr int A_INS = BM / RPI / NLW;           // load instructions per loader wave per slice
  static constexpr int B_INS = BN / RPI / NLW;
  static constexpr int INS = A_INS + B_INS;
  static_assert(BK == 32 || BK == 64, "slice depth");
  static_assert(BM % (RPI * NLW) == 0 && BN % (RPI * NLW) == 0, "load split");
  static_assert(A_INS >= 1 && B_INS >= 1, "load split");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(NST >= 2 && INS * (NST - 2) <= 63, "ring depth / vmcnt range");
  // output staging of one wave: 16 rows of OC columns, 16-byte pad per row
  __host__ __device__ static constexpr int out_cols(int epi) { return epi == EPI_SWIGLU ? WN / 2 : WN; }
  __host__ __device__ static constexpr int pitch(int epi) { return out_cols(epi) * 2 + 16; }
  __host__ __device__ static constexpr int lds(int epi) { return RING + NWAVES * 16 * pitch(epi); }
};

typedef __attribute__((address_space(3))) void lds_void_w;

// Buffer range of the operands, and the offset of rows that are not read:
// kDeadOff + k * 2 stays above kRangeEnd and below 2^32 for K < 2^19.
constexpr unsigned kRangeEnd = 0xffe00000u;
constexpr unsigned kDeadOff = 0xffe80000u;

// 16 bytes per lane, buffer -> LDS: lane i lands at lds + 16 * i.
__device__ __forceinline__ void dma16_w(__amdgpu_buffer_rsrc_t r, unsigned voff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_w*)lds, 16, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm_w() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// vmcnt <= ins * n for a runtime n in [0, NMAX]
template <int INS, int NMAX>
__device__ __forceinline__ void wait_slices(int n) {
  if constexpr (NMAX > 0) {
    if (n >= NMAX) { wait_vm_w<INS * NMAX>(); return; }
    wait_slices<INS, NMAX - 1>(n);
  } else {
    wait_vm_w<0>();
  }
}

template <int CPR>
__device__ __forceinline__ int swz_w(int r, int c) {
  return r * (CPR * 16) + ((c ^ ((r / (16 / CPR)) & (CPR - 1))) << 4);
}

// SPLIT: the launch splits the contraction (p.ksplit > 1) and the kernel
// writes float32 partial sums instead of the epilogue's output.
template <int BM, int BN, int WGM, int WGN, int BK, int NST, int OCC, int EPI, bool SPLIT>
__global__ __launch_bounds__(64 * (WGM * WGN + 4))
__attribute__((amdgpu_waves_per_eu((WGM * WGN + 4) / 4 * OCC, (WGM * WGN + 4) / 4 * OCC)))
void gemm_ws_kernel(const GroupedGemm p, int n_tiles) {
  using C = CfgW<BM, BN, WGM, WGN, BK, NST>;
  static_assert(C::NLW == 4 && (C::NWAVES + C::NLW) % 4 == 0, "waves per SIMD");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool loader = wave >= C::NWAVES;
  const int lw = wave - C::NWAVES;                  // loader index
  const int wm = wave / WGN, wn = wave % WGN;       // compute wave position

  // slot v: the workgroups of one XCD (i % 8) hold consecutive slots
  const int S = gridDim.x;
  const int v = (S % kNumXcd == 0) ? (blockIdx.x % kNumXcd) * (S / kNumXcd) + blockIdx.x / kNumXcd : blockIdx.x;
  // units: tiles, each split into KS runs over K / KS (unit u: tile u / KS,
  // part u % KS)
  const int KS = SPLIT ? p.ksplit : 1;
  const int total = (p.offsets == nullptr ? ceil_div(p.M_max, BM) : ld_table<true>(p.tile_prefix, p.G)) * n_tiles * KS;
  if (v >= total) return;
  const int my_tiles = (total - 1 - v) / S + 1;     // units v, v + S, ...
  const int nk = p.K / BK / KS;                      // slices per unit
  const int nsl = my_tiles * nk;                     // slices of the whole stream

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  // Rows past the tile end (and weight rows past N) are read at offset
  // kDeadOff + k, beyond the buffer's range: the load returns zeros without a
  // memory access.  Their LDS rows feed only outputs that are never stored.
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(A), 0, (int)kRangeEnd, 0x00020000);
  const int lrow = lane / C::CPR;
  const int lslot = lane % C::CPR;

  // ---- loader: the unit and slice that the next refill reads ----
  int ld_t = -1, ld_k = nk;
  unsigned ld_kb = 0;                               // byte offset of the unit's first slice
  unsigned a_off[C::A_INS], b_off[C::B_INS];
  __amdgpu_buffer_rsrc_t b_rsrc = a_rsrc;
  auto ld_setup = [&](int t) __attribute__((always_inline)) {
    // scalar loads only: the ring's loads in flight are not waited for here
    int g, row0, rows, nt;
    const int u = v + t * S;
    const int tile = u / KS;
    ld_kb = (unsigned)((u - tile * KS) * nk) * C::RB;
    decode_tile<BM, true>(p, n_tiles, tile, g, row0, rows, nt);
    const bf16_t* B = static_cast<const bf16_t*>(p.B) + (long long)g * p.b_group_stride;
    b_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(B), 0, (int)kRangeEnd, 0x00020000);
    // instruction q of the wave reads rows r0 .. r0 + RPI - 1, lane row
    // lrow picks its source row out of those
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q) {
      const int r0 = (lw * C::A_INS + q) * C::RPI;
      int src = row0 + min(r0 + lrow, rows - 1);
      if (p.a_rows != nullptr) {
#pragma unroll
        for (int m = 0; m < C::RPI; ++m) {
          const int sm = ld_table<true>(p.a_rows, row0 + min(r0 + m, rows - 1));
          src = lrow == m ? sm : src;
        }
      }
      const int r = r0 + lrow;
      const int c = lslot ^ ((r / (16 / C::CPR)) & (C::CPR - 1));
      a_off[q] = r < rows ? ((unsigned)src * (unsigned)p.lda + c * 8) * 2u : kDeadOff;
    }
#pragma unroll
    for (int q = 0; q < C::B_INS; ++q) {
      const int r = (lw * C::B_INS + q) * C::RPI + lrow;
      int brow;
      bool live;
      if constexpr (EPI == EPI_SWIGLU) {
        // 32-row sub-tiles alternate gate / up rows of the same hidden columns
        const int s = r >> 5, wc = s / C::TN, ls = s % C::TN;
        const int h = nt * (BN / 2) + (wc * (C::TN / 2) + (ls >> 1)) * 32 + (r & 31);
        live = h < p.N;
        brow = (ls & 1) ? p.N + h : h;
      } else {
        brow = nt * BN + r;
        live = brow < p.N;
      }
      const int c = lslot ^ ((r / (16 / C::CPR)) & (C::CPR - 1));
      b_off[q] = live ? ((unsigned)brow * (unsigned)p.K + c * 8) * 2u : kDeadOff;
    }
  };
  // refill ring slot `slot` with the next slice of the stream
  auto load_next = [&](int slot) __attribute__((always_inline)) {
    if (ld_k == nk) {
      ld_k = 0;
      ++ld_t;
      ld_setup(ld_t);
    }
    char* st = smem + slot * C::STAGE;
    const unsigned koff = ld_kb + (unsigned)ld_k * C::RB;
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q) dma16_w(a_rsrc, a_off[q] + koff, st + (lw * C::A_INS + q) * 1024);
#pragma unroll
    for (int q = 0; q < C::B_INS; ++q)
      dma16_w(b_rsrc, b_off[q] + koff, st + C::A_BYTES + (lw * C::B_INS + q) * 1024);
    ++ld_k;
  };

  // ---- consumer: the unit being multiplied ----
  int c_g, c_row0, c_rows, c_nt, c_ks, act_i;
  auto cp_setup = [&](int t) __attribute__((always_inline)) {
    const int u = v + t * S;
    const int tile = u / KS;
    c_ks = u - tile * KS;
    decode_tile<BM, true>(p, n_tiles, tile, c_g, c_row0, c_rows, c_nt);
    // 32-row blocks of this wave that hold at least one row of the tile
    act_i = min(C::TM, max(0, ceil_div(c_rows - wm * C::WM, 32)));
  };

  floatx16_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int fr = lane & 31;              // fragment row inside a 32-row block
  const int fc = lane >> 5;              // which 8-wide half of a 16-deep step

  // epilogue: activation in registers, 16 rows at a time (the half of a
  // 32-row MFMA block held in accumulator registers 8h .. 8h+7) through the
  // wave's staging area, 16-byte row stores; halves without rows of the tile
  // are skipped
  constexpr int OC = C::out_cols(EPI);
  constexpr int PITCH = C::pitch(EPI);
  constexpr int CPO = OC / 8;            // 16-byte chunks per output row
  constexpr int RPO = 64 / CPO;          // rows per pass of the wave
  static_assert(64 % CPO == 0 && 16 % RPO == 0, "store passes");
  char* stg = smem + C::RING + wave * (16 * PITCH);
  auto epilogue = [&]() __attribute__((always_inline)) {
    bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.C);
    const int col0 = (EPI == EPI_SWIGLU) ? c_nt * (BN / 2) + wn * OC : c_nt * BN + wn * OC;
    const bool vec = (p.ldc % 8 == 0) && ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0);
    const int ch = lane % CPO;
    const int n = col0 + ch * 8;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rows_h = min(16, c_rows - wm * C::WM - i * 32 - h * 16);   // rows of this half in the tile
        if (rows_h <= 0) continue;
#pragma unroll
        for (int r = 8 * h; r < 8 * h + 8; ++r) {
          const int row = 8 * ((r & 7) >> 2) + 4 * (lane >> 5) + (r & 3);   // inside the half
          char* srow = stg + row * PITCH;
          if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int q = 0; q < C::TN / 2; ++q)
              *reinterpret_cast<bf16_t*>(srow + q * 64 + fr * 2) =
                  f32_to_bf16_rn(silu_f32(acc[i][2 * q][r]) * acc[i][2 * q + 1][r]);
          } else {
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
              float x = acc[i][j][r];
              if constexpr (EPI == EPI_GELU) x = gelu_bf16out(x);
              *reinterpret_cast<bf16_t*>(srow + j * 64 + fr * 2) = f32_to_bf16_rn(x);
            }
          }
        }
#pragma unroll
        for (int ps = 0; ps < 16 / RPO; ++ps) {
          const int rr = ps * RPO + lane / CPO;
          if (rr < rows_h) {
            const u32x4_t val = *reinterpret_cast<const u32x4_t*>(stg + rr * PITCH + ch * 16);
            bf16_t* dst = Cout + (long long)(c_row0 + wm * C::WM + i * 32 + h * 16 + rr) * p.ldc + n;
            if (vec && n + 8 <= p.N) {
              *reinterpret_cast<u32x4_t*>(dst) = val;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (n + e < p.N) dst[e] = static_cast<bf16_t>((val[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
          }
        }
      }
    }
  };

  // split contraction: the unit's float32 sums straight from the accumulators
  // (lane: column fr of each 32x32 block, rows 8 (r / 4) + 4 (lane / 32) + r % 4)
  auto epilogue_partial = [&]() __attribute__((always_inline)) {
    float* __restrict__ P = p.partial + (size_t)c_ks * p.M_max * p.ldp;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      if (i >= act_i) continue;
#pragma unroll
      for (int jj = 0; jj < C::TN; ++jj) {
        int col;
        if constexpr (EPI == EPI_SWIGLU) {
          const int h = c_nt * (BN / 2) + (wn * (C::TN / 2) + (jj >> 1)) * 32 + fr;
          if (h >= p.N) continue;
          col = (jj & 1) ? p.N + h : h;
        } else {
          col = c_nt * BN + wn * C::WN + jj * 32 + fr;
          if (col >= p.N) continue;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = wm * C::WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (rl < c_rows) P[(size_t)(c_row0 + rl) * p.ldp + col] = acc[i][jj][r];
        }
      }
    }
  };

  // ---- the stream: slice j of the workgroup's units sits in ring slot j % NST ----
  if (loader) {
    for (int s = 0; s < NST - 1 && s < nsl; ++s) load_next(s);
    int slot_l = NST - 1;
    for (int j = 0; j < nsl; ++j) {
      // slice j has landed once at most the younger slices' loads are
      // outstanding (a loader issues nothing else)
      wait_slices<C::INS, NST - 2>(min(NST - 2, nsl - 1 - j));
      __builtin_amdgcn_s_barrier();      // slice j is visible to all; slot j - 1 is free
      if (j + NST - 1 < nsl) load_next(slot_l);
      slot_l = slot_l + 1 == NST ? 0 : slot_l + 1;
    }
    return;
  }
  cp_setup(0);
  int ct = 0, kt = 0, slot_c = 0;
  for (int j = 0; j < nsl; ++j) {
    __builtin_amdgcn_s_barrier();        // slice j has landed
    const char* sa = smem + slot_c * C::STAGE;
    const char* sb = sa + C::A_BYTES;
    // MFMAs of the slice for the ACT 32-row blocks of the wave that hold rows
    // of the tile; fragments of step kk + 1 are read while those of step kk
    // are multiplied
    auto slice = [&](auto act_c) __attribute__((always_inline)) {
      constexpr int ACT = decltype(act_c)::value;
      bf16x8_t af[2][ACT], bfv[2][C::TN];
      auto read_frags = [&](int buf, int kk) __attribute__((always_inline)) {
        const int chk = kk * 2 + fc;
#pragma unroll
        for (int jj = 0; jj < C::TN; ++jj)
          bfv[buf][jj] = *reinterpret_cast<const bf16x8_t*>(sb + swz_w<C::CPR>(wn * C::WN + jj * 32 + fr, chk));
#pragma unroll
        for (int i = 0; i < ACT; ++i)
          af[buf][i] = *reinterpret_cast<const bf16x8_t*>(sa + swz_w<C::CPR>(wm * C::WM + i * 32 + fr, chk));
      };
      read_frags(0, 0);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        if (kk + 1 < C::KK) read_frags((kk + 1) & 1, kk + 1);
#pragma unroll
        for (int i = 0; i < ACT; ++i)
#pragma unroll
          for (int jj = 0; jj < C::TN; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bfv[kk & 1][jj], acc[i][jj], 0, 0, 0);
      }
    };
    static_assert(C::TM <= 4, "row blocks per wave");
    if constexpr (OCC == 1) {
      // straight-line code per block count (the register file has room)
      switch (act_i) {
        case 1: slice(std::integral_constant<int, 1>{}); break;
        case 2: if constexpr (C::TM >= 2) slice(std::integral_constant<int, 2>{}); break;
        case 3: if constexpr (C::TM >= 3) slice(std::integral_constant<int, 3>{}); break;
        case 4: if constexpr (C::TM >= 4) slice(std::integral_constant<int, 4>{}); break;
        default: break;                  // no rows of the tile in this wave's blocks
      }
    } else {
      // one body, blocks past act_i skipped at run time
      bf16x8_t af[2][C::TM], bfv[2][C::TN];
      auto read_frags = [&](int buf, int kk) __attribute__((always_inline)) {
        const int chk = kk * 2 + fc;
#pragma unroll
        for (int jj = 0; jj < C::TN; ++jj)
          bfv[buf][jj] = *reinterpret_cast<const bf16x8_t*>(sb + swz_w<C::CPR>(wn * C::WN + jj * 32 + fr, chk));
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          if (i < act_i) af[buf][i] = *reinterpret_cast<const bf16x8_t*>(sa + swz_w<C::CPR>(wm * C::WM + i * 32 + fr, chk));
      };
      read_frags(0, 0);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        if (kk + 1 < C::KK) read_frags((kk + 1) & 1, kk + 1);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          if (i < act_i) {
#pragma unroll
            for (int jj = 0; jj < C::TN; ++jj)
              acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bfv[kk & 1][jj], acc[i][jj], 0, 0, 0);
          }
      }
    }
    // the fragments are in registers before the next barrier frees the slot
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    slot_c = slot_c + 1 == NST ? 0 : slot_c + 1;

    if (++kt == nk) {
      if constexpr (SPLIT) epilogue_partial();
      else epilogue();
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int jj = 0; jj < C::TN; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
      kt = 0;
      if (++ct < my_tiles) cp_setup(ct);
    }
  }
}

// Sum of the ksplit partial results of each tile (part 0 first, then 1, ...)
// and the epilogue, over the same tiles as the GEMM launch; four columns per
// thread.
template <int BM, int COLS, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GroupedGemm p, int n_tiles) {
  const int total = (p.offsets == nullptr ? ceil_div(p.M_max, BM) : p.tile_prefix[p.G]) * n_tiles;
  const int KS = p.ksplit;
  const size_t part = (size_t)p.M_max * p.ldp;
  bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.C);
  constexpr int C4 = COLS / 4;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int g, row0, rows, nt;
    decode_tile<BM>(p, n_tiles, tile, g, row0, rows, nt);
    const int c0 = nt * COLS;
    const int ncols = min(COLS, p.N - c0);
    for (int i = threadIdx.x; i < rows * C4; i += blockDim.x) {
      const int r = i / C4, c = (i % C4) * 4;
      if (c >= ncols) continue;
      const float* __restrict__ P = p.partial + (size_t)(row0 + r) * p.ldp + c0 + c;
      float a[4] = {0.0f, 0.0f, 0.0f, 0.0f}, b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c + e < ncols) {
            a[e] += P[ks * part + e];
            if constexpr (EPI == EPI_SWIGLU) b[e] += P[ks * part + p.N + e];
          }
        }
      }
      bf16_t* dst = Cout + (size_t)(row0 + r) * p.ldc + c0 + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c + e >= ncols) continue;
        float v = a[e];
        if constexpr (EPI == EPI_SWIGLU) v = silu_f32(a[e]) * b[e];
        if constexpr (EPI == EPI_GELU) v = gelu_bf16out(a[e]);
        dst[e] = f32_to_bf16_rn(v);
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int BK, int NST, int OCC, int EPI>
hipError_t launch_ws(const GroupedGemm& p, hipStream_t s) {
  using C = CfgW<BM, BN, WGM, WGN, BK, NST>;
  constexpr int LDS = C::lds(EPI);
  static_assert(LDS <= 160 * 1024 / OCC, "LDS per workgroup");
  // 32-bit byte offsets below kRangeEnd: one group's weights and the rows of
  // A must span less than that (gathered A: the source rows, which the
  // caller keeps within the same bound; checked here for M_max rows)
  if (p.K % BK != 0 || p.K >= (1 << 19)) return hipErrorInvalidValue;
  const long long b_group_bytes = (long long)((EPI == EPI_SWIGLU) ? 2 * p.N : p.N) * p.K * 2;
  if (b_group_bytes >= (long long)kRangeEnd || (long long)p.lda * 2 * p.M_max >= (long long)kRangeEnd)
    return hipErrorInvalidValue;
  constexpr int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int n_tiles = ceil_div(p.N, cols);
  if (n_tiles == 0 || p.M_max == 0) return hipSuccess;
  const long long tiles = (long long)(p.offsets == nullptr ? ceil_div(p.M_max, BM)
                                                           : p.M_max / BM + std::min(p.G, p.M_max)) * n_tiles;
  const int KS = p.ksplit > 1 ? p.ksplit : 1;
  if (KS > 1 && (p.partial == nullptr || (p.K / BK) % KS != 0 ||
                 p.ldp < ((EPI == EPI_SWIGLU) ? 2 * p.N : p.N)))
    return hipErrorInvalidValue;
  const long long bound = tiles * KS;
  if (bound > 0x7fffffffLL) return hipErrorInvalidValue;
  const int cus = p.cus > 0 ? std::min(p.cus, num_cus()) : num_cus();
  const int blocks = (int)std::min<long long>(bound, (long long)cus * OCC);
  static std::atomic<bool> allowed[64];   // per device: attribute set (host threads may race)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !allowed[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_ws_kernel<BM, BN, WGM, WGN, BK, NST, OCC, EPI, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_ws_kernel<BM, BN, WGM, WGN, BK, NST, OCC, EPI, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) allowed[dev].store(true, std::memory_order_relaxed);
  }
  if (KS == 1) {
    hipLaunchKernelGGL((gemm_ws_kernel<BM, BN, WGM, WGN, BK, NST, OCC, EPI, false>), dim3((unsigned)blocks),
                       dim3(C::THREADS), LDS, s, p, n_tiles);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_ws_kernel<BM, BN, WGM, WGN, BK, NST, OCC, EPI, true>), dim3((unsigned)blocks),
                     dim3(C::THREADS), LDS, s, p, n_tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((splitk_reduce_kernel<BM, cols, EPI>), dim3((unsigned)std::min<long long>(tiles, 4096)),
                     dim3(256), 0, s, p, n_tiles);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_ws_epi(const GroupedGemm& p, int cfg, hipStream_t s) {
  // SwiGLU needs an even number of 32-column blocks per wave (gate / up
  // pairs): the one-row-of-waves layouts fall back to 2x2 waves there
  constexpr bool SW = EPI == EPI_SWIGLU;
  switch (cfg) {
    //                     BM   BN WGM WGN  BK NST OCC
    case 0: return launch_ws<128, 128, 2, 2, 64, 4, 1, EPI>(p, s);
    case 1: return launch_ws<128, 128, 2, 2, 64, 2, 2, EPI>(p, s);
    case 2: return launch_ws<64, 256, 1, 4, 64, 3, 1, EPI>(p, s);
    case 3: return launch_ws<64, 128, 2, 2, 64, 5, 1, EPI>(p, s);
    case 4: return launch_ws<128, 128, 2, 2, 32, 4, 2, EPI>(p, s);
    // waves side by side over the columns: every wave gets the same rows
    case 5: return launch_ws<128, 128, SW ? 2 : 1, SW ? 2 : 4, 64, 4, 1, EPI>(p, s);
    case 6: return launch_ws<128, 128, SW ? 2 : 1, SW ? 2 : 4, 64, 2, 2, EPI>(p, s);
    case 7: return launch_ws<128, 128, SW ? 2 : 1, SW ? 2 : 4, 32, 4, 2, EPI>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int gemm_ws_bm(int cfg) {
  static const int bm[] = {128, 128, 64, 64, 128, 128, 128, 128};
  return (cfg >= 0 && cfg < kGemmWsConfigs) ? bm[cfg] : 0;
}

int gemm_ws_bn(int cfg) {
  static const int bn[] = {128, 128, 256, 128, 128, 128, 128, 128};
  return (cfg >= 0 && cfg < kGemmWsConfigs) ? bn[cfg] : 0;
}

hipError_t launch_gemm_ws(const GroupedGemm& p, int cfg, hipStream_t s) {
  switch (p.epilogue) {
    case EPI_STORE_ACT: return launch_ws_epi<EPI_STORE_ACT>(p, cfg, s);
    case EPI_SWIGLU: return launch_ws_epi<EPI_SWIGLU>(p, cfg, s);
    case EPI_GELU: return launch_ws_epi<EPI_GELU>(p, cfg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
