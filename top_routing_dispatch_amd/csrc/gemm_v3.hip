// bf16 grouped GEMM on 32x32x16 MFMAs for the deep expert FFN shapes (K a
// multiple of BK), with the tile scheduler and epilogues of gemm.hip:
// C[r, n] = sum_k A[r, k] * B_g[n, k] for the rows r of group g.
//   * WGM x WGN waves per workgroup, each owning a WM x WN block of C (TM x TN
//     MFMA blocks): the default 256x256 tile runs eight waves of 128x64 (two
//     per SIMD); the four-wave forms own 128x128 each (one per SIMD,
//     accumulators in the AGPR half of the register file);
//   * K-slices of BK (32 or 64) elements reach LDS either by buffer-to-LDS
//     DMA into NST / NSTB-deep rings (RSD = 0), or through registers (RSD >
//     0): 16-byte buffer loads one slice ahead, then LDS writes into one of
//     two stages, spread over the MFMAs of the slice before;
//   * a wave skips the MFMAs and fragment reads of 32-row blocks that lie past
//     the tile's last row (groups of a few rows pay only for the weight
//     stream, not for MFMAs on padding).
// LDS rows are BK*2 bytes; the 16-byte chunk c of row r sits in slot
// c ^ ((r / (16 / CPR)) % CPR) (CPR chunks per row), so that the 16 rows read
// by one pass of a fragment load cover all 64 banks once.
#include "common.h"

#include <algorithm>
#include <type_traits>

namespace moe {
namespace {

template <int BM, int BN, int WGM, int WGN, int BK, int NST, int NSTB, int RSD = 0>
struct Cfg3 {
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int NWAVES = WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;     // wave tile
  static constexpr int TM = WM / 32, TN = WN / 32;       // 32x32 MFMA blocks per wave
  static constexpr int RB = BK * 2;                      // bytes per LDS row
  static constexpr int CPR = BK / 8;                     // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;                  // rows per 1 KB load instruction
  static constexpr int KK = BK / 16;                     // MFMA k-steps per slice
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int B_RING = NST * A_BYTES;           // the B ring follows the A ring
  // RSD > 0: slices staged in registers (RSD slices in flight per thread) and
  // written to two LDS stages of A_BYTES + B_BYTES; otherwise the DMA rings
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = RSD > 0 ? 2 * STAGE : NST * A_BYTES + NSTB * B_BYTES;
  static constexpr int A_INS = BM / RPI / NWAVES;        // load instructions per wave per slice
  static constexpr int B_INS = BN / RPI / NWAVES;
  static constexpr int INS = A_INS + B_INS;
  static_assert(BK == 32 || BK == 64, "slice depth");
  static_assert(KK % 2 == 0, "fragment double buffering alternates per k-step");
  static_assert(BM % (RPI * NWAVES) == 0 && BN % (RPI * NWAVES) == 0, "load split");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(NST >= 2 && NSTB >= 2, "ring depths");
  static constexpr int NMAX = NST > NSTB ? NST : NSTB;
  // Within one refill the shallower ring's loads are issued first.
  static constexpr bool A_FIRST = NST <= NSTB;
  __host__ __device__ static constexpr bool is_a(int q) { return A_FIRST ? q < A_INS : q >= B_INS; }
  __host__ __device__ static constexpr int a_idx(int q) { return A_FIRST ? q : q - B_INS; }
  __host__ __device__ static constexpr int b_idx(int q) { return A_FIRST ? q - A_INS : q; }
  __host__ __device__ static constexpr int depth(int q) { return is_a(q) ? NST : NSTB; }

};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc3(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane, buffer -> LDS: lane i lands at lds + 16 * i.
__device__ __forceinline__ void dma16_3(__amdgpu_buffer_rsrc_t r, unsigned voff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int CPR>
__device__ __forceinline__ int swz3(int r, int c) {
  return r * (CPR * 16) + ((c ^ ((r / (16 / CPR)) & (CPR - 1))) << 4);
}

template <int BM, int BN, int WGM, int WGN, int BK, int NST, int NSTB, int RSD, int OCC, bool PERS, int EPI,
          typename OutT>
__global__ __launch_bounds__(64 * WGM * WGN)
__attribute__((amdgpu_waves_per_eu(WGM * WGN / 4 * OCC, WGM * WGN / 4 * OCC)))
void gemm_v3_kernel(const GroupedGemm p, int n_tiles) {
  using C = Cfg3<BM, BN, WGM, WGN, BK, NST, NSTB, RSD>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // PERS: a grid of about one workgroup per CU slot walks the tiles that
  // exist (tile, tile + gridDim.x, ...); otherwise one tile per workgroup.
  const int total = PERS ? tile_count<BM>(p, n_tiles) : 0;
  for (int tile = blockIdx.x;; tile += gridDim.x) {
  int g, row0, rows, nt;
  // split tail (EPI_TAIL_PART): this workgroup's unit covers slices
  // [k_unit * nk, (k_unit + 1) * nk) of its tile
  int k_unit = 0, k_units = 1;
  if constexpr (EPI == EPI_TAIL_PART) {
    int main, r;
    tail_units(tile_count<BM>(p, n_tiles), p.round, p.K / BK, main, r, k_units);
    if ((int)blockIdx.x >= k_units * r) return;
    k_unit = (int)blockIdx.x % k_units;
    decode_tile<BM>(p, n_tiles, main + (int)blockIdx.x / k_units, g, row0, rows, nt);
  } else if constexpr (PERS) {
    if (tile >= total) break;
    decode_tile<BM>(p, n_tiles, tile, g, row0, rows, nt);
  } else {
    if (!map_tile<BM>(p, n_tiles, g, row0, rows, nt)) return;
  }
  // 32-row blocks of this wave that hold at least one row of the tile
  const int act_i = min(C::TM, max(0, ceil_div(rows - wm * C::WM, 32)));

  const int K = p.K;
  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(p.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(p.B) + (long long)g * p.b_group_stride;

  // Byte offsets of this wave's load instructions (rows past the tile end
  // clamped to a valid row: their outputs are never stored).
  const int lrow = lane / C::CPR;
  const int lslot = lane % C::CPR;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc3(A, 0xffffffffu);
  const int b_rows = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc3(B, (unsigned)b_rows * (unsigned)K * 2u);
  unsigned a_off[C::A_INS], b_off[C::B_INS];
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int r = (wave * C::A_INS + q) * C::RPI + lrow;
    const int rr = r < rows ? r : rows - 1;
    const unsigned src = p.a_rows ? (unsigned)p.a_rows[row0 + rr] : (unsigned)(row0 + rr);
    const int c = lslot ^ ((r / (16 / C::CPR)) & (C::CPR - 1));
    a_off[q] = (src * (unsigned)p.lda + c * 8) * 2u;
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int r = (wave * C::B_INS + q) * C::RPI + lrow;
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
    const int c = lslot ^ ((r / (16 / C::CPR)) & (C::CPR - 1));
    b_off[q] = ((unsigned)brow * (unsigned)K + c * 8) * 2u;
  }

  // Slice j of A lives in A slot j % NST, slice j of B in B slot j % NSTB.
  // Iteration it refills A with slice it + NST - 1 and B with slice
  // it + NSTB - 1; load instruction q of an iteration belongs to the
  // shallower ring first, then to the deeper one.
  const int nk = K / BK / k_units;
  if (k_unit > 0) {
    const unsigned k_off = (unsigned)(k_unit * nk) * (unsigned)C::RB;
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q) a_off[q] += k_off;
#pragma unroll
    for (int q = 0; q < C::B_INS; ++q) b_off[q] += k_off;
  }
  auto dma_one = [&](int q, int it) __attribute__((always_inline)) {
    const int j = it + C::depth(q) - 1;
    if (C::is_a(q)) {
      const int qa = C::a_idx(q);
      dma16_3(a_rsrc, a_off[qa] + j * (unsigned)C::RB,
              smem + (j % NST) * C::A_BYTES + (wave * C::A_INS + qa) * 1024);
    } else {
      const int qb = C::b_idx(q);
      dma16_3(b_rsrc, b_off[qb] + j * (unsigned)C::RB,
              smem + C::B_RING + (j % NSTB) * C::B_BYTES + (wave * C::B_INS + qb) * 1024);
    }
  };

  floatx16_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // A wave whose A rows all lie past the tile's last row loads no A (those
  // LDS rows feed only 32-row blocks that no wave multiplies).
  const bool a_live = wave * C::A_INS * C::RPI < rows;

  const int fr = lane & 31;              // fragment row inside a 32-row block
  const int fc = lane >> 5;              // which 8-wide half of a 16-deep step
  bf16x8_t af[2][C::TM], bfv[2][C::TN];

  constexpr int MF = C::TM * C::TN;

  // Fragment read r (0 <= r < TM + TN) of 16-deep step kk of the slice at sa
  // (A) / sb (B), numbered in the order of first use by the MFMAs (block row
  // i, then column j): A0, B0..B(TN-1), A1, ..., A(TM-1).
  // act_c: the number of 32-row blocks of the wave that hold rows of the
  // tile when known at compile time, else -1 (act_i at run time).
  auto frag_read1 = [&](auto act_c, int buf, const char* sa, const char* sb, int kk, int r)
                        __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    const int act = ACT >= 0 ? ACT : act_i;
    const int ch = kk * 2 + fc;
    if (r >= 1 && r <= C::TN) {
      bfv[buf][r - 1] = *reinterpret_cast<const bf16x8_t*>(sb + swz3<C::CPR>(wn * C::WN + (r - 1) * 32 + fr, ch));
    } else {
      const int i = r == 0 ? 0 : r - C::TN;
      if (i == 0 || i < act)
        af[buf][i] = *reinterpret_cast<const bf16x8_t*>(sa + swz3<C::CPR>(wm * C::WM + i * 32 + fr, ch));
    }
  };
  auto frag_reads = [&](auto act_c, int buf, const char* sa, const char* sb, int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < C::TM + C::TN; ++r) frag_read1(act_c, buf, sa, sb, kk, r);
  };
  // MFMAs of one 16-deep step on fragment buffer `buf`.
  auto mfma_all = [&](auto act_c, int buf) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    const int act = ACT >= 0 ? ACT : act_i;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      if (i < act) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfv[buf][j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // FULL: every 32-row block of the wave holds rows of the tile.  Its steps
  // are straight-line code, and each step's fragment reads for the next step
  // (and its refill loads) are placed one after each MFMA, so that they issue
  // while the matrix core works instead of in a burst that leaves it idle.
  auto k_loop = [&](auto full_c, auto al_c) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value;
    constexpr bool AL = decltype(al_c)::value;          // this wave loads A rows
    constexpr int WA = AL ? C::A_INS : 0;
    // Loads younger than the later of this wave's A(kt+1) / B(kt+1) when
    // slice kt+1 is awaited: the deeper ring's loads of the same refill, then
    // the refills of the shallower depth minus two iterations.
    constexpr int WAIT = !AL ? C::B_INS * (NSTB - 2)
                         : NST == NSTB ? (WA + C::B_INS) * (NST - 2)
                         : NSTB > NST ? C::B_INS + (WA + C::B_INS) * (NST - 2)
                                      : WA + (WA + C::B_INS) * (NSTB - 2);
    static_assert(WAIT <= 63, "vmcnt range");
    // Load q of iteration it (iteration it refills A with slice it + NST - 1
    // and B with slice it + NSTB - 1); `exists` skips the check that the
    // slice exists, in the steady part of the loop where it always does.
    auto load_q = [&](int q, int it, bool exists) __attribute__((always_inline)) {
      const int j = it + C::depth(q) - 1;
      if ((AL || !C::is_a(q)) && (exists || j < nk)) dma_one(q, it);
    };
    // Prologue: iterations 1-NMAX .. -1 of the same schedule.
#pragma unroll
    for (int it = 1 - C::NMAX; it < 0; ++it) {
#pragma unroll
      for (int q = 0; q < C::INS; ++q)
        if (it + C::depth(q) - 1 >= 0) load_q(q, it, false);
    }
    // Slice `next` has landed for every wave, and every wave is done with the
    // slots refilled next.  While every refill so far was of an existing
    // slice (next + NMAX - 2 < nk), exactly WAIT younger loads are
    // outstanding; in the last iterations everything is awaited.
    auto slice_ready = [&](bool exact) __attribute__((always_inline)) {
      if (exact) wait_vm<WAIT>();
      else wait_vm<0>();
      __builtin_amdgcn_s_barrier();
    };
    using act_t = std::integral_constant<int, FULL ? C::TM : -1>;
    auto load_frags = [&](int buf, int kt, int kk) __attribute__((always_inline)) {
      frag_reads(act_t{}, buf, smem + (kt % NST) * C::A_BYTES, smem + C::B_RING + (kt % NSTB) * C::B_BYTES, kk);
    };
    auto mfma_step = [&](int buf) __attribute__((always_inline)) { mfma_all(act_t{}, buf); };
    // Instruction order of one straight-line step: MFMA m is followed by the
    // reads r with r * MF / NR == m and the loads d with d * MF / ND == m.
    auto interleave = [&](bool reads, bool refill_here) __attribute__((always_inline)) {
      if constexpr (FULL) {
        constexpr int NR = C::TM + C::TN;
        const int nd = refill_here ? (AL ? C::INS : C::B_INS) : 0;
#pragma unroll
        for (int m = 0; m < MF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
          if (reads) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
              if (r * MF / NR == m) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
          }
#pragma unroll
          for (int d = 0; d < C::INS; ++d)
            if (d < nd && d * MF / nd == m) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM load
        }
      }
    };
    // One slice: refill, KK-1 steps that also read the next step's fragments,
    // then (unless it is the last slice) the hand-over to the next slice and
    // the last step.  steady: every refill of this iteration exists.
    auto slice = [&](int kt, bool steady, bool last) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < C::INS; ++q) load_q(q, kt, steady);
#pragma unroll
      for (int kk = 0; kk < C::KK - 1; ++kk) {
        load_frags((kk + 1) & 1, kt, kk + 1);
        mfma_step(kk & 1);
        interleave(true, kk == 0 && steady);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the last step's fragments are in registers before the slot is handed
      // back; the next slice's first fragments are read while this slice's
      // last MFMAs run
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (!last) {
        slice_ready(steady);
        load_frags(0, kt + 1, 0);
      }
      mfma_step(1);
      interleave(!last, false);
      __builtin_amdgcn_sched_barrier(0);
    };
    slice_ready(C::NMAX - 2 < nk);
    load_frags(0, 0, 0);
    const int n_steady = max(0, nk - C::NMAX + 1);  // iterations whose refills all exist
    int kt = 0;
    for (; kt < n_steady && kt < nk - 1; ++kt) slice(kt, true, false);
    for (; kt < nk - 1; ++kt) slice(kt, false, false);
    slice(nk - 1, false, true);
  };
  // Register-staged slices (RSD > 0): each thread loads its 16-byte chunks of
  // slice j (the same chunks the DMA rings move, so the LDS layout and the
  // fragment reads are those above) into register set j % RSD, and writes
  // them to LDS stage j % 2 during the iteration before slice j is
  // multiplied; the loads of slice j + RSD then reuse those registers.  Slice
  // j's loads are thus issued RSD iterations before they are awaited, and
  // one barrier per iteration hands the stages over.
  // act_c: the wave's count of 32-row blocks holding rows of the tile (a
  // compile-time constant here, so that partial tiles get the interleaved
  // schedule too, with their own MFMA count).
  auto k_loop_rs = [&](auto act_c, auto al_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool AL = decltype(al_c)::value;
    constexpr int MFR = ACT * C::TN;                     // MFMAs per step
    constexpr int RS = RSD > 0 ? RSD : 1;
    static_assert(RS <= 2, "register sets");
    constexpr int WL = (AL ? C::A_INS : 0) + C::B_INS;   // loads (and LDS writes) per slice of this wave
    u32x4_t R[RS][C::INS];
    // Load / LDS write w (0 <= w < WL) of this wave's share of a slice: the A
    // chunks first (when the wave loads A), then the B chunks.
    auto gload1 = [&](auto set_c, int j, int w) __attribute__((always_inline)) {
      constexpr int S = decltype(set_c)::value;
      const int q = AL ? w : C::A_INS + w;
      if (q < C::A_INS) R[S][q] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off[q] + j * (unsigned)C::RB, 0, 0);
      else R[S][q] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_off[q - C::A_INS] + j * (unsigned)C::RB, 0, 0);
    };
    auto lwrite1 = [&](auto set_c, int j, int w) __attribute__((always_inline)) {
      constexpr int S = decltype(set_c)::value;
      const int q = AL ? w : C::A_INS + w;
      char* st = smem + (j & 1) * C::STAGE +
                 (q < C::A_INS ? (wave * C::A_INS + q) * 1024 : C::A_BYTES + (wave * C::B_INS + q - C::A_INS) * 1024);
      *reinterpret_cast<u32x4_t*>(st + lane * 16) = R[S][q];
    };
    auto gload = [&](auto set_c, int j) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < WL; ++w) gload1(set_c, j, w);
    };
    auto lwrite = [&](auto set_c, int j) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < WL; ++w) lwrite1(set_c, j, w);
    };
    // the writes and loads of one slice are spread over the first KK - 1
    // steps: step kk takes w in [w_lo(kk), w_lo(kk + 1))
    auto w_lo = [](int kk) { return kk * WL / (C::KK - 1); };
    auto load_frags = [&](int buf, int kt, int kk) __attribute__((always_inline)) {
      const char* sa = smem + (kt & 1) * C::STAGE;
      frag_reads(act_c, buf, sa, sa + C::A_BYTES, kk);
    };
    // fragment reads of a step: A0 and the B blocks always, A1.. as active
    constexpr int NR = (ACT > 1 ? ACT : 1) + C::TN;
    // one MFMA, then the fragment reads, LDS writes and loads that follow it
    auto interleave = [&](bool reads, int nw) __attribute__((always_inline)) {
      if constexpr (MFR > 0) {
#pragma unroll
        for (int m = 0; m < MFR; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
          if (reads) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
              if (r * MFR / NR == m) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
          }
#pragma unroll
          for (int d = 0; d < C::INS; ++d)
            if (d < nw && d * MFR / nw == m) {
              __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // one LDS write
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one load
            }
        }
      }
    };
    // Iteration kt multiplies slice kt (stage kt % 2); wr: slice kt + 1 exists
    // and goes from its registers to the other stage; ld: slice kt + 1 + RS
    // exists and is loaded into the registers just written; last: no next slice.
    auto slice = [&](int kt, auto set_c, bool wr, bool ld, bool last) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < C::KK - 1; ++kk) {
        // The reads of this stage and the writes to the other one go out in
        // the order the schedule below interleaves them (the compiler keeps
        // LDS reads and writes in source order, as it cannot tell the two
        // stages apart).
        const char* sa = smem + (kt & 1) * C::STAGE;
        const int nw = w_lo(kk + 1) - w_lo(kk);
        constexpr int SLOTS = MFR > 0 ? MFR : 1;
#pragma unroll
        for (int m = 0; m < SLOTS; ++m) {
#pragma unroll
          for (int r = 0; r < NR; ++r)
            if (r * SLOTS / NR == m) frag_read1(act_c, (kk + 1) & 1, sa, sa + C::A_BYTES, kk + 1, r);
#pragma unroll
          for (int d = 0; d < C::INS; ++d)
            if (d < nw && d * SLOTS / nw == m) {
              if (wr) lwrite1(set_c, kt + 1, w_lo(kk) + d);
              if (ld) gload1(set_c, kt + 1 + RS, w_lo(kk) + d);
            }
        }
        mfma_all(act_c, kk & 1);
        interleave(true, wr && ld ? nw : 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // this wave's reads of slice kt and writes of slice kt + 1 are done
      // before the barrier; after it every wave's writes are visible and the
      // stage of slice kt may be refilled
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (!last) {
        __builtin_amdgcn_s_barrier();
        load_frags(0, kt + 1, 0);
      }
      mfma_all(act_c, 1);
      interleave(!last, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // register set of the slice written in iteration kt: (kt + 1) % RS
    auto slice_any = [&](int kt, bool wr, bool ld, bool last) __attribute__((always_inline)) {
      if (RS == 1 || (kt + 1) % RS == 0) slice(kt, std::integral_constant<int, 0>{}, wr, ld, last);
      else slice(kt, std::integral_constant<int, RS - 1>{}, wr, ld, last);
    };
    gload(std::integral_constant<int, 0>{}, 0);
    lwrite(std::integral_constant<int, 0>{}, 0);
    if (1 < nk) gload(std::integral_constant<int, 1 % RS>{}, 1);
    if (RS == 2 && 2 < nk) gload(std::integral_constant<int, 0>{}, 2);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    load_frags(0, 0, 0);
    const int n_full = max(0, nk - 1 - RS);   // iterations that write and load
    int kt = 0;
    for (; kt + RS <= n_full; kt += RS) {
      slice(kt, std::integral_constant<int, 1 % RS>{}, true, true, false);
      if constexpr (RS == 2) slice(kt + 1, std::integral_constant<int, 0>{}, true, true, false);
    }
    for (; kt < n_full; ++kt) slice_any(kt, true, true, false);
    for (; kt < nk - 1; ++kt) slice_any(kt, true, false, false);
    slice_any(nk - 1, false, false, true);
  };
  if constexpr (RSD > 0) {
    // one instance per count of active 32-row blocks (a wave with none
    // still loads and writes its share of the slices)
    auto by_act = [&](auto act_c) __attribute__((always_inline)) {
      if (a_live) k_loop_rs(act_c, std::true_type{});
      else k_loop_rs(act_c, std::false_type{});
    };
    static_assert(C::TM <= 4, "active block counts");
    switch (act_i) {
      case 0: by_act(std::integral_constant<int, 0>{}); break;
      case 1: by_act(std::integral_constant<int, 1>{}); break;
      case 2: if constexpr (C::TM >= 2) by_act(std::integral_constant<int, 2>{}); break;
      case 3: if constexpr (C::TM >= 3) by_act(std::integral_constant<int, 3>{}); break;
      default: if constexpr (C::TM >= 4) by_act(std::integral_constant<int, 4>{}); break;
    }
  } else {
    if (act_i == C::TM) {
      if (a_live) k_loop(std::true_type{}, std::true_type{});
      else k_loop(std::true_type{}, std::false_type{});
    } else {
      if (a_live) k_loop(std::false_type{}, std::true_type{});
      else k_loop(std::false_type{}, std::false_type{});
    }
  }
  wait_vm<0>();   // nothing is in flight into LDS when the staging below reuses it

  if (EPI == EPI_TAIL_PART && k_units > 1) {
    // float32 sums of the unit as block blockIdx.x of BM x BN floats (row
    // major); a lane holds column lane % 32 and rows 8 (r / 4) + 4 (lane / 32)
    // + r % 4 of each 32x32 block, and blocks past the tile's rows stay unset.
    // (One unit per tile: the whole sum, stored below like EPI_STORE_ACT.)
    float* __restrict__ P = p.tail_part + (size_t)blockIdx.x * (BM * BN);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      if (i >= act_i) continue;
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * C::WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          P[row * BN + wn * C::WN + j * 32 + (lane & 31)] = acc[i][j][r];
        }
    }
    return;
  }
  // Epilogue: the activation is applied in registers, each wave's output
  // block goes to its own LDS region and is read back as 16-byte row chunks
  // for full-width global stores.  One LDS write instruction covers rows r and
  // r+4; they land on different banks through a 16-byte row pad, or, where the
  // padded block does not fit, by swapping the 64-byte halves of rows with
  // bit 2 of the row index set.
  static_assert(sizeof(OutT) == 2, "16-bit outputs");
  constexpr int OC = (EPI == EPI_SWIGLU) ? C::WN / 2 : C::WN;   // output columns per wave
  constexpr bool PAD = C::NWAVES * C::WM * (OC * 2 + 16) <= C::LDS;
  constexpr int PITCH = OC * 2 + (PAD ? 16 : 0);
  static_assert(C::NWAVES * C::WM * PITCH <= C::LDS, "output staging fits in the rings");
  static_assert(PAD || (OC * 2) % 128 == 0, "half swap needs rows of whole 128-byte pairs");
  auto sbyte = [](int row, int byte) { return PAD ? byte : (byte ^ (((row >> 2) & 1) << 6)); };
  __builtin_amdgcn_s_barrier();          // every wave is done with the ring
  char* stg = smem + wave * (C::WM * PITCH);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    if (i >= act_i) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      char* srow = stg + row * PITCH;
      if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int q = 0; q < C::TN / 2; ++q)
          *reinterpret_cast<bf16_t*>(srow + sbyte(row, q * 64 + (lane & 31) * 2)) =
              f32_to_bf16_rn(silu_f32(acc[i][2 * q][r]) * acc[i][2 * q + 1][r]);
      } else {
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          float v = acc[i][j][r];
          if constexpr (EPI == EPI_GELU) v = gelu_bf16out(v);
          *reinterpret_cast<bf16_t*>(srow + sbyte(row, j * 64 + (lane & 31) * 2)) = f32_to_bf16_rn(v);
        }
      }
    }
  }
  constexpr int CPO = OC / 8;            // 16-byte chunks per output row
  constexpr int RPO = 64 / CPO;          // rows per pass of the wave
  static_assert(64 % CPO == 0 && C::WM % RPO == 0, "store passes");
  OutT* __restrict__ Cout = static_cast<OutT*>(p.C);
  const int col0 = (EPI == EPI_SWIGLU) ? nt * (BN / 2) + wn * OC : nt * BN + wn * OC;
  const int rows_w = min(C::WM, rows - wm * C::WM);   // this wave's rows inside the tile
  const bool vec = (p.ldc % 8 == 0) && ((reinterpret_cast<uintptr_t>(p.C) & 15) == 0);
  const int ch = lane % CPO;
  const int n = col0 + ch * 8;
#pragma unroll
  for (int ps = 0; ps < C::WM / RPO; ++ps) {
    const int rr = ps * RPO + lane / CPO;
    if (rr < rows_w) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + rr * PITCH + sbyte(rr, ch * 16));
      OutT* dst = Cout + (long long)(row0 + wm * C::WM + rr) * p.ldc + n;
      if (vec && n + 8 <= p.N) {
        *reinterpret_cast<u32x4_t*>(dst) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < p.N) dst[e] = static_cast<OutT>((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      }
    }
  }
  if constexpr (!PERS) break;
  __builtin_amdgcn_s_barrier();          // the staging reads are done before the next tile's loads land
  }
}

// Sum of each split-tail tile's units (unit 0 first, then 1, ...) into C,
// rounded to bf16: one workgroup per 16 rows of a tile, four columns per
// thread.  The grid covers `round` tiles (an upper bound of those left over).
template <int BM, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const GroupedGemm p, int n_tiles) {
  int main, r, S;
  tail_units(tile_count<BM>(p, n_tiles), p.round, p.K / 64, main, r, S);
  const int t = blockIdx.x;
  if (t >= r || S == 1) return;      // one unit per tile: stored by the GEMM itself
  int g, row0, rows, nt;
  decode_tile<BM>(p, n_tiles, main + t, g, row0, rows, nt);
  const int rb = blockIdx.y * 16;
  if (rb >= rows) return;
  const float* __restrict__ P = p.tail_part + (size_t)t * S * (BM * BN);
  bf16_t* __restrict__ Cout = static_cast<bf16_t*>(p.C);
  constexpr int C4 = BN / 4;
  for (int i = threadIdx.x; i < 16 * C4; i += blockDim.x) {
    const int rr = rb + i / C4, c = (i % C4) * 4;
    if (rr >= rows) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = P[rr * BN + c + e];
    for (int k = 1; k < S; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += P[(size_t)k * (BM * BN) + rr * BN + c + e];
    }
    const int n = nt * BN + c;
    bf16_t* dst = Cout + (size_t)(row0 + rr) * p.ldc + n;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < p.N) dst[e] = f32_to_bf16_rn(v[e]);
  }
}

inline int m_bound3(const GroupedGemm& p, int bm) {
  if (p.offsets == nullptr) return ceil_div(p.M_max, bm);
  return p.M_max / bm + (p.G < p.M_max ? p.G : p.M_max);
}

template <int BM, int BN, int WGM, int WGN, int BK, int NST, int NSTB, int RSD, int OCC, bool PERS, int EPI>
hipError_t launch_cfg3(const GroupedGemm& p, hipStream_t s) {
  using C = Cfg3<BM, BN, WGM, WGN, BK, NST, NSTB, RSD>;
  if (p.K % BK != 0) return hipErrorInvalidValue;
  const int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int n_tiles = ceil_div(p.N, cols);
  const int m_tiles = m_bound3(p, BM);
  if (m_tiles == 0 || n_tiles == 0) return hipSuccess;
  long long blocks = (long long)m_tiles * n_tiles;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (PERS && p.tail_mode != 0) return hipErrorInvalidValue;
  if (PERS) blocks = std::min<long long>(blocks, (long long)num_cus() * OCC);
  if ((p.tail_mode == 2) != (EPI == EPI_TAIL_PART)) return hipErrorInvalidValue;
  if (p.tail_mode == 2) {
    // at most `round` units, each a block of the float32 buffer
    if (p.round <= 0 || p.tail_part == nullptr || p.tail_cap < p.round || PERS || p.offsets == nullptr)
      return hipErrorInvalidValue;
    blocks = p.round;
  }
  // dynamic LDS above 64 KB has to be allowed explicitly, once per device
  static std::atomic<bool> allowed[64];   // per device: attribute set (host threads may race)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !allowed[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_v3_kernel<BM, BN, WGM, WGN, BK, NST, NSTB, RSD, OCC, PERS, EPI, bf16_t>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) allowed[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL((gemm_v3_kernel<BM, BN, WGM, WGN, BK, NST, NSTB, RSD, OCC, PERS, EPI, bf16_t>), dim3((unsigned)blocks),
                     dim3(C::THREADS), C::LDS, s, p, n_tiles);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_v3_epi(const GroupedGemm& p, int cfg, hipStream_t s) {
  switch (cfg) {
    //                       BM   BN WGM WGN  BK NST NSTB RSD OCC PERS
    // one workgroup per CU
    case 0: return launch_cfg3<256, 256, 2, 4, 64, 2, 3, 0, 1, false, EPI>(p, s);
    case 1: return launch_cfg3<256, 256, 2, 4, 64, 2, 2, 0, 1, false, EPI>(p, s);
    case 2: return launch_cfg3<256, 256, 2, 2, 64, 2, 3, 0, 1, false, EPI>(p, s);
    case 3: return launch_cfg3<256, 256, 2, 2, 64, 2, 2, 0, 1, false, EPI>(p, s);
    case 4: return launch_cfg3<256, 256, 2, 4, 32, 4, 4, 0, 1, false, EPI>(p, s);
    case 11: return launch_cfg3<128, 256, 1, 4, 32, 4, 4, 0, 1, false, EPI>(p, s);
    // two workgroups per CU (<= 80 KB of LDS each)
    case 5: return launch_cfg3<128, 128, 2, 2, 32, 4, 4, 0, 2, false, EPI>(p, s);
    case 6: return launch_cfg3<128, 128, 2, 2, 64, 2, 2, 0, 2, false, EPI>(p, s);
    case 7: return launch_cfg3<128, 128, 2, 2, 64, 2, 3, 0, 2, false, EPI>(p, s);
    case 8: return launch_cfg3<128, 256, 2, 2, 32, 3, 3, 0, 2, false, EPI>(p, s);
    // persistent weight streaming for shallow groups (one m-tile per group)
    case 9: return launch_cfg3<64, 256, 1, 4, 64, 4, 4, 0, 1, true, EPI>(p, s);
    case 10: return launch_cfg3<64, 256, 1, 4, 32, 4, 4, 0, 2, true, EPI>(p, s);
    // register-staged slices, two LDS stages
    case 12: return launch_cfg3<256, 256, 2, 2, 64, 2, 2, 1, 1, false, EPI>(p, s);
    case 13: return launch_cfg3<256, 256, 2, 4, 64, 2, 2, 1, 1, false, EPI>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_tail_reduce(const GroupedGemm& g, hipStream_t s) {
  if (g.tail_mode != 2 || g.round <= 0 || g.tail_part == nullptr || g.epilogue != EPI_TAIL_PART || g.K % 64 != 0)
    return hipErrorInvalidValue;
  const int n_tiles = ceil_div(g.N, 256);
  if (n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((tail_reduce_kernel<256, 256>), dim3((unsigned)g.round, 256 / 16), dim3(256), 0, s, g, n_tiles);
  return hipGetLastError();
}

int gemm_v3_bm(int cfg) {
  static const int bm[] = {256, 256, 256, 256, 256, 128, 128, 128, 128, 64, 64, 128, 256, 256};
  return (cfg >= 0 && cfg < kGemmV3Configs) ? bm[cfg] : 0;
}

hipError_t launch_gemm_v3(const GroupedGemm& p, int cfg, hipStream_t s) {
  if (p.epilogue == EPI_TAIL_PART) {
    // the split tail runs on the 256x256 configurations with one workgroup
    // per CU (DMA rings, register-staged slices)
    if (cfg == 0) return launch_cfg3<256, 256, 2, 4, 64, 2, 3, 0, 1, false, EPI_TAIL_PART>(p, s);
    if (cfg == 13) return launch_cfg3<256, 256, 2, 4, 64, 2, 2, 1, 1, false, EPI_TAIL_PART>(p, s);
    return hipErrorInvalidValue;
  }
  switch (p.epilogue) {
    case EPI_STORE_ACT: return launch_v3_epi<EPI_STORE_ACT>(p, cfg, s);
    case EPI_SWIGLU: return launch_v3_epi<EPI_SWIGLU>(p, cfg, s);
    case EPI_GELU: return launch_v3_epi<EPI_GELU>(p, cfg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
