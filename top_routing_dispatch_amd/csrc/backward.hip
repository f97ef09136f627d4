// Backward pass of the MoE layer, the routing held fixed ("Top-k 路由" page,
// 門控網路的梯度流: the gradient flows through the selected experts' gate
// scores, unselected experts get none; "从 Dense FFN 到 MoE" §9: selected
// experts get the task gradient, the router gets it through the selected
// weights and the balance loss's gradient through the soft importance).
// Kernels here:
//   transpose_bf16   batched [G][R][C] -> [G][C][R] (weights for the
//                    data-gradient GEMMs, which then run on the forward's
//                    grouped kernels);
//   bw_combine       per token: dw[t, j] = <dy[t], y_perm[row]> and
//                    dy_perm[row] = w[t, j] dy[t];
//   bw_act           SwiGLU / GELU backward, elementwise over the expert rows;
//   wgrad            grouped over the contraction: C_g = A_g^T B_g over the
//                    rows of group g (weight gradients; MFMA 16x16x32, the
//                    row slices transposed into LDS);
//   router_grad      per token: d loss / d logits through the combine weights
//                    of the selected experts plus the balance loss;
//   gemm_f32_strided small float32 products of the router (weight gradient
//                    and the input gradient of the router).
// Every sum has a fixed order: the results do not depend on scheduling.
#include "common.h"

#include <cstdlib>

#include <algorithm>

namespace moe {
namespace {

__device__ __forceinline__ float bf(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ in, bf16_t* __restrict__ out,
                                                             int R, int C, const int32_t* __restrict__ offsets) {
  __shared__ bf16_t tile[64][66];
  const long long g = blockIdx.z;
  // a group without rows is never read transposed (the grouped products
  // make no tiles for it): skip it (uniform per workgroup)
  if (offsets != nullptr && offsets[g + 1] == offsets[g]) return;
  const bf16_t* src = in + g * (long long)R * C;
  bf16_t* dst = out + g * (long long)R * C;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // the 16 loads of a thread without branches between them (indices clamped;
  // the clamped copies land in tile entries that are never written out)
  bf16_t v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)
    v[q] = src[(long long)min(r0 + ty + 4 * q, R - 1) * C + min(c0 + tx, C - 1)];
#pragma unroll
  for (int q = 0; q < 16; ++q) tile[ty + 4 * q][tx] = v[q];
  __syncthreads();
  for (int i = ty; i < 64; i += 4)
    if (c0 + i < C && r0 + tx < R) dst[(long long)(c0 + i) * R + r0 + tx] = tile[tx][i];
}

// ---------------------------------------------------------------------------
// One workgroup per token.  Thread i sums the products of elements i, i+256,
// ... in order; the 256 partial sums are added by a fixed tree.
__global__ __launch_bounds__(256) void bw_combine_kernel(const bf16_t* __restrict__ dy, const bf16_t* __restrict__ yp,
                                                         const int32_t* __restrict__ row_of,
                                                         const float* __restrict__ tw, int k, int D,
                                                         float* __restrict__ dw, bf16_t* __restrict__ dyp) {
  __shared__ float red[256];
  const int t = blockIdx.x;
  for (int j = 0; j < k; ++j) {
    const int r = row_of[(long long)t * k + j];
    if (r < 0) {                                          // uniform: dropped, no gradient
      if (threadIdx.x == 0) dw[(long long)t * k + j] = 0.0f;
      continue;
    }
    const float w = tw[(long long)t * k + j];
    float s = 0.0f;
    for (int d = threadIdx.x; d < D; d += 256) {
      const float g = bf(dy[(long long)t * D + d]);
      s = fmaf(g, bf(yp[(long long)r * D + d]), s);
      dyp[(long long)r * D + d] = f32_to_bf16_rn(w * g);
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int h = 128; h >= 1; h >>= 1) {
      if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x == 0) dw[(long long)t * k + j] = red[0];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// SwiGLU: gu = [G | U] (row r: G in 0..F-1, U in F..2F-1), dh = d loss / dH;
//   dG = dh * U * silu'(G), dU = dh * silu(G), silu'(g) = s(g) (1 + g (1 - s(g))).
// GELU: gu = Z (F columns); dZ = dh * (Phi(z) + z phi(z)).
// Rows from rows_valid on (a device count) are skipped.
// Eight consecutive columns per item (F % 8 == 0): 16-byte loads and stores.
__global__ __launch_bounds__(256) void bw_act_kernel(const bf16_t* __restrict__ gu, const bf16_t* __restrict__ dh,
                                                     bf16_t* __restrict__ dgu, const int32_t* __restrict__ rows_valid,
                                                     int rows_max, int F, int swiglu) {
  const int rows = rows_valid ? min(*rows_valid, rows_max) : rows_max;
  const int F8 = F / 8;
  const long long n = (long long)rows * F8;
  const int ldg = swiglu ? 2 * F : F;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const long long r = i / F8;
    const int f = (int)(i % F8) * 8;
    const uint4 gq = *reinterpret_cast<const uint4*>(gu + r * ldg + f);
    const uint4 dq = *reinterpret_cast<const uint4*>(dh + r * F + f);
    const uint4 uq = swiglu ? *reinterpret_cast<const uint4*>(gu + r * ldg + F + f) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, dw4[4] = {dq.x, dq.y, dq.z, dq.w},
                   uw[4] = {uq.x, uq.y, uq.z, uq.w};
    uint32_t o1[4], o2[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t a1 = 0, a2 = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float g = __uint_as_float(h ? (gw[q] & 0xffff0000u) : (gw[q] << 16));
        const float d = __uint_as_float(h ? (dw4[q] & 0xffff0000u) : (dw4[q] << 16));
        uint32_t r1, r2 = 0;
        if (swiglu) {
          const float u = __uint_as_float(h ? (uw[q] & 0xffff0000u) : (uw[q] << 16));
          const float sg = 1.0f / (1.0f + expf(-g));
          r1 = f32_to_bf16_rn(d * u * sg * (1.0f + g * (1.0f - sg)));
          r2 = f32_to_bf16_rn(d * g * sg);
        } else {
          const float cdf = 0.5f * (1.0f + erff(g * 0.70710678118654752f));
          const float pdf = 0.39894228040143268f * expf(-0.5f * g * g);
          r1 = f32_to_bf16_rn(d * (cdf + g * pdf));
        }
        a1 |= r1 << (16 * h);
        a2 |= r2 << (16 * h);
      }
      o1[q] = a1;
      o2[q] = a2;
    }
    *reinterpret_cast<uint4*>(dgu + r * ldg + f) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    if (swiglu) *reinterpret_cast<uint4*>(dgu + r * ldg + F + f) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
  }
}

// ---------------------------------------------------------------------------
// C_g[m, n] = sum over rows r of group g of A[r, m] * B[b_row(r), n]
// (float32 out, [G][M][N]); A [rows][lda] and B [*][ldb] bf16 (lda, ldb,
// M, N multiples of 4).  b_rows (or NULL) maps a row to the B row it reads.
// offsets [G+1] (NULL: one group of rows_max rows).  BMxBN tile per
// workgroup (128x128 on four waves, or 256x256 on eight), 32 rows per slice.  A slice is staged transposed in LDS ([m][r],
// [n][r]) so that the MFMA operands (8 consecutive rows of one column) are
// 16-byte reads: each thread loads an 8-row x 4-column block of A or B (8-byte
// loads), transposes it in registers and stores four 16-byte columns.  The
// next slice's loads are in flight while the current one is multiplied (two
// LDS buffers, one barrier per slice).  Wave tiles of 64x64 or 128x64 (blocks
// of v_mfma_f32_16x16x32_bf16).  Empty groups write zeros.
constexpr int kWgP = 40;                 // LDS row pitch in bf16 (32 rows + pad)

struct WgStage {
  uint2 v[8];
  uint32_t ok;     // bit i: row i of the block exists and the column group is inside C
};

// thread -> operand (0: A, 1: B), 8-row group, 4-column group of the slice.
// Nothing here waits for a load: rows past the group's end and column groups
// past C read a valid element, and wg_store zeroes them from the `ok` bits
// when the values are consumed (slices later).  The row map is read with
// scalar loads: the rows of one wave's threads are the RGW (1 or 2) row
// groups starting at lane 0's, a wave-uniform range, and a scalar load's wait
// does not also wait for the data loads of the slices in flight.
template <int RGW>
__device__ __forceinline__ void wg_load(WgStage& st, const bf16_t* __restrict__ P, int ld,
                                        const int32_t* __restrict__ rows_map, int r_base, int r_hi, int c_base, int C) {
  const bool col_ok = c_base < C;
  const int cc = col_ok ? c_base : 0;
  long long pr[8];
  if (rows_map != nullptr) {                 // uniform per wave (B operand waves)
    const int rb0 = __builtin_amdgcn_readfirstlane(r_base);
    const int rh = __builtin_amdgcn_readfirstlane(r_hi);
    const_i32* rm = (const_i32*)rows_map;
    int sidx[RGW][8];
    if (rb0 + 8 * RGW <= rh) {               // whole range inside the group: one wide scalar load
#pragma unroll
      for (int q = 0; q < RGW; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) sidx[q][i] = rm[rb0 + q * 8 + i];
    } else {
#pragma unroll
      for (int q = 0; q < RGW; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) sidx[q][i] = rm[min(rb0 + q * 8 + i, rh - 1)];
    }
    const int q_l = (r_base - rb0) >> 3;     // 0 .. RGW-1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int v = sidx[0][i];
#pragma unroll
      for (int q = 1; q < RGW; ++q) v = q_l == q ? sidx[q][i] : v;
      pr[i] = (long long)v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = (long long)min(r_base + i, r_hi - 1);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) st.v[i] = *reinterpret_cast<const uint2*>(P + pr[i] * ld + cc);
  uint32_t ok = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) ok |= (col_ok && r_base + i < r_hi) ? (1u << i) : 0u;
  st.ok = ok;
}

// Column c of the LDS slice holds its 32 rows as four 8-row chunks of 16
// bytes; chunk q sits in slot wg_slot<SWZ>(c, q), a permutation of the four
// chunks that depends on the column only through c >> 3, so that the 16-byte
// stores of consecutive threads (columns 4 apart, 80 dwords) and the
// fragment reads (consecutive columns) spread over the banks.  Measured on
// MI355X (LDS bank-conflict cycles of the Mixtral-shaped weight gradients):
// 847M without a permutation, 462M with SWZ 1, 269M with SWZ 2 (the default).
template <int SWZ>
__device__ __forceinline__ int wg_slot(int col, int q) {
  if constexpr (SWZ == 1) return q ^ ((col >> 4) & 3);
  else if constexpr (SWZ == 2) return q ^ (((col >> 3) ^ (col >> 4)) & 3);
  else return q;
}

// slot0 = the slot of the thread's row group in its four columns.
__device__ __forceinline__ void wg_store(const WgStage& st, bf16_t* lds_cols, int slot0) {
  const int r_off = slot0 * 8;
  uint2 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = ((st.ok >> i) & 1u) ? st.v[i] : make_uint2(0u, 0u);
  // column c of the block gets rows 0..7: dword j = row 2j | row 2j+1 << 16
  uint4 o[4];
  uint32_t* w = reinterpret_cast<uint32_t*>(o);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint2 a = v[2 * j], b = v[2 * j + 1];
    w[0 * 4 + j] = (a.x & 0xffffu) | (b.x << 16);
    w[1 * 4 + j] = (a.x >> 16) | (b.x & 0xffff0000u);
    w[2 * 4 + j] = (a.y & 0xffffu) | (b.y << 16);
    w[3 * 4 + j] = (a.y >> 16) | (b.y & 0xffff0000u);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(lds_cols + c * kWgP + r_off) = o[c];
}

template <int BM, int BN, int WGM, int WGN, int SWZ>
__global__ __launch_bounds__(64 * WGM * WGN) void wgrad_kernel(const bf16_t* __restrict__ A, int lda,
                                                               const bf16_t* __restrict__ B, int ldb,
                                                               const int32_t* __restrict__ b_rows,
                                                               const int32_t* __restrict__ offsets, int rows_max,
                                                               int M, int N, float* __restrict__ C) {
  static_assert(BM + BN == 64 * WGM * WGN, "one 8x4 staging block per thread");
  constexpr int WM = BM / WGM, WN = BN / WGN;        // wave tile
  constexpr int TM = WM / 16, TN = WN / 16;           // 16x16 blocks per wave
  constexpr int RGW = 256 / BN;                       // row groups per B wave
  static_assert(BN == 128 || BN == 256, "B waves cover 1 or 2 row groups");
  static_assert(BM % 64 == 0, "A and B threads in separate waves");
  __shared__ __attribute__((aligned(16))) bf16_t S[2][(BM + BN) * kWgP];   // [buffer][A cols, then B cols][row]
  const int g = blockIdx.z;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int r_lo = offsets ? offsets[g] : 0;
  const int r_hi = offsets ? offsets[g + 1] : rows_max;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  // staging role: threads 0..BM-1 load A, BM..BM+BN-1 load B; (8-row group, 4-column group)
  // wave-uniform (BM is a multiple of 64): the operand pointers below are
  // scalar values, so the row map is read with scalar loads
  const bool isb = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64) * 64 >= BM;
  const int sid = isb ? threadIdx.x - BM : threadIdx.x;
  const int ncg = (isb ? BN : BM) / 4;
  const int rg = sid / ncg;
  const int cg = (sid % ncg) * 4;
  const bf16_t* P = isb ? B : A;
  const int ld = isb ? ldb : lda;
  const int32_t* rmap = isb ? b_rows : nullptr;
  const int c_base = (isb ? n0 : m0) + cg;
  const int C_lim = isb ? N : M;
  const int lds_col = (isb ? BM : 0) + cg;
  const int slot_st = wg_slot<SWZ>(lds_col, rg);   // the same for the thread's four columns

  floatx4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][j][q] = 0.0f;

  // Slices j = 0, 1, ... of the group's rows: slice j is multiplied from
  // LDS buffer j % 2; its registers were loaded three slices earlier (four
  // register stages, slice s in stage s % 4), so a load has three slices of
  // MFMA work to arrive in.  The loads and stores run unconditionally (slices
  // past the group's end read clamped rows and store zeros); only the MFMA
  // part is skipped there.  A load guarded by a condition is moved by the
  // compiler down to its use, which would leave nothing in flight.
  const int nsl = (r_hi - r_lo + 31) / 32;
  WgStage st[4];
  if (nsl > 0) {
#pragma unroll
    for (int q = 0; q < 3; ++q) wg_load<RGW>(st[q], P, ld, rmap, r_lo + q * 32 + rg * 8, r_hi, c_base, C_lim);
    wg_store(st[0], &S[0][lds_col * kWgP], slot_st);
  }
  __syncthreads();
  const int fc = lane & 15, fq = lane >> 4;    // fragment column; 8-row chunk (rows 8 fq .. 8 fq + 7)
  // one slice with compile-time register stages: L loads slice j + 3, W
  // stores slice j + 1
  auto slice = [&](int j, WgStage& ld_st, WgStage& wr_st) __attribute__((always_inline)) {
    wg_load<RGW>(ld_st, P, ld, rmap, r_lo + (j + 3) * 32 + rg * 8, r_hi, c_base, C_lim);
    if (j < nsl) {                         // uniform
      const bf16_t* As = S[j & 1];
      const bf16_t* Bs = S[j & 1] + BM * kWgP;
      bf16x8_t fb[TN];
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
        fb[jj] = *reinterpret_cast<const bf16x8_t*>(
            Bs + (wn * WN + jj * 16 + fc) * kWgP + (wg_slot<SWZ>(BM + wn * WN + jj * 16 + fc, fq) << 3));
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(
            As + (wm * WM + i * 16 + fc) * kWgP + (wg_slot<SWZ>(wm * WM + i * 16 + fc, fq) << 3));
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[jj], acc[i][jj], 0, 0, 0);
      }
    }
    wg_store(wr_st, &S[(j + 1) & 1][lds_col * kWgP], slot_st);
    __syncthreads();                       // slice j + 1 is stored; slice j's reads are done
  };
  for (int j = 0; j < nsl; j += 4) {
    slice(j, st[3], st[1]);
    slice(j + 1, st[0], st[2]);
    slice(j + 2, st[1], st[3]);
    slice(j + 3, st[2], st[0]);
  }
  // C block (i, j): lane holds column n = lane & 15, rows m = 4 (lane >> 4) + q
  float* Cg = C + (long long)g * M * N;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + q;
        const int n = n0 + wn * WN + j * 16 + (lane & 15);
        if (m < M && n < N) Cg[(long long)m * N + n] = acc[i][j][q];
      }
}

// ---------------------------------------------------------------------------
__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wave per token, lanes over the experts (EPL per lane).
template <int EPL>
__global__ __launch_bounds__(256) void router_grad_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ idx, const float* __restrict__ tw,
                                                          const float* __restrict__ dw,
                                                          const int32_t* __restrict__ counts, int T, int E, int k,
                                                          int scoring, int renormalize, float alpha,
                                                          float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const bool sig = scoring == SIGMOID_BIAS;
  float s[EPL], pr[EPL], c[EPL], gsel[EPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    s[i] = e < E ? logits[(long long)t * E + e] : 0.0f;
    if (e < E) m = fmaxf(m, s[i]);
    c[i] = e < E ? alpha * (float)E * ((float)counts[e] / ((float)T * (float)k)) / (float)T : 0.0f;
    gsel[i] = 0.0f;
  }
  // soft probabilities of the balance loss (and of the raw-probability gate)
  float z = 0.0f;
  if (sig) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      pr[i] = lane + 64 * i < E ? 1.0f / (1.0f + expf(-s[i])) : 0.0f;
      z += pr[i];
    }
  } else {
    m = wmax(m);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      pr[i] = lane + 64 * i < E ? expf(s[i] - m) : 0.0f;
      z += pr[i];
    }
  }
  z = wsum(z);
  // gate part: the selected slots (k <= 32 scalar loads per wave)
  const int kk = min(k, 64);
  const int my_e = lane < kk ? idx[(long long)t * k + lane] : -1;
  const float my_g = lane < kk ? dw[(long long)t * k + lane] : 0.0f;
  const float my_w = lane < kk ? tw[(long long)t * k + lane] : 0.0f;
  float gdot = wsum(my_g * my_w);                        // <g, w> over the slots
  if (!sig && !renormalize && scoring == SOFTMAX_TOPK) {
    // w = p_sel: ds = p (g~ - <g~, p>) with g~ on the selected experts
    for (int j = 0; j < kk; ++j) {
      const int ej = __shfl(my_e, j);
      const float gj = __shfl(my_g, j);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i == ej) gsel[i] += gj;
    }
    float gp = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) gp += gsel[i] * pr[i] / z;
    gp = wsum(gp);
#pragma unroll
    for (int i = 0; i < EPL; ++i) gsel[i] = (pr[i] / z) * (gsel[i] - gp);
  } else {
    float sa = 0.0f;
    if (sig && renormalize) {
      const float aj = lane < kk ? 1.0f / (1.0f + expf(-logits[(long long)t * E + my_e])) : 0.0f;
      sa = wsum(aj);
    }
    for (int j = 0; j < kk; ++j) {
      const int ej = __shfl(my_e, j);
      const float gj = __shfl(my_g, j);
      const float wj = __shfl(my_w, j);
      float v;
      if (!sig) v = wj * (gj - gdot);                   // renormalised softmax / k-way softmax
      else {
        const float aj = 1.0f / (1.0f + expf(-logits[(long long)t * E + ej]));
        v = renormalize ? aj * (1.0f - aj) * (gj - gdot) / sa : aj * (1.0f - aj) * gj;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i == ej) gsel[i] += v;
    }
  }
  // balance-loss part
  float cp = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) cp += c[i] * pr[i] / z;
  cp = wsum(cp);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) continue;
    float aux;
    if (sig) aux = (c[i] - cp) / z * pr[i] * (1.0f - pr[i]);
    else aux = (pr[i] / z) * (c[i] - cp);
    dlogits[(long long)t * E + e] = gsel[i] + aux;
  }
}

// ---------------------------------------------------------------------------
// C[m, n] = sum_k A(m, k) B(k, n), A(m, k) = A[m am + k ak] (float32),
// B(k, n) = B[k bk + n bn] (BT), float32 out [M][N] (+ C when accumulate).
// 64x64 tile, 4x4 per thread, 16-deep slices through LDS.
// With gridDim.z = S > 1 the contraction is split into S consecutive ranges
// of kc and part z writes C + z M N (added in order by sum_parts_kernel).
template <typename BT>
__global__ __launch_bounds__(256) void gemm_f32_strided_kernel(const float* __restrict__ A, long long am,
                                                               long long ak, const BT* __restrict__ B, long long bk,
                                                               long long bn, int M, int N, int K, int kc,
                                                               float* __restrict__ C) {
  __shared__ float As[16][65], Bs[16][65];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
  const int k_lo = blockIdx.z * kc, k_hi = min(K, k_lo + kc);
  C += (long long)blockIdx.z * M * N;
  float acc[4][4] = {};
  for (int k0 = k_lo; k0 < k_hi; k0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      // consecutive threads walk the stride-1 index of each operand
      int kk, mm;
      if (am == 1) { mm = i & 63; kk = i >> 6; } else { kk = i & 15; mm = i >> 4; }
      const int m = m0 + mm, kq = k0 + kk;
      As[kk][mm] = (m < M && kq < k_hi) ? A[m * am + kq * ak] : 0.0f;
      int kb, nn;
      if (bn == 1) { nn = i & 63; kb = i >> 6; } else { kb = i & 15; nn = i >> 4; }
      const int n = n0 + nn, kr = k0 + kb;
      float bvv = 0.0f;
      if (n < N && kr < k_hi) {
        if constexpr (sizeof(BT) == 2) bvv = bf(B[kr * bk + n * bn]);
        else bvv = B[kr * bk + n * bn];
      }
      Bs[kb][nn] = bvv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[kk][tm + i], Bs[kk][tn + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (m0 + tm + i < M && n0 + tn + j < N) C[(long long)(m0 + tm + i) * N + n0 + tn + j] = acc[i][j];
}

// C[i] = sum over parts z (in order) of P[z n + i]
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ P, int S, long long n,
                                                        float* __restrict__ C) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    float v = 0.0f;
    for (int z = 0; z < S; ++z) v += P[z * n + i];
    C[i] = v;
  }
}

// y[i] = bf16(y[i] + add[i])
__global__ __launch_bounds__(256) void add_f32_to_bf16_kernel(bf16_t* __restrict__ y, const float* __restrict__ add,
                                                              long long n) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    y[i] = f32_to_bf16_rn(bf(y[i]) + add[i]);
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ p, float v, long long n) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = v;
}

inline unsigned grid_for(long long n) { return (unsigned)std::min<long long>((n + 255) / 256, 8192); }

}  // namespace

hipError_t launch_transpose_bf16(const bf16_t* in, bf16_t* out, int G, int R, int C, const int32_t* offsets,
                                 hipStream_t s) {
  if (G <= 0 || R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(ceil_div(C, 64), ceil_div(R, 64), G), dim3(256), 0, s, in, out, R, C, offsets);
  return hipGetLastError();
}

hipError_t launch_bw_combine(const bf16_t* dy, const bf16_t* yp, const int32_t* row_of, const float* tw, int T, int k,
                             int D, float* dw, bf16_t* dyp, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(bw_combine_kernel, dim3(T), dim3(256), 0, s, dy, yp, row_of, tw, k, D, dw, dyp);
  return hipGetLastError();
}

// h [rows, F] from the stored pre-activations gu [rows, nF]: SwiGLU
// silu(g) * u, GELU gelu(g), in float32, rounded to bf16 (the functions of
// the forward's GEMM epilogues); rows = *rows_valid (or rows_max).
__global__ __launch_bounds__(256) void act_fwd_kernel(const bf16_t* __restrict__ gu, bf16_t* __restrict__ h,
                                                      const int32_t* __restrict__ rows_valid, int rows_max, int F,
                                                      int swiglu) {
  const int rows = rows_valid ? min(*rows_valid, rows_max) : rows_max;
  const int F8 = F / 8;
  const long long n = (long long)rows * F8;
  const int ldg = swiglu ? 2 * F : F;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const long long r = i / F8;
    const int f = (int)(i % F8) * 8;
    const uint4 gq = *reinterpret_cast<const uint4*>(gu + r * ldg + f);
    const uint4 uq = swiglu ? *reinterpret_cast<const uint4*>(gu + r * ldg + F + f) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t a = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float g = __uint_as_float(e ? (gw[q] & 0xffff0000u) : (gw[q] << 16));
        float v;
        if (swiglu) v = silu_f32(g) * __uint_as_float(e ? (uw[q] & 0xffff0000u) : (uw[q] << 16));
        else v = gelu_bf16out(g);
        a |= (uint32_t)f32_to_bf16_rn(v) << (16 * e);
      }
      o[q] = a;
    }
    *reinterpret_cast<uint4*>(h + r * F + f) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_act_fwd(const bf16_t* gu, bf16_t* h, const int32_t* rows_valid, int rows_max, int F, bool swiglu,
                          hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  if (F % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(act_fwd_kernel, dim3(grid_for((long long)rows_max * (F / 8))), dim3(256), 0, s, gu, h,
                     rows_valid, rows_max, F, swiglu ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_bw_act(const bf16_t* gu, const bf16_t* dh, bf16_t* dgu, const int32_t* rows_valid, int rows_max,
                         int F, bool swiglu, hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  if (F % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bw_act_kernel, dim3(grid_for((long long)rows_max * (F / 8))), dim3(256), 0, s, gu, dh, dgu,
                     rows_valid, rows_max, F, swiglu ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_wgrad(const bf16_t* A, int lda, const bf16_t* B, int ldb, const int32_t* b_rows,
                        const int32_t* offsets, int G, int rows_max, int M, int N, float* C, hipStream_t s) {
  if (G <= 0 || M <= 0 || N <= 0) return hipSuccess;
  if (lda % 4 != 0 || ldb % 4 != 0 || M % 4 != 0 || N % 4 != 0) return hipErrorInvalidValue;   // 8-byte column groups
  // 256x256 tiles (eight waves) for large outputs: each operand row slice is
  // re-read by half as many workgroups as with 128x128
  const Tuning t = tuning();
  const int forced = t.wgrad_tile != kUnset ? t.wgrad_tile : 0;   // 128 or 256 forces a tile (tuning aid)
  const int swz = t.wgrad_swz != kUnset ? t.wgrad_swz : 2;         // LDS chunk permutation 0 / 1 / 2 (tuning aid)
#define MOE_WG(BM_, BN_, WGM_, WGN_, SWZ_)                                                                   \
  hipLaunchKernelGGL((wgrad_kernel<BM_, BN_, WGM_, WGN_, SWZ_>), dim3(ceil_div(N, BN_), ceil_div(M, BM_), G), \
                     dim3(64 * WGM_ * WGN_), 0, s, A, lda, B, ldb, b_rows, offsets, rows_max, M, N, C)
  if (forced == 256 || (forced != 128 && M >= 256 && N >= 256)) {
    if (swz == 0) MOE_WG(256, 256, 2, 4, 0);
    else if (swz == 1) MOE_WG(256, 256, 2, 4, 1);
    else MOE_WG(256, 256, 2, 4, 2);
  } else {
    if (swz == 0) MOE_WG(128, 128, 2, 2, 0);
    else if (swz == 1) MOE_WG(128, 128, 2, 2, 1);
    else MOE_WG(128, 128, 2, 2, 2);
  }
#undef MOE_WG
  return hipGetLastError();
}

hipError_t launch_router_grad(const float* logits, const int32_t* idx, const float* tw, const float* dw,
                              const int32_t* counts, int T, int E, int k, int scoring, int renormalize, float alpha,
                              float* dlogits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (k > 64) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(T, 4));
  const int epl = ceil_div(E, 64);
#define MOE_RG(N) hipLaunchKernelGGL(router_grad_kernel<N>, grid, dim3(256), 0, s, logits, idx, tw, dw, counts, T, E, k, \
                                     scoring, renormalize, alpha, dlogits)
  if (epl <= 1) MOE_RG(1);
  else if (epl <= 2) MOE_RG(2);
  else if (epl <= 4) MOE_RG(4);
  else if (epl <= 8) MOE_RG(8);
  else if (epl <= 16) MOE_RG(16);
  else return hipErrorInvalidValue;
#undef MOE_RG
  return hipGetLastError();
}

int gemm_f32_split(int M, int N, int K) {
  const long long tiles = (long long)ceil_div(M, 64) * ceil_div(N, 64);
  int sp = 1;
  while (sp < kF32MaxSplit && tiles * sp * 2 <= 512 && K / (sp * 2) >= 256) sp *= 2;
  return sp;
}

hipError_t launch_gemm_f32_strided(const float* A, long long am, long long ak, const void* B, bool b_bf16,
                                   long long bk, long long bn, int M, int N, int K, float* C, float* partial,
                                   hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int sp = partial != nullptr ? gemm_f32_split(M, N, K) : 1;
  const int kc = sp > 1 ? ceil_div(ceil_div(K, sp), 16) * 16 : K;
  const dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(M, 64), (unsigned)sp);
  float* out = sp > 1 ? partial : C;
  if (b_bf16)
    hipLaunchKernelGGL(gemm_f32_strided_kernel<bf16_t>, grid, dim3(256), 0, s, A, am, ak,
                       static_cast<const bf16_t*>(B), bk, bn, M, N, K, kc, out);
  else
    hipLaunchKernelGGL(gemm_f32_strided_kernel<float>, grid, dim3(256), 0, s, A, am, ak,
                       static_cast<const float*>(B), bk, bn, M, N, K, kc, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp == 1) return e;
  const long long n = (long long)M * N;
  hipLaunchKernelGGL(sum_parts_kernel, dim3(grid_for(n)), dim3(256), 0, s, partial, sp, n, C);
  return hipGetLastError();
}

// Chunk bounds of a split contraction (offsets[g] = min(g * chunk, T)) and
// the plane row map r -> r mod E of the router's input gradient.
__global__ __launch_bounds__(256) void router_mfma_aux_kernel(int32_t* __restrict__ offsets, int G, int chunk, int T,
                                                              int32_t* __restrict__ rmap, int E3, int E) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i <= G + E3; i += gridDim.x * 256) {
    if (i <= G) offsets[i] = min(i * chunk, T);
    else rmap[i - G - 1] = (i - G - 1) % E;
  }
}

hipError_t launch_router_grad_mfma(const float* dlog, const bf16_t* x, const bf16_t* w_router, int T, int E, int D,
                                   float* dw_router, float* dx_router, bf16_t* planes, bf16_t* planes_t,
                                   int32_t* aux, float* partial, hipStream_t s) {
  if (T <= 0 || E <= 0 || D <= 0) return hipSuccess;
  const int E3 = 3 * E;
  if (E3 % 4 != 0 || D % 4 != 0 || (dx_router != nullptr && (T % 4 != 0 || w_router == nullptr)))
    return hipErrorInvalidValue;
  hipError_t e = launch_split_bf16x3(dlog, T, E, planes, s);      // [T][3][E]: plane p of logit e at column p E + e
  if (e != hipSuccess) return e;
  // token chunks, so that the output tiles times the chunks fill the chip
  const int bt = (E3 >= 256 && D >= 256) ? 256 : 128;
  const int tiles = ceil_div(E3, bt) * ceil_div(D, bt);
  int G = std::min(kRouterMfmaSplit, std::max(1, ceil_div(2 * num_cus(), tiles)));
  G = std::min(G, std::max(1, T / 256));
  const int chunk = ceil_div(ceil_div(T, G), 32) * 32;
  G = ceil_div(T, chunk);
  int32_t* offsets = aux;
  int32_t* rmap = aux + kRouterMfmaSplit + 1;
  hipLaunchKernelGGL(router_mfma_aux_kernel, dim3(ceil_div(G + 1 + E3, 256)), dim3(256), 0, s, offsets, G, chunk, T,
                     rmap, E3, E);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dW_router: parts [G][3][E][D] over the token chunks and planes, added in that order
  e = launch_wgrad(planes, E3, x, D, nullptr, offsets, G, T, E3, D, partial, s);
  if (e != hipSuccess) return e;
  const long long n = (long long)E * D;
  hipLaunchKernelGGL(sum_parts_kernel, dim3(grid_for(n)), dim3(256), 0, s, partial, 3 * G, n, dw_router);
  e = hipGetLastError();
  if (e != hipSuccess || dx_router == nullptr) return e;
  // dx_router [T][D] = sum over the 3E plane rows r of planes_t[r][t] w_router[r mod E][d]
  e = launch_transpose_bf16(planes, planes_t, 1, T, E3, nullptr, s);
  if (e != hipSuccess) return e;
  return launch_wgrad(planes_t, T, w_router, D, rmap, nullptr, 1, E3, T, D, dx_router, s);
}

hipError_t launch_add_f32_to_bf16(bf16_t* y, const float* add, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(add_f32_to_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, s, y, add, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace moe
