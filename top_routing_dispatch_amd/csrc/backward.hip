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

#include <algorithm>

namespace moe {
namespace {

__device__ __forceinline__ float bf(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ in, bf16_t* __restrict__ out,
                                                             int R, int C) {
  __shared__ bf16_t tile[64][66];
  const long long g = blockIdx.z;
  const bf16_t* src = in + g * (long long)R * C;
  bf16_t* dst = out + g * (long long)R * C;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4)
    if (r0 + i < R && c0 + tx < C) tile[i][tx] = src[(long long)(r0 + i) * C + c0 + tx];
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
__global__ __launch_bounds__(256) void bw_act_kernel(const bf16_t* __restrict__ gu, const bf16_t* __restrict__ dh,
                                                     bf16_t* __restrict__ dgu, const int32_t* __restrict__ rows_valid,
                                                     int rows_max, int F, int swiglu) {
  const int rows = rows_valid ? min(*rows_valid, rows_max) : rows_max;
  const long long n = (long long)rows * F;
  const int ldg = swiglu ? 2 * F : F;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const long long r = i / F;
    const int f = (int)(i % F);
    const float g = bf(gu[r * ldg + f]);
    const float d = bf(dh[r * F + f]);
    if (swiglu) {
      const float u = bf(gu[r * ldg + F + f]);
      const float sg = 1.0f / (1.0f + expf(-g));
      dgu[r * ldg + f] = f32_to_bf16_rn(d * u * sg * (1.0f + g * (1.0f - sg)));
      dgu[r * ldg + F + f] = f32_to_bf16_rn(d * g * sg);
    } else {
      const float cdf = 0.5f * (1.0f + erff(g * 0.70710678118654752f));
      const float pdf = 0.39894228040143268f * expf(-0.5f * g * g);
      dgu[r * ldg + f] = f32_to_bf16_rn(d * (cdf + g * pdf));
    }
  }
}

// Eight bf16 values from p, the first `valid` of them read (valid may be <= 0).
__device__ __forceinline__ uint4 load8_masked(const bf16_t* p, int valid) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = 2 * q < valid ? p[2 * q] : 0u;
    const uint32_t hi = 2 * q + 1 < valid ? p[2 * q + 1] : 0u;
    w[q] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// C_g[m, n] = sum over rows r of group g of A[r, m] * B[b_row(r), n]
// (float32 out, [G][M][N]); A [rows][lda] and B [*][ldb] bf16.  b_rows (or
// NULL) maps a row to the B row it reads.  offsets [G+1] (NULL: one group of
// rows_max rows).  64x64 tile per workgroup, 32 rows per slice; each slice is
// stored transposed in LDS ([m][r], [n][r]) so that the MFMA operands (8
// consecutive rows of one column) are 16-byte reads.  Four waves, 32x32 each
// (2x2 blocks of v_mfma_f32_16x16x32_bf16).  Empty groups write zeros.
__global__ __launch_bounds__(256) void wgrad_kernel(const bf16_t* __restrict__ A, int lda,
                                                    const bf16_t* __restrict__ B, int ldb,
                                                    const int32_t* __restrict__ b_rows,
                                                    const int32_t* __restrict__ offsets, int rows_max, int M, int N,
                                                    float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) bf16_t As[64][40];   // [m][r], 32 rows + pad
  __shared__ __attribute__((aligned(16))) bf16_t Bs[64][40];
  const int g = blockIdx.z;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int r_lo = offsets ? offsets[g] : 0;
  const int r_hi = offsets ? offsets[g + 1] : rows_max;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  floatx4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][j][q] = 0.0f;
  // loader: thread -> (row lr, 8 columns at lc)
  const int lr = threadIdx.x >> 3, lc = (threadIdx.x & 7) * 8;
  for (int r0 = r_lo; r0 < r_hi; r0 += 32) {
    const int r = r0 + lr;
    uint4 av = make_uint4(0u, 0u, 0u, 0u), bv = make_uint4(0u, 0u, 0u, 0u);
    if (r < r_hi) {
      if (m0 + lc + 8 <= M) av = *reinterpret_cast<const uint4*>(A + (long long)r * lda + m0 + lc);
      else av = load8_masked(A + (long long)r * lda + m0 + lc, M - (m0 + lc));
      const long long br = b_rows ? (long long)b_rows[r] : (long long)r;
      if (n0 + lc + 8 <= N) bv = *reinterpret_cast<const uint4*>(B + br * ldb + n0 + lc);
      else bv = load8_masked(B + br * ldb + n0 + lc, N - (n0 + lc));
    }
    __syncthreads();                                   // the previous slice's reads are done
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      As[lc + 2 * q][lr] = (bf16_t)(aw[q] & 0xffffu);
      As[lc + 2 * q + 1][lr] = (bf16_t)(aw[q] >> 16);
      Bs[lc + 2 * q][lr] = (bf16_t)(bw4[q] & 0xffffu);
      Bs[lc + 2 * q + 1][lr] = (bf16_t)(bw4[q] >> 16);
    }
    __syncthreads();
    // lane: column (lane & 15) of a 16-block, rows (lane >> 4) * 8 .. + 7 of the slice
    const int fc = lane & 15, fk = (lane >> 4) * 8;
    bf16x8_t fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(&As[wm * 32 + i * 16 + fc][fk]);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[wn * 32 + j * 16 + fc][fk]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }
  // C block (i, j): lane holds column n = lane & 15, rows m = 4 (lane >> 4) + q
  float* Cg = C + (long long)g * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + q;
        const int n = n0 + wn * 32 + j * 16 + (lane & 15);
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
template <typename BT>
__global__ __launch_bounds__(256) void gemm_f32_strided_kernel(const float* __restrict__ A, long long am,
                                                               long long ak, const BT* __restrict__ B, long long bk,
                                                               long long bn, int M, int N, int K,
                                                               float* __restrict__ C) {
  __shared__ float As[16][65], Bs[16][65];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tm = (threadIdx.x >> 4) * 4, tn = (threadIdx.x & 15) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 16 * 64; i += 256) {
      // consecutive threads walk the stride-1 index of each operand
      int kk, mm;
      if (am == 1) { mm = i & 63; kk = i >> 6; } else { kk = i & 15; mm = i >> 4; }
      const int m = m0 + mm, kq = k0 + kk;
      As[kk][mm] = (m < M && kq < K) ? A[m * am + kq * ak] : 0.0f;
      int kb, nn;
      if (bn == 1) { nn = i & 63; kb = i >> 6; } else { kb = i & 15; nn = i >> 4; }
      const int n = n0 + nn, kr = k0 + kb;
      float bvv = 0.0f;
      if (n < N && kr < K) {
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

hipError_t launch_transpose_bf16(const bf16_t* in, bf16_t* out, int G, int R, int C, hipStream_t s) {
  if (G <= 0 || R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(ceil_div(C, 64), ceil_div(R, 64), G), dim3(256), 0, s, in, out, R, C);
  return hipGetLastError();
}

hipError_t launch_bw_combine(const bf16_t* dy, const bf16_t* yp, const int32_t* row_of, const float* tw, int T, int k,
                             int D, float* dw, bf16_t* dyp, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(bw_combine_kernel, dim3(T), dim3(256), 0, s, dy, yp, row_of, tw, k, D, dw, dyp);
  return hipGetLastError();
}

hipError_t launch_bw_act(const bf16_t* gu, const bf16_t* dh, bf16_t* dgu, const int32_t* rows_valid, int rows_max,
                         int F, bool swiglu, hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  hipLaunchKernelGGL(bw_act_kernel, dim3(grid_for((long long)rows_max * F)), dim3(256), 0, s, gu, dh, dgu, rows_valid,
                     rows_max, F, swiglu ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_wgrad(const bf16_t* A, int lda, const bf16_t* B, int ldb, const int32_t* b_rows,
                        const int32_t* offsets, int G, int rows_max, int M, int N, float* C, hipStream_t s) {
  if (G <= 0 || M <= 0 || N <= 0) return hipSuccess;
  if (lda % 8 != 0 || ldb % 8 != 0) return hipErrorInvalidValue;   // 16-byte row chunks
  hipLaunchKernelGGL(wgrad_kernel, dim3(ceil_div(N, 64), ceil_div(M, 64), G), dim3(256), 0, s, A, lda, B, ldb, b_rows,
                     offsets, rows_max, M, N, C);
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

hipError_t launch_gemm_f32_strided(const float* A, long long am, long long ak, const void* B, bool b_bf16,
                                   long long bk, long long bn, int M, int N, int K, float* C, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ceil_div(M, 64));
  if (b_bf16)
    hipLaunchKernelGGL(gemm_f32_strided_kernel<bf16_t>, grid, dim3(256), 0, s, A, am, ak,
                       static_cast<const bf16_t*>(B), bk, bn, M, N, K, C);
  else
    hipLaunchKernelGGL(gemm_f32_strided_kernel<float>, grid, dim3(256), 0, s, A, am, ak,
                       static_cast<const float*>(B), bk, bn, M, N, K, C);
  return hipGetLastError();
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
