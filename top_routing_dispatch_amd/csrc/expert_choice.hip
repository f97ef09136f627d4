// Expert-choice routing ("Top-k 路由" page, Token-Choice vs Expert-Choice
// table: each expert picks its top-C tokens; "MoE 路由算法" page, 数学机理
// (2) and 深度剖析 ②): the routing probabilities p = softmax(W_g x) over the
// experts, then every expert takes the C tokens with the largest p[:, e]
// (equal values: lower token index first) with gate p[t, e].  Rows are laid
// out expert after expert with the tokens ascending inside an expert, so the
// grouped expert FFN runs unchanged (offsets e C, the token of each row as its
// gather index); a token no expert chose gets nothing from the routed experts
// (the residual path carries it).
//   ec_probs    one wave per token: softmax over the experts in float32
//               (fixed-order butterflies), staged in LDS and written
//               transposed, p^T [E, T], so that an expert's column is a row;
//   ec_select   one workgroup per expert: a bitonic sort in LDS of the keys
//               (p bits << 32 | ~t), descending, takes the first C; a bit
//               mask of the chosen tokens and its word prefix counts give each
//               chosen token its row, e C + (chosen tokens below it);
//   ec_combine  one workgroup per token: the experts that chose it (ascending
//               expert id, from the masks), then y[t] = sum of p[t, e] *
//               y_perm[row] in that order (+ y_shared[t]).
// All integer decisions are exact and every sum has a fixed order.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_max_ec(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum_ec(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

constexpr int kEcTokensPerBlock = 64;

template <int EPL>
__global__ __launch_bounds__(256) void ec_probs_kernel(const float* __restrict__ logits, int T, int E, int C,
                                                       float* __restrict__ pT, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ unselected) {
  __shared__ float sp[64 * EPL][kEcTokensPerBlock + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kEcTokensPerBlock;
  for (int i = 0; i < kEcTokensPerBlock / 4; ++i) {
    const int tl = wave * (kEcTokensPerBlock / 4) + i;
    const int t = t0 + tl;
    if (t >= T) break;                                  // uniform per wave
    float s[EPL], m = -INFINITY;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + 64 * q;
      s[q] = e < E ? logits[(long long)t * E + e] : -INFINITY;
      m = fmaxf(m, s[q]);
    }
    m = wave_max_ec(m);
    float ex[EPL], z = 0.0f;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      ex[q] = lane + 64 * q < E ? expf(s[q] - m) : 0.0f;
      z += ex[q];
    }
    z = wave_sum_ec(z);
#pragma unroll
    for (int q = 0; q < EPL; ++q) sp[lane + 64 * q][tl] = ex[q] / z;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E * kEcTokensPerBlock; i += blockDim.x) {
    const int e = i / kEcTokensPerBlock, j = i % kEcTokensPerBlock;
    if (t0 + j < T) pT[(long long)e * T + t0 + j] = sp[e][j];
  }
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = e * C;
    if (threadIdx.x == 0 && unselected != nullptr) *unselected = 0;
  }
}

// N: keys in LDS (a power of two >= T).  Keys of padding entries are 0, below
// every real key (the token part ~t is nonzero for t < 2^32 - 1).
__global__ __launch_bounds__(1024) void ec_select_kernel(const float* __restrict__ pT, int T, int C, int N,
                                                         int32_t* __restrict__ token_of_row,
                                                         float* __restrict__ row_w, uint32_t* __restrict__ selbits,
                                                         int32_t* __restrict__ selpre) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(smem);
  const int W = (T + 31) / 32;
  uint32_t* bits = reinterpret_cast<uint32_t*>(keys + N);
  int32_t* pre = reinterpret_cast<int32_t*>(bits + W);
  const int e = blockIdx.x;
  const float* col = pT + (long long)e * T;
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    unsigned long long k = 0ull;
    if (i < T) k = ((unsigned long long)__float_as_uint(col[i]) << 32) | (0xffffffffull - (unsigned)i);
    keys[i] = k;
  }
  for (int w = threadIdx.x; w < W; w += blockDim.x) bits[w] = 0u;
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = keys[i], b = keys[ixj];
          const bool up = (i & k) == 0;
          if (up ? (a < b) : (a > b)) { keys[i] = b; keys[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
  for (int j = threadIdx.x; j < C; j += blockDim.x) {
    const unsigned t = 0xffffffffu - (unsigned)(keys[j] & 0xffffffffull);
    atomicOr(&bits[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < W; ++w) { pre[w] = run; run += __popc(bits[w]); }
  }
  __syncthreads();
  for (int w = threadIdx.x; w < W; w += blockDim.x) {
    selbits[(long long)e * W + w] = bits[w];
    selpre[(long long)e * W + w] = pre[w];
  }
  for (int j = threadIdx.x; j < C; j += blockDim.x) {
    const unsigned long long k = keys[j];
    const unsigned t = 0xffffffffu - (unsigned)(k & 0xffffffffull);
    const int rank = pre[t >> 5] + __popc(bits[t >> 5] & ((1u << (t & 31)) - 1u));
    const long long row = (long long)e * C + rank;
    token_of_row[row] = (int)t;
    row_w[row] = __uint_as_float((unsigned)(k >> 32));
  }
}

template <typename ET>
struct EcChunk;
template <> struct EcChunk<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ float elem(const uint4& q, int i) {
    return __uint_as_float(i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w);
  }
  static __device__ __forceinline__ void store(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct EcChunk<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ float elem(const uint4& q, int i) {
    const uint32_t w = (i >> 1) == 0 ? q.x : (i >> 1) == 1 ? q.y : (i >> 1) == 2 ? q.z : q.w;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float v[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_rn(v[2 * i]) | ((uint32_t)f32_to_bf16_rn(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <typename ET>
__global__ __launch_bounds__(256) void ec_combine_kernel(const ET* __restrict__ yp, const float* __restrict__ pT,
                                                         const uint32_t* __restrict__ selbits,
                                                         const int32_t* __restrict__ selpre, const ET* ys, ET* y,
                                                         int T, int E, int C, int D,
                                                         int32_t* __restrict__ unselected) {
  constexpr int N = EcChunk<ET>::N;
  __shared__ int srow[256];
  __shared__ float sw[256];
  __shared__ int wcount[4];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int W = (T + 31) / 32;
  const int e = threadIdx.x;
  bool chosen = false;
  int row = 0;
  float w = 0.0f;
  if (e < E) {
    const uint32_t word = selbits[(long long)e * W + (t >> 5)];
    chosen = (word >> (t & 31)) & 1u;
    if (chosen) {
      row = e * C + selpre[(long long)e * W + (t >> 5)] + __popc(word & ((1u << (t & 31)) - 1u));
      w = pT[(long long)e * T + t];
    }
  }
  const unsigned long long m = __ballot(chosen);
  if (lane == 0) wcount[wave] = __popcll(m);
  __syncthreads();
  int base = 0;
  for (int v = 0; v < wave; ++v) base += wcount[v];
  const int n = wcount[0] + wcount[1] + wcount[2] + wcount[3];
  if (chosen) {
    const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
    srow[pos] = row;
    sw[pos] = w;
  }
  if (threadIdx.x == 0 && n == 0 && unselected != nullptr) atomicAdd(unselected, 1);
  __syncthreads();
  const int chunks = D / N;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    float acc[N];
#pragma unroll
    for (int q = 0; q < N; ++q) acc[q] = 0.0f;
    uint4 vs = make_uint4(0u, 0u, 0u, 0u);
    if (ys != nullptr) vs = *reinterpret_cast<const uint4*>(ys + (long long)t * D + c * N);
    for (int i0 = 0; i0 < n; i0 += 4) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = srow[min(i0 + u, n - 1)];
        v[u] = *reinterpret_cast<const uint4*>(yp + (long long)r * D + c * N);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i0 + u < n) {
          const float ww = sw[i0 + u];
#pragma unroll
          for (int q = 0; q < N; ++q) acc[q] = fmaf(ww, EcChunk<ET>::elem(v[u], q), acc[q]);
        }
      }
    }
    if (ys != nullptr) {
#pragma unroll
      for (int q = 0; q < N; ++q) acc[q] += EcChunk<ET>::elem(vs, q);
    }
    EcChunk<ET>::store(y + (long long)t * D + c * N, acc);
  }
}

}  // namespace

int ec_sort_keys(int T) {
  int n = 1;
  while (n < T) n <<= 1;
  return n;
}

size_t ec_select_lds(int T) {
  const int W = (T + 31) / 32;
  return (size_t)ec_sort_keys(T) * 8 + (size_t)W * 8;
}

hipError_t launch_ec_route(const float* logits, int T, int E, int C, float* pT, int32_t* offsets,
                           int32_t* token_of_row, float* row_w, uint32_t* selbits, int32_t* selpre,
                           int32_t* unselected, hipStream_t s) {
  if (T <= 0 || E <= 0 || E > kEcMaxExperts || T > kEcMaxTokens || C < 0 || C > T) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(T, kEcTokensPerBlock));
  if (E <= 64) hipLaunchKernelGGL(ec_probs_kernel<1>, grid, dim3(256), 0, s, logits, T, E, C, pT, offsets, unselected);
  else if (E <= 128) hipLaunchKernelGGL(ec_probs_kernel<2>, grid, dim3(256), 0, s, logits, T, E, C, pT, offsets, unselected);
  else hipLaunchKernelGGL(ec_probs_kernel<4>, grid, dim3(256), 0, s, logits, T, E, C, pT, offsets, unselected);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = ec_select_lds(T);
  static std::atomic<bool> allowed[64];   // per device: attribute set (host threads may race)
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !allowed[dev].load(std::memory_order_relaxed)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ec_select_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)ec_select_lds(kEcMaxTokens));
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) allowed[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL(ec_select_kernel, dim3((unsigned)E), dim3(1024), lds, s, pT, T, C, ec_sort_keys(T),
                     token_of_row, row_w, selbits, selpre);
  return hipGetLastError();
}

hipError_t launch_ec_combine(const void* y_perm, const float* pT, const uint32_t* selbits, const int32_t* selpre,
                             const void* y_shared, void* y, int T, int E, int C, int D, int act_dtype,
                             int32_t* unselected, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (E > kEcMaxExperts) return hipErrorInvalidValue;
  if (act_dtype == BF16)
    hipLaunchKernelGGL(ec_combine_kernel<bf16_t>, dim3((unsigned)T), dim3(256), 0, s,
                       static_cast<const bf16_t*>(y_perm), pT, selbits, selpre, static_cast<const bf16_t*>(y_shared),
                       static_cast<bf16_t*>(y), T, E, C, D, unselected);
  else
    hipLaunchKernelGGL(ec_combine_kernel<float>, dim3((unsigned)T), dim3(256), 0, s,
                       static_cast<const float*>(y_perm), pT, selbits, selpre, static_cast<const float*>(y_shared),
                       static_cast<float*>(y), T, E, C, D, unselected);
  return hipGetLastError();
}

}  // namespace moe
