// The whole layer forward in one launch, for batches small enough that
// launch latency, not work, sets the time (the Tiny-MoE walk-through's shape:
// 64 tokens, D = 32, four experts of F = 48; "从 Dense FFN 到 MoE" §3-§8).
//
// One workgroup per token.  Routing is cheap at these sizes, so every
// workgroup routes the whole batch itself (no grid-wide synchronisation is
// needed) and then runs only its own token through its experts:
//   0. x and the router weight are staged in LDS as float32;
//   1. router logits s = W_g x of every token in float64 (products of the
//      stored values are exact, the sums are float64), so the selection is
//      taken on float64 scores throughout;
//   2. a group of G = ceil(E / 8) lanes per token, each holding up to eight
//      experts' scores in registers: scoring, top-k (ties to the lower
//      expert) and the soft probabilities of the balance loss ("Top-k 路由"
//      page, Step 2 and its note; "别只比较 Top-k" page, Select and Merge);
//      the workgroup's own token also gets its gate weights;
//   3. the rank of each of the token's assignments among its expert's
//      assignments in (token, slot) order, i.e. the number of earlier tokens
//      that chose the same expert (one ballot per slot); ranks at or past the
//      capacity are dropped ("Top-k 路由" page, 容量因子).  Beside it the
//      token's expert activations of every slot and of the shared experts;
//   4. the token's output: the shared experts' sum plus the weighted outputs
//      of its kept slots ("从 Dense FFN 到 MoE" §6);
//   5. workgroup 0 also: the load statistics f, P, alpha E sum f P, max /
//      mean and drops ("Top-k 路由" page, 負載均衡; "从 Dense FFN 到 MoE" §8),
//      the token sums of P taken in a fixed order, on the threads the
//      token's own steps leave idle.
// Activations and outputs are computed in float32 from the stored values;
// the activation values stay in float32 (LDS) between the two projections.
#include "common.h"

namespace moe {
namespace {

constexpr int kFusedThreads = 256;               // one token per thread in steps 2 and 3
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedMaxK = 8;
constexpr int kFusedMaxE = 64;                   // eight lanes of eight experts; one mask word
constexpr int kFusedPerLane = 8;                 // experts a lane holds in step 2
constexpr int kFusedChunks = 16;                 // token chunks of the P sums
constexpr int kFusedMaxLds = 63 * 1024;          // dynamic LDS, below the 64 KB default

// LDS carve-up (bytes, 16-byte aligned pieces).  Rows of x and W_g are
// padded by four floats so that neighbouring rows start in other banks.
struct FusedLds {
  int x, wr, logits, idx, mask, val, rank, h, part, cnt, psum, total;
};

__host__ __device__ inline int align16(int b) { return (b + 15) & ~15; }
__host__ __device__ inline int fused_row(int D) { return D + 4; }

__host__ __device__ inline FusedLds fused_lds(int T, int D, int E, int k, int F, int SF) {
  FusedLds L{};
  int o = 0;
  L.x = o; o += align16(T * fused_row(D) * 4);        // [T][D+4] float32
  L.wr = o; o += align16(E * fused_row(D) * 4);       // [E][D+4] float32
  L.logits = o; o += align16(T * E * 8);              // [T][E] float64: logits, then probabilities
  L.idx = o; o += align16(T * k * 4);                 // [T][k] selections of every token
  L.mask = o; o += align16(T * 8);                    // [T] bit e: token chose expert e
  L.val = o; o += align16(kFusedMaxK * 8);            // own token: selected p / a / s, then weights
  L.rank = o; o += align16(kFusedWaves * kFusedMaxK * 4);   // per-wave rank counts
  L.h = o; o += align16((k * F + SF) * 4);            // own token's activations: routed, then shared
  L.part = o; o += align16((k + 1) * D * 4);          // per-slot (and shared) output rows
  L.cnt = o; o += align16(E * 4);                     // workgroup 0: counts
  L.psum = o; o += align16((kFusedChunks + 1) * E * 8);   // workgroup 0: chunk sums of P, then f P
  L.total = o;
  return L;
}

// Four consecutive elements as float32 (16-byte float or 8-byte bfloat16 loads).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xffff0000u));
}

// Copies rows [n][D] of global memory into LDS rows of D+4 floats.  Every
// thread's loads of a round of four are issued before its stores.
template <typename T>
__device__ __forceinline__ void stage_rows(const T* __restrict__ g, float* __restrict__ s, int n, int D) {
  const int q = D / 4, total = n * q;
  for (int i0 = threadIdx.x; i0 < total; i0 += 4 * kFusedThreads) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kFusedThreads;
      if (i < total) v[u] = load4(g + (long long)i * 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kFusedThreads;
      if (i < total) *reinterpret_cast<float4*>(s + (i / q) * fused_row(D) + (i % q) * 4) = v[u];
    }
  }
}

// Sum over d < n of x[d] w[d] in float32; x in LDS (float32), w in global memory.
template <typename TW>
__device__ __forceinline__ float dot_f32(const float* __restrict__ x, const TW* __restrict__ w, int n) {
  float s = 0.0f;
#pragma unroll 8
  for (int d = 0; d < n; d += 4) {
    const float4 u = *reinterpret_cast<const float4*>(x + d), v = load4(w + d);
    s = fmaf(u.x, v.x, s);
    s = fmaf(u.y, v.y, s);
    s = fmaf(u.z, v.z, s);
    s = fmaf(u.w, v.w, s);
  }
  return s;
}

// Gate and up rows of one SwiGLU feature against the same x.
template <typename TW>
__device__ __forceinline__ float2 dot2_f32(const float* __restrict__ x, const TW* __restrict__ g,
                                           const TW* __restrict__ u, int n) {
  float sg = 0.0f, su = 0.0f;
#pragma unroll 8
  for (int d = 0; d < n; d += 4) {
    const float4 xv = *reinterpret_cast<const float4*>(x + d), a = load4(g + d), b = load4(u + d);
    sg = fmaf(xv.x, a.x, sg); su = fmaf(xv.x, b.x, su);
    sg = fmaf(xv.y, a.y, sg); su = fmaf(xv.y, b.y, su);
    sg = fmaf(xv.z, a.z, sg); su = fmaf(xv.z, b.z, su);
    sg = fmaf(xv.w, a.w, sg); su = fmaf(xv.w, b.w, su);
  }
  return make_float2(sg, su);
}

// Reductions over the G lanes of a token group (G a power of two <= 8,
// groups aligned in the wave); every lane of the group gets the result.
__device__ __forceinline__ double group_sum(double v, int G) {
  for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double group_max(double v, int G) {
  for (int o = 1; o < G; o <<= 1) {
    const double u = __shfl_xor(v, o);
    v = u > v ? u : v;
  }
  return v;
}

template <typename TA, typename TR>
__global__ __launch_bounds__(kFusedThreads) void fused_layer_kernel(const FusedArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int T = a.T, D = a.D, E = a.E, k = a.k, F = a.F, SF = a.SF;
  const FusedLds L = fused_lds(T, D, E, k, F, SF);
  const int R = fused_row(D);
  float* sxa = reinterpret_cast<float*>(smem + L.x);
  float* swr = reinterpret_cast<float*>(smem + L.wr);
  double* sp = reinterpret_cast<double*>(smem + L.logits);
  int* sidx = reinterpret_cast<int*>(smem + L.idx);
  unsigned long long* smask = reinterpret_cast<unsigned long long*>(smem + L.mask);
  double* sval = reinterpret_cast<double*>(smem + L.val);
  int* srank = reinterpret_cast<int*>(smem + L.rank);
  float* sh = reinterpret_cast<float*>(smem + L.h);
  float* spart = reinterpret_cast<float*>(smem + L.part);
  int* scnt = reinterpret_cast<int*>(smem + L.cnt);
  double* spsum = reinterpret_cast<double*>(smem + L.psum);
  double* sfp = spsum + kFusedChunks * E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x;   // this workgroup's token
  const bool stats_here = blockIdx.x == 0;

  // 0. x and W_g into LDS as float32
  stage_rows(static_cast<const TA*>(a.x), sxa, T, D);
  stage_rows(static_cast<const TR*>(a.w_router), swr, E, D);
  if (stats_here)
    for (int e = tid; e < E; e += kFusedThreads) scnt[e] = 0;
  __syncthreads();

  // 1. logits of every token, float64 sums of exact products
  for (int p = tid; p < T * E; p += kFusedThreads) {
    const float* xr = sxa + (p / E) * R;
    const float* gr = swr + (p % E) * R;
    double s = 0.0;
#pragma unroll 4
    for (int d = 0; d < D; d += 4) {
      const float4 u = *reinterpret_cast<const float4*>(xr + d), v = *reinterpret_cast<const float4*>(gr + d);
      s = fma((double)u.x, (double)v.x, s);
      s = fma((double)u.y, (double)v.y, s);
      s = fma((double)u.z, (double)v.z, s);
      s = fma((double)u.w, (double)v.w, s);
    }
    sp[p] = s;
  }
  __syncthreads();

  // 2. token groups of G lanes; lane `sub` holds experts sub, sub + G, ...
  const int G = E <= 8 ? 1 : E <= 16 ? 2 : E <= 32 ? 4 : 8;
  const int sub = tid & (G - 1);
  for (int t = tid / G; t < T; t += kFusedThreads / G) {
    double* st = sp + t * E;
    // v: the key top-k ranks on: p (softmax first), s (top-k first) or
    // a + b (sigmoid); the row of sp still holds the logits s
    double v[kFusedPerLane];
    double m = -HUGE_VAL, z = 0.0;
#pragma unroll
    for (int i = 0; i < kFusedPerLane; ++i) {
      const int e = sub + i * G;
      v[i] = e < E ? st[e] : 0.0;
      if (e < E) m = v[i] > m ? v[i] : m;
    }
    m = group_max(m, G);
    if (a.scoring == SOFTMAX_TOPK) {
#pragma unroll
      for (int i = 0; i < kFusedPerLane; ++i)
        if (sub + i * G < E) { v[i] = exp(v[i] - m); z += v[i]; }
      z = group_sum(z, G);
#pragma unroll
      for (int i = 0; i < kFusedPerLane; ++i)
        if (sub + i * G < E) v[i] /= z;
    } else if (a.scoring == SIGMOID_BIAS) {
#pragma unroll
      for (int i = 0; i < kFusedPerLane; ++i) {
        const int e = sub + i * G;
        if (e < E) {
          const double af = 1.0 / (1.0 + exp(-v[i]));
          z += af;
          v[i] = a.sel_bias != nullptr ? af + (double)a.sel_bias[e] : af;
        }
      }
      z = group_sum(z, G);
    }
    // top-k: slots in descending key order, ties to the lower expert
    unsigned mine = 0u;                  // bit i: expert sub + i G taken
    unsigned long long tmask = 0ull;
    for (int j = 0; j < k; ++j) {
      int be = -1;
      double best = 0.0;
#pragma unroll
      for (int i = 0; i < kFusedPerLane; ++i) {
        const int e = sub + i * G;
        if (e < E && !((mine >> i) & 1u) && (be < 0 || v[i] > best)) { best = v[i]; be = e; }
      }
      for (int o = 1; o < G; o <<= 1) {
        const double ob = __shfl_xor(best, o);
        const int oe = __shfl_xor(be, o);
        if (oe >= 0 && (be < 0 || ob > best || (ob == best && oe < be))) { best = ob; be = oe; }
      }
      if (be % G == sub) mine |= 1u << (be / G);
      tmask |= 1ull << be;
      if (sub == 0) {
        sidx[t * k + j] = be;
        if (stats_here) atomicAdd(&scnt[be], 1);
        // the own token keeps what its weight is made of: p, s, or the unbiased a
        if (t == t0) sval[j] = a.scoring == SIGMOID_BIAS ? 1.0 / (1.0 + exp(-st[be])) : best;
      }
    }
    if (sub == 0) smask[t] = tmask;
    if (stats_here) {
      // soft probabilities: softmax p for both softmax rules, a / sum a for sigmoid
      if (a.scoring == TOPK_SOFTMAX) {
#pragma unroll
        for (int i = 0; i < kFusedPerLane; ++i)
          if (sub + i * G < E) { v[i] = exp(v[i] - m); z += v[i]; }
        z = group_sum(z, G);
      }
#pragma unroll
      for (int i = 0; i < kFusedPerLane; ++i) {
        const int e = sub + i * G;
        if (e < E) {
          st[e] = a.scoring == SOFTMAX_TOPK ? v[i]
                : a.scoring == TOPK_SOFTMAX ? v[i] / z
                                            : (1.0 / (1.0 + exp(-st[e]))) / z;
        }
      }
    }
    if (t == t0 && sub == 0) {
      // p_sel or a_sel (divided by their sum when renormalising), or the
      // softmax over the selected logits
      const double top = sval[0];
      double sum = 0.0;
      for (int j = 0; j < k; ++j) sum += a.scoring == TOPK_SOFTMAX ? exp(sval[j] - top) : sval[j];
      const bool renorm = a.scoring == TOPK_SOFTMAX || a.renormalize;
      for (int j = 0; j < k; ++j) {
        const double q = a.scoring == TOPK_SOFTMAX ? exp(sval[j] - top) : sval[j];
        const float wj = (float)(renorm ? q / sum : q);
        sval[j] = (double)wj;
        if (a.topk_idx) a.topk_idx[(long long)t0 * k + j] = sidx[t0 * k + j];
        if (a.topk_w) a.topk_w[(long long)t0 * k + j] = wj;
      }
    }
  }
  __syncthreads();

  // 3. ranks of the own token's assignments (earlier tokens with the same
  // expert); beside them the activations of every slot and of the shared
  // experts, and in workgroup 0 the chunk sums of P
  for (int j = 0; j < k; ++j) {
    const int e = sidx[t0 * k + j];
    const unsigned long long hits = __ballot(tid < t0 && ((smask[tid] >> e) & 1ull));
    if (lane == 0) srank[wave * kFusedMaxK + j] = __popcll(hits);
  }
  const float* sx = sxa + t0 * R;
  const TA* __restrict__ w13 = static_cast<const TA*>(a.w13);
  const TA* __restrict__ ws13 = static_cast<const TA*>(a.ws13);
  const int nF = a.activation == SWIGLU ? 2 * F : F;
  const int n_act = k * F + SF;
  const int n_p1 = stats_here ? kFusedChunks * E : 0;
  const int csz = (T + kFusedChunks - 1) / kFusedChunks;
  for (int i = tid; i < n_act + n_p1; i += kFusedThreads) {
    if (i < n_act) {
      float h;
      if (i < k * F) {
        const int j = i / F, f = i % F;
        const TA* gr = w13 + ((long long)sidx[t0 * k + j] * nF + f) * D;
        if (a.activation == SWIGLU) {
          const float2 gu = dot2_f32(sx, gr, gr + (long long)F * D, D);
          h = silu_f32(gu.x) * gu.y;
        } else {
          const float g = dot_f32(sx, gr, D);
          h = 0.5f * g * erfcf(-g * 0.70710678118654752f);   // exact GELU, no cancellation for g < 0
        }
      } else {
        const int f = i - k * F;
        const float2 gu = dot2_f32(sx, ws13 + (long long)f * D, ws13 + (long long)(SF + f) * D, D);
        h = silu_f32(gu.x) * gu.y;
      }
      sh[i] = h;
    } else {
      const int c = (i - n_act) / E, e = (i - n_act) % E;
      double ps = 0.0;
      for (int t = c * csz; t < T && t < (c + 1) * csz; ++t) ps += sp[t * E + e];
      spsum[c * E + e] = ps;
    }
  }
  __syncthreads();
  unsigned kept = 0u;
  for (int j = 0; j < k; ++j) {
    int rank = 0;
#pragma unroll
    for (int w = 0; w < kFusedWaves; ++w) rank += srank[w * kFusedMaxK + j];
    if (rank < a.capacity) kept |= 1u << j;
  }

  // 4. output rows: one per kept slot (weighted), one for the shared experts;
  // workgroup 0 also sums P over the chunks and writes f and P
  const TA* __restrict__ w2 = static_cast<const TA*>(a.w2);
  const TA* __restrict__ ws2 = static_cast<const TA*>(a.ws2);
  const int n_out = (k + (SF > 0 ? 1 : 0)) * D;
  const int n_p2 = stats_here ? E : 0;
  for (int i = tid; i < n_out + n_p2; i += kFusedThreads) {
    if (i < n_out) {
      const int j = i / D, d = i % D;
      float v = 0.0f;
      if (j < k) {
        if ((kept >> j) & 1u)
          v = (float)sval[j] * dot_f32(sh + j * F, w2 + ((long long)sidx[t0 * k + j] * D + d) * F, F);
      } else {
        v = dot_f32(sh + k * F, ws2 + (long long)d * SF, SF);
      }
      spart[i] = v;
    } else {
      const int e = i - n_out;
      double P = 0.0;
      for (int c = 0; c < kFusedChunks; ++c) P += spsum[c * E + e];
      P /= (double)T;
      const int cnt = scnt[e];
      const double f = (double)cnt / (double)(T * k);
      sfp[e] = f * P;
      if (a.counts) a.counts[e] = cnt;
      if (a.stats) {
        a.stats[e] = (float)f;
        a.stats[E + e] = (float)P;
      }
    }
  }
  __syncthreads();
  TA* __restrict__ y = static_cast<TA*>(a.y);
  for (int d = tid; d < D; d += kFusedThreads) {
    float acc = SF > 0 ? spart[k * D + d] : 0.0f;
    for (int j = 0; j < k; ++j) acc += spart[j * D + d];
    y[(long long)t0 * D + d] = from_f32<TA>(acc);
  }

  // 5. the balance loss, max / mean and drops (workgroup 0, its last thread)
  if (stats_here && tid == kFusedThreads - 1) {
    double fp = 0.0;
    int cmax = 0, drop = 0;
    for (int e = 0; e < E; ++e) {
      fp += sfp[e];
      cmax = scnt[e] > cmax ? scnt[e] : cmax;
      drop += scnt[e] > a.capacity ? scnt[e] - a.capacity : 0;
    }
    if (a.stats) {
      a.stats[2 * E] = (float)((double)a.alpha * (double)E * fp);
      a.stats[2 * E + 1] = (float)((double)cmax / ((double)(T * k) / (double)E));
    }
    if (a.dropped) *a.dropped = drop;
  }
}

}  // namespace

bool fused_layer_fits(int act_dtype, int T, int D, int E, int k, int F, int SF) {
  if (T <= 0 || T > kFusedMaxTokens || kFusedMaxTokens > kFusedThreads) return false;
  if (k <= 0 || k > kFusedMaxK || k > E || E > kFusedMaxE) return false;
  if (act_dtype != F32 && act_dtype != BF16) return false;
  if (D <= 0 || D % 4 || F <= 0 || F % 4 || SF < 0 || SF % 4) return false;
  if (D > 4096 || F > 16384 || SF > 16384) return false;     // keeps the LDS arithmetic in int
  return fused_lds(T, D, E, k, F, SF).total <= kFusedMaxLds;
}

hipError_t launch_fused_layer(const FusedArgs& a, int act_dtype, int router_dtype, hipStream_t s) {
  if (!fused_layer_fits(act_dtype, a.T, a.D, a.E, a.k, a.F, a.SF)) return hipErrorInvalidValue;
  if (a.SF > 0 && (a.ws13 == nullptr || a.ws2 == nullptr)) return hipErrorInvalidValue;
  const int lds = fused_lds(a.T, a.D, a.E, a.k, a.F, a.SF).total;
  const dim3 grid((unsigned)a.T), block(kFusedThreads);
  if (act_dtype == F32)
    hipLaunchKernelGGL((fused_layer_kernel<float, float>), grid, block, lds, s, a);
  else if (router_dtype == F32)
    hipLaunchKernelGGL((fused_layer_kernel<bf16_t, float>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((fused_layer_kernel<bf16_t, bf16_t>), grid, block, lds, s, a);
  return hipGetLastError();
}

}  // namespace moe
