// Gate: scoring, top-k selection and combine weights from the router logits.
//
// Scoring rules follow the "Top-k 路由" page (門控函式的數學形式, Step 2 and
// its note on the two softmax orders; Switch keeps the raw top-1 softmax
// value) and the "别只比较 Top-k" page (Score / Select / Merge: sigmoid
// affinity, a bias that takes part in selection only, weights from the
// unbiased affinities).  Top-k per token as in the Tiny-MoE walk-through
// ("从 Dense FFN 到 MoE" §4) and the glossary's TopKRouter.
//
// One wavefront per token.  Lane l holds experts l, l+64, l+128, ...; the
// k (+1) best are found by k (+1) rounds of a wave-wide arg-max with ties to
// the lower expert index, and lane r keeps the r-th pick in a register.
//
// Near-tie refinement: the logits arrive in float32.  Wherever two of the
// k+1 best keys of a token are closer than twice a bound on the float32 error,
// every expert within that distance of the k-th key has its logit recomputed
// as a float64 dot product, and the selection is redone in float64 on those
// candidates.  Every expert outside the candidate set is provably below the
// k-th selected one, so the result equals the selection on exact logits.
#include <float.h>
#include <limits.h>

#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
// Wave-wide arg-max over (value desc, expert asc); every lane gets the result.
template <typename V>
__device__ __forceinline__ void wave_argmax(V& v, int& e) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const V ov = __shfl_xor(v, off);
    const int oe = __shfl_xor(e, off);
    if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
  }
}

// Four consecutive elements (D is a multiple of 4) widened to float.
__device__ __forceinline__ void load4(const void* p, int dt, long long i, float v[4]) {
  if (dt == BF16) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(p) + i);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  } else {
    const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
}

// float64 dot product of token row t with router row e, reduced over the wave.
__device__ double logit_f64(const RouteArgs& a, int t, int e, int lane) {
  double acc = 0.0;
  const long long xo = (long long)t * a.D, wo = (long long)e * a.D;
  for (int d = lane * 4; d < a.D; d += kWave * 4) {
    float xv[4], wv[4];
    load4(a.x, a.act_dtype, xo + d, xv);
    load4(a.w_router, a.router_dtype, wo + d, wv);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = fma((double)xv[q], (double)wv[q], acc);
  }
  return wave_sum_f64(acc);
}

__device__ __forceinline__ float sigmoid_f32(float s) { return 1.0f / (1.0f + expf(-s)); }

template <int EPL>
__global__ __launch_bounds__(256) void route_select_kernel(const RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;                        // uniform per wave
  const int E = a.E, k = a.k;
  const bool sig = a.scoring == SIGMOID_BIAS;
  const float* srow = a.logits + (long long)t * E;

  float s[EPL], key[EPL];
  bool taken[EPL];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    const bool valid = e < E;
    s[i] = valid ? srow[e] : 0.0f;
    float q = -INFINITY;
    if (valid) q = sig ? sigmoid_f32(s[i]) + (a.sel_bias ? a.sel_bias[e] : 0.0f) : s[i];
    key[i] = q;
    taken[i] = !valid;
    amax = fmaxf(amax, fabsf(s[i]));
  }
  amax = wave_max_f32(amax);
  // Margin on |float32 logit - exact logit|.  The logits come from float32
  // sums of 64-deep slices added in float64, whose error is ~1e-7 at
  // D = 7168; the margin is about two orders of magnitude above that.  It is
  // mapped onto the ranking key (sigmoid slope <= 1/4).
  const float eps_s = ldexpf(1.0f + amax, -16);
  const float tau = sig ? 0.25f * eps_s + 1e-6f : eps_s;

  // ---- k (+1) best keys; lane r keeps pick r.
  const int nsel = min(k + 1, E);
  int my_e = -1;
  float my_key = -INFINITY;
  for (int r = 0; r < nsel; ++r) {
    float bv = -INFINITY;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!taken[i] && (be == INT_MAX || key[i] > bv)) { bv = key[i]; be = lane + kWave * i; }
    wave_argmax(bv, be);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i == be) taken[i] = true;
    if (lane == r) { my_e = be; my_key = bv; }
  }

  // ---- near-tie refinement in float64
  const float next_key = __shfl_down(my_key, 1);
  const bool close = (lane + 1 < nsel) && (my_key - next_key <= 2.0f * tau);
  if (__ballot(close) != 0) {
    const float thr = __shfl(my_key, k - 1) - 2.0f * tau;
    double k64[EPL];
    bool cand[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      cand[i] = e < E && key[i] >= thr;
      k64[i] = -INFINITY;
      unsigned long long m = __ballot(cand[i]);
      while (m) {
        const int l = __builtin_ctzll(m);
        m &= m - 1;
        const int ce = l + kWave * i;
        const double s64 = logit_f64(a, t, ce, lane);
        double q64 = s64;
        if (sig) q64 = 1.0 / (1.0 + exp(-s64)) + (a.sel_bias ? (double)a.sel_bias[ce] : 0.0);
        if (lane == l) k64[i] = q64;
      }
    }
    bool tk[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) tk[i] = !cand[i];
    for (int r = 0; r < k; ++r) {
      double bv = -INFINITY;
      int be = INT_MAX;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!tk[i] && (be == INT_MAX || k64[i] > bv)) { bv = k64[i]; be = lane + kWave * i; }
      wave_argmax(bv, be);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i == be) tk[i] = true;
      if (lane == r) my_e = be;
    }
  }

  // ---- weights from the float32 logits
  // s of this lane's pick (lanes r < k): fetch from the owner lane.
  const int pe = (lane < k) ? my_e : 0;
  float s_pick = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float v = __shfl(s[i], pe & 63);
    if ((pe >> 6) == i) s_pick = v;
  }
  const bool slot = lane < k;
  float w = 0.0f;
  float smax = -INFINITY, z = 0.0f;
  if (a.scoring == SOFTMAX_TOPK || a.probs != nullptr) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) m = fmaxf(m, sig ? -INFINITY : s[i]);
    smax = wave_max_f32(m);
  }
  if (a.scoring == SOFTMAX_TOPK) {
    float zz = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) zz += expf(s[i] - smax);
    z = wave_sum_f32(zz);
    const float p = slot ? expf(s_pick - smax) / z : 0.0f;
    if (a.renormalize) {
      const float ps = wave_sum_f32(p);
      w = p / ps;
    } else {
      w = p;
    }
  } else if (a.scoring == TOPK_SOFTMAX) {
    const float msel = wave_max_f32(slot ? s_pick : -INFINITY);
    const float ex = slot ? expf(s_pick - msel) : 0.0f;
    w = ex / wave_sum_f32(ex);
  } else {
    const float af = slot ? sigmoid_f32(s_pick) : 0.0f;
    w = a.renormalize ? af / wave_sum_f32(af) : af;
  }
  if (slot) {
    a.topk_idx[(long long)t * k + lane] = my_e;
    a.topk_w[(long long)t * k + lane] = w;
  }

  // ---- per-token soft probabilities for the balance loss
  if (a.probs != nullptr) {
    float* prow = a.probs + (long long)t * E;
    if (sig) {
      float av[EPL], as = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        av[i] = (lane + kWave * i < E) ? sigmoid_f32(s[i]) : 0.0f;
        as += av[i];
      }
      as = wave_sum_f32(as);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) prow[lane + kWave * i] = av[i] / as;
    } else {
      if (a.scoring != SOFTMAX_TOPK) {
        float zz = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (lane + kWave * i < E) zz += expf(s[i] - smax);
        z = wave_sum_f32(zz);
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) prow[lane + kWave * i] = expf(s[i] - smax) / z;
    }
  }
}

template <int EPL>
hipError_t launch_epl(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(route_select_kernel<EPL>, dim3(ceil_div(a.T, 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_select(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int epl = ceil_div(a.E, kWave);
  if (epl <= 1) return launch_epl<1>(a, s);
  if (epl <= 2) return launch_epl<2>(a, s);
  if (epl <= 4) return launch_epl<4>(a, s);
  if (epl <= 8) return launch_epl<8>(a, s);
  return launch_epl<16>(a, s);
}

}  // namespace moe
