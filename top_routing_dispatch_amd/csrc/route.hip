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
  // Among the k+1 best keys, pick r is "close" to pick r+1 when their float32
  // keys are within 2 tau.  Exactly the picks in a close run get float64
  // keys; when the run reaches the k-th/(k+1)-th boundary, so does every
  // other expert whose key lies within 2 tau below the k-th.  Ranking refined
  // experts by their float64 key and all others by their float32 key then
  // gives the order of the exact keys: any pair with an unrefined member is
  // more than 2 tau apart, far beyond the error of either key.
  const float next_key = __shfl_down(my_key, 1);
  const bool close = (lane + 1 < nsel) && (my_key - next_key <= 2.0f * tau);
  const unsigned long long close_mask = __ballot(close);
  if (close_mask != 0) {
    // pick r needs float64 when it is close to a neighbour
    const bool prev_close = lane > 0 && ((close_mask >> (lane - 1)) & 1ull);
    const bool pick_ref = lane < nsel && (close || prev_close);
    const bool boundary = k < nsel && ((close_mask >> (k - 1)) & 1ull);
    const float thr = __shfl(my_key, k - 1) - 2.0f * tau;
    // per-expert flags: candidate (ranked at all) and refined (float64 key)
    bool cand[EPL], ref[EPL];
    double m64[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      cand[i] = false;
      ref[i] = false;
      m64[i] = (double)key[i];
    }
    // the k+1 picks are candidates; publish which of them are refined
    for (int r = 0; r < nsel; ++r) {
      const int pe_r = __shfl(my_e, r);
      const bool pr = __shfl((int)pick_ref, r) != 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i == pe_r) { cand[i] = true; ref[i] = pr; }
    }
    if (boundary) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E && !cand[i] && key[i] >= thr) { cand[i] = true; ref[i] = true; }
    }
    // float64 logits of the refined experts, up to eight per pass over the
    // token row (the loop is unrolled so several rows' loads are in flight)
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      unsigned long long m = __ballot(ref[i]);
      while (m) {
        constexpr int NB = 4;
        int ce[NB];
        int nb = 0;
        for (; nb < NB && m; ++nb) {
          const int l = __builtin_ctzll(m);
          m &= m - 1;
          ce[nb] = l + kWave * i;
        }
        for (int c = nb; c < NB; ++c) ce[c] = ce[0];
        double acc[NB];
#pragma unroll
        for (int c = 0; c < NB; ++c) acc[c] = 0.0;
        const long long xo = (long long)t * a.D;

        for (int d = lane * 4; d < a.D; d += kWave * 4) {
          float xv[4];
          load4(a.x, a.act_dtype, xo + d, xv);
#pragma unroll
          for (int c = 0; c < NB; ++c) {
            float wv[4];
            load4(a.w_router, a.router_dtype, (long long)ce[c] * a.D + d, wv);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[c] = fma((double)xv[q], (double)wv[q], acc[c]);
          }
        }
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          if (c < nb) {
            const double s64 = wave_sum_f64(acc[c]);
            double q64 = s64;
            if (sig) q64 = 1.0 / (1.0 + exp(-s64)) + (a.sel_bias ? (double)a.sel_bias[ce[c]] : 0.0);
            if (lane == (ce[c] & 63)) m64[i] = q64;
          }
        }
      }
    }
    // rank the candidates: k rounds of (key desc, expert asc)
    bool tk[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) tk[i] = !cand[i];
    for (int r = 0; r < k; ++r) {
      double bv = -INFINITY;
      int be = INT_MAX;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!tk[i] && (be == INT_MAX || m64[i] > bv)) { bv = m64[i]; be = lane + kWave * i; }
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

namespace moe {
namespace {

// hi = rne(w), mid = rne(w - hi), lo = w - hi - mid: every difference is exact
// in float32 and lo has at most 8 significant bits, so hi + mid + lo == w.
__global__ __launch_bounds__(256) void split_bf16x3_kernel(const float* __restrict__ w, int E, int D,
                                                           bf16_t* __restrict__ out) {
  const long long n = (long long)E * D;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const int e = (int)(i / D), d = (int)(i % D);
    const float v = w[i];
    const bf16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    const bf16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    const bf16_t lo = f32_to_bf16(r2);
    bf16_t* o = out + (long long)e * 3 * D + d;
    o[0] = hi;
    o[D] = mid;
    o[2 * D] = lo;
  }
}

}  // namespace

hipError_t launch_split_bf16x3(const float* w, int E, int D, bf16_t* out, hipStream_t s) {
  const long long n = (long long)E * D;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(split_bf16x3_kernel, dim3(blocks), dim3(256), 0, s, w, E, D, out);
  return hipGetLastError();
}

}  // namespace moe
