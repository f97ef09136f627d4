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
// the lower expert index (the maximum by DPP moves across the lanes, then the
// first slot and lane holding it by ballots), and lane r keeps the r-th pick
// in a register.
//
// Near-tie refinement: the logits arrive in float32.  Among the k+1 best keys,
// pick r is "close" to pick r+1 when their float32 keys are within 2 tau (tau
// bounds the float32 error).  The picks in a close run get float64 logits;
// when the run reaches the k-th/(k+1)-th boundary, so does every other expert
// whose key lies within 2 tau below the k-th.  Ranking refined experts by their
// float64 key and all others by their float32 key gives the order of the exact
// keys: any pair with an unrefined member is more than 2 tau apart.  Such
// tokens are refined in their own wavefront, in the selection kernel (up to
// 128 experts) or in a second pass (one wavefront per flagged token).
#include <float.h>
#include <limits.h>

#include "common.h"

namespace moe {
namespace {

// ---- wave-wide reductions ----
// Float max / sum over the 64 lanes by DPP moves (row-local butterflies, then
// the row broadcasts), in a fixed order; the result is read from lane 63 and
// is wave-uniform.  `id` is the identity, which lanes outside a row mask take.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f32(float v, float id) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(v), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_max_u(float v) {
  v = fmaxf(v, dpp_f32<0xb1, 0xf>(v, -INFINITY));    // lane ^ 1
  v = fmaxf(v, dpp_f32<0x4e, 0xf>(v, -INFINITY));    // lane ^ 2
  v = fmaxf(v, dpp_f32<0x141, 0xf>(v, -INFINITY));   // mirror inside 8 lanes
  v = fmaxf(v, dpp_f32<0x140, 0xf>(v, -INFINITY));   // mirror inside 16 lanes
  v = fmaxf(v, dpp_f32<0x142, 0xa>(v, -INFINITY));   // lane 15 of a row into the next
  v = fmaxf(v, dpp_f32<0x143, 0xc>(v, -INFINITY));   // lane 31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_u(float v) {
  v += dpp_f32<0xb1, 0xf>(v, 0.0f);
  v += dpp_f32<0x4e, 0xf>(v, 0.0f);
  v += dpp_f32<0x141, 0xf>(v, 0.0f);
  v += dpp_f32<0x140, 0xf>(v, 0.0f);
  v += dpp_f32<0x142, 0xa>(v, 0.0f);
  v += dpp_f32<0x143, 0xc>(v, 0.0f);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
// Wave-wide arg-max over (value desc, expert asc) for the refinement.
__device__ __forceinline__ void wave_argmax_f64(double& v, int& e) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ov = __shfl_xor(v, off);
    const int oe = __shfl_xor(e, off);
    if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
  }
}

// EL consecutive elements, bf16 (BF) or float32, as raw 16-byte words, and
// widened to float.  The type is a template parameter, and the loads of a
// batch are issued before any is widened, so that they are in flight
// together.
template <bool BF, int EL>
struct RawEl {
  static_assert(EL == 4 || EL == 8, "elements per load");
  static constexpr int NQ = BF ? EL / 8 + (EL % 8 != 0) : EL / 4;
  uint4 q[NQ];
  __device__ __forceinline__ void load(const void* p, long long i) {
    if constexpr (BF) {
      const bf16_t* b = static_cast<const bf16_t*>(p) + i;
      if constexpr (EL == 8) {
        q[0] = *reinterpret_cast<const uint4*>(b);
      } else {
        const uint2 h = *reinterpret_cast<const uint2*>(b);
        q[0] = make_uint4(h.x, h.y, 0u, 0u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NQ; ++j) q[j] = *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i + 4 * j);
    }
  }
  __device__ __forceinline__ float get(int e) const {
    if constexpr (BF) {
      const unsigned u = (&q[0].x)[e >> 1];
      return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
    } else {
      return __uint_as_float((&q[e >> 2].x)[e & 3]);
    }
  }
};

// Input types of the refinement's dot products: 0 = float32 tokens and
// router weight, 1 = bf16 tokens and float32 weight, 2 = both bf16.
constexpr int kDtF32 = 0, kDtBf16F32 = 1, kDtBf16 = 2;

__device__ __forceinline__ float sigmoid_f32(float s) { return 1.0f / (1.0f + expf(-s)); }

// Float32 selection state of one token, held by one wave.
template <int EPL>
struct TokenSel {
  float s[EPL], key[EPL];
  bool taken[EPL];
  int my_e;          // lane r < nsel: the r-th pick
  float my_key;
  float tau;
  int nsel;
};

// Pick with the largest key among the experts not yet taken, ties to the lower
// expert index: the wave maximum of the per-lane maxima, then the first slot
// and lane that hold it (expert lane + 64 i grows with i, then with the lane).
template <int EPL>
__device__ __forceinline__ int wave_pick(const float key[EPL], const bool taken[EPL], float& best) {
  float bv = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (!taken[i]) bv = fmaxf(bv, key[i]);
  best = wave_max_u(bv);
  int be = INT_MAX;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const unsigned long long m = __ballot(!taken[i] && key[i] == best);
    if (be == INT_MAX && m != 0ull) be = __builtin_ctzll(m) + kWave * i;
  }
  return be;
}

template <int EPL>
__device__ __forceinline__ void select_f32(const RouteArgs& a, int t, int lane, TokenSel<EPL>& st) {
  const int E = a.E, k = a.k;
  const bool sig = a.scoring == SIGMOID_BIAS;
  const float* srow = a.logits + (long long)t * E;
  // every load first, with no branch between them (indices clamped, values
  // of lanes past E dropped afterwards): behind a per-slot branch the
  // compiler issued one load at a time
  float sv[EPL], bv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) sv[i] = srow[min(lane + kWave * i, E - 1)];
#pragma unroll
  for (int i = 0; i < EPL; ++i) bv[i] = 0.0f;
  if (sig && a.sel_bias != nullptr) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) bv[i] = a.sel_bias[min(lane + kWave * i, E - 1)];
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    const bool valid = e < E;
    st.s[i] = valid ? sv[i] : 0.0f;
    float q = -INFINITY;
    if (valid) q = sig ? sigmoid_f32(st.s[i]) + bv[i] : st.s[i];
    st.key[i] = q;
    st.taken[i] = !valid;
    amax = fmaxf(amax, fabsf(st.s[i]));
  }
  amax = wave_max_u(amax);
  // Margin on |float32 logit - exact logit|.  The logits come from float32
  // sums of 64-deep slices added in float64, whose error is ~1e-6 at
  // D = 7168; the margin is about two orders of magnitude above that.  It is
  // mapped onto the ranking key (sigmoid slope <= 1/4).
  const float eps_s = ldexpf(1.0f + amax, -16);
  st.tau = sig ? 0.25f * eps_s + 1e-6f : eps_s;
  st.nsel = min(k + 1, E);
  st.my_e = -1;
  st.my_key = -INFINITY;
  for (int r = 0; r < st.nsel; ++r) {
    float bv;
    const int be = wave_pick<EPL>(st.key, st.taken, bv);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i == be) st.taken[i] = true;
    if (lane == r) { st.my_e = be; st.my_key = bv; }
  }
}

// Bit r set: picks r and r+1 are within 2 tau.
template <int EPL>
__device__ __forceinline__ unsigned long long close_mask(const TokenSel<EPL>& st, int lane) {
  const float next_key = __shfl_down(st.my_key, 1);
  return __ballot((lane + 1 < st.nsel) && (st.my_key - next_key <= 2.0f * st.tau));
}

// Softmax statistics of one token's logits over the E experts: the maximum
// and the sum of exp(s - max) (wave-uniform).
template <int EPL>
__device__ __forceinline__ void softmax_stats(const TokenSel<EPL>& st, int lane, int E, float& smax, float& z) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + kWave * i < E) m = fmaxf(m, st.s[i]);
  smax = wave_max_u(m);
  float zz = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + kWave * i < E) zz += expf(st.s[i] - smax);
  z = wave_sum_u(zz);
}

// Combine weights from the float32 logits for the picks my_e of lanes < k,
// written with the expert ids.  smax, z: softmax_stats (SOFTMAX_TOPK only).
template <int EPL>
__device__ __forceinline__ void write_selection(const RouteArgs& a, int t, int lane, const TokenSel<EPL>& st,
                                                int my_e, float smax, float z) {
  const int k = a.k;
  const int pe = (lane < k) ? my_e : 0;
  float s_pick = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const float v = __shfl(st.s[i], pe & 63);
    if ((pe >> 6) == i) s_pick = v;
  }
  const bool slot = lane < k;
  float w = 0.0f;
  if (a.scoring == SOFTMAX_TOPK) {
    const float p = slot ? expf(s_pick - smax) / z : 0.0f;
    w = a.renormalize ? p / wave_sum_u(p) : p;
  } else if (a.scoring == TOPK_SOFTMAX) {
    const float msel = wave_max_u(slot ? s_pick : -INFINITY);
    const float ex = slot ? expf(s_pick - msel) : 0.0f;
    w = ex / wave_sum_u(ex);
  } else {
    const float af = slot ? sigmoid_f32(s_pick) : 0.0f;
    w = a.renormalize ? af / wave_sum_u(af) : af;
  }
  if (slot) {
    a.topk_idx[(long long)t * k + lane] = my_e;
    a.topk_w[(long long)t * k + lane] = w;
  }
}

// Refinement of one token on its wavefront, from the float32 state st and its
// close mask cm: float64 logits for the experts that need them (D-long dot
// products of the stored inputs of types DT, two experts per pass over the
// token's row, 8 (bf16 tokens) or 4 elements per lane and step, UNROLL steps
// of loads in flight), then the candidates ranked and the token's selection
// written.
template <int EPL, int UNROLL, int DT>
__device__ __forceinline__ void refine_token(const RouteArgs& a, int t, int lane, const TokenSel<EPL>& st,
                                          unsigned long long cm, float smax, float z) {
  const bool sig = a.scoring == SIGMOID_BIAS;
  const bool cl = (cm >> lane) & 1ull;
  const bool prev_close = lane > 0 && ((cm >> (lane - 1)) & 1ull);
  const bool pick_ref = lane < st.nsel && (cl || prev_close);
  const bool boundary = a.k < st.nsel && ((cm >> (a.k - 1)) & 1ull);
  const float thr = __shfl(st.my_key, a.k - 1) - 2.0f * st.tau;
  bool cand[EPL], ref[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) { cand[i] = false; ref[i] = false; }
  for (int r = 0; r < st.nsel; ++r) {
    const int pe_r = __shfl(st.my_e, r);
    const bool pr = __shfl((int)pick_ref, r) != 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i == pe_r) { cand[i] = true; ref[i] = pr; }
  }
  if (boundary) {
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < a.E && !cand[i] && st.key[i] >= thr) { cand[i] = true; ref[i] = true; }
  }
  double m64[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) m64[i] = (double)st.key[i];
  const long long xo = (long long)t * a.D;
  // the refined experts, in expert order, four per pass over x
  unsigned long long rm[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) rm[i] = __ballot(ref[i]);
  int slot_i = 0;
  auto next_ref = [&]() -> int {      // next refined expert id, -1 when done (uniform)
    while (slot_i < EPL) {
      unsigned long long m = 0ull;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (i == slot_i) m = rm[i];
      if (m != 0ull) {
        const int l = __builtin_ctzll(m);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (i == slot_i) rm[i] &= rm[i] - 1;
        return l + kWave * slot_i;
      }
      ++slot_i;
    }
    return -1;
  };
  for (;;) {
    int ex[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) ex[j] = next_ref();
    if (ex[0] < 0) break;
    // branch-free body (a missing second expert repeats the first, its sum is
    // dropped), unrolled so that several slices' loads are in flight at once
    long long wo[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) wo[j] = (long long)(ex[j] >= 0 ? ex[j] : ex[0]) * a.D;
    double acc[2] = {0.0, 0.0};
    constexpr int EL = DT == kDtF32 ? 4 : 8;
    constexpr int STEP = kWave * EL;
    for (int d0 = 0; d0 < a.D; d0 += STEP * UNROLL) {
      // UNROLL steps: every load first (lanes past the row's end re-read its
      // last EL elements and add nothing), then the products
      RawEl<DT != kDtF32, EL> xr[UNROLL];
      RawEl<DT == kDtBf16, EL> wr[UNROLL][2];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int d = min(d0 + u * STEP + lane * EL, a.D - EL);
        xr[u].load(a.x, xo + d);
#pragma unroll
        for (int j = 0; j < 2; ++j) wr[u][j].load(a.w_router, wo[j] + d);
      }
      __builtin_amdgcn_sched_barrier(0);     // keep the batch's loads ahead of every product
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const bool in = d0 + u * STEP + lane * EL < a.D;    // a re-read step adds zeros (finite inputs)
#pragma unroll
        for (int q = 0; q < EL; ++q) {
          const double xq = in ? (double)xr[u].get(q) : 0.0;
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[j] = fma(xq, (double)wr[u][j].get(q), acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (ex[j] < 0) continue;
      const double s64 = wave_sum_f64(acc[j]);
      double q64 = s64;
      if (sig) q64 = 1.0 / (1.0 + exp(-s64)) + (a.sel_bias ? (double)a.sel_bias[ex[j]] : 0.0);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i == ex[j]) m64[i] = q64;
    }
  }
  bool tk[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) tk[i] = !cand[i];
  int my_e = -1;
  for (int r = 0; r < a.k; ++r) {
    double bv = -INFINITY;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!tk[i] && (be == INT_MAX || m64[i] > bv)) { bv = m64[i]; be = lane + kWave * i; }
    wave_argmax_f64(bv, be);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i == be) tk[i] = true;
    if (lane == r) my_e = be;
  }
  write_selection(a, t, lane, st, my_e, smax, z);
}

// Pass 2: one wavefront per flagged token (the float32 state recomputed), all
// other waves exit at once.  The loads of the dot products run far ahead.
template <int EPL, int DT>
__global__ __launch_bounds__(256) void route_refine_kernel(const RouteArgs a, const int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T || flags[t] == 0) return;       // uniform per wave
  TokenSel<EPL> st;
  select_f32(a, t, lane, st);
  float smax = 0.0f, z = 1.0f;
  if (a.scoring == SOFTMAX_TOPK) softmax_stats(st, lane, a.E, smax, z);
  refine_token<EPL, 8, DT>(a, t, lane, st, close_mask(st, lane), smax, z);
}

// Pass 1: float32 selection of every token and its probabilities.  FUSED
// (up to 128 experts): the float64 refinement of the tokens that need it in
// the same wavefront, with a lean loop (at most two iterations of loads in
// flight) that keeps the kernel's register footprint small; otherwise a flag
// for pass 2.
template <int EPL, bool FUSED, int DT>
__global__ __launch_bounds__(256) void route_select_kernel(const RouteArgs a, int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;                        // uniform per wave
  const int E = a.E;
  TokenSel<EPL> st;
  select_f32(a, t, lane, st);
  const unsigned long long cm = close_mask(st, lane);
  const bool soft = a.scoring != SIGMOID_BIAS;
  float smax = 0.0f, z = 1.0f;
  if (soft && (a.scoring == SOFTMAX_TOPK || a.probs != nullptr)) softmax_stats(st, lane, E, smax, z);
  if (!FUSED && lane == 0) flags[t] = cm != 0;
  if (FUSED && cm != 0) refine_token<EPL, 2, DT>(a, t, lane, st, cm, smax, z);   // writes the selection
  else write_selection(a, t, lane, st, st.my_e, smax, z);

  if (a.probs != nullptr) {
    float* prow = a.probs + (long long)t * E;
    if (!soft) {
      float av[EPL], as = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        av[i] = (lane + kWave * i < E) ? sigmoid_f32(st.s[i]) : 0.0f;
        as += av[i];
      }
      as = wave_sum_u(as);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) prow[lane + kWave * i] = av[i] / as;
    } else {
      const float rz = 1.0f / z;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) prow[lane + kWave * i] = expf(st.s[i] - smax) * rz;
    }
  }
}

template <int EPL, int DT>
hipError_t launch_epl_dt(const RouteArgs& a, int32_t* flags, hipStream_t s) {
  if constexpr (EPL <= 2) {
    hipLaunchKernelGGL((route_select_kernel<EPL, true, DT>), dim3(ceil_div(a.T, 4)), dim3(256), 0, s, a, flags);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((route_select_kernel<EPL, false, DT>), dim3(ceil_div(a.T, 4)), dim3(256), 0, s, a, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((route_refine_kernel<EPL, DT>), dim3(ceil_div(a.T, 4)), dim3(256), 0, s, a,
                     (const int32_t*)flags);
  return hipGetLastError();
}

template <int EPL>
hipError_t launch_epl(const RouteArgs& a, int32_t* flags, hipStream_t s) {
  if (a.act_dtype != BF16) return launch_epl_dt<EPL, kDtF32>(a, flags, s);   // float32 tokens: float32 weight
  if (a.router_dtype != BF16) return launch_epl_dt<EPL, kDtBf16F32>(a, flags, s);
  return launch_epl_dt<EPL, kDtBf16>(a, flags, s);
}

}  // namespace

hipError_t launch_route_select(const RouteArgs& a, int32_t* flags, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int epl = ceil_div(a.E, kWave);
  if (epl <= 1) return launch_epl<1>(a, flags, s);
  if (epl <= 2) return launch_epl<2>(a, flags, s);
  if (epl <= 4) return launch_epl<4>(a, flags, s);
  if (epl <= 8) return launch_epl<8>(a, flags, s);
  return launch_epl<16>(a, flags, s);
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
