// Dispatch (permute), combine (unpermute) and load statistics.
//
// Dispatch groups the (token, slot) assignments by expert the way the
// Tiny-MoE walk-through's torch.where does ("从 Dense FFN 到 MoE" §5): experts
// in ascending id, and inside one expert the assignments in row-major
// (token, slot) order.  With a capacity C ("Top-k 路由" 容量因子 section) an
// expert keeps its first C assignments in that order; the rest are dropped
// and the residual path carries them ("别只比较 Top-k" mechanism table).
//
// Three small kernels (one, when the batch fits one tile), all deterministic
// (integer atomics only, whose result does not depend on their order):
//   histogram  per 256-token tile, per expert: a bit mask of the tile's tokens
//              that chose the expert (LDS atomicOr), popcounted;
//   scan       per expert over tiles -> tile bases and nominal counts; kept =
//              min(count, C); exclusive scan over experts -> offsets; m-tile
//              prefix for the grouped GEMM; unused row slots set to -1;
//   scatter    rank of a token inside its tile = popcount of the expert's mask
//              below it; row = offsets[e] + tile base + rank, kept if the
//              expert-local rank is below C.
#include "common.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kWordsPerTile = kPermuteTile / 32;

// Build the per-expert token masks of one tile.  Returns, for the calling
// thread's token, a bit per slot that is set for slots to skip (expert id
// out of range, or an id already used by an earlier slot of the same token).
__device__ uint32_t build_masks(const PermuteArgs& a, uint32_t* mask) {
  const int tid = threadIdx.x;
  for (int w = tid; w < a.E * kWordsPerTile; w += blockDim.x) mask[w] = 0u;
  __syncthreads();
  const int t = blockIdx.x * kPermuteTile + tid;
  uint32_t skip = 0u;
  if (t < a.T) {
    const uint32_t bit = 1u << (tid & 31);
    const int word = tid >> 5;
    for (int j = 0; j < a.k; ++j) {
      const int e = a.topk_idx[(long long)t * a.k + j];
      if ((unsigned)e >= (unsigned)a.E) { skip |= 1u << j; continue; }
      const uint32_t old = atomicOr(&mask[e * kWordsPerTile + word], bit);
      if (old & bit) skip |= 1u << j;
    }
  }
  __syncthreads();
  return skip;
}

__global__ __launch_bounds__(kPermuteTile) void hist_kernel(const PermuteArgs a) {
  __shared__ uint32_t mask[kMaxExperts * kWordsPerTile];
  build_masks(a, mask);
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWordsPerTile; ++w) c += __popc(mask[e * kWordsPerTile + w]);
    a.tile_counts[(long long)blockIdx.x * a.E + e] = c;
  }
}

__device__ int block_exclusive_scan(int v, int* s) {
  const int i = threadIdx.x;
  s[i] = v;
  __syncthreads();
  for (int d = 1; d < (int)blockDim.x; d <<= 1) {
    const int u = (i >= d) ? s[i - d] : 0;
    __syncthreads();
    s[i] += u;
    __syncthreads();
  }
  const int incl = s[i];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kMaxExperts) void scan_kernel(const PermuteArgs a, int ntiles) {
  __shared__ int s[kMaxExperts];
  __shared__ int s_total;
  const int e = threadIdx.x;
  int total = 0;
  if (e < a.E) {
    // the counts of 16 tiles are fetched together, then turned into the
    // tiles' base ranks inside expert e
    constexpr int B = 16;
    for (int t0 = 0; t0 < ntiles; t0 += B) {
      int c[B];
#pragma unroll
      for (int u = 0; u < B; ++u)
        c[u] = (t0 + u < ntiles) ? a.tile_counts[(long long)(t0 + u) * a.E + e] : 0;
#pragma unroll
      for (int u = 0; u < B; ++u) {
        if (t0 + u < ntiles) a.tile_counts[(long long)(t0 + u) * a.E + e] = total;
        total += c[u];
      }
    }
    a.counts[e] = total;
  }
  const int kept = (e < a.E) ? min(total, a.capacity) : 0;
  const int off = block_exclusive_scan(kept, s);
  if (e < a.E) a.offsets[e] = off;
  if (e == a.E - 1) { a.offsets[a.E] = off + kept; s_total = off + kept; }
  if (a.tile_prefix != nullptr) {
    const int mt = (e < a.E) ? ceil_div(kept, a.bm) : 0;
    const int mo = block_exclusive_scan(mt, s);
    if (e < a.E) a.tile_prefix[e] = mo;
    if (e == a.E - 1) a.tile_prefix[a.E] = mo + mt;
  }
  __syncthreads();
  for (int r = s_total + e; r < a.rows_cap; r += blockDim.x) a.token_of_row[r] = -1;
}

__global__ __launch_bounds__(kPermuteTile) void scatter_kernel(const PermuteArgs a) {
  __shared__ uint32_t mask[kMaxExperts * kWordsPerTile];
  const uint32_t skip = build_masks(a, mask);
  const int tid = threadIdx.x;
  const int t = blockIdx.x * kPermuteTile + tid;
  if (t >= a.T) return;
  const int word = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
  for (int j = 0; j < a.k; ++j) {
    int row = -1;
    if (!((skip >> j) & 1u)) {
      const int e = a.topk_idx[(long long)t * a.k + j];
      const uint32_t* m = mask + e * kWordsPerTile;
      int rank = __popc(m[word] & below);
      for (int w = 0; w < word; ++w) rank += __popc(m[w]);
      const int r_in_e = a.tile_counts[(long long)blockIdx.x * a.E + e] + rank;
      const int base = a.offsets[e];
      if (r_in_e < a.offsets[e + 1] - base) {
        row = base + r_in_e;
        a.token_of_row[row] = t;
      }
    }
    a.row_of[(long long)t * a.k + j] = row;
  }
}

// All three steps in one workgroup when the batch is a single tile (at most
// kPermuteTile tokens, as in decoding): thread i owns experts 4i .. 4i+3 for
// the counts and the scans, and token i for the scatter.
__global__ __launch_bounds__(kPermuteTile) void permute_one_tile_kernel(const PermuteArgs a) {
  static_assert(kMaxExperts <= 4 * kPermuteTile, "four experts per thread");
  __shared__ uint32_t mask[kMaxExperts * kWordsPerTile];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_scan[kPermuteTile];
  __shared__ int s_total;
  const uint32_t skip = build_masks(a, mask);
  const int tid = threadIdx.x;
  int kept[4], mt[4], sum_k = 0, sum_m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    int c = 0;
    if (e < a.E) {
#pragma unroll
      for (int w = 0; w < kWordsPerTile; ++w) c += __popc(mask[e * kWordsPerTile + w]);
      a.counts[e] = c;
    }
    kept[q] = min(c, a.capacity);
    mt[q] = ceil_div(kept[q], a.bm);
    sum_k += kept[q];
    sum_m += mt[q];
  }
  int off = block_exclusive_scan(sum_k, s_scan);
  int mo = block_exclusive_scan(sum_m, s_scan);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < a.E) {
      a.offsets[e] = off;
      s_off[e] = off;
      if (a.tile_prefix != nullptr) a.tile_prefix[e] = mo;
    }
    off += kept[q];
    mo += mt[q];
    if (e == a.E - 1) {
      a.offsets[a.E] = off;
      s_off[a.E] = off;
      s_total = off;
      if (a.tile_prefix != nullptr) a.tile_prefix[a.E] = mo;
    }
  }
  __syncthreads();
  for (int r = s_total + tid; r < a.rows_cap; r += blockDim.x) a.token_of_row[r] = -1;
  const int t = tid;
  if (t >= a.T) return;
  const int word = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
  for (int j = 0; j < a.k; ++j) {
    int row = -1;
    if (!((skip >> j) & 1u)) {
      const int e = a.topk_idx[(long long)t * a.k + j];
      const uint32_t* m = mask + e * kWordsPerTile;
      int rank = __popc(m[word] & below);
      for (int w = 0; w < word; ++w) rank += __popc(m[w]);
      if (rank < s_off[e + 1] - s_off[e]) {
        row = s_off[e] + rank;
        a.token_of_row[row] = t;
      }
    }
    a.row_of[(long long)t * a.k + j] = row;
  }
}

// x_perm[r] = x[token_of_row[r]] for rows with a token; 16-byte chunks.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ tor,
                                                          uint4* __restrict__ xp, int chunks) {
  const int r = blockIdx.x;
  const int tok = tor[r];
  if (tok < 0) return;
  const uint4* src = x + (long long)tok * chunks;
  uint4* dst = xp + (long long)r * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) dst[c] = src[c];
}

// ---------------------------------------------------------------------------
// combine: y[t] = sum_j w[t,j] * y_perm[row_of[t,j]] (+ y_shared[t])
// ---------------------------------------------------------------------------
template <typename T>
struct Chunk;
template <> struct Chunk<float> {
  static constexpr int N = 4;
  // 16 bytes as loaded, widened only where they are used
  static __device__ __forceinline__ uint4 raw(const float* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ float elem(const uint4& q, int i) {
    return __uint_as_float(i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w);
  }
  static __device__ __forceinline__ void load(const float* p, float v[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Chunk<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ uint4 raw(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ float elem(const uint4& q, int i) {
    const uint32_t w = (i >> 1) == 0 ? q.x : (i >> 1) == 1 ? q.y : (i >> 1) == 2 ? q.z : q.w;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  static __device__ __forceinline__ void load(const bf16_t* p, float v[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float v[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_rn(v[2 * i]) | ((uint32_t)f32_to_bf16_rn(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// A workgroup covers TPB consecutive tokens (TPB * D / N chunk items of N
// elements); their row indices and weights go to LDS once.  Each thread takes
// U items (item i, i + 256, ...) and issues the loads of every item's rows
// (G at a time; U * G = 8, or 4 for k <= 2, where more workgroups do better)
// and shared-expert chunk before the first multiply-add, so that many loads
// are in flight whatever k and D are.  Per
// item the sum runs over the slots in order, as a chain of fused
// multiply-adds, and the shared-expert chunk is added last.
constexpr int kCombineSlots = 1024;           // row indices / weights of a workgroup's tokens in LDS

template <typename T, int G>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ yp, const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ tw, const T* ys, T* y,
                                                      int ntok, int k, int D, int tpb, int cseg) {
  constexpr int N = Chunk<T>::N;
  constexpr int U = G >= 4 ? 8 / G : 4 / G;     // items per thread
  __shared__ int srow[kCombineSlots];
  __shared__ float sw[kCombineSlots];
  const int t0 = blockIdx.x * tpb;
  const int nt = min(tpb, ntok - t0);
  for (int i = threadIdx.x; i < nt * k; i += 256) {
    srow[i] = row_of[(long long)t0 * k + i];
    sw[i] = tw[(long long)t0 * k + i];
  }
  __syncthreads();
  // this workgroup's chunks of each of its tokens: [c0, c0 + cn)
  const int c0 = blockIdx.y * cseg;
  const int cn = min(cseg, D / N - c0);
  const int items = nt * cn;
  for (int base = 0; base < items; base += 256 * U) {
    int tl[U], cc[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = base + (int)threadIdx.x + 256 * u;
      ok[u] = it < items;
      tl[u] = ok[u] ? it / cn : 0;
      cc[u] = ok[u] ? c0 + it % cn : 0;
    }
    float acc[U][N];
    uint4 vs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vs[u] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int q = 0; q < N; ++q) acc[u][q] = 0.0f;
    }
    for (int j0 = 0; j0 < k; j0 += G) {
      uint4 v[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int j = j0 + g;
          const int r = (ok[u] && j < k) ? srow[tl[u] * k + j] : -1;
          if (r >= 0) v[u][g] = Chunk<T>::raw(yp + (long long)r * D + cc[u] * N);
        }
        // the shared-expert chunk is loaded with the first rows, added last
        if (ys != nullptr && j0 == 0 && ok[u]) vs[u] = Chunk<T>::raw(ys + (long long)(t0 + tl[u]) * D + cc[u] * N);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int j = j0 + g;
          const int r = (ok[u] && j < k) ? srow[tl[u] * k + j] : -1;
          if (r >= 0) {
            const float w = sw[tl[u] * k + j];
#pragma unroll
            for (int q = 0; q < N; ++q) acc[u][q] = fmaf(w, Chunk<T>::elem(v[u][g], q), acc[u][q]);
          }
        }
      }
    }
    if (ys != nullptr) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < N; ++q) acc[u][q] += Chunk<T>::elem(vs[u], q);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) Chunk<T>::store(y + (long long)(t0 + tl[u]) * D + cc[u] * N, acc[u]);
  }
}

// ---------------------------------------------------------------------------
// load statistics
// ---------------------------------------------------------------------------
// Column sums of probs over chunks of kStatsChunk tokens.  A block covers 64
// experts x one chunk: thread (e, rg) sums rows rg, rg + 4, ... of the chunk
// (all loads issued before the adds), then the four row groups are added in
// LDS in a fixed order.
__global__ __launch_bounds__(256) void stats_partial_kernel(const StatsArgs a) {
  __shared__ float sp[4][64];
  const int el = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int e = blockIdx.y * 64 + el;
  const int t0 = blockIdx.x * kStatsChunk;
  constexpr int PER = kStatsChunk / 4;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int t = t0 + rg + 4 * i;
    v[i] = (e < a.E && t < a.T) ? a.probs[(long long)t * a.E + e] : 0.0f;
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += v[i];
  sp[rg][el] = s;
  __syncthreads();
  if (rg == 0 && e < a.E)
    a.partial[(long long)blockIdx.x * a.E + e] = (sp[0][el] + sp[1][el]) + (sp[2][el] + sp[3][el]);
}

// f, P, loss, imbalance, dropped.  Thread (e, j) sums the partial chunks
// j, j + TPE, ... of expert e (TPE <= 64 consecutive lanes per expert) and the
// group is combined by a fixed shuffle tree; the scalar results use a fixed
// shuffle tree per wave and then the waves in order.
__global__ __launch_bounds__(kMaxExperts) void stats_final_kernel(const StatsArgs a, int nchunks, int tpe) {
  __shared__ float sP[kMaxExperts];
  __shared__ float wf[kMaxExperts / 64];
  __shared__ int wc[kMaxExperts / 64], wd[kMaxExperts / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = tid / tpe, j = tid % tpe;
  // per-expert counts (issued before the partial sums' adds)
  int c = 0, drop = 0;
  if (tid < a.E) {
    c = a.counts[tid];
    drop = c - min(c, a.capacity);
  }
  float s = 0.0f;
  if (e < a.E) {
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int b = j, q = 0;
    for (; b < nchunks; b += tpe, q = (q + 1) & 3) v[q] += a.partial[(long long)b * a.E + e];
    s = (v[0] + v[1]) + (v[2] + v[3]);
  }
  for (int d = tpe / 2; d >= 1; d >>= 1) s += __shfl_down(s, d, tpe);
  if (j == 0 && e < a.E) {
    const float pe = a.T > 0 ? s / (float)a.T : 0.0f;
    if (a.P) a.P[e] = pe;
    sP[e] = pe;
  }
  __syncthreads();
  const float A = (float)a.T * (float)a.k;
  float fp = 0.0f;
  if (tid < a.E) {
    const float fe = a.T > 0 ? (float)c / A : 0.0f;
    if (a.f) a.f[tid] = fe;
    fp = fe * sP[tid];
  }
  for (int d = 32; d >= 1; d >>= 1) {
    fp += __shfl_down(fp, d);
    c = max(c, __shfl_down(c, d));
    drop += __shfl_down(drop, d);
  }
  if (lane == 0) { wf[wave] = fp; wc[wave] = c; wd[wave] = drop; }
  __syncthreads();
  if (tid == 0) {
    float sf = 0.0f;
    int cm = 0, sd = 0;
    for (int w = 0; w < kMaxExperts / 64; ++w) { sf += wf[w]; cm = max(cm, wc[w]); sd += wd[w]; }
    if (a.aux_loss) *a.aux_loss = a.alpha * (float)a.E * sf;
    if (a.imbalance) *a.imbalance = a.T > 0 ? (float)cm / (A / (float)a.E) : 0.0f;
    if (a.dropped) *a.dropped = sd;
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int ntiles = ceil_div(a.T, kPermuteTile);
  if (ntiles == 1) {
    hipLaunchKernelGGL(permute_one_tile_kernel, dim3(1), dim3(kPermuteTile), 0, s, a);
    return hipGetLastError();
  }
  if (ntiles > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(ntiles), dim3(kPermuteTile), 0, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // one thread per expert (a power of two, at least a wave): the scans take
  // log2(threads) steps
  int threads = 64;
  while (threads < a.E) threads <<= 1;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(threads), 0, s, a, ntiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || ntiles == 0) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(ntiles), dim3(kPermuteTile), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* token_of_row, const int32_t*, int,
                              int rows_cap, int D, int elem_bytes, void* x_perm, hipStream_t s) {
  if (rows_cap == 0) return hipSuccess;
  const int chunks = D * elem_bytes / 16;
  const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(rows_cap), dim3(threads), 0, s,
                     static_cast<const uint4*>(x), token_of_row, static_cast<uint4*>(x_perm), chunks);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_combine_t(const void* y_perm, const int32_t* row_of, const float* topk_w, const void* y_shared,
                            void* y, int ntok, int k, int D, hipStream_t s) {
  const int chunks = D / Chunk<E>::N;
  const int G = k >= 5 ? 8 : k >= 3 ? 4 : k;   // rows loaded together per item
  const int U = G >= 4 ? 8 / G : 4 / G;
  // tokens per workgroup: enough items for every thread's U, within the LDS slots
  int tpb = (256 * U + chunks - 1) / chunks;
  tpb = std::max(1, std::min(tpb, kCombineSlots / k));
  // few tokens with long rows (decode-sized batches): a token's chunks are
  // spread over several workgroups of one pass each, instead of one
  // workgroup taking several dependent passes
  int cseg = chunks;
  if (tpb == 1 && ntok < 1024) cseg = 256 * U;
  const dim3 grid((unsigned)ceil_div(ntok, tpb), (unsigned)ceil_div(chunks, cseg));
  const E* yp = static_cast<const E*>(y_perm);
  const E* ys = static_cast<const E*>(y_shared);
  E* yo = static_cast<E*>(y);
  switch (G) {
    case 1: hipLaunchKernelGGL((combine_kernel<E, 1>), grid, dim3(256), 0, s, yp, row_of, topk_w, ys, yo, ntok, k, D, tpb, cseg); break;
    case 2: hipLaunchKernelGGL((combine_kernel<E, 2>), grid, dim3(256), 0, s, yp, row_of, topk_w, ys, yo, ntok, k, D, tpb, cseg); break;
    case 4: hipLaunchKernelGGL((combine_kernel<E, 4>), grid, dim3(256), 0, s, yp, row_of, topk_w, ys, yo, ntok, k, D, tpb, cseg); break;
    default: hipLaunchKernelGGL((combine_kernel<E, 8>), grid, dim3(256), 0, s, yp, row_of, topk_w, ys, yo, ntok, k, D, tpb, cseg); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* y_perm, const int32_t* row_of, const float* topk_w,
                          const void* y_shared, void* y, int T, int k, int D, int act_dtype,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (act_dtype == BF16) return launch_combine_t<bf16_t>(y_perm, row_of, topk_w, y_shared, y, T, k, D, s);
  return launch_combine_t<float>(y_perm, row_of, topk_w, y_shared, y, T, k, D, s);
}

hipError_t launch_load_stats(const StatsArgs& a, hipStream_t s) {
  const int nchunks = ceil_div(a.T, kStatsChunk);
  if (nchunks > 0) {
    hipLaunchKernelGGL(stats_partial_kernel, dim3(nchunks, ceil_div(a.E, 64)), dim3(256), 0, s, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  int tpe = 1;                          // threads per expert: largest power of two <= 64 with E * tpe <= 1024
  while (tpe < 64 && a.E * tpe * 2 <= kMaxExperts) tpe *= 2;
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kMaxExperts), 0, s, a, nchunks, tpe);
  return hipGetLastError();
}

}  // namespace moe
