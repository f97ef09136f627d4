// Expert-parallel layouts: the part of the two all-to-all exchanges of an
// expert-parallel layer that one GPU holds ("Top-k 路由" page, 通訊拓撲：
// All-to-All figure; "别只比较 Top-k" page, two-All-to-All dispatcher and
// 按目标专家发送 sections).  Experts sit on ranks in contiguous blocks of
// E / R.
//   send:    the permuted rows are expert-major, so the rows bound for rank r
//            are one contiguous run: offsets[r E/R] .. offsets[(r+1) E/R];
//   receive: the all-to-all delivers the sources one after another, each
//            source's rows expert after expert; the local grouped FFN wants
//            them expert after expert (sources in rank order inside an
//            expert).  gather[j] gives the received position of expert-major
//            row j, which the grouped GEMM reads in place (no copy).
// Integer work only; exact and deterministic.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void ep_send_layout_kernel(const int32_t* __restrict__ offsets, int E, int R,
                                                             int32_t* __restrict__ send_counts,
                                                             int32_t* __restrict__ send_offsets) {
  const int per = E / R;
  for (int r = threadIdx.x; r <= R; r += blockDim.x) {
    const int lo = offsets[r * per];               // r == R: offsets[E]
    send_offsets[r] = lo;
    if (r < R) send_counts[r] = offsets[(r + 1) * per] - lo;
  }
}

__device__ __forceinline__ int block_sum_256(int v, int* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int d = 128; d >= 1; d >>= 1) {
    if ((int)threadIdx.x < d) red[threadIdx.x] += red[threadIdx.x + d];
    __syncthreads();
  }
  const int s = red[0];
  __syncthreads();
  return s;
}

// Block b = (source r, local expert e), b = r * El + e: the received run of
// (r, e) starts at the sum of the counts before it in (source, expert) order;
// its expert-major run starts after every row of experts below e and the rows
// of e from sources below r.  Block 0 also writes local_offsets and marks the
// gather entries past the received total with -1.  Rows at or past rows_cap
// are not written (local_offsets are clamped to rows_cap).
__global__ __launch_bounds__(256) void ep_recv_layout_kernel(const int32_t* __restrict__ rc, int R, int El,
                                                             int rows_cap, int32_t* __restrict__ local_offsets,
                                                             int32_t* __restrict__ gather) {
  __shared__ int red[256];
  const int b = blockIdx.x;
  const int r = b / El, e = b % El;
  int s_src = 0, s_dst = 0;
  for (int i = threadIdx.x; i < R * El; i += blockDim.x) {
    const int c = rc[i];
    const int ri = i / El, ei = i % El;
    if (i < b) s_src += c;
    if (ei < e || (ei == e && ri < r)) s_dst += c;
  }
  s_src = block_sum_256(s_src, red);
  s_dst = block_sum_256(s_dst, red);
  const int n = rc[b];
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (s_dst + i < rows_cap) gather[s_dst + i] = s_src + i;
  if (b != 0) return;
  int total = 0;
  for (int i = threadIdx.x; i < R * El; i += blockDim.x) total += rc[i];
  total = block_sum_256(total, red);
  for (int ex = threadIdx.x; ex <= El; ex += blockDim.x) {
    int o = 0;
    for (int i = 0; i < R * El; ++i)
      if (i % El < ex) o += rc[i];
    local_offsets[ex] = min(o, rows_cap);
  }
  for (int j = total + threadIdx.x; j < rows_cap; j += blockDim.x) gather[j] = -1;
}

}  // namespace

hipError_t launch_ep_send_layout(const int32_t* offsets, int E, int R, int32_t* send_counts, int32_t* send_offsets,
                                 hipStream_t s) {
  hipLaunchKernelGGL(ep_send_layout_kernel, dim3(1), dim3(256), 0, s, offsets, E, R, send_counts, send_offsets);
  return hipGetLastError();
}

hipError_t launch_ep_recv_layout(const int32_t* recv_counts, int R, int El, int rows_cap, int32_t* local_offsets,
                                 int32_t* gather, hipStream_t s) {
  hipLaunchKernelGGL(ep_recv_layout_kernel, dim3(R * El), dim3(256), 0, s, recv_counts, R, El, rows_cap,
                     local_offsets, gather);
  return hipGetLastError();
}

}  // namespace moe
