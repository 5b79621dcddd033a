// Sequential merge of per-segment results into true segment start states.
//
// The end state of a segment is affine in its start state, S_end = M S_start +
// S_zero_end, and one exchange of (S_zero_end, M) among the segments recovers
// every segment's exact start state ("Kimi K3 开源日来了", section
// "针对适配的 Infra", KDA context parallelism).  Per (b, h):
//     S = S_in;  for i in 0..G-1:  S_start[i] = S;  S = M[i] S + S_zero_end[i];
//     S_T = S.
// Workgroup = one head and 16 state columns; 256 threads, thread t computes
// row t/2 and columns (t%2)*8..+7 of the slice (threads with t/2 >= D idle).
// The slice of S lives in LDS; M rows stream from L2.  fp32 VALU: the merge is
// a few GFLOP in total and not worth matrix cores.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
// S_T may alias S_in: a workgroup reads its slice of S_in before any write.
__global__ __launch_bounds__(256) void kda_merge_kernel(const float* S_in, const float* __restrict__ Z,
                                                        const float* __restrict__ M,
                                                        float* __restrict__ S_start, float* S_T,
                                                        int BH, int G) {
  __shared__ float s[D][16];
  const int bh = blockIdx.x / (D / 16);
  const int c0 = (blockIdx.x % (D / 16)) * 16;
  const int t = threadIdx.x;
  const int r = t >> 1, cb = (t & 1) * 8;
  const bool active = r < D;
  const size_t hs = (size_t)bh * D * D;
  if (active) {
#pragma unroll
    for (int c = 0; c < 8; ++c) s[r][cb + c] = S_in ? S_in[hs + (size_t)r * D + c0 + cb + c] : 0.f;
  }
  __syncthreads();
  for (int i = 0; i < G; ++i) {
    const size_t gs = ((size_t)i * BH + bh) * D * D;
    float acc[8];
    if (active) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        acc[c] = Z[gs + (size_t)r * D + c0 + cb + c];
        if (S_start) S_start[gs + (size_t)r * D + c0 + cb + c] = s[r][cb + c];
      }
      const float* Mr = M + gs + (size_t)r * D;
      for (int m = 0; m < D; m += 4) {
        const f32x4 mv = *reinterpret_cast<const f32x4*>(Mr + m);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[c] += mv[e] * s[m + e][cb + c];
        }
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s[r][cb + c] = acc[c];
    }
    __syncthreads();
  }
  if (active) {
#pragma unroll
    for (int c = 0; c < 8; ++c) S_T[hs + (size_t)r * D + c0 + cb + c] = s[r][cb + c];
  }
}

hipError_t launch_merge(const float* S_in, const float* Z, const float* M, float* S_start,
                        float* S_T, int BH, int G, int D, hipStream_t stream) {
  if (BH <= 0) return hipSuccess;
  const int nwg = BH * (D / 16);
  if (D == 128)
    hipLaunchKernelGGL((kda_merge_kernel<128>), dim3(nwg), dim3(256), 0, stream, S_in, Z, M, S_start, S_T, BH, G);
  else if (D == 64)
    hipLaunchKernelGGL((kda_merge_kernel<64>), dim3(nwg), dim3(256), 0, stream, S_in, Z, M, S_start, S_T, BH, G);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kda
