// One KDA decode step per (sequence, head), in place on the fp32 state.
//
// The per-request KDA state is fixed-size, so decoding a token touches only
// that state ("Kimi K3 开源日来了", section "针对适配的 Infra").  For one head with
// state S (D x D), gate a = exp(log_alpha), key k, query q, value v, scalar b:
//     D' = Diag(a) S,  u = D'^T k,  w = D'^T q,  delta = b (v - u),
//     S  = D' + k delta^T,  o = S^T q = w + (k.q) delta.
// This is one token of the recurrence S = (I - b k k^T) Diag(a) S + b k v^T,
// o = S^T q, rearranged so that S is read once and written once.
//
// Workgroup = one head, 256 threads.  Thread t owns columns 4*(t%32)..+3 of
// rows t/32 + 8*i (i = 0..D/8-1): every row is read as 32 coalesced 16-byte
// pieces, and the state slice stays in registers between the read and the
// write.  The column reductions over rows finish with a lane shuffle (the two
// row groups of a wave) and an LDS pass over the four waves.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename T, int D>
__global__ __launch_bounds__(256) void kda_decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const T* __restrict__ v, const T* __restrict__ la,
                                                         const T* __restrict__ beta, float* __restrict__ S,
                                                         T* __restrict__ o) {
  constexpr int RPT = D / 8;  // rows per thread
  __shared__ float s_a[D], s_ak[D], s_aq[D];
  __shared__ float s_red[4][2][D];
  __shared__ float s_kq[4];
  const int head = blockIdx.x;
  const int t = threadIdx.x;
  const int cg = t & 31, rg = t >> 5;
  const int wave = t >> 6, lane = t & 63;
  float* Sh = S + (size_t)head * D * D;

  f32x4 st[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    st[i] = (4 * cg < D) ? *reinterpret_cast<const f32x4*>(Sh + (size_t)(rg + 8 * i) * D + 4 * cg) : zero4();

  float kq = 0.f;
  if (t < D) {
    const float kt = to_f32(k[(size_t)head * D + t]);
    const float qt = to_f32(q[(size_t)head * D + t]);
    const float at = expf(to_f32(la[(size_t)head * D + t]));
    s_a[t] = at;
    s_ak[t] = at * kt;
    s_aq[t] = at * qt;
    kq = kt * qt;
  }
  // k.q over the D channels (threads 0..D-1 hold one product each)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
  if (lane == 0) s_kq[wave] = kq;
  __syncthreads();

  float u[4] = {0.f, 0.f, 0.f, 0.f}, w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + 8 * i;
    const float ak = s_ak[r], aq = s_aq[r];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u[c] += ak * st[i][c];
      w[c] += aq * st[i][c];
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u[c] += __shfl_xor(u[c], 32);
    w[c] += __shfl_xor(w[c], 32);
  }
  if (lane < 32 && 4 * cg < D) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s_red[wave][0][4 * cg + c] = u[c];
      s_red[wave][1][4 * cg + c] = w[c];
    }
  }
  __syncthreads();
  if (4 * cg >= D) return;
  const float b = to_f32(beta[head]);
  const float kqs = s_kq[0] + s_kq[1] + s_kq[2] + s_kq[3];
  float dl[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = 4 * cg + c;
    const float uu = s_red[0][0][j] + s_red[1][0][j] + s_red[2][0][j] + s_red[3][0][j];
    dl[c] = b * (to_f32(v[(size_t)head * D + j]) - uu);
  }
  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 4 * cg + c;
      const float ww = s_red[0][1][j] + s_red[1][1][j] + s_red[2][1][j] + s_red[3][1][j];
      o[(size_t)head * D + j] = from_f32<T>(ww + kqs * dl[c]);
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + 8 * i;
    const float ar = s_a[r];
    const float kr = to_f32(k[(size_t)head * D + r]);
    f32x4 x;
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = ar * st[i][c] + kr * dl[c];
    *reinterpret_cast<f32x4*>(Sh + (size_t)r * D + 4 * cg) = x;
  }
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* la,
                         const void* beta, float* S, void* o, int NH, int D, bool bf16_io,
                         hipStream_t stream) {
  if (NH <= 0) return hipSuccess;
#define KDA_DECODE(TY, DD)                                                                        \
  hipLaunchKernelGGL((kda_decode_kernel<TY, DD>), dim3(NH), dim3(256), 0, stream,                \
                     (const TY*)q, (const TY*)k, (const TY*)v, (const TY*)la, (const TY*)beta, S, \
                     (TY*)o)
  if (bf16_io) {
    if (D == 128) KDA_DECODE(bf16, 128);
    else if (D == 64) KDA_DECODE(bf16, 64);
    else return hipErrorInvalidValue;
  } else {
    if (D == 128) KDA_DECODE(float, 128);
    else if (D == 64) KDA_DECODE(float, 64);
    else return hipErrorInvalidValue;
  }
#undef KDA_DECODE
  return hipGetLastError();
}

}  // namespace kda
