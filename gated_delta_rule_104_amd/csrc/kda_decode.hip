// KDA decode per (sequence, head): one token in place on the fp32 state, or a
// few consecutive tokens (speculative decoding's draft tokens) in one pass.
//
// The per-request KDA state is fixed-size, so decoding a token touches only
// that state ("Kimi K3 开源日来了", section "针对适配的 Infra").  For one head with
// state S (D x D), gate a = exp(log_alpha), key k, query q, value v, scalar b:
//     D' = Diag(a) S,  u = D'^T k,  w = D'^T q,  delta = b (v - u),
//     S  = D' + k delta^T,  o = S^T q = w + (k.q) delta.
// This is one token of the recurrence S = (I - b k k^T) Diag(a) S + b k v^T,
// o = S^T q, rearranged so that S is read once and written once.
//
// Workgroup = one head, four waves; wave w owns the D/4 columns
// [w*D/4, (w+1)*D/4) and all D rows of them, so every reduction over rows
// stays inside the wave (lane shuffles) and the waves never wait for each
// other.  Lane l covers 4 columns (l % LPR) of RPL consecutive rows; a row
// slice of the wave is LPR lanes x 16 bytes, so each load instruction reads
// whole 128-byte (D = 128) or 64-byte (D = 64) row pieces.  The gate, key and
// query vectors pass through a per-wave LDS area so that each lane reads its
// rows' values as vectors.  The state is streamed with non-temporal accesses:
// it is touched once per step and is larger than the caches.
//
// Several tokens per call serve speculative decoding, for which the K3 report
// fine-tunes a draft model (blog.csdn.net article on the Kimi K3 report,
// section 二, deployment-aware training): the draft tokens are checked in one
// pass that reads the state once, applies the tokens in registers and writes
// it once, optionally storing the state after each token so that the caller can
// roll back to the last accepted one.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename T>
__device__ __forceinline__ float ld1(const T* p) {
  return to_f32(*p);
}

// ntok consecutive tokens per head: inputs [NH, ntok, D] (beta [NH, ntok]),
// outputs o [NH, ntok, D].  The state is read from S_in once, kept in registers
// across the tokens, and written to S_out once (S_out may alias S_in: every
// lane reads all of its entries before it writes any).  S_pos, when given,
// receives the state after each token at [n, t, h] of [N, ntok, H, D, D].
//
// ONE: the single-token step in place (S_in == S_out, no S_pos), compiled as
// its own kernel so that the hot decode loop keeps its one-pass shape.
template <typename T, int D, bool ONE>
__global__ __launch_bounds__(256) void kda_decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const T* __restrict__ v, const T* __restrict__ la,
                                                         const T* __restrict__ beta, const float* S_in,
                                                         float* S_out, T* __restrict__ o,
                                                         float* __restrict__ S_pos, int ntok_, int H) {
  const int ntok = ONE ? 1 : ntok_;
  constexpr int CPW = D / 4;       // columns per wave
  constexpr int LPR = CPW / 4;     // lanes per row slice (4 columns each)
  constexpr int RG = 64 / LPR;     // row groups per wave
  constexpr int RPL = D / RG;      // consecutive rows per lane
  static_assert(RPL % 4 == 0, "row vectors");
  // per wave: a, a*k, a*q, k for all D channels
  __shared__ __attribute__((aligned(16))) float s_v[4][4][D];
  const int head = blockIdx.x;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int cl = l % LPR, rg = l / LPR;
  const int c0 = wave * CPW + 4 * cl;  // first of the lane's 4 columns
  const int r0 = rg * RPL;             // first of the lane's rows
  const size_t hs = (size_t)head * D * D;

  f32x4 st[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i)
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S_in + hs + (size_t)(r0 + i) * D + c0));

  float* sa = s_v[wave][0];
  float* sak = s_v[wave][1];
  float* saq = s_v[wave][2];
  float* sk = s_v[wave][3];
  // One token's inputs for this lane: its D/64 gate, key and query channels,
  // its four value columns and beta.  With several tokens, token t + 1's are
  // loaded while token t is applied, so only the first token's load latency is
  // exposed (and that one overlaps the state load).
  struct Tok {
    float k[D / 64], q[D / 64], la[D / 64], v[4], b;
  };
  auto load_tok = [&](int t, Tok& x) {
    const size_t tb = ((size_t)head * ntok + t) * D;
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) {
      x.k[jj] = ld1(k + tb + l + 64 * jj);
      x.q[jj] = ld1(q + tb + l + 64 * jj);
      x.la[jj] = ld1(la + tb + l + 64 * jj);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) x.v[c] = ld1(v + tb + c0 + c);
    x.b = ld1(beta + (size_t)head * ntok + t);
  };
  Tok cur;
  if (ntok > 0) load_tok(0, cur);
  for (int t = 0; t < ntok; ++t) {
    const size_t tb = ((size_t)head * ntok + t) * D;  // row of token t
    const bool more = !ONE && t + 1 < ntok;
    Tok nxt;
    if (more) load_tok(t + 1, nxt);
    // gate, key and query: the wave's lanes cover the D channels
    float kq = 0.f;
#pragma unroll
    for (int jj = 0; jj < D / 64; ++jj) {
      const int j = l + 64 * jj;
      const float kt = cur.k[jj], qt = cur.q[jj];
      const float at = expf(cur.la[jj]);
      sa[j] = at;
      sak[j] = at * kt;
      saq[j] = at * qt;
      sk[j] = kt;
      kq += kt * qt;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
    wave_lds_fence();  // this wave's LDS writes before its reads

    float u[4] = {0.f, 0.f, 0.f, 0.f}, w[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i4 = 0; i4 < RPL; i4 += 4) {
      const f32x4 ak = *reinterpret_cast<const f32x4*>(sak + r0 + i4);
      const f32x4 aq = *reinterpret_cast<const f32x4*>(saq + r0 + i4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u[c] += ak[e] * st[i4 + e][c];
          w[c] += aq[e] * st[i4 + e][c];
        }
    }
    // sum over the row groups (lanes with the same column group)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u[c] += __shfl_xor(u[c], off);
        w[c] += __shfl_xor(w[c], off);
      }
    float dl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) dl[c] = cur.b * (cur.v[c] - u[c]);
    if (rg == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[tb + c0 + c] = from_f32<T>(w[c] + kq * dl[c]);
    }
#pragma unroll
    for (int i4 = 0; i4 < RPL; i4 += 4) {
      const f32x4 ar = *reinterpret_cast<const f32x4*>(sa + r0 + i4);
      const f32x4 kr = *reinterpret_cast<const f32x4*>(sk + r0 + i4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int c = 0; c < 4; ++c) st[i4 + e][c] = ar[e] * st[i4 + e][c] + kr[e] * dl[c];
    }
    if (!ONE && S_pos) {
      const int n = head / H, h = head - n * H;
      float* dst = S_pos + (((size_t)n * ntok + t) * H + h) * D * D;
#pragma unroll
      for (int i = 0; i < RPL; ++i)
        __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4*>(dst + (size_t)(r0 + i) * D + c0));
    }
    if (more) cur = nxt;
  }
#pragma unroll
  for (int i = 0; i < RPL; ++i)
    __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4*>(S_out + hs + (size_t)(r0 + i) * D + c0));
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* la,
                         const void* beta, const float* S_in, float* S_out, void* o, float* S_pos,
                         int NH, int H, int ntok, int D, bool bf16_io, hipStream_t stream) {
  if (NH <= 0) return hipSuccess;
  const bool one = ntok == 1 && S_in == S_out && !S_pos;
#define KDA_DECODE(TY, DD)                                                                          \
  do {                                                                                              \
    if (one)                                                                                        \
      hipLaunchKernelGGL((kda_decode_kernel<TY, DD, true>), dim3(NH), dim3(256), 0, stream,        \
                         (const TY*)q, (const TY*)k, (const TY*)v, (const TY*)la, (const TY*)beta,  \
                         S_in, S_out, (TY*)o, nullptr, 1, H);                                       \
    else                                                                                            \
      hipLaunchKernelGGL((kda_decode_kernel<TY, DD, false>), dim3(NH), dim3(256), 0, stream,       \
                         (const TY*)q, (const TY*)k, (const TY*)v, (const TY*)la, (const TY*)beta,  \
                         S_in, S_out, (TY*)o, S_pos, ntok, H);                                      \
  } while (0)
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
