// KDA prefill gradients per head, token by token.
//
// For a loss L with dL/do_t = dO_t and dL/dS_T = dS_T, the gradients of the
// recurrence (blog.csdn.net article on the Kimi K3 report, section 一.1; the
// update itself is the gated delta rule taken for it)
//     D = Diag(a_t) S_{t-1},  u = D^T k_t,  delta = b_t (v_t - u),
//     S_t = D + k_t delta^T,  o_t = S_t^T q_t,          a_t = exp(log_alpha_t)
// follow by running the same steps backwards with the chain rule (training is
// what the K3 report also speeds up with FlashKDA: "Kimi K3 开源日来了", section
// "FlashKDA"):
//     dq_t = S_t dO_t;  dS += q_t dO_t^T
//     dk_t = dS delta + D du;  d_delta = dS^T k_t
//     dbeta_t = d_delta . (v_t - u);  dv_t = b_t d_delta;  du = -b_t d_delta
//     dS += k_t du^T;  dlog_alpha_t = rowsum(D * dS);  dS = Diag(a_t) dS
// and dS0 is the dS left after token 0.
//
// The backward walk needs the state before every token, newest first.  The
// kernel runs the forward recurrence once, keeping the state at the start of
// every 64-token interval in the workspace; then, interval by interval from the
// last, it runs the interval forward again from its checkpoint, keeping each
// token's entering state in the workspace, and walks those tokens backwards.
//
// One workgroup of 4 D threads per head.
//  - Forward passes: thread tid owns column tid / 4 of the state, a quarter of
//    its rows, so u = D^T k is a sum inside the thread and its 3 neighbours.
//    The states go to the workspace row-major; the interval's pass also keeps
//    each token's u for the backward walk.
//  - Backward walk: thread tid owns row i = tid / 4 of the state and of dS,
//    columns [c0, c0 + D/4) with c0 = (tid % 4) D/4.  Sums over a row (dq, dk,
//    dlog_alpha) stay in the thread and its 3 neighbours; the sum over the
//    rows d_delta = dS^T k goes through an LDS transpose (every thread stores
//    its row piece, then adds a quarter column).
//  - The per-token vectors pass through LDS, double-buffered, and the next
//    token's are fetched into registers while the current one runs.
// Every step is evaluated in fp32 on inputs read as fp32.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

template <int D>
struct BwLayout {
  static constexpr int TPR = 4;                // threads per state row
  static constexpr int THREADS = TPR * D;      // one thread per (row, column quarter)
  static constexpr int NW = THREADS / 64;      // waves
  static constexpr int CPT = D / TPR;          // columns per thread
  static_assert(THREADS % 64 == 0 && CPT % 4 == 0, "layout");
};

// Sum of x over the TPR adjacent lanes that share a state row.
template <int D>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int m = 1; m < BwLayout<D>::TPR; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Column sums over all D rows of the workgroup's state layout, into tot[D].
// Every thread first stores its contributions for row i, columns [c0, c0 + CPT)
// into the LDS matrix P (row pitch D + 4 floats) as 16-byte stores (put4).
// col_sum then, after a barrier, has thread tid add a quarter of column
// tid % D (rows (tid / D) D/4 ..); the four quarters meet in quar[4][D], and
// D threads add them into tot.  tot is readable when col_sum returns.
template <int D>
__device__ __forceinline__ void put4(float* P, int i, int col, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<f32x4*>(P + i * (D + 4) + col) = f32x4{x0, x1, x2, x3};
}

template <int D>
__device__ __forceinline__ void col_sum(const float* P, float (*quar)[D], float* tot, int tid) {
  static_assert(BwLayout<D>::THREADS == 4 * D, "one quarter column per thread");
  constexpr int PITCH = D + 4;
  __syncthreads();
  const int j = tid % D, r = tid / D;
  float s = 0.f;
#pragma unroll 8
  for (int rr = 0; rr < D / 4; ++rr) s += P[(r * (D / 4) + rr) * PITCH + j];
  quar[r][j] = s;
  __syncthreads();
  if (tid < D) tot[tid] = (quar[0][tid] + quar[1][tid]) + (quar[2][tid] + quar[3][tid]);
  __syncthreads();
}

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(4 * D, 1) void kda_backward_kernel(BackwardArgs a) {
  using L = BwLayout<D>;
  constexpr int CPT = L::CPT;
  constexpr int NS = D * D;
  // per-token vectors, double-buffered: consecutive commits alternate buffers,
  // so a token's vectors land while the previous token may still be read
  __shared__ float s_k[2][D], s_a[2][D], s_v[2][D], s_q[2][D], s_do[2][D], s_u[2][D];
  __shared__ float s_b[2];
  __shared__ __attribute__((aligned(16))) float s_P[D * (D + 4)];
  __shared__ float quar[4][D];
  __shared__ float s_dd[D];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int i = tid / L::TPR;
  const int part = tid % L::TPR;
  const int c0 = part * CPT;
  const int nt = a.T;
  const int nch = (nt + kBwInterval - 1) / kBwInterval;

  const size_t tok0 = (size_t)bh * nt;
  const T* q = static_cast<const T*>(a.q) + tok0 * D;
  const T* k = static_cast<const T*>(a.k) + tok0 * D;
  const T* v = static_cast<const T*>(a.v) + tok0 * D;
  const T* la = static_cast<const T*>(a.la) + tok0 * D;
  const T* beta = static_cast<const T*>(a.beta) + tok0;
  const T* dO = a.dO ? static_cast<const T*>(a.dO) + tok0 * D : nullptr;
  float* ckpt = a.ws + (size_t)bh * ((size_t)(nch + kBwInterval) * NS + (size_t)kBwInterval * D);
  float* hist = ckpt + (size_t)nch * NS;
  float* hu = hist + (size_t)kBwInterval * NS;  // u of each token of the interval
  const size_t my = (size_t)i * D + c0;  // this thread's first state entry

  // Token vectors: threads < D fetch one channel of the next token into
  // registers while the current token is processed (fetch), and move them to
  // LDS when that token starts (commit, then a barrier).  with_q also takes q,
  // dO and the token's u (kept by the interval's forward pass at hu[tl]) for
  // the backward step.
  float nk = 0.f, nla = 0.f, nv = 0.f, nq = 0.f, ndo = 0.f, nu = 0.f, nb = 0.f;
  auto fetch = [&](int t, bool with_q, int tl = 0) {
    if (tid < D) {
      const size_t o = (size_t)t * D + tid;
      nk = to_f32(k[o]);
      nla = to_f32(la[o]);
      nv = to_f32(v[o]);
      if (with_q) {
        nq = to_f32(q[o]);
        ndo = dO ? to_f32(dO[o]) : 0.f;
        nu = hu[(size_t)tl * D + tid];
      }
    }
    if (tid == 0) nb = to_f32(beta[t]);
  };
  // Returns the buffer the token's vectors are in.  Its barrier also orders
  // every LDS access of the tokens before it against the ones after it.
  int ncommit = 0;
  auto commit = [&](bool with_q) {
    const int cb = ncommit & 1;
    ++ncommit;
    if (tid < D) {
      s_k[cb][tid] = nk;
      s_a[cb][tid] = expf(nla);
      s_v[cb][tid] = nv;
      if (with_q) {
        s_q[cb][tid] = nq;
        s_do[cb][tid] = ndo;
        s_u[cb][tid] = nu;
      }
    }
    if (tid == 0) s_b[cb] = nb;
    __syncthreads();
    return cb;
  };

  // Forward passes in the column layout: thread tid owns column jc = tid / 4,
  // rows [r0, r0 + D/4) with r0 = (tid % 4) D/4, so u_j = sum_i k_i D[i][j] is a
  // sum inside the thread and over the 4 adjacent lanes of the column.  The
  // states go to the workspace row-major, where the backward walk (row layout)
  // reads them after a barrier.
  const int jc = tid >> 2;
  const int r0 = (tid & 3) * (D / 4);
  float Sc[CPT];
  auto store_col = [&](float* dst) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) dst[(size_t)(r0 + m) * D + jc] = Sc[m];
  };
  // one forward token; `next` (or -1) is the token whose vectors to fetch
  // meanwhile; with keep >= 0 the token's u goes to hu[keep]
  auto forward = [&](int next, int keep) {
    const int cb = commit(false);
    if (next >= 0) fetch(next, false);
    float u = 0.f;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      Sc[m] *= s_a[cb][r0 + m];
      u += s_k[cb][r0 + m] * Sc[m];
    }
    u += __shfl_xor(u, 1);
    u += __shfl_xor(u, 2);
    if (keep >= 0 && (tid & 3) == 0) hu[(size_t)keep * D + jc] = u;
    const float w = s_b[cb] * (s_v[cb][jc] - u);
#pragma unroll
    for (int m = 0; m < CPT; ++m) Sc[m] += s_k[cb][r0 + m] * w;
  };

#pragma unroll
  for (int m = 0; m < CPT; ++m) Sc[m] = a.S0 ? a.S0[(size_t)bh * NS + (size_t)(r0 + m) * D + jc] : 0.f;
  if (nt > 0) fetch(0, false);
  for (int t = 0; t < nt; ++t) {
    if (t % kBwInterval == 0) store_col(ckpt + (size_t)(t / kBwInterval) * NS);
    forward(t + 1 < nt ? t + 1 : -1, -1);
  }

  float S[CPT];
  float dS[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) dS[c] = a.dS_T ? a.dS_T[(size_t)bh * NS + my + c] : 0.f;

  for (int ch = nch - 1; ch >= 0; --ch) {
    const int t0 = ch * kBwInterval;
    const int t1 = min(t0 + kBwInterval, nt);
#pragma unroll
    for (int m = 0; m < CPT; ++m) Sc[m] = ckpt[(size_t)ch * NS + (size_t)(r0 + m) * D + jc];
    fetch(t0, false);
    for (int t = t0; t < t1; ++t) {
      store_col(hist + (size_t)(t - t0) * NS);
      forward(t + 1 < t1 ? t + 1 : -1, t - t0);
    }
    // the last token's u (written after its barrier) and every stored state
    // are read below by other threads
    __syncthreads();
    // the entering state of the next token to walk is read one token ahead
    float Sn[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) Sn[c] = hist[(size_t)(t1 - 1 - t0) * NS + my + c];
    fetch(t1 - 1, true, t1 - 1 - t0);
    for (int t = t1 - 1; t >= t0; --t) {
      const int cb = commit(true);
      if (t > t0) fetch(t - 1, true, t - 1 - t0);
      const float ai = s_a[cb][i], ki = s_k[cb][i], qi = s_q[cb][i], b = s_b[cb];
      // D = Diag(a) S_{t-1} (in S); u = D^T k came with the token's vectors
#pragma unroll
      for (int c = 0; c < CPT; ++c) S[c] = ai * Sn[c];
      if (t > t0) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) Sn[c] = hist[(size_t)(t - 1 - t0) * NS + my + c];
      }
      // dq = S_t dO with S_t = D + k delta^T; dS += q dO^T; dk (first part) = dS delta
      float dq = 0.f, dk = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const float del = b * (s_v[cb][c0 + c] - s_u[cb][c0 + c]);
        const float d_o = s_do[cb][c0 + c];
        dq += (S[c] + ki * del) * d_o;
        dS[c] += qi * d_o;
        dk += dS[c] * del;
      }
#pragma unroll
      for (int c = 0; c < CPT; c += 4)
        put4<D>(s_P, i, c0 + c, ki * dS[c], ki * dS[c + 1], ki * dS[c + 2], ki * dS[c + 3]);
      // d_delta = dS^T k
      col_sum<D>(s_P, quar, s_dd, tid);
      float db = 0.f, dla = 0.f;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const float dd = s_dd[c0 + c];
        db += dd * (s_v[cb][c0 + c] - s_u[cb][c0 + c]);
        const float du = -b * dd;
        dk += S[c] * du;
        dS[c] += ki * du;
        dla += S[c] * dS[c];
        dS[c] *= ai;
      }
      dq = row_sum<D>(dq);
      dk = row_sum<D>(dk);
      dla = row_sum<D>(dla);
      db = row_sum<D>(db);
      const size_t o = (tok0 + t) * D;
      if (part == 0) {
        a.dq[o + i] = dq;
        a.dk[o + i] = dk;
        a.dla[o + i] = dla;
      }
      if (tid < L::TPR) {  // the threads of row 0 hold d_delta for all columns
#pragma unroll
        for (int c = 0; c < CPT; ++c) a.dv[o + c0 + c] = b * s_dd[c0 + c];
        if (tid == 0) a.dbeta[tok0 + t] = db;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) a.dS0[(size_t)bh * NS + my + c] = dS[c];
}

hipError_t launch_backward(const BackwardArgs& a, int BH, int D, bool bf16_io, hipStream_t stream) {
  if (BH <= 0) return hipSuccess;
#define KDA_BW(TY, DD) \
  hipLaunchKernelGGL((kda_backward_kernel<TY, DD>), dim3(BH), dim3(4 * DD), 0, stream, a)
  if (bf16_io) {
    if (D == 128) KDA_BW(bf16, 128);
    else KDA_BW(bf16, 64);
  } else {
    if (D == 128) KDA_BW(float, 128);
    else KDA_BW(float, 64);
  }
#undef KDA_BW
  return hipGetLastError();
}

}  // namespace kda
