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
// SPLIT workgroups per head (2 when that still fits the chip in one round),
// each owning DC = D / SPLIT of the state's columns: the forward recurrence and
// d_delta are column by column, so only the row sums (dq, dk, dlog_alpha,
// dbeta) need the other workgroup's half; with SPLIT = 2 each half goes to the
// workspace and a second kernel adds them.  A workgroup has 4 DC threads.
//  - Forward passes: thread tid owns column tid / 4 of its slice, a quarter of
//    the rows, so u = D^T k is a sum inside the thread and its 3 neighbours.
//    The states go to the workspace row-major; the interval's pass also keeps
//    each token's u for the backward walk.
//  - Backward walk: thread tid owns row i = tid / TPR of the slice of the
//    state and of dS, D/4 columns from c0 = (tid % TPR) D/4 (TPR = 4 / SPLIT).
//    Sums over a row (dq, dk, dlog_alpha) stay in the thread and its TPR - 1
//    neighbours; the sum over the rows d_delta = dS^T k goes through an LDS
//    transpose (every thread stores its row piece, then adds a quarter column).
//  - The per-token vectors pass through LDS, double-buffered, and the next
//    token's are fetched into registers while the current one runs.
// Every step is evaluated in fp32 on inputs read as fp32.
#include <algorithm>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

template <int D, int SPLIT>
struct BwLayout {
  static constexpr int DC = D / SPLIT;      // state columns per workgroup
  static constexpr int THREADS = 4 * DC;    // forward: one thread per (column, row quarter)
  static constexpr int TPR = THREADS / D;   // backward: threads per state row
  static constexpr int CPT = DC / TPR;      // backward: columns per thread (D / 4)
  static constexpr int RPT = D / 4;         // forward: rows per thread
  static_assert(THREADS % 64 == 0 && THREADS >= D && TPR >= 1 && CPT % 4 == 0, "layout");
};

// Sum of x over the TPR adjacent lanes that share a state row.
template <int TPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Column sums over all D rows of a workgroup's state slice, into tot[DC].
// Every thread first stores its contributions for row i (CPT columns from c0)
// into the LDS matrix P (row pitch DC + 4 floats) as 16-byte stores (put4).
// col_sum then, after a barrier, has thread tid add a quarter of column
// tid % DC (rows (tid / DC) D/4 ..); the four quarters meet in quar[4][DC], and
// DC threads add them into tot.  tot is readable when col_sum returns.
template <int DC>
__device__ __forceinline__ void put4(float* P, int i, int col, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<f32x4*>(P + i * (DC + 4) + col) = f32x4{x0, x1, x2, x3};
}

template <int D, int DC>
__device__ __forceinline__ void col_sum(const float* P, float (*quar)[DC], float* tot, int tid) {
  constexpr int PITCH = DC + 4;
  __syncthreads();
  const int j = tid % DC, r = tid / DC;
  float s = 0.f;
#pragma unroll 8
  for (int rr = 0; rr < D / 4; ++rr) s += P[(r * (D / 4) + rr) * PITCH + j];
  quar[r][j] = s;
  __syncthreads();
  if (tid < DC) tot[tid] = (quar[0][tid] + quar[1][tid]) + (quar[2][tid] + quar[3][tid]);
  __syncthreads();
}

// Floats of one head's checkpoint / interval area; workgroup half hc of the
// head uses the hc-th 1/SPLIT of it.
__host__ __device__ inline size_t bw_head_floats(int T, int D) {
  return (size_t)((T + kBwInterval - 1) / kBwInterval + kBwInterval) * D * D + (size_t)kBwInterval * D;
}

}  // namespace

template <typename T, int D, int SPLIT>
__global__ __launch_bounds__(4 * (D / SPLIT), 1) void kda_backward_kernel(BackwardArgs a) {
  using L = BwLayout<D, SPLIT>;
  constexpr int DC = L::DC, CPT = L::CPT, RPT = L::RPT, TPR = L::TPR;
  constexpr int NS = D * DC;  // floats of one workgroup's state slice ([D][DC])
  // per-token vectors, double-buffered: consecutive commits alternate buffers,
  // so a token's vectors land while the previous token may still be read
  __shared__ float s_k[2][D], s_a[2][D], s_q[2][D];        // per row
  __shared__ float s_v[2][DC], s_do[2][DC], s_u[2][DC];    // per own column
  __shared__ float s_b[2];
  __shared__ __attribute__((aligned(16))) float s_P[D * (DC + 4)];
  __shared__ float quar[4][DC];
  __shared__ float s_dd[DC];

  const int nbh = gridDim.x / SPLIT;
  const int bh = blockIdx.x / SPLIT, hc = blockIdx.x % SPLIT;
  const int col0 = hc * DC;  // first state column of this workgroup
  const int tid = threadIdx.x;
  const int i = tid / TPR;
  const int part = tid % TPR;
  const int c0 = part * CPT;  // local column
  const int nt = a.T;
  const int nch = (nt + kBwInterval - 1) / kBwInterval;

  const size_t tok0 = (size_t)bh * nt;
  const size_t st0 = (size_t)bh * D * D;  // this head's D x D states
  const T* q = static_cast<const T*>(a.q) + tok0 * D;
  const T* k = static_cast<const T*>(a.k) + tok0 * D;
  const T* v = static_cast<const T*>(a.v) + tok0 * D;
  const T* la = static_cast<const T*>(a.la) + tok0 * D;
  const T* beta = static_cast<const T*>(a.beta) + tok0;
  const T* dO = a.dO ? static_cast<const T*>(a.dO) + tok0 * D : nullptr;
  const size_t hf = bw_head_floats(nt, D);
  float* ckpt = a.ws + (size_t)bh * hf + (size_t)hc * (hf / SPLIT);
  float* hist = ckpt + (size_t)nch * NS;
  float* hu = hist + (size_t)kBwInterval * NS;  // u of each token of the interval, own columns
  // SPLIT = 2: the second half's row sums, [bh][t][3D + 1] after every head's
  // area (the first half writes its own straight to the outputs)
  float* part_sums = a.ws + (size_t)nbh * hf + (size_t)bh * (size_t)nt * (3 * D + 1);
  const size_t my = (size_t)i * DC + c0;  // this thread's first entry of the slice

  // Token vectors: threads < D fetch one row channel (k, log_alpha, q) and
  // threads < DC one own column (v, dO, u) of the next token into registers
  // while the current token is processed (fetch), and move them to LDS when
  // that token starts (commit, then a barrier).  with_q also takes q, dO and
  // the token's u (kept by the interval's forward pass at hu[tl]) for the
  // backward step.
  float nk = 0.f, nla = 0.f, nq = 0.f, nv = 0.f, ndo = 0.f, nu = 0.f, nb = 0.f;
  auto fetch = [&](int t, bool with_q, int tl = 0) {
    const size_t o = (size_t)t * D;
    if (tid < D) {
      nk = to_f32(k[o + tid]);
      nla = to_f32(la[o + tid]);
      if (with_q) nq = to_f32(q[o + tid]);
    }
    if (tid < DC) {
      nv = to_f32(v[o + col0 + tid]);
      if (with_q) {
        ndo = dO ? to_f32(dO[o + col0 + tid]) : 0.f;
        nu = hu[(size_t)tl * DC + tid];
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
      if (with_q) s_q[cb][tid] = nq;
    }
    if (tid < DC) {
      s_v[cb][tid] = nv;
      if (with_q) {
        s_do[cb][tid] = ndo;
        s_u[cb][tid] = nu;
      }
    }
    if (tid == 0) s_b[cb] = nb;
    __syncthreads();
    return cb;
  };

  // Forward passes in the column layout: thread tid owns local column jc =
  // tid / 4, rows [r0, r0 + D/4) with r0 = (tid % 4) D/4, so u_j = sum_i k_i
  // D[i][j] is a sum inside the thread and over the 4 adjacent lanes of the
  // column.  The states go to the workspace as [D][DC] slices, where the
  // backward walk (row layout) reads them after a barrier.
  const int jc = tid >> 2;
  const int r0 = (tid & 3) * RPT;
  float Sc[RPT];
  auto store_col = [&](float* dst) {
#pragma unroll
    for (int m = 0; m < RPT; ++m) dst[(size_t)(r0 + m) * DC + jc] = Sc[m];
  };
  // one forward token; `next` (or -1) is the token whose vectors to fetch
  // meanwhile; with keep >= 0 the token's u goes to hu[keep]
  auto forward = [&](int next, int keep) {
    const int cb = commit(false);
    if (next >= 0) fetch(next, false);
    float u = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      Sc[m] *= s_a[cb][r0 + m];
      u += s_k[cb][r0 + m] * Sc[m];
    }
    u += __shfl_xor(u, 1);
    u += __shfl_xor(u, 2);
    if (keep >= 0 && (tid & 3) == 0) hu[(size_t)keep * DC + jc] = u;
    const float w = s_b[cb] * (s_v[cb][jc] - u);
#pragma unroll
    for (int m = 0; m < RPT; ++m) Sc[m] += s_k[cb][r0 + m] * w;
  };

#pragma unroll
  for (int m = 0; m < RPT; ++m) Sc[m] = a.S0 ? a.S0[st0 + (size_t)(r0 + m) * D + col0 + jc] : 0.f;
  if (nt > 0) fetch(0, false);
  for (int t = 0; t < nt; ++t) {
    if (t % kBwInterval == 0) store_col(ckpt + (size_t)(t / kBwInterval) * NS);
    forward(t + 1 < nt ? t + 1 : -1, -1);
  }

  float S[CPT];
  float dS[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) dS[c] = a.dS_T ? a.dS_T[st0 + (size_t)i * D + col0 + c0 + c] : 0.f;

  for (int ch = nch - 1; ch >= 0; --ch) {
    const int t0 = ch * kBwInterval;
    const int t1 = min(t0 + kBwInterval, nt);
#pragma unroll
    for (int m = 0; m < RPT; ++m) Sc[m] = ckpt[(size_t)ch * NS + (size_t)(r0 + m) * DC + jc];
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
        put4<DC>(s_P, i, c0 + c, ki * dS[c], ki * dS[c + 1], ki * dS[c + 2], ki * dS[c + 3]);
      // d_delta = dS^T k (own columns)
      col_sum<D, DC>(s_P, quar, s_dd, tid);
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
      dq = row_sum<TPR>(dq);
      dk = row_sum<TPR>(dk);
      dla = row_sum<TPR>(dla);
      db = row_sum<TPR>(db);
      const size_t o = (tok0 + t) * D;
      if (SPLIT == 1 || hc == 0) {
        if (part == 0) {
          a.dq[o + i] = dq;
          a.dk[o + i] = dk;
          a.dla[o + i] = dla;
        }
        if (tid == 0) a.dbeta[tok0 + t] = db;
      } else {
        float* ps = part_sums + (size_t)t * (3 * D + 1);
        if (part == 0) {
          ps[i] = dq;
          ps[D + i] = dk;
          ps[2 * D + i] = dla;
        }
        if (tid == 0) ps[3 * D] = db;
      }
      if (tid < TPR) {  // the threads of row 0 hold d_delta for all own columns
#pragma unroll
        for (int c = 0; c < CPT; ++c) a.dv[o + col0 + c0 + c] = b * s_dd[c0 + c];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) a.dS0[st0 + (size_t)i * D + col0 + c0 + c] = dS[c];
}

// SPLIT = 2: adds the second workgroup's row sums of every token, [n] with
// n = BH T (3D + 1), to the first one's, already in dq, dk, dlog_alpha and
// dbeta (one add per element, so the result is deterministic).
__global__ __launch_bounds__(256) void kda_backward_sum_kernel(const float* __restrict__ ps, float* dq, float* dk,
                                                                float* dla, float* dbeta, long long rows, int D) {
  const int W = 3 * D + 1;
  const long long n = rows * W;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (long long)gridDim.x * blockDim.x) {
    const long long row = x / W;
    const int e = (int)(x - row * W);
    const float s = ps[x];
    if (e < D) dq[row * D + e] += s;
    else if (e < 2 * D) dk[row * D + e - D] += s;
    else if (e < 3 * D) dla[row * D + e - 2 * D] += s;
    else dbeta[row] += s;
  }
}

size_t backward_ws_floats(long long BH, int T, int D, int split) {
  return (size_t)BH * bw_head_floats(T, D) + (split == 2 ? (size_t)BH * (size_t)T * (3 * D + 1) : 0);
}

hipError_t launch_backward(const BackwardArgs& a, int BH, int D, int split, hipStream_t stream) {
  if (BH <= 0) return hipSuccess;
#define KDA_BW(TY, DD, SP)                                                                             \
  hipLaunchKernelGGL((kda_backward_kernel<TY, DD, SP>), dim3((long long)BH * SP),                    \
                     dim3(4 * ((DD) / (SP))), 0, stream, a)
#define KDA_BW_D(TY, SP) \
  do {                   \
    if (D == 128) KDA_BW(TY, 128, SP); \
    else KDA_BW(TY, 64, SP);           \
  } while (0)
  if (split == 2) KDA_BW_D(float, 2);
  else KDA_BW_D(float, 1);
#undef KDA_BW_D
#undef KDA_BW
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split != 2 || a.T == 0) return e;
  const long long rows = (long long)BH * a.T;
  const long long n = rows * (3 * D + 1);
  const int blocks = (int)std::min<long long>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(kda_backward_sum_kernel, dim3(blocks), dim3(256), 0, stream,
                     a.ws + (size_t)BH * bw_head_floats(a.T, D), a.dq, a.dk, a.dla, a.dbeta, rows, D);
  return hipGetLastError();
}

}  // namespace kda
