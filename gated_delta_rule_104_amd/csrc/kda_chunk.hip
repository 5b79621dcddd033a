// Chunked KDA evaluation on gfx950: prefill (outputs + end state) and the
// segment pass of the context-parallel decomposition (zero-start end state +
// transfer map).  One template, two modes.
//
// Method.  Per head the recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1}
// + b_t k_t v_t^T, o_t = S_t^T q_t is evaluated 64 tokens at a time: in
// parallel inside a chunk and sequentially across chunks (myzaker "Kimi K3
// 开源日来了", section "FlashKDA").  Within a chunk with start state S and
// per-channel cumulative log-gate g_r = sum_{j<=r} log a_j (kept in log space,
// blog.csdn.net article on the Kimi K3 report, section 一.1), write
//   Qh = q*e^g, Kh = k*e^g, Kb = k*e^-g, Kt = k*e^(g_C - g), Gam = e^(g_C),
//   A = strict_lower(Kh Kb^T),  P = lower(Qh Kb^T),
//   T = (I + diag(b) A)^-1,     Tb = T diag(b).
// Unrolling the recurrence over the chunk gives exactly
//   Delta = Tb (V - Kh S),  O = Qh S + P Delta,  S' = Diag(Gam) S + Kt^T Delta.
// Only the last three depend on S; everything else is S-independent.
//
// Work split.  Columns of S evolve independently once the S-independent
// products are known, so a workgroup owns 16*NC state columns of one
// sequence; several workgroups share a sequence when that is needed to fill
// the 256 compute units.  Inside a workgroup:
//   * NC consumer waves each hold a dk x 16 column slice of S in fp32 MFMA
//     accumulators and run the serial chain for chunk n;
//   * NP = dk/32 producer waves compute chunk n+1's S-independent products into
//     the other half of a double-buffered LDS stage (two pipelines that do not
//     wait on each other inside an iteration; the pages describe FlashKDA's
//     split of intra-chunk work and state passing between independently
//     scheduled thread groups in the same section).
// Three workgroup barriers per chunk separate the producer phases
// (elementwise -> scores -> inverse); the consumer spreads its chain over the
// same three intervals.  The fp32 variant has no room for two stages and runs
// producer and consumer one after the other.
//
// Segment mode runs the same chain on the augmented state [S | M] started at
// [0 | I] (columns >= dv see v = 0), skips q, P and O, and writes S and M.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int CH = 64;  // chunk length

template <typename T, int D, int NC, bool PREFILL>
struct ChunkCfg {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int ES = sizeof(T);
  static constexpr int STAGES = BF ? 2 : 1;
  static constexpr int LAG = STAGES - 1;
  static constexpr int NP = D / 32;
  static constexpr int NW = NC + NP;
  static constexpr int THREADS = 64 * NW;
  static constexpr int E16 = ES / 2;       // 16-byte pieces per 8 elements
  static constexpr int R_TD = D * ES;      // [CH][D] rows (time-major)
  static constexpr int R_DT = CH * ES;     // [D][CH] rows (channel-major)
  static constexpr int R_TT = CH * ES;     // [CH][CH] rows
  static constexpr int R_TI = 16 * ES;     // [16][16] rows
  static constexpr uint32_t S_KH = 0;
  static constexpr uint32_t S_QH = S_KH + CH * R_TD;
  static constexpr uint32_t S_KT = S_QH + (PREFILL ? CH * R_TD : 0);
  static constexpr uint32_t S_TB = S_KT + D * R_DT;
  static constexpr uint32_t S_P = S_TB + CH * R_TT;
  static constexpr uint32_t S_GM = S_P + (PREFILL ? CH * R_TT : 0);
  static constexpr uint32_t STAGE = S_GM + D * 4;
  static constexpr uint32_t X_KB = STAGES * STAGE;
  static constexpr uint32_t X_L = X_KB + CH * R_TD;
  static constexpr uint32_t X_TI = X_L + CH * R_TT;
  static constexpr uint32_t X_BETA = X_TI + 4 * 16 * R_TI;
  static constexpr uint32_t LDS = X_BETA + CH * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(LDS % 16 == 0, "LDS size");
};

// 8 consecutive elements of a token row, as loaded from HBM.
template <typename T> struct Raw8 { u32x4 p[sizeof(T) / 2]; };

template <typename T>
__device__ __forceinline__ void raw_load(Raw8<T>& r, const T* ptr, bool ok) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i)
    r.p[i] = ok ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(ptr) + 16 * i)
                : u32x4{0u, 0u, 0u, 0u};
}

template <typename T>
__device__ __forceinline__ void raw_f32(const Raw8<T>& r, float* out) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(r.p[0][i] << 16);
      out[2 * i + 1] = __uint_as_float(r.p[0][i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(r.p[i >> 2][i & 3]);
  }
}

template <typename T>
__device__ __forceinline__ float exp_dev(float x) {
  if constexpr (sizeof(T) == 2) return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
  else return expf(x);
}

// Producer input registers for one chunk: 4 token rows x 8 channels of
// log_alpha, k and q, plus one beta per lane.
template <typename T> struct ProdRaw {
  Raw8<T> la[4], k[4], q[4];
  uint32_t beta;
};

template <typename T> struct VRegs { T v[16]; };

template <typename T, int D, int NC, bool PREFILL>
struct ChunkKernel {
  using C = ChunkCfg<T, D, NC, PREFILL>;
  char* smem;
  ChunkArgs a;
  const T* q; const T* k; const T* v; const T* la; const T* beta;
  size_t tok0;     // first token of this sequence
  int Tlen, nch;
  int wave, l, g4;  // wave index, lane, 4*(lane/16)
  // consumer
  int col;          // global column of this lane's state slice
  bool isv;         // column reads v (value column) rather than being a map column
  f32x4 S[D / 16];
  f32x4 Dl[4];      // Delta tiles of the current chunk
  bf16x8 SB[D / 32], DB[2];

  __device__ __forceinline__ uint32_t stage(int chunk) const {
    return (C::STAGES == 2 ? (uint32_t)(chunk & 1) : 0u) * C::STAGE;
  }

  // ------------------------------------------------------------ producers
  __device__ __forceinline__ void load_raw(ProdRaw<T>& r, int chunk) const {
    const int pw = wave - NC;
    const int tg = l >> 2, cs = l & 3;
    const int ch = 32 * pw + 8 * cs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = chunk * CH + 4 * tg + i;
      const bool ok = t < Tlen;
      const size_t off = (tok0 + (size_t)(ok ? t : 0)) * D + ch;
      raw_load<T>(r.la[i], la + off, ok);
      raw_load<T>(r.k[i], k + off, ok);
      if constexpr (PREFILL) raw_load<T>(r.q[i], q + off, ok);
    }
    if (pw == 0) {
      const int t = chunk * CH + l;
      if (t < Tlen) {
        if constexpr (sizeof(T) == 2)
          r.beta = (uint32_t)(*reinterpret_cast<const uint16_t*>(beta + tok0 + t)) << 16;
        else
          r.beta = __float_as_uint(beta[tok0 + t]);
      } else {
        r.beta = 0u;
      }
    }
  }

  // Phase 1: cumulative log-gate and the decayed operand tiles of one chunk.
  __device__ __forceinline__ void p1(const ProdRaw<T>& r, uint32_t st) {
    const int pw = wave - NC;
    const int tg = l >> 2, cs = l & 3;
    const int ch = 32 * pw + 8 * cs;
    float g[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw_f32<T>(r.la[i], g[i]);
    float tot[8], inc[8], exc[8], gc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      g[1][c] += g[0][c];
      g[2][c] += g[1][c];
      g[3][c] += g[2][c];
      tot[c] = g[3][c];
      inc[c] = tot[c];
    }
    // inclusive scan of the 4-token totals over the 16 token groups (lane stride 4)
#pragma unroll
    for (int d = 4; d < 64; d *= 2) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float y = __shfl_up(inc[c], d);
        if (l >= d) inc[c] += y;
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float y = __shfl_up(inc[c], 4);
      exc[c] = (l >= 4) ? y : 0.f;
      gc[c] = __shfl(inc[c], 60 + cs);
    }
    float kt[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * tg + i;
      float kk[8], qq[8], vq[8], vkh[8], vkb[8];
      raw_f32<T>(r.k[i], kk);
      if constexpr (PREFILL) raw_f32<T>(r.q[i], qq);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float gg = g[i][c] + exc[c];
        const float eg = exp_dev<T>(gg);
        const float emg = exp_dev<T>(-gg);
        const float et = exp_dev<T>(gc[c] - gg);
        vkh[c] = kk[c] * eg;
        vkb[c] = kk[c] * emg;
        if constexpr (PREFILL) vq[c] = qq[c] * eg;
        kt[i][c] = kk[c] * et;
      }
      if constexpr (C::BF) {
        bf16x8 h, b, qv;
#pragma unroll
        for (int c = 0; c < 8; ++c) { h[c] = (bf16)vkh[c]; b[c] = (bf16)vkb[c]; qv[c] = (bf16)vq[c]; }
        lds_st<bf16x8>(smem, st + C::S_KH + swz<C::R_TD>(row, 2 * ch), h);
        lds_st<bf16x8>(smem, C::X_KB + swz<C::R_TD>(row, 2 * ch), b);
        if constexpr (PREFILL) lds_st<bf16x8>(smem, st + C::S_QH + swz<C::R_TD>(row, 2 * ch), qv);
      } else {
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          f32x4 h = {vkh[4 * hlf], vkh[4 * hlf + 1], vkh[4 * hlf + 2], vkh[4 * hlf + 3]};
          f32x4 b = {vkb[4 * hlf], vkb[4 * hlf + 1], vkb[4 * hlf + 2], vkb[4 * hlf + 3]};
          lds_st<f32x4>(smem, st + C::S_KH + swz<C::R_TD>(row, 4 * (ch + 4 * hlf)), h);
          lds_st<f32x4>(smem, C::X_KB + swz<C::R_TD>(row, 4 * (ch + 4 * hlf)), b);
          if constexpr (PREFILL) {
            f32x4 qv = {vq[4 * hlf], vq[4 * hlf + 1], vq[4 * hlf + 2], vq[4 * hlf + 3]};
            lds_st<f32x4>(smem, st + C::S_QH + swz<C::R_TD>(row, 4 * (ch + 4 * hlf)), qv);
          }
        }
      }
    }
    // Kt^T: channel-major, 4 consecutive tokens per lane and channel
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int rowc = ch + c;
      if constexpr (C::BF) {
        bf16x4 t4;
        t4[0] = (bf16)kt[0][c]; t4[1] = (bf16)kt[1][c]; t4[2] = (bf16)kt[2][c]; t4[3] = (bf16)kt[3][c];
        lds_st<bf16x4>(smem, st + C::S_KT + swz<C::R_DT>(rowc, 2 * 4 * tg), t4);
      } else {
        f32x4 t4 = {kt[0][c], kt[1][c], kt[2][c], kt[3][c]};
        lds_st<f32x4>(smem, st + C::S_KT + swz<C::R_DT>(rowc, 4 * 4 * tg), t4);
      }
    }
    if (tg == 15) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        lds_st<float>(smem, st + C::S_GM + 4 * (ch + c), exp_dev<T>(gc[c]));
    }
    if (pw == 0) lds_st<float>(smem, C::X_BETA + 4 * l, __uint_as_float(r.beta));
  }

  __device__ __forceinline__ void store_tt(uint32_t base, int r, int s, float x) {
    lds_st<T>(smem, base + swz<C::R_TT>(r, C::ES * s), from_f32<T>(x));
  }

  // Phase 2: intra-chunk scores.  Row task (mat, i) computes tiles (i, 0..i) of
  // L = diag(b) A (mat 0) or P (mat 1); an L row task then inverts its
  // diagonal block (I + L_ii) by substitution, one column per lane.
  __device__ __forceinline__ void p2(uint32_t st) {
    const int pw = wave - NC;
    constexpr int NTASK = PREFILL ? 8 : 4;
    for (int task = pw; task < NTASK; task += C::NP) {
      const int mat = PREFILL ? (task & 1) : 0;
      const int i = 3 - (PREFILL ? (task >> 1) : task);
      const uint32_t abase = mat ? st + C::S_QH : st + C::S_KH;
      for (int j = 0; j <= i; ++j) {
        f32x4 acc = zero4();
        if constexpr (C::BF) acc = mma_ll_bf16<C::R_TD>(acc, smem, abase, 16 * i, C::X_KB, 16 * j, D);
        else acc = mma_ll_f32<C::R_TD>(acc, smem, abase, 16 * i, C::X_KB, 16 * j, D);
        const int s = 16 * j + (l & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + g4 + e;
          if (mat == 0) {
            const float b = lds_ld<float>(smem, C::X_BETA + 4 * r);
            store_tt(C::X_L, r, s, s < r ? acc[e] * b : 0.f);
          } else {
            store_tt(st + C::S_P, r, s, s <= r ? acc[e] : 0.f);
          }
        }
      }
      if (mat == 0) {
        wave_lds_fence();
        const int c = l & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sum = (r == c) ? 1.f : 0.f;
#pragma unroll
          for (int m = 0; m < r; ++m)
            sum -= to_f32(lds_ld<T>(smem, C::X_L + swz<C::R_TT>(16 * i + r, C::ES * (16 * i + m)))) * x[m];
          x[r] = sum;
        }
        if (l < 16) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            lds_st<T>(smem, C::X_TI + i * 16 * C::R_TI + swz<C::R_TI>(r, C::ES * c), from_f32<T>(x[r]));
        }
      }
    }
  }

  // acc of a 16x16 tile product A(16x16 from LDS tile at base, rows of RR bytes,
  // row r0, col k0) times B (accumulator tile in registers).
  template <int RR>
  __device__ __forceinline__ f32x4 mma16(uint32_t base, int r0, int k0, f32x4 b, f32x4 acc) const {
    if constexpr (C::BF) {
      bf16x4 af = lds_ld<bf16x4>(smem, base + swz<RR>(r0 + (l & 15), 2 * (k0 + g4)));
      return mfma_bf16_k16(acc, af, pack4(b));
    } else {
      return mma_ar_f32<RR>(acc, smem, base, r0, k0, &b, 1);
    }
  }

  // Phase 3: off-diagonal blocks of T = (I + L)^-1 by block forward
  // substitution, T_ij = -T_ii sum_{m=j}^{i-1} L_im T_mj, then Tb = T diag(b).
  // Column block J of T is one task.
  template <int J>
  __device__ __forceinline__ void p3_col(uint32_t st) {
    f32x4 Tc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Tc[J][e] = to_f32(lds_ld<T>(smem, C::X_TI + J * 16 * C::R_TI + swz<C::R_TI>(g4 + e, C::ES * (l & 15))));
#pragma unroll
    for (int i = J + 1; i < 4; ++i) {
      f32x4 y = zero4();
#pragma unroll
      for (int m = J; m < i; ++m) y = mma16<C::R_TT>(C::X_L, 16 * i, 16 * m, Tc[m], y);
      f32x4 z = mma16<C::R_TI>(C::X_TI + i * 16 * C::R_TI, 0, 0, y, zero4());
      Tc[i] = -z;
    }
    const int s = 16 * J + (l & 15);
    const float b = lds_ld<float>(smem, C::X_BETA + 4 * s);
#pragma unroll
    for (int m = J; m < 4; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) store_tt(st + C::S_TB, 16 * m + g4 + e, s, Tc[m][e] * b);
    }
  }

  __device__ __forceinline__ void p3(uint32_t st) {
    const int pw = wave - NC;
    if (0 % C::NP == pw) p3_col<0>(st);
    if (1 % C::NP == pw) p3_col<1>(st);
    if (2 % C::NP == pw) p3_col<2>(st);
    if (3 % C::NP == pw) p3_col<3>(st);
  }

  // ------------------------------------------------------------ consumers
  __device__ __forceinline__ void load_v(VRegs<T>& vr, int chunk) const {
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = chunk * CH + 16 * ti + g4 + e;
        T x = from_f32<T>(0.f);
        if (isv && t < Tlen) x = v[(tok0 + t) * D + col];
        vr.v[4 * ti + e] = x;
      }
    }
  }

  // Interval 1: Delta = Tb (V - Kh S).
  __device__ __forceinline__ void c1(const VRegs<T>& vr, uint32_t st) {
    f32x4 X[4];
    if constexpr (C::BF) {
#pragma unroll
      for (int m = 0; m < D / 32; ++m) SB[m] = pack8(S[2 * m], S[2 * m + 1]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 y = mma_ar_bf16<C::R_TD>(zero4(), smem, st + C::S_KH, 16 * ti, 0, SB, D / 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) X[ti][e] = to_f32(vr.v[4 * ti + e]) - y[e];
      }
      bf16x8 XB[2] = {pack8(X[0], X[1]), pack8(X[2], X[3])};
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        Dl[ti] = mma_ar_bf16<C::R_TT>(zero4(), smem, st + C::S_TB, 16 * ti, 0, XB, (ti >> 1) + 1);
      DB[0] = pack8(Dl[0], Dl[1]);
      DB[1] = pack8(Dl[2], Dl[3]);
    } else {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 y = mma_ar_f32<C::R_TD>(zero4(), smem, st + C::S_KH, 16 * ti, 0, S, D / 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) X[ti][e] = to_f32(vr.v[4 * ti + e]) - y[e];
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        Dl[ti] = mma_ar_f32<C::R_TT>(zero4(), smem, st + C::S_TB, 16 * ti, 0, X, ti + 1);
    }
  }

  // Interval 2: O = Qh S + P Delta, stored.
  __device__ __forceinline__ void c2(uint32_t st, int chunk) {
    if constexpr (PREFILL) {
      T* o = reinterpret_cast<T*>(a.o);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        f32x4 acc;
        if constexpr (C::BF) {
          acc = mma_ar_bf16<C::R_TD>(zero4(), smem, st + C::S_QH, 16 * ti, 0, SB, D / 32);
          acc = mma_ar_bf16<C::R_TT>(acc, smem, st + C::S_P, 16 * ti, 0, DB, (ti >> 1) + 1);
        } else {
          acc = mma_ar_f32<C::R_TD>(zero4(), smem, st + C::S_QH, 16 * ti, 0, S, D / 16);
          acc = mma_ar_f32<C::R_TT>(acc, smem, st + C::S_P, 16 * ti, 0, Dl, ti + 1);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = chunk * CH + 16 * ti + g4 + e;
          if (t < Tlen) o[(tok0 + t) * D + col] = from_f32<T>(acc[e]);
        }
      }
    }
  }

  // Interval 3: S = Diag(Gam) S + Kt^T Delta.
  __device__ __forceinline__ void c3(uint32_t st) {
#pragma unroll
    for (int ci = 0; ci < D / 16; ++ci) {
      f32x4 gm = lds_ld<f32x4>(smem, st + C::S_GM + 4 * (16 * ci + g4));
      f32x4 acc = S[ci] * gm;
      if constexpr (C::BF) acc = mma_ar_bf16<C::R_DT>(acc, smem, st + C::S_KT, 16 * ci, 0, DB, 2);
      else acc = mma_ar_f32<C::R_DT>(acc, smem, st + C::S_KT, 16 * ci, 0, Dl, 4);
      S[ci] = acc;
    }
  }

  // Pipeline.  Iteration `it` has producers prepare chunk it while consumers
  // run chunk it - LAG; both roles execute the same barrier sequence.  Each
  // role keeps one set of prefetch registers: the loads for the next chunk
  // are issued as soon as the current chunk's registers have been consumed.
  __device__ __forceinline__ void producer_loop() {
    ProdRaw<T> r;
    if (nch > 0) load_raw(r, 0);
    for (int it = 0; it < nch + C::LAG; ++it) {
      const bool w = it < nch;
      if (w) {
        p1(r, stage(it));
        if (it + 1 < nch) load_raw(r, it + 1);
      }
      sync_lds();
      if (w) p2(stage(it));
      sync_lds();
      if (w) p3(stage(it));
      sync_lds();
      if (!C::LAG) sync_lds();
    }
  }

  __device__ __forceinline__ void consumer_loop() {
    VRegs<T> vr;
    if (nch > 0) load_v(vr, 0);
    for (int it = 0; it < nch + C::LAG; ++it) {
      const int cc = it - C::LAG;
      const bool w = cc >= 0;
      if (!C::LAG) {
        sync_lds();
        sync_lds();
        sync_lds();
      }
      if (w) {
        c1(vr, stage(cc));
        if (cc + 1 < nch) load_v(vr, cc + 1);
      }
      if (C::LAG) sync_lds();
      if (w) c2(stage(cc), cc);
      if (C::LAG) sync_lds();
      if (w) c3(stage(cc));
      sync_lds();
    }
  }

  __device__ __forceinline__ void run() {
    const int W = gridDim.x;
    int id = blockIdx.x;
    // Consecutive blockIdx go to different XCDs (round-robin over 8); regroup so
    // that the workgroups sharing a sequence land on one XCD and share its L2.
    if ((W & 7) == 0) id = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int seq = id / a.vsplit;
    const int vs = id - seq * a.vsplit;
    const int gseg = seq / a.BH;
    const int bh = seq - gseg * a.BH;
    tok0 = ((size_t)bh * a.G + gseg) * (size_t)a.Tseg;
    Tlen = a.Tseg;
    nch = (Tlen + CH - 1) / CH;
    wave = threadIdx.x >> 6;
    l = lane_id();
    g4 = 4 * (l >> 4);
    q = reinterpret_cast<const T*>(a.q);
    k = reinterpret_cast<const T*>(a.k);
    v = reinterpret_cast<const T*>(a.v);
    la = reinterpret_cast<const T*>(a.la);
    beta = reinterpret_cast<const T*>(a.beta);

    for (uint32_t i = threadIdx.x * 16; i < C::LDS; i += C::THREADS * 16)
      lds_st<u32x4>(smem, i, u32x4{0u, 0u, 0u, 0u});

    col = vs * 16 * NC + 16 * wave + (l & 15);
    isv = col < D;
    const size_t sbase = (size_t)seq * D * D;
    if (wave < NC) {
#pragma unroll
      for (int ci = 0; ci < D / 16; ++ci)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * ci + g4 + e;
          float x = 0.f;
          if (PREFILL) {
            if (a.S0) x = a.S0[sbase + (size_t)r * D + col];
          } else if (!isv) {
            x = (r == col - D) ? 1.f : 0.f;
          }
          S[ci][e] = x;
        }
    }
    sync_lds();

    if (wave >= NC) {
      producer_loop();
      return;
    }
    consumer_loop();

    if (wave < NC) {
      float* dst;
      int c = col;
      if (PREFILL || isv) dst = a.S_out + sbase;
      else { dst = a.M_out + sbase; c = col - D; }
#pragma unroll
      for (int ci = 0; ci < D / 16; ++ci)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)(16 * ci + g4 + e) * D + c] = S[ci][e];
    }
  }
};

template <typename T, int D, int NC, bool PREFILL>
__global__ __launch_bounds__(64 * (NC + D / 32), 1)
void kda_chunk_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[ChunkCfg<T, D, NC, PREFILL>::LDS];
  ChunkKernel<T, D, NC, PREFILL> kern;
  kern.smem = smem;
  kern.a = a;
  kern.run();
}

template <typename T, int D, int NC, bool PREFILL>
static hipError_t launch_one(const ChunkArgs& a, int nwg, hipStream_t stream) {
  using Cf = ChunkCfg<T, D, NC, PREFILL>;
  hipLaunchKernelGGL((kda_chunk_kernel<T, D, NC, PREFILL>), dim3(nwg), dim3(Cf::THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, bool PREFILL>
static hipError_t launch_nc(const ChunkArgs& a, int nc, int nwg, hipStream_t stream) {
  switch (nc) {
    case 1: return launch_one<T, D, 1, PREFILL>(a, nwg, stream);
    case 2: return launch_one<T, D, 2, PREFILL>(a, nwg, stream);
    case 4: return launch_one<T, D, 4, PREFILL>(a, nwg, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk(const ChunkArgs& a, bool bf16_io, int D, bool prefill, int nc, int nwg,
                        hipStream_t stream) {
  if (bf16_io) {
    if (D == 128) return prefill ? launch_nc<bf16, 128, true>(a, nc, nwg, stream)
                                 : launch_nc<bf16, 128, false>(a, nc, nwg, stream);
    if (D == 64) return prefill ? launch_nc<bf16, 64, true>(a, nc, nwg, stream)
                                : launch_nc<bf16, 64, false>(a, nc, nwg, stream);
  } else {
    if (D == 64) return prefill ? launch_nc<float, 64, true>(a, nc, nwg, stream)
                                : launch_nc<float, 64, false>(a, nc, nwg, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
