// Per-chunk gradients of the prefill: the chunk-parallel part of the backward.
//
// For a loss L with dL/do = dO and dL/dS_T = dS_T, the gradients of a 64-token
// chunk follow from its start state S, the gradient dU = Diag(Gam) dS' with
// respect to its end state (scaled by the chunk's decay), and the chunk's own
// inputs.  With the chunked form of the recurrence (blog.csdn.net article on
// the Kimi K3 report, section 一.1, for the gated delta rule; "Kimi K3
// 开源日来了", section "FlashKDA", for the chunking; training is what the K3
// report also speeds up with FlashKDA)
//   g = cumsum(log alpha),  Qh = q e^g,  Kh = k e^g,  Kb = k e^-g,  Gam = e^(g_C)
//   A = strict_lower(Kh Kb^T),  L = diag(b) A,  P = lower(Qh Kb^T),  T = (I + L)^-1
//   W = V - Kh S,  X = diag(b) W,  Delta = T X
//   O = Qh S + P Delta,  S' = Diag(Gam) (S + Kb^T Delta)
// the chain rule gives, per chunk:
//   dDelta = Kb dU + P^T dO,  Xbar = T^T dDelta,  dv = diag(b) Xbar
//   dP = lower(dO Delta^T),  Abar = diag(b) strict_lower(-Xbar Delta^T) = -strict_lower(dv Delta^T)
//   dQh = dO S^T + dP Kb
//   dKh = -dv S^T + Abar Kb
//   dKb = Delta dU^T + Abar^T Kh + dP^T Qh
//   dbeta_r = sum_j Xbar_rj W_rj - sum_{s<r} (Xbar Delta^T)_rs A_rs = Xbar_r . Y_r,  Y = W - A Delta
//   dq = dQh e^g,  dk = dKh e^g + dKb e^-g
//   dlog_alpha_r = sum_{t >= r} dg_t + rowsum(dU . S) + sum_{s < r} k_s e^-g_s (Delta dU^T)_s
//     with dg = q dq + k (dKh e^g - (dKb - Delta dU^T) e^-g)
// The last line is the gradient with respect to g (g = cumsum(log alpha) within
// the chunk) summed over later tokens, with Gam's part (every token of the
// chunk: rowsum(dU . (S + Kb^T Delta))) taken apart: its Kb^T Delta piece and
// the Delta dU^T piece of dKb cancel for s >= r, so that sum_{s < r} is formed
// directly, which in bf16 products avoids a cancellation between large terms.
//
// The forward equations give Delta = diag(b) Y exactly ((I + diag(b) A) Delta
// = diag(b) W), so for b_r != 0, dbeta_r = dv_r . Delta_r / b_r^2, and no
// product needs Xbar, W or A itself.  The forward pass stores S and Delta of
// every chunk and the reverse chain dS' (and writes dv); only for the rows with
// b below kTinyBeta do they also keep W, A's row and Xbar, from which this
// kernel forms dbeta_r = Xbar_r . (W_r - sum_{s<r} A_rs Delta_s).  Two workgroups
// per (head, chunk), each owning half of the key dimension's columns with one
// wave per 16 columns (4 waves at d = 128).  Each needs about 72 KiB of LDS,
// so two run on a CU at once and one's loads overlap the other's arithmetic.
// Phases, each ended by a workgroup barrier:
//   1. every wave copies its share of dO, Delta and dv into LDS tiles (all
//      loads issued before the first store);
//   2. the 64 x 64 gradients dP, dP^T, Abar, Abar^T (as MFMA A fragments), and
//      in the first half's workgroup dbeta;
//   3. per wave, a 16-column tile of the key dimension: dQh, dKh, dKb (the
//      products with the 64 x 64 gradients on fp32 Kb, Kh, Qh split into two
//      bf16 parts), then the gate's chain rule, written out per (token, channel).
// Operand conventions are those of the chunk kernel: bf16 MFMA 16x16x32 tiles,
// time-major LDS tiles with 32-wide k blocks in the kpos order, and 16x16
// tiles that feed a product as A operands stored in fragment order.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int GCH = 64;  // chunk length
constexpr float G_LOG2E = 1.4426950408889634f;

template <int D>
struct GradCfg {
  static constexpr int NW = D / 32;            // waves per workgroup: 16 columns each, half of D
  static constexpr int THREADS = 64 * NW;
  static constexpr int NCT = 1;                // 16-column tiles per wave
  static constexpr int NKD = D / 32;           // 32-deep k blocks over channels
  static constexpr int NKT = GCH / 32;         // 32-deep k blocks over the chunk's tokens
  static constexpr int R_TD = D * 2;           // bf16 row of a [64][D] tile
  static constexpr int TD_TILE = 16 * R_TD + 16;
  static constexpr int TD_SZ = 4 * TD_TILE;
  // A 64x64 block-triangular matrix as 32-deep A fragments: the 6 of its 8
  // (row tile, k block) slots that hold a nonzero block
  static constexpr int FRC = 6 * 64 * 16;
  static constexpr uint32_t DO = 0;
  static constexpr uint32_t DL = DO + TD_SZ;     // Delta
  static constexpr uint32_t DV = DL + TD_SZ;     // dv
  static constexpr uint32_t DP = DV + TD_SZ;     // dP (lower)
  static constexpr uint32_t DPT = DP + FRC;      // dP^T (upper)
  static constexpr uint32_t AB = DPT + FRC;      // Abar (lower)
  static constexpr uint32_t ABT = AB + FRC;      // Abar^T (upper)
  static constexpr uint32_t BETA = ABT + FRC;    // beta [64] fp32
  static constexpr uint32_t LDS = BETA + 4 * GCH;
  static_assert(2 * LDS <= 160 * 1024, "two workgroups per CU");
  static_assert(LDS % 16 == 0, "LDS alignment");
  static_assert(D / NW == 32, "dbeta: 32 channels of a row per lane");
};

template <int D>
struct GradKernel {
  using C = GradCfg<D>;
  static constexpr int NW = C::NW, NCT = C::NCT, NKD = C::NKD, NKT = C::NKT;
  static constexpr int NP4 = 10;                   // lower blocks (R, S) of the 64x64 gradients
  char* smem;
  BwGradArgs a;
  int wave, l, g4, s0;
  int half;   // which half of the key dimension's columns
  int nrows;  // valid tokens of this chunk
  rsrc_t rq, rk, rla, rbeta, rdo, rdv, rdq, rdk, rdla, rSr, rUr, rW, rDl, rXb, rA;
  uint32_t oTD[NKD];   // A fragments of [64][D] tiles, row tile 0

  __device__ __forceinline__ static uint32_t td(int row, int byte) {
    return (uint32_t)(row >> 4) * C::TD_TILE + swz<C::R_TD>(row & 15, byte);
  }
  // A fragment of row tile t, k block m (channels) of a [64][D] tile
  __device__ __forceinline__ bf16x8 ar(uint32_t tile, int t, int m) const {
    return lds_ld<bf16x8>(smem, tile + oTD[m] + t * C::TD_TILE);
  }
  // Compact slots of the 32-deep A fragments of a 64x64 matrix: row tile t, k
  // block m.  Lower block-triangular (dP, Abar): m <= t/2; upper (their
  // transposes): m >= (t-1)/2.
  __device__ __forceinline__ static constexpr int lo_idx(int t, int m) { return t < 2 ? t : 2 * t - 2 + m; }
  __device__ __forceinline__ static constexpr int up_idx(int t, int m) { return t < 2 ? 2 * t + m : t + 2; }
  __device__ __forceinline__ bf16x8 frlo(uint32_t base, int t, int m) const {
    return lds_ld<bf16x8>(smem, base + (lo_idx(t, m) * 64 + fresh_lane(l)) * 16);
  }
  __device__ __forceinline__ bf16x8 frup(uint32_t base, int t, int m) const {
    return lds_ld<bf16x8>(smem, base + (up_idx(t, m) * 64 + fresh_lane(l)) * 16);
  }
  __device__ __forceinline__ void put16(uint32_t off, const f32x4& v) { lds_st<bf16x4>(smem, off, pack4(v)); }
  // this lane's 4 values of block (R, S) in the slot of a lower / upper matrix
  __device__ __forceinline__ uint32_t slot_lo(uint32_t base, int R, int S) const {
    return base + (lo_idx(R, S / 2) * 64 + fresh_lane(l)) * 16 + (S % 2) * 8;
  }
  __device__ __forceinline__ uint32_t slot_up(uint32_t base, int R, int S) const {
    return base + (up_idx(R, S / 2) * 64 + fresh_lane(l)) * 16 + (S % 2) * 8;
  }
  // x + a.b over bf16 pair e of two 8-element fragments, in fp32
  __device__ __forceinline__ static float dot2(const bf16x8& a, const bf16x8& b, int e, float x) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    const bf16x2 u = {a[2 * e], a[2 * e + 1]}, v = {b[2 * e], b[2 * e + 1]};
    return __builtin_amdgcn_fdot2_f32_bf16(u, v, x, false);
  }

  __device__ __forceinline__ void init_offsets() {
    const int r16 = l & 15;
    const int kg = 8 * (l >> 4);
#pragma unroll
    for (int m = 0; m < NKD; ++m) oTD[m] = swz<C::R_TD>(r16, 2 * (32 * m + kg));
  }

  // ------------------------------------------------------------ phase 1
  // dO and dv (plain channel order) and Delta (the checkpoint, already
  // kpos-ordered) into their LDS tiles, 16 bytes at a time: every load is
  // issued before the first store, so that their latencies overlap.
  __device__ __forceinline__ void copy_tiles() {
    constexpr int PIECES = GCH * D / 8;  // 16-byte pieces of one tile
    constexpr int NL = NW * 64;
    static_assert(PIECES % NL == 0, "each load stays in one tile");
    constexpr int PER = 3 * PIECES / NL, PER_TILE = PIECES / NL;
    const int x0 = wave * 64 + l;
    u32x4 w[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int y = i % PER_TILE * NL + x0;  // piece within tile i / PER_TILE
      const int row = y / (D / 8), p8 = 8 * (y - row * (D / 8));
      const rsrc_t r = i < PER_TILE ? rdo : i < 2 * PER_TILE ? rDl : rdv;
      w[i] = bload128(r, (uint32_t)(row * D + p8) * 2u);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int y = i % PER_TILE * NL + x0;
      const int row = y / (D / 8), p8 = 8 * (y - row * (D / 8));
      if (i < PER_TILE || i >= 2 * PER_TILE) {  // plain channel order: to the kpos positions
        const uint32_t base = i < PER_TILE ? C::DO : C::DV;
        lds_st<u32x2>(smem, base + td(row, 2 * kpos(p8)), u32x2{w[i][0], w[i][1]});
        lds_st<u32x2>(smem, base + td(row, 2 * kpos(p8 + 4)), u32x2{w[i][2], w[i][3]});
      } else {
        lds_st<u32x4>(smem, C::DL + td(row, 2 * p8), w[i]);
      }
    }
  }

  // sum over the 16 lanes of each lane row; lane 15 of the row holds it
  __device__ __forceinline__ static float row_sum16(float x) {
    x += dpp<DPP_ROW_SHR + 1>(x);
    x += dpp<DPP_ROW_SHR + 2>(x);
    x += dpp<DPP_ROW_SHR + 4>(x);
    x += dpp<DPP_ROW_SHR + 8>(x);
    return x;
  }

  // one gradient, rounded to bf16, at (row, column) of the chunk's [64][D] output
  __device__ __forceinline__ static void st_bf16(rsrc_t r, int row, int c, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (bf16)x), r, (uint32_t)(row * D + c) * 2u, 0, 0);
  }

  // Lane l works on column c = D/2 half + 16 wave + l%16 of the head
  // dimension, rows 16t + 4g + e of the chunk (accumulator layout).
  __device__ __forceinline__ int col(int j) const { return half * (D / 2) + 16 * (NCT * wave + j) + s0; }

  // Row c of a checkpoint matrix stored with kpos-ordered rows, k block m: one
  // 16-byte read is the B fragment over that block.
  __device__ __forceinline__ bf16x8 ck_frag(rsrc_t r, int c, int m) const {
    return __builtin_bit_cast(bf16x8, bload128(r, (uint32_t)(c * D + 32 * m + 2 * g4) * 2u));
  }

  // Global data of phase 3, loaded at the start so that the loads are in
  // flight across phases 1 and 2 (the barriers wait only for LDS).  bf16
  // values at this lane's accumulator positions are kept as raw 16-bit loads.
  struct Pre5 {
    bf16x8 sr[NCT][NKD], ur[NCT][NKD];  // S and dS' rows as B fragments over their columns
    uint32_t la[NCT][16], q[NCT][16], k[NCT][16];
  };
  __device__ __forceinline__ uint32_t raw16(rsrc_t r, uint32_t off) const {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  __device__ __forceinline__ static float f16raw(uint32_t x) { return __uint_as_float(x << 16); }
  __device__ __forceinline__ void load_pre5(Pre5& p) const {
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
#pragma unroll
      for (int m = 0; m < NKD; ++m) {
        p.sr[j][m] = ck_frag(rSr, col(j), m);
        p.ur[j][m] = ck_frag(rUr, col(j), m);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 16 * (i >> 2) + g4 + (i & 3);
        const uint32_t off = (uint32_t)(row * D + col(j)) * 2u;
        p.la[j][i] = raw16(rla, off);
        p.q[j][i] = raw16(rq, off);
        p.k[j][i] = raw16(rk, off);
      }
    }
  }

  // dbeta of every row of the chunk, first half's workgroup only: lane x =
  // 64 wave + l takes 32 channels c0 = 32 (x % NW) .. of row x / NW (both
  // tiles and checkpoints in the kpos order), the NW lanes of a row add their
  // parts.  b_r >= kTinyBeta: dbeta_r = (dv_r . Delta_r) / b_r^2.  Otherwise
  // dbeta_r = Xbar_r . (W_r - sum_{s<r} A_rs Delta_s), from the rows the chain
  // kernels keep for such tokens.
  __device__ __forceinline__ void dbeta_rows(size_t tok0) const {
    const int x = wave * 64 + l, row = x / NW, c0 = 32 * (x % NW);
    const float b = lds_ld<float>(smem, C::BETA + 4 * row);
    float part = 0.f;
    if (b >= kTinyBeta) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 dv8 = lds_ld<bf16x8>(smem, C::DV + td(row, 2 * (c0 + 8 * i)));
        const bf16x8 dl8 = lds_ld<bf16x8>(smem, C::DL + td(row, 2 * (c0 + 8 * i)));
#pragma unroll
        for (int e = 0; e < 4; ++e) part = dot2(dv8, dl8, e, part);
      }
    } else {
      // A_rs: block (row/16, s/16) at I(I+1)/2 + J, lane row%16 + 16 ((s%16)/4), value s%4
      const int I = row >> 4;
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)(row * D + c0 + 8 * i) * 2u;
        const bf16x8 xb8 = __builtin_bit_cast(bf16x8, bload128(rXb, off));
        const bf16x8 w8 = __builtin_bit_cast(bf16x8, bload128(rW, off));
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = (float)w8[k];
        for (int s = 0; s < row; ++s) {
          const int J = s >> 4;
          const uint32_t ao = (uint32_t)(((I * (I + 1) / 2 + J) * 256 + ((row & 15) + 16 * ((s & 15) >> 2)) * 4 +
                                          (s & 3)) * 2);
          const float av = f16raw(raw16(rA, ao));
          const bf16x8 d8 = lds_ld<bf16x8>(smem, C::DL + td(s, 2 * (c0 + 8 * i)));
#pragma unroll
          for (int k = 0; k < 8; ++k) y[k] -= av * (float)d8[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) part += (float)xb8[k] * y[k];
      }
    }
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) part += __shfl_xor(part, o);
    if (x % NW == 0 && row < nrows) a.dbeta[tok0 + row] = (bf16)(b >= kTinyBeta ? part / (b * b) : part);
  }

  // ------------------------------------------------------------ phase 2
  // Block (R, S), R >= S, of the 64x64 gradients, from row tiles of dO, dv (R)
  // and of Delta (S), contracting over D.
  template <int R, int S>
  __device__ __forceinline__ void p4_tile() {
    bf16x8 fo[NKD], fd[NKD], fdv[NKD];
#pragma unroll
    for (int m = 0; m < NKD; ++m) {
      fo[m] = ar(C::DO, R, m);
      fd[m] = ar(C::DL, S, m);
      fdv[m] = ar(C::DV, R, m);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 a1 = zero4(), a2 = zero4(), a3 = zero4(), a4 = zero4();
#pragma unroll
    for (int m = 0; m < NKD; ++m) {
      a1 = mfma_bf16_k32(a1, fd[m], fo[m]);    // dP[16R + s0][16S + 4g + e]
      a2 = mfma_bf16_k32(a2, fo[m], fd[m]);    // dP[16R + 4g + e][16S + s0]
      a3 = mfma_bf16_k32(a3, fd[m], fdv[m]);   // -Abar[16R + s0][16S + 4g + e]
      a4 = mfma_bf16_k32(a4, fdv[m], fd[m]);   // -Abar[16R + 4g + e][16S + s0]
    }
    f32x4 v1, v2, v3, v4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool lo1 = R > S || s0 >= g4 + e, st1 = R > S || s0 > g4 + e;  // (row s0, col 4g+e)
      const bool lo2 = R > S || g4 + e >= s0, st2 = R > S || g4 + e > s0;  // (row 4g+e, col s0)
      v1[e] = lo1 ? a1[e] : 0.f;
      v2[e] = lo2 ? a2[e] : 0.f;
      v3[e] = st1 ? -a3[e] : 0.f;
      v4[e] = st2 ? -a4[e] : 0.f;
    }
    put16(slot_lo(C::DP, R, S), v1);
    put16(slot_up(C::DPT, S, R), v2);
    put16(slot_lo(C::AB, R, S), v3);
    put16(slot_up(C::ABT, S, R), v4);
  }
  static constexpr int p4_r(int K) {
    const int rr[NP4] = {3, 3, 3, 3, 2, 2, 2, 1, 1, 0};
    return rr[K];
  }
  static constexpr int p4_s(int K) {
    const int ss[NP4] = {3, 2, 1, 0, 2, 1, 0, 1, 0, 0};
    return ss[K];
  }
  // task K (block (p4_r, p4_s)) runs on wave K % NW
  template <int K>
  __device__ __forceinline__ void p4_tasks() {
    if constexpr (K < NP4) {
      if (K % NW == wave) p4_tile<p4_r(K), p4_s(K)>();
      p4_tasks<K + 1>();
    }
  }

  // ------------------------------------------------------------ phase 3
  // fp32 values a (rows 4g+e of one 16-row tile) and b (the next tile) as a
  // 32-deep B fragment over tokens, split into a bf16 part and the bf16 of the
  // remainder: two products with them carry about 16 bits of the operand.
  __device__ __forceinline__ static void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
    hi = pack8(a, b);
    f32x4 ra, rb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ra[e] = a[e] - (float)hi[e];
      rb[e] = b[e] - (float)hi[4 + e];
    }
    lo = pack8(ra, rb);
  }

  // Key column tile j of this wave (columns c = 16 ct + l%16, ct = NCT w + j),
  // start to end: dQh, dKh, dKb (its Delta dU^T part apart) and rowsum(dU . S),
  // then the gate's chain rule.
  //
  // The products with the 64 x 64 gradients (dP Kb, Abar Kb, Abar^T Kh,
  // dP^T Qh) give each pair of tokens (r, s) a term in dg_r and the opposite
  // one in dg_s; the suffix sum over tokens cancels them except for pairs that
  // straddle the token, so their rounding error would pile up against a small
  // result.  Their operands Kb, Kh, Qh are therefore formed here in fp32, at
  // this lane's own positions (tokens 16t + 4g + e of column c: exactly the
  // positions of its B fragments over tokens), and fed as a bf16 part plus the
  // bf16 of the remainder.
  // Phase 3 runs in two parts: what needs only the chunk's tiles and rows of
  // S and dU (phase5a: rowsum(dU . S), the gate, dO S^T, dv S^T, Delta dU^T)
  // goes before the barrier that hands over the 64 x 64 gradients, so that the
  // waves with fewer of those tasks do it while the others finish theirs.
  struct Part3 {
    f32x4 qv[4], kv[4], eg[4], emg[4], dqh[4], dkh[4], dks[4];
    float dgc;
  };
  // The reverse chain keeps dS', so row c of dU = Diag(Gam) dS' is Gam_c =
  // e^(g_C) (column c's gate over the whole chunk) times row c of dS': the
  // products with dU's row below take that factor after the products.
  __device__ __forceinline__ void phase5a(int j, const Pre5& p, Part3& z) {
    // rows c of S and dS' as B fragments over the state's columns, and
    // rowsum(dS' . S) over the lane's positions
    const bf16x8* sr = p.sr[j];
    const bf16x8* ur = p.ur[j];
    float dgc = 0.f;
#pragma unroll
    for (int m = 0; m < NKD; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) dgc = dot2(sr[m], ur[m], e, dgc);
    // rowsum(dS' . S): the four lane groups (l%16 fixed) hold the rest of the row's sum
    dgc += __shfl_xor(dgc, 16);
    dgc += __shfl_xor(dgc, 32);
    // the gate at this lane's positions: g from log_alpha by a prefix over the
    // lane's 4 rows, then over the lane groups and row tiles
    f32x4* qv = z.qv;
    f32x4* kv = z.kv;
    f32x4* eg = z.eg;
    f32x4* emg = z.emg;
    float gam;  // Gam_c
    {
      float tot[4];
      f32x4 gv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float run = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          run += f16raw(p.la[j][4 * t + e]);
          gv[t][e] = run;
          qv[t][e] = f16raw(p.q[j][4 * t + e]);
          kv[t][e] = f16raw(p.k[j][4 * t + e]);
        }
        tot[t] = run;
      }
      float base = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a0 = __shfl(tot[t], s0), a1 = __shfl(tot[t], s0 + 16), a2 = __shfl(tot[t], s0 + 32),
                    a3 = __shfl(tot[t], s0 + 48);
        const float pre = (g4 > 0 ? a0 : 0.f) + (g4 > 4 ? a1 : 0.f) + (g4 > 8 ? a2 : 0.f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gg = (gv[t][e] + base + pre) * G_LOG2E;
          eg[t][e] = __builtin_amdgcn_exp2f(gg);
          emg[t][e] = __builtin_amdgcn_exp2f(-gg);
        }
        base += (a0 + a1) + (a2 + a3);
      }
      gam = __builtin_amdgcn_exp2f(base * G_LOG2E);
    }
    z.dgc = gam * dgc;  // rowsum(dU . S)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 b = zero4(), q = zero4(), h = zero4();
#pragma unroll
      for (int m = 0; m < NKD; ++m) {
        b = mfma_bf16_k32(b, ar(C::DL, t, m), ur[m]);  // Delta dS'^T
        q = mfma_bf16_k32(q, ar(C::DO, t, m), sr[m]);  // dO S^T
        h = mfma_bf16_k32(h, ar(C::DV, t, m), sr[m]);  // dv S^T
      }
      z.dks[t] = gam * b;  // Delta dU^T
      z.dqh[t] = q;
      z.dkh[t] = -h;  // dKh = -dv S^T + ...
    }
  }

  // dQh += dP Kb;  dKh += Abar Kb;  dKb = Abar^T Kh + dP^T Qh (+ dks), then
  // the gate's chain rule
  __device__ __forceinline__ void phase5b(int j, Part3& z) {
    const int c = col(j);
    const f32x4* qv = z.qv;
    const f32x4* kv = z.kv;
    const f32x4* eg = z.eg;
    const f32x4* emg = z.emg;
    f32x4* dqh = z.dqh;
    f32x4* dkh = z.dkh;
    const f32x4* dks = z.dks;
    const float dgc = z.dgc;
    f32x4 dkb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dkb[t] = zero4();
#pragma unroll
    for (int m = 0; m < NKT; ++m) {
      bf16x8 kbH, kbL, khH, khL, qhH, qhL;
      split8(kv[2 * m] * emg[2 * m], kv[2 * m + 1] * emg[2 * m + 1], kbH, kbL);
      split8(kv[2 * m] * eg[2 * m], kv[2 * m + 1] * eg[2 * m + 1], khH, khL);
      split8(qv[2 * m] * eg[2 * m], qv[2 * m + 1] * eg[2 * m + 1], qhH, qhL);
#pragma unroll
      for (int t = 2 * m; t < 4; ++t) {  // m <= t / 2
        const bf16x8 fdp = frlo(C::DP, t, m), fab = frlo(C::AB, t, m);
        dqh[t] = mfma_bf16_k32(dqh[t], fdp, kbH);
        dqh[t] = mfma_bf16_k32(dqh[t], fdp, kbL);
        dkh[t] = mfma_bf16_k32(dkh[t], fab, kbH);
        dkh[t] = mfma_bf16_k32(dkh[t], fab, kbL);
      }
#pragma unroll
      for (int t = 0; t <= 2 * m + 1; ++t) {  // m >= t / 2
        const bf16x8 fabt = frup(C::ABT, t, m), fdpt = frup(C::DPT, t, m);
        dkb[t] = mfma_bf16_k32(dkb[t], fabt, khH);
        dkb[t] = mfma_bf16_k32(dkb[t], fabt, khL);
        dkb[t] = mfma_bf16_k32(dkb[t], fdpt, qhH);
        dkb[t] = mfma_bf16_k32(dkb[t], fdpt, qhL);
      }
    }
    // the gate's chain rule
    float dg[4][4], ps[4][4];  // dg, and k e^-g (Delta dU^T) for the prefix over earlier tokens
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * t + g4 + e;
        const float dq = dqh[t][e] * eg[t][e];
        const float t1 = dkh[t][e] * eg[t][e], t2 = dkb[t][e] * emg[t][e], t3 = dks[t][e] * emg[t][e];
        st_bf16(rdq, row, c, dq);
        st_bf16(rdk, row, c, t1 + t2 + t3);
        dg[t][e] = qv[t][e] * dq + kv[t][e] * (t1 - t2);
        ps[t][e] = kv[t][e] * t3;
      }
    // dlog_alpha_r = sum_{r' >= r} dg_r' + rowsum(dU . S) + sum_{s < r} ps_s: a
    // suffix and an exclusive prefix over the lane's rows, then over the lane
    // groups and row tiles
    float stot[4], ptot[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float run = 0.f, pre = 0.f;
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        run += dg[t][e];
        dg[t][e] = run;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = ps[t][e];
        ps[t][e] = pre;
        pre += x;
      }
      stot[t] = run;
      ptot[t] = pre;
    }
    float after = 0.f, before = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float a0 = __shfl(ptot[t], s0), a1 = __shfl(ptot[t], s0 + 16), a2 = __shfl(ptot[t], s0 + 32),
                  a3 = __shfl(ptot[t], s0 + 48);
      const float pre = (g4 > 0 ? a0 : 0.f) + (g4 > 4 ? a1 : 0.f) + (g4 > 8 ? a2 : 0.f);
#pragma unroll
      for (int e = 0; e < 4; ++e) ps[t][e] += before + pre;
      before += (a0 + a1) + (a2 + a3);
    }
#pragma unroll
    for (int t = 3; t >= 0; --t) {
      const float a0 = __shfl(stot[t], s0), a1 = __shfl(stot[t], s0 + 16), a2 = __shfl(stot[t], s0 + 32),
                  a3 = __shfl(stot[t], s0 + 48);
      const float post = (g4 < 4 ? a1 : 0.f) + (g4 < 8 ? a2 : 0.f) + (g4 < 12 ? a3 : 0.f);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * t + g4 + e;
        st_bf16(rdla, row, c, (dg[t][e] + post + after) + dgc + ps[t][e]);
      }
      after += (a0 + a1) + (a2 + a3);
    }
  }

  __device__ __forceinline__ void run() {
    const int nch = (a.T + GCH - 1) / GCH;
    // Consecutive blockIdx go to different XCDs (round-robin over 8): regroup
    // so that the two halves of a chunk run on one XCD and share its L2.
    const int nwg = gridDim.x;
    int id = blockIdx.x;
    if ((nwg & 7) == 0) id = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    half = id & 1;
    const int unit = id >> 1;
    const int ncnt = (a.n1 < 0 ? nch : a.n1) - a.n0;  // chunks of each head in this launch
    const int bh = unit / ncnt;
    const int n = a.n0 + (unit - bh * ncnt);
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    l = lane_id();
    g4 = 4 * (l >> 4);
    s0 = l & 15;
    nrows = min(GCH, a.T - n * GCH);
    const size_t tok0 = (size_t)bh * a.T + (size_t)n * GCH;
    const uint32_t in_bytes = (uint32_t)nrows * D * 2u;
    rq = make_rsrc(static_cast<const bf16*>(a.q) + tok0 * D, in_bytes);
    rk = make_rsrc(static_cast<const bf16*>(a.k) + tok0 * D, in_bytes);
    rla = make_rsrc(static_cast<const bf16*>(a.la) + tok0 * D, in_bytes);
    rdo = make_rsrc(a.dO ? static_cast<const bf16*>(a.dO) + tok0 * D : nullptr, a.dO ? in_bytes : 0u);
    rdv = make_rsrc(a.dv + tok0 * D, in_bytes);
    rbeta = make_rsrc(static_cast<const bf16*>(a.beta) + tok0, (uint32_t)nrows * 2u);
    rdq = make_rsrc(a.dq + tok0 * D, in_bytes);
    rdk = make_rsrc(a.dk + tok0 * D, in_bytes);
    rdla = make_rsrc(a.dla + tok0 * D, in_bytes);
    // the chunk's checkpoints from the forward pass and the reverse chain (W,
    // Xbar and A are read only for rows with beta below kTinyBeta)
    const size_t ck = (size_t)bh * nch + n;
    rSr = make_rsrc(a.S_rows + ck * D * D, D * D * 2u);
    rUr = make_rsrc(a.dSp_rows + ck * D * D, D * D * 2u);
    rW = make_rsrc(a.W + ck * GCH * D, GCH * D * 2u);
    rDl = make_rsrc(a.Dl + ck * GCH * D, GCH * D * 2u);
    rXb = make_rsrc(a.Xb + ck * GCH * D, GCH * D * 2u);
    rA = make_rsrc(a.A + ck * NP4 * 256, NP4 * 256 * 2u);
    const bool db = half == 0;  // this workgroup writes dbeta
    init_offsets();
    Pre5 p5;
    load_pre5(p5);
    // zero halves of the 32-deep slots that pair a block of the upper triangle
    // with a stored one (nothing writes them): dP and Abar slots (0, 0) and
    // (2, 1), second half; dP^T and Abar^T slots (1, 0) and (3, 1), first half
    for (int t = threadIdx.x; t < 64 * 2 * 4; t += C::THREADS) {
      const int which = t >> 7, lane = t & 63, sel = (t >> 6) & 1;
      uint32_t off;
      if (which < 2) {
        const uint32_t base = which == 0 ? C::DP : C::AB;
        off = base + (uint32_t)(((sel ? lo_idx(2, 1) : lo_idx(0, 0)) * 64 + lane) * 16 + 8);
      } else {
        const uint32_t base = which == 2 ? C::DPT : C::ABT;
        off = base + (uint32_t)(((sel ? up_idx(3, 1) : up_idx(1, 0)) * 64 + lane) * 16);
      }
      lds_st<u32x2>(smem, off, u32x2{0u, 0u});
    }
    if (wave == 0) {
      const float b = __uint_as_float((uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rbeta, 2 * l, 0, 0) << 16);
      lds_st<float>(smem, C::BETA + 4 * l, b);
    }
    copy_tiles();
    sync_lds();
    p4_tasks<0>();
    if (db) dbeta_rows(tok0);
    Part3 z[NCT];
#pragma unroll
    for (int j = 0; j < NCT; ++j) phase5a(j, p5, z[j]);
    sync_lds();
#pragma unroll
    for (int j = 0; j < NCT; ++j) phase5b(j, z[j]);
  }
};

template <int D>
__global__ __launch_bounds__(GradCfg<D>::THREADS, 2) void kda_bwgrad_kernel(BwGradArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GradCfg<D>::LDS];
  GradKernel<D> k;
  k.smem = smem;
  k.a = a;
  k.run();
}

}  // namespace

hipError_t launch_bwgrad(const BwGradArgs& a, int BH, int D, hipStream_t stream) {
  const long long nch = (a.T + GCH - 1) / GCH;
  const long long n1 = a.n1 < 0 ? nch : a.n1;
  if (a.n0 < 0 || n1 > nch || a.n0 > n1) return hipErrorInvalidValue;
  const long long nwg = 2LL * BH * (n1 - a.n0);  // two workgroups (column halves) per (head, chunk)
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
  if (D == 128) {
    hipLaunchKernelGGL(kda_bwgrad_kernel<128>, dim3((unsigned)nwg), dim3(GradCfg<128>::THREADS), 0, stream, a);
  } else if (D == 64) {
    hipLaunchKernelGGL(kda_bwgrad_kernel<64>, dim3((unsigned)nwg), dim3(GradCfg<64>::THREADS), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kda
