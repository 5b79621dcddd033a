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
//   Qh = q*e^g, Kh = k*e^g, Kb = k*e^-g, Gam = e^(g_C)  (g_C: last row),
//   L = diag(b) strict_lower(Kh Kb^T),  P = lower(Qh Kb^T).
// Unrolling the recurrence over the chunk gives exactly
//   (I + L) Delta = diag(b) (V - Kh S),
//   O = Qh S + P Delta,   S' = Diag(Gam) (S + Kb^T Delta).
// Only the last three depend on S.  The unit lower triangular system is solved
// by 16-row blocks: Delta_i = T_ii (b X_i - sum_{j<i} L_ij Delta_j) with the
// diagonal-block inverses T_ii = (I + L_ii)^-1 computed in advance.  With
// log a >= -1 the factors e^{+-g} stay within [e^-64, e^64] inside a chunk, far
// from the fp32/bf16 range limits.
//
// Work split.  Columns of S evolve independently once the S-independent
// products are known, so a workgroup owns 16*NC state columns of one
// sequence (segment).  Inside a workgroup:
//   * NC consumer waves each hold a dk x 16 column slice of S in fp32 MFMA
//     accumulators and run the serial chain;
//   * NP = dk/32 producer waves load the next chunk and compute its decayed
//     operand tiles.  The pages describe FlashKDA as splitting intra-chunk work
//     and state passing between two independently scheduled thread groups
//     (same section); here the two roles are wavefronts of one workgroup.
// Each chunk takes two workgroup barriers: interval 1 has the producers build
// chunk n+1's elementwise tiles while the consumers run the whole chain of
// chunk n; in interval 2 every wave takes its share of chunk n+1's score tiles
// and diagonal inverses.  Operand tiles live in a double-buffered LDS stage.
// The fp32 variant has no room for two stages and runs the phases in turn.
//
// All global traffic goes through buffer descriptors sized to the sequence, so
// rows past its end read as zero and stores to them are dropped: a ragged last
// chunk needs no branches (zero k, q, log-gate and beta rows leave the state
// and the valid outputs unchanged).
//
// Segment mode runs the same chain on the augmented state [S | M] started at
// [0 | I] (columns >= dv see v = 0), skips q, P and O, and writes S and M.
//
// Prefill can also write the state at every snapshot boundary (a multiple of
// the chunk length, counted over the head's whole sequence): the KDA state of a
// request is kept only at a sparse subset of the 512-token prefix-cache block
// boundaries ("Kimi K3 开源日来了", section "针对适配的 Infra").  The consumer
// waves store their columns of S right after the chunk that closes a boundary.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int CH = 64;  // chunk length
constexpr float LOG2E = 1.4426950408889634f;

template <typename T, int D, int NC, bool PREFILL>
struct ChunkCfg {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int ES = sizeof(T);
  static constexpr int STAGES = BF ? 2 : 1;
  static constexpr int LAG = STAGES - 1;
  static constexpr int NCT = BF ? 2 : 1;   // 16-column state tiles per consumer wave
  static constexpr int NP = D / 32;
  static constexpr int NW = NC + NP;
  static constexpr int THREADS = 64 * NW;
  static constexpr int R_TD = D * ES;      // [CH][D] rows (time-major)
  // [CH][D] tiles are stored as four 16-row blocks, each 16 bytes further along
  // the banks than the previous one, so that the producer's stores (rows 4 apart)
  // do not pile onto the same banks.
  static constexpr int TD_TILE = 16 * R_TD + 16;
  static constexpr int TD_SZ = 4 * TD_TILE;
  static constexpr int R_DT = CH * ES;     // [D][CH] rows (channel-major)
  // Tiles the consumer reads only as MFMA A fragments (-L, P, T_ii) are stored in
  // fragment order: 16-byte lane slots, lane l's slot holding exactly the values
  // its fragment needs, so each fragment is one contiguous, conflict-free read.
  static constexpr int KB = BF ? 32 : 16;  // MFMA depth of the dense products
  static constexpr int JPB = KB / 16;      // 16x16 tiles per 16-byte lane slot of P
  static constexpr int FR16 = 64 * 4 * ES; // one 16x16 tile as 16-deep fragments
  // stage: everything the chain of one chunk reads.  bf16: Kb is kept
  // time-major only; the chain reads it as Kb^T with transposing LDS reads.
  // fp32 (no 16-bit transposing read): a channel-major copy Kb^T sits in the
  // stage and the time-major Kb, which only the score tiles read, in scratch.
  static constexpr uint32_t S_KH = 0;                                   // Kh   [CH][D]
  static constexpr uint32_t S_QH = S_KH + TD_SZ;                        // Qh   [CH][D]
  static constexpr uint32_t S_KB = S_QH + (PREFILL ? TD_SZ : 0);        // Kb [CH][D] (bf16) / Kb^T [D][CH]
  static constexpr uint32_t S_L = S_KB + (BF ? TD_SZ : D * R_DT);       // -L_IJ, J < I: 6 x FR16
  static constexpr uint32_t S_P = S_L + 6 * FR16;                       // P: [4][CH/KB][64] slots
  static constexpr uint32_t S_TI = S_P + (PREFILL ? 4 * (CH / KB) * 64 * 16 : 0);  // T_ii: 4 x FR16
  static constexpr uint32_t S_GM = S_TI + 4 * FR16;                     // Gam  [D] fp32
  static constexpr uint32_t S_BETA = S_GM + D * 4;                      // beta [CH] fp32
  static constexpr uint32_t STAGE = S_BETA + CH * 4;
  // Kb time-major for the score products: in the stage (bf16) or in producer
  // scratch after the stages (fp32)
  static constexpr uint32_t X_KB = STAGES * STAGE;
  static constexpr uint32_t LDS = X_KB + (BF ? 0 : TD_SZ);
  // where the score products find Kb of the chunk in stage st
  __device__ __forceinline__ static uint32_t kb_td(uint32_t st) { return BF ? st + S_KB : X_KB; }
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(LDS % 16 == 0 && STAGE % 16 == 0, "LDS alignment");
};

// Producer input registers for one chunk: 4 token rows x 8 channels of
// log_alpha, k and q, plus one beta per lane (raw bits).
template <typename T> struct ProdRaw {
  Raw8<T> la[4], k[4], q[4];
  uint32_t beta;
};

// Value rows of one chunk for a consumer lane (accumulator layout): 16 rows,
// as loaded (bf16: the lane's two adjacent columns in one dword; fp32: one
// value).  Kept raw so that the prefetch is not waited on until it is used.
struct VRaw { uint32_t r[16]; };

// Operand fragments.  bf16: one v_mfma_f32_16x16x32_bf16 per 32-deep k block;
// fp32: four v_mfma_f32_16x16x4_f32 steps per 16-deep k block.  "ar" fragments
// are LDS A operands against B operands held as accumulator tiles (bf16 tiles
// stored in kpos order, so one 16-byte read per lane); "ll" fragments read both
// operands from LDS, 8 (bf16) or 4 (fp32) consecutive stored positions per lane,
// which is a valid contraction as long as both tiles use the same order.
template <bool BF> struct Frag;
template <> struct Frag<true> {
  typedef bf16x8 A;
  typedef bf16x8 B;
  typedef bf16x4 A16;
  static constexpr int KB = 32;
  __device__ __forceinline__ static B bfrag(const f32x4* t, int m) { return pack8(t[2 * m], t[2 * m + 1]); }
  __device__ __forceinline__ static f32x4 mma(f32x4 acc, A a, B b) { return mfma_bf16_k32(acc, a, b); }
  __device__ __forceinline__ static f32x4 mma16(f32x4 acc, A16 a, f32x4 b) {
    return mfma_bf16_k16(acc, a, pack4(b));
  }
  // an accumulator tile as a 16-deep A operand (it then stands for its transpose)
  __device__ __forceinline__ static A16 a16(f32x4 t) { return pack4(t); }
};
template <> struct Frag<false> {
  typedef f32x4 A;
  typedef f32x4 B;
  typedef f32x4 A16;
  static constexpr int KB = 16;
  __device__ __forceinline__ static B bfrag(const f32x4* t, int m) { return t[m]; }
  __device__ __forceinline__ static f32x4 mma(f32x4 acc, A a, B b) {
    acc = mfma_f32_k4(acc, a[0], b[0]);
    acc = mfma_f32_k4(acc, a[1], b[1]);
    acc = mfma_f32_k4(acc, a[2], b[2]);
    return mfma_f32_k4(acc, a[3], b[3]);
  }
  __device__ __forceinline__ static f32x4 mma16(f32x4 acc, A16 a, f32x4 b) { return mma(acc, a, b); }
  __device__ __forceinline__ static A16 a16(f32x4 t) { return t; }
};

template <typename T, int D, int NC, bool PREFILL, bool BWD = false, bool CKPT = false>
struct ChunkKernel {
  // BWD: the reverse chain of the prefill's gradients (see chain_bw); it uses
  // the prefill's stage layout and producer, visits the chunks last to first,
  // and is built for bf16 inputs (its transposed operands use the 16-bit
  // transposing LDS read).
  // CKPT: the prefill run only for the gradients' checkpoints: no outputs, so
  // neither q nor Qh nor the P tiles.
  static_assert(!BWD || (PREFILL && sizeof(T) == 2), "the backward chain is a bf16 prefill-layout mode");
  static_assert(!CKPT || (PREFILL && !BWD && sizeof(T) == 2), "the checkpoint pass is a bf16 prefill mode");
  static constexpr bool QP = PREFILL && !CKPT;  // q, Qh, P and the outputs are used
  using C = ChunkCfg<T, D, NC, PREFILL>;
  using F = Frag<C::BF>;
  typedef typename F::A16 A16;
  static constexpr int KB = F::KB;
  static constexpr int NKD = D / KB;    // k blocks over channels
  static constexpr int NKT = CH / KB;   // k blocks over the tokens of a chunk
  // stored position of k in tiles read as "ar" A operands
  static constexpr int kp(int k) { return C::BF ? kpos(k) : k; }
  // byte offset of (row, byte) in a [CH][D] tile
  __device__ __forceinline__ static uint32_t td(int row, int byte) {
    return (uint32_t)(row >> 4) * C::TD_TILE + swz<C::R_TD>(row & 15, byte);
  }
  // last k block a lower-triangular row tile ti touches
  static constexpr int tri(int ti) { return (16 * ti + 15) / KB; }
  char* smem;
  ChunkArgs a;
  rsrc_t rq, rk, rv, rla, rbeta, ro;
  int Tlen, nch;
  bf16* ck_w;        // this chunk's checkpoints of W = V - Kh S (rows with tiny beta
  bf16* ck_d;        // only) and Delta (prefill with gradient checkpoints), else null
  int chunk0;        // chunks of the head's sequence before this segment
  size_t ck0;        // gradients' checkpoints: index of this segment's first chunk
  float* snap_head;  // snapshot 0 of this head (prefill with snapshots), else null
  int wave, l;
  // consumer: NCT adjacent 16-column tiles of the state, sharing every A fragment
  static constexpr int NCT = C::NCT;
  int colb;         // global column of this lane in tile 0 (tile j: colb + j, so a
                    // lane's columns are adjacent and move as one 4-byte bf16 pair)
  bool isv;         // columns read v (value columns) rather than being map columns
  bool mskip;       // segment pass: this wave owns map columns and may stop on zero
  bool mzero;       // ... and they have all become exactly zero
  f32x4 S[NCT][D / 16];
  typename F::B sb[NCT][NKD], db[NCT][NKT];
  u32x4 dvq[4];  // reverse chain: the chunk's dv row pieces, stored after the first barrier
  // Per-lane LDS byte offsets of the consumer's A fragments inside a tile of
  // each row size, for row tile 0 (the swizzle term depends only on the lane's
  // row within 16, so row tile t adds 16*t*rowbytes).  [k block]
  // (token-by-token tiles and channel-by-token tiles have the same row size.)
  uint32_t oTD[NKD], oDT[NKT];
  // bf16: per-lane LDS byte offsets of the transposing reads of Kb^T fragments,
  // for row tile pair a (channels 32a .. 32a+31), row tile 0 of the time-major Kb
  uint32_t oTR[D / 32];

  __device__ __forceinline__ uint32_t stage(int chunk) const {
    return (C::STAGES == 2 ? (uint32_t)(chunk & 1) : 0u) * C::STAGE;
  }

  // The chunk that pipeline step `it` works on: the chunks in order, or last to
  // first for the backward chain.  Steps past the end map to chunk indices past
  // either end of the sequence, whose loads (negative offsets become offsets
  // beyond any buffer's size) read zero.
  __device__ __forceinline__ int chunk_of(int it) const { return BWD ? nch - 1 - it : it; }

  // ------------------------------------------------------------ producers
  // Lane (tg = l%16, cs = l/16) of producer wave pw owns tokens 4*tg..4*tg+3 and
  // channels 32*pw + 8*cs .. +7 of the chunk; a channel's 16 token groups are
  // one DPP row, so the prefix sum over tokens runs on row operations.
  // byte offset of token row i of the lane's token group, first of its channels
  __device__ __forceinline__ uint32_t prod_off(int it, int i) const {
    const int ln = fresh_lane(l);
    const int ch = 32 * (wave - NC) + 8 * (ln >> 4);
    return (uint32_t)((chunk_of(it) * CH + 4 * (ln & 15) + i) * D + ch) * C::ES;
  }
  __device__ __forceinline__ void load_la(ProdRaw<T>& r, int chunk) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw_load<T>(r.la[i], rla, prod_off(chunk, i));
  }
  __device__ __forceinline__ void load_kq(ProdRaw<T>& r, int chunk, int i) const {
    raw_load<T>(r.k[i], rk, prod_off(chunk, i));
    if constexpr (QP) raw_load<T>(r.q[i], rq, prod_off(chunk, i));
  }
  __device__ __forceinline__ void load_beta(ProdRaw<T>& r, int chunk) const {
    if (wave == NC) {
      const uint32_t off = (uint32_t)(chunk_of(chunk) * CH + fresh_lane(l)) * C::ES;
      if constexpr (C::BF) r.beta = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rbeta, off, 0, 0);
      else r.beta = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rbeta, off, 0, 0);
    }
  }
  __device__ __forceinline__ void load_raw(ProdRaw<T>& r, int chunk) const {
    load_la(r, chunk);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_kq(r, chunk, i);
    load_beta(r, chunk);
  }

  // Phase 1: cumulative log-gate and the decayed operand tiles of one chunk.
  // bf16 inputs: the gate is accumulated in log2 units and exponentiated with
  // the hardware exp2; fp32 inputs use the accurate library exp.
  // Each register of r is refilled with chunk `next` as soon as it has been
  // read, so the prefetch loads issue spread over this VALU-heavy phase rather
  // than in one burst.
  // The lane's LDS store offsets of phase 1, fixed for the whole loop:
  // [token row i][channel half] in the [CH][D] tiles, and per channel in Kb^T.
  uint32_t p_td[4][2], p_kt[8];
  __device__ __forceinline__ void init_p1_offsets() {
    const int ln = fresh_lane(l);
    const int tg = ln & 15;
    const int ch = 32 * (wave - NC) + 8 * (ln >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf)
        p_td[i][hlf] = C::BF ? td(4 * tg + i, 2 * kp(ch + 4 * hlf)) : td(4 * tg + i, 4 * (ch + 4 * hlf));
#pragma unroll
    for (int c = 0; c < 8; ++c)
      p_kt[c] = C::BF ? 0u : swz<C::R_DT>(ch + c, 4 * 4 * tg);  // (fp32 only)
  }

  __device__ __forceinline__ void p1(ProdRaw<T>& r, uint32_t st, int next) {
    const int ln = fresh_lane(l);
    const int pw = wave - NC;
    const int tg = ln & 15, cs = ln >> 4;
    const int ch = 32 * pw + 8 * cs;
    float g[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      raw_f32<T>(r.la[i], g[i]);
      if constexpr (C::BF) {
#pragma unroll
        for (int c = 0; c < 8; ++c) g[i][c] *= LOG2E;
      }
    }
    load_la(r, next);
    float exc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      g[1][c] += g[0][c];
      g[2][c] += g[1][c];
      g[3][c] += g[2][c];
      // inclusive prefix of the 4-token totals over the 16 token groups of the row
      float x = g[3][c];
      x += dpp<DPP_ROW_SHR + 1>(x);
      x += dpp<DPP_ROW_SHR + 2>(x);
      x += dpp<DPP_ROW_SHR + 4>(x);
      x += dpp<DPP_ROW_SHR + 8>(x);
      exc[c] = dpp<DPP_ROW_SHR + 1>(x);
    }
    // e^g of the chunk's last token (row 3 of token group 15) is Gam
    float eg3[8];
    float kb[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float kk[8], qq[8], vq[8], vkh[8];
      raw_f32<T>(r.k[i], kk);
      if constexpr (QP) raw_f32<T>(r.q[i], qq);
      load_kq(r, next, i);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float gg = g[i][c] + exc[c];
        float eg, emg;
        if constexpr (C::BF) {
          eg = __builtin_amdgcn_exp2f(gg);
          emg = __builtin_amdgcn_exp2f(-gg);
        } else {
          eg = expf(gg);
          emg = expf(-gg);
        }
        if (i == 3) eg3[c] = eg;
        vkh[c] = kk[c] * eg;
        kb[i][c] = kk[c] * emg;
        if constexpr (QP) vq[c] = qq[c] * eg;
      }
      if constexpr (C::BF) {
        // channels ch..ch+3 and ch+4..ch+7 go to their stored positions
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          bf16x4 h, b, qv;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            h[c] = (bf16)vkh[4 * hlf + c];
            b[c] = (bf16)kb[i][4 * hlf + c];
            if constexpr (QP) qv[c] = (bf16)vq[4 * hlf + c];
          }
          const uint32_t o = p_td[i][hlf];
          lds_st<bf16x4>(smem, st + C::S_KH + o, h);
          lds_st<bf16x4>(smem, st + C::S_KB + o, b);
          if constexpr (QP) lds_st<bf16x4>(smem, st + C::S_QH + o, qv);
        }
      } else {
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          f32x4 h = {vkh[4 * hlf], vkh[4 * hlf + 1], vkh[4 * hlf + 2], vkh[4 * hlf + 3]};
          f32x4 b = {kb[i][4 * hlf], kb[i][4 * hlf + 1], kb[i][4 * hlf + 2], kb[i][4 * hlf + 3]};
          lds_st<f32x4>(smem, st + C::S_KH + p_td[i][hlf], h);
          lds_st<f32x4>(smem, C::X_KB + p_td[i][hlf], b);
          if constexpr (QP) {
            f32x4 qv = {vq[4 * hlf], vq[4 * hlf + 1], vq[4 * hlf + 2], vq[4 * hlf + 3]};
            lds_st<f32x4>(smem, st + C::S_QH + p_td[i][hlf], qv);
          }
        }
      }
    }
    // fp32: Kb^T, channel-major, 4 consecutive tokens per lane and channel
    if constexpr (!C::BF) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f32x4 t4 = {kb[0][c], kb[1][c], kb[2][c], kb[3][c]};
        lds_st<f32x4>(smem, st + C::S_KB + p_kt[c], t4);
      }
    }
    if (tg == 15) {
#pragma unroll
      for (int c = 0; c < 8; ++c) lds_st<float>(smem, st + C::S_GM + 4 * (ch + c), eg3[c]);
    }
    if (pw == 0) {
      const float b = C::BF ? __uint_as_float(r.beta << 16) : __uint_as_float(r.beta);
      lds_st<float>(smem, st + C::S_BETA + 4 * ln, b);
    }
    load_beta(r, next);
  }

  // Phase 2, one tile task: block (I, J), J <= I, of the score matrix M = X Kb^T
  // with X = Kh (L, MAT 0) or Qh (P, MAT 1).  The product is taken transposed
  // (A = Kb rows, B = X rows), so lane l ends up holding M[16I + l%16][16J + 4g + e]
  // (g = l/16): exactly its A fragment for the consumer.
  //   MAT 0, J < I : stores -L = -diag(b) M (all strictly lower)
  //   MAT 1        : stores P = lower(M)
  //   MAT 0, J = I : N = L_II (strictly lower), and T_ii = (I + N)^-1 as the exact
  //                  product (I - N)(I + N^2)(I + N^4)(I + N^8) of commuting factors,
  //                  computed in registers.  An accumulator tile of X, used as an A
  //                  operand, stands for X^T; used as a B operand, for X.  Keeping
  //                  both N and N^T as accumulators gives every power and its
  //                  transpose, and Z = T_ii^T = (I + N^T)^-1 is accumulated as
  //                  Z += (N^T)^(2^k) Z from Z = I - N^T.  Z is T_ii's A fragment.
  template <int MAT, int I, int J>
  __device__ __forceinline__ void p2_tile(uint32_t st, int it) {
    constexpr bool DIAG = MAT == 0 && I == J;
    const int ln = fresh_lane(l);
    const int g4 = 4 * (ln >> 4), s0 = ln & 15;
    const uint32_t xbase = (MAT ? st + C::S_QH : st + C::S_KH) + I * C::TD_TILE;
    typename F::A fx[NKD], fb[NKD];
#pragma unroll
    for (int m = 0; m < NKD; ++m) {
      // row s0 of row tile I (J), stored k positions of the lane group: the
      // consumer's fragment offsets (both operands read the same positions,
      // which is a valid contraction in any consistent order)
      fx[m] = lds_ld<typename F::A>(smem, xbase + oTD[m]);
      fb[m] = lds_ld<typename F::A>(smem, C::kb_td(st) + J * C::TD_TILE + oTD[m]);
    }
    float bl = 0.f;
    f32x4 bet4 = zero4();
    if constexpr (MAT == 0) bl = lds_ld<float>(smem, st + C::S_BETA + 4 * (16 * I + s0));
    if constexpr (DIAG) bet4 = lds_ld<f32x4>(smem, st + C::S_BETA + 4 * (16 * I + g4));
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = zero4();
#pragma unroll
    for (int m = 0; m < NKD; ++m) acc = F::mma(acc, fb[m], fx[m]);
    if constexpr (PREFILL && !BWD && C::BF && MAT == 0) {
      // the gradients' checkpoint of this block of strict_lower(Kh Kb^T), for
      // the lane's row (16I + l%16) only if its beta is below kTinyBeta
      if (a.ck_a && bl < kTinyBeta) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (!DIAG || g4 + e < s0) ? acc[e] : 0.f;
        const size_t o = ((ck0 + it) * 10 + I * (I + 1) / 2 + J) * 256 + ln * 4;
        *reinterpret_cast<bf16x4*>(a.ck_a + o) = pack4(v);
      }
    }
    if constexpr (MAT == 0 && !DIAG) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = -bl * acc[e];
      put_frag(st + C::S_L + (I * (I - 1) / 2 + J) * C::FR16 + ln * 4 * C::ES, v);
    } else if constexpr (MAT == 1) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (J < I || g4 + e <= s0) ? acc[e] : 0.f;
      put_frag(st + C::S_P + ((I * (CH / KB) + J / C::JPB) * 64 + ln) * 16 + (J % C::JPB) * 4 * C::ES, v);
    } else {
      f32x4 an = zero4();
#pragma unroll
      for (int m = 0; m < NKD; ++m) an = F::mma(an, fx[m], fb[m]);
      f32x4 Nt, Nn, Z;  // acc(N^T), acc(N), acc(Z)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Nt[e] = g4 + e < s0 ? bl * acc[e] : 0.f;     // N[16I + s0][16I + g4 + e]
        Nn[e] = s0 < g4 + e ? bet4[e] * an[e] : 0.f;  // N[16I + g4 + e][16I + s0]
        Z[e] = (g4 + e == s0 ? 1.f : 0.f) - Nt[e];
      }
      const f32x4 N2 = F::mma16(zero4(), F::a16(Nt), Nn);    // N N
      const f32x4 Nt2 = F::mma16(zero4(), F::a16(Nn), Nt);   // N^T N^T
      Z = F::mma16(Z, F::a16(N2), Z);                        // Z += (N^T)^2 Z
      const f32x4 N4 = F::mma16(zero4(), F::a16(Nt2), N2);   // N^2 N^2
      const f32x4 Nt4 = F::mma16(zero4(), F::a16(N2), Nt2);  // (N^T)^2 (N^T)^2
      Z = F::mma16(Z, F::a16(N4), Z);                        // Z += (N^T)^4 Z
      const f32x4 N8 = F::mma16(zero4(), F::a16(Nt4), N4);   // N^4 N^4
      Z = F::mma16(Z, F::a16(N8), Z);                        // Z += (N^T)^8 Z
      put_frag(st + C::S_TI + I * C::FR16 + ln * 4 * C::ES, Z);
    }
  }

  // 4 values of a 16-deep fragment into its lane slot (bf16: 8 bytes, fp32: 16)
  __device__ __forceinline__ void put_frag(uint32_t off, const f32x4& v) {
    if constexpr (C::BF) lds_st<bf16x4>(smem, off, pack4(v));
    else lds_st<f32x4>(smem, off, v);
  }

  // Phase-2 tasks: the four diagonal L blocks (with their inverses, about twice
  // the work of a tile) first, then the P tiles (prefill only), then the
  // off-diagonal L tiles.  Each task goes to the wave with the least work so far
  // (greedy, at compile time), every wave of the workgroup taking part.  When
  // the consumers compute the previous chunk's outputs in this interval
  // (DEFER_O), or the reverse chain's consumers store dS' and dv in it
  // (DSP_LATE), each consumer wave starts with that step's weight.
  static constexpr int NT2 = QP ? 20 : 10;
  static constexpr int task_wave(int K) {
    int load[C::NW] = {};
    if (DEFER_O || DSP_LATE)
      for (int i = 0; i < NC; ++i) load[i] = DEFER_O ? kOutWeight : kStoreWeight;
    int w = 0;
    for (int k = 0; k <= K; ++k) {
      w = 0;
      for (int i = 1; i < C::NW; ++i)
        if (load[i] < load[w]) w = i;
      load[w] += k < 4 ? 2 : 1;
    }
    return w;
  }
  static constexpr int task_mat(int K) { return K < 4 ? 0 : (QP && K < 14 ? 1 : 0); }
  static constexpr int task_i(int K) {
    if (K < 4) return K;
    int k = K - 4;
    if (QP) {
      if (k < 10) {
        const int ii[10] = {3, 3, 3, 3, 2, 2, 2, 1, 1, 0};
        return ii[k];
      }
      k -= 10;
    }
    const int io[6] = {3, 3, 3, 2, 2, 1};
    return io[k];
  }
  static constexpr int task_j(int K) {
    if (K < 4) return K;
    int k = K - 4;
    if (QP) {
      if (k < 10) {
        const int jj[10] = {3, 2, 1, 0, 2, 1, 0, 1, 0, 0};
        return jj[k];
      }
      k -= 10;
    }
    const int jo[6] = {2, 1, 0, 1, 0, 0};
    return jo[k];
  }

  template <int K>
  __device__ __forceinline__ void p2_task(uint32_t st, int it) {
    if constexpr (K < NT2) {
      constexpr int W = task_wave(K);  // evaluated at compile time
      if (W == wave) p2_tile<task_mat(K), task_i(K), task_j(K)>(st, it);
      p2_task<K + 1>(st, it);
    }
  }

  // it: the chunk whose tiles are built (its index in the segment)
  __device__ __forceinline__ void p2(uint32_t st, int it) {
    if constexpr (BWD) p2_task_bw<0>(st);
    else p2_task<0>(st, it);
  }
  // ------------------------------------------------ backward-chain tile tasks
  // The reverse chain needs the transposes of the forward's A operands: P^T,
  // L^T and T_ii^T.  Block (I, J) of M = X Kb^T (X = Kh or Qh) is computed
  // with A = X rows of row tile I and B = Kb rows of row tile J, so that lane l
  // holds M[16I + 4g + e][16J + l%16] (g = l/16): the accumulator layout of
  // M_IJ, which is exactly the A fragment of M_IJ^T.
  //   MAT 0, I > J : -L_IJ^T (L = diag(b) strict_lower(Kh Kb^T)), slot I(I-1)/2 + J
  //   MAT 1, I >= J: P_IJ^T (P = lower(Qh Kb^T)) in the 32-deep slot of row tile J,
  //                  token block I / 2 (half I % 2)
  //   MAT 0, I = J : T_ii as an accumulator tile (the A fragment of T_ii^T), from
  //                  N = L_ii: T_ii = (I - N)(I + N^2)(I + N^4)(I + N^8), accumulated
  //                  as Z += N^(2^k) Z; N^(2^k) as an A operand is the A fragment
  //                  of the accumulator of (N^T)^(2^k).
  template <int MAT, int I, int J>
  __device__ __forceinline__ void p2_tile_bw(uint32_t st) {
    constexpr bool DIAG = MAT == 0 && I == J;
    const int ln = fresh_lane(l);
    const int g4 = 4 * (ln >> 4), s0 = ln & 15;
    const uint32_t xbase = (MAT ? st + C::S_QH : st + C::S_KH) + I * C::TD_TILE;
    typename F::A fx[NKD], fb[NKD];
#pragma unroll
    for (int m = 0; m < NKD; ++m) {
      fx[m] = lds_ld<typename F::A>(smem, xbase + oTD[m]);
      fb[m] = lds_ld<typename F::A>(smem, C::kb_td(st) + J * C::TD_TILE + oTD[m]);
    }
    f32x4 bet4 = zero4();
    float bl = 0.f;
    if constexpr (MAT == 0) bet4 = lds_ld<f32x4>(smem, st + C::S_BETA + 4 * (16 * I + g4));
    if constexpr (DIAG) bl = lds_ld<float>(smem, st + C::S_BETA + 4 * (16 * I + s0));
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = zero4();
#pragma unroll
    for (int m = 0; m < NKD; ++m) acc = F::mma(acc, fx[m], fb[m]);
    if constexpr (MAT == 0 && !DIAG) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = -bet4[e] * acc[e];
      put_frag(st + C::S_L + (I * (I - 1) / 2 + J) * C::FR16 + ln * 4 * C::ES, v);
    } else if constexpr (MAT == 1) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (I > J || g4 + e >= s0) ? acc[e] : 0.f;
      put_frag(st + C::S_P + ((J * NKT + I / C::JPB) * 64 + ln) * 16 + (I % C::JPB) * 4 * C::ES, v);
    } else {
      f32x4 at = zero4();
#pragma unroll
      for (int m = 0; m < NKD; ++m) at = F::mma(at, fb[m], fx[m]);
      f32x4 Nt, Nn, Z;  // acc(N^T), acc(N), acc(T_ii)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Nn[e] = s0 < g4 + e ? bet4[e] * acc[e] : 0.f;  // N[16I + g4 + e][16I + s0]
        Nt[e] = g4 + e < s0 ? bl * at[e] : 0.f;       // N[16I + s0][16I + g4 + e]
        Z[e] = (g4 + e == s0 ? 1.f : 0.f) - Nn[e];
      }
      const f32x4 N2 = F::mma16(zero4(), F::a16(Nt), Nn);    // N N
      const f32x4 Nt2 = F::mma16(zero4(), F::a16(Nn), Nt);   // N^T N^T
      Z = F::mma16(Z, F::a16(Nt2), Z);                       // Z += N^2 Z
      const f32x4 N4 = F::mma16(zero4(), F::a16(Nt2), N2);   // N^2 N^2
      const f32x4 Nt4 = F::mma16(zero4(), F::a16(N2), Nt2);  // (N^T)^2 (N^T)^2
      Z = F::mma16(Z, F::a16(Nt4), Z);                       // Z += N^4 Z
      const f32x4 Nt8 = F::mma16(zero4(), F::a16(N4), Nt4);  // (N^T)^4 (N^T)^4
      Z = F::mma16(Z, F::a16(Nt8), Z);                       // Z += N^8 Z
      put_frag(st + C::S_TI + I * C::FR16 + ln * 4 * C::ES, Z);
    }
  }

  // The same 20 tasks as the forward's (4 diagonal, 10 P, 6 off-diagonal L),
  // with the same greedy balance over the waves.
  static constexpr int task_i_bw(int K) {
    if (K < 4) return K;
    int k = K - 4;
    if (k < 10) {
      const int ii[10] = {3, 3, 3, 3, 2, 2, 2, 1, 1, 0};
      return ii[k];
    }
    const int io[6] = {3, 3, 3, 2, 2, 1};
    return io[k - 10];
  }
  static constexpr int task_j_bw(int K) {
    if (K < 4) return K;
    int k = K - 4;
    if (k < 10) {
      const int jj[10] = {3, 2, 1, 0, 2, 1, 0, 1, 0, 0};
      return jj[k];
    }
    const int jo[6] = {2, 1, 0, 1, 0, 0};
    return jo[k - 10];
  }
  template <int K>
  __device__ __forceinline__ void p2_task_bw(uint32_t st) {
    if constexpr (K < 20) {
      constexpr int W = task_wave(K);
      if (W == wave) p2_tile_bw<(K >= 4 && K < 14) ? 1 : 0, task_i_bw(K), task_j_bw(K)>(st);
      p2_task_bw<K + 1>(st);
    }
  }


  // ------------------------------------------------------------ consumers
  __device__ __forceinline__ void init_offsets() {
    const int r16 = l & 15;
    // the lane group's k positions start at stored position KB/4 * group
    const int kg = (KB / 4) * (l >> 4);
#pragma unroll
    for (int m = 0; m < NKD; ++m) oTD[m] = swz<C::R_TD>(r16, C::ES * (KB * m + kg));
#pragma unroll
    for (int m = 0; m < NKT; ++m) oDT[m] = swz<C::R_DT>(r16, C::ES * (KB * m + kg));
    if constexpr (C::BF) {
      // lane i of lane group g reads channels 32a + 4(i%4) .. +3 (an even row
      // tile; odd ones are 8 bytes further) of token row 4g + i/4
      const int f = 4 * (l >> 4) + (r16 >> 2), q = r16 & 3;
#pragma unroll
      for (int a = 0; a < D / 32; ++a) oTR[a] = swz<C::R_TD>(f, 2 * kpos(32 * a + 4 * q));
    }
  }

  // bf16 A fragment of Kb^T for state row tile ct (channels 16ct .. 16ct+15) and
  // k block m (tokens 32m .. 32m+31, in the kpos order of the B fragments of
  // Delta), read from the time-major Kb with two transposing 8-byte LDS reads.
  // ds_read_b64_tr_b16 treats the 8-byte reads of a row of 16 lanes as a 16 x 4
  // matrix E (lane i, element j) and returns E[4e + i/4][i % 4] as element e of
  // lane i (checked on gfx950 with a probe of known LDS contents).  So lane i of
  // lane group g, reading channels 16ct + 4(i%4) .. +3 of token 32m + 16h + 4g +
  // i/4, receives tokens 32m + 16h + 4g + e of channel 16ct + i: half h of its
  // fragment.
  __device__ __forceinline__ bf16x8 kbt_frag(uint32_t st, int ct, int m) const { return tr_frag(st + C::S_KB, ct, m); }
  // the same for any time-major [CH][D] tile of the stage at `tile`
  __device__ __forceinline__ bf16x8 tr_frag(uint32_t tile, int ct, int m) const {
    const uint32_t base = tile + oTR[ct >> 1] + 8u * (uint32_t)(ct & 1);
    const bf16x4 lo = lds_tr16(smem, base + (uint32_t)(2 * m) * C::TD_TILE);
    const bf16x4 hi = lds_tr16(smem, base + (uint32_t)(2 * m + 1) * C::TD_TILE);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  // A fragment of row tile `t` and k block m of an LDS tile at `base`.
  // (row tile t of a [CH][D] tile starts TD_TILE bytes after tile t-1; other
  // tiles are plain, 16 * R bytes per row tile)
  template <int TSTRIDE>
  __device__ __forceinline__ typename F::A ar(uint32_t base, const uint32_t* o, int t, int m) const {
    return lds_ld<typename F::A>(smem, base + o[m] + t * TSTRIDE);
  }

  // Lane l holds rows 16*ti + 4*(l/16) + e of its columns (accumulator layout).
  __device__ __forceinline__ void load_v(VRaw& vr, int it) const {
    static_assert(NCT == (C::BF ? 2 : 1), "bf16 lanes own a column pair, fp32 lanes one column");
    const int ln = fresh_lane(l);
    const int g4 = 4 * (ln >> 4);
    const int chunk = chunk_of(it);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // map columns (segment pass) read v = 0: their offset is past any buffer end
        const uint32_t off = ((uint32_t)((chunk * CH + 16 * ti + g4 + e) * D + colb) * C::ES) |
                             (isv ? 0u : 0x80000000u);
        vr.r[4 * ti + e] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0);
      }
    }
  }

  // value of row i (of 16) in column tile j
  __device__ __forceinline__ static float vval(const VRaw& vr, int j, int i) {
    if constexpr (C::BF) return __uint_as_float(j == 0 ? vr.r[i] << 16 : vr.r[i] & 0xffff0000u);
    else return __uint_as_float(vr.r[i]);
  }

  // With three waves per SIMD (segment pass with 8 consumer waves) registers are
  // tighter, and operand fragments are fetched in smaller batches.
  static constexpr bool TIGHT = C::NW > 8;
  // One producer prefetch set (one chunk ahead) instead of two: the
  // three-waves-per-SIMD variant, and fp32 at D = 128, whose 8-byte-per-element
  // rows make two sets too large for 256 registers.
  static constexpr bool ONESET = TIGHT || (!C::BF && D > 64);
  // The outputs O = Qh S + P Delta feed nothing later in the chain, so with a
  // double-buffered stage (bf16 prefill) the consumers compute chunk n's in the
  // second interval, beside chunk n+1's score tiles, instead of in the first,
  // whose length the chain sets; their score-tile share shrinks to match.  The
  // bf16 copies of S (sb) and Delta (db) stay live across the barrier.
  static constexpr bool DEFER_O = QP && !BWD && C::LAG && C::BF;
  // The checkpoint pass stores the start state of chunk n + 1 (the end state of
  // chunk n) after the first barrier of the step that ran chunk n's chain, so
  // that the 32 KiB of stores drain beside the score tiles instead of inside
  // the chain (the first chunk's start state is stored in its chain).
  static constexpr bool CK_LATE = CKPT && C::LAG;
  // Likewise the reverse chain stores dS' of chunk c - 1 (the gradient at
  // chunk c's start, which its chain has just formed) after the first barrier.
  static constexpr bool DSP_LATE = BWD && C::LAG;
  // and its dv rows, kept in registers until then.
  static constexpr bool DV_LATE = BWD && C::LAG;
  // row t of this lane's dv pieces of chunk `chunk` (dv is the output o here)
  __device__ __forceinline__ void store_dv(int chunk, int t, const u32x4& d) const {
    __builtin_amdgcn_raw_buffer_store_b128(
        d, ro, (uint32_t)((chunk * CH + 16 * t + 4 * (l >> 4) + (l & 3)) * D + (colb & ~7)) * 2u, 0, 0);
  }
  // Weight of the outputs of one chunk in score-tile units (a tile is one unit,
  // a diagonal block with its inverse two) when handing out the score tiles.
  // Per-wave timestamps put the outputs at about 2.1K cycles against about
  // 0.55K per unit, but measured over weights 0 to 8 the call is fastest at 1
  // or 2 (h32_t64k 0.617-0.622 ms against 0.628-0.639 for 3 and for outputs
  // computed in the first interval; 6 and 8 were slower still).
  static constexpr int kOutWeight = 2;
  // Likewise the reverse chain's dS' and dv stores (48 KiB per chunk-head),
  // which the consumer waves issue in this interval.
  static constexpr int kStoreWeight = 3;
  static constexpr int C1B = 2;                    // row tiles per batch in c1
  static constexpr int C3B = TIGHT ? 2 : D / 32;   // state row tiles per batch in c3

  // X_t = b_t (v_t - (Kh S)_t) for row tiles H0 .. H0+C1B-1 (fragments fetched
  // first).  X enters holding -v, so the products accumulate Kh S onto it and X
  // ends as one multiply by -b.
  template <int H0>
  __device__ __forceinline__ void c1_part(uint32_t st, f32x4 (*X)[4]) {
    typename F::A fk[C1B][NKD];
#pragma unroll
    for (int h = 0; h < C1B; ++h)
#pragma unroll
      for (int m = 0; m < NKD; ++m) fk[h][m] = ar<C::TD_TILE>(st + C::S_KH, oTD, H0 + h, m);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NKD; ++m)
#pragma unroll
      for (int h = 0; h < C1B; ++h)
#pragma unroll
        for (int j = 0; j < NCT; ++j) X[j][H0 + h] = F::mma(X[j][H0 + h], fk[h][m], sb[j][m]);
    const int kk = 4 * (l >> 4);
#pragma unroll
    for (int h = 0; h < C1B; ++h) {
      const f32x4 bet = lds_ld<f32x4>(smem, st + C::S_BETA + 4 * (16 * (H0 + h) + kk));
      if constexpr (PREFILL && !BWD && NCT == 2) {
        // W = V - Kh S = -X here, kept for the rows with beta below kTinyBeta
        if (ck_w) store_tile_bf16(ck_w, X[0], X[1], H0 + h, -1.f, &bet);
      }
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) X[j][H0 + h][e] = -bet[e] * X[j][H0 + h][e];
    }
  }

  // Tight variant of the X computation: one k block at a time over all four row
  // tiles, so only that block of the bf16 copy of S is live (the segment pass
  // has no later use for it).  X enters holding -v, as in c1_part.
  template <int M>
  __device__ __forceinline__ void c1_kblock(uint32_t st, f32x4 (*X)[4]) {
    typename F::A fk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) fk[t] = ar<C::TD_TILE>(st + C::S_KH, oTD, t, M);
    typename F::B bm[NCT];
#pragma unroll
    for (int j = 0; j < NCT; ++j) bm[j] = F::bfrag(S[j], M);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < NCT; ++j) X[j][t] = F::mma(X[j][t], fk[t], bm[j]);
  }
  template <int M>
  __device__ __forceinline__ void c1_kblocks(uint32_t st, f32x4 (*X)[4]) {
    if constexpr (M < NKD) {
      c1_kblock<M>(st, X);
      c1_kblocks<M + 1>(st, X);
    }
  }

  // Delta from (I + L) Delta = diag(b) (V - Kh S) by 16-row blocks:
  // Delta_i = T_ii (X_i + sum_{j<i} (-L_ij) Delta_j).  X holds -v on entry.
  __device__ __forceinline__ void c1(f32x4 (*X)[4], uint32_t st) {
    if constexpr (TIGHT) {
      c1_kblocks<0>(st, X);
      const int kk = 4 * (l >> 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4 bet = lds_ld<f32x4>(smem, st + C::S_BETA + 4 * (16 * t + kk));
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) X[j][t][e] = -bet[e] * X[j][t][e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int m = 0; m < NKD; ++m) sb[j][m] = F::bfrag(S[j], m);
      c1_part<0>(st, X);
      c1_part<2>(st, X);
    }
    A16 ft[4], fl[4][4];
    const uint32_t lo = (uint32_t)fresh_lane(l) * 4 * C::ES;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      ft[ti] = lds_ld<A16>(smem, st + C::S_TI + ti * C::FR16 + lo);
#pragma unroll
      for (int jj = 0; jj < ti; ++jj)
        fl[ti][jj] = lds_ld<A16>(smem, st + C::S_L + (ti * (ti - 1) / 2 + jj) * C::FR16 + lo);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 Dl[NCT][4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        f32x4 rr = X[j][ti];
#pragma unroll
        for (int jj = 0; jj < ti; ++jj) rr = F::mma16(rr, fl[ti][jj], Dl[j][jj]);  // fl holds -L
        Dl[j][ti] = F::mma16(zero4(), ft[ti], rr);
      }
    }
    if constexpr (PREFILL && !BWD && NCT == 2) {
      if (ck_d) {
#pragma unroll
        for (int t = 0; t < 4; ++t) store_tile_bf16(ck_d, Dl[0], Dl[1], t, 1.f);
      }
    }
#pragma unroll
    for (int j = 0; j < NCT; ++j)
#pragma unroll
      for (int m = 0; m < NKT; ++m) db[j][m] = F::bfrag(Dl[j], m);
  }

  // O = Qh S + P Delta, stored (rows past the sequence end are dropped).  Two
  // halves of two row tiles each keep the prefetched fragments small.
  template <int H0>
  __device__ __forceinline__ void c2_half(uint32_t st, int chunk) {
    const int kk = 4 * (l >> 4);
    const int ln = fresh_lane(l);
    typename F::A fq[2][NKD], fp[2][NKT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ti = H0 + h;
#pragma unroll
      for (int m = 0; m < NKD; ++m) fq[h][m] = ar<C::TD_TILE>(st + C::S_QH, oTD, ti, m);
#pragma unroll
      for (int m = 0; m <= tri(ti); ++m)
        fp[h][m] = lds_ld<typename F::A>(smem, st + C::S_P + ((ti * NKT + m) * 64 + ln) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 O[NCT][2];
#pragma unroll
    for (int j = 0; j < NCT; ++j) O[j][0] = O[j][1] = zero4();
#pragma unroll
    for (int m = 0; m < NKD; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < NCT; ++j) O[j][h] = F::mma(O[j][h], fq[h][m], sb[j][m]);
#pragma unroll
    for (int m = 0; m < NKT; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < NCT; ++j)
          if (m <= tri(H0 + h)) O[j][h] = F::mma(O[j][h], fp[h][m], db[j][m]);
    const uint32_t ob = (uint32_t)((chunk * CH + kk) * D + colb) * C::ES;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t off = ob + (uint32_t)((16 * (H0 + h) + e) * D * C::ES);
        if constexpr (C::BF)
          __builtin_amdgcn_raw_buffer_store_b32(cvt2(O[0][h][e], O[1][h][e]), ro, off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[0][h][e]), ro, off, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void c2(uint32_t st, int chunk) {
    if constexpr (QP && !BWD) {
      if (!a.o) return;
      c2_half<0>(st, chunk);
      c2_half<2>(st, chunk);
    }
  }

  // S = Diag(Gam) (S + Kb^T Delta) for state row tiles C0 .. C0 + C3B - 1.
  template <int C0>
  __device__ __forceinline__ void c3_part(uint32_t st) {
    constexpr int NH = C3B;
    const int kk = 4 * (l >> 4);
    typename F::A fk[NH][NKT];
    f32x4 gm[NH];
#pragma unroll
    for (int ci = 0; ci < NH; ++ci) {
#pragma unroll
      for (int m = 0; m < NKT; ++m) {
        if constexpr (C::BF) fk[ci][m] = kbt_frag(st, C0 + ci, m);
        else fk[ci][m] = ar<16 * C::R_DT>(st + C::S_KB, oDT, C0 + ci, m);
      }
      gm[ci] = lds_ld<f32x4>(smem, st + C::S_GM + 4 * (16 * (C0 + ci) + kk));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NKT; ++m)
#pragma unroll
      for (int ci = 0; ci < NH; ++ci)
#pragma unroll
        for (int j = 0; j < NCT; ++j) S[j][C0 + ci] = F::mma(S[j][C0 + ci], fk[ci][m], db[j][m]);
#pragma unroll
    for (int ci = 0; ci < NH; ++ci)
#pragma unroll
      for (int j = 0; j < NCT; ++j) S[j][C0 + ci] = S[j][C0 + ci] * gm[ci];
  }

  template <int C0>
  __device__ __forceinline__ void c3_from(uint32_t st) {
    if constexpr (C0 < D / 16) {
      c3_part<C0>(st);
      c3_from<C0 + C3B>(st);
    }
  }
  __device__ __forceinline__ void c3(uint32_t st) { c3_from<0>(st); }

  // This lane's entries of the state, at row r, columns c .. c + NCT - 1 of a
  // D x D fp32 matrix at dst.
  __device__ __forceinline__ void store_state(float* dst, int c) const {
    const rsrc_t r = make_rsrc(dst, D * D * 4);
    const uint32_t vo = (uint32_t)(4 * (l >> 4) * D + c) * 4;  // the lane's first entry
#pragma unroll
    for (int ci = 0; ci < D / 16; ++ci)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int so = (16 * ci + e) * D * 4;
        if constexpr (NCT == 2) {
          const u32x2 x = {__float_as_uint(S[0][ci][e]), __float_as_uint(S[1][ci][e])};
          __builtin_amdgcn_raw_buffer_store_b64(x, r, vo, so, 0);
        } else {
#pragma unroll
          for (int j = 0; j < NCT; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[j][ci][e]), r, vo + 4 * j, so, 0);
        }
      }
  }

  // Row-major bf16 D-wide matrices with the positions inside every 32-wide
  // block of a row in the kpos order (the layout the per-chunk gradients read
  // the state, dS' and Delta in: a row of one gives an MFMA fragment over its
  // columns in one 16-byte read).  A lane holds two adjacent columns of four
  // rows; the lanes 2j, 2j+1, 2j+8, 2j+9 of a 16-lane row hold the columns of
  // position group j (positions 8j .. 8j+7 of the block: columns 4j .. 4j+3 and
  // 4j+16 .. 4j+19), so after a 4 x 4 transpose among them each stores one row
  // of the group with one 16-byte store instead of four 4-byte ones.
  // rows 16t + 4(l/16) + e of the lane's columns (dword e: the two bf16)
  __device__ __forceinline__ void store_kpos_rows(rsrc_t r, int t, u32x4 d) const {
    const int r16 = l & 15;
    d = transpose4<DPP_ROW_ROR8>(d, (r16 & 8) != 0, (r16 & 1) != 0);
    const int row = 16 * t + 4 * (l >> 4) + 2 * ((r16 >> 3) & 1) + (r16 & 1);
    const int pos = (colb & ~31) + 8 * ((r16 & 7) >> 1);
    __builtin_amdgcn_raw_buffer_store_b128(d, r, (uint32_t)(row * D + pos) * 2u, 0, 0);
  }

  // This lane's entries of the state (bf16 columns only) as bf16 into a
  // row-major D x D matrix in the layout above.
  __device__ __forceinline__ void store_state_bf16(bf16* rows) const {
    if constexpr (C::BF) {
      const rsrc_t rr = make_rsrc(rows, D * D * 2);
#pragma unroll
      for (int ci = 0; ci < D / 16; ++ci)
        store_kpos_rows(rr, ci, u32x4{cvt2(S[0][ci][0], S[1][ci][0]), cvt2(S[0][ci][1], S[1][ci][1]),
                                      cvt2(S[0][ci][2], S[1][ci][2]), cvt2(S[0][ci][3], S[1][ci][3])});
    }
  }

  // Row tile t of a [CH][D] matrix held in accumulators (x[j]: this lane's
  // columns colb + j), scaled by `sc`, as bf16 into a row-major [CH][D] matrix
  // in the layout above.  With `bet` (the beta of the lane's rows 16t +
  // 4(l/16) + e), only the rows whose beta is below kTinyBeta are stored (one
  // 4-byte store each).
  __device__ __forceinline__ void store_tile_bf16(bf16* dst, const f32x4* x0, const f32x4* x1, int t, float sc,
                                                  const f32x4* bet = nullptr) const {
    const rsrc_t r = make_rsrc(dst, CH * D * 2);
    if (!bet) {
      store_kpos_rows(r, t, u32x4{cvt2(sc * x0[t][0], sc * x1[t][0]), cvt2(sc * x0[t][1], sc * x1[t][1]),
                                  cvt2(sc * x0[t][2], sc * x1[t][2]), cvt2(sc * x0[t][3], sc * x1[t][3])});
      return;
    }
    const int g4 = 4 * (l >> 4);
    const uint32_t pc = (uint32_t)kpos(colb);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((*bet)[e] < kTinyBeta)
        __builtin_amdgcn_raw_buffer_store_b32(cvt2(sc * x0[t][e], sc * x1[t][e]), r,
                                              (uint32_t)((16 * t + g4 + e) * D + pc) * 2u, 0, 0);
  }

  // Snapshot after chunk cc when it closes a snapshot interval of the sequence.
  __device__ __forceinline__ void snapshot(int cc) const {
    if constexpr (PREFILL && !BWD) {
      if (!snap_head) return;
      const int gc = chunk0 + cc + 1;
      if (gc % a.snap_chunks) return;
      const int j = gc / a.snap_chunks - 1;
      if (j >= a.nsnap) return;  // a ragged last chunk ends short of the boundary
      store_state(snap_head + (size_t)j * a.H * D * D, colb);
    }
  }

  __device__ __forceinline__ void chain(VRaw& vr, int cc) {
    // The value rows seed the accumulators of Kh S (as -v), which frees their
    // registers for the next chunk's rows before the chain's products start.
    // The three-waves-per-SIMD variant has no registers to spare for rows in
    // flight during the products and loads them after the solve.  The loads are
    // issued on every path (rows past the end read zero), as for the producers.
    f32x4 X[NCT][4];
#pragma unroll
    for (int j = 0; j < NCT; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) X[j][t][e] = -vval(vr, j, 4 * t + e);
    if constexpr (!TIGHT) load_v(vr, cc + 1);
    if constexpr (PREFILL && !BWD) {
      // checkpoints for the gradients: the start state of every chunk, and its
      // Delta and, for the rows with beta below kTinyBeta, W = V - Kh S
      // (stored from c1)
      ck_w = ck_d = nullptr;
      if (a.ck_rows) {
        const size_t o = ck0 + cc;
        if (!CK_LATE || cc == 0) store_state_bf16(a.ck_rows + o * D * D);
        ck_w = a.ck_w + o * CH * D;
        ck_d = a.ck_d + o * CH * D;
      }
    }
    c1(X, stage(cc));
    if constexpr (TIGHT) load_v(vr, cc + 1);
    if constexpr (!DEFER_O) c2(stage(cc), cc);
    c3(stage(cc));
    snapshot(cc);
  }

  // Backward chain of one chunk (pipeline step cc, chunk chunk_of(cc)), run
  // last chunk to first.  S holds dS', the gradient of the loss with respect
  // to the chunk's end state (dS_T for the last chunk), for this wave's
  // columns.  With the chunk's forward S' = Diag(Gam) (S + Kb^T Delta),
  // (I + L) Delta = diag(b) (V - Kh S) and O = Qh S + P Delta, the chain rule
  // gives, column by column (nothing here depends on the forward state):
  //   dU = Diag(Gam) dS'                     (dS' is stored: the per-chunk gradients use it)
  //   dDelta = Kb dU + P^T dO
  //   Xbar = (I + L)^-T dDelta               (block back substitution with T_ii^T, L^T)
  //   dS = dU + Qh^T dO - Kh^T diag(b) Xbar  (the gradient at the chunk's start)
  // The value registers hold the chunk's dO rows (the v pointer is dO here).
  __device__ __forceinline__ void chain_bw(VRaw& vr, int cc) {
    if constexpr (BWD) {
      const uint32_t st = stage(cc);
      const int chunk = chunk_of(cc);
      const int kk = 4 * (l >> 4);
      // dO of the chunk as B fragments over its tokens
      typename F::B dob[NCT][NKT];
      {
        f32x4 dt[NCT][4];
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) dt[j][t][e] = vval(vr, j, 4 * t + e);
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int m = 0; m < NKT; ++m) dob[j][m] = F::bfrag(dt[j], m);
      }
      load_v(vr, cc + 1);
      // dS' for the per-chunk gradients: the launch's first chunk's here, the
      // others' after the first barrier of the step before (DSP_LATE)
      if (!DSP_LATE || cc == 0) store_state_bf16(a.dSp_rows + (ck0 + chunk) * D * D);
      // dU = Diag(Gam) dS', in place
#pragma unroll
      for (int ci = 0; ci < D / 16; ++ci) {
        const f32x4 gm = lds_ld<f32x4>(smem, st + C::S_GM + 4 * (16 * ci + kk));
#pragma unroll
        for (int j = 0; j < NCT; ++j) S[j][ci] = S[j][ci] * gm;
      }
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int m = 0; m < NKD; ++m) sb[j][m] = F::bfrag(S[j], m);
      // dS = dU + Qh^T dO + ...: the Qh^T dO part needs nothing from this
      // chunk's solve, so it is issued first
#pragma unroll
      for (int ci = 0; ci < D / 16; ++ci) {
        typename F::A fq[NKT];
#pragma unroll
        for (int m = 0; m < NKT; ++m) fq[m] = tr_frag(st + C::S_QH, ci, m);
#pragma unroll
        for (int m = 0; m < NKT; ++m)
#pragma unroll
          for (int j = 0; j < NCT; ++j) S[j][ci] = F::mma(S[j][ci], fq[m], dob[j][m]);
      }
      // dDelta = Kb dU + P^T dO, row tile by row tile
      f32x4 Xb[NCT][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        typename F::A fk[NKD], fp[NKT];
#pragma unroll
        for (int m = 0; m < NKD; ++m) fk[m] = ar<C::TD_TILE>(st + C::S_KB, oTD, t, m);
#pragma unroll
        for (int m = t / C::JPB; m < NKT; ++m)
          fp[m] = lds_ld<typename F::A>(smem, st + C::S_P + ((t * NKT + m) * 64 + fresh_lane(l)) * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
          f32x4 acc = zero4();
#pragma unroll
          for (int m = 0; m < NKD; ++m) acc = F::mma(acc, fk[m], sb[j][m]);
#pragma unroll
          for (int m = t / C::JPB; m < NKT; ++m) acc = F::mma(acc, fp[m], dob[j][m]);
          Xb[j][t] = acc;
        }
      }
      // Xbar_t = T_tt^T (dDelta_t - sum_{u > t} L_ut^T Xbar_u), from the last row tile
      {
        A16 ft[4], fl[4][4];
        const uint32_t lo = (uint32_t)fresh_lane(l) * 4 * C::ES;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          ft[t] = lds_ld<A16>(smem, st + C::S_TI + t * C::FR16 + lo);
#pragma unroll
          for (int u = t + 1; u < 4; ++u)
            fl[t][u] = lds_ld<A16>(smem, st + C::S_L + (u * (u - 1) / 2 + t) * C::FR16 + lo);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 3; t >= 0; --t) {
#pragma unroll
          for (int j = 0; j < NCT; ++j) {
            f32x4 rr = Xb[j][t];
#pragma unroll
            for (int u = t + 1; u < 4; ++u) rr = F::mma16(rr, fl[t][u], Xb[j][u]);  // fl holds -L^T
            Xb[j][t] = F::mma16(zero4(), ft[t], rr);
          }
        }
      }
      // dv = diag(b) Xbar (the output o pointer is dv here, in the inputs'
      // dtype), and Xbar itself for the rows with beta below kTinyBeta (the
      // per-chunk gradients recover every other row's from dv)
      {
        bf16* xb = a.ck_xb + (ck0 + chunk) * CH * D;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 bet = lds_ld<f32x4>(smem, st + C::S_BETA + 4 * (16 * t + kk));
          store_tile_bf16(xb, Xb[0], Xb[1], t, 1.f, &bet);
          // dv is row-major in plain column order: the four lanes of a quad
          // hold 8 adjacent columns, and after a 4 x 4 transpose each stores
          // one of their rows with one 16-byte store
          const int q = l & 3;
          const u32x4 d = transpose4<DPP_QUAD_SWAP2>(
              u32x4{cvt2(bet[0] * Xb[0][t][0], bet[0] * Xb[1][t][0]), cvt2(bet[1] * Xb[0][t][1], bet[1] * Xb[1][t][1]),
                    cvt2(bet[2] * Xb[0][t][2], bet[2] * Xb[1][t][2]), cvt2(bet[3] * Xb[0][t][3], bet[3] * Xb[1][t][3])},
              (q & 2) != 0, (q & 1) != 0);
          if constexpr (DV_LATE)
            dvq[t] = d;
          else
            store_dv(chunk, t, d);
        }
      }
      // -diag(b) Xbar as B fragments over the chunk's tokens
      typename F::B yb[NCT][NKT];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4 bet = lds_ld<f32x4>(smem, st + C::S_BETA + 4 * (16 * t + kk));
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) Xb[j][t][e] = -bet[e] * Xb[j][t][e];
      }
#pragma unroll
      for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int m = 0; m < NKT; ++m) yb[j][m] = F::bfrag(Xb[j], m);
      // ... + Kh^T (-diag(b) Xbar), state row tile by row tile
#pragma unroll
      for (int ci = 0; ci < D / 16; ++ci) {
        typename F::A fh[NKT];
#pragma unroll
        for (int m = 0; m < NKT; ++m) fh[m] = tr_frag(st + C::S_KH, ci, m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NKT; ++m)
#pragma unroll
          for (int j = 0; j < NCT; ++j) S[j][ci] = F::mma(S[j][ci], fh[m], yb[j][m]);
      }
    }
  }

  // Segment pass: once a wave's map columns are all exactly zero they stay
  // zero for finite inputs (their value rows are zero, and every step of the
  // chain is linear in the columns it updates), so the wave stops running the
  // chain for them and keeps only its share of the score tiles.  The columns are
  // checked after every second chunk.
  __device__ __forceinline__ void chain_step(VRaw& vr, int cc) {
    if constexpr (BWD) {
      chain_bw(vr, cc);
      return;
    }
    if constexpr (!PREFILL) {
      if (mzero) return;
    }
    chain(vr, cc);
    if constexpr (!PREFILL) {
      if (mskip && (cc & 1)) mzero = state_is_zero();
    }
  }

  // every state entry of the wave is +0 or -0 (a wave-uniform answer)
  __device__ __forceinline__ bool state_is_zero() const {
    uint32_t acc = 0u;
#pragma unroll
    for (int j = 0; j < NCT; ++j)
#pragma unroll
      for (int ci = 0; ci < D / 16; ++ci)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc |= __float_as_uint(S[j][ci][e]);
    return __builtin_amdgcn_ballot_w64((acc & 0x7fffffffu) != 0u) == 0u;
  }

  // Pipeline.  Iteration `it` prepares chunk it and runs the serial chain of
  // chunk it - LAG: interval 1 has the producer waves build the elementwise
  // tiles while the consumer waves run the chain; in interval 2 every wave
  // takes its share of the score tiles and diagonal inverses.  Producer waves
  // keep one set of prefetch registers, refilled as soon as the current
  // chunk's are consumed.
  // One producer iteration: build chunk `it` from the registers in r and refill
  // r with chunk it + PD: right away for PD = 1, and for PD = 2 once the first
  // barrier has passed (the rest of the workgroup is then busy with the score
  // tiles, and the data has a whole iteration to arrive).
  //
  // The prefetch loads are issued on every path, also past the last chunk
  // (buffer loads beyond the sequence read zero): the compiler's count of
  // loads in flight must be the same on all paths, or it waits for every
  // load, including the prefetch of the next chunk, before using a register set.
  //
  // Every step runs the elementwise phase with its loads, also the last one of
  // a two-stage pipeline, which prepares a chunk past the end (zero inputs)
  // into the stage nobody reads any more: with no data-dependent branches
  // around the loads, the compiler counts them exactly.  That step's score
  // tiles and their barrier are skipped, by every wave alike.
  template <int PD>
  __device__ __forceinline__ void producer_step(ProdRaw<T>& r, int it) {
    stamp(it, 0);
    p1(r, stage(it), it + PD);
    stamp(it, 1);
    sync_lds();
    stamp(it, 2);
    if (C::LAG && it == nch) return;
    p2(stage(it), it);
    stamp(it, 3);
    sync_lds();
    stamp(it, 4);
    if (!C::LAG) sync_lds();
  }

  // Producer inputs are prefetched two chunks ahead (two register sets, the
  // loop unrolled by two with the odd step peeled off, so that the loop's back
  // edge always follows both steps), except in the ONESET variants, which keep
  // one set and prefetch one chunk ahead.
#ifdef KDA_PHASE_STAMPS
  // Profiling build only: per-wave timestamps (s_memtime, shader-clock cycles)
  // at the phase boundaries of pipeline steps kStampFirst .. +kStampSteps - 1:
  // the step's start, the end of the elementwise phase (producers) or of the
  // chain (consumers), after the first barrier, the end of the score tiles,
  // after the second barrier; [workgroup][step][wave][5].
  unsigned long long* stp = nullptr;
  __device__ __forceinline__ void stamp(int it, int k) const {
    const int c = it - kStampFirst;
    if (!stp || c < 0 || c >= kStampSteps) return;
    const unsigned long long t = __builtin_amdgcn_s_memtime();
    if (l == 0) stp[((size_t)c * kStampWaves + wave) * 5 + k] = t;
  }
#else
  __device__ __forceinline__ void stamp(int, int) const {}
#endif

  __device__ __forceinline__ void producer_loop() {
    init_offsets();
    init_p1_offsets();
    const int n = nch + C::LAG;
    if constexpr (ONESET) {
      ProdRaw<T> r;
      load_raw(r, 0);
      for (int it = 0; it < n; ++it) producer_step<1>(r, it);
    } else {
      ProdRaw<T> ra, rb;
      load_raw(ra, 0);
      load_raw(rb, 1);
      int it = 0;
      for (; it + 1 < n; it += 2) {
        producer_step<2>(ra, it);
        producer_step<2>(rb, it + 1);
      }
      if (it < n) producer_step<2>(ra, it);
    }
  }

  __device__ __forceinline__ void consumer_loop() {
    VRaw vr;
    init_offsets();
    if (nch > 0) load_v(vr, 0);
    for (int it = 0; it < nch + C::LAG; ++it) {
      const int cc = it - C::LAG;
      stamp(it, 0);
      if (C::LAG && cc >= 0) chain_step(vr, cc);
      stamp(it, 1);
      sync_lds();
      stamp(it, 2);
      if constexpr (CK_LATE) {
        if (a.ck_rows && cc >= 0 && cc + 1 < nch) store_state_bf16(a.ck_rows + (ck0 + cc + 1) * D * D);
      }
      if constexpr (DSP_LATE) {
        if (cc >= 0 && chunk_of(cc) >= 1) store_state_bf16(a.dSp_rows + (ck0 + chunk_of(cc) - 1) * D * D);
      }
      if constexpr (DV_LATE) {
        if (cc >= 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) store_dv(chunk_of(cc), t, dvq[t]);
        }
      }
      if (C::LAG && it == nch) {  // the chunk past the end: no score tiles
        if constexpr (DEFER_O) {
          if (cc >= 0) c2(stage(cc), cc);
        }
        break;
      }
      p2(stage(it), it);
      if constexpr (DEFER_O) {
        if (cc >= 0) c2(stage(cc), cc);
      }
      stamp(it, 3);
      sync_lds();
      stamp(it, 4);
      if (!C::LAG) {
        chain_step(vr, cc);
        sync_lds();
      }
    }
  }

  __device__ __forceinline__ void run() {
    const int W = gridDim.x;
    int id = blockIdx.x;
    // Consecutive blockIdx go to different XCDs (round-robin over 8); regroup so
    // that the workgroups sharing a sequence land on one XCD and share its L2.
    // With one workgroup per sequence nothing is shared, and the launch order is
    // kept: the sequences that run while others exit at once (the split
    // prefill's segment 0) then spread over all XCDs instead of filling one.
    if ((W & 7) == 0 && a.vsplit > 1) id = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
    const int seq = id / a.vsplit;
    const int vs = id - seq * a.vsplit;
    const int gseg = seq / a.BH;
    const int bh = seq - gseg * a.BH;
    const int seg0 = a.t0 + gseg * a.Tseg;  // first token of this segment
    const size_t tok0 = (size_t)bh * a.Ttot + seg0;
    Tlen = min(a.Tseg, a.Tend - seg0);
    nch = (Tlen + CH - 1) / CH;
    chunk0 = seg0 / CH;
    ck0 = (size_t)bh * ((a.Ttot + CH - 1) / CH) + chunk0;
    // Segments with corrected heads: whether this one runs, and how far (the
    // decision is the same for every wave of the workgroup, taken before any
    // barrier).
    const int rec = (gseg - a.flag_g0) * a.BH + bh;
    // whether record r (>= 0) says the map has not vanished
    auto rec_live = [&](int r) -> bool {
      const uint32_t* f = a.seg_flag + (size_t)r * kFlagSlots;
      uint32_t x = 0u;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) x |= f[i];
      return x != 0u;
    };
    bool pred_live = true;  // FLAG_FIX: the previous segment's map had not vanished
    if (a.flag_mode != FLAG_NONE) {
      const bool has_rec = gseg >= a.flag_g0;
      const bool live = has_rec && a.flag_mode != FLAG_HEAD && rec_live(rec);
      if (a.flag_mode == FLAG_FIX) pred_live = gseg > a.flag_g0 && rec_live(rec - a.BH);
      switch (a.flag_mode) {
        case FLAG_HEAD: nch = min(nch, a.head_chunks); break;
        case FLAG_SLOW_ONLY: if (!has_rec || !live) return; break;
        case FLAG_FAST_ONLY: if (has_rec && live) return; break;
        case FLAG_FIX:
          if (!has_rec) return;
          if (!live) nch = min(nch, a.head_chunks);
          break;
        default: break;
      }
      // a walk cut short reads nothing past its chunks (the prefetch of the
      // chunks after them then reads zeros without touching memory)
      Tlen = min(Tlen, nch * CH);
    }
    snap_head = nullptr;
    if (PREFILL && a.snap) {
      const int b = bh / a.H, h = bh - b * a.H;
      snap_head = a.snap + ((size_t)b * a.nsnap * a.H + h) * D * D;
    }
    wave = threadIdx.x >> 6;
    l = lane_id();
#ifdef KDA_PHASE_STAMPS
    if constexpr (PREFILL && NC + D / 32 <= kStampWaves) {
      const size_t per = (size_t)kStampSteps * kStampWaves * 5;
      if (a.stamps && (size_t)(blockIdx.x + 1) * per <= a.stamps_n) stp = a.stamps + blockIdx.x * per;
    }
#endif
    const int g4 = 4 * (l >> 4);
    const uint32_t rowbytes = (uint32_t)Tlen * D * C::ES;
    const size_t base = tok0 * D * C::ES;
    rk = make_rsrc(reinterpret_cast<const char*>(a.k) + base, rowbytes);
    // a missing v (the backward chain's dO may be absent) reads as zeros
    rv = make_rsrc(a.v ? reinterpret_cast<const char*>(a.v) + base : nullptr, a.v ? rowbytes : 0u);
    rla = make_rsrc(reinterpret_cast<const char*>(a.la) + base, rowbytes);
    rbeta = make_rsrc(reinterpret_cast<const char*>(a.beta) + tok0 * C::ES, (uint32_t)Tlen * C::ES);
    if constexpr (QP) rq = make_rsrc(reinterpret_cast<const char*>(a.q) + base, rowbytes);
    // without o (a forward pass run for its state checkpoints) every store is
    // dropped; the backward chain writes dv through it
    if constexpr (PREFILL)
      ro = make_rsrc(a.o ? reinterpret_cast<const char*>(a.o) + base : nullptr, a.o ? rowbytes : 0u);

    // Every LDS byte the kernel reads is written by it first, except the halves
    // of the 32-deep P lane slots that pair a diagonal tile with the tile above
    // it (tiles (0,1) and (2,3); for the backward chain's P^T, tiles (1,0) and
    // (3,2) of P^T): nothing writes them, and they must hold the zeros of P's
    // upper triangle.
    if constexpr (QP && C::JPB == 2) {
      for (uint32_t t = threadIdx.x; t < 2u * 64u * C::STAGES; t += C::THREADS) {
        // forward: slots (I = 2, m = 1) and (I = 0, m = 0), second half;
        // backward: slots (J = 3, m = 1) and (J = 1, m = 0), first half
        const uint32_t slot = BWD ? ((t & 64u) ? 3u * (CH / KB) + 1u : 1u * (CH / KB))
                                  : ((t & 64u) ? 2u * (CH / KB) + 1u : 0u);
        lds_st<u32x2>(smem, (t >> 7) * C::STAGE + C::S_P + (slot * 64u + (t & 63u)) * 16u + (BWD ? 0u : 8u),
                      u32x2{0u, 0u});
      }
    }

    colb = vs * 16 * NC * NCT + 16 * NCT * wave + NCT * (l & 15);
    isv = PREFILL || colb < D;  // a wave's tiles lie on one side of D
    mskip = !PREFILL && a.map_skip && __builtin_amdgcn_readfirstlane(isv ? 0 : 1);
    // the head walk carries the map columns only
    mzero = !PREFILL && a.flag_mode == FLAG_HEAD && __builtin_amdgcn_readfirstlane(isv ? 1 : 0);
    const size_t sbase = (size_t)seq * D * D;
    // prefill start state: one per sequence, or (s0_first) S0 [BH, D, D] for
    // segment 0 and zero for the others; when correcting a head whose previous
    // segment's map vanished, that segment's zero-start end state (Z_prev)
    const float* s0 = nullptr;
    if (PREFILL && a.flag_mode == FLAG_FIX && !pred_live) s0 = a.Z_prev + sbase;
    else if (PREFILL && a.S0) s0 = !a.s0_first ? a.S0 + sbase : gseg == 0 ? a.S0 + (size_t)bh * D * D : nullptr;
    if (wave < NC) {
      if (PREFILL && NCT == 2 && s0) {
        // the lane's two adjacent columns of a row as one 8-byte load
        const rsrc_t rs = make_rsrc(s0, D * D * 4);
#pragma unroll
        for (int ci = 0; ci < D / 16; ++ci)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u32x2 x = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)((16 * ci + g4 + e) * D + colb) * 4u, 0, 0));
            S[0][ci][e] = __uint_as_float(x[0]);
            S[NCT - 1][ci][e] = __uint_as_float(x[1]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < NCT; ++j)
#pragma unroll
          for (int ci = 0; ci < D / 16; ++ci)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 16 * ci + g4 + e;
              const int c = colb + j;
              float x = 0.f;
              if (PREFILL) {
                if (s0) x = s0[(size_t)r * D + c];
              } else if (!isv) {
                x = (r == c - D) ? 1.f : 0.f;
              }
              S[j][ci][e] = x;
            }
      }
      // Retire the start-state loads here: left pending into the chunk loop, they
      // make the compiler wait for every load and store in flight at the top of
      // each iteration (its count at the loop header merges in this path).
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited for
    }
    sync_lds();

    if (wave >= NC) {
      producer_loop();
      return;
    }
    consumer_loop();

    if (!PREFILL && a.flag_mode == FLAG_HEAD) {
      // the segment's record: one word per consumer wave, nonzero while any of
      // the wave's map columns is not exactly zero
      const bool live = !isv && !state_is_zero();
      if (l == 0) a.seg_flag[(size_t)rec * kFlagSlots + vs * NC + wave] = live ? 1u : 0u;
      return;
    }
    // prefill over several segments: every segment's end state (Z_out), or only
    // the last one's (S_out, if given)
    float* dst;
    int c = colb;
    if (PREFILL) {
      if (a.Z_out) {
        dst = a.Z_out + sbase;
      } else {
        if (a.G > 1 && gseg != a.G - 1) return;
        if (!a.S_out) return;
        dst = a.S_out + (size_t)bh * D * D;
      }
    } else if (isv) {
      dst = a.S_out + sbase;
    } else {
      dst = a.M_out + sbase;
      c = colb - D;
    }
    store_state(dst, c);
  }
};

template <typename T, int D, int NC, bool PREFILL, bool BWD = false, bool CKPT = false>
__global__ __launch_bounds__(64 * (NC + D / 32), 1)
void kda_chunk_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[ChunkCfg<T, D, NC, PREFILL>::LDS];
  ChunkKernel<T, D, NC, PREFILL, BWD, CKPT> kern;
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
    case 4:
      if constexpr (sizeof(T) == 2) return launch_one<T, D, 4, PREFILL>(a, nwg, stream);
      else return hipErrorInvalidValue;
    case 8:
      if constexpr (sizeof(T) == 2 && !PREFILL && D == 128) return launch_one<T, D, 8, PREFILL>(a, nwg, stream);
      else return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int D, int NC>
static hipError_t launch_bwd_one(const ChunkArgs& a, int nwg, hipStream_t stream) {
  using Cf = ChunkCfg<bf16, D, NC, true>;
  hipLaunchKernelGGL((kda_chunk_kernel<bf16, D, NC, true, true>), dim3(nwg), dim3(Cf::THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const ChunkArgs& a, int D, int nc, int nwg, hipStream_t stream) {
  if (D == 128) {
    switch (nc) {
      case 1: return launch_bwd_one<128, 1>(a, nwg, stream);
      case 2: return launch_bwd_one<128, 2>(a, nwg, stream);
      case 4: return launch_bwd_one<128, 4>(a, nwg, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (D == 64) {
    switch (nc) {
      case 1: return launch_bwd_one<64, 1>(a, nwg, stream);
      case 2: return launch_bwd_one<64, 2>(a, nwg, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

template <int D, int NC>
static hipError_t launch_ckpt_one(const ChunkArgs& a, int nwg, hipStream_t stream) {
  using Cf = ChunkCfg<bf16, D, NC, true>;
  hipLaunchKernelGGL((kda_chunk_kernel<bf16, D, NC, true, false, true>), dim3(nwg), dim3(Cf::THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_chunk_ckpt(const ChunkArgs& a, int D, int nc, int nwg, hipStream_t stream) {
  if (D == 128) {
    switch (nc) {
      case 1: return launch_ckpt_one<128, 1>(a, nwg, stream);
      case 2: return launch_ckpt_one<128, 2>(a, nwg, stream);
      case 4: return launch_ckpt_one<128, 4>(a, nwg, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (D == 64) {
    switch (nc) {
      case 1: return launch_ckpt_one<64, 1>(a, nwg, stream);
      case 2: return launch_ckpt_one<64, 2>(a, nwg, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk(const ChunkArgs& a, bool bf16_io, int D, bool prefill, int nc, int nwg,
                        hipStream_t stream) {
  if (bf16_io) {
    if (D == 128) return prefill ? launch_nc<bf16, 128, true>(a, nc, nwg, stream)
                                 : launch_nc<bf16, 128, false>(a, nc, nwg, stream);
    if (D == 64) return prefill ? launch_nc<bf16, 64, true>(a, nc, nwg, stream)
                                : launch_nc<bf16, 64, false>(a, nc, nwg, stream);
  } else {
    if (D == 128) return prefill ? launch_nc<float, 128, true>(a, nc, nwg, stream)
                                 : launch_nc<float, 128, false>(a, nc, nwg, stream);
    if (D == 64) return prefill ? launch_nc<float, 64, true>(a, nc, nwg, stream)
                                : launch_nc<float, 64, false>(a, nc, nwg, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
