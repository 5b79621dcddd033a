// Internal launch interface between the C-ABI layer (kda_api.hip) and the
// kernel translation units.  Host-side only types; no validation here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "kda_device.hpp"

namespace kda {

// One chunked pass over `G * BH` independent sequences (segments).  Sequence
// s = g * BH + bh reads tokens [t0 + g*Tseg, min(t0 + (g+1)*Tseg, Tend)) of head
// bh, whose rows start at token bh * Ttot of the [BH, Ttot, D] inputs.
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* la;
  const void* beta;
  const float* S0;  // prefill: start state of every segment [G*BH, D, D] or null
  void* o;          // prefill: outputs [BH, Ttot, D]
  float* S_out;     // prefill: S_T [BH, D, D] (end of the last segment);
                    // segment pass: zero-start end states [G*BH, D, D]
  float* M_out;     // segment pass: transfer maps [G*BH, D, D]
  int BH;
  int G;
  int Tseg;         // tokens per segment (the last one may be shorter)
  int Ttot;         // tokens per head (row stride of a head in tokens)
  int t0 = 0;       // first token of segment 0
  int Tend = 0;     // end of the covered tokens (t0 + G*Tseg or less, <= Ttot)
  int vsplit;       // workgroups per sequence (each owns 16 * nc * chunk_tiles_per_wave columns)
  // prefill only: state snapshots [B, nsnap, H, D, D] after every snap_chunks
  // chunks of a head's whole sequence (null: none).  With snapshots and G > 1,
  // Tseg must be a multiple of the chunk length.
  float* snap = nullptr;
  int snap_chunks = 1;
  int nsnap = 0;
  int H = 1;        // heads per sequence batch entry (bh = b * H + h)
  // segment pass: a wave stops updating its map columns once they are all
  // exactly zero (they stay zero for finite inputs); 0 keeps updating them
  int map_skip = 1;
  // gradients' checkpoints, bf16 row-major matrices with the positions inside
  // each 32-wide block of a row in the kpos order (null: none), indexed by the
  // chunk of the head's whole sequence (nch = ceil(Ttot / 64) per head; a
  // launch may cover the chunks from t0 / 64 on).  Prefill (bf16,
  // one segment per head): the start state of every chunk [BH, nch, D, D] and
  // its Delta [BH, nch, CH, D]; for the rows (tokens) with beta < kTinyBeta
  // only, W = V - Kh S [BH, nch, CH, D] and the row's part of the strictly
  // lower blocks of Kh Kb^T [BH, nch, 10, 64 lanes, 4] (block (I, J), J <= I,
  // at I(I+1)/2 + J; lane l holds row 16I + l%16, columns 16J + 4(l/16) + e).
  // Backward chain: dS' (the gradient with respect to the chunk's end state)
  // [BH, nch, D, D] of every chunk, and
  // Xbar [BH, nch, CH, D] of its rows with beta < kTinyBeta (dv through o).
  bf16* ck_rows = nullptr;
  bf16* ck_w = nullptr;
  bf16* ck_d = nullptr;
  bf16* ck_a = nullptr;
  bf16* dSp_rows = nullptr;
  bf16* ck_xb = nullptr;
  // Segments started from zero whose heads are corrected afterwards (the
  // split prefill): one record of kFlagSlots words per (segment, bh), nonzero
  // when the segment's transfer map was not exactly zero after head_chunks
  // chunks.  Segment g of this launch (g >= flag_g0) has record
  // (g - flag_g0) * BH + bh; see FlagMode for what each launch does with it.
  uint32_t* seg_flag = nullptr;
  int flag_mode = 0;
  int flag_g0 = 0;
  int head_chunks = 0;
  // prefill: the end state of every segment [G*BH, D, D] (null: S_out only)
  float* Z_out = nullptr;
  // prefill: S0 is segment 0's start state [BH, D, D] and the other segments
  // start from zero (0: S0 holds one start state per sequence)
  int s0_first = 0;
  // FLAG_FIX: the end state of the segment before each sequence's, from zero
  // (the first one's: from the true start) [G*BH, D, D]; a sequence whose
  // previous segment's map vanished starts from it instead of S0
  const float* Z_prev = nullptr;
  // profiling build (KDA_PHASE_STAMPS) only: phase timestamps of every
  // workgroup of this launch, stamps_n entries (see the chunk kernel)
  unsigned long long* stamps = nullptr;
  size_t stamps_n = 0;
};

// Phase timestamps of the profiling build: pipeline steps and waves recorded
// per workgroup.
constexpr int kStampFirst = 32;
constexpr int kStampSteps = 16;
constexpr int kStampWaves = 8;

// Words per segment record (one per consumer wave of the segment pass, up to
// D/16 of them).
constexpr int kFlagSlots = 8;

enum FlagMode {
  FLAG_NONE = 0,
  // segment pass: walk the first head_chunks chunks of the map columns only
  // (the state columns stay idle) and write the records instead of Z and M
  FLAG_HEAD = 1,
  // segment pass: run only the segments with a nonzero record
  FLAG_SLOW_ONLY = 2,
  // prefill: skip the segments with a nonzero record (segments below flag_g0
  // have none and always run)
  FLAG_FAST_ONLY = 3,
  // prefill: segments with a zero record walk only their first head_chunks
  // chunks, the others all of theirs; segments below flag_g0 do nothing.  A
  // segment whose previous one has a zero record (or is the first, below
  // flag_g0) starts from Z_prev, the others from S0
  FLAG_FIX = 4,
};

// Reverse chain of the prefill gradients (bf16 inputs, one segment per head):
// S0 = dS_T [BH, D, D] or null, S_out = dS0, v = dO, o = dv [BH, T, D],
// dSp_rows and ck_xb as above; nc
// consumer waves per workgroup ({1, 2, 4} at D = 128, {1, 2} at D = 64).
hipError_t launch_chunk_bwd(const ChunkArgs& a, int D, int nc, int nwg, hipStream_t stream);

// Prefill run only for the gradients' checkpoints (bf16; a.o null, q unused):
// the ck_* pointers above; nc as for launch_chunk_bwd.
hipError_t launch_chunk_ckpt(const ChunkArgs& a, int D, int nc, int nwg, hipStream_t stream);

// 16-column state tiles each consumer wave of the chunk kernel owns.
inline int chunk_tiles_per_wave(bool bf16_io) { return bf16_io ? 2 : 1; }

// prefill: columns = D; segment pass: columns = 2*D (state + map).
// nc = consumer waves per workgroup: {1, 2, 4} for bf16, {1, 2} for fp32;
// nwg = G * BH * vsplit.
hipError_t launch_chunk(const ChunkArgs& a, bool bf16_io, int D, bool prefill, int nc, int nwg,
                        hipStream_t stream);

// ntok tokens per head ([NH, ntok, D] inputs, beta [NH, ntok]); S_out may alias
// S_in; S_pos [N, ntok, H, D, D] (NH = N * H) or null.
hipError_t launch_decode(const void* q, const void* k, const void* v, const void* la,
                         const void* beta, const float* S_in, float* S_out, void* o, float* S_pos,
                         int NH, int H, int ntok, int D, bool bf16_io, hipStream_t stream);

// Prefill gradients over [BH, T, D] fp32 inputs, token by token, split
// workgroups (1 or 2) per head.  The workspace holds, per head,
// (ceil(T / kBwInterval) + kBwInterval) fp32 D x D states (a checkpoint at the
// start of every interval and the entering state of every token of the
// interval being walked) and kBwInterval fp32 D-vectors (u = D^T k of each
// token of that interval), then, with two workgroups per head, the second
// one's row sums of every token (BH T (3D + 1) floats).
constexpr int kBwInterval = 64;
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* la;
  const void* beta;
  const float* S0;    // [BH, D, D] or null (= 0)
  const void* dO;     // [BH, T, D] or null (= 0)
  const float* dS_T;  // [BH, D, D] or null (= 0)
  float* dq;          // [BH, T, D]
  float* dk;          // [BH, T, D]
  float* dv;          // [BH, T, D]
  float* dla;         // [BH, T, D]
  float* dbeta;       // [BH, T]
  float* dS0;         // [BH, D, D]
  float* ws;
  int T;
};
size_t backward_ws_floats(long long BH, int T, int D, int split);

// Rows (tokens) whose beta is below this get the gradient checkpoints that
// only they need (W, Xbar and their part of Kh Kb^T); every other row's dbeta
// follows from dv and Delta, which are proportional to its beta.
constexpr float kTinyBeta = 0x1p-30f;

// Per-chunk gradients of the prefill (bf16 inputs), two workgroups per
// (head, chunk): from the chunk's start state (the forward's checkpoint), its
// Delta, dS' (from the reverse chain) and dv (the reverse chain's output).
struct BwGradArgs {
  const void* q;
  const void* k;
  const void* la;
  const void* beta;
  const void* dO;      // [BH, T, D] or null (= 0)
  const bf16* dv;      // [BH, T, D], written by the reverse chain
  // checkpoints, bf16 row-major with kpos-ordered positions (ChunkArgs::ck_*):
  const bf16* S_rows;  // the start state of every chunk [BH, nch, D, D]
  const bf16* Dl;      // Delta of every chunk [BH, nch, CH, D]
  const bf16* dSp_rows; // dS' of every chunk [BH, nch, D, D] (dU = Diag(Gam) dS')
  // rows with beta < kTinyBeta only:
  const bf16* W;       // W = V - Kh S [BH, nch, CH, D]
  const bf16* A;       // strictly lower blocks of Kh Kb^T [BH, nch, 10, 64, 4]
  const bf16* Xb;      // Xbar [BH, nch, CH, D]
  bf16* dq;            // [BH, T, D], the inputs' dtype
  bf16* dk;
  bf16* dla;
  bf16* dbeta;         // [BH, T]
  int T;
  // chunks [n0, n1) of every head (n1 < 0: to the last one)
  int n0 = 0;
  int n1 = -1;
};
hipError_t launch_bwgrad(const BwGradArgs& a, int BH, int D, hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, int BH, int D, int split, hipStream_t stream);

// flags: records of the G segments as in ChunkArgs::seg_flag (record i * BH + bh;
// a zero record means that segment's map is exactly zero), or null: every map
// is applied.  With records, S_start[i] is written only where segment i - 1's
// map did not vanish (elsewhere the start state is Z[i - 1], or S_in for i = 0,
// and is read from there), and the chain runs only through the segments whose
// map did not vanish.
hipError_t launch_merge(const float* S_in, const float* Z, const float* M, float* S_start,
                        float* S_T, int BH, int G, int D, hipStream_t stream,
                        const uint32_t* flags = nullptr);

// Reads n_la gate values and n_beta betas (bf16 or fp32) on `stream`, waits for
// the result, and sets *bits_out to bit 0 if a log_alpha value lies outside
// [-1, 0] or is not finite and bit 1 if a beta lies outside [0, 1] or is not
// finite.  Synchronises `stream`.  n_la is a multiple of 8 and la 16-byte
// aligned; beta may have any element alignment.
hipError_t check_gates(const void* la, long long n_la, const void* beta, long long n_beta, bool bf16_io,
                       hipStream_t stream, unsigned int* bits_out);

}  // namespace kda
