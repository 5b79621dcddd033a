/*
 * libkda -- Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).
 *
 * KDA is a delta-rule linear attention with a channel-wise forget gate whose
 * per-head state is a fixed-size dk x dv matrix ("Kimi K3 深度解析", section 3.1;
 * blog.csdn.net article on the Kimi K3 report, section 一.1).  Per head and
 * token t, with state S (dk x dv), gate alpha_t in (0,1]^dk and scalar beta_t:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                  (the output reads the updated state)
 *
 * No output scale and no normaliser is applied: q and k are used as given.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer to a contiguous row-major array,
 *    aligned to 16 bytes.  The caller owns all memory; the library allocates
 *    and frees no device memory inside these calls, and synchronises nothing
 *    except in the check mode described below.
 *  - `dtype` gives the element type of q, k, v, log_alpha, beta and o.  States
 *    (S0, S_T, S, S_zero_end, M, S_in, S_start) are always fp32.
 *  - The gate is passed in log space: log_alpha = log(alpha), one value per key
 *    channel, and must lie in [-1, 0]; beta must lie in [0, 1].  The pages
 *    describe the gate as lower-bounded so that long sequences neither overflow
 *    nor underflow (blog.csdn.net article, section 一.1); the kernels rely on
 *    the bound (|cumulative log-decay| <= 64 inside a 64-token chunk).  By
 *    default nothing checks it: a gate below the bound can give inf or NaN
 *    outputs with KDA_OK.  With the "check" option set (below), every call that
 *    takes log_alpha and beta first reduces them on the device, waits for the
 *    answer (it synchronises `stream`), and returns KDA_ERR_PRECONDITION,
 *    launching nothing else, when a value is out of range or not finite.
 *  - Supported head sizes: dk == dv == 64 or 128, for both dtypes.
 *  - Errors: arguments are validated on the host before anything is launched;
 *    on error nothing is written and a status != KDA_OK is returned, with a
 *    description in kda_last_error() (thread-local).  Work is enqueued
 *    asynchronously on `stream`; a launch failure returns KDA_ERR_HIP.
 *  - Calls never abort the process.  The only global state is per device and
 *    created on first use: the compute-unit count, the check flag, and for the
 *    sequence-split prefill a second stream (with two events) per caller
 *    stream, kept for the process lifetime; plus the process-wide options.
 *  - Options (kda_set_option): process-wide tuning and debugging switches,
 *    read from the environment once, at the first call that needs them, and
 *    changed at run time with kda_set_option.  Every choice they make gives the
 *    same result up to rounding.  See kda_set_option for the list.
 */
#ifndef LIBKDA_H
#define LIBKDA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 8

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,         /* a required pointer is NULL                    */
  KDA_ERR_SHAPE = 2,        /* negative size, dk != dv, or size overflow      */
  KDA_ERR_UNSUPPORTED = 3,  /* head size / dtype combination not built        */
  KDA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned               */
  KDA_ERR_WORKSPACE = 5,    /* a required workspace is missing or too small   */
  KDA_ERR_PRECONDITION = 6, /* check mode: log_alpha outside [-1, 0] or beta
                               outside [0, 1] (or not finite)                 */
  KDA_ERR_HIP = 7           /* the HIP runtime reported an error              */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * Chunked prefill of B*H independent heads over T tokens.
 * Evaluates the recurrence above exactly (up to rounding) in 64-token chunks:
 * parallel inside a chunk, sequential across chunks ("Kimi K3 开源日来了",
 * section "FlashKDA").
 *   q, k, log_alpha : [B, H, T, dk]   dtype
 *   v               : [B, H, T, dv]   dtype
 *   beta            : [B, H, T]       dtype, in [0, 1]
 *   S0              : [B, H, dk, dv]  fp32 start states, or NULL for zero
 *   o               : [B, H, T, dv]   dtype, written
 *   S_T             : [B, H, dk, dv]  fp32 end states, written; may alias S0
 *   workspace       : device scratch of workspace_bytes bytes, or NULL
 * Any T >= 0 is accepted (a last partial chunk is masked); T == 0 copies S0
 * (or zeros) to S_T.
 *
 * With few heads and a long sequence, the call can cut every sequence into G
 * segments and apply the context-parallel decomposition of the same section
 * ("针对适配的 Infra", KDA context parallelism) on this GPU (kda_prefill_plan
 * reports the cut).  By default every segment is prefilled at once, segment 0
 * from S0 and the others from zero, outputs included.  A short walk over the
 * first chunks of every later segment's transfer map decides, on the device,
 * whether the map is exactly zero there (it then stays zero).  If so, the
 * segment's outputs past those chunks and its end state are already the true
 * ones up to rounding, and only those first chunks are prefilled again from
 * the segment's true start state (from a merge of the segments' end states
 * and maps).  If not, the segment takes the longer way: its zero-start state
 * and map from the segment pass, then its whole prefill again from its start
 * state.  Option "fixup" 0 selects the earlier pipeline instead: the first T0
 * tokens prefilled directly beside the segment pass over the G - 1 segments
 * after them, the merge, then the prefill of those G segments.
 * The split path needs kda_prefill_workspace_bytes() of workspace (fp32
 * states, 3G - 2 per head, and G - 1 small segment records; 3G - 1 states
 * with fixup 0); with a smaller or NULL workspace the call runs the
 * single-pass path instead.  The workspace is only used by work enqueued by
 * this call; calls on one stream may share it.
 * The segment pass runs on a second stream of the library's own, one per
 * (device, caller stream) pair (created at the first split call on that stream,
 * default priority), forked from and joined back to `stream` with events, so
 * all of the call's work is ordered after earlier work on `stream` and before
 * later work on it, and split calls on different caller streams do not wait for
 * each other.
 */
size_t kda_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, kda_dtype dtype);

kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* beta, const float* S0, void* o, float* S_T, int B, int H,
                             int T, int dk, int dv, kda_dtype dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * Same arguments and results as kda_chunk_prefill without the workspace: the
 * sequence-split path takes its workspace from a scratch array the library
 * holds on each device (64 MiB, a file-scope device array that the device keeps
 * until the process ends), and the call itself allocates nothing.  The split
 * plan of every shape fits it on a 256-CU device with the default options; a
 * plan that needs more (e.g. a large "split" option) returns KDA_ERR_WORKSPACE
 * and launches nothing.  Nothing in the scratch array has to start at any value
 * (every byte the call reads there it has written first), but all calls on one
 * device share it: calls that can overlap on one device (on different streams,
 * or from different threads) race and must not be issued; calls on one stream
 * are ordered and safe.
 */
kda_status kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                                     const void* beta, const float* S0, void* o, float* S_T, int B, int H,
                                     int T, int dk, int dv, kda_dtype dtype, hipStream_t stream);

/*
 * kda_chunk_prefill that also keeps state snapshots for prefix caching.  The
 * KDA state of a request has a fixed size and is stored only at a sparse subset
 * of the 512-token block boundaries that prefix matching uses ("Kimi K3
 * 开源日来了", section "针对适配的 Infra", prefix-cache paragraph); a cache hit
 * then resumes from the longest stored boundary.
 *   snap_interval : tokens between snapshots, a positive multiple of 64 (the
 *                   chunk length; 512 or a multiple of it in the pages' use), or
 *                   0 for none
 *   S_snap        : [B, T / snap_interval, H, dk, dv] fp32 (floor division):
 *                   entry [b, j, h] is head (b, h)'s state after its first
 *                   (j + 1) * snap_interval tokens.  Required (16-byte aligned)
 *                   when that count is nonzero, ignored otherwise; must not
 *                   overlap any other argument.
 * Every other argument, the workspace and the paths taken are as for
 * kda_chunk_prefill, whose outputs this call reproduces bit for bit.
 * Errors: KDA_ERR_SHAPE for a negative interval or one that is not a multiple
 * of 64; the rest as for kda_chunk_prefill.
 */
kda_status kda_chunk_prefill_snap(const void* q, const void* k, const void* v, const void* log_alpha,
                                  const void* beta, const float* S0, void* o, float* S_T,
                                  float* S_snap, int snap_interval, int B, int H, int T, int dk,
                                  int dv, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * The cut kda_chunk_prefill would use for this shape when given
 * kda_prefill_workspace_bytes() of workspace: a first part of *T0 tokens
 * prefilled directly, then *G segments of *Tseg tokens (the last one possibly
 * shorter, ending at T).  *G == 1 (*T0 == 0, *Tseg == T) means the
 * single-pass path.  With the default pipeline *T0 is 0 and segment 0 starts
 * from S0; with option "fixup" 0, *T0 > 0.  T0 and Tseg are multiples of 64
 * on the split path.  Writes nothing else and launches nothing.
 */
kda_status kda_prefill_plan(int B, int H, int T, int dk, int dv, kda_dtype dtype, int* T0, int* G,
                            int* Tseg);

/*
 * Last step of the context-parallel decomposition (same section): every
 * segment, once its true start state is known, runs its own prefill.  Here all
 * G = ceil(T / Tseg) segments of all B*H heads run in one call, segment i
 * covering tokens [i*Tseg, min((i+1)*Tseg, T)) and starting from S_start[i].
 *   q, k, v, log_alpha, beta, o : as for kda_chunk_prefill (T >= 1 tokens)
 *   S_start : [G, B, H, dk, dv] fp32 start states, or NULL for zero
 *   S_T     : [B, H, dk, dv] fp32, written with the end state of the last segment
 * With S_start from kda_segment_transfer + kda_segment_merge this reproduces
 * kda_chunk_prefill over the whole sequence.  Tseg >= 1; S_T must not alias
 * S_start.
 */
kda_status kda_chunk_prefill_segments(const void* q, const void* k, const void* v,
                                      const void* log_alpha, const void* beta, const float* S_start,
                                      void* o, float* S_T, int B, int H, int T, int Tseg, int dk,
                                      int dv, kda_dtype dtype, hipStream_t stream);

/*
 * One decode step for N*H independent heads: applies the recurrence for one
 * token to the fp32 state held in place (the state is the fixed-size per-request
 * KDA cache, "Kimi K3 开源日来了", section "针对适配的 Infra").
 *   q, k, log_alpha : [N, H, dk]      dtype
 *   v               : [N, H, dv]      dtype
 *   beta            : [N, H]          dtype
 *   S               : [N, H, dk, dv]  fp32, read and overwritten
 *   o               : [N, H, dv]      dtype, written
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* beta, float* S, void* o, int N, int H, int dk, int dv,
                           kda_dtype dtype, hipStream_t stream);

/*
 * Several consecutive tokens per sequence in one pass over the state: the
 * verification step of speculative decoding, for which the K3 report
 * fine-tunes a draft model (blog.csdn.net article on the Kimi K3 report,
 * section 二, deployment-aware training).  Equivalent to ntok calls of
 * kda_decode_step, reading and writing the state once.
 *   q, k, log_alpha : [N, H, ntok, dk]   dtype
 *   v               : [N, H, ntok, dv]   dtype
 *   beta            : [N, H, ntok]       dtype (any element alignment)
 *   S_in            : [N, H, dk, dv]     fp32 state before the tokens
 *   S_out           : [N, H, dk, dv]     fp32, written with the state after all
 *                                        ntok tokens; may alias S_in (in place)
 *   o               : [N, H, ntok, dv]   dtype, written
 *   S_pos           : [N, ntok, H, dk, dv] fp32 or NULL: entry [n, t, h] is the
 *                     state after token t, the rollback point when only tokens
 *                     0..t are accepted; must not overlap any other argument
 * ntok == 0 copies S_in to S_out.  Errors: as for kda_decode_step.
 */
kda_status kda_decode_tokens(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* beta, const float* S_in, float* S_out, void* o, float* S_pos,
                             int N, int H, int ntok, int dk, int dv, kda_dtype dtype, hipStream_t stream);

/*
 * First half of the context-parallel decomposition ("Kimi K3 开源日来了",
 * section "针对适配的 Infra", KDA Context Parallelism): the sequence of every
 * (b, h), of T = G * Tseg tokens, is cut into G segments; for each segment this
 * computes, independently of the others,
 *   S_zero_end : [G, B, H, dk, dv]  fp32, its end state when started from zero
 *   M          : [G, B, H, dk, dk]  fp32, its transfer map, so that the end
 *                state from any start state X is  M X + S_zero_end.
 *   k, log_alpha : [B, H, T, dk] dtype;  v : [B, H, T, dv];  beta : [B, H, T].
 * Tseg >= 1.  q is not needed.
 */
kda_status kda_segment_transfer(const void* k, const void* v, const void* log_alpha,
                                const void* beta, float* S_zero_end, float* M, int B, int H, int G,
                                int Tseg, int dk, int dv, kda_dtype dtype, hipStream_t stream);

/*
 * Second half: the exchange that recovers each segment's true start state
 * (same section).  Per (b, h), sequentially over segments i = 0..G-1:
 *     S_start[i] = S;   S = M[i] S + S_zero_end[i];       and finally S_T = S,
 * starting from S = S_in (NULL for zero).  All arrays fp32:
 *   S_in [B,H,dk,dv] or NULL; S_zero_end [G,B,H,dk,dv]; M [G,B,H,dk,dk];
 *   S_start [G,B,H,dk,dv] or NULL (not written); S_T [B,H,dk,dv].
 * S_T may alias S_in; it must not alias S_zero_end, M or S_start.
 */
kda_status kda_segment_merge(const float* S_in, const float* S_zero_end, const float* M,
                             float* S_start, float* S_T, int B, int H, int G, int dk, int dv,
                             hipStream_t stream);

/*
 * Gradients of the prefill, for training (the K3 report credits FlashKDA with
 * faster training as well as inference: myzaker "Kimi K3 开源日来了", section
 * "FlashKDA").  For a loss L with dL/do = dO and dL/dS_T = dS_T this computes
 * the gradients with respect to every input of kda_chunk_prefill
 * (reverse-mode chain rule).
 *   q, k, v, log_alpha, beta, S0 : as for kda_chunk_prefill (S0 NULL = zero)
 *   dO   : [B, H, T, dv] dtype, or NULL (= 0)
 *   dS_T : [B, H, dk, dv] fp32, or NULL (= 0)
 *   dq, dk_, dlog_alpha : [B, H, T, dk] dtype;  dv_ : [B, H, T, dv] dtype;
 *   dbeta : [B, H, T] dtype;  dS0 : [B, H, dk, dv] fp32.
 * Each gradient takes the dtype of the input it belongs to (the states' is
 * fp32), as autograd frameworks expect.
 * bf16 inputs run in the chunked form, on the matrix cores (bf16 operands,
 * fp32 accumulation): a forward pass that keeps, for every 64-token chunk, its
 * start state S and Delta; beside it the reverse chain over the chunks
 * (dS' -> dS, which needs no forward state), which keeps dU = Diag(Gam) dS'
 * of every chunk and writes dv_; then every (head, chunk)'s remaining
 * gradients in parallel.  For tokens with beta below 2^-30 the two chains
 * also keep W = V - Kh S, Xbar and the token's row of strict_lower(Kh Kb^T),
 * from which such a token's dbeta is formed.  fp32
 * inputs run the recurrence's token steps backwards in fp32, token by token,
 * one workgroup (or two, each with half of the state's columns) per head.
 * The workspace (device memory, at least kda_backward_workspace_bytes for the
 * same dtype, 16-byte aligned) holds, for bf16, room for those per-chunk
 * values (bf16: S and dS' dk x dv each, W, Delta and Xbar 64 x dv each, the
 * 64 x 64 lower blocks; 117 KiB per chunk-head at d = 128) and one fp32 end
 * state per head; for fp32, a state
 * checkpoint every 64 tokens, the entering
 * states and vectors u = (Diag(alpha) S)^T k of one 64-token interval, per
 * head, and the two halves' row sums.  Its contents on return are undefined.
 * No output may alias an input or the workspace.  The bf16 path forks part of
 * its work to the same per-caller-stream side stream as the sequence-split
 * prefill.  Errors: KDA_ERR_NULL for a missing required pointer,
 * KDA_ERR_WORKSPACE for a missing workspace or one below the required size.
 */
size_t kda_backward_workspace_bytes(int B, int H, int T, int dk, int dv, kda_dtype dtype);
kda_status kda_prefill_backward(const void* q, const void* k, const void* v, const void* log_alpha,
                                const void* beta, const float* S0, const void* dO, const float* dS_T,
                                void* dq, void* dk_, void* dv_, void* dlog_alpha, void* dbeta,
                                float* dS0, int B, int H, int T, int dk, int dv, kda_dtype dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Process-wide options.  Each starts from the environment variable of the same
 * name in capitals with a KDA_ prefix (KDA_SPLIT, ...), read once, at the first
 * call that needs the options; kda_set_option changes one for every later call
 * (thread-safe; calls already enqueued are not affected).  value -1 restores the
 * library's default.  Names:
 *   "split"            segments of the sequence-split prefill (after the first
 *                      part with fixup 0; 0 = never split, >= 2 = that many;
 *                      default: chosen from the shape and the compute-unit
 *                      count)
 *   "fixup"            0: the split prefill's earlier pipeline (first part
 *                      beside the segment pass, merge, prefill of every
 *                      segment); default 1 (segments from zero, heads
 *                      corrected)
 *   "head_chunks"      chunks of every segment's map walked before deciding
 *                      whether it has vanished, and prefilled again when it
 *                      has (1..1024; default 4)
 *   "transfer_cost16"  with fixup 0: the first part's length ratio, in 16ths
 *                      (1..64)
 *   "map_skip"         0: the segment pass keeps updating transfer-map columns
 *                      that have become exactly zero (same results bit for bit
 *                      for finite inputs); default 1
 *   "nc"               consumer waves per workgroup of the chunk kernels
 *                      (1, 2, 4, 8 where built; default: chosen from the shape)
 *   "bw_split"         workgroups per head of the backward's chunk kernels (1 or
 *                      2; default: chosen from the shape)
 *   "bw_overlap"       bf16 backward from 16 chunks per head: 1 runs the
 *                      reverse chain in two launches (later half of the
 *                      chunks, then earlier half) and the later half's per-chunk
 *                      gradients beside the earlier half's chain, on the side
 *                      stream; 0 (default) runs the chain whole, then every
 *                      chunk's gradients.  Same results bit for bit
 *   "check"            1: validate log_alpha and beta on the device before every
 *                      call that reads them (see the conventions above); default 0
 *   "log"              1: print every launch's shape to stderr; default 0
 * kda_set_option returns KDA_ERR_SHAPE for an unknown name or a value the option
 * does not take; kda_get_option writes the value in effect (-1: default).
 */
kda_status kda_set_option(const char* name, long long value);
kda_status kda_get_option(const char* name, long long* value);

/*
 * Profiling only.  In a library built with KDA_PHASE_STAMPS (build.py
 * --stamps, libkda_stamps.so), every later sequence-split prefill records,
 * for each workgroup of its main launch (the prefill of every segment from
 * zero), the shader clock (s_memtime) of every wave at five points of
 * pipeline steps 32 .. 47: the step's start, the end of the elementwise phase
 * (producer waves) or of the chain (consumer waves), after the first barrier,
 * the end of the score tiles, after the second barrier.  With the environment
 * variable KDA_STAMP_TARGET set to "ckpt" or "reverse" when this is called,
 * the bf16 prefill backward's checkpoint pass or its reverse chain (in the
 * reverse chain, step i is chunk nch - 1 - i) records them instead.
 *   stamps : device buffer of count 64-bit entries, indexed
 *            [workgroup][step - 32][wave][point] with 8 wave slots; a
 *            workgroup whose entries do not fit records nothing; NULL (or
 *            count 0) stops recording
 * The regular library returns KDA_ERR_UNSUPPORTED and records nothing.
 */
kda_status kda_debug_phase_stamps(unsigned long long* stamps, size_t count);

/*
 * Profiling only (any build): the duration of the main launch (the prefill of
 * every segment from zero) of sequence-split prefills, timed with HIP events
 * recorded on the caller's stream around that launch, so that the calls
 * themselves are not synchronised.
 *   kda_debug_time_main_launches(count): arms count event pairs (1 .. 256)
 *     for the next count sequence-split prefills on the current device, and
 *     forgets what an earlier arming recorded; 0 disarms.  KDA_ERR_SHAPE for a
 *     count out of range.
 *   kda_debug_main_launch_ms(ms, count, recorded): *recorded = the launches
 *     timed since the arming; waits for them and writes the first
 *     min(count, *recorded) durations in milliseconds to ms (host memory).
 * One caller at a time: calls that overlap on other threads may take each
 * other's pairs.
 */
kda_status kda_debug_time_main_launches(int count);
kda_status kda_debug_main_launch_ms(float* ms, int count, int* recorded);

const char* kda_status_string(kda_status status);
const char* kda_last_error(void);
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_H */
