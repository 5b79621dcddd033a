// C-ABI of libkda: host-side validation, launch geometry and error mapping.
// Every check runs before anything is enqueued, so a rejected call writes
// nothing.  See include/libkda.h for the contract of each entry point.
#include "../../include/libkda.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kda_launch.hpp"

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status fail(kda_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kda_status ok() {
  g_err[0] = '\0';
  return KDA_OK;
}

kda_status hip_fail(hipError_t e, const char* what) {
  return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------------ options
// Process-wide switches (see kda_set_option in libkda.h).  Each starts from its
// environment variable, read once; -1 means the library's default.
enum Opt {
  OPT_SPLIT, OPT_COST16, OPT_MAP_SKIP, OPT_NC, OPT_BW_SPLIT, OPT_CHECK, OPT_LOG, OPT_FIXUP, OPT_HEAD,
  OPT_BW_OVERLAP, OPT_COUNT
};
struct OptDesc {
  const char* name;
  const char* env;
};
const OptDesc kOpts[OPT_COUNT] = {{"split", "KDA_SPLIT"},       {"transfer_cost16", "KDA_TRANSFER_COST16"},
                                  {"map_skip", "KDA_MAP_SKIP"}, {"nc", "KDA_NC"},
                                  {"bw_split", "KDA_BW_SPLIT"}, {"check", "KDA_CHECK"},
                                  {"log", "KDA_LOG"},           {"fixup", "KDA_FIXUP"},
                                  {"head_chunks", "KDA_HEAD_CHUNKS"}, {"bw_overlap", "KDA_BW_OVERLAP"}};
std::atomic<long long> g_opt[OPT_COUNT];
std::once_flag g_opt_once;

bool opt_valid(int o, long long v) {
  if (v == -1) return true;
  switch (o) {
    case OPT_SPLIT: return v == 0 || (v >= 2 && v <= 4096);
    case OPT_COST16: return v >= 1 && v <= 64;
    case OPT_NC: return v == 1 || v == 2 || v == 4 || v == 8;
    case OPT_BW_SPLIT: return v == 1 || v == 2;
    case OPT_HEAD: return v >= 1 && v <= 1024;
    default: return v == 0 || v == 1;  // map_skip, check, log, fixup, bw_overlap
  }
}

void init_opts() {
  for (int o = 0; o < OPT_COUNT; ++o) {
    long long v = -1;
    if (const char* env = getenv(kOpts[o].env)) {
      char* end = nullptr;
      const long long x = strtoll(env, &end, 10);
      if (end != env && opt_valid(o, x)) v = x;
      else if (o == OPT_LOG && env[0]) v = 1;  // any non-numeric KDA_LOG turns logging on
    }
    g_opt[o].store(v, std::memory_order_relaxed);
  }
}

long long opt(Opt o) {
  std::call_once(g_opt_once, init_opts);
  return g_opt[o].load(std::memory_order_relaxed);
}

bool log_on() { return opt(OPT_LOG) == 1; }

// Compute units of the current device (cached per device id).
int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Workgroups per head of the fp32 (token-step) backward: two, each with half
// of the state's columns, when that still fits the chip in one round; option
// bw_split forces the choice.
int bw_split(long long BH) {
  if (const long long v = opt(OPT_BW_SPLIT); v == 1 || v == 2) return (int)v;
  return 2 * BH <= cu_count() ? 2 : 1;
}

// Option map_skip = 0 keeps the segment pass updating map columns that have
// become exactly zero (for tests that compare both ways); by default it stops.
bool map_skip_enabled() { return opt(OPT_MAP_SKIP) != 0; }

// Consumer waves per workgroup (each owns chunk_tiles_per_wave(bf16) 16-column
// state tiles): the smallest of 1, 2, 4 (fp32: 1, 2) that divides the column
// tiles and still launches no more workgroups than there are compute units, so
// that the sequences run in one round with their columns split as far as that
// allows (else the largest).  A second round walks whole sequences again: at
// 160 heads x 8192 tokens two workgroups per head took 0.785 ms against 0.475
// for one, at 100 heads x 2048 four took 0.208 ms against 0.106 for two.
// Option nc overrides for tuning and tests, where that count is built.
int pick_nc(long long nseq, int ncol_tiles, bool bf16_io, bool allow8 = false) {
  const int ncmax = bf16_io ? (allow8 ? 8 : 4) : 2;
  const int tw = kda::chunk_tiles_per_wave(bf16_io);
  const long long v = opt(OPT_NC);
  if (v > 0 && v <= ncmax && ncol_tiles % (v * tw) == 0) return (int)v;
  const long long cus = cu_count();
  // 8 consumer waves (segment pass, 2*D columns in one workgroup): when one
  // workgroup per sequence fills one round of the chip but 4 waves would need
  // two, one round of the larger workgroups wins (measured: about 1.8x the
  // per-workgroup time, with no duplicated producer work).
  if (ncmax == 8 && ncol_tiles == 8 * tw && nseq <= cus && 2 * nseq > cus) return 8;
  int largest = 1;
  for (int nc = 1; nc <= ncmax; nc <<= 1) {
    if (ncol_tiles % (nc * tw)) continue;
    if (nseq * (ncol_tiles / (nc * tw)) <= cus) return nc;
    largest = nc;
  }
  return largest;
}

// Prefill of few heads over a long sequence: rather than splitting each head's
// state columns over many workgroups (each of which then repeats the whole
// per-chunk preparation), cut the sequence and use the context-parallel
// decomposition.
//
// Default (option fixup = 1): G segments of Tseg tokens (the last one may be
// shorter).  Segment 0 starts from S0, every other one from zero, and all of
// them are prefilled at once, outputs included.  A segment's true outputs
// differ from its zero-start ones by O_M S_start, where O_M is what the
// segment's transfer map contributes to each output; once the map is exactly
// zero (it stays zero for finite inputs) that term is exactly zero.  So a short
// walk over the first head_chunks chunks of every segment's map decides, per
// (segment, head), whether the map has vanished there.  If it has, only those
// first chunks are walked again from the true start state, after the merge;
// if not, the segment takes the path below (its zero-start end state and map
// from the segment pass, then its whole prefill again).  Which of the two a
// segment takes is decided on the device, so nothing waits on the host.
//
// Option fixup = 0: the first T0 tokens start from the known S0 and are simply
// prefilled; meanwhile the segment pass computes the zero-start end state and
// transfer map of each of the next G - 1 segments of Tseg tokens.  A sequential
// merge then gives the true start state of each of the G remaining segments
// (the last one ends at T and may be shorter), which are prefilled
// independently.  The result is the same recurrence.
//
// T0 is chosen so that the direct prefill and the segment pass, which run side
// by side, end together.  The segment pass skips q and the outputs but carries
// twice the state columns, and stops updating map columns once they have
// decayed to exact zero; running beside the prefill it costs about 12/16 of it
// per token when the gates decay as fast as in the 64K-token, 32-head workload
// (10/16 to 15/16 measured there: 12/16 fastest, 15/16 3% slower) and about
// 15/16 when the map never reaches zero (11/16 to 19/16 within 1% of each
// other).  Option transfer_cost16 overrides the ratio for tuning.
struct PrefillPlan {
  bool split = false;
  int T0 = 0, G = 1, Tseg = 0;
  size_t ws = 0;
};

constexpr int kTransferCost16 = 12;  // segment pass / prefill time per token, in 16ths
constexpr int kHeadChunks = 4;       // chunks walked to decide whether a segment's map has vanished

int head_chunks() {
  const long long v = opt(OPT_HEAD);
  return v >= 1 && v <= 1024 ? (int)v : kHeadChunks;
}

bool fixup_enabled() { return opt(OPT_FIXUP) != 0; }

PrefillPlan plan_prefill(long long BH, int T, int D, kda_dtype dt) {
  PrefillPlan pl;
  pl.Tseg = T;
  if (dt != KDA_BF16 || BH <= 0 || T <= 0) return pl;
  const long long cus = cu_count();
  const int ntiles = D / 16;
  long long G = opt(OPT_SPLIT);  // 0: never; >= 2: that many segments (after the first part)
  if (G >= 0) {
    if (G < 2) return pl;
  } else {
    // worth it when one pass cannot fill the chip without 4+ workgroups per head
    if (BH * ntiles / 4 >= cus || T < 4096) return pl;
    // one round of segment prefills: with G * BH above the CU count the last
    // workgroups would walk a whole segment again on their own (at 48 heads,
    // 6 segments took 1.36 ms against 0.95 ms for 5)
    G = cus / BH;
    if (G > T / 1024) G = T / 1024;
    if (G < 2) return pl;
  }
  if (fixup_enabled()) {
    // G equal segments, the first from S0
    const long long Tseg = ((T + G - 1) / G + 63) / 64 * 64;
    const long long Geff = (T + Tseg - 1) / Tseg;
    if (Geff < 2) return pl;
    pl.split = true;
    pl.T0 = 0;
    pl.G = (int)Geff;
    pl.Tseg = (int)Tseg;
    // Z of all G segments, M and start states of the G - 1 after the first,
    // and their records
    pl.ws = (size_t)(3 * Geff - 2) * BH * D * D * sizeof(float) +
            (size_t)(Geff - 1) * BH * kda::kFlagSlots * sizeof(uint32_t);
    return pl;
  }
  long long cost16 = opt(OPT_COST16);
  if (cost16 < 1 || cost16 > 64) cost16 = kTransferCost16;
  for (; G >= 2; --G) {
    // T = T0 + (G - 1) * Tseg + last, 0 < last <= Tseg, T0 ~ (cost16/16) Tseg
    const long long unit = 64LL * (16 * G + cost16);
    long long Tseg = (16LL * T + unit - 1) / unit * 64;
    long long T0 = cost16 * Tseg / 16 / 64 * 64;
    if (T0 < 64) T0 = 64;
    if (T - T0 > G * Tseg) T0 = (T - G * Tseg + 63) / 64 * 64;
    const long long last = T - T0 - (G - 1) * Tseg;
    if (last <= 0 || last > Tseg || T0 >= T) continue;
    pl.split = true;
    pl.T0 = (int)T0;
    pl.G = (int)G;
    pl.Tseg = (int)Tseg;
    // Z and M of G - 1 segments, the direct part's end state, G start states
    pl.ws = (size_t)(3 * G - 1) * BH * D * D * sizeof(float);
    return pl;
  }
  return pl;
}

// A second stream on which the segment pass runs beside the direct prefill of
// the first part (default priority, non-blocking, kept for the process
// lifetime), with the events that fork it from and join it to the caller's
// stream: one per (device, caller stream), so that split calls issued on
// independent streams do not queue behind each other.  The table holds
// kSideSlots caller streams per device; past that, a caller stream shares the
// slot its handle hashes to (still correct, only no longer independent).  The
// mutex keeps one call's record/wait sequence whole.
struct SideStream {
  hipStream_t owner = nullptr;  // the caller stream this slot serves
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipEvent_t mid = nullptr, mid2 = nullptr;  // two more cross-stream points (the chunked backward)
  std::mutex mu;
};
constexpr int kSideSlots = 64;

kda_status side_stream(hipStream_t caller, SideStream** out) {
  static std::mutex mu;
  static SideStream* table[64][kSideSlots] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(KDA_ERR_UNSUPPORTED, "device %d out of range", dev);
  const uint64_t hsh = (reinterpret_cast<uintptr_t>(caller) >> 4) * 0x9E3779B97F4A7C15ull;
  const int home = (int)(hsh >> 58);  // 0 .. 63
  std::lock_guard<std::mutex> lk(mu);
  SideStream** row = table[dev];
  for (int i = 0; i < kSideSlots; ++i) {
    const int slot = (home + i) % kSideSlots;
    if (row[slot] && row[slot]->owner == caller) {
      *out = row[slot];
      return KDA_OK;
    }
    if (!row[slot]) {
      SideStream* ss = new SideStream();
      ss->owner = caller;
      if ((e = hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking)) != hipSuccess ||
          (e = hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming)) != hipSuccess ||
          (e = hipEventCreateWithFlags(&ss->join, hipEventDisableTiming)) != hipSuccess ||
          (e = hipEventCreateWithFlags(&ss->mid, hipEventDisableTiming)) != hipSuccess ||
          (e = hipEventCreateWithFlags(&ss->mid2, hipEventDisableTiming)) != hipSuccess) {
        delete ss;  // (a partly created stream or event is left to process exit)
        return hip_fail(e, "creating the side stream");
      }
      row[slot] = ss;
      *out = ss;
      return KDA_OK;
    }
  }
  *out = row[home];  // table full: share
  return KDA_OK;
}

// With the check option set: log_alpha (n_la values) and beta (n_beta) are
// read on the device and KDA_ERR_PRECONDITION is returned if any is out of
// range or not finite.  Synchronises `stream`.
kda_status check_gates(const void* la, long long n_la, const void* beta, long long n_beta, kda_dtype dt,
                       hipStream_t stream) {
  if (opt(OPT_CHECK) != 1 || (n_la == 0 && n_beta == 0)) return KDA_OK;
  unsigned int bits = 0u;
  const hipError_t e = kda::check_gates(la, n_la, beta, n_beta, dt == KDA_BF16, stream, &bits);
  if (e != hipSuccess) return hip_fail(e, "input check");
  if (bits & 1u)
    return fail(KDA_ERR_PRECONDITION, "log_alpha has values outside [-1, 0] or not finite (check mode)");
  if (bits & 2u) return fail(KDA_ERR_PRECONDITION, "beta has values outside [0, 1] or not finite (check mode)");
  return KDA_OK;
}

kda_status check_dims(int dk, int dv) {
  if (dk != dv) return fail(KDA_ERR_SHAPE, "dk (%d) must equal dv (%d)", dk, dv);
  if (dk != 64 && dk != 128) return fail(KDA_ERR_UNSUPPORTED, "head size %d not supported (64 or 128)", dk);
  return KDA_OK;
}

kda_status check_dtype(kda_dtype dt) {
  if (dt != KDA_F32 && dt != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return KDA_OK;
}

#define KDA_REQUIRE(p, name)                                                     \
  do {                                                                           \
    if (!(p)) return fail(KDA_ERR_NULL, "%s is NULL", name);                     \
    if (!aligned(p)) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

#define KDA_OPTIONAL(p, name)                                                    \
  do {                                                                           \
    if ((p) && !aligned(p)) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

const long long kMaxElems = (1LL << 40);

// Kernels address one sequence through a 32-bit buffer range.
kda_status check_seq_bytes(long long T, int dk, kda_dtype dt) {
  const long long es = dt == KDA_BF16 ? 2 : 4;
  if ((T + 64) * dk * es > INT32_MAX)
    return fail(KDA_ERR_UNSUPPORTED, "sequence of %lld tokens exceeds 2 GiB per tensor and head", T);
  return KDA_OK;
}

// Prefill of G = ceil(T / Tseg) consecutive segments of every head, each from its
// own start state (Sst: [G, BH, D, D] or null for zero); S_T receives the end
// state of the last segment.
struct Snap {
  float* p = nullptr;  // [B, nsnap, H, D, D] or null
  int chunks = 0;      // chunks per snapshot interval
  int n = 0;
  int H = 1;
};

// Phase timestamps of the profiling build (kda_debug_phase_stamps), and the
// launch that records them: 0 the sequence-split prefill's main launch, 1 the
// backward's checkpoint pass, 2 the backward's reverse chain.
std::atomic<unsigned long long*> g_stamps{nullptr};
std::atomic<size_t> g_stamps_n{0};
std::atomic<int> g_stamp_target{0};

// Events around the main launch of the next sequence-split prefills
// (kda_debug_time_main_launches): pair i brackets the i-th armed launch.
constexpr int kMaxTimedLaunches = 256;
struct MainTimer {
  std::mutex mu;
  int dev = -1;
  int cap = 0;    // armed pairs
  int n = 0;      // pairs recorded so far
  int made = 0;   // pairs created on `dev`
  hipEvent_t ev[2 * kMaxTimedLaunches] = {};
};
MainTimer g_mt;

// The next armed event pair on the current device, or nulls when none is armed.
void main_timer_slot(hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  std::lock_guard<std::mutex> lk(g_mt.mu);
  int dev = -1;
  if (g_mt.n >= g_mt.cap || hipGetDevice(&dev) != hipSuccess || dev != g_mt.dev) return;
  *start = g_mt.ev[2 * g_mt.n];
  *stop = g_mt.ev[2 * g_mt.n + 1];
  ++g_mt.n;
}

// Per-segment control of a prefill launch in the split path with corrected
// heads (ChunkArgs::seg_flag and the fields after it).
struct SegCtl {
  uint32_t* rec = nullptr;
  int mode = kda::FLAG_NONE;
  int g0 = 0;
  int head = 0;
  float* Z_out = nullptr;
  bool s0_first = false;
  const float* Z_prev = nullptr;
};

// Prefill of the G = ceil((Tend - t0) / Tseg) consecutive segments of tokens
// [t0, Tend) of every head (sequences of T tokens), segment i from Sst[i] (null:
// zero; with sc.s0_first, Sst [BH, D, D] is segment 0's start and the others
// start from zero); S_T (if not null) receives the end state of the last
// segment.  nc = 0 picks the consumer-wave count.
kda_status launch_segment_prefill(const void* q, const void* k, const void* v, const void* log_alpha,
                                  const void* beta, const float* Sst, void* o, float* S_T,
                                  long long BH, int T, int t0, int Tend, int Tseg, int D, bool bf,
                                  hipStream_t stream, const char* what, const Snap& sn = Snap(),
                                  int nc = 0, kda::bf16* ck_rows = nullptr, kda::bf16* ck_w = nullptr,
                                  kda::bf16* ck_d = nullptr, kda::bf16* ck_a = nullptr,
                                  const SegCtl& sc = SegCtl()) {
  const int n = Tend - t0;
  const int G = n > 0 ? (int)(((long long)n + Tseg - 1) / Tseg) : 1;  // no tokens: copy the start state
  const long long nseq = BH * G;
  const int nt = D / 16;
  if (nc == 0) nc = pick_nc(nseq, nt, bf);
  kda::ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
  a.S0 = Sst; a.o = o; a.S_out = S_T; a.M_out = nullptr;
  a.BH = (int)BH; a.G = G; a.Tseg = Tseg; a.Ttot = T; a.t0 = t0; a.Tend = Tend;
  a.vsplit = nt / (nc * kda::chunk_tiles_per_wave(bf));
  a.snap = sn.n > 0 ? sn.p : nullptr; a.snap_chunks = sn.chunks > 0 ? sn.chunks : 1;
  a.nsnap = sn.n; a.H = sn.H;
  a.ck_rows = ck_rows; a.ck_w = ck_w; a.ck_d = ck_d; a.ck_a = ck_a;
  a.seg_flag = sc.rec; a.flag_mode = sc.mode; a.flag_g0 = sc.g0; a.head_chunks = sc.head;
  a.Z_out = sc.Z_out; a.s0_first = sc.s0_first ? 1 : 0; a.Z_prev = sc.Z_prev;
  const int stamp_target = g_stamp_target.load(std::memory_order_relaxed);
  if ((sc.mode == kda::FLAG_FAST_ONLY && stamp_target == 0) || (ck_rows && stamp_target == 1)) {
    a.stamps = g_stamps.load(std::memory_order_relaxed);
    a.stamps_n = g_stamps_n.load(std::memory_order_relaxed);
  }
  const long long nwg = nseq * a.vsplit;
  if (nwg > INT32_MAX) return fail(KDA_ERR_SHAPE, "problem too large");
  if (log_on())
    fprintf(stderr, "[libkda] %s BH=%lld T=%d tokens [%d,%d) Tseg=%d G=%d D=%d nc=%d vsplit=%d grid=%lld\n",
            what, BH, T, t0, Tend, Tseg, G, D, nc, a.vsplit, nwg);
  // with checkpoints (and no outputs) the checkpoint-only variant runs
  const hipError_t e = ck_rows ? kda::launch_chunk_ckpt(a, D, nc, (int)nwg, stream)
                               : kda::launch_chunk(a, bf, D, true, nc, (int)nwg, stream);
  if (e != hipSuccess) return hip_fail(e, what);
  return KDA_OK;
}

// Validation shared by the prefill entry points.
kda_status check_prefill_args(const void* q, const void* k, const void* v, const void* log_alpha,
                              const void* beta, void* o, float* S_T, int B, int H, int T, int dk,
                              int dv, kda_dtype dtype) {
  if (B < 0 || H < 0 || T < 0) return fail(KDA_ERR_SHAPE, "negative size B=%d H=%d T=%d", B, H, T);
  kda_status st;
  if ((st = check_dtype(dtype)) != KDA_OK) return st;
  if ((st = check_dims(dk, dv)) != KDA_OK) return st;
  const long long BH = (long long)B * H;
  if (BH * T * dk > kMaxElems || BH > (1LL << 30)) return fail(KDA_ERR_SHAPE, "problem too large");
  if ((st = check_seq_bytes(T, dk, dtype)) != KDA_OK) return st;
  if (BH == 0) return KDA_OK;
  KDA_REQUIRE(S_T, "S_T");
  if (T > 0) {
    KDA_REQUIRE(q, "q");
    KDA_REQUIRE(k, "k");
    KDA_REQUIRE(v, "v");
    KDA_REQUIRE(log_alpha, "log_alpha");
    KDA_REQUIRE(beta, "beta");
    KDA_REQUIRE(o, "o");
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

kda_status kda_set_option(const char* name, long long value) {
  if (!name) return fail(KDA_ERR_NULL, "option name is NULL");
  for (int o = 0; o < OPT_COUNT; ++o) {
    if (strcmp(name, kOpts[o].name) != 0) continue;
    if (!opt_valid(o, value)) return fail(KDA_ERR_SHAPE, "option %s does not take the value %lld", name, value);
    opt((Opt)o);  // environment defaults first, so they do not overwrite this later
    g_opt[o].store(value, std::memory_order_relaxed);
    return ok();
  }
  return fail(KDA_ERR_SHAPE, "unknown option '%s'", name);
}

kda_status kda_get_option(const char* name, long long* value) {
  if (!name || !value) return fail(KDA_ERR_NULL, "option name or value pointer is NULL");
  for (int o = 0; o < OPT_COUNT; ++o) {
    if (strcmp(name, kOpts[o].name) != 0) continue;
    *value = opt((Opt)o);
    return ok();
  }
  return fail(KDA_ERR_SHAPE, "unknown option '%s'", name);
}

const char* kda_last_error(void) { return g_err; }

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "null pointer";
    case KDA_ERR_SHAPE: return "invalid shape";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_ALIGN: return "misaligned pointer";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_PRECONDITION: return "input precondition violated";
    case KDA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

kda_status kda_debug_phase_stamps(unsigned long long* stamps, size_t count) {
#ifdef KDA_PHASE_STAMPS
  if (!stamps) count = 0;
  const char* t = getenv("KDA_STAMP_TARGET");
  g_stamp_target.store(t && !strcmp(t, "ckpt") ? 1 : t && !strcmp(t, "reverse") ? 2 : 0, std::memory_order_relaxed);
  g_stamps.store(count ? stamps : nullptr, std::memory_order_relaxed);
  g_stamps_n.store(count, std::memory_order_relaxed);
  return ok();
#else
  (void)stamps;
  (void)count;
  return fail(KDA_ERR_UNSUPPORTED, "phase timestamps need the profiling build (KDA_PHASE_STAMPS)");
#endif
}

kda_status kda_debug_time_main_launches(int count) {
  if (count < 0 || count > kMaxTimedLaunches)
    return fail(KDA_ERR_SHAPE, "count %d out of range (0 .. %d)", count, kMaxTimedLaunches);
  std::lock_guard<std::mutex> lk(g_mt.mu);
  g_mt.cap = g_mt.n = 0;
  if (count == 0) return ok();
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != g_mt.dev) {  // events belong to the device current when they were created
    for (int i = 0; i < 2 * g_mt.made; ++i) (void)hipEventDestroy(g_mt.ev[i]);
    g_mt.made = 0;
    g_mt.dev = dev;
  }
  for (; g_mt.made < count; ++g_mt.made)
    if ((e = hipEventCreate(&g_mt.ev[2 * g_mt.made])) != hipSuccess ||
        (e = hipEventCreate(&g_mt.ev[2 * g_mt.made + 1])) != hipSuccess)
      return hip_fail(e, "hipEventCreate");
  g_mt.cap = count;
  return ok();
}

kda_status kda_debug_main_launch_ms(float* ms, int count, int* recorded) {
  if (!recorded) return fail(KDA_ERR_NULL, "recorded is NULL");
  if (count < 0) return fail(KDA_ERR_SHAPE, "count %d is negative", count);
  if (count > 0 && !ms) return fail(KDA_ERR_NULL, "ms is NULL");
  std::lock_guard<std::mutex> lk(g_mt.mu);
  *recorded = g_mt.n;
  for (int i = 0; i < g_mt.n && i < count; ++i) {
    hipError_t e = hipEventSynchronize(g_mt.ev[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], g_mt.ev[2 * i], g_mt.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "reading the launch events");
  }
  return ok();
}

size_t kda_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, kda_dtype dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || dk != dv || (dk != 64 && dk != 128)) return 0;
  return plan_prefill((long long)B * H, T, dk, dtype).ws;
}

kda_status kda_prefill_plan(int B, int H, int T, int dk, int dv, kda_dtype dtype, int* T0, int* G,
                            int* Tseg) {
  if (!T0 || !G || !Tseg) return fail(KDA_ERR_NULL, "T0, G and Tseg must not be NULL");
  if (B < 0 || H < 0 || T < 0) return fail(KDA_ERR_SHAPE, "negative size B=%d H=%d T=%d", B, H, T);
  kda_status st;
  if ((st = check_dtype(dtype)) != KDA_OK) return st;
  if ((st = check_dims(dk, dv)) != KDA_OK) return st;
  const PrefillPlan pl = plan_prefill((long long)B * H, T, dk, dtype);
  *T0 = pl.split ? pl.T0 : 0;
  *G = pl.split ? pl.G : 1;
  *Tseg = pl.split ? pl.Tseg : T;
  return ok();
}

}  // extern "C"

namespace {

// Scratch of the no-allocation prefill entry point: the sequence-split path's
// states and segment records when the caller cannot pass a workspace.  Every
// default plan on a 256-CU device fits (at most 48 MiB: one head of d = 128
// cut into 256 segments); each device the library runs on holds its own copy
// until the process ends.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) char scratch[kScratchBytes];

// The scratch array's device address on the current device, looked up once per
// device (with that device current) with hipGetSymbolAddress.  The array's name
// in host code is only a host-side stand-in and must never be passed to a
// kernel or a copy.
kda_status scratch_ptr(void** out) {
  static std::mutex mu;
  static void* cache[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(KDA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    cache[dev] = p;
  }
  *out = cache[dev];
  return KDA_OK;
}

// The split prefill with corrected segment heads (plan T0 = 0): G segments of
// Ts tokens, segment 0 from S0.  The workspace holds Z [G, BH, D, D] (the
// zero-start end states; segment 0's from S0), M and the start states
// [G - 1, BH, D, D] of segments 1 .. G-1, and their records [G - 1, BH,
// kFlagSlots].  On the caller's stream, with the segment pass's step on the
// side stream:
//  1. the head walk: the first head_chunks chunks of every later segment's
//     transfer map, which writes the records (nonzero: the map has not
//     vanished there);
//  2. beside each other: the prefill of segment 0 and of every segment whose map
//     vanished, from zero, outputs and end states included; and the segment
//     pass over the others (their Z and M);
//  3. the merge, which runs the chain only through the segments whose map did
//     not vanish (after a segment whose map vanished, the next one's start
//     state is that segment's zero-start end state, read from Z directly);
//  4. the prefill from the true start states: the first head_chunks chunks of
//     the segments whose map vanished (their outputs are replaced), the whole
//     of the others.
kda_status prefill_split_heads(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const float* S0, void* o, float* S_T, long long BH,
                               int T, int D, bool bf, int G, int Ts, float* ws, const Snap& sn,
                               hipStream_t stream) {
  const int G1 = G - 1;
  const size_t nS = (size_t)BH * D * D;
  float* Z = ws;              // [G]
  float* M = Z + G * nS;      // [G - 1], segments 1 .. G-1
  float* Sst = M + G1 * nS;   // [G - 1]
  uint32_t* rec = reinterpret_cast<uint32_t*>(Sst + G1 * nS);
  const int head = head_chunks();
  SideStream* ss = nullptr;
  kda_status st;
  if ((st = side_stream(stream, &ss)) != KDA_OK) return st;
  // the segment pass's launches cover segments 1 .. G-1
  kda::ChunkArgs t;
  t.q = nullptr; t.k = k; t.v = v; t.la = log_alpha; t.beta = beta;
  t.S0 = nullptr; t.o = nullptr; t.S_out = nullptr; t.M_out = nullptr;
  t.BH = (int)BH; t.G = G1; t.Tseg = Ts; t.Ttot = T; t.t0 = Ts; t.Tend = T;
  const int nt2 = 2 * D / 16, nc2 = pick_nc(BH * G1, nt2, bf, D == 128);
  t.vsplit = nt2 / (nc2 * kda::chunk_tiles_per_wave(bf));
  t.map_skip = map_skip_enabled();
  t.seg_flag = rec; t.flag_g0 = 0; t.head_chunks = head;
  const int nwg2 = (int)(BH * G1 * t.vsplit);
  const int nc1 = D / 16 / kda::chunk_tiles_per_wave(bf);  // one workgroup per sequence
  if (log_on())
    fprintf(stderr, "[libkda] prefill split BH=%lld T=%d D=%d: %d x %d-token segments, heads of %d chunks "
            "corrected; transfer nc=%d vsplit=%d\n", BH, T, D, G, Ts, head, nc2, t.vsplit);
  hipError_t e;
  // 1. the head walk
  t.flag_mode = kda::FLAG_HEAD;
  if ((e = kda::launch_chunk(t, bf, D, false, nc2, nwg2, stream)) != hipSuccess)
    return hip_fail(e, "kda_chunk_prefill head walk");
  {
    // 2. the segment pass over the segments whose map did not vanish (side
    //    stream), beside the prefill of all the others from zero
    std::lock_guard<std::mutex> lk(ss->mu);
    if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess ||
        (e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess)
      return hip_fail(e, "kda_chunk_prefill fork");
    t.flag_mode = kda::FLAG_SLOW_ONLY;
    t.S_out = Z + nS;
    t.M_out = M;
    if ((e = kda::launch_chunk(t, bf, D, false, nc2, nwg2, ss->s)) != hipSuccess)
      return hip_fail(e, "kda_chunk_prefill segment pass");
    SegCtl sc;
    sc.rec = rec; sc.mode = kda::FLAG_FAST_ONLY; sc.g0 = 1; sc.Z_out = Z; sc.s0_first = true;
    hipEvent_t t0 = nullptr, t1 = nullptr;  // profiling hook: this launch's duration
    main_timer_slot(&t0, &t1);
    if (t0 && (e = hipEventRecord(t0, stream)) != hipSuccess) st = hip_fail(e, "kda_chunk_prefill event");
    if (st == KDA_OK)
      st = launch_segment_prefill(q, k, v, log_alpha, beta, S0, o, nullptr, BH, T, 0, T, Ts, D, bf, stream,
                                  "kda_chunk_prefill zero-start segments", sn, nc1, nullptr, nullptr, nullptr,
                                  nullptr, sc);
    if (st == KDA_OK && t1 && (e = hipEventRecord(t1, stream)) != hipSuccess)
      st = hip_fail(e, "kda_chunk_prefill event");
    // join even if the launch above failed, so the side stream's work is waited for
    if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess ||
        (e = hipStreamWaitEvent(stream, ss->join, 0)) != hipSuccess)
      return hip_fail(e, "kda_chunk_prefill join");
    if (st != KDA_OK) return st;
  }
  // 3. the merge, from segment 0's end state
  if ((e = kda::launch_merge(Z, Z + nS, M, Sst, S_T, (int)BH, G1, D, stream, rec)) != hipSuccess)
    return hip_fail(e, "kda_chunk_prefill merge");
  // 4. the heads (or whole segments) again from the true start states
  SegCtl sc;
  sc.rec = rec; sc.mode = kda::FLAG_FIX; sc.g0 = 0; sc.head = head; sc.Z_prev = Z;
  return launch_segment_prefill(q, k, v, log_alpha, beta, Sst, o, nullptr, BH, T, Ts, T, Ts, D, bf, stream,
                                "kda_chunk_prefill corrected heads", sn, nc1, nullptr, nullptr, nullptr,
                                nullptr, sc);
}

// The prefill with or without snapshots.  noalloc: the split path's workspace is
// the library's scratch array (workspace / workspace_bytes are ignored), and a
// plan that needs more than the array holds is refused.
kda_status prefill_impl(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                        const float* S0, void* o, float* S_T, float* S_snap, int snap_interval, int B, int H,
                        int T, int dk, int dv, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                        bool noalloc, hipStream_t stream) {
  kda_status st = check_prefill_args(q, k, v, log_alpha, beta, o, S_T, B, H, T, dk, dv, dtype);
  if (st != KDA_OK) return st;
  if (snap_interval < 0 || snap_interval % 64)
    return fail(KDA_ERR_SHAPE, "snap_interval must be 0 or a positive multiple of 64 (got %d)",
                snap_interval);
  const long long BH = (long long)B * H;
  if (BH == 0) return ok();
  KDA_OPTIONAL(S0, "S0");
  KDA_OPTIONAL(workspace, "workspace");
  Snap sn;
  if (snap_interval > 0 && T / snap_interval > 0) {
    KDA_REQUIRE(S_snap, "S_snap");
    sn.p = S_snap;
    sn.chunks = snap_interval / 64;
    sn.n = T / snap_interval;
    sn.H = H;
  }
  if (T > 0 && (st = check_gates(log_alpha, BH * T * dk, beta, BH * T, dtype, stream)) != KDA_OK) return st;
  const bool bf = dtype == KDA_BF16;
  const int D = dk;
  const PrefillPlan pl = plan_prefill(BH, T, D, dtype);
  if (noalloc) {
    workspace = nullptr;
    workspace_bytes = 0;
    if (pl.split) {
      if (pl.ws > kScratchBytes)
        return fail(KDA_ERR_WORKSPACE,
                    "the sequence-split plan needs %zu bytes of scratch; the no-allocation entry point "
                    "holds %zu", pl.ws, kScratchBytes);
      if ((st = scratch_ptr(&workspace)) != KDA_OK) return st;
      workspace_bytes = kScratchBytes;
    }
  }
  if (pl.split && workspace && workspace_bytes >= pl.ws && pl.T0 == 0) {
    st = prefill_split_heads(q, k, v, log_alpha, beta, S0, o, S_T, BH, T, D, bf, pl.G, pl.Tseg,
                             static_cast<float*>(workspace), sn, stream);
    return st == KDA_OK ? ok() : st;
  }
  if (pl.split && workspace && workspace_bytes >= pl.ws) {
    const int G = pl.G, G1 = G - 1, T0 = pl.T0, Ts = pl.Tseg;
    const size_t nS = (size_t)BH * D * D;
    float* Z = static_cast<float*>(workspace);  // [G-1] zero-start end states
    float* M = Z + G1 * nS;                     // [G-1] transfer maps
    float* S1 = M + G1 * nS;                    // end state of the direct part
    float* Sst = S1 + nS;                       // [G] start states of the segments
    SideStream* ss = nullptr;
    if ((st = side_stream(stream, &ss)) != KDA_OK) return st;
    kda::ChunkArgs t;
    t.q = nullptr; t.k = k; t.v = v; t.la = log_alpha; t.beta = beta;
    t.S0 = nullptr; t.o = nullptr; t.S_out = Z; t.M_out = M;
    t.BH = (int)BH; t.G = G1; t.Tseg = Ts; t.Ttot = T; t.t0 = T0; t.Tend = T0 + G1 * Ts;
    const int nt2 = 2 * D / 16, nc2 = pick_nc(BH * G1, nt2, bf, D == 128);
    t.vsplit = nt2 / (nc2 * kda::chunk_tiles_per_wave(bf));
    t.map_skip = map_skip_enabled();
    // the direct part: one workgroup per head (all of a head's column tiles) when
    // the segment pass leaves room for it, else the usual choice
    const int nc0 = BH * (G1 * t.vsplit + 1) <= cu_count() ? D / 16 / kda::chunk_tiles_per_wave(bf) : 0;
    if (log_on())
      fprintf(stderr, "[libkda] prefill split BH=%lld T=%d D=%d: direct [0,%d), %d x %d-token segments; "
              "transfer nc=%d vsplit=%d\n", BH, T, D, T0, G, Ts, nc2, t.vsplit);
    hipError_t e;
    {
      // 1. beside each other: the direct prefill of tokens [0, T0) from S0, and
      //    the segment pass over the G - 1 segments that follow it
      std::lock_guard<std::mutex> lk(ss->mu);
      if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess ||
          (e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess)
        return hip_fail(e, "kda_chunk_prefill fork");
      if ((e = kda::launch_chunk(t, bf, D, false, nc2, (int)(BH * G1 * t.vsplit), ss->s)) != hipSuccess)
        return hip_fail(e, "kda_chunk_prefill segment pass");
      st = launch_segment_prefill(q, k, v, log_alpha, beta, S0, o, S1, BH, T, 0, T0, T0, D, bf, stream,
                                  "kda_chunk_prefill direct part", sn, nc0);
      // join even if the launch above failed, so the side stream's work is waited for
      if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess ||
          (e = hipStreamWaitEvent(stream, ss->join, 0)) != hipSuccess)
        return hip_fail(e, "kda_chunk_prefill join");
      if (st != KDA_OK) return st;
    }
    // 2. merge, from the direct part's end state, into the start states of all G
    //    segments (the merged state after segment G-2 is the last one's start)
    if ((e = kda::launch_merge(S1, Z, M, Sst, Sst + G1 * nS, (int)BH, G1, D, stream)) != hipSuccess)
      return hip_fail(e, "kda_chunk_prefill merge");
    // 3. prefill of every segment from its start state (Tseg and T0 are multiples
    //    of the chunk length, as snapshots need)
    st = launch_segment_prefill(q, k, v, log_alpha, beta, Sst, o, S_T, BH, T, T0, T, Ts, D, bf, stream,
                                "kda_chunk_prefill segment prefill", sn);
    return st == KDA_OK ? ok() : st;
  }
  st = launch_segment_prefill(q, k, v, log_alpha, beta, S0, o, S_T, BH, T, 0, T, T > 0 ? T : 1, D, bf,
                              stream, "kda_chunk_prefill", sn);
  return st == KDA_OK ? ok() : st;
}

// Workspace of the chunked backward (bf16 inputs), per chunk-head: the start
// state and dS' (bf16 D x D each), W = V - Kh S, Delta and
// Xbar (bf16 64 x D each), all row-major with kpos-ordered positions, and the
// 10 lower 16x16 blocks of strict_lower(Kh Kb^T) (bf16, lane order); then the
// forward pass's end state, which is not needed (fp32 [BH, D, D]).  W, Xbar
// and the blocks are written (and read) only in the rows of tokens with beta
// below kTinyBeta.  In floats.
constexpr long long kAckElems = 10 * 256;  // bf16 elements of the blocks of one chunk
size_t chunk_bw_ws_floats(long long BH, int T, int D) {
  const long long nch = (T + 63) / 64;
  return (size_t)(BH * nch * ((2 * D + 3 * 64) * D + kAckElems) / 2 + BH * D * D);
}

// Gradients of the prefill in the chunked form (bf16 inputs; arguments already
// validated):
//  1. beside each other: the forward pass from S0, which keeps the start state
//     and Delta of every chunk (its outputs are not written), on the side
//     stream; and the reverse chain from dS_T over the chunks, last to first,
//     which keeps dS' of every chunk and writes dv and dS0 (it
//     needs no forward state).  For the rows with beta below kTinyBeta only,
//     they also keep W = V - Kh S, the row of strict_lower(Kh Kb^T) and Xbar;
//  2. the per-chunk gradients, two workgroups (column halves) per (head, chunk).
// With the overlap (option bw_overlap 1, from kBwOverlapChunks chunks per
// head) the reverse chain runs as two launches, the later half of the chunks
// and then the earlier half (dS at the halves' boundary carried in dS0, which
// each workgroup reads before it writes), and the later half's gradients run
// on the side stream as soon as the forward pass and that half of the reverse
// chain are done: on the CUs the forward pass leaves, beside the earlier half
// of the reverse chain.  The earlier half's gradients follow it on the
// caller's stream.  It is off by default: the gradients running beside the
// earlier half slow that half, which is the critical path, about as much as
// the idle CUs gain.
constexpr long long kBwOverlapChunks = 16;
kda_status chunk_backward(const void* q, const void* k, const void* v, const void* log_alpha, const void* beta,
                          const float* S0, const void* dO, const float* dS_T, void* dq, void* dk_, void* dv_,
                          void* dlog_alpha, void* dbeta, float* dS0, int B, int H, int T, int D, float* ws,
                          hipStream_t stream) {
  const long long BH = (long long)B * H;
  const long long nch = (T + 63) / 64;
  const size_t nS = (size_t)BH * nch * D * D, nC = (size_t)BH * nch * 64 * D;  // elements per array
  kda::bf16* S_rows = reinterpret_cast<kda::bf16*>(ws);
  kda::bf16* dSp_rows = S_rows + nS;
  kda::bf16* W = dSp_rows + nS;
  kda::bf16* Dl = W + nC;
  kda::bf16* Xb = Dl + nC;
  kda::bf16* Ack = Xb + nC;
  float* ST = reinterpret_cast<float*>(Ack + (size_t)BH * nch * kAckElems);  // [BH, D, D], discarded
  const int nt = D / 16;
  kda::ChunkArgs r;
  r.q = q; r.k = k; r.v = dO; r.la = log_alpha; r.beta = beta;
  r.S0 = dS_T; r.o = dv_; r.S_out = dS0; r.M_out = nullptr;
  r.BH = (int)BH; r.G = 1; r.Tseg = T > 0 ? T : 1; r.Ttot = T; r.t0 = 0; r.Tend = T;
  r.dSp_rows = dSp_rows;
  r.ck_xb = Xb;
  if (g_stamp_target.load(std::memory_order_relaxed) == 2) {
    r.stamps = g_stamps.load(std::memory_order_relaxed);
    r.stamps_n = g_stamps_n.load(std::memory_order_relaxed);
  }
  // The forward pass and the reverse chain run side by side: their column
  // split is chosen so that both together fill the chip once.
  const int ncb = pick_nc(2 * BH, nt, true);
  r.vsplit = nt / (ncb * kda::chunk_tiles_per_wave(true));
  if (BH * r.vsplit > INT32_MAX) return fail(KDA_ERR_SHAPE, "problem too large");
  const bool overlap = opt(OPT_BW_OVERLAP) == 1 && nch >= kBwOverlapChunks;
  const int c1 = overlap ? (int)(nch / 2) : 0;  // first chunk of the later half
  if (log_on())
    fprintf(stderr, "[libkda] backward BH=%lld T=%d D=%d: reverse chain nc=%d vsplit=%d, %lld x %lld chunk gradients%s\n",
            BH, T, D, ncb, r.vsplit, BH, nch, overlap ? ", the later half's beside the earlier half's chain" : "");
  hipError_t e;
  if (T == 0) {  // dS0 = dS_T
    if ((e = kda::launch_chunk_bwd(r, D, ncb, (int)(BH * r.vsplit), stream)) != hipSuccess)
      return hip_fail(e, "kda_prefill_backward reverse chain");
    return ok();
  }
  kda::BwGradArgs g;
  g.q = q; g.k = k; g.la = log_alpha; g.beta = beta; g.dO = dO;
  g.dv = static_cast<const kda::bf16*>(dv_);
  g.S_rows = S_rows; g.W = W; g.Dl = Dl; g.A = Ack; g.dSp_rows = dSp_rows; g.Xb = Xb;
  g.dq = static_cast<kda::bf16*>(dq); g.dk = static_cast<kda::bf16*>(dk_);
  g.dla = static_cast<kda::bf16*>(dlog_alpha); g.dbeta = static_cast<kda::bf16*>(dbeta); g.T = T;
  SideStream* ss = nullptr;
  kda_status st;
  if ((st = side_stream(stream, &ss)) != KDA_OK) return st;
  std::lock_guard<std::mutex> lk(ss->mu);
  if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess || (e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess)
    return hip_fail(e, "kda_prefill_backward fork");
  st = launch_segment_prefill(q, k, v, log_alpha, beta, S0, nullptr, ST, BH, T, 0, T, T, D, true, ss->s,
                              "kda_prefill_backward forward checkpoints", Snap(), ncb, S_rows, W, Dl, Ack);
  if (!overlap) {
    if (st == KDA_OK && (e = kda::launch_chunk_bwd(r, D, ncb, (int)(BH * r.vsplit), stream)) != hipSuccess)
      st = hip_fail(e, "kda_prefill_backward reverse chain");
    // join even if a launch above failed, so the side stream's work is waited for
    if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess || (e = hipStreamWaitEvent(stream, ss->join, 0)) != hipSuccess)
      return hip_fail(e, "kda_prefill_backward join");
    if (st != KDA_OK) return st;
    if ((e = kda::launch_bwgrad(g, (int)BH, D, stream)) != hipSuccess)
      return hip_fail(e, "kda_prefill_backward gradients");
    return ok();
  }
  // the reverse chain's later half (the tokens from 64 c1 on), from dS_T into
  // dS0, then its earlier half, from dS0 into dS0
  kda::ChunkArgs rh = r, rl = r;
  rh.t0 = 64 * c1; rh.Tseg = T - rh.t0;
  rl.S0 = dS0; rl.Tseg = 64 * c1; rl.Tend = 64 * c1;
  kda::BwGradArgs gh = g, gl = g;
  gh.n0 = c1; gh.n1 = (int)nch;
  gl.n0 = 0; gl.n1 = c1;
  if (st == KDA_OK && (e = hipEventRecord(ss->mid, ss->s)) != hipSuccess) st = hip_fail(e, "kda_prefill_backward event");
  if (st == KDA_OK && (e = kda::launch_chunk_bwd(rh, D, ncb, (int)(BH * r.vsplit), stream)) != hipSuccess)
    st = hip_fail(e, "kda_prefill_backward reverse chain");
  if (st == KDA_OK && (e = hipEventRecord(ss->mid2, stream)) != hipSuccess) st = hip_fail(e, "kda_prefill_backward event");
  if (st == KDA_OK && (e = kda::launch_chunk_bwd(rl, D, ncb, (int)(BH * r.vsplit), stream)) != hipSuccess)
    st = hip_fail(e, "kda_prefill_backward reverse chain");
  // side stream, after the forward pass: the later half's gradients once that
  // half of the reverse chain is done
  if (st == KDA_OK && (e = hipStreamWaitEvent(ss->s, ss->mid2, 0)) != hipSuccess) st = hip_fail(e, "kda_prefill_backward wait");
  if (st == KDA_OK && (e = kda::launch_bwgrad(gh, (int)BH, D, ss->s)) != hipSuccess)
    st = hip_fail(e, "kda_prefill_backward gradients");
  // caller's stream, after the earlier half of the chain: that half's
  // gradients once the forward pass is done
  if (st == KDA_OK && (e = hipStreamWaitEvent(stream, ss->mid, 0)) != hipSuccess) st = hip_fail(e, "kda_prefill_backward wait");
  if (st == KDA_OK && (e = kda::launch_bwgrad(gl, (int)BH, D, stream)) != hipSuccess)
    st = hip_fail(e, "kda_prefill_backward gradients");
  // join even if a launch above failed, so the side stream's work is waited for
  if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess || (e = hipStreamWaitEvent(stream, ss->join, 0)) != hipSuccess)
    return hip_fail(e, "kda_prefill_backward join");
  return st == KDA_OK ? ok() : st;
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill_snap(const void* q, const void* k, const void* v, const void* log_alpha,
                                  const void* beta, const float* S0, void* o, float* S_T,
                                  float* S_snap, int snap_interval, int B, int H, int T, int dk,
                                  int dv, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return prefill_impl(q, k, v, log_alpha, beta, S0, o, S_T, S_snap, snap_interval, B, H, T, dk, dv, dtype,
                      workspace, workspace_bytes, false, stream);
}

kda_status kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                                     const void* beta, const float* S0, void* o, float* S_T, int B, int H,
                                     int T, int dk, int dv, kda_dtype dtype, hipStream_t stream) {
  return prefill_impl(q, k, v, log_alpha, beta, S0, o, S_T, nullptr, 0, B, H, T, dk, dv, dtype, nullptr, 0,
                      true, stream);
}

kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* beta, const float* S0, void* o, float* S_T, int B, int H,
                             int T, int dk, int dv, kda_dtype dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return kda_chunk_prefill_snap(q, k, v, log_alpha, beta, S0, o, S_T, nullptr, 0, B, H, T, dk, dv,
                                dtype, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_prefill_segments(const void* q, const void* k, const void* v,
                                      const void* log_alpha, const void* beta, const float* S_start,
                                      void* o, float* S_T, int B, int H, int T, int Tseg, int dk,
                                      int dv, kda_dtype dtype, hipStream_t stream) {
  if (Tseg < 1) return fail(KDA_ERR_SHAPE, "Tseg must be >= 1 (got %d)", Tseg);
  kda_status st = check_prefill_args(q, k, v, log_alpha, beta, o, S_T, B, H, T, dk, dv, dtype);
  if (st != KDA_OK) return st;
  const long long BH = (long long)B * H;
  if (BH == 0) return ok();
  KDA_OPTIONAL(S_start, "S_start");
  if (T == 0) return fail(KDA_ERR_SHAPE, "T must be >= 1 for a segmented prefill");
  if ((st = check_gates(log_alpha, BH * T * dk, beta, BH * T, dtype, stream)) != KDA_OK) return st;
  st = launch_segment_prefill(q, k, v, log_alpha, beta, S_start, o, S_T, BH, T, 0, T, Tseg, dk,
                              dtype == KDA_BF16, stream, "kda_chunk_prefill_segments");
  return st == KDA_OK ? ok() : st;
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* beta, float* S, void* o, int N, int H, int dk, int dv,
                           kda_dtype dtype, hipStream_t stream) {
  if (N < 0 || H < 0) return fail(KDA_ERR_SHAPE, "negative size N=%d H=%d", N, H);
  kda_status st;
  if ((st = check_dtype(dtype)) != KDA_OK) return st;
  if ((st = check_dims(dk, dv)) != KDA_OK) return st;
  const long long NH = (long long)N * H;
  if (NH > INT32_MAX) return fail(KDA_ERR_SHAPE, "problem too large");
  if (NH == 0) return ok();
  KDA_REQUIRE(q, "q");
  KDA_REQUIRE(k, "k");
  KDA_REQUIRE(v, "v");
  KDA_REQUIRE(log_alpha, "log_alpha");
  if (!beta) return fail(KDA_ERR_NULL, "beta is NULL");  // [N,H] rows: any element alignment
  KDA_REQUIRE(S, "S");
  KDA_REQUIRE(o, "o");
  if ((st = check_gates(log_alpha, NH * dk, beta, NH, dtype, stream)) != KDA_OK) return st;
  hipError_t e = kda::launch_decode(q, k, v, log_alpha, beta, S, S, o, nullptr, (int)NH, H, 1, dk,
                                    dtype == KDA_BF16, stream);
  if (e != hipSuccess) return hip_fail(e, "kda_decode_step launch");
  return ok();
}

kda_status kda_decode_tokens(const void* q, const void* k, const void* v, const void* log_alpha,
                             const void* beta, const float* S_in, float* S_out, void* o, float* S_pos,
                             int N, int H, int ntok, int dk, int dv, kda_dtype dtype, hipStream_t stream) {
  if (N < 0 || H < 0 || ntok < 0) return fail(KDA_ERR_SHAPE, "negative size N=%d H=%d ntok=%d", N, H, ntok);
  kda_status st;
  if ((st = check_dtype(dtype)) != KDA_OK) return st;
  if ((st = check_dims(dk, dv)) != KDA_OK) return st;
  const long long NH = (long long)N * H;
  if (NH > INT32_MAX || NH * ntok * dk > kMaxElems) return fail(KDA_ERR_SHAPE, "problem too large");
  if (NH == 0) return ok();
  KDA_REQUIRE(S_in, "S_in");
  KDA_REQUIRE(S_out, "S_out");
  KDA_OPTIONAL(S_pos, "S_pos");
  if (ntok > 0) {
    KDA_REQUIRE(q, "q");
    KDA_REQUIRE(k, "k");
    KDA_REQUIRE(v, "v");
    KDA_REQUIRE(log_alpha, "log_alpha");
    if (!beta) return fail(KDA_ERR_NULL, "beta is NULL");  // [N,H,ntok] rows: any element alignment
    KDA_REQUIRE(o, "o");
    if ((st = check_gates(log_alpha, NH * ntok * dk, beta, NH * ntok, dtype, stream)) != KDA_OK) return st;
  }
  hipError_t e = kda::launch_decode(q, k, v, log_alpha, beta, S_in, S_out, o, ntok > 0 ? S_pos : nullptr,
                                    (int)NH, H, ntok, dk, dtype == KDA_BF16, stream);
  if (e != hipSuccess) return hip_fail(e, "kda_decode_tokens launch");
  return ok();
}

kda_status kda_segment_transfer(const void* k, const void* v, const void* log_alpha,
                                const void* beta, float* S_zero_end, float* M, int B, int H, int G,
                                int Tseg, int dk, int dv, kda_dtype dtype, hipStream_t stream) {
  if (B < 0 || H < 0 || G < 0) return fail(KDA_ERR_SHAPE, "negative size B=%d H=%d G=%d", B, H, G);
  if (Tseg < 1) return fail(KDA_ERR_SHAPE, "Tseg must be >= 1 (got %d)", Tseg);
  if ((long long)G * Tseg > INT32_MAX) return fail(KDA_ERR_SHAPE, "G * Tseg exceeds 2^31 tokens");
  kda_status st;
  if ((st = check_dtype(dtype)) != KDA_OK) return st;
  if ((st = check_dims(dk, dv)) != KDA_OK) return st;
  const long long BH = (long long)B * H;
  const long long nseq = BH * G;
  if (nseq * Tseg * dk > kMaxElems || nseq > (1LL << 30)) return fail(KDA_ERR_SHAPE, "problem too large");
  if ((st = check_seq_bytes(Tseg, dk, dtype)) != KDA_OK) return st;
  if (nseq == 0) return ok();
  KDA_REQUIRE(k, "k");
  KDA_REQUIRE(v, "v");
  KDA_REQUIRE(log_alpha, "log_alpha");
  KDA_REQUIRE(beta, "beta");
  KDA_REQUIRE(S_zero_end, "S_zero_end");
  KDA_REQUIRE(M, "M");
  if ((st = check_gates(log_alpha, nseq * Tseg * dk, beta, nseq * Tseg, dtype, stream)) != KDA_OK) return st;
  const int ntiles = (dv + dk) / 16;
  const int nc = pick_nc(nseq, ntiles, dtype == KDA_BF16, dk == 128);
  kda::ChunkArgs a;
  a.q = nullptr; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
  a.S0 = nullptr; a.o = nullptr; a.S_out = S_zero_end; a.M_out = M;
  a.BH = (int)BH; a.G = G; a.Tseg = Tseg; a.Ttot = G * Tseg; a.t0 = 0; a.Tend = G * Tseg;
  a.vsplit = ntiles / (nc * kda::chunk_tiles_per_wave(dtype == KDA_BF16));
  a.map_skip = map_skip_enabled();
  const long long nwg = nseq * a.vsplit;
  if (nwg > INT32_MAX) return fail(KDA_ERR_SHAPE, "problem too large");
  if (log_on())
    fprintf(stderr, "[libkda] transfer BH=%lld G=%d Tseg=%d D=%d nc=%d vsplit=%d grid=%lld\n", BH, G,
            Tseg, dk, nc, a.vsplit, nwg);
  hipError_t e = kda::launch_chunk(a, dtype == KDA_BF16, dk, false, nc, (int)nwg, stream);
  if (e != hipSuccess) return hip_fail(e, "kda_segment_transfer launch");
  return ok();
}

kda_status kda_segment_merge(const float* S_in, const float* S_zero_end, const float* M,
                             float* S_start, float* S_T, int B, int H, int G, int dk, int dv,
                             hipStream_t stream) {
  if (B < 0 || H < 0 || G < 0) return fail(KDA_ERR_SHAPE, "negative size B=%d H=%d G=%d", B, H, G);
  kda_status st;
  if ((st = check_dims(dk, dv)) != KDA_OK) return st;
  const long long BH = (long long)B * H;
  if (BH * G * dk * dk > kMaxElems || BH > (1LL << 24)) return fail(KDA_ERR_SHAPE, "problem too large");
  if (BH == 0) return ok();
  KDA_REQUIRE(S_T, "S_T");
  KDA_OPTIONAL(S_in, "S_in");
  KDA_OPTIONAL(S_start, "S_start");
  if (G > 0) {
    KDA_REQUIRE(S_zero_end, "S_zero_end");
    KDA_REQUIRE(M, "M");
  }
  hipError_t e = kda::launch_merge(S_in, S_zero_end, M, S_start, S_T, (int)BH, G, dk, stream);
  if (e != hipSuccess) return hip_fail(e, "kda_segment_merge launch");
  return ok();
}

size_t kda_backward_workspace_bytes(int B, int H, int T, int dk, int dv, kda_dtype dtype) {
  if (B <= 0 || H <= 0 || T < 0 || dk != dv || (dk != 64 && dk != 128)) return 0;
  if (dtype == KDA_BF16) return chunk_bw_ws_floats((long long)B * H, T, dk) * sizeof(float);
  if (dtype == KDA_F32)
    return kda::backward_ws_floats((long long)B * H, T, dk, bw_split((long long)B * H)) * sizeof(float);
  return 0;
}

kda_status kda_prefill_backward(const void* q, const void* k, const void* v, const void* log_alpha,
                                const void* beta, const float* S0, const void* dO, const float* dS_T,
                                void* dq, void* dk_, void* dv_, void* dlog_alpha, void* dbeta,
                                float* dS0, int B, int H, int T, int dk, int dv, kda_dtype dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || H < 0 || T < 0) return fail(KDA_ERR_SHAPE, "negative size B=%d H=%d T=%d", B, H, T);
  kda_status st;
  if ((st = check_dtype(dtype)) != KDA_OK) return st;
  if ((st = check_dims(dk, dv)) != KDA_OK) return st;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX || BH * T * dk > kMaxElems) return fail(KDA_ERR_SHAPE, "problem too large");
  if (BH == 0) return ok();
  KDA_REQUIRE(dS0, "dS0");
  KDA_OPTIONAL(S0, "S0");
  KDA_OPTIONAL(dS_T, "dS_T");
  if (T > 0) {
    KDA_REQUIRE(q, "q");
    KDA_REQUIRE(k, "k");
    KDA_REQUIRE(v, "v");
    KDA_REQUIRE(log_alpha, "log_alpha");
    if (!beta) return fail(KDA_ERR_NULL, "beta is NULL");  // [B,H,T]: any element alignment
    KDA_OPTIONAL(dO, "dO");
    KDA_REQUIRE(dq, "dq");
    KDA_REQUIRE(dk_, "dk_");
    KDA_REQUIRE(dv_, "dv_");
    KDA_REQUIRE(dlog_alpha, "dlog_alpha");
    if (!dbeta) return fail(KDA_ERR_NULL, "dbeta is NULL");
  }
  const bool bf = dtype == KDA_BF16;
  const int split = bw_split(BH);
  const size_t need = (bf ? chunk_bw_ws_floats(BH, T, dk) : kda::backward_ws_floats(BH, T, dk, split)) * sizeof(float);
  if (!workspace) return fail(KDA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(workspace)) return fail(KDA_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (T > 0 && (st = check_gates(log_alpha, BH * T * dk, beta, BH * T, dtype, stream)) != KDA_OK) return st;
  if (bf) return chunk_backward(q, k, v, log_alpha, beta, S0, dO, dS_T, dq, dk_, dv_, dlog_alpha, dbeta, dS0, B, H,
                                T, dk, static_cast<float*>(workspace), stream);
  kda::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta; a.S0 = S0; a.dO = dO; a.dS_T = dS_T;
  a.dq = static_cast<float*>(dq); a.dk = static_cast<float*>(dk_); a.dv = static_cast<float*>(dv_);
  a.dla = static_cast<float*>(dlog_alpha); a.dbeta = static_cast<float*>(dbeta); a.dS0 = dS0;
  a.ws = static_cast<float*>(workspace);
  a.T = T;
  hipError_t e = kda::launch_backward(a, (int)BH, dk, split, stream);
  if (e != hipSuccess) return hip_fail(e, "kda_prefill_backward launch");
  return ok();
}

}  // extern "C"
