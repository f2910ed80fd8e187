// rkl_api.hip -- the C ABI declared in include/rkl.h: argument checks,
// workspace layout and launch sequences.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "rkl.h"
#include "rkl_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define RKL_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(RKL_DEVICE_ERROR, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// Per-kernel device time (rkl_kernel_timing / rkl_kernel_times): while the
// calling thread has timing on, every kernel a call launches carries two
// events that the launch itself stamps with the kernel's begin and end
// (rkl::set_launch_events), so timing adds no packets to the stream.  Events
// come from a per-thread, per-device pool and go back to it once read.
struct TimedLaunch {
  const char* name;
  hipEvent_t begin, end;
  int device;
};
thread_local bool g_timing = false;
thread_local std::vector<TimedLaunch> g_timed;
thread_local std::vector<std::vector<hipEvent_t>> g_event_pool;   // [device]

static hipError_t pooled_events(hipEvent_t* a, hipEvent_t* b, int* device) {
  hipError_t e = hipGetDevice(device);
  if (e != hipSuccess) return e;
  if ((int)g_event_pool.size() <= *device) g_event_pool.resize(*device + 1);
  std::vector<hipEvent_t>& pool = g_event_pool[*device];
  hipEvent_t* out[2] = {a, b};
  for (hipEvent_t* o : out) {
    if (!pool.empty()) {
      *o = pool.back();
      pool.pop_back();
    } else if ((e = hipEventCreate(o)) != hipSuccess) {
      if (o == b) pool.push_back(*a);
      return e;
    }
  }
  return hipSuccess;
}

static void release_events(hipEvent_t a, hipEvent_t b, int device) {
  if ((int)g_event_pool.size() <= device) g_event_pool.resize(device + 1);
  g_event_pool[device].push_back(a);
  g_event_pool[device].push_back(b);
}

// A kernel launch (a launch_* call returning hipError_t) on stream `st`, timed
// when timing is on.  A launch_* call that launched nothing (an empty fill)
// records no entry.
#define RKL_LAUNCH(name, st, expr)                                                      \
  do {                                                                                  \
    hipEvent_t evb_ = nullptr, eve_ = nullptr;                                          \
    int evd_ = 0;                                                                       \
    if (g_timing) {                                                                     \
      RKL_TRY(pooled_events(&evb_, &eve_, &evd_));                                      \
      rkl::set_launch_events(evb_, eve_);                                               \
    }                                                                                   \
    const hipError_t el_ = (expr);                                                      \
    const bool launched_ = !rkl::launch_events_pending();                               \
    rkl::set_launch_events(nullptr, nullptr);                                           \
    if (g_timing) {                                                                     \
      if (launched_ && el_ == hipSuccess)                                               \
        g_timed.push_back(TimedLaunch{name, evb_, eve_, evd_});                         \
      else                                                                              \
        release_events(evb_, eve_, evd_);                                               \
    }                                                                                   \
    if (el_ != hipSuccess) return fail(RKL_DEVICE_ERROR, "%s: %s", #expr, hipGetErrorString(el_)); \
  } while (0)

constexpr int64_t kMaxDim = (int64_t)1 << 30;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Tuning knobs, read from the environment at every call (cheap next to a
// launch) so that one process can exercise several settings.  The workgroup
// orders and the tiles per backward workgroup never change a result bit, nor
// does a backward chunk width that is a whole number of dh segments (the
// default); other widths move where dh's fp32 sum is split, i.e. its
// rounding.  The workspace size depends on the width.

// The GEMM operands' per-lane DMA offsets are formed with 24-bit multiplies
// (row < 256 times the row pitch in bytes), so a pitch must stay below 2^24
// bytes: the dz chunk width and the token count of a backward call are capped
// at 2^22.
constexpr int64_t kMaxPitchElems = (int64_t)1 << 22;

// Vocabulary columns per backward chunk for N rows: as many whole
// kChunkUnit (65536) columns as keep the chunk's fp16 dz within 2 GiB, at
// least one unit (262144 columns at N <= 4096, 65536 for N > 8192).  Fewer chunks mean fewer launches and no narrow tail
// chunk; chunks on segment boundaries keep dh's bits independent of N.
// RKL_VOCAB_CHUNK overrides it (a multiple of 256; widths that are not a
// multiple of kDhSegment change where dh's sum is split, i.e. its rounding).
int64_t vocab_chunk(int64_t N) {
  if (const char* s = std::getenv("RKL_VOCAB_CHUNK")) {
    int64_t v = std::atoll(s);
    if (v < 256) v = 256;
    if (v > kMaxPitchElems) v = kMaxPitchElems;
    return round_up(v, 256);
  }
  const int64_t budget = (int64_t)1 << 31;   // bytes of fp16 dz per chunk
  int64_t units = budget / (2 * (N > 0 ? N : 1) * (int64_t)rkl::kChunkUnit);
  if (units < 1) units = 1;
  const int64_t C = units * rkl::kChunkUnit;
  return C < kMaxPitchElems ? C : kMaxPitchElems;
}

// Vocabulary tiles one backward dz workgroup sweeps (does not change
// results).  Measured at N = 4096, H = 2048, V = 151936: with both
// projections one per workgroup is fastest (the finer grain balances the
// last wave; 2 and 3 ran 1.3 and 2.7 % slower); with one projection per job
// (teacher logits, log-probability / entropy, top-k) the pipeline fill and
// the epilogue weigh twice as much per job, and two per workgroup ran
// bwd_dz_tiles 3.1 / 3.7 / 3.5 % faster than one (2790 / 2518 / 2531 us
// against 2880 / 2614 / 2622).  RKL_BWD_TILES overrides it.
int bwd_tiles_per_group(int mode) {
  if (const char* s = std::getenv("RKL_BWD_TILES")) {
    const int v = std::atoi(s);
    return v < 1 ? 1 : (v > 64 ? 64 : v);
  }
  return (mode == rkl::kModeHidden || mode == rkl::kModeHiddenTeachers) ? 1 : 2;
}

// Whether the dz kernel makes its share of the fp16 W_s copy after the
// stream, from the k-tile loaded again, rather than from the stream's own
// stage (same bits): when each workgroup runs one job (both projections) and
// converts at most one k-tile (Hs / 64 <= token tiles).  Mid-stream, the
// copy's stores hold up the next k-step's barrier.  RKL_LATE_W16=0 turns it
// off.
bool late_w16(int mode, int tiles_per_group, int64_t Hs, int64_t ntok) {
  if (const char* s = std::getenv("RKL_LATE_W16"))
    if (s[0] == '0') return false;
  return (mode == rkl::kModeHidden || mode == rkl::kModeHiddenTeachers) && tiles_per_group == 1 &&
         Hs / 64 <= ntok;   // 64-deep k-tiles
}

// Workgroup order of the fused kernels (panel_order): GS vocabulary runs x TG
// token tiles resident together.  Does not change results.  Measured at
// N = 4096, H = 2048, V = 151936: the forward is fastest with 2 x 16, the
// backward dz kernel (which also streams its dz stores) with 4 x 8.
struct Order {
  int gs, tg;
};
Order read_order(const char* env, Order dflt) {
  if (const char* s = std::getenv(env)) {
    int a = 0, b = 0;
    if (std::sscanf(s, "%d,%d", &a, &b) == 2 && a >= 1 && b >= 1 && a <= 4096 && b <= 4096) return Order{a, b};
  }
  return dflt;
}
Order fwd_order() { return read_order("RKL_FWD_ORDER", Order{2, 16}); }

Order bwd_order() { return read_order("RKL_BWD_ORDER", Order{4, 8}); }

// Column tiles per panel in the dh GEMM's workgroup order (RKL_DH_PANEL;
// does not change results).  Measured at N = 4096, H = 2048 (16 x 16 tiles,
// one workgroup per CU): panels of 8 columns, i.e. 4 row tiles x 8 column
// tiles per XCD, run dh 2.8 % faster than whole rows of 16 (2 x 16 per XCD:
// every XCD then streams all of W's columns); 4 and 2 are slower again.
int dh_panel(int ntn) {
  const char* s = std::getenv("RKL_DH_PANEL");
  const int v = s ? std::atoi(s) : 8;
  return v < 1 ? 1 : (v > ntn ? ntn : v);
}

// Forward split plan: depends on V only (so a row's result never depends on N).
struct Split {
  int tiles_per_split, nsplit;
};
Split fwd_split(int64_t V) {
  const int64_t ntv = ceil_div(V, rkl::kFwdTileV);
  int64_t tps = ceil_div(ntv, 200);   // 3 at V = 151936: 198 splits (measured fastest)
  if (const char* s = std::getenv("RKL_FWD_TILES")) {   // tiles per split (changes rounding only)
    const int v = std::atoi(s);
    if (v >= 1 && v <= 1024) tps = v;
  }
  return Split{(int)tps, (int)ceil_div(ntv, tps)};
}

// Splits per forward workgroup.  A workgroup streams its splits' vocabulary
// tiles as one pipeline, so longer runs save pipeline fills, but the fused
// kernels hold one workgroup per CU, so a ragged last wave of workgroups
// costs as long as a full one.  The choice minimises waves of kCUs
// workgroups x (tiles per workgroup + a fill of about a tenth of a tile),
// and is taken when it beats one split per workgroup by more than 1 %.
// Measured forward times at H = 2048, V = 151936 (us, the choice against
// one split per workgroup, each after warm-up in one process): N = 4096
// (8 groups of 25 splits, 256 workgroups) 4444 / 4549 on one box and
// 4296 / 4329 on another; N = 8192 (4 groups of 50) 8468 / 8564; N = 16384
// (2 groups of 99) 16839 / 17196; N = 1000 (29 groups of 7, 232
// workgroups: one ragged wave against seven) 1197 / 1240; N = 4224 (groups
// of 2) 4762 / 4734, within the noise.  With several teachers chosen per row
// (uneven), token tiles differ in work -- a tile that straddles a teacher
// boundary runs a teacher pass per teacher -- and long workgroups would
// leave the slowest tiles' workgroups running alone: one split per
// workgroup lets the CUs balance them (K = 4, N = 4096, rows in random
// order: forward 5.29 against 6.63 ms; in runs of 1024 rows, which no tile
// straddles, 4.78 against 4.60 ms).  Does not change results.
// RKL_FWD_SPLITS_PER_WG overrides it.
constexpr int64_t kCUs = 256;   // MI355X compute units
int fwd_splits_per_wg(int nsplit, int tiles_per_split, int64_t ntok, bool uneven) {
  if (const char* s = std::getenv("RKL_FWD_SPLITS_PER_WG")) {
    const int v = std::atoi(s);
    if (v >= 1) return v < nsplit ? v : nsplit;
  }
  if (uneven) return 1;
  if (ntok < 1) ntok = 1;
  auto cost = [&](int spw) {
    const int64_t waves = ceil_div(ceil_div(nsplit, spw) * ntok, kCUs);
    return (double)waves * ((double)spw * tiles_per_split + 0.1);
  };
  int best = 1;
  double best_cost = cost(1);
  for (int spw = 2; spw <= nsplit; ++spw) {
    const double c = cost(spw);
    if (c <= best_cost) {   // ties go to the longer runs
      best = spw;
      best_cost = c;
    }
  }
  return best_cost < 0.99 * cost(1) ? best : 1;
}

size_t fwd_ws_bytes(int64_t N, int64_t V, bool tiled) {
  if (!tiled) return 0;
  return align256((size_t)fwd_split(V).nsplit * 5 * (size_t)N * sizeof(float));
}

// Whether the dh GEMM runs one workgroup per (tile, vocabulary segment),
// writing segment sums that a reduce adds in order, instead of one
// workgroup per tile summing every segment: when the tiles alone would not
// fill the CUs (N below 4096 at Hs = 2048).  Same bits either way.  Measured
// at Hs = 2048, V = 151936 (ten 16384-column segments), split against one
// workgroup per tile: dh 500 against 1921 us at N = 512 (32 tiles), 737
// against 1903 at N = 1024, 1221 + 34 (the reduce) against 1888 at N = 2048.
// RKL_DH_SPLIT = 0 / 1 forces it off / on.
bool dh_split(int64_t N, int64_t Hs) {
  if (const char* s = std::getenv("RKL_DH_SPLIT")) {
    if (s[0] == '0') return false;
    if (s[0] == '1') return true;
  }
  return ceil_div(N, rkl::kDhTileM) * ceil_div(Hs, rkl::kDhTileN) < kCUs;
}

// dh segments a chunk [c0, c0 + width) overlaps (segments end at absolute
// multiples of kDhSegment).
int64_t dh_segments(int64_t c0, int64_t width) {
  return (c0 + width - 1) / rkl::kDhSegment - c0 / rkl::kDhSegment + 1;
}

struct BwdLayout {
  int64_t hrows, ldz, npad, nchunks, nseg;
  size_t off_h16, off_dz, off_w16, off_dhp, off_scale, total;
};
// [scale block: rkl::kScaleWmag + nchunks words][h16: hrows x Hs fp16][dz chunk:
// npad x ldz fp16][fp16 W_s chunk copy][dh segment sums nseg x N x Hs fp32,
// when dh is split]; npad = N rounded up to the 128-token tile (the dz
// kernel writes those rows as zero)
BwdLayout bwd_layout(int64_t N, int64_t V, int64_t Hs) {
  BwdLayout L{};
  L.hrows = round_up(N, 64);
  L.npad = round_up(N, rkl::kFwdTileN);
  const int64_t C = vocab_chunk(N);
  L.ldz = round_up(V < C ? V : C, 64);
  L.nchunks = ceil_div(V, C);
  // most segments one chunk overlaps
  L.nseg = 0;
  for (int64_t c0 = 0; c0 < V; c0 += C) {
    const int64_t n = dh_segments(c0, (V - c0) < C ? (V - c0) : C);
    if (n > L.nseg) L.nseg = n;
  }
  L.off_scale = 0;
  L.off_h16 = align256((size_t)(rkl::kScaleWmag + L.nchunks) * 4);
  L.off_dz = L.off_h16 + align256((size_t)Hs * L.hrows * 2);
  L.off_w16 = L.off_dz + align256((size_t)L.npad * L.ldz * 2);
  // the fp16 W_s copy covers every 256-row vocabulary tile of a chunk
  L.off_dhp = L.off_w16 + align256((size_t)round_up(L.ldz, rkl::kFwdTileV) * Hs * 2);
  L.total = L.off_dhp + (dh_split(N, Hs) ? align256((size_t)L.nseg * N * Hs * 4) : 0);
  return L;
}

size_t ws_bytes(int64_t N, int64_t V, int64_t Hs, int64_t Ht) {
  (void)Ht;
  if (Hs == 0) return 0;   // both sides as logits: row kernels need no workspace
  const size_t f = fwd_ws_bytes(N, V, true);
  const size_t b = bwd_layout(N, V, Hs).total;
  return f > b ? f : b;
}

// Per-row teachers: the rows are first grouped by teacher id (a stable
// sort) so that a 128-row tile mixes teachers only at group boundaries; the
// fused kernels then run one teacher pass per tile instead of one per teacher
// present.  The grouped copies live in front of the regular workspace:
// [perm][teacher ids][mask bytes][h_s rows][h_t rows][loss or grad][stats][dh].
struct GroupLayout {
  size_t off_perm, off_tid, off_mask, off_hs, off_ht, off_row, off_stats, off_dh, total;
};
GroupLayout group_layout(int64_t N, int64_t Hs, int64_t Ht) {
  GroupLayout G{};
  size_t o = 0;
  G.off_perm = o;  o += align256((size_t)N * 4);
  G.off_tid = o;   o += align256((size_t)N * 4);
  G.off_mask = o;  o += align256((size_t)N);
  G.off_hs = o;    o += align256((size_t)N * Hs * 2);
  G.off_ht = o;    o += align256((size_t)N * Ht * 2);
  G.off_row = o;   o += align256((size_t)N * 4);
  G.off_stats = o; o += align256((size_t)N * 16);
  G.off_dh = o;    o += align256((size_t)N * Hs * 4);
  G.total = o;
  return G;
}

int check_dims(int64_t N, int64_t V, int64_t Hs, int64_t Ht, bool teacher_hidden, bool student_hidden) {
  if (N < 0 || N > kMaxDim) return fail(RKL_INVALID_ARG, "N=%lld out of range [0, 2^30]", (long long)N);
  if (V < 1 || V > kMaxDim) return fail(RKL_INVALID_ARG, "V=%lld out of range [1, 2^30]", (long long)V);
  if (student_hidden) {
    if (Hs <= 0 || Hs > 65536) return fail(RKL_INVALID_ARG, "Hs=%lld out of range", (long long)Hs);
    if (Hs % 64) return fail(RKL_UNSUPPORTED, "Hs=%lld is not a multiple of 64", (long long)Hs);
  } else if (Hs != 0) {
    return fail(RKL_INVALID_ARG, "Hs must be 0 when the student is given as logits");
  }
  if (teacher_hidden) {
    if (Ht <= 0 || Ht > 65536) return fail(RKL_INVALID_ARG, "Ht=%lld out of range", (long long)Ht);
    if (Ht % 64) return fail(RKL_UNSUPPORTED, "Ht=%lld is not a multiple of 64", (long long)Ht);
  }
  if (N * V > ((int64_t)1 << 40)) return fail(RKL_INVALID_ARG, "N*V too large");
  return RKL_OK;
}

#define NEED16(p, name)                                                                              \
  do {                                                                                               \
    if (!(p)) return fail(RKL_INVALID_ARG, "%s is NULL", name);                                      \
    if (!aligned16(p)) return fail(RKL_INVALID_ARG, "%s is not 16-byte aligned", name);             \
  } while (0)
#define NEED4(p, name)                                                                               \
  do {                                                                                               \
    if (!(p)) return fail(RKL_INVALID_ARG, "%s is NULL", name);                                      \
    if (!aligned4(p)) return fail(RKL_INVALID_ARG, "%s is not 4-byte aligned", name);               \
  } while (0)
#define OPT4(p, name)                                                                                \
  do {                                                                                               \
    if ((p) && !aligned4(p)) return fail(RKL_INVALID_ARG, "%s is not 4-byte aligned", name);        \
  } while (0)

// ---------------------------------------------------------------------------
// forward / backward bodies shared by the hidden and logits entry points
// ---------------------------------------------------------------------------
// mode: y != NULL -> log-probability / entropy (out0 = log p(y), out1 =
// entropy); else reverse KL (out0 = loss) with the teacher as hidden states
// (z_t NULL) or as logits.
int mode_of(const float* z_t, const int32_t* y, const int32_t* teacher) {
  if (y) return rkl::kModeLogprobEntropy;
  if (z_t) return rkl::kModeTeacherLogits;
  return teacher ? rkl::kModeHiddenTeachers : rkl::kModeHidden;
}

// Per-row teachers: K weights of [V, Ht] each, back to back.
struct Teachers {
  const int32_t* teacher = nullptr;   // NULL: one teacher
  int K = 1;
  int64_t stride = 0;
};

// Rows of the given logits (rkl_forward_logits / rkl_backward_logits): token
// n reads row rows[n] of buffers that hold nrows rows; rows NULL: row n.
struct ZRows {
  const int32_t* rows = nullptr;
  int64_t nrows = 0;
};

int forward_tiled(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s, const rkl_bf16* W_s,
                  const rkl_bf16* h_t, const rkl_bf16* W_t, const float* z_t, const int32_t* y,
                  const uint8_t* row_mask, float* out0, float* out1, float* stats, void* ws, size_t ws_bytes_given,
                  hipStream_t s, Teachers tch = Teachers{}, float* merged = nullptr, ZRows zr = ZRows{}) {
  const size_t need = fwd_ws_bytes(N, V, true);
  if (ws_bytes_given < need)
    return fail(RKL_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes_given, need);
  if (N == 0) return RKL_OK;
  NEED16(ws, "workspace");
  const Split sp = fwd_split(V);
  rkl::FwdParams p{};
  p.N = (int)N; p.V = (int)V; p.Hs = (int)Hs; p.Ht = (int)Ht;
  p.h_s = h_s; p.W_s = W_s; p.h_t = h_t; p.W_t = W_t; p.z_t = z_t; p.y = y;
  p.z_rows = zr.rows; p.z_nrows = (int)(zr.rows ? zr.nrows : N);
  p.teacher = tch.teacher; p.K = tch.K; p.wt_stride = tch.stride;
  p.partial = static_cast<float*>(ws);
  p.tiles_per_split = sp.tiles_per_split;
  p.nsplit = sp.nsplit;
  p.ntok = (int)ceil_div(N, rkl::kFwdTileN);
  p.splits_per_wg = fwd_splits_per_wg(p.nsplit, p.tiles_per_split, p.ntok, tch.teacher && tch.K > 1);
  p.order_gs = fwd_order().gs;
  p.order_tg = fwd_order().tg;
  const int mode = mode_of(z_t, y, tch.teacher);
  RKL_LAUNCH("fwd_tiles", s, rkl::launch_fwd_tiles(p, mode, s));
  if (merged) {   // one vocabulary shard: its merged statistics, not finalised
    RKL_LAUNCH("fwd_combine", s, rkl::launch_fwd_merge(p.partial, p.nsplit, p.N, merged, s));
    return RKL_OK;
  }
  RKL_LAUNCH("fwd_combine", s, rkl::launch_fwd_combine(p.partial, p.nsplit, p.N, row_mask, mode == rkl::kModeLogprobEntropy, out0, out1,
                                  stats, s));
  return RKL_OK;
}

// Top-k estimator: the support of every row and the teacher's
// log-probabilities on it (rkl_*_topk).
struct TopK {
  bool on = false;
  int K = 0;
  const int32_t* S = nullptr;
  const float* lpt_S = nullptr;
  const float* lps = nullptr;   // the student's log-probabilities on S from the forward (NULL: recomputed)
};

int backward_tiled(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s, const rkl_bf16* W_s,
                   const rkl_bf16* h_t, const rkl_bf16* W_t, const float* z_t, const int32_t* y,
                   const uint8_t* row_mask, const float* grad, const float* grad_h, const float* stats, float* dh,
                   float* dW, int accumulate, void* ws, size_t ws_bytes_given, hipStream_t s,
                   Teachers tch = Teachers{}, TopK topk = TopK{}, ZRows zr = ZRows{}) {
  const int mode = topk.on ? rkl::kModeTopK : mode_of(z_t, y, tch.teacher);
  if (N > kMaxPitchElems)
    return fail(RKL_UNSUPPORTED, "N=%lld rows exceed the backward's limit of 2^22 per call", (long long)N);
  const BwdLayout L = bwd_layout(N, V, Hs);
  if (ws_bytes_given < L.total)
    return fail(RKL_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes_given, L.total);
  if (N == 0) {
    // an empty selection still produces a (zero) dW unless the caller accumulates
    if (!accumulate) RKL_LAUNCH("fill_zero", s, rkl::launch_fill_zero(dW, V * Hs * (int64_t)sizeof(float), s));
    return RKL_OK;
  }
  NEED16(ws, "workspace");
  char* base = static_cast<char*>(ws);
  uint32_t* scales = reinterpret_cast<uint32_t*>(base + L.off_scale);
  uint16_t* h16 = reinterpret_cast<uint16_t*>(base + L.off_h16);
  uint16_t* dz = reinterpret_cast<uint16_t*>(base + L.off_dz);
  uint16_t* w16 = reinterpret_cast<uint16_t*>(base + L.off_w16);
  RKL_LAUNCH("grad_scale", s, rkl::launch_grad_scale(grad, grad_h, row_mask, stats, (int)N, mode,
                                 (int)L.nchunks, scales, s));
  RKL_LAUNCH("absmax_bf16", s, rkl::launch_absmax_bf16(h_s, N * Hs, scales, s));
  RKL_LAUNCH("convert_h", s, rkl::launch_convert_h(h_s, (int)N, (int)Hs, scales, h16, (int)L.hrows, s));
  const int64_t C = vocab_chunk(N);
  for (int64_t c0 = 0, chunk = 0; c0 < V; c0 += C, ++chunk) {
    uint32_t* wmag = scales + rkl::kScaleWmag + chunk;
    const int64_t width = (V - c0) < C ? (V - c0) : C;
    const int64_t kpad = round_up(width, 64);
    rkl::BwdParams b{};
    b.N = (int)N; b.V = (int)V; b.Hs = (int)Hs; b.Ht = (int)Ht;
    b.h_s = h_s; b.W_s = W_s; b.h_t = h_t; b.W_t = W_t; b.z_t = z_t;
    b.z_rows = zr.rows; b.z_nrows = (int)(zr.rows ? zr.nrows : N);
    b.row_mask = row_mask; b.grad = grad; b.grad_h = grad_h; b.y = y; b.stats = stats;
    b.teacher = tch.teacher; b.K = tch.K; b.wt_stride = tch.stride;
    b.scales = scales; b.wmag = wmag; b.dz = dz; b.w16 = w16; b.ldz = (int)L.ldz; b.c0 = (int)c0;
    b.kpad = (int)kpad;
    b.ntv = (int)ceil_div(kpad, rkl::kFwdTileV);
    b.tiles_per_group = bwd_tiles_per_group(mode);
    b.ngroups = (int)ceil_div(b.ntv, b.tiles_per_group);
    b.ntok = (int)ceil_div(N, rkl::kFwdTileN);
    b.order_gs = bwd_order().gs;
    b.order_tg = bwd_order().tg;
    b.late_w16 = late_w16(mode, b.tiles_per_group, Hs, b.ntok) ? 1 : 0;
    RKL_LAUNCH("bwd_dz_tiles", s, rkl::launch_bwd_dz(b, mode, s));
    if (topk.on && topk.K > 0)
      RKL_LAUNCH("topk_dz_add", s, rkl::launch_topk_dz_add(h_s, W_s, (int)N, (int)V, (int)Hs, topk.K, topk.S,
                                                          topk.lpt_S, topk.lps, row_mask, grad, stats, scales, dz,
                                                          (int)L.ldz,
                                                          (int)c0, (int)width, s));
    RKL_LAUNCH("w_rescale", s, rkl::launch_w_rescale(W_s + c0 * Hs, (int)width, b.ntv, (int)Hs, wmag, w16, s));

    rkl::DwParams w{};
    w.scales = scales; w.dz = dz; w.ldz = (int)L.ldz; w.N = (int)N; w.kpad = (int)kpad; w.width = (int)width;
    w.h16 = h16; w.hrows = (int)L.hrows; w.H = (int)Hs;
    w.dW = dW + c0 * Hs; w.accumulate = accumulate;
    w.ntm = (int)ceil_div(width, rkl::kDwTileM);
    w.ntn = (int)ceil_div(Hs, rkl::kDwTileN);
    RKL_LAUNCH("dw_gemm", s, rkl::launch_dw(w, s));

    rkl::DhParams h{};
    h.scales = scales; h.wmag = wmag; h.dz = dz; h.ldz = (int)L.ldz; h.N = (int)N; h.npad = (int)L.npad; h.kpad = (int)kpad;
    h.width = (int)width; h.c0 = (int)c0;
    h.w16 = w16; h.H = (int)Hs; h.dh = dh; h.accumulate = c0 > 0;
    h.ntm = (int)ceil_div(N, rkl::kDhTileM);
    h.ntn = (int)ceil_div(Hs, rkl::kDhTileN);
    h.panel = dh_panel(h.ntn);
    h.nseg = (int)dh_segments(c0, kpad);
    h.partial = dh_split(N, Hs) ? reinterpret_cast<float*>(base + L.off_dhp) : nullptr;
    RKL_LAUNCH("dh_gemm", s, rkl::launch_dh(h, s));
    if (h.partial) RKL_LAUNCH("dh_reduce", s, rkl::launch_dh_reduce(h, s));
  }
  return RKL_OK;
}

// Merge of G vocabulary shards' partials (rkl_combine_shards*).
int combine_shards(int64_t G, int64_t N, const float* partials, const uint8_t* row_mask, bool lpe, float* out0,
                   float* out1, float* stats, hipStream_t s) {
  if (G < 1 || G > ((int64_t)1 << 20)) return fail(RKL_INVALID_ARG, "G=%lld shards out of range [1, 2^20]", (long long)G);
  if (N < 0 || N > kMaxDim) return fail(RKL_INVALID_ARG, "N=%lld out of range [0, 2^30]", (long long)N);
  if (G * 5 * N > ((int64_t)1 << 40)) return fail(RKL_INVALID_ARG, "G*N too large");
  if (N == 0) return RKL_OK;
  NEED4(partials, "partials"); NEED4(stats, "stats");
  if (lpe) { NEED4(out0, "logp"); NEED4(out1, "entropy"); }
  else NEED4(out0, "loss");
  RKL_LAUNCH("fwd_combine", s, rkl::launch_fwd_combine(partials, (int)G, (int)N, row_mask, lpe, out0, out1, stats, s));
  return RKL_OK;
}

}  // namespace

int rkl::set_last_error(int code, const char* msg) {
  g_err = msg;
  return code;
}

// The library is built with hidden visibility; only the C ABI is exported.
#pragma GCC visibility push(default)
extern "C" {

const char* rkl_last_error(void) { return g_err.c_str(); }

const char* rkl_version(void) { return "rkl 0.1 gfx950"; }

int rkl_kernel_timing(int enable) {
  g_timing = enable != 0;
  return RKL_OK;
}

int rkl_kernel_times(int cap, const char** names, double* total_ms, int* launches, int* count) {
  if (cap < 0 || (cap > 0 && (!names || !total_ms || !launches)) || !count)
    return fail(RKL_INVALID_ARG, "need cap >= 0, arrays of cap entries and a count");
  std::vector<TimedLaunch> recs;
  recs.swap(g_timed);
  int n = 0;
  int rc = RKL_OK;
  for (const TimedLaunch& r : recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.end);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.begin, r.end);
    release_events(r.begin, r.end, r.device);
    if (e != hipSuccess) {
      rc = fail(RKL_DEVICE_ERROR, "kernel timing event: %s", hipGetErrorString(e));
      continue;
    }
    int k = 0;
    while (k < n && k < cap && std::strcmp(names[k], r.name) != 0) ++k;
    if (k == n) {
      if (n < cap) {
        names[n] = r.name;
        total_ms[n] = 0.0;
        launches[n] = 0;
      }
      ++n;
    }
    if (k < cap) {
      total_ms[k] += ms;
      launches[k] += 1;
    }
  }
  *count = n;
  return rc;
}

size_t rkl_workspace_bytes(int64_t N, int64_t V, int64_t Hs, int64_t Ht) {
  if (N < 0 || N > kMaxDim || V < 1 || V > kMaxDim || Hs < 0 || Ht < 0) return 0;
  return ws_bytes(N, V, Hs, Ht);
}

size_t rkl_workspace_bytes_teachers(int64_t N, int64_t V, int64_t Hs, int64_t Ht) {
  if (N < 0 || N > kMaxDim || V < 1 || V > kMaxDim || Hs < 0 || Ht < 0) return 0;
  return group_layout(N, Hs, Ht).total + ws_bytes(N, V, Hs, Ht);
}

int rkl_compact_rows(const uint8_t* mask, int64_t T, int32_t* row_idx, int32_t* n_rows_dev, int64_t* n_rows_host,
                     rkl_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T < 0 || T >= ((int64_t)1 << 31)) return fail(RKL_INVALID_ARG, "T=%lld out of range", (long long)T);
  NEED4(n_rows_dev, "n_rows_dev");
  if (T > 0) {
    if (!mask) return fail(RKL_INVALID_ARG, "mask is NULL");
    NEED4(row_idx, "row_idx");
  }
  RKL_LAUNCH("compact", s, rkl::launch_compact(mask, (int)T, row_idx, n_rows_dev, s));
  if (n_rows_host) {
    int32_t n = 0;
    RKL_TRY(hipMemcpyAsync(&n, n_rows_dev, sizeof(n), hipMemcpyDeviceToHost, s));
    RKL_TRY(hipStreamSynchronize(s));
    *n_rows_host = n;
  }
  return RKL_OK;
}

int rkl_gather_rows(const void* src, int64_t T, int64_t row_bytes, const int32_t* row_idx, int64_t N, void* dst,
                    rkl_stream_t stream) {
  if (T < 0 || N < 0 || N > T) return fail(RKL_INVALID_ARG, "need 0 <= N <= T (N=%lld, T=%lld)", (long long)N, (long long)T);
  if (N >= ((int64_t)1 << 31)) return fail(RKL_INVALID_ARG, "N too large");
  if (row_bytes <= 0 || row_bytes % 4) return fail(RKL_INVALID_ARG, "row_bytes=%lld must be a positive multiple of 4", (long long)row_bytes);
  if (N == 0) return RKL_OK;
  if (!src || !dst || !row_idx) return fail(RKL_INVALID_ARG, "NULL pointer");
  const bool need16 = row_bytes % 16 == 0;
  if (need16 ? !(aligned16(src) && aligned16(dst)) : !(aligned4(src) && aligned4(dst)))
    return fail(RKL_INVALID_ARG, "src/dst misaligned");
  RKL_LAUNCH("gather", static_cast<hipStream_t>(stream), rkl::launch_gather(src, row_bytes, row_idx, N, dst, static_cast<hipStream_t>(stream)));
  return RKL_OK;
}

int rkl_scatter_rows(const void* src, int64_t N, int64_t row_bytes, const int32_t* row_idx, int64_t T, void* dst,
                     rkl_stream_t stream) {
  if (T < 0 || N < 0 || N > T) return fail(RKL_INVALID_ARG, "need 0 <= N <= T (N=%lld, T=%lld)", (long long)N, (long long)T);
  if (T >= ((int64_t)1 << 31)) return fail(RKL_INVALID_ARG, "T too large");
  if (row_bytes <= 0 || row_bytes % 4) return fail(RKL_INVALID_ARG, "row_bytes=%lld must be a positive multiple of 4", (long long)row_bytes);
  if (T == 0) return RKL_OK;
  if (!dst || (N > 0 && (!src || !row_idx))) return fail(RKL_INVALID_ARG, "NULL pointer");
  const bool need16 = row_bytes % 16 == 0;
  if (need16 ? !(aligned16(dst) && (N == 0 || aligned16(src))) : !(aligned4(dst) && (N == 0 || aligned4(src))))
    return fail(RKL_INVALID_ARG, "src/dst misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  RKL_LAUNCH("fill_zero", s, rkl::launch_fill_zero(dst, T * row_bytes, s));
  if (N > 0) RKL_LAUNCH("scatter", s, rkl::launch_scatter(src, row_bytes, row_idx, N, dst, s));
  return RKL_OK;
}

int rkl_forward_hidden(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s, const rkl_bf16* W_s,
                       const rkl_bf16* h_t, const rkl_bf16* W_t, const uint8_t* row_mask, float* loss, float* stats,
                       void* workspace, size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, Hs, Ht, true, true)) return rc;
  if (N > 0) {
    NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); NEED16(h_t, "h_t"); NEED16(W_t, "W_t");
    NEED4(loss, "loss"); NEED4(stats, "stats");
  }
  return forward_tiled(N, V, Hs, Ht, h_s, W_s, h_t, W_t, nullptr, nullptr, row_mask, loss, nullptr, stats, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

int rkl_forward_hidden_shard(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s, const rkl_bf16* W_s,
                             const rkl_bf16* h_t, const rkl_bf16* W_t, float* partial, void* workspace,
                             size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, Hs, Ht, true, true)) return rc;
  if (N > 0) {
    NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); NEED16(h_t, "h_t"); NEED16(W_t, "W_t");
    NEED4(partial, "partial");
  }
  return forward_tiled(N, V, Hs, Ht, h_s, W_s, h_t, W_t, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                       workspace, workspace_bytes, static_cast<hipStream_t>(stream), Teachers{}, partial);
}

int rkl_forward_logits_shard(int64_t N, int64_t V, int64_t Hs, const rkl_bf16* h_s, const rkl_bf16* W_s,
                             const float* z_s, const float* z_t, float* partial, void* workspace,
                             size_t workspace_bytes, rkl_stream_t stream) {
  const bool student_hidden = h_s != nullptr || W_s != nullptr;
  if (student_hidden && z_s) return fail(RKL_INVALID_ARG, "give the student as (h_s, W_s) or as z_s, not both");
  if (int rc = check_dims(N, V, Hs, 0, false, student_hidden)) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N > 0) {
    NEED16(z_t, "z_t"); NEED4(partial, "partial");
    if (student_hidden) { NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); }
    else NEED16(z_s, "z_s");
  }
  if (student_hidden)
    return forward_tiled(N, V, Hs, 0, h_s, W_s, nullptr, nullptr, z_t, nullptr, nullptr, nullptr, nullptr, nullptr,
                         workspace, workspace_bytes, s, Teachers{}, partial);
  if (N == 0) return RKL_OK;
  RKL_LAUNCH("fwd_rows_logits", s, rkl::launch_fwd_rows_logits(z_s, z_t, nullptr, (int)N, (int)N, (int)V, nullptr, nullptr, nullptr, partial, s));
  return RKL_OK;
}

int rkl_combine_shards(int64_t G, int64_t N, const float* partials, const uint8_t* row_mask, float* loss,
                       float* stats, rkl_stream_t stream) {
  return combine_shards(G, N, partials, row_mask, false, loss, nullptr, stats, static_cast<hipStream_t>(stream));
}

int rkl_forward_logprob_entropy_shard(int64_t N, int64_t V, int64_t H, const rkl_bf16* h, const rkl_bf16* W,
                                      const int32_t* y, float* partial, void* workspace, size_t workspace_bytes,
                                      rkl_stream_t stream) {
  if (int rc = check_dims(N, V, H, 0, false, true)) return rc;
  if (N > 0) {
    NEED16(h, "h"); NEED16(W, "W"); NEED4(y, "y"); NEED4(partial, "partial");
  }
  return forward_tiled(N, V, H, 0, h, W, nullptr, nullptr, nullptr, y, nullptr, nullptr, nullptr, nullptr, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream), Teachers{}, partial);
}

int rkl_combine_shards_logprob_entropy(int64_t G, int64_t N, const float* partials, const uint8_t* row_mask,
                                       float* logp, float* entropy, float* stats, rkl_stream_t stream) {
  return combine_shards(G, N, partials, row_mask, true, logp, entropy, stats, static_cast<hipStream_t>(stream));
}

// z_rows / T of the logits entry points: the row index, and the rows the
// logits buffers hold.
static int check_z_rows(int64_t N, const int32_t* z_rows, int64_t T, ZRows& zr) {
  if (!z_rows) return RKL_OK;
  if (T < 1 || T > kMaxDim)
    return fail(RKL_INVALID_ARG, "T=%lld rows of the logits out of range [1, 2^30] with z_rows", (long long)T);
  if (N > 0) NEED4(z_rows, "z_rows");
  zr.rows = z_rows;
  zr.nrows = T;
  return RKL_OK;
}

int rkl_forward_logits(int64_t N, int64_t V, int64_t Hs, const rkl_bf16* h_s, const rkl_bf16* W_s, const float* z_s,
                       const float* z_t, const int32_t* z_rows, int64_t T, const uint8_t* row_mask, float* loss,
                       float* stats, void* workspace, size_t workspace_bytes, rkl_stream_t stream) {
  const bool student_hidden = h_s != nullptr || W_s != nullptr;
  if (student_hidden && z_s) return fail(RKL_INVALID_ARG, "give the student as (h_s, W_s) or as z_s, not both");
  if (int rc = check_dims(N, V, Hs, 0, false, student_hidden)) return rc;
  ZRows zr;
  if (int rc = check_z_rows(N, z_rows, T, zr)) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N > 0) {
    NEED16(z_t, "z_t");
    NEED4(loss, "loss"); NEED4(stats, "stats");
    if (student_hidden) { NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); }
    else NEED16(z_s, "z_s");
  }
  if (student_hidden)
    return forward_tiled(N, V, Hs, 0, h_s, W_s, nullptr, nullptr, z_t, nullptr, row_mask, loss, nullptr, stats,
                         workspace, workspace_bytes, s, Teachers{}, nullptr, zr);
  if (N == 0) return RKL_OK;
  RKL_LAUNCH("fwd_rows_logits", s, rkl::launch_fwd_rows_logits(z_s, z_t, zr.rows, (int)(zr.rows ? zr.nrows : N), (int)N,
                                                              (int)V, row_mask, loss, stats, nullptr, s));
  return RKL_OK;
}

int rkl_backward_hidden(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s, const rkl_bf16* W_s,
                        const rkl_bf16* h_t, const rkl_bf16* W_t, const uint8_t* row_mask, const float* grad_loss,
                        const float* stats, float* dh_s, float* dW_s, int accumulate_dW, void* workspace,
                        size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, Hs, Ht, true, true)) return rc;
  NEED16(dW_s, "dW_s");
  if (N > 0) {
    NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); NEED16(h_t, "h_t"); NEED16(W_t, "W_t");
    NEED4(stats, "stats"); NEED16(dh_s, "dh_s"); OPT4(grad_loss, "grad_loss");
  }
  return backward_tiled(N, V, Hs, Ht, h_s, W_s, h_t, W_t, nullptr, nullptr, row_mask, grad_loss, nullptr, stats, dh_s,
                        dW_s, accumulate_dW != 0, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int rkl_backward_logits(int64_t N, int64_t V, int64_t Hs, const rkl_bf16* h_s, const rkl_bf16* W_s, const float* z_s,
                        const float* z_t, const int32_t* z_rows, int64_t T, const uint8_t* row_mask,
                        const float* grad_loss, const float* stats, float* dh_s, float* dW_s, int accumulate_dW,
                        float* dz_s, void* workspace, size_t workspace_bytes, rkl_stream_t stream) {
  const bool student_hidden = h_s != nullptr || W_s != nullptr;
  if (student_hidden && z_s) return fail(RKL_INVALID_ARG, "give the student as (h_s, W_s) or as z_s, not both");
  if (int rc = check_dims(N, V, Hs, 0, false, student_hidden)) return rc;
  ZRows zr;
  if (int rc = check_z_rows(N, z_rows, T, zr)) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (student_hidden) {
    if (dz_s) return fail(RKL_INVALID_ARG, "dz_s must be NULL when the student is given as hidden states");
    NEED16(dW_s, "dW_s");
    if (N > 0) {
      NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); NEED16(z_t, "z_t");
      NEED4(stats, "stats"); NEED16(dh_s, "dh_s"); OPT4(grad_loss, "grad_loss");
    }
    return backward_tiled(N, V, Hs, 0, h_s, W_s, nullptr, nullptr, z_t, nullptr, row_mask, grad_loss, nullptr, stats,
                          dh_s, dW_s, accumulate_dW != 0, workspace, workspace_bytes, s, Teachers{}, TopK{}, zr);
  }
  if (dh_s || dW_s) return fail(RKL_INVALID_ARG, "dh_s and dW_s must be NULL when the student is given as logits");
  if (N == 0) return RKL_OK;
  NEED16(z_s, "z_s"); NEED16(z_t, "z_t"); NEED4(stats, "stats"); NEED16(dz_s, "dz_s"); OPT4(grad_loss, "grad_loss");
  RKL_LAUNCH("bwd_rows_logits", s, rkl::launch_bwd_rows_logits(z_s, z_t, zr.rows, (int)(zr.rows ? zr.nrows : N), (int)N,
                                                              (int)V, row_mask, grad_loss, stats, dz_s, s));
  return RKL_OK;
}

int rkl_forward_logprob_entropy(int64_t N, int64_t V, int64_t H, const rkl_bf16* h, const rkl_bf16* W,
                                const int32_t* y, const uint8_t* row_mask, float* logp, float* entropy, float* stats,
                                void* workspace, size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, H, 0, false, true)) return rc;
  if (N > 0) {
    NEED16(h, "h"); NEED16(W, "W"); NEED4(y, "y");
    NEED4(logp, "logp"); NEED4(entropy, "entropy"); NEED4(stats, "stats");
  }
  return forward_tiled(N, V, H, 0, h, W, nullptr, nullptr, nullptr, y, row_mask, logp, entropy, stats, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

int rkl_backward_logprob_entropy(int64_t N, int64_t V, int64_t H, const rkl_bf16* h, const rkl_bf16* W,
                                 const int32_t* y, const uint8_t* row_mask, const float* grad_logp,
                                 const float* grad_entropy, const float* stats, float* dh, float* dW,
                                 int accumulate_dW, void* workspace, size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, H, 0, false, true)) return rc;
  NEED16(dW, "dW");
  if (N > 0) {
    NEED16(h, "h"); NEED16(W, "W"); NEED4(y, "y"); NEED4(stats, "stats"); NEED16(dh, "dh");
    OPT4(grad_logp, "grad_logp"); OPT4(grad_entropy, "grad_entropy");
  }
  return backward_tiled(N, V, H, 0, h, W, nullptr, nullptr, nullptr, y, row_mask, grad_logp, grad_entropy, stats, dh,
                        dW, accumulate_dW != 0, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int rkl_forward_topk(int64_t N, int64_t V, int64_t H, int64_t K, const rkl_bf16* h, const rkl_bf16* W,
                     const int32_t* y, const int32_t* support, const float* logpt_support, const float* logpt_y,
                     const uint8_t* row_mask, float* loss, float* stats, float* logps_support, void* workspace,
                     size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, H, 0, false, true)) return rc;
  if (K < 0 || K > V) return fail(RKL_INVALID_ARG, "K=%lld support entries out of range [0, V]", (long long)K);
  if (N * K > ((int64_t)1 << 40)) return fail(RKL_INVALID_ARG, "N*K too large");
  if (N > 0) {
    NEED16(h, "h"); NEED16(W, "W"); NEED4(y, "y"); NEED4(logpt_y, "logpt_y");
    NEED4(loss, "loss"); NEED4(stats, "stats");
    if (K > 0) { NEED4(support, "support"); NEED4(logpt_support, "logpt_support"); OPT4(logps_support, "logps_support"); }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the student's log-sum-exp and log p(y) over the whole vocabulary (the
  // log-probability forward; its log p(y) goes to `loss` for the moment)
  if (int rc = forward_tiled(N, V, H, 0, h, W, nullptr, nullptr, nullptr, y, row_mask, loss, nullptr, stats,
                             workspace, workspace_bytes, s))
    return rc;
  if (N == 0) return RKL_OK;
  RKL_LAUNCH("topk_terms", s, rkl::launch_topk_terms(h, W, (int)N, (int)V, (int)H, (int)K, y, support, logpt_support,
                                                    logpt_y, row_mask, loss, stats, K > 0 ? logps_support : nullptr,
                                                    s));
  return RKL_OK;
}

int rkl_backward_topk(int64_t N, int64_t V, int64_t H, int64_t K, const rkl_bf16* h, const rkl_bf16* W,
                      const int32_t* y, const int32_t* support, const float* logpt_support, const uint8_t* row_mask,
                      const float* grad_loss, const float* stats, const float* logps_support, float* dh, float* dW,
                      int accumulate_dW, void* workspace, size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, H, 0, false, true)) return rc;
  if (K < 0 || K > V) return fail(RKL_INVALID_ARG, "K=%lld support entries out of range [0, V]", (long long)K);
  if (N * K > ((int64_t)1 << 40)) return fail(RKL_INVALID_ARG, "N*K too large");
  NEED16(dW, "dW");
  if (N > 0) {
    NEED16(h, "h"); NEED16(W, "W"); NEED4(y, "y"); NEED4(stats, "stats"); NEED16(dh, "dh");
    OPT4(grad_loss, "grad_loss");
    if (K > 0) { NEED4(support, "support"); NEED4(logpt_support, "logpt_support"); OPT4(logps_support, "logps_support"); }
  }
  TopK t;
  t.on = true; t.K = (int)K; t.S = support; t.lpt_S = logpt_support; t.lps = K > 0 ? logps_support : nullptr;
  return backward_tiled(N, V, H, 0, h, W, nullptr, nullptr, nullptr, y, row_mask, grad_loss, nullptr, stats, dh, dW,
                        accumulate_dW != 0, workspace, workspace_bytes, static_cast<hipStream_t>(stream), Teachers{},
                        t);
}

int rkl_forward_hidden_teachers(int64_t N, int64_t V, int64_t Hs, int64_t Ht, int64_t K, const rkl_bf16* h_s,
                                const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t, const int32_t* teacher,
                                const uint8_t* row_mask, float* loss, float* stats, void* workspace,
                                size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, Hs, Ht, true, true)) return rc;
  if (K < 1 || K > 31) return fail(RKL_INVALID_ARG, "K=%lld teachers out of range [1, 31]", (long long)K);
  if (N > 0) {
    NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); NEED16(h_t, "h_t"); NEED16(W_t, "W_t"); NEED4(teacher, "teacher");
    NEED4(loss, "loss"); NEED4(stats, "stats");
  }
  const GroupLayout G = group_layout(N, Hs, Ht);
  const size_t need = G.total + ws_bytes(N, V, Hs, Ht);
  if (workspace_bytes < need)
    return fail(RKL_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (N == 0) return RKL_OK;
  NEED16(workspace, "workspace");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* g = static_cast<char*>(workspace);
  int32_t* perm = reinterpret_cast<int32_t*>(g + G.off_perm);
  int32_t* tid = reinterpret_cast<int32_t*>(g + G.off_tid);
  uint8_t* mask = row_mask ? reinterpret_cast<uint8_t*>(g + G.off_mask) : nullptr;
  rkl_bf16* hs = reinterpret_cast<rkl_bf16*>(g + G.off_hs);
  rkl_bf16* ht = reinterpret_cast<rkl_bf16*>(g + G.off_ht);
  float* loss_g = reinterpret_cast<float*>(g + G.off_row);
  float* stats_g = reinterpret_cast<float*>(g + G.off_stats);
  RKL_LAUNCH("group_by_teacher", s, rkl::launch_group_by_teacher(teacher, row_mask, (int)N, (int)K, perm, tid, mask, s));
  RKL_LAUNCH("gather", s, rkl::launch_gather(h_s, Hs * 2, perm, N, hs, s));
  RKL_LAUNCH("gather", s, rkl::launch_gather(h_t, Ht * 2, perm, N, ht, s));
  Teachers t;
  t.teacher = tid; t.K = (int)K; t.stride = V * Ht;
  if (int rc = forward_tiled(N, V, Hs, Ht, hs, W_s, ht, W_t, nullptr, nullptr, mask, loss_g, nullptr, stats_g,
                             g + G.total, workspace_bytes - G.total, s, t))
    return rc;
  RKL_LAUNCH("scatter", s, rkl::launch_scatter(loss_g, 4, perm, N, loss, s));
  RKL_LAUNCH("scatter", s, rkl::launch_scatter(stats_g, 16, perm, N, stats, s));
  return RKL_OK;
}

int rkl_backward_hidden_teachers(int64_t N, int64_t V, int64_t Hs, int64_t Ht, int64_t K, const rkl_bf16* h_s,
                                 const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t,
                                 const int32_t* teacher, const uint8_t* row_mask, const float* grad_loss,
                                 const float* stats, float* dh_s, float* dW_s, int accumulate_dW, void* workspace,
                                 size_t workspace_bytes, rkl_stream_t stream) {
  if (int rc = check_dims(N, V, Hs, Ht, true, true)) return rc;
  if (K < 1 || K > 31) return fail(RKL_INVALID_ARG, "K=%lld teachers out of range [1, 31]", (long long)K);
  NEED16(dW_s, "dW_s");
  if (N > 0) {
    NEED16(h_s, "h_s"); NEED16(W_s, "W_s"); NEED16(h_t, "h_t"); NEED16(W_t, "W_t"); NEED4(teacher, "teacher");
    NEED4(stats, "stats"); NEED16(dh_s, "dh_s"); OPT4(grad_loss, "grad_loss");
  }
  if (N > kMaxPitchElems)
    return fail(RKL_UNSUPPORTED, "N=%lld rows exceed the backward's limit of 2^22 per call", (long long)N);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GroupLayout G = group_layout(N, Hs, Ht);
  const size_t need = G.total + bwd_layout(N, V, Hs).total;
  if (workspace_bytes < need)
    return fail(RKL_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  Teachers t;
  t.K = (int)K; t.stride = V * Ht;
  if (N == 0)   // nothing to group: only dW is written (zeros unless accumulating)
    return backward_tiled(N, V, Hs, Ht, h_s, W_s, h_t, W_t, nullptr, nullptr, row_mask, grad_loss, nullptr, stats,
                          dh_s, dW_s, accumulate_dW != 0, workspace, workspace_bytes, s, t);
  NEED16(workspace, "workspace");
  char* g = static_cast<char*>(workspace);
  int32_t* perm = reinterpret_cast<int32_t*>(g + G.off_perm);
  int32_t* tid = reinterpret_cast<int32_t*>(g + G.off_tid);
  uint8_t* mask = row_mask ? reinterpret_cast<uint8_t*>(g + G.off_mask) : nullptr;
  rkl_bf16* hs = reinterpret_cast<rkl_bf16*>(g + G.off_hs);
  rkl_bf16* ht = reinterpret_cast<rkl_bf16*>(g + G.off_ht);
  float* grad_g = grad_loss ? reinterpret_cast<float*>(g + G.off_row) : nullptr;
  float* stats_g = reinterpret_cast<float*>(g + G.off_stats);
  float* dh_g = reinterpret_cast<float*>(g + G.off_dh);
  RKL_LAUNCH("group_by_teacher", s, rkl::launch_group_by_teacher(teacher, row_mask, (int)N, (int)K, perm, tid, mask, s));
  RKL_LAUNCH("gather", s, rkl::launch_gather(h_s, Hs * 2, perm, N, hs, s));
  RKL_LAUNCH("gather", s, rkl::launch_gather(h_t, Ht * 2, perm, N, ht, s));
  if (grad_loss) RKL_LAUNCH("gather", s, rkl::launch_gather(grad_loss, 4, perm, N, grad_g, s));
  RKL_LAUNCH("gather", s, rkl::launch_gather(stats, 16, perm, N, stats_g, s));
  t.teacher = tid;
  if (int rc = backward_tiled(N, V, Hs, Ht, hs, W_s, ht, W_t, nullptr, nullptr, mask, grad_g, nullptr, stats_g, dh_g,
                              dW_s, accumulate_dW != 0, g + G.total, workspace_bytes - G.total, s, t))
    return rc;
  RKL_LAUNCH("scatter", s, rkl::launch_scatter(dh_g, Hs * 4, perm, N, dh_s, s));
  return RKL_OK;
}

}  // extern "C"
#pragma GCC visibility pop
