// C ABI of the DSpark round (declared in include/dspark.h): argument checks,
// workspace layout, launch order and the per-kernel event timing.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <vector>

#include "dspark.h"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace: [header | scheduler ranks | tile stats (B + 1 rows) | block stats | request state | slot list |
// residual tile mass | U rows of the last drawn tokens | acceptance pass: row
// statistics, row argmax, tile masses | lazy verification: row counters, request progress |
// resident draft round: phase flags, exit counter].  Header words: 0 status, 1 residual slot count, 2 scheduler
// ticket, 3 scheduler first failure.  The header and the scheduler ranks are all
// that dspark_schedule touches, at offsets that do not depend on V and r.
constexpr size_t kHeaderBytes = 256;
struct Layout {
  size_t header, sched, tstat, bstat, req, slots, rsum, hrows, rowinfo, rowarg, tmass, vsync, grid, total;
  int n_tiles, n_blk;
};

bool schedule_sizes_ok(int B, int gamma) {
  return B >= 1 && gamma >= 1 && gamma <= 16 && (long long)B * gamma <= 8192;
}

bool sizes_ok(int B, int gamma, int V, int r) {
  return B >= 1 && gamma >= 1 && gamma <= 16 && V >= 1 && r >= 1 &&
         (long long)B * (gamma + 1) <= (1ll << 31) / 4;
}

Layout layout(int B, int gamma, int V, int r) {
  Layout L{};
  L.n_tiles = (V + kTile - 1) / kTile;
  L.n_blk = (V + kBlock - 1) / kBlock;
  size_t off = 0;
  L.header = off;
  off = align_up(off + kHeaderBytes);
  L.sched = off;  // candidate ranks, then Theta of every cut (best-cut rule)
  off = align_up(off + (size_t)B * gamma * sizeof(int32_t));
  off = align_up(off + ((size_t)B * gamma + 1) * sizeof(double));
  L.tstat = off;  // one spare row (B) takes the records of padding slots
  off = align_up(off + (size_t)(B + 1) * L.n_tiles * sizeof(TileStatRef));  // the larger record (fp32 logits)
  L.bstat = off;
  off = align_up(off + (size_t)B * (gamma + 1) * L.n_blk * sizeof(BlockStat));
  L.req = off;
  off = align_up(off + (size_t)B * sizeof(ReqState));
  L.slots = off;
  off = align_up(off + (size_t)B * sizeof(int32_t));
  L.rsum = off;
  off = align_up(off + (size_t)B * L.n_tiles * sizeof(float));
  L.hrows = off;  // U rows of the tokens drawn at the previous block position
  off = align_up(off + (size_t)B * r * sizeof(uint16_t));
  // acceptance pass: target row statistics and the tile masses of every position
  L.rowinfo = off;
  off = align_up(off + (size_t)B * gamma * 2 * sizeof(double));
  L.rowarg = off;
  off = align_up(off + (size_t)B * gamma * sizeof(int32_t));
  L.tmass = off;
  off = align_up(off + (size_t)B * gamma * L.n_tiles * sizeof(float));
  L.vsync = off;  // lazy verification: blocks done per target row, then the decided positions per request
  off = align_up(off + ((size_t)B * (gamma + 1) + B) * sizeof(uint32_t));
  L.grid = off;  // resident draft round: phase flags of the workgroups and the exit counter
  off = align_up(off + (size_t)kResidentGridWords * sizeof(uint32_t));
  L.total = off;
  return L;
}

template <typename T> T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool dtype_ok(int d) { return d == DSPARK_BF16 || d == DSPARK_F32; }

// ---------------------------------------------------------------------------
// Kernel timing with HIP events (off unless enabled per class).
// ---------------------------------------------------------------------------
struct ProfState {
  std::mutex mu;
  int period[kNumClasses] = {};    // 0: off; k: every k-th launch of the class is timed
  unsigned seen[kNumClasses] = {}; // launches of the class since it was enabled
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[kNumClasses];
  // event pairs that were read back, reused by later scopes (creating events on
  // every launch costs host time that shows up in the timed region)
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
};
ProfState& prof() {
  static ProfState p;
  return p;
}

}  // namespace

namespace {
thread_local KernelEvents* t_events = nullptr;

struct SetupKey {
  const void* fn;
  int dev, threads;
  size_t lds;
  bool operator<(const SetupKey& o) const {
    if (fn != o.fn) return fn < o.fn;
    if (dev != o.dev) return dev < o.dev;
    if (threads != o.threads) return threads < o.threads;
    return lds < o.lds;
  }
};
}  // namespace

hipError_t kernel_setup(const void* fn, int threads, size_t lds, int* groups) {
  static std::mutex mu;
  static std::map<SetupKey, int> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const SetupKey key{fn, dev, threads, lds};
  std::lock_guard<std::mutex> g(mu);
  auto it = done.find(key);
  if (it != done.end()) {
    *groups = it->second;
    return hipSuccess;
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess || per_cu < 1) {
    per_cu = 1;
    (void)hipGetLastError();  // handled here: not to be reported with a later launch
  }
  *groups = cus * per_cu;
  done.emplace(key, *groups);
  return hipSuccess;
}


KernelEvents* kernel_events() { return t_events; }

thread_local int t_hip_error = 0;
int hip_failed(hipError_t e) {
  t_hip_error = (int)e;
  return DSPARK_EHIP;
}

ProfileScope::ProfileScope(int c, hipStream_t) : cls(c), ev{nullptr, nullptr, 0}, outer(t_events), on(false) {
  {
    ProfState& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (p.period[cls] <= 0 || p.seen[cls]++ % (unsigned)p.period[cls] != 0) return;
    if (!p.pool.empty()) {
      ev.start = p.pool.back().first, ev.stop = p.pool.back().second;
      p.pool.pop_back();
    }
  }
  if (!ev.start) {
    if (hipEventCreate(&ev.start) != hipSuccess) return;
    if (hipEventCreate(&ev.stop) != hipSuccess) {
      (void)hipEventDestroy(ev.start);
      return;
    }
  }
  on = true;
  t_events = &ev;
}

ProfileScope::~ProfileScope() {
  if (!on) return;
  t_events = outer;
  ProfState& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (ev.launches == 0) {  // nothing was launched: nothing to time
    p.pool.emplace_back(ev.start, ev.stop);
    return;
  }
  p.ev[cls].emplace_back(ev.start, ev.stop);
}

}  // namespace dspark

using namespace dspark;

#define DSPARK_TRY(expr)                         \
  do {                                           \
    const hipError_t e_ = (expr);                \
    if (e_ != hipSuccess) return hip_failed(e_); \
  } while (0)

namespace {

// Arguments of the scheduler over `workspace` (its part of the layout and the
// status word), or DSPARK_EINVAL with nothing enqueued.
int schedule_args_ok(const float* conf, const double* sps_B, const double* sps_val, int n_points, int B, int gamma,
                     int rule, double param, int32_t* budget) {
  if (!schedule_sizes_ok(B, gamma)) return DSPARK_EINVAL;
  if (rule < DSPARK_SCHED_EARLY_STOP || rule > DSPARK_SCHED_THRESHOLD) return DSPARK_EINVAL;
  const bool table = rule == DSPARK_SCHED_EARLY_STOP || rule == DSPARK_SCHED_ARGMAX;
  if (table && (n_points < 2 || n_points > 1024 || !sps_B || !sps_val)) return DSPARK_EINVAL;
  if (!(param == param)) return DSPARK_EINVAL;  // NaN
  if (!conf || !budget) return DSPARK_EINVAL;
  return DSPARK_OK;
}

int schedule_args(const float* conf, const float* tau, const double* sps_B, const double* sps_val, int n_points,
                  int B, int gamma, int rule, double param, int32_t* budget, void* workspace, ScheduleArgs& a) {
  const int ok = schedule_args_ok(conf, sps_B, sps_val, n_points, B, gamma, rule, param, budget);
  if (ok != DSPARK_OK) return ok;
  if (!workspace) return DSPARK_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return DSPARK_EINVAL;
  const bool table = rule == DSPARK_SCHED_EARLY_STOP || rule == DSPARK_SCHED_ARGMAX;
  a = ScheduleArgs{};
  a.conf = conf, a.tau = tau, a.sps_B = sps_B, a.sps_val = sps_val, a.n_points = table ? n_points : 0;
  a.B = B, a.gamma = gamma, a.rule = rule, a.param = param, a.budget = budget;
  a.status = at<uint32_t>(workspace, 0);
  a.ticket = a.status + 2, a.stop_enc = a.status + 3;
  a.rank = at<int32_t>(workspace, align_up(kHeaderBytes));
  a.theta = at<double>(workspace, align_up(kHeaderBytes) + align_up((size_t)B * gamma * sizeof(int32_t)));
  return DSPARK_OK;
}

int draft_args_ok(const void* base_logits, int logits_dtype, const void* U, const void* W, int factor_dtype,
                  int w_layout, const int32_t* prev0, const float* temperature, int B, int gamma, int V, int r,
                  int32_t* draft_tokens, float* draft_logq, double* draft_lse, void* workspace) {
  if (!sizes_ok(B, gamma, V, r) || !dtype_ok(logits_dtype) || !dtype_ok(factor_dtype)) return DSPARK_EINVAL;
  if (w_layout != DSPARK_W_VOCAB_MAJOR) return DSPARK_EINVAL;
  if (!base_logits || !U || !W || !prev0 || !temperature || !draft_tokens || !draft_logq || !draft_lse ||
      !workspace)
    return DSPARK_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return DSPARK_EINVAL;
  return DSPARK_OK;
}

// Which implementation of the draft round runs (dspark_set_draft_path).
std::atomic<int>& draft_path() {
  static std::atomic<int> p{DSPARK_DRAFT_PER_POSITION};
  return p;
}

// The draft round on validated arguments; with `sched`, the scheduler too: one
// GEMM and one draw per position, the scheduler in the launch of the last draw
// when that draw uses the fast kernel, else after it.  On the resident path
// (when it fits) one launch runs the whole round and the scheduler follows it.
int draft_round(const void* base_logits, int logits_dtype, const void* U, const void* W, int factor_dtype,
                const int32_t* prev0, const float* temperature, uint64_t seed, const int32_t* pos_offset, int B,
                int gamma, int V, int r, int32_t* draft_tokens, float* draft_logq, double* draft_lse,
                void* workspace, hipStream_t s, const ScheduleArgs* sched) {
  const Layout L = layout(B, gamma, V, r);
  uint32_t* status = at<uint32_t>(workspace, L.header);

  GemmArgs g{};
  g.base = base_logits, g.U = U, g.Wt = W, g.prev0 = prev0, g.draft = draft_tokens;
  g.temperature = temperature;
  g.B = B, g.gamma = gamma, g.V = V, g.r = r, g.n_tiles = L.n_tiles;
  g.tstat = at<TileStatRef>(workspace, L.tstat);
  g.status = status;

  DraftSelectArgs d{};
  d.base = base_logits, d.U = U, d.Wt = W, d.prev0 = prev0, d.temperature = temperature;
  d.pos_offset = pos_offset, d.tstat = g.tstat, d.seed = seed;
  d.B = B, d.gamma = gamma, d.V = V, d.r = r, d.n_tiles = L.n_tiles;
  d.draft = draft_tokens, d.logq = draft_logq, d.lse = draft_lse, d.status = status;
  // the streaming GEMM takes the U rows of the previous tokens from this table
  // (filled by the draw of the previous position) instead of gathering them
  if (draft_path().load(std::memory_order_relaxed) == DSPARK_DRAFT_RESIDENT) {
    // the whole round in one launch, W2 kept on chip
    hipError_t e;
    {
      ProfileScope ps(kClsDraftRound, s);
      e = launch_draft_resident(d, logits_dtype, factor_dtype, at<uint32_t>(workspace, L.grid), s);
    }
    if (e == hipSuccess) {
      if (sched) {
        ProfileScope ps(kClsSchedule, s);
        DSPARK_TRY(launch_schedule(*sched, s));
      }
      return DSPARK_OK;
    }
    if (e != hipErrorNotSupported) return hip_failed(e);
  }

  const bool table = factor_dtype == DSPARK_BF16 && (r == 128 || r == 256);
  d.hrows = table ? at<void>(workspace, L.hrows) : nullptr;

  for (int pos = 0; pos < gamma; ++pos) {
    g.pos = pos;
    g.hrows = pos > 0 ? d.hrows : nullptr;
    d.pos = pos;
    {
      ProfileScope ps(kClsDraftGemm, s);
      DSPARK_TRY(launch_gemm_stats(g, logits_dtype, factor_dtype, false, s));
    }
    if (sched && pos == gamma - 1) {
      // the last draw and the scheduler, both bound by latency, in one launch
      ProfileScope ps(kClsDraftSelect, s);
      const hipError_t e = launch_draft_select_schedule(d, *sched, logits_dtype, factor_dtype, s);
      if (e == hipSuccess) return DSPARK_OK;
      if (e != hipErrorNotSupported) return hip_failed(e);
    }
    {
      ProfileScope ps(kClsDraftSelect, s);
      DSPARK_TRY(launch_draft_select(d, logits_dtype, factor_dtype, s));
    }
  }
  if (sched) {
    ProfileScope ps(kClsSchedule, s);
    DSPARK_TRY(launch_schedule(*sched, s));
  }
  return DSPARK_OK;
}

}  // namespace

extern "C" {

int dspark_abi_version(void) { return DSPARK_ABI_VERSION; }

const char* dspark_error_string(int code) {
  switch (code) {
    case DSPARK_OK: return "ok";
    case DSPARK_EINVAL: return "invalid argument";
    case DSPARK_EHIP: return "HIP runtime error";
    case DSPARK_EDATA: return "invalid input data found on the device";
    default: return "unknown error";
  }
}

int dspark_last_hip_error(const char** name) {
  if (name) *name = hipGetErrorName(static_cast<hipError_t>(t_hip_error));
  return t_hip_error;
}

size_t dspark_workspace_bytes(int B, int gamma, int V, int r) {
  if (!sizes_ok(B, gamma, V, r)) return 0;
  return layout(B, gamma, V, r).total;
}

size_t dspark_schedule_workspace_bytes(int B, int gamma) {
  if (!schedule_sizes_ok(B, gamma)) return 0;
  return align_up(kHeaderBytes) + align_up((size_t)B * gamma * sizeof(int32_t)) +
         align_up(((size_t)B * gamma + 1) * sizeof(double));
}

int dspark_pack_w2(const void* W, int factor_dtype, int V, int r, void* W_packed, void* stream) {
  if (!W || !W_packed || V < 1 || r < 1 || !dtype_ok(factor_dtype)) return DSPARK_EINVAL;
  const int es = factor_dtype == DSPARK_BF16 ? 2 : 4;
  DSPARK_TRY(launch_pack_w2(W, W_packed, es, V, r, static_cast<hipStream_t>(stream)));
  return DSPARK_OK;
}

int dspark_set_draft_path(int path) {
  if (path != DSPARK_DRAFT_PER_POSITION && path != DSPARK_DRAFT_RESIDENT) return DSPARK_EINVAL;
  return draft_path().exchange(path);
}

int dspark_set_resident_wait_bound(double seconds, double* previous) {
  if (!(seconds >= 0.0 && seconds <= 60.0)) return DSPARK_EINVAL;
  const uint64_t prev = set_resident_wait_ticks((uint64_t)(seconds * 1e8));
  if (previous) *previous = (double)prev * 1e-8;
  return DSPARK_OK;
}

int dspark_draft_round(const void* base_logits, int logits_dtype, const void* U, const void* W,
                       int factor_dtype, int w_layout, const int32_t* prev0, const float* temperature,
                       uint64_t seed, const int32_t* pos_offset, int B, int gamma, int V, int r,
                       int32_t* draft_tokens, float* draft_logq, double* draft_lse, void* workspace,
                       void* stream) {
  const int ok = draft_args_ok(base_logits, logits_dtype, U, W, factor_dtype, w_layout, prev0, temperature, B, gamma, V, r,
                               draft_tokens, draft_logq, draft_lse, workspace);
  if (ok != DSPARK_OK) return ok;
  return draft_round(base_logits, logits_dtype, U, W, factor_dtype, prev0, temperature, seed, pos_offset, B, gamma,
                     V, r, draft_tokens, draft_logq, draft_lse, workspace, static_cast<hipStream_t>(stream),
                     nullptr);
}

int dspark_draft_schedule(const void* base_logits, int logits_dtype, const void* U, const void* W,
                          int factor_dtype, int w_layout, const int32_t* prev0, const float* temperature, uint64_t seed,
                          const int32_t* pos_offset, int B, int gamma, int V, int r, int32_t* draft_tokens,
                          float* draft_logq, double* draft_lse, const float* conf, const float* tau,
                          const double* sps_B, const double* sps_val, int n_points, int rule, double param,
                          int32_t* budget, void* workspace, void* stream) {
  ScheduleArgs a;
  int ok = schedule_args(conf, tau, sps_B, sps_val, n_points, B, gamma, rule, param, budget, workspace, a);
  if (ok != DSPARK_OK) return ok;
  ok = draft_args_ok(base_logits, logits_dtype, U, W, factor_dtype, w_layout, prev0, temperature, B, gamma, V, r, draft_tokens,
                     draft_logq, draft_lse, workspace);
  if (ok != DSPARK_OK) return ok;
  return draft_round(base_logits, logits_dtype, U, W, factor_dtype, prev0, temperature, seed, pos_offset, B, gamma,
                     V, r, draft_tokens, draft_logq, draft_lse, workspace, static_cast<hipStream_t>(stream), &a);
}

int dspark_schedule_ex(const float* conf, const float* tau, const double* sps_B, const double* sps_val,
                       int n_points, int B, int gamma, int rule, double param, int32_t* budget,
                       void* workspace, void* stream) {
  ScheduleArgs a;
  const int ok = schedule_args(conf, tau, sps_B, sps_val, n_points, B, gamma, rule, param, budget, workspace, a);
  if (ok != DSPARK_OK) return ok;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ProfileScope ps(kClsSchedule, s);
  DSPARK_TRY(launch_schedule(a, s));
  return DSPARK_OK;
}

int dspark_schedule_static(const float* conf, const double* sps_B, const double* sps_val, int n_points, int B,
                           int gamma, int32_t* budget, uint32_t* status, void* stream) {
  // arguments first: nothing is enqueued (not even the first call's clearing) for bad ones
  int ok = schedule_args_ok(conf, sps_B, sps_val, n_points, B, gamma, DSPARK_SCHED_EARLY_STOP, 0.0, budget);
  if (ok != DSPARK_OK) return ok;
  if (dspark_schedule_workspace_bytes(B, gamma) > kStaticScheduleBytes) return DSPARK_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  DSPARK_TRY(static_schedule_scratch(&scratch, s));
  ScheduleArgs a;
  ok = schedule_args(conf, nullptr, sps_B, sps_val, n_points, B, gamma, DSPARK_SCHED_EARLY_STOP, 0.0, budget,
                     scratch, a);
  if (ok != DSPARK_OK) return ok;
  if (status) a.status = status;
  ProfileScope ps(kClsSchedule, s);
  DSPARK_TRY(launch_schedule(a, s));
  return DSPARK_OK;
}

int dspark_schedule(const float* conf, const double* sps_B, const double* sps_val, int n_points,
                    int B, int gamma, int32_t* budget, void* workspace, void* stream) {
  return dspark_schedule_ex(conf, nullptr, sps_B, sps_val, n_points, B, gamma, DSPARK_SCHED_EARLY_STOP, 0.0,
                            budget, workspace, stream);
}

int dspark_verify(const void* target_logits, const void* base_logits, int logits_dtype, const void* U,
                  const void* W, int factor_dtype, int w_layout, const int32_t* prev0, const int32_t* draft_tokens,
                  const float* draft_logq, const double* draft_lse, const int32_t* budget,
                  const float* temperature, uint64_t seed, const int32_t* pos_offset, int B, int gamma,
                  int V, int r, int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                  float* debug_logp_logq, float* debug_residual, void* workspace, void* stream) {
  if (!sizes_ok(B, gamma, V, r) || !dtype_ok(logits_dtype) || !dtype_ok(factor_dtype)) return DSPARK_EINVAL;
  if (w_layout != DSPARK_W_VOCAB_MAJOR) return DSPARK_EINVAL;
  if (!target_logits || !base_logits || !U || !W || !prev0 || !draft_tokens || !draft_logq || !draft_lse ||
      !temperature || !out_tokens || !num_accepted || !num_emitted || !workspace)
    return DSPARK_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return DSPARK_EINVAL;
  const Layout L = layout(B, gamma, V, r);
  hipStream_t s = static_cast<hipStream_t>(stream);

  VerifyArgs a{};
  a.target = target_logits, a.base = base_logits, a.U = U, a.Wt = W, a.prev0 = prev0;
  a.draft = draft_tokens, a.draft_logq = draft_logq, a.draft_lse = draft_lse, a.budget = budget;
  a.temperature = temperature, a.pos_offset = pos_offset, a.seed = seed;
  a.B = B, a.gamma = gamma, a.V = V, a.r = r, a.n_blk = L.n_blk, a.n_tiles = L.n_tiles;
  a.bstat = at<BlockStat>(workspace, L.bstat);
  a.rowcnt = at<uint32_t>(workspace, L.vsync);
  a.vstate = a.rowcnt + (size_t)B * (gamma + 1);
  a.req = at<ReqState>(workspace, L.req);
  a.slot_req = at<int32_t>(workspace, L.slots);
  a.slot_count = at<uint32_t>(workspace, L.header) + 1;
  a.rsum = at<float>(workspace, L.rsum);
  a.out_tokens = out_tokens, a.num_accepted = num_accepted, a.num_emitted = num_emitted;
  a.debug_logp_logq = debug_logp_logq, a.debug_residual = debug_residual;
  a.status = at<uint32_t>(workspace, L.header);

  {
    // target rows read up to the first rejection; statistics, tests and final tokens in one pass
    ProfileScope ps(kClsRowStats, s);
    DSPARK_TRY(launch_verify_lazy(a, logits_dtype, s));
  }
  {
    GemmArgs g{};
    g.base = base_logits, g.target = target_logits, g.U = U, g.Wt = W, g.prev0 = prev0;
    g.draft = draft_tokens, g.temperature = temperature, g.draft_lse = draft_lse, g.req = a.req;
    g.slot_req = a.slot_req, g.slot_count = a.slot_count;
    g.B = B, g.gamma = gamma, g.V = V, g.r = r, g.n_tiles = L.n_tiles;
    g.rsum = a.rsum, g.status = a.status;
    ProfileScope ps(kClsResidualGemm, s);
    DSPARK_TRY(launch_gemm_stats(g, logits_dtype, factor_dtype, true, s));
  }
  {
    ProfileScope ps(kClsResidualSelect, s);
    DSPARK_TRY(launch_residual_select(a, logits_dtype, factor_dtype, s));
  }
  if (debug_residual) DSPARK_TRY(launch_residual_debug(a, logits_dtype, factor_dtype, s));
  return DSPARK_OK;
}

int dspark_acceptance(const void* target_logits, const void* base_logits, int logits_dtype, const void* U,
                      const void* W, int factor_dtype, int w_layout, const int32_t* prev0, const int32_t* draft_tokens,
                      const double* draft_lse, const float* temperature, int B, int gamma, int V, int r,
                      double* c_star, void* workspace, void* stream) {
  if (!sizes_ok(B, gamma, V, r) || !dtype_ok(logits_dtype) || !dtype_ok(factor_dtype)) return DSPARK_EINVAL;
  if (w_layout != DSPARK_W_VOCAB_MAJOR) return DSPARK_EINVAL;
  if (!target_logits || !base_logits || !U || !W || !prev0 || !draft_tokens || !draft_lse || !temperature ||
      !c_star || !workspace)
    return DSPARK_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return DSPARK_EINVAL;
  const Layout L = layout(B, gamma, V, r);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // block statistics of target rows 0..gamma (all of them)
  VerifyArgs v{};
  v.target = target_logits, v.temperature = temperature, v.budget = nullptr;
  v.B = B, v.gamma = gamma, v.V = V, v.r = r, v.n_blk = L.n_blk, v.n_tiles = L.n_tiles;
  v.bstat = at<BlockStat>(workspace, L.bstat);
  v.slot_count = at<uint32_t>(workspace, L.header) + 1;
  v.status = at<uint32_t>(workspace, L.header);
  DSPARK_TRY(launch_row_stats(v, logits_dtype, s));

  AcceptanceArgs c{};
  c.bstat = v.bstat, c.temperature = temperature, c.draft = draft_tokens;
  c.tile_mass = at<float>(workspace, L.tmass);
  c.rowinfo = at<double2>(workspace, L.rowinfo);
  c.rowarg = at<int32_t>(workspace, L.rowarg);
  c.c_star = c_star;
  c.B = B, c.gamma = gamma, c.V = V, c.n_blk = L.n_blk, c.n_tiles = L.n_tiles;
  c.status = v.status;
  DSPARK_TRY(launch_row_info(c, s));

  // tile masses of min(p, q) for every (request, row): the residual-mode pass
  GemmArgs g{};
  g.base = base_logits, g.target = target_logits, g.U = U, g.Wt = W, g.prev0 = prev0;
  g.draft = draft_tokens, g.temperature = temperature, g.draft_lse = draft_lse;
  g.tv = 1, g.rowinfo = c.rowinfo;
  g.B = B, g.gamma = gamma, g.V = V, g.r = r, g.n_tiles = L.n_tiles;
  g.rsum = at<float>(workspace, L.tmass), g.status = v.status;
  {
    ProfileScope ps(kClsAcceptance, s);
    DSPARK_TRY(launch_gemm_stats(g, logits_dtype, factor_dtype, true, s, &c.n_parts));
  }
  DSPARK_TRY(launch_acceptance_finish(c, s));
  return DSPARK_OK;
}

int dspark_status(void* workspace, void* stream) {
  if (!workspace) return DSPARK_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  DSPARK_TRY(hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s));
  DSPARK_TRY(hipStreamSynchronize(s));
  if (word) {
    DSPARK_TRY(hipMemsetAsync(workspace, 0, sizeof(word), s));
    DSPARK_TRY(hipStreamSynchronize(s));
    return DSPARK_EDATA;
  }
  return DSPARK_OK;
}

int dspark_profile_enable(int kernel_class, int enabled) {
  if (kernel_class < 0 || kernel_class >= kNumClasses) return DSPARK_EINVAL;
  if (enabled < 0) return DSPARK_EINVAL;
  ProfState& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.period[kernel_class] = enabled;
  p.seen[kernel_class] = 0;
  return DSPARK_OK;
}

int dspark_profile_read(int kernel_class, int* launches, double* total_ms) {
  if (kernel_class < 0 || kernel_class >= kNumClasses || !launches || !total_ms) return DSPARK_EINVAL;
  ProfState& p = prof();
  std::vector<std::pair<hipEvent_t, hipEvent_t>> evs;
  {
    std::lock_guard<std::mutex> g(p.mu);
    evs.swap(p.ev[kernel_class]);
  }
  double tot = 0.0;
  int rc = DSPARK_OK;
  for (auto& e : evs) {
    float ms = 0.0f;
    hipError_t he = hipEventSynchronize(e.second);
    if (he == hipSuccess) he = hipEventElapsedTime(&ms, e.first, e.second);
    if (he != hipSuccess) rc = hip_failed(he);
    tot += ms;
  }
  {
    std::lock_guard<std::mutex> g(p.mu);
    p.pool.insert(p.pool.end(), evs.begin(), evs.end());
  }
  *launches = (int)evs.size();
  *total_ms = tot;
  return rc;
}

}  // extern "C"
