// Host-side launchers of the DSpark kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "device.hpp"

namespace dspark {

enum KernelClass : int {
  kClsDraftGemm = 0, kClsDraftSelect = 1, kClsRowStats = 2, kClsAccept = 3,
  kClsResidualGemm = 4, kClsResidualSelect = 5, kClsSchedule = 6, kClsAcceptance = 7, kClsDraftRound = 8,
  kNumClasses = 9,
};

// Kernel timing (measurement support).  While a ProfileScope of an enabled
// class is open, the launches inside it carry its two events in their dispatch:
// `start` takes the first kernel's start time and `stop` each kernel's end time,
// so the interval covers kernel execution and the gaps between the scope's own
// kernels, not the dispatch of the first one.
struct KernelEvents {
  hipEvent_t start, stop;
  int launches;
};
KernelEvents* kernel_events();  // the innermost open scope's events, or NULL
// Records `e` as this thread's last HIP failure (dspark_last_hip_error) and
// returns DSPARK_EHIP.
int hip_failed(hipError_t e);

struct ProfileScope {
  ProfileScope(int cls, hipStream_t s);
  ~ProfileScope();
  int cls;
  KernelEvents ev;
  KernelEvents* outer;
  bool on;
};

// One-time set-up of a kernel on the current device, safe under concurrent host
// threads (done once per kernel, device and LDS size, under a lock): raises the
// kernel's dynamic-LDS limit to `lds` when that exceeds 64 KB and stores in
// *groups the device's CU count times the workgroups of `threads` threads that
// fit on one CU (1 per CU if the occupancy query fails).  Returns the error of a
// failed device query or attribute call (nothing is cached then).
hipError_t kernel_setup(const void* fn, int threads, size_t lds, int* groups);

// Launch of a kernel taking one argument struct, timed by the open ProfileScope.
// Errors are left for hipGetLastError(), as with the <<<>>> launch.
template <typename Arg, typename A>
void launch(void (*k)(Arg), dim3 grid, dim3 block, size_t lds, hipStream_t s, const A& a) {
  KernelEvents* e = kernel_events();
  if (!e) {
    k<<<grid, block, lds, s>>>(a);
    return;
  }
  Arg arg = a;
  void* args[] = {&arg};
  if (hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, lds, s,
                         e->launches == 0 ? e->start : nullptr, e->stop, 0) == hipSuccess)
    ++e->launches;
}

// Arguments of the fused Markov-bias GEMM with its softmax-statistics epilogue.
// Draft mode: one slot per request, base row `pos`; writes TileRec<logit type>
// [B + 1][n_tiles] (8 bytes a record for bf16 logits, 16 for fp32).
// Residual mode: slots are the requests listed in slot_req[0..*slot_count), each
// at its own row req[b].n; writes the residual mass of every tile [B][n_tiles].
struct GemmArgs {
  const void* base;          // [B, gamma, V]
  const void* target;        // [B, gamma+1, V]        (residual mode)
  const void* U;             // [V, r]
  const void* Wt;            // [V, r]
  const int32_t* prev0;      // [B]
  const int32_t* draft;      // [B, gamma]
  const float* temperature;  // [B]
  const double* draft_lse;   // [B, gamma]             (residual mode)
  const void* hrows;         // [B, r] U rows of the previous tokens, or NULL (draft mode)
  const ReqState* req;       // [B]                    (residual mode)
  const int32_t* slot_req;   // [B]                    (residual mode)
  const uint32_t* slot_count;//                        (residual mode)
  int tv;                    // residual mode as the acceptance pass: every (request, row)
  const double2* rowinfo;    // [B, gamma] target row max and ln-sum-exp    (acceptance pass)
  int B, gamma, V, r, n_tiles, pos;
  void* tstat;               // draft mode output: TileRec<logit type> records
  float* rsum;               // residual mode output
  uint32_t* status;
};

// `parts` (acceptance pass, may be NULL) receives the number of partial sums
// written per slot row of rsum: n_tiles, or one per workgroup of the streaming pass.
hipError_t launch_gemm_stats(const GemmArgs& a, int logits_dtype, int factor_dtype, bool residual,
                             hipStream_t s, int* parts = nullptr);

struct DraftSelectArgs {
  const void* base;
  const void* U;
  const void* Wt;
  const int32_t* prev0;
  const float* temperature;
  const int32_t* pos_offset;
  const void* tstat;         // TileRec<logit type> records of position pos
  uint64_t seed;
  int B, gamma, V, r, n_tiles, pos;
  int32_t* draft;
  float* logq;
  double* lse;
  void* hrows;               // [B, r] or NULL: receives U[x] of the token drawn
  uint32_t* status;
};

hipError_t launch_draft_select(const DraftSelectArgs& a, int logits_dtype, int factor_dtype,
                               hipStream_t s);

// The whole draft round (every position: contraction, statistics, draw) in one
// cooperative launch that keeps W2 on chip; hipErrorNotSupported when the sizes,
// types or the device do not fit it (the caller then launches per position).
// `grid_words` (kResidentGridWords words of the workspace, zero between calls)
// holds the launch's phase flags.
constexpr int kResidentGridWords = 1024 + 64;
hipError_t launch_draft_resident(const DraftSelectArgs& d, int logits_dtype, int factor_dtype,
                                 uint32_t* grid_words, hipStream_t s);
// Sets the bound of the resident round's device-wide waits (s_memrealtime
// ticks, 100 MHz) for later launches; returns the previous bound.
uint64_t set_resident_wait_ticks(uint64_t ticks);

struct VerifyArgs {
  const void* target;
  const void* base;
  const void* U;
  const void* Wt;
  const int32_t* prev0;
  const int32_t* draft;
  const float* draft_logq;
  const double* draft_lse;
  const int32_t* budget;
  const float* temperature;
  const int32_t* pos_offset;
  uint64_t seed;
  int B, gamma, V, r, n_blk, n_tiles;
  BlockStat* bstat;          // [B, gamma+1, n_blk]
  uint32_t* rowcnt;          // [B, gamma+1] work items of each target row done (lazy pass; zero between calls)
  uint32_t* vstate;          // [B] progress word of the lazy pass (rows complete, positions accepted, done)
  ReqState* req;             // [B]
  int32_t* slot_req;         // [B]
  uint32_t* slot_count;
  float* rsum;               // [B, n_tiles]
  int32_t* out_tokens;
  int32_t* num_accepted;
  int32_t* num_emitted;
  float* debug_logp_logq;
  float* debug_residual;
  uint32_t* status;
};

hipError_t launch_row_stats(const VerifyArgs& a, int logits_dtype, hipStream_t s);
hipError_t launch_verify_lazy(const VerifyArgs& a, int logits_dtype, hipStream_t s);
hipError_t launch_residual_select(const VerifyArgs& a, int logits_dtype, int factor_dtype,
                                  hipStream_t s);
hipError_t launch_residual_debug(const VerifyArgs& a, int logits_dtype, int factor_dtype,
                                 hipStream_t s);

// Acceptance pass helpers: statistics of target rows 0..gamma-1 from their
// block statistics, and the per-position sum of the tile masses.
struct AcceptanceArgs {
  const BlockStat* bstat;    // [B, gamma+1, n_blk]
  const float* temperature;
  const int32_t* draft;      // [B, gamma]
  const float* tile_mass;    // [B * gamma, n_tiles]
  double2* rowinfo;          // [B, gamma]
  int32_t* rowarg;           // [B, gamma] lowest index of the row maximum
  double* c_star;            // [B, gamma]
  int B, gamma, V, n_blk, n_tiles;
  int n_parts;               // partial sums per position in tile_mass
  uint32_t* status;
};
hipError_t launch_row_info(const AcceptanceArgs& a, hipStream_t s);
hipError_t launch_acceptance_finish(const AcceptanceArgs& a, hipStream_t s);

struct ScheduleArgs {
  const float* conf;
  const float* tau;          // [gamma] Sequential Temperature Scaling, or NULL
  const double* sps_B;
  const double* sps_val;
  int n_points, B, gamma;
  int rule;                  // dspark_schedule_rule
  double param;              // fixed length or score threshold
  int32_t* budget;
  uint32_t* status;
  int32_t* rank;       // [B * gamma] position of each candidate in the admission order
  uint32_t* ticket;    // workgroups finished (returns to 0)
  uint32_t* stop_enc;  // first failing position m as 0x7fffffff - m, 0 if none (returns to 0)
  double* theta;       // [B * gamma + 1] Theta after the first m candidates (best-cut rule)
};

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t s);

// The library-held scratch of dspark_schedule_static: the scheduler's workspace
// layout (header, ranks, Theta) at its largest size, B gamma = 8192.
constexpr size_t kStaticScheduleBytes = 256 + 8192 * 4 + 65792;
// Device address of that scratch on the current device (looked up once per
// device); the first call on a device also enqueues, on `s`, the clearing of
// its header words.
hipError_t static_schedule_scratch(void** ptr, hipStream_t s);
int schedule_groups(const ScheduleArgs& a);        // workgroups of one scheduler launch
size_t schedule_lds_bytes(const ScheduleArgs& a);  // its dynamic LDS

// The draw of position d.pos and the scheduler in one launch (B + schedule_groups
// workgroups).  Returns hipErrorNotSupported, having enqueued nothing, when the
// draw needs the general kernel (more than 4096 tiles).
hipError_t launch_draft_select_schedule(const DraftSelectArgs& d, const ScheduleArgs& s, int logits_dtype,
                                        int factor_dtype, hipStream_t stream);

// W2 [r, V] row-major -> [V, r] row-major (elements of 2 or 4 bytes).
hipError_t launch_pack_w2(const void* w, void* out, int elem_bytes, int V, int r, hipStream_t s);

}  // namespace dspark
