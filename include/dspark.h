/*
 * dspark.h -- C ABI of the DSpark draft/verify round on AMD MI355X (gfx950).
 *
 * One round of DSpark speculative decoding over a serving batch of B requests:
 *   dspark_draft_round  semi-autoregressive drafting of a gamma-token block
 *   dspark_schedule     confidence-driven verify budgets (prefix scheduler)
 *   dspark_verify       lossless rejection sampling against the target
 *
 * Sources (the pages):
 *   [P1] "DSpark, la bozza che sa quando fermarsi" (paithon.it), section
 *        "Un po' di autoregressione basta": eq. p_k (backbone logits U_k plus a
 *        prefix-dependent bias B_k), the Markov head B = W1 W2 of rank 256.
 *   [P2] same page, section "Verificare meglio, non di più": eq. a_j = prod c_i,
 *        eq. Theta = tau * SPS(B), greedy admission with an early stop.
 *   [P3] "Les mathématiques derrière l'accélération ..." (seventnews.com),
 *        section "La garantie de l'échantillonnage par rejet": accept with
 *        probability min(1, p/q), stop at the first rejection, resample it from
 *        the residual distribution.
 *   [P4] "DeepSeek发布DSpark" (learnblockchain.cn), section "DSpark 是什么？":
 *        a bonus token after a fully accepted block.
 *   [P5] "DSpark, la bozza ..." (paithon.it), section "Che cosa resta da
 *        verificare", and "DSpark : le pari de DeepSeek ..." (aitalk.it),
 *        section "Vérifier seulement ce qui compte": in production the cut is
 *        estimated from confidences two steps old and the early stop is
 *        removed; scores are recalibrated position by position, left to right
 *        (Sequential Temperature Scaling), keeping their order.
 *
 * Conventions for every call:
 *   - Tensor arguments are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Layouts are dense row-major.
 *   - `workspace` is a device buffer of at least dspark_workspace_bytes(B,
 *     gamma, V, r) bytes (dspark_schedule alone: dspark_schedule_workspace_bytes
 *     (B, gamma)), 256-byte aligned, zero-filled before its first use, owned by
 *     the caller.  Every call that completes leaves the counters it uses at
 *     zero again; after a call that returned DSPARK_EHIP, zero the workspace
 *     before reusing it.  Calls that share a workspace must be ordered on one stream,
 *     with one exception: dspark_schedule touches only its own part of the
 *     workspace and the status word (atomically), so it may run on another
 *     stream concurrently with dspark_draft_round of the same round.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  Every
 *     call only enqueues work on it and returns; nothing synchronises the host
 *     except dspark_status().
 *   - Return value: DSPARK_OK, or a negative error code.  Host-checkable
 *     argument errors return DSPARK_EINVAL before anything is enqueued; a failed
 *     launch returns DSPARK_EHIP.  Data errors found on the device (a token id
 *     outside [0, V), a budget outside [0, gamma], a negative or NaN
 *     temperature, a confidence outside (0, 1), a step-rate table whose batch
 *     sizes are not strictly increasing or whose rates are not positive and
 *     finite) set a bit in the workspace's status word; the offending value is
 *     clamped so that every kernel stays in bounds (with a bad table the budgets
 *     are unspecified), and dspark_status() reports DSPARK_EDATA.  Arguments that
 *     live in device memory (the table included) are checked there, not on the
 *     host, so that no call synchronises.
 *   - Sizes: B >= 1, 1 <= gamma <= 16, V >= 1, r >= 1.
 *   - Randomness: Philox4x32-10 (Salmon et al., SC'11) keyed by `seed`, with
 *     counter (draw index / 4, block position + pos_offset[b], request b,
 *     stream); the same (seed, pos_offset) reproduces a round bit for bit.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_ABI_VERSION 5

enum dspark_status_code {
  DSPARK_OK = 0,
  DSPARK_EINVAL = -1, /* bad argument (checked on the host) */
  DSPARK_EHIP = -2,   /* a HIP runtime call or kernel launch failed */
  DSPARK_EDATA = -3   /* bad input data found on the device (see dspark_status) */
};

enum dspark_dtype {
  DSPARK_BF16 = 0, /* bfloat16 */
  DSPARK_F32 = 1   /* IEEE float32 */
};

/* Layout of the Markov head's second factor W2, an r x V matrix on the pages
 * ([P1]: B = W1 W2).  Every call that reads W2 takes the layout explicitly. */
enum dspark_w_layout {
  DSPARK_W_VOCAB_MAJOR = 0, /* [V, r] row-major: row v holds column v of W2, the
                               r values one vocabulary column contracts over
                               contiguous.  The only layout the round reads. */
  DSPARK_W_RANK_MAJOR = 1   /* [r, V] row-major: W2 as the pages print it.  Not
                               read by the round (DSPARK_EINVAL): pack it once
                               with dspark_pack_w2. */
};

/* Verify-budget rules of dspark_schedule_ex. */
enum dspark_schedule_rule {
  DSPARK_SCHED_EARLY_STOP = 0, /* the greedy prefix scheduler with its early stop ([P2]) */
  DSPARK_SCHED_ARGMAX = 1,     /* the production rule: best cut, no early stop ([P5]) */
  DSPARK_SCHED_FIXED = 2,      /* baseline: every request verifies min(param, gamma) tokens */
  DSPARK_SCHED_THRESHOLD = 3   /* baseline: verify while the score exceeds param */
};

/* Implementations of the draft round (dspark_set_draft_path). */
enum dspark_draft_path {
  DSPARK_DRAFT_PER_POSITION = 0, /* one contraction and one draw launch per position (default) */
  DSPARK_DRAFT_RESIDENT = 1      /* one cooperative launch for the whole round, W2 held on chip,
                                    where it fits (else per position) */
};

/* Version of this ABI (DSPARK_ABI_VERSION of the built library). */
int dspark_abi_version(void);

/* Static text for a return code. */
const char* dspark_error_string(int code);

/* The HIP error behind the calling thread's most recent DSPARK_EHIP return
 * (a hipError_t value; 0 if this thread has had none), and, when `name` is not
 * NULL, its name from the HIP runtime (a static string) in *name.  Each
 * DSPARK_EHIP return overwrites it; other returns leave it as it was. */
int dspark_last_hip_error(const char** name);

/* Bytes of device workspace the three calls need for these sizes (0 if a size
 * is out of range).  One workspace serves draft, schedule and verify. */
size_t dspark_workspace_bytes(int B, int gamma, int V, int r);

/* Bytes of device workspace dspark_schedule needs on its own (0 if a size is
 * out of range: B >= 1, 1 <= gamma <= 16, B * gamma <= 8192); never more than
 * dspark_workspace_bytes for the same B and gamma. */
size_t dspark_schedule_workspace_bytes(int B, int gamma);

/*
 * dspark_pack_w2 -- the Markov head's second factor ([P1], section "Un po' di
 * autoregressione basta": B = W1 W2 with W2 of r rows by V columns) from the
 * pages' [r, V] layout into the vocabulary-major [V, r] layout the round reads
 * (DSPARK_W_VOCAB_MAJOR): W_packed[v, rho] = W[rho, v].  W2 is a static weight,
 * so a caller holding it as [r, V] packs it once and passes W_packed to every
 * round.
 *
 *   W         [r, V] factor_dtype   device, read only
 *   W_packed  [V, r] factor_dtype   device, written; must not overlap W
 * Errors: DSPARK_EINVAL for a NULL pointer, V or r < 1, or an unknown dtype;
 * DSPARK_EHIP for a failed launch.  Only enqueues work on `stream`.
 */
int dspark_pack_w2(const void* W, int factor_dtype, int V, int r, void* W_packed, void* stream);

/* Selects the implementation dspark_draft_round and dspark_draft_schedule use
 * from now on, process-wide (a dspark_draft_path value); returns the previous
 * one, or DSPARK_EINVAL for an unknown value.  Both implementations compute
 * the same draft round ([P1] eq. p_k) with the same arithmetic.  On MI355X the
 * per-position launches are the faster ones at the sizes measured (the
 * resident round's two device-wide waits per position cost more than the
 * kernel boundaries they replace), so they are the default.  The resident
 * round is a cooperative launch; where it does not fit (see dspark_draft_round)
 * or the HIP runtime refuses it (as it does while another process on the GPU
 * holds the device's cooperative-launch resources), the call takes the
 * per-position launches instead, with the same results. */
int dspark_set_draft_path(int path);

/* Bound, in seconds (0 to 60; default 0.2), of each device-wide wait of the
 * resident draft round, for launches enqueued after the call, process-wide.  A
 * wait that passes its bound stops waiting and sets a bit of the workspace
 * status word (dspark_status then returns DSPARK_EDATA): the round's outputs
 * are then unspecified, every memory access stays in bounds and the launch
 * completes, leaving the workspace fit for the next call.  Only a GPU shared
 * with other work that holds CUs for that long stalls the round; a bound of 0
 * forces the stall path.  The previous bound goes to *previous when it is not
 * NULL.  DSPARK_EINVAL for a bound outside [0, 60] or NaN. */
int dspark_set_resident_wait_bound(double seconds, double* previous);

/*
 * dspark_draft_round -- [P1] eq. p_k with the Markov head.
 *
 * For k = 1..gamma, for every request b:
 *   d_k(v) = base_logits[b, k-1, v] + sum_rho U[x_{k-1}, rho] * W[v, rho]
 *   q_k    = softmax(d_k / T_b)   (T_b = temperature[b]; T_b = 0 means argmax)
 *   x_k   ~ q_k                    (x_0 = prev0[b])
 * The Markov bias is computed on the fly and never written to memory.
 *
 *   base_logits  [B, gamma, V]  logits_dtype   backbone logits U_k of [P1]
 *   U            [V, r]         factor_dtype   first factor W1 of [P1]
 *   W            [V, r]         factor_dtype   second factor W2 of [P1] stored
 *                                              vocabulary-major: row v holds
 *                                              column v of W2 (W2 = W^T)
 *   w_layout     DSPARK_W_VOCAB_MAJOR (anything else: DSPARK_EINVAL, nothing
 *                enqueued; a [r, V] W2 is packed with dspark_pack_w2)
 *   prev0        [B] int32      last committed token of each request
 *   temperature  [B] float32    >= 0; 0 = greedy
 *   seed                        Philox key
 *   pos_offset   [B] int32 or NULL (= 0): absolute position of the block, so
 *                                that successive rounds draw fresh numbers
 * Outputs:
 *   draft_tokens [B, gamma] int32   x_1..x_gamma
 *   draft_logq   [B, gamma] float32 ln q_k(x_k) (0 for greedy requests)
 *   draft_lse    [B, gamma] float64 ln sum_v exp(d_k(v) / T_b) (for greedy
 *                                   requests: max_v d_k(v)); kept in fp64 so
 *                                   that dspark_verify can rebuild q_k exactly
 * The round runs as one contraction launch and one draw launch per position.
 * After dspark_set_draft_path(DSPARK_DRAFT_RESIDENT) it runs instead, where it
 * fits (bf16 logits and factors, r = 256, V a multiple of 8 with at most
 * 20 x 64 columns per CU: V <= 163840 on a 256-CU MI355X, B <= 2048), as one
 * cooperative launch that keeps W2 in registers across the gamma positions
 * (every CU takes part).  Both give the same results, bit for bit.
 */
int dspark_draft_round(const void* base_logits, int logits_dtype,
                       const void* U, const void* W, int factor_dtype, int w_layout,
                       const int32_t* prev0, const float* temperature,
                       uint64_t seed, const int32_t* pos_offset,
                       int B, int gamma, int V, int r,
                       int32_t* draft_tokens, float* draft_logq, double* draft_lse,
                       void* workspace, void* stream);

/*
 * dspark_schedule -- [P2] hardware-aware prefix scheduler.
 *
 *   a[b, j] = fl32(a[b, j-1] * conf[b, j]), a[b, -1] = 1      (eq. a_j)
 *   Q[b, j] = floor(a[b, j] * 2^32)
 * Candidates (b, j) are taken in decreasing Q (ties: lower b, then lower j).
 * With tau_0 = B * 2^32, N_0 = B (verify batch in tokens, one per request) and
 * t(N) = 1 / SPS(N) linear between the table points (first value below the
 * first point, last segment extended beyond the last one), candidate m is
 * admitted iff (tau_m + Q_m) * t(N_m) > tau_m * t(N_m + 1) in float64, i.e.
 * iff Theta = tau * SPS(N) strictly grows (eq. Theta); the first failure ends
 * the scan.  budget[b] = number of admitted candidates of request b.
 *
 *   conf     [B, gamma] float32  confidence scores, each in (0, 1)
 *   sps_B    [n_points] float64  batch sizes in tokens, strictly increasing
 *   sps_val  [n_points] float64  steps per second at those sizes, > 0 and finite
 *            (a table that breaks either rule is reported as a data error)
 *   budget   [B] int32 out       verify budgets in [0, gamma]
 * Limits: n_points in [2, 1024], B * gamma <= 8192.  The position of each
 * candidate in the order above is computed directly (the number of candidates
 * before it) rather than by sorting, so every admission test runs in parallel
 * with exactly the stated arithmetic.
 */
int dspark_schedule(const float* conf, const double* sps_B, const double* sps_val,
                    int n_points, int B, int gamma, int32_t* budget,
                    void* workspace, void* stream);

/*
 * dspark_schedule_static -- dspark_schedule that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory: code under HIP
 * stream/graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arithmetic, limits and budgets are exactly those of dspark_schedule.
 *
 *   conf, sps_B, sps_val, n_points, B, gamma, budget: as for dspark_schedule
 *   status   device uint32 or NULL: the data-error bits of this call (scores
 *            outside (0, 1), a bad table) are ORed into it, as into the
 *            workspace's status word (the caller zeroes it); NULL drops them.
 * Scratch: instead of a workspace the call uses one library-held device array
 * of 98816 bytes per GPU (the largest scheduler workspace, B * gamma <= 8192),
 * held until the process ends.  Its counters return to zero at the end of every
 * call.  All calls on one GPU share it: calls that overlap on one GPU (another
 * stream, another host thread) race and must not be made.  The call makes no
 * hipMalloc / hipFree and calls no allocating library routine; the first call
 * on a device looks up the array's address and enqueues one small clearing
 * kernel on `stream`.
 * Errors: DSPARK_EINVAL as for dspark_schedule (B * gamma > 8192 included);
 * DSPARK_EHIP for a failed lookup or launch.
 */
int dspark_schedule_static(const float* conf, const double* sps_B, const double* sps_val, int n_points,
                           int B, int gamma, int32_t* budget, uint32_t* status, void* stream);

/*
 * dspark_schedule_ex -- dspark_schedule with Sequential Temperature Scaling and
 * a choice of rule ([P2], [P5]).
 *
 *   tau      [gamma] float32 or NULL: when given, every score is first
 *            rescaled to c' = 1 / (1 + exp(-z / tau[j])), z = ln c - ln(1 - c),
 *            evaluated in float64 and rounded once to float32 (kept inside
 *            (0, 1)); tau > 0.  The rules below then use c'.
 *   rule     DSPARK_SCHED_EARLY_STOP: exactly dspark_schedule.
 *            DSPARK_SCHED_ARGMAX: candidates in the same order; the number m
 *              admitted maximises Theta_m = tau_m / t(N_m) over m = 0..B*gamma
 *              (tau_m = B 2^32 + the first m values Q, N_m = B + m, one
 *              float64 division), the smallest such m on ties.  The production
 *              scheduler applies this rule to confidence scores two rounds old:
 *              the caller passes those.
 *            DSPARK_SCHED_FIXED: budget[b] = min(max(param, 0), gamma) (MTP-k).
 *            DSPARK_SCHED_THRESHOLD: budget[b] = number of leading positions j
 *              with c'[b, j] > (float)param.
 *   sps_B, sps_val, n_points: as for dspark_schedule; only read by the first
 *            two rules (may be NULL for the others).
 * Workspace: dspark_schedule_workspace_bytes(B, gamma).  Errors: an unknown
 * rule or a NaN param returns DSPARK_EINVAL; a non-positive tau gives NaN or
 * extreme scores that are clamped.
 */
int dspark_schedule_ex(const float* conf, const float* tau, const double* sps_B, const double* sps_val,
                       int n_points, int B, int gamma, int rule, double param, int32_t* budget,
                       void* workspace, void* stream);

/*
 * dspark_draft_schedule -- dspark_draft_round followed by dspark_schedule_ex on
 * the same stream and workspace, in one call ([P1], [P2]).  The scheduler reads
 * only the confidence scores, so it does not depend on the draft: its
 * workgroups run in the same launch as the draw of the last block position
 * (both are bound by memory latency, not bandwidth), when that draw uses the
 * kernel for rows of at most 4096 tiles (V <= 262144); otherwise it is a launch
 * of its own after the draft round.  Outputs, arithmetic and errors are those
 * of the two calls; the arguments are theirs (budget as in dspark_schedule_ex).
 * Workspace: dspark_workspace_bytes(B, gamma, V, r).
 */
int dspark_draft_schedule(const void* base_logits, int logits_dtype, const void* U, const void* W,
                          int factor_dtype, int w_layout, const int32_t* prev0, const float* temperature, uint64_t seed,
                          const int32_t* pos_offset, int B, int gamma, int V, int r, int32_t* draft_tokens,
                          float* draft_logq, double* draft_lse, const float* conf, const float* tau,
                          const double* sps_B, const double* sps_val, int n_points, int rule, double param,
                          int32_t* budget, void* workspace, void* stream);

/*
 * dspark_verify -- [P3] lossless verification with the [P4] bonus token.
 *
 * For request b with budget L = budget[b] (NULL: L = gamma), target row j of
 * target_logits predicts block position j+1.  For k = 1..L:
 *   p_k = softmax(target_logits[b, k-1] / T_b)
 *   accept x_k iff u < min(1, p_k(x_k) / q_k(x_k)), u = uniform draw;
 * the first rejection at position n+1 draws its replacement from
 *   max(0, p_{n+1} - q_{n+1}) normalised (p_{n+1} if that has no mass),
 * with q_{n+1} rebuilt from base_logits, U, W and draft_lse; if all L are
 * accepted a bonus token is drawn from p_{L+1}.  Greedy requests (T_b = 0)
 * accept x_k iff it is the target argmax (lowest index on ties) and emit the
 * target argmax.
 *
 *   target_logits [B, gamma+1, V] logits_dtype
 *   base_logits, U, W, w_layout, prev0, temperature, seed, pos_offset: as
 *                 given to dspark_draft_round for the same round
 *   draft_tokens, draft_logq, draft_lse: its outputs
 *   budget       [B] int32 or NULL
 * Outputs:
 *   out_tokens   [B, gamma+1] int32: x_1..x_n, final token, then -1
 *   num_accepted [B] int32 n;  num_emitted [B] int32 n + 1
 *   debug_logp_logq [B, gamma, 2] float32 or NULL: (ln p_k(x_k), ln q_k(x_k))
 *                 at the positions k = 1..min(n + 1, L) whose test ran, for
 *                 sampled requests (untouched elsewhere)
 *   debug_residual  [B, V] float32 or NULL: the normalised residual row of
 *                 requests that rejected (untouched elsewhere)
 */
int dspark_verify(const void* target_logits, const void* base_logits, int logits_dtype,
                  const void* U, const void* W, int factor_dtype, int w_layout,
                  const int32_t* prev0, const int32_t* draft_tokens,
                  const float* draft_logq, const double* draft_lse,
                  const int32_t* budget, const float* temperature,
                  uint64_t seed, const int32_t* pos_offset,
                  int B, int gamma, int V, int r,
                  int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
                  float* debug_logp_logq, float* debug_residual,
                  void* workspace, void* stream);

/*
 * dspark_acceptance -- the analytic acceptance rate of every drafted position
 * ("DSpark, la bozza ...", section "Verificare meglio, non di più", eq. c*_k:
 * one minus the total-variation distance between the draft and target
 * distributions, the label the confidence head is trained on).
 *
 *   c_star[b, k-1] = sum_v min(p_k(v), q_k(v)),   k = 1..gamma
 * with p_k = softmax(target_logits[b, k-1] / T_b) and q_k the draft
 * distribution of position k rebuilt from base_logits, U, W and the drafted
 * prefix (x_0 = prev0[b], x_j = draft_tokens[b, j-1]) and normalised by
 * draft_lse[b, k-1] -- i.e. the probability that the accept test of position k
 * passes given that x_1..x_{k-1} were accepted.  Greedy requests (T_b = 0):
 * 1 if draft_tokens[b, k-1] is the target row's lowest-index maximum, else 0.
 *
 *   target_logits [B, gamma+1, V], base_logits [B, gamma, V], U, W, w_layout,
 *   prev0, temperature: as for dspark_verify; draft_tokens, draft_lse: the outputs of
 *   dspark_draft_round for the same inputs.
 *   c_star        [B, gamma] float64 out.
 * Reads every target and backbone row once plus W2 per group of 128 positions;
 * tile masses are fp32, their sum fp64.  Shares the workspace of the other
 * calls (ordered on one stream: it empties the residual work list).
 */
int dspark_acceptance(const void* target_logits, const void* base_logits, int logits_dtype,
                      const void* U, const void* W, int factor_dtype, int w_layout,
                      const int32_t* prev0, const int32_t* draft_tokens, const double* draft_lse,
                      const float* temperature, int B, int gamma, int V, int r,
                      double* c_star, void* workspace, void* stream);

/* Synchronises `stream`, returns DSPARK_EDATA if any call on this workspace
 * found bad data since the last dspark_status() (and clears the word), else
 * DSPARK_OK; DSPARK_EHIP if the stream reports an error. */
int dspark_status(void* workspace, void* stream);

/* Timing of individual kernels (measurement support).  While enabled, every
 * `enabled`-th launch of the kernel class `kernel_class` (the first, then every
 * enabled-th after it; 0 turns timing off) carries a pair of HIP events in its
 * dispatch (hipExtLaunchKernel), which take the kernel's own start and end
 * times on the caller's stream.  A timed launch costs a few microseconds of
 * extra dispatch time, so a sample keeps that out of a timed region.  dspark_profile_read() waits for the recorded
 * events and returns the number of timed launches and their summed duration in
 * ms, then clears the record.  Classes: 0 draft GEMM + softmax statistics, 1 draft
 * sample, 2 verification pass (target row statistics up to the first
 * rejection, accept tests, bonus and greedy tokens), 3 unused, 4 residual
 * statistics, 5 residual sample, 6 scheduler, 7 acceptance-pass GEMM, 8 the
 * resident draft round (a cooperative launch: its events are recorded on the
 * stream around the launch, so they include its dispatch). */
int dspark_profile_enable(int kernel_class, int enabled);
int dspark_profile_read(int kernel_class, int* launches, double* total_ms);

/* Reference rates of the device (measurement support, not part of a round:
 * the roofline of the kernels above is also reported against these).  Both
 * only enqueue one kernel on `stream`; the caller times it.  `sink` is a
 * device uint32 that is written only in a case that does not occur (it keeps
 * the work from being optimised away).
 *   dspark_peak_stream_read: reads the `bytes` (a positive multiple of 16)
 *     of the device buffer `buf` once: every wavefront one contiguous 8 KB
 *     chunk, its eight 16-byte streaming loads per lane all in flight.
 *   dspark_peak_mfma_bf16: `blocks` workgroups of 4 wavefronts, each running
 *     `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16 chains:
 *     blocks * 4 * iters * 4 * 32768 flops.
 * Errors: DSPARK_EINVAL for a NULL pointer or a size out of range. */
int dspark_peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int dspark_peak_mfma_bf16(int blocks, int iters, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
