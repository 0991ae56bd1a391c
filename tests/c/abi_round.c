/*
 * One DSpark draft-and-verify round called from C through the library's ABI
 * (include/dspark.h), with device buffers from the HIP runtime's C API: the
 * boundary used the way a C or C++ serving engine would use it, with no Python
 * and no PyTorch in the process.
 *
 * Inputs come from a counter-based integer hash (lowbias32) so that a second
 * implementation (tests/test_gpu_c_abi.py, numpy) regenerates them bit for bit:
 *   target [B, GAMMA + 1, V] bf16   sign (1 + m / 128) 2^e, e in [-2, 1]
 *   base   [B, GAMMA, V]     bf16   the target row of the same position with the
 *                                   two lowest mantissa bits flipped by the hash
 *   U, W   [V, R]            bf16   e in [-7, -4]  (W vocabulary-major)
 *   prev0, temperature, confidence scores, a 4-point step-rate table.
 * The round: dspark_draft_schedule (early-stop rule), then dspark_verify.
 *
 * Usage: abi_round OUTPUT_FILE
 * Writes draft tokens, draft ln q, draft ln-sum-exp, budgets, emitted tokens,
 * accepted and emitted counts, in that order, as raw little-endian arrays;
 * returns 0, or 1 with a message on any error.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dspark.h"

enum { B = 64, GAMMA = 4, V = 12392, R = 128, NPTS = 4 };
static const uint64_t SEED = 12345;

static uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

/* element i of the stream `salt` */
static uint32_t hash_at(uint32_t salt, uint32_t i) { return mix(i * 0x9E3779B9U + salt); }

static uint16_t bf16_from(uint32_t h, int e0) {
  const uint32_t s = h >> 31, m = h & 127u, e = (uint32_t)(e0 + 127) + ((h >> 7) & 3u);
  return (uint16_t)((s << 15) | (e << 7) | m);
}

static int fail(const char* what, int code) {
  fprintf(stderr, "abi_round: %s failed (%d)\n", what, code);
  return 1;
}

#define HIP_OK(call)                                            \
  do {                                                          \
    hipError_t e_ = (call);                                     \
    if (e_ != hipSuccess) return fail(#call, (int)e_);          \
  } while (0)

static int to_device(void** dev, const void* host, size_t bytes) {
  if (hipMalloc(dev, bytes) != hipSuccess) return -1;
  return hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) == hipSuccess ? 0 : -1;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: abi_round OUTPUT_FILE\n");
    return 1;
  }
  if (dspark_abi_version() != DSPARK_ABI_VERSION) return fail("dspark_abi_version", dspark_abi_version());

  const size_t n_tgt = (size_t)B * (GAMMA + 1) * V, n_base = (size_t)B * GAMMA * V, n_fac = (size_t)V * R;
  uint16_t* target = malloc(n_tgt * 2);
  uint16_t* base = malloc(n_base * 2);
  uint16_t* U = malloc(n_fac * 2);
  uint16_t* W = malloc(n_fac * 2);
  if (!target || !base || !U || !W) return fail("malloc", 0);
  for (size_t i = 0; i < n_tgt; ++i) target[i] = bf16_from(hash_at(1u, (uint32_t)i), -2);
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < GAMMA; ++j)
      for (int v = 0; v < V; ++v) {
        const size_t ib = ((size_t)b * GAMMA + j) * V + v, it = ((size_t)b * (GAMMA + 1) + j) * V + v;
        base[ib] = (uint16_t)(target[it] ^ (hash_at(2u, (uint32_t)ib) & 3u));
      }
  for (size_t i = 0; i < n_fac; ++i) U[i] = bf16_from(hash_at(3u, (uint32_t)i), -7);
  for (size_t i = 0; i < n_fac; ++i) W[i] = bf16_from(hash_at(4u, (uint32_t)i), -7);
  int32_t prev0[B];
  float temperature[B], conf[B * GAMMA];
  for (int b = 0; b < B; ++b) {
    prev0[b] = (int32_t)(hash_at(5u, (uint32_t)b) % (uint32_t)V);
    temperature[b] = b % 4 == 3 ? 0.0f : (b % 2 ? 0.7f : 1.0f);
  }
  for (int i = 0; i < B * GAMMA; ++i) conf[i] = (float)(1u + hash_at(6u, (uint32_t)i) % 998u) / 1000.0f;
  const double sps_B[NPTS] = {1.0, 8.0, 64.0, 512.0};
  double sps_val[NPTS];
  for (int i = 0; i < NPTS; ++i) sps_val[i] = 1e6 / (20000.0 + 5.0 * sps_B[i]);

  void *d_target, *d_base, *d_U, *d_W, *d_prev0, *d_T, *d_conf, *d_sB, *d_sV;
  if (to_device(&d_target, target, n_tgt * 2) || to_device(&d_base, base, n_base * 2) ||
      to_device(&d_U, U, n_fac * 2) || to_device(&d_W, W, n_fac * 2) || to_device(&d_prev0, prev0, sizeof prev0) ||
      to_device(&d_T, temperature, sizeof temperature) || to_device(&d_conf, conf, sizeof conf) ||
      to_device(&d_sB, sps_B, sizeof sps_B) || to_device(&d_sV, sps_val, sizeof sps_val))
    return fail("device inputs", 0);

  const size_t ws_bytes = dspark_workspace_bytes(B, GAMMA, V, R);
  if (ws_bytes == 0) return fail("dspark_workspace_bytes", 0);
  void *ws, *d_draft, *d_logq, *d_lse, *d_budget, *d_out, *d_nacc, *d_nem;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemset(ws, 0, ws_bytes));  /* zero-filled before its first use */
  HIP_OK(hipMalloc(&d_draft, B * GAMMA * 4));
  HIP_OK(hipMalloc(&d_logq, B * GAMMA * 4));
  HIP_OK(hipMalloc(&d_lse, B * GAMMA * 8));
  HIP_OK(hipMalloc(&d_budget, B * 4));
  HIP_OK(hipMalloc(&d_out, B * (GAMMA + 1) * 4));
  HIP_OK(hipMalloc(&d_nacc, B * 4));
  HIP_OK(hipMalloc(&d_nem, B * 4));

  int rc = dspark_draft_schedule(d_base, DSPARK_BF16, d_U, d_W, DSPARK_BF16, DSPARK_W_VOCAB_MAJOR, d_prev0, d_T, SEED,
                                 NULL, B, GAMMA, V, R, d_draft, d_logq, d_lse, d_conf, NULL, d_sB, d_sV, NPTS,
                                 DSPARK_SCHED_EARLY_STOP, 0.0, d_budget, ws, NULL);
  if (rc != DSPARK_OK) return fail("dspark_draft_schedule", rc);
  rc = dspark_verify(d_target, d_base, DSPARK_BF16, d_U, d_W, DSPARK_BF16, DSPARK_W_VOCAB_MAJOR, d_prev0, d_draft,
                     d_logq, d_lse, d_budget, d_T, SEED, NULL, B, GAMMA, V, R, d_out, d_nacc, d_nem, NULL, NULL, ws,
                     NULL);
  if (rc != DSPARK_OK) return fail("dspark_verify", rc);
  rc = dspark_status(ws, NULL);  /* synchronises the stream */
  if (rc != DSPARK_OK) return fail("dspark_status", rc);

  int32_t draft[B * GAMMA], budget[B], out[B * (GAMMA + 1)], nacc[B], nem[B];
  float logq[B * GAMMA];
  double lse[B * GAMMA];
  HIP_OK(hipMemcpy(draft, d_draft, sizeof draft, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(logq, d_logq, sizeof logq, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, d_lse, sizeof lse, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(budget, d_budget, sizeof budget, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(nacc, d_nacc, sizeof nacc, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(nem, d_nem, sizeof nem, hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) return fail("fopen", 0);
  fwrite(draft, sizeof draft, 1, f);
  fwrite(logq, sizeof logq, 1, f);
  fwrite(lse, sizeof lse, 1, f);
  fwrite(budget, sizeof budget, 1, f);
  fwrite(out, sizeof out, 1, f);
  fwrite(nacc, sizeof nacc, 1, f);
  fwrite(nem, sizeof nem, 1, f);
  if (fclose(f) != 0) return fail("fclose", 0);

  long verified = 0, accepted = 0;
  for (int b = 0; b < B; ++b) verified += budget[b], accepted += nacc[b];
  printf("abi_round ok: B=%d gamma=%d V=%d r=%d, %ld positions verified, %ld accepted\n", B, GAMMA, V, R, verified,
         accepted);

  hipFree(ws);
  hipFree(d_draft), hipFree(d_logq), hipFree(d_lse), hipFree(d_budget), hipFree(d_out), hipFree(d_nacc), hipFree(d_nem);
  hipFree(d_target), hipFree(d_base), hipFree(d_U), hipFree(d_W), hipFree(d_prev0), hipFree(d_T), hipFree(d_conf);
  hipFree(d_sB), hipFree(d_sV);
  free(target), free(base), free(U), free(W);
  return 0;
}
