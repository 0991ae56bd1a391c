/*
 * Plain fp64 CPU oracle of one DSpark draft-and-verify round, in C, with host
 * pointers: the ref_ entry points.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline of the benchmark load this library; it shares no code, header or
 * table with the HIP path.  It computes what oracle/dspark.py computes (the
 * same readings of the pages, the same sampler and random-number layout), as
 * straight loops over requests (OpenMP) and vocabulary entries, so that whole
 * batches at the measured sizes finish in seconds.
 *
 * Sources (the pages):
 *   "DSpark, la bozza che sa quando fermarsi" (paithon.it): section "Un po' di
 *     autoregressione basta" (eq. p_k: draft logits U_k plus the Markov bias
 *     B(x_{k-1}, .) = row x_{k-1} of W1 W2, rank 256) and section "Verificare
 *     meglio, non di piu" (prefix survival a_j = prod c_i, Theta = tau SPS(B),
 *     greedy admission that stops when Theta stops growing).
 *   "Les mathematiques derriere l'acceleration ..." (seventnews.com), section
 *     "La garantie de l'echantillonnage par rejet": accept x_k with probability
 *     min(1, p/q), stop at the first rejection, resample from the residual.
 *   "DeepSeek DSpark" (learnblockchain.cn), section "DSpark shi shen me": the
 *     bonus token after a fully accepted block.
 * Readings where the pages are silent (written down in the design notes):
 *   the three-level Gumbel-max sampler (blocks of 4096, tiles of 64), the
 *   Philox4x32-10 counter layout, the uniform map, temperatures below 2^-64
 *   taken as greedy, the residual falling back to p when its mass is zero,
 *   the verify batch counting tokens, the decision margins and their 1e-6 flag.
 *
 * Layouts: base [B, gamma, V], target [B, gamma+1, V] (bf16 as uint16 bits, or
 * fp32), U [V, r] and W [r, V] (W2 as the pages print it), row-major.
 * Every entry point returns 0, or -1 for an argument it rejects.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TILE 64
#define BLOCK (TILE * 64)
#define MARGIN_FLAG 1.0e-6

enum { DRAFT_TOP = 0, DRAFT_MID = 1, DRAFT_LEAF = 2, ACCEPT = 3, FINAL_TOP = 4, FINAL_MID = 5, FINAL_LEAF = 6 };

/* ---------------------------------------------------------------- inputs */

static double elem(const void* p, int dtype, size_t i) {
  if (dtype == 0) {  /* bf16: the upper half of an fp32 bit pattern */
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

static double effective_temperature(float T) {
  double t = (double)T;
  return t >= ldexp(1.0, -64) ? t : 0.0;  /* NaN and negatives compare false: greedy */
}

/* ---------------------------------------------------------------- Philox4x32-10
 * J. K. Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):
 * per round, words 0 and 2 are multiplied by two odd constants; the high
 * halves of the products are xored with words 1 and 3 and the round key, the
 * low halves become the new words 1 and 3; the key advances by two Weyl
 * increments between rounds.  Counter (n div 4, position, request, stream),
 * key (seed mod 2^32, seed div 2^32), draw n is output word n mod 4. */
static uint32_t philox_word(uint64_t seed, uint32_t stream, uint32_t request, uint32_t position, uint32_t n) {
  uint32_t c0 = n >> 2, c1 = position, c2 = request, c3 = stream;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0, c1 = lo1, c2 = n2, c3 = lo0;
  }
  switch (n & 3u) {
    case 0: return c0;
    case 1: return c1;
    case 2: return c2;
    default: return c3;
  }
}

/* u = (floor(w / 2^9) + 1/2) 2^-23, strictly inside (0, 1) */
static double uniform_of(uint32_t w) { return ((double)(w >> 9) + 0.5) * ldexp(1.0, -23); }

static double gumbel_of(double u) { return -log(-log(u)); }

/* ---------------------------------------------------------------- sampler */

static double logsumexp(const double* x, int n) {
  if (n <= 0) return -INFINITY;
  double m = -INFINITY;
  for (int i = 0; i < n; ++i)
    if (x[i] > m) m = x[i];
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += exp(x[i] - m);
  return m + log(s);
}

/* Largest entry (lowest index among equal ones) and its relative margin over
 * the runner-up, the denominator widened by the entries' condition numbers
 * when `cond` is given. */
static int pick(const double* v, const double* cond, int n, double* margin) {
  int i = 0;
  for (int k = 1; k < n; ++k)
    if (v[k] > v[i]) i = k;
  if (n == 1) {
    *margin = INFINITY;
    return i;
  }
  int j = -1;
  for (int k = 0; k < n; ++k)
    if (k != i && (j < 0 || v[k] > v[j])) j = k;
  double v1 = v[i], v2 = v[j];
  if (v2 == -INFINITY) {
    *margin = INFINITY;
    return i;
  }
  double scale = fmax(1.0, fmax(fabs(v1), fabs(v2)));
  if (cond) scale += fmax(cond[i], cond[j]);
  *margin = (v1 - v2) / scale;
  return i;
}

/* Sum of cond_mass over [lo, hi) divided by exp(lam): how much cancellation
 * produced a candidate's mass (0 without cond_mass). */
static double kappa(const double* cond_mass, int lo, int hi, double lam) {
  if (!cond_mass || lam == -INFINITY) return 0.0;
  double s = 0.0;
  for (int v = lo; v < hi; ++v) s += cond_mass[v];
  return s / exp(lam);
}

/* One draw from the distribution proportional to exp(s): block, then tile
 * inside the block, then element inside the tile, each an exact Gumbel-max
 * draw from the conditional distribution of its children. */
static int tree_sample(const double* s, int V, uint64_t seed, const int streams[3], uint32_t request,
                       uint32_t position, const double* cond_mass, double* margin_out) {
  const int nblk = (V + BLOCK - 1) / BLOCK;
  double* blk_lam = (double*)malloc(sizeof(double) * (size_t)nblk);
  double* val = (double*)malloc(sizeof(double) * (size_t)(nblk > TILE ? nblk : TILE));
  double* cond = (double*)malloc(sizeof(double) * (size_t)(nblk > TILE ? nblk : TILE));
  for (int k = 0; k < nblk; ++k) {
    int lo = k * BLOCK, hi = lo + BLOCK < V ? lo + BLOCK : V;
    blk_lam[k] = logsumexp(s + lo, hi - lo);
  }
  double row_lam = logsumexp(blk_lam, nblk);
  for (int k = 0; k < nblk; ++k) {
    val[k] = blk_lam[k] - row_lam + gumbel_of(uniform_of(philox_word(seed, streams[0], request, position, k)));
    int lo = k * BLOCK, hi = lo + BLOCK < V ? lo + BLOCK : V;
    cond[k] = kappa(cond_mass, lo, hi, blk_lam[k]);
  }
  double m_top, m_mid, m_leaf;
  int k = pick(val, cond_mass ? cond : NULL, nblk, &m_top);

  int lo = k * BLOCK, hi = lo + BLOCK < V ? lo + BLOCK : V;
  int nt = (hi - lo + TILE - 1) / TILE;
  double t_lam[TILE];
  for (int t = 0; t < nt; ++t) {
    int a = lo + t * TILE, e = a + TILE < hi ? a + TILE : hi;
    t_lam[t] = logsumexp(s + a, e - a);
    val[t] = t_lam[t] - blk_lam[k] + gumbel_of(uniform_of(philox_word(seed, streams[1], request, position, t)));
    cond[t] = kappa(cond_mass, a, e, t_lam[t]);
  }
  int t = pick(val, cond_mass ? cond : NULL, nt, &m_mid);

  int tl = lo + t * TILE, th = tl + TILE < hi ? tl + TILE : hi;
  for (int e = 0; e < th - tl; ++e) {
    val[e] = s[tl + e] - t_lam[t] + gumbel_of(uniform_of(philox_word(seed, streams[2], request, position, e)));
    if (cond_mass) cond[e] = isfinite(s[tl + e]) ? cond_mass[tl + e] / exp(s[tl + e]) : 0.0;
  }
  int e = pick(val, cond_mass ? cond : NULL, th - tl, &m_leaf);
  free(blk_lam);
  free(val);
  free(cond);
  *margin_out = fmin(m_top, fmin(m_mid, m_leaf));
  return tl + e;
}

static int argmax_first(const double* x, int n) {
  int i = 0;
  for (int k = 1; k < n; ++k)
    if (x[k] > x[i]) i = k;
  return i;
}

/* Draft logits at one position: d_v = base_v + sum_rho U[prev, rho] W[rho, v]. */
static void draft_logits(const void* base_row, int ldt, size_t base_off, const void* U, const void* W, int fdt,
                         int prev, int V, int r, double* d, double* h) {
  for (int rho = 0; rho < r; ++rho) h[rho] = elem(U, fdt, (size_t)prev * r + rho);
  for (int v = 0; v < V; ++v) d[v] = 0.0;
  for (int rho = 0; rho < r; ++rho) {
    const double hr = h[rho];
    for (int v = 0; v < V; ++v) d[v] += hr * elem(W, fdt, (size_t)rho * V + v);
  }
  for (int v = 0; v < V; ++v) d[v] = elem(base_row, ldt, base_off + v) + d[v];
}

/* ---------------------------------------------------------------- entry points */

int ref_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* Draft round: for k = 1..gamma, d = base[b, k-1] + U[x_{k-1}] W; greedy rows
 * take the lowest-index maximum (ln q = 0, lse = max d); others draw x_k from
 * softmax(d / T) with streams 0/1/2 at position k + pos_offset[b]
 * (ln q = s[x] - lse(s), lse = lse(s)).  margin: smallest decision margin. */
int ref_draft_round(const void* base, int logits_dtype, const void* U, const void* W, int factor_dtype,
                    const int32_t* prev0, const float* temperature, uint64_t seed, const int32_t* pos_offset,
                    const int32_t* req_ids, int B, int gamma, int V, int r, int32_t* tokens, double* logq,
                    double* lse, double* margin) {
  if (!base || !U || !W || !prev0 || !temperature || !tokens || !logq || !lse || !margin) return -1;
  if (B < 1 || gamma < 1 || V < 1 || r < 1 || (logits_dtype != 0 && logits_dtype != 1) ||
      (factor_dtype != 0 && factor_dtype != 1))
    return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int b = 0; b < B; ++b) {
    double* d = (double*)malloc(sizeof(double) * (size_t)V);
    double* s = (double*)malloc(sizeof(double) * (size_t)V);
    double* h = (double*)malloc(sizeof(double) * (size_t)r);
    const double T = effective_temperature(temperature[b]);
    const uint32_t rq = (uint32_t)(req_ids ? req_ids[b] : b), off = (uint32_t)(pos_offset ? pos_offset[b] : 0);
    static const int streams[3] = {DRAFT_TOP, DRAFT_MID, DRAFT_LEAF};
    int prev = prev0[b];
    if (prev < 0 || prev >= V) bad = 1, prev = 0;
    for (int k = 1; k <= gamma; ++k) {
      draft_logits(base, logits_dtype, ((size_t)b * gamma + (k - 1)) * V, U, W, factor_dtype, prev, V, r, d, h);
      const size_t o = (size_t)b * gamma + (k - 1);
      int x;
      double m;
      if (T == 0.0) {
        x = argmax_first(d, V);
        for (int v = 0; v < V; ++v) s[v] = d[v] - d[x];
        pick(s, NULL, V, &m);
        logq[o] = 0.0;
        lse[o] = d[x];
      } else {
        for (int v = 0; v < V; ++v) s[v] = d[v] / T;
        const double ls = logsumexp(s, V);
        x = tree_sample(s, V, seed, streams, rq, (uint32_t)k + off, NULL, &m);
        logq[o] = s[x] - ls;
        lse[o] = ls;
      }
      tokens[o] = x;
      margin[o] = m;
      prev = x;
    }
    free(d);
    free(s);
    free(h);
  }
  return bad ? -1 : 0;
}

/* Verification of one drafted block per request: positions 1..L accepted
 * with probability min(1, p/q) (greedy: iff the target argmax), stopping at
 * the first rejection; the final token from the normalised residual
 * max(0, p - q) of the rejected row (p if that has no mass) or, after a fully
 * accepted block, from target row L (streams 4/5/6 at position n + 1 +
 * pos_offset); greedy requests emit the target argmax.  logp/logq_out hold
 * ln p_k(x_k) and ln q_k(x_k) at tested positions (NaN elsewhere); the
 * optional residual_out [B, V] (NULL to skip) the row the final token of a
 * sampled request is drawn from after a rejection (NaN rows elsewhere). */
int ref_verify(const void* target, const void* base, int logits_dtype, const void* U, const void* W,
               int factor_dtype, const int32_t* prev0, const int32_t* draft_tokens, const float* temperature,
               uint64_t seed, const int32_t* budget, const int32_t* pos_offset, const int32_t* req_ids, int B,
               int gamma, int V, int r, int32_t* out_tokens, int32_t* num_accepted, int32_t* num_emitted,
               double* logp_out, double* logq_out, double* margin, int32_t* rows_flagged, double* residual_out) {
  if (!target || !base || !U || !W || !prev0 || !draft_tokens || !temperature || !out_tokens || !num_accepted ||
      !num_emitted || !logp_out || !logq_out || !margin || !rows_flagged)
    return -1;
  if (B < 1 || gamma < 1 || V < 1 || r < 1 || (logits_dtype != 0 && logits_dtype != 1) ||
      (factor_dtype != 0 && factor_dtype != 1))
    return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int b = 0; b < B; ++b) {
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    double* d = (double*)malloc(sizeof(double) * (size_t)V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    double* h = (double*)malloc(sizeof(double) * (size_t)r);
    static const int streams[3] = {FINAL_TOP, FINAL_MID, FINAL_LEAF};
    int L = budget ? budget[b] : gamma;
    if (L < 0 || L > gamma) bad = 1, L = L < 0 ? 0 : gamma;
    const double T = effective_temperature(temperature[b]);
    const uint32_t rq = (uint32_t)(req_ids ? req_ids[b] : b), pos0 = (uint32_t)(pos_offset ? pos_offset[b] : 0);
    int xs[17];
    xs[0] = prev0[b];
    for (int k = 1; k <= gamma; ++k) xs[k] = draft_tokens[(size_t)b * gamma + k - 1];
    for (int k = 0; k <= gamma; ++k)
      if (xs[k] < 0 || xs[k] >= V) bad = 1, xs[k] = 0;
    margin[b] = INFINITY;
    rows_flagged[b] = 0;
    for (int k = 0; k < gamma; ++k) logp_out[(size_t)b * gamma + k] = NAN, logq_out[(size_t)b * gamma + k] = NAN;
    /* optional [B, V] output: the distribution the final token is drawn from
     * after a rejection (the normalised residual, or p where the residual has
     * no mass); NaN on rows that hold no such draw */
    double* const res_row = residual_out ? residual_out + (size_t)b * V : NULL;
    if (res_row)
      for (int v = 0; v < V; ++v) res_row[v] = NAN;
    int n = 0;
    for (int k = 1; k <= L; ++k) {
      for (int v = 0; v < V; ++v) z[v] = elem(target, logits_dtype, ((size_t)b * (gamma + 1) + (k - 1)) * V + v);
      const int x = xs[k];
      int ok;
      if (T == 0.0) {
        ok = x == argmax_first(z, V);
      } else {
        for (int v = 0; v < V; ++v) w[v] = z[v] / T;
        const double lp = z[x] / T - logsumexp(w, V);
        draft_logits(base, logits_dtype, ((size_t)b * gamma + (k - 1)) * V, U, W, factor_dtype, xs[k - 1], V, r, d, h);
        for (int v = 0; v < V; ++v) d[v] = d[v] / T;
        const double lq = d[x] - logsumexp(d, V);
        const double ln_u = log(uniform_of(philox_word(seed, ACCEPT, rq, (uint32_t)k + pos0, 0)));
        ok = ln_u < lp - lq;  /* u < min(1, p/q), since ln u < 0 */
        const double m = fabs(ln_u - (lp - lq)) / fmax(1.0, fmax(fabs(ln_u), fabs(lp) + fabs(lq)));
        if (m < margin[b]) margin[b] = m;
        rows_flagged[b] += m < MARGIN_FLAG;
        logp_out[(size_t)b * gamma + k - 1] = lp;
        logq_out[(size_t)b * gamma + k - 1] = lq;
      }
      if (!ok) break;
      ++n;
    }
    for (int v = 0; v < V; ++v) z[v] = elem(target, logits_dtype, ((size_t)b * (gamma + 1) + n) * V + v);
    int y;
    double m = INFINITY;
    if (T == 0.0) {
      y = argmax_first(z, V);
    } else if (n < L) {
      for (int v = 0; v < V; ++v) w[v] = z[v] / T;
      const double lzp = logsumexp(w, V);
      for (int v = 0; v < V; ++v) p[v] = exp(w[v] - lzp);
      draft_logits(base, logits_dtype, ((size_t)b * gamma + n) * V, U, W, factor_dtype, xs[n], V, r, d, h);
      for (int v = 0; v < V; ++v) d[v] = d[v] / T;
      const double lzq = logsumexp(d, V);
      double mass = 0.0;
      for (int v = 0; v < V; ++v) {
        q[v] = exp(d[v] - lzq);
        const double rv = p[v] - q[v];
        d[v] = rv > 0.0 ? rv : 0.0;  /* the residual */
        mass += d[v];
      }
      if (mass > 0.0) {
        for (int v = 0; v < V; ++v) {
          w[v] = d[v] > 0.0 ? log(d[v]) : -INFINITY;
          q[v] = p[v] + q[v];  /* cancellation scale of each residual entry */
        }
        y = tree_sample(w, V, seed, streams, rq, (uint32_t)(n + 1) + pos0, q, &m);
        if (res_row)
          for (int v = 0; v < V; ++v) res_row[v] = d[v] / mass;
      } else {
        y = tree_sample(w, V, seed, streams, rq, (uint32_t)(n + 1) + pos0, NULL, &m);
        if (res_row)
          for (int v = 0; v < V; ++v) res_row[v] = p[v];
      }
      if (m < margin[b]) margin[b] = m;
      rows_flagged[b] += m < MARGIN_FLAG;
    } else {
      for (int v = 0; v < V; ++v) w[v] = z[v] / T;
      y = tree_sample(w, V, seed, streams, rq, (uint32_t)(n + 1) + pos0, NULL, &m);
      if (m < margin[b]) margin[b] = m;
      rows_flagged[b] += m < MARGIN_FLAG;
    }
    for (int i = 0; i <= gamma; ++i) out_tokens[(size_t)b * (gamma + 1) + i] = -1;
    for (int i = 0; i < n; ++i) out_tokens[(size_t)b * (gamma + 1) + i] = xs[i + 1];
    out_tokens[(size_t)b * (gamma + 1) + n] = y;
    num_accepted[b] = n;
    num_emitted[b] = n + 1;
    free(z);
    free(d);
    free(p);
    free(q);
    free(w);
    free(h);
  }
  return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- scheduler */

/* 1/SPS at a verify batch of N tokens: linear between the table points, the
 * first value below the first point, the last segment extended beyond the
 * last point. */
static double step_time(double N, const double* sB, const double* tt, int n) {
  if (N <= sB[0]) return tt[0];
  int i = 0;
  while (i + 1 < n - 1 && sB[i + 1] <= N) ++i;
  const double frac = (N - sB[i]) / (sB[i + 1] - sB[i]);
  return tt[i] + (tt[i + 1] - tt[i]) * frac;
}

typedef struct {
  int64_t q;
  int b, j;
} Cand;

static int cand_cmp(const void* x, const void* y) {
  const Cand* a = (const Cand*)x;
  const Cand* c = (const Cand*)y;
  if (a->q != c->q) return a->q > c->q ? -1 : 1;  /* larger Q first */
  if (a->b != c->b) return a->b < c->b ? -1 : 1;
  return a->j < c->j ? -1 : (a->j > c->j);
}

/* Budgets from the greedy early-stop prefix scheduler: a_{b,j} = fl32 product
 * of the scores left to right, Q = floor(a 2^32); candidates by decreasing Q
 * (then request, then position); from tau_0 = B 2^32 and N_0 = B, candidate m
 * is admitted iff (tau_m + Q) t(N_m) > tau_m t(N_m + 1), and the first failure
 * ends the scan.  min_gap: smallest relative gap of a comparison made. */
int ref_schedule(const float* conf, const double* sps_B, const double* sps_val, int n_points, int B, int gamma,
                 int32_t* budget, double* min_gap) {
  if (!conf || !sps_B || !sps_val || !budget || n_points < 2 || B < 1 || gamma < 1) return -1;
  for (int i = 0; i + 1 < n_points; ++i)
    if (!(sps_B[i + 1] > sps_B[i])) return -1;
  double* tt = (double*)malloc(sizeof(double) * (size_t)n_points);
  for (int i = 0; i < n_points; ++i) tt[i] = 1.0 / sps_val[i];
  Cand* c = (Cand*)malloc(sizeof(Cand) * (size_t)B * (size_t)gamma);
  int bad = 0;
  for (int b = 0; b < B; ++b) {
    volatile float acc = 1.0f;  /* one fp32 rounding per factor */
    for (int j = 0; j < gamma; ++j) {
      const float cj = conf[(size_t)b * gamma + j];
      if (!(cj > 0.0f && cj < 1.0f)) bad = 1;
      acc = acc * cj;
      Cand* e = &c[(size_t)b * gamma + j];
      e->q = (int64_t)floor((double)acc * 4294967296.0);
      e->b = b, e->j = j;
    }
  }
  if (bad) {
    free(tt);
    free(c);
    return -1;
  }
  qsort(c, (size_t)B * (size_t)gamma, sizeof(Cand), cand_cmp);
  int64_t tau = (int64_t)B << 32;
  int64_t N = B;
  double gap = INFINITY;
  for (int b = 0; b < B; ++b) budget[b] = 0;
  for (size_t m = 0; m < (size_t)B * (size_t)gamma; ++m) {
    const double lhs = (double)(tau + c[m].q) * step_time((double)N, sps_B, tt, n_points);
    const double rhs = (double)tau * step_time((double)(N + 1), sps_B, tt, n_points);
    const double den = fmax(fabs(lhs), fabs(rhs));
    if (den > 0.0 && fabs(lhs - rhs) / den < gap) gap = fabs(lhs - rhs) / den;
    if (!(lhs > rhs)) break;
    tau += c[m].q;
    N += 1;
    budget[c[m].b] = c[m].j + 1;
  }
  if (min_gap) *min_gap = gap;
  free(tt);
  free(c);
  return 0;
}
