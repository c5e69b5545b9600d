/*
 * spec_oracle.c -- plain, slow, float64 CPU oracle of the speculative-decoding
 * verify / accept / resample step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header
 * or constant table with the HIP implementation; the two meet only through
 * the seeded inputs.
 *
 * What it follows (pages: "Decodificación Especulativa y EAGLE", lesson 25 of
 * ai-engineering.academy, and Perplexity's "Accelerating Sonar through
 * speculation"):
 *   - section "La Regla de Exactitud": for each drafted x_t draw r ~ U(0,1);
 *     accept iff r < p(x_t)/q(x_t); otherwise draw the replacement from the
 *     normalised positive part (p - q)+ and stop;
 *   - section "El Concepto", steps 3-4: scan left to right, keep the longest
 *     accepted prefix; if every draft is accepted draw a bonus token from the
 *     target row after the last draft;
 *   - section "La Regla de Exactitud", greedy case: at temperature 0 accept iff
 *     argmax(p) == x_t, else emit argmax(p) and stop;
 *   - the listing in section "Desarrolla": the same temperature divides the
 *     target and the draft logits before the softmax.
 * Readings taken where the pages are silent (see the design notes):
 *   - accept test in product form r*q < p (strict), so q = 0 < p accepts;
 *   - the residual is the pointwise vector (p - q)+, not p minus the scalar
 *     q(x_t) (the listing subtracts the scalar; the rule's formula does not);
 *   - argmax ties go to the lowest index; NaN entries never win a greedy row;
 *   - sampling is an exponential race: winner = argmax_v (ln w_v - ln E_v)
 *     with E_v = -ln U_v, U_v from Philox4x32-10 keyed by the seed and
 *     counter (v >> 2, position, request, 0), word v & 3; the accept uniform
 *     r_t is word 0 of counter (0, t, request, 1).  w_v is a probability:
 *     (p - q)+ after a rejection, p itself for the bonus (z_v / T - lse), so
 *     the race keys and the near-tie window below do not move when a
 *     constant is added to a row's logits;
 *   - U(x) = (2*(x >> 9) + 1) * 2^-24, an exact value in (0, 1).
 *
 * It also holds the draft-side sampler that precedes verification
 * (oracle_draft_sample, at the end of this file): one token per request from
 * softmax(z / T) by the same kind of race on its own Philox stream (tag 2),
 * or the argmax at T = 0; the commit step that follows it
 * (oracle_commit_tokens): the emitted tokens appended to each request's
 * token history on the device; and greedy verification of a draft tree
 * (oracle_tree_verify_greedy): the longest root-to-node path whose every
 * token is the argmax of its parent's target row.
 *
 * Philox4x32-10 is written from its published definition (Salmon, Moraes,
 * Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): ten
 * rounds of two 32x32->64 multiplies, with a Weyl-sequence key schedule.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2 /* test-only input type: exact float64 logits */

/* flags written per request */
#define OR_FLAG_ACCEPT_NEAR_TIE 1u  /* some evaluated |r*q - p| < 1e-6 * max(p, r*q) */
#define OR_FLAG_RACE_NEAR_TIE 2u    /* best - second < 1e-6 * max(1, |best|), keys ln w - ln E */
#define OR_FLAG_RESIDUAL_EMPTY 4u   /* no token had p > q; raced on p instead */

/* ---------------------------------------------------------------- Philox */

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u; /* round multipliers */
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u; /* key increments */
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* U(x) = (2*(x>>9) + 1) / 2^24: 2^23 equally spaced points strictly in (0,1). */
double oracle_u01(uint32_t x) {
  return (2.0 * (double)(x >> 9) + 1.0) / 16777216.0;
}

static uint32_t philox_word(uint64_t seed, uint32_t c0, uint32_t c1, uint32_t c2,
                            uint32_t c3, int word) {
  uint32_t ctr[4] = {c0, c1, c2, c3};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  return out[word];
}

/* Accept uniform r_t for request b, draft position t. */
double oracle_accept_uniform(uint64_t seed, int32_t b, int32_t t) {
  return oracle_u01(philox_word(seed, 0u, (uint32_t)t, (uint32_t)b, 1u, 0));
}

/* Exponential variate E_v = -ln U_v of the race at (request b, position pos). */
double oracle_race_exponential(uint64_t seed, int32_t b, int32_t pos, int32_t v) {
  uint32_t x = philox_word(seed, (uint32_t)v >> 2, (uint32_t)pos, (uint32_t)b, 0u, v & 3);
  return -log(oracle_u01(x));
}

/* Exponential variate of the draft-side sampler at (request b, draft step). */
double oracle_draft_exponential(uint64_t seed, int32_t b, int32_t step, int32_t v) {
  uint32_t x = philox_word(seed, (uint32_t)v >> 2, (uint32_t)step, (uint32_t)b, 2u, v & 3);
  return -log(oracle_u01(x));
}

/* ---------------------------------------------------------------- inputs */

static double logit(const void* base, int dtype, int64_t row, int32_t V, int32_t v) {
  int64_t i = row * (int64_t)V + v;
  if (dtype == OR_F32) return (double)((const float*)base)[i];
  if (dtype == OR_F64) return ((const double*)base)[i];
  /* bf16: the stored 16 bits are the top half of a float32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Largest non-NaN value of a row (-inf if none). */
static double row_max(const void* base, int dtype, int64_t row, int32_t V) {
  double m = -INFINITY;
  for (int32_t v = 0; v < V; ++v) {
    double z = logit(base, dtype, row, V, v);
    if (z > m) m = z;
  }
  return m;
}

/* Greedy argmax: lowest index attaining the maximum; -1 if no finite maximum. */
static int32_t row_argmax(const void* base, int dtype, int64_t row, int32_t V) {
  double m = -INFINITY;
  int32_t idx = -1;
  for (int32_t v = 0; v < V; ++v) {
    double z = logit(base, dtype, row, V, v);
    if (z > m) {
      m = z;
      idx = v;
    }
  }
  if (!isfinite(m)) return -1;
  return idx;
}

/* log-sum-exp of row/T, max-shifted; NaN/inf results signal a bad row. */
static double row_lse(const void* base, int dtype, int64_t row, int32_t V, double T) {
  double m = row_max(base, dtype, row, V);
  if (!isfinite(m)) return NAN;
  double s = 0.0;
  for (int32_t v = 0; v < V; ++v) s += exp(logit(base, dtype, row, V, v) / T - m / T);
  return m / T + log(s);
}

/* ---------------------------------------------------------------- one request */

typedef struct {
  int dtype;
  const void* target;
  const void* draft;
  int32_t B, V, max_k, n_draft_rows;
  const int32_t* offsets;
  const int32_t* tokens;
  const float* temperature;
  uint64_t seed;
} oracle_inputs;

typedef struct {
  int32_t* accept_len;   /* [B] */
  int32_t* out_tokens;   /* [n_draft_rows + B] */
  double* p_at;          /* [n_draft_rows] or NULL */
  double* q_at;          /* [n_draft_rows] or NULL */
  uint32_t* flags;       /* [B] or NULL */
  double* race_best;     /* [B] or NULL: winning race key (oracle scale) */
  double* race_gap;      /* [B] or NULL: best - second-best race key */
} oracle_outputs;

static void fail_request(const oracle_inputs* in, const oracle_outputs* o, int32_t b,
                         int offsets_ok) {
  o->accept_len[b] = -1;
  if (!offsets_ok) return;
  int32_t k = in->offsets[b + 1] - in->offsets[b];
  for (int32_t i = 0; i <= k; ++i) o->out_tokens[in->offsets[b] + b + i] = -1;
  for (int32_t t = 0; t < k; ++t) {
    if (o->p_at) o->p_at[in->offsets[b] + t] = NAN;
    if (o->q_at) o->q_at[in->offsets[b] + t] = NAN;
  }
}

void oracle_verify_one(const oracle_inputs* in, const oracle_outputs* o, int32_t b) {
  const int32_t V = in->V;
  if (o->flags) o->flags[b] = 0;
  if (o->race_best) o->race_best[b] = NAN;
  if (o->race_gap) o->race_gap[b] = NAN;

  /* validate the request's slice of the packed layout */
  int32_t off = in->offsets[b], off1 = in->offsets[b + 1];
  int offsets_ok = off >= 0 && off1 <= in->n_draft_rows && off1 - off >= 0 &&
                   off1 - off <= in->max_k;
  if (!offsets_ok) {
    fail_request(in, o, b, 0);
    return;
  }
  const int32_t K = off1 - off;
  const int64_t trow0 = (int64_t)off + b; /* target row t of b is trow0 + t */
  const int64_t drow0 = off;              /* draft row t of b is drow0 + t */
  const double T = (double)in->temperature[b];
  if (!isfinite(T) || T < 0.0 || (T > 0.0 && K > 0 && in->draft == NULL)) {
    fail_request(in, o, b, 1);
    return;
  }
  for (int32_t t = 0; t < K; ++t) {
    int32_t x = in->tokens[off + t];
    if (x < 0 || x >= V) {
      fail_request(in, o, b, 1);
      return;
    }
  }

  int32_t n, y;
  if (T == 0.0) {
    /* greedy rule: accept x_t iff argmax(p_t) == x_t; emit argmax at the stop */
    int32_t g[64];
    for (int32_t t = 0; t <= K; ++t) {
      g[t] = row_argmax(in->target, in->dtype, trow0 + t, V);
      if (g[t] < 0) {
        fail_request(in, o, b, 1);
        return;
      }
    }
    n = K;
    for (int32_t t = 0; t < K; ++t) {
      if (g[t] != in->tokens[off + t]) {
        n = t;
        break;
      }
    }
    y = g[n];
    for (int32_t t = 0; t < K; ++t) {
      if (o->p_at) o->p_at[off + t] = NAN;
      if (o->q_at) o->q_at[off + t] = NAN;
    }
  } else {
    /* sampled: p_t = softmax(P_t / T), q_t = softmax(Q_t / T) */
    double lp[64], lq[64];
    for (int32_t t = 0; t <= K; ++t) {
      lp[t] = row_lse(in->target, in->dtype, trow0 + t, V, T);
      if (!isfinite(lp[t])) {
        fail_request(in, o, b, 1);
        return;
      }
    }
    for (int32_t t = 0; t < K; ++t) {
      lq[t] = row_lse(in->draft, in->dtype, drow0 + t, V, T);
      if (!isfinite(lq[t])) {
        fail_request(in, o, b, 1);
        return;
      }
    }
    /* left-to-right ratio test; every position's p/q is reported */
    n = K;
    for (int32_t t = 0; t < K; ++t) {
      int32_t x = in->tokens[off + t];
      double p = exp(logit(in->target, in->dtype, trow0 + t, V, x) / T - lp[t]);
      double q = exp(logit(in->draft, in->dtype, drow0 + t, V, x) / T - lq[t]);
      if (o->p_at) o->p_at[off + t] = p;
      if (o->q_at) o->q_at[off + t] = q;
      if (n < K) continue; /* already stopped: later positions are not tested */
      double r = oracle_accept_uniform(in->seed, b, t);
      /* relative: two tiny probabilities are not a near-tie by themselves */
      if (fabs(r * q - p) < 1e-6 * fmax(p, r * q) && o->flags)
        o->flags[b] |= OR_FLAG_ACCEPT_NEAR_TIE;
      if (!(r * q < p)) n = t;
    }

    /* race: residual (p_n - q_n)+ after a rejection, else bonus from p_K */
    int residual = n < K;
    int any_positive = 0;
    if (residual) {
      for (int32_t v = 0; v < V && !any_positive; ++v) {
        double p = exp(logit(in->target, in->dtype, trow0 + n, V, v) / T - lp[n]);
        double q = exp(logit(in->draft, in->dtype, drow0 + n, V, v) / T - lq[n]);
        if (p - q > 0.0) any_positive = 1;
      }
      if (!any_positive && o->flags) o->flags[b] |= OR_FLAG_RESIDUAL_EMPTY;
    }
    double best = -INFINITY, second = -INFINITY;
    y = -1;
    for (int32_t v = 0; v < V; ++v) {
      double key;
      double e = oracle_race_exponential(in->seed, b, n, v);
      if (residual && any_positive) {
        double p = exp(logit(in->target, in->dtype, trow0 + n, V, v) / T - lp[n]);
        double q = exp(logit(in->draft, in->dtype, drow0 + n, V, v) / T - lq[n]);
        double w = p - q;
        if (!(w > 0.0)) continue;
        key = log(w) - log(e);
      } else {
        key = logit(in->target, in->dtype, trow0 + n, V, v) / T - lp[n] - log(e);
      }
      if (key > best) {
        second = best;
        best = key;
        y = v;
      } else if (key > second) {
        second = key;
      }
    }
    if (o->race_best) o->race_best[b] = best;
    if (o->race_gap) o->race_gap[b] = best - second;
    if (best - second < 1e-6 * fmax(1.0, fabs(best)) && o->flags)
      o->flags[b] |= OR_FLAG_RACE_NEAR_TIE;
  }

  o->accept_len[b] = n;
  for (int32_t i = 0; i < n; ++i) o->out_tokens[trow0 + i] = in->tokens[off + i];
  o->out_tokens[trow0 + n] = y;
  for (int32_t i = n + 1; i <= K; ++i) o->out_tokens[trow0 + i] = -1;
}

/*
 * Batch entry: evaluates the requests listed in `reqs` (all B when reqs is
 * NULL), each with its own request index b (the Philox counter uses b).
 * Output arrays are laid out for the whole batch; entries of requests not
 * evaluated are left untouched.  Returns 0, or -1 on a bad argument.
 */
int oracle_spec_verify(int dtype, const void* target, const void* draft, int32_t B, int32_t V,
                       int32_t max_k, int32_t n_draft_rows, const int32_t* offsets,
                       const int32_t* tokens, const float* temperature, uint64_t seed,
                       const int32_t* reqs, int32_t n_reqs, int32_t* accept_len,
                       int32_t* out_tokens, double* p_at, double* q_at, uint32_t* flags,
                       double* race_best, double* race_gap) {
  if (!target || !offsets || !temperature || !accept_len || !out_tokens) return -1;
  if (B < 1 || V < 1 || max_k < 0 || max_k > 63) return -1;
  if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F64) return -1;
  oracle_inputs in = {dtype, target, draft, B, V, max_k, n_draft_rows, offsets, tokens,
                      temperature, seed};
  oracle_outputs o = {accept_len, out_tokens, p_at, q_at, flags, race_best, race_gap};
  if (reqs) {
    for (int32_t i = 0; i < n_reqs; ++i) {
      if (reqs[i] < 0 || reqs[i] >= B) return -1;
      oracle_verify_one(&in, &o, reqs[i]);
    }
  } else {
    for (int32_t b = 0; b < B; ++b) oracle_verify_one(&in, &o, b);
  }
  return 0;
}

/*
 * Draft-side sampler: the drafting step that precedes verification.  The
 * lesson's concept (section "El Concepto", step 1) and its listing draw each
 * draft token from softmax(q / T); Perplexity's draft-target scheme takes the
 * top token at every draft step (greedy drafting, T = 0).  Row b of `logits`
 * is the draft model's output for request b at draft step `step`.
 *   T == 0: x = lowest index attaining the row maximum;
 *   T > 0:  x = argmax_v (ln q_v - ln E_v) with E_v = -ln U_v, U_v from
 *           Philox4x32-10 keyed by the seed, counter (v >> 2, step, b, 2),
 *           word v & 3 (stream tag 2, apart from the verify step's tags 0
 *           and 1); ties to the lowest index.  An exponential race, so x is
 *           an exact draw from softmax(z / T).
 * q_at[b] = exp(z_x / T - lse(z / T)) for T > 0 (NaN when T == 0).  A near
 * tie (best - second < 1e-6 * max(1, |best|)) sets flags[b] bit 2.  A bad
 * temperature (negative, NaN, infinite) or a row with no finite maximum
 * gives x = -1.  Returns 0, or -1 on a bad argument.
 */
int oracle_draft_sample(int dtype, const void* logits, int32_t B, int32_t V,
                        const float* temperature, uint64_t seed, int32_t step, int32_t* tokens,
                        double* q_at, uint32_t* flags, double* race_gap) {
  if (!logits || !temperature || !tokens || B < 1 || V < 1) return -1;
  if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F64) return -1;
  for (int32_t b = 0; b < B; ++b) {
    const double T = (double)temperature[b];
    if (flags) flags[b] = 0;
    if (q_at) q_at[b] = NAN;
    if (race_gap) race_gap[b] = NAN;
    tokens[b] = -1;
    if (!isfinite(T) || T < 0.0) continue;
    if (T == 0.0) {
      tokens[b] = row_argmax(logits, dtype, b, V);
      continue;
    }
    const double lse = row_lse(logits, dtype, b, V, T);
    if (!isfinite(lse)) continue;
    double best = -INFINITY, second = -INFINITY;
    int32_t x = -1;
    for (int32_t v = 0; v < V; ++v) {
      double key =
          logit(logits, dtype, b, V, v) / T - lse - log(oracle_draft_exponential(seed, b, step, v));
      if (key > best) {
        second = best;
        best = key;
        x = v;
      } else if (key > second) {
        second = key;
      }
    }
    tokens[b] = x;
    if (x >= 0 && q_at) q_at[b] = exp(logit(logits, dtype, b, V, x) / T - lse);
    if (race_gap) race_gap[b] = best - second;
    if (best - second < 1e-6 * fmax(1.0, fabs(best)) && flags) flags[b] |= OR_FLAG_RACE_NEAR_TIE;
  }
  return 0;
}

/*
 * Commit step after verification (Perplexity's page, section on MTP
 * scheduling: once the verify step has decided, a kernel writes the
 * accepted tokens into their places on the device, so the host never waits
 * for the outcome).  For request b with n = accept_len[b] and history row
 * seq_tokens[b * seq_stride .. + capacity), length L = seq_len[b]:
 *   - a failed verify (n < 0), n > K_b, or a slice outside the packed
 *     layout (offsets as in the verify step, K_b <= max_k): status -1;
 *   - L < 0 or L + n + 1 > capacity: status -2;
 *   - otherwise the n + 1 emitted tokens out_tokens[offsets[b] + b + i],
 *     i = 0..n, are written at positions L..L+n, seq_len[b] = L + n + 1,
 *     next_tokens[b] = the last of them, status n + 1.
 * A failed request keeps its history and length and gets next_tokens -1.
 */
int oracle_commit_tokens(int32_t B, int32_t max_k, int32_t n_draft_rows, const int32_t* offsets,
                         const int32_t* accept_len, const int32_t* out_tokens,
                         int32_t* seq_tokens, int64_t seq_stride, int32_t* seq_len,
                         int32_t capacity, int32_t* next_tokens, int32_t* status) {
  if (B < 1 || !offsets || !accept_len || !out_tokens || !seq_tokens || !seq_len ||
      !next_tokens || !status || capacity < 0 || seq_stride < capacity)
    return -1;
  for (int32_t b = 0; b < B; ++b) {
    next_tokens[b] = -1;
    const int32_t off = offsets[b], off1 = offsets[b + 1], n = accept_len[b];
    const int slice_ok = off >= 0 && off1 >= off && off1 <= n_draft_rows && off1 - off <= max_k;
    if (!slice_ok || n < 0 || n > off1 - off) {
      status[b] = -1;
      continue;
    }
    const int32_t L = seq_len[b];
    if (L < 0 || (int64_t)L + n + 1 > capacity) {
      status[b] = -2;
      continue;
    }
    for (int32_t i = 0; i <= n; ++i)
      seq_tokens[(int64_t)b * seq_stride + L + i] = out_tokens[(int64_t)off + b + i];
    seq_len[b] = L + n + 1;
    next_tokens[b] = out_tokens[(int64_t)off + b + n];
    status[b] = n + 1;
  }
  return 0;
}

/* ---------------------------------------------------------------- tree verify */

/* Greedy verification of a draft tree ("Decodificación Especulativa y EAGLE",
 * section on tree attention verification: every node of the tree is scored in
 * one target pass, each node seeing only its ancestors, and the result is the
 * longest prefix along any accepted root-to-node path; Perplexity's post,
 * section "EAGLE": the chosen sequence is followed by one extra token from the
 * target).  With the greedy rule of section "La Regla de Exactitud" a draft
 * node is accepted when its parent is accepted and its token is the argmax of
 * the parent's target row.
 *
 * Request b owns nodes i = 0..N_b-1, N_b = node_offsets[b+1] - node_offsets[b],
 * at packed rows node_offsets[b] + i.  Node 0 is the root (the last committed
 * token; its parent and token entries are not read).  Node i >= 1 has parent
 * parents[off + i] in [0, i) and token tokens[off + i] in [0, V).  Target row
 * of node i: the distribution of the token that follows the path root..i.
 *
 * Per request:
 *   g_i = argmax of node i's row (lowest index on ties), for every node;
 *   accepted(0) = 1; accepted(i) = accepted(parent) and token_i == g_parent;
 *   depth(0) = 0; depth(i) = depth(parent) + 1;
 *   c = the accepted node of greatest depth, lowest index among equals (two
 *       accepted nodes of equal depth need siblings with equal tokens);
 *   d = depth(c); path = root = a_0, a_1, ..., a_d = c (each the parent of the
 *       next).
 * Outputs: accept_len[b] = d; out_tokens[off + j] = token of a_{j+1} for j < d,
 * out_tokens[off + d] = g_c, -1 after; accept_nodes[off + j] = a_j for j <= d,
 * -1 after.  Failures set accept_len[b] = -1: a slice outside [0, n_rows) or
 * N_b outside [1, max_nodes] (nothing else written), or a parent outside
 * [0, i), a token outside [0, V), a row with no finite maximum (the request's
 * outputs filled with -1).
 */
int oracle_tree_verify_greedy(int dtype, const void* target, int32_t B, int32_t V,
                              int32_t max_nodes, int32_t n_rows, const int32_t* node_offsets,
                              const int32_t* parents, const int32_t* tokens,
                              int32_t* accept_len, int32_t* out_tokens,
                              int32_t* accept_nodes) {
  if (B < 1 || V < 1 || max_nodes < 1 || max_nodes > 1024 || !target || !node_offsets ||
      !parents || !tokens || !accept_len || !out_tokens || !accept_nodes)
    return -1;
  int32_t g[1024], depth[1024], path[1024];
  unsigned char acc[1024];
  for (int32_t b = 0; b < B; ++b) {
    const int32_t off = node_offsets[b], off1 = node_offsets[b + 1];
    const int32_t N = off1 - off;
    if (off < 0 || off1 > n_rows || off1 < off || N < 1 || N > max_nodes) {
      accept_len[b] = -1;
      continue;
    }
    int ok = 1;
    for (int32_t i = 1; i < N && ok; ++i) {
      const int32_t par = parents[off + i], tok = tokens[off + i];
      if (par < 0 || par >= i || tok < 0 || tok >= V) ok = 0;
    }
    for (int32_t i = 0; i < N && ok; ++i) {
      g[i] = row_argmax(target, dtype, (int64_t)off + i, V);
      if (g[i] < 0) ok = 0;
    }
    if (!ok) {
      accept_len[b] = -1;
      for (int32_t i = 0; i < N; ++i) {
        out_tokens[off + i] = -1;
        accept_nodes[off + i] = -1;
      }
      continue;
    }
    /* acceptance and depth, parents before children */
    acc[0] = 1;
    depth[0] = 0;
    for (int32_t i = 1; i < N; ++i) {
      const int32_t par = parents[off + i];
      acc[i] = acc[par] && tokens[off + i] == g[par];
      depth[i] = depth[par] + 1;
    }
    int32_t c = 0;
    for (int32_t i = 1; i < N; ++i)
      if (acc[i] && depth[i] > depth[c]) c = i;
    const int32_t d = depth[c];
    int32_t u = c;
    for (int32_t j = d; j >= 0; --j) {
      path[j] = u;
      u = j > 0 ? parents[off + u] : u;
    }
    accept_len[b] = d;
    for (int32_t j = 0; j < N; ++j) {
      out_tokens[off + j] = j < d ? tokens[off + path[j + 1]] : (j == d ? g[c] : -1);
      accept_nodes[off + j] = j <= d ? path[j] : -1;
    }
  }
  return 0;
}
