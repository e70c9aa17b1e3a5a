/*
 * CPU oracle for speculative-decoding verification — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C99 in fp64.  It is used by the tests, by the
 * smoke check and by the benchmark's CPU-baseline leg, and by nothing on the
 * product path.  It shares no code, header, table or helper with the GPU
 * library; both only read the same seeded input arrays.
 *
 * Sources (web pages; p = target distribution, q = draft distribution):
 *  [LOTOOK]  lotook.com "What is speculative decoding?" explainer — section
 *            "단계별로 어떻게 작동할까요" (the four steps of one cycle: draft K,
 *            one target pass giving K+1 distributions, left-to-right accept /
 *            reject, resample at the first rejection or take a bonus token)
 *            and the FAQ on losslessness (greedy accepts only the target's
 *            top choice).
 *  [ARISER]  ariser.io "Speculative Decoding: 작은 모델이 먼저 쓰면 큰 모델도
 *            빨라진다" — section "같은 분포를 지키는 작은 장치" (accept x ~ q with
 *            probability min(1, p(x)/q(x)); on rejection draw from
 *            normalize(max(0, p - q)); temperature / top-p must already be
 *            applied to p and q) and its two-token worked example.
 *  [TAPS]    aitrends.kr "TAPS: 추측 샘플링을 위한 작업 인지형 제안 분포 연구" —
 *            section "방법론" (merged-tree verification: ancestor-preserving
 *            mask, one target pass, keep the longest accepted path) and
 *            section "코드 예제" (merged mask block layout).
 *  [SUBSPEC] hip-studyrecord.tistory.com SubSpec review — Method, part 2
 *            "Token 생성과정" (greedy verify narrative: accept the agreeing
 *            prefix, replace the first disagreeing token, drop the rest).
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes): accept iff u * q'(x) < p'(x) with u in [0,1); inverse CDF over
 * ascending vocabulary ids, first j with C_j > u*S; argmax ties -> lowest id;
 * top-p orders by raw logit, keeps whole tie groups, stops when the tempered
 * cumulative mass first reaches top_p, top_p >= 1 disables it; an
 * out-of-range draft token is rejected (sampling) / a mismatch (greedy);
 * a tree child is checked against the target's top choice at its parent and
 * the deepest accepted node wins, lowest node index on ties.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* per-request flag bits */
#define FLAG_ACCEPT_NEAR 1   /* a uniform within 1e-6 relative of p'/q' */
#define FLAG_CDF_NEAR 2      /* u*S within 1e-6 relative of a CDF step */
#define FLAG_TOPP_NEAR 4     /* an alternative nucleus near top_p changes the output */
#define FLAG_FALLBACK 8      /* residual mass S <= S_RESOLUTION, drew from p' instead */
#define FLAG_TOKEN_RANGE 16  /* a draft token outside [0, V) */
#define FLAG_TOPP_EDGE 32    /* some row's nucleus edge lies within 1e-6 of top_p
                                (informational: p', q' may legitimately differ) */
#define FLAG_S_NEAR 64       /* residual mass within a factor 4 of S_RESOLUTION */

#define REL_TOL 1e-6
/* Residual mass at or below which the residual is taken as empty and the
 * replacement is drawn from p' (reading: S = 0 cannot happen after a
 * rejection in exact arithmetic; at 2^-20 of the unit mass, twice the total
 * rounding of p' and q' held as float32 values, max(0, p' - q') carries no
 * resolvable mass, and normalising it would only amplify rounding). */
#define S_RESOLUTION 9.5367431640625e-07

/* ------------------------------------------------------------------ */
/* input widening: every stored value becomes the fp64 number it encodes */

static double logit_at(const void *base, int dtype, size_t i) {
  if (dtype == ORC_F32) return (double)((const float *)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------ */
/* one row's distribution after temperature and top-p ([ARISER]: p and q must
 * reflect the sampling settings).  Fills prob[V]; info[] = {max logit, Z (sum
 * of exp((l-max)/T)), kept mass (as a fraction of Z), tau, cum mass before the
 * cut group, cum mass after the cut group, cut group index}.               */

typedef struct {
  double value;
  int index;
} Entry;

static int by_value_desc(const void *a, const void *b) {
  const Entry *x = (const Entry *)a, *y = (const Entry *)b;
  if (x->value > y->value) return -1;
  if (x->value < y->value) return 1;
  return (x->index > y->index) - (x->index < y->index);
}

/* cut_shift: 0 = the defined nucleus; -1 = stop one group earlier; +1 = one
 * group later (used only to test whether a near-boundary choice matters). */
static void row_distribution(const void *logits, int dtype, size_t off, int V,
                             double T, double top_p, int cut_shift,
                             double *prob, Entry *scratch, double *info) {
  double m = -INFINITY;
  for (int j = 0; j < V; ++j) {
    double l = logit_at(logits, dtype, off + j);
    if (l > m) m = l;
  }
  double Z = 0.0;
  for (int j = 0; j < V; ++j) {
    double e = exp((logit_at(logits, dtype, off + j) - m) / T);
    prob[j] = e;
    Z += e;
  }
  for (int j = 0; j < V; ++j) prob[j] /= Z;
  double tau = -INFINITY, before = 0.0, after = 1.0, kept = 1.0;
  int cut_group = -1;
  if (top_p < 1.0) {
    for (int j = 0; j < V; ++j) {
      scratch[j].value = logit_at(logits, dtype, off + j);
      scratch[j].index = j;
    }
    qsort(scratch, (size_t)V, sizeof(Entry), by_value_desc);
    /* walk tie groups from the top, accumulating tempered mass */
    double cum = 0.0;
    int g = 0, start = 0, target_group = -1;
    /* first pass: find the defined cut group */
    while (start < V) {
      int end = start;
      double gm = 0.0;
      while (end < V && scratch[end].value == scratch[start].value) {
        gm += prob[scratch[end].index];
        ++end;
      }
      if (cum + gm >= top_p) {
        target_group = g;
        before = cum;
        after = cum + gm;
        break;
      }
      cum += gm;
      start = end;
      ++g;
    }
    if (target_group < 0) target_group = g - 1; /* rounding: keep everything */
    cut_group = target_group;
    int want = target_group + cut_shift;
    if (want < 0) want = 0;
    /* second pass: locate the wanted group's value */
    start = 0;
    g = 0;
    while (start < V) {
      int end = start;
      while (end < V && scratch[end].value == scratch[start].value) ++end;
      tau = scratch[start].value;
      if (g == want) break;
      start = end;
      ++g;
    }
    kept = 0.0;
    for (int j = 0; j < V; ++j)
      if (logit_at(logits, dtype, off + j) >= tau) kept += prob[j];
    for (int j = 0; j < V; ++j)
      prob[j] = (logit_at(logits, dtype, off + j) >= tau) ? prob[j] / kept : 0.0;
  }
  if (info) {
    info[0] = m;
    info[1] = Z;
    info[2] = kept;
    info[3] = tau;
    info[4] = before;
    info[5] = after;
    info[6] = (double)cut_group;
  }
}

/* Exposed for tests: the post-temperature, post-top-p distribution of one row. */
int oracle_row_distribution(const void *logits, int dtype, int V, double T,
                            double top_p, double *out_prob, double *out_info) {
  if (!logits || !out_prob || V < 1 || !(T > 0.0)) return -1;
  Entry *scratch = (Entry *)malloc(sizeof(Entry) * (size_t)V);
  if (!scratch) return -2;
  row_distribution(logits, dtype, 0, V, T, top_p, 0, out_prob, scratch, out_info);
  free(scratch);
  return 0;
}

/* ------------------------------------------------------------------ */
/* sampling verify of one request ([LOTOOK] four steps; [ARISER] rule)    */

typedef struct {
  int n;            /* accepted drafts */
  int token;        /* replacement (n < K) or bonus (n == K) */
  double S;         /* residual mass */
  int flags;
} SampleResult;

static SampleResult verify_one_request(
    const void *target, const void *draft, int dtype, const int32_t *tok,
    const float *ua, float us, double T, double top_p, int K, int V,
    int alt_row /* -1 none; else row r in [0, 2K] (target rows 0..K, draft K+1..2K) */,
    int alt_shift, double **P, double **Q, Entry *scratch, double *r,
    double *out_p, double *out_q, double (*infos)[7]) {
  SampleResult res = {0, -1, 0.0, 0};
  size_t rowV = (size_t)V;
  /* distributions p'_0..p'_K and q'_0..q'_{K-1} */
  for (int i = 0; i <= K; ++i) {
    int shift = (alt_row == i) ? alt_shift : 0;
    row_distribution(target, dtype, (size_t)i * rowV, V, T, top_p, shift, P[i],
                     scratch, infos ? infos[i] : NULL);
  }
  for (int i = 0; i < K; ++i) {
    int shift = (alt_row == K + 1 + i) ? alt_shift : 0;
    row_distribution(draft, dtype, (size_t)i * rowV, V, T, top_p, shift, Q[i],
                     scratch, infos ? infos[K + 1 + i] : NULL);
  }
  /* probabilities at the draft tokens (diagnostics for every position) */
  for (int i = 0; i < K; ++i) {
    int x = tok[i];
    int ok = (x >= 0 && x < V);
    if (out_p) out_p[i] = ok ? P[i][x] : 0.0;
    if (out_q) out_q[i] = ok ? Q[i][x] : 0.0;
  }
  /* left to right: accept x_i iff u_i * q'(x_i) < p'(x_i); stop at the first rejection */
  int n = K;
  for (int i = 0; i < K; ++i) {
    int x = tok[i];
    if (x < 0 || x >= V) {
      res.flags |= FLAG_TOKEN_RANGE;
      n = i;
      break;
    }
    double a = P[i][x], c = Q[i][x], u = (double)ua[i];
    if (c > 0.0) {
      double ratio = a / c;
      if (fabs(u - ratio) <= REL_TOL * ratio) res.flags |= FLAG_ACCEPT_NEAR;
    }
    if (!(u * c < a)) {
      n = i;
      break;
    }
  }
  res.n = n;
  /* residual (first rejection) or bonus (all accepted) */
  double S = 0.0;
  if (n < K) {
    for (int j = 0; j < V; ++j) {
      double d = P[n][j] - Q[n][j];
      r[j] = d > 0.0 ? d : 0.0;
      S += r[j];
    }
    if (S > 0.25 * S_RESOLUTION && S < 4.0 * S_RESOLUTION) res.flags |= FLAG_S_NEAR;
    if (!(S > S_RESOLUTION)) {
      res.flags |= FLAG_FALLBACK;
      S = 0.0;
      for (int j = 0; j < V; ++j) {
        r[j] = P[n][j];
        S += r[j];
      }
    }
  } else {
    for (int j = 0; j < V; ++j) {
      r[j] = P[K][j];
      S += r[j];
    }
  }
  res.S = S;
  /* inverse CDF over ascending ids: smallest j with C_j > u*S */
  double t = (double)us * S, C = 0.0, Cprev = 0.0;
  int pick = -1;
  for (int j = 0; j < V; ++j) {
    Cprev = C;
    C += r[j];
    if (C > t) {
      pick = j;
      break;
    }
  }
  if (pick < 0) {
    for (int j = V - 1; j >= 0; --j)
      if (r[j] > 0.0) {
        pick = j;
        break;
      }
    res.flags |= FLAG_CDF_NEAR;
  } else {
    double gap = fmin(t - Cprev, C - t);
    if (gap <= REL_TOL * t) res.flags |= FLAG_CDF_NEAR;
  }
  res.token = pick;
  return res;
}

/*
 * Sampling verify of B requests.
 *   target [B, K+1, V], draft [B, K, V] (dtype ORC_F32 / ORC_BF16 bit patterns)
 *   tokens [B, K]; u_accept [B, K]; u_sample [B]; T > 0; top_p in (0, 1].
 * Outputs: out_accepted [B]; out_tokens [B, K+1] (accepted drafts, the
 * replacement or bonus, then -1); optional out_p/out_q [B, K] (p'(x_i),
 * q'(x_i)), out_S [B] (residual mass), out_flags [B] (FLAG_* bits),
 * out_row_info [B, 2K+1, 7] (see row_distribution).
 *
 * The other nucleus membership (top_p < 1).  Where a row's cumulative mass
 * before or after its cut group lies within 1e-6 of top_p, the request is
 * verified again with that one row's cut moved one group earlier (before
 * near) or later (after near), every other row as defined.  Each such
 * variant is alternative a = 2 * row + (0: earlier, 1: later), row in
 * [0, 2K] (target rows 0..K, draft rows K+1..2K).  Optional outputs, all
 * indexed [B, 2K+1, 2]: out_alt_n (the accepted length under the variant,
 * -1 where no variant is taken), out_alt_token (its replacement or bonus),
 * out_alt_S (its residual mass); out_alt_p / out_alt_q [B, 2K+1, 2, K] its
 * p'(x_i), q'(x_i).  FLAG_TOPP_NEAR marks a request where some variant's
 * accepted length or token differs from the defined one.
 */
int oracle_verify_sample(const void *target, const void *draft, int dtype,
                         const int32_t *tokens, const float *u_accept,
                         const float *u_sample, double T, double top_p, int B,
                         int K, int V, int32_t *out_accepted, int32_t *out_tokens,
                         double *out_p, double *out_q, double *out_S,
                         int32_t *out_flags, double *out_row_info,
                         int32_t *out_alt_n, int32_t *out_alt_token, double *out_alt_S,
                         double *out_alt_p, double *out_alt_q) {
  if (!target || !draft || !tokens || !u_accept || !u_sample || !out_accepted ||
      !out_tokens)
    return -1;
  if (B < 1 || K < 1 || V < 1 || !(T > 0.0) || !(top_p > 0.0)) return -2;
  size_t esz = dtype == ORC_F32 ? 4 : 2;
  double **P = (double **)malloc(sizeof(double *) * (size_t)(K + 1));
  double **Q = (double **)malloc(sizeof(double *) * (size_t)K);
  double *buf = (double *)malloc(sizeof(double) * (size_t)V * (size_t)(2 * K + 2));
  Entry *scratch = (Entry *)malloc(sizeof(Entry) * (size_t)V);
  double(*infos)[7] = (double(*)[7])malloc(sizeof(double) * 7 * (size_t)(2 * K + 1));
  if (!P || !Q || !buf || !scratch || !infos) {
    free(P); free(Q); free(buf); free(scratch); free(infos);
    return -3;
  }
  for (int i = 0; i <= K; ++i) P[i] = buf + (size_t)i * V;
  for (int i = 0; i < K; ++i) Q[i] = buf + (size_t)(K + 1 + i) * V;
  double *r = buf + (size_t)(2 * K + 1) * V;
  for (int b = 0; b < B; ++b) {
    const char *tb = (const char *)target + (size_t)b * (K + 1) * V * esz;
    const char *db = (const char *)draft + (size_t)b * K * V * esz;
    const int32_t *tok = tokens + (size_t)b * K;
    const float *ua = u_accept + (size_t)b * K;
    SampleResult res = verify_one_request(
        tb, db, dtype, tok, ua, u_sample[b], T, top_p, K, V, -1, 0, P, Q, scratch, r,
        out_p ? out_p + (size_t)b * K : NULL, out_q ? out_q + (size_t)b * K : NULL,
        infos);
    /* a nucleus whose edge sits within 1e-6 of top_p: does the other choice
     * change what is emitted? */
    const size_t nalt = (size_t)(2 * K + 1) * 2;
    if (out_alt_n)
      for (size_t a = 0; a < nalt; ++a) {
        out_alt_n[(size_t)b * nalt + a] = -1;
        if (out_alt_token) out_alt_token[(size_t)b * nalt + a] = -1;
        if (out_alt_S) out_alt_S[(size_t)b * nalt + a] = 0.0;
      }
    if (top_p < 1.0) {
      /* infos[] of the defined request, kept: the variants below overwrite
       * nothing of it (they pass no info buffer) */
      for (int row = 0; row < 2 * K + 1; ++row) {
        double before = infos[row][4], after = infos[row][5];
        int shifts[2] = {0, 0};
        if (infos[row][6] > 0.0 && fabs(before - top_p) <= REL_TOL) shifts[0] = -1;
        if (fabs(after - top_p) <= REL_TOL) shifts[1] = +1;
        if (shifts[0] || shifts[1]) res.flags |= FLAG_TOPP_EDGE;
        for (int s = 0; s < 2; ++s) {
          if (!shifts[s]) continue;
          const size_t a = (size_t)b * nalt + (size_t)(2 * row + s);
          SampleResult alt = verify_one_request(
              tb, db, dtype, tok, ua, u_sample[b], T, top_p, K, V, row, shifts[s], P, Q,
              scratch, r, out_alt_p ? out_alt_p + a * (size_t)K : NULL,
              out_alt_q ? out_alt_q + a * (size_t)K : NULL, NULL);
          if (alt.n != res.n || alt.token != res.token) res.flags |= FLAG_TOPP_NEAR;
          if (out_alt_n) out_alt_n[a] = alt.n;
          if (out_alt_token) out_alt_token[a] = alt.token;
          if (out_alt_S) out_alt_S[a] = alt.S;
        }
      }
      if (out_row_info)
        memcpy(out_row_info + (size_t)b * (2 * K + 1) * 7, infos,
               sizeof(double) * 7 * (size_t)(2 * K + 1));
      /* restore nothing: each request recomputes its rows from scratch */
    } else if (out_row_info) {
      memcpy(out_row_info + (size_t)b * (2 * K + 1) * 7, infos,
             sizeof(double) * 7 * (size_t)(2 * K + 1));
    }
    out_accepted[b] = res.n;
    int32_t *ot = out_tokens + (size_t)b * (K + 1);
    for (int i = 0; i <= K; ++i) ot[i] = -1;
    for (int i = 0; i < res.n; ++i) ot[i] = tok[i];
    ot[res.n] = res.token;
    if (out_S) out_S[b] = res.S;
    if (out_flags) out_flags[b] = res.flags;
  }
  free(P); free(Q); free(buf); free(scratch); free(infos);
  return 0;
}

/* ------------------------------------------------------------------ */
/* greedy (temperature 0): accept while the draft equals the target's top
 * choice ([LOTOOK] FAQ; [SUBSPEC] verify step), emit the top choice at the
 * first mismatch or after the last position (bonus).                    */

static int row_argmax(const void *logits, int dtype, size_t off, int V) {
  int best = 0;
  double bv = logit_at(logits, dtype, off);
  for (int j = 1; j < V; ++j) {
    double v = logit_at(logits, dtype, off + j);
    if (v > bv) { /* strict: equal values keep the lower id */
      bv = v;
      best = j;
    }
  }
  return best;
}

int oracle_verify_greedy(const void *target, int dtype, const int32_t *tokens,
                         int B, int K, int V, int32_t *out_accepted,
                         int32_t *out_tokens, int32_t *out_argmax) {
  if (!target || !tokens || !out_accepted || !out_tokens) return -1;
  if (B < 1 || K < 1 || V < 1) return -2;
  int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
  if (!a) return -3;
  for (int b = 0; b < B; ++b) {
    size_t base = (size_t)b * (K + 1) * V;
    for (int i = 0; i <= K; ++i) a[i] = row_argmax(target, dtype, base + (size_t)i * V, V);
    const int32_t *tok = tokens + (size_t)b * K;
    int n = K;
    for (int i = 0; i < K; ++i)
      if (tok[i] != a[i]) {
        n = i;
        break;
      }
    int32_t *ot = out_tokens + (size_t)b * (K + 1);
    for (int i = 0; i <= K; ++i) ot[i] = -1;
    for (int i = 0; i < n; ++i) ot[i] = tok[i];
    ot[n] = a[n];
    out_accepted[b] = n;
    if (out_argmax)
      for (int i = 0; i <= K; ++i) out_argmax[(size_t)b * (K + 1) + i] = a[i];
  }
  free(a);
  return 0;
}

/* ------------------------------------------------------------------ */
/* The target's logits from its final hidden states and the vocabulary
 * matrix, fused in front of greedy verification.  The one target pass of
 * [LOTOOK]'s four steps ends in this product: l[r][v] = sum_k h[r][k] *
 * w[v][k], h and w bf16 bit patterns.  Every product is exact in fp64; the
 * sum runs in k order in fp64.  absdot[r][v] = sum_k |h[r][k] w[v][k]|
 * bounds the rounding of any fp32 evaluation of the same sum (by
 * (d - 1) 2^-24 absdot / (1 - (d - 1) 2^-24), whatever the order).      */

static double bf16_value(uint16_t bits) {
  const uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static void lmhead_row(const uint16_t *hrow, const uint16_t *weight, int d, int V, double *h,
                       double *logits, double *absdot) {
  for (int k = 0; k < d; ++k) h[k] = bf16_value(hrow[k]);
  for (int v = 0; v < V; ++v) {
    const uint16_t *w = weight + (size_t)v * d;
    double s = 0.0, a = 0.0;
    for (int k = 0; k < d; ++k) {
      const double p = h[k] * bf16_value(w[k]);
      s += p;
      a += fabs(p);
    }
    logits[v] = s;
    if (absdot) absdot[v] = a;
  }
}

int oracle_lmhead_logits(const uint16_t *hidden, const uint16_t *weight, int R, int d, int V,
                         double *out_logits, double *out_absdot) {
  if (!hidden || !weight || !out_logits) return -1;
  if (R < 1 || d < 1 || V < 1) return -2;
  double *h = (double *)malloc(sizeof(double) * (size_t)d);
  if (!h) return -3;
  for (int r = 0; r < R; ++r)
    lmhead_row(hidden + (size_t)r * d, weight, d, V, h, out_logits + (size_t)r * V,
               out_absdot ? out_absdot + (size_t)r * V : NULL);
  free(h);
  return 0;
}

/* Greedy verification on the fused logits: the top choice of each of the
 * K+1 rows (lowest id on ties), then the rule of oracle_verify_greedy.  */
int oracle_lmhead_greedy(const uint16_t *hidden, const uint16_t *weight, const int32_t *tokens,
                         int B, int K, int d, int V, int32_t *out_accepted, int32_t *out_tokens,
                         int32_t *out_argmax) {
  if (!hidden || !weight || !tokens || !out_accepted || !out_tokens) return -1;
  if (B < 1 || K < 1 || d < 1 || V < 1) return -2;
  double *h = (double *)malloc(sizeof(double) * (size_t)d);
  double *row = (double *)malloc(sizeof(double) * (size_t)V);
  int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
  if (!h || !row || !a) {
    free(h);
    free(row);
    free(a);
    return -3;
  }
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i <= K; ++i) {
      lmhead_row(hidden + ((size_t)b * (K + 1) + i) * d, weight, d, V, h, row, NULL);
      int best = 0;
      for (int v = 1; v < V; ++v)
        if (row[v] > row[best]) best = v; /* strict: ties keep the lower id */
      a[i] = best;
    }
    const int32_t *tok = tokens + (size_t)b * K;
    int n = K;
    for (int i = 0; i < K; ++i)
      if (tok[i] != a[i]) {
        n = i;
        break;
      }
    int32_t *ot = out_tokens + (size_t)b * (K + 1);
    for (int i = 0; i <= K; ++i) ot[i] = -1;
    for (int i = 0; i < n; ++i) ot[i] = tok[i];
    ot[n] = a[n];
    out_accepted[b] = n;
    if (out_argmax)
      for (int i = 0; i <= K; ++i) out_argmax[(size_t)b * (K + 1) + i] = a[i];
  }
  free(h);
  free(row);
  free(a);
  return 0;
}

/* ------------------------------------------------------------------ */
/* greedy verification of a merged tree ([TAPS] "방법론": one target pass
 * over all paths under an ancestor-preserving mask, keep the longest
 * accepted path).                                                       */

/* 1 if mask rows equal the ancestor-or-self closure of parents (with
 * parents[0] = -1 and 0 <= parents[i] < i), else 0. */
static int tree_is_valid(const int32_t *parents, const uint8_t *mask, int N) {
  if (parents[0] != -1) return 0;
  for (int i = 1; i < N; ++i)
    if (parents[i] < 0 || parents[i] >= i) return 0;
  for (int i = 0; i < N; ++i) {
    for (int j = 0; j < N; ++j) {
      int anc = 0;
      for (int k = i; k >= 0; k = parents[k])
        if (k == j) {
          anc = 1;
          break;
        }
      if ((mask[(size_t)i * N + j] != 0) != anc) return 0;
    }
  }
  return 1;
}

int oracle_tree_is_valid(const int32_t *parents, const uint8_t *mask, int N) {
  if (!parents || !mask || N < 1) return -1;
  return tree_is_valid(parents, mask, N);
}

int oracle_verify_tree(const void *target, int dtype, const int32_t *parents,
                       const int32_t *node_tokens, const uint8_t *anc_mask, int B,
                       int N, int V, int32_t *out_path_len, int32_t *out_path_nodes,
                       int32_t *out_tokens, int32_t *out_valid, int32_t *out_argmax) {
  if (!target || !parents || !node_tokens || !anc_mask || !out_path_len ||
      !out_path_nodes || !out_tokens)
    return -1;
  if (B < 1 || N < 1 || V < 1) return -2;
  int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
  int *match = (int *)malloc(sizeof(int) * (size_t)N);
  int *acc = (int *)malloc(sizeof(int) * (size_t)N);
  int *depth = (int *)malloc(sizeof(int) * (size_t)N);
  if (!a || !match || !acc || !depth) {
    free(a); free(match); free(acc); free(depth);
    return -3;
  }
  for (int b = 0; b < B; ++b) {
    const int32_t *par = parents + (size_t)b * N;
    const int32_t *tok = node_tokens + (size_t)b * N;
    const uint8_t *mask = anc_mask + (size_t)b * N * N;
    if (out_valid) out_valid[b] = tree_is_valid(par, mask, N);
    /* node i's row holds the target's next-token logits after root..i */
    for (int i = 0; i < N; ++i)
      a[i] = row_argmax(target, dtype, ((size_t)b * N + i) * (size_t)V, V);
    /* a child is right if it is the target's top choice after its parent */
    match[0] = 1;
    for (int i = 1; i < N; ++i) {
      int p = par[i];
      match[i] = (p >= 0 && p < N && tok[i] == a[p]) ? 1 : 0;
    }
    /* accepted = every node on its mask row (ancestors and itself) is right */
    for (int i = 0; i < N; ++i) {
      acc[i] = 1;
      depth[i] = -1;
      for (int j = 0; j < N; ++j)
        if (mask[(size_t)i * N + j]) {
          depth[i] += 1;
          if (!match[j]) acc[i] = 0;
        }
    }
    /* deepest accepted node, lowest index on ties */
    int best = 0;
    for (int i = 1; i < N; ++i)
      if (acc[i] && depth[i] > depth[best]) best = i;
    int d = depth[best] < 0 ? 0 : depth[best];
    int32_t *pn = out_path_nodes + (size_t)b * N;
    int32_t *ot = out_tokens + (size_t)b * N;
    for (int i = 0; i < N; ++i) {
      pn[i] = -1;
      ot[i] = -1;
    }
    /* the path: the best node's mask row minus the root, ordered by depth */
    for (int j = 1; j < N; ++j)
      if (mask[(size_t)best * N + j] && depth[j] >= 1 && depth[j] <= d) {
        pn[depth[j] - 1] = j;
        ot[depth[j] - 1] = tok[j];
      }
    if (d < N) ot[d] = a[best]; /* the target's next token after the path */
    out_path_len[b] = d;
    if (out_argmax)
      for (int i = 0; i < N; ++i) out_argmax[(size_t)b * N + i] = a[i];
  }
  free(a); free(match); free(acc); free(depth);
  return 0;
}

/* ------------------------------------------------------------------------
 * KV-cache commit after one cycle.  Both models keep their own cache; the
 * entries of rejected drafts are cut away before the next cycle (LOTOOK,
 * section on the KV cache), and a drafter that shares the target's layers
 * has its temporary entries overwritten with the target's values (SubSpec
 * review, Method part 2, step 4 "Update KV").  For a merged tree verified in
 * one pass (TAPS, "방법론") the accepted path's entries are gathered into
 * consecutive slots.
 *
 * Cache layout [L][2][B][H][S][D], elements of es bytes (the bytes are
 * copied, never interpreted).  Request b's cycle wrote its entries at slots
 * c .. c+N-1 (c = cache_len[b]): slot c + i holds node i of the tree, or
 * position i of a linear draft (node / position 0 is the root, the token
 * emitted by the previous cycle).  The accepted path is the root and then
 * path_nodes[b][0 .. d-1] (d = path_len[b]), or positions 1 .. d when
 * path_nodes is NULL.  After the commit slot c + j holds the entry of path
 * element j (j = 0 .. d), every other slot is unchanged, and new_len[b] =
 * c + 1 + d.  Definition is out of place: every committed entry is the
 * cache's entry before the call.  The mirror, if given, receives the same
 * d + 1 entries at the same slots.
 *
 * A request whose inputs are inconsistent (d outside [0, N-1], c < 0,
 * c + N > S, or path nodes not strictly increasing within [1, N-1]) is left
 * untouched and gets new_len[b] = -1.
 *
 * kv_out (and mirror_out) must hold a copy of the cache (and mirror) before
 * the call; kv_in is the cache before the call.
 * ------------------------------------------------------------------------ */
int oracle_kv_commit(const void *kv_in, void *kv_out, void *mirror_out, int es, int L, int B,
                     int H, int S, int D, const int32_t *cache_len, const int32_t *path_len,
                     const int32_t *path_nodes, int N, int32_t *new_len) {
  if (!kv_in || !kv_out || !cache_len || !path_len || !new_len) return -1;
  if (es < 1 || L < 1 || B < 1 || H < 1 || S < 1 || D < 1 || N < 1) return -2;
  const size_t row = (size_t)D * (size_t)es;
  const unsigned char *src = (const unsigned char *)kv_in;
  unsigned char *dst = (unsigned char *)kv_out;
  unsigned char *mir = (unsigned char *)mirror_out;
  for (int b = 0; b < B; ++b) {
    const int c = cache_len[b];
    const int d = path_len[b];
    int ok = d >= 0 && d <= N - 1 && c >= 0 && (long)c + N <= S;
    if (ok && path_nodes) {
      int prev = 0;
      for (int j = 0; j < d && ok; ++j) {
        const int p = path_nodes[(size_t)b * N + j];
        if (p <= prev || p > N - 1) ok = 0;
        prev = p;
      }
    }
    if (!ok) {
      new_len[b] = -1;
      continue;
    }
    for (int l = 0; l < L; ++l)
      for (int kv = 0; kv < 2; ++kv)
        for (int h = 0; h < H; ++h) {
          const size_t base = ((((size_t)l * 2 + kv) * B + b) * H + h) * (size_t)S * row;
          for (int j = 0; j <= d; ++j) {
            const int node = j == 0 ? 0 : (path_nodes ? path_nodes[(size_t)b * N + j - 1] : j);
            const unsigned char *from = src + base + (size_t)(c + node) * row;
            memcpy(dst + base + (size_t)(c + j) * row, from, row);
            if (mir) memcpy(mir + base + (size_t)(c + j) * row, from, row);
          }
        }
    new_len[b] = c + 1 + d;
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Merging two drafters' trees under one root (TAPS, "방법론": one target
 * pass over both trees under an ancestor-preserving mask; "코드 예제": the
 * block layout) and routing by confidence (TAPS: the tree whose nodes have
 * the higher mean predicted probability).
 *
 * Per request: tree t (t = 1, 2) has n_t + 1 nodes in BFS order, parents
 * [n_t + 1] (node 0 the root, parent -1; 0 <= parent[i] < i otherwise),
 * tokens [n_t + 1], conf [n_t + 1] (the drafter's probability of each
 * node's token; the root's entry is not used).  The merged tree has
 * N = n1 + n2 + 1 nodes: node 0 = the shared root (tree 1's root token);
 * nodes 1..n1 = tree 1's nodes 1..n1 with their parents; nodes
 * n1+1..n1+n2 = tree 2's nodes 1..n2, parent 0 staying 0 and parent p > 0
 * becoming p + n1.  The mask row of node i is its ancestor-or-self set.
 * Confidence of a tree: the mean of conf over its non-root nodes, summed
 * in node order in fp64 (0 for a tree without nodes); route = 1 if tree 2's
 * is larger, else 0.  A request with an invalid tree gets route -1,
 * parents and tokens -1, a zero mask, confidences 0.
 * ------------------------------------------------------------------------ */
static int parents_ok(const int32_t *p, int n) {
  if (p[0] != -1) return 0;
  for (int i = 1; i <= n; ++i)
    if (p[i] < 0 || p[i] >= i) return 0;
  return 1;
}

int oracle_tree_merge(const int32_t *parents1, const int32_t *tokens1, const float *conf1,
                      int n1, const int32_t *parents2, const int32_t *tokens2,
                      const float *conf2, int n2, int B, int32_t *out_parents,
                      int32_t *out_tokens, uint8_t *out_mask, double *out_conf,
                      int32_t *out_route) {
  if (!parents1 || !tokens1 || !conf1 || !parents2 || !tokens2 || !conf2 || !out_parents ||
      !out_tokens || !out_mask || !out_conf || !out_route)
    return -1;
  if (n1 < 0 || n2 < 0 || B < 1 || n1 + n2 + 1 > 64) return -2;
  const int N = n1 + n2 + 1;
  for (int b = 0; b < B; ++b) {
    const int32_t *p1 = parents1 + (size_t)b * (n1 + 1), *p2 = parents2 + (size_t)b * (n2 + 1);
    const int32_t *t1 = tokens1 + (size_t)b * (n1 + 1), *t2 = tokens2 + (size_t)b * (n2 + 1);
    const float *c1 = conf1 + (size_t)b * (n1 + 1), *c2 = conf2 + (size_t)b * (n2 + 1);
    int32_t *par = out_parents + (size_t)b * N, *tok = out_tokens + (size_t)b * N;
    uint8_t *mask = out_mask + (size_t)b * N * N;
    memset(mask, 0, (size_t)N * N);
    if (!parents_ok(p1, n1) || !parents_ok(p2, n2)) {
      for (int i = 0; i < N; ++i) par[i] = tok[i] = -1;
      out_conf[2 * b] = out_conf[2 * b + 1] = 0.0;
      out_route[b] = -1;
      continue;
    }
    for (int i = 0; i <= n1; ++i) {
      par[i] = p1[i];
      tok[i] = t1[i];
    }
    for (int i = 1; i <= n2; ++i) {
      par[n1 + i] = p2[i] == 0 ? 0 : p2[i] + n1;
      tok[n1 + i] = t2[i];
    }
    for (int i = 0; i < N; ++i)
      for (int j = i; j >= 0; j = par[j]) mask[(size_t)i * N + j] = 1;
    double s1 = 0.0, s2 = 0.0;
    for (int i = 1; i <= n1; ++i) s1 += (double)c1[i];
    for (int i = 1; i <= n2; ++i) s2 += (double)c2[i];
    const double m1 = n1 > 0 ? s1 / n1 : 0.0, m2 = n2 > 0 ? s2 / n2 : 0.0;
    out_conf[2 * b] = m1;
    out_conf[2 * b + 1] = m2;
    out_route[b] = m2 > m1 ? 1 : 0;
  }
  return 0;
}
