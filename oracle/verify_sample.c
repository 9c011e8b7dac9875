/*
 * verify_sample.c -- CPU oracle of the verify step's sampling epilogue
 * (test infrastructure only; the product library neither links nor calls
 * it, and shares no code with it).
 *
 * What is computed, per verify row m (Splash engine article, section
 * "Exact, up to top-32"; qwen-spec page, section on the fused sampling
 * kernel and the sampling paragraph after it):
 *
 *  1. Candidates: the top_k (1..32) logits of the row, ordered by value,
 *     larger first, equal values by smaller token index (a reading: the page
 *     does not say how ties are broken).
 *  2. Target probabilities p over the candidates: temperature T over those
 *     entries (softmax of logit / T), truncated to the shortest prefix whose
 *     mass reaches top_p, renormalised.  Tokens outside the prefix have p = 0.
 *     T == 0 is greedy: p is 1 on the first candidate (the argmax).
 *  3. Accept test of the drafted token d with the draft's probability q(d):
 *     accept when u * q(d) < p(d) (u uniform in [0, 1), given).
 *  4. On rejection a token is drawn from the residual max(p - q, 0),
 *     normalised, by inverting its cumulative sum at v * R (v uniform in
 *     [0, 1), given; R the residual mass), scanning the candidates in their
 *     order and taking the first whose cumulative sum exceeds v * R.  If the
 *     residual has no mass (possible only through rounding) the same
 *     inversion is applied to p.  The emitted token is d when accepted, the
 *     drawn token otherwise.
 *
 * Arithmetic is IEEE double without contraction; the margin of each discrete
 * decision (accept test, draw) is returned so that a test can tell a clear
 * decision from one inside rounding distance.
 *
 * Status codes: 0 ok, -1 invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define VS_MAX_TOPK 32
#define VS_MAX_DRAFT 16

typedef struct {
  float value;
  int32_t index;
} vs_entry;

/* larger value first; equal values: smaller index first */
static int vs_order(const void *a, const void *b) {
  const vs_entry *x = (const vs_entry *)a;
  const vs_entry *y = (const vs_entry *)b;
  if (x->value > y->value) return -1;
  if (x->value < y->value) return 1;
  return (x->index > y->index) - (x->index < y->index);
}

/* Step 1: the k first entries of each row in the candidate order. */
int vs_topk(const float *logits, int M, int64_t V, int k, int32_t *idx,
            float *val) {
  if (logits == NULL || idx == NULL || val == NULL || M < 1 || V < 1 ||
      k < 1 || k > VS_MAX_TOPK || k > V)
    return -1;
  vs_entry *row = (vs_entry *)malloc((size_t)V * sizeof(vs_entry));
  if (row == NULL) return -1;
  for (int m = 0; m < M; ++m) {
    for (int64_t i = 0; i < V; ++i) {
      row[i].value = logits[(size_t)m * (size_t)V + (size_t)i];
      row[i].index = (int32_t)i;
    }
    qsort(row, (size_t)V, sizeof(vs_entry), vs_order);
    for (int i = 0; i < k; ++i) {
      idx[(size_t)m * k + i] = row[i].index;
      val[(size_t)m * k + i] = row[i].value;
    }
  }
  free(row);
  return 0;
}

/* q(t) from the draft's candidate list of one row (0 when absent). */
static double draft_prob(const int32_t *didx, const double *dq, int kd,
                         int32_t t) {
  for (int j = 0; j < kd; ++j)
    if (didx[j] == t) return dq[j];
  return 0.0;
}

/*
 * Steps 2-4 for M rows whose candidates (k of them, in candidate order) are
 * given.  Outputs per row: p[k] (0 beyond the kept prefix), greedy token,
 * accept flag, emitted token, and the two margins:
 *   accept_margin = p(d) - u q(d)   (the test accepts when it is > 0);
 *   draw_margin   = min over candidates i of |C_i - v R| / R, C_i the
 *                   cumulative residual (or p) sum through i -- the relative
 *                   distance of the draw point from the nearest boundary
 *                   (1 when no draw was made).
 */
int vs_sample(const int32_t *top_idx, const float *top_val, int M, int k,
              double T, double top_p, const int32_t *draft_tok,
              const int32_t *draft_idx, const double *draft_q, int kd,
              const double *u, const double *v, double *p_out,
              int32_t *greedy, int32_t *accept, int32_t *token,
              double *accept_margin, double *draw_margin) {
  if (top_idx == NULL || top_val == NULL || M < 1 || k < 1 ||
      k > VS_MAX_TOPK || kd < 0 || kd > VS_MAX_DRAFT || !(T >= 0.0) ||
      !(top_p > 0.0 && top_p <= 1.0) || draft_tok == NULL || u == NULL ||
      v == NULL || p_out == NULL || greedy == NULL || accept == NULL ||
      token == NULL || accept_margin == NULL || draw_margin == NULL ||
      (kd > 0 && (draft_idx == NULL || draft_q == NULL)))
    return -1;
  for (int m = 0; m < M; ++m) {
    const int32_t *ti = top_idx + (size_t)m * k;
    const float *tv = top_val + (size_t)m * k;
    double *p = p_out + (size_t)m * k;
    const int32_t *di = kd > 0 ? draft_idx + (size_t)m * kd : NULL;
    const double *dq = kd > 0 ? draft_q + (size_t)m * kd : NULL;

    /* step 2: target probabilities */
    if (T == 0.0) {
      p[0] = 1.0;
      for (int i = 1; i < k; ++i) p[i] = 0.0;
    } else {
      double z = 0.0;
      for (int i = 0; i < k; ++i) {
        p[i] = exp(((double)tv[i] - (double)tv[0]) / T);
        z += p[i];
      }
      for (int i = 0; i < k; ++i) p[i] /= z;
      int n = k;
      double c = 0.0;
      for (int i = 0; i < k; ++i) {
        c += p[i];
        if (c >= top_p) {
          n = i + 1;
          break;
        }
      }
      double kept = 0.0;
      for (int i = 0; i < n; ++i) kept += p[i];
      for (int i = 0; i < k; ++i) p[i] = i < n ? p[i] / kept : 0.0;
    }
    greedy[m] = ti[0];

    /* step 3: accept test of the drafted token */
    const int32_t d = draft_tok[m];
    double pd = 0.0;
    for (int i = 0; i < k; ++i)
      if (ti[i] == d) pd = p[i];
    const double qd = kd > 0 ? draft_prob(di, dq, kd, d) : 0.0;
    accept_margin[m] = pd - u[m] * qd;
    accept[m] = u[m] * qd < pd;
    draw_margin[m] = 1.0;
    if (accept[m]) {
      token[m] = d;
      continue;
    }

    /* step 4: residual draw */
    double r[VS_MAX_TOPK];
    double R = 0.0;
    for (int i = 0; i < k; ++i) {
      const double qi = kd > 0 ? draft_prob(di, dq, kd, ti[i]) : 0.0;
      r[i] = p[i] > qi ? p[i] - qi : 0.0;
      R += r[i];
    }
    if (!(R > 0.0)) {
      for (int i = 0; i < k; ++i) r[i] = p[i];
      R = 1.0;
    }
    const double target = v[m] * R;
    int pick = -1;
    double c = 0.0, closest = INFINITY;
    for (int i = 0; i < k; ++i) {
      if (r[i] <= 0.0) continue;
      c += r[i];
      const double gap = fabs(c - target) / R;
      if (gap < closest) closest = gap;
      if (pick < 0 && c > target) pick = i;
    }
    if (pick < 0) /* rounding left the point past the last boundary */
      for (int i = k - 1; i >= 0; --i)
        if (r[i] > 0.0) {
          pick = i;
          break;
        }
    token[m] = ti[pick];
    draw_margin[m] = closest;
  }
  return 0;
}
