/*
 * gdn_state.c -- CPU oracle of the Gated DeltaNet state step of a verify pass
 * (test infrastructure only; the product library neither links nor calls it,
 * and shares no code with it).
 *
 * The pages (Splash engine article, section "What one step reads"; qwen-spec
 * page, the paragraph on the hybrid model) fix the state: per recurrent layer
 * and value head a 128 x 128 fp32 matrix, read and written back every step;
 * each tree node's output comes from the shared state after the context plus
 * the updates along the node's own path; after the check the accepted path is
 * written into the state.  The update itself is not printed there; the
 * reading taken is the published gated delta rule, per token t with keys and
 * queries k_t, q_t (length dk), value v_t (length dv), gate alpha_t and
 * writing strength beta_t:
 *
 *     S <- alpha_t * S * (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T
 *     o_t = S q_t            (S is dv x dk, row-major; o after the update)
 *
 * Key heads: q and k come per key head; with H value heads and Hk key heads
 * (Hk divides H), value head h reads key head h / (H / Hk).
 *
 * Tree: node i has parent[i] (-1 for a child of the context's last token;
 * parents precede children).  Node i's output is o_i = S_i q_i, where S_i is
 * the state after applying, in order from the root down, the updates of every
 * node on the path to i, i included.  Commit: the updates of the accepted
 * nodes path[0..a-1] are applied to the state in that order.
 *
 * Everything is computed straight from the definition with full matrices in
 * IEEE double, no contraction.  Status: 0 ok, -1 invalid argument.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* S (dv x dk, double) <- alpha S (I - beta k k^T) + beta v k^T */
static void apply_update(double *S, int dv, int dk, const float *k,
                         const float *v, double alpha, double beta) {
  double *P = (double *)malloc((size_t)dk * dk * sizeof(double));
  double *T = (double *)malloc((size_t)dv * dk * sizeof(double));
  /* P = I - beta k k^T */
  for (int a = 0; a < dk; ++a)
    for (int b = 0; b < dk; ++b)
      P[a * dk + b] = (a == b ? 1.0 : 0.0) - beta * (double)k[a] * (double)k[b];
  /* T = S P */
  for (int r = 0; r < dv; ++r)
    for (int b = 0; b < dk; ++b) {
      double acc = 0.0;
      for (int a = 0; a < dk; ++a) acc += S[r * dk + a] * P[a * dk + b];
      T[r * dk + b] = acc;
    }
  for (int r = 0; r < dv; ++r)
    for (int b = 0; b < dk; ++b)
      S[r * dk + b] = alpha * T[r * dk + b] + beta * (double)v[r] * (double)k[b];
  free(P);
  free(T);
}

/*
 * Node outputs of one layer: S0 [H][dv][dk], q/k [M][Hk][dk], v [M][H][dv],
 * alpha/beta [M][H], parent [M]; out [M][H][dv] (double).
 */
int gdn_tree_out(const float *S0, int H, int Hk, int dv, int dk, int M,
                 const float *q, const float *k, const float *v,
                 const float *alpha, const float *beta, const int32_t *parent,
                 double *out) {
  if (S0 == NULL || q == NULL || k == NULL || v == NULL || alpha == NULL ||
      beta == NULL || parent == NULL || out == NULL || H < 1 || Hk < 1 ||
      H % Hk != 0 || dv < 1 || dk < 1 || M < 1)
    return -1;
  const int G = H / Hk;
  for (int i = 0; i < M; ++i)
    if (parent[i] < -1 || parent[i] >= i) return -1;
  double *S = (double *)malloc((size_t)dv * dk * sizeof(double));
  int *path = (int *)malloc((size_t)M * sizeof(int));
  for (int i = 0; i < M; ++i) {
    /* the path root .. i */
    int depth = 0;
    for (int n = i; n >= 0; n = parent[n]) path[depth++] = n;
    for (int h = 0; h < H; ++h) {
      for (int e = 0; e < dv * dk; ++e)
        S[e] = (double)S0[(size_t)h * dv * dk + e];
      for (int s = depth - 1; s >= 0; --s) {
        const int n = path[s];
        apply_update(S, dv, dk, k + ((size_t)n * Hk + h / G) * dk,
                     v + ((size_t)n * H + h) * dv,
                     (double)alpha[(size_t)n * H + h],
                     (double)beta[(size_t)n * H + h]);
      }
      const float *qi = q + ((size_t)i * Hk + h / G) * dk;
      for (int r = 0; r < dv; ++r) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += S[r * dk + c] * (double)qi[c];
        out[((size_t)i * H + h) * dv + r] = acc;
      }
    }
  }
  free(S);
  free(path);
  return 0;
}

/*
 * Commit of the accepted nodes path[0..a-1] (in that order) to L layers of
 * states S [L][H][dv][dk] (double, updated in place); k [L][M][Hk][dk],
 * v [L][M][H][dv], alpha/beta [L][M][H].
 */
int gdn_commit(double *S, int L, int H, int Hk, int dv, int dk, int M,
               const float *k,
               const float *v, const float *alpha, const float *beta,
               const int32_t *path, int a) {
  if (S == NULL || k == NULL || v == NULL || alpha == NULL || beta == NULL ||
      (a > 0 && path == NULL) || L < 1 || H < 1 || Hk < 1 || H % Hk != 0 ||
      dv < 1 || dk < 1 || M < 1 || a < 0 || a > M)
    return -1;
  const int G = H / Hk;
  for (int s = 0; s < a; ++s)
    if (path[s] < 0 || path[s] >= M) return -1;
  for (int l = 0; l < L; ++l)
    for (int h = 0; h < H; ++h) {
      double *Sh = S + ((size_t)l * H + h) * dv * dk;
      for (int s = 0; s < a; ++s) {
        const size_t t = ((size_t)l * M + path[s]) * H + h;
        const size_t tk = ((size_t)l * M + path[s]) * Hk + h / G;
        apply_update(Sh, dv, dk, k + tk * dk, v + t * dv, (double)alpha[t],
                     (double)beta[t]);
      }
    }
  return 0;
}
