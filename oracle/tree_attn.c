/*
 * tree_attn.c -- CPU oracle of tree-verify attention over a paged int8 KV
 * cache (test infrastructure only; the product library neither links nor
 * calls it, and shares no code with it).
 *
 * What the pages fix: the attention layers have 24 query heads, 4 KV heads
 * and head dimension 256 (Splash engine article, the model listing in "The
 * engine hard-codes the model"); a KV page holds 32 tokens in int8 with an
 * fp32 scale per token per head (same article, the section on the paged KV
 * pool); the verify pass reads the cache in place and every tree node sees
 * the context and its own ancestors through a mask (qwen-spec page, Notes and
 * the hybrid-model paragraph).
 *
 * Readings taken where the pages are silent:
 *  - The tree's own keys and values sit in the cache right after the context:
 *    node j at logical position ctx_len + j.
 *  - Node i sees positions p < ctx_len and the tree positions of its
 *    ancestors and of itself: bit j of anc[i] set.
 *  - Logical position p lives in page page_table[p / 32], slot p % 32.  Per
 *    physical page and KV head, keys are [32 tokens][D] int8, values are
 *    stored transposed, [D][32 tokens] int8, and each has one fp32 scale per
 *    token: k = k8 * k_scale, v = v8 * v_scale.
 *  - Query head h reads KV head h / (Hq / Hkv).  Scores are scale * q . k,
 *    then a softmax over the visible positions, output sum_p w_p v_p.
 *  - Queries arrive as bf16 bit patterns [M][Hq][D].
 *
 * Straight from the definition, IEEE double, no blocking.
 *
 * Besides the outputs o[i][h][d] = sum_p w_p v_p[d], it can return
 * absw[i][h][d] = sum_p w_p |v_p[d]|, the same weights applied to the
 * magnitudes of the values.  That sum is the scale of the rounding error of
 * any evaluation that rounds the terms w_p v_p[d] (or w_p times the value
 * scale) to a shorter format before adding them: a term rounded to relative
 * precision u moves the output by at most u * w_p |v_p[d]|.  Pass NULL when
 * it is not needed.
 * Status: 0 ok, -1 invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* physical page of logical position p */
static int64_t page_of(const int32_t *page_table, int64_t p) {
  return page_table[p / 32];
}

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int ta_tree_attention(const uint16_t *q, int M, int Hq, int Hkv, int D,
                      const int8_t *k_pages, const int8_t *v_pages,
                      const float *k_scale, const float *v_scale,
                      const int32_t *page_table, int pool_pages,
                      int64_t ctx_len, const uint32_t *anc, double scale,
                      double *out, double *absw) {
  if (q == NULL || k_pages == NULL || v_pages == NULL || k_scale == NULL ||
      v_scale == NULL || page_table == NULL || anc == NULL || out == NULL ||
      M < 1 || M > 32 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 1 ||
      pool_pages < 1 || ctx_len < 0)
    return -1;
  const int64_t total = ctx_len + M;
  const int64_t lpages = (total + 31) / 32;
  for (int64_t lp = 0; lp < lpages; ++lp)
    if (page_table[lp] < 0 || page_table[lp] >= pool_pages) return -1;
  const int G = Hq / Hkv;
  double *s = (double *)malloc((size_t)total * sizeof(double));
  unsigned char *vis = (unsigned char *)malloc((size_t)total);
  if (s == NULL || vis == NULL) {
    free(s);
    free(vis);
    return -1;
  }
  for (int i = 0; i < M; ++i) {
    for (int64_t p = 0; p < total; ++p)
      vis[p] = p < ctx_len ? 1 : (unsigned char)((anc[i] >> (p - ctx_len)) & 1u);
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const uint16_t *qi = q + ((size_t)i * Hq + h) * D;
      double mx = -INFINITY;
      for (int64_t p = 0; p < total; ++p) {
        if (!vis[p]) continue;
        const int64_t pp = page_of(page_table, p);
        const int slot = (int)(p % 32);
        const size_t base = (size_t)(pp * Hkv + g);
        const double ks = (double)k_scale[base * 32 + slot];
        double dot = 0.0;
        for (int d = 0; d < D; ++d) {
          const int8_t k8 = k_pages[(base * 32 + slot) * D + d];
          dot += bf16_to_double(qi[d]) * ((double)k8 * ks);
        }
        s[p] = scale * dot;
        if (s[p] > mx) mx = s[p];
      }
      double den = 0.0;
      for (int64_t p = 0; p < total; ++p) {
        if (!vis[p]) continue;
        s[p] = exp(s[p] - mx);
        den += s[p];
      }
      double *o = out + ((size_t)i * Hq + h) * D;
      double *ao = absw == NULL ? NULL : absw + ((size_t)i * Hq + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (ao != NULL)
        for (int d = 0; d < D; ++d) ao[d] = 0.0;
      for (int64_t p = 0; p < total; ++p) {
        if (!vis[p]) continue;
        const int64_t pp = page_of(page_table, p);
        const int slot = (int)(p % 32);
        const size_t base = (size_t)(pp * Hkv + g);
        const double vs = (double)v_scale[base * 32 + slot];
        const double w = s[p] / den;
        for (int d = 0; d < D; ++d) {
          const int8_t v8 = v_pages[base * 32 * (size_t)D + (size_t)d * 32 + slot];
          o[d] += w * ((double)v8 * vs);
          if (ao != NULL) ao[d] += w * fabs((double)v8 * vs);
        }
      }
    }
  }
  free(s);
  free(vis);
  return 0;
}
