/*
 * Oracle for prefix-reuse ("bipartite") attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (the HIP library) never calls it and
 * shares no source with it.
 *
 * What it computes is the plain definition of the attention the Bat page
 * ("Bat: Efficient Generative Recommender Serving with Bipartite Attention")
 * describes for generative-recommender prefill:
 *   - neither the history nor the items carry positions, and the two
 *     groups can trade places (section "This paper's idea", and "Why it
 *     works": permutation invariance), so there is no positional encoding
 *     and no causal mask;
 *   - one group (the prefix: a user's history, or a set of cached items)
 *     has its key/value cache built once and reused (section "Problem",
 *     "Why this problem is worth solving"); reusing it is only exact if the
 *     prefix tokens never look at the fresh group, so prefix rows see the
 *     prefix only (the UG-Separation page's abstract keeps user-side tokens
 *     purely user-side so that their computation can be cached);
 *   - the fresh group (the suffix) sees the prefix and itself; attention is
 *     bidirectional inside a group (the GBLA page's abstract: bidirectional
 *     encoder attention).
 * The attention itself is scaled dot-product softmax attention (the pages do
 * not print Bipartite Attention's internals; softmax is the plain reading).
 *
 * Everything is float64, two passes per row (max, then exp-sum and the
 * normalised weighted sum), over contiguous K/V: no tiling, no online
 * softmax, no block table.  Inputs may be float32 or bfloat16 bit patterns;
 * both widen to float64 exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to double. */
static double load_elem(const void *base, int64_t idx, int dtype) {
  if (dtype == ORACLE_F64) return ((const double *)base)[idx];
  if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * General masked softmax attention for one head.
 *   q [n_q, D], k [n_k, D], v [n_k, D] (row-major, dtype as given)
 *   mask [n_q, n_k]: 1 where query i may attend to key j
 *   out [n_q, D], lse [n_q] (natural log) in float64
 * S_ij = scale * <q_i, k_j>;  LSE_i = log sum_{visible j} exp(S_ij);
 * O_i = sum_{visible j} exp(S_ij - LSE_i) v_j.
 * A row with no visible key has LSE = -inf and O = 0 (the empty partial).
 */
void oracle_attention_masked(int n_q, int n_k, int D, int dtype, const void *q,
                             const void *k, const void *v, const uint8_t *mask,
                             double scale, double *out, double *lse) {
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (n_k > 0 ? n_k : 1));
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_q; ++i) {
      /* pass 1: scores of visible keys and their maximum */
      double mx = -INFINITY;
      for (int j = 0; j < n_k; ++j) {
        if (!mask[(int64_t)i * n_k + j]) continue;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += load_elem(q, (int64_t)i * D + d, dtype) *
                 load_elem(k, (int64_t)j * D + d, dtype);
        s[j] = scale * dot;
        if (s[j] > mx) mx = s[j];
      }
      double *o = out + (int64_t)i * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (mx == -INFINITY) {
        lse[i] = -INFINITY;
        continue;
      }
      /* pass 2: log-sum-exp, then the normalised weighted sum of values */
      double sum = 0.0;
      for (int j = 0; j < n_k; ++j)
        if (mask[(int64_t)i * n_k + j]) sum += exp(s[j] - mx);
      double l = mx + log(sum);
      lse[i] = l;
      for (int j = 0; j < n_k; ++j) {
        if (!mask[(int64_t)i * n_k + j]) continue;
        double w = exp(s[j] - l);
        for (int d = 0; d < D; ++d)
          o[d] += w * load_elem(v, (int64_t)j * D + d, dtype);
      }
    }
    free(s);
  }
}

/*
 * Batched prefill, suffix rows only, heads interleaved as in the packed
 * token-major layout [tokens, H, D].
 *
 * For request r:
 *   suffix tokens  rows cu_s[r] .. cu_s[r+1]-1 of q / k_s / v_s
 *   prefix tokens  rows cu_p[r] .. cu_p[r+1]-1 of k_p / v_p, already in the
 *                  order the request sees them (for an item prefix: the
 *                  items' tokens in block-table order)
 * A suffix row sees every prefix token and every suffix token of its own
 * request, so its visible set is the whole concatenated sequence [P; U].
 *
 * Selection: if n_sel < 0 every (suffix row, head) pair is computed and
 * out is [total_suffix, H, D], lse is [H, total_suffix].  Otherwise only the
 * pairs (sel_row[i], sel_head[i]) are computed and out is [n_sel, D], lse is
 * [n_sel].
 */
int oracle_prefill_suffix(int B, int H, int D, int dtype, const void *q,
                          const void *k_s, const void *v_s, const int32_t *cu_s,
                          const void *k_p, const void *v_p, const int32_t *cu_p,
                          double scale, int n_sel, const int32_t *sel_row,
                          const int32_t *sel_head, double *out, double *lse) {
  const int64_t total_s = cu_s[B];
  const int64_t n_pairs = n_sel < 0 ? total_s * H : (int64_t)n_sel;
  int bad = 0;
#pragma omp parallel
  {
    int64_t cap = 0;
    double *s = NULL;
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < n_pairs; ++t) {
      int64_t row;
      int h;
      if (n_sel < 0) {
        row = t / H;
        h = (int)(t % H);
      } else {
        row = sel_row[t];
        h = sel_head[t];
      }
      if (row < 0 || row >= total_s || h < 0 || h >= H) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      /* the request that owns this suffix row */
      int r = 0;
      while (cu_s[r + 1] <= row) ++r;
      const int64_t p0 = cu_p[r], n_p = cu_p[r + 1] - cu_p[r];
      const int64_t s0 = cu_s[r], n_s = cu_s[r + 1] - cu_s[r];
      const int64_t n = n_p + n_s;
      if (n > cap) {
        free(s);
        cap = n;
        s = (double *)malloc(sizeof(double) * cap);
      }
      const int64_t qo = (row * H + h) * D;
      /* pass 1: scores over [P; U] and their maximum */
      double mx = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        const void *kb = j < n_p ? k_p : k_s;
        const int64_t tok = j < n_p ? p0 + j : s0 + (j - n_p);
        const int64_t ko = (tok * H + h) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += load_elem(q, qo + d, dtype) * load_elem(kb, ko + d, dtype);
        s[j] = scale * dot;
        if (s[j] > mx) mx = s[j];
      }
      /* pass 2 */
      double sum = 0.0;
      for (int64_t j = 0; j < n; ++j) sum += exp(s[j] - mx);
      const double l = mx + log(sum);
      double *o = n_sel < 0 ? out + (row * H + h) * D : out + t * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        const void *vb = j < n_p ? v_p : v_s;
        const int64_t tok = j < n_p ? p0 + j : s0 + (j - n_p);
        const int64_t vo = (tok * H + h) * D;
        const double w = exp(s[j] - l);
        for (int d = 0; d < D; ++d) o[d] += w * load_elem(vb, vo + d, dtype);
      }
      if (n_sel < 0)
        lse[(int64_t)h * total_s + row] = l;
      else
        lse[t] = l;
    }
    free(s);
  }
  return bad ? -1 : 0;
}

/* Number of OpenMP threads the library will use (reported beside timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
