/*
 * AirCache oracle: a plain, slow, single-threaded CPU implementation, in
 * double precision, of the post-prefill visual KV-cache compression pass.
 *
 * Source of every step: the paper-notes page "AirCache: Activating Inter-Modal
 * Relevancy KV Cache Compression for Efficient Large Vision-Language Model
 * Inference" (ICCV 2025), sections "Elite Observation Window" (key design 1),
 * "Layer-wise KV Cache Budget Allocation" (key design 2) and the training-free
 * procedure (prefill, then one budget-and-compress step over all layers).
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers. The HIP library never
 * links, loads or calls this file, and this file includes nothing from it.
 *
 * Every floating-point quantity is computed in double precision from inputs
 * widened exactly (float32 or bfloat16 bit patterns). Build with
 * -ffp-contract=off so that no multiply-add is fused behind the reader's back.
 *
 * Readings where the page leaves a step open (each also listed in the design
 * notes of the repository):
 *  - multi-head: per-head attention with D = head_dim; query head h reads
 *    KV head h / (H_q / H_kv); step 1 averages the per-head softmax rows over
 *    the query heads and yields one elite set per (layer, sample); step 2
 *    averages over all query heads and all elite rows;
 *  - step 2 normalises each elite row over the N_v visual keys plus the N_tk
 *    elite text keys only, with no causal mask;
 *  - skewness uses the sample standard deviation (n - 1); sigma = 0 gives 0;
 *  - cross-layer normalisation is mean-1 scaling per sample; skewness is first
 *    shifted by min(0, min_l s_k) so that it is non-negative (all-zero after
 *    the shift gives 1 for every layer);
 *  - r = ratio * N_v as a real number, floored once at the end, clamped to
 *    [0, N_v];
 *  - top-r selection by I_v, equal scores go to the lower index, kept indices
 *    are emitted in ascending order;
 *  - compacted layout per (layer, sample, KV head): kept visual rows in
 *    ascending order, then all text rows, samples packed one after another;
 *  - the per-KV-head selection (group-wise top-K) keeps each KV head's own
 *    top-r_hat by the I_v of its query heads, with the layer's budget r_hat
 *    set from the I_v over all query heads as in the shared selection;
 *  - int8 quantisation of the kept cache: symmetric range [-127, 127], one
 *    scale per (layer, sample, KV head) for K and one for V, codes rounded
 *    half to even in float32;
 *  - the visual observation window: the last k visual tokens as the
 *    observation rows, each normalised over the N_v visual keys.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int L, B, Hq, Hkv, D, Nv, Nt;
  int dtype; /* 0: float32, 1: bfloat16 bit patterns */
  double alpha;
  double ratio;
} orc_desc;

static double elem(const void *base, size_t i, int dtype) {
  if (dtype == 0) return (double)((const float *)base)[i];
  uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static size_t q_index(const orc_desc *w, int b, int h, int j) {
  return (((size_t)b * w->Hq + h) * w->Nt + j) * (size_t)w->D;
}

static size_t k_index(const orc_desc *w, int b, int g, int s) {
  return (((size_t)b * w->Hkv + g) * (size_t)(w->Nv + w->Nt) + s) * (size_t)w->D;
}

/* Scaled dot product q_{b,h,jq} . k_{b,g,s} / sqrt(D). */
static double logit(const orc_desc *w, const void *q_l, const void *k_l, int b,
                    int h, int jq, int g, int s) {
  size_t qi = q_index(w, b, h, jq), ki = k_index(w, b, g, s);
  double acc = 0.0;
  for (int d = 0; d < w->D; ++d) acc += elem(q_l, qi + d, w->dtype) * elem(k_l, ki + d, w->dtype);
  return acc / sqrt((double)w->D);
}

/* Softmax of z[0..n) in place: exp(z - max) / sum. */
static void softmax(double *z, int n) {
  double m = z[0];
  for (int i = 1; i < n; ++i)
    if (z[i] > m) m = z[i];
  double s = 0.0;
  for (int i = 0; i < n; ++i) {
    z[i] = exp(z[i] - m);
    s += z[i];
  }
  for (int i = 0; i < n; ++i) z[i] /= s;
}

/*
 * Step 1, elite observation window (text-only attention and the elite set).
 * For every query head: the softmax row of the last text query over the N_t
 * text keys. pbar = mean of those rows over the query heads. The elite set is
 * { j : pbar[j] >= alpha * max(pbar) }, written in ascending order.
 * Returns N_tk. pbar receives N_t values.
 */
int orc_elite_select(const orc_desc *w, const void *q_l, const void *k_l, int b,
                     double *pbar, int32_t *elite) {
  const int G = w->Hq / w->Hkv;
  double *z = (double *)malloc(sizeof(double) * (size_t)w->Nt);
  for (int j = 0; j < w->Nt; ++j) pbar[j] = 0.0;
  for (int h = 0; h < w->Hq; ++h) {
    int g = h / G;
    for (int j = 0; j < w->Nt; ++j) z[j] = logit(w, q_l, k_l, b, h, w->Nt - 1, g, w->Nv + j);
    softmax(z, w->Nt);
    for (int j = 0; j < w->Nt; ++j) pbar[j] += z[j];
  }
  for (int j = 0; j < w->Nt; ++j) pbar[j] /= (double)w->Hq;
  double pmax = pbar[0];
  for (int j = 1; j < w->Nt; ++j)
    if (pbar[j] > pmax) pmax = pbar[j];
  int n = 0;
  for (int j = 0; j < w->Nt; ++j)
    if (pbar[j] >= w->alpha * pmax) elite[n++] = j;
  free(z);
  return n;
}

/*
 * Step 2, cross-modal attention of the elite queries and visual importance.
 * For every query head h and elite query j: softmax over the columns
 * [visual keys 0..N_v-1, elite text keys], then I_v[i] is the mean over all
 * (h, j) rows of the probability at visual column i.
 */
void orc_cross_score(const orc_desc *w, const void *q_l, const void *k_l, int b,
                     const int32_t *elite, int ntk, double *iv) {
  const int G = w->Hq / w->Hkv;
  const int ncol = w->Nv + ntk;
  double *z = (double *)malloc(sizeof(double) * (size_t)ncol);
  for (int i = 0; i < w->Nv; ++i) iv[i] = 0.0;
  for (int h = 0; h < w->Hq; ++h) {
    int g = h / G;
    for (int e = 0; e < ntk; ++e) {
      int jq = elite[e];
      for (int c = 0; c < w->Nv; ++c) z[c] = logit(w, q_l, k_l, b, h, jq, g, c);
      for (int e2 = 0; e2 < ntk; ++e2) z[w->Nv + e2] = logit(w, q_l, k_l, b, h, jq, g, w->Nv + elite[e2]);
      softmax(z, ncol);
      for (int i = 0; i < w->Nv; ++i) iv[i] += z[i];
    }
  }
  for (int i = 0; i < w->Nv; ++i) iv[i] /= (double)w->Hq * (double)ntk;
  free(z);
}

/*
 * Step 2 with one selection per KV head (the group-wise top-K of the
 * edge-device survey page, section 10.1 on GQA/MQA: the query heads that
 * share a KV head decide together). For KV head g, I_v^g[i] is the mean,
 * over the G query heads h with h / G = g and the elite rows j, of the
 * probability at visual column i of the same row softmax as orc_cross_score.
 * iv_g: [H_kv][N_v].
 */
void orc_cross_score_groups(const orc_desc *w, const void *q_l, const void *k_l, int b,
                            const int32_t *elite, int ntk, double *iv_g) {
  const int G = w->Hq / w->Hkv;
  const int ncol = w->Nv + ntk;
  double *z = (double *)malloc(sizeof(double) * (size_t)ncol);
  for (int i = 0; i < w->Hkv * w->Nv; ++i) iv_g[i] = 0.0;
  for (int h = 0; h < w->Hq; ++h) {
    int g = h / G;
    double *row_sum = iv_g + (size_t)g * w->Nv;
    for (int e = 0; e < ntk; ++e) {
      int jq = elite[e];
      for (int c = 0; c < w->Nv; ++c) z[c] = logit(w, q_l, k_l, b, h, jq, g, c);
      for (int e2 = 0; e2 < ntk; ++e2) z[w->Nv + e2] = logit(w, q_l, k_l, b, h, jq, g, w->Nv + elite[e2]);
      softmax(z, ncol);
      for (int i = 0; i < w->Nv; ++i) row_sum[i] += z[i];
    }
  }
  for (int i = 0; i < w->Hkv * w->Nv; ++i) iv_g[i] /= (double)G * (double)ntk;
  free(z);
}

/*
 * Step 3, layer strength and skewness of I_v.
 * s_t = sum I_v; s_k = n / ((n-1)(n-2)) * sum(((I_v - mu) / sigma)^3) with mu
 * the mean and sigma the sample standard deviation; sigma = 0 gives s_k = 0.
 */
void orc_layer_stats(const double *iv, int n, double *s_t, double *s_k) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += iv[i];
  /* sigma and the skewness do not change when every value is shifted by the
   * same amount; working on y = I_v - I_v[0] keeps an exactly constant vector
   * exactly zero, so its sigma is 0 rather than a rounding residue. */
  const double x0 = iv[0];
  double sy = 0.0;
  for (int i = 0; i < n; ++i) sy += iv[i] - x0;
  double mu = sy / (double)n;
  double v = 0.0;
  for (int i = 0; i < n; ++i) v += ((iv[i] - x0) - mu) * ((iv[i] - x0) - mu);
  double sigma = sqrt(v / (double)(n - 1));
  double k3 = 0.0;
  if (sigma > 0.0) {
    for (int i = 0; i < n; ++i) {
      double t = ((iv[i] - x0) - mu) / sigma;
      k3 += t * t * t;
    }
    k3 *= (double)n / ((double)(n - 1) * (double)(n - 2));
  }
  *s_t = s;
  *s_k = k3;
}

/*
 * Step 4, budget of every layer of one sample (L layers, ascending order).
 * s't = s_t * L / sum(s_t); shift m = min(0, min s_k), u = s_k - m,
 * s'k = u * L / sum(u) (1 for every layer when sum(u) = 0);
 * x = 0.5 * (s't + s'k) * (ratio * N_v); budget = clamp(floor(x), 0, N_v).
 * mode picks the allocation rule: 0 the page's (strength and skewness,
 * "Layer-wise KV Cache Budget Allocation", the r_hat equation); the variants
 * of that section's allocation ablation table, read as the same equation with
 * one term: 1 uniform, x = ratio * N_v; 2 strength only, x = s't * ratio *
 * N_v; 3 skewness only, x = s'k * ratio * N_v; 4 the pyramid allocation the
 * table names (budgets falling with depth; the page gives no formula), read
 * as the plainest linear pyramid with the same mean, x = r 2 (L - l) / (L + 1)
 * for layer l = 0 .. L - 1 (the sum over layers is L r, the first layer gets
 * 2 L r / (L + 1), the last 2 r / (L + 1)).
 */
void orc_budget(const double *s_t, const double *s_k, int L, double ratio, int Nv, int mode,
                double *x, int32_t *budget) {
  double st_sum = 0.0, m = 0.0, u_sum = 0.0;
  for (int l = 0; l < L; ++l) st_sum += s_t[l];
  for (int l = 0; l < L; ++l)
    if (s_k[l] < m) m = s_k[l];
  for (int l = 0; l < L; ++l) u_sum += s_k[l] - m;
  double r = ratio * (double)Nv;
  for (int l = 0; l < L; ++l) {
    double stn = s_t[l] * (double)L / st_sum;
    double skn = (u_sum > 0.0) ? (s_k[l] - m) * (double)L / u_sum : 1.0;
    x[l] = mode == 1   ? r
           : mode == 2 ? stn * r
           : mode == 3 ? skn * r
           : mode == 4 ? r * (double)(2 * (L - l)) / (double)(L + 1)
                       : 0.5 * (stn + skn) * r;
    double f = floor(x[l]);
    if (!(f > 0.0)) f = 0.0; /* also maps NaN to 0 */
    if (f > (double)Nv) f = (double)Nv;
    budget[l] = (int32_t)f;
  }
}

typedef struct {
  double score;
  int32_t index;
} scored;

static int by_score_desc(const void *a, const void *b) {
  const scored *x = (const scored *)a, *y = (const scored *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->index > y->index) - (x->index < y->index);
}

static int by_int_asc(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/*
 * Step 5, top-k selection of the visual tokens of one layer: order by
 * (I_v descending, index ascending), keep the first k, write them ascending.
 */
void orc_topk(const double *iv, int n, int k, int32_t *kept) {
  scored *s = (scored *)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) {
    s[i].score = iv[i];
    s[i].index = i;
  }
  qsort(s, (size_t)n, sizeof(scored), by_score_desc);
  for (int i = 0; i < k; ++i) kept[i] = s[i].index;
  qsort(kept, (size_t)k, sizeof(int32_t), by_int_asc);
  free(s);
}

/*
 * Step 6, compaction of one sample of one layer: for each KV head, the kept
 * visual rows (in the order given) followed by all text rows, copied byte for
 * byte into out_seg, laid out [H_kv][k + N_t][D].
 */
void orc_gather(const orc_desc *w, const void *src_l, int b, const int32_t *kept, int k,
                void *out_seg) {
  const size_t esz = (w->dtype == 0) ? 4 : 2;
  const size_t row = (size_t)w->D * esz;
  const char *src = (const char *)src_l;
  char *dst = (char *)out_seg;
  for (int g = 0; g < w->Hkv; ++g) {
    for (int i = 0; i < k; ++i) {
      memcpy(dst, src + k_index(w, b, g, kept[i]) * esz, row);
      dst += row;
    }
    for (int j = 0; j < w->Nt; ++j) {
      memcpy(dst, src + k_index(w, b, g, w->Nv + j) * esz, row);
      dst += row;
    }
  }
}

/*
 * Step 6 with one selection per KV head: as orc_gather, with head g's kept
 * visual rows read from kept_g + g * kept_stride (k of them, in the order
 * given).
 */
void orc_gather_groups(const orc_desc *w, const void *src_l, int b, const int32_t *kept_g, int kept_stride,
                       int k, void *out_seg) {
  const size_t esz = (w->dtype == 0) ? 4 : 2;
  const size_t row = (size_t)w->D * esz;
  const char *src = (const char *)src_l;
  char *dst = (char *)out_seg;
  for (int g = 0; g < w->Hkv; ++g) {
    const int32_t *kept = kept_g + (size_t)g * kept_stride;
    for (int i = 0; i < k; ++i) {
      memcpy(dst, src + k_index(w, b, g, kept[i]) * esz, row);
      dst += row;
    }
    for (int j = 0; j < w->Nt; ++j) {
      memcpy(dst, src + k_index(w, b, g, w->Nv + j) * esz, row);
      dst += row;
    }
  }
}

/*
 * int8 quantisation of one head's kept cache, after the token compression
 * (the UniCache blog, section 6.3 on stacking quantisation with compression:
 * compress first, then quantise; one scale per head, the head's largest
 * absolute value over the quantisation range). The page fixes neither the
 * range nor the rounding; read as the symmetric range [-127, 127], scale
 * s = max|x| / 127 and code q = round-half-to-even(x / s), with s = 0 and
 * every code 0 for an all-zero head. The quantised code is an integer
 * decided by floating point, so it is decided in float32 (the inputs are
 * float32, or bfloat16, which widens to float32 exactly): one float32
 * division per element, correctly rounded, then rintf.
 * seg: n elements in the descriptor's dtype; codes: n int8; *scale: s.
 */
void orc_quantize_i8(const void *seg, int dtype, size_t n, int8_t *codes, float *scale) {
  float m = 0.0f;
  for (size_t i = 0; i < n; ++i) {
    const float x = (float)elem(seg, i, dtype);
    const float a = x < 0.0f ? -x : x;
    if (a > m) m = a;
  }
  const float s = m / 127.0f;
  for (size_t i = 0; i < n; ++i) {
    const float x = (float)elem(seg, i, dtype);
    float q = 0.0f;
    if (s > 0.0f) q = rintf(x / s);
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    codes[i] = (int8_t)q;
  }
  *scale = s;
}

/*
 * Decode attention over one compacted (layer, sample) segment, the consumer
 * of the compacted cache: the KV-cache primer page (devpress.csdn.net),
 * section 2.1 "到底缓存什么？", the o_t equation, with one new query per head
 * and no mask (the incremental step sees only cached positions, section 2.2).
 * For each query head h, with KV head g = h / (H_q / H_kv):
 *   o_h = softmax(q_h . K_g^T / sqrt(D)) V_g
 * over the n rows of head g in the segment, laid out [H_kv][n][D] as
 * orc_gather writes it. q: [H_q][D] in the descriptor's dtype; o: [H_q][D].
 */
void orc_decode_attention(const orc_desc *w, const void *k_seg, const void *v_seg, int n, const void *q,
                          double *o) {
  const int G = w->Hq / w->Hkv, D = w->D;
  const double scale = sqrt((double)D);
  double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int h = 0; h < w->Hq; ++h) {
    const int g = h / G;
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += elem(q, (size_t)h * D + d, w->dtype) * elem(k_seg, ((size_t)g * n + j) * D + d, w->dtype);
      z[j] = acc / scale;
    }
    softmax(z, n);
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += z[j] * elem(v_seg, ((size_t)g * n + j) * D + d, w->dtype);
      o[(size_t)h * D + d] = acc;
    }
  }
  free(z);
}

/*
 * Decode attention over one segment of the int8 cache: orc_decode_attention
 * with every cached value read as code * scale (the quantisation's reading,
 * value = code times the scale of its KV head, for K and for V), dequantised
 * exactly in double precision. kq_seg, vq_seg: int8 [H_kv][n][D]; k_scale,
 * v_scale: [H_kv]; q: [H_q][D] in the descriptor's dtype; o: [H_q][D].
 */
void orc_decode_attention_i8(const orc_desc *w, const int8_t *kq_seg, const int8_t *vq_seg, const float *k_scale,
                             const float *v_scale, int n, const void *q, double *o) {
  const int G = w->Hq / w->Hkv, D = w->D;
  const double scale = sqrt((double)D);
  double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int h = 0; h < w->Hq; ++h) {
    const int g = h / G;
    const double ks = (double)k_scale[g], vs = (double)v_scale[g];
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += elem(q, (size_t)h * D + d, w->dtype) * ((double)kq_seg[((size_t)g * n + j) * D + d] * ks);
      z[j] = acc / scale;
    }
    softmax(z, n);
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += z[j] * ((double)vq_seg[((size_t)g * n + j) * D + d] * vs);
      o[(size_t)h * D + d] = acc;
    }
  }
  free(z);
}

/*
 * The window ablation's visual window (AirCache paper-notes page, "消融实验",
 * the window table's visual-window row, read with "Elite Observation Window"):
 * the observation rows are the last kwin visual tokens instead of the elite
 * text tokens. Each such row's softmax runs over the N_v visual keys (the
 * window's own keys are among them; no causal mask, as for the elite rows),
 * and I_v[i] is the mean over every query head and window row of the
 * probability at visual key i. With iv_groups non-NULL, also the mean over
 * the query heads of each KV head only ([H_kv][N_v]).
 * q_all: [B][H_q][N_v + N_t][D] (every position's query); k_l as elsewhere.
 */
void orc_visual_window(const orc_desc *w, const void *q_all, const void *k_l, int b, int kwin, double *iv,
                       double *iv_groups) {
  const int G = w->Hq / w->Hkv, D = w->D, S = w->Nv + w->Nt;
  double *z = (double *)malloc(sizeof(double) * (size_t)w->Nv);
  for (int i = 0; i < w->Nv; ++i) iv[i] = 0.0;
  if (iv_groups)
    for (int i = 0; i < w->Hkv * w->Nv; ++i) iv_groups[i] = 0.0;
  for (int h = 0; h < w->Hq; ++h) {
    const int g = h / G;
    const size_t qh = ((size_t)b * w->Hq + h) * (size_t)S;
    for (int r = 0; r < kwin; ++r) {
      const int jq = w->Nv - kwin + r;
      for (int c = 0; c < w->Nv; ++c) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
          acc += elem(q_all, (qh + jq) * D + d, w->dtype) * elem(k_l, k_index(w, b, g, c) + d, w->dtype);
        z[c] = acc / sqrt((double)D);
      }
      softmax(z, w->Nv);
      for (int c = 0; c < w->Nv; ++c) {
        iv[c] += z[c];
        if (iv_groups) iv_groups[(size_t)g * w->Nv + c] += z[c];
      }
    }
  }
  for (int c = 0; c < w->Nv; ++c) iv[c] /= (double)w->Hq * (double)kwin;
  if (iv_groups)
    for (int i = 0; i < w->Hkv * w->Nv; ++i) iv_groups[i] /= (double)G * (double)kwin;
  free(z);
}

/*
 * Prefill attention of one layer and sample, the attention whose keys the
 * pass later scores: the KV-cache primer page (devpress.csdn.net), section
 * 2.1 "到底缓存什么？", the o_t equation applied at every position t of the
 * regrouped sequence (visual tokens first, then text), so position t attends
 * to the keys 0..t:
 *   o_{h,t} = softmax(q_{h,t} . K_g[0..t]^T / sqrt(D)) V_g[0..t],  g = h / (H_q / H_kv).
 * q_all: [B][H_q][N_v + N_t][D] (every position's query); k_l, v_l:
 * [B][H_kv][N_v + N_t][D]; rows row0 .. row0 + nrows - 1 of every query head
 * of sample b go to o [H_q][nrows][D].
 */
void orc_prefill_attention(const orc_desc *w, const void *q_all, const void *k_l, const void *v_l, int b,
                           int row0, int nrows, double *o) {
  const int G = w->Hq / w->Hkv, D = w->D, S = w->Nv + w->Nt;
  const double scale = sqrt((double)D);
  double *z = (double *)malloc(sizeof(double) * (size_t)S);
  for (int h = 0; h < w->Hq; ++h) {
    const int g = h / G;
    const size_t qh = ((size_t)b * w->Hq + h) * (size_t)S;
    for (int r = 0; r < nrows; ++r) {
      const int t = row0 + r;
      for (int s = 0; s <= t; ++s) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
          acc += elem(q_all, (qh + t) * D + d, w->dtype) * elem(k_l, k_index(w, b, g, s) + d, w->dtype);
        z[s] = acc / scale;
      }
      softmax(z, t + 1);
      for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int s = 0; s <= t; ++s) acc += z[s] * elem(v_l, k_index(w, b, g, s) + d, w->dtype);
        o[((size_t)h * nrows + r) * D + d] = acc;
      }
    }
  }
  free(z);
}

/*
 * The whole pass. Arrays indexed [l][b] are row-major with B columns.
 *   elite [L][B][N_t] (first n_elite valid), pbar [L][B][N_t],
 *   iv [L][B][N_v], s_t, s_k, x [L][B], budget [L][B],
 *   out_off [L][B+1] element offsets of each sample's segment in the layer,
 *   kept [L][B][N_v] (first budget valid).
 * k_out / v_out: per-layer output buffers, or NULL to skip compaction.
 * Returns 0, or -1 on an invalid descriptor.
 */
int orc_run(const orc_desc *w, const void *const *q, const void *const *k,
            const void *const *v, int32_t *elite, int32_t *n_elite, double *pbar,
            double *iv, double *s_t, double *s_k, double *x, int32_t *budget,
            int64_t *out_off, int32_t *kept, void *const *k_out, void *const *v_out) {
  if (w->L < 1 || w->B < 1 || w->Hq < 1 || w->Hkv < 1 || w->Hq % w->Hkv != 0 || w->D < 1 ||
      w->Nv < 3 || w->Nt < 1 || (w->dtype != 0 && w->dtype != 1))
    return -1;
  const int L = w->L, B = w->B;
  for (int l = 0; l < L; ++l) {
    for (int b = 0; b < B; ++b) {
      size_t lb = (size_t)l * B + b;
      int32_t *el = elite + lb * w->Nt;
      int ntk = orc_elite_select(w, q[l], k[l], b, pbar + lb * w->Nt, el);
      n_elite[lb] = ntk;
      orc_cross_score(w, q[l], k[l], b, el, ntk, iv + lb * w->Nv);
      orc_layer_stats(iv + lb * w->Nv, w->Nv, &s_t[lb], &s_k[lb]);
    }
  }
  double *st = (double *)malloc(sizeof(double) * (size_t)L);
  double *sk = (double *)malloc(sizeof(double) * (size_t)L);
  double *xx = (double *)malloc(sizeof(double) * (size_t)L);
  int32_t *bb = (int32_t *)malloc(sizeof(int32_t) * (size_t)L);
  for (int b = 0; b < B; ++b) {
    for (int l = 0; l < L; ++l) {
      st[l] = s_t[(size_t)l * B + b];
      sk[l] = s_k[(size_t)l * B + b];
    }
    orc_budget(st, sk, L, w->ratio, w->Nv, 0, xx, bb);
    for (int l = 0; l < L; ++l) {
      x[(size_t)l * B + b] = xx[l];
      budget[(size_t)l * B + b] = bb[l];
    }
  }
  free(st);
  free(sk);
  free(xx);
  free(bb);
  for (int l = 0; l < L; ++l) {
    int64_t off = 0;
    for (int b = 0; b < B; ++b) {
      size_t lb = (size_t)l * B + b;
      out_off[(size_t)l * (B + 1) + b] = off;
      orc_topk(iv + lb * w->Nv, w->Nv, budget[lb], kept + lb * w->Nv);
      const size_t esz = (w->dtype == 0) ? 4 : 2;
      if (k_out) orc_gather(w, k[l], b, kept + lb * w->Nv, budget[lb], (char *)k_out[l] + (size_t)off * esz);
      if (v_out) orc_gather(w, v[l], b, kept + lb * w->Nv, budget[lb], (char *)v_out[l] + (size_t)off * esz);
      off += (int64_t)w->Hkv * (budget[lb] + w->Nt) * w->D;
    }
    out_off[(size_t)l * (B + 1) + B] = off;
  }
  return 0;
}
