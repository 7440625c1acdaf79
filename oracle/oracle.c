/*
 * CPU oracle for level-wise histogram GBDT tree growth (squared error).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this file.  The GPU library never links, calls or
 * includes it, and it shares no code with the GPU library: its own structs,
 * its own loops, its own build line (gcc, -ffp-contract=off, no fast-math).
 *
 * Plain, single-threaded, FP64.  It follows the pages step by step:
 *
 *  - "Module Design: Training Core" (MPSBoost spec), section 2, "Single
 *    Mathematical Semantics": g_i = prediction_i - label_i, h_i = 1,
 *    score(G,H) = G^2/(H+lambda), weight(G,H) = -G/(H+lambda),
 *    gain = 0.5*(score_left + score_right - score_parent) - gamma.
 *  - same page, section 3, "Tree Model": flat node array with feature,
 *    threshold bin, children, leaf value, gain, flags; the stable tie-break
 *    (larger gain, then smaller feature, then smaller threshold bin, then the
 *    first candidate), strict FP64 '>' with no epsilon, gain must be strictly
 *    positive, bin <= threshold_bin goes left, and the parameter / child
 *    constraints (min_samples_leaf, min_child_weight, strictly positive
 *    Hessian on both children; violators never compete).
 *  - same page, section 6, "Tree Growth": the seven level-wise steps.
 *  - same page, section 7, "CPU Oracle": FP64 count/G/H accumulated per bin in
 *    the supplied row-index order; nodes written breadth-first to a flat array.
 *
 * One reading is added where the pages are silent (listed with the others in
 * the design notes): the gradient is put on a per-tree fixed-point grid
 * before any histogram is taken.  With M = max_i |g_i|, M < 2^e (frexp),
 * L = ceil(log2 n) and S = 52 - e - L, the grid value is
 * k_i = rint(ldexp(g_i, S)) (round half to even) and the gradient used from
 * then on is ldexp(k_i, -S).  Every partial sum of those values over any row
 * subset is an integer multiple of 2^-S below 2^52 * 2^-S in magnitude, so
 * the FP64 row-order sums below are exact; an int64 shadow of each sum is
 * kept and checked against the FP64 value.  M = 0 gives S = 0.
 *
 * Depth: the root is depth 0; splits are tried at depths 0 .. max_depth-1;
 * nodes at depth max_depth are leaves.  Breadth-first numbering: within a
 * level, parents are visited in node-index order, each splitting parent
 * appends its left child and then its right child.
 */
#define _POSIX_C_SOURCE 199309L
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_RANGE (-3)
#define ORC_E_INTERNAL (-7)
#define ORC_LEAF 1u

#define ORC_SQUARED_ERROR 0
#define ORC_LOGISTIC 1

typedef struct {
  double reg_lambda;
  double gamma;
  double min_child_weight;
  double learning_rate;
  int32_t min_samples_leaf;
  int32_t max_depth;
  int32_t objective; /* ORC_SQUARED_ERROR or ORC_LOGISTIC */
  int32_t pad;
} orc_params;

typedef struct {
  int32_t feature;
  int32_t threshold_bin;
  int32_t left;
  int32_t right;
  double leaf_value;
  double gain;
  uint32_t flags;
  int32_t depth;
  int64_t count;  /* rows in the node */
  int64_t gsum_q; /* sum of the fixed-point gradients k_i over the node */
  int64_t hsum_q; /* logistic: sum of the fixed-point Hessians over the node (0 otherwise) */
} orc_node;

typedef struct {
  double gain;
  int32_t feature;
  int32_t threshold_bin;
  int64_t n_left;
  int64_t gq_left;
  int32_t valid;
  int32_t pad;
  double h_left; /* the left child's Hessian sum (FP64) */
} orc_split;

static double now_s(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

/* Parameter rules of the Tree Model section. */
int orc_validate_params(const orc_params* p) {
  if (!p) return ORC_E_ARG;
  if (!isfinite(p->reg_lambda) || !isfinite(p->gamma) || !isfinite(p->min_child_weight) ||
      !isfinite(p->learning_rate))
    return ORC_E_ARG;
  if (p->min_samples_leaf < 1) return ORC_E_ARG;
  if (p->min_child_weight < 0.0) return ORC_E_ARG;
  if (p->reg_lambda < 0.0) return ORC_E_ARG;
  if (p->gamma < 0.0) return ORC_E_ARG;
  if (p->max_depth < 0 || p->max_depth > 20) return ORC_E_ARG;
  if (p->objective != ORC_SQUARED_ERROR && p->objective != ORC_LOGISTIC) return ORC_E_ARG;
  return ORC_OK;
}

int32_t orc_ceil_log2(int64_t n) {
  int32_t L = 0;
  while (((int64_t)1 << L) < n) ++L;
  return L;
}

/*
 * Gradients (Single Mathematical Semantics: g = prediction - label, h = 1)
 * and the per-tree fixed-point grid described in the header.
 */
int orc_gradient_grid(int64_t n, const double* pred, const float* label, int64_t* k_out,
                      int32_t* scale_out, double* g_out) {
  if (n < 1 || !pred || !label || !k_out || !scale_out) return ORC_E_ARG;
  double M = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double g = pred[i] - (double)label[i];
    if (!isfinite(g)) return ORC_E_RANGE;
    if (g_out) g_out[i] = g;
    double a = fabs(g);
    if (a > M) M = a;
  }
  int32_t S = 0;
  if (M > 0.0) {
    int e = 0;
    (void)frexp(M, &e); /* M = m * 2^e, 0.5 <= m < 1, so M < 2^e */
    S = 52 - e - orc_ceil_log2(n);
  }
  for (int64_t i = 0; i < n; ++i) {
    double g = pred[i] - (double)label[i];
    k_out[i] = (int64_t)rint(ldexp(g, S));
  }
  *scale_out = S;
  return ORC_OK;
}

/*
 * exp(x) for x <= 0, written out from a published method: Cody and Waite's
 * argument reduction ("Software Manual for the Elementary Functions", 1980)
 * and the Taylor series of e^r.  k = rint(x / ln 2) and
 * r = (x - k*LN2_HI) - k*LN2_LO, where LN2_HI holds the first 42 significant
 * bits of ln 2 (so k*LN2_HI is exact for |k| < 2^11) and LN2_LO = ln 2 - LN2_HI
 * rounded to FP64; then |r| <= ln(2)/2 and e^r = sum_{j=0..13} r^j / j!
 * (the first omitted term is below 2^-57 relative), summed by Horner's rule
 * from the highest power, and e^x = 2^k * e^r (ldexp, exact for the normal
 * results that x in [-700, 0] gives).  Every step is one IEEE FP64 operation,
 * so the result is the same on any machine that rounds to nearest even.
 * Arguments below -700 give 0 (the callers need e^-|p| only to about 1e-304).
 */
static const double ORC_LN2_HI = 0x1.62e42fefa3800p-1;
static const double ORC_LN2_LO = 0x1.ef35793c76730p-45;
static const double ORC_INV_LN2 = 0x1.71547652b82fep+0;

double orc_exp_neg(double x) {
  if (!(x <= 0.0)) return NAN;
  if (x < -700.0) return 0.0;
  const double kd = rint(x * ORC_INV_LN2);
  const double r = (x - kd * ORC_LN2_HI) - kd * ORC_LN2_LO;
  /* 1/j! for j = 13 down to 0 */
  static const double inv_fact[14] = {
      1.0 / 6227020800.0, 1.0 / 479001600.0, 1.0 / 39916800.0, 1.0 / 3628800.0, 1.0 / 362880.0,
      1.0 / 40320.0,      1.0 / 5040.0,      1.0 / 720.0,      1.0 / 120.0,     1.0 / 24.0,
      1.0 / 6.0,          0.5,               1.0,              1.0};
  double poly = inv_fact[0];
  for (int j = 1; j < 14; ++j) poly = poly * r + inv_fact[j];
  return ldexp(poly, (int)kd);
}

/*
 * Sigmoid binary cross-entropy on the raw score ("Gradient boosted trees
 * (spec model)", gbtBinaryCrossentropyGradSpec: the gradient of the
 * sigmoid's cross-entropy with respect to the prediction).  With
 * s = 1 / (1 + e^-p): g = s - y.  The pages give no Hessian; the reading
 * used is its second derivative, h = s (1 - s), which the Training Core's
 * Newton-form weight -G/(H+lambda) and gain take where squared error has
 * h = 1.  Both come from z = e^-|p| and d = 1 + z, so that neither loses
 * accuracy for large |p|: s = 1/d for p >= 0 and z/d otherwise, and
 * h = z / (d*d), each one IEEE operation at a time.
 */
void orc_logistic_gh(double p, double y, double* g, double* h) {
  const double z = orc_exp_neg(-fabs(p));
  const double d = 1.0 + z;
  const double s = p >= 0.0 ? 1.0 / d : z / d;
  *g = s - y;
  *h = z / (d * d);
}

/*
 * Grid exponent of one quantity for the logistic objective (reading): with
 * M the largest magnitude (frexp exponent e, M < 2^e), S = 52 - e - L as for
 * squared error, but at most 30 - e, so every fixed-point value fits 31 bits
 * (a resolution of 2^-30 of M) while every sum over any rows stays exact.
 */
static int32_t orc_logistic_scale(double M, int64_t n) {
  if (!(M > 0.0)) return 0;
  int e = 0;
  (void)frexp(M, &e);
  int32_t S = 52 - e - orc_ceil_log2(n);
  if (S > 30 - e) S = 30 - e;
  return S;
}

/* Gradients and Hessians of the logistic objective on their per-tree grids. */
int orc_logistic_grid(int64_t n, const double* pred, const float* label, int64_t* kg, int64_t* kh,
                      int32_t* sg_out, int32_t* sh_out) {
  if (n < 1 || !pred || !label || !kg || !kh || !sg_out || !sh_out) return ORC_E_ARG;
  double Mg = 0.0, Mh = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double g, h;
    if (!isfinite(pred[i]) || !isfinite((double)label[i])) return ORC_E_RANGE;
    orc_logistic_gh(pred[i], (double)label[i], &g, &h);
    if (!isfinite(g) || !isfinite(h)) return ORC_E_RANGE;
    if (fabs(g) > Mg) Mg = fabs(g);
    if (h > Mh) Mh = h;
  }
  const int32_t Sg = orc_logistic_scale(Mg, n);
  const int32_t Sh = orc_logistic_scale(Mh, n);
  for (int64_t i = 0; i < n; ++i) {
    double g, h;
    orc_logistic_gh(pred[i], (double)label[i], &g, &h);
    kg[i] = (int64_t)rint(ldexp(g, Sg));
    kh[i] = (int64_t)rint(ldexp(h, Sh));
  }
  *sg_out = Sg;
  *sh_out = Sh;
  return ORC_OK;
}

/*
 * One node's histogram (CPU Oracle section: count/G/H per bin, accumulated in
 * the supplied row order, FP64).  gq is the int64 shadow of G on the grid.
 * Returns ORC_E_INTERNAL if an FP64 sum ever differs from its shadow.
 */
int orc_node_histogram(const uint8_t* bins, int32_t F, const int32_t* bin_offset,
                       int32_t total_bins, const int32_t* rows, int64_t n_rows, const int64_t* k,
                       int32_t S, uint32_t* cnt, int64_t* gq, double* g, double* h,
                       const int64_t* kh, int32_t Sh, int64_t* hq) {
  memset(cnt, 0, sizeof(uint32_t) * (size_t)total_bins);
  memset(gq, 0, sizeof(int64_t) * (size_t)total_bins);
  if (hq) memset(hq, 0, sizeof(int64_t) * (size_t)total_bins);
  for (int32_t b = 0; b < total_bins; ++b) {
    g[b] = 0.0;
    h[b] = 0.0;
  }
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t i = rows[r];
    const double gi = ldexp((double)k[i], -S);
    /* h_i = 1 for squared error; the logistic objective's grid value otherwise */
    const double hi = kh ? ldexp((double)kh[i], -Sh) : 1.0;
    for (int32_t f = 0; f < F; ++f) {
      const int32_t b = bin_offset[f] + (int32_t)bins[i * (int64_t)F + f];
      cnt[b] += 1u;
      g[b] = g[b] + gi;
      h[b] = h[b] + hi;
      gq[b] += k[i];
      if (kh && hq) hq[b] += kh[i];
    }
  }
  for (int32_t b = 0; b < total_bins; ++b) {
    if (g[b] != ldexp((double)gq[b], -S)) return ORC_E_INTERNAL;
    if (kh ? (hq && h[b] != ldexp((double)hq[b], -Sh)) : h[b] != (double)cnt[b]) return ORC_E_INTERNAL;
  }
  return ORC_OK;
}

static double score(double G, double H, double lambda) {
  const double num = G * G;
  const double den = H + lambda;
  return num / den;
}

/*
 * Split selection for one node (Tree Model section).  Candidates are visited
 * feature-major, thresholds ascending, t = 0 .. n_bins[f]-2; a candidate
 * enters the comparison only if both children meet min_samples_leaf and
 * min_child_weight and have strictly positive Hessian.  The best starts at
 * gain 0.0 and is replaced only on a strictly larger FP64 gain, which gives
 * exactly: larger gain, then smaller feature, then smaller bin, then first,
 * with a strictly positive gain required.
 */
int orc_best_split(int32_t F, const int32_t* n_bins, const int32_t* bin_offset,
                   const uint32_t* cnt, const int64_t* gq, const double* g, const double* h,
                   double G_v, double H_v, int64_t n_v, const orc_params* p, orc_split* out) {
  memset(out, 0, sizeof(*out));
  out->feature = -1;
  out->threshold_bin = -1;
  double best = 0.0;
  const double lambda = p->reg_lambda;
  const double score_parent = score(G_v, H_v, lambda);
  for (int32_t f = 0; f < F; ++f) {
    double GL = 0.0, HL = 0.0;
    int64_t nL = 0, gqL = 0;
    for (int32_t t = 0; t + 1 < n_bins[f]; ++t) {
      const int32_t b = bin_offset[f] + t;
      GL = GL + g[b];
      HL = HL + h[b];
      nL += cnt[b];
      gqL += gq[b];
      const int64_t nR = n_v - nL;
      const double GR = G_v - GL;
      const double HR = H_v - HL;
      if (nL < p->min_samples_leaf || nR < p->min_samples_leaf) continue;
      if (HL < p->min_child_weight || HR < p->min_child_weight) continue;
      if (!(HL > 0.0) || !(HR > 0.0)) continue;
      const double sL = score(GL, HL, lambda);
      const double sR = score(GR, HR, lambda);
      const double sum = sL + sR;
      const double diff = sum - score_parent;
      const double half = 0.5 * diff;
      const double gain = half - p->gamma;
      if (gain > best) {
        best = gain;
        out->gain = gain;
        out->feature = f;
        out->threshold_bin = t;
        out->n_left = nL;
        out->gq_left = gqL;
        out->h_left = HL;
        out->valid = 1;
      }
    }
  }
  return ORC_OK;
}

/* Leaf weight (Single Mathematical Semantics). */
double orc_leaf_weight(double G, double H, double lambda) {
  const double den = H + lambda;
  return -G / den;
}

/* Stable partition: bin <= threshold goes left, order kept on both sides. */
int64_t orc_partition(const uint8_t* bins, int32_t F, const int32_t* rows, int64_t n_rows,
                      int32_t feature, int32_t threshold_bin, int32_t* left_out,
                      int32_t* right_out) {
  int64_t nl = 0, nr = 0;
  for (int64_t r = 0; r < n_rows; ++r) {
    const int32_t i = rows[r];
    if ((int32_t)bins[(int64_t)i * F + feature] <= threshold_bin)
      left_out[nl++] = i;
    else
      right_out[nr++] = i;
  }
  return nl;
}

typedef struct {
  int32_t id;
  int64_t off; /* offset of the node's rows in the current level buffer */
  int64_t count;
} orc_active;

/*
 * Boosting: n_trees trees grown level by level (Tree Growth section, steps
 * 1-7), predictions updated after each tree as pred_i + (eta * w).
 *
 * pred: [n] in/out.  nodes: [n_trees][2^(max_depth+1)-1].  n_nodes, scale:
 * [n_trees].  Optional outputs (NULL to skip): pred_per_tree [n_trees][n];
 * for tree dump_tree only: dump_cnt/dump_gq [max_nodes][total_bins]
 * (histograms of every node at depth < max_depth, zero elsewhere),
 * dump_leaf_of_row [n], dump_k [n]; timing [2] = total and histogram seconds.
 */
int orc_train(int64_t n, int32_t F, const uint8_t* bins, const int32_t* n_bins, const float* label,
              const orc_params* p, int32_t n_trees, double* pred, orc_node* nodes,
              int32_t* n_nodes, int32_t* scale, double* pred_per_tree, int32_t dump_tree,
              uint32_t* dump_cnt, int64_t* dump_gq, int32_t* dump_leaf_of_row, int64_t* dump_k,
              double* timing, int32_t* scale_h, int64_t* dump_hq, int64_t* dump_kh) {
  int rc = orc_validate_params(p);
  if (rc) return rc;
  if (n < 1 || n > 0x7fffffffLL || F < 1 || !bins || !n_bins || !label || !pred || !nodes ||
      !n_nodes || !scale || n_trees < 0)
    return ORC_E_ARG;
  int32_t* bin_offset = (int32_t*)malloc(sizeof(int32_t) * (size_t)(F + 1));
  if (!bin_offset) return ORC_E_INTERNAL;
  bin_offset[0] = 0;
  for (int32_t f = 0; f < F; ++f) {
    if (n_bins[f] < 1 || n_bins[f] > 256) {
      free(bin_offset);
      return ORC_E_ARG;
    }
    bin_offset[f + 1] = bin_offset[f] + n_bins[f];
  }
  const int32_t TB = bin_offset[F];
  for (int64_t i = 0; i < n; ++i) {
    if (!isfinite((double)label[i]) || !isfinite(pred[i])) {
      free(bin_offset);
      return ORC_E_RANGE;
    }
    for (int32_t f = 0; f < F; ++f)
      if ((int32_t)bins[i * F + f] >= n_bins[f]) {
        free(bin_offset);
        return ORC_E_RANGE;
      }
  }
  const int32_t D = p->max_depth;
  const int32_t max_nodes = (1 << (D + 1)) - 1;
  double t_total = 0.0, t_hist = 0.0;

  const int logistic = p->objective == ORC_LOGISTIC;
  int64_t* k = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
  int64_t* kh = logistic ? (int64_t*)malloc(sizeof(int64_t) * (size_t)n) : NULL;
  int64_t* hqv = logistic ? (int64_t*)malloc(sizeof(int64_t) * (size_t)TB) : NULL;
  int32_t* buf_a = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  int32_t* buf_b = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  int32_t* tmp_r = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  int32_t* leaf_of_row = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  orc_active* act = (orc_active*)malloc(sizeof(orc_active) * (size_t)(max_nodes + 1));
  orc_active* nxt = (orc_active*)malloc(sizeof(orc_active) * (size_t)(max_nodes + 1));
  uint32_t* cnt = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)TB);
  int64_t* gq = (int64_t*)malloc(sizeof(int64_t) * (size_t)TB);
  double* hg = (double*)malloc(sizeof(double) * (size_t)TB);
  double* hh = (double*)malloc(sizeof(double) * (size_t)TB);
  if (!k || !buf_a || !buf_b || !tmp_r || !leaf_of_row || !act || !nxt || !cnt || !gq || !hg || !hh ||
      (logistic && (!kh || !hqv))) {
    rc = ORC_E_INTERNAL;
    goto done;
  }

  for (int32_t t = 0; t < n_trees; ++t) {
    const double t0 = now_s();
    const int dump = (t == dump_tree);
    orc_node* tree = nodes + (size_t)t * (size_t)max_nodes;
    int32_t S = 0, Sh = 0;
    /* gradients (and, for the logistic objective, Hessians) and grids */
    if (logistic)
      rc = orc_logistic_grid(n, pred, label, k, kh, &S, &Sh);
    else
      rc = orc_gradient_grid(n, pred, label, k, &S, NULL);
    if (rc) goto done;
    scale[t] = S;
    if (scale_h) scale_h[t] = Sh;
    if (dump && dump_k) memcpy(dump_k, k, sizeof(int64_t) * (size_t)n);
    if (dump && dump_kh && logistic) memcpy(dump_kh, kh, sizeof(int64_t) * (size_t)n);
    if (dump && dump_hq) memset(dump_hq, 0, sizeof(int64_t) * (size_t)max_nodes * (size_t)TB);
    if (dump && dump_cnt) memset(dump_cnt, 0, sizeof(uint32_t) * (size_t)max_nodes * (size_t)TB);
    if (dump && dump_gq) memset(dump_gq, 0, sizeof(int64_t) * (size_t)max_nodes * (size_t)TB);

    /* step 1 at the root: one active node with rows 0..n-1 in order */
    int32_t count_nodes = 1;
    int32_t n_act = 1;
    int32_t* cur = buf_a;
    int32_t* nb = buf_b;
    for (int64_t i = 0; i < n; ++i) cur[i] = (int32_t)i;
    act[0].id = 0;
    act[0].off = 0;
    act[0].count = n;
    memset(&tree[0], 0, sizeof(orc_node));
    tree[0].depth = 0;
    tree[0].count = n;
    {
      int64_t s = 0, sh = 0;
      for (int64_t i = 0; i < n; ++i) {
        s += k[i];
        if (logistic) sh += kh[i];
      }
      tree[0].gsum_q = s;
      tree[0].hsum_q = sh;
    }

    for (int32_t d = 0; d < D && n_act > 0; ++d) {
      int32_t n_nxt = 0;
      int64_t nb_off = 0;
      for (int32_t a = 0; a < n_act; ++a) {
        const int32_t v = act[a].id;
        const int32_t* rows = cur + act[a].off;
        const int64_t nv = act[a].count;
        /* step 2: histogram of the node, rows in order */
        const double th = now_s();
        rc = orc_node_histogram(bins, F, bin_offset, TB, rows, nv, k, S, cnt, gq, hg, hh, kh, Sh, hqv);
        t_hist += now_s() - th;
        if (rc) goto done;
        if (dump && dump_cnt) memcpy(dump_cnt + (size_t)v * TB, cnt, sizeof(uint32_t) * (size_t)TB);
        if (dump && dump_gq) memcpy(dump_gq + (size_t)v * TB, gq, sizeof(int64_t) * (size_t)TB);
        if (dump && dump_hq && logistic) memcpy(dump_hq + (size_t)v * TB, hqv, sizeof(int64_t) * (size_t)TB);
        /* node totals, row order */
        double Gv = 0.0, Hv = 0.0;
        for (int64_t r = 0; r < nv; ++r) {
          Gv = Gv + ldexp((double)k[rows[r]], -S);
          Hv = Hv + (logistic ? ldexp((double)kh[rows[r]], -Sh) : 1.0);
        }
        if (Gv != ldexp((double)tree[v].gsum_q, -S) ||
            (logistic && Hv != ldexp((double)tree[v].hsum_q, -Sh))) {
          rc = ORC_E_INTERNAL;
          goto done;
        }
        /* steps 3-4: split selection with the constraint filter */
        orc_split sp;
        orc_best_split(F, n_bins, bin_offset, cnt, gq, hg, hh, Gv, Hv, nv, p, &sp);
        if (sp.valid) {
          /* step 5: stable partition into the next level buffer */
          int32_t* left = nb + nb_off;
          const int64_t nl = orc_partition(bins, F, rows, nv, sp.feature, sp.threshold_bin, left, tmp_r);
          if (nl != sp.n_left) {
            rc = ORC_E_INTERNAL;
            goto done;
          }
          memcpy(left + nl, tmp_r, sizeof(int32_t) * (size_t)(nv - nl));
          /* step 6: append the children breadth-first */
          const int32_t lc = count_nodes, rcn = count_nodes + 1;
          count_nodes += 2;
          tree[v].feature = sp.feature;
          tree[v].threshold_bin = sp.threshold_bin;
          tree[v].left = lc;
          tree[v].right = rcn;
          tree[v].gain = sp.gain;
          tree[v].leaf_value = 0.0;
          tree[v].flags = 0u;
          memset(&tree[lc], 0, sizeof(orc_node));
          memset(&tree[rcn], 0, sizeof(orc_node));
          tree[lc].depth = d + 1;
          tree[rcn].depth = d + 1;
          tree[lc].count = nl;
          tree[rcn].count = nv - nl;
          tree[lc].gsum_q = sp.gq_left;
          tree[rcn].gsum_q = tree[v].gsum_q - sp.gq_left;
          if (logistic) {
            int64_t hl = 0;
            for (int64_t r = 0; r < nl; ++r) hl += kh[left[r]];
            if (ldexp((double)hl, -Sh) != sp.h_left) {
              rc = ORC_E_INTERNAL;
              goto done;
            }
            tree[lc].hsum_q = hl;
            tree[rcn].hsum_q = tree[v].hsum_q - hl;
          }
          nxt[n_nxt].id = lc;
          nxt[n_nxt].off = nb_off;
          nxt[n_nxt].count = nl;
          ++n_nxt;
          nxt[n_nxt].id = rcn;
          nxt[n_nxt].off = nb_off + nl;
          nxt[n_nxt].count = nv - nl;
          ++n_nxt;
          nb_off += nv;
        } else {
          /* step 6: freeze as a leaf */
          tree[v].feature = -1;
          tree[v].threshold_bin = -1;
          tree[v].left = -1;
          tree[v].right = -1;
          tree[v].gain = 0.0;
          tree[v].flags = ORC_LEAF;
          tree[v].leaf_value = orc_leaf_weight(Gv, Hv, p->reg_lambda);
          for (int64_t r = 0; r < nv; ++r) leaf_of_row[rows[r]] = v;
        }
      }
      {
        orc_active* sw = act;
        act = nxt;
        nxt = sw;
      }
      n_act = n_nxt;
      {
        int32_t* sw = cur;
        cur = nb;
        nb = sw;
      }
    }
    /* nodes at depth D (or any still active) become leaves */
    for (int32_t a = 0; a < n_act; ++a) {
      const int32_t v = act[a].id;
      const int32_t* rows = cur + act[a].off;
      const int64_t nv = act[a].count;
      double Gv = 0.0, Hv = 0.0;
      for (int64_t r = 0; r < nv; ++r) {
        Gv = Gv + ldexp((double)k[rows[r]], -S);
        Hv = Hv + (logistic ? ldexp((double)kh[rows[r]], -Sh) : 1.0);
      }
      tree[v].feature = -1;
      tree[v].threshold_bin = -1;
      tree[v].left = -1;
      tree[v].right = -1;
      tree[v].gain = 0.0;
      tree[v].flags = ORC_LEAF;
      tree[v].leaf_value = orc_leaf_weight(Gv, Hv, p->reg_lambda);
      for (int64_t r = 0; r < nv; ++r) leaf_of_row[rows[r]] = v;
    }
    n_nodes[t] = count_nodes;
    if (dump && dump_leaf_of_row) memcpy(dump_leaf_of_row, leaf_of_row, sizeof(int32_t) * (size_t)n);
    /* step 7, after the tree: each row adds (eta * w) of the leaf whose
       partitioned row list holds it */
    for (int64_t i = 0; i < n; ++i) {
      const double delta = p->learning_rate * tree[leaf_of_row[i]].leaf_value;
      pred[i] = pred[i] + delta;
    }
    if (pred_per_tree) memcpy(pred_per_tree + (size_t)t * (size_t)n, pred, sizeof(double) * (size_t)n);
    t_total += now_s() - t0;
  }
  rc = ORC_OK;
done:
  if (timing) {
    timing[0] = t_total;
    timing[1] = t_hist;
  }
  free(bin_offset);
  free(k);
  free(kh);
  free(hqv);
  free(buf_a);
  free(buf_b);
  free(tmp_r);
  free(leaf_of_row);
  free(act);
  free(nxt);
  free(cnt);
  free(gq);
  free(hg);
  free(hh);
  return rc;
}

/*
 * Feature binning: the "Quantized" state between validation and training in
 * the Training Core page's state machine (section 5).  The pages name the
 * state but not the rule; the reading used here: feature f has n_bins[f]
 * bins and n_bins[f] - 1 strictly increasing upper bounds
 * upper[bin_offset[f] + k], and a value's bin is how many of those bounds are
 * strictly below it (a value equal to a bound stays in the lower bin).  Each
 * value is compared with every bound of its feature in turn; nothing is
 * searched or skipped.  A NaN value compares below nothing and gets bin 0.
 * Returns -1 when a bound is NaN or the bounds of a feature are not strictly
 * increasing (out is then not written), else the number of NaN values.
 */
int64_t orc_bin_features(int64_t n_rows, int32_t F, const float* raw, const int32_t* n_bins,
                         const int32_t* bin_offset, const float* upper, uint8_t* out) {
  for (int32_t f = 0; f < F; ++f) {
    const float* u = upper + bin_offset[f];
    for (int32_t k = 0; k + 1 < n_bins[f]; ++k) {
      if (isnan(u[k])) return -1;
      if (k + 2 < n_bins[f] && !(u[k] < u[k + 1])) return -1;
    }
  }
  int64_t n_nan = 0;
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int32_t f = 0; f < F; ++f) {
      const float x = raw[r * F + f];
      const float* u = upper + bin_offset[f];
      int32_t below = 0;
      for (int32_t k = 0; k + 1 < n_bins[f]; ++k)
        if (u[k] < x) ++below;
      if (isnan(x)) ++n_nan;
      out[r * F + f] = (uint8_t)below;
    }
  }
  return n_nan;
}

/*
 * Ensemble forward pass: "Gradient boosted trees (spec model)", section
 * Forward pass.  One tree is traversed from its root: at a split node the
 * row goes to the left child when its bin of the node's feature is <= the
 * node's threshold bin, else to the right child (the same routing as the
 * Training Core page's Tree Model section), until a leaf, whose value is the
 * tree's output.  The ensemble adds the learning rate times each tree's
 * output to the initial prediction.  Reading (the spec names the sum, not
 * its rounding): the trees are added one at a time in their order,
 * out = ((base + eta*w_1) + eta*w_2) + ..., one IEEE rounding per product and
 * per sum -- the sequence that step 7 of the Tree Growth section applies
 * after each tree -- so the prediction of a training row equals its
 * prediction at the end of training bit for bit.
 *
 * trees: n_trees node arrays of tree_stride nodes each (tree t at
 * nodes + t * tree_stride) with n_nodes[t] nodes.  Returns ORC_OK, or
 * ORC_E_ARG when a visited node's children or feature are out of range or a
 * walk takes more steps than the tree has nodes (out is then incomplete).
 */
int orc_predict(int64_t n, int32_t F, const uint8_t* bins, int32_t n_trees, const orc_node* nodes,
                int32_t tree_stride, const int32_t* n_nodes, double base, double eta, double* out) {
  if (n < 0 || F < 1 || n_trees < 0 || tree_stride < 1 || (n > 0 && (!bins || !out))) return ORC_E_ARG;
  for (int64_t i = 0; i < n; ++i) out[i] = base;
  for (int32_t t = 0; t < n_trees; ++t) {
    const orc_node* tree = nodes + (size_t)t * (size_t)tree_stride;
    const int32_t nn = n_nodes[t];
    if (nn < 1 || nn > tree_stride) return ORC_E_ARG;
    for (int64_t i = 0; i < n; ++i) {
      int32_t v = 0;
      int32_t steps = 0;
      while (!(tree[v].flags & ORC_LEAF)) {
        const int32_t f = tree[v].feature;
        if (f < 0 || f >= F || ++steps > nn) return ORC_E_ARG;
        const int32_t next = ((int32_t)bins[i * (int64_t)F + f] <= tree[v].threshold_bin) ? tree[v].left
                                                                                          : tree[v].right;
        if (next < 0 || next >= nn) return ORC_E_ARG;
        v = next;
      }
      const double term = eta * tree[v].leaf_value;
      out[i] = out[i] + term;
    }
  }
  return ORC_OK;
}

/*
 * Bin bounds: how the bounds of the "Quantized" state (Training Core, state
 * machine, section 5) are chosen.  The page names the state only; two
 * readings are provided, both ending in bounds that strictly increase so
 * that orc_bin_features accepts them.  For feature f with B = n_bins[f]
 * bins, the B - 1 bounds u_1 .. u_{B-1} go to upper[bin_offset[f] + k - 1];
 * the entry after them (never read by the binning) is set to +inf.
 *
 *  Both take zeros of either sign as +0, so the bounds are unique.
 *  method 0, equal width: lo and hi are the least and greatest finite values
 *    of the feature (NaN and +-inf skipped; lo = hi = 0 if there is none);
 *    u_k = (float)(lo + (hi - lo) * (k / B)), evaluated in FP64 one operation
 *    at a time (k / B, the product, the sum), then rounded to FP32.
 *  method 1, quantile: the sample is the rows 0, s, 2s, ... with
 *    s = ceil(n / ORC_QUANTILE_SAMPLE) (every row when n <= ORC_QUANTILE_SAMPLE),
 *    a row sample as GBDT libraries use to build bins; its m finite values
 *    (NaN and +-inf skipped, as for the range above) sorted ascending as
 *    v_0 <= ... <= v_{m-1}; u_k is v_r with r = ceil(k m / B) - 1, so at least
 *    k m / B of them lie at or below u_k (m = 0: every u_k = 0).
 *
 * Then, for k = 2 .. B-1, a bound that is not above its predecessor is raised
 * to next_up(u_{k-1}): the next FP32 value above it among zero and the normal
 * values (0 for a negative value whose next value would be subnormal; the
 * least positive normal value for a zero; a positive value's next
 * representable value; +inf stays +inf).
 */
#define ORC_QUANTILE_SAMPLE 32768

static float orc_next_up(float x) {
  if (isinf(x) && x > 0.0f) return x;
  if (x == 0.0f) return 1.17549435e-38f; /* FLT_MIN */
  uint32_t b;
  memcpy(&b, &x, 4);
  b = x > 0.0f ? b + 1u : b - 1u;
  float y;
  memcpy(&y, &b, 4);
  if (y < 0.0f && y > -1.17549435e-38f) y = 0.0f; /* would be subnormal */
  return y;
}

static int orc_cmp_float(const void* a, const void* b) {
  const float x = *(const float*)a, y = *(const float*)b;
  return (x > y) - (x < y);
}

int orc_feature_bounds(int64_t n, int32_t F, const float* raw, const int32_t* n_bins, int32_t method,
                       float* upper) {
  if (n < 0 || F < 1 || (n > 0 && !raw) || !n_bins || !upper) return ORC_E_ARG;
  if (method != 0 && method != 1) return ORC_E_ARG;
  const int64_t step = n <= ORC_QUANTILE_SAMPLE ? 1 : (n + ORC_QUANTILE_SAMPLE - 1) / ORC_QUANTILE_SAMPLE;
  float* buf = (float*)malloc(sizeof(float) * (size_t)(ORC_QUANTILE_SAMPLE + 1));
  if (!buf) return ORC_E_INTERNAL;
  int64_t off = 0;
  for (int32_t f = 0; f < F; ++f) {
    const int32_t B = n_bins[f];
    if (B < 1 || B > 256) {
      free(buf);
      return ORC_E_ARG;
    }
    float* u = upper + off; /* u[k - 1] = u_k */
    if (method == 0) {
      int have = 0;
      float lo = 0.0f, hi = 0.0f;
      for (int64_t i = 0; i < n; ++i) {
        float x = raw[i * F + f];
        if (!isfinite(x)) continue;
        if (x == 0.0f) x = 0.0f;
        if (!have || x < lo) lo = x;
        if (!have || x > hi) hi = x;
        have = 1;
      }
      for (int32_t k = 1; k < B; ++k) {
        const double t = (double)k / (double)B;
        const double w = (double)hi - (double)lo;
        const double m = w * t;
        u[k - 1] = (float)((double)lo + m);
      }
    } else {
      int64_t m = 0;
      for (int64_t i = 0; i < n; i += step) {
        const float x = raw[i * F + f];
        if (isfinite(x)) buf[m++] = x == 0.0f ? 0.0f : x;
      }
      qsort(buf, (size_t)m, sizeof(float), orc_cmp_float);
      for (int32_t k = 1; k < B; ++k) {
        if (m == 0) {
          u[k - 1] = 0.0f;
        } else {
          const int64_t r = ((int64_t)k * m + B - 1) / B - 1;
          u[k - 1] = buf[r];
        }
      }
    }
    for (int32_t k = 2; k < B; ++k)
      if (!(u[k - 1] > u[k - 2])) u[k - 1] = orc_next_up(u[k - 2]);
    upper[off + B - 1] = INFINITY;
    off += B;
  }
  free(buf);
  return ORC_OK;
}
