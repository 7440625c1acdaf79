/*
 * Seeded synthetic inputs for level-wise histogram GBDT training.
 *
 * This module holds input generation only: pre-binned uint8 feature matrices
 * (row-major [n][F]) and float32 regression labels.  It contains none of the
 * boosting arithmetic (gradients, histograms, gains, partitions); both the
 * oracle and the GPU path consume the bytes it writes.
 *
 * Random numbers come from a counter-based SplitMix64: the value for
 * (seed, stream, counter) is the SplitMix64 output mix(s0 + (counter+1)*gamma)
 * with s0 = mix(seed ^ mix(stream)), so any cell can be generated
 * independently of every other one and generation order does not matter.
 * Streams: 1 = bins, 2 = structure / weights, 3 = label noise.
 *
 * Workloads (seed = 1000 + k for workload k):
 *   1: 4,096 x 8, 32 uniform bins; label = (b0+b1+b2)/32 + 0.1 N(0,1)
 *   2: 1,000,000 x 32, 256 uniform bins; label = random depth-4 tree + 0.5 N
 *   3: 581,012 x 54 (a covtype-shaped stand-in): 10 Gaussian features binned
 *      equal-width into 256 bins on [-4,4), 44 binary features with ~5% ones;
 *      integer label 1..7
 *   4: 10,000,000 x 100, 256 Zipf(1.2)-occupied bins; sparse linear label
 *   5: 50,000,000 x 28, 64 uniform bins; sin/product label
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

uint64_t dg_u64(uint64_t seed, uint64_t stream, uint64_t ctr) {
  uint64_t s0 = mix64(seed ^ mix64(stream + GOLDEN));
  return mix64(s0 + (ctr + 1) * GOLDEN);
}

/* uniform in [0,1) with 53 random bits; draw c uses counter 2c */
double dg_uniform(uint64_t seed, uint64_t stream, uint64_t c) {
  return (double)(dg_u64(seed, stream, 2 * c) >> 11) * 0x1.0p-53;
}

/* standard normal by Box-Muller from counters 2c and 2c+1 */
double dg_normal(uint64_t seed, uint64_t stream, uint64_t c) {
  double u1 = (double)(dg_u64(seed, stream, 2 * c) >> 11) * 0x1.0p-53;
  double u2 = (double)(dg_u64(seed, stream, 2 * c + 1) >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(1.0 - u1));
  return r * cos(6.283185307179586 * u2);
}

uint64_t dg_fnv1a64(const void* data, size_t nbytes) {
  const unsigned char* p = (const unsigned char*)data;
  uint64_t h = 0xcbf29ce484222325ULL;
  for (size_t i = 0; i < nbytes; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ULL;
  }
  return h;
}

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

int dg_config_shape(int k, int64_t* n, int32_t* F) {
  switch (k) {
    case 1: *n = 4096; *F = 8; return 0;
    case 2: *n = 1000000; *F = 32; return 0;
    case 3: *n = 581012; *F = 54; return 0;
    case 4: *n = 10000000; *F = 100; return 0;
    case 5: *n = 50000000; *F = 28; return 0;
    default: return -1;
  }
}

int dg_config_nbins(int k, int32_t* n_bins) {
  int64_t n; int32_t F;
  if (dg_config_shape(k, &n, &F)) return -1;
  for (int f = 0; f < F; ++f) {
    switch (k) {
      case 1: n_bins[f] = 32; break;
      case 2: n_bins[f] = 256; break;
      case 3: n_bins[f] = f < 10 ? 256 : 2; break;
      case 4: n_bins[f] = 256; break;
      case 5: n_bins[f] = 64; break;
    }
  }
  return 0;
}

/*
 * Rows [r0, r1) of workload k.  bins is [r1-r0][F] row-major, label [r1-r0].
 * Row i of any range equals row i of the full workload.  Rows from n on are
 * held-out rows drawn by the same recipe (counters past the training rows).
 */
int dg_config_rows(int k, int64_t r0, int64_t r1, uint8_t* bins, float* label) {
  int64_t n; int32_t F;
  if (dg_config_shape(k, &n, &F)) return -1;
  if (r0 < 0 || r0 > r1 || r1 > ((int64_t)1 << 36)) return -2;
  const uint64_t seed = 1000 + (uint64_t)k;

  /* workload 2: the hidden depth-4 tree (15 internal nodes, BFS order) */
  int tree_feat[15], tree_thr[15];
  double tree_leaf[16];
  /* workload 4: Zipf table and the sparse linear support */
  double zipf_cdf[256];
  int lin_feat[20];
  double lin_w[20];
  if (k == 2) {
    for (int j = 0; j < 15; ++j) {
      tree_feat[j] = (int)floor(32.0 * dg_uniform(seed, 2, 2 * j));
      tree_thr[j] = (int)floor(255.0 * dg_uniform(seed, 2, 2 * j + 1));
    }
    for (int l = 0; l < 16; ++l) tree_leaf[l] = dg_normal(seed, 2, 100 + l);
  }
  if (k == 4) {
    double acc = 0.0;
    for (int r = 1; r <= 256; ++r) {
      acc += pow((double)r, -1.2);
      zipf_cdf[r - 1] = acc;
    }
    int perm[100];
    for (int j = 0; j < 100; ++j) perm[j] = j;
    for (int j = 0; j < 20; ++j) {
      int r = j + (int)floor((double)(100 - j) * dg_uniform(seed, 2, j));
      if (r > 99) r = 99;
      int t = perm[j]; perm[j] = perm[r]; perm[r] = t;
      lin_feat[j] = perm[j];
      lin_w[j] = -5.0 + 10.0 * dg_uniform(seed, 2, 100 + j);
    }
  }

  #pragma omp parallel for schedule(static)
  for (int64_t i = r0; i < r1; ++i) {
    uint8_t* row = bins + (i - r0) * (int64_t)F;
    const uint64_t c0 = (uint64_t)i * (uint64_t)F;
    double y = 0.0;
    switch (k) {
      case 1: {
        for (int f = 0; f < F; ++f)
          row[f] = (uint8_t)clampi((int)floor(32.0 * dg_uniform(seed, 1, c0 + f)), 0, 31);
        y = (row[0] + row[1] + row[2]) / 32.0 + 0.1 * dg_normal(seed, 3, (uint64_t)i);
        break;
      }
      case 2: {
        for (int f = 0; f < F; ++f)
          row[f] = (uint8_t)clampi((int)floor(256.0 * dg_uniform(seed, 1, c0 + f)), 0, 255);
        int node = 0;
        for (int d = 0; d < 4; ++d)
          node = (row[tree_feat[node]] <= tree_thr[node]) ? 2 * node + 1 : 2 * node + 2;
        y = tree_leaf[node - 15] + 0.5 * dg_normal(seed, 3, (uint64_t)i);
        break;
      }
      case 3: {
        double z[10];
        for (int f = 0; f < F; ++f) {
          if (f < 10) {
            z[f] = dg_normal(seed, 1, c0 + f);
            row[f] = (uint8_t)clampi((int)floor((z[f] + 4.0) * 32.0), 0, 255);
          } else {
            row[f] = dg_uniform(seed, 1, c0 + f) < 0.05 ? 1 : 0;
          }
        }
        double v = 4.0 + z[0] - 0.8 * z[1] + 0.5 * z[2] * z[3] +
                   1.5 * ((double)row[10] - (double)row[11]) +
                   0.6 * dg_normal(seed, 3, (uint64_t)i);
        v = rint(v);
        y = v < 1.0 ? 1.0 : (v > 7.0 ? 7.0 : v);
        break;
      }
      case 4: {
        const double tot = zipf_cdf[255];
        for (int f = 0; f < F; ++f) {
          double t = dg_uniform(seed, 1, c0 + f) * tot;
          int lo = 0, hi = 255; /* smallest r with cdf[r] > t */
          while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (zipf_cdf[mid] > t) hi = mid; else lo = mid + 1;
          }
          row[f] = (uint8_t)lo;
        }
        for (int j = 0; j < 20; ++j) y += lin_w[j] * (double)row[lin_feat[j]] / 255.0;
        y += dg_normal(seed, 3, (uint64_t)i);
        break;
      }
      case 5: {
        for (int f = 0; f < F; ++f)
          row[f] = (uint8_t)clampi((int)floor(64.0 * dg_uniform(seed, 1, c0 + f)), 0, 63);
        double v[6];
        for (int j = 0; j < 6; ++j) v[j] = ((double)row[j] + 0.5) / 64.0;
        y = sin(6.283185307179586 * v[0]) + v[1] * v[2] + sin(3.141592653589793 * v[3]) * v[4] - v[5] +
            0.3 * dg_normal(seed, 3, (uint64_t)i);
        break;
      }
    }
    label[i - r0] = (float)y;
  }
  return 0;
}

/*
 * Generic random workload for tests: feature f has n_bins[f] bins.
 * bin_kind 0: uniform bins; 1: skewed (bin 0 with probability 1/2, else uniform);
 * label_kind 0: N(0,1); 1: dyadic values k/8 with k uniform in [-64, 64];
 *            2: sum of the first min(F,3) bins scaled by 1/16 plus 0.25 N(0,1).
 */
int dg_random(int64_t n, int32_t F, const int32_t* n_bins, uint64_t seed, int bin_kind,
              int label_kind, uint8_t* bins, float* label) {
  if (n < 0 || F <= 0) return -1;
  for (int f = 0; f < F; ++f)
    if (n_bins[f] < 1 || n_bins[f] > 256) return -2;
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint8_t* row = bins + i * (int64_t)F;
    const uint64_t c0 = (uint64_t)i * (uint64_t)F;
    for (int f = 0; f < F; ++f) {
      double u = dg_uniform(seed, 1, c0 + f);
      int b;
      if (bin_kind == 1) {
        b = u < 0.5 ? 0 : (int)floor((u - 0.5) * 2.0 * n_bins[f]);
      } else {
        b = (int)floor(u * n_bins[f]);
      }
      row[f] = (uint8_t)clampi(b, 0, n_bins[f] - 1);
    }
    double y;
    if (label_kind == 1) {
      int kk = (int)floor(129.0 * dg_uniform(seed, 3, (uint64_t)i)) - 64;
      if (kk > 64) kk = 64;
      y = kk / 8.0;
    } else if (label_kind == 2) {
      y = 0.0;
      for (int f = 0; f < F && f < 3; ++f) y += row[f] / 16.0;
      y += 0.25 * dg_normal(seed, 3, (uint64_t)i);
    } else {
      y = dg_normal(seed, 3, (uint64_t)i);
    }
    label[i] = (float)y;
  }
  return 0;
}
