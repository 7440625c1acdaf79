// HIP kernels (gfx950) and the C ABI of the level-wise histogram GBDT hot
// path.  The operations are those of "Module Design: Training Core"
// (MPSBoost spec), sections 2, 3 and 6; see include/gbdt.h for the contract
// of each entry point.
//
// Compiled with -ffp-contract=off: every FP64 expression below is evaluated
// as written, one IEEE rounding per operation, no fused multiply-add.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <type_traits>
#include <vector>

#include "gbdt.h"
#include "gbdt_internal.h"
#include "gbdt_device.h"

#pragma clang fp contract(off)

namespace gbdt {

// ------------------------------------------------------------------ errors --

static thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return GBDT_E_DEVICE;
}

#define GBDT_LAUNCH_CHECK(what)                        \
  do {                                                 \
    hipError_t e_ = hipGetLastError();                 \
    if (e_ != hipSuccess) return hip_fail(e_, (what)); \
  } while (0)

// ------------------------------------------------------------ diagnostics --

struct DiagState {
  bool enabled = false;
  int32_t capacity = 0;
  int32_t count = 0;
  bool open = false;
  std::vector<hipEvent_t> ev;  // 2 per record
  std::vector<int32_t> kind;
};
static DiagState g_diag;

void diag_begin(int kind, hipStream_t s) {
  if (!g_diag.enabled || g_diag.count >= g_diag.capacity) return;
  g_diag.kind[g_diag.count] = kind;
  (void)hipEventRecord(g_diag.ev[2 * g_diag.count], s);
  g_diag.open = true;
}

void diag_end(hipStream_t s) {
  if (!g_diag.open) return;
  (void)hipEventRecord(g_diag.ev[2 * g_diag.count + 1], s);
  ++g_diag.count;
  g_diag.open = false;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WsLayout ws_layout(int64_t n_rows, int32_t max_list, int32_t total_bins) {
  WsLayout L{};
  if (n_rows < 1) n_rows = 1;
  if (max_list < 1) max_list = 1;
  if (total_bins < 1) total_bins = 1;
  L.status_cap = (n_rows + kPartTileRows - 1) / kPartTileRows + int64_t(max_list) + 2;
  L.hpart_tiles = int64_t(kHistTargetTiles) + int64_t(max_list) + 2;
  L.tdesc_cap = L.status_cap;
  size_t off = 0;
  L.ctrl = off;
  off = align256(off + sizeof(WsCtrl));
  L.tdesc = off;
  off = align256(off + sizeof(TileDesc) * size_t(L.tdesc_cap));
  L.hdesc = off;
  off = align256(off + sizeof(TileDesc) * size_t(L.hpart_tiles));
  L.gpart = off;
  off = align256(off + 2 * (sizeof(double) + sizeof(int64_t)) * kGradBlocks);
  L.prefix = off;
  off = align256(off + sizeof(int32_t) * (size_t(max_list) + 2));
  L.hprefix = off;
  off = align256(off + sizeof(int32_t) * (size_t(max_list) + 2));
  L.hmulti = off;
  off = align256(off + sizeof(int32_t) * (4 + 4 * (size_t(max_list) + 2)));
  L.fcand = off;
  off = align256(off + sizeof(FindCand) * size_t(max_list) * size_t(find_chunks(total_bins)));
  L.status = off;
  off = align256(off + sizeof(uint64_t) * size_t(L.status_cap));
  L.status2 = off;
  off = align256(off + sizeof(uint64_t) * size_t(L.status_cap));
  L.gstage = off;
  off = align256(off + sizeof(PlanEntry) * (size_t(max_list) + 2));
  L.hpart = off;
  size_t hp = sizeof(uint64_t) * size_t(L.hpart_tiles) * size_t(total_bins);
  // the setup-time bin census of gbdt_pack_matrix reuses this region
  size_t census = sizeof(uint32_t) * size_t(GBDT_MAX_FEATURES) * GBDT_MAX_BINS;
  off = align256(off + (hp > census ? hp : census));
  L.total = off;
  return L;
}

int32_t hist_tile_rows(int64_t rows_bound, int64_t n_rows, int32_t target, int32_t min_rows) {
  const int64_t tmax = (int64_t(1) << pack_bits_for(n_rows)) - 1;
  int64_t t = (rows_bound + target - 1) / target;
  if (t < min_rows) t = min_rows;
  if (t > tmax) t = tmax;
  if (t < 1) t = 1;
  return int32_t(t);
}

// ------------------------------------------------------- device helpers --

// Sum of a 64-bit value over the 64 lanes of a wave with DPP lane moves (no
// LDS round trips): pairs and quads, half rows, rows, then rows 0+1 into row
// 1, 2+3 into row 3, and row 1 into row 3.  Every lane must be active; the
// total is returned in every lane (read from lane 63).  Exact mod 2^64.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t wave_sum_dpp(uint64_t v) {
  v += dpp_u64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_u64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_u64<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_u64<0x140, 0xF>(v);  // row_mirror
  v += dpp_u64<0x142, 0xA>(v);  // row_bcast:15 (rows 1 and 3 receive)
  v += dpp_u64<0x143, 0xC>(v);  // row_bcast:31 (rows 2 and 3 receive)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double wave_max(double v) {
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------- planner --
// Standalone planner launch for the per-call entry points: plans
// list[0..*list_len) (see plan_tiles).
__global__ void __launch_bounds__(1024) k_plan(const gbdt_node* __restrict__ nodes,
                                               const int32_t* __restrict__ list,
                                               const int32_t* __restrict__ list_len,
                                               int32_t list_cap, int32_t tile_rows,
                                               int32_t max_tiles, int32_t* __restrict__ prefix,
                                               TileDesc* __restrict__ desc,
                                               WsCtrl* __restrict__ ctrl,
                                               uint64_t* __restrict__ status,
                                               const gbdt_split* __restrict__ splits,
                                               const int32_t* __restrict__ feature_col,
                                               int32_t n_features, int32_t* __restrict__ multi) {
  __shared__ PlanLds lds;
  const int32_t raw = *list_len;
  if (threadIdx.x == 0 && (raw < 0 || raw > list_cap)) dev_error(&ctrl->err, GBDT_E_SHAPE);
  const int32_t n = clamp_len(list_len, list_cap);
  plan_tiles(nodes, list, n, tile_rows, max_tiles, prefix, desc, status, ctrl, splits, feature_col,
             n_features, multi, lds, status == nullptr);
}

// -------------------------------------------------------------- gradients --
// Pass 1: g_i = pred_i - (double)label_i; per-block max |g| (Training Core
// section 2; the grid of the fixed-point reading).
__global__ void __launch_bounds__(256) k_grad_max(const double* __restrict__ pred,
                                                  const float* __restrict__ label, int64_t n,
                                                  double* __restrict__ part,
                                                  WsCtrl* __restrict__ ctrl) {
  __shared__ double sh[4];
  double m = 0.0;
  bool bad = false;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  // four rows per thread per step, their loads issued together
  for (int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i0 < n; i0 += 4 * stride) {
    double p[4];
    float l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      p[u] = i < n ? pred[i] : 0.0;
      l[u] = i < n ? label[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double g = p[u] - (double)l[u];
      if (!isfinite(g)) bad = true;
      m = fmax(m, fabs(g));
    }
  }
  if (bad) dev_error(&ctrl->err, GBDT_E_RANGE);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    double r = fmax(fmax(sh[0], sh[1]), fmax(sh[2], sh[3]));
    part[blockIdx.x] = r;
  }
}

// Pass 2: M = max of the partial maxima (every block derives the same S),
// S = 52 - e - L, q_i = rint(ldexp(g_i, S)) and the sum of q.  QT: int64, or
// int32 for the tree driver when L >= 22 (then |q_i| <= 2^(52-L) <= 2^30).
template <typename QT>
__global__ void __launch_bounds__(256) k_grad_q(const double* __restrict__ pred,
                                                const float* __restrict__ label, int64_t n,
                                                int32_t log2n, const double* __restrict__ part,
                                                int32_t nparts, QT* __restrict__ q,
                                                int32_t* __restrict__ scale,
                                                int64_t* __restrict__ psum) {
  __shared__ double shm[4];
  __shared__ int64_t shs[4];
  double m = 0.0;
#pragma unroll
  for (int j = 0; j < kGradBlocks / 256; ++j) {
    const int i = j * 256 + threadIdx.x;
    if (i < nparts) m = fmax(m, part[i]);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) shm[threadIdx.x >> 6] = m;
  __syncthreads();
  const double M = fmax(fmax(shm[0], shm[1]), fmax(shm[2], shm[3]));
  int32_t S = 0;
  if (M > 0.0) {
    int e = 0;
    (void)frexp(M, &e);
    S = 52 - e - log2n;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = S;
  int64_t s = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i0 < n; i0 += 4 * stride) {
    double p[4];
    float l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      p[u] = i < n ? pred[i] : 0.0;
      l[u] = i < n ? label[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n) {
        const double g = p[u] - (double)l[u];
        const int64_t k = (int64_t)rint(ldexp(g, S));
        q[i] = (QT)k;
        s += k;
      }
    }
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) shs[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) psum[blockIdx.x] = shs[0] + shs[1] + shs[2] + shs[3];
}

// sum of q from the per-block partial sums (exact: integers)
__global__ void __launch_bounds__(kGradBlocks) k_grad_sum(const int64_t* __restrict__ psum,
                                                          int32_t nparts, int64_t* __restrict__ gsum) {
  __shared__ int64_t sh[kGradBlocks / 64];
  int64_t v = (int32_t)threadIdx.x < nparts ? psum[threadIdx.x] : 0;
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t t = 0;
    for (int w = 0; w < kGradBlocks / 64; ++w) t += sh[w];
    *gsum = t;
  }
}

// ------------------------------------------------- logistic objective --
// e^x for -700 <= x <= 0 (0 below -700): Cody and Waite's argument reduction,
// x = k ln 2 + r with k = rint(x / ln 2) and r = (x - k LN2_HI) - k LN2_LO
// (LN2_HI: the first 42 significant bits of ln 2, so k LN2_HI is exact;
// LN2_LO: the rest, rounded), then e^r by its Taylor series to degree 13
// (|r| <= ln(2)/2, the first omitted term below 2^-57 of the sum) in Horner
// form from the highest power, and e^x = 2^k e^r.  One IEEE FP64 operation at
// a time (no contraction in this library), so any IEEE host computing the
// same sequence gets the same bits.
__device__ __forceinline__ double exp_nonpos(double x) {
  if (x < -700.0) return 0.0;
  constexpr double kInvLn2 = 0x1.71547652b82fep+0;
  constexpr double kLn2Hi = 0x1.62e42fefa3800p-1;
  constexpr double kLn2Lo = 0x1.ef35793c76730p-45;
  // 1/j! for j = 13 .. 0, each correctly rounded
  constexpr double kInvFact[14] = {
      0x1.6124613a86d09p-33, 0x1.1eed8eff8d898p-29, 0x1.ae64567f544e4p-26, 0x1.27e4fb7789f5cp-22,
      0x1.71de3a556c734p-19, 0x1.a01a01a01a01ap-16, 0x1.a01a01a01a01ap-13, 0x1.6c16c16c16c17p-10,
      0x1.1111111111111p-7,  0x1.5555555555555p-5,  0x1.5555555555555p-3,  0x1.0000000000000p-1,
      0x1.0000000000000p+0,  0x1.0000000000000p+0};
  const double k = rint(x * kInvLn2);
  const double r = (x - k * kLn2Hi) - k * kLn2Lo;
  double p = kInvFact[0];
#pragma unroll
  for (int j = 1; j < 14; ++j) p = p * r + kInvFact[j];
  return ldexp(p, (int)k);
}

// Sigmoid cross-entropy on the raw score p ("Gradient boosted trees (spec
// model)", gbtBinaryCrossentropyGradSpec): g = sigmoid(p) - y, and the
// second derivative h = sigmoid(p) (1 - sigmoid(p)) as the Hessian, both from
// z = e^-|p| and d = 1 + z: sigmoid = 1/d for p >= 0, z/d otherwise;
// h = z / (d d).
__device__ __forceinline__ void logistic_gh(double p, double y, double& g, double& h) {
  const double z = exp_nonpos(-fabs(p));
  const double d = 1.0 + z;
  const double s = p >= 0.0 ? 1.0 / d : z / d;
  g = s - y;
  h = z / (d * d);
}

// Pass 1 of the logistic objective: per-block max |g| and max h (a
// non-finite prediction, label, g or h sets GBDT_E_RANGE).
__global__ void __launch_bounds__(256) k_lgrad_max(const double* __restrict__ pred,
                                                   const float* __restrict__ label, int64_t n,
                                                   double* __restrict__ part_g,
                                                   double* __restrict__ part_h,
                                                   WsCtrl* __restrict__ ctrl) {
  __shared__ double shg[4], shh[4];
  double mg = 0.0, mh = 0.0;
  bool bad = false;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i0 < n; i0 += 4 * stride) {
    double p[4];
    float l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      p[u] = i < n ? pred[i] : 0.0;
      l[u] = i < n ? label[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // (rows past n are skipped: at p = 0 their h = 1/4 would enter the max)
      if (i0 + u * stride >= n) continue;
      if (!isfinite(p[u]) || !isfinite((double)l[u])) {
        bad = true;
        continue;
      }
      double g, h;
      logistic_gh(p[u], (double)l[u], g, h);
      if (!isfinite(g) || !isfinite(h)) bad = true;
      mg = fmax(mg, fabs(g));
      mh = fmax(mh, h);
    }
  }
  if (bad) dev_error(&ctrl->err, GBDT_E_RANGE);
  mg = wave_max(mg);
  mh = wave_max(mh);
  if ((threadIdx.x & 63) == 0) {
    shg[threadIdx.x >> 6] = mg;
    shh[threadIdx.x >> 6] = mh;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    part_g[blockIdx.x] = fmax(fmax(shg[0], shg[1]), fmax(shg[2], shg[3]));
    part_h[blockIdx.x] = fmax(fmax(shh[0], shh[1]), fmax(shh[2], shh[3]));
  }
}

// The logistic objective's grid exponent for a largest magnitude M: the
// squared-error grid 52 - e - L, but at most 30 - e, so every fixed-point
// value fits 31 bits (M < 2^e); 0 when M = 0.
__device__ __forceinline__ int32_t logistic_scale(double M, int32_t log2n) {
  if (!(M > 0.0)) return 0;
  int e = 0;
  (void)frexp(M, &e);
  const int32_t S = 52 - e - log2n;
  return S < 30 - e ? S : 30 - e;
}

// Pass 2: both grids from the partial maxima (every block derives the same
// S and Sh), q = rint(ldexp(g, S)) and qh = rint(ldexp(h, Sh)) as int32, and
// per-block sums of each.
__global__ void __launch_bounds__(256) k_lgrad_q(const double* __restrict__ pred,
                                                 const float* __restrict__ label, int64_t n,
                                                 int32_t log2n, const double* __restrict__ part_g,
                                                 const double* __restrict__ part_h, int32_t nparts,
                                                 int32_t* __restrict__ q, int32_t* __restrict__ qh,
                                                 int32_t* __restrict__ scale,
                                                 int32_t* __restrict__ scale_h,
                                                 int64_t* __restrict__ psum,
                                                 int64_t* __restrict__ psum_h) {
  __shared__ double shg[4], shh[4];
  __shared__ int64_t ssg[4], ssh[4];
  double mg = 0.0, mh = 0.0;
#pragma unroll
  for (int j = 0; j < kGradBlocks / 256; ++j) {
    const int i = j * 256 + threadIdx.x;
    if (i < nparts) {
      mg = fmax(mg, part_g[i]);
      mh = fmax(mh, part_h[i]);
    }
  }
  mg = wave_max(mg);
  mh = wave_max(mh);
  if ((threadIdx.x & 63) == 0) {
    shg[threadIdx.x >> 6] = mg;
    shh[threadIdx.x >> 6] = mh;
  }
  __syncthreads();
  const int32_t S = logistic_scale(fmax(fmax(shg[0], shg[1]), fmax(shg[2], shg[3])), log2n);
  const int32_t Sh = logistic_scale(fmax(fmax(shh[0], shh[1]), fmax(shh[2], shh[3])), log2n);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *scale = S;
    *scale_h = Sh;
  }
  int64_t sg = 0, sh = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i0 < n; i0 += 4 * stride) {
    double p[4];
    float l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      p[u] = i < n ? pred[i] : 0.0;
      l[u] = i < n ? label[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n) {
        double g, h;
        logistic_gh(p[u], (double)l[u], g, h);
        const int32_t kg = (int32_t)rint(ldexp(g, S));
        const int32_t kh = (int32_t)rint(ldexp(h, Sh));
        q[i] = kg;
        qh[i] = kh;
        sg += kg;
        sh += kh;
      }
    }
  }
  sg = wave_sum(sg);
  sh = wave_sum(sh);
  if ((threadIdx.x & 63) == 0) {
    ssg[threadIdx.x >> 6] = sg;
    ssh[threadIdx.x >> 6] = sh;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    psum[blockIdx.x] = ssg[0] + ssg[1] + ssg[2] + ssg[3];
    psum_h[blockIdx.x] = ssh[0] + ssh[1] + ssh[2] + ssh[3];
  }
}

// Range check of caller-supplied fixed-point gradients (the per-call
// histogram entry point): |q_i| <= 2^(52 - ceil(log2 n)) for every row, the
// bound the packed LDS cells are sized for.  The tree driver's q comes from
// k_grad_q, which meets it by construction (|g| < 2^e, so |g 2^S| < 2^(52-L)).
__global__ void __launch_bounds__(256) k_check_q(const int64_t* __restrict__ q, int64_t n,
                                                 int64_t bound, WsCtrl* __restrict__ ctrl) {
  bool bad = false;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t x = q[i];
    bad |= (x > bound) || (x < -bound);
  }
  if (bad) dev_error(&ctrl->err, GBDT_E_OVERFLOW);
}

// -------------------------------------------------------------- histogram --
constexpr int kHistThreads = 1024;

// q of row r from a buffer of int64 or, with Q32, int32 elements (the tree
// driver stores q as int32 in its row buffers when |q| <= 2^30).
template <bool Q32>
__device__ __forceinline__ int64_t q_at(const void* q, int64_t r) {
  if (Q32) return (int64_t) reinterpret_cast<const int32_t*>(q)[r];
  return reinterpret_cast<const int64_t*>(q)[r];
}
// An LDS address as a pointer: a 32-bit byte address used by the ds
// instruction as it stands (the dynamic LDS of the histogram starts at 0).
typedef __attribute__((address_space(3))) uint64_t LdsU64;

// A 64-bit value moved within each quad of lanes by a DPP quad_perm (CTL).
template <int CTL>
__device__ __forceinline__ uint64_t dpp_quad64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTL, 0xf, 0xf, false);
  return ((uint64_t)hi << 32) | lo;
}
// The q of batch u for every lane of a row, from the lane of its quad that
// loaded it: quad position u (rows of 4 or 8 lanes), or u within each pair
// (rows of 2 lanes).  u is a constant after unrolling.
template <int D>
__device__ __forceinline__ uint64_t quad_bcast_batch(uint64_t v, int u) {
  constexpr bool P = D == 2;
  switch (u & 3) {
    case 0: return dpp_quad64<P ? 0xA0 : 0x00>(v);
    case 1: return dpp_quad64<P ? 0xF5 : 0x55>(v);
    case 2: return dpp_quad64<0xAA>(v);
    default: return dpp_quad64<0xFF>(v);
  }
}

// Vector load of UNIT bytes (4, 8 or 16) as dwords.
template <int UNIT>
struct VecLoad;
template <>
struct VecLoad<4> {
  static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* d) {
    d[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  static __device__ __forceinline__ void store(uint8_t* p, const uint32_t* d) {
    *reinterpret_cast<uint32_t*>(p) = d[0];
  }
};
template <>
struct VecLoad<8> {
  static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* d) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    d[0] = v.x;
    d[1] = v.y;
  }
  static __device__ __forceinline__ void store(uint8_t* p, const uint32_t* d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(d[0], d[1]);
  }
};
template <>
struct VecLoad<16> {
  static __device__ __forceinline__ void load(const uint8_t* p, uint32_t* d) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  }
  static __device__ __forceinline__ void store(uint8_t* p, const uint32_t* d) {
    *reinterpret_cast<uint4*>(p) = make_uint4(d[0], d[1], d[2], d[3]);
  }
};

// Widest of 16, 8, 4 bytes that divides the row stride of a block.
inline int load_unit_for(int32_t block_stride) {
  if (block_stride % 16 == 0) return 16;
  if (block_stride % 8 == 0) return 8;
  return 4;
}

// Filtered histogram tiles (the last level of a tree whose partition before
// it was skipped): the tile reads rows of its parent's segment and adds only
// those that go to the child it builds -- bin <= threshold for the left
// child, > threshold for the right one, the stable partition's rule
// ("Module Design: Training Core", section 6, step 5).  A tile descriptor
// marks it in n_left: 2 keeps the left-going rows, 3 the right-going ones;
// feature and threshold_bin carry the parent's split (the feature as its
// matrix column).  The row's split value is the field at `sh` (width mask)
// of the dword at base + row * stride.
struct RowFilter {
  const uint8_t* base;
  int64_t stride;
  uint32_t sh, mask;
  int32_t thr;
  bool left;
};

__device__ __forceinline__ bool tile_filtered(const TileDesc& td) { return td.n_left >= 2; }

__device__ inline RowFilter row_filter(const TileDesc& td, const uint8_t* bins, int64_t row_capacity,
                                       int32_t n_blocks, int32_t block_features, int32_t block_stride,
                                       int32_t n_features, int32_t n_bit, int32_t bit_stride,
                                       int32_t n_nib, int32_t nib_stride, WsCtrl* ctrl) {
  RowFilter f;
  const int32_t nbc = n_features - n_bit;  // first bit column
  const int32_t nbyte = nbc - n_nib;       // first nibble column
  const int32_t c = td.feature;
  const uint8_t* bits = bins + int64_t(n_blocks) * row_capacity * block_stride;
  const uint8_t* nibs = bits + row_capacity * bit_stride;
  f.left = td.n_left == 2;
  f.thr = td.threshold_bin;
  if (c < 0 || c >= n_features || td.n_left > 3) {
    // (not a valid split: no row is kept, and the error word is set)
    if (threadIdx.x == 0 && ctrl != nullptr) dev_error(&ctrl->err, GBDT_E_INTERNAL);
    f.base = bins;
    f.stride = 0;
    f.sh = 0u;
    f.mask = 0u;
    f.thr = -1;
    f.left = true;
  } else if (c >= nbc) {
    const int32_t k = c - nbc;
    f.base = bits + 4 * (k >> 5);
    f.stride = bit_stride;
    f.sh = (uint32_t)(k & 31);
    f.mask = 1u;
  } else if (c >= nbyte) {
    const int32_t k = c - nbyte;
    f.base = nibs + 4 * (k >> 3);
    f.stride = nib_stride;
    f.sh = 4u * (uint32_t)(k & 7);
    f.mask = 15u;
  } else {
    const int32_t b = c / block_features;
    const int32_t j = c - b * block_features;
    f.base = bins + int64_t(b) * row_capacity * block_stride + (j & ~3);
    f.stride = block_stride;
    f.sh = 8u * (uint32_t)(j & 3);
    f.mask = 0xffu;
  }
  return f;
}

__device__ __forceinline__ uint32_t filter_dword(const RowFilter& f, int64_t row) {
  return *reinterpret_cast<const uint32_t*>(f.base + row * f.stride);
}

__device__ __forceinline__ bool filter_keep(const RowFilter& f, uint32_t dw) {
  return ((int32_t)((dw >> f.sh) & f.mask) <= f.thr) == f.left;
}

// Histogram of a tile's bit features (the bit block), with 2 LDS slots per
// bit feature k (its bins 0 and 1).  Per feature the rarer value is
// accumulated -- the skip bin, 0 when none is set, is the frequent one -- by
// walking the set bits of (word ^ inverse mask) of each row: one LDS atomic
// per rare cell; the frequent bin is the tile total minus the rare one.
// Lanes are (row group, word of 32 bit features).
constexpr int kBitStage = 1024;   // bit features whose output table is staged in LDS
constexpr int kMaxBitWords = 128; // words per row of the bit block, at most

template <int NW, bool Q32, bool FILT>
__device__ void hist_bit_block(const TileDesc& td, const RowFilter& flt, int32_t tile,
                               const uint8_t* __restrict__ bins,
                               int64_t row_capacity, int32_t n_blocks, int32_t block_stride,
                               int32_t n_features, int32_t n_bit, int32_t bit_stride,
                               const int32_t* __restrict__ col_feature, const void* __restrict__ q,
                               const int32_t* __restrict__ bin_offset,
                               const int32_t* __restrict__ skip_bin, int32_t total_bins,
                               int32_t lds_bins, int32_t bits,
                               int64_t* __restrict__ hist_g, uint32_t* __restrict__ hist_cnt,
                               uint64_t* __restrict__ partial, WsCtrl* __restrict__ ctrl,
                               uint64_t* lds, uint32_t* s_inv, int32_t* s_bit, uint64_t* sh_tot) {
  const int32_t nbc = n_features - n_bit;
  const int32_t nwords = bit_stride >> 2;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  if (2 * n_bit > lds_bins) {
    if (threadIdx.x == 0) dev_error(&ctrl->err, GBDT_E_SHAPE);
    return;
  }
  for (int32_t b = threadIdx.x; b < 2 * n_bit; b += blockDim.x) lds[b] = 0ull;
  for (int32_t w = threadIdx.x; w < nwords; w += blockDim.x) s_inv[w] = 0u;
  __syncthreads();
  // per bit feature: its global bins and whether its skip bin is 1
  for (int32_t kk = threadIdx.x; kk < n_bit; kk += blockDim.x) {
    int32_t f = col_feature[nbc + kk];
    f = f < 0 ? 0 : (f >= n_features ? n_features - 1 : f);
    const int32_t lo = bin_offset[f];
    const int32_t nb = bin_offset[f + 1] - lo;
    const int32_t sk = skip_bin != nullptr ? skip_bin[f] : -1;
    const uint32_t inv = (sk == 1 && nb == 2) ? 1u : 0u;
    if (inv) atomicOr(&s_inv[kk >> 5], 1u << (kk & 31));
    if (kk < kBitStage) s_bit[kk] = (lo << 2) | ((nb == 2 ? 1 : 0) << 1) | (int32_t)inv;
  }
  __syncthreads();
  const int64_t r0 = td.r0;
  const int64_t r1 = td.r1;
  const int32_t rpi = (int32_t)blockDim.x / nwords;  // rows per step
  const int32_t w = (int32_t)threadIdx.x % nwords;
  const int32_t rg = (int32_t)threadIdx.x / nwords;
  const uint32_t inv = s_inv[w < nwords ? w : 0];
  const int32_t kbase = 32 * w;
  const uint32_t valid = kbase + 32 <= n_bit ? 0xffffffffu
                                             : (kbase >= n_bit ? 0u : ((1u << (n_bit - kbase)) - 1u));
  const uint32_t* __restrict__ wb = reinterpret_cast<const uint32_t*>(
      bins + int64_t(n_blocks) * row_capacity * block_stride);
  uint64_t tot = 0ull;
  constexpr int BATCH = 4;
  if (rg < rpi) {
    for (int64_t r = r0 + rg; r < r1; r += int64_t(BATCH) * rpi) {
      uint32_t x[BATCH], fx[BATCH];
      int64_t qq[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t rr = r + int64_t(u) * rpi;
        const bool ok = rr < r1;
        x[u] = ok ? wb[rr * nwords + w] : 0u;
        qq[u] = ok ? q_at<Q32>(q, rr) : 0;
        if (FILT) fx[u] = ok ? filter_dword(flt, rr) : 0u;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t rr = r + int64_t(u) * rpi;
        if (rr >= r1) continue;
        if (FILT && !filter_keep(flt, fx[u])) continue;
        const uint64_t pk = ((uint64_t)qq[u] << bits) + 1ull;
        tot += pk;
        uint32_t m = (x[u] ^ inv) & valid;
        while (m) {
          const int32_t t = __builtin_ctz(m);
          m &= m - 1u;
          const int32_t slot = 2 * (kbase + t) + (int32_t)(1u ^ ((inv >> t) & 1u));
          __hip_atomic_fetch_add(&lds[slot], pk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  }
  const uint64_t t0 = wave_sum_dpp((w == 0 && rg < rpi) ? tot : 0ull);
  if (lane == 0) sh_tot[wid] = t0;
  __syncthreads();
  uint64_t tile_total = 0ull;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) tile_total += sh_tot[ww];
  // the frequent bin of each bit feature: tile total minus the rare one
  for (int32_t kk = threadIdx.x; kk < n_bit; kk += blockDim.x) {
    const int32_t iv = (int32_t)((s_inv[kk >> 5] >> (kk & 31)) & 1u);
    lds[2 * kk + iv] = tile_total - lds[2 * kk + (1 - iv)];
  }
  __syncthreads();
  const uint64_t mask = (1ull << bits) - 1ull;
  const int32_t v = td.node;
  for (int32_t e = threadIdx.x; e < 2 * n_bit; e += blockDim.x) {
    const int32_t kk = e >> 1, b = e & 1;
    int32_t lo, two;
    if (kk < kBitStage) {
      lo = s_bit[kk] >> 2;
      two = (s_bit[kk] >> 1) & 1;
    } else {
      int32_t f = col_feature[nbc + kk];
      f = f < 0 ? 0 : (f >= n_features ? n_features - 1 : f);
      lo = bin_offset[f];
      two = bin_offset[f + 1] - lo == 2;
    }
    if (b == 1 && !two) continue;  // a one-bin feature
    const uint64_t xv = lds[e];
    if (td.ntiles == 1) {
      const uint64_t c = xv & mask;
      hist_g[int64_t(v) * total_bins + lo + b] = (int64_t)(xv - c) >> bits;
      hist_cnt[int64_t(v) * total_bins + lo + b] = (uint32_t)c;
    } else {
      partial[int64_t(tile) * total_bins + lo + b] = xv;
    }
  }
}

// The nibble block: lanes are (row group, word of 8 nibble features).  Each
// row's word gives 8 cells; every cell except the feature's skip bin (its
// most frequent bin, derived from the tile total at the end) adds the packed
// (q << bits) + 1 to its LDS slot with one 64-bit atomic.  Feature k's 16
// slots are rotated by k (slot 16 k + ((b + k) & 15)), so equal bins of
// different features fall in different bank pairs, and each lane walks its 8
// nibbles starting at nibble (row group & 7), so the lanes of a quarter-wave
// address several features at once.
template <int NW, bool Q32, bool FILT>
__device__ void hist_nib_block(const TileDesc& td, const RowFilter& flt, int32_t tile,
                               const uint8_t* __restrict__ bins,
                               int64_t row_capacity, int32_t n_blocks, int32_t block_stride,
                               int32_t n_features, int32_t n_bit, int32_t bit_stride, int32_t n_nib,
                               int32_t nib_stride, const int32_t* __restrict__ col_feature,
                               const void* __restrict__ q, const int32_t* __restrict__ bin_offset,
                               const int32_t* __restrict__ skip_bin, int32_t total_bins,
                               int32_t lds_bins, int32_t bits, int64_t* __restrict__ hist_g,
                               uint32_t* __restrict__ hist_cnt, uint64_t* __restrict__ partial,
                               WsCtrl* __restrict__ ctrl, uint64_t* lds, uint32_t* s_skip,
                               uint64_t* sh_tot) {
  const int32_t nbyte = n_features - n_bit - n_nib;  // nibble k is column nbyte + k
  const int32_t nwords = nib_stride >> 2;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  if (kNibSlots * n_nib > lds_bins || nwords > kMaxBitWords) {
    if (threadIdx.x == 0) dev_error(&ctrl->err, GBDT_E_SHAPE);
    return;
  }
  for (int32_t b = threadIdx.x; b < kNibSlots * n_nib; b += blockDim.x) lds[b] = 0ull;
  // per word: the skip bins of its 8 features as nibbles (16 = none: no cell matches)
  for (int32_t w = threadIdx.x; w < nwords; w += blockDim.x) {
    uint32_t sk = 0u, none = 0u;
    for (int32_t t = 0; t < 8; ++t) {
      const int32_t kk = 8 * w + t;
      int32_t b = -1;
      if (kk < n_nib && skip_bin != nullptr) {
        int32_t f = col_feature[nbyte + kk];
        f = f < 0 ? 0 : (f >= n_features ? n_features - 1 : f);
        b = skip_bin[f];
      }
      if (b >= 0 && b < 16)
        sk |= uint32_t(b) << (4 * t);
      else
        none |= 1u << t;
    }
    s_skip[2 * w] = sk;
    s_skip[2 * w + 1] = none;
  }
  __syncthreads();
  const int64_t r0 = td.r0;
  const int64_t r1 = td.r1;
  const int32_t rpi = (int32_t)blockDim.x / nwords;  // rows per step
  const int32_t w = (int32_t)threadIdx.x % nwords;
  const int32_t rg = (int32_t)threadIdx.x / nwords;
  const uint32_t skw = s_skip[2 * (w < nwords ? w : 0)];
  const uint32_t none = s_skip[2 * (w < nwords ? w : 0) + 1];
  const int32_t kbase = 8 * w;
  const int32_t nval = n_nib - kbase < 8 ? n_nib - kbase : 8;  // this word's features
  const int32_t rot = rg & 7;
  const uint32_t* __restrict__ wb = reinterpret_cast<const uint32_t*>(
      bins + int64_t(n_blocks) * row_capacity * block_stride + row_capacity * bit_stride);
  uint64_t tot = 0ull;
  constexpr int BATCH = 4;
  if (rg < rpi) {
    for (int64_t r = r0 + rg; r < r1; r += int64_t(BATCH) * rpi) {
      uint32_t x[BATCH], fx[BATCH];
      int64_t qq[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t rr = r + int64_t(u) * rpi;
        const bool ok = rr < r1;
        x[u] = ok ? wb[rr * nwords + w] : 0u;
        qq[u] = ok ? q_at<Q32>(q, rr) : 0;
        if (FILT) fx[u] = ok ? filter_dword(flt, rr) : 0u;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int64_t rr = r + int64_t(u) * rpi;
        if (rr >= r1) continue;
        if (FILT && !filter_keep(flt, fx[u])) continue;
        const uint64_t pk = ((uint64_t)qq[u] << bits) + 1ull;
        tot += pk;
        const uint32_t diff = x[u] ^ skw;
#pragma unroll 1
        for (int m = 0; m < 8; ++m) {
          const int32_t t = (m + rot) & 7;
          if (t >= nval) continue;
          const bool is_skip = ((diff >> (4 * t)) & 15u) == 0u && !((none >> t) & 1u);
          if (is_skip) continue;
          const int32_t kk = kbase + t;
          const int32_t b = (int32_t)((x[u] >> (4 * t)) & 15u);
          __hip_atomic_fetch_add(&lds[kNibSlots * kk + ((b + kk) & 15)], pk, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  }
  const uint64_t t0 = wave_sum_dpp((w == 0 && rg < rpi) ? tot : 0ull);
  if (lane == 0) sh_tot[wid] = t0;
  __syncthreads();
  uint64_t tile_total = 0ull;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) tile_total += sh_tot[ww];
  // each feature's skip bin: the tile total minus its other bins
  for (int32_t kk = threadIdx.x; kk < n_nib; kk += blockDim.x) {
    const uint32_t sk = s_skip[2 * (kk >> 3)], nn = s_skip[2 * (kk >> 3) + 1];
    if ((nn >> (kk & 7)) & 1u) continue;
    const int32_t sb = (int32_t)((sk >> (4 * (kk & 7))) & 15u);
    uint64_t rest = 0ull;
    for (int32_t b = 0; b < 16; ++b)
      if (b != sb) rest += lds[kNibSlots * kk + ((b + kk) & 15)];
    lds[kNibSlots * kk + ((sb + kk) & 15)] = tile_total - rest;
  }
  __syncthreads();
  const uint64_t mask = (1ull << bits) - 1ull;
  const int32_t v = td.node;
  for (int32_t e = threadIdx.x; e < kNibSlots * n_nib; e += blockDim.x) {
    const int32_t kk = e >> 4, b = e & 15;
    int32_t f = col_feature[nbyte + kk];
    f = f < 0 ? 0 : (f >= n_features ? n_features - 1 : f);
    const int32_t lo = bin_offset[f];
    if (b >= bin_offset[f + 1] - lo) continue;
    const uint64_t xv = lds[kNibSlots * kk + ((b + kk) & 15)];
    if (td.ntiles == 1) {
      const uint64_t c = xv & mask;
      hist_g[int64_t(v) * total_bins + lo + b] = (int64_t)(xv - c) >> bits;
      hist_cnt[int64_t(v) * total_bins + lo + b] = (uint32_t)c;
    } else {
      partial[int64_t(tile) * total_bins + lo + b] = xv;
    }
  }
}

// One workgroup = one (tile of one node's rows, column block); the block
// index n_blocks is the bit block (hist_bit_block).
//
// Byte blocks (at most 32 columns, rows of at most 8 dwords).  Lanes are
// (row group rg, dword c of the row) with D lanes per row (D = the row's
// dwords rounded up to a power of two); each lane loads one dword of a row
// and adds the packed cell (q << bits) + 1 to the LDS slot of each of its 4
// bytes with a 64-bit LDS atomic.  The LDS histogram is bank-skewed: the
// slot of (copy k, column j, bin b) is 32 b + 4 D k + j, so a slot's bank
// pair (slot mod 16 for 8-byte slots) does not depend on the bin.  gfx950
// serves a wave's 64-bit LDS atomic one quarter-wave (16 lanes) at a time
// and a quarter takes as many passes as lanes meet on one bank pair; each
// lane therefore walks its 4 bytes in a rotated order (byte (m + rot) & 3 in
// step m) chosen so that the 16 lanes of every quarter-wave always address
// 16 different bank pairs, whatever the bin values (a hot bin included):
//   D = 8: rot = (rg & 1) + 2 ((c >> 2) xor ((rg >> 1) & 1)), one copy (32
//   columns); rows of adjacent quarter-waves then never share a (column,
//   byte) slot, so a hot bin cannot make consecutive passes of one
//   instruction update the same address (the earlier rot = (rg & 1) +
//   2 (c >> 2) shared it between all rows of one parity);
//   D = 4: rot = rg & 3, one copy;
//   D = 2 or 1: rot = rg & 3 and 4 / D copies picked by (rg >> 2), summed at
//   the end.
// The slot's byte address, bin * 256 + lane offset, is one v_perm_b32 of the
// row dword and a register holding the lane's four offsets.  Rows past the
// tile end add 0; lanes past the row's dwords and padding bytes (always 0)
// land in columns that are never read.  256 bin rows are allocated, so any
// byte value stays inside the allocation; the first lds_bins / 32 rows are
// zeroed and read back.  A node covered by one tile writes its decoded
// histogram straight to hist; otherwise the tile writes its packed partial
// (global bin order) for k_hist_reduce.  NARROW: 0 byte blocks only; 1 a bit
// block too; 2 a nibble block (and maybe a bit block) too -- each variant
// carries only the code its layout needs.
template <int D, int NARROW, bool Q32, bool IDS = false, bool FILT = false>
__global__ void GBDT_SGPR_CAP GBDT_TWO_GROUPS __launch_bounds__(kHistThreads) k_hist(
    const uint8_t* __restrict__ bins, int64_t row_capacity, int32_t n_blocks,
    int32_t block_features, int32_t block_stride, int32_t n_features, int32_t n_bit,
    int32_t bit_stride, const int32_t* __restrict__ col_feature, const void* __restrict__ q,
    const int32_t* __restrict__ bin_offset, const int32_t* __restrict__ skip_bin,
    int32_t total_bins, int32_t lds_bins, const TileDesc* __restrict__ desc, int32_t bits,
    int64_t* __restrict__ hist_g, uint32_t* __restrict__ hist_cnt,
    uint64_t* __restrict__ partial, WsCtrl* __restrict__ ctrl, const int32_t* __restrict__ guard,
    int32_t n_nib, int32_t nib_stride, const int32_t* __restrict__ ridx, int64_t id_blk_pitch,
    int32_t id_row_pitch, int32_t id_tiles) {
  static_assert(D == 1 || D == 2 || D == 4 || D == 8, "lanes per row");
  static_assert(!IDS || NARROW == 0, "index mode reads byte blocks only");
  static_assert(!(IDS && FILT), "filtered tiles read rows in order");
  if (failed(guard)) return;
  constexpr int RPW = 64 / D;               // rows per wave per batch
  constexpr int RPI = kHistThreads / D;     // rows per workgroup per batch
  constexpr int BATCH = D >= 4 ? D : 4;     // batches per step (1024 rows a step for D >= 4)
  constexpr int NCOPY = D >= 4 ? 1 : 4 / D; // histogram copies (bank skew of narrow rows)
  constexpr int W = 4 * D;                  // slots of one copy in a bin row
  constexpr int NW = kHistThreads / 64;
  // All LDS is dynamic, so the histogram slots start at LDS address 0 and a
  // v_perm result is the atomic's address as it stands; the small tables
  // follow the kLdsHistBudgetBins slots.
  extern __shared__ uint64_t lds[];
  uint64_t* const sh_tot = lds + kLdsHistBudgetBins;                        // [NW]
  int32_t* const s_fbins = reinterpret_cast<int32_t*>(sh_tot + NW);        // [kHistRowSlots]
  int32_t* const s_fgb = s_fbins + kHistRowSlots;                          // [kHistRowSlots]
  uint32_t* const s_inv = reinterpret_cast<uint32_t*>(s_fgb + kHistRowSlots);  // [kMaxBitWords]
  int32_t* const s_bit = reinterpret_cast<int32_t*>(s_inv + kMaxBitWords);  // [kBitStage]
  // id_tiles > 0 (index mode with the interleaved copy; byte blocks only): a
  // 1-D grid in which workgroup w takes block (w / 8) % n_blocks of tile
  // (w / (8 n_blocks)) 8 + w % 8.  Workgroups go to the XCDs in turn, so
  // w % 8 -- the tile's residue -- names the XCD: the blocks of one tile,
  // which read the same q and, gathering, a row's cache lines, all run on
  // one XCD, next to each other in time, and its L2 serves them all.
  int32_t tile = blockIdx.x;
  int32_t blk = blockIdx.y;
  if (NARROW == 0 && id_tiles > 0) {
    const int32_t w = blockIdx.x;
    blk = (w >> 3) % n_blocks;
    tile = (w / (8 * n_blocks)) * 8 + (w & 7);
    if (tile >= id_tiles) return;
  }
  const TileDesc td = desc[tile];
  // FILT: every tile of the plan is filtered (a plan either filters all its
  // tiles or none)
  RowFilter flt{};
  if constexpr (FILT) {
    if (td.node >= 0)
      flt = row_filter(td, bins, row_capacity, n_blocks, block_features, block_stride, n_features,
                       n_bit, bit_stride, n_nib, nib_stride, blk == 0 ? ctrl : nullptr);
  }
  if (NARROW > 0 && blk >= n_blocks) {  // the narrow blocks: bits, then nibbles
    if (td.node < 0) return;
    if (blk == n_blocks && n_bit > 0) {
      if ((bit_stride >> 2) > kMaxBitWords) {  // the host checks bit_stride <= 4 * kMaxBitWords
        if (threadIdx.x == 0) dev_error(&ctrl->err, GBDT_E_SHAPE);
        return;
      }
      hist_bit_block<NW, Q32, FILT>(td, flt, td.slot, bins, row_capacity, n_blocks, block_stride, n_features, n_bit,
                         bit_stride, col_feature, q, bin_offset, skip_bin, total_bins, lds_bins, bits,
                         hist_g, hist_cnt, partial, ctrl, lds, s_inv, s_bit, sh_tot);
    } else if constexpr (NARROW == 2) {
      if (blk == n_blocks + (n_bit > 0 ? 1 : 0) && n_nib > 0)
        hist_nib_block<NW, Q32, FILT>(td, flt, td.slot, bins, row_capacity, n_blocks, block_stride, n_features, n_bit,
                           bit_stride, n_nib, nib_stride, col_feature, q, bin_offset, skip_bin,
                           total_bins, lds_bins, bits, hist_g, hist_cnt, partial, ctrl, lds, s_inv,
                           sh_tot);
    }
    return;
  }
  if (blk >= n_blocks) return;
  // The column table (lane j of wave 0: column f0 + j) is needed only by the
  // output, so its loads are issued here and consumed after the row loop.
  const int32_t nbc = n_features - n_bit - n_nib;
  const int32_t f0 = blk * block_features;  // first byte column of the block
  const int32_t c1 = f0 + block_features < nbc ? f0 + block_features : nbc;
  const int32_t nf = c1 - f0;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const bool tval = lane < nf;
  int32_t tf = col_feature != nullptr ? col_feature[tval ? f0 + lane : f0] : (tval ? f0 + lane : f0);
  tf = tf < 0 ? 0 : (tf >= n_features ? n_features - 1 : tf);
  int32_t t_lo = 0, t_hi = 0;
  if (wid == 0) {
    t_lo = bin_offset[tf];
    t_hi = bin_offset[tf + 1];
  }
  asm volatile("" ::: "memory");
  if (td.node < 0) return;  // beyond the plan
  const int32_t rows_out = lds_bins >> 5;  // bin rows zeroed and read back (<= 256)
  {
    uint4* z = reinterpret_cast<uint4*>(lds);
    for (int32_t i = threadIdx.x; i < rows_out * (kHistRowSlots / 2); i += kHistThreads)
      z[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (wid == 0 && lane < kHistRowSlots) {
    s_fbins[lane] = tval ? t_hi - t_lo : 0;
    s_fgb[lane] = t_lo;
  }
  // lane roles and the four LDS byte offsets of the lane's bytes
  const int32_t c = threadIdx.x % D;
  const int32_t rg = threadIdx.x / D;
  const int32_t rot = D == 8 ? (((rg & 1) + 2 * (((c >> 2) ^ (rg >> 1)) & 1)) & 3) : (rg & 3);
  const int32_t copy = NCOPY == 1 ? 0 : ((rg >> 2) & (NCOPY - 1));
  uint32_t offs = 0u;
  uint32_t sel[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t bm = (uint32_t)((m + rot) & 3);
    const uint32_t off = 8u * (uint32_t)(copy * W + 4 * c + (int32_t)bm);  // < 256
    offs |= off << (8 * m);
    // result byte 0 = offs byte m, byte 1 = row byte bm, bytes 2-3 = 0
    sel[m] = (uint32_t)m | ((4u + bm) << 8) | 0x0c0c0000u;
  }
  const int32_t nd = block_stride >> 2;  // dwords of a row (>= 1)
  const uint32_t lane_off = 4u * (uint32_t)(c < nd ? c : nd - 1);  // loads stay inside the row
  const int64_t r0 = td.r0;
  const int64_t r1 = td.r1;
  __syncthreads();
  // A stage covers SROWS = RPI * H rows in H batches.  Within a stage each
  // wave owns H * RPW consecutive rows, batch u of them rows
  // [first + u RPW, first + (u + 1) RPW): a wave reads whole runs of cache
  // lines, so no line is shared by waves that may drift apart in time (with
  // batches RPI rows apart, a line at each 8-row boundary was fetched by two
  // waves, and the 50M x 28 root read 40 bytes per 32-byte row).  The loop
  // is an NS-stage pipeline: while one stage's atomics run, the loads of the
  // next NS - 1 stages are in flight, and each stage reloads NS stages ahead
  // as soon as its atomics are issued.  Loads are unconditional: a row past
  // the tile end reads the tile's last row (the wave's first row of the
  // stage is < r1, so it exists); the reloads after the last stage read rows
  // that are never used.  Loop bounds are wave-uniform.
  constexpr int H = BATCH / 2;
  // (three or four stages keep more loads in flight but measured the same)
  constexpr int NS = 2;
  constexpr int32_t SROWS = RPI * H;
  // rows are addressed from the tile's first row: a uniform base plus a
  // 32-bit lane offset (a tile holds < 2^24 rows of at most 32 bytes)
  const int32_t nt = (int32_t)(r1 - r0);    // rows of the tile
  // IDS: the tile's positions r0 .. r1 hold the row ids ridx[r0 ..] of the
  // matrix, whose row id's block starts at bins + blk id_blk_pitch + id
  // id_row_pitch (block-major: row_capacity block_stride and block_stride;
  // interleaved: block_stride and n_blocks block_stride); a row id outside
  // the matrix is clamped to its last row, so no load leaves the matrix
  const uint8_t* __restrict__ tb = IDS ? bins + int64_t(blk) * id_blk_pitch
                                       : bins + (int64_t(blk) * row_capacity + r0) * block_stride;
  const int32_t* __restrict__ trid = IDS ? ridx + r0 : nullptr;
  const uint32_t last_row = (uint32_t)(row_capacity > 0 ? row_capacity - 1 : 0);
  auto row_dword_at = [&](uint32_t rc) -> uint32_t {
    if constexpr (IDS) {
      const uint32_t id = (uint32_t)trid[rc];
      return *reinterpret_cast<const uint32_t*>(
          tb + (int64_t(id < last_row ? id : last_row) * id_row_pitch + lane_off));
    } else {
      return *reinterpret_cast<const uint32_t*>(tb + (__umul24(rc, (uint32_t)block_stride) + lane_off));
    }
  };
  constexpr uint32_t QSH = Q32 ? 2u : 3u;  // log2 of q's element size
  const char* __restrict__ tq = reinterpret_cast<const char*>(q) + (r0 << QSH);
  const int32_t first_row = wid * (H * RPW) + lane / D;  // the lane's first row in the tile
  // (the wave's row base in a scalar register, so the loop exits are
  // uniform branches and the load counters stay exact across them)
  int32_t base = __builtin_amdgcn_readfirstlane(wid * (H * RPW));
  if (base < nt) {
    const int32_t lr = nt - 1;
    // q: with D >= 2 lanes per row, lane (row group, c) loads q of its row
    // in batch c % H of the stage, so one load per stage serves H batches and
    // batch u's q is taken from a lane of the same quad with a DPP move
    // (c % H == u: quad position u, or u and u + 2 for D == 2 pairs); with
    // D == 1 every lane loads its own row's q per batch.
    constexpr int NQ = D >= 2 ? 1 : H;
    // q stays in its stored width until it is used (a widening right after
    // the load would make the wave wait for it there)
    using QT = typename std::conditional<Q32, int32_t, int64_t>::type;
    uint32_t xs[NS][H];
    QT qs[NS][NQ];
    uint32_t fs[NS][NQ];  // FILT: the split dwords of the rows whose q the lane loads
    // Rows past the tile end are clamped to its last row and added like any
    // other row; the exact correction after the loop subtracts those copies
    // (packed sums are exact mod 2^64), so the loop needs no masks.  Lanes
    // past the row's dwords reread its last dword into columns >= 4 nd,
    // which are never read.  The empty asm takes the loaded values as
    // operands where they are used, so the compiler can neither drop a load
    // nor wait for it early.
    auto load_half = [&](int32_t first, uint32_t* x, QT* qq, uint32_t* ff) {
#pragma unroll
      for (int u = 0; u < H; ++u) {
        const int32_t rr = first + u * RPW + (lane / D);
        const uint32_t rc = (uint32_t)(rr < lr ? rr : lr);
        x[u] = row_dword_at(rc);
        if (D == 1) {
          qq[u < NQ ? u : 0] = *reinterpret_cast<const QT*>(tq + (rc << QSH));
          if (FILT) ff[u < NQ ? u : 0] = filter_dword(flt, r0 + rc);
        }
      }
      if (D >= 2) {
        const int32_t rr = first + (c % H) * RPW + (lane / D);
        const uint32_t rc = (uint32_t)(rr < lr ? rr : lr);
        qq[0] = *reinterpret_cast<const QT*>(tq + (rc << QSH));
        if (FILT) ff[0] = filter_dword(flt, r0 + rc);
      }
    };
    // (FILT: a row the filter drops adds the packed value 0)
    auto add_half = [&](uint32_t* x, QT* qq, uint32_t* ff) {
      uint64_t pkh = 0ull;
      if (D >= 2) {
        asm volatile("" : "+v"(qq[0]));
        pkh = ((uint64_t)(int64_t)qq[0] << bits) | 1ull;
        if (FILT) {
          asm volatile("" : "+v"(ff[0]));
          if (!filter_keep(flt, ff[0])) pkh = 0ull;
        }
      }
#pragma unroll
      for (int u = 0; u < H; ++u) {
        uint64_t pk;
        if (D >= 2) {
          asm volatile("" : "+v"(x[u]));
          pk = quad_bcast_batch<D>(pkh, u);
        } else {
          asm volatile("" : "+v"(x[u]), "+v"(qq[u < NQ ? u : 0]));
          pk = ((uint64_t)(int64_t)qq[u < NQ ? u : 0] << bits) | 1ull;
          if (FILT) {
            asm volatile("" : "+v"(ff[u < NQ ? u : 0]));
            if (!filter_keep(flt, ff[u < NQ ? u : 0])) pk = 0ull;
          }
        }
        // (FILT: a dropped row's lanes issue no atomics; a kept row's
        // packed value is never 0, its count bit being set)
        if (FILT && pk == 0ull) continue;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t a = __builtin_amdgcn_perm(x[u], offs, sel[m]);
          __hip_atomic_fetch_add(reinterpret_cast<LdsU64*>((uintptr_t)a), pk, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    };
    // The first stages are issued in stage order (the empty asm with a
    // memory clobber keeps the compiler from interleaving them), so the load
    // counter at the loop head is the same from the prologue as from the
    // previous iteration, and stage 0 waits only for its own loads.
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      load_half(base + st * SROWS, xs[st], qs[st], fs[st]);
      asm volatile("" ::: "memory");
    }
    // the tile's last row, for the correction below, loaded with the first
    // rows so that no round trip follows the loop
    uint32_t x_last = row_dword_at((uint32_t)lr);
    QT q_last = *reinterpret_cast<const QT*>(tq + (uint32_t(lr) << QSH));
    uint32_t f_last = FILT ? filter_dword(flt, r0 + lr) : 0u;
    // The wave needs `todo` stages (wave-uniform).  Each loop iteration
    // adds NS stages and reloads each NS stages ahead, unconditionally; the
    // last 1..NS stages are added after the loop from the buffers already
    // loaded.  The loop thus has one exit and its back edge one load-counter
    // state, so a stage waits only for its own loads.
    int32_t todo = (nt - base + SROWS - 1) / SROWS;
    const int32_t stages = todo;
    while (todo > NS) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        add_half(xs[st], qs[st], fs[st]);
        load_half(base + (st + NS) * SROWS, xs[st], qs[st], fs[st]);
      }
      base += NS * SROWS;
      todo -= NS;
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
      if (st < todo) add_half(xs[st], qs[st], fs[st]);
    asm volatile("" : "+v"(x_last), "+v"(q_last), "+v"(f_last));
    // the lane visited rows first_row + u RPW + s SROWS, u < H, s < stages;
    // those at or past nt were row lr
    int32_t valid = 0;
#pragma unroll
    for (int u = 0; u < H; ++u) {
      const int32_t r = first_row + u * RPW;
      valid += r < nt ? (nt - r + SROWS - 1) / SROWS : 0;
    }
    const int32_t extra = stages * H - valid;
    if (extra > 0) {
      const uint32_t x = x_last;
      const int64_t qq = (int64_t)q_last;
      const uint64_t one = (FILT && !filter_keep(flt, f_last)) ? 0ull : (((uint64_t)qq << bits) | 1ull);
      const uint64_t pk = one * (0ull - (uint64_t)extra);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a = __builtin_amdgcn_perm(x, offs, sel[m]);
        __hip_atomic_fetch_add(reinterpret_cast<LdsU64*>((uintptr_t)a), pk, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
  __syncthreads();
  // Output in three steps, so that global writes run along the bins: (1)
  // thread t reads column t % 32 of bin rows t / 32 + 32 i (consecutive
  // threads on consecutive columns, i.e. distinct bank pairs), summing the
  // copies; (2) after a barrier it writes them back transposed, column j at
  // j * RP + ((cb + j) mod RP) with RP = R rounded up to a power of two (the
  // rotation keeps consecutive columns on distinct bank pairs; nf * RP <=
  // 8192 slots); (3) after another barrier consecutive threads take
  // consecutive bins of one column and write the decoded histogram or the
  // packed partial at global bin s_fgb[j] + cb.  Bin-row order had each
  // wave's 64 writes land a feature's bin count apart, one cache line each
  // (10M x 100 histogram levels: 18 us of 80).
  const uint64_t mask = (1ull << bits) - 1ull;
  const int32_t v = td.node;
  const int32_t R = rows_out;
  int32_t lrp = 0;  // log2 of RP
  while ((1 << lrp) < R) ++lrp;
  const int32_t RP = 1 << lrp;
  constexpr int MAXV = 256 / (kHistThreads / kHistRowSlots);  // bin rows per thread
  const int32_t oc = (int32_t)threadIdx.x & (kHistRowSlots - 1);
  const int32_t orow = (int32_t)threadIdx.x / kHistRowSlots;
  uint64_t xv[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int32_t cb = orow + i * (kHistThreads / kHistRowSlots);
    uint64_t x = 0ull;
    if (oc < nf && cb < R) {
#pragma unroll
      for (int k = 0; k < NCOPY; ++k) x += lds[cb * kHistRowSlots + k * W + oc];
    }
    xv[i] = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int32_t cb = orow + i * (kHistThreads / kHistRowSlots);
    if (oc < nf && cb < R) lds[oc * RP + ((cb + oc) & (RP - 1))] = xv[i];
  }
  __syncthreads();
  for (int32_t r = threadIdx.x; r < nf * RP; r += kHistThreads) {
    const int32_t j = r >> lrp;
    const int32_t cb = r & (RP - 1);
    const int32_t fn = s_fbins[j];
    if (fn > R && cb == 0) dev_error(&ctrl->err, GBDT_E_SHAPE);
    if (cb >= fn || cb >= R) continue;
    const uint64_t x = lds[j * RP + ((cb + j) & (RP - 1))];
    const int64_t gidx = int64_t(s_fgb[j]) + cb;
    if (td.ntiles == 1) {
      const uint64_t cc = x & mask;
      hist_g[int64_t(v) * total_bins + gidx] = (int64_t)(x - cc) >> bits;
      hist_cnt[int64_t(v) * total_bins + gidx] = (uint32_t)cc;
    } else {
      partial[int64_t(td.slot) * total_bins + gidx] = x;
    }
  }
}

// Sums the packed partials of every multi-tile node.  The planner lists those
// nodes (multi[0] = count; entry m, (node, first tile, end tile, list
// position), at multi + 4 + 4 m); workgroups stride over (node, 64-bin
// chunk) items.  A workgroup owns 64 bins of one node; its 16 waves take the
// node's tiles round-robin (loads batched four deep) and combine through
// LDS.  The sums are exact integers, so any order gives the same bits.  The
// first item's entry is loaded with the count (entries up to list_cap are
// allocated), so the partials are the second round trip.
__global__ void __launch_bounds__(1024) k_hist_reduce(const int32_t* __restrict__ multi,
                                                     int32_t list_cap,
                                                     int32_t max_tiles, int32_t bits,
                                                     int32_t total_bins,
                                                     const uint64_t* __restrict__ partial,
                                                     int64_t* __restrict__ hist_g,
                                                     uint32_t* __restrict__ hist_cnt,
                                                     const int32_t* __restrict__ guard) {
  if (failed(guard)) return;
  __shared__ int64_t sg[16][64];
  __shared__ uint64_t sc[16][64];
  const int4* __restrict__ ent = reinterpret_cast<const int4*>(multi + 4);
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int32_t nbc = (total_bins + 63) / 64;
  const uint64_t mask = (1ull << bits) - 1ull;
  const int32_t m0 = (int32_t)blockIdx.x / nbc;
  int4 e = ent[m0 < list_cap ? m0 : list_cap - 1];
  const int32_t nm = clamp_len(multi, list_cap);
  // work items (multi-tile node m, 64-bin chunk) in a grid-stride loop: a
  // level with no multi-tile node ends after one load per workgroup
  for (int32_t it = blockIdx.x; it < nm * nbc; it += gridDim.x) {
    const int32_t m = it / nbc;
    const int32_t b = (it - m * nbc) * 64 + lane;
    const bool inb = b < total_bins;
    if (m != m0) e = ent[m];
    const int32_t t0 = e.y < 0 ? 0 : e.y;
    int32_t t1 = e.z;
    if (t1 > max_tiles) t1 = max_tiles;  // an over-full plan is already flagged
    int64_t g = 0;
    uint64_t c = 0;
    for (int32_t t = t0 + wid; t < t1; t += 16 * 4) {
      uint64_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int32_t tt = t + 16 * u;
        x[u] = (inb && tt < t1) ? partial[int64_t(tt) * total_bins + b] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t cc = x[u] & mask;
        g += (int64_t)(x[u] - cc) >> bits;
        c += cc;
      }
    }
    sg[wid][lane] = g;
    sc[wid][lane] = c;
    __syncthreads();
    if (wid == 0 && inb) {
      int64_t gg = 0;
      uint64_t ccs = 0;
      for (int w = 0; w < 16; ++w) {
        gg += sg[w][lane];
        ccs += sc[w][lane];
      }
      const int32_t v = e.x < 0 ? 0 : e.x;
      hist_g[int64_t(v) * total_bins + b] = gg;
      hist_cnt[int64_t(v) * total_bins + b] = (uint32_t)ccs;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ subtraction --
__global__ void __launch_bounds__(256) k_subtract(int64_t* __restrict__ hist_g,
                                                  uint32_t* __restrict__ hist_cnt,
                                                  int32_t total_bins,
                                                  const gbdt_pair* __restrict__ pairs,
                                                  const int32_t* __restrict__ n_pairs,
                                                  int32_t pair_cap, WsCtrl* __restrict__ ctrl) {
  const int32_t n = clamp_len(n_pairs, pair_cap);
  const int32_t j = blockIdx.y;
  if (j >= n) return;
  const gbdt_pair pr = pairs[j];
  const int64_t P = int64_t(pr.parent) * total_bins, Sm = int64_t(pr.smaller) * total_bins,
                Lg = int64_t(pr.larger) * total_bins;
  bool bad = false;
  for (int32_t b = blockIdx.x * blockDim.x + threadIdx.x; b < total_bins;
       b += gridDim.x * blockDim.x) {
    const uint32_t cp = hist_cnt[P + b], cs = hist_cnt[Sm + b];
    bad |= cs > cp;
    hist_cnt[Lg + b] = cp - cs;
    hist_g[Lg + b] = hist_g[P + b] - hist_g[Sm + b];
  }
  if (bad) dev_error(&ctrl->err, GBDT_E_INTERNAL);
}

// ------------------------------------------------------------- split find --
struct FindParams {
  double lambda, gamma, mcw;
  int32_t msl;
};

__device__ __forceinline__ double score_of(double G, double H, double lambda) {
  const double num = G * G;
  const double den = H + lambda;
  return num / den;
}


// DPP lane move of a 32-bit value; lanes whose source is outside the row (or
// whose row is masked off) read 0, the identity of both combines below.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int32_t dpp_i32(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int64_t dpp_i64(int64_t v) {
  return (int64_t)dpp_u64<CTRL, ROW_MASK>((uint64_t)v);
}
// A 64-bit value of lane l (wave-uniform l).
__device__ __forceinline__ int64_t read_lane_i64(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// One step of the inclusive segmented scan: the running value of the lane
// CTRL moves in from (earlier lanes) is added unless this lane's run already
// holds a segment head.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void seg_scan_step(int32_t& fl, int64_t& g, int32_t& c) {
  const int32_t fu = dpp_i32<CTRL, ROW_MASK>(fl);
  const int64_t gu = dpp_i64<CTRL, ROW_MASK>(g);
  const int32_t cu = dpp_i32<CTRL, ROW_MASK>(c);
  if (!fl) {
    g += gu;
    c += cu;
    fl = fu;
  }
}

// The same step with the logistic objective's Hessian sums as a third value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void seg_scan_step(int32_t& fl, int64_t& g, int32_t& c, int64_t& h) {
  const int32_t fu = dpp_i32<CTRL, ROW_MASK>(fl);
  const int64_t gu = dpp_i64<CTRL, ROW_MASK>(g);
  const int32_t cu = dpp_i32<CTRL, ROW_MASK>(c);
  const int64_t hu = dpp_i64<CTRL, ROW_MASK>(h);
  if (!fl) {
    g += gu;
    c += cu;
    h += hu;
    fl = fu;
  }
}

// Candidate order: larger gain, then larger key (key = INT32_MAX - global
// bin, so the smaller feature and then the smaller threshold win).  The
// empty candidate is (0.0, 0): all zero bits.  Gains compared here are only
// ever positive, so IEEE equality is bit equality.
__device__ __forceinline__ bool better(double g1, int32_t k1, double g2, int32_t k2) {
  return g1 > g2 || (g1 == g2 && k1 > k2);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(double& g, int32_t& key) {
  const double og = __longlong_as_double(dpp_i64<CTRL, ROW_MASK>(__double_as_longlong(g)));
  const int32_t ok = dpp_i32<CTRL, ROW_MASK>(key);
  if (better(og, ok, g, key)) {
    g = og;
    key = ok;
  }
}

// One workgroup of THREADS per node.  The node's histogram is read in passes
// of THREADS * E bins in global bin order (feature-major, bins ascending);
// thread t holds E consecutive bins in registers.  A
// segmented prefix sum (segments = features) -- serial inside the thread,
// a DPP scan of the per-thread tails across the wave, the waves' tails
// through LDS, and a carry across passes -- gives every bin's left totals
// (G_L, n_L); each candidate's gain is evaluated exactly as the formula is
// written, and the workgroup keeps the largest gain, ties to the smaller
// global bin.  The loads that do not depend on the node id are issued with
// the list loads; the thread that owns the winning bin writes the split.
// With sub_par / sub_sib (the tree driver), a node whose entry names a parent
// is the larger child of a split pair: its histogram is the parent's minus
// its built sibling's (exact integers), computed here and written to its own
// slot for the next level; a negative count sets GBDT_E_INTERNAL.
// HESS (the logistic objective): H of a bin range is its sum of fixed-point
// Hessians (hist_h, grid *scale_h) instead of its row count; the scan
// carries it as a third value, the larger sibling's Hessian histogram is
// derived like its G, and split_h[v] gets the winner's left Hessian sum.
template <int THREADS, int E, bool HESS>
__global__ void __launch_bounds__(THREADS) k_find(
    int64_t* __restrict__ hist_g, uint32_t* __restrict__ hist_cnt,
    const int32_t* __restrict__ bin_offset, const int32_t* __restrict__ bin_feature,
    const int32_t* __restrict__ n_bins, int32_t total_bins, const gbdt_node* __restrict__ nodes,
    const int32_t* __restrict__ list, const int32_t* __restrict__ list_len, int32_t list_cap,
    FindParams fp, const int32_t* __restrict__ scale, gbdt_split* __restrict__ splits,
    const int32_t* __restrict__ sub_par, const int32_t* __restrict__ sub_sib,
    int32_t* __restrict__ err, int32_t n_chunks, FindCand* __restrict__ cand,
    const int32_t* __restrict__ guard, int64_t* __restrict__ hist_h,
    const int32_t* __restrict__ scale_h, int64_t* __restrict__ split_h) {
  constexpr int NW = THREADS / 64;
  if (failed(guard)) return;
  __shared__ int64_t sw_g[NW];
  __shared__ int32_t sw_c[NW];
  __shared__ int32_t sw_f[NW];
  __shared__ int64_t sw_h[HESS ? NW : 1];
  __shared__ int64_t s_carry_g;
  __shared__ int32_t s_carry_c;
  __shared__ int64_t s_carry_h;
  __shared__ double r_gain[NW];
  __shared__ int32_t r_key[NW];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int32_t j = blockIdx.x;  // < list_cap (the grid)
  const int32_t chunk = blockIdx.y;
  const int32_t raw_len = *list_len;
  const int32_t v = list[j];
  const int32_t S = *scale;
  const int32_t par = sub_par != nullptr ? sub_par[j] : -1;
  const int32_t sib = sub_par != nullptr ? sub_sib[j] : -1;
  // this workgroup's bins [blo, bhi): all of them, or with n_chunks > 1 the
  // features whose first bin lies in [chunk * kFindChunk, + kFindChunk)
  int32_t blo = 0, bhi = total_bins;
  if (n_chunks > 1) {
    const int32_t nlo = chunk * kFindChunk;
    const int32_t nhi = nlo + kFindChunk < total_bins ? nlo + kFindChunk : total_bins;
    const int32_t fa = bin_feature[nlo < total_bins ? nlo : total_bins - 1];
    const int32_t fz = bin_feature[nhi - 1];
    const int32_t oa = bin_offset[fa];
    const int32_t ff = oa < nlo ? fa + 1 : fa;  // the chunk's first feature
    blo = ff <= fz ? bin_offset[ff] : 0;
    bhi = ff <= fz ? bin_offset[fz + 1] : 0;
    if (nlo >= total_bins) blo = bhi = 0;
  }
  int32_t f[E + 2];  // features of bins b0-1 .. b0+E of the first pass
  {
    const int32_t b0 = blo + threadIdx.x * E;
#pragma unroll
    for (int e = 0; e < E + 2; ++e) {
      const int32_t b = b0 - 1 + e;
      const bool inb = b >= blo && b < bhi;
      const int32_t fv = bin_feature[inb ? b : 0];
      f[e] = inb ? fv : -1 - e;
    }
  }
  asm volatile("" ::: "memory");
  const int32_t n = raw_len < 0 ? 0 : (raw_len > list_cap ? list_cap : raw_len);
  if (j >= n) return;
  const gbdt_node nd = nodes[v];
  int64_t* __restrict__ hg = hist_g + int64_t(v) * total_bins;
  uint32_t* __restrict__ hc = hist_cnt + int64_t(v) * total_bins;
  const bool derive = par >= 0;
  const int64_t* __restrict__ hg_p = hist_g + int64_t(derive ? par : v) * total_bins;
  const uint32_t* __restrict__ hc_p = hist_cnt + int64_t(derive ? par : v) * total_bins;
  const int64_t* __restrict__ hg_s = hist_g + int64_t(derive ? sib : v) * total_bins;
  const uint32_t* __restrict__ hc_s = hist_cnt + int64_t(derive ? sib : v) * total_bins;
  // the Hessian histograms (HESS only)
  int64_t* __restrict__ hh = HESS ? hist_h + int64_t(v) * total_bins : nullptr;
  const int64_t* __restrict__ hh_p = HESS ? hist_h + int64_t(derive ? par : v) * total_bins : nullptr;
  const int64_t* __restrict__ hh_s = HESS ? hist_h + int64_t(derive ? sib : v) * total_bins : nullptr;
  const int32_t Sh = HESS ? *scale_h : 0;
  bool bad = false;

  double best_gain = 0.0;
  int32_t best_key = 0;
  int32_t best_thr = -1, best_f = -1, best_nl = 0;
  int64_t best_gl = 0, best_hl = 0;
  if (threadIdx.x == 0) {
    s_carry_g = 0;
    s_carry_c = 0;
    s_carry_h = 0;
  }
  for (int32_t pass = blo; pass < bhi; pass += THREADS * E) {
    const int32_t b0 = pass + threadIdx.x * E;
    if (pass > blo) {
#pragma unroll
      for (int e = 0; e < E + 2; ++e) {
        const int32_t b = b0 - 1 + e;
        const bool inb = b >= blo && b < bhi;
        const int32_t fv = bin_feature[inb ? b : 0];
        f[e] = inb ? fv : -1 - e;
      }
    }
    int64_t g[E];
    int32_t c[E];
    int64_t h[E];
    int32_t fo[E];  // first global bin of the feature of bin b0 + e
    if (derive) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int32_t b = b0 + e;
        const bool inb = b < bhi;
        const uint32_t cp = inb ? hc_p[b] : 0u, cs = inb ? hc_s[b] : 0u;
        g[e] = inb ? hg_p[b] - hg_s[b] : 0;
        c[e] = (int32_t)(cp - cs);
        bad |= cs > cp;
        if constexpr (HESS) {
          h[e] = inb ? hh_p[b] - hh_s[b] : 0;
          bad |= h[e] < 0;
        }
        fo[e] = bin_offset[inb ? f[e + 1] : 0];
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int32_t b = b0 + e;
        const bool inb = b < bhi;
        g[e] = inb ? hg[b] : 0;
        c[e] = inb ? (int32_t)hc[b] : 0;
        if constexpr (HESS) h[e] = inb ? hh[b] : 0;
        fo[e] = bin_offset[inb ? f[e + 1] : 0];
      }
    }
    const double Gv = ldexp((double)nd.gsum, -S);
    const double Hv = HESS ? ldexp((double)nd.hsum, -Sh) : (double)nd.count;
    const double sP = score_of(Gv, Hv, fp.lambda);
    const int64_t nv = nd.count;
    // serial segmented scan inside the thread
    int32_t first_head = E;
    int64_t rg = 0, rh = 0;
    int32_t rc = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool head = (b0 + e >= bhi) || (f[e] != f[e + 1]);
      if (head && first_head == E) first_head = e;
      rg = head ? g[e] : rg + g[e];
      rc = head ? c[e] : rc + c[e];
      g[e] = rg;
      c[e] = rc;
      if constexpr (HESS) {
        rh = head ? h[e] : rh + h[e];
        h[e] = rh;
      }
    }
    // segmented scan of the thread tails across the wave (DPP row shifts,
    // then rows 0 -> 1, 2 -> 3, row 1 -> rows 2 and 3)
    int32_t fl = first_head < E ? 1 : 0;
    int64_t wg = rg, wh = rh;
    int32_t wc = rc;
    if constexpr (HESS) {
      seg_scan_step<0x111, 0xF>(fl, wg, wc, wh);
      seg_scan_step<0x112, 0xF>(fl, wg, wc, wh);
      seg_scan_step<0x114, 0xF>(fl, wg, wc, wh);
      seg_scan_step<0x118, 0xF>(fl, wg, wc, wh);
      seg_scan_step<0x142, 0xA>(fl, wg, wc, wh);
      seg_scan_step<0x143, 0xC>(fl, wg, wc, wh);
    } else {
      seg_scan_step<0x111, 0xF>(fl, wg, wc);  // row_shr:1
      seg_scan_step<0x112, 0xF>(fl, wg, wc);  // row_shr:2
      seg_scan_step<0x114, 0xF>(fl, wg, wc);  // row_shr:4
      seg_scan_step<0x118, 0xF>(fl, wg, wc);  // row_shr:8
      seg_scan_step<0x142, 0xA>(fl, wg, wc);  // row_bcast:15
      seg_scan_step<0x143, 0xC>(fl, wg, wc);  // row_bcast:31
    }
    if (lane == 63) {
      sw_g[wid] = wg;
      sw_c[wid] = wc;
      sw_f[wid] = fl;
      if constexpr (HESS) sw_h[wid] = wh;
    }
    __syncthreads();
    // the open segment entering this wave: a segmented scan of the wave
    // tails across lanes 0..NW-1 (row 0, DPP row shifts), read at lane
    // wid - 1 -- the pass's carry when no wave before this one holds a
    // segment head -- with no serial walk over the waves
    int64_t cgw, chw = 0;
    int32_t ccw;
    {
      const bool in = lane < NW;
      int32_t tf = in ? sw_f[lane] : 0;
      int64_t tg = in ? sw_g[lane] : 0;
      int32_t tc = in ? sw_c[lane] : 0;
      int64_t th = (HESS && in) ? sw_h[HESS ? lane : 0] : 0;
      if constexpr (HESS) {
        seg_scan_step<0x111, 0xF>(tf, tg, tc, th);
        seg_scan_step<0x112, 0xF>(tf, tg, tc, th);
        seg_scan_step<0x114, 0xF>(tf, tg, tc, th);
        seg_scan_step<0x118, 0xF>(tf, tg, tc, th);
      } else {
        seg_scan_step<0x111, 0xF>(tf, tg, tc);
        seg_scan_step<0x112, 0xF>(tf, tg, tc);
        seg_scan_step<0x114, 0xF>(tf, tg, tc);
        seg_scan_step<0x118, 0xF>(tf, tg, tc);
      }
      const int wv = __builtin_amdgcn_readfirstlane(wid);
      cgw = s_carry_g;
      ccw = s_carry_c;
      if constexpr (HESS) chw = s_carry_h;
      if (wv > 0) {
        const int32_t f = __builtin_amdgcn_readlane(tf, wv - 1);
        const int64_t g = read_lane_i64(tg, wv - 1);
        const int32_t cc = __builtin_amdgcn_readlane(tc, wv - 1);
        cgw = f ? g : cgw + g;
        ccw = f ? cc : ccw + cc;
        if constexpr (HESS) {
          const int64_t hh = read_lane_i64(th, wv - 1);
          chw = f ? hh : chw + hh;
        }
      }
    }
    const int64_t incl_g = fl ? wg : cgw + wg;  // open segment at this thread's end
    const int32_t incl_c = fl ? wc : ccw + wc;
    const int64_t incl_h = fl ? wh : chw + wh;
    // the open segment entering this thread: the previous lane's, or the
    // wave's carry in lane 0 (wave_shr:1 gives lane 0 a zero)
    int64_t cin_g = dpp_i64<0x138, 0xF>(incl_g);
    int32_t cin_c = dpp_i32<0x138, 0xF>(incl_c);
    int64_t cin_h = HESS ? dpp_i64<0x138, 0xF>(incl_h) : 0;
    if (lane == 0) {
      cin_g = cgw;
      cin_c = ccw;
      cin_h = chw;
    }
    __syncthreads();
    if (threadIdx.x == THREADS - 1) {
      s_carry_g = incl_g;
      s_carry_c = incl_c;
      if constexpr (HESS) s_carry_h = incl_h;
    }
    // candidates: bin b with its right neighbour in the same feature
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int32_t b = b0 + e;
      if (b >= bhi) break;
      const int64_t gl = e < first_head ? g[e] + cin_g : g[e];
      const int32_t nlc = e < first_head ? c[e] + cin_c : c[e];
      const int64_t hl = HESS ? (e < first_head ? h[e] + cin_h : h[e]) : 0;
      if (f[e + 2] != f[e + 1]) continue;
      const int64_t nl = nlc;
      const int64_t nr = nv - nl;
      const double GL = ldexp((double)gl, -S);
      const double HL = HESS ? ldexp((double)hl, -Sh) : (double)nl;
      const double GR = Gv - GL;
      const double HR = Hv - HL;
      if (nl >= fp.msl && nr >= fp.msl && HL >= fp.mcw && HR >= fp.mcw && HL > 0.0 && HR > 0.0) {
        const double sL = score_of(GL, HL, fp.lambda);
        const double sR = score_of(GR, HR, fp.lambda);
        const double sum = sL + sR;
        const double diff = sum - sP;
        const double half = 0.5 * diff;
        const double gain = half - fp.gamma;
        const int32_t key = 0x7fffffff - b;
        if (gain > 0.0 && better(gain, key, best_gain, best_key)) {
          best_gain = gain;
          best_key = key;
          best_gl = gl;
          best_hl = hl;
          best_nl = nlc;
          best_f = f[e + 1];
          best_thr = b - fo[e];
        }
      }
    }
    if (derive) {
      // the derived histogram, for the next level: each bin's value is its
      // in-thread running sum minus the previous bin's (or itself at a head).
      // Stored last, so no wait above covers these writes.
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int32_t b = b0 + e;
        if (b < bhi) {
          const bool head = e == 0 || f[e] != f[e + 1];
          hg[b] = head ? g[e] : g[e] - g[e - 1 < 0 ? 0 : e - 1];
          hc[b] = (uint32_t)(head ? c[e] : c[e] - c[e - 1 < 0 ? 0 : e - 1]);
          if constexpr (HESS) hh[b] = head ? h[e] : h[e] - h[e - 1 < 0 ? 0 : e - 1];
        }
      }
    }
    __syncthreads();
  }
  if (bad) dev_error(err, GBDT_E_INTERNAL);
  // argmax over the wave (DPP), then over the waves
  double wg_gain = best_gain;
  int32_t wg_key = best_key;
  argmax_step<0xB1, 0xF>(wg_gain, wg_key);   // quad_perm [1,0,3,2]
  argmax_step<0x4E, 0xF>(wg_gain, wg_key);   // quad_perm [2,3,0,1]
  argmax_step<0x141, 0xF>(wg_gain, wg_key);  // row_half_mirror
  argmax_step<0x140, 0xF>(wg_gain, wg_key);  // row_mirror
  argmax_step<0x142, 0xA>(wg_gain, wg_key);  // row_bcast:15
  argmax_step<0x143, 0xC>(wg_gain, wg_key);  // row_bcast:31
  if (lane == 63) {
    r_gain[wid] = wg_gain;
    r_key[wid] = wg_key;
  }
  __syncthreads();
  // the waves' best in lanes 0..NW-1 (empty candidates beyond), reduced
  // within row 0 by DPP; every lane of the row then holds the best
  double top_gain = lane < NW ? r_gain[lane] : 0.0;
  int32_t top_key = lane < NW ? r_key[lane] : 0;
  argmax_step<0xB1, 0xF>(top_gain, top_key);   // quad_perm [1,0,3,2]
  argmax_step<0x4E, 0xF>(top_gain, top_key);   // quad_perm [2,3,0,1]
  argmax_step<0x141, 0xF>(top_gain, top_key);  // row_half_mirror
  argmax_step<0x140, 0xF>(top_gain, top_key);  // row_mirror
  top_gain = __longlong_as_double(read_lane_i64(__double_as_longlong(top_gain), 0));
  top_key = __builtin_amdgcn_readlane(top_key, 0);
  if (n_chunks > 1) {
    // this chunk's best candidate for the merge (key 0: none)
    FindCand* __restrict__ c = cand + int64_t(j) * n_chunks + chunk;
    if (top_key != 0 && top_gain > 0.0) {
      if (best_key == top_key) {
        FindCand x;
        x.gain = best_gain;
        x.key = best_key;
        x.feature = best_f;
        x.threshold_bin = best_thr;
        x.n_left = best_nl;
        x.g_left = best_gl;
        x.h_left = best_hl;
        *c = x;
      }
    } else if (threadIdx.x == 0) {
      FindCand x;
      x.gain = 0.0;
      x.key = 0;
      x.feature = -1;
      x.threshold_bin = -1;
      x.n_left = 0;
      x.g_left = 0;
      x.h_left = 0;
      *c = x;
    }
    return;
  }
  if (top_key != 0 && top_gain > 0.0) {
    // the owner of the winning bin (each bin has one owner) writes the split
    if (best_key == top_key) {
      gbdt_split sp;
      sp.gain = best_gain;
      sp.feature = best_f;
      sp.threshold_bin = best_thr;
      sp.g_left = best_gl;
      sp.n_left = best_nl;
      sp.valid = 1;
      splits[v] = sp;
      if constexpr (HESS) split_h[v] = best_hl;
    }
  } else if (threadIdx.x == 0) {
    gbdt_split sp;
    sp.gain = 0.0;
    sp.feature = -1;
    sp.threshold_bin = -1;
    sp.g_left = 0;
    sp.n_left = 0;
    sp.valid = 0;
    splits[v] = sp;
    if constexpr (HESS) split_h[v] = 0;
  }
}

// Merge of the chunked split search: one wave per listed node takes the best
// of its chunks' candidates (larger gain, then the larger key: the smaller
// global bin; keys are unique across chunks) and writes the split, or an
// invalid split when no chunk has one.
__global__ void __launch_bounds__(64) k_find_merge(const int32_t* __restrict__ list,
                                                   const int32_t* __restrict__ list_len,
                                                   int32_t list_cap, int32_t n_chunks,
                                                   const FindCand* __restrict__ cand,
                                                   gbdt_split* __restrict__ splits,
                                                   const int32_t* __restrict__ guard,
                                                   int64_t* __restrict__ split_h) {
  if (failed(guard)) return;
  const int32_t j = blockIdx.x;
  const int32_t raw = *list_len;
  const int32_t n = raw < 0 ? 0 : (raw > list_cap ? list_cap : raw);
  if (j >= n) return;
  const int32_t v = list[j];
  const int lane = threadIdx.x;
  double bg = 0.0;
  int32_t bk = 0, bc = -1;
  for (int32_t c = lane; c < n_chunks; c += 64) {
    const FindCand x = cand[int64_t(j) * n_chunks + c];
    if (x.key != 0 && better(x.gain, x.key, bg, bk)) {
      bg = x.gain;
      bk = x.key;
      bc = c;
    }
  }
  double wg = bg;
  int32_t wk = bk;
  argmax_step<0xB1, 0xF>(wg, wk);
  argmax_step<0x4E, 0xF>(wg, wk);
  argmax_step<0x141, 0xF>(wg, wk);
  argmax_step<0x140, 0xF>(wg, wk);
  argmax_step<0x142, 0xA>(wg, wk);
  argmax_step<0x143, 0xC>(wg, wk);
  const int32_t top_k = __builtin_amdgcn_readlane(wk, 63);  // the wave's best key (row_bcast:31 ends in lane 63)
  if (top_k != 0) {
    if (bk == top_k && bc >= 0) {
      const FindCand x = cand[int64_t(j) * n_chunks + bc];
      gbdt_split sp;
      sp.gain = x.gain;
      sp.feature = x.feature;
      sp.threshold_bin = x.threshold_bin;
      sp.g_left = x.g_left;
      sp.n_left = x.n_left;
      sp.valid = 1;
      splits[v] = sp;
      if (split_h != nullptr) split_h[v] = x.h_left;
    }
  } else if (lane == 0) {
    gbdt_split sp;
    sp.gain = 0.0;
    sp.feature = -1;
    sp.threshold_bin = -1;
    sp.g_left = 0;
    sp.n_left = 0;
    sp.valid = 0;
    splits[v] = sp;
  }
}

// -------------------------------------------------------------- partition --
// Stable partition in one pass with a decoupled look-back across the tiles
// of a node.  The tile is the workgroup's id and a tile waits only on
// lower-numbered tiles.  Each XCD dispatches its share of a grid's
// workgroups in increasing id order, so the lowest unfinished tile is
// always resident (every earlier workgroup on its XCD has finished) and
// never waits: the chain drains without an atomic tile counter at the start
// of each tile's critical path.  Each status word packs a 2-bit state
// (1 = tile count available, 2 = inclusive prefix available) with a 32-bit
// value; the wait is bounded and reports GBDT_E_INTERNAL if it runs out.
constexpr uint64_t kStAgg = 1ull << 62;
constexpr uint64_t kStInc = 2ull << 62;
constexpr uint64_t kStMask = 3ull << 62;

__device__ __forceinline__ void st_publish(uint64_t* p, uint64_t word) {
  __hip_atomic_store(p, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t st_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kPartThreads = 1024;
constexpr int kPartWaves = kPartThreads / 64;

// Wave 0 of the workgroup: exclusive count of left rows over the tiles of the
// node before `tile`, 64 predecessors per step.  Tiles before the node's first
// tile count as an inclusive prefix of 0, so the walk stops there.
__device__ int64_t lookback_excl(uint64_t* status, int32_t tile, int32_t tfirst, bool* ok) {
  const int lane = threadIdx.x & 63;
  int64_t excl = 0;
  int32_t idx = tile - 1;
  uint32_t spins = 0;
  while (true) {
    const int32_t p = idx - lane;
    const uint64_t w = p >= tfirst ? st_load(&status[p]) : kStInc;
    const uint64_t st = w & kStMask;
    const uint64_t inc = __ballot(st == kStInc);
    const uint64_t zero = __ballot(st == 0ull);
    const int first_inc = inc ? (__ffsll((unsigned long long)inc) - 1) : 64;
    const uint64_t need = first_inc >= 63 ? ~0ull : ((2ull << first_inc) - 1ull);
    if (zero & need) {
      if (++spins > (1u << 20)) {
        *ok = false;
        return excl;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    const int64_t val = ((need >> lane) & 1ull) ? (int64_t)(uint32_t)(w & 0xffffffffull) : 0;
    excl += wave_sum(val);
    if (first_inc < 64) return excl;
    idx -= 64;
  }
}

// The same over status words that carry two counts, bits 0-30 and 31-61
// (two-level partitions): their exclusive sums in *lo and *hi.
__device__ void lookback_excl2(uint64_t* status, int32_t tile, int32_t tfirst, int64_t* lo,
                               int64_t* hi, bool* ok) {
  const int lane = threadIdx.x & 63;
  int64_t e0 = 0, e1 = 0;
  int32_t idx = tile - 1;
  uint32_t spins = 0;
  while (true) {
    const int32_t p = idx - lane;
    const uint64_t w = p >= tfirst ? st_load(&status[p]) : kStInc;
    const uint64_t st = w & kStMask;
    const uint64_t inc = __ballot(st == kStInc);
    const uint64_t zero = __ballot(st == 0ull);
    const int first_inc = inc ? (__ffsll((unsigned long long)inc) - 1) : 64;
    const uint64_t need = first_inc >= 63 ? ~0ull : ((2ull << first_inc) - 1ull);
    if (zero & need) {
      if (++spins > (1u << 20)) {
        *ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    // both counts in one 64-bit sum, bits 0-31 and 32-63: a step adds at
    // most one inclusive prefix (< 2^31) and 63 tile counts (< 2^13 each),
    // so the low half never carries into the high one
    const uint64_t v = ((need >> lane) & 1ull)
                           ? ((w & 0x7fffffffull) | (((w >> 31) & 0x7fffffffull) << 32))
                           : 0ull;
    const uint64_t sum = wave_sum(v);
    e0 += (int64_t)(sum & 0xffffffffull);
    e1 += (int64_t)(sum >> 32);
    if (first_inc < 64) break;
    idx -= 64;
  }
  *lo = e0;
  *hi = e1;
}

// Where a partition tile reads each row's value of a split feature (matrix
// column c): from dword dw of the rows' first moved block, held in registers,
// when the feature is a byte column of that block (dw >= 0); otherwise from
// the dword at base + row * stride.  The value is (dword >> sh) & mask.
struct SplitVal {
  const uint8_t* base;
  uint32_t stride, sh, mask;
  int32_t dw;
};
__device__ __forceinline__ SplitVal split_val(int32_t c, int32_t b0, bool rows_in_regs,
                                              const uint8_t* sbins, int64_t row_capacity,
                                              int32_t n_blocks, int32_t block_features,
                                              int32_t block_stride, int32_t n_features, int32_t n_bit,
                                              int32_t bit_stride, int32_t n_nib, int32_t nib_stride) {
  SplitVal v;
  const int32_t nbc = n_features - n_bit;
  const int32_t nbyte = nbc - n_nib;
  const uint8_t* bits = sbins + int64_t(n_blocks) * row_capacity * block_stride;
  v.dw = -1;
  if (c >= nbc) {
    const int32_t k = c - nbc;
    v.base = bits + 4 * (k >> 5);
    v.stride = (uint32_t)bit_stride;
    v.sh = (uint32_t)(k & 31);
    v.mask = 1u;
  } else if (c >= nbyte) {
    const int32_t k = c - nbyte;
    v.base = bits + row_capacity * bit_stride + 4 * (k >> 3);
    v.stride = (uint32_t)nib_stride;
    v.sh = 4u * (uint32_t)(k & 7);
    v.mask = 15u;
  } else {
    const int32_t b = c / block_features;
    const int32_t j = c - b * block_features;
    v.base = sbins + int64_t(b) * row_capacity * block_stride + (j & ~3);
    v.stride = (uint32_t)block_stride;
    v.sh = 8u * (uint32_t)(j & 3);
    v.mask = 0xffu;
    if (rows_in_regs && b == b0) v.dw = j >> 2;
  }
  return v;
}

// ND dwords of one row (4-byte aligned) as wide loads and stores: the first
// min(ND, 4) dwords in `a`, the rest in `b` (two register quads, so each
// load writes its own aligned registers).
template <int ND>
struct RowData {
  static_assert(ND >= 1 && ND <= 8, "row of 1..8 dwords");
  uint4 a, b;
};
template <int N>
__device__ __forceinline__ uint4 load_dwords(const uint8_t* p) {
  if constexpr (N == 4) return *reinterpret_cast<const uint4*>(p);
  if constexpr (N == 3) { const uint3 v = *reinterpret_cast<const uint3*>(p); return make_uint4(v.x, v.y, v.z, 0u); }
  if constexpr (N == 2) { const uint2 v = *reinterpret_cast<const uint2*>(p); return make_uint4(v.x, v.y, 0u, 0u); }
  if constexpr (N == 1) return make_uint4(*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u);
  return make_uint4(0u, 0u, 0u, 0u);
}
template <int N>
__device__ __forceinline__ void store_dwords(uint8_t* p, const uint4& v) {
  if constexpr (N == 4) *reinterpret_cast<uint4*>(p) = v;
  if constexpr (N == 3) *reinterpret_cast<uint3*>(p) = make_uint3(v.x, v.y, v.z);
  if constexpr (N == 2) *reinterpret_cast<uint2*>(p) = make_uint2(v.x, v.y);
  if constexpr (N == 1) *reinterpret_cast<uint32_t*>(p) = v.x;
}
// Dword i (uniform, < ND) of a row held in registers.
template <int ND>
__device__ __forceinline__ uint32_t row_dword(const RowData<ND> d, uint32_t i) {
  uint32_t v = d.a.x;
  if (ND > 1) v = i == 1 ? d.a.y : v;
  if (ND > 2) v = i == 2 ? d.a.z : v;
  if (ND > 3) v = i == 3 ? d.a.w : v;
  if (ND > 4) v = i == 4 ? d.b.x : v;
  if (ND > 5) v = i == 5 ? d.b.y : v;
  if (ND > 6) v = i == 6 ? d.b.z : v;
  if (ND > 7) v = i == 7 ? d.b.w : v;
  return v;
}
template <int ND>
__device__ __forceinline__ void row_load(const uint8_t* p, RowData<ND>& d) {
  d.a = load_dwords<(ND < 4 ? ND : 4)>(p);
  if constexpr (ND > 4) d.b = load_dwords<ND - 4>(p + 16);
}
template <int ND>
__device__ __forceinline__ void row_store(uint8_t* p, const RowData<ND>& d) {
  store_dwords<(ND < 4 ? ND : 4)>(p, d.a);
  if constexpr (ND > 4) store_dwords<ND - 4>(p + 16, d.b);
}
// One workgroup per tile of K * kPartThreads rows of a splitting node (tile
// = workgroup id).  Thread t owns rows t + k kPartThreads of the tile and
// moves each whole row itself: the row's bytes of a column block (ND dwords)
// with one or two wide loads and stores, its q and row id, so a wave's
// accesses cover 64 consecutive source rows and two runs of destinations
// (left and right).  The tile descriptor carries the node's split, so right
// after it arrives the workgroup issues every load that does not depend on
// the destinations: q, row ids and, for every row of the thread, the first
// moved block -- the one holding the split feature, whose byte is then taken
// from the registers, so no line of the tile is fetched twice (a narrow
// split feature adds one dword load per row for its bit or nibble).  Then it
// ballots the go-left flags, publishes its left count, looks back for the
// exclusive prefix (decoupled look-back) and stores; the other blocks and
// the narrow blocks are loaded and stored row by row after that.  IDS
// (index mode): the positions hold row ids of the matrix instead of rows; a
// tile moves each position's id and q, with the split byte read from the
// matrix at the id.
//
// FOUR (two-level partition): the tiles cover the segment of a grandparent
// g, whose rows are in g's level order; each row goes through g's split to
// child a (left) or b (right) and through that child's split (when it has
// one) to a's or b's left or right child, and the four classes are written
// stably to the grandchildren's segments [a1 | a2 | b1 | b2] of g's segment
// -- the order two successive stable partitions would leave ("Module
// Design: Training Core", section 6, step 5, applied at two levels at once).
// Each class's rank comes from the tile's per-(row k, wave) counts and two
// decoupled look-backs run side by side: wave 0 over (a1, a2) in status,
// wave 1 over (b1, b2) in status2.
template <int ND, int K, bool Q32OUT, bool NIB, bool IDS = false, bool FOUR = false>
__global__ void GBDT_SGPR_CAP __launch_bounds__(kPartThreads) k_partition(
    const uint8_t* __restrict__ sbins, const void* __restrict__ sq,
    const int32_t* __restrict__ srid, uint8_t* __restrict__ dbins, void* __restrict__ dq,
    int32_t* __restrict__ drid, int64_t row_capacity, int32_t n_blocks, int32_t block_features,
    int32_t block_stride, int32_t n_features, int32_t n_bit, int32_t bit_stride,
    const TileDesc* __restrict__ desc, uint64_t* __restrict__ status, WsCtrl* __restrict__ ctrl,
    int32_t qsh /* log2 of the source q's element size: 2 (int32) or 3 (int64) */,
    int32_t n_nib, int32_t nib_stride, const uint8_t* __restrict__ scols,
    uint64_t* __restrict__ status2) {
  static_assert(K == 2 || K == 4 || (K == 8 && IDS), "rows per thread");
  static_assert(!IDS || !NIB, "index mode moves no narrow block");
  static_assert(!(IDS && FOUR), "two-level partitions move rows");
  constexpr int TILE = K * kPartThreads;
  constexpr int NCNT = K * kPartWaves;  // per-(row k, wave) left counts
  // an int32 destination q is the low half of the source element
  using QT = typename std::conditional<Q32OUT, int32_t, int64_t>::type;
  // (FOUR: two arrays of packed class counts, (a1 | a2 << 16) and (b1 | b2 << 16))
  __shared__ int32_t s_cnt[FOUR ? 2 * NCNT : NCNT];
  __shared__ int32_t s_excl;
  __shared__ int32_t s_excl4[4];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int32_t tile = (int32_t)blockIdx.x;
  const int32_t total = ctrl->plan_total;
  if (tile >= total) return;
  const TileDesc td = desc[tile];
  const int32_t tfirst = td.tfirst;
  const int32_t tlast = td.tfirst + td.ntiles - 1;
  const int32_t tin = tile - tfirst;
  const int64_t r0 = td.r0;
  const int64_t span = int64_t(td.r1) - td.r0;
  const int32_t rows_all = (int32_t)(span < 0 ? 0 : (span > TILE ? TILE : span));
  // a listed node must carry a valid split; otherwise nothing is moved, the
  // tile still publishes (so later tiles never wait on it) and the error word
  // is set.  The descriptor's feature is the split's matrix column: a byte
  // column (c < nbyte = n_features - n_nib - n_bit), a nibble (c - nbyte) of
  // the nibble block or a bit (c - (n_features - n_bit)) of the bit block.
  bool split_ok = td.split_valid && td.feature >= 0 && td.feature < n_features;
  // FOUR: the children's splits (thresholds, whether each splits) and counts
  const int32_t n_a = td.n_left;
  const int32_t n_b = td.count - td.n_left;
  const bool has2 = FOUR && td.split2 >= 0;
  const bool has3 = FOUR && td.split3 >= 0;
  const int32_t c2 = has2 ? (td.split2 >> 8) : 0, thr2 = has2 ? (td.split2 & 0xff) : 0;
  const int32_t c3 = has3 ? (td.split3 >> 8) : 0, thr3 = has3 ? (td.split3 & 0xff) : 0;
  if constexpr (FOUR) {
    split_ok = split_ok && c2 < n_features && c3 < n_features && n_a >= 0 && n_b >= 0 &&
               td.n2 >= 0 && td.n2 <= n_a && td.n3 >= 0 && td.n3 <= n_b;
  }
  int32_t rows = split_ok ? rows_all : 0;
  const int32_t nbc = n_features - n_bit;  // the first bit column
  const int32_t nbyte = nbc - n_nib;
  const int32_t sc = split_ok ? td.feature : 0;
  const bool fbit = sc >= nbc;
  const bool fnib = NIB && !fbit && sc >= nbyte;
  const bool fnarrow = fbit || fnib;
  const int32_t fblk = fnarrow ? 0 : sc / block_features;
  const int32_t fcol = fnarrow ? 0 : sc % block_features;
  const int32_t fk = fbit ? sc - nbc : (fnib ? sc - nbyte : 0);
  const int32_t nwords = bit_stride >> 2;
  const uint8_t* __restrict__ fcolp = sbins + int64_t(fblk) * row_capacity * block_stride + fcol;
  const uint8_t* __restrict__ sbits = sbins + int64_t(n_blocks) * row_capacity * block_stride;
  const uint8_t* __restrict__ snibs = sbits + row_capacity * bit_stride;
  // the split feature's word in a narrow block (bit k: word k >> 5; nibble k: word k >> 3)
  const uint32_t* __restrict__ fwordp =
      fbit ? reinterpret_cast<const uint32_t*>(sbits) + (fk >> 5)
           : reinterpret_cast<const uint32_t*>(snibs) + (fk >> 3);
  // loads that need only the descriptor, unconditional (a row past the tile
  // end rereads its last row and is ignored), so none waits behind a branch
  int32_t fb[K];
  QT qv[K];
  RowData<ND> rd[K];  // the first moved block of each row of the thread
  // Addresses are a uniform base at the tile's first row plus a 32-bit lane
  // offset (a tile spans at most 8192 rows of at most 512 bytes).
  // block 0 here means the first block moved: the split feature's own block
  // (any block for a narrow split feature), so its byte always comes from
  // the rows' registers; the other blocks follow in order
  const int32_t b0 = fnarrow ? 0 : fblk;
  const int64_t b0off = int64_t(b0) * row_capacity * block_stride;
  const uint8_t* __restrict__ tb = sbins + b0off + r0 * block_stride;
  const uint32_t bs = (uint32_t)block_stride;
  // With every row's first block (the split feature's) loaded early, the
  // split byte comes from those registers: a separate load of the split
  // bytes would bring each line of the tile in twice when the cache has
  // evicted it before the rows are read.  (uniform)
  const bool from_rows = !IDS && !fnarrow && n_blocks > 0;
  // IDS (index mode): position r0 + i holds row id srid[r0 + i] (the position
  // itself when srid is NULL) of the matrix sbins; only ids and q move, and
  // the split byte is read at the row id (clamped into the matrix), from the
  // column-major copy scols (column c's byte of row r at c row_capacity + r)
  // when there is one: a node's rows, in ascending id order, then share a
  // cache line per 128 consecutive ids instead of per 128 / block_stride
  const bool from_cols = IDS && scols != nullptr;  // (uniform)
  int32_t rids[K];
  // FOUR: each row's values of the children's split features (x2: a's, x3:
  // b's).  The 4096-row tiles (K = 4) take them from the rows' registers
  // only: the planner gives two-level plans those tiles only for layouts of
  // one byte block (the registers of separate loads would cost the kernel
  // its second workgroup per CU); a child split outside the registers' block
  // is then an error and the tile moves nothing.
  constexpr bool CHILD_LOADS = FOUR && K < 4;
  SplitVal sv2{}, sv3{};
  uint32_t x2[CHILD_LOADS ? K : 1], x3[CHILD_LOADS ? K : 1];
  if constexpr (FOUR) {
    const bool regs = n_blocks > 0;  // the rows' first moved block is held in registers
    sv2 = split_val(c2, b0, regs, sbins, row_capacity, n_blocks, block_features, block_stride,
                    n_features, n_bit, bit_stride, n_nib, nib_stride);
    sv3 = split_val(c3, b0, regs, sbins, row_capacity, n_blocks, block_features, block_stride,
                    n_features, n_bit, bit_stride, n_nib, nib_stride);
#pragma unroll
    for (int k = 0; k < (CHILD_LOADS ? K : 1); ++k) x2[k] = x3[k] = 0u;
    if (!CHILD_LOADS && ((has2 && sv2.dw < 0) || (has3 && sv3.dw < 0))) {
      split_ok = false;
      rows = 0;
    }
  }
  if (rows > 0) {
    const char* __restrict__ tq = reinterpret_cast<const char*>(sq) + (r0 << qsh);
    const uint32_t lr = (uint32_t)(rows - 1);
    // otherwise one dword load per row (the byte's aligned dword, or the
    // bit's word), issued first: loads complete in order, so the flags wait
    // only for these while the rows are still in flight
    const uint32_t frow = fbit ? (uint32_t)nwords * 4u : (fnib ? (uint32_t)nib_stride : bs);
    if constexpr (IDS) {
      const uint8_t* __restrict__ tf = fcolp - (fcol & 3);
      const int64_t last = row_capacity > 0 ? row_capacity - 1 : 0;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t i = (uint32_t)(k * kPartThreads) + threadIdx.x;
        const uint32_t ic = i < lr ? i : lr;
        rids[k] = srid != nullptr ? srid[r0 + ic] : (int32_t)(r0 + ic);
      }
      const uint8_t* __restrict__ tcol = from_cols ? scols + int64_t(sc) * row_capacity : nullptr;
      bool bad_id = false;  // (an id outside the matrix is clamped into it and reported)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        bad_id |= rids[k] < 0 || rids[k] > last;
        const int64_t id = rids[k] < 0 ? 0 : (rids[k] > last ? last : rids[k]);
        fb[k] = from_cols ? (int32_t)tcol[id]
                          : (int32_t)*reinterpret_cast<const uint32_t*>(tf + id * int64_t(frow));
      }
      if (bad_id) dev_error(&ctrl->err, GBDT_E_INTERNAL);
    } else if (!from_rows) {
      const uint8_t* __restrict__ tf =
          (fnarrow ? reinterpret_cast<const uint8_t*>(fwordp) : fcolp - (fcol & 3)) + r0 * int64_t(frow);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t i = (uint32_t)(k * kPartThreads) + threadIdx.x;
        const uint32_t ic = i < lr ? i : lr;
        fb[k] = (int32_t)*reinterpret_cast<const uint32_t*>(tf + ic * frow);
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint32_t i = (uint32_t)(k * kPartThreads) + threadIdx.x;
      const uint32_t ic = i < lr ? i : lr;
      // an int32 destination reads the low half of the source element
      // (int32 or int64: the driver narrows only q that fit); an int64 one
      // comes from an int64 source
      qv[k] = *reinterpret_cast<const QT*>(tq + (ic << qsh));
      // with no byte block (ND == 1, block_stride 0) this rereads the first
      // dword of the bit block, and the value is never stored
      if constexpr (!IDS) row_load<ND>(tb + ic * bs, rd[k]);
    }
    if constexpr (CHILD_LOADS) {
      // (loaded with the rows; a feature of the registers' block needs none)
      const uint8_t* __restrict__ t2 = sv2.base + r0 * int64_t(sv2.stride);
      const uint8_t* __restrict__ t3 = sv3.base + r0 * int64_t(sv3.stride);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t i = (uint32_t)(k * kPartThreads) + threadIdx.x;
        const uint32_t ic = i < lr ? i : lr;
        if (has2 && sv2.dw < 0) x2[k] = *reinterpret_cast<const uint32_t*>(t2 + ic * sv2.stride);
        if (has3 && sv3.dw < 0) x3[k] = *reinterpret_cast<const uint32_t*>(t3 + ic * sv3.stride);
      }
    }
    if (from_rows) {
      const uint32_t fdw = (uint32_t)fcol >> 2;
      const uint32_t fsh = 8u * (uint32_t)(fcol & 3);
#pragma unroll
      for (int k = 0; k < K; ++k) fb[k] = (int32_t)((row_dword<ND>(rd[k], fdw) >> fsh) & 0xffu);
    } else {
      const uint32_t fsh = from_cols ? 0u
                           : fbit ? (uint32_t)(fk & 31)
                                  : (fnib ? 4u * (uint32_t)(fk & 7) : 8u * (uint32_t)(fcol & 3));
      const uint32_t fmask = fbit ? 1u : (fnib ? 15u : 0xffu);
#pragma unroll
      for (int k = 0; k < K; ++k) fb[k] = (int32_t)(((uint32_t)fb[k] >> fsh) & fmask);
    }
  }
  if (!split_ok && threadIdx.x == 0) dev_error(&ctrl->err, GBDT_E_INTERNAL);

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t seg_end = int64_t(td.begin) + td.count;
  bool bad_pos = false;
  int32_t dpos[K];
  // Wave w's exclusive scan of count array cnt (the (row k, wave) counts in
  // row order, in place); returns the tile's total.
  auto scan_counts = [&](int32_t* cnt) -> int32_t {
    constexpr int E = NCNT >= 64 ? NCNT / 64 : 1;  // counts per lane
    int32_t c[E];
    int32_t own = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = lane * E + e;
      c[e] = idx < NCNT ? cnt[idx] : 0;
      own += c[e];
    }
    const int32_t x = wave_incl_scan(own);
    int32_t run = x - own;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int idx = lane * E + e;
      if (idx < NCNT) cnt[idx] = run;
      run += c[e];
    }
    return __builtin_amdgcn_readlane(x, 63);
  };
  if constexpr (!FOUR) {
    uint64_t bal[K];  // go-left flags of the wave's rows k (a row's own flag is its bit)
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int32_t i = k * kPartThreads + threadIdx.x;
      bal[k] = __ballot((i < rows) && (fb[k] <= td.threshold_bin));
      if (lane == 0) s_cnt[k * kPartWaves + wid] = __popcll(bal[k]);
    }
    __syncthreads();
    // wave 0: exclusive scan of the (row k, wave) counts in row order, then
    // publish the tile's left count at once (so later tiles never wait long),
    // look back for the exclusive prefix of the node's earlier tiles and
    // publish the inclusive one
    if (wid == 0) {
      const int32_t acc = scan_counts(s_cnt);
      if (lane == 0) st_publish(&status[tile], (tin == 0 ? kStInc : kStAgg) | (uint64_t)(uint32_t)acc);
      int64_t excl = 0;
      bool ok = true;
      if (tin > 0) excl = lookback_excl(status, tile, tfirst, &ok);
      if (lane == 0) {
        if (!ok) dev_error(&ctrl->err, GBDT_E_INTERNAL);
        if (tin > 0) st_publish(&status[tile], kStInc | (uint64_t)(uint32_t)(excl + acc));
        s_excl = (int32_t)excl;
        if (tile == tlast && excl + acc != td.n_left) dev_error(&ctrl->err, GBDT_E_INTERNAL);
      }
    }
    __syncthreads();
    const int32_t excl = s_excl;
    const int64_t lbase = int64_t(td.begin) + excl;
    const int64_t rbase = int64_t(td.begin) + td.n_left + (int64_t(tin) * TILE - excl);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int32_t i = k * kPartThreads + threadIdx.x;
      dpos[k] = -1;
      if (i < rows) {
        const int32_t rl = s_cnt[k * kPartWaves + wid] + __popcll(bal[k] & lt_mask);
        const bool left = (bal[k] >> lane) & 1ull;
        const int64_t d = left ? lbase + rl : rbase + (i - rl);
        // a split record whose left count disagrees with the rows could send a
        // row outside its node's segment: such a row is not written
        const bool in_seg = d >= td.begin && d < seg_end;
        bad_pos |= !in_seg;
        dpos[k] = in_seg ? (int32_t)d : -1;
      }
    }
  } else {
    // class of each row: 0 a1, 1 a2, 2 b1, 3 b2 (a child without a split
    // keeps all its rows in its first class), two bits per row k in one
    // register, and the (row k, wave) counts of every class; the ballots
    // are taken again for the ranks after the look-back (the registers of
    // per-row ranks would cost the kernel its second workgroup per CU)
    uint32_t cls = 0u;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int32_t i = k * kPartThreads + threadIdx.x;
      const bool valid = i < rows;
      // (the children's split values: from the rows' registers or their loads)
      const uint32_t w2 = sv2.dw >= 0 ? row_dword<ND>(rd[k], (uint32_t)sv2.dw) : x2[CHILD_LOADS ? k : 0];
      const uint32_t w3 = sv3.dw >= 0 ? row_dword<ND>(rd[k], (uint32_t)sv3.dw) : x3[CHILD_LOADS ? k : 0];
      const int32_t v2 = (int32_t)((w2 >> sv2.sh) & sv2.mask);
      const int32_t v3 = (int32_t)((w3 >> sv3.sh) & sv3.mask);
      const bool ga = fb[k] <= td.threshold_bin;
      const bool l2 = ga ? (!has2 || v2 <= thr2) : (!has3 || v3 <= thr3);
      const uint32_t c = (ga ? 0u : 2u) | (l2 ? 0u : 1u);
      cls |= c << (2 * k);
      asm volatile("" : "+v"(cls));
      const uint64_t m0 = __ballot(valid && c == 0u);
      const uint64_t m1 = __ballot(valid && c == 1u);
      const uint64_t m2 = __ballot(valid && c == 2u);
      const uint64_t m3 = __ballot(valid && c == 3u);
      if (lane == 0) {
        s_cnt[k * kPartWaves + wid] = __popcll(m0) | (__popcll(m1) << 16);
        s_cnt[NCNT + k * kPartWaves + wid] = __popcll(m2) | (__popcll(m3) << 16);
      }
    }
    // (the empty asm keeps the classes computed here: sunk past the barrier,
    // they would keep every row's split values live instead)
    asm volatile("" : "+v"(cls));
    __syncthreads();
    // wave 0 scans, publishes and looks back over (a1, a2) in status, wave 1
    // over (b1, b2) in status2; each checks its child's totals at the last tile
    if (wid < 2) {
      const int32_t acc = scan_counts(s_cnt + wid * NCNT);
      const int64_t lo = acc & 0xffff, hi = acc >> 16;
      uint64_t* __restrict__ st = wid == 0 ? status : status2;
      if (lane == 0)
        st_publish(&st[tile], (tin == 0 ? kStInc : kStAgg) | ((uint64_t)hi << 31) | (uint64_t)lo);
      int64_t e0 = 0, e1 = 0;
      bool ok = true;
      if (tin > 0) lookback_excl2(st, tile, tfirst, &e0, &e1, &ok);
      if (lane == 0) {
        if (!ok) dev_error(&ctrl->err, GBDT_E_INTERNAL);
        if (tin > 0) st_publish(&st[tile], kStInc | ((uint64_t)(e1 + hi) << 31) | (uint64_t)(e0 + lo));
        s_excl4[2 * wid] = (int32_t)e0;
        s_excl4[2 * wid + 1] = (int32_t)e1;
        if (tile == tlast) {
          const int64_t want0 = wid == 0 ? td.n2 : td.n3;
          const int64_t want1 = wid == 0 ? n_a - td.n2 : n_b - td.n3;
          if (e0 + lo != want0 || e1 + hi != want1) dev_error(&ctrl->err, GBDT_E_INTERNAL);
        }
      }
    }
    __syncthreads();
    // the grandchildren's segments: a1 at begin, a2 after a1, b1 at begin + n_a, b2 after b1
    const int64_t B0 = int64_t(td.begin) + s_excl4[0];
    const int64_t B1 = int64_t(td.begin) + td.n2 + s_excl4[1];
    const int64_t B2 = int64_t(td.begin) + n_a + s_excl4[2];
    const int64_t B3 = int64_t(td.begin) + n_a + td.n3 + s_excl4[3];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int32_t i = k * kPartThreads + threadIdx.x;
      const bool valid = i < rows;
      const int32_t c = (int32_t)((cls >> (2 * k)) & 3u);
      const uint64_t m0 = __ballot(valid && c == 0);
      const uint64_t m1 = __ballot(valid && c == 1);
      const uint64_t m2 = __ballot(valid && c == 2);
      const uint64_t m3 = __ballot(valid && c == 3);
      dpos[k] = -1;
      if (valid) {
        const uint64_t mine = c == 0 ? m0 : (c == 1 ? m1 : (c == 2 ? m2 : m3));
        const int32_t pk = s_cnt[(c >> 1) * NCNT + k * kPartWaves + wid];
        const int32_t off = (c & 1) ? (pk >> 16) : (pk & 0xffff);
        const int64_t base = c == 0 ? B0 : (c == 1 ? B1 : (c == 2 ? B2 : B3));
        const int64_t d = base + off + __popcll(mine & lt_mask);
        const bool in_seg = d >= td.begin && d < seg_end;
        bad_pos |= !in_seg;
        dpos[k] = in_seg ? (int32_t)d : -1;
      }
    }
  }
  if (bad_pos) dev_error(&ctrl->err, GBDT_E_INTERNAL);
  // q of every row, then the first moved block
#pragma unroll
  for (int k = 0; k < K; ++k)
    if (dpos[k] >= 0) reinterpret_cast<QT*>(dq)[dpos[k]] = qv[k];
  // row ids (moved only when the destination has them)
  if (drid != nullptr) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t sr = r0 + k * kPartThreads + threadIdx.x;
      if (dpos[k] >= 0) drid[dpos[k]] = IDS ? rids[k] : (srid != nullptr ? srid[sr] : (int32_t)sr);
    }
  }
  if constexpr (IDS) return;
  if (n_blocks > 0) {
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (dpos[k] >= 0) row_store<ND>(dbins + b0off + int64_t(dpos[k]) * block_stride, rd[k]);
  }
  // the other byte blocks, double-buffered: block b + 1 is loaded before
  // block b is stored (loads are unconditional, from clamped rows).  Tiles
  // of more than two rows per thread are used only with one block (the
  // registers of two buffers would not fit); the plain loop covers them.
  // (j-th block after the first: block j - 1 below b0, block j above it)
  auto other_block = [&](int32_t j) { return j <= b0 ? j - 1 : j; };
  if constexpr (K > 2) {
    for (int32_t j = 1; j < n_blocks; ++j) {
      const int64_t boff = int64_t(other_block(j)) * row_capacity * block_stride;
      const uint8_t* __restrict__ tbb = sbins + boff + r0 * block_stride;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t i = (uint32_t)(k * kPartThreads) + threadIdx.x;
        int32_t d = dpos[k];
        asm volatile("" : "+v"(d));  // (no destination address hoisted out of the block loop)
        if (d >= 0) {
          RowData<ND> x;
          row_load<ND>(tbb + i * bs, x);
          row_store<ND>(dbins + boff + int64_t(d) * block_stride, x);
        }
      }
    }
  } else if (n_blocks > 1) {
    RowData<ND> nx[K];
    auto load_block = [&](int32_t j, RowData<ND>* dst) {
      const uint8_t* __restrict__ src = sbins + int64_t(other_block(j)) * row_capacity * block_stride;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int32_t i = k * kPartThreads + threadIdx.x;
        row_load<ND>(src + (r0 + (i < rows ? i : rows - 1)) * block_stride, dst[k]);
      }
    };
    auto store_block = [&](int32_t j, const RowData<ND>* src) {
      uint8_t* __restrict__ dstp = dbins + int64_t(other_block(j)) * row_capacity * block_stride;
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (dpos[k] >= 0) row_store<ND>(dstp + int64_t(dpos[k]) * block_stride, src[k]);
    };
    if (rows > 0) load_block(1, nx);
    int32_t b = 1;
    while (b < n_blocks) {
      if (b + 1 < n_blocks && rows > 0) load_block(b + 1, rd);
      store_block(b, nx);
      if (++b >= n_blocks) break;
      if (b + 1 < n_blocks && rows > 0) load_block(b + 1, nx);
      store_block(b, rd);
      ++b;
    }
  }
  // the narrow blocks (bit words, then nibble words): nw words per row, 4 at
  // a time, rows in groups of at most 4 per thread
  auto move_words = [&](const uint8_t* __restrict__ sblk, uint8_t* __restrict__ dblk, int32_t nw) {
    constexpr int GB = K < 4 ? K : 4;
    const uint32_t rowb = (uint32_t)nw * 4u;
    const uint8_t* __restrict__ tw = sblk + r0 * int64_t(rowb);
    uint8_t* __restrict__ dw = dblk;
    int32_t w0 = 0;
    for (; w0 + 4 <= nw; w0 += 4) {
#pragma unroll
      for (int kb = 0; kb < K; kb += GB) {
        RowData<4> x[GB];
#pragma unroll
        for (int e = 0; e < GB; ++e) {
          const uint32_t i = (uint32_t)((kb + e) * kPartThreads) + threadIdx.x;
          if (dpos[kb + e] >= 0) row_load<4>(tw + (i * rowb + 4u * (uint32_t)w0), x[e]);
        }
#pragma unroll
        for (int e = 0; e < GB; ++e) {
          // (the empty asm keeps the 64-bit destination addresses from being
          // hoisted out of the word loop, where all K would stay live)
          int32_t d = dpos[kb + e];
          asm volatile("" : "+v"(d));
          if (d >= 0) row_store<4>(dw + int64_t(d) * rowb + 4 * w0, x[e]);
        }
      }
    }
    for (; w0 < nw; ++w0) {
      uint32_t x[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const uint32_t i = (uint32_t)(k * kPartThreads) + threadIdx.x;
        if (dpos[k] >= 0) x[k] = *reinterpret_cast<const uint32_t*>(tw + (i * rowb + 4u * (uint32_t)w0));
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        int32_t d = dpos[k];
        asm volatile("" : "+v"(d));
        if (d >= 0) {
          RowData<1> one;
          one.a = make_uint4(x[k], 0u, 0u, 0u);
          row_store<1>(dw + int64_t(d) * rowb + 4 * w0, one);
        }
      }
    }
  };
  uint8_t* __restrict__ dbits = dbins + int64_t(n_blocks) * row_capacity * block_stride;
  if (n_bit > 0) move_words(sbits, dbits, nwords);
  if (NIB && n_nib > 0) move_words(snibs, dbits + row_capacity * bit_stride, nib_stride >> 2);
}

// ------------------------------------------------------ prediction update --
// Forward pass of one tree over the rows of X in their original order, in two
// launches.  k_compact_tree copies the tree into a table of 8 bytes per node
// (left child; where the split feature's bin sits in a row's dwords -- byte
// blocks, then bit words, then nibble words -- and the threshold) plus a
// table of leaf values by node, checking each node.  k_update is persistent
// (a few workgroups per CU): each workgroup first copies the node table into
// LDS (64 KiB for a depth-12 tree), then walks rows in a grid-stride loop,
// ROWS rows per lane at once, each lane holding its rows' bins (every block,
// MAXDW dwords at most) in registers.  The walk is branch-free: every step
// reads each row's node, picks the split feature's dword with a select tree
// over the bits of its index, extracts the bin with one bit-field extract and
// moves the row to a child.  Leaves (and nodes that fail the check) point to
// themselves with a threshold no bin exceeds, so a row that reaches one stays
// there and the step needs no test; the wave stops when none of its rows
// moved.  The node a row ends on is then checked once, and the leaf value
// read from global memory.  HBM traffic is the bins once and the predictions
// read and written once, sequentially in rows -- no gather or scatter through
// row ids.  Trees must be breadth-first with right = left + 1; a node whose
// children are not in (id, n_nodes) stops the walk and sets GBDT_E_INTERNAL
// (the row keeps its prediction).  A tree too large for LDS is walked from
// the global table (TREE_IN_LDS = false).
constexpr int kUpdThreads = 1024;
constexpr int kUpdMaxRowBytes = 256;
constexpr size_t kUpdTreeLds = 64 * 1024;
constexpr uint32_t kLeafThr = 0xffffu;  // the threshold field of a leaf's entry
constexpr uint32_t kBadThr = 0xfffeu;   // ... of a node that fails the check

// One workgroup.  Entry of a split node v: e.x = left child, e.y = dword
// index (6 bits) | shift << 6 (5 bits) | bin width << 11 (5 bits: 8 byte, 4
// nibble, 1 bit) | threshold << 16.  A row's dwords are its byte blocks,
// then, from dword word_base, its bit words and nibble words.  Entry of a leaf: e.x = v, e.y = kLeafThr
// << 16 (width 0: the bin reads as 0, so the row stays), with its value at
// lval[v]; of a failing node: e.x = v, e.y = kBadThr << 16.
__global__ void __launch_bounds__(1024) k_compact_tree(const gbdt_node* __restrict__ nodes,
                                                       const int32_t* __restrict__ n_nodes_dev,
                                                       int32_t max_nodes, int32_t n_features,
                                                       const int32_t* __restrict__ feature_col,
                                                       int32_t n_blocks, int32_t block_features,
                                                       int32_t block_stride, int32_t n_bit,
                                                       uint2* __restrict__ ctab,
                                                       double* __restrict__ lval,
                                                       int32_t* __restrict__ driver_nodes,
                                                       WsCtrl* __restrict__ ctrl, int32_t bit_stride,
                                                       int32_t n_nib, int32_t word_base) {
  __shared__ int32_t s_bad;
  // driver mode (driver_nodes = the tree's node count): a tree whose kernels
  // recorded an error is dropped -- node count 0, so the update that follows
  // changes no prediction
  if (driver_nodes != nullptr && failed(&ctrl->err)) {
    if (threadIdx.x == 0) *driver_nodes = 0;
    return;
  }
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  int32_t nn = *n_nodes_dev;
  if (nn > max_nodes) nn = max_nodes;
  for (int32_t v = threadIdx.x; v < nn; v += blockDim.x) {
    const int4 nd = *reinterpret_cast<const int4*>(&nodes[v]);
    uint2 e = make_uint2((uint32_t)v, kBadThr << 16);  // a failing node, until shown otherwise
    if (nd.z < 0) {
      e.y = kLeafThr << 16;
      lval[v] = nodes[v].leaf_value;
    } else if (nd.z <= v || nd.z + 1 >= nn || nd.w != nd.z + 1 || nd.x < 0 || nd.x >= n_features) {
      // (stays a failing node)
    } else {
      const int32_t c = feature_col != nullptr ? feature_col[nd.x] : nd.x;
      const int32_t nbc = n_features - n_bit;  // the first bit column
      const int32_t nbyte = nbc - n_nib;       // the first nibble column
      uint32_t loc;
      if (c >= 0 && c < nbyte) {
        const int32_t blk = c / block_features;
        const int32_t byte = blk * block_stride + (c - blk * block_features);
        loc = (uint32_t)(byte >> 2) | ((uint32_t)(8 * (byte & 3)) << 6) | (8u << 11);
      } else if (c >= nbyte && c < nbc) {  // a nibble: after the bit words in the row's dwords
        const int32_t kk = c - nbyte;
        loc = (uint32_t)(word_base + (bit_stride >> 2) + (kk >> 3)) | ((uint32_t)(4 * (kk & 7)) << 6) |
              (4u << 11);
      } else {
        const int32_t kk = c - nbc;
        loc = (uint32_t)(word_base + (kk >> 5)) | ((uint32_t)(kk & 31) << 6) | (1u << 11);
      }
      // (a bin threshold at or above kBadThr would read as a leaf or bad
      // node: bins are at most 255)
      if (c >= 0 && c < n_features && nd.y >= 0 && nd.y < (int32_t)kBadThr) {
        e.x = (uint32_t)nd.z;
        e.y = loc | ((uint32_t)nd.y << 16);
      }
    }
    if (e.y == (kBadThr << 16)) s_bad = 1;
    ctab[v] = e;
  }
  // driver mode: a node that fails the check drops the whole tree before any
  // row is updated (outside the driver the walk reports the rows that meet it)
  if (driver_nodes != nullptr) {
    __syncthreads();
    if (threadIdx.x == 0 && s_bad) {
      dev_error(&ctrl->err, GBDT_E_INTERNAL);
      *driver_nodes = 0;
    }
  }
}

// ND1 > 0: byte blocks of ND1 dwords each, every block loaded with one or
// two wide loads (a 16-byte load and one of 4, 8 or 12 bytes), then the bit
// words; ND1 == 0: any layout, one dword per load.  (10M x 100, four blocks
// of 28 bytes: one dword per load moved the rows at 3.6 TB/s.)
template <int MAXDW, int ROWS, bool TREE_IN_LDS, int ND1, bool NIB>
__global__ void GBDT_SGPR_CAP __launch_bounds__(kUpdThreads) k_update(
    double* __restrict__ pred, int64_t n, const uint8_t* __restrict__ bins, int64_t row_capacity,
    int32_t n_blocks, int32_t block_stride, int32_t bit_stride,
    const uint2* __restrict__ ctab_g, const double* __restrict__ lval,
    const int32_t* __restrict__ n_nodes_dev, int32_t max_nodes, double eta,
    WsCtrl* __restrict__ ctrl, int32_t nib_stride) {
  static_assert((MAXDW & (MAXDW - 1)) == 0, "MAXDW is a power of two");
  extern __shared__ uint64_t smem[];
  int32_t nn = *n_nodes_dev;
  if (nn > max_nodes) nn = max_nodes;
  if (nn < 1) {
    if (blockIdx.x == 0 && threadIdx.x == 0) dev_error(&ctrl->err, GBDT_E_INTERNAL);
    return;
  }
  const uint2* ctab = ctab_g;
  if (TREE_IN_LDS) {
    uint2* ct = reinterpret_cast<uint2*>(smem);
    for (int32_t v = threadIdx.x; v < nn; v += kUpdThreads) ct[v] = ctab_g[v];
    __syncthreads();
    ctab = ct;
  }
  const int32_t dw = block_stride >> 2;
  const int32_t ndw = n_blocks * dw;            // byte-block dwords of a row
  const int32_t nwords = bit_stride >> 2;       // then its bit words
  const int32_t nnw = nib_stride >> 2;          // then its nibble words
  const uint32_t* __restrict__ bitw =
      reinterpret_cast<const uint32_t*>(bins + int64_t(n_blocks) * row_capacity * block_stride);
  const uint32_t* __restrict__ nibw = bitw + row_capacity * nwords;
  bool bad = false;
  const int64_t stride = int64_t(gridDim.x) * kUpdThreads * ROWS;
  for (int64_t base = int64_t(blockIdx.x) * kUpdThreads * ROWS + threadIdx.x; base < n;
       base += stride) {
    uint32_t row[ROWS][MAXDW];
    int32_t v[ROWS];
    bool live[ROWS];
    double pv[ROWS];
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
      const int64_t i0 = base + int64_t(u) * kUpdThreads;
      live[u] = i0 < n;
      v[u] = 0;
      const int64_t i = live[u] ? i0 : n - 1;  // a valid row: loads need no branch
      pv[u] = pred[i];
      // dword x of the row: byte block b, dword xb of its run (a uniform
      // walk, no division), then the bit words.  The loads are unconditional
      // (uniform pointer selects), so all of them are in flight together.
      // Dwords past the row's words keep what their load read (the row's
      // first dword): no node refers to them, and zeroing them made the
      // wave wait for every load issued so far, block by block.
      const uint32_t* __restrict__ bp =
          reinterpret_cast<const uint32_t*>(bins + i * block_stride);
      const uint32_t* __restrict__ wp = bitw + i * nwords;
      const uint32_t* __restrict__ np = nibw + i * nnw;
      if constexpr (ND1 > 0) {
        // byte blocks of ND1 dwords each (block_stride = 4 ND1): block b's
        // dwords with one or two wide loads into row dwords b ND1 ..; then
        // the bit and nibble words, one load each, from dword NBM ND1 on
        // (MAXDW 8: one block, NBM 1).  Every load is unconditional (a block
        // past n_blocks, or a word past the row's, rereads the row's first
        // block or dword and is never referred to), so all are in flight
        // together: with a branch per block the wave waited for every load
        // issued so far at each block.
        static_assert(ND1 <= MAXDW, "a byte block fits the row registers");
        constexpr int NBM = MAXDW == 8 ? 1 : MAXDW / ND1;
#pragma unroll
        for (int b = 0; b < NBM; ++b) {
          RowData<ND1> rdat;
          row_load<ND1>(bins + (int64_t(b < n_blocks ? b : 0) * row_capacity + i) * block_stride, rdat);
          const uint32_t w8[8] = {rdat.a.x, rdat.a.y, rdat.a.z, rdat.a.w,
                                  rdat.b.x, rdat.b.y, rdat.b.z, rdat.b.w};
#pragma unroll
          for (int x = 0; x < ND1; ++x) row[u][b * ND1 + x] = w8[x];
        }
#pragma unroll
        for (int x = NBM * ND1; x < MAXDW; ++x) {
          const int32_t k = x - NBM * ND1;
          const bool in_bits = k < nwords;
          const bool in_nibs = NIB && !in_bits && k - nwords < nnw;
          row[u][x] = *(in_bits ? wp + k : (in_nibs ? np + (k - nwords) : bp));
        }
      } else {
        int32_t xb = 0;
        int64_t boff = 0;  // dwords from bins to block b's run
#pragma unroll
        for (int x = 0; x < MAXDW; ++x) {
          const bool in_bytes = x < ndw;
          const bool in_bits = !in_bytes && x < ndw + nwords;
          const bool in_nibs = NIB && !in_bytes && !in_bits && x < ndw + nwords + nnw;
          const uint32_t* p = in_bytes ? bp + boff + xb
                                       : (in_bits ? wp + (x - ndw) : (in_nibs ? np + (x - ndw - nwords) : bp));
          row[u][x] = *p;
          if (in_bytes && ++xb == dw) {
            xb = 0;
            boff += (row_capacity * block_stride) >> 2;
          }
        }
      }
    }
    // the walk: branch-free steps until no row of the wave moves (a row on a
    // leaf or a failing node stays there)
    for (int step = 0; step <= GBDT_MAX_DEPTH; ++step) {
      bool walking = false;
#pragma unroll
      for (int u = 0; u < ROWS; ++u) {
        const uint2 e = ctab[v[u]];
        // the split feature's dword: a select tree over the bits of its index
        const uint32_t kk = e.y;
        uint32_t t[MAXDW];
#pragma unroll
        for (int x = 0; x < MAXDW; ++x) t[x] = row[u][x];
#pragma unroll
        for (int lvl = 0, w = MAXDW; w > 1; ++lvl, w >>= 1) {
          const bool hi = (kk >> lvl) & 1u;
#pragma unroll
          for (int x = 0; x < w / 2; ++x) t[x] = hi ? t[2 * x + 1] : t[2 * x];
        }
        // the bin: width (e.y >> 11) & 31 bits at shift (e.y >> 6) & 31
        const uint32_t bv = __builtin_amdgcn_ubfe(t[0], (e.y >> 6) & 31u, (e.y >> 11) & 31u);
        const int32_t next = (int32_t)e.x + (bv <= (e.y >> 16) ? 0 : 1);
        walking |= next != v[u];
        v[u] = next;
      }
      if (!__any(walking)) break;
    }
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
      if (!live[u]) continue;
      // a leaf, or a failing node / no leaf within the depth bound
      if ((ctab[v[u]].y >> 16) != kLeafThr) {
        bad = true;
        continue;
      }
      const int64_t i = base + int64_t(u) * kUpdThreads;
      const double delta = eta * lval[v[u]];
      pred[i] = pv[u] + delta;
    }
  }
  if (bad) dev_error(&ctrl->err, GBDT_E_INTERNAL);
}

template <int MAXDW, int ND1 = 0, bool NIB = false>
static void launch_update(bool in_lds, int rows, dim3 grid, size_t lds, hipStream_t s, double* pred,
                          int64_t n, const gbdt_matrix* X, const uint2* ctab, const double* lval,
                          const int32_t* n_nodes, int32_t max_nodes, double eta, WsCtrl* ctrl) {
  // two rows per lane only where both rows' bins fit registers without scratch
  constexpr int R2 = MAXDW <= 16 ? 2 : 1;
  auto kern = in_lds ? (rows == 2 ? k_update<MAXDW, R2, true, ND1, NIB> : k_update<MAXDW, 1, true, ND1, NIB>)
                     : (rows == 2 ? k_update<MAXDW, R2, false, ND1, NIB> : k_update<MAXDW, 1, false, ND1, NIB>);
  hipLaunchKernelGGL(kern, grid, dim3(kUpdThreads), lds, s, pred, n, X->bins, X->row_capacity,
                     X->n_blocks, X->block_stride, X->bit_stride, ctab, lval, n_nodes, max_nodes, eta,
                     ctrl, X->nib_stride);
}

// ------------------------------------------------------- setup: packing --
// One thread per row: byte columns into their blocks (feature of column c =
// col_feature[c], identity when NULL), bit features into the bit words.
__global__ void __launch_bounds__(256) k_pack(const uint8_t* __restrict__ src, int64_t n,
                                              int32_t F, uint8_t* __restrict__ dst,
                                              int64_t row_capacity, int32_t n_blocks,
                                              int32_t block_features, int32_t block_stride,
                                              int32_t n_bit, int32_t bit_stride,
                                              const int32_t* __restrict__ col_feature,
                                              const int32_t* __restrict__ n_bins,
                                              WsCtrl* __restrict__ ctrl, int32_t n_nib,
                                              int32_t nib_stride) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t nbc = F - n_bit - n_nib;
  bool bad = false;
  for (int32_t b = 0; b < n_blocks; ++b) {
    uint8_t* d = dst + int64_t(b) * row_capacity * block_stride + i * block_stride;
    for (int32_t jj = 0; jj < block_stride; ++jj) {
      const int32_t c = b * block_features + jj;
      uint8_t x = 0;
      if (jj < block_features && c < nbc) {
        int32_t f = col_feature != nullptr ? col_feature[c] : c;
        f = f < 0 ? 0 : (f >= F ? F - 1 : f);
        x = src[i * F + f];
        bad |= (int32_t)x >= n_bins[f];
      }
      d[jj] = x;
    }
  }
  if (n_bit > 0) {
    uint32_t* wd = reinterpret_cast<uint32_t*>(dst + int64_t(n_blocks) * row_capacity * block_stride +
                                               i * bit_stride);
    for (int32_t w = 0; w < (bit_stride >> 2); ++w) {
      uint32_t word = 0u;
      for (int32_t t = 0; t < 32; ++t) {
        const int32_t kk = 32 * w + t;
        if (kk >= n_bit) break;
        int32_t f = col_feature[F - n_bit + kk];  // bit k is column F - n_bit + k
        f = f < 0 ? 0 : (f >= F ? F - 1 : f);
        const uint8_t x = src[i * F + f];
        bad |= (int32_t)x >= n_bins[f] || x > 1;
        word |= uint32_t(x & 1) << t;
      }
      wd[w] = word;
    }
  }
  if (n_nib > 0) {
    uint32_t* wd = reinterpret_cast<uint32_t*>(dst + int64_t(n_blocks) * row_capacity * block_stride +
                                               row_capacity * bit_stride + i * nib_stride);
    for (int32_t w = 0; w < (nib_stride >> 2); ++w) {
      uint32_t word = 0u;
      for (int32_t t = 0; t < 8; ++t) {
        const int32_t kk = 8 * w + t;
        if (kk >= n_nib) break;
        int32_t f = col_feature[nbc + kk];
        f = f < 0 ? 0 : (f >= F ? F - 1 : f);
        const uint8_t x = src[i * F + f];
        bad |= (int32_t)x >= n_bins[f] || x > 15;
        word |= uint32_t(x & 15) << (4 * t);
      }
      wd[w] = word;
    }
  }
  if (bad) dev_error(&ctrl->err, GBDT_E_RANGE);
}

// bin census for the skip-bin choice: counts[f][bin] over all rows
__global__ void __launch_bounds__(256) k_census(const uint8_t* __restrict__ src, int64_t n,
                                                int32_t F, uint32_t* __restrict__ counts) {
  __shared__ uint32_t c[64 * 256];
  const int32_t fg = blockIdx.y * 64;
  const int32_t nf = (F - fg) < 64 ? (F - fg) : 64;
  for (int t = threadIdx.x; t < 64 * 256; t += blockDim.x) c[t] = 0u;
  __syncthreads();
  const int64_t rows_per_block = (n + gridDim.x - 1) / gridDim.x;
  const int64_t a = int64_t(blockIdx.x) * rows_per_block;
  int64_t e = a + rows_per_block;
  if (e > n) e = n;
  for (int64_t x = a * nf + threadIdx.x; x < e * nf; x += blockDim.x) {
    const int64_t i = x / nf;
    const int32_t f = (int32_t)(x - i * nf);
    atomicAdd(&c[f * 256 + src[i * F + fg + f]], 1u);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nf * 256; t += blockDim.x)
    if (c[t]) atomicAdd(&counts[int64_t(fg) * 256 + t], c[t]);
}

__global__ void __launch_bounds__(64) k_pick_skip(const uint32_t* __restrict__ counts, int32_t F,
                                                  const int32_t* __restrict__ n_bins,
                                                  int32_t* __restrict__ skip_bin) {
  const int32_t f = blockIdx.x;
  if (f >= F || threadIdx.x != 0) return;
  uint32_t best = 0u;
  int32_t bi = -1;
  for (int32_t c = 0; c < n_bins[f]; ++c) {
    const uint32_t x = counts[int64_t(f) * 256 + c];
    if (x > best) {
      best = x;
      bi = c;
    }
  }
  skip_bin[f] = bi;
}

// The byte blocks of a block-major matrix interleaved row by row (index
// mode's gather copy): dword d of row r's block b goes to dword
// r pd + b nd + d (pd dwords per row, the padding after the blocks zero), for
// every row below row_capacity.  One thread per destination dword, so the
// stores are coalesced and each source read covers a row's block.
__global__ void __launch_bounds__(256) k_interleave(const uint32_t* __restrict__ src,
                                                    uint32_t* __restrict__ dst, int64_t row_capacity,
                                                    int32_t n_blocks, int32_t nd, int32_t pd) {
  const int64_t total = row_capacity * pd;
  for (int64_t o = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; o < total;
       o += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = o / pd;
    const int32_t e = (int32_t)(o - r * pd);
    const int32_t b = e / nd;
    dst[o] = b < n_blocks ? src[(int64_t(b) * row_capacity + r) * nd + (e - b * nd)] : 0u;
  }
}

// The byte columns of a block-major matrix one after another (index mode's
// split-byte copy): column c = b block_features + j of row r goes to byte
// c row_capacity + r.  One thread per destination byte (coalesced stores).
__global__ void __launch_bounds__(256) k_columns(const uint8_t* __restrict__ src,
                                                 uint8_t* __restrict__ dst, int64_t row_capacity,
                                                 int32_t n_cols, int32_t block_features,
                                                 int32_t block_stride) {
  const int64_t total = row_capacity * n_cols;
  for (int64_t o = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; o < total;
       o += int64_t(gridDim.x) * blockDim.x) {
    const int32_t c = (int32_t)(o / row_capacity);
    const int64_t r = o - int64_t(c) * row_capacity;
    const int32_t b = c / block_features;
    dst[o] = src[(int64_t(b) * row_capacity + r) * block_stride + (c - b * block_features)];
  }
}

__global__ void k_zero_u32(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// ------------------------------------------------------------ host checks --

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static int check_ws(void* ws, size_t ws_bytes, const WsLayout& L) {
  if (ws == nullptr || !aligned(ws, 256)) return fail(GBDT_E_ARG, "workspace is null or not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(GBDT_E_ARG, "workspace too small: need " + std::to_string(L.total) + " bytes, got " +
                                std::to_string(ws_bytes));
  return GBDT_OK;
}

int check_matrix(const gbdt_matrix& X) {
  if (X.bins == nullptr) return fail(GBDT_E_ARG, "matrix bins pointer is null");
  if (X.n_rows < 0 || X.n_rows > 0x7fffffffLL) return fail(GBDT_E_ARG, "n_rows out of range");
  if (X.row_capacity < X.n_rows) return fail(GBDT_E_SHAPE, "row_capacity < n_rows");
  if (X.n_features < 1 || X.n_features > GBDT_MAX_FEATURES) return fail(GBDT_E_ARG, "n_features out of range");
  if (X.n_bit_features < 0 || X.n_bit_features > X.n_features)
    return fail(GBDT_E_ARG, "n_bit_features out of range");
  if ((X.col_feature == nullptr) != (X.feature_col == nullptr))
    return fail(GBDT_E_ARG, "col_feature and feature_col must both be set or both be NULL");
  if (X.n_nib_features < 0 || X.n_nib_features > X.n_features - X.n_bit_features)
    return fail(GBDT_E_ARG, "n_nib_features out of range");
  if (X.col_feature == nullptr && (X.n_bit_features != 0 || X.n_nib_features != 0))
    return fail(GBDT_E_ARG, "bit and nibble blocks need the column maps");
  if (X.n_nib_features > 0 &&
      (X.nib_stride < 4 * ((X.n_nib_features + 7) / 8) || (X.nib_stride & 3) || X.nib_stride > 4 * kMaxBitWords))
    return fail(GBDT_E_ARG, "bad nib_stride");
  if (X.n_nib_features == 0 && X.nib_stride != 0) return fail(GBDT_E_ARG, "nib_stride without nibble features");
  const int32_t nbc = X.n_features - X.n_bit_features - X.n_nib_features;
  if (nbc > 0) {
    if (X.block_features < 1 || X.block_stride < X.block_features || (X.block_stride & 3) ||
        X.block_stride > 1024)
      return fail(GBDT_E_ARG, "bad block_features / block_stride");
    if (int64_t(X.n_blocks) * X.block_features < nbc || int64_t(X.n_blocks - 1) * X.block_features >= nbc)
      return fail(GBDT_E_SHAPE, "n_blocks does not match the byte columns / block_features");
  } else if (X.n_blocks != 0) {
    return fail(GBDT_E_SHAPE, "n_blocks must be 0 when every feature is a bit");
  }
  if (X.n_bit_features > 0 &&
      (X.bit_stride < 4 * ((X.n_bit_features + 31) / 32) || (X.bit_stride & 3) ||
       X.bit_stride > 4 * kMaxBitWords))
    return fail(GBDT_E_ARG, "bad bit_stride");
  if (!aligned(X.bins, 4)) return fail(GBDT_E_ARG, "bins not 4-byte aligned");
  return GBDT_OK;
}

static int check_features(const gbdt_features& ft, int32_t n_features) {
  if (ft.n_features != n_features) return fail(GBDT_E_SHAPE, "feature table does not match the matrix");
  if (ft.total_bins < 1 || ft.total_bins > GBDT_MAX_FEATURES * GBDT_MAX_BINS)
    return fail(GBDT_E_ARG, "total_bins out of range");
  if (!ft.n_bins || !ft.bin_offset || !ft.bin_feature) return fail(GBDT_E_ARG, "feature table pointer is null");
  return GBDT_OK;
}


bool same_layout(const gbdt_matrix& a, const gbdt_matrix& b) {
  return a.n_rows == b.n_rows && a.row_capacity == b.row_capacity && a.n_features == b.n_features &&
         a.n_blocks == b.n_blocks && a.block_features == b.block_features &&
         a.block_stride == b.block_stride && a.n_bit_features == b.n_bit_features &&
         a.bit_stride == b.bit_stride && a.col_feature == b.col_feature &&
         a.feature_col == b.feature_col && a.n_nib_features == b.n_nib_features &&
         a.nib_stride == b.nib_stride;
}

int check_hist_inputs(const gbdt_rows& src, const gbdt_features& ft) {
  int rc = check_matrix(src.X);
  if (rc) return rc;
  rc = check_features(ft, src.X.n_features);
  if (rc) return rc;
  if (!src.q) return fail(GBDT_E_ARG, "q is null");
  if (ft.max_block_bins < 1 || ft.max_block_bins > kLdsHistBudgetBins)
    return fail(GBDT_E_UNSUPPORTED, "max_block_bins outside the LDS histogram budget");
  if (src.X.n_features > src.X.n_bit_features + src.X.n_nib_features &&
      (src.X.block_stride > kHistMaxBlockStride || src.X.block_features > kHistRowSlots))
    return fail(GBDT_E_UNSUPPORTED, "a column block wider than 32 bytes");
  if (2 * src.X.n_bit_features > ft.max_block_bins)
    return fail(GBDT_E_SHAPE, "max_block_bins below 2 slots per bit feature");
  if (kNibSlots * src.X.n_nib_features > ft.max_block_bins)
    return fail(GBDT_E_SHAPE, "max_block_bins below 16 slots per nibble feature");
  return GBDT_OK;
}

int check_partition_inputs(const gbdt_rows& src, const gbdt_rows& dst) {
  int rc = check_matrix(src.X);
  if (rc) return rc;
  rc = check_matrix(dst.X);
  if (rc) return rc;
  if (!same_layout(src.X, dst.X)) return fail(GBDT_E_SHAPE, "source and destination layouts differ");
  if (!src.q || !dst.q) return fail(GBDT_E_ARG, "q pointer is null");
  if (src.X.n_blocks > 0 && src.X.block_stride > kHistMaxBlockStride)
    return fail(GBDT_E_UNSUPPORTED, "a column block wider than 32 bytes");
  return GBDT_OK;
}

template <int N, bool Q, bool F>
static auto hist_kernel(int D) -> decltype(&k_hist<8, N, Q>) {
  return D == 8   ? k_hist<8, N, Q, false, F>
         : D == 4 ? k_hist<4, N, Q, false, F>
         : D == 2 ? k_hist<2, N, Q, false, F>
                  : k_hist<1, N, Q, false, F>;
}

template <int N>
static auto hist_kernel_q(int D, bool q32, bool filt) -> decltype(&k_hist<8, N, true>) {
  return filt ? (q32 ? hist_kernel<N, true, true>(D) : hist_kernel<N, false, true>(D))
              : (q32 ? hist_kernel<N, true, false>(D) : hist_kernel<N, false, false>(D));
}

int launch_hist(const gbdt_rows& src, const gbdt_features& ft, const TileDesc* desc,
                int64_t max_tiles, int64_t* hist_g, uint32_t* hist_cnt, uint64_t* hpart,
                WsCtrl* ctrl, hipStream_t s, bool q32, bool guard, bool ids,
                const uint8_t* rows_ix, bool filt) {
  const int64_t n_rows = src.X.n_rows > 0 ? src.X.n_rows : 1;
  const int32_t bits = pack_bits_for(n_rows);
  const bool has_bytes = src.X.n_features > src.X.n_bit_features + src.X.n_nib_features;
  const bool has_bits = src.X.n_bit_features > 0 || src.X.n_nib_features > 0;  // narrow blocks
  // byte blocks: 256 bin rows of 32 slots (any byte value stays inside);
  // the bit block: 2 slots per bit feature
  // (both within kLdsHistBudgetBins slots), then the kernel's small tables
  const size_t lds = sizeof(uint64_t) * size_t(kLdsHistBudgetBins + kHistThreads / 64) +
                     sizeof(int32_t) * size_t(2 * kHistRowSlots + kMaxBitWords + kBitStage);
  const int32_t nd = has_bytes ? src.X.block_stride / 4 : 1;  // dwords per row (<= 8)
  const int D = nd <= 1 ? 1 : (nd <= 2 ? 2 : (nd <= 4 ? 4 : 8));
  const int narrow = src.X.n_nib_features > 0 ? 2 : (src.X.n_bit_features > 0 ? 1 : 0);
  // (index mode: two or more byte blocks of at most 32 columns are at least
  // 17 columns, 5 dwords, wide, so D = 8)
  if (ids && (narrow != 0 || src.rid == nullptr || D != 8))
    return fail(GBDT_E_INTERNAL, "index mode needs byte blocks of 5 to 8 dwords and row ids");
  if (ids && filt) return fail(GBDT_E_INTERNAL, "filtered histogram tiles read rows in order");
  auto kern = ids ? (q32 ? k_hist<8, 0, true, true> : k_hist<8, 0, false, true>)
              : narrow == 2 ? hist_kernel_q<2>(D, q32, filt)
              : narrow == 1 ? hist_kernel_q<1>(D, q32, filt)
                            : hist_kernel_q<0>(D, q32, filt);
  (void)has_bits;
  const unsigned gy = (unsigned)(src.X.n_blocks + (src.X.n_bit_features > 0 ? 1 : 0) +
                                 (src.X.n_nib_features > 0 ? 1 : 0));
  // index mode gathers from the interleaved copy when there is one (row id's
  // block b at rows_ix + id pitch + b block_stride), with the XCD-aware 1-D
  // grid: ceil(max_tiles / 8) groups of 8 tiles times n_blocks blocks
  // (the root level of index mode reads X in row order, on the same grid)
  const bool ix = ids && rows_ix != nullptr;
  const bool xgrid = rows_ix != nullptr && narrow == 0 && src.X.n_blocks >= 1;
  const int64_t bs = src.X.block_stride;
  const int64_t id_blk_pitch = ix ? bs : src.X.row_capacity * bs;
  const int32_t id_row_pitch = ix ? interleave_pitch(src.X) : (int32_t)bs;
  const dim3 grid = xgrid ? dim3((unsigned)((max_tiles + 7) / 8 * 8 * src.X.n_blocks), 1u)
                          : dim3((unsigned)max_tiles, gy);
  diag_begin(kDiagHist, s);
  hipLaunchKernelGGL(kern, grid, dim3(kHistThreads), lds, s, ix ? rows_ix : src.X.bins,
                     src.X.row_capacity, src.X.n_blocks, src.X.block_features, src.X.block_stride,
                     src.X.n_features, src.X.n_bit_features, src.X.bit_stride, src.X.col_feature,
                     src.q, ft.bin_offset, ft.skip_bin, ft.total_bins, ft.max_block_bins, desc, bits,
                     hist_g, hist_cnt, hpart, ctrl, guard ? &ctrl->err : nullptr, src.X.n_nib_features,
                     src.X.nib_stride, ids ? src.rid : nullptr, id_blk_pitch, id_row_pitch,
                     xgrid ? (int32_t)max_tiles : 0);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_hist");
  return GBDT_OK;
}

int launch_hist_reduce(const int32_t* multi, int32_t list_cap, int64_t max_tiles, int64_t n_rows,
                       int32_t total_bins,
                       const uint64_t* hpart, int64_t* hist_g, uint32_t* hist_cnt, hipStream_t s,
                       const int32_t* guard) {
  const int32_t bits = pack_bits_for(n_rows > 0 ? n_rows : 1);
  // multi-tile nodes hold more than one tile of rows each, so there are at
  // most max_tiles / 2 of them; the grid covers up to kReduceNodeSlots of
  // them at once (never more than kReduceGrid workgroups: most levels have
  // few or no multi-tile nodes, and empty workgroups still take dispatch
  // time), the grid-stride loop the rest
  int64_t gy = max_tiles / 2 < list_cap ? max_tiles / 2 : list_cap;
  if (gy > kReduceNodeSlots) gy = kReduceNodeSlots;
  if (gy < 1) gy = 1;
  int64_t grid = int64_t((total_bins + 63) / 64) * gy;
  if (grid > kReduceGrid) grid = kReduceGrid;
  diag_begin(kDiagHistReduce, s);
  hipLaunchKernelGGL(k_hist_reduce, dim3((unsigned)grid), dim3(1024), 0, s, multi, list_cap,
                     (int32_t)max_tiles, bits, total_bins, hpart, hist_g, hist_cnt, guard);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_hist_reduce");
  return GBDT_OK;
}

template <bool HESS>
static int launch_find_t(int64_t* hist_g, uint32_t* hist_cnt, const gbdt_features& ft,
                         const gbdt_node* nodes, const int32_t* list, const int32_t* list_len,
                         int32_t list_cap, const gbdt_params& p, const int32_t* scale,
                         gbdt_split* splits, const int32_t* sub_par, const int32_t* sub_sib,
                         WsCtrl* ctrl, hipStream_t s, FindCand* cand, const int32_t* guard,
                         int64_t* hist_h, const int32_t* scale_h, int64_t* split_h) {
  FindParams fp{p.reg_lambda, p.gamma, p.min_child_weight, p.min_samples_leaf};
  const int32_t nch = cand != nullptr ? find_chunks(ft.total_bins) : 1;
  int32_t* err = ctrl != nullptr ? &ctrl->err : nullptr;
  diag_begin(kDiagFind, s);
  if (nch > 1) {
    // whole features of up to kFindChunk + 255 bins: one or two passes of
    // 1024 threads x 2 bins
    hipLaunchKernelGGL((k_find<1024, 2, HESS>), dim3((unsigned)list_cap, (unsigned)nch), dim3(1024), 0,
                       s, hist_g, hist_cnt, ft.bin_offset, ft.bin_feature, ft.n_bins, ft.total_bins,
                       nodes, list, list_len, list_cap, fp, scale, splits, sub_par, sub_sib, err, nch,
                       cand, guard, hist_h, scale_h, split_h);
    GBDT_LAUNCH_CHECK("k_find");
    hipLaunchKernelGGL(k_find_merge, dim3((unsigned)list_cap), dim3(64), 0, s, list, list_len,
                       list_cap, nch, (const FindCand*)cand, splits, guard, split_h);
    diag_end(s);
    GBDT_LAUNCH_CHECK("k_find_merge");
    return GBDT_OK;
  }
  // 1024 threads with the fewest bins per thread (1, 2, 3, 4, 6 or 8) that cover
  // the bins in one pass (several passes of 8 above 8192 bins): a thread's
  // scan and its candidates' FP64 divisions are a serial chain, so the
  // node's latency falls with the bins per thread
  const int32_t tb = ft.total_bins;
  int threads = 1024;
  auto kern = tb <= 1024   ? k_find<1024, 1, HESS>
              : tb <= 2048 ? k_find<1024, 2, HESS>
              : tb <= 3072 ? k_find<1024, 3, HESS>
              : tb <= 4096 ? k_find<1024, 4, HESS>
              : tb <= 6144 ? k_find<1024, 6, HESS>
                           : k_find<1024, 8, HESS>;
  if (list_cap > 256 && tb <= 4096) {
    threads = 512;
    kern = tb <= 512    ? k_find<512, 1, HESS>
           : tb <= 1024 ? k_find<512, 2, HESS>
           : tb <= 1536 ? k_find<512, 3, HESS>
           : tb <= 2048 ? k_find<512, 4, HESS>
           : tb <= 3072 ? k_find<512, 6, HESS>
                        : k_find<512, 8, HESS>;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)list_cap), dim3(threads), 0, s, hist_g, hist_cnt,
                     ft.bin_offset, ft.bin_feature, ft.n_bins, ft.total_bins, nodes, list,
                     list_len, list_cap, fp, scale, splits, sub_par, sub_sib, err, 1,
                     (FindCand*)nullptr, guard, hist_h, scale_h, split_h);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_find");
  return GBDT_OK;
}

int launch_find(int64_t* hist_g, uint32_t* hist_cnt, const gbdt_features& ft, const gbdt_node* nodes,
                const int32_t* list, const int32_t* list_len, int32_t list_cap, const gbdt_params& p,
                const int32_t* scale, gbdt_split* splits, const int32_t* sub_par,
                const int32_t* sub_sib, WsCtrl* ctrl, hipStream_t s, FindCand* cand,
                const int32_t* guard, int64_t* hist_h, const int32_t* scale_h, int64_t* split_h) {
  if (hist_h != nullptr)
    return launch_find_t<true>(hist_g, hist_cnt, ft, nodes, list, list_len, list_cap, p, scale, splits,
                               sub_par, sub_sib, ctrl, s, cand, guard, hist_h, scale_h, split_h);
  return launch_find_t<false>(hist_g, hist_cnt, ft, nodes, list, list_len, list_cap, p, scale, splits,
                              sub_par, sub_sib, ctrl, s, cand, guard, nullptr, nullptr, nullptr);
}

// ------------------------------------------------------- feature binning --
// Raw FP32 values to uint8 bins: the "Quantized" state that "Module Design:
// Training Core" (section 5, state machine) puts between validation and
// training.  Feature f has n_bins[f] bins and n_bins[f] - 1 strictly
// increasing FP32 upper bounds at upper[bin_offset[f] + k], k < n_bins[f] - 1
// (the entry at k = n_bins[f] - 1 is not read).  A value's bin is the number
// of its feature's bounds strictly below it: x <= upper[0] gives bin 0, a
// value above every bound the last bin.  Only comparisons, so exact.  A NaN
// value gets bin 0 and sets GBDT_E_RANGE, and so do bounds that are NaN or
// not strictly increasing (checked one global bin per thread).
//
// Each thread bins 16 consecutive values of the row-major matrix per step
// (four 16-byte loads, one 16-byte store), in a grid-stride loop; the
// feature index advances incrementally, with no division per value.  The
// bounds (and each feature's offset and bound count) are staged in LDS when
// they fit (LDS = true), else read from global memory.  With the bounds in
// LDS, each value first guesses its bin from the line through its feature's
// first and last bound and keeps the guess when the two bounds around it
// confirm it (one pair of lookups; exact, since only the comparisons
// decide); otherwise, and always without LDS, it searches by binary lifting
// with a fixed 8 steps (at most 255 bounds), written out per value so the
// compiler interleaves the searches of a thread's 16 values.
constexpr int kBinThreads = 256;
constexpr int kBinGrid = 4096;
constexpr size_t kBinLdsBytes = 64 * 1024;

__device__ __forceinline__ uint32_t bin_of(const float* __restrict__ t, int32_t nb, float x) {
  int32_t c = 0;
#pragma unroll
  for (int32_t s = 128; s >= 1; s >>= 1) {
    const int32_t probe = c + s - 1;
    if (probe < nb && t[probe] < x) c += s;
  }
  return (uint32_t)c;
}

// bounds of a feature of nb bins (a feature table holds 1..256 bins)
__device__ __forceinline__ int32_t bin_bounds(int32_t nb) { return nb < 1 ? 0 : (nb > 256 ? 255 : nb - 1); }

// LDS words of k_bin: the skewed bounds, a word per feature, and (aligned
// to 8 bytes) a (first bound, 1 / spacing) pair per feature.
__host__ __device__ inline size_t bin_lds_words(int32_t tb, int32_t F) {
  return ((size_t(tb) + 2 * size_t(F) + 1) & ~size_t(1)) + 2 * size_t(F);
}

template <bool LDS>
__global__ void __launch_bounds__(kBinThreads) k_bin(const float* __restrict__ raw, int64_t n_vals,
                                                     int32_t F, const int32_t* __restrict__ n_bins,
                                                     const int32_t* __restrict__ bin_offset,
                                                     const int32_t* __restrict__ bin_feature,
                                                     int32_t total_bins, const float* __restrict__ upper,
                                                     uint8_t* __restrict__ out, WsCtrl* __restrict__ ctrl) {
  // LDS: the bounds, feature f's from bin_offset[f] + f (the skew by f puts
  // bound k of different features in different banks: with 64 bins per
  // feature they would otherwise all share one bank), then one word per
  // feature, its offset << 8 | its bound count
  extern __shared__ float s_bin[];
  const float* tab = upper;
  const int32_t* offs = bin_offset;
  uint32_t* s_meta = reinterpret_cast<uint32_t*>(s_bin + total_bins + F);  // offset << 8 | bound count
  float2* s_gs = reinterpret_cast<float2*>(s_bin + ((size_t(total_bins) + 2 * size_t(F) + 1) & ~size_t(1)));
  if constexpr (LDS) {
    for (int32_t i = threadIdx.x; i < total_bins; i += blockDim.x) s_bin[i + bin_feature[i]] = upper[i];
    for (int32_t f = threadIdx.x; f < F; f += blockDim.x) {
      const int32_t nb = bin_bounds(n_bins[f]);
      s_meta[f] = ((uint32_t)(bin_offset[f] + f) << 8) | (uint32_t)nb;
      // the guess's line through the first and last bound (0 slope when the
      // spacing is not a finite positive number)
      const float u0 = nb > 0 ? upper[bin_offset[f]] : 0.0f;
      const float u1 = nb > 0 ? upper[bin_offset[f] + nb - 1] : 0.0f;
      float inv = 0.0f;
      if (nb >= 2 && u1 > u0) {
        inv = (float)(nb - 1) / (u1 - u0);
        if (!(inv <= 3.0e38f)) inv = 0.0f;
      }
      s_gs[f] = make_float2(u0, inv);
    }
    __syncthreads();
    tab = s_bin;
  }
  const int64_t G = int64_t(gridDim.x) * blockDim.x;
  int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  {
    // the bounds, one global bin per thread: bound k of feature f is read
    // when k < n_bins[f] - 1 and compared with bound k + 1 below the last
    bool bad = false;
    for (int64_t i = c; i < total_bins; i += G) {
      const int32_t fb = bin_feature[i];
      const int32_t k = (int32_t)i - bin_offset[fb], nb = n_bins[fb] - 1;
      if (k < nb) {
        const float u = upper[i];
        bad |= u != u || (k + 1 < nb && !(u < upper[i + 1]));
      }
    }
    if (bad) dev_error(&ctrl->err, GBDT_E_RANGE);
  }
  const int64_t nchunks = (n_vals + 15) / 16;
  if (c >= nchunks) return;
  int32_t f = (int32_t)((c * 16) % F);
  const int32_t step_f = (int32_t)((G * 16) % F);
  bool nan = false;
  for (; c < nchunks; c += G) {
    const int64_t i0 = c * 16;
    const bool full = i0 + 16 <= n_vals;
    float v[16];
    if (full) {
      const float4* p = reinterpret_cast<const float4*>(raw + i0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 x = p[q];
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = i0 + e < n_vals ? raw[i0 + e] : 0.0f;
    }
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    int32_t fe = f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      int32_t o, nb;
      if constexpr (LDS) {
        const uint32_t mt = s_meta[fe];
        o = (int32_t)(mt >> 8);
        nb = (int32_t)(mt & 0xffu);
      } else {
        o = offs[fe];
        nb = bin_bounds(n_bins[fe]);
      }
      nan |= v[e] != v[e];
      uint32_t bin;
      if constexpr (LDS) {
        // guess from the line through the first and last bound (exact for
        // equal-width bounds up to rounding), kept if the two bounds around it
        // confirm it, else the full search
        const float2 gs = s_gs[fe];
        float t = (v[e] - gs.x) * gs.y;
        t = fminf(fmaxf(t, 0.0f), (float)nb);
        const int32_t gg = (int32_t)ceilf(t);
        const float lo = tab[o + (gg > 0 ? gg - 1 : 0)];
        const float hi = tab[o + (gg < nb ? gg : 0)];
        const bool ok = (gg == 0 || lo < v[e]) && (gg == nb || !(hi < v[e]));
        bin = ok ? (uint32_t)gg : bin_of(tab + o, nb, v[e]);
      } else {
        bin = bin_of(tab + o, nb, v[e]);
      }
      w[e >> 2] |= bin << (8 * (e & 3));
      fe = fe + 1 == F ? 0 : fe + 1;
    }
    if (full) {
      *reinterpret_cast<uint4*>(out + i0) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (i0 + e < n_vals) out[i0 + e] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
    }
    f += step_f;
    if (f >= F) f -= F;
  }
  if (nan) dev_error(&ctrl->err, GBDT_E_RANGE);
}

// ------------------------------------------------------------ bin bounds --
// How the bounds of the "Quantized" state (Training Core, section 5) are
// chosen; the page names the state only.  Equal width: u_k = lo + (hi - lo)
// (k / B) over each feature's finite range, in FP64 one operation at a time
// and rounded to FP32.  Quantile: u_k is the ceil(k m / B)-th smallest of the
// m finite values in a row sample (rows 0, s, 2s, ..., at most kQuantSample
// of them), as GBDT libraries sample rows to build bins.  Then bounds that do
// not increase are raised to next_up of their predecessor.
constexpr int kQuantSample = 32768;
constexpr int kBoundThreads = 1024;

// Order-preserving key of a float (larger float, larger key), -0 taken as
// +0; finite values only come through here.
__device__ __forceinline__ uint32_t float_key(float x) {
  const uint32_t b = x == 0.0f ? 0u : __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The next FP32 value above x among zero and the normal values: FLT_MIN for
// a zero, 0 for a negative value whose next value would be subnormal, +inf
// stays +inf.
__device__ __forceinline__ float next_up_normal(float x) {
  if (x == __int_as_float(0x7f800000)) return x;
  if (x == 0.0f) return __uint_as_float(0x00800000u);
  uint32_t b = __float_as_uint(x);
  b = x > 0.0f ? b + 1u : b - 1u;
  float y = __uint_as_float(b);
  if (y < 0.0f && y > -__uint_as_float(0x00800000u)) y = 0.0f;
  return y;
}

// Raise bounds that do not increase, in order (one thread per feature).
__device__ __forceinline__ void strictly_increasing(float* u, int32_t nb) {
  for (int32_t k = 1; k < nb; ++k)
    if (!(u[k] > u[k - 1])) u[k] = next_up_normal(u[k - 1]);
}

__global__ void __launch_bounds__(256) k_range_init(uint32_t* __restrict__ kmin,
                                                    uint32_t* __restrict__ kmax, int32_t F) {
  for (int32_t f = blockIdx.x * 256 + threadIdx.x; f < F; f += gridDim.x * 256) {
    kmin[f] = 0xffffffffu;
    kmax[f] = 0u;
  }
}

// Least and greatest finite value of each feature, as order-preserving keys:
// per workgroup in LDS, then one device atomic per feature and workgroup.
// Each thread takes runs of 16 consecutive values (four 16-byte loads), the
// feature index advancing by one per value.
__global__ void __launch_bounds__(kBinThreads) k_range(const float* __restrict__ raw, int64_t n_vals,
                                                       int32_t F, uint32_t* __restrict__ kmin,
                                                       uint32_t* __restrict__ kmax) {
  extern __shared__ uint32_t s_key[];  // [F] minima, then [F] maxima
  for (int32_t f = threadIdx.x; f < F; f += blockDim.x) {
    s_key[f] = 0xffffffffu;
    s_key[F + f] = 0u;
  }
  __syncthreads();
  const int64_t stride = int64_t(gridDim.x) * blockDim.x * 16;
  for (int64_t v0 = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 16; v0 < n_vals; v0 += stride) {
    float x[16];
    if (v0 + 16 <= n_vals) {
      const float4* p = reinterpret_cast<const float4*>(raw + v0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = p[q];
        x[4 * q] = t.x;
        x[4 * q + 1] = t.y;
        x[4 * q + 2] = t.z;
        x[4 * q + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) x[q] = v0 + q < n_vals ? raw[v0 + q] : __int_as_float(0x7fc00000);
    }
    int32_t f = (int32_t)(v0 % F);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (isfinite(x[q])) {
        const uint32_t k = float_key(x[q]);
        atomicMin(&s_key[f], k);
        atomicMax(&s_key[F + f], k);
      }
      if (++f == F) f = 0;
    }
  }
  __syncthreads();
  for (int32_t f = threadIdx.x; f < F; f += blockDim.x) {
    if (s_key[f] != 0xffffffffu) atomicMin(&kmin[f], s_key[f]);
    if (s_key[F + f] != 0u) atomicMax(&kmax[f], s_key[F + f]);
  }
}

// Equal-width bounds from the ranges (one thread per feature).
__global__ void __launch_bounds__(256) k_bounds_width(const uint32_t* __restrict__ kmin,
                                                      const uint32_t* __restrict__ kmax, int32_t F,
                                                      const int32_t* __restrict__ n_bins,
                                                      const int32_t* __restrict__ bin_offset,
                                                      float* __restrict__ upper) {
  const int32_t f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const bool have = kmin[f] != 0xffffffffu;
  const float lo = have ? key_float(kmin[f]) : 0.0f;
  const float hi = have ? key_float(kmax[f]) : 0.0f;
  const int32_t B = n_bins[f];
  float* u = upper + bin_offset[f];
  for (int32_t k = 1; k < B; ++k) {
    const double t = (double)k / (double)B;
    const double w = (double)hi - (double)lo;
    const double m = w * t;
    u[k - 1] = (float)((double)lo + m);
  }
  strictly_increasing(u, B - 1);
  u[B - 1] = __int_as_float(0x7f800000);
}

// Quantile bounds: one workgroup per feature sorts the keys of its sampled
// finite values in LDS (bitonic, non-finite values as the largest key, past
// the m finite ones) and reads the ranks off.
__global__ void __launch_bounds__(kBoundThreads) k_bounds_quantile(const float* __restrict__ raw,
                                                                   int64_t n, int32_t F, int64_t step,
                                                                   int32_t cnt, int32_t P,
                                                                   const int32_t* __restrict__ n_bins,
                                                                   const int32_t* __restrict__ bin_offset,
                                                                   float* __restrict__ upper) {
  extern __shared__ uint32_t s_sort[];  // [P] keys, P a power of two >= cnt
  __shared__ int32_t s_m[kBoundThreads / 64];
  const int32_t f = blockIdx.x;
  int32_t mine = 0;
  for (int32_t j = threadIdx.x; j < P; j += kBoundThreads) {
    uint32_t k = 0xffffffffu;
    if (j < cnt) {
      const float x = raw[int64_t(j) * step * F + f];
      if (isfinite(x)) {
        k = float_key(x);
        ++mine;
      }
    }
    s_sort[j] = k;
  }
  mine = wave_sum(mine);
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = mine;
  __syncthreads();
  int32_t m = 0;
  for (int w = 0; w < kBoundThreads / 64; ++w) m += s_m[w];
  // bitonic sort, ascending
  for (int32_t size = 2; size <= P; size <<= 1) {
    for (int32_t half = size >> 1; half > 0; half >>= 1) {
      for (int32_t t = threadIdx.x; t < P / 2; t += kBoundThreads) {
        const int32_t i = 2 * t - (t & (half - 1));  // low index of the pair
        const int32_t j = i + half;
        const bool up = (i & size) == 0;
        const uint32_t a = s_sort[i], b = s_sort[j];
        if ((a > b) == up) {
          s_sort[i] = b;
          s_sort[j] = a;
        }
      }
      __syncthreads();
    }
  }
  const int32_t B = n_bins[f];
  float* u = upper + bin_offset[f];
  for (int32_t k = 1 + threadIdx.x; k < B; k += kBoundThreads) {
    if (m == 0) {
      u[k - 1] = 0.0f;
    } else {
      const int64_t r = (int64_t(k) * m + B - 1) / B - 1;
      u[k - 1] = key_float(s_sort[r]);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    strictly_increasing(u, B - 1);
    u[B - 1] = __int_as_float(0x7f800000);
  }
}

template <int K, bool Q, bool N, bool F>
static auto partition_kernel_f(int32_t nd) -> decltype(&k_partition<1, K, Q, N>) {
  switch (nd) {
    case 1: return k_partition<1, K, Q, N, false, F>;
    case 2: return k_partition<2, K, Q, N, false, F>;
    case 3: return k_partition<3, K, Q, N, false, F>;
    case 4: return k_partition<4, K, Q, N, false, F>;
    case 5: return k_partition<5, K, Q, N, false, F>;
    case 6: return k_partition<6, K, Q, N, false, F>;
    case 7: return k_partition<7, K, Q, N, false, F>;
    case 8: return k_partition<8, K, Q, N, false, F>;
    default: return nullptr;
  }
}

// The row-moving kernel for rows of nd dwords; four: the two-level form.
template <int K, bool Q, bool N>
static auto partition_kernel(int32_t nd, bool four) -> decltype(&k_partition<1, K, Q, N>) {
  return four ? partition_kernel_f<K, Q, N, true>(nd) : partition_kernel_f<K, Q, N, false>(nd);
}

int launch_partition(const gbdt_rows& src, const gbdt_rows& dst, const TileDesc* desc,
                     uint64_t* status, WsCtrl* ctrl, int64_t max_tiles, int32_t tile_rows,
                     hipStream_t s, bool qin32, bool qout32, bool ids, const uint8_t* cols,
                     bool four, uint64_t* status2) {
  const int32_t nd = src.X.n_blocks > 0 ? src.X.block_stride / 4 : 1;
  if (qin32 && !qout32) return fail(GBDT_E_INTERNAL, "an int64 q destination needs an int64 source");
  if (four && (ids || status2 == nullptr))
    return fail(GBDT_E_INTERNAL, "two-level partitions move rows and need a second status array");
  decltype(&k_partition<1, 2, false, false>) kern = nullptr;
  const bool nib = src.X.n_nib_features > 0;
  if (ids) {
    if (nib || src.X.n_bit_features > 0 || src.X.n_blocks < 1 || dst.rid == nullptr)
      return fail(GBDT_E_INTERNAL, "index mode needs byte blocks and row ids");
    if (tile_rows == 2 * kPartThreads)
      kern = qout32 ? k_partition<1, 2, true, false, true> : k_partition<1, 2, false, false, true>;
    else if (tile_rows == 8 * kPartThreads)
      kern = qout32 ? k_partition<1, 8, true, false, true> : k_partition<1, 8, false, false, true>;
    else
      return fail(GBDT_E_INTERNAL, "unsupported partition tile size");
  } else if (tile_rows == 2 * kPartThreads)
    kern = nib ? (qout32 ? partition_kernel<2, true, true>(nd, four) : partition_kernel<2, false, true>(nd, four))
               : (qout32 ? partition_kernel<2, true, false>(nd, four)
                         : partition_kernel<2, false, false>(nd, four));
  else if (tile_rows == 4 * kPartThreads && qout32 && nd <= 7)
    kern = nib ? partition_kernel<4, true, true>(nd, four) : partition_kernel<4, true, false>(nd, four);
  else
    return fail(GBDT_E_INTERNAL, "unsupported partition tile size");
  if (kern == nullptr) return fail(GBDT_E_UNSUPPORTED, "a column block wider than 32 bytes");
  diag_begin(kDiagPartition, s);
  hipLaunchKernelGGL(kern, dim3((unsigned)max_tiles), dim3(kPartThreads), 0, s, src.X.bins, src.q,
                     src.rid, dst.X.bins, dst.q, dst.rid, src.X.row_capacity, src.X.n_blocks,
                     src.X.block_features, src.X.block_stride, src.X.n_features,
                     src.X.n_bit_features, src.X.bit_stride, desc, status, ctrl, qin32 ? 2 : 3,
                     src.X.n_nib_features, src.X.nib_stride, ids ? cols : nullptr,
                     four ? status2 : nullptr);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_partition");
  return GBDT_OK;
}

}  // namespace gbdt

using namespace gbdt;

// ==================================================================== C ABI ==

extern "C" {

int gbdt_abi_version(void) { return GBDT_ABI_VERSION; }

int gbdt_diag_enable(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return fail(GBDT_E_ARG, "capacity out of range");
  if (g_diag.capacity < capacity) {
    const int32_t old = g_diag.capacity;
    g_diag.ev.resize(size_t(2) * capacity);
    g_diag.kind.resize(capacity);
    for (int32_t i = 2 * old; i < 2 * capacity; ++i) {
      hipError_t e = hipEventCreateWithFlags(&g_diag.ev[i], hipEventDisableSystemFence);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    g_diag.capacity = capacity;
  }
  g_diag.count = 0;
  g_diag.open = false;
  g_diag.enabled = true;
  return GBDT_OK;
}

int gbdt_diag_disable(void) {
  g_diag.enabled = false;
  return GBDT_OK;
}

int gbdt_diag_read(int32_t max_records, int32_t* kinds, float* ms, int32_t* n_out) {
  if (!kinds || !ms || !n_out || max_records < 0) return fail(GBDT_E_ARG, "null argument");
  const int32_t n = g_diag.count < max_records ? g_diag.count : max_records;
  if (g_diag.count > 0) {
    hipError_t e = hipEventSynchronize(g_diag.ev[2 * g_diag.count - 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  }
  for (int32_t i = 0; i < n; ++i) {
    kinds[i] = g_diag.kind[i];
    float t = 0.f;
    hipError_t e = hipEventElapsedTime(&t, g_diag.ev[2 * i], g_diag.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    ms[i] = t;
  }
  *n_out = n;
  g_diag.count = 0;
  return GBDT_OK;
}

const char* gbdt_last_error(void) { return g_last_error.c_str(); }

int gbdt_validate_params(const gbdt_params* p) {
  if (!p) return fail(GBDT_E_ARG, "params is null");
  if (!std::isfinite(p->reg_lambda) || !std::isfinite(p->gamma) ||
      !std::isfinite(p->min_child_weight) || !std::isfinite(p->learning_rate))
    return fail(GBDT_E_ARG, "every floating parameter must be finite");
  if (p->min_samples_leaf < 1) return fail(GBDT_E_ARG, "min_samples_leaf must be >= 1");
  if (p->min_child_weight < 0.0) return fail(GBDT_E_ARG, "min_child_weight must be >= 0");
  if (p->reg_lambda < 0.0) return fail(GBDT_E_ARG, "reg_lambda must be >= 0");
  if (p->gamma < 0.0) return fail(GBDT_E_ARG, "gamma must be >= 0");
  if (p->max_depth < 0 || p->max_depth > GBDT_MAX_DEPTH) return fail(GBDT_E_ARG, "max_depth out of range");
  if (p->objective != GBDT_OBJECTIVE_SQUARED_ERROR && p->objective != GBDT_OBJECTIVE_LOGISTIC)
    return fail(GBDT_E_ARG, "unknown objective");
  return GBDT_OK;
}

size_t gbdt_workspace_bytes(int64_t n_rows, int32_t max_list, int32_t total_bins) {
  return ws_layout(n_rows, max_list, total_bins).total;
}

int gbdt_choose_layout(int32_t n_features, const int32_t* n_bins_host, int32_t pack,
                       gbdt_matrix* X, int32_t* max_block_bins, int32_t* col_feature_host,
                       int32_t* feature_col_host) {
  if (!X || !n_bins_host || !max_block_bins || !col_feature_host || !feature_col_host)
    return fail(GBDT_E_ARG, "null argument");
  if (n_features < 1 || n_features > GBDT_MAX_FEATURES) return fail(GBDT_E_ARG, "n_features out of range");
  for (int32_t f = 0; f < n_features; ++f)
    if (n_bins_host[f] < 1 || n_bins_host[f] > GBDT_MAX_BINS) return fail(GBDT_E_ARG, "n_bins out of range");
  // byte columns first (feature order), then the nibble features, then the
  // bit features (each in feature order)
  const bool bits = (pack & GBDT_PACK_BITS) != 0;
  const bool nibs = (pack & GBDT_PACK_NIBBLES) != 0;
  auto is_bit = [&](int32_t f) { return bits && n_bins_host[f] <= 2; };
  auto is_nib = [&](int32_t f) { return nibs && !is_bit(f) && n_bins_host[f] <= 16; };
  std::vector<int32_t> cols;
  int32_t n_bit = 0, n_nib = 0;
  for (int32_t f = 0; f < n_features; ++f)
    if (!is_bit(f) && !is_nib(f)) cols.push_back(f);
  const int32_t nbc = (int32_t)cols.size();
  for (int32_t f = 0; f < n_features; ++f)
    if (is_nib(f)) {
      cols.push_back(f);
      ++n_nib;
    }
  for (int32_t f = 0; f < n_features; ++f)
    if (is_bit(f)) {
      cols.push_back(f);
      ++n_bit;
    }
  if (2 * n_bit > kLdsHistBudgetBins) return fail(GBDT_E_UNSUPPORTED, "too many bit features for the LDS budget");
  if (kNibSlots * n_nib > kLdsHistBudgetBins)
    return fail(GBDT_E_UNSUPPORTED, "too many nibble features for the LDS budget");
  int32_t worst = 2 * n_bit > kNibSlots * n_nib ? 2 * n_bit : kNibSlots * n_nib;
  int32_t bf = 0, nb = 0;
  if (nbc > 0) {
    // fewest blocks of equal width, at most 32 columns (8 dwords per row);
    // the histogram of a byte block takes 32 LDS slots per bin row
    nb = (nbc + kHistRowSlots - 1) / kHistRowSlots;
    bf = (nbc + nb - 1) / nb;
    nb = (nbc + bf - 1) / bf;
    int32_t bmax = 0;
    for (int32_t c = 0; c < nbc; ++c) bmax = n_bins_host[cols[c]] > bmax ? n_bins_host[cols[c]] : bmax;
    if (kHistRowSlots * bmax > worst) worst = kHistRowSlots * bmax;
  }
  X->n_features = n_features;
  X->n_blocks = nb;
  X->block_features = bf;
  X->block_stride = nbc > 0 ? ((bf + 3) & ~3) : 0;
  X->n_bit_features = n_bit;
  X->bit_stride = n_bit > 0 ? 4 * ((n_bit + 31) / 32) : 0;
  X->n_nib_features = n_nib;
  X->nib_stride = n_nib > 0 ? 4 * ((n_nib + 7) / 8) : 0;
  X->col_feature = nullptr;
  X->feature_col = nullptr;
  for (int32_t c = 0; c < n_features; ++c) {
    col_feature_host[c] = cols[c];
    feature_col_host[cols[c]] = c;
  }
  *max_block_bins = worst;
  return GBDT_OK;
}

int gbdt_choose_blocking(int32_t n_features, const int32_t* n_bins_host, gbdt_matrix* X,
                         int32_t* max_block_bins) {
  if (!X || !n_bins_host || !max_block_bins) return fail(GBDT_E_ARG, "null argument");
  if (n_features < 1 || n_features > GBDT_MAX_FEATURES) return fail(GBDT_E_ARG, "n_features out of range");
  std::vector<int32_t> cf(n_features), fc(n_features);
  return gbdt_choose_layout(n_features, n_bins_host, 0, X, max_block_bins, cf.data(), fc.data());
}

int gbdt_read_error(void* ws, void* stream) {
  if (!ws) return fail(GBDT_E_ARG, "workspace is null");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  WsCtrl c;
  hipError_t e = hipMemcpyAsync(&c, ws, sizeof(WsCtrl), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the error word");
  if (c.err != 0) {
    int32_t zero[2] = {0, 0};
    e = hipMemcpyAsync(ws, zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "clearing the error word");
    return fail(c.err, "device-side check failed (code " + std::to_string(c.err) + ")");
  }
  return GBDT_OK;
}

int gbdt_feature_bounds(const float* raw, int64_t n_rows, const gbdt_features* ft, int32_t method,
                        float* upper, void* ws, size_t ws_bytes, void* stream) {
  if (!ft || !upper) return fail(GBDT_E_ARG, "null argument");
  if (method != GBDT_BOUNDS_EQUAL_WIDTH && method != GBDT_BOUNDS_QUANTILE)
    return fail(GBDT_E_ARG, "unknown bounds method");
  if (n_rows < 0 || n_rows > 0x7fffffffLL) return fail(GBDT_E_ARG, "n_rows out of range");
  if (n_rows > 0 && !raw) return fail(GBDT_E_ARG, "null argument");
  if (ft->n_features < 1 || ft->n_features > GBDT_MAX_FEATURES) return fail(GBDT_E_ARG, "n_features out of range");
  int rc = check_features(*ft, ft->n_features);
  if (rc) return rc;
  if (!aligned(raw, 16) || !aligned(upper, 4)) return fail(GBDT_E_ARG, "raw must be 16-byte aligned");
  const WsLayout L = ws_layout(n_rows < 1 ? 1 : n_rows, 1, ft->total_bins);
  rc = check_ws(ws, ws_bytes, L);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int32_t F = ft->n_features;
  diag_begin(kDiagBounds, s);
  if (method == GBDT_BOUNDS_EQUAL_WIDTH) {
    uint32_t* kmin = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.hpart);
    uint32_t* kmax = kmin + F;
    const unsigned fg = (unsigned)((F + 255) / 256);
    hipLaunchKernelGGL(k_range_init, dim3(fg), dim3(256), 0, s, kmin, kmax, F);
    GBDT_LAUNCH_CHECK("k_range_init");
    const int64_t n_vals = n_rows * F;
    if (n_vals > 0) {
      int64_t grid = (n_vals + 16 * kBinThreads - 1) / (16 * kBinThreads);
      if (grid > kBinGrid) grid = kBinGrid;
      hipLaunchKernelGGL(k_range, dim3((unsigned)grid), dim3(kBinThreads), 2 * sizeof(uint32_t) * size_t(F), s,
                         raw, n_vals, F, kmin, kmax);
      GBDT_LAUNCH_CHECK("k_range");
    }
    hipLaunchKernelGGL(k_bounds_width, dim3(fg), dim3(256), 0, s, (const uint32_t*)kmin,
                       (const uint32_t*)kmax, F, ft->n_bins, ft->bin_offset, upper);
    GBDT_LAUNCH_CHECK("k_bounds_width");
  } else {
    const int64_t step = n_rows <= kQuantSample ? 1 : (n_rows + kQuantSample - 1) / kQuantSample;
    const int32_t cnt = n_rows == 0 ? 0 : int32_t((n_rows + step - 1) / step);
    int32_t P = 2;
    while (P < cnt) P <<= 1;
    hipLaunchKernelGGL(k_bounds_quantile, dim3((unsigned)F), dim3(kBoundThreads), sizeof(uint32_t) * size_t(P), s,
                       raw, n_rows, F, step, cnt, P, ft->n_bins, ft->bin_offset, upper);
    GBDT_LAUNCH_CHECK("k_bounds_quantile");
  }
  diag_end(s);
  return GBDT_OK;
}

int gbdt_bin_features(const float* raw, int64_t n_rows, const gbdt_features* ft, const float* upper,
                      uint8_t* bins_out, void* ws, size_t ws_bytes, void* stream) {
  if (!ft || !upper) return fail(GBDT_E_ARG, "null argument");
  if (n_rows < 0 || n_rows > 0x7fffffffLL) return fail(GBDT_E_ARG, "n_rows out of range");
  if (n_rows > 0 && (!raw || !bins_out)) return fail(GBDT_E_ARG, "null argument");
  if (ft->n_features < 1 || ft->n_features > GBDT_MAX_FEATURES) return fail(GBDT_E_ARG, "n_features out of range");
  int rc = check_features(*ft, ft->n_features);
  if (rc) return rc;
  if (!aligned(raw, 16) || !aligned(bins_out, 16)) return fail(GBDT_E_ARG, "raw and bins_out must be 16-byte aligned");
  const WsLayout L = ws_layout(n_rows < 1 ? 1 : n_rows, 1, 1);
  rc = check_ws(ws, ws_bytes, L);
  if (rc) return rc;
  if (n_rows == 0) return GBDT_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  WsCtrl* ctrl = reinterpret_cast<WsCtrl*>(static_cast<char*>(ws) + L.ctrl);
  const int32_t F = ft->n_features;
  const int64_t n_vals = n_rows * F;
  int64_t grid = (n_vals + 16 * kBinThreads - 1) / (16 * kBinThreads);
  if (grid > kBinGrid) grid = kBinGrid;
  const size_t lds = sizeof(float) * bin_lds_words(ft->total_bins, F);
  diag_begin(kDiagBin, s);
  if (lds <= kBinLdsBytes)
    hipLaunchKernelGGL(k_bin<true>, dim3((unsigned)grid), dim3(kBinThreads), lds, s, raw, n_vals, F, ft->n_bins,
                       ft->bin_offset, ft->bin_feature, ft->total_bins, upper, bins_out, ctrl);
  else
    hipLaunchKernelGGL(k_bin<false>, dim3((unsigned)grid), dim3(kBinThreads), 0, s, raw, n_vals, F, ft->n_bins,
                       ft->bin_offset, ft->bin_feature, ft->total_bins, upper, bins_out, ctrl);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_bin");
  return GBDT_OK;
}

int gbdt_pack_matrix(const uint8_t* rowmajor, const gbdt_matrix* dst, const gbdt_features* ft,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!rowmajor || !dst || !ft) return fail(GBDT_E_ARG, "null argument");
  int rc = check_matrix(*dst);
  if (rc) return rc;
  rc = check_features(*ft, dst->n_features);
  if (rc) return rc;
  const WsLayout L = ws_layout(dst->n_rows, 1, ft->total_bins);
  rc = check_ws(ws, ws_bytes, L);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  WsCtrl* ctrl = reinterpret_cast<WsCtrl*>(w + L.ctrl);
  const int64_t n = dst->n_rows;
  if (n > 0) {
    const int64_t grid = (n + 255) / 256;
    diag_begin(kDiagPack, s);
    hipLaunchKernelGGL(k_pack, dim3((unsigned)grid), dim3(256), 0, s, rowmajor, n,
                       dst->n_features, dst->bins, dst->row_capacity, dst->n_blocks,
                       dst->block_features, dst->block_stride, dst->n_bit_features,
                       dst->bit_stride, dst->col_feature, ft->n_bins, ctrl, dst->n_nib_features,
                       dst->nib_stride);
    diag_end(s);
    GBDT_LAUNCH_CHECK("k_pack");
  }
  if (ft->skip_bin) {
    uint32_t* counts = reinterpret_cast<uint32_t*>(w + L.hpart);
    const int64_t nc = int64_t(dst->n_features) * 256;
    diag_begin(kDiagPack, s);
    hipLaunchKernelGGL(k_zero_u32, dim3(256), dim3(256), 0, s, counts, nc);
    diag_end(s);
    GBDT_LAUNCH_CHECK("k_zero_u32");
    if (n > 0) {
      int64_t gx = n / 4096 + 1;
      if (gx > 512) gx = 512;
      const int32_t gy = (dst->n_features + 63) / 64;
      diag_begin(kDiagPack, s);
      hipLaunchKernelGGL(k_census, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, rowmajor, n,
                         dst->n_features, counts);
      diag_end(s);
      GBDT_LAUNCH_CHECK("k_census");
    }
    diag_begin(kDiagPack, s);
    hipLaunchKernelGGL(k_pick_skip, dim3((unsigned)dst->n_features), dim3(64), 0, s, counts,
                       dst->n_features, ft->n_bins, ft->skip_bin);
    diag_end(s);
    GBDT_LAUNCH_CHECK("k_pick_skip");
  }
  return GBDT_OK;
}

int gbdt_interleave_rows(const gbdt_matrix* X, uint8_t* out, void* stream) {
  if (!X || !out) return fail(GBDT_E_ARG, "null argument");
  int rc = check_matrix(*X);
  if (rc) return rc;
  if (!aligned(out, 4)) return fail(GBDT_E_ARG, "out not 4-byte aligned");
  if (X->n_blocks < 1 || X->block_stride < 4) return GBDT_OK;
  const int32_t pd = interleave_pitch(*X) / 4;
  const int64_t total = X->row_capacity * pd;
  if (total == 0) return GBDT_OK;
  int64_t grid = (total + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  diag_begin(kDiagPack, s);
  hipLaunchKernelGGL(k_interleave, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(X->bins), reinterpret_cast<uint32_t*>(out),
                     X->row_capacity, X->n_blocks, X->block_stride / 4, pd);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_interleave");
  return GBDT_OK;
}

int32_t gbdt_interleave_pitch(const gbdt_matrix* X) {
  if (!X || X->n_blocks < 1 || X->block_stride < 4) return 0;
  return interleave_pitch(*X);
}

int gbdt_column_major(const gbdt_matrix* X, uint8_t* out, void* stream) {
  if (!X || !out) return fail(GBDT_E_ARG, "null argument");
  int rc = check_matrix(*X);
  if (rc) return rc;
  const int32_t n_cols = X->n_features - X->n_bit_features - X->n_nib_features;
  const int64_t total = n_cols > 0 && X->n_blocks > 0 ? X->row_capacity * n_cols : 0;
  if (total == 0) return GBDT_OK;
  int64_t grid = (total + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  diag_begin(kDiagPack, s);
  hipLaunchKernelGGL(k_columns, dim3((unsigned)grid), dim3(256), 0, s, X->bins, out, X->row_capacity,
                     n_cols, X->block_features, X->block_stride);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_columns");
  return GBDT_OK;
}

int gbdt_compute_gradients(const double* pred, const float* label, int64_t n, int64_t* q,
                           int32_t* scale, int64_t* gsum, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!gsum) return fail(GBDT_E_ARG, "null argument");
  const WsLayout L = ws_layout(n < 1 ? 1 : n, 1, 1);
  const int rc = check_ws(ws, ws_bytes, L);
  if (rc) return rc;
  char* w = static_cast<char*>(ws);
  return launch_gradients(pred, label, n, q, false, scale, gsum, reinterpret_cast<double*>(w + L.gpart),
                          reinterpret_cast<WsCtrl*>(w + L.ctrl), reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace gbdt {

int launch_gradients(const double* pred, const float* label, int64_t n, void* q, bool q32,
                     int32_t* scale, int64_t* gsum, double* part, WsCtrl* ctrl, hipStream_t s) {
  if (!pred || !label || !q || !scale) return fail(GBDT_E_ARG, "null argument");
  if (n < 1 || n > 0x7fffffffLL) return fail(GBDT_E_ARG, "n out of range");
  if (q32 && ceil_log2(n) < 22) return fail(GBDT_E_INTERNAL, "int32 q needs ceil(log2 n) >= 22");
  int64_t* psum = reinterpret_cast<int64_t*>(part + kGradBlocks);
  const int32_t blocks = grad_blocks(n);
  diag_begin(kDiagGradMax, s);
  hipLaunchKernelGGL(k_grad_max, dim3((unsigned)blocks), dim3(256), 0, s, pred, label, n, part, ctrl);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_grad_max");
  diag_begin(kDiagGradQ, s);
  if (q32)
    hipLaunchKernelGGL(k_grad_q<int32_t>, dim3((unsigned)blocks), dim3(256), 0, s, pred, label, n,
                       ceil_log2(n), part, blocks, static_cast<int32_t*>(q), scale, psum);
  else
    hipLaunchKernelGGL(k_grad_q<int64_t>, dim3((unsigned)blocks), dim3(256), 0, s, pred, label, n,
                       ceil_log2(n), part, blocks, static_cast<int64_t*>(q), scale, psum);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_grad_q");
  if (gsum != nullptr) {
    hipLaunchKernelGGL(k_grad_sum, dim3(1), dim3(kGradBlocks), 0, s, (const int64_t*)psum, blocks, gsum);
    GBDT_LAUNCH_CHECK("k_grad_sum");
  }
  return GBDT_OK;
}

int launch_gradients_logistic(const double* pred, const float* label, int64_t n, int32_t* q,
                              int32_t* qh, int32_t* scale, int32_t* scale_h, double* part,
                              WsCtrl* ctrl, hipStream_t s) {
  if (!pred || !label || !q || !qh || !scale || !scale_h) return fail(GBDT_E_ARG, "null argument");
  if (n < 1 || n > 0x7fffffffLL) return fail(GBDT_E_ARG, "n out of range");
  double* part_h = part + 2 * kGradBlocks;
  int64_t* psum = reinterpret_cast<int64_t*>(part + kGradBlocks);
  int64_t* psum_h = reinterpret_cast<int64_t*>(part + 3 * kGradBlocks);
  const int32_t blocks = grad_blocks(n);
  diag_begin(kDiagGradMax, s);
  hipLaunchKernelGGL(k_lgrad_max, dim3((unsigned)blocks), dim3(256), 0, s, pred, label, n, part, part_h,
                     ctrl);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_lgrad_max");
  diag_begin(kDiagGradQ, s);
  hipLaunchKernelGGL(k_lgrad_q, dim3((unsigned)blocks), dim3(256), 0, s, pred, label, n, ceil_log2(n),
                     (const double*)part, (const double*)part_h, blocks, q, qh, scale, scale_h, psum,
                     psum_h);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_lgrad_q");
  return GBDT_OK;
}

int update_predictions(double* pred, const gbdt_matrix* X, const gbdt_node* nodes,
                       int32_t* n_nodes, int32_t max_nodes, double learning_rate, void* ws,
                       size_t ws_bytes, hipStream_t s, bool driver) {
  if (!pred || !X || !nodes || !n_nodes) return fail(GBDT_E_ARG, "null argument");
  int rc = check_matrix(*X);
  if (rc) return rc;
  if (max_nodes < 1) return fail(GBDT_E_ARG, "max_nodes must be >= 1");
  if (!std::isfinite(learning_rate)) return fail(GBDT_E_ARG, "learning_rate must be finite");
  const int64_t n = X->n_rows;
  if (n == 0) return GBDT_OK;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return fail(GBDT_E_ARG, "workspace is null or misaligned");
  WsCtrl* ctrl = reinterpret_cast<WsCtrl*>(static_cast<char*>(ws));
  const int64_t row_bytes = int64_t(X->n_blocks) * X->block_stride + X->bit_stride + X->nib_stride;
  if (row_bytes > kUpdMaxRowBytes) return fail(GBDT_E_UNSUPPORTED, "rows wider than 256 bytes");
  const WsLayout L = ws_layout(n, 1, 1);
  const size_t tables = size_t(max_nodes) * (sizeof(uint2) + sizeof(double));
  if (ws_bytes < L.total || tables > L.total - L.hpart)
    return fail(GBDT_E_ARG, "workspace too small for the tree tables");
  uint2* ctab = reinterpret_cast<uint2*>(static_cast<char*>(ws) + L.hpart);
  double* lval = reinterpret_cast<double*>(static_cast<char*>(ws) + L.hpart +
                                           sizeof(uint2) * size_t(max_nodes));
  // the node table goes to LDS (8 B per node); leaf values (by node) stay
  // in global memory (read once per row, after the walk)
  const size_t node_table = size_t(max_nodes) * sizeof(uint2);
  const bool in_lds = node_table <= kUpdTreeLds;
  const size_t lds = in_lds ? node_table : 0;
  const int64_t ndw = row_bytes / 4;
  const int rows = ndw <= 16 ? 2 : 1;
  int64_t grid = (n + int64_t(kUpdThreads) * rows - 1) / (int64_t(kUpdThreads) * rows);
  if (grid > 512) grid = 512;  // persistent: the tree is copied to LDS once per workgroup
  // byte blocks of 1..8 dwords: wide loads per block (one block of any
  // width within 8 row dwords, or several of 5..8 dwords whose blocks and
  // narrow words fit: the narrow words then start at dword (MAXDW / nd1) nd1)
  const int32_t nd1 = X->n_blocks >= 1 && (X->block_stride & 3) == 0 && X->block_stride >= 4 &&
                              X->block_stride <= 32 && (X->n_blocks == 1 || X->block_stride >= 20)
                          ? X->block_stride / 4
                          : 0;
  const int32_t nwords_all = (X->bit_stride + X->nib_stride) / 4;
  const int32_t maxdw_multi = ndw <= 16 ? 16 : 32;
  const bool multi = X->n_nib_features == 0 && !(ndw <= 8 && nd1 > 0) && ndw <= 32 && nd1 >= 5 &&
                     X->n_blocks * nd1 > 8 && X->n_blocks <= maxdw_multi / nd1 &&
                     nwords_all <= maxdw_multi - (maxdw_multi / nd1) * nd1;
  const int32_t word_base = multi ? (maxdw_multi / nd1) * nd1 : X->n_blocks * (X->block_stride / 4);
  diag_begin(kDiagUpdate, s);
  hipLaunchKernelGGL(k_compact_tree, dim3(1), dim3(1024), 0, s, nodes, n_nodes, max_nodes,
                     X->n_features, X->feature_col, X->n_blocks, X->block_features, X->block_stride,
                     X->n_bit_features, ctab, lval, driver ? n_nodes : nullptr, ctrl, X->bit_stride,
                     X->n_nib_features, word_base);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_compact_tree");
  diag_begin(kDiagUpdate, s);
  if (X->n_nib_features > 0) {  // a nibble block: the general row loads
    if (ndw <= 8)
      launch_update<8, 0, true>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval,
                                n_nodes, max_nodes, learning_rate, ctrl);
    else if (ndw <= 16)
      launch_update<16, 0, true>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval,
                                 n_nodes, max_nodes, learning_rate, ctrl);
    else if (ndw <= 32)
      launch_update<32, 0, true>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval,
                                 n_nodes, max_nodes, learning_rate, ctrl);
    else
      launch_update<64, 0, true>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval,
                                 n_nodes, max_nodes, learning_rate, ctrl);
  } else if (ndw <= 8 && nd1 > 0) {
    auto go = [&](auto tag) {
      launch_update<8, decltype(tag)::value>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X,
                                             ctab, lval, n_nodes, max_nodes, learning_rate, ctrl);
    };
    switch (nd1) {
      case 1: go(std::integral_constant<int, 1>()); break;
      case 2: go(std::integral_constant<int, 2>()); break;
      case 3: go(std::integral_constant<int, 3>()); break;
      case 4: go(std::integral_constant<int, 4>()); break;
      case 5: go(std::integral_constant<int, 5>()); break;
      case 6: go(std::integral_constant<int, 6>()); break;
      case 7: go(std::integral_constant<int, 7>()); break;
      default: go(std::integral_constant<int, 8>()); break;
    }
  } else if (multi) {
    auto go = [&](auto tag) {
      if (maxdw_multi == 16)
        launch_update<16, decltype(tag)::value>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n,
                                                X, ctab, lval, n_nodes, max_nodes, learning_rate, ctrl);
      else
        launch_update<32, decltype(tag)::value>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n,
                                                X, ctab, lval, n_nodes, max_nodes, learning_rate, ctrl);
    };
    switch (nd1) {
      case 5: go(std::integral_constant<int, 5>()); break;
      case 6: go(std::integral_constant<int, 6>()); break;
      case 7: go(std::integral_constant<int, 7>()); break;
      default: go(std::integral_constant<int, 8>()); break;
    }
  } else if (ndw <= 8)
    launch_update<8>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval, n_nodes,
                     max_nodes, learning_rate, ctrl);
  else if (ndw <= 16)
    launch_update<16>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval, n_nodes,
                      max_nodes, learning_rate, ctrl);
  else if (ndw <= 32)
    launch_update<32>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval, n_nodes,
                      max_nodes, learning_rate, ctrl);
  else
    launch_update<64>(in_lds, rows, dim3((unsigned)grid), lds, s, pred, n, X, ctab, lval, n_nodes,
                      max_nodes, learning_rate, ctrl);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_update");
  return GBDT_OK;
}

}  // namespace gbdt

extern "C" {

int gbdt_build_histograms(const gbdt_rows* src, const gbdt_features* ft, const gbdt_node* nodes,
                          const int32_t* list, const int32_t* list_len, int32_t list_cap,
                          int64_t rows_bound, int64_t* hist_g, uint32_t* hist_cnt, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!src || !ft || !nodes || !list || !list_len || !hist_g || !hist_cnt)
    return fail(GBDT_E_ARG, "null argument");
  int rc = check_hist_inputs(*src, *ft);
  if (rc) return rc;
  if (list_cap < 0 || rows_bound < 0) return fail(GBDT_E_ARG, "negative capacity");
  if (list_cap == 0) return GBDT_OK;
  const WsLayout L = ws_layout(src->X.n_rows, list_cap, ft->total_bins);
  rc = check_ws(ws, ws_bytes, L);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  WsCtrl* ctrl = reinterpret_cast<WsCtrl*>(w + L.ctrl);
  int32_t* hprefix = reinterpret_cast<int32_t*>(w + L.hprefix);
  int32_t* hmulti = reinterpret_cast<int32_t*>(w + L.hmulti);
  TileDesc* hdesc = reinterpret_cast<TileDesc*>(w + L.hdesc);
  uint64_t* hpart = reinterpret_cast<uint64_t*>(w + L.hpart);
  const int32_t gy = src->X.n_blocks + (src->X.n_bit_features > 0 ? 1 : 0) + (src->X.n_nib_features > 0 ? 1 : 0);
  const int32_t T = hist_tile_rows(
      rows_bound, src->X.n_rows, hist_target_tiles(gy, src->X.n_rows),
      hist_min_tile_rows(ft->total_bins, int64_t(src->X.n_blocks) * src->X.block_stride + src->X.bit_stride +
                                             src->X.nib_stride));
  const int64_t max_tiles = (rows_bound + T - 1) / T + list_cap;
  if (max_tiles > L.hpart_tiles) return fail(GBDT_E_SHAPE, "too many histogram tiles for the workspace");
  diag_begin(kDiagPlan, s);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, s, nodes, list, list_len, list_cap, T,
                     (int32_t)max_tiles, hprefix, hdesc, ctrl, (uint64_t*)nullptr,
                     (const gbdt_split*)nullptr, (const int32_t*)nullptr, 0, hmulti);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_plan");
  if (src->X.n_rows > 0) {
    const int64_t nq = src->X.n_rows;
    const int64_t q_bound = int64_t(1) << (52 - ceil_log2(nq));
    const int64_t gq = (nq + 255) / 256 < 1024 ? (nq + 255) / 256 : 1024;
    hipLaunchKernelGGL(k_check_q, dim3((unsigned)gq), dim3(256), 0, s, src->q, nq, q_bound, ctrl);
    GBDT_LAUNCH_CHECK("k_check_q");
  }
  rc = launch_hist(*src, *ft, hdesc, max_tiles, hist_g, hist_cnt, hpart, ctrl, s);
  if (rc) return rc;
  return launch_hist_reduce(hmulti, list_cap, max_tiles, src->X.n_rows,
                            ft->total_bins, hpart, hist_g, hist_cnt, s);
}

int gbdt_subtract_histograms(int64_t* hist_g, uint32_t* hist_cnt, int32_t total_bins,
                             const gbdt_pair* pairs, const int32_t* n_pairs, int32_t pair_cap,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!hist_g || !hist_cnt || !pairs || !n_pairs) return fail(GBDT_E_ARG, "null argument");
  if (total_bins < 1 || pair_cap < 0) return fail(GBDT_E_ARG, "bad size");
  if (pair_cap == 0) return GBDT_OK;
  const WsLayout L = ws_layout(1, 1, 1);
  if (!ws || ws_bytes < sizeof(WsCtrl)) return fail(GBDT_E_ARG, "workspace too small");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  WsCtrl* ctrl = reinterpret_cast<WsCtrl*>(static_cast<char*>(ws) + L.ctrl);
  int32_t gx = (total_bins + 255) / 256;
  if (gx > 64) gx = 64;
  diag_begin(kDiagSubtract, s);
  hipLaunchKernelGGL(k_subtract, dim3((unsigned)gx, (unsigned)pair_cap), dim3(256), 0, s, hist_g,
                     hist_cnt, total_bins, pairs, n_pairs, pair_cap, ctrl);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_subtract");
  return GBDT_OK;
}

int gbdt_find_best_splits(const int64_t* hist_g, const uint32_t* hist_cnt,
                          const gbdt_features* ft, const gbdt_node* nodes, const int32_t* list,
                          const int32_t* list_len, int32_t list_cap, const gbdt_params* p,
                          const int32_t* scale, gbdt_split* splits, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!hist_g || !hist_cnt || !ft || !nodes || !list || !list_len || !p || !scale || !splits)
    return fail(GBDT_E_ARG, "null argument");
  int rc = gbdt_validate_params(p);
  if (rc) return rc;
  if (ft->total_bins < 1 || !ft->bin_offset || !ft->bin_feature || !ft->n_bins)
    return fail(GBDT_E_ARG, "bad feature table");
  if (list_cap < 0) return fail(GBDT_E_ARG, "negative capacity");
  if (list_cap == 0) return GBDT_OK;
  // a workspace sized for list_cap entries and these bins holds the chunked
  // search's candidates; without one the search runs one workgroup per node
  FindCand* cand = nullptr;
  if (ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255) == 0) {
    const WsLayout L = ws_layout(1, list_cap, ft->total_bins);
    if (ws_bytes >= L.total) cand = reinterpret_cast<FindCand*>(static_cast<char*>(ws) + L.fcand);
  }
  // without the subtraction lists the kernel only reads the histograms
  return launch_find(const_cast<int64_t*>(hist_g), const_cast<uint32_t*>(hist_cnt), *ft, nodes, list,
                     list_len, list_cap, *p, scale, splits, nullptr, nullptr, nullptr,
                     reinterpret_cast<hipStream_t>(stream), cand);
}

int gbdt_partition_rows(const gbdt_rows* src, const gbdt_rows* dst, const gbdt_node* nodes,
                        const gbdt_split* splits, const int32_t* list, const int32_t* list_len,
                        int32_t list_cap, int64_t rows_bound, void* ws, size_t ws_bytes,
                        void* stream) {
  if (!src || !dst || !nodes || !splits || !list || !list_len) return fail(GBDT_E_ARG, "null argument");
  int rc = check_partition_inputs(*src, *dst);
  if (rc) return rc;
  if (list_cap < 0 || rows_bound < 0) return fail(GBDT_E_ARG, "negative capacity");
  if (list_cap == 0) return GBDT_OK;
  const WsLayout L = ws_layout(src->X.n_rows, list_cap, 1);
  rc = check_ws(ws, ws_bytes, L);
  if (rc) return rc;
  const int32_t ptr = part_tile_rows(src->X.n_rows, src->X.n_blocks, src->X.block_stride, false);
  const int64_t max_tiles = (rows_bound + ptr - 1) / ptr + list_cap;
  if (max_tiles > L.status_cap) return fail(GBDT_E_SHAPE, "too many partition tiles for the workspace");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  WsCtrl* ctrl = reinterpret_cast<WsCtrl*>(w + L.ctrl);
  int32_t* prefix = reinterpret_cast<int32_t*>(w + L.prefix);
  TileDesc* tdesc = reinterpret_cast<TileDesc*>(w + L.tdesc);
  uint64_t* status = reinterpret_cast<uint64_t*>(w + L.status);
  diag_begin(kDiagPlan, s);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, s, nodes, list, list_len, list_cap,
                     ptr, (int32_t)max_tiles, prefix, tdesc, ctrl, status, splits,
                     src->X.feature_col, src->X.n_features, (int32_t*)nullptr);
  diag_end(s);
  GBDT_LAUNCH_CHECK("k_plan");
  return launch_partition(*src, *dst, tdesc, status, ctrl, max_tiles, ptr, s);
}

int gbdt_update_predictions(double* pred, const gbdt_matrix* X, const gbdt_node* nodes,
                            const int32_t* n_nodes, int32_t max_nodes, double learning_rate,
                            void* ws, size_t ws_bytes, void* stream) {
  return gbdt::update_predictions(pred, X, nodes, const_cast<int32_t*>(n_nodes), max_nodes,
                                  learning_rate, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream),
                                  false);
}

}  // extern "C"
