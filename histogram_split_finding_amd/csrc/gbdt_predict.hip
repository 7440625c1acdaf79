// Ensemble forward pass over a binned matrix: "Gradient boosted trees (spec
// model)", section Forward pass.  Each tree is traversed from its root (a row
// goes left when its bin of the node's feature is <= the node's threshold
// bin, the routing of "Module Design: Training Core", section 3) to a leaf;
// the ensemble adds the learning rate times each tree's leaf value to the
// initial prediction, tree by tree in order, one rounding per product and
// per sum -- the sequence step 7 of the Tree Growth section applies during
// training, so training rows get their training-time predictions bit for
// bit.
//
// Two kernels.  k_compact_ensemble (one workgroup per tree) checks every
// node and writes an 8-byte table entry per node (left child or leaf tag;
// where the split feature's bin sits in a row's dwords, and the threshold)
// plus the leaf values, both at the node's own index.  k_predict walks the
// rows: a launch takes a run of trees whose tables fit LDS together (64 KiB,
// 8192 entries), copies them there once per workgroup, and each lane loads
// its row's dwords once and walks every tree of the run in order,
// accumulating the prediction in a register; the prediction is read (or
// started from the base score) and written once per launch.  Trees larger
// than LDS are walked from the global table.

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>

#include "gbdt.h"
#include "gbdt_device.h"
#include "gbdt_internal.h"

#pragma clang fp contract(off)

namespace gbdt {

namespace {

constexpr int kPredThreads = 1024;
constexpr int kPredMaxRowBytes = 256;
constexpr int64_t kPredLdsEntries = 8192;  // 64 KiB of 8-byte table entries
constexpr uint32_t kPLeaf = 0x80000000u;
constexpr uint32_t kPBad = 0x40000000u;

// One workgroup per tree t: entry v of the tree at ctab[t * stride + v], its
// leaf value (leaves only) at lval[t * stride + v].  A node is accepted when
// it is a leaf, or a split whose children are right = left + 1, both after it
// and below the tree's node count, one level deeper than it (root depth 0,
// at most GBDT_MAX_DEPTH), and whose feature exists: then every walk reaches
// a leaf within GBDT_MAX_DEPTH steps.  Otherwise GBDT_E_ARG is recorded.
__global__ void __launch_bounds__(256) k_compact_ensemble(
    const gbdt_node* __restrict__ trees, const int32_t* __restrict__ n_nodes, int32_t stride,
    int32_t n_features, const int32_t* __restrict__ feature_col, int32_t n_blocks,
    int32_t block_features, int32_t block_stride, int32_t n_bit, uint2* __restrict__ ctab,
    double* __restrict__ lval, WsCtrl* __restrict__ ctrl, int32_t bit_stride, int32_t n_nib) {
  const int32_t t = blockIdx.x;
  const gbdt_node* __restrict__ tree = trees + int64_t(t) * stride;
  const int32_t nn = n_nodes[t];
  bool bad = nn < 1 || nn > stride || tree[0].depth != 0;
  const int32_t nbc = n_features - n_bit;  // the first bit column
  const int32_t nbyte = nbc - n_nib;       // the first nibble column
  for (int32_t v = threadIdx.x; v < (nn > 0 && nn <= stride ? nn : 0); v += blockDim.x) {
    const gbdt_node nd = tree[v];
    uint2 e;
    e.y = 0u;
    if (nd.flags & GBDT_NODE_LEAF) {
      e.x = kPLeaf | (uint32_t)v;
      lval[int64_t(t) * stride + v] = nd.leaf_value;
    } else {
      const bool kids = nd.left > v && nd.left + 1 < nn && nd.right == nd.left + 1;
      const bool deep = kids && nd.depth >= 0 && nd.depth < GBDT_MAX_DEPTH &&
                        tree[nd.left].depth == nd.depth + 1 && tree[nd.right].depth == nd.depth + 1;
      const int32_t c = (nd.feature >= 0 && nd.feature < n_features)
                            ? (feature_col != nullptr ? feature_col[nd.feature] : nd.feature)
                            : -1;
      if (!deep || c < 0 || c >= n_features || nd.threshold_bin < 0 || nd.threshold_bin > 0xffff) {
        e.x = kPBad;
        bad = true;
      } else {
        uint32_t loc;
        if (c < nbyte) {
          const int32_t blk = c / block_features;
          const int32_t byte = blk * block_stride + (c - blk * block_features);
          loc = (uint32_t)(byte >> 2) | ((uint32_t)(8 * (byte & 3)) << 6);
        } else if (c < nbc) {  // a nibble, after the bit words in the row's dwords
          const int32_t kk = c - nbyte;
          loc = (uint32_t)(n_blocks * (block_stride >> 2) + (bit_stride >> 2) + (kk >> 3)) |
                ((uint32_t)(4 * (kk & 7)) << 6) | (2u << 11);
        } else {
          const int32_t kk = c - nbc;
          loc = (uint32_t)(n_blocks * (block_stride >> 2) + (kk >> 5)) | ((uint32_t)(kk & 31) << 6) |
                (1u << 11);
        }
        e.x = (uint32_t)nd.left;
        e.y = loc | ((uint32_t)nd.threshold_bin << 16);
      }
    }
    ctab[int64_t(t) * stride + v] = e;
  }
  if (bad) dev_error(&ctrl->err, GBDT_E_ARG);
}

// Row i's dwords: byte block b's run of block_stride / 4 dwords for each b in
// turn, then the bit words, then the nibble words; entries past them are 0.
// The loads are unconditional (uniform pointer selects), so all are in flight
// together.
template <int MAXDW>
__device__ __forceinline__ void load_row(const uint8_t* __restrict__ bins, int64_t i,
                                         int64_t row_capacity, int32_t block_stride, int32_t ndw,
                                         int32_t nwords, const uint32_t* __restrict__ bitw,
                                         int32_t nnw, const uint32_t* __restrict__ nibw,
                                         uint32_t (&row)[MAXDW]) {
  const int32_t dw = block_stride >> 2;
  const uint32_t* __restrict__ bp = reinterpret_cast<const uint32_t*>(bins + i * block_stride);
  const uint32_t* __restrict__ wp = bitw + i * nwords;
  const uint32_t* __restrict__ np = nibw + i * nnw;
  int32_t xb = 0;
  int64_t boff = 0;
#pragma unroll
  for (int x = 0; x < MAXDW; ++x) {
    const bool in_bytes = x < ndw;
    const bool in_bits = !in_bytes && x < ndw + nwords;
    const bool in_nibs = !in_bytes && !in_bits && x < ndw + nwords + nnw;
    const uint32_t* p =
        in_bytes ? bp + boff + xb : (in_bits ? wp + (x - ndw) : (in_nibs ? np + (x - ndw - nwords) : bp));
    const uint32_t val = *p;
    row[x] = (in_bytes || in_bits || in_nibs) ? val : 0u;
    if (in_bytes && ++xb == dw) {
      xb = 0;
      boff += (row_capacity * block_stride) >> 2;
    }
  }
}

// Trees [t0, t1) for every row: out[i] = (started ? out[i] : base) + eta*w
// for each tree in order.
template <int MAXDW, bool IN_LDS>
__global__ void __launch_bounds__(kPredThreads) k_predict(
    double* __restrict__ out, int64_t n, const uint8_t* __restrict__ bins, int64_t row_capacity,
    int32_t n_blocks, int32_t block_stride, int32_t bit_stride, const uint2* __restrict__ ctab_g,
    const double* __restrict__ lval, int32_t t0, int32_t t1, int32_t stride, double base,
    int32_t started, double eta, const int32_t* __restrict__ guard, int32_t nib_stride) {
  static_assert((MAXDW & (MAXDW - 1)) == 0, "MAXDW is a power of two");
  extern __shared__ uint64_t smem[];
  if (failed(guard)) return;
  const uint2* ctab = ctab_g + int64_t(t0) * stride;
  if (IN_LDS) {
    uint2* ct = reinterpret_cast<uint2*>(smem);
    const int32_t m = (t1 - t0) * stride;
    for (int32_t v = threadIdx.x; v < m; v += kPredThreads) ct[v] = ctab[v];
    __syncthreads();
    ctab = ct;
  }
  const int32_t ndw = n_blocks * (block_stride >> 2);
  const int32_t nwords = bit_stride >> 2;
  const int32_t nnw = nib_stride >> 2;
  const uint32_t* __restrict__ bitw =
      reinterpret_cast<const uint32_t*>(bins + int64_t(n_blocks) * row_capacity * block_stride);
  const uint32_t* __restrict__ nibw = bitw + row_capacity * nwords;
  const int64_t gstride = int64_t(gridDim.x) * kPredThreads;
  for (int64_t i0 = int64_t(blockIdx.x) * kPredThreads + threadIdx.x; i0 - threadIdx.x < n;
       i0 += gstride) {
    const bool live = i0 < n;
    const int64_t i = live ? i0 : n - 1;  // a valid row: the loads need no branch
    uint32_t row[MAXDW];
    load_row<MAXDW>(bins, i, row_capacity, block_stride, ndw, nwords, bitw, nnw, nibw, row);
    double pv = started ? out[i] : base;
    for (int32_t t = 0; t < t1 - t0; ++t) {
      const uint2* __restrict__ tab = ctab + int64_t(t) * stride;
      int32_t v = 0;
      uint32_t fin = 0u;  // the leaf's entry once reached
      // every accepted tree ends its walks within GBDT_MAX_DEPTH steps
      for (int step = 0; step <= GBDT_MAX_DEPTH; ++step) {
        const uint2 e = tab[v];
        const bool leaf = (e.x & kPLeaf) != 0u;
        uint32_t s[MAXDW];
#pragma unroll
        for (int x = 0; x < MAXDW; ++x) s[x] = row[x];
        const uint32_t kk = e.y & 63u;
#pragma unroll
        for (int lvl = 0, w = MAXDW; w > 1; ++lvl, w >>= 1) {
          const bool hi = (kk >> lvl) & 1u;
#pragma unroll
          for (int x = 0; x < w / 2; ++x) s[x] = hi ? s[2 * x + 1] : s[2 * x];
        }
        const uint32_t shift = (e.y >> 6) & 31u;
        const uint32_t wcode = (e.y >> 11) & 3u;  // 0 byte, 1 bit, 2 nibble
        const uint32_t vmask = wcode == 1u ? 1u : (wcode == 2u ? 15u : 0xffu);
        const uint32_t bv = (s[0] >> shift) & vmask;
        const int32_t next = (int32_t)e.x + (bv <= (e.y >> 16) ? 0 : 1);
        const bool moving = fin == 0u && !leaf;
        fin = fin != 0u ? fin : (leaf ? e.x : 0u);
        v = moving ? next : v;
        if (!__any(moving)) break;
      }
      const double term = eta * lval[(int64_t(t0) + t) * stride + (fin & ~kPLeaf)];
      pv = pv + term;
    }
    if (live) out[i] = pv;
  }
}

template <int MAXDW>
void launch_predict(bool in_lds, dim3 grid, size_t lds, hipStream_t s, double* out, int64_t n,
                    const gbdt_matrix& X, const uint2* ctab, const double* lval, int32_t t0, int32_t t1,
                    int32_t stride, double base, int32_t started, double eta, const int32_t* guard) {
  auto kern = in_lds ? k_predict<MAXDW, true> : k_predict<MAXDW, false>;
  hipLaunchKernelGGL(kern, grid, dim3(kPredThreads), lds, s, out, n, X.bins, X.row_capacity,
                     X.n_blocks, X.block_stride, X.bit_stride, ctab, lval, t0, t1, stride, base,
                     started, eta, guard, X.nib_stride);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Scratch of gbdt_predict_noalloc, for callers that cannot allocate: the
// control block (error word), the compact tables and the leaf values of one
// call, at most kNoAllocBytes.  Every GPU the library runs on holds its own
// copy until the process ends.  Host code never uses this name as an
// address: it takes each device's address from hipGetSymbolAddress once.
constexpr size_t kNoAllocBytes = size_t(16) << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch's address on the current device (looked up on the first call
// on that device).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GBDT_E_UNSUPPORTED, "device index beyond 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(GBDT_E_DEVICE, "scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GBDT_OK;
}

// The control block starts each call at zero (a kernel, not a memset node,
// so the call can be captured into a graph), and the call's error word is
// copied to the caller's status at its end.
__global__ void __launch_bounds__(64) k_clear_ctrl(WsCtrl* __restrict__ ctrl) {
  reinterpret_cast<int32_t*>(ctrl)[threadIdx.x] = 0;
}
__global__ void __launch_bounds__(64) k_copy_status(const WsCtrl* __restrict__ ctrl,
                                                    int32_t* __restrict__ status) {
  if (threadIdx.x == 0) *status = ctrl->err;
}

int predict_impl(const gbdt_matrix* X, const gbdt_node* trees, const int32_t* n_nodes,
                 int32_t n_trees, int32_t tree_stride, double base_score, double learning_rate,
                 double* out, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace

}  // namespace gbdt

using namespace gbdt;

extern "C" {

size_t gbdt_predict_workspace_bytes(int32_t n_trees, int32_t tree_stride) {
  if (n_trees < 0 || tree_stride < 1) return 0;
  const size_t m = size_t(n_trees) * size_t(tree_stride);
  return sizeof(WsCtrl) + align256(m * sizeof(uint2)) + align256(m * sizeof(double));
}

int gbdt_predict(const gbdt_matrix* X, const gbdt_node* trees, const int32_t* n_nodes,
                 int32_t n_trees, int32_t tree_stride, double base_score, double learning_rate,
                 double* out, void* ws, size_t ws_bytes, void* stream) {
  return predict_impl(X, trees, n_nodes, n_trees, tree_stride, base_score, learning_rate, out, ws,
                      ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

int gbdt_predict_noalloc(const gbdt_matrix* X, const gbdt_node* trees, const int32_t* n_nodes,
                         int32_t n_trees, int32_t tree_stride, double base_score,
                         double learning_rate, double* out, int32_t* status, void* stream) {
  if (!status) return fail(GBDT_E_ARG, "status is null");
  if (n_trees < 0 || tree_stride < 1) return fail(GBDT_E_ARG, "n_trees or tree_stride out of range");
  const size_t need = gbdt_predict_workspace_bytes(n_trees, tree_stride);
  if (need > kNoAllocBytes)
    return fail(GBDT_E_ARG, "n_trees * tree_stride needs " + std::to_string(need) +
                                " bytes of scratch; gbdt_predict_noalloc holds " +
                                std::to_string(kNoAllocBytes) + " (use gbdt_predict with a workspace)");
  void* ws = nullptr;
  int rc = scratch_ptr(&ws);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  WsCtrl* ctrl = static_cast<WsCtrl*>(ws);
  hipLaunchKernelGGL(k_clear_ctrl, dim3(1), dim3(64), 0, s, ctrl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "k_clear_ctrl");
  rc = predict_impl(X, trees, n_nodes, n_trees, tree_stride, base_score, learning_rate, out, ws,
                    kNoAllocBytes, s);
  if (rc) return rc;
  hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(64), 0, s, ctrl, status);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "k_copy_status");
  return GBDT_OK;
}

}  // extern "C"

namespace gbdt {
namespace {

int predict_impl(const gbdt_matrix* X, const gbdt_node* trees, const int32_t* n_nodes,
                 int32_t n_trees, int32_t tree_stride, double base_score, double learning_rate,
                 double* out, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!X) return fail(GBDT_E_ARG, "X is null");
  int rc = check_matrix(*X);
  if (rc) return rc;
  if (n_trees < 0 || tree_stride < 1 || tree_stride > (1 << 24))
    return fail(GBDT_E_ARG, "n_trees or tree_stride out of range");
  if (n_trees > 0 && (!trees || !n_nodes)) return fail(GBDT_E_ARG, "trees or n_nodes is null");
  if (!std::isfinite(base_score) || !std::isfinite(learning_rate))
    return fail(GBDT_E_ARG, "base_score and learning_rate must be finite");
  const int64_t n = X->n_rows;
  if (n == 0) return GBDT_OK;
  if (!out) return fail(GBDT_E_ARG, "out is null");
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255)) return fail(GBDT_E_ARG, "workspace is null or misaligned");
  if (ws_bytes < gbdt_predict_workspace_bytes(n_trees, tree_stride))
    return fail(GBDT_E_ARG, "workspace smaller than gbdt_predict_workspace_bytes()");
  const int64_t row_bytes = int64_t(X->n_blocks) * X->block_stride + X->bit_stride + X->nib_stride;
  if (row_bytes > kPredMaxRowBytes) return fail(GBDT_E_UNSUPPORTED, "rows wider than 256 bytes");
  char* w = static_cast<char*>(ws);
  WsCtrl* ctrl = reinterpret_cast<WsCtrl*>(w);
  const size_t m = size_t(n_trees) * size_t(tree_stride);
  uint2* ctab = reinterpret_cast<uint2*>(w + sizeof(WsCtrl));
  double* lval = reinterpret_cast<double*>(w + sizeof(WsCtrl) + align256(m * sizeof(uint2)));
  if (n_trees > 0) {
    diag_begin(kDiagPredict, s);
    hipLaunchKernelGGL(k_compact_ensemble, dim3((unsigned)n_trees), dim3(256), 0, s, trees, n_nodes,
                       tree_stride, X->n_features, X->feature_col, X->n_blocks, X->block_features,
                       X->block_stride, X->n_bit_features, ctab, lval, ctrl, X->bit_stride,
                       X->n_nib_features);
    diag_end(s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "k_compact_ensemble");
  }
  // runs of trees whose tables fit LDS together; one launch per run (with no
  // trees, one launch writes the base score)
  const bool in_lds = tree_stride <= kPredLdsEntries;
  const int32_t per = in_lds ? int32_t(kPredLdsEntries / tree_stride) : 1;
  int64_t grid = (n + kPredThreads - 1) / kPredThreads;
  if (grid > 512) grid = 512;  // persistent: the tables are copied to LDS once per workgroup
  const int64_t ndw = row_bytes / 4;
  const int32_t* guard = &ctrl->err;
  int32_t t0 = 0;
  do {
    const int32_t t1 = n_trees - t0 < per ? n_trees : t0 + per;
    const size_t lds = in_lds ? size_t(t1 - t0) * tree_stride * sizeof(uint2) : 0;
    diag_begin(kDiagPredict, s);
    if (ndw <= 8)
      launch_predict<8>(in_lds, dim3((unsigned)grid), lds, s, out, n, *X, ctab, lval, t0, t1, tree_stride,
                        base_score, t0 > 0, learning_rate, guard);
    else if (ndw <= 16)
      launch_predict<16>(in_lds, dim3((unsigned)grid), lds, s, out, n, *X, ctab, lval, t0, t1,
                         tree_stride, base_score, t0 > 0, learning_rate, guard);
    else if (ndw <= 32)
      launch_predict<32>(in_lds, dim3((unsigned)grid), lds, s, out, n, *X, ctab, lval, t0, t1,
                         tree_stride, base_score, t0 > 0, learning_rate, guard);
    else
      launch_predict<64>(in_lds, dim3((unsigned)grid), lds, s, out, n, *X, ctab, lval, t0, t1,
                         tree_stride, base_score, t0 > 0, learning_rate, guard);
    diag_end(s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "k_predict");
    t0 = t1;
  } while (t0 < n_trees);
  return GBDT_OK;
}

}  // namespace
}  // namespace gbdt
