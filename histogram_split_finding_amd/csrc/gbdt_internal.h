// Internal declarations shared by the HIP translation units of libgbdt.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "gbdt.h"

namespace gbdt {

// Split search over wide histograms: a node's features are cut into chunks
// (a feature belongs to the chunk of its first bin, chunks of kFindChunk
// bins), one workgroup per (node, chunk), and a merge picks each node's
// best chunk candidate.
constexpr int kFindChunk = 2048;
constexpr int kFindChunkMinBins = 4096;  // histograms of more bins take the chunked search
inline int32_t find_chunks(int32_t total_bins) {
  return total_bins > kFindChunkMinBins ? (total_bins + kFindChunk - 1) / kFindChunk : 1;
}
// The best candidate of one (node, chunk): gain and order key (0 = none).
struct FindCand {
  double gain;
  int32_t key, feature, threshold_bin, n_left;
  int64_t g_left;
  int64_t h_left;  // the logistic objective's left Hessian sum (0 otherwise)
};
static_assert(sizeof(FindCand) == 40, "candidate record is 40 bytes");

// Workspace layout.  Offsets are multiples of 256 bytes.
struct WsCtrl {
  int32_t err;          // first device-side error code (0 = none)
  int32_t err_detail;   // call-specific detail (e.g. offending node)
  uint32_t unused0;
  int32_t plan_total;   // tiles planned by the last planner launch
  int32_t pad[60];
};
static_assert(sizeof(WsCtrl) == 256, "control block is 256 bytes");

constexpr int kGradBlocks = 1024;     // grid of the gradient kernels
// A wave's SGPRs are allocated in blocks of 16 plus a fixed 16 from an
// 800-entry file per SIMD (measured on gfx950): kernels reporting at most 80
// SGPRs keep eight waves per SIMD, i.e. two 1024-thread workgroups per CU;
// 81 already drops a 1024-thread kernel to one workgroup per CU.
#define GBDT_SGPR_CAP __attribute__((amdgpu_num_sgpr(80)))
// Eight waves per SIMD (two 1024-thread workgroups per CU) also caps a
// wave at 64 VGPRs (512 per SIMD lane); the attribute makes the register
// allocator hold to that.
#define GBDT_TWO_GROUPS __attribute__((amdgpu_waves_per_eu(8, 8)))

constexpr int kPartTileRows = 2048;   // rows per partition tile (the smaller size; bounds use it)
constexpr int kPartTileRowsLarge = 4096;
constexpr int64_t kPartLargeRows = int64_t(1) << 22;  // matrices from this size take the larger tiles

// Whether the tree driver moves row ids instead of rows (index mode): for
// rows of two or more byte blocks, no narrow block, squared error.  Each
// level's partition then moves every row's id and q only (8 bytes each way
// instead of the whole row), and the histogram reads the rows of the
// original matrix through the ids; on 10M rows of 4 x 28 bytes a probe of
// the two patterns put a level at 0.2-0.5 ms against 0.6 ms for moving rows.
// One-block rows (28 bytes and less) move faster than they gather at all but
// the first levels, so they keep the row-moving partition.
inline bool grow_moves_ids(const gbdt_matrix& X, bool logistic) {
  return !logistic && X.n_blocks >= 2 && X.n_bit_features == 0 && X.n_nib_features == 0;
}

// Rows per partition tile for a matrix of n rows in n_blocks byte blocks of
// block_stride bytes whose q moves as int32 (q32) or int64: large matrices of
// one block of at most 28 bytes with int32 q take 4096-row tiles (four rows
// per thread, each loaded whole before the look-back), which halves the
// tiles, and so the look-back chain, of the 2048-row ones; wider rows or
// int64 q would take that kernel past the 64 registers of two workgroups per
// CU.  Small matrices keep more tiles than workgroup slots, and several
// blocks need the registers for double-buffering the blocks.
// In index mode (ids: only row ids and q move) every large matrix takes
// 8192-row tiles: the kernel holds no rows in registers, and fewer tiles
// shorten the look-back chains (10M x 100: 3.88 -> 3.75 -> 3.68 ms per tree
// from 2048- to 4096- to 8192-row tiles).
constexpr int kPartTileRowsIds = 8192;
// Two-level partitions (four) take the 4096-row tiles only when every split
// byte is in the one block they hold in registers (no narrow block).
inline int32_t part_tile_rows(int64_t n_rows, int32_t n_blocks, int32_t block_stride, bool q32,
                              bool ids = false, bool four = false, bool narrow = false) {
  if (ids) return n_rows < kPartLargeRows ? kPartTileRows : kPartTileRowsIds;
  if (n_rows < kPartLargeRows || n_blocks > 1 || block_stride > 28 || !q32) return kPartTileRows;
  if (four && (narrow || n_blocks < 1)) return kPartTileRows;
  return kPartTileRowsLarge;
}
constexpr int kHistMinTileRows = 1024;
constexpr int kHistTargetTiles = 1024;    // workgroups per histogram launch to aim for
constexpr int kHistMinTargetTiles = 128;
constexpr int kReduceNodeSlots = 64;  // multi-tile nodes the partial-reduction grid covers at once
constexpr int kReduceGrid = 512;      // at most this many reduction workgroups
constexpr int kLdsHistBudgetBins = 8192;  // LDS slots (8 bytes) of one histogram workgroup: 64 KiB
constexpr int kHistRowSlots = 32;          // LDS slots per bin row of a byte block's histogram
constexpr int kHistMaxBlockStride = 32;    // bytes per row of a byte block, at most (8 dwords)
constexpr int kNibSlots = 16;              // LDS slots per feature of the nibble block's histogram

// Work assignment of one tile (written by the planner).  A partition plan
// also carries the node's split, so a partition tile needs no second load.
// A two-level (4-way) partition plan has one entry per grandparent g: its
// segment and split, and the splits of its children a (left) and b (right),
// each packed as (matrix column << 8) | threshold_bin, or -1 when that child
// does not split; n2 (n3) is the number of a's (b's) rows that go to a's
// (b's) left child, all of a's (b's) rows when it does not split.
struct TileDesc {
  int32_t node;    // node id
  int32_t r0, r1;  // rows [r0, r1) of the tile
  int32_t ntiles;  // tiles of the node
  int32_t tfirst;  // first tile of the node
  int32_t slot;    // the tile's index in its plan: histogram plans launch largest tiles
                   // first, and a tile's partial lives at this index
  int32_t begin;   // the node's segment
  int32_t count;
  int32_t feature;        // partition plans: the node's split
  int32_t threshold_bin;
  int32_t n_left;
  int32_t split_valid;
  int32_t split2, n2;     // two-level partition plans: child a's split and left rows
  int32_t split3, n3;     // child b's
};
static_assert(sizeof(TileDesc) == 64, "tile descriptor is 64 bytes");

// One entry of a partition plan as the level kernel stages it: the node,
// its segment and its split (the feature as its matrix column).
struct PlanEntry {
  int32_t node, begin, count, feature, threshold_bin, n_left;
};

// Two tile plans live in the workspace at once: the partition plan
// (tdesc, prefix, status, ctrl->plan_total) and the histogram plan
// (hdesc, hprefix), so the level kernel of the tree driver can write this
// level's partition plan and the next level's histogram plan together.
struct WsLayout {
  size_t ctrl;        // WsCtrl
  size_t tdesc;       // TileDesc[tdesc_cap]: partition plan
  size_t hdesc;       // TileDesc[hpart_tiles]: histogram plan
  size_t gpart;       // double[kGradBlocks] maxima, then int64[kGradBlocks] sums; the
                      // logistic objective's Hessian maxima and sums follow
  size_t prefix;      // int32[max_list + 2]: partition plan
  size_t hprefix;     // int32[max_list + 2]: histogram plan
  size_t hmulti;      // int32[4 + 4 (max_list + 2)]: histogram plan, nodes of several tiles:
                      // the count, then (node, first tile, end tile, list position) each
  size_t fcand;       // FindCand[max_list * find_chunks]: split search, best per chunk
  size_t status;      // uint64[status_cap]
  size_t status2;     // uint64[status_cap]: the second look-back of two-level partitions
  size_t gstage;      // PlanEntry[max_list]: a level's splitting nodes, for the two-level
                      // partition planned one level later
  size_t hpart;       // uint64[hpart_tiles * total_bins]
  size_t total;
  int64_t status_cap;
  int64_t hpart_tiles;
  int64_t tdesc_cap;
};

WsLayout ws_layout(int64_t n_rows, int32_t max_list, int32_t total_bins);

// Error plumbing (thread-local text).
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);

inline int32_t ceil_log2(int64_t n) {
  int32_t L = 0;
  while ((int64_t(1) << L) < n) ++L;
  return L;
}

// Fixed-point packing of one histogram cell in LDS: (q << bits) + 1, so the
// low `bits` bits count rows and the rest sums q.  Exact while a tile holds
// fewer than 2^bits rows and 2*bits + 52 - ceil(log2 n) <= 63.
inline int32_t pack_bits_for(int64_t n_rows) {
  int32_t L = ceil_log2(n_rows < 1 ? 1 : n_rows);
  int32_t b = (11 + L) / 2;
  if (b > 24) b = 24;
  return b;
}

int32_t hist_tile_rows(int64_t rows_bound, int64_t n_rows, int32_t target, int32_t min_rows);

// Fewest rows of a histogram tile for a layout of row_bytes bytes per row
// (all column blocks) and total_bins bins: a tile's rows should carry at
// least as many bytes as the packed partial it may write (8 bytes per bin),
// between kHistMinTileRows and 8192 rows (1M x 32 columns of 256 bins: 2048
// rows per tile, 2346 -> 2464 trees/s).
inline int32_t hist_min_tile_rows(int64_t total_bins, int64_t row_bytes) {
  const int64_t t = row_bytes > 0 ? (8 * total_bins) / row_bytes : kHistMinTileRows;
  return int32_t(t < kHistMinTileRows ? kHistMinTileRows : (t > 8192 ? 8192 : t));
}

// Histogram tiles per launch to aim for: about kHistTargetTiles workgroups
// over the tile x column-block grid (gy blocks) for matrices of n_rows >=
// kPartLargeRows, a quarter of that below (fewer, longer tiles: less partial
// output and reduction per level where levels are latency-bound; the
// covtype-shaped depth-10 tree 432 -> 423 us, 1M x 32 324 -> 321 us, while
// 10M x 100 and 50M x 28 lose 2-4 % with the smaller target), and at least
// kHistMinTargetTiles tiles.
inline int32_t hist_target_tiles(int32_t gy, int64_t n_rows) {
  const int32_t base = n_rows < kPartLargeRows ? kHistTargetTiles / 4 : kHistTargetTiles;
  const int32_t t = base / (gy < 1 ? 1 : gy);
  return t < kHistMinTargetTiles ? kHistMinTargetTiles : t;
}

// Most rows one histogram tile may hold for n rows: the packed LDS cells
// count a tile's rows in `bits` bits.
inline int32_t hist_tile_max(int64_t n_rows) {
  return int32_t((int64_t(1) << pack_bits_for(n_rows < 1 ? 1 : n_rows)) - 1);
}

// Histogram tile rows for a level that builds `rows` rows (device and host):
// about `target` tiles of equal size, at least min(min_rows, tile_max) rows
// and at most tile_max.  A node's last tile is partial, so a level has at
// most target + nodes tiles; the plan launches them largest first.
__host__ __device__ inline int32_t hist_tile_rows_for(int32_t rows, int32_t tile_max, int32_t target,
                                                      int32_t min_rows) {
  int32_t t = (rows + target - 1) / target;
  const int32_t lo = min_rows < tile_max ? min_rows : tile_max;
  if (t < lo) t = lo;
  if (t > tile_max) t = tile_max;
  return t < 1 ? 1 : t;
}

// Argument checks and launches shared by the per-call entry points and the
// tree driver (the driver's level kernel writes the tile plans itself).
bool same_layout(const gbdt_matrix& a, const gbdt_matrix& b);
int check_matrix(const gbdt_matrix& X);
int check_hist_inputs(const gbdt_rows& src, const gbdt_features& ft);
int check_partition_inputs(const gbdt_rows& src, const gbdt_rows& dst);
// Whether the tree driver moves rows only after every second level: in
// row-moving mode, for depths 2 to 12 (the level kernel then plans every
// filtered and two-level plan in one pass).  The odd levels' histograms are
// then built from the parents' unpartitioned rows (filtered tiles), and a
// two-level partition follows each odd level but the last.
inline bool grow_alternates(bool moves_ids, int32_t max_depth) {
  return !moves_ids && max_depth >= 2 && max_depth <= 12;
}

// Row pitch in bytes of index mode's row-interleaved copy: the row's
// n_blocks * block_stride bytes rounded up to a power of two up to 128 (so no
// row straddles a 128-byte cache line), else to a multiple of 128.
inline int32_t interleave_pitch(const gbdt_matrix& X) {
  const int32_t p = X.n_blocks * X.block_stride;
  if (p > 128) return (p + 127) / 128 * 128;
  int32_t q = 4;
  while (q < p) q *= 2;
  return q;
}

// q32: src.q holds int32 elements (the tree driver's row buffers, see
// driver_q32); otherwise int64 as the ABI declares.  ids (index mode, byte
// blocks only): a tile's rows are the rows src.rid names (their q in src.q
// at the tile's positions), read from the matrix src.X, or from rows_ix, its
// byte blocks interleaved row by row, when that is not NULL.  filt: the
// plan's tiles are filtered (each reads rows of a parent's segment and keeps
// those going to the child it builds; rows in order only).
int launch_hist(const gbdt_rows& src, const gbdt_features& ft, const TileDesc* desc,
                int64_t max_tiles, int64_t* hist_g, uint32_t* hist_cnt, uint64_t* hpart,
                WsCtrl* ctrl, hipStream_t s, bool q32 = false, bool guard = false, bool ids = false,
                const uint8_t* rows_ix = nullptr, bool filt = false);
int launch_hist_reduce(const int32_t* multi, int32_t list_cap, int64_t max_tiles, int64_t n_rows,
                       int32_t total_bins, const uint64_t* hpart, int64_t* hist_g,
                       uint32_t* hist_cnt, hipStream_t s, const int32_t* guard = nullptr);
// hist_h / scale_h / split_h: the logistic objective's Hessian histograms,
// grid and per-split left Hessian sums (nullptr for squared error, H = count).
int launch_find(int64_t* hist_g, uint32_t* hist_cnt, const gbdt_features& ft, const gbdt_node* nodes,
                const int32_t* list, const int32_t* list_len, int32_t list_cap, const gbdt_params& p,
                const int32_t* scale, gbdt_split* splits, const int32_t* sub_par,
                const int32_t* sub_sib, WsCtrl* ctrl, hipStream_t s, FindCand* cand = nullptr,
                const int32_t* guard = nullptr, int64_t* hist_h = nullptr,
                const int32_t* scale_h = nullptr, int64_t* split_h = nullptr);
// qin32 / qout32: src.q / dst.q hold int32 elements (the tree driver's row
// buffers); otherwise int64.  ids (index mode, byte blocks only): only each
// position's row id (src.rid, NULL = the position itself) and q move, into
// dst.rid and dst.q; the split byte is read from the matrix src.X at the row
// id, from cols, the matrix's byte columns one after another, when that is
// not NULL.  four: a two-level plan (one entry per grandparent, its
// children's splits in the descriptors), whose second look-back runs over
// status2; row-moving only.
int launch_partition(const gbdt_rows& src, const gbdt_rows& dst, const TileDesc* desc,
                     uint64_t* status, WsCtrl* ctrl, int64_t max_tiles, int32_t tile_rows,
                     hipStream_t s, bool qin32 = false, bool qout32 = false, bool ids = false,
                     const uint8_t* cols = nullptr, bool four = false, uint64_t* status2 = nullptr);

// Blocks of the gradient kernels for n rows: each leaves a partial max |g|
// and a partial sum of q in the workspace (gpart).
inline int32_t grad_blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return int32_t(b < kGradBlocks ? b : kGradBlocks);
}
// Gradients and the fixed-point grid (gbdt_compute_gradients); q32: q gets
// int32 elements (the tree driver, ceil(log2 n) >= 22), otherwise int64.
// part: the workspace's gpart region (partial maxima, then partial sums).
// With gsum == nullptr the sum of q is left as grad_blocks(n) partial sums
// at part + kGradBlocks (the tree driver adds them up itself).
int launch_gradients(const double* pred, const float* label, int64_t n, void* q, bool q32,
                     int32_t* scale, int64_t* gsum, double* part, WsCtrl* ctrl, hipStream_t s);
// The logistic objective's gradients and Hessians (int32 each, see gbdt.h):
// part as above with the Hessian maxima at part + 2 kGradBlocks and their
// per-block sums after them; the sums stay as per-block partials.
int launch_gradients_logistic(const double* pred, const float* label, int64_t n, int32_t* q,
                              int32_t* qh, int32_t* scale, int32_t* scale_h, double* part,
                              WsCtrl* ctrl, hipStream_t s);

// Whether the tree driver stores q as int32 (in its original-order buffer and
// its two row buffers): exact when every |q| <= 2^(52 - ceil(log2 n)) fits 31
// bits, i.e. n > 2^21 rows (|q| <= 2^30); it saves 4 of 8 bytes per row in
// every histogram and every partition.
inline bool driver_q32(int64_t n_rows) { return ceil_log2(n_rows) >= 22; }

// Step 7 (gbdt_update_predictions).  driver: the tree driver's mode -- the
// update does nothing once the workspace error word is set, and the tree's
// node count (n_nodes, device) is set to 0 when the word is set or a node of
// the tree fails the structure check, so no failed tree is exported and no
// prediction moves.
int update_predictions(double* pred, const gbdt_matrix* X, const gbdt_node* nodes,
                       int32_t* n_nodes, int32_t max_nodes, double learning_rate, void* ws,
                       size_t ws_bytes, hipStream_t s, bool driver);

// Per-kernel device timing (the backend's diagnostics): when enabled, every
// launch of the library is bracketed by two hipEvents on its stream.
enum DiagKind {
  kDiagGradMax = 1, kDiagGradQ, kDiagPlan, kDiagHist, kDiagHistReduce, kDiagSubtract, kDiagFind,
  kDiagTreeInit, kDiagLevel, kDiagPartition, kDiagUpdate, kDiagPack, kDiagBin, kDiagPredict,
  kDiagBounds
};
void diag_begin(int kind, hipStream_t s);
void diag_end(hipStream_t s);

}  // namespace gbdt
