/*
 * gbdt.h -- C ABI of the MI355X (gfx950) level-wise histogram GBDT hot path
 * for squared-error boosting, with the sigmoid cross-entropy (logistic)
 * objective as a second one in the tree driver.
 *
 * What the calls compute is fixed by "Module Design: Training Core"
 * (MPSBoost spec):
 *   section 2 (Single Mathematical Semantics): g_i = prediction_i - label_i,
 *     h_i = 1, score(G,H) = G^2/(H+lambda), weight(G,H) = -G/(H+lambda),
 *     gain = 0.5*(score_left + score_right - score_parent) - gamma;
 *   section 3 (Tree Model): flat node array, stable tie-break (larger gain,
 *     then smaller feature, then smaller threshold bin, then the first
 *     candidate) on strict FP64 '>', strictly positive gain, bin <=
 *     threshold_bin goes left, parameter and child constraints;
 *   section 4 (Backend Interface): POD views and preallocated outputs, the
 *     caller decides when, the library decides how;
 *   section 6 (Tree Growth): the seven level-wise steps;
 *   section 7 (CPU Oracle): no hidden CPU fallback -- a call that cannot run
 *     on the GPU returns an error.
 * The per-level batching (one launch per level for all nodes, smaller child
 * built and larger child obtained by subtraction) follows the idea of the
 * ExaBoost PR "[cuda] hybrid level-batched tree growth" (its batched
 * construct / subtract / find / sync and batched apply commits); the kernels
 * are written for gfx950 from that description, not ported.
 *
 * Fixed-point gradients.  Within one tree the gradient of row i is carried as
 * the int64 q_i = rint(ldexp(g_i, S)) with S = 52 - e - ceil(log2 n), where
 * max_i |g_i| < 2^e (frexp exponent); S = 0 when every g_i is 0.  Every sum of
 * q over any row subset is exact in int64 and, times 2^-S, exact in FP64, so
 * histograms do not depend on the order of accumulation.
 *
 * Conventions for every call:
 *  - Pointers are device pointers (hipMalloc or torch tensors) unless marked
 *    "host".  All buffers are caller-owned; the library allocates nothing.
 *  - stream is a hipStream_t passed as void*.  Calls enqueue work on it and
 *    return without synchronising.  Calls on one stream run in order.
 *  - Return value: GBDT_OK or a negative gbdt_status.  Conditions checkable
 *    on the host are checked before anything is enqueued, and on failure no
 *    output is touched.  Conditions only visible on the device (a bin out of
 *    range, a fixed-point bound, an internal consistency check) are recorded
 *    in the workspace's error word; gbdt_read_error() returns it.
 *  - gbdt_last_error() returns a thread-local description of the last failure.
 *  - Every call that takes a workspace needs at least gbdt_workspace_bytes()
 *    bytes, 256-byte aligned.  Calls that share a workspace must be ordered
 *    (same stream).  The workspace must be zero-filled once before first use
 *    (its error word); after that the library keeps it consistent.
 */
#ifndef GBDT_H_
#define GBDT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GBDT_ABI_VERSION 7
#define GBDT_MAX_DEPTH 16       /* deepest tree the level loop supports */
#define GBDT_MAX_FEATURES 4096
#define GBDT_MAX_BINS 256       /* bins per feature */

typedef enum {
  GBDT_OK = 0,
  GBDT_E_ARG = -1,          /* null / misaligned pointer, bad size or parameter */
  GBDT_E_SHAPE = -2,        /* inconsistent shapes or capacities */
  GBDT_E_RANGE = -3,        /* a value out of range: bin >= n_bins, non-finite g */
  GBDT_E_OVERFLOW = -4,     /* a fixed-point bound would be exceeded */
  GBDT_E_DEVICE = -5,       /* HIP runtime error */
  GBDT_E_UNSUPPORTED = -6,  /* shape outside what the kernels support */
  GBDT_E_INTERNAL = -7      /* a device-side consistency check failed */
} gbdt_status;

/* Node flags. */
#define GBDT_NODE_LEAF 1u

/*
 * Objectives (gbdt_params.objective).  Squared error: g = pred - label, h = 1
 * (Training Core, section 2).  Logistic: the sigmoid cross-entropy of "Gradient
 * boosted trees (spec model)" (gbtBinaryCrossentropyGradSpec) on the raw score,
 * g = sigmoid(pred) - label and, as the pages give no Hessian, its second
 * derivative h = sigmoid(pred) (1 - sigmoid(pred)); with z = e^-|pred| (0 when
 * |pred| > 700) and d = 1 + z: sigmoid = 1/d (pred >= 0) or z/d, h = z/(d*d),
 * e^x from a Cody-Waite reduction and the degree-13 Taylor series, one IEEE
 * FP64 operation at a time.  g and h each get a per-tree fixed-point grid
 * (S = min(52 - e - ceil(log2 n), 30 - e), so every value fits 31 bits); the
 * Hessian sums H replace the row counts in min_child_weight, H > 0, the gain
 * and the leaf weight.
 */
#define GBDT_OBJECTIVE_SQUARED_ERROR 0
#define GBDT_OBJECTIVE_LOGISTIC 1

/*
 * Bin matrix, column-blocked, with an optional bit block.
 *
 * Byte columns: the first n_features - n_bit_features columns hold one uint8
 * bin each.  They are cut into n_blocks groups of block_features (the last
 * group may be shorter; n_blocks is 0 when every feature is a bit).  Block b
 * is a row-major [row_capacity][block_stride] uint8 array starting at
 * bins + b * row_capacity * block_stride; byte j of a row in block b is
 * byte column c = b * block_features + j (bytes past the block's columns are
 * padding, 0).  block_stride is a multiple of 4, so each row of a block is a
 * run of whole dwords that consecutive lanes load with coalesced accesses.
 *
 * Bit block (n_bit_features > 0): features with at most 2 bins stored as one
 * bit each (the idea of the ExaBoost PR's commit that packs two 4-bit cells
 * per byte when every column has at most 16 bins, taken to 1 bit for binary
 * features).  It is a row-major [row_capacity][bit_stride] array of uint32
 * words starting right after the byte blocks, at
 * bins + n_blocks * row_capacity * block_stride; bit k of a row (the k-th bit
 * feature) is bit (k & 31) of word k >> 5.  bit_stride is a multiple of 4 and
 * at least 4 * ceil(n_bit_features / 32).
 *
 * Nibble block (n_nib_features > 0): features of 3 to 16 bins stored as one
 * 4-bit cell each, eight to a word (the ExaBoost PR's commit that stores two
 * cells per byte when every column fits 16 bins, here for the columns that
 * do).  A row-major [row_capacity][nib_stride] array of uint32 words starting
 * after the bit block, at bins + n_blocks * row_capacity * block_stride +
 * row_capacity * bit_stride; nibble k of a row is bits 4 (k & 7) .. 4 (k & 7)
 * + 3 of word k >> 3.  nib_stride is a multiple of 4 and at least
 * 4 * ceil(n_nib_features / 8).
 *
 * Columns are numbered byte columns first, then the nibble features, then the
 * bit features: with nbyte = n_features - n_nib_features - n_bit_features,
 * column c < nbyte is a byte column, nbyte + k is nibble k and
 * n_features - n_bit_features + k is bit k.  col_feature (device,
 * [n_features]) names each column's feature; feature_col (device,
 * [n_features]) is its inverse.  Both NULL means the identity (byte column c
 * is feature c), which requires no bit or nibble features.  Host struct
 * holding device pointers.
 */
typedef struct gbdt_matrix {
  uint8_t* bins;
  int64_t n_rows;
  int64_t row_capacity;
  int32_t n_features;
  int32_t n_blocks;
  int32_t block_features;
  int32_t block_stride;
  int32_t n_bit_features;
  int32_t bit_stride;
  const int32_t* col_feature;
  const int32_t* feature_col;
  int32_t n_nib_features;
  int32_t nib_stride;
} gbdt_matrix;

/*
 * Feature table (host struct, device arrays).  n_bins[f] in [1, 256];
 * bin_offset[f] = sum of n_bins[g] for g < f (bin_offset[F] = total_bins);
 * bin_feature[b] = the feature of global bin b ([total_bins]); skip_bin[f] is
 * a bin of a bit feature f whose count and gradient sum the histogram kernel
 * derives from the node total instead of accumulating (the most frequent bin,
 * set by gbdt_pack_matrix), or -1; byte features ignore it.  The choice
 * changes speed only, never a bit of the result.  max_block_bins is the
 * histogram kernel's LDS slot count: at least 32 times the most bins of any
 * byte feature (a byte block's histogram takes 32 slots per bin row) and 2
 * per bit feature, at most 8192 (written by gbdt_choose_blocking /
 * gbdt_choose_layout).
 */
typedef struct gbdt_features {
  int32_t n_features;
  int32_t total_bins;
  int32_t max_block_bins; /* host value: LDS slots of one histogram workgroup */
  int32_t pad;
  const int32_t* n_bins;
  const int32_t* bin_offset;
  const int32_t* bin_feature;
  int32_t* skip_bin;
} gbdt_features;

/*
 * Rows in one order: the bin matrix, the fixed-point gradients q and the
 * original row id of each position (rid == NULL means position == row id).
 * Host struct holding device pointers.
 */
typedef struct gbdt_rows {
  gbdt_matrix X;
  int64_t* q;
  int32_t* rid;
} gbdt_rows;

/*
 * Flat breadth-first tree node (Training Core, section 3).  Leaves carry
 * GBDT_NODE_LEAF, feature = threshold_bin = left = right = -1, gain = 0 and
 * their weight in leaf_value; internal nodes carry the split, the child ids
 * and the gain, and leaf_value = 0.  The working fields say where the node's
 * rows sit in the row order of its level: positions [begin, begin + count),
 * with gsum = sum of q over them and, for the logistic objective, hsum = sum
 * of the fixed-point Hessians (0 for squared error, where H is the count).
 */
typedef struct gbdt_node {
  int32_t feature;
  int32_t threshold_bin;
  int32_t left;
  int32_t right;
  double leaf_value;
  double gain;
  uint32_t flags;
  int32_t depth;
  int32_t begin;
  int32_t count;
  int64_t gsum;
  int64_t hsum;
} gbdt_node; /* 64 bytes */

/*
 * Best split of a node: FP64 gain, split feature and bin, and the left
 * child's fixed-point gradient sum and row count.  valid = 1 iff a candidate
 * with strictly positive gain passed every constraint.
 */
typedef struct gbdt_split {
  double gain;
  int32_t feature;
  int32_t threshold_bin;
  int64_t g_left;
  int32_t n_left;
  int32_t valid;
} gbdt_split; /* 32 bytes */

/* Sibling triple for subtraction: hist[larger] = hist[parent] - hist[smaller]. */
typedef struct gbdt_pair {
  int32_t parent;
  int32_t smaller;
  int32_t larger;
  int32_t pad;
} gbdt_pair;

/*
 * Training parameters (Training Core, section 3): min_samples_leaf >= 1,
 * min_child_weight >= 0, reg_lambda >= 0, gamma >= 0, every float finite;
 * 0 <= max_depth <= GBDT_MAX_DEPTH; objective one of GBDT_OBJECTIVE_*.
 * Host struct.
 */
typedef struct gbdt_params {
  double reg_lambda;
  double gamma;
  double min_child_weight;
  double learning_rate;
  int32_t min_samples_leaf;
  int32_t max_depth;
  int32_t objective;
  int32_t pad;
} gbdt_params;

/* ---------------------------------------------------------------- setup -- */

/* Library ABI version (GBDT_ABI_VERSION). */
int gbdt_abi_version(void);

/* Thread-local text describing the last non-OK status of this thread. */
const char* gbdt_last_error(void);

/* Parameter rules of Training Core section 3: GBDT_OK or GBDT_E_ARG. */
int gbdt_validate_params(const gbdt_params* p /* host */);

/*
 * Workspace size for every call below, for matrices of up to n_rows rows,
 * lists of up to max_list entries and histograms of total_bins bins.
 */
size_t gbdt_workspace_bytes(int64_t n_rows, int32_t max_list, int32_t total_bins);

/*
 * Column blocking for features with n_bins_host[f] bins (host array): writes
 * n_features, n_blocks, block_features and block_stride of *X (no bit block:
 * n_bit_features 0, identity columns, NULL maps) and *max_block_bins: the
 * fewest blocks of equal width with at most 32 features each (rows of at
 * most 8 dwords), and 32 LDS slots per bin row of the widest feature (at
 * most 8192 slots, 64 KiB).
 */
int gbdt_choose_blocking(int32_t n_features, const int32_t* n_bins_host, gbdt_matrix* X /* host */,
                         int32_t* max_block_bins /* host */);

/*
 * Layout with narrow blocks.  pack is a set of flags: GBDT_PACK_BITS makes
 * every feature of at most 2 bins a bit, GBDT_PACK_NIBBLES makes every
 * feature of 3 to 16 bins a 4-bit cell; the others are byte columns (each
 * kind in feature order); with pack == 0 as gbdt_choose_blocking.  Writes the
 * layout fields of *X (the map pointers are left NULL: the caller uploads
 * col_feature_host / feature_col_host, host arrays of n_features entries that
 * this call fills, and stores the device copies in X), and *max_block_bins
 * (the LDS slots one histogram workgroup needs: 32 per bin of the widest
 * byte feature, 2 per bit feature for the bit block, 16 per nibble feature
 * for the nibble block).
 */
#define GBDT_PACK_BITS 1
#define GBDT_PACK_NIBBLES 2
int gbdt_choose_layout(int32_t n_features, const int32_t* n_bins_host, int32_t pack,
                       gbdt_matrix* X /* host */, int32_t* max_block_bins /* host */,
                       int32_t* col_feature_host /* host */, int32_t* feature_col_host /* host */);

/*
 * Packs a row-major uint8 [n_rows][n_features] bin matrix (device) into the
 * column-blocked layout of *dst (dst->bins allocated by the caller with
 * n_blocks * row_capacity * block_stride + row_capacity * bit_stride bytes;
 * bit features must have at most 2 bins), checks every bin against
 * n_bins (a violation sets GBDT_E_RANGE in the error word) and writes
 * ft->skip_bin (most frequent bin of each feature, smallest on ties; used for
 * bit features).
 * Setup step, not part of the per-tree path.
 */
int gbdt_pack_matrix(const uint8_t* rowmajor, const gbdt_matrix* dst /* host */,
                     const gbdt_features* ft /* host */, void* ws, size_t ws_bytes, void* stream);

/*
 * Feature binning: the "Quantized" state of the Training Core page's state
 * machine (section 5), the step that turns raw values into the bins every
 * other call reads.  raw (device, FP32, [n_rows][n_features] row-major,
 * 16-byte aligned) is written to bins_out (device, uint8, same shape and
 * layout, 16-byte aligned; the input of gbdt_pack_matrix).  Feature f has
 * ft->n_bins[f] bins and ft->n_bins[f] - 1 strictly increasing FP32 upper
 * bounds at upper[ft->bin_offset[f] + k] (device, [total_bins]; the entry at
 * k = n_bins[f] - 1 is not read).  A value's bin is the number of its
 * feature's bounds strictly below it: x <= the first bound gives bin 0, x
 * above every bound gives n_bins[f] - 1; -inf and +inf are ordinary values.
 * Comparisons only, so the result is exact.  A NaN value is written as bin 0
 * and sets GBDT_E_RANGE in the error word; so do bounds that are NaN or not
 * strictly increasing.  Uses the workspace's error word only (size from
 * gbdt_workspace_bytes(n_rows, 1, 1)).  ft needs n_bins, bin_offset and
 * bin_feature.  Host-checked errors (null or misaligned pointers, sizes)
 * return before anything is enqueued; with n_rows = 0 nothing is enqueued
 * (raw and bins_out may then be NULL).  Setup step, not part of the per-tree
 * path.
 */
int gbdt_bin_features(const float* raw, int64_t n_rows, const gbdt_features* ft /* host */,
                      const float* upper, uint8_t* bins_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Bin bounds for gbdt_bin_features: how the bounds of the "Quantized" state
 * (Training Core, section 5) are chosen, which the page leaves open.  For
 * feature f with B = ft->n_bins[f] bins, writes B - 1 strictly increasing
 * bounds u_1 .. u_{B-1} to upper[bin_offset[f] + k - 1] (device, FP32,
 * [total_bins]) and +inf after them.
 *   GBDT_BOUNDS_EQUAL_WIDTH: lo and hi are the feature's least and greatest
 *     finite values over all rows (NaN and +-inf skipped; 0 and 0 if there is
 *     none), u_k = (float)(lo + (hi - lo) * (k / B)) evaluated in FP64 one
 *     operation at a time.
 *   GBDT_BOUNDS_QUANTILE: the finite values of the row sample 0, s, 2s, ...
 *     with s = ceil(n_rows / 32768) (every row up to 32768 rows), m of them,
 *     sorted ascending; u_k is the one at rank ceil(k m / B) - 1 (0 when
 *     m = 0).  At least k m / B of the sample lies at or below u_k.
 * Zeros of either sign count as +0 in both.
 * Then each bound that is not above its predecessor is raised to the next
 * FP32 value above it among zero and the normal values (FLT_MIN after a
 * zero, 0 after a negative value whose successor is subnormal).
 * raw: device FP32 [n_rows][n_features] row-major, 16-byte aligned.
 * ws: at least gbdt_workspace_bytes(n_rows, 1, total_bins) bytes.  Setup
 * step, not part of the per-tree path; ft needs n_bins and bin_offset.
 */
#define GBDT_BOUNDS_EQUAL_WIDTH 0
#define GBDT_BOUNDS_QUANTILE 1
int gbdt_feature_bounds(const float* raw, int64_t n_rows, const gbdt_features* ft /* host */,
                        int32_t method, float* upper, void* ws, size_t ws_bytes, void* stream);

/*
 * Diagnostics (Training Core section 4, diagnostics()): per-kernel device
 * time.  While enabled, each kernel launch of the library is bracketed by two
 * hipEvents on its stream (up to `capacity` launches are kept).
 * gbdt_diag_read waits for the last one, copies (kind, milliseconds) of each
 * launch into host arrays and clears the record.  Kinds: 1 gradient max,
 * 2 gradient grid, 3 tile planner, 4 histogram, 5 histogram partial reduce,
 * 6 subtraction, 7 split search, 8 tree init, 9 level bookkeeping,
 * 10 partition, 11 prediction update, 12 packing, 13 binning, 14 ensemble
 * prediction, 15 bin bounds.  One process-wide record;
 * not for concurrent use from several threads.
 */
int gbdt_diag_enable(int32_t capacity);
int gbdt_diag_disable(void);
int gbdt_diag_read(int32_t max_records, int32_t* kinds /* host */, float* ms /* host */,
                   int32_t* n_out /* host */);

/* Reads (synchronously) and clears the workspace error word. */
int gbdt_read_error(void* ws, void* stream);

/* ------------------------------------------------------- hot-path calls -- */

/*
 * Step 1 of a tree (Training Core section 2): g_i = pred_i - (double)label_i,
 * h_i = 1 (not stored), the per-tree grid S and q_i = rint(ldexp(g_i, S)).
 * Writes q[n], *scale (S) and *gsum (sum of q) in device memory; nothing is
 * read back.  A non-finite g sets GBDT_E_RANGE.
 */
int gbdt_compute_gradients(const double* pred, const float* label, int64_t n, int64_t* q,
                           int32_t* scale, int64_t* gsum, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Step 2 (Training Core sections 6-7): for every node v = list[j],
 * j < *list_len (device count), adds to hist_g[v][b] / hist_cnt[v][b] the sum
 * of q and the number of rows among positions [nodes[v].begin,
 * nodes[v].begin + nodes[v].count) of src whose bin of feature f equals c,
 * for every global bin b = bin_offset[f] + c.  The slots of listed nodes are
 * overwritten (their previous contents are ignored); other slots are not
 * touched.  hist_g, hist_cnt: [slots][total_bins], slot = node id.
 * Requires block_stride <= 32 bytes (GBDT_E_UNSUPPORTED otherwise) and
 * ft->max_block_bins at least 32 times the bins of every byte feature; a
 * feature with more bins sets GBDT_E_SHAPE.
 * rows_bound bounds the sum of the listed counts (sizes the launch);
 * list_cap bounds *list_len.  Requires |q_i| <= 2^(52 - ceil(log2 n_rows))
 * (as written by gbdt_compute_gradients); a violation, found by a check of
 * every q of src before the histograms, sets GBDT_E_OVERFLOW.
 * Requires every bin < n_bins[f] and padding bytes 0, which holds for rows
 * written by gbdt_pack_matrix (which checks the bins) and gbdt_partition_rows;
 * other bytes give wrong counts but never an access outside the buffers.
 */
int gbdt_build_histograms(const gbdt_rows* src /* host */, const gbdt_features* ft /* host */,
                          const gbdt_node* nodes, const int32_t* list, const int32_t* list_len,
                          int32_t list_cap, int64_t rows_bound, int64_t* hist_g,
                          uint32_t* hist_cnt, void* ws, size_t ws_bytes, void* stream);

/*
 * Sibling subtraction: for each pairs[j], j < *n_pairs,
 * hist[larger] = hist[parent] - hist[smaller] elementwise over G (int64) and
 * count (uint32).  Exact, so identical to building the larger child directly.
 * A count that would go negative sets GBDT_E_INTERNAL.
 */
int gbdt_subtract_histograms(int64_t* hist_g, uint32_t* hist_cnt, int32_t total_bins,
                             const gbdt_pair* pairs, const int32_t* n_pairs, int32_t pair_cap,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Steps 3-4 (Training Core sections 2-3): for each node v = list[j], scans
 * every candidate (f, t), t in [0, n_bins[f]-2], of hist[v]: left = bins
 * <= t, right = the rest; a candidate competes only if both children have
 * >= min_samples_leaf rows, Hessian >= min_child_weight and Hessian > 0; the
 * gain is evaluated in FP64 as 0.5*((s_L + s_R) - s_P) - gamma with
 * s = (G*G)/(H+lambda), G = ldexp(sum q, -S), H = count (IEEE operations in
 * that order, no contraction).  splits[v] gets the candidate with the largest
 * gain, ties to the smaller feature, then the smaller bin; valid = 1 iff that
 * gain is strictly positive.  Node totals come from nodes[v].gsum / count;
 * S from *scale.  ws may be NULL; a 256-byte aligned workspace of at least
 * gbdt_workspace_bytes(1, list_cap, total_bins) bytes lets a histogram of
 * more than 4096 bins be searched by several workgroups per node (chunks of
 * whole features) and a merge; the result is the same either way.
 */
int gbdt_find_best_splits(const int64_t* hist_g, const uint32_t* hist_cnt,
                          const gbdt_features* ft /* host */, const gbdt_node* nodes,
                          const int32_t* list, const int32_t* list_len, int32_t list_cap,
                          const gbdt_params* p /* host */, const int32_t* scale,
                          gbdt_split* splits, void* ws, size_t ws_bytes, void* stream);

/*
 * Step 5 (Training Core section 3 routing, section 6 step 5): for each node
 * v = list[j] with s = splits[v], the rows at positions [begin, begin+count)
 * of src (bins of every block, q and row id) are written to the same
 * positions of dst, rows with bin(s.feature) <= s.threshold_bin first, each
 * side in its original order (stable).  Rows of unlisted nodes are not
 * touched.  The left count must equal s.n_left, else GBDT_E_INTERNAL.
 * src->rid == NULL means identity; dst->rid == NULL skips the row ids (the
 * level-wise driver does not need them).  Requires block_stride <= 32 bytes
 * (GBDT_E_UNSUPPORTED otherwise).
 */
int gbdt_partition_rows(const gbdt_rows* src /* host */, const gbdt_rows* dst /* host */,
                        const gbdt_node* nodes, const gbdt_split* splits, const int32_t* list,
                        const int32_t* list_len, int32_t list_cap, int64_t rows_bound, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Step 7 (Training Core section 6), by the forward pass of "Gradient boosted
 * trees (spec model)" (Forward pass): every row i of X (rows in their
 * original order) is routed from node 0 -- bin <= threshold_bin goes left,
 * otherwise right -- to a leaf v, and pred[i] = pred[i] + (learning_rate *
 * nodes[v].leaf_value), two roundings.  nodes is a flat breadth-first tree
 * of *n_nodes (device count, <= max_nodes) nodes in which siblings are
 * adjacent (right = left + 1, as the level-wise driver writes them); a node
 * whose children break that, are not larger than its own id or not below
 * *n_nodes, or whose feature or threshold_bin is out of range (threshold_bin
 * outside [0, 65533]), stops the walk, leaves the row's prediction unchanged
 * and sets GBDT_E_INTERNAL.  With pred holding a
 * base score, one call per tree gives the ensemble prediction of held-out
 * rows.
 */
int gbdt_update_predictions(double* pred, const gbdt_matrix* X /* host */, const gbdt_node* nodes,
                            const int32_t* n_nodes, int32_t max_nodes, double learning_rate,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Ensemble forward pass ("Gradient boosted trees (spec model)", Forward pass:
 * each tree traversed from its root, a row going left when its bin of the
 * node's feature is <= threshold_bin; the initial prediction plus the
 * learning rate times each tree's output):
 *   out[i] = ((base_score + learning_rate * w_1(i)) + learning_rate * w_2(i)) + ...
 * with the trees added one at a time in order, one rounding per product and
 * per sum -- the sequence the training's prediction update applies, so rows
 * of the training matrix get their training-time predictions bit for bit.
 *
 * X: the rows (device, any layout the other calls accept; rows in X's
 * order).  trees: device, n_trees node arrays of tree_stride gbdt_node each
 * (tree t at trees + t * tree_stride), as gbdt_grow_tree writes them:
 * breadth-first, right = left + 1 after the node, each child one level
 * deeper than its parent (root depth 0, at most GBDT_MAX_DEPTH).  n_nodes:
 * device int32[n_trees], the node count of each tree.  out: device
 * double[n_rows], written (not read).  ws: at least
 * gbdt_predict_workspace_bytes(n_trees, tree_stride) bytes, 256-byte aligned,
 * error word zero.  A tree that fails those structure checks sets GBDT_E_ARG
 * in the error word, and then out is not written at all (nor when the word
 * was already set).  n_trees = 0 writes base_score to every row.
 */
size_t gbdt_predict_workspace_bytes(int32_t n_trees, int32_t tree_stride);
int gbdt_predict(const gbdt_matrix* X /* host */, const gbdt_node* trees, const int32_t* n_nodes,
                 int32_t n_trees, int32_t tree_stride, double base_score, double learning_rate,
                 double* out, void* ws, size_t ws_bytes, void* stream);

/*
 * gbdt_predict for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and the same bits as gbdt_predict, with the
 * workspace replaced by a scratch area the library holds on each GPU
 * (16 MiB: gbdt_predict_workspace_bytes(n_trees, tree_stride) must not
 * exceed 16777216, else GBDT_E_ARG before anything is enqueued).  The call
 * allocates nothing.  The current device must be the one stream runs on.
 * status: device int32, written at the end of the call with 0 or the
 * device-side error code (GBDT_E_ARG for a malformed tree, in which case out
 * is not written).  Every call on one GPU shares that GPU's scratch, which
 * starts each call cleared: calls that may overlap on one GPU (different
 * streams, or different host threads) race and must be serialised by the
 * caller.
 */
int gbdt_predict_noalloc(const gbdt_matrix* X /* host */, const gbdt_node* trees,
                         const int32_t* n_nodes, int32_t n_trees, int32_t tree_stride,
                         double base_score, double learning_rate, double* out, int32_t* status,
                         void* stream);

/* ------------------------------------------------------ level-wise driver -- */

/*
 * Device buffers for gbdt_grow_tree (host struct of device pointers); sizes
 * from gbdt_grow_sizes.  pp[0], pp[1]: two row orders (bins in the blocking
 * of X and q; rid may be NULL) used in turn by the partition of each level.
 * In index mode (gbdt_grow_moves_ids) the partition moves row ids instead of
 * rows: pp[k].rid must then be set and pp[k].X.bins is not read (it may be
 * NULL).
 * q and the row buffers' q are working storage of 8 bytes per row: when
 * ceil(log2 n_rows) >= 22 (n_rows > 2^21), every |q| <= 2^(52 - ceil(log2 n))
 * <= 2^30 and the driver keeps q as int32 in the first 4 n bytes (exact);
 * otherwise as int64.  The logistic objective's grids keep every value within
 * 31 bits, so its q is int32 at any n.
 */
typedef struct gbdt_grow_buffers {
  gbdt_rows pp[2];
  int64_t* q;            /* [n] gradients in row-id order (int32 [n] when n > 2^21) */
  int64_t* hist_g;       /* [hist_slots][total_bins] */
  uint32_t* hist_cnt;    /* [hist_slots][total_bins] */
  gbdt_split* splits;    /* [max_nodes] */
  int32_t* lists;        /* [list_words] */
  void* ctrl;            /* [ctrl_bytes] */
  void* ws;
  size_t ws_bytes;
  /* logistic objective only (NULL otherwise): the fixed-point Hessians in
     row-id order, int32 [n]; the Hessian histograms [hist_slots][total_bins];
     the left child's Hessian sum of each split [max_nodes].  The row
     buffers' rid arrays (then required, int32 [n] each) carry the Hessians
     through the partitions. */
  int32_t* qh;
  int64_t* hist_h;
  int64_t* split_h;
  /* index mode only, optional (NULL: not used): X's byte blocks interleaved
     row by row, as gbdt_interleave_rows writes them (row_capacity rows of
     gbdt_interleave_pitch bytes).
     When set, index mode's histograms read the rows they reach through row
     ids from here: a row's blocks then share cache lines, and the
     workgroups of one tile's blocks run on one XCD and share its L2. */
  uint8_t* rows_ix;
  /* index mode only, optional (NULL: not used): X's byte columns one after
     another, as gbdt_column_major writes them.  When set, index mode's
     partition reads each row's split byte from here: a node's rows, whose
     ids ascend, then share one cache line per 128 ids of the split column. */
  uint8_t* cols;
} gbdt_grow_buffers;

/*
 * 1 when gbdt_grow_tree runs X with the objective in index mode, else 0: for
 * rows of two or more byte blocks with no bit or nibble block, squared
 * error.  Each level's partition then moves every row's id and q only,
 * stably, as "Module Design: Training Core" (section 6, step 5) partitions
 * row indices, and the histogram of a node reads its rows of X through the
 * ids (the ExaBoost PR's kernels gather through data indices the same way);
 * wide rows are cheaper to gather than to move at every level.  Other
 * layouts move whole rows into node order and stream them.
 */
int gbdt_grow_moves_ids(const gbdt_matrix* X /* host */, int32_t objective);

/*
 * The levels of gbdt_grow_tree whose histograms are built from the parents'
 * unpartitioned rows, as a bit mask (bit d: level d), or 0.  In row-moving
 * mode (gbdt_grow_moves_ids 0) with 2 <= max_depth <= 12 these are the odd
 * levels: rows move only after each odd level but the last, by one stable
 * two-level partition of every grandparent's segment into its
 * grandchildren's segments, and each histogram tile of an odd level reads
 * its parent's segment and adds only the rows that go to the child it
 * builds (bin <= threshold_bin for a left child; "Module Design: Training
 * Core", section 6, steps 3 and 5).  The histograms, nodes and row orders
 * of the built levels are the same as with one partition per level; only
 * the work differs.  Host only; NULL arguments give 0.
 */
int64_t gbdt_grow_filtered_levels(const gbdt_matrix* X /* host */, const gbdt_params* p /* host */);

/*
 * X's byte blocks interleaved row by row: row r's block b (block_stride
 * bytes) at out + r * P + b * block_stride, for r < row_capacity, where
 * P = gbdt_interleave_pitch(X); the P - n_blocks * block_stride bytes after
 * a row's blocks are written as 0.  out: device, 4-byte aligned (128-byte
 * aligned keeps each row inside whole cache lines), at least row_capacity *
 * P bytes, not overlapping X, written and nothing else; the bit and nibble
 * blocks are not copied.  The rows_ix buffer of gbdt_grow_tree's index mode,
 * written once per matrix (enqueued on stream; no host sync).  Errors:
 * GBDT_E_ARG for a null or misaligned pointer, the matrix checks of
 * gbdt_build_histograms.
 */
int gbdt_interleave_rows(const gbdt_matrix* X /* host */, uint8_t* out, void* stream);

/*
 * Row pitch P in bytes of gbdt_interleave_rows' copy: n_blocks *
 * block_stride rounded up to a power of two when at most 128 (so a gathered
 * row never straddles two 128-byte cache lines), else to a multiple of 128;
 * 0 for a matrix with no byte block.
 */
int32_t gbdt_interleave_pitch(const gbdt_matrix* X /* host */);

/*
 * X's byte columns one after another: byte column c's bin of row r at
 * out + c * row_capacity + r, for c < n_features - n_bit_features -
 * n_nib_features and r < row_capacity.  out: device, at least row_capacity
 * bytes per byte column, not overlapping X, written and nothing else.  The
 * cols buffer of gbdt_grow_tree's index mode, written once per matrix
 * (enqueued on stream; no host sync).  Errors: GBDT_E_ARG for a null
 * pointer, the matrix checks of gbdt_build_histograms.
 */
int gbdt_column_major(const gbdt_matrix* X /* host */, uint8_t* out, void* stream);

/* Sizes (in elements / bytes as named) of the driver's buffers. */
typedef struct gbdt_grow_sizes_t {
  int64_t max_nodes;     /* 2^(max_depth+1) - 1 */
  int64_t hist_slots;    /* 2^max_depth - 1 (at least 1) */
  int64_t list_words;
  int64_t ctrl_bytes;
  int64_t ws_bytes;
} gbdt_grow_sizes_t;

int gbdt_grow_sizes(int64_t n_rows, int32_t total_bins, int32_t max_depth,
                    gbdt_grow_sizes_t* out /* host */);

/*
 * One boosting step (Training Core section 6, steps 1-7): gradients from
 * pred and label, the tree grown level by level into nodes_out
 * ([max_nodes], breadth-first; *n_nodes_dev gets the node count), and
 * pred updated with learning_rate times the leaf weights.  All levels are
 * enqueued without host synchronisation.
 *
 * Failure (Training Core section 5: a failed fit exports no model; section 8:
 * backend errors leave no partial model): when a device-side check records an
 * error in b->ws's error word (a non-finite gradient, a partition count that
 * disagrees with its split, an internal bound), every later kernel of the
 * tree does nothing, *n_nodes_dev is set to 0 and no prediction is changed;
 * the same holds for every later call while the word stays set (it is
 * sticky until gbdt_read_error clears it).  So after a batch of trees, one
 * gbdt_read_error tells whether all of them completed, and the first tree
 * with 0 nodes is the one that failed.
 */
int gbdt_grow_tree(const gbdt_matrix* X /* host */, const gbdt_features* ft /* host */,
                   const float* label, double* pred, const gbdt_params* p /* host */,
                   gbdt_node* nodes_out, int32_t* n_nodes_dev, const gbdt_grow_buffers* b /* host */,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GBDT_H_ */
