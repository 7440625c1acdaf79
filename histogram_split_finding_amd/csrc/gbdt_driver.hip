// Level-wise tree growth driver: the seven steps of "Module Design: Training
// Core" (MPSBoost spec), section 6, run on the device without a host round
// trip per level.  The host enqueues a fixed sequence of launches per level;
// the level's node lists, counts and tile plans live in device memory and are
// written by k_level, so every launch is sized by a static bound and surplus
// workgroups exit early (the one-sync-per-level idea of the ExaBoost PR,
// taken to zero host syncs per tree).
//
// Per level d: histograms of the listed nodes (root, or the smaller child of
// every split pair) and the reduction of multi-tile partials; split search,
// which also derives each larger sibling's histogram (parent minus smaller);
// k_level (breadth-first children, frozen leaves, next level's lists, this
// level's partition plan and the next level's histogram plan); and the
// stable partition of the splitting nodes' rows into the other row buffer
// (skipped at the last level).  After the last level every row is routed
// through the finished tree and its prediction updated.

#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "gbdt.h"
#include "gbdt_internal.h"
#include "gbdt_device.h"

#pragma clang fp contract(off)

namespace gbdt {

struct TreeCtrl {
  int32_t scale;
  int32_t n_leaves;
  int64_t gsum_root;
  int32_t scale_h;  // the logistic objective's Hessian grid (0 otherwise)
  int32_t pad0;
  int32_t level_start[GBDT_MAX_DEPTH + 2];
  int32_t level_count[GBDT_MAX_DEPTH + 2];
  int32_t n_build[GBDT_MAX_DEPTH + 2];
  int32_t n_find[GBDT_MAX_DEPTH + 2];
  int32_t n_split[GBDT_MAX_DEPTH + 2];
};

// Per-level lists (level d occupies words [2^d - 1, 2^(d+1) - 1) of each):
// nodes whose histograms are built, nodes searched for a split (with, for a
// larger sibling, its parent and built sibling, else -1), splitting nodes;
// then the leaves of the tree.
struct ListLayout {
  int64_t per_type;  // 2^D - 1 words
  int64_t build, find, find_par, find_sib, split, leaves, total;
};

static ListLayout list_layout(int32_t D) {
  ListLayout L{};
  const int64_t m = (int64_t(1) << D) - 1;
  L.per_type = m < 1 ? 1 : m;
  L.build = 0;
  L.find = L.per_type;
  L.find_par = 2 * L.per_type;
  L.find_sib = 3 * L.per_type;
  L.split = 4 * L.per_type;
  L.leaves = 5 * L.per_type;
  L.total = L.leaves + (int64_t(1) << D) + 4;
  return L;
}

// Where the level kernel writes the two tile plans.
struct PlanArgs {
  int32_t* prefix;   // partition plan
  TileDesc* desc;
  uint64_t* status;
  uint64_t* status2;   // the second look-back of two-level partition plans
  PlanEntry* gstage;   // the splitting nodes of the last level that filtered its children
  int32_t* hprefix;  // histogram plan
  int32_t* hmulti;
  TileDesc* hdesc;
  WsCtrl* ctrl;
  const int32_t* feature_col;  // the matrix's map (partition plans store split columns)
  int32_t n_features;
};

// -G / (H + lambda), with H the row count (squared error, h = 1) or, for the
// logistic objective (hess), the node's Hessian sum on its grid Sh.
__device__ __forceinline__ double leaf_weight(int64_t gsum, int32_t count, int64_t hsum, int32_t S,
                                              int32_t Sh, bool hess, double lambda) {
  const double G = ldexp((double)gsum, -S);
  const double H = hess ? ldexp((double)hsum, -Sh) : (double)count;
  const double den = H + lambda;
  return -G / den;
}

__device__ __forceinline__ void make_leaf(gbdt_node* nd, double w) {
  nd->feature = -1;
  nd->threshold_bin = -1;
  nd->left = -1;
  nd->right = -1;
  nd->leaf_value = w;
  nd->gain = 0.0;
  nd->flags = GBDT_NODE_LEAF;
}

// Step 1 at the root: node 0 holds every row, lists of level 0 and the
// histogram plan of the root (tile_rows, max_tiles: the first level's).
__global__ void __launch_bounds__(1024) k_tree_init(gbdt_node* __restrict__ nodes,
                                                    gbdt_split* __restrict__ splits,
                                                    TreeCtrl* __restrict__ tc,
                                                    int32_t* __restrict__ lists, ListLayout LL,
                                                    int32_t n, int64_t min_split, int32_t D,
                                                    double lambda, int32_t* __restrict__ n_nodes_out,
                                                    PlanArgs pa, int32_t tile_rows,
                                                    int32_t max_tiles,
                                                    const int64_t* __restrict__ psum,
                                                    int32_t nparts,
                                                    const int32_t* __restrict__ guard,
                                                    const int64_t* __restrict__ psum_h) {
  __shared__ PlanLds lds;
  __shared__ int64_t s_part[1024 / 64];
  __shared__ int64_t s_parth[1024 / 64];
  // after an error (e.g. a non-finite gradient) the tree is not started: it
  // has no nodes, and the later kernels of the tree do nothing
  if (failed(guard)) {
    if (threadIdx.x == 0) *n_nodes_out = 0;
    return;
  }
  // the root's sum of q from the gradient kernels' per-block partial sums
  {
    int64_t v = 0, vh = 0;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) {
      v += psum[i];
      if (psum_h != nullptr) vh += psum_h[i];
    }
    v = wave_sum(v);
    vh = wave_sum(vh);
    if ((threadIdx.x & 63) == 0) {
      s_part[threadIdx.x >> 6] = v;
      s_parth[threadIdx.x >> 6] = vh;
    }
  }
  for (int i = threadIdx.x; i < GBDT_MAX_DEPTH + 2; i += blockDim.x) {
    tc->level_start[i] = 0;
    tc->level_count[i] = 0;
    tc->n_build[i] = 0;
    tc->n_find[i] = 0;
    tc->n_split[i] = 0;
  }
  __syncthreads();
  const bool grow = D >= 1 && (int64_t)n >= min_split;
  if (threadIdx.x == 0) {
    gbdt_node r;
    r.feature = -1;
    r.threshold_bin = -1;
    r.left = -1;
    r.right = -1;
    r.leaf_value = 0.0;
    r.gain = 0.0;
    r.flags = 0u;
    r.depth = 0;
    r.begin = 0;
    r.count = n;
    int64_t gs = 0, hs = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
      gs += s_part[w];
      hs += s_parth[w];
    }
    tc->gsum_root = gs;
    r.gsum = gs;
    r.hsum = hs;
    tc->level_start[0] = 0;
    tc->level_count[0] = 1;
    tc->n_leaves = 0;
    splits[0].valid = 0;
    if (D == 0) {
      make_leaf(&r, leaf_weight(r.gsum, n, r.hsum, tc->scale, tc->scale_h, psum_h != nullptr, lambda));
      lists[LL.leaves] = 0;
      tc->n_leaves = 1;
    } else if (grow) {
      lists[LL.build] = 0;
      lists[LL.find] = 0;
      lists[LL.find_par] = -1;
      lists[LL.find_sib] = -1;
      tc->n_build[0] = 1;
      tc->n_find[0] = 1;
    }
    nodes[0] = r;
    *n_nodes_out = 1;
  }
  __syncthreads();
  plan_tiles(nodes, lists + LL.build, grow ? 1 : 0, tile_rows, max_tiles, pa.hprefix, pa.hdesc,
             nullptr, pa.ctrl, nullptr, nullptr, 0, pa.hmulti, lds, true);
}

// Steps 3-6 bookkeeping for level d, one workgroup: each level-d node either
// splits (its children are appended breadth-first: left then right, in the
// order of the parents) or is frozen as a leaf with weight -G/(H+lambda).
// Writes the lists of level d+1 (nodes to build, sibling pairs, nodes to
// search), the splitting nodes of level d (for the partition) and appends
// the new leaves.
__global__ void __launch_bounds__(1024) k_level(int32_t d, int32_t D, gbdt_node* __restrict__ nodes,
                                                gbdt_split* __restrict__ splits,
                                                TreeCtrl* __restrict__ tc,
                                                int32_t* __restrict__ lists, ListLayout LL,
                                                int64_t min_split, double lambda,
                                                int32_t* __restrict__ n_nodes_out, PlanArgs pa,
                                                int32_t part_tile, int32_t part_max_tiles,
                                                int32_t hist_tile_max,
                                                int32_t hist_target, int32_t hist_min_rows,
                                                int32_t hist_max_tiles_next,
                                                const int32_t* __restrict__ guard,
                                                const int64_t* __restrict__ split_h,
                                                int32_t filt_next, int32_t four) {
  __shared__ PlanLds lds;
  __shared__ int32_t shm[7 * 17];
  __shared__ int32_t s_fcol[GBDT_MAX_FEATURES];  // the matrix column of each feature
  // after an error nothing of the level is written, and the partition that
  // follows finds an empty plan (it reads no other sign of the failure: a
  // partition tile that stopped early would stall its successors'
  // look-back)
  if (failed(guard)) {
    if (threadIdx.x == 0) pa.ctrl->plan_total = 0;
    return;
  }
  // the feature -> matrix column map, loaded with the level's first loads
  // (the plans' split columns then cost no dependent round trip); the block
  // scans below synchronise before its first use
  const int32_t nfeat = pa.n_features < GBDT_MAX_FEATURES ? pa.n_features : GBDT_MAX_FEATURES;
  for (int32_t f = threadIdx.x; f < nfeat; f += blockDim.x)
    s_fcol[f] = pa.feature_col != nullptr ? pa.feature_col[f] : f;
  auto column_of = [&](const gbdt_split& sp) -> int32_t {
    return (!sp.valid || sp.feature < 0 || sp.feature >= nfeat) ? -1 : s_fcol[sp.feature];
  };
  for (int c = threadIdx.x; c < kPlanSizeBuckets; c += blockDim.x) lds.bucket[c] = 0;
  const int32_t first = tc->level_start[d];
  const int32_t cnt = tc->level_count[d];
  const int32_t S = tc->scale;
  const int32_t Sh = tc->scale_h;
  const bool hess = split_h != nullptr;  // the logistic objective
  const int32_t leaf_base = tc->n_leaves;
  const int32_t child_first = first + cnt;
  const bool last = (d + 1 == D);
  const int32_t per = (cnt + blockDim.x - 1) / blockDim.x;
  const int32_t i0 = threadIdx.x * per;
  int32_t i1 = i0 + per;
  if (i1 > cnt) i1 = cnt;
  // at most one level node per thread: the plans are staged from registers
  // (no second read of the lists, nodes and splits just written)
  const bool fast = cnt <= (int32_t)blockDim.x;

  // counts: splits, pairs, searched children, leaves, partition tiles, rows
  // the next level builds (the smaller child of each pair), two-level
  // partition entries
  int32_t c[7] = {0, 0, 0, 0, 0, 0, 0};
  int32_t my_small = -1;  // fast path: the smaller child's rows of this thread's pair
  // four (two-level partition of the level's grandparents): the thread of
  // each even position i holds child a = first + i of grandparent i / 2 (b
  // is a + 1), staged by the previous level's kernel in gstage; the entry
  // carries both children's splits, and a grandparent neither of whose
  // children splits moves nothing
  PlanEntry g4{};
  gbdt_split sa{}, sb{};
  bool need4 = false;
  if (four && fast && i0 < i1 && (i0 & 1) == 0 && i0 + 1 < cnt) {
    sa = splits[first + i0];
    sb = splits[first + i0 + 1];
    g4 = pa.gstage[i0 >> 1];
    need4 = (sa.valid && sa.feature >= 0 && sa.feature < nfeat) ||
            (sb.valid && sb.feature >= 0 && sb.feature < nfeat);
    if (need4 && !last) {
      c[6] = 1;
      c[4] = tiles_of(g4.count, part_tile);
    }
  }
  for (int32_t i = i0; i < i1; ++i) {
    const int32_t v = first + i;
    const gbdt_split s = splits[v];
    const int32_t count = nodes[v].count;
    if (s.valid) {
      const int32_t nl = s.n_left, nr = count - s.n_left;
      ++c[0];
      if (last) {
        c[3] += 2;
      } else {
        if (!four) c[4] += tiles_of(count, part_tile);
        if ((int64_t)(nl > nr ? nl : nr) >= min_split) {
          ++c[1];
          c[2] += ((int64_t)nl >= min_split) + ((int64_t)nr >= min_split);
          // (a filtered next level reads the parent's rows)
          const int32_t rows = filt_next ? count : (nl <= nr ? nl : nr);
          c[5] += rows;
          my_small = rows;
        }
      }
    } else {
      ++c[3];
    }
  }
  int32_t r[7], t[7];
  block_exclusive_scan_multi<7>(c, r, t, shm);
  // histogram tile rows of the next level from the rows it actually builds:
  // about hist_target tiles, none below hist_min_rows (or above the packed
  // cells' limit)
  const int32_t hist_tile_rows_next = hist_tile_rows_for(t[5], hist_tile_max, hist_target, hist_min_rows);
  {
    int32_t nt = 0;
    if (fast) {
      nt = my_small >= 0 ? tiles_of(my_small, hist_tile_rows_next) : 0;
    } else if (!last) {
      for (int32_t i = i0; i < i1; ++i) {
        const int32_t v = first + i;
        const gbdt_split sp = splits[v];
        if (!sp.valid) continue;
        const int32_t nl = sp.n_left, nr = nodes[v].count - sp.n_left;
        if ((int64_t)(nl > nr ? nl : nr) >= min_split)
          nt += tiles_of(filt_next ? nodes[v].count : (nl <= nr ? nl : nr), hist_tile_rows_next);
      }
    }
    int32_t tot;
    r[5] = block_exclusive_scan(nt, &tot, shm);
    t[5] = tot;
  }
  int32_t r_split = r[0], r_pair = r[1], r_find = r[2], r_leaf = r[3];
  const int32_t t_split = t[0], t_pair = t[1], t_find = t[2], t_leaf = t[3];
  PlanEntry* stP = lds.stage;                    // partition plan entries
  PlanEntry* stH = lds.stage + kPlanStage / 2;   // next level's histogram plan entries
  int32_t* spP = lds.spre;
  int32_t* spH = lds.spre + kPlanStage;

  const int64_t lvl_off = (int64_t(1) << d) - 1;
  const int64_t nxt_off = (int64_t(1) << (d + 1)) - 1;
  int32_t* split_list = lists + LL.split + lvl_off;
  int32_t* leaves = lists + LL.leaves;
  int32_t* build_n = lists + LL.build + nxt_off;
  int32_t* find_n = lists + LL.find + nxt_off;
  int32_t* find_par_n = lists + LL.find_par + nxt_off;
  int32_t* find_sib_n = lists + LL.find_sib + nxt_off;

  for (int32_t i = i0; i < i1; ++i) {
    const int32_t v = first + i;
    const gbdt_split s = splits[v];
    gbdt_node nd = nodes[v];
    if (s.valid) {
      const int32_t lc = child_first + 2 * r_split;
      const int32_t rc = lc + 1;
      const int32_t nl = s.n_left, nr = nd.count - s.n_left;
      if (fast && !last) {
        PlanEntry pe;
        pe.node = v;
        pe.begin = nd.begin;
        pe.count = nd.count < 0 ? 0 : nd.count;
        pe.feature = column_of(s);
        pe.threshold_bin = s.threshold_bin;
        pe.n_left = s.n_left;
        if (!four) {
          stP[r_split] = pe;
          spP[r_split] = r[4];
        }
        // (the next level filters its children and partitions this level's
        // rows two levels at once: it reads this node's entry by position)
        if (filt_next && pa.gstage != nullptr) pa.gstage[r_split] = pe;
      }
      nd.feature = s.feature;
      nd.threshold_bin = s.threshold_bin;
      nd.left = lc;
      nd.right = rc;
      nd.gain = s.gain;
      nd.leaf_value = 0.0;
      nd.flags = 0u;
      nodes[v] = nd;
      gbdt_node L, R;
      L.feature = R.feature = -1;
      L.threshold_bin = R.threshold_bin = -1;
      L.left = L.right = R.left = R.right = -1;
      L.leaf_value = R.leaf_value = 0.0;
      L.gain = R.gain = 0.0;
      L.flags = R.flags = 0u;
      L.depth = R.depth = d + 1;
      L.begin = nd.begin;
      L.count = nl;
      L.gsum = s.g_left;
      R.begin = nd.begin + nl;
      R.count = nr;
      R.gsum = nd.gsum - s.g_left;
      L.hsum = hess ? split_h[v] : 0;
      R.hsum = hess ? nd.hsum - L.hsum : 0;
      if (last) {
        make_leaf(&L, leaf_weight(L.gsum, L.count, L.hsum, S, Sh, hess, lambda));
        make_leaf(&R, leaf_weight(R.gsum, R.count, R.hsum, S, Sh, hess, lambda));
        leaves[leaf_base + r_leaf] = lc;
        leaves[leaf_base + r_leaf + 1] = rc;
        r_leaf += 2;
      } else if ((int64_t)(nl > nr ? nl : nr) >= min_split) {
        // the smaller child is built; the larger one is derived in the
        // split search (parent minus smaller)
        const int32_t sm = (nl <= nr) ? lc : rc;
        if (fast) {
          PlanEntry pe;
          pe.node = sm;
          if (filt_next) {
            // a filtered tile: the parent's rows, of which it keeps those
            // going to sm (n_left 2: the left child, 3: the right one)
            pe.begin = nd.begin;
            pe.count = nd.count < 0 ? 0 : nd.count;
            pe.feature = column_of(s);
            pe.threshold_bin = s.threshold_bin;
            pe.n_left = sm == lc ? 2 : 3;
          } else {
            pe.begin = sm == lc ? L.begin : R.begin;
            pe.count = sm == lc ? nl : nr;
            pe.feature = pe.threshold_bin = pe.n_left = 0;
          }
          stH[r_pair] = pe;
          spH[r_pair] = r[5];
        }
        build_n[r_pair] = sm;
        ++r_pair;
        if ((int64_t)nl >= min_split) {
          find_n[r_find] = lc;
          find_par_n[r_find] = lc == sm ? -1 : v;
          find_sib_n[r_find] = lc == sm ? -1 : sm;
          ++r_find;
        }
        if ((int64_t)nr >= min_split) {
          find_n[r_find] = rc;
          find_par_n[r_find] = rc == sm ? -1 : v;
          find_sib_n[r_find] = rc == sm ? -1 : sm;
          ++r_find;
        }
      }
      nodes[lc] = L;
      nodes[rc] = R;
      splits[lc].valid = 0;
      splits[rc].valid = 0;
      split_list[r_split] = v;
      ++r_split;
    } else {
      make_leaf(&nd, leaf_weight(nd.gsum, nd.count, nd.hsum, S, Sh, hess, lambda));
      nodes[v] = nd;
      leaves[leaf_base + r_leaf] = v;
      ++r_leaf;
    }
  }
  if (threadIdx.x == 0) {
    tc->n_split[d] = t_split;
    tc->level_start[d + 1] = child_first;
    tc->level_count[d + 1] = 2 * t_split;
    if (!last) {
      tc->n_build[d + 1] = t_pair;
      tc->n_find[d + 1] = t_find;
    }
    tc->n_leaves = leaf_base + t_leaf;
    *n_nodes_out = child_first + 2 * t_split;
    if (fast) {
      spP[four ? t[6] : t_split] = t[4];
      spH[t_pair] = t[5];
      lds.n_multi = 0;
    }
  }
  if (need4 && !last) {
    PlanEntry pe = g4;
    pe.count = pe.count < 0 ? 0 : pe.count;
    const int32_t ca = column_of(sa), cb = column_of(sb);
    stP[r[6]] = pe;
    lds.ext[r[6]] = make_int4(ca >= 0 ? ((ca << 8) | (sa.threshold_bin & 0xff)) : -1,
                              ca >= 0 ? sa.n_left : g4.n_left,
                              cb >= 0 ? ((cb << 8) | (sb.threshold_bin & 0xff)) : -1,
                              cb >= 0 ? sb.n_left : g4.count - g4.n_left);
    spP[r[6]] = r[4];
  }
  if (last) return;
  // (the driver filters only levels whose parents fit this path)
  if ((filt_next || four) && !fast) {
    if (threadIdx.x == 0) dev_error(&pa.ctrl->err, GBDT_E_INTERNAL);
    return;
  }
  __syncthreads();  // the lists, the children's counts and the staged entries are visible
  // this level's partition plan (splitting nodes; none when the next level
  // is filtered: its rows are not moved) and the next level's histogram plan
  // (nodes to build)
  if (fast) {
    if (four)
      plan_emit(stP, spP, &lds.n_multi, t[6], part_tile, part_max_tiles, pa.prefix, pa.desc,
                pa.status, pa.ctrl, true, nullptr, nullptr, lds.ext, pa.status2);
    else if (!filt_next)
      plan_emit(stP, spP, &lds.n_multi, t_split, part_tile, part_max_tiles, pa.prefix, pa.desc,
                pa.status, pa.ctrl, true, nullptr, nullptr);
    plan_emit(stH, spH, &lds.n_multi, t_pair, hist_tile_rows_next, hist_max_tiles_next, pa.hprefix,
              pa.hdesc, nullptr, pa.ctrl, false, pa.hmulti, lds.bucket);
  } else {
    plan_tiles(nodes, split_list, t_split, part_tile, part_max_tiles, pa.prefix, pa.desc,
               pa.status, pa.ctrl, splits, pa.feature_col, pa.n_features, nullptr, lds, false);
    plan_tiles(nodes, build_n, t_pair, hist_tile_rows_next, hist_max_tiles_next, pa.hprefix,
               pa.hdesc, nullptr, pa.ctrl, nullptr, nullptr, 0, pa.hmulti, lds, true);
  }
}

// Nodes of fewer rows than this cannot split: each child needs
// min_samples_leaf rows and, for squared error (H = count), a Hessian of
// min_child_weight.  The logistic objective's Hessian is not a count, so only
// min_samples_leaf bounds it there.
static int64_t min_split_count(const gbdt_params* p, int64_t n) {
  double mc = p->objective == GBDT_OBJECTIVE_LOGISTIC ? 0.0 : std::ceil(p->min_child_weight);
  int64_t m = p->min_samples_leaf;
  if (mc > double(n) + 1.0) return 2 * (n + 1);
  if (int64_t(mc) > m) m = int64_t(mc);
  if (m < 1) m = 1;
  return 2 * m;
}

}  // namespace gbdt

using namespace gbdt;

extern "C" {

int gbdt_grow_sizes(int64_t n_rows, int32_t total_bins, int32_t max_depth, gbdt_grow_sizes_t* out) {
  if (!out) return fail(GBDT_E_ARG, "out is null");
  if (max_depth < 0 || max_depth > GBDT_MAX_DEPTH) return fail(GBDT_E_ARG, "max_depth out of range");
  if (n_rows < 1 || n_rows > 0x7fffffffLL) return fail(GBDT_E_ARG, "n_rows out of range");
  if (total_bins < 1) return fail(GBDT_E_ARG, "total_bins out of range");
  out->max_nodes = (int64_t(1) << (max_depth + 1)) - 1;
  out->hist_slots = (int64_t(1) << max_depth) - 1;
  if (out->hist_slots < 1) out->hist_slots = 1;
  out->list_words = list_layout(max_depth).total;
  out->ctrl_bytes = int64_t((sizeof(TreeCtrl) + 255) & ~size_t(255));
  out->ws_bytes = int64_t(ws_layout(n_rows, int32_t(1) << max_depth, total_bins).total);
  return GBDT_OK;
}

int gbdt_grow_moves_ids(const gbdt_matrix* X, int32_t objective) {
  if (!X) return 0;
  return grow_moves_ids(*X, objective == GBDT_OBJECTIVE_LOGISTIC) ? 1 : 0;
}

int64_t gbdt_grow_filtered_levels(const gbdt_matrix* X, const gbdt_params* p) {
  if (!X || !p) return 0;
  if (!grow_alternates(grow_moves_ids(*X, p->objective == GBDT_OBJECTIVE_LOGISTIC), p->max_depth)) return 0;
  int64_t m = 0;
  for (int32_t d = 1; d < p->max_depth; d += 2) m |= int64_t(1) << d;
  return m;
}

int gbdt_grow_tree(const gbdt_matrix* X, const gbdt_features* ft, const float* label, double* pred,
                   const gbdt_params* p, gbdt_node* nodes_out, int32_t* n_nodes_dev,
                   const gbdt_grow_buffers* b, void* stream) {
  if (!X || !ft || !label || !pred || !p || !nodes_out || !n_nodes_dev || !b)
    return fail(GBDT_E_ARG, "null argument");
  int rc = gbdt_validate_params(p);
  if (rc) return rc;
  const int64_t n = X->n_rows;
  if (n < 1 || n > 0x7fffffffLL) return fail(GBDT_E_ARG, "n_rows out of range");
  if (ft->n_features != X->n_features) return fail(GBDT_E_SHAPE, "feature table does not match the matrix");
  if (!b->q || !b->hist_g || !b->hist_cnt || !b->splits || !b->lists || !b->ctrl || !b->ws)
    return fail(GBDT_E_ARG, "a driver buffer is null");
  const bool logistic = p->objective == GBDT_OBJECTIVE_LOGISTIC;
  // index mode: the row buffers carry row ids and q only (their bins are not
  // read and may be NULL)
  const bool ids = grow_moves_ids(*X, logistic);
  for (int k = 0; k < 2; ++k) {
    const gbdt_rows& r = b->pp[k];
    if (!r.q) return fail(GBDT_E_ARG, "a row buffer's q is null");
    if (ids && !r.rid) return fail(GBDT_E_ARG, "index mode needs the row buffers' rid");
    if (!ids && !r.X.bins) return fail(GBDT_E_ARG, "a row buffer's bins are null");
    if (!ids && !same_layout(r.X, *X)) return fail(GBDT_E_SHAPE, "row buffers must have the layout of X");
    if (logistic && !r.rid) return fail(GBDT_E_ARG, "the logistic objective needs the row buffers' rid");
  }
  if (logistic && (!b->qh || !b->hist_h || !b->split_h))
    return fail(GBDT_E_ARG, "the logistic objective needs qh, hist_h and split_h");
  if (ids && b->rows_ix && (reinterpret_cast<uintptr_t>(b->rows_ix) & 3u))
    return fail(GBDT_E_ARG, "rows_ix not 4-byte aligned");
  const int32_t D = p->max_depth;
  gbdt_grow_sizes_t sz;
  rc = gbdt_grow_sizes(n, ft->total_bins, D, &sz);
  if (rc) return rc;
  if (b->ws_bytes < size_t(sz.ws_bytes)) return fail(GBDT_E_ARG, "workspace too small for this tree");

  gbdt_rows src;
  src.X = *X;
  src.q = b->q;
  // the logistic objective's Hessians travel with the rows in the rid slot
  src.rid = logistic ? b->qh : nullptr;
  rc = check_hist_inputs(src, *ft);
  if (rc) return rc;
  if (!ids) {
    rc = check_partition_inputs(b->pp[0], b->pp[1]);
    if (rc) return rc;
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  TreeCtrl* tc = reinterpret_cast<TreeCtrl*>(b->ctrl);
  const ListLayout LL = list_layout(D);
  const int64_t min_split = min_split_count(p, n);
  const WsLayout WL = ws_layout(n, int32_t(1) << D, ft->total_bins);
  char* w = static_cast<char*>(b->ws);
  PlanArgs pa;
  pa.ctrl = reinterpret_cast<WsCtrl*>(w + WL.ctrl);
  pa.prefix = reinterpret_cast<int32_t*>(w + WL.prefix);
  pa.desc = reinterpret_cast<TileDesc*>(w + WL.tdesc);
  pa.status = reinterpret_cast<uint64_t*>(w + WL.status);
  pa.hprefix = reinterpret_cast<int32_t*>(w + WL.hprefix);
  pa.hmulti = reinterpret_cast<int32_t*>(w + WL.hmulti);
  pa.hdesc = reinterpret_cast<TileDesc*>(w + WL.hdesc);
  pa.status2 = reinterpret_cast<uint64_t*>(w + WL.status2);
  pa.gstage = reinterpret_cast<PlanEntry*>(w + WL.gstage);
  pa.feature_col = X->feature_col;
  pa.n_features = X->n_features;
  uint64_t* hpart = reinterpret_cast<uint64_t*>(w + WL.hpart);
  // per level: histogram tile rows and launch bounds (level d builds at most
  // 2^(d-1) nodes holding at most n/2 rows; the root builds n rows)
  int32_t h_rows[GBDT_MAX_DEPTH + 1];
  int64_t h_tiles[GBDT_MAX_DEPTH + 1];
  int64_t p_tiles[GBDT_MAX_DEPTH + 1];
  // the level kernel sizes levels >= 1 from their actual rows (about
  // `target` tiles of at least min(min_rows, tile_max) rows, at most
  // tile_max); the bound below holds for every size it can choose
  const int32_t tile_max = hist_tile_max(n);
  // q is int32 (original order and both row buffers) when that is exact:
  // always for the logistic objective's 31-bit grids
  const bool q32 = logistic || driver_q32(n);
  const int32_t part_tile =
      part_tile_rows(n, X->n_blocks, X->block_stride, q32, ids, grow_alternates(ids, p->max_depth),
                     X->n_bit_features > 0 || X->n_nib_features > 0);
  const int32_t target = hist_target_tiles(X->n_blocks + (X->n_bit_features > 0 ? 1 : 0) +
                                               (X->n_nib_features > 0 ? 1 : 0),
                                           n);
  const int32_t min_rows =
      hist_min_tile_rows(ft->total_bins,
                         int64_t(X->n_blocks) * X->block_stride + X->bit_stride + X->nib_stride);
  // Row-moving mode moves rows only after every second level (alt): the
  // histograms of an odd level are built from the parents' unmoved rows
  // (each tile reads its parent's segment and keeps the rows that go to the
  // child it builds), and after it one two-level partition moves each
  // grandparent's rows straight into its grandchildren's order.  That trades
  // every other full row move for reading the larger children's rows once.
  // Index mode keeps one partition per level (filtering would gather both
  // children's rows), and so do trees deeper than 12 levels (the level
  // kernel plans filtered and two-level plans in one pass only up to 1,024
  // nodes).
  const bool alt = grow_alternates(ids, D);
  for (int32_t d = 0; d <= D; ++d) {
    const int32_t cap_build = d == 0 ? 1 : (int32_t(1) << (d - 1));
    const int64_t rows_build = (d == 0 || (alt && (d & 1))) ? n : n / 2;
    h_rows[d] = hist_tile_rows(rows_build, n, target, min_rows);
    if (d == 0) {
      h_tiles[d] = (rows_build + h_rows[d] - 1) / h_rows[d] + cap_build;
    } else {
      // tiles <= t_eff <= target + nodes, or rows / tile_max + nodes when
      // tile_max caps the size
      const int64_t by_max = (rows_build + tile_max - 1) / tile_max;
      h_tiles[d] = (by_max > target ? by_max : target) + cap_build;
    }
    p_tiles[d] = (n + part_tile - 1) / part_tile + (int64_t(1) << d);
    if (h_tiles[d] > WL.hpart_tiles || p_tiles[d] > WL.status_cap)
      return fail(GBDT_E_INTERNAL, "tile bound exceeds the workspace");
  }

  // every kernel of the tree after the gradients stops once an error is
  // recorded in the workspace (see failed())
  const int32_t* guard = &pa.ctrl->err;
  // (the sum of q stays as per-block partial sums; k_tree_init adds them)
  double* gpart = reinterpret_cast<double*>(w + WL.gpart);
  if (logistic)
    rc = launch_gradients_logistic(pred, label, n, reinterpret_cast<int32_t*>(b->q), b->qh, &tc->scale,
                                   &tc->scale_h, gpart, pa.ctrl, s);
  else
    rc = launch_gradients(pred, label, n, b->q, q32, &tc->scale, nullptr, gpart, pa.ctrl, s);
  if (rc) return rc;
  diag_begin(kDiagTreeInit, s);
  hipLaunchKernelGGL(k_tree_init, dim3(1), dim3(1024), 0, s, nodes_out, b->splits, tc, b->lists, LL,
                     (int32_t)n, min_split, D, p->reg_lambda, n_nodes_dev, pa, h_rows[0],
                     (int32_t)h_tiles[0],
                     reinterpret_cast<const int64_t*>(gpart + kGradBlocks), grad_blocks(n), guard,
                     logistic ? reinterpret_cast<const int64_t*>(gpart + 3 * kGradBlocks) : nullptr);
  diag_end(s);
  {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "k_tree_init");
  }

  int32_t n_moves = 0;  // partitions so far (they alternate between the two row buffers)
  for (int32_t d = 0; d < D; ++d) {
    const gbdt_rows& dst = b->pp[n_moves & 1];
    const int64_t lvl_off = (int64_t(1) << d) - 1;
    const int32_t cap_lvl = int32_t(1) << d;
    const int32_t cap_build = d == 0 ? 1 : (int32_t(1) << (d - 1));
    // (index mode: the rows of the original matrix, through the row ids of
    // the level's order; the root reads X in row order)
    gbdt_rows hsrc = src;
    if (ids) hsrc.X = *X;
    const bool filt = alt && (d & 1);
    rc = launch_hist(hsrc, *ft, pa.hdesc, h_tiles[d], b->hist_g, b->hist_cnt, hpart, pa.ctrl, s, q32,
                     true, ids && src.rid != nullptr, ids ? b->rows_ix : nullptr, filt);
    if (rc) return rc;
    rc = launch_hist_reduce(pa.hmulti, cap_build, h_tiles[d], n, ft->total_bins, hpart, b->hist_g,
                            b->hist_cnt, s, guard);
    if (rc) return rc;
    if (logistic) {
      // the Hessian histograms: the same kernels over the same tile plan with
      // the Hessians (the rows' rid slot) as the summed value; the counts they
      // write are the same ones again
      gbdt_rows hs = src;
      hs.q = reinterpret_cast<int64_t*>(src.rid);
      rc = launch_hist(hs, *ft, pa.hdesc, h_tiles[d], b->hist_h, b->hist_cnt, hpart, pa.ctrl, s, true,
                       true, false, nullptr, filt);
      if (rc) return rc;
      rc = launch_hist_reduce(pa.hmulti, cap_build, h_tiles[d], n, ft->total_bins, hpart, b->hist_h,
                              b->hist_cnt, s, guard);
      if (rc) return rc;
    }
    rc = launch_find(b->hist_g, b->hist_cnt, *ft, nodes_out, b->lists + LL.find + lvl_off,
                     &tc->n_find[d], cap_lvl, *p, &tc->scale, b->splits,
                     b->lists + LL.find_par + lvl_off, b->lists + LL.find_sib + lvl_off, pa.ctrl, s,
                     reinterpret_cast<FindCand*>(w + WL.fcand), guard, logistic ? b->hist_h : nullptr,
                     &tc->scale_h, b->split_h);
    if (rc) return rc;
    // (alt: after an even level the next one filters; after an odd one the
    // rows move two levels at once)
    const bool filt_next = alt && !(d & 1) && d + 1 < D;
    const bool four = alt && (d & 1) && d + 1 < D;
    diag_begin(kDiagLevel, s);
    hipLaunchKernelGGL(k_level, dim3(1), dim3(1024), 0, s, d, D, nodes_out, b->splits, tc, b->lists,
                       LL, min_split, p->reg_lambda, n_nodes_dev, pa, part_tile, (int32_t)p_tiles[d],
                       tile_max, target, min_rows, (int32_t)h_tiles[d + 1], guard,
                       logistic ? b->split_h : nullptr, filt_next ? 1 : 0, four ? 1 : 0);
    diag_end(s);
    {
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "k_level");
    }
    // the rows of the last level's children are never read again: the
    // prediction update routes rows through the finished tree instead
    if (alt ? four : d + 1 < D) {
      rc = launch_partition(hsrc, dst, pa.desc, pa.status, pa.ctrl, p_tiles[d], part_tile, s, q32, q32,
                            ids, ids ? b->cols : nullptr, four, pa.status2);
      if (rc) return rc;
      src = dst;
      ++n_moves;
    }
  }
  // step 7 in driver mode: a tree that failed (or whose structure does not
  // check out) gets n_nodes = 0 and leaves every prediction unchanged
  rc = update_predictions(pred, X, nodes_out, n_nodes_dev, int32_t(sz.max_nodes), p->learning_rate,
                          b->ws, b->ws_bytes, s, true);
  return rc;
}

}  // extern "C"
