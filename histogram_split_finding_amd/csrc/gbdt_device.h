// Device helpers shared by the HIP translation units of libgbdt: error word,
// wave and workgroup scans, and the tile planner (run by one workgroup).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gbdt.h"
#include "gbdt_internal.h"

namespace gbdt {

__device__ __forceinline__ void dev_error(int32_t* err, int code) { atomicCAS(err, 0, code); }

// The tree driver hands its kernels the workspace error word as `guard`:
// once a kernel of the tree has recorded an error, every later kernel of the
// tree (and of later trees, until the word is read and cleared) does nothing,
// so no tree is finished and no prediction changes after a failure.  The
// per-call entry points pass nullptr.
__device__ __forceinline__ bool failed(const int32_t* guard) {
  return guard != nullptr &&
         __hip_atomic_load(guard, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// DPP lane move of a 32-bit value: lanes whose source lies outside the row,
// or whose row is masked off, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int32_t dpp_move_i32(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive sum over lanes 0..lane of a wave (every lane active): shifts by
// 1, 2, 4 and 8 within each row of 16 lanes, then row 0's total into row 1
// and row 2's into row 3 (row_bcast:15), then rows 0-1's total into rows 2
// and 3 (row_bcast:31).  VALU lane moves, no LDS round trips.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x) {
  x += dpp_move_i32<0x111, 0xF>(x);  // row_shr:1
  x += dpp_move_i32<0x112, 0xF>(x);  // row_shr:2
  x += dpp_move_i32<0x114, 0xF>(x);  // row_shr:4
  x += dpp_move_i32<0x118, 0xF>(x);  // row_shr:8
  x += dpp_move_i32<0x142, 0xA>(x);  // row_bcast:15
  x += dpp_move_i32<0x143, 0xC>(x);  // row_bcast:31
  return x;
}

// The same within row 0 only (lanes 0..15): enough for the at most 16 wave
// totals of a workgroup.
__device__ __forceinline__ int32_t row_incl_scan(int32_t x) {
  x += dpp_move_i32<0x111, 0xF>(x);
  x += dpp_move_i32<0x112, 0xF>(x);
  x += dpp_move_i32<0x114, 0xF>(x);
  x += dpp_move_i32<0x118, 0xF>(x);
  return x;
}

// Exclusive scan of one int32 per thread across a workgroup (blockDim.x a
// multiple of 64, <= 1024).  Returns the exclusive prefix; *total = sum.
// Each wave scans with lane moves and writes its total; after one barrier
// every wave scans the wave totals itself (lanes 0..15) and takes its own
// offset with a lane read.
__device__ inline int32_t block_exclusive_scan(int32_t v, int32_t* total, int32_t* sh /*[32]*/) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = (blockDim.x + 63) >> 6;
  const int32_t x = wave_incl_scan(v);
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  const int32_t t = row_incl_scan(lane < nw ? sh[lane] : 0);
  const int32_t before = wid > 0 ? __builtin_amdgcn_readlane(t, wid - 1) : 0;
  *total = __builtin_amdgcn_readlane(t, nw - 1);
  __syncthreads();  // (sh may be reused)
  return before + x - v;
}

// Exclusive scans of K int32 values per thread across a workgroup at once
// (one barrier for all K, as block_exclusive_scan).  sh: LDS [K * 17].
template <int K>
__device__ inline void block_exclusive_scan_multi(const int32_t (&v)[K], int32_t (&excl)[K],
                                                  int32_t (&total)[K], int32_t* sh) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = (blockDim.x + 63) >> 6;
  int32_t x[K];
#pragma unroll
  for (int k = 0; k < K; ++k) x[k] = wave_incl_scan(v[k]);
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < K; ++k) sh[k * 17 + wid] = x[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int32_t t = row_incl_scan(lane < nw ? sh[k * 17 + lane] : 0);
    const int32_t before = wid > 0 ? __builtin_amdgcn_readlane(t, wid - 1) : 0;
    excl[k] = before + x[k] - v[k];
    total[k] = __builtin_amdgcn_readlane(t, nw - 1);
  }
  __syncthreads();
}

__device__ __forceinline__ int32_t clamp_len(const int32_t* len, int32_t cap) {
  int32_t n = *len;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

constexpr int kPlanLdsEntries = 8192;  // list entries whose tile prefix is kept in LDS
constexpr int kPlanStage = 2048;       // list entries whose node data is kept in LDS
constexpr int kPlanStage4 = 512;       // entries of a two-level partition plan (grandparents)

constexpr int kPlanSizeBuckets = 64;  // size classes of the histogram tiles' largest-first order
constexpr int kPlanSortMinTiles = 768;  // smaller histogram plans (about one round) keep node order

// LDS of the planner: sh [32], spre [kPlanLdsEntries + 1], stage
// [kPlanStage], the size-class counters of the largest-first order, and the
// children's splits of a two-level partition plan's entries (split2, n2,
// split3, n3 of the tile descriptor).
struct PlanLds {
  int32_t sh[32];
  int32_t n_multi;
  int32_t spre[kPlanLdsEntries + 1];
  PlanEntry stage[kPlanStage];
  int32_t bucket[kPlanSizeBuckets];
  int4 ext[kPlanStage4];
};

// Size class of a tile of `size` rows (tiles hold at most tile_rows): 0 for
// the largest, kPlanSizeBuckets - 1 for the smallest.
__device__ __forceinline__ int32_t tile_size_class(int32_t size, int32_t tile_rows) {
  // tile_rows < 2^24, so size * 64 fits 32 bits
  const uint32_t k = ((uint32_t)(size < 0 ? 0 : size) * (uint32_t)kPlanSizeBuckets) /
                     ((uint32_t)tile_rows + 1u);
  return kPlanSizeBuckets - 1 - (int32_t)(k > kPlanSizeBuckets - 1 ? kPlanSizeBuckets - 1 : k);
}

// Launch position of a tile of class cls in a histogram plan: the tiles are
// ordered by size class, largest first, so that the workgroups dispatched
// last -- whose end is the launch's end -- carry the smallest tiles.  The
// order within a class is arbitrary; each tile keeps its own index as its
// partial slot, so no result depends on it.  bucket[] holds the classes'
// next positions.
__device__ __forceinline__ int32_t tile_order(int32_t* bucket, int32_t cls) {
  return atomicAdd(&bucket[cls], 1);
}

// Counts the tiles of a node of `count` rows into their size classes: its
// full tiles and, if any, its last partial tile (an empty node has one empty
// tile).
__device__ __forceinline__ void count_node_tiles(int32_t* bucket, int32_t count, int32_t tile_rows) {
  const int32_t c = count < 0 ? 0 : count;
  const int32_t full = c / tile_rows;
  const int32_t rem = c - full * tile_rows;
  if (full > 0) atomicAdd(&bucket[tile_size_class(tile_rows, tile_rows)], full);
  if (rem > 0 || c == 0) atomicAdd(&bucket[tile_size_class(rem, tile_rows)], 1);
}

// bucket[c] := first launch position of class c (exclusive prefix of the
// counts), by wave 0 (one class per lane); the workgroup synchronises
// around it.
__device__ __forceinline__ void tile_order_prefix(int32_t* bucket) {
  static_assert(kPlanSizeBuckets == 64, "one size class per lane");
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int32_t v = bucket[lane];
    bucket[lane] = wave_incl_scan(v) - v;
  }
  __syncthreads();
}

// The matrix column of a split's feature (-1 for an invalid split or a
// feature outside the map's range).
__device__ __forceinline__ int32_t split_column(const gbdt_split& sp, const int32_t* feature_col,
                                                int32_t n_features) {
  if (!sp.valid || sp.feature < 0 || sp.feature >= n_features) return -1;
  return feature_col != nullptr ? feature_col[sp.feature] : sp.feature;
}

__device__ __forceinline__ int32_t tiles_of(int32_t c, int32_t tile_rows) {
  if (c < 0) c = 0;
  return c == 0 ? 1 : (c + tile_rows - 1) / tile_rows;
}

// Second half of a tile plan, from entries already staged in LDS: stage[j]
// the j-th list entry and spre[0..n] the exclusive prefix of its tiles
// (spre[n] = total), both visible to the workgroup.  Writes prefix[0..n],
// the multi-tile list (multi != nullptr), the plan total and cleared
// look-back status (status != nullptr) and every tile's descriptor (from LDS
// only), then descriptors with node -1 up to max_tiles.  with_split: the
// entries carry a split (partition plans).  *n_multi (LDS) must be 0 and
// visible, like the staged entries.  ext (LDS, or nullptr): the children's
// splits of a two-level partition plan, ext[j] = (split2, n2, split3, n3);
// status2 then receives cleared look-back words too.
__device__ inline void plan_emit(const PlanEntry* stage, const int32_t* spre, int32_t* n_multi,
                                 int32_t n, int32_t tile_rows, int32_t max_tiles,
                                 int32_t* __restrict__ prefix, TileDesc* __restrict__ desc,
                                 uint64_t* __restrict__ status, WsCtrl* __restrict__ ctrl,
                                 bool with_split, int32_t* __restrict__ multi,
                                 int32_t* bucket /* LDS [kPlanSizeBuckets] or nullptr */,
                                 const int4* ext = nullptr, uint64_t* __restrict__ status2 = nullptr) {
  const int32_t total = spre[n];
  for (int32_t j = threadIdx.x; j <= n; j += blockDim.x) {
    prefix[j] = spre[j];
    if (multi != nullptr && j < n && spre[j + 1] - spre[j] > 1)
      reinterpret_cast<int4*>(multi + 4)[atomicAdd(n_multi, 1)] =
          make_int4(stage[j].node, spre[j], spre[j + 1], j);
  }
  if (threadIdx.x == 0) {
    if (total > max_tiles) dev_error(&ctrl->err, GBDT_E_SHAPE);
    if (status != nullptr) {
      ctrl->plan_total = total < max_tiles ? total : max_tiles;
    }
  }
  const int32_t lim = total < max_tiles ? total : max_tiles;
  // with `bucket`, the tiles' size classes are counted per node first (not
  // when the plan overflows: its positions must stay below max_tiles)
  if (total > max_tiles || total <= kPlanSortMinTiles) bucket = nullptr;
  if (bucket != nullptr) {
    for (int32_t j = threadIdx.x; j < n; j += blockDim.x) count_node_tiles(bucket, stage[j].count, tile_rows);
    tile_order_prefix(bucket);
  }
  {
    for (int32_t t = threadIdx.x; t < lim; t += blockDim.x) {
      int32_t lo = 0, hi = n - 1;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (spre[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const PlanEntry pe = stage[lo];
      const int32_t tf = spre[lo];
      TileDesc d;
      d.node = pe.node;
      d.r0 = pe.begin + (t - tf) * tile_rows;
      d.r1 = d.r0 + tile_rows < pe.begin + pe.count ? d.r0 + tile_rows : pe.begin + pe.count;
      int32_t pos = t;
      if (bucket != nullptr) pos = tile_order(bucket, tile_size_class(d.r1 - d.r0, tile_rows));
      d.ntiles = spre[lo + 1] - tf;
      d.tfirst = tf;
      d.begin = pe.begin;
      d.count = pe.count;
      d.feature = pe.feature;
      d.threshold_bin = pe.threshold_bin;
      d.n_left = pe.n_left;
      d.split_valid = with_split && pe.feature >= 0;
      d.slot = t;
      if (ext != nullptr) {
        const int4 x = ext[lo];
        d.split2 = x.x;
        d.n2 = x.y;
        d.split3 = x.z;
        d.n3 = x.w;
      } else {
        d.split2 = d.split3 = -1;
        d.n2 = d.n3 = 0;
      }
      desc[pos] = d;
      if (status != nullptr) status[t] = 0ull;
      if (status2 != nullptr) status2[t] = 0ull;
    }
  }
  // surplus tiles of a histogram launch find node -1; a partition launch's
  // stop at ctrl->plan_total (50M rows: 12K scattered writes spared)
  if (status == nullptr)
    for (int32_t t = lim + threadIdx.x; t < max_tiles; t += blockDim.x) desc[t].node = -1;
  __syncthreads();
  if (threadIdx.x == 0 && multi != nullptr) multi[0] = *n_multi;
}

// Tile plan of the nodes list[0..n), run by every thread of one workgroup:
// tiles per node (ceil(count / tile_rows), at least one), their exclusive
// prefix (prefix[n] = total), one descriptor per tile (a workgroup of the
// launch that follows reads its whole assignment with one load), for a
// histogram plan descriptors with node -1 for the launch's tiles [total,
// max_tiles), and, for a partition plan (status != nullptr), a cleared
// look-back status array and the plan total in ctrl (its launch's surplus
// tiles stop there), and (splits != nullptr) each node's
// split in its tiles' descriptors (the split feature as its matrix column:
// feature_col[feature], or the feature itself when feature_col is NULL),
// and (multi != nullptr) the list positions
// of the nodes with more than one tile (multi[0] = their count, then from
// multi + 4 one int4 (node, first tile, end tile, list position) each, in
// no particular order; for the partial reduction).  More tiles than max_tiles sets
// GBDT_E_SHAPE; the surplus is not planned.  Each entry's node (and split)
// is read once; up to kPlanStage entries are kept in LDS, so writing the
// descriptors reads no global memory.  The list and the nodes' counts must
// be visible to the workgroup (written before a barrier or a previous
// launch).
__device__ inline void plan_tiles(const gbdt_node* __restrict__ nodes, const int32_t* __restrict__ list,
                                  int32_t n, int32_t tile_rows, int32_t max_tiles,
                                  int32_t* __restrict__ prefix, TileDesc* __restrict__ desc,
                                  uint64_t* __restrict__ status, WsCtrl* __restrict__ ctrl,
                                  const gbdt_split* __restrict__ splits,
                                  const int32_t* __restrict__ feature_col, int32_t n_features,
                                  int32_t* __restrict__ multi, PlanLds& L, bool by_size) {
  const bool staged = n <= kPlanStage;
  const bool in_lds = n <= kPlanLdsEntries;
  const int32_t per = (n + blockDim.x - 1) / blockDim.x;
  const int32_t j0 = threadIdx.x * per;
  int32_t local = 0;
  for (int32_t j = j0; j < j0 + per && j < n; ++j) {
    const int32_t v = list[j];
    const gbdt_node nd = nodes[v];
    local += tiles_of(nd.count, tile_rows);
    if (staged) {
      PlanEntry pe;
      pe.node = v;
      pe.begin = nd.begin;
      pe.count = nd.count < 0 ? 0 : nd.count;
      pe.feature = pe.threshold_bin = pe.n_left = 0;
      if (splits != nullptr) {
        const gbdt_split sp = splits[v];
        pe.feature = split_column(sp, feature_col, n_features);
        pe.threshold_bin = sp.threshold_bin;
        pe.n_left = sp.n_left;
      }
      L.stage[j] = pe;
    }
  }
  if (threadIdx.x == 0) L.n_multi = 0;
  for (int c = threadIdx.x; c < kPlanSizeBuckets; c += blockDim.x) L.bucket[c] = 0;
  int32_t total;
  int32_t excl = block_exclusive_scan(local, &total, L.sh);
  if (staged) {
    for (int32_t j = j0; j < j0 + per && j < n; ++j) {
      L.spre[j] = excl;
      excl += tiles_of(L.stage[j].count, tile_rows);
    }
    if (threadIdx.x == 0) L.spre[n] = total;
    __syncthreads();
    plan_emit(L.stage, L.spre, &L.n_multi, n, tile_rows, max_tiles, prefix, desc, status, ctrl,
              splits != nullptr, multi, by_size ? L.bucket : nullptr);
    return;
  }
  // long lists: the prefix in LDS (up to kPlanLdsEntries) or global memory,
  // entries read from global memory
  for (int32_t j = j0; j < j0 + per && j < n; ++j) {
    prefix[j] = excl;
    if (in_lds) L.spre[j] = excl;
    const int32_t nt = tiles_of(nodes[list[j]].count, tile_rows);
    if (multi != nullptr && nt > 1)
      reinterpret_cast<int4*>(multi + 4)[atomicAdd(&L.n_multi, 1)] = make_int4(list[j], excl, excl + nt, j);
    excl += nt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (multi != nullptr) multi[0] = L.n_multi;
    prefix[n] = total;
    if (in_lds) L.spre[n] = total;
    if (total > max_tiles) dev_error(&ctrl->err, GBDT_E_SHAPE);
    if (status != nullptr) {
      ctrl->plan_total = total < max_tiles ? total : max_tiles;
    }
  }
  __syncthreads();
  const int32_t lim = total < max_tiles ? total : max_tiles;
  // an overflowing plan keeps positions below max_tiles; a plan of one round
  // of workgroups has no tail to shorten
  if (total > max_tiles || total <= kPlanSortMinTiles) by_size = false;
  if (by_size) {
    for (int32_t j = threadIdx.x; j < n; j += blockDim.x)
      count_node_tiles(L.bucket, nodes[list[j]].count, tile_rows);
    tile_order_prefix(L.bucket);
  }
  {
  for (int32_t t = threadIdx.x; t < lim; t += blockDim.x) {
    const int32_t* pre = in_lds ? L.spre : prefix;
    int32_t lo = 0, hi = n - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int32_t v = list[lo];
    const gbdt_node nd = nodes[v];
    PlanEntry pe;
    pe.node = v;
    pe.begin = nd.begin;
    pe.count = nd.count < 0 ? 0 : nd.count;
    pe.feature = pe.threshold_bin = pe.n_left = 0;
    if (splits != nullptr) {
      const gbdt_split sp = splits[v];
      pe.feature = split_column(sp, feature_col, n_features);
      pe.threshold_bin = sp.threshold_bin;
      pe.n_left = sp.n_left;
    }
    const int32_t tf = pre[lo];
    TileDesc d;
    d.node = pe.node;
    d.r0 = pe.begin + (t - tf) * tile_rows;
    d.r1 = d.r0 + tile_rows < pe.begin + pe.count ? d.r0 + tile_rows : pe.begin + pe.count;
    d.ntiles = pre[lo + 1] - tf;
    d.tfirst = tf;
    d.begin = pe.begin;
    d.count = pe.count;
    d.feature = pe.feature;
    d.threshold_bin = pe.threshold_bin;
    d.n_left = pe.n_left;
    d.split_valid = splits != nullptr && pe.feature >= 0;
    d.slot = t;
    d.split2 = d.split3 = -1;
    d.n2 = d.n3 = 0;
    int32_t pos = t;
    if (by_size) pos = tile_order(L.bucket, tile_size_class(d.r1 - d.r0, tile_rows));
    desc[pos] = d;
    if (status != nullptr) status[t] = 0ull;
  }
  }
  // surplus tiles of a histogram launch find node -1; a partition launch's
  // stop at ctrl->plan_total (50M rows: 12K scattered writes spared)
  if (status == nullptr)
    for (int32_t t = lim + threadIdx.x; t < max_tiles; t += blockDim.x) desc[t].node = -1;
  __syncthreads();
}

}  // namespace gbdt
