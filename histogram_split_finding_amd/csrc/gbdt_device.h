// Device helpers shared by the HIP translation units of libgbdt: error word,
// wave and workgroup scans, and the tile planner (run by one workgroup).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gbdt.h"
#include "gbdt_internal.h"

namespace gbdt {

__device__ __forceinline__ void dev_error(int32_t* err, int code) { atomicCAS(err, 0, code); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Exclusive scan of one int32 per thread across a workgroup (blockDim.x a
// multiple of 64, <= 1024).  Returns the exclusive prefix; *total = sum.
__device__ inline int32_t block_exclusive_scan(int32_t v, int32_t* total, int32_t* sh /*[32]*/) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  int32_t x = v;
  for (int off = 1; off < 64; off <<= 1) {
    int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int w = 0; w < nw; ++w) {
      int32_t t = sh[w];
      sh[w] = acc;
      acc += t;
    }
    sh[31] = acc;
  }
  __syncthreads();
  int32_t res = sh[wid] + x - v;
  *total = sh[31];
  __syncthreads();
  return res;
}

__device__ __forceinline__ int32_t clamp_len(const int32_t* len, int32_t cap) {
  int32_t n = *len;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

constexpr int kPlanLdsEntries = 8192;

// Tile plan of the nodes list[0..n), run by every thread of one workgroup:
// tiles per node (ceil(count / tile_rows), at least one), their exclusive
// prefix (prefix[n] = total), one descriptor per tile (a workgroup of the
// launch that follows reads its whole assignment with one load), descriptors
// with node -1 for the launch's tiles [total, max_tiles), and, for a
// partition plan (status != nullptr), a cleared look-back status array and
// the ticket and plan total in ctrl.  More tiles than max_tiles sets
// GBDT_E_SHAPE; the surplus is not planned.  sh: LDS [32];
// spre: LDS [kPlanLdsEntries + 1].  The list and the nodes' counts must be
// visible to the workgroup (written before a barrier or a previous launch).
__device__ inline void plan_tiles(const gbdt_node* __restrict__ nodes, const int32_t* __restrict__ list,
                                  int32_t n, int32_t tile_rows, int32_t max_tiles,
                                  int32_t* __restrict__ prefix, TileDesc* __restrict__ desc,
                                  uint64_t* __restrict__ status, WsCtrl* __restrict__ ctrl,
                                  int32_t* sh, int32_t* spre) {
  const int32_t per = (n + blockDim.x - 1) / blockDim.x;
  const int32_t j0 = threadIdx.x * per;
  int32_t local = 0;
  for (int32_t j = j0; j < j0 + per && j < n; ++j) {
    int32_t c = nodes[list[j]].count;
    if (c < 0) c = 0;
    local += c == 0 ? 1 : (c + tile_rows - 1) / tile_rows;
  }
  int32_t total;
  int32_t excl = block_exclusive_scan(local, &total, sh);
  const bool in_lds = n <= kPlanLdsEntries;
  for (int32_t j = j0; j < j0 + per && j < n; ++j) {
    prefix[j] = excl;
    if (in_lds) spre[j] = excl;
    int32_t c = nodes[list[j]].count;
    if (c < 0) c = 0;
    excl += c == 0 ? 1 : (c + tile_rows - 1) / tile_rows;
  }
  if (threadIdx.x == 0) {
    prefix[n] = total;
    if (in_lds) spre[n] = total;
    if (total > max_tiles) dev_error(&ctrl->err, GBDT_E_SHAPE);
    if (status != nullptr) {
      ctrl->plan_total = total < max_tiles ? total : max_tiles;
      ctrl->ticket = 0u;
    }
  }
  __syncthreads();
  const int32_t lim = total < max_tiles ? total : max_tiles;
  for (int32_t t = threadIdx.x; t < lim; t += blockDim.x) {
    const int32_t* pre = in_lds ? spre : prefix;
    int32_t lo = 0, hi = n - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int32_t v = list[lo];
    const gbdt_node nd = nodes[v];
    const int32_t tf = pre[lo];
    const int32_t nt = pre[lo + 1] - tf;
    const int32_t cnt = nd.count < 0 ? 0 : nd.count;
    TileDesc d;
    d.node = v;
    d.r0 = nd.begin + (t - tf) * tile_rows;
    d.r1 = d.r0 + tile_rows < nd.begin + cnt ? d.r0 + tile_rows : nd.begin + cnt;
    d.ntiles = nt;
    d.tfirst = tf;
    d.j = lo;
    d.begin = nd.begin;
    d.count = cnt;
    desc[t] = d;
    if (status != nullptr) status[t] = 0ull;
  }
  for (int32_t t = lim + threadIdx.x; t < max_tiles; t += blockDim.x) desc[t].node = -1;
  __syncthreads();
}

}  // namespace gbdt
