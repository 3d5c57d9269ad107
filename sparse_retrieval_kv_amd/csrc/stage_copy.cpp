// Host tier through the copy engines: the kept host-resident blocks go from
// the pinned host pools to the HBM staging pages as hipMemcpy2DAsync /
// hipMemcpyAsync calls on a side stream (openGauss DataVec page "KV Cache
// Query-Based Computation Inference Acceleration", sections "Feature
// Description" and "Overall Solution": the offload part of the KV cache is
// kept in host DDR and the blocks retrieved at a decode round are loaded
// into HBM before attention).
//
// The host learns which blocks to copy from a device list (the kept ids, or
// the residency planner's (block, slot) pairs) copied to pinned host memory,
// then issues one copy per run: consecutive blocks that sit on consecutive
// host pages and go to consecutive staging pages.  A (page, KV head) tile is
// 32 KiB contiguous in both pools and the heads of a page are adjacent, so a
// run of one head's tiles is a 2-D copy (pitch: one page), and a run of
// whole pages -- every head keeps the same blocks, as in the per-sequence
// selection -- is one contiguous copy.
#include <hip/hip_runtime_api.h>

#include <vector>

#include "rkv.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr size_t kTileBytes = (size_t)kBlock * kDim * 2;  // one (page, head) tile

struct Pools {
  const uint16_t* host_k;
  const uint16_t* host_v;
  uint16_t* k_pages;
  uint16_t* v_pages;
  int n_kv;
};

// Head h's K and V tiles of n consecutive host pages hp.. to n consecutive
// device pages dp.. (h < 0: every head, i.e. whole pages).
hipError_t copy_run(const Pools& p, int64_t hp, int64_t dp, int64_t n, int h,
                    hipStream_t side) {
  const size_t page_bytes = kTileBytes * p.n_kv;
  const char* srcs[2] = {reinterpret_cast<const char*>(p.host_k),
                         reinterpret_cast<const char*>(p.host_v)};
  char* dsts[2] = {reinterpret_cast<char*>(p.k_pages), reinterpret_cast<char*>(p.v_pages)};
  for (int t = 0; t < 2; ++t) {
    hipError_t e;
    if (h < 0) {
      e = hipMemcpyAsync(dsts[t] + dp * page_bytes, srcs[t] + hp * page_bytes,
                         (size_t)n * page_bytes, hipMemcpyHostToDevice, side);
    } else if (n == 1) {
      e = hipMemcpyAsync(dsts[t] + dp * page_bytes + h * kTileBytes,
                         srcs[t] + hp * page_bytes + h * kTileBytes, kTileBytes,
                         hipMemcpyHostToDevice, side);
    } else {
      e = hipMemcpy2DAsync(dsts[t] + dp * page_bytes + h * kTileBytes, page_bytes,
                           srcs[t] + hp * page_bytes + h * kTileBytes, page_bytes,
                           kTileBytes, (size_t)n, hipMemcpyHostToDevice, side);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One list's copies: pairs (block j, staging page dp) in list order; blocks
// without a host page or out of range are skipped.  Runs are cut wherever
// the next pair is not (j + 1, dp + 1) on host page hp + 1.
hipError_t copy_list(const Pools& p, const int32_t* host_row, int max_blocks,
                     int64_t n_host_pages, const int32_t* js, const int64_t* dps,
                     int n, int h, hipStream_t side, int64_t* copied) {
  int64_t run_hp = -1, run_dp = -1, run_n = 0;
  int prev_j = -2;
  for (int i = 0; i <= n; ++i) {
    int j = -1;
    int64_t hp = -1, dp = -1;
    if (i < n) {
      j = js[i];
      dp = dps[i];
      if (j >= 0 && j < max_blocks) hp = host_row[j];
      if (hp < 0 || hp >= n_host_pages) j = -1;  // nothing to copy
    }
    const bool extends = run_n > 0 && j >= 0 && j == prev_j + 1 &&
                         hp == run_hp + run_n && dp == run_dp + run_n;
    if (!extends && run_n > 0) {
      const hipError_t e = copy_run(p, run_hp, run_dp, run_n, h, side);
      if (e != hipSuccess) return e;
      *copied += run_n;
      run_n = 0;
    }
    if (j >= 0) {
      if (run_n == 0) {
        run_hp = hp;
        run_dp = dp;
      }
      ++run_n;
    }
    prev_j = j;
  }
  return hipSuccess;
}

}  // namespace

hipError_t issue_stage_copies(const StageCopyArgs& a, int64_t* tiles_copied) {
  Pools p{a.host_k, a.host_v, a.k_pages, a.v_pages, a.n_kv};
  std::vector<int64_t> dps;
  std::vector<int32_t> js;
  int64_t copied = 0;
  for (int b = 0; b < a.batch; ++b) {
    const int32_t* host_row = a.host_table + (int64_t)b * a.max_blocks;
    // whole pages when every head of the sequence copies the same pairs
    const int bh0 = b * a.n_kv;
    const int n0 = a.count(bh0);
    bool same = a.whole_pages;
    for (int h = 1; same && h < a.n_kv; ++h) {
      const int bh = bh0 + h;
      same = a.count(bh) == n0;
      for (int i = 0; i < n0 && same; ++i)
        same = a.block(bh, i) == a.block(bh0, i) && a.slot(bh, i) == a.slot(bh0, i);
    }
    for (int h = 0; h < (same ? 1 : a.n_kv); ++h) {
      const int bh = bh0 + h;
      const int n = a.count(bh);
      js.resize(n);
      dps.resize(n);
      for (int i = 0; i < n; ++i) {
        js[i] = a.block(bh, i);
        const int s = a.slot(bh, i);
        dps[i] = (s >= 0 && s < a.slots_per_seq)
                     ? a.stage_page0 + (int64_t)b * a.slots_per_seq + s
                     : -1;
        if (dps[i] < 0 || dps[i] >= a.n_pages) js[i] = -1;
      }
      int64_t c = 0;
      const hipError_t e = copy_list(p, host_row, a.max_blocks, a.n_host_pages, js.data(),
                                     dps.data(), n, same ? -1 : h, a.side, &c);
      if (e != hipSuccess) return e;
      copied += same ? c * a.n_kv : c;
    }
  }
  if (tiles_copied) *tiles_copied = copied;
  return hipSuccess;
}

}  // namespace rkv
