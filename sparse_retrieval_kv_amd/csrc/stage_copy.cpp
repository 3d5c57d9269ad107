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
//
// A copy command costs about 10 us of copy-engine time however small it is,
// and the commands of one stream run one after another, so a caller may ask
// (rkv_params.copy_lanes) for the copies to be spread over copy lanes:
// streams of the library's own, forked from the caller's side stream by an
// event and joined back to it by one event each.  On MI355X four lanes run
// 32 KiB copies about 3x and 512 KiB copies 2x faster than one stream (the
// latter at the host link's rate); sixteen run slower than one.  The lanes
// are ordinary streams of the process, which shares the runtime's hardware
// queues among all its streams, so they are off unless asked for.
#include <hip/hip_runtime_api.h>

#include <mutex>
#include <vector>

#include "rkv.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr size_t kTileBytes = (size_t)kBlock * kDim * 2;  // one (page, head) tile

constexpr int kMaxLanes = RKV_MAX_COPY_LANES;
constexpr int kMaxDevices = 64;
// a command's fixed cost, in bytes of transfer at the host link's rate
constexpr size_t kCommandBytes = (size_t)512 << 10;

// The copy lanes of one device, created as calls ask for them (with that
// device current) and kept until the process ends (default priority,
// non-blocking).
struct Lanes {
  bool have_fork = false;
  int made = 0;  // lanes with both their stream and their join event
  hipEvent_t fork;
  hipStream_t stream[kMaxLanes];
  hipEvent_t join[kMaxLanes];
};
std::mutex g_lanes_mutex;  // held while a call forks, fills and joins lanes
Lanes g_lanes[kMaxDevices];

// The current device's lanes, at least n of them.
hipError_t lanes_of_current_device(int n, Lanes** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  Lanes& L = g_lanes[dev];
  if (!L.have_fork) {
    e = hipEventCreateWithFlags(&L.fork, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    L.have_fork = true;
  }
  while (L.made < n) {
    e = hipStreamCreateWithFlags(&L.stream[L.made], hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    e = hipEventCreateWithFlags(&L.join[L.made], hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipStreamDestroy(L.stream[L.made]);
      return e;
    }
    ++L.made;
  }
  *out = &L;
  return hipSuccess;
}

// Where a call's copy commands go: the side stream alone (n = 1), or each
// command to the lane with the least work queued by this call.
struct LaneQueue {
  int n = 1;
  hipStream_t stream[kMaxLanes];
  size_t load[kMaxLanes] = {};
  bool used[kMaxLanes] = {};
  hipStream_t pick(size_t bytes) {
    int best = 0;
    for (int i = 1; i < n; ++i)
      if (load[i] < load[best]) best = i;
    load[best] += bytes + kCommandBytes;
    used[best] = true;
    return stream[best];
  }
};

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
                    LaneQueue& lanes) {
  const size_t page_bytes = kTileBytes * p.n_kv;
  const char* srcs[2] = {reinterpret_cast<const char*>(p.host_k),
                         reinterpret_cast<const char*>(p.host_v)};
  char* dsts[2] = {reinterpret_cast<char*>(p.k_pages), reinterpret_cast<char*>(p.v_pages)};
  for (int t = 0; t < 2; ++t) {
    hipError_t e;
    if (h < 0) {
      const size_t bytes = (size_t)n * page_bytes;
      e = hipMemcpyAsync(dsts[t] + dp * page_bytes, srcs[t] + hp * page_bytes, bytes,
                         hipMemcpyHostToDevice, lanes.pick(bytes));
    } else if (n == 1) {
      e = hipMemcpyAsync(dsts[t] + dp * page_bytes + h * kTileBytes,
                         srcs[t] + hp * page_bytes + h * kTileBytes, kTileBytes,
                         hipMemcpyHostToDevice, lanes.pick(kTileBytes));
    } else {
      e = hipMemcpy2DAsync(dsts[t] + dp * page_bytes + h * kTileBytes, page_bytes,
                           srcs[t] + hp * page_bytes + h * kTileBytes, page_bytes,
                           kTileBytes, (size_t)n, hipMemcpyHostToDevice,
                           lanes.pick((size_t)n * kTileBytes));
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
                     int n, int h, LaneQueue& lanes, int64_t* copied) {
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
      const hipError_t e = copy_run(p, run_hp, run_dp, run_n, h, lanes);
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

// Every list's copies, queued on the lanes.
hipError_t issue_on_lanes(const StageCopyArgs& a, LaneQueue& lanes, int64_t* tiles_copied) {
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
                                     dps.data(), n, same ? -1 : h, lanes, &c);
      if (e != hipSuccess) return e;
      copied += same ? c * a.n_kv : c;
    }
  }
  if (tiles_copied) *tiles_copied = copied;
  return hipSuccess;
}

}  // namespace

// Without lanes the copies go on the side stream.  With n lanes they start
// once the side stream's earlier work is done (the fork event), and the side
// stream's later work waits for every lane that got a copy (the join
// events).
hipError_t issue_stage_copies(const StageCopyArgs& a, int64_t* tiles_copied) {
  LaneQueue lanes;
  if (a.lanes < 2) {
    lanes.stream[0] = a.side;
    return issue_on_lanes(a, lanes, tiles_copied);
  }
  const int n = a.lanes < kMaxLanes ? a.lanes : kMaxLanes;
  std::lock_guard<std::mutex> lock(g_lanes_mutex);
  Lanes* L = nullptr;
  hipError_t e = lanes_of_current_device(n, &L);
  if (e == hipSuccess) e = hipEventRecord(L->fork, a.side);
  for (int i = 0; i < n && e == hipSuccess; ++i)
    e = hipStreamWaitEvent(L->stream[i], L->fork, 0);
  if (e != hipSuccess) return e;
  lanes.n = n;
  for (int i = 0; i < n; ++i) lanes.stream[i] = L->stream[i];
  const hipError_t issued = issue_on_lanes(a, lanes, tiles_copied);
  // join whatever was queued, also after a failed copy call
  for (int i = 0; i < n; ++i) {
    if (!lanes.used[i]) continue;
    e = hipEventRecord(L->join[i], L->stream[i]);
    if (e == hipSuccess) e = hipStreamWaitEvent(a.side, L->join[i], 0);
    if (e != hipSuccess) return e;
  }
  return issued;
}

}  // namespace rkv
