// Host tier: stage selected offload blocks from pinned host memory into HBM
// (gfx950).
//
// openGauss DataVec page "KV Cache Query-Based Computation Inference
// Acceleration", sections "Feature Description" and "Overall Solution": the
// offload part of the KV cache lives in host DDR, and at each decode round
// the blocks picked by the retrieval step are loaded back into HBM before
// attention.  Sections "Configuration Parameters": sequences longer than the
// offload boundary keep their offload region on the host.
//
// One 256-thread workgroup copies the K tile and the V tile (32 KiB each) of
// one selected (sequence, KV head, rank r) block from the host pool to the
// HBM staging page stage_page0 + b * k_cap + r.  The kernel reads the pinned
// host memory directly (16-byte loads, all issued before the first store,
// 16 per thread), so a whole step's staging is one launch with no host
// round trip for the selected ids.
#include "rkv.h"
#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kStageThreads = 256;
constexpr int kTile16 = kBlock * kDim * 2 / 16;  // 16-byte pieces per tile

// K and V tiles (32 KiB each) from src to dst (16-byte piece offsets), every
// load issued before the first store.
__device__ __forceinline__ void copy_tiles(const uint4* __restrict__ src_k,
                                           const uint4* __restrict__ src_v,
                                           int64_t src, uint4* __restrict__ dst_k,
                                           uint4* __restrict__ dst_v, int64_t dst) {
  constexpr int kPer = kTile16 / kStageThreads;  // 8 pieces per thread per tile
  uint4 kv[kPer], vv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    kv[u] = src_k[src + u * kStageThreads + threadIdx.x];
    vv[u] = src_v[src + u * kStageThreads + threadIdx.x];
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    dst_k[dst + u * kStageThreads + threadIdx.x] = kv[u];
    dst_v[dst + u * kStageThreads + threadIdx.x] = vv[u];
  }
}

// Merged-list entries of the init and local blocks (from the block table).
__device__ __forceinline__ int write_fixed_entries_stage(const Regions& R, int k,
                                                         const int32_t* trow,
                                                         int32_t* mrow) {
  const int lstart = R.local_start > R.n_init ? R.local_start : R.n_init;
  for (int i = threadIdx.x; i < R.n_init; i += blockDim.x) mrow[i] = trow[i];
  for (int i = lstart + threadIdx.x; i < R.nb; i += blockDim.x)
    mrow[R.n_init + k + (i - lstart)] = trow[i];
  return R.n_init + k + (R.nb - lstart);
}

__global__ __launch_bounds__(kStageThreads) void stage_kernel(
    const uint4* __restrict__ host_k, const uint4* __restrict__ host_v,
    int64_t n_host_pages, const int32_t* __restrict__ host_table,
    int max_blocks, const int32_t* __restrict__ sel_ids,
    const int32_t* __restrict__ n_sel, int k_cap, int n_kv,
    uint4* __restrict__ k_pages, uint4* __restrict__ v_pages, int64_t n_pages,
    int64_t stage_page0) {
  const int64_t item = blockIdx.x;  // (bh, r), r fastest
  const int r = (int)(item % k_cap);
  const int bh = (int)(item / k_cap);
  const int b = bh / n_kv, h = bh - b * n_kv;
  int ns = n_sel[bh];
  if (r == 0 && (ns < 0 || ns > k_cap)) report_bounds(kBoundsCount, ns);
  ns = ns < k_cap ? ns : k_cap;
  if (r >= ns) return;
  const int j = sel_ids[(int64_t)bh * k_cap + r];
  if (j < 0 || j >= max_blocks) {
    report_bounds(kBoundsBlock, j);
    return;
  }
  const int hp = host_table[(int64_t)b * max_blocks + j];
  if ((uint64_t)(int64_t)hp >= (uint64_t)n_host_pages) {
    if (hp != -1) report_bounds(kBoundsHostPage, hp);  // -1: block in HBM
    return;
  }
  const int64_t dst_page = stage_page0 + (int64_t)b * k_cap + r;
  if (dst_page < 0 || dst_page >= n_pages) return;
  copy_tiles(host_k, host_v, ((int64_t)hp * n_kv + h) * kTile16, k_pages, v_pages,
             (dst_page * n_kv + h) * kTile16);
}


// ---------------------------------------------------------------------------
// Residency across steps.  Staging slot r (of slot_cap >= k_cap) of
// (sequence b, KV head h) is the head-h slice of page
// stage_page0 + b * slot_cap + r; slot_ids[b][h][r] names the logical block
// whose K/V the slot holds (-1: none).  A kept block that already sits in a
// slot is not copied again; the blocks new to the kept set take, in
// ascending order, the slots that hold no kept block, first-in first-out:
// in slot order starting at the list's cursor, which then moves past the
// last slot filled.  With more slots than kept blocks, a dropped block
// stays resident for a while and costs no copy if it is kept again.
// Results are those of staging every kept block: the merged table points
// each kept host-resident block at its slot.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;

struct ResArgs {
  int n_kv, init_tokens, local_tokens;
  const int32_t* host_table;
  const int32_t* table;
  const int32_t* lens;
  int max_blocks;
  const int32_t* sel_ids;
  const int32_t* n_sel;
  int k_cap;
  int slot_cap;
  int32_t* slot_ids;
  int32_t* slot_cursor;  // [bh]: next slot to fill, first-in first-out
  int2* copies;       // [bh][k_cap]: (block, slot) to copy
  int32_t* n_copies;  // [bh]
  int32_t* n_staged;  // optional copy of n_copies
  int64_t stage_page0;
  int32_t* merged;
  int32_t* n_merged;
  int m_cap;
  // split mode (non-null): merged keeps the entries whose pages are in HBM
  // before this call's copies; merged_new [bh][k_cap] gets the staging pages
  // of the blocks copied now
  int32_t* merged_new;
  int32_t* n_new;
};

// Position of this thread's flag among the set flags of the workgroup (in
// thread order) and the total; `sh` holds kPlanWaves words.
__device__ __forceinline__ int plan_scan(bool flag, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  if (lane == 0) sh[wave] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int c = sh[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + below;
}

__global__ __launch_bounds__(kPlanThreads) void stage_plan_kernel(ResArgs a) {
  __shared__ uint32_t selbits[RKV_MAX_BLOCKS / 32];
  __shared__ uint32_t heldbits[RKV_MAX_BLOCKS / 32];
  __shared__ uint16_t rank_of[RKV_MAX_BLOCKS];
  __shared__ uint16_t free_slots[RKV_MAX_BLOCKS];
  __shared__ uint16_t new_ranks[RKV_MAX_BLOCKS];
  __shared__ int sh[kPlanWaves];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.n_kv;
  const int max_blocks = a.max_blocks;
  const int k_cap = a.k_cap;
  const int S = a.slot_cap;
  const int L = clamp_len(a.lens[b], max_blocks * kBlock);
  const Regions R = regions_of(L, a.init_tokens, a.local_tokens);
  int k = a.n_sel[bh];
  if (tid == 0 && (k < 0 || k > R.n_off || k > k_cap)) report_bounds(kBoundsCount, k);
  k = k < 0 ? 0 : k;
  k = k < R.n_off ? k : R.n_off;
  k = k < k_cap ? k : k_cap;
  const int32_t* trow = a.table + (int64_t)b * max_blocks;
  const int32_t* hrow = a.host_table + (int64_t)b * max_blocks;
  const int32_t* srow = a.sel_ids + (int64_t)bh * k_cap;
  int32_t* slots = a.slot_ids + (int64_t)bh * S;
  int32_t* mrow = a.merged + (int64_t)bh * a.m_cap;
  const int64_t page0 = a.stage_page0 + (int64_t)b * S;
  int cursor = a.slot_cursor[bh];
  cursor = (cursor < 0 || cursor >= S) ? 0 : cursor;
  auto in_off = [&](int j) { return j >= R.n_init && j < R.n_init + R.n_off; };
  auto bit = [](const uint32_t* bits, int j) { return (bits[j >> 5] >> (j & 31)) & 1u; };

  for (int i = tid; i < RKV_MAX_BLOCKS / 32; i += kPlanThreads) {
    selbits[i] = 0u;
    heldbits[i] = 0u;
  }
  __syncthreads();
  // the kept set and each kept block's rank
  for (int q = tid; q < k; q += kPlanThreads) {
    const int j = srow[q];
    if (in_off(j)) {
      atomicOr(&selbits[j >> 5], 1u << (j & 31));
      rank_of[j] = (uint16_t)q;
    }
  }
  __syncthreads();
  // slots whose block stays kept keep it (one slot per block); the others
  // are free, listed first-in first-out (slot order from the cursor)
  int n_free = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int i = base + tid;
    const int r = i < S ? (cursor + i) % S : 0;
    bool is_free = false;
    if (i < S) {
      const int j = slots[r];
      bool keep = j >= 0 && j < max_blocks && in_off(j) && bit(selbits, j) &&
                  hrow[j] >= 0;
      if (keep) keep = (atomicOr(&heldbits[j >> 5], 1u << (j & 31)) &
                        (1u << (j & 31))) == 0u;
      if (keep) {
        mrow[R.n_init + rank_of[j]] = (int32_t)(page0 + r);
      } else {
        is_free = true;
      }
    }
    int tot;
    const int pos = plan_scan(is_free, sh, &tot);
    if (is_free) free_slots[n_free + pos] = (uint16_t)r;
    n_free += tot;
  }
  // kept blocks: in HBM already (table page), held in a slot (done above),
  // or new (ascending rank)
  int n_new = 0;
  for (int base = 0; base < k; base += kPlanThreads) {
    const int q = base + tid;
    bool is_new = false;
    if (q < k) {
      const int j = srow[q];
      if (!in_off(j)) {
        mrow[R.n_init + q] = -1;
      } else if (hrow[j] < 0) {
        mrow[R.n_init + q] = trow[j];
      } else {
        is_new = !bit(heldbits, j);
      }
    }
    int tot;
    const int pos = plan_scan(is_new, sh, &tot);
    if (is_new) new_ranks[n_new + pos] = (uint16_t)q;
    n_new += tot;
  }
  // (LDS lists are visible: plan_scan ends with a barrier)
  const int n_cp = n_new < n_free ? n_new : n_free;
  int2* crow = a.copies + (int64_t)bh * k_cap;
  for (int i = tid; i < n_cp; i += kPlanThreads) {
    const int q = new_ranks[i], r = free_slots[i];
    const int j = srow[q];
    slots[r] = j;
    crow[i] = make_int2(j, r);
    mrow[R.n_init + q] = (int32_t)(page0 + r);
  }
  // more kept host blocks than slots (slot_cap below the kept count): the
  // blocks without a slot get page -1 and the list reports n_staged = -1
  for (int i = n_cp + tid; i < n_new; i += kPlanThreads)
    mrow[R.n_init + new_ranks[i]] = -1;
  // a free slot that is not reused keeps its block's data and its id, so
  // the block costs no copy if it is kept again later
  if (tid == 0 && n_cp > 0) a.slot_cursor[bh] = (free_slots[n_cp - 1] + 1) % S;
  const int cnt = write_fixed_entries_stage(R, k, trow, mrow);
  int n_res = cnt;
  if (a.merged_new) {  // uniform: split the table
    // positions of the entries copied now (the kept-block bits are no
    // longer needed: reused as a position bitmap)
    __syncthreads();
    for (int i = tid; i < RKV_MAX_BLOCKS / 32; i += kPlanThreads) selbits[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n_cp; i += kPlanThreads) {
      const int e = R.n_init + new_ranks[i];
      atomicOr(&selbits[e >> 5], 1u << (e & 31));
    }
    int32_t* nrow = a.merged_new + (int64_t)bh * k_cap;
    for (int i = tid; i < n_cp; i += kPlanThreads)
      nrow[i] = (int32_t)(page0 + free_slots[i]);
    __syncthreads();
    // the other entries, in order, compacted in place (every value of a
    // round is read before the round's scan, whose barrier precedes the
    // writes, and a round writes only below its own first entry)
    n_res = 0;
    for (int base = 0; base < cnt; base += kPlanThreads) {
      const int e = base + tid;
      const int v = e < cnt ? mrow[e] : -1;
      const bool keep = e < cnt && v != -1 && !bit(selbits, e);
      int tot;
      const int pos = plan_scan(keep, sh, &tot);
      if (keep) mrow[n_res + pos] = v;
      n_res += tot;
    }
  }
  if (tid == 0) {
    a.n_merged[bh] = n_res;
    a.n_copies[bh] = n_cp;
    if (a.n_staged) a.n_staged[bh] = n_new > n_cp ? -1 : n_cp;
    if (a.merged_new) a.n_new[bh] = n_cp;
  }
}

// Copy item (bh, i < n_copies[bh]): the K and V tiles of head h of block j
// from the host pools to slot r.
__global__ __launch_bounds__(kStageThreads) void stage_copy_kernel(
    const uint4* __restrict__ host_k, const uint4* __restrict__ host_v,
    int64_t n_host_pages, const int32_t* __restrict__ host_table,
    int max_blocks, const int2* __restrict__ copies,
    const int32_t* __restrict__ n_copies, int k_cap, int slot_cap, int n_kv,
    uint4* __restrict__ k_pages, uint4* __restrict__ v_pages, int64_t n_pages,
    int64_t stage_page0) {
  const int64_t item = blockIdx.x;  // (bh, i), i fastest
  const int i = (int)(item % k_cap);
  const int bh = (int)(item / k_cap);
  const int b = bh / n_kv, h = bh - b * n_kv;
  if (i >= n_copies[bh]) return;
  const int2 c = copies[(int64_t)bh * k_cap + i];
  if (c.x < 0 || c.x >= max_blocks || c.y < 0 || c.y >= slot_cap) return;
  const int hp = host_table[(int64_t)b * max_blocks + c.x];
  if ((uint64_t)(int64_t)hp >= (uint64_t)n_host_pages) {
    report_bounds(kBoundsHostPage, hp);
    return;
  }
  const int64_t dst_page = stage_page0 + (int64_t)b * slot_cap + c.y;
  if (dst_page < 0 || dst_page >= n_pages) return;
  copy_tiles(host_k, host_v, ((int64_t)hp * n_kv + h) * kTile16, k_pages, v_pages,
             (dst_page * n_kv + h) * kTile16);
}

// Prefill-time offload: item (b, j, h) copies head h of the device page of
// offload block j of sequence b (blocks [n_init, local_start) for its
// length) to host page host_table[b][j] of the pinned pools, K and V tiles,
// every load issued before the first store.  The copies are bound by the
// host link, so a small grid walks the items: the rest of the GPU stays free
// for the representation build that runs beside it.
__global__ __launch_bounds__(kStageThreads) void offload_kernel(
    const uint4* __restrict__ k_pages, const uint4* __restrict__ v_pages,
    int64_t n_pages, const int32_t* __restrict__ table, int max_blocks,
    const int32_t* __restrict__ lens, int batch, int n_kv, int init_tokens,
    int local_tokens, const int32_t* __restrict__ host_table,
    uint4* __restrict__ host_k, uint4* __restrict__ host_v, int64_t n_host_pages) {
  const int64_t items = (int64_t)batch * max_blocks * n_kv;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    // (b, j, h), h fastest
    const int h = (int)(item % n_kv);
    const int64_t rest = item / n_kv;
    const int j = (int)(rest % max_blocks);
    const int b = (int)(rest / max_blocks);
    const int L = clamp_len(lens[b], max_blocks * kBlock);
    const Regions R = regions_of(L, init_tokens, local_tokens);
    if (j < R.n_init || j >= R.n_init + R.n_off) continue;
    const int hp = host_table[(int64_t)b * max_blocks + j];
    if ((uint64_t)(int64_t)hp >= (uint64_t)n_host_pages) {
      if (hp != -1) report_bounds(kBoundsHostPage, hp);  // -1: block stays in HBM
      continue;
    }
    const int page = table[(int64_t)b * max_blocks + j];
    if ((uint64_t)(int64_t)page >= (uint64_t)n_pages) {
      report_bounds(kBoundsPage, page);
      continue;
    }
    copy_tiles(k_pages, v_pages, ((int64_t)page * n_kv + h) * kTile16, host_k, host_v,
               ((int64_t)hp * n_kv + h) * kTile16);
  }
}

}  // namespace

hipError_t launch_stage(const uint16_t* host_k, const uint16_t* host_v,
                        int64_t n_host_pages, const int32_t* host_table,
                        int max_blocks, const int32_t* sel_ids,
                        const int32_t* n_sel, int k_cap, int batch, int n_kv,
                        uint16_t* k_pages, uint16_t* v_pages, int64_t n_pages,
                        int64_t stage_page0, hipStream_t stream) {
  const int64_t items = (int64_t)batch * n_kv * k_cap;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(stage_kernel, dim3((unsigned)items), dim3(kStageThreads), 0,
                     stream, reinterpret_cast<const uint4*>(host_k),
                     reinterpret_cast<const uint4*>(host_v), n_host_pages,
                     host_table, max_blocks, sel_ids, n_sel, k_cap, n_kv,
                     reinterpret_cast<uint4*>(k_pages),
                     reinterpret_cast<uint4*>(v_pages), n_pages, stage_page0);
  return hipGetLastError();
}

size_t resident_workspace_bytes(int batch, int n_kv, int k_cap) {
  const size_t lists = (size_t)batch * n_kv;
  return lists * k_cap * sizeof(int2) + (lists * sizeof(int32_t) + 255) / 256 * 256;
}

namespace {

ResArgs resident_args(const Method& m, const int32_t* host_table, const int32_t* table,
                      const int32_t* lens, int max_blocks, const int32_t* sel_ids,
                      const int32_t* n_sel, int k_cap, int batch, int slot_cap,
                      int32_t* slot_ids, int32_t* slot_cursor, int64_t stage_page0,
                      int32_t* merged, int32_t* n_merged, int m_cap,
                      int32_t* n_staged, void* workspace) {
  const int lists = batch * m.n_kv_heads;
  ResArgs a;
  a.n_kv = m.n_kv_heads;
  a.init_tokens = m.init_tokens;
  a.local_tokens = m.local_tokens;
  a.host_table = host_table;
  a.table = table;
  a.lens = lens;
  a.max_blocks = max_blocks;
  a.sel_ids = sel_ids;
  a.n_sel = n_sel;
  a.k_cap = k_cap;
  a.slot_cap = slot_cap;
  a.slot_ids = slot_ids;
  a.slot_cursor = slot_cursor;
  a.copies = static_cast<int2*>(workspace);
  a.n_copies = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                          (size_t)lists * k_cap * sizeof(int2));
  a.n_staged = n_staged;
  a.stage_page0 = stage_page0;
  a.merged = merged;
  a.n_merged = n_merged;
  a.m_cap = m_cap;
  a.merged_new = nullptr;
  a.n_new = nullptr;
  return a;
}

}  // namespace

hipError_t launch_stage_plan(const Method& m, const int32_t* host_table,
                             const int32_t* table, const int32_t* lens,
                             int max_blocks, const int32_t* sel_ids,
                             const int32_t* n_sel, int k_cap, int batch,
                             int slot_cap, int32_t* slot_ids, int32_t* slot_cursor,
                             int64_t stage_page0, int32_t* merged,
                             int32_t* n_merged, int m_cap, int32_t* n_staged,
                             void* workspace, hipStream_t stream, int32_t* merged_new,
                             int32_t* n_new) {
  const int lists = batch * m.n_kv_heads;
  if (lists == 0) return hipSuccess;
  ResArgs a = resident_args(m, host_table, table, lens, max_blocks, sel_ids, n_sel,
                            k_cap, batch, slot_cap, slot_ids, slot_cursor, stage_page0,
                            merged, n_merged, m_cap, n_staged, workspace);
  a.merged_new = merged_new;
  a.n_new = n_new;
  hipLaunchKernelGGL(stage_plan_kernel, dim3(lists), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_stage_copy(const Method& m, const uint16_t* host_k,
                             const uint16_t* host_v, int64_t n_host_pages,
                             const int32_t* host_table, int max_blocks, int k_cap,
                             int batch, int slot_cap, uint16_t* k_pages,
                             uint16_t* v_pages, int64_t n_pages, int64_t stage_page0,
                             const void* workspace, hipStream_t stream) {
  const int lists = batch * m.n_kv_heads;
  if (lists == 0) return hipSuccess;
  const int2* copies = static_cast<const int2*>(workspace);
  const int32_t* n_copies = reinterpret_cast<const int32_t*>(
      static_cast<const char*>(workspace) + (size_t)lists * k_cap * sizeof(int2));
  const int64_t items = (int64_t)lists * k_cap;
  hipLaunchKernelGGL(stage_copy_kernel, dim3((unsigned)items), dim3(kStageThreads), 0,
                     stream, reinterpret_cast<const uint4*>(host_k),
                     reinterpret_cast<const uint4*>(host_v), n_host_pages, host_table,
                     max_blocks, copies, n_copies, k_cap, slot_cap, m.n_kv_heads,
                     reinterpret_cast<uint4*>(k_pages), reinterpret_cast<uint4*>(v_pages),
                     n_pages, stage_page0);
  return hipGetLastError();
}

hipError_t launch_stage_resident(const Method& m, const uint16_t* host_k,
                                 const uint16_t* host_v, int64_t n_host_pages,
                                 const int32_t* host_table, const int32_t* table,
                                 const int32_t* lens, int max_blocks,
                                 const int32_t* sel_ids, const int32_t* n_sel,
                                 int k_cap, int batch, int slot_cap,
                                 int32_t* slot_ids, int32_t* slot_cursor,
                                 uint16_t* k_pages, uint16_t* v_pages,
                                 int64_t n_pages, int64_t stage_page0,
                                 int32_t* merged, int32_t* n_merged, int m_cap,
                                 int32_t* n_staged, void* workspace,
                                 hipStream_t stream) {
  const int lists = batch * m.n_kv_heads;
  if (lists == 0) return hipSuccess;
  hipError_t e = launch_stage_plan(m, host_table, table, lens, max_blocks, sel_ids,
                                   n_sel, k_cap, batch, slot_cap, slot_ids, slot_cursor,
                                   stage_page0, merged, n_merged, m_cap, n_staged,
                                   workspace, stream);
  if (e != hipSuccess) return e;
  const ResArgs a = resident_args(m, host_table, table, lens, max_blocks, sel_ids, n_sel,
                                  k_cap, batch, slot_cap, slot_ids, slot_cursor,
                                  stage_page0, merged, n_merged, m_cap, n_staged,
                                  workspace);
  const int64_t items = (int64_t)lists * k_cap;
  hipLaunchKernelGGL(stage_copy_kernel, dim3((unsigned)items), dim3(kStageThreads), 0,
                     stream, reinterpret_cast<const uint4*>(host_k),
                     reinterpret_cast<const uint4*>(host_v), n_host_pages, host_table,
                     max_blocks, a.copies, a.n_copies, k_cap, slot_cap, m.n_kv_heads,
                     reinterpret_cast<uint4*>(k_pages), reinterpret_cast<uint4*>(v_pages),
                     n_pages, stage_page0);
  return hipGetLastError();
}

hipError_t launch_offload(const Method& m, const uint16_t* k_pages,
                          const uint16_t* v_pages, int64_t n_pages,
                          const int32_t* table, int max_blocks, const int32_t* lens,
                          int batch, const int32_t* host_table, uint16_t* host_k,
                          uint16_t* host_v, int64_t n_host_pages,
                          hipStream_t stream) {
  const int64_t items = (int64_t)batch * max_blocks * m.n_kv_heads;
  if (items == 0) return hipSuccess;
  // 64 workgroups keep 4 MiB of copies in flight, far more than the host
  // link needs, and leave the other compute units free
  const int64_t wgs = items < 64 ? items : 64;
  hipLaunchKernelGGL(offload_kernel, dim3((unsigned)wgs), dim3(kStageThreads), 0,
                     stream, reinterpret_cast<const uint4*>(k_pages),
                     reinterpret_cast<const uint4*>(v_pages), n_pages, table,
                     max_blocks, lens, batch, m.n_kv_heads, m.init_tokens,
                     m.local_tokens, host_table, reinterpret_cast<uint4*>(host_k),
                     reinterpret_cast<uint4*>(host_v), n_host_pages);
  return hipGetLastError();
}

RKV_BOUNDS_SETTER(set_bounds_word_stage)

}  // namespace rkv
