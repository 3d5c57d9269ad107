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
#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kStageThreads = 256;
constexpr int kTile16 = kBlock * kDim * 2 / 16;  // 16-byte pieces per tile

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
  ns = ns < k_cap ? ns : k_cap;
  if (r >= ns) return;
  const int j = sel_ids[(int64_t)bh * k_cap + r];
  if (j < 0 || j >= max_blocks) return;
  const int hp = host_table[(int64_t)b * max_blocks + j];
  if ((uint64_t)(int64_t)hp >= (uint64_t)n_host_pages) return;
  const int64_t dst_page = stage_page0 + (int64_t)b * k_cap + r;
  if (dst_page < 0 || dst_page >= n_pages) return;
  const int64_t src = ((int64_t)hp * n_kv + h) * kTile16;
  const int64_t dst = (dst_page * n_kv + h) * kTile16;
  constexpr int kPer = kTile16 / kStageThreads;  // 8 pieces per thread per tile
  uint4 kv[kPer], vv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    kv[u] = host_k[src + u * kStageThreads + threadIdx.x];
    vv[u] = host_v[src + u * kStageThreads + threadIdx.x];
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    k_pages[dst + u * kStageThreads + threadIdx.x] = kv[u];
    v_pages[dst + u * kStageThreads + threadIdx.x] = vv[u];
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

}  // namespace rkv
