// Block representation vectors and decode-token append (gfx950).
//
// A representation is the fp32 mean of a block's 128 keys per KV head
// (openGauss DataVec page "KV Cache Query-Based Computation Inference
// Acceleration", sections "Feature Description" / "Overall Solution":
// representation vectors are extracted block by block).
//
// One wave reduces one (page, head) tile of 32 KiB.  Lane (c, g) with
// c = lane % 16 and g = lane / 16 reads the 16-byte chunk c (dims 8c..8c+7)
// of rows g, g+4, ..., g+124: each load instruction covers four whole
// 256-byte rows, 1 KiB contiguous.  Column sums are kept in fp32 and the
// four row groups are folded with two cross-lane adds.
#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

struct Sum8 {
  float v[8];
};

__device__ __forceinline__ void add_chunk(Sum8& s, uint4 w) {
  s.v[0] += bf16lo(w.x);
  s.v[1] += bf16hi(w.x);
  s.v[2] += bf16lo(w.y);
  s.v[3] += bf16hi(w.y);
  s.v[4] += bf16lo(w.z);
  s.v[5] += bf16hi(w.z);
  s.v[6] += bf16lo(w.w);
  s.v[7] += bf16hi(w.w);
}

// Fold the four row groups and write the mean of dims 8c..8c+7 (lanes 0-15).
__device__ __forceinline__ void finish_rep(Sum8& s, int lane, float* dst) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s.v[i] += __shfl_xor(s.v[i], 16);
    s.v[i] += __shfl_xor(s.v[i], 32);
  }
  if (lane < 16) {
    const float inv = 1.0f / 128.0f;  // exact power of two
    float4* o = reinterpret_cast<float4*>(dst + lane * 8);
    o[0] = make_float4(s.v[0] * inv, s.v[1] * inv, s.v[2] * inv, s.v[3] * inv);
    o[1] = make_float4(s.v[4] * inv, s.v[5] * inv, s.v[6] * inv, s.v[7] * inv);
  }
}

__global__ __launch_bounds__(256) void build_reps_kernel(
    const uint16_t* __restrict__ k_pages, int64_t n_pages,
    const int32_t* __restrict__ table, int max_blocks,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ block_begin,
    int batch, int n_kv, float* __restrict__ reps) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)batch * max_blocks * n_kv;
  if (item >= total) return;
  const int h = (int)(item % n_kv);
  const int64_t rest = item / n_kv;
  const int j = (int)(rest % max_blocks);
  const int b = (int)(rest / max_blocks);
  // the page id is requested together with the lengths (j < max_blocks
  // always holds), so the tile's loads wait for one round trip, not two
  const int page = table[(int64_t)b * max_blocks + j];
  const int L = clamp_len(lens[b], max_blocks * kBlock);
  int j0 = block_begin ? block_begin[b] : 0;
  j0 = j0 < 0 ? 0 : j0;
  if (j < j0 || j >= (L >> 7)) return;
  if ((uint64_t)(int64_t)page >= (uint64_t)n_pages) {
    report_bounds(kBoundsPage, page);
    return;
  }
  const uint16_t* K = k_pages + ((int64_t)page * n_kv + h) * (kBlock * kDim);
  const int c = lane & 15, g = lane >> 4;
  // all 32 loads of the tile in flight at once, then summed in row order
  uint4 w[32];
#pragma unroll
  for (int it = 0; it < 32; ++it)
    w[it] = *reinterpret_cast<const uint4*>(K + (it * 4 + g) * kDim + c * 8);
  Sum8 s = {};
#pragma unroll
  for (int it = 0; it < 32; ++it) add_chunk(s, w[it]);
  finish_rep(s, lane,
             reps + (((int64_t)b * n_kv + h) * max_blocks + j) * kDim);
}

// One wave per (sequence, KV head): write K row and V column of slot L-1;
// when the slot is the block's last, also write that block's representation
// (rows 0..126 from the pool, row 127 from k_new).
__global__ __launch_bounds__(64) void append_kv_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_pages, uint16_t* __restrict__ v_pages,
    int64_t n_pages, const int32_t* __restrict__ table, int max_blocks,
    const int32_t* __restrict__ lens, int n_kv, float* __restrict__ reps) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / n_kv, h = bh - b * n_kv;
  const int L = clamp_len(lens[b], max_blocks * kBlock);
  if (L <= 0) return;
  const int pos = L - 1, j = pos >> 7, slot = pos & 127;
  const int page = table[(int64_t)b * max_blocks + j];
  if ((uint64_t)(int64_t)page >= (uint64_t)n_pages) {
    report_bounds(kBoundsPage, page);
    return;
  }
  const int64_t base = ((int64_t)page * n_kv + h) * (kBlock * kDim);
  const uint16_t* kn = k_new + (int64_t)bh * kDim;
  const uint16_t* vn = v_new + (int64_t)bh * kDim;
  reinterpret_cast<uint32_t*>(k_pages + base + slot * kDim)[lane] =
      reinterpret_cast<const uint32_t*>(kn)[lane];
  v_pages[base + lane * kBlock + slot] = vn[lane];
  v_pages[base + (lane + 64) * kBlock + slot] = vn[lane + 64];
  if (slot != kBlock - 1 || reps == nullptr) return;
  const uint16_t* K = k_pages + base;
  const int c = lane & 15, g = lane >> 4;
  Sum8 s = {};
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const int t = it * 4 + g;
    const uint16_t* src = (t == kBlock - 1) ? kn : K + t * kDim;
    add_chunk(s, *reinterpret_cast<const uint4*>(src + c * 8));
  }
  finish_rep(s, lane, reps + ((int64_t)bh * max_blocks + j) * kDim);
}


// Streaming-read probe (a measurement helper, not part of the method): one
// wave per 16 KiB chunk, chunks dealt round robin over the grid, sixteen
// 16-byte loads in flight per lane (the access shape of the attention
// kernel's tiles); the data is folded into one XOR per wave so the loads
// cannot be elided.
__global__ __launch_bounds__(64) void read_probe_kernel(const uint4* __restrict__ src,
                                                        int64_t n16,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  const int64_t n_chunks = n16 / 1024;
  uint32_t x = 0;
  for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const uint4* p = src + c * 1024;
    uint4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = p[u * 64 + lane];
#pragma unroll
    for (int u = 0; u < 16; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (blockIdx.x == 0) {
    for (int64_t i = n_chunks * 1024 + lane; i < n16; i += 64) {
      const uint4 v = src[i];
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) atomicXor(sink, x);
}

}  // namespace

hipError_t launch_build_reps(const uint16_t* k_pages, int64_t n_pages,
                             const int32_t* table, int max_blocks,
                             const int32_t* lens, const int32_t* block_begin,
                             int batch, int n_kv_heads, float* reps,
                             hipStream_t stream) {
  const int64_t items = (int64_t)batch * max_blocks * n_kv_heads;
  if (items == 0) return hipSuccess;
  const int64_t wgs = (items + 3) / 4;
  hipLaunchKernelGGL(build_reps_kernel, dim3((unsigned)wgs), dim3(256), 0,
                     stream, k_pages, n_pages, table, max_blocks, lens,
                     block_begin, batch, n_kv_heads, reps);
  return hipGetLastError();
}

hipError_t launch_append_kv(const uint16_t* k_new, const uint16_t* v_new,
                            uint16_t* k_pages, uint16_t* v_pages,
                            int64_t n_pages, const int32_t* table,
                            int max_blocks, const int32_t* lens, int batch,
                            int n_kv_heads, float* reps, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kv_kernel, dim3(batch * n_kv_heads), dim3(64), 0,
                     stream, k_new, v_new, k_pages, v_pages, n_pages, table,
                     max_blocks, lens, n_kv_heads, reps);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                             int n_cu, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  // four waves per compute unit (one per SIMD), as the attention split
  const int64_t waves = (int64_t)(n_cu > 0 ? n_cu : 256) * 4;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)waves), dim3(64), 0, stream,
                     static_cast<const uint4*>(buf), n16, sink);
  return hipGetLastError();
}

RKV_BOUNDS_SETTER(set_bounds_word_reps)

}  // namespace rkv
