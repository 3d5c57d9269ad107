// Inner-product retrieval, exact top-k and block-table merge (gfx950).
//
// openGauss DataVec page "KV Cache Query-Based Computation Inference
// Acceleration", section "Overall Solution": the current token's query is
// scored against every offload-block representation by inner product, the
// top-K closest blocks are kept and joined with the initial-token and
// sliding-window blocks.  Defaults and the dense switch: same page,
// "Configuration Parameters".
//
// One workgroup of 1024 threads handles one (sequence, KV head):
//  1. the group's query heads are summed once (sum_g q_g . r = (sum_g q_g) . r);
//  2. eight lanes score one representation (512 B, one 128-byte line per
//     lane-octet per load), 128 representations per pass; scores become
//     order-preserving uint32 keys in LDS;
//  3. a 4-pass 8-bit radix select over the keys finds the k-th largest key T
//     (LDS histogram; one wave turns it into "how many above" with a
//     reversed wave scan);
//  4. an ordered compaction keeps every key > T and the lowest-index keys
//     == T, writing the ids ascending, and the merged page list is written
//     (init blocks, kept blocks, local blocks).
#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// fp32 -> uint32 whose unsigned order is the float order (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0 + +0 = +0 under round-to-nearest
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup (thread order).
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int t = lane < kSelWaves ? sh[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < kSelWaves; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < kSelWaves) sh[kSelWaves + lane] = s - t;
  }
  __syncthreads();
  const int r = x - v + sh[kSelWaves + wave];
  __syncthreads();  // sh may be reused by the caller's next scan
  return r;
}

// Merged page list: init blocks, the given kept offload blocks (written by
// the caller), then local blocks.  Returns the entry count.
__device__ __forceinline__ int write_fixed_entries(
    const Regions& R, int k, const int32_t* trow, int32_t* mrow) {
  const int lstart = R.local_start > R.n_init ? R.local_start : R.n_init;
  for (int i = threadIdx.x; i < R.n_init; i += blockDim.x) mrow[i] = trow[i];
  for (int i = lstart + threadIdx.x; i < R.nb; i += blockDim.x)
    mrow[R.n_init + k + (i - lstart)] = trow[i];
  return R.n_init + k + (R.nb - lstart);
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    Method m, const uint16_t* __restrict__ q, const float* __restrict__ reps,
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ prompt_lens, int max_blocks,
    int32_t* __restrict__ sel_ids, int32_t* __restrict__ n_sel, int k_cap,
    int32_t* __restrict__ merged, int32_t* __restrict__ n_merged, int m_cap) {
  extern __shared__ uint32_t keys[];  // [max_blocks]
  __shared__ float qs[kDim];
  __shared__ uint32_t hist[256];
  __shared__ int scan_sh[2 * kSelWaves];
  __shared__ int sh_digit, sh_above;

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / m.n_kv_heads, h = bh - b * m.n_kv_heads;
  const int L = clamp_len(lens[b], max_blocks * kBlock);
  const Regions R = regions_of(L, m.init_tokens, m.local_tokens);
  const int plen = prompt_lens ? prompt_lens[b] : lens[b];
  const bool dense = plen < m.dense_boundary || m.topk_ppm >= kPpmOne;
  const int n = R.n_off;
  int k = dense ? n : topk_of(n, m.topk_ppm);
  k = k < n ? k : n;

  const int32_t* trow = table + (int64_t)b * max_blocks;
  int32_t* srow = sel_ids + (int64_t)bh * k_cap;
  int32_t* mrow = merged ? merged + (int64_t)bh * m_cap : nullptr;

  if (k == n) {  // keep every offload block (dense switch, or k covers all)
    for (int r = tid; r < k; r += kSelThreads) {
      srow[r] = R.n_init + r;
      if (mrow) mrow[R.n_init + r] = trow[R.n_init + r];
    }
  } else if (k > 0) {
    // 1. summed query of the group
    if (tid < kDim) {
      const uint16_t* qh = q + ((int64_t)b * m.n_q_heads + h * m.group) * kDim;
      float s = 0.f;
      for (int g = 0; g < m.group; ++g) s += __uint_as_float((uint32_t)qh[g * kDim + tid] << 16);
      qs[tid] = s;
    }
    __syncthreads();
    // 2. scores -> keys; lane octet o = tid % 8 covers floats 4(o+8i)..+3
    const int o = tid & 7;
    float4 qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qv[i] = *reinterpret_cast<const float4*>(&qs[4 * (o + 8 * i)]);
    const float* rbase =
        reps + ((int64_t)bh * max_blocks + R.n_init) * kDim;
#pragma unroll 4
    for (int base = 0; base < n; base += kSelThreads / 8) {
      const int jj = base + (tid >> 3);
      float part = 0.f;
      if (jj < n) {
        const float4* p = reinterpret_cast<const float4*>(rbase + (int64_t)jj * kDim);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = p[o + 8 * i];
          part += v.x * qv[i].x + v.y * qv[i].y + v.z * qv[i].z + v.w * qv[i].w;
        }
      }
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 4);
      if (o == 0 && jj < n) keys[jj] = order_key(part);
    }
    __syncthreads();

    // 3. radix select of the k-th largest key, most significant digit first
    uint32_t prefix = 0, pmask = 0;
    int remaining = k;  // keys still to take among those matching prefix
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < n; j += kSelThreads) {
        const uint32_t key = keys[j];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        const int lane = tid;
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        const uint32_t s = h0 + h1 + h2 + h3;
        uint32_t incl = s;  // sum over lanes >= this lane
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_down(incl, off);
          if (lane + off < 64) incl += y;
        }
        const uint32_t a3 = incl - s;  // count in bins above 4*lane+3
        const uint32_t a2 = a3 + h3, a1 = a2 + h2, a0 = a1 + h1;
        const uint32_t rem = (uint32_t)remaining;
        if (a3 < rem && rem <= a3 + h3) { sh_digit = 4 * lane + 3; sh_above = (int)a3; }
        if (a2 < rem && rem <= a2 + h2) { sh_digit = 4 * lane + 2; sh_above = (int)a2; }
        if (a1 < rem && rem <= a1 + h1) { sh_digit = 4 * lane + 1; sh_above = (int)a1; }
        if (a0 < rem && rem <= a0 + h0) { sh_digit = 4 * lane;     sh_above = (int)a0; }
      }
      __syncthreads();
      remaining -= sh_above;
      prefix |= (uint32_t)sh_digit << shift;
      pmask |= 255u << shift;
    }
    const uint32_t T = prefix;  // the k-th largest key; take `remaining` of == T

    // 4. ordered compaction over contiguous per-thread index ranges
    const int per = (n + kSelThreads - 1) / kSelThreads;
    const int j0 = tid * per;
    const int j1 = j0 + per < n ? j0 + per : n;
    int gt = 0, eq = 0;
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = keys[j];
      gt += key > T;
      eq += key == T;
    }
    const int eq_before = block_exclusive_scan(eq, scan_sh);
    int take_eq = remaining - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
    int out = block_exclusive_scan(gt + take_eq, scan_sh);
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = keys[j];
      bool keep = key > T;
      if (key == T && take_eq > 0) {
        keep = true;
        --take_eq;
      }
      if (keep) {
        srow[out] = R.n_init + j;
        if (mrow) mrow[R.n_init + out] = trow[R.n_init + j];
        ++out;
      }
    }
  }
  if (mrow) {
    const int cnt = write_fixed_entries(R, k, trow, mrow);
    if (tid == 0) n_merged[bh] = cnt;
  }
  if (tid == 0) n_sel[bh] = k;
}

// Standalone merge from given selections.  Ids outside the offload range
// are written as page -1 (the attention kernel skips such entries).
__global__ __launch_bounds__(256) void merge_kernel(
    Method m, const int32_t* __restrict__ table, int max_blocks,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ sel_ids,
    const int32_t* __restrict__ n_sel, int k_cap,
    int32_t* __restrict__ merged, int32_t* __restrict__ n_merged, int m_cap) {
  const int bh = blockIdx.x;
  const int b = bh / m.n_kv_heads;
  const int L = clamp_len(lens[b], max_blocks * kBlock);
  const Regions R = regions_of(L, m.init_tokens, m.local_tokens);
  int k = n_sel[bh];
  k = k < 0 ? 0 : k;
  k = k < R.n_off ? k : R.n_off;
  k = k < k_cap ? k : k_cap;
  const int32_t* trow = table + (int64_t)b * max_blocks;
  const int32_t* srow = sel_ids + (int64_t)bh * k_cap;
  int32_t* mrow = merged + (int64_t)bh * m_cap;
  for (int r = threadIdx.x; r < k; r += blockDim.x) {
    const int j = srow[r];
    const bool ok = j >= R.n_init && j < R.n_init + R.n_off;
    mrow[R.n_init + r] = ok ? trow[j] : -1;
  }
  const int cnt = write_fixed_entries(R, k, trow, mrow);
  if (threadIdx.x == 0) n_merged[bh] = cnt;
}

}  // namespace

hipError_t launch_select(const Method& m, const uint16_t* q, const float* reps,
                         const int32_t* table, const int32_t* lens,
                         const int32_t* prompt_lens, int batch, int max_blocks,
                         int32_t* sel_ids, int32_t* n_sel, int k_cap,
                         int32_t* merged, int32_t* n_merged, int m_cap,
                         hipStream_t stream) {
  const int groups = batch * m.n_kv_heads;
  if (groups == 0) return hipSuccess;
  const size_t lds = (size_t)max_blocks * sizeof(uint32_t);
  hipLaunchKernelGGL(select_kernel, dim3(groups), dim3(kSelThreads), lds,
                     stream, m, q, reps, table, lens, prompt_lens, max_blocks,
                     sel_ids, n_sel, k_cap, merged, n_merged, m_cap);
  return hipGetLastError();
}

hipError_t launch_merge(const Method& m, const int32_t* table, int max_blocks,
                        const int32_t* lens, const int32_t* sel_ids,
                        const int32_t* n_sel, int k_cap, int batch,
                        int32_t* merged, int32_t* n_merged, int m_cap,
                        hipStream_t stream) {
  const int groups = batch * m.n_kv_heads;
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(groups), dim3(256), 0, stream, m,
                     table, max_blocks, lens, sel_ids, n_sel, k_cap, merged,
                     n_merged, m_cap);
  return hipGetLastError();
}

}  // namespace rkv
