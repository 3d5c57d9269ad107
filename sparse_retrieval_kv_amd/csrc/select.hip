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
//  3. one wave (no workgroup barriers) runs a 4-pass 8-bit radix select over
//     the keys to find the k-th largest key T (LDS histogram, reversed wave
//     scan);
//  4. the same wave compacts in index order with ballots: every key > T and
//     the lowest-index keys == T, ids ascending; the merged page list gets
//     the init blocks, the kept blocks and the local blocks.
#include "rkv.h"
#include "rkv_device.h"
#include "rkv_internal.h"

namespace rkv {
namespace {

constexpr int kSelThreads = 1024;

// fp32 -> uint32 whose unsigned order is the float order (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0 + +0 = +0 under round-to-nearest
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact top-k of keys[0..n) (1 <= k < n) by one wave: a 4-pass 8-bit radix
// select finds the k-th largest key T (LDS histogram, reversed wave scan),
// then an ordered ballot compaction keeps every key > T and the
// lowest-index keys == T, writing the kept ids ascending to srow and
// replacing each key by its rank + 1 (0 when not kept).
__device__ __forceinline__ void select_in_wave(uint32_t* keys, int n, int k,
                                               int id0, int32_t* srow,
                                               uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;  // keys still to take among those matching prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    for (int j = lane; j < n; j += 64) {
      const uint32_t key = keys[j];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
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
    int digit = -1, above = 0;
    if (a3 < rem && rem <= a3 + h3) { digit = 4 * lane + 3; above = (int)a3; }
    if (a2 < rem && rem <= a2 + h2) { digit = 4 * lane + 2; above = (int)a2; }
    if (a1 < rem && rem <= a1 + h1) { digit = 4 * lane + 1; above = (int)a1; }
    if (a0 < rem && rem <= a0 + h0) { digit = 4 * lane;     above = (int)a0; }
    // exactly one lane found the digit holding the remaining-th key
    const uint64_t who = __ballot(digit >= 0);
    const int src = __builtin_ctzll(who);
    digit = __shfl(digit, src);
    above = __shfl(above, src);
    remaining -= above;
    prefix |= (uint32_t)digit << shift;
    pmask |= 255u << shift;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  const uint32_t T = prefix;  // the k-th largest key; take `remaining` of == T
  int out = 0;
  for (int base = 0; base < n; base += 64) {
    const int j = base + lane;
    const uint32_t key = j < n ? keys[j] : 0u;
    const bool eq = j < n && key == T;
    const uint64_t eqm = __ballot(eq);
    const int eq_rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(eqm >> 32),
                            __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
    const bool keep = (j < n && key > T) || (eq && eq_rank < remaining);
    const uint64_t km = __ballot(keep);
    const int pos = out + __builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32),
                              __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
    if (keep) srow[pos] = id0 + j;
    if (j < n) keys[j] = keep ? (uint32_t)(pos + 1) : 0u;
    out += __popcll(km);
    remaining -= __popcll(eqm);
  }
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

// Decode-token append folded into the selection launch (one wave): write
// the K row and the V column of slot L-1 and, when the slot completes its
// block, that block's representation (rows 0..126 from the pool, row 127
// from k_new).  The selection never reads this token or this block's
// representation: the block holding slot L-1 is the sequence's last, which
// is always local.
struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pages;
  uint16_t* v_pages;
  int64_t n_pages;
  float* reps;
};

__device__ __forceinline__ void append_in_wave(const AppendArgs& ap, int bh, int h,
                                               int n_kv, int L, int max_blocks,
                                               const int32_t* trow) {
  const int lane = threadIdx.x & 63;
  if (L <= 0) return;
  const int pos = L - 1, j = pos >> 7, slot = pos & 127;
  const int page = trow[j];
  if ((uint64_t)(int64_t)page >= (uint64_t)ap.n_pages) return;
  const int64_t base = ((int64_t)page * n_kv + h) * (kBlock * kDim);
  const uint16_t* kn = ap.k_new + (int64_t)bh * kDim;
  const uint16_t* vn = ap.v_new + (int64_t)bh * kDim;
  reinterpret_cast<uint32_t*>(ap.k_pages + base + slot * kDim)[lane] =
      reinterpret_cast<const uint32_t*>(kn)[lane];
  ap.v_pages[base + lane * kBlock + slot] = vn[lane];
  ap.v_pages[base + (lane + 64) * kBlock + slot] = vn[lane + 64];
  if (slot != kBlock - 1 || ap.reps == nullptr) return;
  const uint16_t* K = ap.k_pages + base;
  const int c = lane & 15, g = lane >> 4;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const int t = it * 4 + g;
    const uint16_t* src = (t == kBlock - 1) ? kn : K + t * kDim;
    const uint4 w = *reinterpret_cast<const uint4*>(src + c * 8);
    acc[0] += bf16lo(w.x); acc[1] += bf16hi(w.x);
    acc[2] += bf16lo(w.y); acc[3] += bf16hi(w.y);
    acc[4] += bf16lo(w.z); acc[5] += bf16hi(w.z);
    acc[6] += bf16lo(w.w); acc[7] += bf16hi(w.w);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i] += __shfl_xor(acc[i], 16);
    acc[i] += __shfl_xor(acc[i], 32);
  }
  if (lane < 16) {
    const float inv = 1.0f / 128.0f;
    float4* o = reinterpret_cast<float4*>(ap.reps + ((int64_t)bh * max_blocks + j) * kDim + lane * 8);
    o[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    o[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
}

struct SelArgs {
  Method m;
  const uint16_t* q;
  const float* reps;
  const int32_t* table;
  const int32_t* lens;
  const int32_t* prompt_lens;
  int max_blocks;
  int32_t* sel_ids;
  int32_t* n_sel;
  int k_cap;
  int32_t* merged;
  int32_t* n_merged;
  int m_cap;
};

constexpr int kTabRegs = RKV_MAX_BLOCKS / kSelThreads;  // table entries per thread
constexpr int kSlots = kSelThreads / 8;                  // reps per scoring round

// Everything that does not depend on the sequence length -- the length, the
// query, this thread's block-table entries and the first round of
// representations -- is requested at once, so the selection costs about one
// memory round trip before its LDS work.
template <bool APPEND>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelArgs a, AppendArgs ap) {
  extern __shared__ uint32_t keys[];  // [max_blocks]: scores, then ranks
  __shared__ float qs[kDim];
  __shared__ uint32_t hist[256];

  const Method& m = a.m;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / m.n_kv_heads, h = bh - b * m.n_kv_heads;
  const int max_blocks = a.max_blocks;
  const int32_t* trow = a.table + (int64_t)b * max_blocks;

  // --- requests independent of the length ---
  const int lraw = a.lens[b];
  const int plen = a.prompt_lens ? a.prompt_lens[b] : lraw;
  float qsum = 0.f;
  if (tid < kDim) {
    const uint16_t* qh = a.q + ((int64_t)b * m.n_q_heads + h * m.group) * kDim;
    for (int g = 0; g < m.group; ++g)
      qsum += __uint_as_float((uint32_t)qh[g * kDim + tid] << 16);
  }
  int tab[kTabRegs];
#pragma unroll
  for (int i = 0; i < kTabRegs; ++i) {
    const int j = tid + kSelThreads * i;
    tab[i] = j < max_blocks ? trow[j] : -1;
  }
  // offload blocks start at ceil(init/128) whenever there are any
  int ib = (int)(((int64_t)m.init_tokens + 127) >> 7);
  ib = ib < max_blocks ? ib : max_blocks;
  const int n_cap = max_blocks - ib;  // rows of reps that exist after ib
  const float* rbase = a.reps + ((int64_t)bh * max_blocks + ib) * kDim;
  const int o = tid & 7;
  float4 v[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int jj = u * kSlots + (tid >> 3);
    const float4* p = reinterpret_cast<const float4*>(
        rbase + (int64_t)(jj < n_cap ? jj : 0) * kDim);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[u][i] = n_cap > 0 ? p[o + 8 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // --- regions and k ---
  const int L = clamp_len(lraw, max_blocks * kBlock);
  const Regions R = regions_of(L, m.init_tokens, m.local_tokens);
  const bool dense = plen < m.dense_boundary || m.topk_ppm >= kPpmOne;
  const int n = R.n_off;  // when n > 0, R.n_init == ib
  int k = dense ? n : topk_of(n, m.topk_ppm);
  k = k < n ? k : n;
  int32_t* srow = a.sel_ids + (int64_t)bh * a.k_cap;
  int32_t* mrow = a.merged ? a.merged + (int64_t)bh * a.m_cap : nullptr;

  if (k > 0 && k < n) {
    if (tid < kDim) qs[tid] = qsum;
    __syncthreads();
    float4 qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qv[i] = *reinterpret_cast<const float4*>(&qs[4 * (o + 8 * i)]);
    // scores -> order keys; lane octet o covers floats 4(o+8i)..+3 of a rep
    for (int base = 0; base < n; base += 4 * kSlots) {
      if (base > 0) {  // later rounds: only when n > 512
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int jj = base + u * kSlots + (tid >> 3);
          const float4* p = reinterpret_cast<const float4*>(
              rbase + (int64_t)(jj < n ? jj : 0) * kDim);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[u][i] = p[o + 8 * i];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = base + u * kSlots + (tid >> 3);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          part += v[u][i].x * qv[i].x + v[u][i].y * qv[i].y +
                  v[u][i].z * qv[i].z + v[u][i].w * qv[i].w;
        part += __shfl_xor(part, 1);
        part += __shfl_xor(part, 2);
        part += __shfl_xor(part, 4);
        if (o == 0 && jj < n) keys[jj] = order_key(part);
      }
    }
    __syncthreads();
    // wave 0 selects; the last wave appends the decoded token meanwhile
    if (tid < 64) select_in_wave(keys, n, k, R.n_init, srow, hist);
    if (APPEND && tid >= kSelThreads - 64)
      append_in_wave(ap, bh, h, m.n_kv_heads, L, max_blocks, trow);
    __syncthreads();  // ranks in keys[] are visible to every thread
  } else {
    for (int r = tid; r < k; r += kSelThreads) srow[r] = R.n_init + r;
    if (APPEND && tid >= kSelThreads - 64)
      append_in_wave(ap, bh, h, m.n_kv_heads, L, max_blocks, trow);
  }

  // merged page list from the block-table entries each thread holds
  if (mrow) {
    const int lstart = R.local_start > R.n_init ? R.local_start : R.n_init;
#pragma unroll
    for (int i = 0; i < kTabRegs; ++i) {
      const int j = tid + kSelThreads * i;
      if (j >= R.nb) continue;
      int dst = -1;
      if (j < R.n_init) {
        dst = j;
      } else if (j >= lstart) {
        dst = R.n_init + k + (j - lstart);
      } else if (k == n) {
        dst = j;
      } else if (k > 0) {
        const uint32_t rank = keys[j - R.n_init];
        if (rank) dst = R.n_init + (int)rank - 1;
      }
      if (dst >= 0) mrow[dst] = tab[i];
    }
    if (tid == 0) a.n_merged[bh] = R.n_init + k + (R.nb - lstart);
  }
  if (tid == 0) a.n_sel[bh] = k;
}

// Standalone merge from given selections.  Ids outside the offload range
// are written as page -1 (the attention kernel skips such entries).  A kept
// block that lives in host memory (host_table entry >= 0) is taken from its
// staging page stage_page0 + b * k_cap + r (host tier); every other block
// from the block table.
__global__ __launch_bounds__(256) void merge_kernel(
    Method m, const int32_t* __restrict__ table, int max_blocks,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ sel_ids,
    const int32_t* __restrict__ n_sel, int k_cap,
    const int32_t* __restrict__ host_table, int64_t stage_page0,
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
    int page = -1;
    if (ok) {
      const bool on_host = host_table && host_table[(int64_t)b * max_blocks + j] >= 0;
      page = on_host ? (int)(stage_page0 + (int64_t)b * k_cap + r) : trow[j];
    }
    mrow[R.n_init + r] = page;
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
                         const AppendOp* append, hipStream_t stream) {
  const int groups = batch * m.n_kv_heads;
  if (groups == 0) return hipSuccess;
  const size_t lds = (size_t)max_blocks * sizeof(uint32_t);
  SelArgs a{m, q, reps, table, lens, prompt_lens, max_blocks, sel_ids, n_sel,
            k_cap, merged, n_merged, m_cap};
  if (append) {
    AppendArgs ap{append->k_new, append->v_new, append->k_pages, append->v_pages,
                  append->n_pages, append->reps};
    hipLaunchKernelGGL(select_kernel<true>, dim3(groups), dim3(kSelThreads), lds,
                       stream, a, ap);
  } else {
    AppendArgs ap{};
    hipLaunchKernelGGL(select_kernel<false>, dim3(groups), dim3(kSelThreads), lds,
                       stream, a, ap);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const Method& m, const int32_t* table, int max_blocks,
                        const int32_t* lens, const int32_t* sel_ids,
                        const int32_t* n_sel, int k_cap, int batch,
                        const int32_t* host_table, int64_t stage_page0,
                        int32_t* merged, int32_t* n_merged, int m_cap,
                        hipStream_t stream) {
  const int groups = batch * m.n_kv_heads;
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(groups), dim3(256), 0, stream, m,
                     table, max_blocks, lens, sel_ids, n_sel, k_cap, host_table,
                     stage_page0, merged, n_merged, m_cap);
  return hipGetLastError();
}

}  // namespace rkv
