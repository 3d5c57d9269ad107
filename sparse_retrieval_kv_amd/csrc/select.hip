// Inner-product retrieval, exact top-k and block-table merge (gfx950).
//
// openGauss DataVec page "KV Cache Query-Based Computation Inference
// Acceleration", section "Overall Solution": the current token's query is
// scored against every offload-block representation by inner product, the
// top-K closest blocks are kept and joined with the initial-token and
// sliding-window blocks.  Defaults and the dense switch: same page,
// "Configuration Parameters".
//
// Two launches per selection:
//  1. score_kernel: one wave per 32 representations (16 KiB) of one
//     (sequence, KV head) -- 16 or 8 when that gives too few waves to cover
//     the compute units twice -- so the scan of even one sequence is spread
//     over most compute units (one compute unit alone streams only a few
//     tens of GB/s).  The group's query heads are summed once
//     (sum_g q_g . r = (sum_g q_g) . r); eight lanes score one
//     representation; the fp32 scores go to the workspace.  Extra workgroups append the decoded token meanwhile.
//  2. topk_kernel: one 1024-thread workgroup per (sequence, KV head) -- in
//     the per-sequence selection mode each of them sums the scores of all
//     KV heads of its sequence, in head order, so all find the same set --
//     holds the scores as order-preserving uint32 keys and the block-table
//     entries in registers, finds the k-th largest
//     key T by a 4-pass 8-bit radix select over an LDS histogram (wave-
//     aggregated atomics), then keeps every key > T and the lowest-index
//     keys == T with one workgroup scan, writing the kept ids ascending and
//     the merged page list (init blocks, kept blocks, local blocks).
#include "rkv.h"
#include "rkv_device.h"
#include "rkv_internal.h"

#include <type_traits>

namespace rkv {
namespace {



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
  if ((uint64_t)(int64_t)page >= (uint64_t)ap.n_pages) {
    report_bounds(kBoundsPage, page);
    return;
  }
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
  int ib;        // first offload block: min(ceil(init / 128), max_blocks)
  int n_chunks;  // score chunks per (sequence, KV head)
  int spec_end;  // chunks ending at or below this block load before the length
  int n_bh;      // batch * n_kv_heads
  uint32_t* keys;  // workspace [batch][n_kv_heads][max_blocks]
  int32_t* sel_ids;
  int32_t* n_sel;
  int k_cap;
  int32_t* merged;
  int32_t* n_merged;
  int m_cap;
};

constexpr int kScoreThreads = 64;
constexpr int kScoreMaxRounds = 4;  // 8 representations per round
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTabRegs = RKV_MAX_BLOCKS / kTopkThreads;  // blocks per thread

// Regions, k and whether scores are needed, from the raw lengths.
struct Pick {
  Regions R;
  int k;
  bool ranked;  // 0 < k < n_off: the top-k needs the scores
};

__device__ __forceinline__ Pick pick_of(const Method& m, int lraw, int plen,
                                        int max_blocks) {
  Pick p;
  const int L = clamp_len(lraw, max_blocks * kBlock);
  p.R = regions_of(L, m.init_tokens, m.local_tokens);
  const bool dense = plen < m.dense_boundary || m.topk_ppm >= kPpmOne;
  const int n = p.R.n_off;
  int k = dense ? n : topk_of(n, m.topk_ppm);
  p.k = k < n ? k : n;
  p.ranked = p.k > 0 && p.k < n;
  return p;
}

// Wave item = (bh, chunk c): representations of blocks
// [ib + C c, ib + C c + C) of the offload range, C = 8 * ROUNDS.  Items past
// the score grid append the decoded token of sequence-head item - n_bh *
// n_chunks (one wave).
template <bool APPEND, int ROUNDS>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(SelArgs a,
                                                              AppendArgs ap) {
  constexpr int kScoreRounds = ROUNDS;
  constexpr int kScoreChunk = 8 * ROUNDS;
  __shared__ __attribute__((aligned(16))) float qs[kDim];
  const Method& m = a.m;
  const int tid = threadIdx.x;
  const int64_t item = blockIdx.x;
  const int max_blocks = a.max_blocks;
  const int64_t n_items = (int64_t)a.n_chunks * a.n_bh;
  if (item >= n_items) {
    if (APPEND) {
      const int bh = (int)(item - n_items);
      const int b = bh / m.n_kv_heads, h = bh - b * m.n_kv_heads;
      const int L = clamp_len(a.lens[b], max_blocks * kBlock);
      append_in_wave(ap, bh, h, m.n_kv_heads, L, max_blocks,
                     a.table + (int64_t)b * max_blocks);
    }
    return;
  }
  const int bh = (int)(item / a.n_chunks);
  const int c = (int)(item - (int64_t)bh * a.n_chunks);
  const int b = bh / m.n_kv_heads, h = bh - b * m.n_kv_heads;

  // --- requests independent of the length: the group's query rows (lane
  // tid holds dims 2 tid and 2 tid + 1 of each) and the lengths; and, for a
  // chunk inside every possible offload range (below spec_end), its
  // representations, all issued before any of them is waited for.  A chunk
  // past spec_end waits for the length and loads only if it is in range: in
  // a batch of ragged lengths most of those chunks lie past their
  // sequence's offload end. ---
  const int o = tid & 7, slot = tid >> 3;  // lane octet o of slot 0..7
  const int j0 = a.ib + c * kScoreChunk;
  const bool spec = j0 + kScoreChunk <= a.spec_end;  // uniform
  float4 v[kScoreRounds][4];
  auto load_reps = [&]() {
#pragma unroll
    for (int u = 0; u < kScoreRounds; ++u) {
      int j = j0 + u * 8 + slot;
      j = j < max_blocks ? j : max_blocks - 1;
      const float4* p = reinterpret_cast<const float4*>(
          a.reps + ((int64_t)bh * max_blocks + j) * kDim);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[u][i] = p[o + 8 * i];
    }
  };
  // the rest of the item once the representations are requested: the
  // group's query heads summed in head order, this chunk's share of the
  // offload range, the scores
  auto finish = [&](auto early) {
    const uint32_t* qh = reinterpret_cast<const uint32_t*>(
        a.q + ((int64_t)b * m.n_q_heads + h * m.group) * kDim);
    uint32_t qw[RKV_MAX_GROUP];
#pragma unroll
    for (int g = 0; g < RKV_MAX_GROUP; ++g)
      qw[g] = g < m.group ? qh[g * (kDim / 2) + tid] : 0u;
    const int lraw = a.lens[b];
    // the pointer is chosen, not the value, so that this load goes out with
    // the others instead of after the length arrives
    const int plen = (a.prompt_lens ? a.prompt_lens : a.lens)[b];
    float qsum0 = 0.f, qsum1 = 0.f;  // dims 2 tid and 2 tid + 1
#pragma unroll
    for (int g = 0; g < RKV_MAX_GROUP; ++g) {
      if (g < m.group) {
        qsum0 += bf16lo(qw[g]);
        qsum1 += bf16hi(qw[g]);
      }
    }
    const Pick pk = pick_of(m, lraw, plen, max_blocks);
    const int ls = pk.R.n_init + pk.R.n_off;  // offload end
    if (!pk.ranked || j0 >= ls) return;  // uniform over the wave
    if (!decltype(early)::value) load_reps();
    *reinterpret_cast<float2*>(&qs[2 * tid]) = make_float2(qsum0, qsum1);
    __syncthreads();
    float4 qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qv[i] = *reinterpret_cast<const float4*>(&qs[4 * (o + 8 * i)]);
    uint32_t* krow = a.keys + (int64_t)bh * max_blocks;
#pragma unroll
    for (int u = 0; u < kScoreRounds; ++u) {
      const int j = j0 + u * 8 + slot;
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part += v[u][i].x * qv[i].x + v[u][i].y * qv[i].y +
                v[u][i].z * qv[i].z + v[u][i].w * qv[i].w;
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 4);
      if (o == 0 && j < ls) krow[j] = __float_as_uint(part);
    }
  };
  if (spec) {
    load_reps();
    finish(std::true_type());
  } else {
    finish(std::false_type());
  }
}

// Inclusive prefix sum over the 64 lanes of a wave in lane order: row
// shifts by 1, 2, 4, 8 within each row of 16 lanes, then the last lane of
// row 0 / row 2 is broadcast into rows 1 / 3 and the last lane of row 1
// into rows 2 and 3 (DPP row_shr and row_bcast).
__device__ __forceinline__ uint32_t wave_prefix_incl(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);
  return x;
}

// Inclusive workgroup scan helper: returns the sum of `x` over the waves
// before this one and the total; `sh` holds kTopkWaves words.
__device__ __forceinline__ uint32_t waves_before(uint32_t x, uint32_t* sh,
                                                 uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t y = sh[w];
    before += w < wave ? y : 0u;
    all += y;
  }
  __syncthreads();  // sh may be reused right after
  *total = all;
  return before;
}


__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsh[kTopkWaves];
  __shared__ int sdig[3];
  const Method& m = a.m;
  const int tid = threadIdx.x, lane = tid & 63;
  // one workgroup per (b, h).  Per sequence, every workgroup of sequence b
  // sums the scores of all its heads in the same order, so all of them find
  // the same selection; each writes its own head's rows.
  const int b = blockIdx.x / m.n_kv_heads;
  const int bh = blockIdx.x;
  const int n_sum = m.per_sequence ? m.n_kv_heads : 1;
  const int max_blocks = a.max_blocks;
  const int32_t* trow = a.table + (int64_t)b * max_blocks;
  const uint32_t* krow =
      a.keys + (int64_t)(m.per_sequence ? b * m.n_kv_heads : bh) * max_blocks;

  // --- requests independent of the length ---
  const int lraw = a.lens[b];
  // the pointer is chosen, not the value, so that this load goes out with
  // the others instead of after the length arrives
  const int plen = (a.prompt_lens ? a.prompt_lens : a.lens)[b];
  int tab[kTabRegs];
  uint32_t key[kTabRegs];
  float sc[kTabRegs];
  // table entries and (first) scores in one batch of loads, no loop
  // between them, so that they share one memory round trip
#pragma unroll
  for (int i = 0; i < kTabRegs; ++i) {
    const int j = tid + kTopkThreads * i;
    const bool in = j < max_blocks;
    tab[i] = in ? trow[j] : -1;
    sc[i] = in ? __uint_as_float(krow[j]) : 0.f;
  }
  // per sequence: the other heads' scores, added in head order.  When
  // every block fits one thread (max_blocks <= 1024), heads 1..8 join the
  // batch above: their loads use a clamped index, so no lane condition
  // makes the compiler wait for them early.
  const bool one_reg = max_blocks <= kTopkThreads;
  int h_rest = 1;
  if (one_reg && n_sum > 1) {  // uniform
    const int jc = tid < max_blocks ? tid : max_blocks - 1;
    float t1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      t1[u] = 1 + u < n_sum ? __uint_as_float(krow[(int64_t)(1 + u) * max_blocks + jc])
                            : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (1 + u < n_sum && tid < max_blocks) sc[0] += t1[u];
    h_rest = 9;
  }
  // the rest four heads per round trip (eight at a time over all registers
  // needs 95 registers and ran slower)
  for (int h0 = h_rest; h0 < n_sum; h0 += 4) {
    float t[4][kTabRegs];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < kTabRegs; ++i) {
        const int j = tid + kTopkThreads * i;
        t[u][i] = (h0 + u < n_sum && j < max_blocks)
                      ? __uint_as_float(krow[(int64_t)(h0 + u) * max_blocks + j])
                      : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < kTabRegs; ++i)
        if (h0 + u < n_sum && tid + kTopkThreads * i < max_blocks) sc[i] += t[u][i];
  }
  // raw fp32 scores -> order keys
#pragma unroll
  for (int i = 0; i < kTabRegs; ++i) key[i] = order_key(sc[i]);
  if (tid < 256) hist[tid] = 0u;

  const Pick pk = pick_of(m, lraw, plen, max_blocks);
  const Regions& R = pk.R;
  const int k = pk.k;
  const int ls = R.n_init + R.n_off;
  int32_t* srow = a.sel_ids + (int64_t)bh * a.k_cap;
  int32_t* mrow = a.merged ? a.merged + (int64_t)bh * a.m_cap : nullptr;
  const int lstart = R.local_start > R.n_init ? R.local_start : R.n_init;

  // rank + 1 of each kept offload block this thread holds (0: not kept)
  int rank1[kTabRegs];
#pragma unroll
  for (int i = 0; i < kTabRegs; ++i) rank1[i] = 0;

  if (pk.ranked) {  // uniform over the workgroup
    __syncthreads();  // hist zeroed
    uint32_t prefix = 0, pmask = 0;
    int remaining = k;  // keys still to take among those matching prefix
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int i = 0; i < kTabRegs; ++i) {
        const int j = tid + kTopkThreads * i;
        if (kTopkThreads * i >= ls) break;  // uniform
        const bool has = j >= R.n_init && j < ls && (key[i] & pmask) == prefix;
        const uint32_t d = (key[i] >> shift) & 255u;
        // lanes sharing the first active lane's digit add with one atomic
        const uint64_t act = __ballot(has);
        if (act == 0) continue;
        const int first = __builtin_ctzll(act);
        const uint32_t d0 = __builtin_amdgcn_readlane(d, first);
        const uint64_t same = __ballot(has && d == d0);
        if (lane == first) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
        if (has && d != d0) atomicAdd(&hist[d], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
        const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        hist[4 * lane] = 0u;
        hist[4 * lane + 1] = 0u;
        hist[4 * lane + 2] = 0u;
        hist[4 * lane + 3] = 0u;
        const uint32_t s4 = h0 + h1 + h2 + h3;
        const uint32_t incl = wave_prefix_incl(s4);
        const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
        const uint32_t a3 = total - incl;  // count in bins above 4*lane+3
        const uint32_t a2 = a3 + h3, a1 = a2 + h2, a0 = a1 + h1;
        const uint32_t rem = (uint32_t)remaining;
        int digit = -1, above = 0, cnt = 0;
        if (a3 < rem && rem <= a3 + h3) { digit = 4 * lane + 3; above = (int)a3; cnt = (int)h3; }
        if (a2 < rem && rem <= a2 + h2) { digit = 4 * lane + 2; above = (int)a2; cnt = (int)h2; }
        if (a1 < rem && rem <= a1 + h1) { digit = 4 * lane + 1; above = (int)a1; cnt = (int)h1; }
        if (a0 < rem && rem <= a0 + h0) { digit = 4 * lane;     above = (int)a0; cnt = (int)h0; }
        // exactly one lane holds the digit of the remaining-th key
        if (digit >= 0) {
          sdig[0] = digit;
          sdig[1] = above;
          sdig[2] = cnt;
        }
      }
      __syncthreads();
      remaining -= sdig[1];
      prefix |= (uint32_t)sdig[0] << shift;
      pmask |= 255u << shift;
      // every key left in the chosen bin is taken: the class is settled
      if (remaining == sdig[2]) break;  // uniform
    }
    // keys whose masked value exceeds the prefix are kept, and the first
    // `remaining` keys (in block order) whose masked value equals it
    uint32_t gt_carry = 0, eq_carry = 0;
#pragma unroll
    for (int i = 0; i < kTabRegs; ++i) {
      if (kTopkThreads * i >= ls) break;  // uniform
      const int j = tid + kTopkThreads * i;
      const bool cand = j >= R.n_init && j < ls;
      const uint32_t mk = key[i] & pmask;
      const bool gt = cand && mk > prefix, eq = cand && mk == prefix;
      const uint64_t gm = __ballot(gt), em = __ballot(eq);
      // gt counts in the low 16 bits, eq counts in the high 16 (n < 2^16)
      const uint32_t wcnt = (uint32_t)__popcll(gm) | ((uint32_t)__popcll(em) << 16);
      uint32_t tot;
      const uint32_t wb = waves_before(wcnt, wsh, &tot);
      const uint32_t gt_before = gt_carry + (wb & 0xffffu) + (uint32_t)lanes_below(gm);
      const uint32_t eq_before = eq_carry + (wb >> 16) + (uint32_t)lanes_below(em);
      const uint32_t rem = (uint32_t)remaining;
      const uint32_t pos = gt_before + (eq_before < rem ? eq_before : rem);
      if ((gt || (eq && eq_before < rem)) && pos < (uint32_t)k) {
        srow[pos] = j;
        rank1[i] = (int)pos + 1;
      }
      gt_carry += tot & 0xffffu;
      eq_carry += tot >> 16;
    }
  } else {
    for (int r = tid; r < k; r += kTopkThreads) srow[r] = R.n_init + r;
  }

  // merged page list from the block-table entries each thread holds
  if (mrow) {
#pragma unroll
    for (int i = 0; i < kTabRegs; ++i) {
      const int j = tid + kTopkThreads * i;
      if (j >= R.nb) continue;
      int dst = -1;
      if (j < R.n_init) {
        dst = j;
      } else if (j >= lstart) {
        dst = R.n_init + k + (j - lstart);
      } else if (k == R.n_off) {
        dst = j;
      } else if (rank1[i]) {
        dst = R.n_init + rank1[i] - 1;
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
  if (k < 0 || k > R.n_off || k > k_cap) report_bounds(kBoundsCount, k);
  k = k < 0 ? 0 : k;
  k = k < R.n_off ? k : R.n_off;
  k = k < k_cap ? k : k_cap;
  const int32_t* trow = table + (int64_t)b * max_blocks;
  const int32_t* srow = sel_ids + (int64_t)bh * k_cap;
  int32_t* mrow = merged + (int64_t)bh * m_cap;
  for (int r = threadIdx.x; r < k; r += blockDim.x) {
    const int j = srow[r];
    const bool ok = j >= R.n_init && j < R.n_init + R.n_off;
    if (!ok) report_bounds(kBoundsBlock, j);
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

size_t select_keys_bytes(int batch, int n_kv_heads, int max_blocks) {
  return (size_t)batch * n_kv_heads * max_blocks * sizeof(uint32_t);
}

hipError_t launch_score(const Method& m, const uint16_t* q, const float* reps,
                        const int32_t* table, const int32_t* lens,
                        const int32_t* prompt_lens, int batch, int max_blocks,
                        uint32_t* scores, const AppendOp* append,
                        hipStream_t stream) {
  const int groups = batch * m.n_kv_heads;
  if (groups == 0) return hipSuccess;
  int ib = (int)(((int64_t)m.init_tokens + 127) >> 7);
  ib = ib < max_blocks ? ib : max_blocks;
  // 32 representations per score wave, fewer when that leaves less than
  // two waves per compute unit: a small scan is latency-bound, and its
  // share of one compute unit's bandwidth is what its waves wait for
  const int64_t want = 2 * (int64_t)device_cu_count();
  int rounds = kScoreMaxRounds;
  while (rounds > 1 &&
         (int64_t)groups * ((max_blocks - ib + 8 * rounds - 1) / (8 * rounds)) < want)
    rounds >>= 1;
  const int chunk = 8 * rounds;
  const int n_chunks = (max_blocks - ib + chunk - 1) / chunk;
  // A batch of one requests every chunk's representations with the length
  // (only the window's chunks are read in vain).  In a batch, only chunks
  // inside every ranked list's offload range: a list needs scores only when
  // its prompt is not below the dense boundary, so L >= dense_boundary and
  // its offload range reaches at least block (dense_boundary - local) / 128.
  int spec_end = max_blocks;
  if (batch > 1) {
    const int64_t lo = m.dense_boundary > m.local_tokens
                           ? ((int64_t)m.dense_boundary - m.local_tokens) / kBlock
                           : 0;
    spec_end = (int)(lo < ib ? ib : (lo > max_blocks ? max_blocks : lo));
  }
  SelArgs a{m, q, reps, table, lens, prompt_lens, max_blocks, ib, n_chunks, spec_end,
            groups, scores, nullptr, nullptr, 0, nullptr, nullptr, 0};
  const int64_t score_wgs = (int64_t)groups * n_chunks;
  AppendArgs ap{};
  if (append)
    ap = AppendArgs{append->k_new, append->v_new, append->k_pages, append->v_pages,
                    append->n_pages, append->reps};
  const dim3 sgrid((unsigned)(score_wgs + (append ? groups : 0)));
  if (sgrid.x > 0) {
#define RKV_SCORE_LAUNCH(R)                                                      \
  if (append)                                                                    \
    hipLaunchKernelGGL((score_kernel<true, R>), sgrid, dim3(kScoreThreads), 0,   \
                       stream, a, ap);                                           \
  else                                                                           \
    hipLaunchKernelGGL((score_kernel<false, R>), sgrid, dim3(kScoreThreads), 0,  \
                       stream, a, ap);
    if (rounds == 1) {
      RKV_SCORE_LAUNCH(1)
    } else if (rounds == 2) {
      RKV_SCORE_LAUNCH(2)
    } else {
      RKV_SCORE_LAUNCH(4)
    }
#undef RKV_SCORE_LAUNCH
  }
  return hipGetLastError();
}

hipError_t launch_topk(const Method& m, const int32_t* table, const int32_t* lens,
                       const int32_t* prompt_lens, int batch, int max_blocks,
                       const uint32_t* scores, int32_t* sel_ids, int32_t* n_sel,
                       int k_cap, int32_t* merged, int32_t* n_merged, int m_cap,
                       hipStream_t stream) {
  const int groups = batch * m.n_kv_heads;
  if (groups == 0) return hipSuccess;
  // the top-k only reads the scores
  SelArgs a{m, nullptr, nullptr, table, lens, prompt_lens, max_blocks, 0, 0, 0,
            groups, const_cast<uint32_t*>(scores), sel_ids, n_sel, k_cap,
            merged, n_merged, m_cap};
  hipLaunchKernelGGL(topk_kernel, dim3(groups), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select(const Method& m, const uint16_t* q, const float* reps,
                         const int32_t* table, const int32_t* lens,
                         const int32_t* prompt_lens, int batch, int max_blocks,
                         int32_t* sel_ids, int32_t* n_sel, int k_cap,
                         int32_t* merged, int32_t* n_merged, int m_cap,
                         void* workspace, const AppendOp* append,
                         hipStream_t stream) {
  uint32_t* scores = static_cast<uint32_t*>(workspace);
  hipError_t e = launch_score(m, q, reps, table, lens, prompt_lens, batch,
                              max_blocks, scores, append, stream);
  if (e != hipSuccess) return e;
  return launch_topk(m, table, lens, prompt_lens, batch, max_blocks, scores,
                     sel_ids, n_sel, k_cap, merged, n_merged, m_cap, stream);
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

RKV_BOUNDS_SETTER(set_bounds_word_select)

}  // namespace rkv
