// Split-K paged decode attention with log-sum-exp combine (gfx950).
//
// softmax(q K^T / sqrt(d)) V for one query token per head (rkmt.cn ATB
// KV-cache article, section 1.1), reading K/V pages through a block table
// (same article, section 2.2), over the merged block list of each
// (sequence, KV head).  Partial softmax results are merged by their
// log-sum-exp (partial results merged the FlashDecoding way, CSDN "KV cache"
// survey, section "Share--KV cache共享").
//
// Work partition.  Every merged block is cut into two 64-token halves
// ("units"); the units of all (sequence, KV head) lists, taken in order,
// form one range of T units that is split evenly over a fixed number W of
// waves (default two per compute unit), taken in a virtual order that puts
// the waves sharing a compute unit next to each other, so every compute
// unit streams the same share.  A wave's range meets one or a few lists;
// for each list it writes one partial (m, l, acc) into slot v + list (v: the
// wave's virtual index).  Walking the range, every step to the next piece
// moves to the next wave or the next list or both, so v + list never repeats
// and a list's pieces sit in consecutive slots; the wave holding a list's
// first unit records the first slot and the piece count.  T is known only on the
// device, so every wave derives the partition from n_merged itself: ragged
// batches stay balanced and no host round trip is needed.  A batch of one
// sequence (all its lists equally long) instead deals each list's units
// round robin over a fixed set of waves, so that a wave can request its
// page ids before it knows the list length (strided_body).  Within a list, a
// wave's loads are software-pipelined: unit u+1's K tile is requested right
// after unit u's V tile, so about 32 KiB per wave stay in flight while unit
// u's softmax and PV products run.
//
// MFMA math for one 64-token unit (query heads padded to 16):
//   S^T[16 tokens x 16 heads] = K_tile[16 x 128] . Q^T[128 x 16]
//     with v_mfma_f32_16x16x32_bf16, four K-steps of 32 dims per tile,
//     four tiles per unit.  The accumulator layout (lane l holds rows
//     4(l/16)+r, column l%16) puts four tokens of head l%16 in each lane.
//   O[16 heads x 16 dims] += P[16 x 32 tokens] . V[32 tokens x 16 dims]
//     with the same instruction: the two S^T tiles of a 32-token pair are
//     exactly the A-operand layout of P (row = head l%16, eight tokens per
//     lane group), so P never leaves the registers.  P is split into a bf16
//     high part and a bf16 residual (two MFMAs) so the weights keep ~16
//     significant bits; V is bf16 already.
// Token order inside a unit is chosen so that every load is 16 contiguous
// bytes per lane: in pair pp, lane group g owns tokens 32pp+8g .. 32pp+8g+7.
//   K tile (pair pp, half e): row m holds token 32pp + 8(m/4) + 4e + m%4,
//   V: lane (col, g) reads dim 16n+col, tokens 32pp+8g..+7 (one 16-byte
//   piece of the dim-major V tile).
// Every (page, head) K and V tile is read exactly once.
//
// For a batch of one, attn_select_mfma_kernel also takes over the top-k and
// the merge (openGauss DataVec page, "Overall Solution"): each wave of a
// list finds the list's selection from the inner-product scores itself and
// builds the merged page list in its LDS, so a decode step needs no
// separate top-k launch (see select_strided_body).
#include "rkv_device.h"
#include "rkv_internal.h"

#include <math.h>

#include <type_traits>

namespace rkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -INFINITY;
constexpr int kUnit = 64;  // tokens per work unit (half a block)

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Zero the bf16 lanes of a V piece whose token index (tok0 + j) >= valid.
__device__ __forceinline__ uint4 mask_tokens(uint4 v, int tok0, int valid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (tok0 + 2 * i) < valid ? 0x0000ffffu : 0u;
    const uint32_t hi = (tok0 + 2 * i + 1) < valid ? 0xffff0000u : 0u;
    w[i] &= (lo | hi);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Split 8 fp32 weights into bf16 high parts and bf16 residuals.
__device__ __forceinline__ void split_hi_lo(const float (&p)[8], bf16x8& hi,
                                            bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __float_as_uint(p[2 * i]) & 0xffff0000u;
    const uint32_t b = __float_as_uint(p[2 * i + 1]) & 0xffff0000u;
    const uint32_t ra = __float_as_uint(p[2 * i] - __uint_as_float(a));
    const uint32_t rb = __float_as_uint(p[2 * i + 1] - __uint_as_float(b));
    h[i] = (a >> 16) | b;
    l[i] = (ra >> 16) | (rb & 0xffff0000u);
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
  lo = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  int64_t n_pages;
  const int32_t* merged;
  const int32_t* n_merged;
  const int32_t* lens;
  float* part_acc;   // [n_slots][group][128]
  float2* part_ml;   // [n_slots][group]
  int* n_pieces;     // [batch * n_kv]: pieces of each non-empty list
  int* first_slot;   // [batch * n_kv]: slot of a list's first piece (range split)
  int m_cap, max_len, batch, n_kv, group, n_waves, n_slots;
  int comb_spec;     // pieces per combine lane requested before the count
  int n_cu;          // compute units of the device
  int per_list;      // > 0: waves per list of the single-sequence partition
  float scale_log2;  // scale * log2(e)
  // shared-prefix cascade (c_waves > 0): waves n_waves .. n_waves + c_waves - 1
  // of the range-split launch attend the shared blocks, c_q sequences per
  // wave; merged / n_merged then hold each list's private entries only
  const int32_t* c_table;  // block-table row of sequence 0: the shared pages
  const uint32_t* c_mask;  // [batch * n_kv][c_words]: attended shared blocks
  int c_words;             // mask words per list
  int c_q;                 // sequences per cascade wave (16 / group, <= batch)
  int c_groups;            // sequence groups: ceil(batch / c_q)
  int c_chunks;            // chunks of shared blocks per (KV head, group)
  int c_chunk_blocks;      // shared blocks per chunk (<= 64)
  int c_shared;            // shared blocks named by the caller
  int c_waves;             // n_kv * c_groups * c_chunks, or 0
  int64_t c_slot0;         // first cascade slot; wave cw writes c_q slots
  // a previous part of every row's attention to fold in (prev_lse null:
  // none), and where to leave each row's log-sum-exp (null: nowhere)
  const float* prev_out;   // [batch][n_q][128], normalized
  const float* prev_lse;   // [batch][n_q]: log2 of the row's softmax sum
  float* lse_out;          // [batch][n_q]
};

// ---------------------------------------------------------------------------
// The unit partition, shared by the split kernel and the combine.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int units_of(const AttnArgs& a, int bh) {
  int n = a.n_merged[bh];
  if (n < 0 || n > a.m_cap) report_bounds(kBoundsCount, n);
  n = n < 0 ? 0 : (n > a.m_cap ? a.m_cap : n);
  return 2 * n;
}

// A merged entry's page id outside the pool contributes nothing; -1 is the
// merge's own mark for a block it left out and is not reported.
__device__ __forceinline__ void report_page(int page) {
  if (page != -1) report_bounds(kBoundsPage, page);
}

// units_of for a lane's list bh, 0 past the last list.  The load is made
// from a valid index on every lane and masked afterwards: a load under a
// lane condition makes the compiler wait for it where the branch rejoins.
__device__ __forceinline__ int units_or_zero(const AttnArgs& a, int bh, int NB) {
  const int u = units_of(a, bh < NB ? bh : NB - 1);
  return bh < NB ? u : 0;
}

// The T units are split evenly over W waves in a virtual order in which the
// waves that share a compute unit are neighbours: when the grid fills an
// idle GPU, workgroup w runs on compute unit w mod n_cu (workgroups are
// dealt round robin over the 8 XCDs and, within an XCD, over its compute
// units), so waves w, w + n_cu, w + 2 n_cu, ... share one.  Each compute
// unit then streams its share of the units (+-1) -- a compute unit's
// bandwidth, not a wave's, is what is shared.  The placement only steers
// speed: any placement gives the same results.
__device__ __forceinline__ int virtual_wave(int w, int W, int n_cu) {
  if (n_cu <= 0 || W % n_cu != 0) return w;
  return (w % n_cu) * (W / n_cu) + w / n_cu;
}

// With at least as many units as waves, wave v takes units
// [v T / W, (v+1) T / W); with fewer, wave v < T takes unit v alone (so the
// waves holding units are consecutive in both cases).
__device__ __forceinline__ int64_t unit_start(int v, int64_t T, int W) {
  if (T >= W) return (int64_t)v * T / W;
  return v < T ? v : T;
}

// The virtual wave whose range holds unit u (0 <= u < T): the largest v
// with unit_start(v) <= u.
__device__ __forceinline__ int wave_of(int64_t u, int64_t T, int W) {
  if (T >= W) return (int)(((u + 1) * W - 1) / T);
  return (int)u;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// ---------------------------------------------------------------------------
// Per-wave timestamps of the folded-selection launch (a library built with
// RKV_WAVE_STAMPS; compiled out otherwise).  Lane 0 keeps s_memrealtime
// values (100 MHz) in LDS and writes them out once, when the wave ends, so
// that no global store sits in the wave's memory counter while it runs.
// Slots: kStampStart, kStampScores (scores and table row arrived),
// kStampSearch (selection found), kStampVreq (first unit's V tile
// requested), kStampList (merged list in LDS), kStampDone (partials
// written), kStampHwId (XCC_ID << 32 | HW_ID), then kStampUnit0 + i: the
// wave's i-th unit attended (i < kStampUnits).
// ---------------------------------------------------------------------------
constexpr int kStampStart = 0, kStampScores = 1, kStampSearch = 2, kStampVreq = 3,
              kStampList = 4, kStampDone = 5, kStampHwId = 6, kStampUnit0 = 7;
constexpr int kStampUnits = kWaveStampSlots - kStampUnit0;

#ifdef RKV_WAVE_STAMPS
__device__ unsigned long long rkv_wave_stamps[kWaveStampWaves][kWaveStampSlots];
__shared__ unsigned long long stamp_lds[kWaveStampSlots];
__device__ __forceinline__ void stamp(int k) {
  if (threadIdx.x == 0) stamp_lds[k] = __builtin_amdgcn_s_memrealtime();
}
// stamp k once x is computed (x is made to depend on)
__device__ __forceinline__ void stamp_after(int k, uint32_t x) {
  if (__builtin_amdgcn_readfirstlane(x) != 0x9e3779b9u) stamp(k);
}
__device__ __forceinline__ void stamp_begin() {
  if (threadIdx.x == 0) {
    for (int k = 0; k < kWaveStampSlots; ++k) stamp_lds[k] = 0;
    stamp_lds[kStampHwId] =
        ((unsigned long long)__builtin_amdgcn_s_getreg(63508) << 32) |  // XCC_ID
        (unsigned)__builtin_amdgcn_s_getreg(63492);                     // HW_ID
  }
  stamp(kStampStart);
}
__device__ __forceinline__ void stamp_flush() {
  __builtin_amdgcn_s_waitcnt(0);
  stamp(kStampDone);
  if (threadIdx.x == 0 && blockIdx.x < (unsigned)kWaveStampWaves)
    for (int k = 0; k < kWaveStampSlots; ++k) rkv_wave_stamps[blockIdx.x][k] = stamp_lds[k];
}
#else
__device__ __forceinline__ void stamp(int) {}
__device__ __forceinline__ void stamp_after(int, uint32_t) {}
__device__ __forceinline__ void stamp_begin() {}
__device__ __forceinline__ void stamp_flush() {}
#endif

// ---------------------------------------------------------------------------
// One unit's K and V tiles.
// ---------------------------------------------------------------------------

// K tile of unit hf (tokens 64hf..64hf+63) into the S^T A-operand layout:
// tile t (16 tokens) and K-step kk, lane (col, grp) -> token row(t, col),
// dims 8*(4kk+grp)..+7.
__device__ __forceinline__ void load_k_unit(uint4 (&kf)[4][4], const uint16_t* K,
                                            int hf, int col, int grp) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = kUnit * hf + 32 * (t >> 1) + 8 * (col >> 2) + 4 * (t & 1) + (col & 3);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kf[t][kk] = ld16(K + row * kDim + (4 * kk + grp) * 8);
  }
}

// V tile of unit hf into the PV B-operand layout: pair pp, dim tile n8,
// lane (col, grp) -> dim 16*n8+col, tokens 64hf+32pp+8grp..+7.
__device__ __forceinline__ void load_v_unit(uint4 (&vf)[2][8], const uint16_t* V,
                                            int hf, int col, int grp) {
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int n8 = 0; n8 < 8; ++n8)
      vf[pp][n8] = ld16(V + (16 * n8 + col) * kBlock + kUnit * hf + 32 * pp + 8 * grp);
}

// ---------------------------------------------------------------------------
// Math policies: MFMA (query heads packed against K tiles) and VALU.
// ---------------------------------------------------------------------------

struct MfmaMath {
  typedef f32x4 Scores[4];
  bf16x8 bq[4];
  f32x4 acc[8];
  float m_run, l_run;

  // Q^T as the B operand: lane (col, grp) holds head col, dims of chunk
  // 4kk+grp (8 bf16) for kk = 0..3; padded heads are zero.  Every lane
  // loads a valid row (padded lanes the group's last) and the padding is
  // zeroed after the load: a branch around the loads would make the
  // compiler wait for them at the branch's end.
  __device__ __forceinline__ void begin(const AttnArgs& a, int b, int h, int col,
                                        int grp) {
    const int G = a.group;
    const int row = col < G ? col : G - 1;
    const uint16_t* qrow = a.q + ((int64_t)b * a.n_kv * G + h * G + row) * kDim;
    uint4 v[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) v[kk] = ld16(qrow + (4 * kk + grp) * 8);
    const uint32_t keep = col < G ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      bq[kk] = as_bf16x8(make_uint4(v[kk].x & keep, v[kk].y & keep, v[kk].z & keep,
                                    v[kk].w & keep));
#pragma unroll
    for (int n8 = 0; n8 < 8; ++n8) acc[n8] = (f32x4){0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;
  }

  __device__ __forceinline__ void scores(const uint4 (&kf)[4][4], Scores& s) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[t][kk]),
                                                       bq[kk], s[t], 0, 0, 0);
    }
  }

  __device__ __forceinline__ void accumulate(Scores& s, uint4 (&vf)[2][8],
                                             int valid, float sl2, int col, int grp) {
    (void)col;
    // log2-domain logits, mask past the sequence end, unit max per head
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[t][r] * sl2;
        const int tok = 32 * (t >> 1) + 8 * grp + 4 * (t & 1) + r;
        x = tok < valid ? x : kNegInf;
        s[t][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(s[t][r] - m_new);
        s[t][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // accumulator rows are heads 4*grp + r; their alpha lives in lane 4*grp+r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) acc[n8][r] *= ar;
    }
    if (valid < kUnit) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
          vf[pp][n8] = mask_tokens(vf[pp][n8], 32 * pp + 8 * grp, valid);
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const float p8[8] = {s[2 * pp][0],     s[2 * pp][1],     s[2 * pp][2],
                           s[2 * pp][3],     s[2 * pp + 1][0], s[2 * pp + 1][1],
                           s[2 * pp + 1][2], s[2 * pp + 1][3]};
      bf16x8 ph, pl;
      split_hi_lo(p8, ph, pl);
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) {
        const bf16x8 v = as_bf16x8(vf[pp][n8]);
        acc[n8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, v, acc[n8], 0, 0, 0);
        acc[n8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, v, acc[n8], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void finish(const AttnArgs& a, int64_t slot, int lane,
                                         int col, int grp) {
    const int G = a.group;
    // the four lane groups of a head hold disjoint token subsets of l
    float lt = l_run + __shfl_xor(l_run, 16);
    lt += __shfl_xor(lt, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 4 * grp + r;
      if (hh < G) {
        float* dst = a.part_acc + (slot * G + hh) * kDim + col;
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8) dst[16 * n8] = acc[n8][r];
      }
    }
    if (lane < G) a.part_ml[slot * G + lane] = make_float2(m_run, lt);
  }
};

// Vector-ALU variant with the same memory schedule (same units, same
// per-lane 16-byte pieces, same token order): q.k by v_dot2_f32_bf16 on bf16
// pairs, p.v by fp32 FMAs, so the two variants differ only in where the dot
// products run.
//   QK: lane (col, grp) holds 32 dims (chunks 4kk+grp) of token row col of
//       each tile; partial dots for the G heads are summed over the four lane
//       groups, leaving S[token(t, col)][head] in every lane of column col.
//   PV: lane (col, grp) owns dims 16n+col and tokens 32pp+8grp..+7; the
//       weights of those tokens are fetched from the lanes that own their
//       rows, and the per-lane partial sums are folded over the lane groups
//       once per list piece.
__device__ __forceinline__ float dot8(uint4 k, uint4 q, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x),
                                      __builtin_bit_cast(bf16x2, q.x), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y),
                                      __builtin_bit_cast(bf16x2, q.y), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z),
                                      __builtin_bit_cast(bf16x2, q.z), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w),
                                      __builtin_bit_cast(bf16x2, q.w), c, false);
  return c;
}

template <int G>
struct ValuMath {
  typedef float Scores[4][G];
  uint4 qv[G][4];
  float acc[8][G];
  float m_run[G], l_run[G];

  __device__ __forceinline__ void begin(const AttnArgs& a, int b, int h, int col,
                                        int grp) {
    (void)col;
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qv[hh][kk] = ld16(a.q + ((int64_t)b * a.n_kv * G + h * G + hh) * kDim +
                          (4 * kk + grp) * 8);
#pragma unroll
    for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) acc[n8][hh] = 0.f;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m_run[hh] = kNegInf;
      l_run[hh] = 0.f;
    }
  }

  __device__ __forceinline__ void scores(const uint4 (&kf)[4][4], Scores& s) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float c = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) c = dot8(kf[t][kk], qv[hh][kk], c);
        c += __shfl_xor(c, 16);
        c += __shfl_xor(c, 32);
        s[t][hh] = c;
      }
  }

  __device__ __forceinline__ void accumulate(Scores& s, uint4 (&vf)[2][8],
                                             int valid, float sl2, int col, int grp) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = 32 * (t >> 1) + 8 * (col >> 2) + 4 * (t & 1) + (col & 3);
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
        s[t][hh] = tok < valid ? s[t][hh] * sl2 : kNegInf;
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 4; ++t) mx = fmaxf(mx, s[t][hh]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[hh], mx);
      const float alpha = fast_exp2(m_run[hh] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s[t][hh] = fast_exp2(s[t][hh] - m_new);
        ps += s[t][hh];
      }
      l_run[hh] = l_run[hh] * alpha + ps;  // over this lane's token rows
      m_run[hh] = m_new;
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) acc[n8][hh] *= alpha;
    }
    if (valid < kUnit) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
          vf[pp][n8] = mask_tokens(vf[pp][n8], 32 * pp + 8 * grp, valid);
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // weight of token 32pp+8grp+j: tile 2pp+(j>=4), row 4grp+(j&3)
        float w[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          w[hh] = __shfl(s[2 * pp + (j >> 2)][hh], 16 * grp + 4 * grp + (j & 3));
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8) {
          const uint4 v = vf[pp][n8];
          const uint32_t vw = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y
                            : (j >> 1) == 2 ? v.z : v.w;
          const float x = (j & 1) ? bf16hi(vw) : bf16lo(vw);
#pragma unroll
          for (int hh = 0; hh < G; ++hh) acc[n8][hh] = fmaf(w[hh], x, acc[n8][hh]);
        }
      }
    }
  }

  __device__ __forceinline__ void finish(const AttnArgs& a, int64_t slot, int lane,
                                         int col, int grp) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float lt = l_run[hh];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) lt += __shfl_xor(lt, o);
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) {
        float x = acc[n8][hh];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        if (grp == 0) a.part_acc[(slot * G + hh) * kDim + 16 * n8 + col] = x;
      }
      if (lane == 0) a.part_ml[slot * G + hh] = make_float2(m_run[hh], lt);
    }
  }
};

// ---------------------------------------------------------------------------
// Split kernel: one wave per range of units.
// ---------------------------------------------------------------------------

// Units [u0, u1) of list bh, written to partial slot `slot`.
template <class Math>
__device__ __forceinline__ void run_piece(const AttnArgs& a, Math& math, int bh,
                                          int u0, int u1, int64_t slot, int lane,
                                          int col, int grp) {
  const int b = bh / a.n_kv, h = bh - b * a.n_kv;
  const int32_t* mrow = a.merged + (int64_t)bh * a.m_cap;
  const int n = units_of(a, bh) >> 1;
  const int L = clamp_len(a.lens[b], a.max_len);
  const int last_valid = L - (((L + 127) >> 7) - 1) * kBlock;
  const int64_t head_off = (int64_t)h * (kBlock * kDim);
  const int64_t page_stride = (int64_t)a.n_kv * (kBlock * kDim);
  // an out-of-range page id is read from page 0 (always present) and its
  // unit is skipped
  auto page_ok = [&](int p) { return (uint64_t)(int64_t)p < (uint64_t)a.n_pages; };
  auto tile_of = [&](int p) {
    return (page_ok(p) ? (int64_t)p * page_stride : 0) + head_off;
  };
  auto valid_of = [&](int u) {
    const int e = u >> 1;
    const int v = (e == n - 1 ? last_valid : kBlock) - kUnit * (u & 1);
    return v < 0 ? 0 : (v > kUnit ? kUnit : v);
  };

  math.begin(a, b, h, col, grp);
  int page = mrow[u0 >> 1];
  int64_t tile = tile_of(page);
  uint4 kf[4][4];
  load_k_unit(kf, a.k_pages + tile, u0 & 1, col, grp);
  // page id of the entry after the current one, requested one unit early
  int page_next = ((u0 >> 1) + 1 < n) ? mrow[(u0 >> 1) + 1] : 0;

  for (int u = u0; u < u1; ++u) {
    typename Math::Scores s;
    math.scores(kf, s);
    __builtin_amdgcn_sched_barrier(0);
    uint4 vf[2][8];
    load_v_unit(vf, a.v_pages + tile, u & 1, col, grp);
    const bool cur_ok = page_ok(page);
    if (!cur_ok) report_page(page);
    const int valid = valid_of(u);
    if (u + 1 < u1) {  // prefetch the next unit's K tile
      if (u & 1) {     // the next unit starts the next entry
        page = page_next;
        tile = tile_of(page);
        const int e2 = (u >> 1) + 2;
        page_next = e2 < n ? mrow[e2] : 0;
      }
      load_k_unit(kf, a.k_pages + tile, (u + 1) & 1, col, grp);
    }
    if (!cur_ok || valid == 0) continue;
    math.accumulate(s, vf, valid, a.scale_log2, col, grp);
  }
  math.finish(a, slot, lane, col, grp);
}

template <class Math>
__device__ __forceinline__ void split_body(const AttnArgs& a) {
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int W = a.n_waves;
  const int w = virtual_wave(blockIdx.x, W, a.n_cu);
  const int NB = a.batch * a.n_kv;
  // the unit counts of the first 4 x 64 lists are requested together and
  // kept in registers (a loop of loads would wait for each group in turn,
  // and the walk below would read them again)
  constexpr int kHeld = 4;
  int held[kHeld];
#pragma unroll
  for (int g = 0; g < kHeld; ++g) held[g] = units_or_zero(a, 64 * g + lane, NB);
  int64_t T = 0;
#pragma unroll
  for (int g = 0; g < kHeld; ++g) T += wave_sum_i(held[g]);
  for (int base = 64 * kHeld; base < NB; base += 64)
    T += wave_sum_i(units_or_zero(a, base + lane, NB));
  if (T == 0) return;
  const int64_t lo = unit_start(w, T, W), hi = unit_start(w + 1, T, W);
  if (lo >= hi) return;
  Math math;
  int64_t run = 0;  // units of the lists before this group of 64
  for (int base = 0; base < NB && run < hi; base += 64) {
    const int bh = base + lane;
    const int gi = base >> 6;
    const int u = gi == 0 ? held[0]
                : gi == 1 ? held[1]
                : gi == 2 ? held[2]
                : gi == 3 ? held[3]
                : units_or_zero(a, bh, NB);
    const int incl = wave_incl_scan(u, lane);
    const int64_t s0 = run + incl - u, s1 = run + incl;
    uint64_t hit = __ballot(u > 0 && s0 < hi && s1 > lo);
    while (hit) {
      const int src = __builtin_ctzll(hit);
      hit &= hit - 1;
      const int pbh = base + src;
      const int64_t ps = run + __shfl(incl - u, src);
      const int pu = __shfl(u, src);
      const int64_t a0 = lo > ps ? lo : ps;
      const int64_t a1 = hi < ps + pu ? hi : ps + pu;
      // the list's pieces are those of waves wave_of(ps) .. wave_of(ps +
      // pu - 1), in slots wave + list; the wave holding the list's first
      // unit records where they start and how many there are
      if (a0 == ps && lane == 0) {
        const int w0 = wave_of(ps, T, W);
        a.first_slot[pbh] = w0 + pbh;
        a.n_pieces[pbh] = wave_of(ps + pu - 1, T, W) - w0 + 1;
      }
      run_piece(a, math, pbh, (int)(a0 - ps), (int)(a1 - ps), (int64_t)w + pbh,
                lane, col, grp);
    }
    run += __shfl(incl, 63);
  }
}

// The unit loop of the single-sequence partition for wave c of list bh,
// whose list has `units` units (L: the sequence length).  The wave's units
// are c, c + P, c + 2P, ...; it takes them last first, so that its first unit
// lies in the list's tail (the window blocks), whose page the folded
// selection knows before it has found the kept blocks.  page_at(i) gives the
// page id of the wave's i-th unit (unit c + i P).  With PRE, the first unit's
// K and V tiles (page pre_page) were requested by the caller into kf / vf.
template <bool PRE, class Math, class PageAt>
__device__ __forceinline__ void strided_loop(const AttnArgs& a, Math& math, int bh,
                                             int c, int units, int L,
                                             PageAt page_at, int lane, int col,
                                             int grp, uint4 (&kf)[4][4],
                                             uint4 (&vf)[2][8], int pre_page) {
  const int P = a.per_list;
  const int h = bh % a.n_kv;
  if (c >= units) return;  // uniform over the wave
  if (c == 0 && lane == 0) a.n_pieces[bh] = units < P ? units : P;
  const int n_mine = (units - c + P - 1) / P;
  const int n = units >> 1;
  const int last_valid = L - (((L + 127) >> 7) - 1) * kBlock;
  const int64_t head_off = (int64_t)h * (kBlock * kDim);
  const int64_t page_stride = (int64_t)a.n_kv * (kBlock * kDim);
  auto page_ok = [&](int p) { return (uint64_t)(int64_t)p < (uint64_t)a.n_pages; };
  auto tile_of = [&](int p) {
    return (page_ok(p) ? (int64_t)p * page_stride : 0) + head_off;
  };
  auto valid_of = [&](int u) {
    const int e = u >> 1;
    const int v = (e == n - 1 ? last_valid : kBlock) - kUnit * (u & 1);
    return v < 0 ? 0 : (v > kUnit ? kUnit : v);
  };

  int i = n_mine - 1;
  int page = PRE ? pre_page : page_at(i);
  int64_t tile = tile_of(page);
  if (!PRE) load_k_unit(kf, a.k_pages + tile, (c + i * P) & 1, col, grp);
  int page_next = i > 0 ? page_at(i - 1) : 0;
  // one unit: its scores, its V tile (unless requested ahead), the next
  // unit's K tile, then its softmax and PV products
  auto unit = [&](auto load_v) {
    const int u = c + i * P;
    typename Math::Scores s;
    math.scores(kf, s);
    __builtin_amdgcn_sched_barrier(0);
    if (decltype(load_v)::value) load_v_unit(vf, a.v_pages + tile, u & 1, col, grp);
    const bool cur_ok = page_ok(page);
    if (!cur_ok) report_page(page);
    const int valid = valid_of(u);
    if (i > 0) {  // prefetch the next unit's K tile
      page = page_next;
      tile = tile_of(page);
      page_next = i > 1 ? page_at(i - 2) : 0;
      load_k_unit(kf, a.k_pages + tile, (u - P) & 1, col, grp);
    }
    if (cur_ok && valid > 0) math.accumulate(s, vf, valid, a.scale_log2, col, grp);
#ifdef RKV_WAVE_STAMPS
    if constexpr (std::is_same<Math, MfmaMath>::value) {
      const int ord = n_mine - 1 - i;  // the wave's ord-th unit
      if (ord < kStampUnits) stamp_after(kStampUnit0 + ord, __float_as_uint(math.l_run));
    }
#endif
  };
  if (PRE) {
    unit(std::false_type());
    --i;
  }
  for (; i >= 0; --i) unit(std::true_type());
  math.finish(a, (int64_t)bh * P + c, lane, col, grp);
}

// Single-sequence partition (batch of one: every list has the same length,
// since the regions and k depend only on the sequence).  Wave w takes list
// w mod NB and, as piece c = w / NB of P per list, the list's units c,
// c + P, c + 2P, ...: its units sit at positions that do not depend on the
// list length, so the page ids of its first 64 units are requested together
// with the length -- one dependent memory round trip fewer before the first
// K tile than the range split.  Each list's units are dealt evenly (+-1 per
// wave) and the pieces are numbered by c.
template <class Math>
__device__ __forceinline__ void strided_body(const AttnArgs& a) {
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int NB = a.batch * a.n_kv;
  const int P = a.per_list;
  const int bh = (int)(blockIdx.x % (unsigned)NB);
  const int c = (int)(blockIdx.x / (unsigned)NB);
  const int b = bh / a.n_kv, h = bh - b * a.n_kv;
  const int32_t* mrow = a.merged + (int64_t)bh * a.m_cap;
  // --- one memory round trip: the list length, the sequence length, the
  // page ids of this wave's first 64 units and the query rows ---
  const int units = units_of(a, bh);
  const int L = clamp_len(a.lens[b], a.max_len);
  const int64_t e_lane = ((int64_t)c + (int64_t)lane * P) >> 1;
  const int pref = e_lane < a.m_cap ? mrow[e_lane] : 0;
  Math math;
  math.begin(a, b, h, col, grp);
  // L is used only past the branch in strided_loop; without this use the
  // compiler would request it only after n_merged has arrived (a second
  // round trip)
  __asm__ volatile("" ::"s"(L));
  // page id of this wave's i-th unit: requested above for i < 64
  auto page_at = [&](int i) {
    return i < 64 ? __shfl(pref, i) : mrow[(c + (int64_t)i * P) >> 1];
  };
  uint4 kf[4][4];
  uint4 vf[2][8];
  strided_loop<false>(a, math, bh, c, units, L, page_at, lane, col, grp, kf, vf, 0);
}

// ---------------------------------------------------------------------------
// Shared-prefix cascade (CSDN survey, section "Share--KV cache共享": cascade
// inference attends a prefix shared by several requests once for all of
// them and merges the partial results with the private suffix's the
// FlashDecoding way; ATB article, section 2.1: pages shared by reference
// count).  When the first c_shared logical blocks of every sequence sit on
// the same pages, a (page, KV head) tile of that prefix is read once for a
// group of c_q = 16 / group sequences, whose query heads fill the 16 MFMA
// columns together; a column whose sequence did not keep the block is
// masked out.  Each cascade wave takes one chunk of the prefix for one (KV
// head, group) and leaves one piece per sequence of the group.
// ---------------------------------------------------------------------------
struct CascadeMath : MfmaMath {
  // columns c = q * G + hh: query head hh of sequence b0 + q (zero padding
  // past the group or the batch); every lane loads a valid row
  __device__ __forceinline__ void begin_group(const AttnArgs& a, int b0, int h,
                                              int col, int grp) {
    const int G = a.group;
    const int q = col / G, hh = col - q * G;
    const bool ok = q < a.c_q && b0 + q < a.batch;
    const int b = ok ? b0 + q : b0;
    const uint16_t* qrow = a.q + ((int64_t)b * a.n_kv * G + h * G + (ok ? hh : 0)) * kDim;
    uint4 v[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) v[kk] = ld16(qrow + (4 * kk + grp) * 8);
    const uint32_t keep = ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      bq[kk] = as_bf16x8(make_uint4(v[kk].x & keep, v[kk].y & keep, v[kk].z & keep,
                                    v[kk].w & keep));
#pragma unroll
    for (int n8 = 0; n8 < 8; ++n8) acc[n8] = (f32x4){0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;
  }

  // One full 64-token unit; col_ok: this lane's column attends the block.
  // A column with no logit yet keeps m = -inf and l = 0 (exponents are
  // taken against 0 then, so no -inf - -inf appears).
  __device__ __forceinline__ void accumulate_cols(Scores& s, uint4 (&vf)[2][8],
                                                  bool col_ok, float sl2, int grp) {
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = col_ok ? s[t][r] * sl2 : kNegInf;
        s[t][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_base = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_base);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(s[t][r] - m_base);
        s[t][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) acc[n8][r] *= ar;
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const float p8[8] = {s[2 * pp][0],     s[2 * pp][1],     s[2 * pp][2],
                           s[2 * pp][3],     s[2 * pp + 1][0], s[2 * pp + 1][1],
                           s[2 * pp + 1][2], s[2 * pp + 1][3]};
      bf16x8 ph, pl;
      split_hi_lo(p8, ph, pl);
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) {
        const bf16x8 v = as_bf16x8(vf[pp][n8]);
        acc[n8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, v, acc[n8], 0, 0, 0);
        acc[n8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, v, acc[n8], 0, 0, 0);
      }
    }
  }

  // Column c's rows go to slot slot0 + c / G, row c mod G (a piece per
  // sequence of the group, in the ordinary G-row layout).
  __device__ __forceinline__ void finish_group(const AttnArgs& a, int64_t slot0,
                                               int lane, int col, int grp) {
    const int G = a.group;
    const int QG = a.c_q * G;
    float lt = l_run + __shfl_xor(l_run, 16);
    lt += __shfl_xor(lt, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 4 * grp + r;
      if (c < QG) {
        const int q = c / G;
        float* dst = a.part_acc + ((slot0 + q) * G + (c - q * G)) * kDim + col;
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8) dst[16 * n8] = acc[n8][r];
      }
    }
    if (lane < QG) {
      const int q = lane / G;
      a.part_ml[(slot0 + q) * G + (lane - q * G)] = make_float2(m_run, lt);
    }
  }
};

__device__ __forceinline__ void cascade_body(const AttnArgs& a) {
  __shared__ int cpage[64];      // the chunk's attended blocks: pages
  __shared__ uint32_t cqm[64];   // ... and which sequences of the group attend
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int cw = (int)blockIdx.x - a.n_waves;
  const int chunk = cw % a.c_chunks;
  const int hg = cw / a.c_chunks;
  const int g = hg % a.c_groups, h = hg / a.c_groups;
  const int Q = a.c_q;
  const int b0 = g * Q;
  const int j0 = chunk * a.c_chunk_blocks;
  int j1 = j0 + a.c_chunk_blocks;
  j1 = j1 < a.c_shared ? j1 : a.c_shared;

  // --- one round trip: block j0 + lane's page (table row 0) and, per
  // sequence of the group, its attended bit (clamped indexes, masked) ---
  const int j = j0 + lane;
  const int jc = j < a.c_shared ? j : a.c_shared - 1;
  const int page_raw = a.c_table[jc];
  uint32_t words[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int b = b0 + q < a.batch ? b0 + q : a.batch - 1;
    words[q] = a.c_mask[((int64_t)b * a.n_kv + h) * a.c_words + (jc >> 5)];
  }
  uint32_t qm = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const bool in = q < Q && b0 + q < a.batch;
    qm |= (in && ((words[q] >> (jc & 31)) & 1u)) ? 1u << q : 0u;
  }
  const bool any = j < j1 && qm != 0u;
  const uint64_t am = __ballot(any);
  const int n_att = __popcll(am);
  const int pos = lanes_below(am);
  // lanes without a block write slot 63, which is an entry only when every
  // lane has one
  cpage[any ? pos : 63] = page_raw;
  cqm[any ? pos : 63] = qm;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  CascadeMath math;
  math.begin_group(a, b0, h, col, grp);
  const int q_col = col / a.group;
  const int64_t head_off = (int64_t)h * (kBlock * kDim);
  const int64_t page_stride = (int64_t)a.n_kv * (kBlock * kDim);
  auto page_ok = [&](int p) { return (uint64_t)(int64_t)p < (uint64_t)a.n_pages; };
  auto tile_of = [&](int p) { return (page_ok(p) ? (int64_t)p * page_stride : 0) + head_off; };
  const int n_u = 2 * n_att;
  uint4 kf[4][4];
  uint4 vf[2][8];
  if (n_u > 0) {  // uniform
    int page = cpage[0];
    int64_t tile = tile_of(page);
    load_k_unit(kf, a.k_pages + tile, 0, col, grp);
    for (int u = 0; u < n_u; ++u) {
      typename CascadeMath::Scores sc;
      math.scores(kf, sc);
      __builtin_amdgcn_sched_barrier(0);
      load_v_unit(vf, a.v_pages + tile, u & 1, col, grp);
      const bool cur_ok = page_ok(page);
      if (!cur_ok) report_page(page);
      const uint32_t m_cur = cqm[u >> 1];
      if (u + 1 < n_u) {  // the next unit's K tile
        page = cpage[(u + 1) >> 1];
        tile = tile_of(page);
        load_k_unit(kf, a.k_pages + tile, (u + 1) & 1, col, grp);
      }
      const bool col_ok = q_col < 16 && ((m_cur >> q_col) & 1u) != 0u;
      if (cur_ok) math.accumulate_cols(sc, vf, col_ok, a.scale_log2, grp);
    }
  }
  math.finish_group(a, a.c_slot0 + (int64_t)cw * Q, lane, col, grp);
}

// ---------------------------------------------------------------------------
// Top-k and merge inside the attention launch (batch of one).
//
// The selection of a (sequence, KV head) list depends only on the list's
// scores, the sequence length and the parameters, and fits one wave when
// max_blocks <= 1024 (16 blocks per lane).  So instead of a separate top-k
// launch, every one of the list's P attention waves finds the selection
// itself from the same inputs -- the same set, since the set is defined by
// its values alone -- builds the merged page list in its own LDS and then
// runs the single-sequence unit loop on it.  The list's first wave also
// writes sel_ids, n_sel, merged and n_merged, as the top-k launch would.
//
// Selection (openGauss page, "Overall Solution": the top-K blocks by
// inner product): scores become order keys (unsigned order = float order);
// the k-th largest key T is found by deciding its bits from the top, one
// count of keys >= candidate per bit (ballots over the wave), stopping as
// soon as exactly k keys are >= T.  Kept: every key > T and, when the
// search ran to the last bit, the lowest-index keys == T up to k.  Lane l
// holds blocks l, l + 64, ..., so ascending (register, lane) is ascending
// block order.
// ---------------------------------------------------------------------------
constexpr int kFusedRegs = kFusedMaxBlocks / 64;

struct SelectIn {
  const int32_t* table;      // [1][max_blocks]
  const uint32_t* scores;    // [n_kv][max_blocks] raw fp32 bits
  const int32_t* prompt_lens;  // [1] or null (then lens)
  int max_blocks;
  int init_tokens, local_tokens, topk_ppm, dense_boundary;
  int32_t* sel_ids;   // [n_kv][k_cap]
  int32_t* n_sel;     // [n_kv]
  int k_cap;
  int32_t* merged;    // [n_kv][m_cap]
  int32_t* n_merged;  // [n_kv]
};

// The kept offload blocks of one list as per-lane bit masks (bit i: block
// lane + 64 i), for lists whose offload range ends within the first NR
// registers; cbits marks the offload blocks, 0 < k < n_off.
template <int NR>
__device__ __forceinline__ uint32_t kept_blocks(const uint32_t (&key)[kFusedRegs],
                                                uint32_t cbits, int k, int n_off,
                                                int lane) {
  // non-offload blocks as key 0: every threshold tried below is >= 1, so
  // they are never counted.  An offload block has key 0 only for the score
  // bit pattern 0xffffffff (a negative NaN): it ranks below every other
  // key, and if T stays 0 the tie pass below takes such blocks lowest index
  // first, as for any tied key.
  uint32_t keyc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) keyc[i] = ((cbits >> i) & 1u) ? key[i] : 0u;
  uint32_t T = 0;
  int cT = n_off;  // offload keys >= T
  // the bit mask and the candidate in scalar registers, so that a pass's
  // only vector work is its compares (with the loop counter and the
  // candidate in vector registers, every pass waited on the vector unit
  // two more times)
  for (uint32_t bm = 0x80000000u; bm != 0u;
       bm = (uint32_t)__builtin_amdgcn_readfirstlane((int)(bm >> 1))) {
    if (cT == k) break;  // exactly k keys >= T: they are the top k
    const uint32_t t = T | bm;
    // every compare of the pass first, then the counts: a count read
    // right after its compare waits for the vector unit's mask write
    uint64_t m[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) m[i] = __ballot(keyc[i] >= t);
    __builtin_amdgcn_sched_barrier(0);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) cnt += __popcll(m[i]);
    cnt = __builtin_amdgcn_readfirstlane(cnt);
    T = cnt >= k ? t : T;
    cT = cnt >= k ? cnt : cT;
  }
  uint32_t kbits = 0;
  if (cT == k) {  // here T >= 1 (k < n_off)
#pragma unroll
    for (int i = 0; i < NR; ++i) kbits |= keyc[i] >= T ? 1u << i : 0u;
    return kbits;
  }
  // T is the k-th largest key: keys > T, then the lowest blocks with key T
  int g = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i)
    g += __popcll(__ballot(((cbits >> i) & 1u) && key[i] > T));
  const int need = k - g;
  int eq_before = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const bool c = ((cbits >> i) & 1u) != 0u;
    const bool eq = c && key[i] == T;
    const uint64_t em = __ballot(eq);
    const bool take = (c && key[i] > T) || (eq && eq_before + lanes_below(em) < need);
    kbits |= take ? 1u << i : 0u;
    eq_before += __popcll(em);
  }
  return kbits;
}

template <class Math>
__device__ __forceinline__ void select_strided_body(const AttnArgs& a,
                                                    const SelectIn& f) {
  __shared__ int mlist[kFusedMaxBlocks + 1];  // + a spare slot
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int NB = a.n_kv;  // one sequence
  const int bh = (int)(blockIdx.x % (unsigned)NB);
  const int c = (int)(blockIdx.x / (unsigned)NB);
  const int mb = f.max_blocks;
  const uint32_t* srow_in = f.scores + (int64_t)bh * mb;

  // --- one memory round trip: lengths, the block-table row, the list's
  // scores and the query rows (clamped indexes, no lane conditions) ---
  const int lraw_v = a.lens[0];
  const int plen_v = (f.prompt_lens ? f.prompt_lens : a.lens)[0];
  // (the whole table row first: the first tile's page needs only it, and
  // loads arrive in the order they were requested)
  int tab[kFusedRegs];
  uint32_t raw[kFusedRegs];
#pragma unroll
  for (int i = 0; i < kFusedRegs; ++i) {
    int j = lane + 64 * i;
    j = j < mb ? j : mb - 1;
    tab[i] = f.table[j];
  }
#pragma unroll
  for (int i = 0; i < kFusedRegs; ++i) {
    int j = lane + 64 * i;
    j = j < mb ? j : mb - 1;
    raw[i] = srow_in[j];
  }
  Math math;
  math.begin(a, 0, bh, col, grp);
  // the lengths are the same on every lane: scalar registers from here on,
  // so the region arithmetic and the selection's branches stay scalar
  const int lraw = __builtin_amdgcn_readfirstlane(lraw_v);
  const int plen = __builtin_amdgcn_readfirstlane(plen_v);
#ifdef RKV_WAVE_STAMPS
  {
    uint32_t x = 0;  // every score and table entry has arrived
#pragma unroll
    for (int i = 0; i < kFusedRegs; ++i) x ^= raw[i] ^ (uint32_t)tab[i];
    stamp_after(kStampScores, x);
  }
#endif

  // --- regions and k, as the top-k launch takes them ---
  const int Ls = clamp_len(lraw, mb * kBlock);
  const Regions R = regions_of(Ls, f.init_tokens, f.local_tokens);
  const bool dense = plen < f.dense_boundary || f.topk_ppm >= kPpmOne;
  int k = dense ? R.n_off : topk_of(R.n_off, f.topk_ppm);
  k = k < R.n_off ? k : R.n_off;
  const bool ranked = k > 0 && k < R.n_off;
  const int ls = R.n_init + R.n_off;  // offload end (= first local block)
  const int lstart = R.local_start > R.n_init ? R.local_start : R.n_init;
  const int n_m = R.n_init + k + (R.nb - lstart);

  // --- the wave's first unit (its last in list order) is requested now,
  // before the selection, when its block does not depend on it: an init
  // block, a window block, or any block when every offload block is kept.
  // Entry e of the merged list is block e below n_init + k and block
  // lstart + (e - n_init - k) from there on.  A wave whose first unit is a
  // kept block (or that has no unit) requests block 0's tile instead and
  // does not use it: the code stays straight, since a load under a branch
  // would make the selection below wait for it where the branch rejoins. ---
  const int P = a.per_list;
  const int units = 2 * n_m;
  const int n_first = c < units ? (units - c + P - 1) / P : 0;
  const int u_first = c + (n_first - 1) * P;
  const int e_first = u_first >> 1;
  const bool early = n_first > 0 && (!ranked || e_first < R.n_init || e_first >= R.n_init + k);
  int j0 = e_first < R.n_init + k ? e_first : lstart + (e_first - R.n_init - k);
  j0 = early ? j0 : 0;
  int t0 = tab[0];
#pragma unroll
  for (int i = 1; i < kFusedRegs; ++i) t0 = (j0 >> 6) == i ? tab[i] : t0;
  const int early_page = __shfl(t0, j0 & 63);
  const int64_t early_tile =
      ((uint64_t)(int64_t)early_page < (uint64_t)a.n_pages
           ? (int64_t)early_page * a.n_kv * (kBlock * kDim) : 0) +
      (int64_t)bh * (kBlock * kDim);
  uint4 kf[4][4];
  uint4 vf[2][8];
  // only the K tile now: a compute unit keeps about one unit's K and V
  // (32 KiB) per wave pair in flight, and a wave asking for more stalls at
  // the request until earlier data returns -- the selection would then
  // start only after that.  The V tile follows the selection.
  load_k_unit(kf, a.k_pages + early_tile, u_first & 1, col, grp);
  __builtin_amdgcn_sched_barrier(0);

  // per-lane bit masks over the registers (bit i: block lane + 64 i): the
  // list's offload blocks and the kept ones
  uint32_t key[kFusedRegs];
#pragma unroll
  for (int i = 0; i < kFusedRegs; ++i) key[i] = order_key(__uint_as_float(raw[i]));
  uint32_t cbits = 0, kbits = 0;
#pragma unroll
  for (int i = 0; i < kFusedRegs; ++i) {
    const int j = lane + 64 * i;
    cbits |= (j >= R.n_init && j < ls) ? 1u << i : 0u;
  }
  if (ranked)  // uniform
    kbits = (ls + 63) >> 6 <= 8 ? kept_blocks<8>(key, cbits, k, R.n_off, lane)
                                : kept_blocks<16>(key, cbits, k, R.n_off, lane);
  stamp_after(kStampSearch, kbits);
  load_v_unit(vf, a.v_pages + early_tile, u_first & 1, col, grp);
  __builtin_amdgcn_sched_barrier(0);
  stamp(kStampVreq);

  // --- merged page list (init blocks, kept blocks, local blocks), with
  // selects only: entry dst of block j, -1 when j is not attended (its LDS
  // write then goes to a spare slot) ---
  const bool writer = c == 0;
  const bool all_kept = k == R.n_off;
  int32_t* sel_out = f.sel_ids + (int64_t)bh * f.k_cap;
  int32_t* m_out = f.merged + (int64_t)bh * a.m_cap;
  int pos_before = 0;
#pragma unroll
  for (int i = 0; i < kFusedRegs; ++i) {
    if (64 * i < R.nb) {  // uniform
      const int j = lane + 64 * i;
      const bool kj = ((kbits >> i) & 1u) != 0u;
      const uint64_t km = __ballot(kj);
      const int pos = pos_before + lanes_below(km);
      const bool offl = j >= R.n_init && j < lstart;
      int dst = j >= lstart ? R.n_init + k + (j - lstart) : j;
      dst = (offl && !all_kept) ? (kj ? R.n_init + pos : -1) : dst;
      dst = j < R.nb ? dst : -1;
      mlist[dst >= 0 ? dst : kFusedMaxBlocks] = tab[i];
      if (writer) {  // uniform
        if (dst >= 0) m_out[dst] = tab[i];
        if (kj) sel_out[pos] = j;
      }
      pos_before += __popcll(km);
    }
  }
  if (writer && !ranked)
    for (int r = lane; r < k; r += 64) sel_out[r] = R.n_init + r;
  if (writer && lane == 0) {
    f.n_sel[bh] = k;
    f.n_merged[bh] = n_m;
  }
  __syncthreads();  // the list in LDS is complete (one wave per workgroup)
  stamp(kStampList);

  const int L = clamp_len(lraw, a.max_len);
  auto page_at = [&](int i) { return mlist[(c + i * P) >> 1]; };
  if (early)
    strided_loop<true>(a, math, bh, c, 2 * n_m, L, page_at, lane, col, grp, kf, vf,
                       early_page);
  else
    strided_loop<false>(a, math, bh, c, 2 * n_m, L, page_at, lane, col, grp, kf, vf, 0);
  stamp_flush();
}

__global__ __launch_bounds__(64) void attn_select_mfma_kernel(AttnArgs a,
                                                              SelectIn f) {
  stamp_begin();
  select_strided_body<MfmaMath>(a, f);
}

template <class Math, bool STRIDED>
__device__ __forceinline__ void attn_body(const AttnArgs& a) {
  if constexpr (STRIDED) {
    strided_body<Math>(a);
  } else {
    if constexpr (std::is_same<Math, MfmaMath>::value) {
      if (blockIdx.x >= (unsigned)a.n_waves) {  // shared-prefix cascade waves
        cascade_body(a);
        return;
      }
    }
    split_body<Math>(a);
  }
}

template <bool STRIDED>
__global__ __launch_bounds__(64) void attn_mfma_kernel(AttnArgs a) {
  attn_body<MfmaMath, STRIDED>(a);
}

template <int G, bool STRIDED>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
  attn_body<ValuMath<G>, STRIDED>(a);
}

// ---------------------------------------------------------------------------
// Combine: one wave per (sequence, query head, 32-dim slice), so that even a
// batch of one sequence spreads the partial reads over many compute units.
// A list's pieces sit in consecutive slots: from slot list * P in the
// single-sequence partition (known up front, so the first pieces are
// requested together with the piece count), from the recorded first slot in
// the range split.  Lane (pg, d4) takes pieces pg, pg + 8, ... (up to 16
// requested at once) over the float4 d4 of the slice and folds them with a
// running maximum; the eight piece groups are then merged by log-sum-exp in
// a fixed butterfly order.
// ---------------------------------------------------------------------------
constexpr int kCombSlices = 4;   // 32-dim slices per query head
constexpr int kCombGroups = 8;   // piece groups per wave
constexpr int kCombDepth = 16;   // pieces in flight per lane
constexpr int kCombSpecMax = 20; // pieces per lane requested with the count

__device__ __forceinline__ void lse_fold(float& m, float& l, float4& acc, float m2,
                                         float l2, const float4& acc2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;  // both sides empty
  const float s1 = fast_exp2(m - mn), s2 = fast_exp2(m2 - mn);
  acc.x = acc.x * s1 + acc2.x * s2;
  acc.y = acc.y * s1 + acc2.y * s2;
  acc.z = acc.z * s1 + acc2.z * s2;
  acc.w = acc.w * s1 + acc2.w * s2;
  l = l * s1 + l2 * s2;
  m = mn;
}

__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int pg = lane >> 3, d4 = lane & 7;
  const int bq = blockIdx.x / kCombSlices, slice = blockIdx.x % kCombSlices;
  const int G = a.group;
  const int Hq = a.n_kv * G;
  const int b = bq / Hq, qh = bq - b * Hq;
  const int bh = b * a.n_kv + qh / G, hh = qh - (qh / G) * G;
  const bool strided = a.per_list > 0;  // uniform
  const int dim0 = 32 * slice + 4 * d4;
  float4* dst = reinterpret_cast<float4*>(out + (int64_t)bq * kDim + dim0);

  // single-sequence partition: the first `spec` pieces per lane are
  // requested together with the piece count (spec: the host's estimate of a
  // list's pieces per lane; 0 in the range split, whose slots are known
  // only from first_slot)
  const int P = strided ? a.per_list : a.n_slots;
  const int64_t sslot0 = strided ? (int64_t)bh * P : 0;
  const int spec = a.comb_spec;
  float2 ml0[kCombSpecMax];
  float4 v0[kCombSpecMax];
#pragma unroll
  for (int u = 0; u < kCombSpecMax; ++u) {
    if (u < spec) {
      const int i = pg + u * kCombGroups;
      const int64_t slot = sslot0 + (i < P ? i : P - 1);
      ml0[u] = a.part_ml[slot * G + hh];
      v0[u] = *reinterpret_cast<const float4*>(a.part_acc + (slot * G + hh) * kDim + dim0);
    }
  }
  const int units = units_of(a, bh);
  int np = a.n_pieces[bh];
  int fs = a.first_slot[bh];
  int64_t slot0 = sslot0;
  if (!strided) {  // uniform
    fs = fs < 0 ? 0 : (fs > a.n_slots - 1 ? a.n_slots - 1 : fs);
    slot0 = fs;
  }
  const int np_cap = strided ? P : a.n_slots - fs;
  np = units == 0 ? 0 : (np < 1 ? 1 : (np > np_cap ? np_cap : np));
  float m = kNegInf, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kCombSpecMax; ++u) {
    const int i = pg + u * kCombGroups;
    if (u < spec && i < np && ml0[u].y > 0.f) lse_fold(m, l, acc, ml0[u].x, ml0[u].y, v0[u]);
  }
  for (int base = pg + spec * kCombGroups; base < np; base += kCombDepth * kCombGroups) {
    float2 ml[kCombDepth];
    float4 v[kCombDepth];
#pragma unroll
    for (int u = 0; u < kCombDepth; ++u) {
      const int i = base + u * kCombGroups;
      if (i < np) {
        const int64_t slot = slot0 + i;
        ml[u] = a.part_ml[slot * G + hh];
        v[u] = *reinterpret_cast<const float4*>(a.part_acc + (slot * G + hh) * kDim + dim0);
      } else {
        ml[u] = make_float2(kNegInf, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombDepth; ++u)
      if (ml[u].y > 0.f) lse_fold(m, l, acc, ml[u].x, ml[u].y, v[u]);
  }
  // shared-prefix cascade: the pieces the (KV head, group) chunk waves left
  // for this sequence (chunk c's in slot c_slot0 + (wave * c_q + q))
  if (a.c_waves > 0) {  // uniform
    const int g = b / a.c_q, q = b - g * a.c_q;
    const int64_t cbase =
        a.c_slot0 + (int64_t)((qh / G) * a.c_groups + g) * a.c_chunks * a.c_q + q;
    for (int c = pg; c < a.c_chunks; c += kCombGroups) {
      const int64_t slot = cbase + (int64_t)c * a.c_q;
      const float2 mlc = a.part_ml[slot * G + hh];
      const float4 vc =
          *reinterpret_cast<const float4*>(a.part_acc + (slot * G + hh) * kDim + dim0);
      if (mlc.y > 0.f) lse_fold(m, l, acc, mlc.x, mlc.y, vc);
    }
  }
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    float4 a2;
    a2.x = __shfl_xor(acc.x, off);
    a2.y = __shfl_xor(acc.y, off);
    a2.z = __shfl_xor(acc.z, off);
    a2.w = __shfl_xor(acc.w, off);
    lse_fold(m, l, acc, m2, l2, a2);
  }
  // a previous part of the row (its normalized output and log2 softmax
  // sum): one more piece with m = its log-sum-exp and l = 1
  if (a.prev_lse) {  // uniform
    const float pm = a.prev_lse[bq];
    const float4 po =
        *reinterpret_cast<const float4*>(a.prev_out + (int64_t)bq * kDim + dim0);
    if (pm > kNegInf) lse_fold(m, l, acc, pm, 1.f, po);
  }
  if (pg == 0) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    *dst = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (a.lse_out && slice == 0 && lane == 0)
    a.lse_out[bq] = l > 0.f ? m + log2f(l) : kNegInf;
}

// Shared-prefix cascade, first launch: per (sequence, KV head) list, the
// shared blocks it attends as a bit mask and its merged table without them.
// A sequence's shared end is the caller's count of shared blocks, cut before
// its last block (the decoded token's, never shared) and at its first block
// whose page is not sequence 0's.  Below that end the list attends its init
// blocks, its kept blocks and its window blocks; those entries are always a
// prefix of the merged list (init, kept, window blocks, each ascending), so
// the private table is the rest of the row.
struct CascadePrep {
  const int32_t* table;  // [batch][max_blocks]
  int max_blocks;
  const int32_t* lens;
  const int32_t* merged;
  const int32_t* n_merged;
  int m_cap;
  const int32_t* sel_ids;  // the kept ids the merged table was built from
  const int32_t* n_sel;
  int k_cap;
  int shared, words, n_kv, init_tokens, local_tokens;
  uint32_t* mask;          // [lists][words]
  int32_t* merged_priv;    // [lists][m_cap]
  int32_t* n_priv;         // [lists]
};

constexpr int kMaxSharedWords = RKV_MAX_BLOCKS / 32;

__global__ __launch_bounds__(64) void cascade_prep_kernel(CascadePrep c) {
  __shared__ uint32_t bits[kMaxSharedWords];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / c.n_kv;
  const int L = clamp_len(c.lens[b], c.max_blocks * kBlock);
  const Regions R = regions_of(L, c.init_tokens, c.local_tokens);
  const int lstart = R.local_start > R.n_init ? R.local_start : R.n_init;
  int se = L > 0 ? (L - 1) >> 7 : 0;
  se = se < c.shared ? se : c.shared;
  const int32_t* row = c.table + (int64_t)b * c.max_blocks;
  for (int j0 = 0; j0 < se; j0 += 64) {  // uniform
    const int j = j0 + lane;
    const int jc = j < se ? j : se - 1;
    const uint64_t dm = __ballot(j < se && row[jc] != c.table[jc]);
    if (dm != 0) {
      se = j0 + __builtin_ctzll(dm);
      break;
    }
  }
  for (int w = lane; w < c.words; w += 64) bits[w] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // kept ids below the shared end (ascending: stop at the first chunk that
  // reaches it)
  int ns = c.n_sel[bh];
  if (ns < 0 || ns > c.k_cap) report_bounds(kBoundsCount, ns);
  ns = ns < 0 ? 0 : (ns > c.k_cap ? c.k_cap : ns);
  const int32_t* srow = c.sel_ids + (int64_t)bh * c.k_cap;
  int n_kept_sh = 0;
  for (int r0 = 0; r0 < ns; r0 += 64) {  // uniform
    const int r = r0 + lane;
    const int id = srow[r < ns ? r : ns - 1];
    const bool in = r < ns && id >= 0 && id < se;
    if (in) atomicOr(&bits[id >> 5], 1u << (id & 31));
    n_kept_sh += __popcll(__ballot(in));
    if (__ballot(r < ns && id >= se) != 0) break;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // init blocks [0, min(n_init, se)) and window blocks [lstart, se)
  const int init_end = R.n_init < se ? R.n_init : se;
  auto range_bits = [](int lo, int a0, int a1) {  // bits of [a0, a1) in word [lo, lo + 32)
    const int s0 = a0 > lo ? a0 - lo : 0;
    const int s1 = a1 < lo + 32 ? a1 - lo : 32;
    if (s1 <= s0) return 0u;
    const uint32_t hi = s1 >= 32 ? 0xffffffffu : (1u << s1) - 1u;
    return hi & ~((1u << s0) - 1u);
  };
  uint32_t* mrow = c.mask + (int64_t)bh * c.words;
  for (int w = lane; w < c.words; w += 64)
    mrow[w] = bits[w] | range_bits(32 * w, 0, init_end) | range_bits(32 * w, lstart, se);
  int n_m = c.n_merged[bh];
  if (n_m < 0 || n_m > c.m_cap) report_bounds(kBoundsCount, n_m);
  n_m = n_m < 0 ? 0 : (n_m > c.m_cap ? c.m_cap : n_m);
  int n_sh = init_end + n_kept_sh + (se > lstart ? se - lstart : 0);
  n_sh = n_sh < n_m ? n_sh : n_m;
  const int32_t* src = c.merged + (int64_t)bh * c.m_cap + n_sh;
  int32_t* dst = c.merged_priv + (int64_t)bh * c.m_cap;
  for (int e = lane; e < n_m - n_sh; e += 64) dst[e] = src[e];
  if (lane == 0) c.n_priv[bh] = n_m - n_sh;
}

}  // namespace

AttnPlan plan_attention(int batch, int n_q_heads, int n_kv_heads, int waves,
                        int m_cap, int n_cu) {
  AttnPlan p;
  (void)m_cap;
  // two waves per compute unit (one per SIMD pair): the whole split runs in
  // one round, each wave streaming its own run of units
  p.n_cu = n_cu > 0 ? n_cu : 256;
  p.n_waves = waves > 0 ? waves : 2 * p.n_cu;
  const int64_t lists = (int64_t)batch * (n_kv_heads > 0 ? n_kv_heads : 0);
  // a single sequence takes the length-independent strided partition: P
  // waves per list, slot list * P + c for wave c of a list; the range split
  // writes slot v + list for virtual wave v, at most W + lists slots
  p.per_list = 0;
  if (batch == 1 && n_kv_heads > 0) {
    p.per_list = p.n_waves / n_kv_heads;
    if (p.per_list < 1) p.per_list = 1;
  }
  p.n_slots = p.per_list > 0 ? lists * p.per_list : p.n_waves + lists;
  const int group = n_kv_heads > 0 ? n_q_heads / n_kv_heads : 0;
  p.partial_bytes = (size_t)p.n_slots * group * kDim * sizeof(float);
  p.ml_bytes = (size_t)p.n_slots * group * 2 * sizeof(float);
  // piece counts, then first slots
  p.count_bytes = ((size_t)lists * 2 * sizeof(int) + 255) / 256 * 256;
  // single-sequence partition: a list has per_list pieces at most; the
  // combine's eight lanes per slice request them before knowing the count
  int spec = (p.per_list + 7) / 8;
  p.comb_spec = p.per_list > 0 ? (spec < 1 ? 1 : (spec > 20 ? 20 : spec)) : 0;
  p.total_bytes = p.partial_bytes + p.ml_bytes + p.count_bytes;
  return p;
}

namespace {

AttnArgs attn_args(const Method& m, const AttnPlan& plan, float scale,
                   const uint16_t* q, const uint16_t* k_pages,
                   const uint16_t* v_pages, int64_t n_pages,
                   const int32_t* merged, const int32_t* n_merged, int m_cap,
                   const int32_t* lens, int batch, void* workspace) {
  AttnArgs a;
  a.q = q;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.n_pages = n_pages;
  a.merged = merged;
  a.n_merged = n_merged;
  a.lens = lens;
  a.part_acc = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) +
                                        plan.partial_bytes);
  a.n_pieces = reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                      plan.partial_bytes + plan.ml_bytes);
  a.first_slot = a.n_pieces + (int64_t)batch * m.n_kv_heads;
  a.n_slots = plan.n_slots;
  a.comb_spec = plan.comb_spec;
  a.n_cu = plan.n_cu;
  a.m_cap = m_cap;
  a.max_len = m_cap * kBlock;
  a.batch = batch;
  a.n_kv = m.n_kv_heads;
  a.group = m.group;
  a.n_waves = plan.n_waves;
  a.per_list = plan.per_list;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.c_table = nullptr;
  a.c_mask = nullptr;
  a.c_words = a.c_q = a.c_groups = a.c_chunks = a.c_chunk_blocks = 0;
  a.c_shared = a.c_waves = 0;
  a.c_slot0 = 0;
  a.prev_out = nullptr;
  a.prev_lse = nullptr;
  a.lse_out = nullptr;
  return a;
}

hipError_t launch_combine(const Method& m, const AttnArgs& a, int batch,
                          float* out, hipStream_t stream) {
  hipLaunchKernelGGL(attn_combine_kernel,
                     dim3((unsigned)(batch * m.n_q_heads * kCombSlices)), dim3(64), 0,
                     stream, a, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_attn(const Method& m, bool use_mfma,
                              const AttnPlan& plan, float scale,
                              const uint16_t* q, const uint16_t* k_pages,
                              const uint16_t* v_pages, int64_t n_pages,
                              const int32_t* merged, const int32_t* n_merged,
                              int m_cap, const int32_t* lens, int batch,
                              float* out, void* workspace, hipStream_t stream,
                              const float* prev_out, const float* prev_lse,
                              float* lse_out) {
  if (batch == 0) return hipSuccess;
  AttnArgs a = attn_args(m, plan, scale, q, k_pages, v_pages, n_pages, merged,
                         n_merged, m_cap, lens, batch, workspace);
  a.prev_out = prev_out;
  a.prev_lse = prev_lse;
  a.lse_out = lse_out;
  const int64_t waves =
      plan.per_list > 0 ? (int64_t)batch * m.n_kv_heads * plan.per_list : plan.n_waves;
  const dim3 grid((unsigned)waves), block(64);
  const bool strided = plan.per_list > 0;
  if (use_mfma) {
    if (strided)
      hipLaunchKernelGGL(attn_mfma_kernel<true>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<false>, grid, block, 0, stream, a);
  } else {
#define RKV_VALU_CASE(G)                                                        \
  case G:                                                                       \
    if (strided)                                                                \
      hipLaunchKernelGGL((attn_valu_kernel<G, true>), grid, block, 0, stream, a); \
    else                                                                        \
      hipLaunchKernelGGL((attn_valu_kernel<G, false>), grid, block, 0, stream, a); \
    break;
    switch (m.group) {
      RKV_VALU_CASE(1)
      RKV_VALU_CASE(2)
      RKV_VALU_CASE(4)
      RKV_VALU_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef RKV_VALU_CASE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(m, a, batch, out, stream);
}

namespace {
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

CascadePlan plan_cascade(int batch, int n_q_heads, int n_kv_heads, int waves,
                         int m_cap, int n_cu, int shared_blocks) {
  CascadePlan c;
  c.attn = plan_attention(batch, n_q_heads, n_kv_heads, waves, m_cap, n_cu);
  c.q = c.groups = c.chunks = c.chunk_blocks = c.waves = c.words = 0;
  c.shared = shared_blocks;
  c.slot0 = c.attn.n_slots;
  c.mask_off = c.priv_off = c.npriv_off = c.attn.total_bytes;
  c.total_bytes = c.attn.total_bytes;
  // nothing to share with fewer than two sequences (a batch of one takes the
  // single-sequence partition)
  if (batch < 2 || shared_blocks <= 0 || n_kv_heads <= 0 || c.attn.per_list > 0) return c;
  const int group = n_q_heads / n_kv_heads;
  c.q = 16 / group > 1 ? 16 / group : 1;
  c.q = c.q < batch ? c.q : batch;
  c.groups = (batch + c.q - 1) / c.q;
  // about one cascade wave per compute unit, chunks of at most 64 blocks
  const int combos = n_kv_heads * c.groups;
  int chunks = c.attn.n_cu / combos;
  const int min_chunks = (shared_blocks + 63) / 64;
  chunks = chunks < min_chunks ? min_chunks : chunks;
  chunks = chunks > shared_blocks ? shared_blocks : chunks;
  c.chunk_blocks = (shared_blocks + chunks - 1) / chunks;
  c.chunks = (shared_blocks + c.chunk_blocks - 1) / c.chunk_blocks;
  c.waves = combos * c.chunks;
  c.words = (shared_blocks + 31) / 32;
  // cascade slots after the range split's, c_q per cascade wave
  AttnPlan& p = c.attn;
  c.slot0 = p.n_slots;
  p.n_slots += c.waves * c.q;
  p.partial_bytes = (size_t)p.n_slots * group * kDim * sizeof(float);
  p.ml_bytes = (size_t)p.n_slots * group * 2 * sizeof(float);
  p.total_bytes = p.partial_bytes + p.ml_bytes + p.count_bytes;
  const size_t lists = (size_t)batch * n_kv_heads;
  c.mask_off = round256(p.total_bytes);
  c.priv_off = c.mask_off + round256(lists * c.words * sizeof(uint32_t));
  c.npriv_off = c.priv_off + round256(lists * (size_t)m_cap * sizeof(int32_t));
  c.total_bytes = c.npriv_off + round256(lists * sizeof(int32_t));
  return c;
}

hipError_t launch_decode_attn_cascade(const Method& m, const CascadePlan& plan,
                                      float scale, const uint16_t* q,
                                      const uint16_t* k_pages, const uint16_t* v_pages,
                                      int64_t n_pages, const int32_t* merged,
                                      const int32_t* n_merged, int m_cap,
                                      const int32_t* sel_ids, const int32_t* n_sel,
                                      int k_cap, const int32_t* table, int max_blocks,
                                      const int32_t* lens, int batch, float* out,
                                      void* workspace, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (plan.waves == 0)
    return launch_decode_attn(m, true, plan.attn, scale, q, k_pages, v_pages, n_pages,
                              merged, n_merged, m_cap, lens, batch, out, workspace,
                              stream);
  char* ws = static_cast<char*>(workspace);
  uint32_t* mask = reinterpret_cast<uint32_t*>(ws + plan.mask_off);
  int32_t* merged_priv = reinterpret_cast<int32_t*>(ws + plan.priv_off);
  int32_t* n_priv = reinterpret_cast<int32_t*>(ws + plan.npriv_off);
  CascadePrep c;
  c.table = table;
  c.max_blocks = max_blocks;
  c.lens = lens;
  c.merged = merged;
  c.n_merged = n_merged;
  c.m_cap = m_cap;
  c.sel_ids = sel_ids;
  c.n_sel = n_sel;
  c.k_cap = k_cap;
  c.shared = plan.shared;
  c.words = plan.words;
  c.n_kv = m.n_kv_heads;
  c.init_tokens = m.init_tokens;
  c.local_tokens = m.local_tokens;
  c.mask = mask;
  c.merged_priv = merged_priv;
  c.n_priv = n_priv;
  hipLaunchKernelGGL(cascade_prep_kernel, dim3((unsigned)(batch * m.n_kv_heads)),
                     dim3(64), 0, stream, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnArgs a = attn_args(m, plan.attn, scale, q, k_pages, v_pages, n_pages, merged_priv,
                         n_priv, m_cap, lens, batch, workspace);
  a.c_table = table;
  a.c_mask = mask;
  a.c_words = plan.words;
  a.c_q = plan.q;
  a.c_groups = plan.groups;
  a.c_chunks = plan.chunks;
  a.c_chunk_blocks = plan.chunk_blocks;
  a.c_shared = plan.shared;
  a.c_waves = plan.waves;
  a.c_slot0 = plan.slot0;
  hipLaunchKernelGGL(attn_mfma_kernel<false>,
                     dim3((unsigned)(plan.attn.n_waves + plan.waves)), dim3(64), 0,
                     stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(m, a, batch, out, stream);
}

bool fused_select_attn_ok(const Method& m, bool use_mfma, const AttnPlan& plan,
                          int batch, int max_blocks) {
  return batch == 1 && use_mfma && !m.per_sequence && plan.per_list > 0 &&
         max_blocks <= kFusedMaxBlocks;
}

hipError_t launch_select_attn(const Method& m, bool use_mfma, const AttnPlan& plan,
                              float scale, const uint16_t* q,
                              const uint16_t* k_pages, const uint16_t* v_pages,
                              int64_t n_pages, const int32_t* table, int max_blocks,
                              const int32_t* lens, const int32_t* prompt_lens,
                              const uint32_t* scores, int32_t* sel_ids,
                              int32_t* n_sel, int k_cap, int32_t* merged,
                              int32_t* n_merged, int m_cap, float* out,
                              void* workspace, hipStream_t stream) {
  if (!fused_select_attn_ok(m, use_mfma, plan, 1, max_blocks)) return hipErrorInvalidValue;
  const AttnArgs a = attn_args(m, plan, scale, q, k_pages, v_pages, n_pages, merged,
                               n_merged, m_cap, lens, 1, workspace);
  SelectIn f;
  f.table = table;
  f.scores = scores;
  f.prompt_lens = prompt_lens;
  f.max_blocks = max_blocks;
  f.init_tokens = m.init_tokens;
  f.local_tokens = m.local_tokens;
  f.topk_ppm = m.topk_ppm;
  f.dense_boundary = m.dense_boundary;
  f.sel_ids = sel_ids;
  f.n_sel = n_sel;
  f.k_cap = k_cap;
  f.merged = merged;
  f.n_merged = n_merged;
  const dim3 grid((unsigned)((int64_t)m.n_kv_heads * plan.per_list)), block(64);
  hipLaunchKernelGGL(attn_select_mfma_kernel, grid, block, 0, stream, a, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(m, a, 1, out, stream);
}

RKV_BOUNDS_SETTER(set_bounds_word_attn)

hipError_t read_wave_stamps(uint64_t* dst, int waves) {
#ifdef RKV_WAVE_STAMPS
  if (waves < 0 || waves > kWaveStampWaves) return hipErrorInvalidValue;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(rkv_wave_stamps),
                             (size_t)waves * kWaveStampSlots * sizeof(uint64_t), 0,
                             hipMemcpyDeviceToHost);
#else
  (void)dst;
  (void)waves;
  return hipErrorNotSupported;
#endif
}

}  // namespace rkv
