// Split-K paged decode attention with log-sum-exp combine (gfx950).
//
// softmax(q K^T / sqrt(d)) V for one query token per head (rkmt.cn ATB
// KV-cache article, section 1.1), reading K/V pages through a block table
// (same article, section 2.2), over the merged block list of each
// (sequence, KV head).  The list is cut into chunks of `chunk` blocks; one
// wave computes the online-softmax partial (m, l, acc) of one chunk for all
// query heads of the group, and a second kernel merges the partials of a
// head by their log-sum-exp (partial results merged the FlashDecoding way,
// CSDN "KV cache" survey, section "Share--KV cache共享").
//
// MFMA schedule for one 128-token block (query heads padded to 16):
//   S^T[16 tokens x 16 heads] = K_tile[16 x 128] . Q^T[128 x 16]
//     with v_mfma_f32_16x16x32_bf16, four K-steps of 32 dims per tile,
//     eight tiles per block.  The accumulator layout (lane l holds rows
//     4(l/16)+r, column l%16) puts four tokens of head l%16 in each lane.
//   O[16 heads x 16 dims] += P[16 x 32 tokens] . V[32 tokens x 16 dims]
//     with the same instruction: the two S^T tiles of a 32-token pair are
//     exactly the A-operand layout of P (row = head l%16, eight tokens per
//     lane group), so P never leaves the registers.  P is split into a bf16
//     high part and a bf16 residual (two MFMAs) so the weights keep ~16
//     significant bits; V is bf16 already.
// Token order inside a block is chosen so that every load is 16 contiguous
// bytes per lane: in pair pp, lane group g owns tokens 32pp+8g .. 32pp+8g+7.
//   K tile (pair pp, half e): row m holds token 32pp + 8(m/4) + 4e + m%4,
//   V: lane (col, g) reads dim 16n+col, tokens 32pp+8g..+7 (one 16-byte
//   piece of the dim-major V tile).
// Every block's (page, head) K and V tiles are read exactly once.
#include "rkv_device.h"
#include "rkv_internal.h"

#include <math.h>

namespace rkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -INFINITY;

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
  float* part_acc;   // [B*Hq][n_chunks][128]
  float2* part_ml;   // [B*Hq][n_chunks]
  int m_cap, max_len, batch, n_kv, group, chunk, n_chunks;
  float scale_log2;  // scale * log2(e)
};

// Work item = (chunk i, sequence-head bh), chunk-major so that the first
// chunks of every (b, h) come first.
__global__ __launch_bounds__(64) void attn_mfma_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int n_bh = a.batch * a.n_kv;
  const int i = blockIdx.x / n_bh;
  const int bh = blockIdx.x - i * n_bh;
  int n = a.n_merged[bh];
  n = n < 0 ? 0 : (n > a.m_cap ? a.m_cap : n);
  const int e0 = i * a.chunk;
  if (e0 >= n) return;
  const int e1 = e0 + a.chunk < n ? e0 + a.chunk : n;
  const int b = bh / a.n_kv, h = bh - b * a.n_kv;
  const int G = a.group;
  const int Hq = a.n_kv * G;
  const int L = clamp_len(a.lens[b], a.max_len);
  const int last_valid = L - (((L + 127) >> 7) - 1) * kBlock;

  // Q^T as the B operand: lane (col, grp) holds head col, dims of chunk
  // 4kk+grp (8 bf16) for kk = 0..3; padded heads are zero.
  bf16x8 bq[4];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * Hq + h * G + col) * kDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col < G) v = ld16(qrow + (4 * kk + grp) * 8);
      bq[kk] = as_bf16x8(v);
    }
  }

  f32x4 acc[8];
#pragma unroll
  for (int n8 = 0; n8 < 8; ++n8) acc[n8] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const int32_t* mrow = a.merged + (int64_t)bh * a.m_cap;

  for (int e = e0; e < e1; ++e) {
    const int page = mrow[e];
    if ((uint64_t)(int64_t)page >= (uint64_t)a.n_pages) continue;
    const int valid = (e == n - 1) ? last_valid : kBlock;
    const int64_t tile = ((int64_t)page * a.n_kv + h) * (kBlock * kDim);
    const uint16_t* K = a.k_pages + tile;
    const uint16_t* V = a.v_pages + tile;

    uint4 kf[8][4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int row = 32 * (t >> 1) + 8 * (col >> 2) + 4 * (t & 1) + (col & 3);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kf[t][kk] = ld16(K + row * kDim + (4 * kk + grp) * 8);
    }
    uint4 vf[4][8];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8)
        vf[pp][n8] = ld16(V + (16 * n8 + col) * kBlock + 32 * pp + 8 * grp);

    f32x4 s[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      s[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[t][kk]),
                                                       bq[kk], s[t], 0, 0, 0);
    }

    // log2-domain logits, mask past the sequence end, block max per head
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[t][r] * a.scale_log2;
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
    for (int t = 0; t < 8; ++t)
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

    if (valid < kBlock) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
          vf[pp][n8] = mask_tokens(vf[pp][n8], 32 * pp + 8 * grp, valid);
    }

#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
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

  // the four lane groups of a head hold disjoint token subsets of l
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  const int64_t head0 = (int64_t)b * Hq + h * G;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * grp + r;
    if (hh < G) {
      float* dst = a.part_acc + ((head0 + hh) * a.n_chunks + i) * kDim + col;
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) dst[16 * n8] = acc[n8][r];
    }
  }
  if (lane < G) a.part_ml[(head0 + lane) * a.n_chunks + i] = make_float2(m_run, lt);
}

// Vector-ALU variant with the same memory schedule (same tiles, same
// per-lane 16-byte pieces, same token order): the q.k products use
// v_dot2_f32_bf16 on bf16 pairs and the p.v products fp32 FMAs, so the two
// variants differ only in where the dot products run.
//   QK: lane (col, grp) holds 32 dims (chunks 4kk+grp) of token row col of
//       each tile; partial dots for the G heads are summed over the four lane
//       groups, leaving S[token(t, col)][head] in every lane of column col.
//   PV: lane (col, grp) owns dims 16n+col and tokens 32pp+8grp..+7; the
//       weights of those tokens are fetched from the lanes that own their
//       rows, and the per-lane partial sums are folded over the lane groups
//       once per work item.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int n_bh = a.batch * a.n_kv;
  const int i = blockIdx.x / n_bh;
  const int bh = blockIdx.x - i * n_bh;
  int n = a.n_merged[bh];
  n = n < 0 ? 0 : (n > a.m_cap ? a.m_cap : n);
  const int e0 = i * a.chunk;
  if (e0 >= n) return;
  const int e1 = e0 + a.chunk < n ? e0 + a.chunk : n;
  const int b = bh / a.n_kv, h = bh - b * a.n_kv;
  const int Hq = a.n_kv * G;
  const int L = clamp_len(a.lens[b], a.max_len);
  const int last_valid = L - (((L + 127) >> 7) - 1) * kBlock;

  uint4 qv[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qv[hh][kk] = ld16(a.q + ((int64_t)b * Hq + h * G + hh) * kDim +
                        (4 * kk + grp) * 8);

  float acc[8][G];
#pragma unroll
  for (int n8 = 0; n8 < 8; ++n8)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) acc[n8][hh] = 0.f;
  float m_run[G], l_run[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_run[hh] = kNegInf;
    l_run[hh] = 0.f;
  }
  const int32_t* mrow = a.merged + (int64_t)bh * a.m_cap;

  for (int e = e0; e < e1; ++e) {
    const int page = mrow[e];
    if ((uint64_t)(int64_t)page >= (uint64_t)a.n_pages) continue;
    const int valid = (e == n - 1) ? last_valid : kBlock;
    const int64_t tile = ((int64_t)page * a.n_kv + h) * (kBlock * kDim);
    const uint16_t* K = a.k_pages + tile;
    const uint16_t* V = a.v_pages + tile;

    uint4 kf[8][4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int row = 32 * (t >> 1) + 8 * (col >> 2) + 4 * (t & 1) + (col & 3);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kf[t][kk] = ld16(K + row * kDim + (4 * kk + grp) * 8);
    }
    uint4 vf[4][8];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8)
        vf[pp][n8] = ld16(V + (16 * n8 + col) * kBlock + 32 * pp + 8 * grp);

    // S[t][hh] for token row col of tile t, summed over the lane groups
    float s[8][G];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float c = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) c = dot8(kf[t][kk], qv[hh][kk], c);
        c += __shfl_xor(c, 16);
        c += __shfl_xor(c, 32);
        const int tok = 32 * (t >> 1) + 8 * (col >> 2) + 4 * (t & 1) + (col & 3);
        s[t][hh] = tok < valid ? c * a.scale_log2 : kNegInf;
      }
    float alpha[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 8; ++t) mx = fmaxf(mx, s[t][hh]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[hh], mx);
      alpha[hh] = fast_exp2(m_run[hh] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        s[t][hh] = fast_exp2(s[t][hh] - m_new);
        ps += s[t][hh];
      }
      l_run[hh] = l_run[hh] * alpha[hh] + ps;  // over this lane's token rows
      m_run[hh] = m_new;
#pragma unroll
      for (int n8 = 0; n8 < 8; ++n8) acc[n8][hh] *= alpha[hh];
    }

    if (valid < kBlock) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int n8 = 0; n8 < 8; ++n8)
          vf[pp][n8] = mask_tokens(vf[pp][n8], 32 * pp + 8 * grp, valid);
    }
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
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

  const int64_t head0 = (int64_t)b * Hq + h * G;
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
      if (grp == 0)
        a.part_acc[((head0 + hh) * a.n_chunks + i) * kDim + 16 * n8 + col] = x;
    }
    if (lane == 0)
      a.part_ml[(head0 + hh) * a.n_chunks + i] = make_float2(m_run[hh], lt);
  }
}

// One 128-thread workgroup per (sequence, query head): merge the partials of
// its active chunks in chunk order.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a,
                                                           float* __restrict__ out) {
  const int bq = blockIdx.x;
  const int G = a.group;
  const int Hq = a.n_kv * G;
  const int b = bq / Hq, qh = bq - b * Hq;
  int n = a.n_merged[b * a.n_kv + qh / G];
  n = n < 0 ? 0 : (n > a.m_cap ? a.m_cap : n);
  const int nc = (n + a.chunk - 1) / a.chunk;
  const float2* ml = a.part_ml + (int64_t)bq * a.n_chunks;
  const float* pa = a.part_acc + (int64_t)bq * a.n_chunks * kDim + threadIdx.x;
  float M = kNegInf;
  for (int c = 0; c < nc; ++c) {
    const float2 v = ml[c];
    if (v.y > 0.f) M = fmaxf(M, v.x);
  }
  float num = 0.f, den = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float2 v = ml[c];
    if (v.y > 0.f) {
      const float w = fast_exp2(v.x - M);
      den += w * v.y;
      num += w * pa[(int64_t)c * kDim];
    }
  }
  out[(int64_t)bq * kDim + threadIdx.x] = den > 0.f ? num / den : 0.f;
}

}  // namespace

AttnPlan plan_attention(int batch, int n_q_heads, int n_kv_heads, int m_cap,
                        int split_blocks) {
  AttnPlan p;
  int chunk = split_blocks;
  if (chunk <= 0) {
    // about 16K potential work items: one block per item for single
    // sequences, more for large batches (each item streams chunk x 64 KiB)
    const int64_t cells = (int64_t)batch * n_kv_heads * m_cap;
    chunk = (int)(cells / 16384);
    chunk = chunk < 1 ? 1 : (chunk > 64 ? 64 : chunk);
  }
  if (chunk > m_cap) chunk = m_cap > 0 ? m_cap : 1;
  p.chunk = chunk;
  p.n_chunks = (m_cap + chunk - 1) / chunk;
  const size_t heads = (size_t)batch * n_q_heads * (size_t)p.n_chunks;
  p.partial_bytes = heads * kDim * sizeof(float);
  p.ml_bytes = heads * 2 * sizeof(float);
  return p;
}

hipError_t launch_decode_attn(const Method& m, bool use_mfma,
                              const AttnPlan& plan, float scale,
                              const uint16_t* q, const uint16_t* k_pages,
                              const uint16_t* v_pages, int64_t n_pages,
                              const int32_t* merged, const int32_t* n_merged,
                              int m_cap, const int32_t* lens, int batch,
                              float* out, void* workspace, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
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
  a.m_cap = m_cap;
  a.max_len = m_cap * kBlock;
  a.batch = batch;
  a.n_kv = m.n_kv_heads;
  a.group = m.group;
  a.chunk = plan.chunk;
  a.n_chunks = plan.n_chunks;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int64_t items = (int64_t)plan.n_chunks * batch * m.n_kv_heads;
  if (items > 0) {
    const dim3 grid((unsigned)items), block(64);
    if (use_mfma) {
      hipLaunchKernelGGL(attn_mfma_kernel, grid, block, 0, stream, a);
    } else {
      switch (m.group) {
        case 1: hipLaunchKernelGGL(attn_valu_kernel<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(attn_valu_kernel<2>, grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL(attn_valu_kernel<4>, grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL(attn_valu_kernel<8>, grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_combine_kernel, dim3(batch * m.n_q_heads), dim3(128),
                     0, stream, a, out);
  return hipGetLastError();
}

}  // namespace rkv
