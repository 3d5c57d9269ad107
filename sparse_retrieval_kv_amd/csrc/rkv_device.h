// Device helpers shared by the HIP kernel files (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

// bf16 bit pattern(s) -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Out-of-range device values the kernels clamp or skip.  Debug builds
// (RKV_DEBUG) record the first one into a caller-given device word (kind in
// the top byte, the value in the low 32 bits; see rkv_debug_set_report);
// other builds compile the reports out.
constexpr unsigned kBoundsLength = 1;    // a length outside [0, max]
constexpr unsigned kBoundsPage = 2;      // a page id outside the device pool
constexpr unsigned kBoundsBlock = 3;     // a block id outside the list's range
constexpr unsigned kBoundsCount = 4;     // a list count above its capacity
constexpr unsigned kBoundsHostPage = 5;  // a host page id outside the host pool

#ifdef RKV_DEBUG
// one per code object; set by this file's RKV_BOUNDS_SETTER function
static __device__ unsigned long long* rkv_bounds_word;
__device__ __forceinline__ void report_bounds(unsigned kind, int64_t value) {
  unsigned long long* w = rkv_bounds_word;
  if (w != nullptr)
    atomicCAS(w, 0ull, ((unsigned long long)kind << 56) |
                           (unsigned long long)(uint32_t)value);
}
#define RKV_BOUNDS_SETTER(name)                                              \
  hipError_t name(unsigned long long* word) {                                \
    return hipMemcpyToSymbol(HIP_SYMBOL(rkv_bounds_word), &word, sizeof(word)); \
  }
#else
__device__ __forceinline__ void report_bounds(unsigned, int64_t) {}
#define RKV_BOUNDS_SETTER(name) \
  hipError_t name(unsigned long long*) { return hipErrorNotSupported; }
#endif

// Current length of sequence b, clamped to [0, max_len].
__device__ __forceinline__ int clamp_len(int L, int max_len) {
  if (L < 0 || L > max_len) report_bounds(kBoundsLength, L);
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// Block split of a sequence of L tokens (openGauss page, "Overall
// Solution"): init blocks [0, n_init), offload [n_init, local_start) when
// local_start > n_init, local blocks [max(local_start, n_init), nb).
struct Regions {
  int nb, n_init, local_start, n_off;
};

__device__ __forceinline__ Regions regions_of(int L, int init_tokens,
                                              int local_tokens) {
  Regions r;
  if (L <= 0) {
    r.nb = r.n_init = r.local_start = r.n_off = 0;
    return r;
  }
  r.nb = (L + 127) >> 7;
  const int ib = (int)(((int64_t)init_tokens + 127) >> 7);
  r.n_init = ib < r.nb ? ib : r.nb;
  int tail = L - local_tokens;
  tail = tail > 0 ? tail : 0;
  const int ls = tail >> 7;
  r.local_start = ls < r.nb - 1 ? ls : r.nb - 1;
  r.n_off = r.local_start > r.n_init ? r.local_start - r.n_init : 0;
  return r;
}

// k = ceil(n * ppm / 10^6) in exact integer arithmetic.
__device__ __forceinline__ int topk_of(int n_off, int ppm) {
  return (int)(((int64_t)n_off * ppm + 999999) / 1000000);
}

// fp32 -> uint32 whose unsigned order is the float order (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0 + +0 = +0 under round-to-nearest
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Set bits of a wave mask in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-wide sum / max over all 64 lanes.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace rkv
