// rkv_decode_step_static: the decode step with its two workspaces taken from
// a scratch array the library keeps in device memory, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The step's kernels are the ones
// rkv_decode_step launches; only where their scratch lives differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rkv.h"
#include "rkv_internal.h"

namespace {

// One copy per GPU, from the library's first use on that GPU until the
// process ends.  In host code `scratch` names a host-side stand-in: kernels
// get the device address that hipGetSymbolAddress returns for the current
// device, never the array's name.
static __device__ __align__(256) unsigned char scratch[RKV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The current device's scratch address, looked up once per device with that
// device current.
rkv_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return rkv::report(RKV_ERR_HIP, "rkv_decode_step_static: hipGetDevice: %s",
                       hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return rkv::report(RKV_ERR_UNSUPPORTED,
                       "rkv_decode_step_static: device %d beyond the %d supported",
                       dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return rkv::report(RKV_ERR_HIP,
                         "rkv_decode_step_static: hipGetSymbolAddress of the scratch "
                         "array on device %d: %s", dev, hipGetErrorString(e));
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return RKV_OK;
}

}  // namespace

extern "C" rkv_status rkv_decode_step_static(
    const rkv_params* params, const uint16_t* k_new, const uint16_t* v_new,
    uint16_t* k_pages, uint16_t* v_pages, int64_t n_pages, const uint16_t* q,
    float* reps, const int32_t* block_table, const int32_t* lens,
    const int32_t* prompt_lens, int32_t batch, int32_t max_blocks,
    int32_t* sel_ids, int32_t* n_sel, int32_t k_cap, int32_t* merged,
    int32_t* n_merged, int32_t m_cap, float* out, hipStream_t stream) {
  if (params == nullptr)
    return rkv::report(RKV_ERR_INVALID_ARG, "params is NULL");
  // select workspace first (rounded to 256 bytes), the attention workspace
  // after it: disjoint, both 256-byte aligned
  const size_t sel = (rkv_select_workspace_size(params, batch, max_blocks) + 255) /
                     256 * 256;
  const size_t att = rkv_attn_workspace_size(params, batch, m_cap);
  if (sel + att > (size_t)RKV_STATIC_SCRATCH_BYTES)
    return rkv::report(RKV_ERR_UNSUPPORTED,
                       "rkv_decode_step_static: this shape needs %zu bytes of "
                       "scratch (select %zu + attention %zu), above the static "
                       "limit of %zu bytes; use rkv_decode_step with caller "
                       "workspaces", sel + att, sel, att,
                       (size_t)RKV_STATIC_SCRATCH_BYTES);
  void* base = nullptr;
  const rkv_status s = scratch_address(&base);
  if (s != RKV_OK) return s;
  char* b = static_cast<char*>(base);
  return rkv::decode_step_impl(params, k_new, v_new, k_pages, v_pages, n_pages, q,
                               reps, block_table, lens, prompt_lens, batch,
                               max_blocks, sel_ids, n_sel, k_cap, merged, n_merged,
                               m_cap, out, b, sel, b + sel,
                               (size_t)RKV_STATIC_SCRATCH_BYTES - sel, stream);
}
