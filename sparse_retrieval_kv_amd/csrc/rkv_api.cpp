// Host side of the C ABI declared in include/rkv.h: argument validation,
// workspace sizing, error reporting and kernel dispatch.  Nothing here
// allocates device memory; every launch goes on the caller's stream.
#include "rkv.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <string>

#include "rkv_internal.h"

namespace {

thread_local std::string g_last_error;

rkv_status fail(rkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

rkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return RKV_OK;
  return fail(RKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

#define RKV_REQUIRE(cond, status, ...) \
  do {                                 \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

// Checks shared by every call; fills the kernels' view of the parameters.
rkv_status check_params(const rkv_params* p, rkv::Method* m) {
  RKV_REQUIRE(p != nullptr, RKV_ERR_INVALID_ARG, "params is NULL");
  RKV_REQUIRE(p->block_size == RKV_BLOCK_SIZE, RKV_ERR_UNSUPPORTED,
              "block_size %d unsupported (only 128)", p->block_size);
  RKV_REQUIRE(p->head_dim == RKV_HEAD_DIM, RKV_ERR_UNSUPPORTED,
              "head_dim %d unsupported (only 128)", p->head_dim);
  RKV_REQUIRE(p->n_q_heads > 0 && p->n_kv_heads > 0, RKV_ERR_INVALID_ARG,
              "head counts must be positive (q %d, kv %d)", p->n_q_heads,
              p->n_kv_heads);
  RKV_REQUIRE(p->n_q_heads % p->n_kv_heads == 0, RKV_ERR_INVALID_ARG,
              "n_q_heads %d is not a multiple of n_kv_heads %d",
              p->n_q_heads, p->n_kv_heads);
  RKV_REQUIRE(p->n_q_heads / p->n_kv_heads <= RKV_MAX_GROUP,
              RKV_ERR_UNSUPPORTED, "group size %d above %d",
              p->n_q_heads / p->n_kv_heads, RKV_MAX_GROUP);
  RKV_REQUIRE(p->init_tokens >= 0 && p->local_tokens >= 0, RKV_ERR_INVALID_ARG,
              "init_tokens / local_tokens must be >= 0");
  RKV_REQUIRE(p->topk_ppm >= 0 && p->topk_ppm <= RKV_PPM_ONE,
              RKV_ERR_INVALID_ARG, "topk_ppm %d outside [0, 1000000]",
              p->topk_ppm);
  RKV_REQUIRE(p->dense_boundary >= 0, RKV_ERR_INVALID_ARG,
              "dense_boundary must be >= 0");
  RKV_REQUIRE(isfinite(p->scale), RKV_ERR_INVALID_ARG, "scale is not finite");
  RKV_REQUIRE(p->attn_impl >= RKV_ATTN_AUTO && p->attn_impl <= RKV_ATTN_VALU,
              RKV_ERR_INVALID_ARG, "attn_impl %d unknown", p->attn_impl);
  RKV_REQUIRE(p->split_waves >= 0 && p->split_waves <= (1 << 16),
              RKV_ERR_INVALID_ARG, "split_waves %d outside [0, 65536]",
              p->split_waves);
  RKV_REQUIRE(p->select_mode == RKV_SELECT_PER_HEAD ||
                  p->select_mode == RKV_SELECT_PER_SEQUENCE,
              RKV_ERR_INVALID_ARG, "select_mode %d unknown", p->select_mode);
  RKV_REQUIRE(p->copy_lanes >= 0 && p->copy_lanes <= RKV_MAX_COPY_LANES,
              RKV_ERR_INVALID_ARG, "copy_lanes %d outside [0, %d]", p->copy_lanes,
              RKV_MAX_COPY_LANES);
  if (m) {
    m->per_sequence = p->select_mode == RKV_SELECT_PER_SEQUENCE;
    m->n_q_heads = p->n_q_heads;
    m->n_kv_heads = p->n_kv_heads;
    m->group = p->n_q_heads / p->n_kv_heads;
    m->init_tokens = p->init_tokens;
    m->local_tokens = p->local_tokens;
    m->topk_ppm = p->topk_ppm;
    m->dense_boundary = p->dense_boundary;
  }
  return RKV_OK;
}

rkv_status check_sizes(int32_t batch, int32_t max_blocks) {
  RKV_REQUIRE(batch >= 0, RKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  RKV_REQUIRE(max_blocks >= 1 && max_blocks <= RKV_MAX_BLOCKS,
              RKV_ERR_INVALID_ARG, "max_blocks %d outside [1, %d]",
              max_blocks, RKV_MAX_BLOCKS);
  return RKV_OK;
}

// Call extent: keeps every grid of the call within a dispatch's 32-bit
// work-item count (the largest is the staging copy's 256 work-items per
// list entry: 2^31 at the limit).
rkv_status check_extent(const rkv_params* p, int32_t batch, int64_t row) {
  const int64_t rows = (int64_t)batch * p->n_q_heads;
  const int64_t entries = (int64_t)batch * p->n_kv_heads * (row > 1 ? row : 1);
  RKV_REQUIRE(rows <= RKV_MAX_QUERY_ROWS, RKV_ERR_UNSUPPORTED,
              "batch * n_q_heads = %lld above %d", (long long)rows,
              RKV_MAX_QUERY_ROWS);
  RKV_REQUIRE(entries <= RKV_MAX_LIST_ENTRIES, RKV_ERR_UNSUPPORTED,
              "batch * n_kv_heads * %lld = %lld above %d", (long long)row,
              (long long)entries, RKV_MAX_LIST_ENTRIES);
  return RKV_OK;
}

int64_t max3(int64_t a, int64_t b, int64_t c) {
  const int64_t m = a > b ? a : b;
  return m > c ? m : c;
}

rkv_status check_pool(const void* pool, int64_t n_pages, const char* name) {
  RKV_REQUIRE(pool != nullptr, RKV_ERR_INVALID_ARG, "%s is NULL", name);
  RKV_REQUIRE(aligned16(pool), RKV_ERR_INVALID_ARG,
              "%s is not 16-byte aligned", name);
  RKV_REQUIRE(n_pages >= 1, RKV_ERR_INVALID_ARG, "n_pages %lld < 1",
              (long long)n_pages);
  return RKV_OK;
}

int64_t topk_cap(const rkv_params* p, int32_t max_blocks) {
  const bool dense_possible =
      p->dense_boundary > 0 || p->topk_ppm >= RKV_PPM_ONE;
  if (dense_possible) return max_blocks;
  return ((int64_t)max_blocks * p->topk_ppm + RKV_PPM_ONE - 1) / RKV_PPM_ONE;
}

#define RKV_TRY(expr)                  \
  do {                                 \
    rkv_status s_ = (expr);            \
    if (s_ != RKV_OK) return s_;       \
  } while (0)

}  // namespace

extern "C" {

rkv_params rkv_params_default(int32_t n_q_heads, int32_t n_kv_heads) {
  rkv_params p;
  p.block_size = RKV_BLOCK_SIZE;
  p.head_dim = RKV_HEAD_DIM;
  p.n_q_heads = n_q_heads;
  p.n_kv_heads = n_kv_heads;
  p.init_tokens = 1024;
  p.local_tokens = 7192;
  p.topk_ppm = 200000;
  p.dense_boundary = 32768;
  p.scale = 1.0f / sqrtf((float)RKV_HEAD_DIM);
  p.attn_impl = RKV_ATTN_AUTO;
  p.split_waves = 0;
  p.select_mode = RKV_SELECT_PER_HEAD;
  p.copy_lanes = 0;
  return p;
}

int32_t rkv_abi_version(void) { return RKV_ABI_VERSION; }

const char* rkv_status_string(rkv_status s) {
  switch (s) {
    case RKV_OK: return "ok";
    case RKV_ERR_INVALID_ARG: return "invalid argument";
    case RKV_ERR_UNSUPPORTED: return "unsupported";
    case RKV_ERR_WORKSPACE: return "workspace too small";
    case RKV_ERR_HIP: return "HIP error";
    case RKV_ERR_BOUNDS: return "out-of-range device value";
  }
  return "unknown status";
}

const char* rkv_last_error(void) { return g_last_error.c_str(); }

rkv_status rkv_build_reps(const rkv_params* params, const uint16_t* k_pages,
                          int64_t n_pages, const int32_t* block_table,
                          int32_t max_blocks, const int32_t* lens,
                          const int32_t* block_begin, int32_t batch,
                          float* reps, hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_extent(params, batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_REQUIRE(block_table && lens && reps, RKV_ERR_INVALID_ARG,
              "block_table, lens and reps must not be NULL");
  RKV_REQUIRE(aligned16(reps), RKV_ERR_INVALID_ARG, "reps is not 16-byte aligned");
  return hip_status(rkv::launch_build_reps(k_pages, n_pages, block_table,
                                           max_blocks, lens, block_begin, batch,
                                           m.n_kv_heads, reps, stream),
                    "rkv_build_reps launch");
}

rkv_status rkv_append_kv(const rkv_params* params, const uint16_t* k_new,
                         const uint16_t* v_new, uint16_t* k_pages,
                         uint16_t* v_pages, int64_t n_pages,
                         const int32_t* block_table, int32_t max_blocks,
                         const int32_t* lens, int32_t batch, float* reps,
                         hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_extent(params, batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_REQUIRE(k_new && v_new && block_table && lens, RKV_ERR_INVALID_ARG,
              "k_new, v_new, block_table and lens must not be NULL");
  RKV_REQUIRE(aligned16(k_new) && aligned16(v_new) && (!reps || aligned16(reps)),
              RKV_ERR_INVALID_ARG, "k_new, v_new and reps must be 16-byte aligned");
  return hip_status(rkv::launch_append_kv(k_new, v_new, k_pages, v_pages,
                                          n_pages, block_table, max_blocks,
                                          lens, batch, m.n_kv_heads, reps,
                                          stream),
                    "rkv_append_kv launch");
}

int32_t rkv_topk_capacity(const rkv_params* params, int32_t max_blocks) {
  if (!params || max_blocks < 0) return 0;
  return (int32_t)topk_cap(params, max_blocks);
}

size_t rkv_select_workspace_size(const rkv_params* params, int32_t batch,
                                 int32_t max_blocks) {
  if (!params || batch <= 0 || max_blocks <= 0 || params->n_kv_heads <= 0) return 0;
  return rkv::select_keys_bytes(batch, params->n_kv_heads, max_blocks);
}

namespace {

rkv_status select_common(const rkv_params* params, const uint16_t* q,
                         const float* reps, const int32_t* block_table,
                         const int32_t* lens, const int32_t* prompt_lens,
                         int32_t batch, int32_t max_blocks, int32_t* sel_ids,
                         int32_t* n_sel, int32_t k_cap, int32_t* merged,
                         int32_t* n_merged, int32_t m_cap, void* workspace,
                         size_t workspace_bytes, const rkv::AppendOp* append,
                         hipStream_t stream, const char* what) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_extent(params, batch, max_blocks));
  RKV_REQUIRE(q && reps && block_table && lens && n_sel && (sel_ids || k_cap == 0),
              RKV_ERR_INVALID_ARG,
              "q, reps, block_table, lens, sel_ids and n_sel must not be NULL");
  RKV_REQUIRE(aligned16(q) && aligned16(reps), RKV_ERR_INVALID_ARG,
              "q and reps must be 16-byte aligned");
  RKV_REQUIRE(k_cap >= topk_cap(params, max_blocks), RKV_ERR_INVALID_ARG,
              "k_cap %d below the required %lld", k_cap,
              (long long)topk_cap(params, max_blocks));
  if (merged) {
    RKV_REQUIRE(n_merged != nullptr, RKV_ERR_INVALID_ARG,
                "n_merged must not be NULL when merged is given");
    RKV_REQUIRE(m_cap >= max_blocks, RKV_ERR_INVALID_ARG,
                "m_cap %d below max_blocks %d", m_cap, max_blocks);
  }
  const size_t need = rkv_select_workspace_size(params, batch, max_blocks);
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace),
              RKV_ERR_WORKSPACE, "select workspace %zu bytes, need %zu",
              workspace_bytes, need);
  return hip_status(rkv::launch_select(m, q, reps, block_table, lens,
                                       prompt_lens, batch, max_blocks, sel_ids,
                                       n_sel, k_cap, merged, n_merged, m_cap,
                                       workspace, append, stream),
                    what);
}

}  // namespace

rkv_status rkv_select(const rkv_params* params, const uint16_t* q,
                      const float* reps, const int32_t* block_table,
                      const int32_t* lens, const int32_t* prompt_lens,
                      int32_t batch, int32_t max_blocks, int32_t* sel_ids,
                      int32_t* n_sel, int32_t k_cap, int32_t* merged,
                      int32_t* n_merged, int32_t m_cap, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return select_common(params, q, reps, block_table, lens, prompt_lens, batch,
                       max_blocks, sel_ids, n_sel, k_cap, merged, n_merged,
                       m_cap, workspace, workspace_bytes, nullptr, stream,
                       "rkv_select launch");
}

rkv_status rkv_append_select(const rkv_params* params, const uint16_t* k_new,
                             const uint16_t* v_new, uint16_t* k_pages,
                             uint16_t* v_pages, int64_t n_pages,
                             const uint16_t* q, float* reps,
                             const int32_t* block_table, const int32_t* lens,
                             const int32_t* prompt_lens, int32_t batch,
                             int32_t max_blocks, int32_t* sel_ids,
                             int32_t* n_sel, int32_t k_cap, int32_t* merged,
                             int32_t* n_merged, int32_t m_cap, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_REQUIRE(k_new && v_new, RKV_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
  RKV_REQUIRE(aligned16(k_new) && aligned16(v_new), RKV_ERR_INVALID_ARG,
              "k_new and v_new must be 16-byte aligned");
  const rkv::AppendOp op{k_new, v_new, k_pages, v_pages, n_pages, reps};
  return select_common(params, q, reps, block_table, lens, prompt_lens, batch,
                       max_blocks, sel_ids, n_sel, k_cap, merged, n_merged,
                       m_cap, workspace, workspace_bytes, &op, stream,
                       "rkv_append_select launch");
}

rkv_status rkv_merge_table(const rkv_params* params, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* lens,
                           const int32_t* sel_ids, const int32_t* n_sel,
                           int32_t k_cap, int32_t batch,
                           const int32_t* host_table, int64_t stage_page0,
                           int32_t* merged, int32_t* n_merged, int32_t m_cap,
                           hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_REQUIRE(block_table && lens && sel_ids && n_sel && merged && n_merged,
              RKV_ERR_INVALID_ARG, "a required pointer is NULL");
  RKV_REQUIRE(k_cap >= 0, RKV_ERR_INVALID_ARG, "k_cap %d < 0", k_cap);
  RKV_TRY(check_extent(params, batch, max3(max_blocks, k_cap, m_cap)));
  RKV_REQUIRE(m_cap >= max_blocks, RKV_ERR_INVALID_ARG,
              "m_cap %d below max_blocks %d", m_cap, max_blocks);
  RKV_REQUIRE(!host_table || (stage_page0 >= 0 &&
                               stage_page0 + (int64_t)batch * k_cap <= (int64_t)INT32_MAX),
              RKV_ERR_INVALID_ARG,
              "with a host table, stage_page0 must be >= 0 and staging page "
              "ids must fit int32");
  return hip_status(rkv::launch_merge(m, block_table, max_blocks, lens, sel_ids,
                                      n_sel, k_cap, batch, host_table, stage_page0,
                                      merged, n_merged, m_cap, stream),
                    "rkv_merge_table launch");
}

namespace {

// The staging kernels read the host pools directly: they must be pinned host
// memory mapped into the device address space.
rkv_status host_views(const uint16_t* host_k, const uint16_t* host_v,
                      const uint16_t* dev_view[2]) {
  const uint16_t* pools[2] = {host_k, host_v};
  for (int i = 0; i < 2; ++i) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, pools[i]) != hipSuccess ||
        attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr ||
        attr.hostPointer != static_cast<const void*>(pools[i])) {
      (void)hipGetLastError();
      return fail(RKV_ERR_INVALID_ARG,
                  "%s is not pinned host memory mapped for the device",
                  i == 0 ? "host_k" : "host_v");
    }
    dev_view[i] = static_cast<const uint16_t*>(attr.devicePointer);
  }
  return RKV_OK;
}

}  // namespace

rkv_status rkv_stage_blocks(const rkv_params* params, const uint16_t* host_k,
                            const uint16_t* host_v, int64_t n_host_pages,
                            const int32_t* host_table, int32_t max_blocks,
                            const int32_t* sel_ids, const int32_t* n_sel,
                            int32_t k_cap, int32_t batch, uint16_t* k_pages,
                            uint16_t* v_pages, int64_t n_pages,
                            int64_t stage_page0, hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_TRY(check_pool(host_k, n_host_pages, "host_k"));
  RKV_TRY(check_pool(host_v, n_host_pages, "host_v"));
  RKV_REQUIRE(host_table && sel_ids && n_sel, RKV_ERR_INVALID_ARG,
              "host_table, sel_ids and n_sel must not be NULL");
  RKV_REQUIRE(k_cap >= 1, RKV_ERR_INVALID_ARG, "k_cap %d < 1", k_cap);
  RKV_TRY(check_extent(params, batch, max3(max_blocks, k_cap, 1)));
  RKV_REQUIRE(stage_page0 >= 0 &&
                  stage_page0 + (int64_t)batch * k_cap <= n_pages &&
                  stage_page0 + (int64_t)batch * k_cap <= (int64_t)INT32_MAX,
              RKV_ERR_INVALID_ARG,
              "staging pages [%lld, +%lld) do not fit in the %lld-page pool",
              (long long)stage_page0, (long long)batch * k_cap,
              (long long)n_pages);
  const uint16_t* dev_view[2] = {nullptr, nullptr};
  RKV_TRY(host_views(host_k, host_v, dev_view));
  return hip_status(rkv::launch_stage(dev_view[0], dev_view[1], n_host_pages,
                                      host_table, max_blocks, sel_ids, n_sel,
                                      k_cap, batch, m.n_kv_heads, k_pages,
                                      v_pages, n_pages, stage_page0, stream),
                    "rkv_stage_blocks launch");
}

rkv_status rkv_offload_blocks(const rkv_params* params, const uint16_t* k_pages,
                              const uint16_t* v_pages, int64_t n_pages,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* lens, int32_t batch,
                              const int32_t* host_table, uint16_t* host_k,
                              uint16_t* host_v, int64_t n_host_pages,
                              hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_TRY(check_pool(host_k, n_host_pages, "host_k"));
  RKV_TRY(check_pool(host_v, n_host_pages, "host_v"));
  RKV_REQUIRE(block_table && lens && host_table, RKV_ERR_INVALID_ARG,
              "block_table, lens and host_table must not be NULL");
  RKV_TRY(check_extent(params, batch, max_blocks));
  const uint16_t* dev_view[2] = {nullptr, nullptr};
  RKV_TRY(host_views(host_k, host_v, dev_view));
  return hip_status(rkv::launch_offload(m, k_pages, v_pages, n_pages, block_table,
                                        max_blocks, lens, batch, host_table,
                                        const_cast<uint16_t*>(dev_view[0]),
                                        const_cast<uint16_t*>(dev_view[1]),
                                        n_host_pages, stream),
                    "rkv_offload_blocks launch");
}

size_t rkv_stage_workspace_size(const rkv_params* params, int32_t batch,
                                int32_t k_cap) {
  if (!params || params->n_kv_heads <= 0 || batch <= 0 || k_cap <= 0) return 0;
  return rkv::resident_workspace_bytes(batch, params->n_kv_heads, k_cap);
}

rkv_status rkv_stage_resident(const rkv_params* params, const uint16_t* host_k,
                              const uint16_t* host_v, int64_t n_host_pages,
                              const int32_t* host_table,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* lens, const int32_t* sel_ids,
                              const int32_t* n_sel, int32_t k_cap, int32_t batch,
                              int32_t slot_cap, int32_t* slot_ids,
                              int32_t* slot_cursor, uint16_t* k_pages,
                              uint16_t* v_pages, int64_t n_pages,
                              int64_t stage_page0, int32_t* merged,
                              int32_t* n_merged, int32_t m_cap, int32_t* n_staged,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_TRY(check_pool(host_k, n_host_pages, "host_k"));
  RKV_TRY(check_pool(host_v, n_host_pages, "host_v"));
  RKV_REQUIRE(host_table && block_table && lens && sel_ids && n_sel && slot_ids &&
                  slot_cursor && merged && n_merged,
              RKV_ERR_INVALID_ARG, "a required pointer is NULL");
  RKV_REQUIRE(k_cap >= 1 && k_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "k_cap %d outside [1, %d]", k_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(slot_cap >= 1 && slot_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "slot_cap %d outside [1, %d]", slot_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(m_cap >= max_blocks, RKV_ERR_INVALID_ARG,
              "m_cap %d below max_blocks %d", m_cap, max_blocks);
  RKV_TRY(check_extent(params, batch, max3(m_cap, k_cap, slot_cap)));
  RKV_REQUIRE(stage_page0 >= 0 &&
                  stage_page0 + (int64_t)batch * slot_cap <= n_pages &&
                  stage_page0 + (int64_t)batch * slot_cap <= (int64_t)INT32_MAX,
              RKV_ERR_INVALID_ARG,
              "staging pages [%lld, +%lld) do not fit in the %lld-page pool",
              (long long)stage_page0, (long long)batch * slot_cap,
              (long long)n_pages);
  const size_t need = rkv_stage_workspace_size(params, batch, k_cap);
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace),
              RKV_ERR_WORKSPACE, "staging workspace %zu bytes, need %zu",
              workspace_bytes, need);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "workspace is not 16-byte aligned");
  const uint16_t* dev_view[2] = {nullptr, nullptr};
  RKV_TRY(host_views(host_k, host_v, dev_view));
  return hip_status(rkv::launch_stage_resident(
                        m, dev_view[0], dev_view[1], n_host_pages, host_table,
                        block_table, lens, max_blocks, sel_ids, n_sel, k_cap,
                        batch, slot_cap, slot_ids, slot_cursor, k_pages, v_pages,
                        n_pages, stage_page0,
                        merged, n_merged, m_cap, n_staged, workspace, stream),
                    "rkv_stage_resident launch");
}

rkv_status rkv_stage_plan(const rkv_params* params, const int32_t* host_table,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* lens, const int32_t* sel_ids,
                          const int32_t* n_sel, int32_t k_cap, int32_t batch,
                          int32_t slot_cap, int32_t* slot_ids, int32_t* slot_cursor,
                          int64_t n_pages, int64_t stage_page0, int32_t* merged,
                          int32_t* n_merged, int32_t m_cap, int32_t* merged_new,
                          int32_t* n_new, int32_t* n_staged, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_REQUIRE(host_table && block_table && lens && sel_ids && n_sel && slot_ids &&
                  slot_cursor && merged && n_merged,
              RKV_ERR_INVALID_ARG, "a required pointer is NULL");
  RKV_REQUIRE((merged_new == nullptr) == (n_new == nullptr), RKV_ERR_INVALID_ARG,
              "merged_new and n_new must be given together");
  RKV_REQUIRE(k_cap >= 1 && k_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "k_cap %d outside [1, %d]", k_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(slot_cap >= 1 && slot_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "slot_cap %d outside [1, %d]", slot_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(m_cap >= max_blocks, RKV_ERR_INVALID_ARG,
              "m_cap %d below max_blocks %d", m_cap, max_blocks);
  RKV_REQUIRE(n_pages >= 1, RKV_ERR_INVALID_ARG, "n_pages %lld < 1",
              (long long)n_pages);
  RKV_TRY(check_extent(params, batch, max3(m_cap, k_cap, slot_cap)));
  RKV_REQUIRE(stage_page0 >= 0 &&
                  stage_page0 + (int64_t)batch * slot_cap <= n_pages &&
                  stage_page0 + (int64_t)batch * slot_cap <= (int64_t)INT32_MAX,
              RKV_ERR_INVALID_ARG,
              "staging pages [%lld, +%lld) do not fit in the %lld-page pool",
              (long long)stage_page0, (long long)batch * slot_cap,
              (long long)n_pages);
  const size_t need = rkv_stage_workspace_size(params, batch, k_cap);
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace),
              RKV_ERR_WORKSPACE, "staging workspace %zu bytes, need %zu",
              workspace_bytes, need);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "workspace is not 16-byte aligned");
  return hip_status(rkv::launch_stage_plan(m, host_table, block_table, lens, max_blocks,
                                           sel_ids, n_sel, k_cap, batch, slot_cap,
                                           slot_ids, slot_cursor, stage_page0, merged,
                                           n_merged, m_cap, n_staged, workspace, stream,
                                           merged_new, n_new),
                    "rkv_stage_plan launch");
}

rkv_status rkv_stage_copy(const rkv_params* params, const uint16_t* host_k,
                          const uint16_t* host_v, int64_t n_host_pages,
                          const int32_t* host_table, int32_t max_blocks, int32_t k_cap,
                          int32_t batch, int32_t slot_cap, uint16_t* k_pages,
                          uint16_t* v_pages, int64_t n_pages, int64_t stage_page0,
                          const void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_TRY(check_pool(host_k, n_host_pages, "host_k"));
  RKV_TRY(check_pool(host_v, n_host_pages, "host_v"));
  RKV_REQUIRE(host_table != nullptr, RKV_ERR_INVALID_ARG, "host_table is NULL");
  RKV_REQUIRE(k_cap >= 1 && k_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "k_cap %d outside [1, %d]", k_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(slot_cap >= 1 && slot_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "slot_cap %d outside [1, %d]", slot_cap, RKV_MAX_BLOCKS);
  RKV_TRY(check_extent(params, batch, max3(k_cap, slot_cap, 1)));
  RKV_REQUIRE(stage_page0 >= 0 &&
                  stage_page0 + (int64_t)batch * slot_cap <= n_pages &&
                  stage_page0 + (int64_t)batch * slot_cap <= (int64_t)INT32_MAX,
              RKV_ERR_INVALID_ARG,
              "staging pages [%lld, +%lld) do not fit in the %lld-page pool",
              (long long)stage_page0, (long long)batch * slot_cap,
              (long long)n_pages);
  const size_t need = rkv_stage_workspace_size(params, batch, k_cap);
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace),
              RKV_ERR_WORKSPACE, "staging workspace %zu bytes, need %zu",
              workspace_bytes, need);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "workspace is not 16-byte aligned");
  const uint16_t* dev_view[2] = {nullptr, nullptr};
  RKV_TRY(host_views(host_k, host_v, dev_view));
  return hip_status(rkv::launch_stage_copy(m, dev_view[0], dev_view[1], n_host_pages,
                                           host_table, max_blocks, k_cap, batch,
                                           slot_cap, k_pages, v_pages, n_pages,
                                           stage_page0, workspace, stream),
                    "rkv_stage_copy launch");
}

size_t rkv_stage_host_list_size(const rkv_params* params, int32_t batch,
                                int32_t k_cap) {
  if (!params || params->n_kv_heads <= 0 || batch <= 0 || k_cap <= 0) return 0;
  const size_t lists = (size_t)batch * params->n_kv_heads;
  return lists * k_cap * 2 * sizeof(int32_t) + lists * sizeof(int32_t);
}

namespace {

// The host list of the copy-engine staging calls must be pinned host memory
// (the device writes it with an asynchronous copy).
rkv_status check_host_list(const void* host_list, size_t bytes, size_t need) {
  RKV_REQUIRE(host_list != nullptr, RKV_ERR_INVALID_ARG, "host_list is NULL");
  RKV_REQUIRE(bytes >= need, RKV_ERR_WORKSPACE, "host_list %zu bytes, need %zu",
              bytes, need);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_list) != hipSuccess ||
      attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(RKV_ERR_INVALID_ARG, "host_list is not pinned host memory");
  }
  return RKV_OK;
}

rkv_status copy_issue(const rkv::StageCopyArgs& a, int64_t* tiles, hipEvent_t done,
                      const char* what) {
  hipError_t e = rkv::issue_stage_copies(a, tiles);
  if (e == hipSuccess && done) e = hipEventRecord(done, a.side);
  return hip_status(e, what);
}

}  // namespace

rkv_status rkv_stage_blocks_async(const rkv_params* params, const uint16_t* host_k,
                                  const uint16_t* host_v, int64_t n_host_pages,
                                  const int32_t* host_table_host, int32_t max_blocks,
                                  const int32_t* sel_ids, const int32_t* n_sel,
                                  int32_t k_cap, int32_t batch, uint16_t* k_pages,
                                  uint16_t* v_pages, int64_t n_pages,
                                  int64_t stage_page0, void* host_list,
                                  size_t host_list_bytes, hipStream_t stream,
                                  hipStream_t side, hipEvent_t done) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_TRY(check_pool(host_k, n_host_pages, "host_k"));
  RKV_TRY(check_pool(host_v, n_host_pages, "host_v"));
  RKV_REQUIRE(host_table_host && sel_ids && n_sel, RKV_ERR_INVALID_ARG,
              "host_table_host, sel_ids and n_sel must not be NULL");
  RKV_REQUIRE(k_cap >= 1, RKV_ERR_INVALID_ARG, "k_cap %d < 1", k_cap);
  RKV_TRY(check_extent(params, batch, max3(max_blocks, k_cap, 1)));
  RKV_REQUIRE(stage_page0 >= 0 &&
                  stage_page0 + (int64_t)batch * k_cap <= n_pages &&
                  stage_page0 + (int64_t)batch * k_cap <= (int64_t)INT32_MAX,
              RKV_ERR_INVALID_ARG,
              "staging pages [%lld, +%lld) do not fit in the %lld-page pool",
              (long long)stage_page0, (long long)batch * k_cap,
              (long long)n_pages);
  const uint16_t* dev_view[2] = {nullptr, nullptr};
  RKV_TRY(host_views(host_k, host_v, dev_view));
  const size_t lists = (size_t)batch * m.n_kv_heads;
  const size_t ids_bytes = lists * k_cap * sizeof(int32_t);
  RKV_TRY(check_host_list(host_list, host_list_bytes, ids_bytes + lists * sizeof(int32_t)));
  if (lists == 0) return RKV_OK;
  int32_t* ids = static_cast<int32_t*>(host_list);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(host_list) + ids_bytes);
  hipError_t e = hipMemcpyAsync(ids, sel_ids, ids_bytes, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(counts, n_sel, lists * sizeof(int32_t), hipMemcpyDeviceToHost,
                       stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "rkv_stage_blocks_async: kept ids to the host");
  rkv::StageCopyArgs a;
  a.host_k = host_k;
  a.host_v = host_v;
  a.n_host_pages = n_host_pages;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.n_pages = n_pages;
  a.host_table = host_table_host;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.n_kv = m.n_kv_heads;
  a.stage_page0 = stage_page0;
  a.slots_per_seq = k_cap;
  a.whole_pages = m.per_sequence;
  a.ids = ids;
  a.pairs = nullptr;
  a.counts = counts;
  a.row = k_cap;
  a.side = side;
  a.lanes = params->copy_lanes;
  return copy_issue(a, nullptr, done, "rkv_stage_blocks_async copies");
}

rkv_status rkv_stage_resident_async(
    const rkv_params* params, const uint16_t* host_k, const uint16_t* host_v,
    int64_t n_host_pages, const int32_t* host_table, const int32_t* host_table_host,
    const int32_t* block_table, int32_t max_blocks, const int32_t* lens,
    const int32_t* sel_ids, const int32_t* n_sel, int32_t k_cap, int32_t batch,
    int32_t slot_cap, int32_t* slot_ids, int32_t* slot_cursor, uint16_t* k_pages,
    uint16_t* v_pages, int64_t n_pages, int64_t stage_page0, int32_t* merged,
    int32_t* n_merged, int32_t m_cap, int32_t* n_staged, void* workspace,
    size_t workspace_bytes, void* host_list, size_t host_list_bytes,
    hipStream_t stream, hipStream_t side, hipEvent_t done) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_TRY(check_pool(host_k, n_host_pages, "host_k"));
  RKV_TRY(check_pool(host_v, n_host_pages, "host_v"));
  RKV_REQUIRE(host_table && host_table_host && block_table && lens && sel_ids && n_sel &&
                  slot_ids && slot_cursor && merged && n_merged,
              RKV_ERR_INVALID_ARG, "a required pointer is NULL");
  RKV_REQUIRE(k_cap >= 1 && k_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "k_cap %d outside [1, %d]", k_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(slot_cap >= 1 && slot_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "slot_cap %d outside [1, %d]", slot_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(m_cap >= max_blocks, RKV_ERR_INVALID_ARG,
              "m_cap %d below max_blocks %d", m_cap, max_blocks);
  RKV_TRY(check_extent(params, batch, max3(m_cap, k_cap, slot_cap)));
  RKV_REQUIRE(stage_page0 >= 0 &&
                  stage_page0 + (int64_t)batch * slot_cap <= n_pages &&
                  stage_page0 + (int64_t)batch * slot_cap <= (int64_t)INT32_MAX,
              RKV_ERR_INVALID_ARG,
              "staging pages [%lld, +%lld) do not fit in the %lld-page pool",
              (long long)stage_page0, (long long)batch * slot_cap,
              (long long)n_pages);
  const size_t need = rkv_stage_workspace_size(params, batch, k_cap);
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace),
              RKV_ERR_WORKSPACE, "staging workspace %zu bytes, need %zu",
              workspace_bytes, need);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "workspace is not 16-byte aligned");
  const uint16_t* dev_view[2] = {nullptr, nullptr};
  RKV_TRY(host_views(host_k, host_v, dev_view));
  const size_t lists = (size_t)batch * m.n_kv_heads;
  const size_t pair_bytes = lists * k_cap * 2 * sizeof(int32_t);
  const size_t list_bytes = pair_bytes + lists * sizeof(int32_t);
  RKV_TRY(check_host_list(host_list, host_list_bytes, list_bytes));
  if (lists == 0) return RKV_OK;
  // the planner on the device; its (block, slot) list and counts to the host
  hipError_t e = rkv::launch_stage_plan(m, host_table, block_table, lens, max_blocks,
                                        sel_ids, n_sel, k_cap, batch, slot_cap,
                                        slot_ids, slot_cursor, stage_page0, merged,
                                        n_merged, m_cap, n_staged, workspace, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(host_list, workspace, list_bytes, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return hip_status(e, "rkv_stage_resident_async: planner and its list to the host");
  rkv::StageCopyArgs a;
  a.host_k = host_k;
  a.host_v = host_v;
  a.n_host_pages = n_host_pages;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.n_pages = n_pages;
  a.host_table = host_table_host;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.n_kv = m.n_kv_heads;
  a.stage_page0 = stage_page0;
  a.slots_per_seq = slot_cap;
  a.whole_pages = m.per_sequence;
  a.ids = nullptr;
  a.pairs = static_cast<const int32_t*>(host_list);
  a.counts = reinterpret_cast<const int32_t*>(static_cast<char*>(host_list) + pair_bytes);
  a.row = k_cap;
  a.side = side;
  a.lanes = params->copy_lanes;
  return copy_issue(a, nullptr, done, "rkv_stage_resident_async copies");
}

size_t rkv_attn_workspace_size(const rkv_params* params, int32_t batch,
                               int32_t m_cap) {
  if (!params || params->n_q_heads <= 0 || params->n_kv_heads <= 0 ||
      batch < 0 || m_cap < 1 || params->split_waves < 0)
    return 0;
  const rkv::AttnPlan p = rkv::plan_attention(
      batch, params->n_q_heads, params->n_kv_heads, params->split_waves, m_cap,
      rkv::device_cu_count());
  return p.total_bytes;
}

rkv_status rkv_decode_attn(const rkv_params* params, const uint16_t* q,
                           const uint16_t* k_pages, const uint16_t* v_pages,
                           int64_t n_pages, const int32_t* merged,
                           const int32_t* n_merged, int32_t m_cap,
                           const int32_t* lens, int32_t batch, float* out,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_REQUIRE(batch >= 0, RKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  RKV_REQUIRE(m_cap >= 1 && m_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "m_cap %d outside [1, %d]", m_cap, RKV_MAX_BLOCKS);
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_REQUIRE(q && merged && n_merged && lens && out, RKV_ERR_INVALID_ARG,
              "q, merged, n_merged, lens and out must not be NULL");
  RKV_REQUIRE(aligned16(q) && aligned16(out), RKV_ERR_INVALID_ARG,
              "q and out must be 16-byte aligned");
  const bool use_mfma = params->attn_impl != RKV_ATTN_VALU;
  RKV_REQUIRE(use_mfma || m.group == 1 || m.group == 2 || m.group == 4 ||
                  m.group == 8,
              RKV_ERR_UNSUPPORTED,
              "the VALU attention variant supports groups 1, 2, 4 and 8 (got %d)",
              m.group);
  RKV_TRY(check_extent(params, batch, m_cap));
  const rkv::AttnPlan plan = rkv::plan_attention(
      batch, m.n_q_heads, m.n_kv_heads, params->split_waves, m_cap,
      rkv::device_cu_count());
  const size_t need = plan.total_bytes;
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace != nullptr),
              RKV_ERR_WORKSPACE, "attention workspace %zu bytes, need %zu",
              workspace_bytes, need);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "workspace is not 16-byte aligned");
  return hip_status(
      rkv::launch_decode_attn(m, use_mfma, plan,
                              params->scale, q, k_pages, v_pages, n_pages,
                              merged, n_merged, m_cap, lens, batch, out,
                              workspace, stream),
      "rkv_decode_attn launch");
}

rkv_status rkv_decode_attn_lse(const rkv_params* params, const uint16_t* q,
                               const uint16_t* k_pages, const uint16_t* v_pages,
                               int64_t n_pages, const int32_t* merged,
                               const int32_t* n_merged, int32_t m_cap,
                               const int32_t* lens, int32_t batch,
                               const float* prev_out, const float* prev_lse,
                               float* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_REQUIRE(batch >= 0, RKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  RKV_REQUIRE(m_cap >= 1 && m_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "m_cap %d outside [1, %d]", m_cap, RKV_MAX_BLOCKS);
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_REQUIRE(q && merged && n_merged && lens && out, RKV_ERR_INVALID_ARG,
              "q, merged, n_merged, lens and out must not be NULL");
  RKV_REQUIRE((prev_out == nullptr) == (prev_lse == nullptr), RKV_ERR_INVALID_ARG,
              "prev_out and prev_lse must be given together");
  RKV_REQUIRE(aligned16(q) && aligned16(out) && aligned16(prev_out),
              RKV_ERR_INVALID_ARG, "q, out and prev_out must be 16-byte aligned");
  RKV_REQUIRE(prev_out == nullptr || prev_out != out, RKV_ERR_INVALID_ARG,
              "prev_out must not be out");
  const bool use_mfma = params->attn_impl != RKV_ATTN_VALU;
  RKV_REQUIRE(use_mfma || m.group == 1 || m.group == 2 || m.group == 4 ||
                  m.group == 8,
              RKV_ERR_UNSUPPORTED,
              "the VALU attention variant supports groups 1, 2, 4 and 8 (got %d)",
              m.group);
  RKV_TRY(check_extent(params, batch, m_cap));
  const rkv::AttnPlan plan = rkv::plan_attention(
      batch, m.n_q_heads, m.n_kv_heads, params->split_waves, m_cap,
      rkv::device_cu_count());
  const size_t need = plan.total_bytes;
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace != nullptr),
              RKV_ERR_WORKSPACE, "attention workspace %zu bytes, need %zu",
              workspace_bytes, need);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "workspace is not 16-byte aligned");
  return hip_status(
      rkv::launch_decode_attn(m, use_mfma, plan, params->scale, q, k_pages, v_pages,
                              n_pages, merged, n_merged, m_cap, lens, batch, out,
                              workspace, stream, prev_out, prev_lse, lse),
      "rkv_decode_attn_lse launch");
}

size_t rkv_attn_cascade_workspace_size(const rkv_params* params, int32_t batch,
                                       int32_t m_cap, int32_t shared_blocks) {
  if (!params || params->n_q_heads <= 0 || params->n_kv_heads <= 0 ||
      batch < 0 || m_cap < 1 || params->split_waves < 0 || shared_blocks < 0)
    return 0;
  const rkv::CascadePlan p = rkv::plan_cascade(
      batch, params->n_q_heads, params->n_kv_heads, params->split_waves, m_cap,
      rkv::device_cu_count(), shared_blocks);
  return p.total_bytes;
}

rkv_status rkv_decode_attn_cascade(const rkv_params* params, const uint16_t* q,
                                   const uint16_t* k_pages, const uint16_t* v_pages,
                                   int64_t n_pages, const int32_t* merged,
                                   const int32_t* n_merged, int32_t m_cap,
                                   const int32_t* sel_ids, const int32_t* n_sel,
                                   int32_t k_cap, const int32_t* block_table,
                                   int32_t max_blocks, int32_t shared_blocks,
                                   const int32_t* lens, int32_t batch, float* out,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  rkv::Method m;
  RKV_TRY(check_params(params, &m));
  RKV_REQUIRE(batch >= 0, RKV_ERR_INVALID_ARG, "batch %d < 0", batch);
  RKV_REQUIRE(m_cap >= 1 && m_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "m_cap %d outside [1, %d]", m_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(max_blocks >= 1 && max_blocks <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "max_blocks %d outside [1, %d]", max_blocks, RKV_MAX_BLOCKS);
  RKV_REQUIRE(k_cap >= 1 && k_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "k_cap %d outside [1, %d]", k_cap, RKV_MAX_BLOCKS);
  RKV_REQUIRE(shared_blocks >= 0 && shared_blocks <= max_blocks, RKV_ERR_INVALID_ARG,
              "shared_blocks %d outside [0, max_blocks = %d]", shared_blocks,
              max_blocks);
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_REQUIRE(q && merged && n_merged && sel_ids && n_sel && block_table && lens && out,
              RKV_ERR_INVALID_ARG,
              "q, merged, n_merged, sel_ids, n_sel, block_table, lens and out must "
              "not be NULL");
  RKV_REQUIRE(aligned16(q) && aligned16(out), RKV_ERR_INVALID_ARG,
              "q and out must be 16-byte aligned");
  RKV_REQUIRE(params->attn_impl != RKV_ATTN_VALU, RKV_ERR_UNSUPPORTED,
              "the shared-prefix cascade runs on the MFMA attention only");
  RKV_TRY(check_extent(params, batch, max3(m_cap, k_cap, max_blocks)));
  const rkv::CascadePlan plan = rkv::plan_cascade(
      batch, m.n_q_heads, m.n_kv_heads, params->split_waves, m_cap,
      rkv::device_cu_count(), shared_blocks);
  const size_t need = plan.total_bytes;
  RKV_REQUIRE(workspace_bytes >= need && (need == 0 || workspace != nullptr),
              RKV_ERR_WORKSPACE, "cascade attention workspace %zu bytes, need %zu",
              workspace_bytes, need);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "workspace is not 16-byte aligned");
  return hip_status(
      rkv::launch_decode_attn_cascade(m, plan, params->scale, q, k_pages, v_pages,
                                      n_pages, merged, n_merged, m_cap, sel_ids, n_sel,
                                      k_cap, block_table, max_blocks, lens, batch, out,
                                      workspace, stream),
      "rkv_decode_attn_cascade launch");
}

namespace {

// Checks of rkv_select_attend (also the attention half of rkv_decode_step).
rkv_status select_attend_checks(const rkv_params* params, rkv::Method* m,
                                const uint16_t* q, const uint16_t* k_pages,
                                const uint16_t* v_pages, int64_t n_pages,
                                const int32_t* block_table, int32_t max_blocks,
                                const int32_t* lens, int32_t batch,
                                const int32_t* sel_ids, const int32_t* n_sel,
                                int32_t k_cap, const int32_t* merged,
                                const int32_t* n_merged, int32_t m_cap,
                                const float* out, const void* workspace,
                                size_t workspace_bytes, rkv::AttnPlan* plan) {
  RKV_TRY(check_params(params, m));
  RKV_TRY(check_sizes(batch, max_blocks));
  RKV_REQUIRE(k_cap >= 0, RKV_ERR_INVALID_ARG, "k_cap %d < 0", k_cap);
  RKV_REQUIRE(m_cap >= max_blocks && m_cap <= RKV_MAX_BLOCKS, RKV_ERR_INVALID_ARG,
              "m_cap %d outside [max_blocks %d, %d]", m_cap, max_blocks,
              RKV_MAX_BLOCKS);
  RKV_TRY(check_extent(params, batch, max3(max_blocks, k_cap, m_cap)));
  RKV_TRY(check_pool(k_pages, n_pages, "k_pages"));
  RKV_TRY(check_pool(v_pages, n_pages, "v_pages"));
  RKV_REQUIRE(q && block_table && lens && n_sel && (sel_ids || k_cap == 0) &&
                  merged && n_merged && out,
              RKV_ERR_INVALID_ARG,
              "q, block_table, lens, sel_ids, n_sel, merged, n_merged and out "
              "must not be NULL");
  RKV_REQUIRE(aligned16(q) && aligned16(out), RKV_ERR_INVALID_ARG,
              "q and out must be 16-byte aligned");
  RKV_REQUIRE(k_cap >= topk_cap(params, max_blocks), RKV_ERR_INVALID_ARG,
              "k_cap %d below the required %lld", k_cap,
              (long long)topk_cap(params, max_blocks));
  const bool use_mfma = params->attn_impl != RKV_ATTN_VALU;
  RKV_REQUIRE(use_mfma || m->group == 1 || m->group == 2 || m->group == 4 ||
                  m->group == 8,
              RKV_ERR_UNSUPPORTED,
              "the VALU attention variant supports groups 1, 2, 4 and 8 (got %d)",
              m->group);
  *plan = rkv::plan_attention(batch, m->n_q_heads, m->n_kv_heads,
                              params->split_waves, m_cap, rkv::device_cu_count());
  RKV_REQUIRE(workspace_bytes >= plan->total_bytes &&
                  (plan->total_bytes == 0 || workspace != nullptr),
              RKV_ERR_WORKSPACE, "attention workspace %zu bytes, need %zu",
              workspace_bytes, plan->total_bytes);
  RKV_REQUIRE(aligned16(workspace), RKV_ERR_INVALID_ARG,
              "attention workspace is not 16-byte aligned");
  return RKV_OK;
}

// Top-k + merge from the scores, then attention: one fused launch where
// fused_select_attn_ok holds, else the top-k launch and rkv_decode_attn's.
hipError_t select_attend_launch(const rkv_params* params, const rkv::Method& m,
                                const rkv::AttnPlan& plan, const uint16_t* q,
                                const uint16_t* k_pages, const uint16_t* v_pages,
                                int64_t n_pages, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* lens,
                                const int32_t* prompt_lens, int32_t batch,
                                const uint32_t* scores, int32_t* sel_ids,
                                int32_t* n_sel, int32_t k_cap, int32_t* merged,
                                int32_t* n_merged, int32_t m_cap, float* out,
                                void* workspace, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const bool use_mfma = params->attn_impl != RKV_ATTN_VALU;
  if (rkv::fused_select_attn_ok(m, use_mfma, plan, batch, max_blocks))
    return rkv::launch_select_attn(m, use_mfma, plan, params->scale, q, k_pages,
                                   v_pages, n_pages, block_table, max_blocks, lens,
                                   prompt_lens, scores, sel_ids, n_sel, k_cap,
                                   merged, n_merged, m_cap, out, workspace, stream);
  hipError_t e = rkv::launch_topk(m, block_table, lens, prompt_lens, batch,
                                  max_blocks, scores, sel_ids, n_sel, k_cap,
                                  merged, n_merged, m_cap, stream);
  if (e != hipSuccess) return e;
  return rkv::launch_decode_attn(m, use_mfma, plan, params->scale, q, k_pages,
                                 v_pages, n_pages, merged, n_merged, m_cap, lens,
                                 batch, out, workspace, stream);
}

}  // namespace

rkv_status rkv_select_attend(const rkv_params* params, const uint16_t* q,
                             const uint16_t* k_pages, const uint16_t* v_pages,
                             int64_t n_pages, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* lens,
                             const int32_t* prompt_lens, int32_t batch,
                             const float* scores, int32_t* sel_ids,
                             int32_t* n_sel, int32_t k_cap, int32_t* merged,
                             int32_t* n_merged, int32_t m_cap, float* out,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  rkv::Method m;
  rkv::AttnPlan plan;
  RKV_TRY(select_attend_checks(params, &m, q, k_pages, v_pages, n_pages, block_table,
                               max_blocks, lens, batch, sel_ids, n_sel, k_cap,
                               merged, n_merged, m_cap, out, workspace,
                               workspace_bytes, &plan));
  RKV_REQUIRE(scores != nullptr && (reinterpret_cast<uintptr_t>(scores) & 3u) == 0,
              RKV_ERR_INVALID_ARG, "scores must be a 4-byte aligned, non-NULL pointer");
  return hip_status(
      select_attend_launch(params, m, plan, q, k_pages, v_pages, n_pages, block_table,
                           max_blocks, lens, prompt_lens, batch,
                           reinterpret_cast<const uint32_t*>(scores), sel_ids,
                           n_sel, k_cap, merged, n_merged, m_cap, out, workspace,
                           stream),
      "rkv_select_attend launch");
}

rkv_status rkv_decode_step(const rkv_params* params, const uint16_t* k_new,
                           const uint16_t* v_new, uint16_t* k_pages,
                           uint16_t* v_pages, int64_t n_pages, const uint16_t* q,
                           float* reps, const int32_t* block_table,
                           const int32_t* lens, const int32_t* prompt_lens,
                           int32_t batch, int32_t max_blocks, int32_t* sel_ids,
                           int32_t* n_sel, int32_t k_cap, int32_t* merged,
                           int32_t* n_merged, int32_t m_cap, float* out,
                           void* select_workspace, size_t select_workspace_bytes,
                           void* attn_workspace, size_t attn_workspace_bytes,
                           hipStream_t stream) {
  return rkv::decode_step_impl(params, k_new, v_new, k_pages, v_pages, n_pages, q,
                               reps, block_table, lens, prompt_lens, batch,
                               max_blocks, sel_ids, n_sel, k_cap, merged, n_merged,
                               m_cap, out, select_workspace, select_workspace_bytes,
                               attn_workspace, attn_workspace_bytes, stream);
}

rkv_status rkv_debug_set_report(uint64_t* word) {
  RKV_REQUIRE(word == nullptr || (reinterpret_cast<uintptr_t>(word) & 7u) == 0,
              RKV_ERR_INVALID_ARG, "word must be 8-byte aligned");
  unsigned long long* w = reinterpret_cast<unsigned long long*>(word);
  hipError_t e = rkv::set_bounds_word_attn(w);
  if (e == hipErrorNotSupported) {
    (void)hipGetLastError();
    return fail(RKV_ERR_UNSUPPORTED, "this library was built without RKV_DEBUG");
  }
  if (e == hipSuccess) e = rkv::set_bounds_word_reps(w);
  if (e == hipSuccess) e = rkv::set_bounds_word_select(w);
  if (e == hipSuccess) e = rkv::set_bounds_word_stage(w);
  return hip_status(e, "rkv_debug_set_report");
}

rkv_status rkv_debug_check(uint64_t* word, hipStream_t stream) {
  RKV_REQUIRE(word != nullptr && (reinterpret_cast<uintptr_t>(word) & 7u) == 0,
              RKV_ERR_INVALID_ARG, "word must be a non-NULL, 8-byte aligned pointer");
  hipError_t e = hipStreamSynchronize(stream);
  uint64_t v = 0;
  if (e == hipSuccess) e = hipMemcpy(&v, word, sizeof(v), hipMemcpyDeviceToHost);
  const uint64_t zero = 0;
  if (e == hipSuccess && v != 0)
    e = hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_status(e, "rkv_debug_check");
  if (v == 0) return RKV_OK;
  static const char* const kinds[] = {"?", "length", "page id", "block id", "count",
                                      "host page id"};
  const unsigned kind = (unsigned)(v >> 56);
  return fail(RKV_ERR_BOUNDS, "out-of-range %s %d met by a kernel (clamped or skipped)",
              kinds[kind < 6 ? kind : 0], (int)(int32_t)(uint32_t)v);
}

rkv_status rkv_debug_wave_stamps(uint64_t* dst, int32_t waves) {
  RKV_REQUIRE(waves >= 0 && waves <= RKV_WAVE_STAMP_WAVES, RKV_ERR_INVALID_ARG,
              "waves %d outside [0, %d]", waves, RKV_WAVE_STAMP_WAVES);
  RKV_REQUIRE(dst != nullptr || waves == 0, RKV_ERR_INVALID_ARG, "dst is NULL");
  const hipError_t e = rkv::read_wave_stamps(dst, waves);
  if (e == hipErrorNotSupported)
    return fail(RKV_ERR_UNSUPPORTED, "this library was built without RKV_WAVE_STAMPS");
  return hip_status(e, "rkv_debug_wave_stamps");
}

rkv_status rkv_read_probe(const void* buffer, size_t bytes, uint32_t* sink,
                          hipStream_t stream) {
  RKV_REQUIRE(buffer && sink, RKV_ERR_INVALID_ARG, "buffer and sink must not be NULL");
  RKV_REQUIRE(aligned16(buffer), RKV_ERR_INVALID_ARG, "buffer is not 16-byte aligned");
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e, "rkv_read_probe device query");
  return hip_status(rkv::launch_read_probe(buffer, (int64_t)bytes, sink, n_cu, stream),
                    "rkv_read_probe launch");
}

}  // extern "C"

namespace rkv {

rkv_status report(rkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

rkv_status decode_step_impl(const rkv_params* params, const uint16_t* k_new,
                           const uint16_t* v_new, uint16_t* k_pages,
                           uint16_t* v_pages, int64_t n_pages, const uint16_t* q,
                           float* reps, const int32_t* block_table,
                           const int32_t* lens, const int32_t* prompt_lens,
                           int32_t batch, int32_t max_blocks, int32_t* sel_ids,
                           int32_t* n_sel, int32_t k_cap, int32_t* merged,
                           int32_t* n_merged, int32_t m_cap, float* out,
                           void* select_workspace, size_t select_workspace_bytes,
                           void* attn_workspace, size_t attn_workspace_bytes,
                           hipStream_t stream) {
  rkv::Method m;
  rkv::AttnPlan plan;
  RKV_TRY(select_attend_checks(params, &m, q, k_pages, v_pages, n_pages, block_table,
                               max_blocks, lens, batch, sel_ids, n_sel, k_cap,
                               merged, n_merged, m_cap, out, attn_workspace,
                               attn_workspace_bytes, &plan));
  RKV_REQUIRE(reps != nullptr && aligned16(reps), RKV_ERR_INVALID_ARG,
              "reps must be a 16-byte aligned, non-NULL pointer");
  RKV_REQUIRE(k_new && v_new, RKV_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
  RKV_REQUIRE(aligned16(k_new) && aligned16(v_new), RKV_ERR_INVALID_ARG,
              "k_new and v_new must be 16-byte aligned");
  const size_t need = rkv_select_workspace_size(params, batch, max_blocks);
  RKV_REQUIRE(select_workspace_bytes >= need && (need == 0 || select_workspace),
              RKV_ERR_WORKSPACE, "select workspace %zu bytes, need %zu",
              select_workspace_bytes, need);
  {
    // the two workspaces must not overlap: the attention waves of a list
    // read the scores while other waves write partials
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(select_workspace);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(attn_workspace);
    const bool disjoint = need == 0 || plan.total_bytes == 0 ||
                          s0 + need <= a0 || a0 + plan.total_bytes <= s0;
    RKV_REQUIRE(disjoint, RKV_ERR_INVALID_ARG,
                "the select workspace [%p, +%zu) and the attention workspace "
                "[%p, +%zu) overlap", select_workspace, need, attn_workspace,
                plan.total_bytes);
  }
  uint32_t* scores = static_cast<uint32_t*>(select_workspace);
  const rkv::AppendOp op{k_new, v_new, k_pages, v_pages, n_pages, reps};
  hipError_t e = rkv::launch_score(m, q, reps, block_table, lens, prompt_lens, batch,
                                   max_blocks, scores, &op, stream);
  if (e != hipSuccess) return hip_status(e, "rkv_decode_step launch");
  return hip_status(
      select_attend_launch(params, m, plan, q, k_pages, v_pages, n_pages, block_table,
                           max_blocks, lens, prompt_lens, batch, scores, sel_ids,
                           n_sel, k_cap, merged, n_merged, m_cap, out,
                           attn_workspace, stream),
      "rkv_decode_step launch");
}

int device_cu_count() {
  static std::atomic<int> cache[64];  // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;  // no device visible (host-only use): MI355X's count
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace rkv
