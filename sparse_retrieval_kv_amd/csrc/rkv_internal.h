// Internal interface between the host API (rkv_api.cpp) and the kernel
// files.  Each launcher enqueues its kernel(s) on `stream` and returns the
// launch status; all argument checking happens in rkv_api.cpp before these
// are called.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "rkv.h"

namespace rkv {

constexpr int kBlock = 128;   // tokens per block / page
constexpr int kDim = 128;     // head dimension
constexpr int kPpmOne = 1000000;

// Region and selection parameters as the kernels see them.
struct Method {
  int n_q_heads, n_kv_heads, group;
  int init_tokens, local_tokens, topk_ppm, dense_boundary;
  bool per_sequence;  // one selection per sequence (scores summed over heads)
};

hipError_t launch_build_reps(const uint16_t* k_pages, int64_t n_pages,
                             const int32_t* table, int max_blocks,
                             const int32_t* lens, const int32_t* block_begin,
                             int batch, int n_kv_heads, float* reps,
                             hipStream_t stream);

hipError_t launch_append_kv(const uint16_t* k_new, const uint16_t* v_new,
                            uint16_t* k_pages, uint16_t* v_pages,
                            int64_t n_pages, const int32_t* table,
                            int max_blocks, const int32_t* lens, int batch,
                            int n_kv_heads, float* reps, hipStream_t stream);

// Optional decode-token append carried out by the selection launch.
struct AppendOp {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pages;
  uint16_t* v_pages;
  int64_t n_pages;
  float* reps;  // may be null
};

// Workspace of launch_select: one uint32 order key per (sequence, KV head,
// block).
size_t select_keys_bytes(int batch, int n_kv_heads, int max_blocks);

hipError_t launch_select(const Method& m, const uint16_t* q, const float* reps,
                         const int32_t* table, const int32_t* lens,
                         const int32_t* prompt_lens, int batch, int max_blocks,
                         int32_t* sel_ids, int32_t* n_sel, int k_cap,
                         int32_t* merged, int32_t* n_merged, int m_cap,
                         void* workspace, const AppendOp* append,
                         hipStream_t stream);

// The two launches of launch_select on their own: fp32 inner-product
// scores of the offload blocks (raw bits, [batch][n_kv_heads][max_blocks];
// entries outside a list's offload range are not written), with the
// optional decode-token append; then the top-k and merge from such scores.
hipError_t launch_score(const Method& m, const uint16_t* q, const float* reps,
                        const int32_t* table, const int32_t* lens,
                        const int32_t* prompt_lens, int batch, int max_blocks,
                        uint32_t* scores, const AppendOp* append,
                        hipStream_t stream);
hipError_t launch_topk(const Method& m, const int32_t* table, const int32_t* lens,
                       const int32_t* prompt_lens, int batch, int max_blocks,
                       const uint32_t* scores, int32_t* sel_ids, int32_t* n_sel,
                       int k_cap, int32_t* merged, int32_t* n_merged, int m_cap,
                       hipStream_t stream);

hipError_t launch_merge(const Method& m, const int32_t* table, int max_blocks,
                        const int32_t* lens, const int32_t* sel_ids,
                        const int32_t* n_sel, int k_cap, int batch,
                        const int32_t* host_table, int64_t stage_page0,
                        int32_t* merged, int32_t* n_merged, int m_cap,
                        hipStream_t stream);

hipError_t launch_stage(const uint16_t* host_k, const uint16_t* host_v,
                        int64_t n_host_pages, const int32_t* host_table,
                        int max_blocks, const int32_t* sel_ids,
                        const int32_t* n_sel, int k_cap, int batch, int n_kv,
                        uint16_t* k_pages, uint16_t* v_pages, int64_t n_pages,
                        int64_t stage_page0, hipStream_t stream);

// Prefill-time offload of the offload-region pages into pinned host pools.
hipError_t launch_offload(const Method& m, const uint16_t* k_pages,
                          const uint16_t* v_pages, int64_t n_pages,
                          const int32_t* table, int max_blocks, const int32_t* lens,
                          int batch, const int32_t* host_table, uint16_t* host_k,
                          uint16_t* host_v, int64_t n_host_pages,
                          hipStream_t stream);

// Host tier with residency across steps (slot planner + copy of the blocks
// new to the kept set).  Workspace: copy list + per-list counts.
size_t resident_workspace_bytes(int batch, int n_kv, int k_cap);
hipError_t launch_stage_resident(const Method& m, const uint16_t* host_k,
                                 const uint16_t* host_v, int64_t n_host_pages,
                                 const int32_t* host_table, const int32_t* table,
                                 const int32_t* lens, int max_blocks,
                                 const int32_t* sel_ids, const int32_t* n_sel,
                                 int k_cap, int batch, int slot_cap,
                                 int32_t* slot_ids, int32_t* slot_cursor,
                                 uint16_t* k_pages, uint16_t* v_pages,
                                 int64_t n_pages, int64_t stage_page0,
                                 int32_t* merged, int32_t* n_merged, int m_cap,
                                 int32_t* n_staged, void* workspace,
                                 hipStream_t stream);

// The residency planner alone (the first launch of launch_stage_resident):
// slot state, merged table and the (block, slot) copy list in the workspace
// ([batch * n_kv][k_cap] int32 pairs, then [batch * n_kv] counts).
hipError_t launch_stage_plan(const Method& m, const int32_t* host_table,
                             const int32_t* table, const int32_t* lens,
                             int max_blocks, const int32_t* sel_ids,
                             const int32_t* n_sel, int k_cap, int batch,
                             int slot_cap, int32_t* slot_ids, int32_t* slot_cursor,
                             int64_t stage_page0, int32_t* merged,
                             int32_t* n_merged, int m_cap, int32_t* n_staged,
                             void* workspace, hipStream_t stream,
                             int32_t* merged_new = nullptr, int32_t* n_new = nullptr);
// The copy launch of launch_stage_resident alone, over the copy list a
// launch_stage_plan left in `workspace`.
hipError_t launch_stage_copy(const Method& m, const uint16_t* host_k,
                             const uint16_t* host_v, int64_t n_host_pages,
                             const int32_t* host_table, int max_blocks, int k_cap,
                             int batch, int slot_cap, uint16_t* k_pages,
                             uint16_t* v_pages, int64_t n_pages, int64_t stage_page0,
                             const void* workspace, hipStream_t stream);

// Copy-engine staging from a host copy of a list: kept ids (pairs null; the
// r-th kept block goes to slot r) or (block, slot) pairs, rows of `row`
// entries per (sequence, KV head), with counts.  Slot s of sequence b is page
// stage_page0 + b * slots_per_seq + s.  Issues the copies on `side` and
// returns the number of (page, head) tiles copied.
struct StageCopyArgs {
  const uint16_t* host_k;
  const uint16_t* host_v;
  int64_t n_host_pages;
  uint16_t* k_pages;
  uint16_t* v_pages;
  int64_t n_pages;
  const int32_t* host_table;  // HOST [batch][max_blocks]
  int max_blocks, batch, n_kv;
  int64_t stage_page0;
  int slots_per_seq;
  bool whole_pages;  // copy whole pages when all heads of a sequence agree
  const int32_t* ids;     // [lists][row] kept ids, or null
  const int32_t* pairs;   // [lists][row][2] (block, slot), or null
  const int32_t* counts;  // [lists]
  int row;
  hipStream_t side;
  int lanes;  // >= 2: copies spread over that many streams of the library
  int count(int bh) const {
    const int n = counts[bh];
    return n < 0 ? 0 : (n > row ? row : n);
  }
  int block(int bh, int i) const {
    return pairs ? pairs[2 * ((int64_t)bh * row + i)] : ids[(int64_t)bh * row + i];
  }
  int slot(int bh, int i) const {
    return pairs ? pairs[2 * ((int64_t)bh * row + i) + 1] : i;
  }
};
hipError_t issue_stage_copies(const StageCopyArgs& a, int64_t* tiles_copied);

// Split-K decode attention over a fixed number of waves: the 64-token units
// of all merged lists are spread evenly over `n_waves` waves; the workspace
// holds one partial per (wave, list) piece: n_waves + lists slots of
// `group` heads for the range split, lists * per_list for the
// single-sequence partition.
struct AttnPlan {
  int n_waves;
  int n_slots;           // partial slots
  int comb_spec;         // combine pieces per lane requested speculatively
  int n_cu;              // compute units of the device
  int per_list;          // > 0: single-sequence partition, waves per list
  size_t partial_bytes;  // fp32 [n_slots][group][kDim]
  size_t ml_bytes;       // float2 [n_slots][group]
  size_t count_bytes;    // int [lists] piece counts, int [lists] first slots (padded)
  size_t total_bytes;
};
AttnPlan plan_attention(int batch, int n_q_heads, int n_kv_heads, int waves,
                        int m_cap, int n_cu);

// Compute units of the current device (queried once per device).
int device_cu_count();

hipError_t launch_decode_attn(const Method& m, bool use_mfma,
                              const AttnPlan& plan, float scale,
                              const uint16_t* q, const uint16_t* k_pages,
                              const uint16_t* v_pages, int64_t n_pages,
                              const int32_t* merged, const int32_t* n_merged,
                              int m_cap, const int32_t* lens, int batch,
                              float* out, void* workspace, hipStream_t stream,
                              const float* prev_out = nullptr,
                              const float* prev_lse = nullptr, float* lse_out = nullptr);

// Top-k + merge folded into the attention launch, for the shapes
// fused_select_attn_ok accepts (a batch of one, MFMA, per-head selection,
// max_blocks <= kFusedMaxBlocks): every wave of a list finds the list's
// selection from the scores itself (the list's first wave also writes
// sel_ids / n_sel / merged / n_merged), then attends exactly as
// launch_decode_attn's single-sequence partition does; then the combine.
constexpr int kFusedMaxBlocks = 1024;
// Per-wave timestamps of the folded-selection launch (built with
// RKV_WAVE_STAMPS): kWaveStampSlots 64-bit values for each of the launch's
// first kWaveStampWaves waves; read_wave_stamps copies the first `waves`
// rows to host memory (hipErrorNotSupported in other builds).
constexpr int kWaveStampWaves = RKV_WAVE_STAMP_WAVES;
constexpr int kWaveStampSlots = RKV_WAVE_STAMP_SLOTS;
hipError_t read_wave_stamps(uint64_t* dst, int waves);
bool fused_select_attn_ok(const Method& m, bool use_mfma, const AttnPlan& plan,
                          int batch, int max_blocks);
hipError_t launch_select_attn(const Method& m, bool use_mfma, const AttnPlan& plan,
                              float scale,
                              const uint16_t* q, const uint16_t* k_pages,
                              const uint16_t* v_pages, int64_t n_pages,
                              const int32_t* table, int max_blocks,
                              const int32_t* lens, const int32_t* prompt_lens,
                              const uint32_t* scores, int32_t* sel_ids,
                              int32_t* n_sel, int k_cap, int32_t* merged,
                              int32_t* n_merged, int m_cap, float* out,
                              void* workspace, hipStream_t stream);

// Shared-prefix cascade decode: the range split over each list's private
// entries plus cascade waves over the shared prefix, after a preparation
// launch (shared-block masks and private merged tables), then the combine.
// Workspace: the range split's (with c_waves * c_q more slots), then the
// masks, the private merged tables and their counts.
struct CascadePlan {
  AttnPlan attn;         // n_slots includes the cascade slots
  int q, groups, chunks, chunk_blocks, waves, words, shared;
  int64_t slot0;         // first cascade slot
  size_t mask_off, priv_off, npriv_off;  // byte offsets in the workspace
  size_t total_bytes;
};
CascadePlan plan_cascade(int batch, int n_q_heads, int n_kv_heads, int waves,
                         int m_cap, int n_cu, int shared_blocks);
hipError_t launch_decode_attn_cascade(const Method& m, const CascadePlan& plan,
                                      float scale, const uint16_t* q,
                                      const uint16_t* k_pages, const uint16_t* v_pages,
                                      int64_t n_pages, const int32_t* merged,
                                      const int32_t* n_merged, int m_cap,
                                      const int32_t* sel_ids, const int32_t* n_sel,
                                      int k_cap, const int32_t* table, int max_blocks,
                                      const int32_t* lens, int batch, float* out,
                                      void* workspace, hipStream_t stream);

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                             int n_cu, hipStream_t stream);

// Debug builds: point each kernel file's bounds-report word at `word` (null:
// off) for the current device.  Other builds: hipErrorNotSupported.
hipError_t set_bounds_word_attn(unsigned long long* word);
hipError_t set_bounds_word_reps(unsigned long long* word);
hipError_t set_bounds_word_select(unsigned long long* word);
hipError_t set_bounds_word_stage(unsigned long long* word);

// Sets the calling thread's error text (rkv_last_error) and returns s.
rkv_status report(rkv_status s, const char* fmt, ...);

// Body of rkv_decode_step (validation, then the launches) with the two
// workspaces as given; also behind the entry point that takes them from the
// library's static scratch.
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
                            hipStream_t stream);

}  // namespace rkv
