// Internal interface between the C-ABI host code (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "iq_device.h"

namespace iq {

struct CacheView {
  uint8_t* k_codes;
  uint16_t* k_norms;
  uint8_t* v_codes;
  uint16_t* v_norms;
  int32_t num_pages;
  int32_t hkv;
  int32_t bits;  // 3 or 4: record width
};

// The 4-bit quantiser (codebook.hip), computed once per process.
struct Codebook4 {
  double level[16];       // ascending Lloyd-Max levels of N(0, 1)
  float thr[15];          // fp32 decision thresholds (midpoints; thr[7] = 0)
  float alpha;            // scale of the f16 level operands
  double alpha_rel_err;   // worst relative error of the eight f16 magnitudes
  uint16_t level_f16[8];  // f16 bits of alpha * level[8 + k]
  Levels4 lv;             // the kernels' form
};
const Codebook4& codebook4();

// Rotation buffer: fp32 matrices [hkv][32][4][4], then fp32 quaternion staging
// [hkv][32][2][4].
inline size_t rotation_matrix_bytes(int hkv) { return (size_t)hkv * 32 * 16 * sizeof(float); }
inline size_t rotation_total_bytes(int hkv) {
  return rotation_matrix_bytes(hkv) + (size_t)hkv * 32 * 8 * sizeof(float);
}

hipError_t launch_rotation_init(const float* quats_dev, int hkv, float* rot_dev,
                                hipStream_t stream);

hipError_t launch_quantize_append(const CacheView& c, const float* rot, const void* k,
                                  const void* v, int dtype, int n_tokens, const int32_t* seq_idx,
                                  const int32_t* pos, const int32_t* block_table, int max_pages,
                                  hipStream_t stream);

// Caller choices for one decode call (iq_decode_options in the C ABI); zero
// fields leave the choice to the planner.
struct DecodeOptions {
  int waves;            // 0, 4 or 8 waves per workgroup
  int pages_per_split;  // 0 or pages per split of the host plan
  int rounds;           // 0 or workgroups per CU the plan is made for
  int plan;             // 0 auto, 1 host plan, 2 device-balanced plan
  int merge;            // 0 auto (a merge kernel), 1 merge workgroups in the split launch, 2 a merge kernel
  int deterministic;    // nonzero: each wave takes a fixed share of its split's pages
};

struct DecodePlan {
  int splits;           // workgroups per (sequence, kv head); balanced: slots per workspace row
  int pages_per_split;
  int waves;            // waves per workgroup: 4 (one short pass) or 8 (long streams)
  int balanced;         // several sequences: the split plan is made on the device
  int grid_x;           // balanced: workgroups launched (the plan's plus spare ones)
  int plan_wgs;         // balanced: workgroups the pages are spread over
  int merge;            // as DecodeOptions::merge (0: decided at launch)
  int deterministic;
  int cus;              // compute units planned for
};
DecodePlan plan_decode(int batch, int hkv, int max_seq_len, int num_cus, const DecodeOptions& o);
size_t decode_workspace_bytes(int batch, int hq, const DecodePlan& plan);
// Whether a call with this plan merges in the split launch (else a merge kernel follows).
bool decode_fused_merge(const DecodePlan& plan, int batch, int hkv, int hq, int bits, bool append);

// Decode workspace: arrival counters first (a fixed region, so that any later
// call finds them where the last one left them: zero), then the split
// partials.  The counters must be zero before a buffer's first use; every
// call leaves them zero.
constexpr size_t kWsCounterBytes = 16384;
constexpr int kMaxCounterUnits = (int)(kWsCounterBytes / 8);  // (sequence, kv head) pairs

// k_new / v_new non-null: a decode step, which first appends each sequence's
// token at position seq_lens[b] - 1 (rows [B][Hkv][128] of kv_dtype).
hipError_t launch_decode(const CacheView& c, const float* rot, const void* q, int q_dtype,
                         int batch, int hq, const int32_t* block_table, int max_pages,
                         const int32_t* seq_lens, const DecodePlan& plan, float softmax_scale,
                         float* out, void* workspace, const void* k_new, const void* v_new,
                         int kv_dtype, hipStream_t stream);

// Merge of the split partials ([B][Hq][splits] rows of m, l and acc[128]):
// normalise and, with `rotate`, apply T^T (rot = the rotation buffer).
// n_splits (nullable, device int[B]): the slots sequence b used.
hipError_t launch_decode_merge(bool rotate, const float* rot, const float* ws_acc, const float* ws_ml,
                               int splits, int batch, int hq, int group, const int32_t* n_splits,
                               float* out, hipStream_t stream);

// Uncompressed baseline (dense.hip): paged cache of bf16 (format 0) or FP8
// E4M3 (format 1) values, K token-major [pages][hkv][64][128], V
// coordinate-major [pages][hkv][128][64]; FP8 values are x / scale.
struct DenseCacheView {
  uint8_t* k;
  uint8_t* v;
  int32_t num_pages;
  int32_t hkv;
  int32_t format;
  float k_scale, v_scale;  // FP8 only; positive
};
hipError_t launch_dense_append(const DenseCacheView& c, const void* k, const void* v, int dtype,
                               int n_tokens, const int32_t* seq_idx, const int32_t* pos,
                               const int32_t* block_table, int max_pages, hipStream_t stream);
DecodePlan plan_dense_decode(int batch, int hkv, int max_seq_len, int num_cus);
hipError_t launch_dense_decode(const DenseCacheView& c, const void* q, int batch, int hq,
                               const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                               const DecodePlan& plan, float softmax_scale, float* out,
                               void* workspace, hipStream_t stream);
// Chunked causal prefill of one sequence over the uncompressed cache (q bf16
// [n_q][hq][128], query i at position q_start + i); no workspace.
hipError_t launch_dense_prefill(const DenseCacheView& c, const void* q, int n_q, int hq, int q_start,
                                const int32_t* block_table, int max_pages, float softmax_scale, float* out,
                                hipStream_t stream);
// Streaming read of `bytes` (a multiple of 16) at `buf`; one word per thread
// of the fixed grid goes to `sink`.
constexpr int kProbeBlocks = 2048, kProbeThreads = 256;
hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// Longest causal key range of one prefill call, in pages (the page ids of the
// range are staged in LDS): 4096 pages = 262,144 tokens.
constexpr int kPrefillMaxPages = 4096;

struct PrefillPlan {
  int row_tiles;        // workgroups per kv head along the query rows
  int kv_splits;        // workgroups along the key range
  int waves;            // 8: eight waves of 16 rows; 4: four waves of 32 rows
};
PrefillPlan plan_prefill(int n_q, int hq, int hkv, int q_start, int num_cus);
size_t prefill_workspace_bytes(int n_q, int hq, const PrefillPlan& plan);
hipError_t launch_prefill(const CacheView& c, const float* rot, const void* q, int q_dtype,
                          int n_q, int hq, int q_start, const int32_t* block_table,
                          int max_pages, const PrefillPlan& plan, float softmax_scale,
                          float* out, void* workspace, hipStream_t stream);
// Several sequences in one launch: sequence b's queries are rows cu_q[b] ..
// cu_q[b+1]-1 (device), its first at position q_starts[b] (device), its
// block-table row block_table + b * max_pages; plan.row_tiles covers the
// longest query count.
// A chunk quantise-appended by the prefill launch itself: tokens new_start ..
// new_start + n_new - 1 of the (one) sequence, rows [n_new][hkv][128] of
// dtype; counters = the workspace's counter region (zero at rest).
struct PrefillAppend {
  const void* k;
  const void* v;
  int dtype, n_new, new_start;
  uint32_t* counters;
};
// Whether the whole prefill grid can be resident at once (the fused append's
// waits need it).
bool prefill_append_fused(const PrefillPlan& plan, int hkv, int bits, int num_cus);
hipError_t launch_prefill_args(const CacheView& c, const float* rot, const void* q, int q_dtype,
                               int batch, int n_q, int hq, const int32_t* cu_q, int q_start,
                               const int32_t* q_starts, const int32_t* block_table, int max_pages,
                               const PrefillPlan& plan, float softmax_scale, float* out,
                               const PrefillAppend* app, hipStream_t stream);
// Quantise-append of tokens pos0 .. pos0 + n_tokens - 1 of one sequence
// (block-table row block_table); the same records as launch_quantize_append.
hipError_t launch_quantize_append_range(const CacheView& c, const float* rot, const void* k,
                                        const void* v, int dtype, int n_tokens, int pos0,
                                        const int32_t* block_table, int max_pages, hipStream_t stream);
hipError_t launch_prefill_varlen(const CacheView& c, const float* rot, const void* q, int q_dtype,
                                 int batch, int n_q, int hq, const int32_t* cu_q, int q_start,
                                 const int32_t* q_starts, const int32_t* block_table, int max_pages,
                                 const PrefillPlan& plan, float softmax_scale, float* out,
                                 void* workspace, hipStream_t stream);

}  // namespace iq
