// C ABI of libisoquant: argument validation, split planning and launches.
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so argument errors are reported (and testable) without a GPU;
// nothing is enqueued when a check fails.  No entry point synchronises the
// host (FreeToken v0.2.0 release notes, Kernels #726).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "../../include/isoquant.h"
#include "iq_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The no-allocation decode step's scratch: one array per GPU the library runs
// on.  Host code never uses the array's name as an address (on the host it is
// a stand-in, not device memory): it uses the address hipGetSymbolAddress
// returns for the current device, kept per device.
static __device__ __align__(256) uint8_t scratch[IQ_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);  // the same address whoever stores it
  return q;
}

bool cache_ok(const iq_cache* c) {
  return c && c->k_codes_dev && c->k_norms_dev && c->v_codes_dev && c->v_norms_dev &&
         c->num_pages > 0 && c->n_kv_heads > 0 && (c->bits == 0 || c->bits == 3 || c->bits == 4);
}

iq::CacheView view(const iq_cache* c) {
  return iq::CacheView{c->k_codes_dev, c->k_norms_dev, c->v_codes_dev, c->v_norms_dev,
                       c->num_pages, c->n_kv_heads, c->bits == 4 ? 4 : 3};
}

bool scale_ok(float s) { return isfinite(s) && s >= 0.f; }

bool dense_ok(const iq_dense_cache* c) {
  return c && c->k_dev && c->v_dev && c->num_pages > 0 && c->n_kv_heads > 0 && c->n_kv_heads <= 65535 &&
         (c->format == IQ_KV_BF16 ||
          (c->format == IQ_KV_FP8_E4M3 && scale_ok(c->k_scale) && scale_ok(c->v_scale)));
}

iq::DenseCacheView dense_view(const iq_dense_cache* c) {
  const bool fp8 = c->format == IQ_KV_FP8_E4M3;
  return iq::DenseCacheView{static_cast<uint8_t*>(c->k_dev), static_cast<uint8_t*>(c->v_dev), c->num_pages,
                            c->n_kv_heads, c->format,
                            fp8 && c->k_scale > 0.f ? c->k_scale : 1.0f,
                            fp8 && c->v_scale > 0.f ? c->v_scale : 1.0f};
}

bool dtype_ok(int32_t d) { return d == IQ_F32 || d == IQ_BF16 || d == IQ_F16; }

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

iq_status launch_status(hipError_t e) { return e == hipSuccess ? IQ_OK : IQ_ERR_LAUNCH; }

float resolve_scale(float s) { return (s > 0.f && isfinite(s)) ? s : 1.0f / sqrtf(128.0f); }

// Decode options -> the planner's form; false for a field outside its values.
bool decode_options(const iq_decode_options* o, iq::DecodeOptions* out) {
  *out = iq::DecodeOptions{};
  if (!o) return true;
  if ((o->waves != 0 && o->waves != 4 && o->waves != 8) || o->pages_per_split < 0 || o->rounds < 0 ||
      o->rounds > 64 || o->plan < IQ_PLAN_AUTO || o->plan > IQ_PLAN_BALANCED || o->merge < IQ_MERGE_AUTO ||
      o->merge > IQ_MERGE_KERNEL)
    return false;
  out->waves = o->waves;
  out->pages_per_split = o->pages_per_split;
  out->rounds = o->rounds;
  out->plan = o->plan == IQ_PLAN_HOST ? 1 : 0;
  out->merge = o->merge == IQ_MERGE_FUSED ? 1 : o->merge == IQ_MERGE_KERNEL ? 2 : 0;
  out->deterministic = o->deterministic != 0;
  return true;
}

static_assert(IQ_DECODE_COUNTER_BYTES == iq::kWsCounterBytes, "counter region size");

// Shared by iq_decode_attention(_ex) and iq_decode_step(_ex): k_new null for attention alone.
iq_status decode_call(const iq_cache* cache, const void* rot_dev, const void* q_dev, int32_t q_dtype,
                      int32_t batch, int32_t n_q_heads, const void* k_new_dev, const void* v_new_dev,
                      int32_t kv_dtype, const int32_t* block_table_dev, int32_t max_pages_per_seq,
                      const int32_t* seq_lens_dev, int32_t max_seq_len, float softmax_scale, float* out_dev,
                      void* workspace_dev, size_t workspace_bytes, const iq_decode_options* options,
                      hipStream_t stream) {
  if (!cache_ok(cache) || !rot_dev || !q_dev || !dtype_ok(q_dtype) || batch < 1 || batch > 65535 ||
      n_q_heads < 1 || !block_table_dev || max_pages_per_seq < 1 || !seq_lens_dev || max_seq_len < 0 ||
      !out_dev || !workspace_dev)
    return IQ_ERR_INVALID_ARG;
  if (k_new_dev && (!v_new_dev || !dtype_ok(kv_dtype))) return IQ_ERR_INVALID_ARG;
  iq::DecodeOptions opts;
  if (!decode_options(options, &opts)) return IQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)max_pages_per_seq * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  if (cache->n_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;
  if (n_q_heads / cache->n_kv_heads > IQ_MAX_GROUP) return IQ_ERR_UNSUPPORTED;
  const iq::DecodePlan plan = iq::plan_decode(batch, cache->n_kv_heads, max_seq_len, device_cu_count(), opts);
  if (workspace_bytes < iq::decode_workspace_bytes(batch, n_q_heads, plan)) return IQ_ERR_WORKSPACE;
  return launch_status(iq::launch_decode(view(cache), reinterpret_cast<const float*>(rot_dev), q_dev,
                                         q_dtype, batch, n_q_heads, block_table_dev, max_pages_per_seq,
                                         seq_lens_dev, plan, resolve_scale(softmax_scale), out_dev,
                                         workspace_dev, k_new_dev, v_new_dev, kv_dtype, stream));
}

}  // namespace

extern "C" {

const char* iq_status_string(int32_t status) {
  switch (status) {
    case IQ_OK: return "ok";
    case IQ_ERR_INVALID_ARG: return "invalid argument";
    case IQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case IQ_ERR_WORKSPACE: return "workspace too small";
    case IQ_ERR_LAUNCH: return "HIP copy or kernel launch failed";
    case IQ_ERR_DEVICE: return "no usable HIP device";
    case IQ_ERR_SCRATCH: return "call needs more scratch than the library's static array holds";
    default: return "unknown status";
  }
}

int32_t iq_version(void) { return 10000; }

iq_status iq_codebook(int32_t bits, double* levels_host, float* thresholds_host, float* level_scale) {
  if ((bits != 3 && bits != 4) || !levels_host || !thresholds_host) return IQ_ERR_INVALID_ARG;
  if (bits == 3) {
    for (int k = 0; k < 4; ++k) {
      levels_host[4 + k] = iq::kLevel3[k];
      levels_host[3 - k] = -iq::kLevel3[k];
    }
    for (int k = 0; k < 3; ++k) {
      thresholds_host[4 + k] = iq::kThr3[k];
      thresholds_host[2 - k] = -iq::kThr3[k];
    }
    thresholds_host[3] = 0.0f;
    if (level_scale) *level_scale = iq::kLevelScale;
    return IQ_OK;
  }
  const iq::Codebook4& cb = iq::codebook4();
  for (int k = 0; k < 16; ++k) levels_host[k] = cb.level[k];
  for (int k = 0; k < 15; ++k) thresholds_host[k] = cb.thr[k];
  if (level_scale) *level_scale = cb.alpha;
  return IQ_OK;
}

size_t iq_rotation_bytes(int32_t n_kv_heads) {
  return n_kv_heads > 0 ? iq::rotation_total_bytes(n_kv_heads) : 0;
}

iq_status iq_rotation_init(const float* quats_host, int32_t n_kv_heads, void* rot_dev,
                           size_t rot_bytes, hipStream_t stream) {
  if (!quats_host || !rot_dev || n_kv_heads < 1 || n_kv_heads > 65535) return IQ_ERR_INVALID_ARG;
  if (rot_bytes < iq::rotation_total_bytes(n_kv_heads)) return IQ_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n_kv_heads * 32 * 2; ++i) {
    double n = 0;
    for (int k = 0; k < 4; ++k) {
      const double v = quats_host[4 * i + k];
      if (!isfinite(v)) return IQ_ERR_INVALID_ARG;
      n += v * v;
    }
    if (!(n > 0) || !isfinite(n)) return IQ_ERR_INVALID_ARG;
  }
  float* mats = reinterpret_cast<float*>(rot_dev);
  float* staging = reinterpret_cast<float*>(reinterpret_cast<char*>(rot_dev) +
                                            iq::rotation_matrix_bytes(n_kv_heads));
  const size_t qbytes = (size_t)n_kv_heads * 32 * 8 * sizeof(float);
  if (hipMemcpyAsync(staging, quats_host, qbytes, hipMemcpyHostToDevice, stream) != hipSuccess)
    return IQ_ERR_LAUNCH;
  return launch_status(iq::launch_rotation_init(staging, n_kv_heads, mats, stream));
}

iq_status iq_quantize_append(const iq_cache* cache, const void* rot_dev, const void* k_dev,
                             const void* v_dev, int32_t dtype, int32_t n_tokens,
                             const int32_t* seq_idx_dev, const int32_t* pos_dev,
                             const int32_t* block_table_dev, int32_t max_pages_per_seq,
                             hipStream_t stream) {
  if (!cache_ok(cache) || !rot_dev || !dtype_ok(dtype) || n_tokens < 0 || max_pages_per_seq < 1)
    return IQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return IQ_OK;
  if (!k_dev || !v_dev || !seq_idx_dev || !pos_dev || !block_table_dev) return IQ_ERR_INVALID_ARG;
  return launch_status(iq::launch_quantize_append(view(cache), reinterpret_cast<const float*>(rot_dev),
                                                  k_dev, v_dev, dtype, n_tokens, seq_idx_dev, pos_dev,
                                                  block_table_dev, max_pages_per_seq, stream));
}

size_t iq_decode_workspace_bytes_ex(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t max_seq_len, const iq_decode_options* options) {
  iq::DecodeOptions opts;
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || max_seq_len < 0 || !decode_options(options, &opts))
    return 0;
  const iq::DecodePlan plan = iq::plan_decode(batch, n_kv_heads, max_seq_len, device_cu_count(), opts);
  return iq::decode_workspace_bytes(batch, n_q_heads, plan);
}

iq_status iq_decode_describe(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t max_seq_len,
                             int32_t bits, int32_t step, const iq_decode_options* options,
                             iq_decode_plan_info* info) {
  iq::DecodeOptions opts;
  if (!info || batch < 1 || batch > 65535 || n_q_heads < 1 || n_kv_heads < 1 || n_kv_heads > 65535 ||
      max_seq_len < 0 || (bits != 0 && bits != 3 && bits != 4) || n_q_heads % n_kv_heads != 0 ||
      !decode_options(options, &opts))
    return IQ_ERR_INVALID_ARG;
  if (n_q_heads / n_kv_heads > IQ_MAX_GROUP) return IQ_ERR_UNSUPPORTED;
  const iq::DecodePlan plan = iq::plan_decode(batch, n_kv_heads, max_seq_len, device_cu_count(), opts);
  const bool fused = iq::decode_fused_merge(plan, batch, n_kv_heads, n_q_heads, bits == 4 ? 4 : 3, step != 0);
  info->waves = plan.waves;
  info->splits = plan.splits;
  info->pages_per_split = plan.pages_per_split;
  info->balanced = plan.balanced;
  info->fused_merge = fused ? 1 : 0;
  info->workgroups = plan.balanced ? plan.grid_x
                                   : plan.splits * n_kv_heads * batch + (fused ? batch * n_q_heads : 0);
  return IQ_OK;
}

size_t iq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t max_seq_len) {
  return iq_decode_workspace_bytes_ex(batch, n_q_heads, n_kv_heads, max_seq_len, nullptr);
}

iq_status iq_decode_attention(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                              int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                              const int32_t* block_table_dev, int32_t max_pages_per_seq,
                              const int32_t* seq_lens_dev, int32_t max_seq_len, float softmax_scale,
                              float* out_dev, void* workspace_dev, size_t workspace_bytes,
                              hipStream_t stream) {
  return decode_call(cache, rot_dev, q_dev, q_dtype, batch, n_q_heads, nullptr, nullptr, 0, block_table_dev,
                     max_pages_per_seq, seq_lens_dev, max_seq_len, softmax_scale, out_dev, workspace_dev,
                     workspace_bytes, nullptr, stream);
}

iq_status iq_decode_attention_ex(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                                 int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                 const int32_t* block_table_dev, int32_t max_pages_per_seq,
                                 const int32_t* seq_lens_dev, int32_t max_seq_len, float softmax_scale,
                                 float* out_dev, void* workspace_dev, size_t workspace_bytes,
                                 const iq_decode_options* options, hipStream_t stream) {
  return decode_call(cache, rot_dev, q_dev, q_dtype, batch, n_q_heads, nullptr, nullptr, 0, block_table_dev,
                     max_pages_per_seq, seq_lens_dev, max_seq_len, softmax_scale, out_dev, workspace_dev,
                     workspace_bytes, options, stream);
}

iq_status iq_decode_step(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                         int32_t q_dtype, int32_t batch, int32_t n_q_heads, const void* k_new_dev,
                         const void* v_new_dev, int32_t kv_dtype, const int32_t* block_table_dev,
                         int32_t max_pages_per_seq, const int32_t* seq_lens_dev, int32_t max_seq_len,
                         float softmax_scale, float* out_dev, void* workspace_dev,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!k_new_dev) return IQ_ERR_INVALID_ARG;
  return decode_call(cache, rot_dev, q_dev, q_dtype, batch, n_q_heads, k_new_dev, v_new_dev, kv_dtype,
                     block_table_dev, max_pages_per_seq, seq_lens_dev, max_seq_len, softmax_scale, out_dev,
                     workspace_dev, workspace_bytes, nullptr, stream);
}

iq_status iq_decode_step_noalloc(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                                 int32_t q_dtype, int32_t batch, int32_t n_q_heads, const void* k_new_dev,
                                 const void* v_new_dev, int32_t kv_dtype, const int32_t* block_table_dev,
                                 int32_t max_pages_per_seq, const int32_t* seq_lens_dev, int32_t max_seq_len,
                                 float softmax_scale, float* out_dev, hipStream_t stream) {
  if (!cache_ok(cache) || !rot_dev || !q_dev || !dtype_ok(q_dtype) || !k_new_dev || !v_new_dev ||
      !dtype_ok(kv_dtype) || batch < 1 || batch > 65535 || n_q_heads < 1 || !block_table_dev ||
      max_pages_per_seq < 1 || !seq_lens_dev || max_seq_len < 0 || !out_dev)
    return IQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)max_pages_per_seq * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  if (cache->n_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;
  if (n_q_heads / cache->n_kv_heads > IQ_MAX_GROUP) return IQ_ERR_UNSUPPORTED;
  iq::DecodeOptions opts{};
  opts.merge = 2;  // the merge kernel: no counter in the array has to start at zero
  const iq::DecodePlan plan = iq::plan_decode(batch, cache->n_kv_heads, max_seq_len, device_cu_count(), opts);
  if (iq::decode_workspace_bytes(batch, n_q_heads, plan) > (size_t)IQ_NOALLOC_SCRATCH_BYTES)
    return IQ_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return IQ_ERR_DEVICE;
  return launch_status(iq::launch_decode(view(cache), reinterpret_cast<const float*>(rot_dev), q_dev,
                                         q_dtype, batch, n_q_heads, block_table_dev, max_pages_per_seq,
                                         seq_lens_dev, plan, resolve_scale(softmax_scale), out_dev, ws,
                                         k_new_dev, v_new_dev, kv_dtype, stream));
}

iq_status iq_decode_step_ex(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                            int32_t q_dtype, int32_t batch, int32_t n_q_heads, const void* k_new_dev,
                            const void* v_new_dev, int32_t kv_dtype, const int32_t* block_table_dev,
                            int32_t max_pages_per_seq, const int32_t* seq_lens_dev, int32_t max_seq_len,
                            float softmax_scale, float* out_dev, void* workspace_dev,
                            size_t workspace_bytes, const iq_decode_options* options, hipStream_t stream) {
  if (!k_new_dev) return IQ_ERR_INVALID_ARG;
  return decode_call(cache, rot_dev, q_dev, q_dtype, batch, n_q_heads, k_new_dev, v_new_dev, kv_dtype,
                     block_table_dev, max_pages_per_seq, seq_lens_dev, max_seq_len, softmax_scale, out_dev,
                     workspace_dev, workspace_bytes, options, stream);
}

iq_status iq_dense_append(const iq_dense_cache* cache, const void* k_dev, const void* v_dev,
                          int32_t dtype, int32_t n_tokens, const int32_t* seq_idx_dev,
                          const int32_t* pos_dev, const int32_t* block_table_dev,
                          int32_t max_pages_per_seq, hipStream_t stream) {
  if (!dense_ok(cache) || !dtype_ok(dtype) || n_tokens < 0 || max_pages_per_seq < 1)
    return IQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return IQ_OK;
  if (!k_dev || !v_dev || !seq_idx_dev || !pos_dev || !block_table_dev) return IQ_ERR_INVALID_ARG;
  return launch_status(iq::launch_dense_append(dense_view(cache), k_dev, v_dev, dtype, n_tokens,
                                               seq_idx_dev, pos_dev, block_table_dev,
                                               max_pages_per_seq, stream));
}

size_t iq_dense_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t max_seq_len) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || max_seq_len < 0) return 0;
  const iq::DecodePlan plan = iq::plan_dense_decode(batch, n_kv_heads, max_seq_len, device_cu_count());
  return iq::decode_workspace_bytes(batch, n_q_heads, plan);
}

iq_status iq_dense_decode_attention(const iq_dense_cache* cache, const void* q_dev, int32_t q_dtype,
                                    int32_t batch, int32_t n_q_heads, const int32_t* block_table_dev,
                                    int32_t max_pages_per_seq, const int32_t* seq_lens_dev,
                                    int32_t max_seq_len, float softmax_scale, float* out_dev,
                                    void* workspace_dev, size_t workspace_bytes, hipStream_t stream) {
  if (!dense_ok(cache) || !q_dev || !dtype_ok(q_dtype) || batch < 1 || batch > 65535 ||
      n_q_heads < 1 || !block_table_dev || max_pages_per_seq < 1 || !seq_lens_dev ||
      max_seq_len < 0 || !out_dev || !workspace_dev)
    return IQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  if ((int64_t)max_seq_len > (int64_t)max_pages_per_seq * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  if (q_dtype != IQ_BF16 || n_q_heads / cache->n_kv_heads > IQ_MAX_GROUP) return IQ_ERR_UNSUPPORTED;
  const iq::DecodePlan plan = iq::plan_dense_decode(batch, cache->n_kv_heads, max_seq_len, device_cu_count());
  if (workspace_bytes < iq::decode_workspace_bytes(batch, n_q_heads, plan)) return IQ_ERR_WORKSPACE;
  return launch_status(iq::launch_dense_decode(dense_view(cache), q_dev, batch, n_q_heads, block_table_dev,
                                               max_pages_per_seq, seq_lens_dev, plan,
                                               resolve_scale(softmax_scale), out_dev, workspace_dev,
                                               stream));
}

iq_status iq_dense_prefill_attention(const iq_dense_cache* cache, const void* q_dev, int32_t q_dtype,
                                     int32_t n_q, int32_t n_q_heads, int32_t q_start_pos,
                                     const int32_t* block_table_dev, int32_t max_pages, float softmax_scale,
                                     float* out_dev, hipStream_t stream) {
  if (!dense_ok(cache) || !q_dev || !dtype_ok(q_dtype) || n_q < 0 || n_q_heads < 1 || q_start_pos < 0 ||
      !block_table_dev || max_pages < 1 || !out_dev)
    return IQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  if ((int64_t)q_start_pos + n_q > (int64_t)max_pages * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  if (n_q == 0) return IQ_OK;
  const int group = n_q_heads / cache->n_kv_heads;
  if (q_dtype != IQ_BF16 || !pow2(group) || group > 128) return IQ_ERR_UNSUPPORTED;
  if ((int64_t)q_start_pos + n_q > (int64_t)iq::kPrefillMaxPages * IQ_PAGE_TOKENS) return IQ_ERR_UNSUPPORTED;
  if ((n_q + 128 / group - 1) / (128 / group) > 65535) return IQ_ERR_UNSUPPORTED;
  return launch_status(iq::launch_dense_prefill(dense_view(cache), q_dev, n_q, n_q_heads, q_start_pos,
                                                block_table_dev, max_pages, resolve_scale(softmax_scale),
                                                out_dev, stream));
}

size_t iq_probe_sink_bytes(void) {
  return (size_t)iq::kProbeBlocks * iq::kProbeThreads * sizeof(uint32_t);
}

iq_status iq_probe_read(const void* buf_dev, size_t bytes, void* sink_dev, size_t sink_bytes,
                        hipStream_t stream) {
  if (!buf_dev || !sink_dev || bytes == 0 || bytes % 16 != 0 || sink_bytes < iq_probe_sink_bytes())
    return IQ_ERR_INVALID_ARG;
  return launch_status(iq::launch_probe_read(buf_dev, bytes, static_cast<uint32_t*>(sink_dev), stream));
}

size_t iq_prefill_workspace_bytes(int32_t n_q, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t q_start_pos) {
  if (n_q < 1 || n_q_heads < 1 || n_kv_heads < 1 || q_start_pos < 0) return 0;
  const iq::PrefillPlan plan = iq::plan_prefill(n_q, n_q_heads, n_kv_heads, q_start_pos, device_cu_count());
  return iq::prefill_workspace_bytes(n_q, n_q_heads, plan);
}

iq_status iq_prefill_attention_ex(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                                  int32_t q_dtype, int32_t n_q, int32_t n_q_heads, int32_t q_start_pos,
                                  const int32_t* block_table_dev, int32_t max_pages, float softmax_scale,
                                  float* out_dev, void* workspace_dev, size_t workspace_bytes,
                                  const iq_prefill_options* options, hipStream_t stream) {
  if (!cache_ok(cache) || !rot_dev || !q_dev || !dtype_ok(q_dtype) || n_q < 0 || n_q_heads < 1 ||
      q_start_pos < 0 || !block_table_dev || max_pages < 1 || !out_dev)
    return IQ_ERR_INVALID_ARG;
  const int waves = options ? options->waves : 0;
  if (waves != 0 && waves != 4 && waves != 8) return IQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  if ((int64_t)q_start_pos + n_q > (int64_t)max_pages * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  if (n_q == 0) return IQ_OK;
  const int group = n_q_heads / cache->n_kv_heads;
  if (!pow2(group) || group > 128 || cache->n_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;
  if ((int64_t)q_start_pos + n_q > (int64_t)iq::kPrefillMaxPages * IQ_PAGE_TOKENS)
    return IQ_ERR_UNSUPPORTED;
  iq::PrefillPlan plan = iq::plan_prefill(n_q, n_q_heads, cache->n_kv_heads, q_start_pos, device_cu_count());
  if (waves == 4) plan.waves = 4;
  if (plan.row_tiles > 65535) return IQ_ERR_UNSUPPORTED;
  const size_t need = iq::prefill_workspace_bytes(n_q, n_q_heads, plan);
  if (need > 0 && (!workspace_dev || workspace_bytes < need)) return IQ_ERR_WORKSPACE;
  return launch_status(iq::launch_prefill(view(cache), reinterpret_cast<const float*>(rot_dev), q_dev,
                                          q_dtype, n_q, n_q_heads, q_start_pos, block_table_dev, max_pages,
                                          plan, resolve_scale(softmax_scale), out_dev, workspace_dev,
                                          stream));
}

iq_status iq_prefill_attention(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                               int32_t q_dtype, int32_t n_q, int32_t n_q_heads, int32_t q_start_pos,
                               const int32_t* block_table_dev, int32_t max_pages, float softmax_scale,
                               float* out_dev, void* workspace_dev, size_t workspace_bytes,
                               hipStream_t stream) {
  return iq_prefill_attention_ex(cache, rot_dev, q_dev, q_dtype, n_q, n_q_heads, q_start_pos, block_table_dev,
                                 max_pages, softmax_scale, out_dev, workspace_dev, workspace_bytes, nullptr,
                                 stream);
}

size_t iq_prefill_append_workspace_bytes(int32_t n_q, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t q_start_pos) {
  if (n_q < 0 || n_q_heads < 1 || n_kv_heads < 1 || q_start_pos < 0) return 0;
  const size_t base = n_q > 0 ? iq_prefill_workspace_bytes(n_q, n_q_heads, n_kv_heads, q_start_pos) : 0;
  return iq::kWsCounterBytes + base;
}

int32_t iq_prefill_append_launches(int32_t n_q, int32_t n_q_heads, int32_t n_kv_heads, int32_t bits) {
  if (n_q < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0 || (bits != 3 && bits != 4))
    return IQ_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return IQ_ERR_DEVICE;
  const int cus = device_cu_count();
  const iq::PrefillPlan plan = iq::plan_prefill(n_q, n_q_heads, n_kv_heads, 0, cus);
  return iq::prefill_append_fused(plan, n_kv_heads, bits, cus) ? 1 : 2;
}

iq_status iq_prefill_append(const iq_cache* cache, const void* rot_dev, const void* k_new_dev,
                            const void* v_new_dev, int32_t kv_dtype, int32_t n_new, int32_t new_start,
                            const void* q_dev, int32_t q_dtype, int32_t n_q, int32_t n_q_heads,
                            int32_t q_start_pos, const int32_t* block_table_dev, int32_t max_pages,
                            float softmax_scale, float* out_dev, void* workspace_dev,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!cache_ok(cache) || !rot_dev || n_new < 0 || new_start < 0 || n_q < 0 || n_q_heads < 1 ||
      q_start_pos < 0 || !block_table_dev || max_pages < 1 || !workspace_dev)
    return IQ_ERR_INVALID_ARG;
  if (n_new > 0 && (!k_new_dev || !v_new_dev || !dtype_ok(kv_dtype))) return IQ_ERR_INVALID_ARG;
  if (n_q > 0 && (!q_dev || !dtype_ok(q_dtype) || !out_dev)) return IQ_ERR_INVALID_ARG;
  if ((int64_t)new_start + n_new > (int64_t)max_pages * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  if ((int64_t)q_start_pos + n_q > (int64_t)max_pages * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  const int group = n_q_heads / cache->n_kv_heads;
  if (n_q > 0) {
    if (!pow2(group) || group > 128 || cache->n_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;
    if ((int64_t)q_start_pos + n_q > (int64_t)iq::kPrefillMaxPages * IQ_PAGE_TOKENS) return IQ_ERR_UNSUPPORTED;
  }
  if (workspace_bytes < iq_prefill_append_workspace_bytes(n_q, n_q_heads, cache->n_kv_heads, q_start_pos))
    return IQ_ERR_WORKSPACE;
  const iq::CacheView c = view(cache);
  const float* rot = reinterpret_cast<const float*>(rot_dev);
  if (n_q == 0)
    return n_new == 0 ? IQ_OK
                      : launch_status(iq::launch_quantize_append_range(c, rot, k_new_dev, v_new_dev, kv_dtype,
                                                                       n_new, new_start, block_table_dev,
                                                                       max_pages, stream));
  const int cus = device_cu_count();
  const iq::PrefillPlan plan = iq::plan_prefill(n_q, n_q_heads, cache->n_kv_heads, q_start_pos, cus);
  if (plan.row_tiles > 65535) return IQ_ERR_UNSUPPORTED;
  const float scale = resolve_scale(softmax_scale);
  if (n_new > 0 && iq::prefill_append_fused(plan, cache->n_kv_heads, c.bits, cus)) {
    const iq::PrefillAppend app{k_new_dev, v_new_dev, kv_dtype, n_new, new_start,
                                reinterpret_cast<uint32_t*>(workspace_dev)};
    return launch_status(iq::launch_prefill_args(c, rot, q_dev, q_dtype, 1, n_q, n_q_heads, nullptr,
                                                 q_start_pos, nullptr, block_table_dev, max_pages, plan,
                                                 scale, out_dev, &app, stream));
  }
  if (n_new > 0) {
    const hipError_t e = iq::launch_quantize_append_range(c, rot, k_new_dev, v_new_dev, kv_dtype, n_new,
                                                          new_start, block_table_dev, max_pages, stream);
    if (e != hipSuccess) return IQ_ERR_LAUNCH;
  }
  return launch_status(iq::launch_prefill(c, rot, q_dev, q_dtype, n_q, n_q_heads, q_start_pos, block_table_dev,
                                          max_pages, plan, scale, out_dev,
                                          static_cast<uint8_t*>(workspace_dev) + iq::kWsCounterBytes, stream));
}

iq_status iq_prefill_attention_varlen(const iq_cache* cache, const void* rot_dev, const void* q_dev,
                                      int32_t q_dtype, int32_t batch, int32_t n_q_heads, int32_t total_q,
                                      const int32_t* cu_q_dev, const int32_t* q_start_dev,
                                      int32_t max_q_per_seq, int32_t max_kv_len,
                                      const int32_t* block_table_dev, int32_t max_pages_per_seq,
                                      float softmax_scale, float* out_dev, void* workspace_dev,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!cache_ok(cache) || !rot_dev || !dtype_ok(q_dtype) || batch < 1 || batch > 65535 ||
      n_q_heads < 1 || total_q < 0 || max_q_per_seq < 0 || max_kv_len < 0 ||
      max_pages_per_seq < 1 || !block_table_dev || !cu_q_dev || !q_start_dev)
    return IQ_ERR_INVALID_ARG;
  if (n_q_heads % cache->n_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  if ((int64_t)max_q_per_seq > (int64_t)max_kv_len || max_q_per_seq > total_q) return IQ_ERR_INVALID_ARG;
  if ((int64_t)max_kv_len > (int64_t)max_pages_per_seq * IQ_PAGE_TOKENS) return IQ_ERR_INVALID_ARG;
  if (total_q == 0 || max_q_per_seq == 0) return IQ_OK;
  if (!q_dev || !out_dev) return IQ_ERR_INVALID_ARG;
  const int group = n_q_heads / cache->n_kv_heads;
  if (!pow2(group) || group > 128 || cache->n_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;
  if ((int64_t)max_kv_len > (int64_t)iq::kPrefillMaxPages * IQ_PAGE_TOKENS) return IQ_ERR_UNSUPPORTED;
  const iq::PrefillPlan plan =
      iq::plan_prefill(max_q_per_seq, n_q_heads, cache->n_kv_heads, 0, device_cu_count());
  if (plan.row_tiles > 65535) return IQ_ERR_UNSUPPORTED;
  const size_t need = iq::prefill_workspace_bytes(total_q, n_q_heads, plan);
  if (need > 0 && (!workspace_dev || workspace_bytes < need)) return IQ_ERR_WORKSPACE;
  return launch_status(iq::launch_prefill_varlen(view(cache), reinterpret_cast<const float*>(rot_dev),
                                                 q_dev, q_dtype, batch, total_q, n_q_heads, cu_q_dev, 0,
                                                 q_start_dev, block_table_dev, max_pages_per_seq, plan,
                                                 resolve_scale(softmax_scale), out_dev, workspace_dev,
                                                 stream));
}

}  // extern "C"
