/*
 * libisoquant — IsoQuant compressed-space attention for AMD Instinct MI355X
 * (gfx950).  C ABI: plain pointers and sizes, no C++ or framework types.
 *
 * The method ("RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via
 * Fused Compressed-Space Attention", abstract): each key/value head vector
 * (d = 128) is put through a normalised Walsh-Hadamard transform and then 32
 * block-diagonal SO(4) rotations, each given by a pair of unit quaternions
 * (256 stored parameters per head), and is then scalar-quantised to 3 bits;
 * attention runs on the packed tensors without materialising full-precision
 * K/V.  The query is rotated into the same orthogonal space and the value
 * accumulator is rotated back once at the end.
 *
 * Quantiser: n = ||x||_2 (stored as fp16), u = (T x) sqrt(d) / n, code =
 * number of the seven nearest-centroid thresholds that u reaches; centroids
 * are the 8 Gaussian Lloyd-Max levels +-0.2451, +-0.7560, +-1.3440, +-2.1520
 * scaled by n / sqrt(d).  One record = 48 bytes of codes + 2 bytes of norm.
 *
 * Conventions for every entry point
 *   - Pointers named *_dev are device memory on the current HIP device; the
 *     caller allocates and owns all of them (cache, rotation, inputs,
 *     outputs, workspace).  The library never allocates or frees device
 *     memory and keeps no pointer after returning.
 *   - Every call is asynchronous on `stream` (0 = the null stream) and does
 *     not synchronise the host (FreeToken v0.2.0 release notes, Kernels:
 *     attention metadata must not block the host, #726).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns a negative iq_status and enqueues nothing.  A
 *     failed kernel launch returns IQ_ERR_LAUNCH.
 *   - Device-side contract (not checked): block-table entries lie in
 *     [0, num_pages); sequence lengths and positions fit the block table;
 *     each cache slot is written by at most one token of a call.
 *   - Byte offsets are computed in 64 bits (caches larger than 2^31 bytes
 *     are supported; FreeToken v0.2.0 release notes, GGUF Support #699:
 *     kernels must not run past 32-bit offsets).
 *   - Functions are re-entrant; calls that write the same cache slots or the
 *     same workspace on overlapping streams race.
 */
#ifndef ISOQUANT_H
#define ISOQUANT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IQ_OK = 0,
  IQ_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad dtype, bad quaternion */
  IQ_ERR_UNSUPPORTED = -2,   /* valid but outside what the kernels handle     */
  IQ_ERR_WORKSPACE = -3,     /* workspace smaller than the *_workspace_bytes   */
  IQ_ERR_LAUNCH = -4,        /* HIP reported an error for a copy or launch     */
  IQ_ERR_DEVICE = -5,        /* no usable HIP device                           */
  IQ_ERR_SCRATCH = -6        /* the call needs more than the static scratch    */
} iq_status;

typedef enum { IQ_F32 = 0, IQ_BF16 = 1, IQ_F16 = 2 } iq_dtype;

enum {
  IQ_HEAD_DIM = 128,         /* d                                               */
  IQ_PAGE_TOKENS = 64,       /* tokens per cache page                           */
  IQ_CODE_BYTES = 48,        /* 128 codes x 3 bits                              */
  IQ_CODE_BYTES4 = 64,       /* 128 codes x 4 bits (4-bit caches)               */
  IQ_ROT_PARAMS = 256,       /* stored rotation parameters per kv head          */
  IQ_MAX_GROUP = 16          /* query heads per kv head handled by decode       */
};

/*
 * One layer's paged cache, in four caller-owned device arrays:
 *   k_codes, v_codes : uint8  [num_pages][n_kv_heads][64][48]
 *   k_norms, v_norms : uint16 [num_pages][n_kv_heads][64]   (fp16 bit patterns)
 * Token t of a sequence lives in page block_table[seq][t / 64], slot t % 64
 * (FreeToken v0.1.3 release notes, Engine #367: paged KV reserved at allocation
 * granularity).
 * Code record layout (48 bytes, coordinates 0..127): four 12-byte groups, group
 * g holding coordinates 32g..32g+31.  In a group, the bytes at offsets b, 4+b
 * and 8+b (b = 0..3) form a 24-bit little-endian integer ("byte lane" b); the
 * 3-bit code of coordinate 32g + 4s + b is at bits 3s..3s+2 of byte lane b.
 * K pages hold the records slot after slot: record (page, head, slot) starts
 * at byte ((page * n_kv_heads + head) * 64 + slot) * 48 of k_codes.
 * V pages hold the same records in the order the decode matrix cores read
 * them: the 3,072 bytes of (page, head) are 64 regions of 48 bytes, region
 * n + 16 q (n, q < 16, 4) made of four 12-byte chunks c; byte lane r (bytes r,
 * 4 + r, 8 + r) of chunk c of region (n, q) is byte lane n % 4 of group n / 4
 * of the record in slot 16 c + 4 q + r.  Norm arrays are slot-ordered for
 * both.  The struct is read during the call only.
 *
 * bits = 4 selects the 4-bit variant of the same pipeline (FreeToken issue
 * #141, Proposed Solution: the rotation-based KV quantisers listed there span
 * 3 and 4 bits): codes are the 16-level Gaussian Lloyd-Max quantiser's (see
 * iq_codebook), 64 bytes per record, k_codes/v_codes [num_pages][n_kv_heads][64][64].
 * A stored nibble is sign-magnitude: code c (0..15, ascending levels) is stored
 * as c - 8 for c >= 8 and 15 - c below.  Record: dword d (bytes 4d..4d+3)
 * holds coordinates 8d..8d+7, byte b of it coordinate 8d + b in its low nibble
 * and 8d + 4 + b in its high one.  V blocks (4,096 bytes per (page, head)):
 * 64 regions of 64 bytes; region n + 16 jq (n < 16, jq < 4) is 16 dwords, dword
 * 4p + 2 th + q (p < 4, th < 2, q < 2) holds in byte r the token of slot
 * 32 th + 16 q + 4 jq + r, its coordinate c = 32 (n / 4) + 4p + n % 4 in the low
 * nibble and c + 16 in the high one.  bits = 0 or 3: the 3-bit records above.
 * Every entry point taking an iq_cache handles both widths.
 */
typedef struct {
  uint8_t *k_codes_dev;
  uint16_t *k_norms_dev;
  uint8_t *v_codes_dev;
  uint16_t *v_norms_dev;
  int32_t num_pages;
  int32_t n_kv_heads;
  int32_t bits;              /* 0 or 3: 3-bit records; 4: 4-bit records; else invalid */
} iq_cache;

/* Human-readable text for a status code (static storage). */
const char *iq_status_string(int32_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t iq_version(void);

/*
 * The scalar quantiser of a record width, as the kernels apply it (host
 * only; no device is needed).  bits = 3: the eight Gaussian Lloyd-Max levels
 * the specification of this path fixes (the pages name 3-bit scalar
 * quantisation and print no levels); bits = 4:
 * the 16-level Gaussian Lloyd-Max quantiser, computed by Lloyd's iteration
 * (thresholds at the midpoints of adjacent levels, each level the mean of
 * N(0, 1) over its cell) once per process.
 *
 * levels_host     : 2^bits doubles, written: the ascending levels.
 * thresholds_host : 2^bits - 1 floats, written: the fp32 decision thresholds;
 *                   code = number of thresholds u reaches (u >= t).
 * level_scale     : may be null; written: alpha, the factor applied to the
 *                   levels before they are rounded to the f16 operands of the
 *                   matrix cores (1/alpha is folded into the norm factors).
 * Errors          : IQ_ERR_INVALID_ARG for bits not 3 or 4 or a null array.
 */
iq_status iq_codebook(int32_t bits, double *levels_host, float *thresholds_host,
                      float *level_scale);

/*
 * Rotation setup ("RotaryQuant ...", abstract: WHT followed by block-diagonal
 * SO(4) rotations; FreeToken issue #141, Proposed Solution: quaternion
 * rotations).  One rotation per kv head, shared by K, V and that head's query
 * group.
 *
 * quats_host : host float[n_kv_heads][32][2][4]; [h][b][0] = q_L, [h][b][1] = q_R,
 *              components (w, x, y, z) with w real.  Need not be unit: each is
 *              normalised.  Block b maps coordinates 4b..4b+3, read as the
 *              quaternion v = v0 + v1 i + v2 j + v3 k, to q_L * v * conj(q_R).
 * rot_dev    : device buffer of at least iq_rotation_bytes(n_kv_heads) bytes,
 *              written by this call; pass it unchanged to the other calls.
 * Errors     : IQ_ERR_INVALID_ARG for null pointers, n_kv_heads < 1, a buffer
 *              that is too small, or a quaternion of zero or non-finite norm.
 */
size_t iq_rotation_bytes(int32_t n_kv_heads);
iq_status iq_rotation_init(const float *quats_host, int32_t n_kv_heads, void *rot_dev,
                           size_t rot_bytes, hipStream_t stream);

/*
 * Quantise and append ("RotaryQuant ...", abstract: 3-bit scalar quantisation
 * after the rotation).  For every token i and kv head h, quantises K[i][h] and
 * V[i][h] and stores the records in slot pos[i] % 64 of page
 * block_table[seq_idx[i]][pos[i] / 64].
 *
 * k_dev, v_dev     : [n_tokens][n_kv_heads][128] of `dtype` (IQ_F32/IQ_BF16/IQ_F16).
 * seq_idx_dev      : int32[n_tokens], row of the block table of each token.
 * pos_dev          : int32[n_tokens], absolute position of each token.
 * block_table_dev  : int32[*][max_pages_per_seq], row-major.
 * n_tokens == 0 is a no-op.  Inputs with non-finite values give unspecified codes.
 * A token whose position lies outside the block table, or whose table entry is
 * not a page of the cache, is skipped: no record is written for it.
 */
iq_status iq_quantize_append(const iq_cache *cache, const void *rot_dev, const void *k_dev,
                             const void *v_dev, int32_t dtype, int32_t n_tokens,
                             const int32_t *seq_idx_dev, const int32_t *pos_dev,
                             const int32_t *block_table_dev, int32_t max_pages_per_seq,
                             hipStream_t stream);

/*
 * Decode attention on the packed cache ("RotaryQuant ...", abstract; the
 * context is split across workgroups as in FreeToken v0.2.0 release notes,
 * Kernels #729, and an all -inf chunk yields no NaN, #654).  Every query head
 * h of sequence b attends all seq_lens[b] cached tokens of kv head
 * h / (n_q_heads / n_kv_heads); the caller appends the current token first.
 *
 * q_dev          : [batch][n_q_heads][128] of q_dtype.
 * block_table_dev: int32[batch][max_pages_per_seq].
 * seq_lens_dev   : int32[batch], each in [0, max_seq_len].
 * max_seq_len    : host-side upper bound of seq_lens, used to plan the splits.
 * softmax_scale  : <= 0 selects 1/sqrt(128).
 * out_dev        : float[batch][n_q_heads][128], in the original (unrotated) space.
 *                  A sequence of length 0 gives zeros.
 * workspace_dev  : at least iq_decode_workspace_bytes(...) bytes.  Its first
 *                  IQ_DECODE_COUNTER_BYTES bytes are arrival counters and must
 *                  be zero before the buffer's first decode call (zero a new
 *                  buffer once); every call leaves them zero.  The rest holds
 *                  the per-split partials (m, l, accumulator) of this call,
 *                  any contents on entry.
 * Unsupported: n_q_heads / n_kv_heads > IQ_MAX_GROUP.
 * Splits and their merge: the context of each (sequence, kv head) is split
 * across workgroups; the partials are merged by a second kernel, or (on
 * request, see iq_decode_options.merge) by merge workgroups of the same
 * launch, which wait for the split workgroups of their (sequence, kv head)
 * through the counters (only where the runtime's occupancy calculator says
 * the whole grid is resident at once).
 * Determinism: by default the waves of a workgroup take the pages of their
 * split as they become free, so the order of the f16 rounding of softmax
 * weights can differ between runs (the results agree to about 2^-11 of a
 * weight, far inside the 1e-3 tolerance); iq_decode_options.deterministic
 * fixes the order (bit-identical results for a fixed plan).
 */
enum { IQ_DECODE_COUNTER_BYTES = 16384 };
size_t iq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t max_seq_len);
iq_status iq_decode_attention(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                              int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                              const int32_t *block_table_dev, int32_t max_pages_per_seq,
                              const int32_t *seq_lens_dev, int32_t max_seq_len,
                              float softmax_scale, float *out_dev, void *workspace_dev,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * Choices a caller may fix for one decode call (the _ex entry points below;
 * the context split by length and CU count, FreeToken v0.2.0 release notes,
 * Kernels #729).  A zero field leaves the choice to the planner; a null
 * pointer means all zeros, which is what the plain entry points use.  The
 * same options must be given to iq_decode_workspace_bytes_ex and to the call.
 *   waves           : 0, 4 or 8 waves per workgroup.
 *   pages_per_split : 0, or pages per split of the host plan (capped at 64 per wave).
 *   rounds          : 0, or the workgroups per CU the plan is made for (more,
 *                     shorter splits).
 *   plan            : IQ_PLAN_AUTO (device-balanced for 2..64 sequences, else the
 *                     host plan), IQ_PLAN_HOST (splits of equal page ranges
 *                     planned from max_seq_len), IQ_PLAN_BALANCED (= AUTO).
 *   merge           : IQ_MERGE_AUTO / IQ_MERGE_KERNEL: a merge kernel follows
 *                     the split launch; IQ_MERGE_FUSED: merge workgroups join the
 *                     split launch where allowed (host plan, four waves, the
 *                     whole grid resident at once), else a merge kernel.
 *   deterministic   : nonzero: wave w of a workgroup takes pages w, w + W, ...
 *                     of its split in order: bit-identical results for a fixed
 *                     plan, run after run.
 * Errors: IQ_ERR_INVALID_ARG for a field outside these values.
 */
typedef enum { IQ_PLAN_AUTO = 0, IQ_PLAN_HOST = 1, IQ_PLAN_BALANCED = 2 } iq_decode_plan;
typedef enum { IQ_MERGE_AUTO = 0, IQ_MERGE_FUSED = 1, IQ_MERGE_KERNEL = 2 } iq_decode_merge;
typedef struct {
  int32_t waves;
  int32_t pages_per_split;
  int32_t rounds;
  int32_t plan;
  int32_t merge;
  int32_t deterministic;
} iq_decode_options;
size_t iq_decode_workspace_bytes_ex(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t max_seq_len, const iq_decode_options *options);
iq_status iq_decode_attention_ex(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                                 int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                 const int32_t *block_table_dev, int32_t max_pages_per_seq,
                                 const int32_t *seq_lens_dev, int32_t max_seq_len,
                                 float softmax_scale, float *out_dev, void *workspace_dev,
                                 size_t workspace_bytes, const iq_decode_options *options,
                                 hipStream_t stream);

/*
 * Decode step = quantise-append of each sequence's current token followed by
 * decode attention, fused ("RotaryQuant ...", abstract: the quantiser and the
 * packed-tensor attention form one fused GPU pipeline): the append runs inside
 * the decode kernel, in the workgroup that reads the sequence's last page, so
 * a step is two launches instead of three.  Equivalent to iq_quantize_append of the
 * tokens (seq_idx = b, pos = seq_lens[b] - 1) followed by iq_decode_attention
 * with the same arguments: the same records are written, and the attention
 * uses the new token.
 *
 * k_new_dev, v_new_dev : [batch][n_kv_heads][128] of kv_dtype (IQ_F32/IQ_BF16/IQ_F16),
 *                        the K and V rows of the token at position seq_lens[b] - 1.
 * Other arguments and the workspace are those of iq_decode_attention.  A
 * sequence with seq_lens[b] = 0 appends nothing and gives zeros.  The table
 * entry of the new token's page must be a page of the cache (otherwise no
 * record is written and the attention reads an unspecified page).
 */
iq_status iq_decode_step(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                         int32_t q_dtype, int32_t batch, int32_t n_q_heads, const void *k_new_dev,
                         const void *v_new_dev, int32_t kv_dtype, const int32_t *block_table_dev,
                         int32_t max_pages_per_seq, const int32_t *seq_lens_dev,
                         int32_t max_seq_len, float softmax_scale, float *out_dev,
                         void *workspace_dev, size_t workspace_bytes, hipStream_t stream);
/*
 * The launch plan a decode call with these arguments would use (host only;
 * the merge choice asks the HIP runtime's occupancy calculator about the
 * current device, so without a usable device fused_merge reads 0).  bits: 3
 * or 4 (the cache's record width); step: nonzero for iq_decode_step(_ex).
 * Writes *info; IQ_ERR_INVALID_ARG for arguments the call would refuse for
 * the same reasons.
 */
typedef struct {
  int32_t waves;            /* waves per workgroup                                   */
  int32_t splits;           /* host plan: splits per (sequence, kv head); balanced:
                               partial-row slots per query head                      */
  int32_t pages_per_split;  /* host plan: pages per split; balanced: the cap         */
  int32_t balanced;         /* 1: the split plan is made on the device from the lengths */
  int32_t fused_merge;      /* 1: merge workgroups in the split launch; 0: a merge kernel */
  int32_t workgroups;       /* workgroups of the split launch                        */
} iq_decode_plan_info;
iq_status iq_decode_describe(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t max_seq_len,
                             int32_t bits, int32_t step, const iq_decode_options *options,
                             iq_decode_plan_info *info);

/*
 * iq_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments and results as iq_decode_step without the workspace:
 * the split partials live in a static device array of the library
 * (IQ_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends), located
 * once per device on the first call made with that device current.  The call
 * allocates and frees nothing.  Every call on a GPU shares that GPU's array,
 * so calls that overlap on one GPU (other streams, other host threads) race;
 * nothing in the array needs to start at zero (the merge always runs as a
 * second kernel).  IQ_ERR_SCRATCH (nothing enqueued) when the call's plan
 * needs more than the array holds (iq_decode_workspace_bytes of the same
 * arguments > IQ_NOALLOC_SCRATCH_BYTES); IQ_ERR_DEVICE when the array cannot
 * be located on the current device; other errors as iq_decode_step.
 */
enum { IQ_NOALLOC_SCRATCH_BYTES = 32 << 20 };
iq_status iq_decode_step_noalloc(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                                 int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                 const void *k_new_dev, const void *v_new_dev, int32_t kv_dtype,
                                 const int32_t *block_table_dev, int32_t max_pages_per_seq,
                                 const int32_t *seq_lens_dev, int32_t max_seq_len, float softmax_scale,
                                 float *out_dev, hipStream_t stream);

/* iq_decode_step with the options of iq_decode_attention_ex. */
iq_status iq_decode_step_ex(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                            int32_t q_dtype, int32_t batch, int32_t n_q_heads, const void *k_new_dev,
                            const void *v_new_dev, int32_t kv_dtype, const int32_t *block_table_dev,
                            int32_t max_pages_per_seq, const int32_t *seq_lens_dev,
                            int32_t max_seq_len, float softmax_scale, float *out_dev,
                            void *workspace_dev, size_t workspace_bytes,
                            const iq_decode_options *options, hipStream_t stream);

/*
 * Chunked causal prefill attention of one sequence on the packed cache
 * ("RotaryQuant ...", abstract; FreeToken issue #141, Proposed Solution:
 * faster prefill with GQA).  Query i sits at position q_start_pos + i and
 * attends cached keys 0 .. q_start_pos + i.  The GQA-grouped QK^T and PV are
 * dense contractions and run on the matrix cores (f16 inputs, fp32 accumulate).
 *
 * q_dev          : [n_q][n_q_heads][128] of q_dtype.
 * block_table_dev: int32[max_pages] of this sequence.
 * out_dev        : float[n_q][n_q_heads][128], original space.
 * workspace_dev  : at least iq_prefill_workspace_bytes(...) bytes (currently 0).
 * Unsupported: q_start_pos + n_q > 262,144 (the causal range's page ids are
 * staged on chip), or n_q_heads / n_kv_heads not a power of two up to 128.
 */
size_t iq_prefill_workspace_bytes(int32_t n_q, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t q_start_pos);
iq_status iq_prefill_attention(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                               int32_t q_dtype, int32_t n_q, int32_t n_q_heads,
                               int32_t q_start_pos, const int32_t *block_table_dev,
                               int32_t max_pages, float softmax_scale, float *out_dev,
                               void *workspace_dev, size_t workspace_bytes, hipStream_t stream);
/*
 * iq_prefill_attention with a choice of workgroup shape (same results up to
 * the order of the fp32 sums): waves 0 or 8 = eight waves of 16 query rows
 * (the default), 4 = four waves of 32 rows.  A null pointer means 0.
 * IQ_ERR_INVALID_ARG for another value.
 */
typedef struct {
  int32_t waves;
} iq_prefill_options;
iq_status iq_prefill_attention_ex(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                                  int32_t q_dtype, int32_t n_q, int32_t n_q_heads,
                                  int32_t q_start_pos, const int32_t *block_table_dev,
                                  int32_t max_pages, float softmax_scale, float *out_dev,
                                  void *workspace_dev, size_t workspace_bytes,
                                  const iq_prefill_options *options, hipStream_t stream);

/*
 * Quantise-append of a chunk fused with the chunked prefill over it
 * ("RotaryQuant ...", abstract: quantiser and packed-tensor attention as one
 * fused GPU pipeline; FreeToken v0.2.0 release notes, Kernels #632: extend
 * attention, a prefill chunk attending the cache it extends).  The same
 * records and the same attention as iq_quantize_append of the chunk's tokens
 * (sequence 0 of the one-row block table, positions new_start .. new_start +
 * n_new - 1) followed by iq_prefill_attention with the other arguments.
 * When the runtime's occupancy calculator says the whole prefill grid is
 * resident at once, one launch does both: the prefill workgroups of each kv
 * head first quantise a share of the chunk's 64-token blocks, store the
 * records device-coherent and count them in; a workgroup waits for the count
 * only before it requests the first page holding appended tokens (the waits
 * are bounded, about a second; a wait that runs out leaves NaN rows).  The
 * waits need every workgroup of the launch to get a CU: work of other
 * streams only delays that, but two such launches (or fused-merge decode
 * launches) overlapping on one GPU can hold each other's CUs until the waits
 * run out, so overlapping calls are the caller's to avoid.  Otherwise the
 * two kernels run one after the other.
 *
 * k_new_dev, v_new_dev : [n_new][n_kv_heads][128] of kv_dtype.
 * workspace_dev        : at least iq_prefill_append_workspace_bytes(...) bytes;
 *                        its first IQ_DECODE_COUNTER_BYTES bytes are counters that
 *                        must be zero before the buffer's first use (every call
 *                        leaves them zero).
 * n_new = 0: the prefill alone; n_q = 0: the append alone.  Other arguments,
 * limits and errors as iq_quantize_append and iq_prefill_attention;
 * IQ_ERR_INVALID_ARG also when new_start + n_new exceeds the block table.
 */
size_t iq_prefill_append_workspace_bytes(int32_t n_q, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t q_start_pos);
/* Kernels an iq_prefill_append call with n_new > 0 and n_q > 0 launches on the
 * current device: 1 (fused) or 2; IQ_ERR_INVALID_ARG / IQ_ERR_DEVICE as a
 * negative value. */
int32_t iq_prefill_append_launches(int32_t n_q, int32_t n_q_heads, int32_t n_kv_heads, int32_t bits);
iq_status iq_prefill_append(const iq_cache *cache, const void *rot_dev, const void *k_new_dev,
                            const void *v_new_dev, int32_t kv_dtype, int32_t n_new, int32_t new_start,
                            const void *q_dev, int32_t q_dtype, int32_t n_q, int32_t n_q_heads,
                            int32_t q_start_pos, const int32_t *block_table_dev, int32_t max_pages,
                            float softmax_scale, float *out_dev, void *workspace_dev,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Batched variable-length chunked prefill: several sequences' query chunks in
 * one launch (the same attention as iq_prefill_attention for each sequence;
 * "RotaryQuant ...", abstract, and FreeToken issue #141, Proposed Solution).
 *
 * q_dev          : [total_q][n_q_heads][128] of q_dtype; sequence b's queries are
 *                  rows cu_q[b] .. cu_q[b+1]-1, query i of it at position
 *                  q_start[b] + i, attending that sequence's keys 0 .. q_start[b] + i.
 * cu_q_dev       : int32[batch + 1], nondecreasing, cu_q[0] = 0, cu_q[batch] <= total_q.
 * q_start_dev    : int32[batch].
 * max_q_per_seq  : host bound of cu_q[b+1] - cu_q[b] (sizes the grid).
 * max_kv_len     : host bound of q_start[b] + cu_q[b+1] - cu_q[b].
 * block_table_dev: int32[batch][max_pages_per_seq].
 * out_dev        : float[total_q][n_q_heads][128], original space; rows of no
 *                  sequence are not written.
 * Unsupported: max_kv_len > 262,144, or n_q_heads / n_kv_heads not a power of two
 * up to 128.  Device data beyond the bounds breaks the contract (wrong results,
 * never reads outside the table or the cache).  total_q = 0 is a no-op.
 */
iq_status iq_prefill_attention_varlen(const iq_cache *cache, const void *rot_dev, const void *q_dev,
                                      int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                      int32_t total_q, const int32_t *cu_q_dev,
                                      const int32_t *q_start_dev, int32_t max_q_per_seq,
                                      int32_t max_kv_len, const int32_t *block_table_dev,
                                      int32_t max_pages_per_seq, float softmax_scale, float *out_dev,
                                      void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/*
 * Uncompressed baseline ("RotaryQuant ...", abstract: the packed attention
 * avoids materialising full-precision KV state; this is that state) and the
 * FP8 fallback (FreeToken issue #141, Proposed Solution: standard FP8 KV as
 * the fallback format).  A paged cache of bf16 or FP8 values and its decode
 * attention on the same paging, split planning and merge as the packed path,
 * so that the packed cache's byte reduction is measured as time on the same
 * GPU.  Numerics: exact products of the stored values and the query (bf16,
 * or f16 for FP8), fp32 accumulation, softmax weights as high + low parts.
 *
 * One layer's cache, in two caller-owned device arrays:
 *   k_dev : [num_pages][n_kv_heads][64][128]   token-major
 *   v_dev : [num_pages][n_kv_heads][128][64]   coordinate-major
 * of uint16 bf16 bits (format IQ_KV_BF16) or uint8 FP8 bytes (IQ_KV_FP8_E4M3:
 * OCP E4M3, 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
 * finite value 448, no infinities).  FP8 holds x / scale, rounded to nearest
 * even and saturated at +-448: byte = e4m3(float(x) * float(1 / k_scale)) for
 * K and likewise for V; the attention reads e4m3 * scale.  Scales must be
 * positive and finite (0 selects 1); bf16 ignores them.
 * Token t of a sequence lives in page block_table[seq][t / 64], slot t % 64.
 */
typedef enum { IQ_KV_BF16 = 0, IQ_KV_FP8_E4M3 = 1 } iq_kv_format;
typedef struct {
  void *k_dev;
  void *v_dev;
  int32_t num_pages;
  int32_t n_kv_heads;
  int32_t format;            /* iq_kv_format */
  float k_scale, v_scale;    /* FP8 only */
} iq_dense_cache;

/* As iq_quantize_append (same arguments, skip rules and errors): stores the K
 * and V rows of each token, rounded to bf16 (nearest even) or encoded as FP8,
 * in its slot.  IQ_ERR_INVALID_ARG also for an unknown format or a negative or
 * non-finite scale. */
iq_status iq_dense_append(const iq_dense_cache *cache, const void *k_dev, const void *v_dev,
                          int32_t dtype, int32_t n_tokens, const int32_t *seq_idx_dev,
                          const int32_t *pos_dev, const int32_t *block_table_dev,
                          int32_t max_pages_per_seq, hipStream_t stream);

/* As iq_decode_attention over the bf16 or FP8 cache: out = softmax(scale q K^T) V
 * per query head over the stored values, fp32 [batch][n_q_heads][128].  q_dtype must be IQ_BF16
 * (IQ_ERR_UNSUPPORTED otherwise); group limit and workspace rules as there (its
 * partials follow the counter region, which it leaves untouched). */
size_t iq_dense_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t max_seq_len);
iq_status iq_dense_decode_attention(const iq_dense_cache *cache, const void *q_dev,
                                    int32_t q_dtype, int32_t batch, int32_t n_q_heads,
                                    const int32_t *block_table_dev, int32_t max_pages_per_seq,
                                    const int32_t *seq_lens_dev, int32_t max_seq_len,
                                    float softmax_scale, float *out_dev, void *workspace_dev,
                                    size_t workspace_bytes, hipStream_t stream);

/* Chunked causal prefill of one sequence over the bf16 or FP8 cache: the
 * attention of iq_prefill_attention (query i at position q_start_pos + i
 * attends keys 0 .. q_start_pos + i) over the stored values, fp32
 * [n_q][n_q_heads][128].  q_dtype must be IQ_BF16 (IQ_ERR_UNSUPPORTED
 * otherwise); other limits, the block table and errors as iq_prefill_attention;
 * no workspace. */
iq_status iq_dense_prefill_attention(const iq_dense_cache *cache, const void *q_dev, int32_t q_dtype,
                                     int32_t n_q, int32_t n_q_heads, int32_t q_start_pos,
                                     const int32_t *block_table_dev, int32_t max_pages,
                                     float softmax_scale, float *out_dev, hipStream_t stream);

/*
 * Measurement aid: the achievable HBM read rate of this GPU, against which the
 * decode kernels' rates are also reported.  Reads `bytes` (a multiple of 16,
 * buffer 16-byte aligned) at buf_dev once, with 16-byte loads from a fixed
 * grid; each thread writes one word (the XOR of what it read) to sink_dev,
 * which must hold iq_probe_sink_bytes() bytes.  IQ_ERR_INVALID_ARG for null
 * pointers, a size of 0 or not a multiple of 16, or a short sink.
 */
size_t iq_probe_sink_bytes(void);
iq_status iq_probe_read(const void *buf_dev, size_t bytes, void *sink_dev, size_t sink_bytes,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ISOQUANT_H */
