// Quantise-append: K/V head vectors -> packed 3-bit (48-byte) or 4-bit
// (64-byte) records + fp16 norms in a 64-token paged cache.
//
// "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention", abstract: Walsh-Hadamard transform, then
// block-diagonal SO(4) rotations, then low-bit scalar quantisation.  Per vector
// x: n = ||x||, u = (B H x) / n (H unnormalised, so u = T x sqrt(d) / n),
// code = number of thresholds u reaches, record = packed codes, norm = fp16(n).
//
// Mapping: four lanes per vector, 32 consecutive coordinates per lane (lane
// quarter j = coordinates 32j..32j+31).  The first half of the grid handles K,
// the second V; consecutive quads take consecutive (token, head) vectors, so a
// wave reads 16 contiguous 256-byte rows and writes 16 x 48 contiguous bytes
// per page run.  All arithmetic is fp32 on the vector ALUs.
#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

// Appends of at most this many vectors (K and V together) take the
// latency-oriented kernel.
constexpr long long kSmallAppendVectors = 16384;

// Grid (token blocks of 64, kv heads, K|V): a workgroup quantises 64
// consecutive input tokens of one kv head and one tensor, a quad of lanes per
// vector.  When the 64 tokens are one whole page of one sequence (positions
// p0 .. p0 + 63, p0 a multiple of 64: a prefill chunk), their K records and
// norms land contiguously, and the V block -- whose matrix-core order
// interleaves the page's tokens -- is assembled in LDS and written as 3,072
// contiguous bytes; otherwise each quad stores its own record.
// The first 14 argument dwords (everything the first loads need) are
// preloaded into SGPRs; the cache pointers follow from the argument segment.
// BITS = 4: the 4-bit records (nibbles, see iq_device.h); a quad lane's
// quarter is then record dwords 4j..4j+3, and its V bytes pair coordinates
// 32j + 4p + b and 32j + 16 + 4p + b of the token.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void quantize_append_kernel(
    const void* __restrict__ k, const void* __restrict__ v, const int32_t* __restrict__ seq_idx,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_table, int n_tok,
    int hkv, int max_pages, const float* __restrict__ rot, int num_pages,
    uint8_t* __restrict__ k_codes, uint16_t* __restrict__ k_norms, uint8_t* __restrict__ v_codes,
    uint16_t* __restrict__ v_norms, Levels4 lv, int pos0) {
  constexpr int kRecB = BITS == 4 ? kRec4 : kRec;
  const int tl = threadIdx.x >> 2, j = threadIdx.x & 3;
  const int head = blockIdx.y, which = blockIdx.z;
  const int t0 = blockIdx.x * 64;
  const int tok = t0 + tl;
  const bool valid = tok < n_tok;
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kPage * kRecB];  // the page's V block
  // the head's rotation blocks, read from LDS by the transform (loaded once
  // per workgroup instead of 32 16-byte loads per lane)
  __shared__ __attribute__((aligned(16))) float s_rot[kRotFloats];

  // The destination is looked up while the vector is transformed: position
  // and sequence first, then the page id, all before the arithmetic.
  // (seq_idx and pos null: one sequence, token i at position pos0 + i)
  const int p = valid ? (pos ? pos[tok] : pos0 + tok) : -1;
  const int si = valid ? (seq_idx ? seq_idx[tok] : 0) : -1;
  const int p0 = pos ? pos[t0] : pos0 + t0, s0 = seq_idx ? seq_idx[t0] : 0;
  float x[32];
  const size_t vi = (size_t)(valid ? tok : t0) * hkv + head;
  load32(which ? v : k, vi * kD + 32 * j, DT, x);
  // a position outside the table or a page id outside the cache is skipped
  const bool in_table = (unsigned)p < (unsigned)max_pages * kPage;
  const int page = in_table ? block_table[(size_t)si * max_pages + (p >> 6)] : -1;
  const bool stored = (unsigned)page < (unsigned)num_pages;
  if (threadIdx.x < kRotFloats / 4)
    reinterpret_cast<f4*>(s_rot)[threadIdx.x] =
        reinterpret_cast<const f4*>(rot + (size_t)head * kRotFloats)[threadIdx.x];
  // one whole page: every token in order, all stored (uniform for the
  // workgroup); the barrier also publishes the rotation blocks
  const bool whole = __syncthreads_and(valid && si == s0 && p == p0 + tl && (p0 & 63) == 0 && stored);

  uint32_t sel[8];
  const float n = quad_codes<BITS>(x, j, s_rot, lv, sel);

  const int slot = p & 63;
  const size_t blk = (size_t)page * hkv + head;  // (page, kv head) block
  quad_store<BITS, PlainStore>(which, stored, whole, j, slot, sel, n,
                               (which ? v_codes : k_codes) + blk * (kPage * kRecB),
                               (which ? v_norms : k_norms) + blk * kPage, s_v, threadIdx.x);
}

// Few vectors (a decode step appends one token per sequence): the latency
// of one vector is what counts.  Here 32 lanes share a vector, lane r holding
// coordinates 4r..4r+3 and SO(4) block r, so the transform is a handful of
// register and lane-exchange steps per lane; lane r's four codes are selector
// r % 8 of group r / 8, and the eight lanes of a group OR their bit fields
// into the group's three dwords.  Loads of the position, the rotation block
// and the vector go out together, the page id as soon as the position lands.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void quantize_small_kernel(
    const void* __restrict__ k, const void* __restrict__ v, const int32_t* __restrict__ seq_idx,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_table,
    const float* __restrict__ rot, int n_vec, int hkv, int max_pages, int num_pages,
    uint8_t* __restrict__ k_codes, uint16_t* __restrict__ k_norms, uint8_t* __restrict__ v_codes,
    uint16_t* __restrict__ v_norms, Levels4 lv, int pos0) {
  const int gv = blockIdx.x * 8 + (threadIdx.x >> 5);  // K vectors first, then V
  const int r = threadIdx.x & 31;
  if (gv >= 2 * n_vec) return;  // whole half-waves leave together
  const int which = gv >= n_vec;
  const int vi = gv - (which ? n_vec : 0);  // token * hkv + head
  const int tok = vi / hkv;
  const int head = vi - tok * hkv;

  const int p = pos ? pos[tok] : pos0 + tok;
  const int si = seq_idx ? seq_idx[tok] : 0;
  const f4* mrow = reinterpret_cast<const f4*>(rot + (size_t)head * kRotFloats + 16 * r);
  const f4 m0 = mrow[0], m1 = mrow[1], m2 = mrow[2], m3 = mrow[3];
  float x0, x1, x2, x3;
  {
    const size_t idx = (size_t)vi * kD + 4 * r;
    if (DT == 0) {
      const f4 a = *reinterpret_cast<const f4*>(reinterpret_cast<const float*>(which ? v : k) + idx);
      x0 = a[0]; x1 = a[1]; x2 = a[2]; x3 = a[3];
    } else {
      const u2 a = *reinterpret_cast<const u2*>(reinterpret_cast<const uint16_t*>(which ? v : k) + idx);
      const uint32_t w0 = a[0], w1 = a[1];
      if (DT == 1) {
        x0 = __builtin_bit_cast(float, w0 << 16);
        x1 = __builtin_bit_cast(float, w0 & 0xFFFF0000u);
        x2 = __builtin_bit_cast(float, w1 << 16);
        x3 = __builtin_bit_cast(float, w1 & 0xFFFF0000u);
      } else {
        x0 = half_bits_to_float(w0 & 0xFFFFu);
        x1 = half_bits_to_float(w0 >> 16);
        x2 = half_bits_to_float(w1 & 0xFFFFu);
        x3 = half_bits_to_float(w1 >> 16);
      }
    }
  }
  // a position outside the table or a page id outside the cache is skipped
  const bool in_table = (unsigned)p < (unsigned)max_pages * kPage;
  const int page = in_table ? block_table[(size_t)si * max_pages + (p >> 6)] : -1;

  float n;
  if constexpr (BITS == 3) {
    u3 w;
    quantize_lanes32<false>(x0, x1, x2, x3, m0, m1, m2, m3, r, n, w);
    if ((unsigned)page >= (unsigned)num_pages) return;
    const size_t blk = (size_t)page * hkv + head;  // (page, kv head) block
    place_record(which, r, w, n, (which ? v_codes : k_codes) + blk * (kPage * kRec),
                 (which ? v_norms : k_norms) + blk * kPage, p & 63);
  } else {
    const uint32_t w = quantize_lanes32_4(x0, x1, x2, x3, m0, m1, m2, m3, r, which, lv, n);
    if ((unsigned)page >= (unsigned)num_pages) return;
    const size_t blk = (size_t)page * hkv + head;
    place_record4(which, r, w, n, (which ? v_codes : k_codes) + blk * (kPage * kRec4),
                  (which ? v_norms : k_norms) + blk * kPage, p & 63);
  }
}

namespace {

hipError_t launch_append(const CacheView& c, const float* rot, const void* k, const void* v, int dtype,
                         int n_tokens, const int32_t* seq_idx, const int32_t* pos, int pos0,
                         const int32_t* block_table, int max_pages, hipStream_t stream) {
  const Levels4 lv = c.bits == 4 ? codebook4().lv : Levels4{};
  const long long n_vec = (long long)n_tokens * c.hkv;
  if (2 * n_vec <= kSmallAppendVectors) {
    const unsigned blocks = (unsigned)((2 * n_vec + 7) / 8);
#define IQ_SMALL(DT, B)                                                                          \
  hipLaunchKernelGGL((quantize_small_kernel<DT, B>), dim3(blocks), dim3(256), 0, stream, k, v,   \
                     seq_idx, pos, block_table, rot, (int)n_vec, c.hkv, max_pages,               \
                     c.num_pages, c.k_codes, c.k_norms, c.v_codes, c.v_norms, lv, pos0)
#define IQ_SMALL_B(B)            \
  if (dtype == 0) IQ_SMALL(0, B); \
  else if (dtype == 1) IQ_SMALL(1, B); \
  else IQ_SMALL(2, B)
    if (c.bits == 4) { IQ_SMALL_B(4); }
    else { IQ_SMALL_B(3); }
#undef IQ_SMALL_B
#undef IQ_SMALL
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((n_tokens + 63) / 64), (unsigned)c.hkv, 2);
#define IQ_QUADS(DT, B)                                                                           \
  hipLaunchKernelGGL((quantize_append_kernel<DT, B>), grid, dim3(256), 0, stream, k, v, seq_idx,   \
                     pos, block_table, n_tokens, c.hkv, max_pages, rot, c.num_pages, c.k_codes,     \
                     c.k_norms, c.v_codes, c.v_norms, lv, pos0)
#define IQ_QUADS_B(B)            \
  if (dtype == 0) IQ_QUADS(0, B); \
  else if (dtype == 1) IQ_QUADS(1, B); \
  else IQ_QUADS(2, B)
  if (c.bits == 4) { IQ_QUADS_B(4); }
  else { IQ_QUADS_B(3); }
#undef IQ_QUADS_B
#undef IQ_QUADS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_append(const CacheView& c, const float* rot, const void* k, const void* v,
                                  int dtype, int n_tokens, const int32_t* seq_idx,
                                  const int32_t* pos, const int32_t* block_table, int max_pages,
                                  hipStream_t stream) {
  return launch_append(c, rot, k, v, dtype, n_tokens, seq_idx, pos, 0, block_table, max_pages, stream);
}

hipError_t launch_quantize_append_range(const CacheView& c, const float* rot, const void* k,
                                        const void* v, int dtype, int n_tokens, int pos0,
                                        const int32_t* block_table, int max_pages, hipStream_t stream) {
  return launch_append(c, rot, k, v, dtype, n_tokens, nullptr, nullptr, pos0, block_table, max_pages, stream);
}

}  // namespace iq
