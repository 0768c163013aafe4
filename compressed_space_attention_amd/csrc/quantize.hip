// Quantise-append: K/V head vectors -> 48-byte 3-bit records + fp16 norms in
// a 64-token paged cache.
//
// "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention", abstract: Walsh-Hadamard transform, then
// block-diagonal SO(4) rotations, then 3-bit scalar quantisation.  Per vector
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

__global__ __launch_bounds__(256) void quantize_append_kernel(
    const void* __restrict__ k, const void* __restrict__ v, int dtype, long long n_vec,
    int hkv, const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ block_table, int max_pages, const float* __restrict__ rot,
    uint8_t* __restrict__ k_codes, uint16_t* __restrict__ k_norms, uint8_t* __restrict__ v_codes,
    uint16_t* __restrict__ v_norms) {
  const long long gv = (long long)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int j = threadIdx.x & 3;
  if (gv >= 2 * n_vec) return;  // whole quads leave together
  const int which = gv >= n_vec;
  const long long vi = gv - (which ? n_vec : 0);  // token * hkv + head
  const int tok = (int)(vi / hkv);
  const int head = (int)(vi - (long long)tok * hkv);

  float x[32];
  load32(which ? v : k, (size_t)vi * kD + 32 * j, dtype, x);

  float ss0 = 0.f, ss1 = 0.f, ss2 = 0.f, ss3 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    ss0 = fmaf(x[i], x[i], ss0);
    ss1 = fmaf(x[i + 1], x[i + 1], ss1);
    ss2 = fmaf(x[i + 2], x[i + 2], ss2);
    ss3 = fmaf(x[i + 3], x[i + 3], ss3);
  }
  float ss = (ss0 + ss1) + (ss2 + ss3);
  ss += quad_xor1(ss);
  ss += quad_xor2(ss);
  const float n = sqrtf(ss);

  wht128_quad(x, j);
  float z[32];
  so4_forward_quarter(rot + (size_t)head * kRotFloats, j, x, z);

  uint32_t sel[8];
  if (n > 0.f) {
    const float inv_n = 1.0f / n;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sel[s] = code_of(z[4 * s] * inv_n) | (code_of(z[4 * s + 1] * inv_n) << 8) |
               (code_of(z[4 * s + 2] * inv_n) << 16) | (code_of(z[4 * s + 3] * inv_n) << 24);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) sel[s] = 0x04040404u;  // zero vector: level +0.2451 * 0
  }
  u3 w;
  selectors_to_group(sel, w.x, w.y, w.z);

  const int p = pos[tok];
  const int page = block_table[(size_t)seq_idx[tok] * max_pages + (p >> 6)];
  const int slot = p & 63;
  const size_t rec = ((size_t)page * hkv + head) * kPage + slot;
  if (!which) {
    *reinterpret_cast<u3*>(k_codes + rec * kRec + 12 * j) = w;
    if (j == 0) k_norms[rec] = float_to_half_sat(n);
    return;
  }
  // V: byte lane b of this group goes to region n = 4j + b (quad q of the
  // slot), chunk c = slot / 16, byte lane r = slot % 4 -- the order in which
  // the decode matrix cores consume V (see the cache layout in isoquant.h).
  uint8_t* blk = v_codes + ((size_t)page * hkv + head) * (kPage * kRec);
  const int c = slot >> 4, q = (slot >> 2) & 3, r = slot & 3;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint8_t* dst = blk + (4 * j + b + 16 * q) * kRec + 12 * c + r;
    dst[0] = (uint8_t)(w.x >> (8 * b));
    dst[4] = (uint8_t)(w.y >> (8 * b));
    dst[8] = (uint8_t)(w.z >> (8 * b));
  }
  if (j == 0) v_norms[rec] = float_to_half_sat(n);
}

hipError_t launch_quantize_append(const CacheView& c, const float* rot, const void* k, const void* v,
                                  int dtype, int n_tokens, const int32_t* seq_idx,
                                  const int32_t* pos, const int32_t* block_table, int max_pages,
                                  hipStream_t stream) {
  const long long n_vec = (long long)n_tokens * c.hkv;
  const long long blocks = (2 * n_vec + 63) / 64;
  hipLaunchKernelGGL(quantize_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, v,
                     dtype, n_vec, c.hkv, seq_idx, pos, block_table, max_pages, rot, c.k_codes,
                     c.k_norms, c.v_codes, c.v_norms);
  return hipGetLastError();
}

}  // namespace iq
