// Device helpers shared by the IsoQuant HIP kernels (gfx950, wave64).
//
// Method ("RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention", abstract): normalised Walsh-Hadamard transform,
// then 32 block-diagonal SO(4) rotations, then 3-bit scalar quantisation; the
// attention kernels read the packed codes directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {

constexpr int kD = 128;        // head dimension
constexpr int kPage = 64;      // tokens per page
constexpr int kRec = 48;       // code bytes per vector (3-bit records)
constexpr int kRec4 = 64;      // code bytes per vector (4-bit records)
constexpr int kBlocks = 32;    // SO(4) blocks per head
constexpr int kRotFloats = kBlocks * 16;  // fp32 4x4 matrices per kv head

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

struct __attribute__((aligned(4))) u3 {
  uint32_t x, y, z;
};

// ---------------------------------------------------------------------------
// 3-bit quantiser constants: the Gaussian Lloyd-Max levels that the
// specification of this path fixes (positive half; the pages name 3-bit
// scalar quantisation but print no levels), and the decision thresholds =
// midpoints between adjacent levels, as fp32 (the middle threshold is 0).
// ---------------------------------------------------------------------------
constexpr double kLevel3[4] = {0.2451, 0.7560, 1.3440, 2.1520};
constexpr float kThr3[3] = {0.50055f, 1.05f, 1.748f};
// code = number of the seven thresholds (-t3, -t2, -t1, 0, t1, t2, t3) that u
// reaches (ties reach).  By symmetry it is 4 + m for u >= 0 with m = the
// number of positive thresholds |u| reaches, and 3 - m' = m' ^ 3 for u < 0
// with m' = the number |u| strictly exceeds; |u| > t is tested as a >= t with
// a = the float one ulp below |u| (an integer decrement of the bits).  So one
// magnitude count of three comparisons serves both signs and needs no
// threshold selection.  u + 0 turns -0 into +0 (which codes 4, like +0).  A
// NaN codes 3 or 4 (its vector's norm is NaN then).
__host__ __device__ __forceinline__ uint32_t code_of(float u) {
  const uint32_t b = __builtin_bit_cast(uint32_t, u + 0.0f);
  const uint32_t neg = (uint32_t)((int32_t)b >> 31);  // all ones iff u < 0
  const float a = fabsf(__builtin_bit_cast(float, b + neg));
  const uint32_t m4 = 4u + (uint32_t)(a >= kThr3[0]) + (uint32_t)(a >= kThr3[1]) +
                      (uint32_t)(a >= kThr3[2]);
  return m4 ^ (neg & 7u);  // u < 0: 7 - (4 + m') = 3 - m'
}

// The matrix-core kernels consume the levels as f16 operands.  They carry
// alpha * level with alpha = 1.7670845, chosen so that all four magnitudes
// land within 1.7e-5 (relative) of an f16 value (plain f16 levels are off by
// up to 1.9e-4); 1/alpha is folded into the per-token norm factor.
constexpr float kLevelScale = 1.7670845f;
constexpr uint16_t kLevelF16[8] = {0xC39B, 0xC0C0, 0xBD58, 0xB6EE,   // codes 0..3 (negative)
                                   0x36EE, 0x3D58, 0x40C0, 0x439B};  // codes 4..7
constexpr uint32_t bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return a | (b << 8) | (c << 16) | (d << 24);
}
constexpr uint32_t kLo0123 = bytes4(kLevelF16[0] & 255, kLevelF16[1] & 255, kLevelF16[2] & 255,
                                    kLevelF16[3] & 255);
constexpr uint32_t kLo4567 = bytes4(kLevelF16[4] & 255, kLevelF16[5] & 255, kLevelF16[6] & 255,
                                    kLevelF16[7] & 255);
constexpr uint32_t kHi0123 = bytes4(kLevelF16[0] >> 8, kLevelF16[1] >> 8, kLevelF16[2] >> 8,
                                    kLevelF16[3] >> 8);
constexpr uint32_t kHi4567 = bytes4(kLevelF16[4] >> 8, kLevelF16[5] >> 8, kLevelF16[6] >> 8,
                                    kLevelF16[7] >> 8);

// ---------------------------------------------------------------------------
// Packed record layout.  A 48-byte record is four 12-byte groups (group g =
// coordinates 32g..32g+31), each three little-endian dwords w0, w1, w2.  Byte
// lane b (byte b of w0, w1, w2) is a 24-bit integer holding the codes of
// coordinates 32g + 4s + b at bits 3s..3s+2, s = 0..7.
//
// "Selector" z_s = the four codes of coordinates 4s..4s+3 of the group, one
// per byte: exactly the byte-select operand v_perm_b32 takes, so a selector
// turns into four f16 levels with four v_perm_b32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void group_to_selectors(uint32_t w0, uint32_t w1, uint32_t w2,
                                                   uint32_t z[8]) {
  z[0] = w0 & 0x07070707u;
  z[1] = (w0 >> 3) & 0x07070707u;
  z[2] = ((w0 >> 6) & 0x03030303u) | ((w1 << 2) & 0x04040404u);
  z[3] = (w1 >> 1) & 0x07070707u;
  z[4] = (w1 >> 4) & 0x07070707u;
  z[5] = ((w1 >> 7) & 0x01010101u) | ((w2 << 1) & 0x06060606u);
  z[6] = (w2 >> 2) & 0x07070707u;
  z[7] = (w2 >> 5) & 0x07070707u;
}

__host__ __device__ __forceinline__ void selectors_to_group(const uint32_t z[8], uint32_t& w0,
                                                   uint32_t& w1, uint32_t& w2) {
  w0 = z[0] | (z[1] << 3) | ((z[2] & 0x03030303u) << 6);
  w1 = ((z[2] >> 2) & 0x01010101u) | (z[3] << 1) | (z[4] << 4) | ((z[5] & 0x01010101u) << 7);
  w2 = ((z[5] >> 1) & 0x03030303u) | (z[6] << 2) | (z[7] << 5);
}

// Four codes (one selector) -> four f16 levels (alpha-scaled) in two dwords:
// the first holds coordinates 4s, 4s+1 and the second 4s+2, 4s+3.
__device__ __forceinline__ u2 selector_to_f16(uint32_t z) {
  const uint32_t l = __builtin_amdgcn_perm(kLo4567, kLo0123, z);  // low bytes of 4 levels
  const uint32_t h = __builtin_amdgcn_perm(kHi4567, kHi0123, z);  // high bytes
  return u2{__builtin_amdgcn_perm(h, l, 0x05010400u), __builtin_amdgcn_perm(h, l, 0x07030602u)};
}

// ---------------------------------------------------------------------------
// 4-bit records (the 4-bit member of the same family: 16 Gaussian Lloyd-Max
// levels, symmetric about 0).  A stored nibble is sign-magnitude: bit 3 marks
// the negative side, bits 0-2 index the magnitude (0 = smallest); code c of
// the 15-threshold quantiser (c = number of thresholds u reaches, 0..15) is
// stored as c - 8 for c >= 8 and 15 - c below.  A 64-byte record: dword d holds
// coordinates 8d..8d+7, byte b of it coordinate 8d+b in its low nibble and
// 8d+4+b in its high one.
//
// The host computes the codebook (Lloyd's iteration) and passes it to the
// kernels as this struct: the seven positive thresholds (the negative ones
// mirror them exactly) and v_perm_b32 tables of the f16 bytes of alpha times
// the eight magnitudes.
// ---------------------------------------------------------------------------
struct Levels4 {
  float t[7];                                // positive decision thresholds, ascending
  uint32_t lo0123, lo4567, hi0123, hi4567;   // f16 low / high bytes of alpha * magnitude k
};

// Nibble of u.  Nonnegative u (including -0): the magnitudes whose lower
// threshold it reaches; negative u: 8 + the thresholds |u| exceeds (a tie
// belongs to the upper code on either side).  "|u| > t" is "x >= t" for x the
// float just below |u| (|u| > 0 there), so one binary search over the seven
// ascending thresholds (three comparisons) serves both sides.
__host__ __device__ __forceinline__ uint32_t nibble_of(float u, const Levels4& lv) {
  const bool neg = !(u >= 0.0f);
  const float a = fabsf(u);
  const float x = neg ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) - 1u) : a;
  const bool b2 = x >= lv.t[3];
  const bool b1 = x >= (b2 ? lv.t[5] : lv.t[1]);
  const float t0 = b2 ? (b1 ? lv.t[6] : lv.t[4]) : (b1 ? lv.t[2] : lv.t[0]);
  const bool b0 = x >= t0;
  return (neg ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

// Four nibbles (one per byte, bits 0-3) -> four f16 levels (alpha-scaled) in
// two dwords, ordered like the bytes.
__device__ __forceinline__ u2 nibbles_to_f16(uint32_t z, const Levels4& lv) {
  const uint32_t k = z & 0x07070707u;
  const uint32_t l = __builtin_amdgcn_perm(lv.lo4567, lv.lo0123, k);
  const uint32_t h = __builtin_amdgcn_perm(lv.hi4567, lv.hi0123, k) | ((z << 4) & 0x80808080u);
  return u2{__builtin_amdgcn_perm(h, l, 0x05010400u), __builtin_amdgcn_perm(h, l, 0x07030602u)};
}

// The eight f16 levels of one record dword (coordinates 8d..8d+7 in order).
__device__ __forceinline__ h8 dword4_to_h8(uint32_t w, const Levels4& lv) {
  const u2 a = nibbles_to_f16(w & 0x0F0F0F0Fu, lv), b = nibbles_to_f16((w >> 4) & 0x0F0F0F0Fu, lv);
  return __builtin_bit_cast(h8, u4{a[0], a[1], b[0], b[1]});
}

// ---------------------------------------------------------------------------
// Small numeric helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fp32 -> fp16 bits, round to nearest even, saturating finite values at 65504.
__device__ __forceinline__ uint16_t float_to_half_sat(float x) {
  _Float16 h = (_Float16)x;
  uint16_t b = __builtin_bit_cast(uint16_t, h);
  if ((b & 0x7FFFu) == 0x7C00u) b = (b & 0x8000u) | 0x7BFFu;
  return b;
}

// load32 in two halves, so that a load can be issued well before its data is
// needed: the raw 16-byte chunks (8 for fp32, 4 for the 16-bit types), then
// their conversion.
__device__ __forceinline__ void load32_raw(const void* base, size_t idx, int dtype, u4 r[8]) {
  if (dtype == 0) {
    const u4* p = reinterpret_cast<const u4*>(reinterpret_cast<const float*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = p[i];
  } else {
    const u4* p = reinterpret_cast<const u4*>(reinterpret_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = p[i];
  }
}
__device__ __forceinline__ void raw_to_f32(const u4 r[8], int dtype, float x[32]) {
  if (dtype == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * i + k] = __builtin_bit_cast(float, (uint32_t)r[i][k]);  // rvalue: see the note on bit casts
  } else if (dtype == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * i + 2 * k] = __builtin_bit_cast(float, r[i][k] << 16);
        x[8 * i + 2 * k + 1] = __builtin_bit_cast(float, r[i][k] & 0xFFFF0000u);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * i + 2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r[i][k] & 0xFFFFu));
        x[8 * i + 2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(r[i][k] >> 16));
      }
  }
}

// Load 32 consecutive elements (128-bit aligned) as fp32.
__device__ __forceinline__ void load32(const void* base, size_t idx, int dtype, float x[32]) {
  u4 r[8];
  load32_raw(base, idx, dtype, r);
  raw_to_f32(r, dtype, x);
}

// 2^x on the transcendental unit (v_exp_f32).  Results below 2^-126 flush to
// zero, which is harmless for softmax weights relative to a running maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest of the eight non-negative fp16 values held in two u2 pairs, as
// fp16 bits (non-negative fp16 bit patterns order like the values).
typedef uint16_t us2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t max_half_bits(const u2& a, const u2& b) {
  const us2 m0 = __builtin_elementwise_max(__builtin_bit_cast(us2, (uint32_t)a[0]),
                                            __builtin_bit_cast(us2, (uint32_t)a[1]));
  const us2 m1 = __builtin_elementwise_max(__builtin_bit_cast(us2, (uint32_t)b[0]),
                                            __builtin_bit_cast(us2, (uint32_t)b[1]));
  const us2 m = __builtin_elementwise_max(m0, m1);
  return m[0] > m[1] ? m[0] : m[1];
}

// ---------------------------------------------------------------------------
// Lane exchanges inside a quad of lanes, on the DPP path (full-rate VALU, no
// LDS crossbar): xor 1 = quad_perm [1,0,3,2], xor 2 = quad_perm [2,3,0,1].
// ---------------------------------------------------------------------------
template <int QUAD_PERM>
__device__ __forceinline__ float quad_swap(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), QUAD_PERM,
                                                            0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor1(float v) { return quad_swap<0xB1>(v); }
__device__ __forceinline__ float quad_xor2(float v) { return quad_swap<0x4E>(v); }

// Exchanges across rows (16 lanes) and halves (32 lanes) with the gfx950
// permlane swaps: with both operands equal to v, lane l of the two results
// holds v[l] and v[l ^ 16] (resp. v[l ^ 32]) in some order, so any
// symmetric combination of the pair is a butterfly reduction step.
//
// Note on bit casts: clang lowers __builtin_bit_cast of an ext_vector element
// lvalue (v[1], v.y) as a load from the vector's first element, so every bit
// cast here and elsewhere takes a converted rvalue ((uint32_t)v[1]).
__device__ __forceinline__ u2 pair_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return u2{(uint32_t)r[0], (uint32_t)r[1]};
}
__device__ __forceinline__ u2 pair_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return u2{(uint32_t)r[0], (uint32_t)r[1]};
}
__device__ __forceinline__ float max_xor16(float v) {
  const u2 p = pair_xor16(__builtin_bit_cast(uint32_t, v));
  return fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const u2 p = pair_xor32(__builtin_bit_cast(uint32_t, v));
  return fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const u2 p = pair_xor16(__builtin_bit_cast(uint32_t, v));
  return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const u2 p = pair_xor32(__builtin_bit_cast(uint32_t, v));
  return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}
__device__ __forceinline__ uint32_t umax_xor16(uint32_t v) {
  const u2 p = pair_xor16(v);
  return max(p[0], p[1]);
}
__device__ __forceinline__ uint32_t umax_xor32(uint32_t v) {
  const u2 p = pair_xor32(v);
  return max(p[0], p[1]);
}

// Exchanges with lane ^ 4 and lane ^ 8 inside rows of 16 (DPP row shifts /
// rotation), and bitwise-or / sum reductions over them.
__device__ __forceinline__ float lane_xor4_f(float v) {
  const int iv = __builtin_bit_cast(int, v);
  const int t = __builtin_amdgcn_update_dpp(iv, iv, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0, 2
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(t, iv, 0x114, 0xF, 0xA, false));
}
__device__ __forceinline__ float lane_xor8_f(float v) {
  const int iv = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(iv, iv, 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float add_xor4(float v) { return v + lane_xor4_f(v); }
__device__ __forceinline__ uint32_t or_xor1(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t or_xor2(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t or_xor4(uint32_t v) {
  return v | __builtin_bit_cast(uint32_t, lane_xor4_f(__builtin_bit_cast(float, v)));
}

// ---------------------------------------------------------------------------
// Rotate one 128-vector held by the 32 lanes of a half-wave: lane r holds
// coordinates 4r..4r+3 (x0..x3) and the rows m0..m3 of SO(4) block r.
// n = ||x|| (every lane); z0..z3 = coordinates 4r..4r+3 of B H x.  The
// Walsh-Hadamard butterflies at coordinate distance 1 and 2 are in registers,
// 4..64 are lane exchanges 1..16; u = (B H x) / n with H unnormalised equals
// T x sqrt(d) / n.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rotate_lanes32(float x0, float x1, float x2, float x3,
                                               const f4& m0, const f4& m1, const f4& m2,
                                               const f4& m3, int r, float& n, float& z0, float& z1,
                                               float& z2, float& z3) {
  float ss = fmaf(x3, x3, fmaf(x2, x2, fmaf(x1, x1, x0 * x0)));
  ss += quad_xor1(ss);
  ss += quad_xor2(ss);
  ss = add_xor4(ss);
  ss += lane_xor8_f(ss);
  ss = sum_xor16(ss);
  n = sqrtf(ss);
  {
    const float a0 = x0 + x1, a1 = x0 - x1, a2 = x2 + x3, a3 = x2 - x3;
    x0 = a0 + a2; x2 = a0 - a2; x1 = a1 + a3; x3 = a1 - a3;
  }
  // lower lane keeps y + partner, upper lane partner - y
  float sg = (r & 1) ? -1.0f : 1.0f;
  x0 = fmaf(sg, x0, quad_xor1(x0)); x1 = fmaf(sg, x1, quad_xor1(x1));
  x2 = fmaf(sg, x2, quad_xor1(x2)); x3 = fmaf(sg, x3, quad_xor1(x3));
  sg = (r & 2) ? -1.0f : 1.0f;
  x0 = fmaf(sg, x0, quad_xor2(x0)); x1 = fmaf(sg, x1, quad_xor2(x1));
  x2 = fmaf(sg, x2, quad_xor2(x2)); x3 = fmaf(sg, x3, quad_xor2(x3));
  sg = (r & 4) ? -1.0f : 1.0f;
  x0 = fmaf(sg, x0, lane_xor4_f(x0)); x1 = fmaf(sg, x1, lane_xor4_f(x1));
  x2 = fmaf(sg, x2, lane_xor4_f(x2)); x3 = fmaf(sg, x3, lane_xor4_f(x3));
  sg = (r & 8) ? -1.0f : 1.0f;
  x0 = fmaf(sg, x0, lane_xor8_f(x0)); x1 = fmaf(sg, x1, lane_xor8_f(x1));
  x2 = fmaf(sg, x2, lane_xor8_f(x2)); x3 = fmaf(sg, x3, lane_xor8_f(x3));
  {
    // swap pair (A, B) = (own, partner) on the lower row, (partner, own) on
    // the upper one: the butterfly is A + (+-1) B on both
    sg = (r & 16) ? -1.0f : 1.0f;
    u2 q;
    q = pair_xor16(__builtin_bit_cast(uint32_t, x0));
    x0 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)q[1]), __builtin_bit_cast(float, (uint32_t)q[0]));
    q = pair_xor16(__builtin_bit_cast(uint32_t, x1));
    x1 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)q[1]), __builtin_bit_cast(float, (uint32_t)q[0]));
    q = pair_xor16(__builtin_bit_cast(uint32_t, x2));
    x2 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)q[1]), __builtin_bit_cast(float, (uint32_t)q[0]));
    q = pair_xor16(__builtin_bit_cast(uint32_t, x3));
    x3 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)q[1]), __builtin_bit_cast(float, (uint32_t)q[0]));
  }
  z0 = m0[0] * x0 + m0[1] * x1 + m0[2] * x2 + m0[3] * x3;
  z1 = m1[0] * x0 + m1[1] * x1 + m1[2] * x2 + m1[3] * x3;
  z2 = m2[0] * x0 + m2[1] * x1 + m2[2] * x2 + m2[3] * x3;
  z3 = m3[0] * x0 + m3[1] * x1 + m3[2] * x2 + m3[3] * x3;
}

// 3-bit record of rotate_lanes32's vector: w = the three dwords of group r/8
// of the packed record (every lane of the group).
// The bit fields of selector s (four codes, one per byte) in a group's three
// dwords: the codes of selector s sit at bits 3s .. 3s+2 of each byte lane's
// 24-bit field, whose bytes are dword k's bytes (k = 0, 1, 2), so dword k
// gets the codes shifted by 3s - 8k, kept to the bits of their own bytes.
// OR-ing the fields of selectors 0..7 gives selectors_to_group.
template <bool SHIFTS>
__host__ __device__ __forceinline__ void selector_fields(int s, uint32_t sel, uint32_t& w0, uint32_t& w1,
                                                         uint32_t& w2) {
  if constexpr (SHIFTS) {
    auto field = [&](int k) {
      // sel shifted left by 3s - 8k (right where negative): one 64-bit shift
      const uint32_t part = (uint32_t)(((uint64_t)sel << 32) >> (32 - 3 * s + 8 * k));
      const uint32_t m = ((0x07u << (3 * s)) >> (8 * k)) & 0xFFu;
      return part & (m * 0x01010101u);
    };
    w0 = field(0);
    w1 = field(1);
    w2 = field(2);
  } else {
    w0 = w1 = w2 = 0;
    switch (s) {
      case 0: w0 = sel; break;
      case 1: w0 = sel << 3; break;
      case 2: w0 = (sel & 0x03030303u) << 6; w1 = (sel >> 2) & 0x01010101u; break;
      case 3: w1 = sel << 1; break;
      case 4: w1 = sel << 4; break;
      case 5: w1 = (sel & 0x01010101u) << 7; w2 = (sel >> 1) & 0x03030303u; break;
      case 6: w2 = sel << 2; break;
      default: w2 = sel << 5; break;
    }
  }
}

// SHIFTS: place the selector's fields with lane-dependent shifts and masks
// (no branches; measured faster inside the decode step) instead of a switch
// over the selector index (measured faster in the standalone one-token
// append, where the compiler overlaps it with the page-id load).  Both give
// the same dwords.
template <bool SHIFTS>
__device__ __forceinline__ void quantize_lanes32(float x0, float x1, float x2, float x3,
                                                 const f4& m0, const f4& m1, const f4& m2,
                                                 const f4& m3, int r, float& n, u3& w) {
  float z0, z1, z2, z3;
  rotate_lanes32(x0, x1, x2, x3, m0, m1, m2, m3, r, n, z0, z1, z2, z3);
  uint32_t sel = 0x04040404u;  // zero vector: every code 4
  if (n > 0.f) {
    const float inv_n = 1.0f / n;
    sel = code_of(z0 * inv_n) | (code_of(z1 * inv_n) << 8) | (code_of(z2 * inv_n) << 16) |
          (code_of(z3 * inv_n) << 24);
  }
  // selector s of group g: its bit fields in the group's three dwords
  uint32_t w0, w1, w2;
  selector_fields<SHIFTS>(r & 7, sel, w0, w1, w2);
  w.x = or_xor4(or_xor2(or_xor1(w0)));
  w.y = or_xor4(or_xor2(or_xor1(w1)));
  w.z = or_xor4(or_xor2(or_xor1(w2)));
}

// Store the record of quantize_lanes32 into one (page, kv head) block:
// `codes` = its 3,072 code bytes, `norms` = its 64 fp16 norms.  K blocks are
// slot-ordered (lane 8g writes group g); V blocks are in the matrix-core
// order of the decode kernels: byte lane b of group g goes to region 4g + b
// of quad (slot / 4) % 4, chunk slot / 16, byte lane slot % 4 (lane 8g + b
// writes it).  Works for global and LDS destinations alike.
__device__ __forceinline__ void place_record(bool is_v, int r, const u3& w, float n, uint8_t* codes,
                                             uint16_t* norms, int slot) {
  const int s = r & 7, g = r >> 3;
  if (!is_v) {
    if (s == 0) *reinterpret_cast<u3*>(codes + slot * kRec + 12 * g) = w;
  } else if (s < 4) {
    const int c = slot >> 4, q = (slot >> 2) & 3, rr = slot & 3;
    uint8_t* dst = codes + (4 * g + s + 16 * q) * kRec + 12 * c + rr;
    dst[0] = (uint8_t)(w.x >> (8 * s));
    dst[4] = (uint8_t)(w.y >> (8 * s));
    dst[8] = (uint8_t)(w.z >> (8 * s));
  }
  if (r == 0) norms[slot] = float_to_half_sat(n);
}

// 4-bit record of rotate_lanes32's vector.  Returns the dword this lane
// stores: for K (is_v false) lane r = 2d holds record dword d (its own four
// nibbles low, lane 2d+1's high); for V lane r = 8a + p (p < 4) holds the
// four V-block bytes of coordinates c = 32a + 4p + b (low nibble) and c + 16
// (high nibble, from lane r + 4).  Every lane of the half-wave must call it.
__device__ __forceinline__ uint32_t quantize_lanes32_4(float x0, float x1, float x2, float x3,
                                                       const f4& m0, const f4& m1, const f4& m2,
                                                       const f4& m3, int r, bool is_v,
                                                       const Levels4& lv, float& n) {
  float z0, z1, z2, z3;
  rotate_lanes32(x0, x1, x2, x3, m0, m1, m2, m3, r, n, z0, z1, z2, z3);
  uint32_t sel = 0;  // zero vector: every nibble 0 (code 8, level +0.128 * 0)
  if (n > 0.f) {
    const float inv_n = 1.0f / n;
    sel = nibble_of(z0 * inv_n, lv) | (nibble_of(z1 * inv_n, lv) << 8) |
          (nibble_of(z2 * inv_n, lv) << 16) | (nibble_of(z3 * inv_n, lv) << 24);
  }
  const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sel, 0xB1, 0xF, 0xF, true);
  const uint32_t p4 = __builtin_bit_cast(uint32_t, lane_xor4_f(__builtin_bit_cast(float, sel)));
  return sel | ((is_v ? p4 : p1) << 4);
}

// Store the 4-bit record of quantize_lanes32_4 (w = its return value) into one
// (page, kv head) block: `codes` = its 4,096 code bytes, `norms` = its 64 fp16
// norms.  K blocks are slot-ordered; V blocks are in the matrix-core order of
// the decode kernels: the byte of (slot, coordinates c, c + 16), c = 32a + 4p
// + b, is byte slot % 4 of dword 4p + 2 th + q of region (4a + b) + 16 jq, for
// slot = 32 th + 16 q + 4 jq + slot % 4.  Global and LDS destinations alike.
__device__ __forceinline__ void place_record4(bool is_v, int r, uint32_t w, float n, uint8_t* codes,
                                              uint16_t* norms, int slot) {
  if (!is_v) {
    if ((r & 1) == 0) *reinterpret_cast<uint32_t*>(codes + slot * kRec4 + 2 * r) = w;
  } else if ((r & 4) == 0) {
    const int a = r >> 3, p = r & 3;
    const int th = slot >> 5, q = (slot >> 4) & 1, jq = (slot >> 2) & 3, rr = slot & 3;
    uint8_t* dst = codes + (4 * a + 16 * jq) * 64 + 4 * (4 * p + 2 * th + q) + rr;
#pragma unroll
    for (int b = 0; b < 4; ++b) dst[64 * b] = (uint8_t)(w >> (8 * b));
  }
  if (r == 0) norms[slot] = float_to_half_sat(n);
}

// x[k] += s * (x[k] of the quad partner), k = 0..7, partner = lane ^ 1
// (QUAD_PERM 0xB1) or lane ^ 2 (0x4E): one v_fmac_f32 with the partner's value
// taken through DPP per element (the compiler keeps a separate DPP move for
// this multiply-add form).  A VALU write followed by a DPP read of the same
// register needs two wait states, which the compiler does not insert around
// inline asm (it does not count the block's outputs as vector-ALU writes):
// hence an s_nop before the block (for the writes that precede it) and one
// after it (for a DPP read of its outputs that may follow); within the block
// no element is read after the block has written it.  Partner lanes outside
// EXEC read as 0 (bound_ctrl), as with the DPP moves elsewhere.
template <int QUAD_PERM>
__device__ __forceinline__ void fmac_quad_xor8(float* x, float s) {
  static_assert(QUAD_PERM == 0xB1 || QUAD_PERM == 0x4E, "quad exchange");
  if constexpr (QUAD_PERM == 0xB1) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1"
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
          "+v"(x[7])
        : "v"(s));
  } else {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
        "s_nop 1"
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
          "+v"(x[7])
        : "v"(s));
  }
}

// ---------------------------------------------------------------------------
// Unnormalised Walsh-Hadamard transform (Sylvester order) of a 128-vector held
// by the four lanes of a quad, 32 consecutive coordinates each: lane quarter
// j = lane % 4 holds coordinates 32j..32j+31.  Coordinate distances 1..16 are
// in-register butterflies; 32 and 64 are DPP exchanges within the quad.
//
// Returns sigma = +-1 and leaves x = sigma * (H x) on the lane.  A cross-lane
// butterfly step is x' = s x + p (p = the partner's value, s = -1 on the upper
// lane of the pair); each lane computes t = x + s p instead, one fused
// multiply-add with the partner's value taken through DPP, and carries the
// factor: x' = s t exactly, since round-to-nearest is symmetric in sign.  The
// partner two lanes away carries the same first factor s1, so the second step
// leaves t' = t + s2 t_partner with x'' = s1 s2 t'.  Callers fold sigma = s1 s2
// into a later scale factor.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wht128_quad(float x[32], int j) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  const float s1 = (j & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 8) fmac_quad_xor8<0xB1>(x + i, s1);
  const float s2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 8) fmac_quad_xor8<0x4E>(x + i, s2);
  return s1 * s2;
}

// The same transform with the quarters on lanes l, l^XOR_A (j^1) and
// l^XOR_B (j^2) of a wave (generic lane exchange; used where the quarters of
// a vector must sit 16 lanes apart).
template <int XOR_A, int XOR_B>
__device__ __forceinline__ void wht128_spread(float x[32], int j) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  const float s1 = (j & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fmaf(s1, x[i], __shfl_xor(x[i], XOR_A));
  const float s2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fmaf(s2, x[i], __shfl_xor(x[i], XOR_B));
}

// z = M_b y for the 8 blocks of quarter j (blocks 8j..8j+7); rot = one kv
// head's [32][4][4] row-major fp32 matrices.
__device__ __forceinline__ void so4_forward_quarter(const float* __restrict__ rot, int j,
                                                    const float y[32], float z[32]) {
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) {
    const f4* m = reinterpret_cast<const f4*>(rot + (8 * j + bb) * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f4 row = m[r];
      z[4 * bb + r] = row[0] * y[4 * bb] + row[1] * y[4 * bb + 1] + row[2] * y[4 * bb + 2] +
                      row[3] * y[4 * bb + 3];
    }
  }
}

// One vector held by a quad of lanes (lane quarter j = coordinates 32j ..
// 32j + 31 in x): its norm (returned) and codes.  sel[bb] holds the codes
// (3-bit) or nibbles (4-bit) of coordinates 32j + 4bb .. + 3, one per byte;
// s_rot is the kv head's rotation blocks in LDS.  The quantise-append kernel
// and the fused append of the chunked prefill both code vectors through this
// one function, so their records are byte-identical.
template <int BITS>
__device__ __forceinline__ float quad_codes(float x[32], int j, const float* s_rot, const Levels4& lv,
                                            uint32_t sel[8]) {
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

  // x = sigma * (H x): the rotated coordinates below carry sigma too, which
  // inv_n takes back (an exact sign change)
  const float sigma = wht128_quad(x, j);
  // SO(4) block by block (blocks 8j .. 8j + 7 of the quarter), each block's
  // four outputs turned into codes at once: sel[bb] holds the codes (3-bit)
  // or nibbles (4-bit) of coordinates 32j + 4bb .. + 3, one per byte.  The
  // zero vector is coded through inv_n = 0: every u is then +-0, which codes
  // as 4 (resp. nibble 0 = code 8), so no coordinate needs a branch.  The
  // empty asm makes each block's rotation rows (LDS) depend on the previous
  // block's codes: otherwise the compiler reads all 32 rows up front and holds
  // 128 of them in registers (204 VGPRs instead of 62, a third of the waves).
  {
    const float inv_n = sigma * (n > 0.f ? 1.0f / n : 0.f);
    uint32_t prev = 0;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      int off = (8 * j + bb) * 16;
      asm volatile("" : "+v"(off) : "v"(prev));
      const f4* m = reinterpret_cast<const f4*>(s_rot + off);
      uint32_t w = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f4 row = m[r];
        const float zr = row[0] * x[4 * bb] + row[1] * x[4 * bb + 1] + row[2] * x[4 * bb + 2] +
                         row[3] * x[4 * bb + 3];
        uint32_t c;
        if constexpr (BITS == 3) c = code_of(zr * inv_n);
        else c = nibble_of(zr * inv_n, lv);
        w |= c << (8 * r);
      }
      sel[bb] = w;
      prev = w;
    }
  }

  return n;
}


// Stores of the quantisers: plain ones, and device-scope ones (complete where
// every XCD sees them, not in this XCD's L2) for records that workgroups of
// the same launch on other XCDs read.  Vector stores only.
struct PlainStore {
  static __device__ __forceinline__ void b8(uint8_t* p, uint32_t v) { *p = (uint8_t)v; }
  static __device__ __forceinline__ void b16(uint16_t* p, uint32_t v) { *p = (uint16_t)v; }
  static __device__ __forceinline__ void b96(uint8_t* p, const u3& w) { *reinterpret_cast<u3*>(p) = w; }
  static __device__ __forceinline__ void b128(uint8_t* p, const u4& w) { *reinterpret_cast<u4*>(p) = w; }
};
typedef uint32_t u3v __attribute__((ext_vector_type(3)));
struct DeviceStore {
  static __device__ __forceinline__ void b8(uint8_t* p, uint32_t v) {
    asm volatile("global_store_byte %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
  }
  static __device__ __forceinline__ void b16(uint16_t* p, uint32_t v) {
    asm volatile("global_store_short %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
  }
  static __device__ __forceinline__ void b96(uint8_t* p, const u3& w) {
    const u3v v = {w.x, w.y, w.z};
    asm volatile("global_store_dwordx3 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
  }
  static __device__ __forceinline__ void b128(uint8_t* p, const u4& w) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(w) : "memory");
  }
};

// The record of quad_codes' vector in `slot` of a (page, kv head) block:
// codes = the block's code bytes, norms = its 64 fp16 norms.  K records are
// slot-ordered; V bytes go to the matrix-core order of the decode kernels
// (see the cache layout in isoquant.h).  whole: the workgroup's 256 threads
// (64 quads) hold the page's 64 slots in order, so the V block is assembled in
// s_v (LDS) and written out as one contiguous run after a workgroup barrier
// (every thread of the workgroup must call this then); otherwise each quad
// stores its own bytes.  stored = false: nothing is written (the vector's
// position or page lies outside the table or the cache).  t = the thread's
// index in the workgroup.
// UNIFORM_BARRIER: the barrier of a V record is taken whether or not the page
// is whole (for callers whose workgroup halves code different blocks).
template <int BITS, class S, bool UNIFORM_BARRIER = false>
__device__ __forceinline__ void quad_store(bool is_v, bool stored, bool whole, int j, int slot,
                                           const uint32_t sel[8], float n, uint8_t* codes,
                                           uint16_t* norms, uint8_t* s_v, int t) {
  constexpr int kRecB = BITS == 4 ? kRec4 : kRec;
  if constexpr (BITS == 3) {
    u3 w;
    selectors_to_group(sel, w.x, w.y, w.z);
    if (!is_v) {
      if (stored) S::b96(codes + slot * kRec + 12 * j, w);
    } else if (stored) {
      // byte lane b of this group goes to region n = 4j + b (quad q of the
      // slot), chunk c = slot / 16, byte lane r = slot % 4
      const int c = slot >> 4, q = (slot >> 2) & 3, r = slot & 3;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int off = (4 * j + b + 16 * q) * kRec + 12 * c + r;
        const uint32_t b0 = (w.x >> (8 * b)) & 0xFF, b1 = (w.y >> (8 * b)) & 0xFF, b2 = (w.z >> (8 * b)) & 0xFF;
        if (whole) {
          s_v[off] = (uint8_t)b0; s_v[off + 4] = (uint8_t)b1; s_v[off + 8] = (uint8_t)b2;
        } else {
          S::b8(codes + off, b0); S::b8(codes + off + 4, b1); S::b8(codes + off + 8, b2);
        }
      }
    }
  } else {
    if (!is_v) {
      // record dword 4j + kk: byte b = coordinate 32j + 8kk + b (low nibble,
      // selector 2kk) and 32j + 8kk + 4 + b (high nibble, selector 2kk + 1)
      u4 w;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) w[kk] = sel[2 * kk] | (sel[2 * kk + 1] << 4);
      if (stored) S::b128(codes + slot * kRec4 + 16 * j, w);
    } else if (stored) {
      // coordinates 32j + 4p + b (selector p) and + 16 (selector p + 4) share
      // byte slot % 4 of dword 4p + 2 th + q of region (4j + b) + 16 jq
      // (slot = 32 th + 16 q + 4 jq + r)
      const int th = slot >> 5, q = (slot >> 4) & 1, jq = (slot >> 2) & 3, r = slot & 3;
      const int base = (4 * j + 16 * jq) * 64 + 4 * (2 * th + q) + r;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint32_t v = sel[pp] | (sel[pp + 4] << 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int off = base + 64 * b + 16 * pp;
          if (whole) s_v[off] = (uint8_t)(v >> (8 * b));
          else S::b8(codes + off, (v >> (8 * b)) & 0xFF);
        }
      }
    }
  }
  if (stored && j == 0) S::b16(norms + slot, float_to_half_sat(n));
  if (is_v && (whole || UNIFORM_BARRIER)) {
    __syncthreads();
    constexpr int kChunks = kPage * kRecB / 16;
    if (whole && t < kChunks) S::b128(codes + 16 * t, reinterpret_cast<const u4*>(s_v)[t]);
  }
}

}  // namespace iq
