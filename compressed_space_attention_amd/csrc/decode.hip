// Decode attention directly on the packed 3-bit cache.
//
// "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention", abstract: attention runs on packed 3-bit
// tensors without materialising full-precision K/V.  The query is rotated into
// the cache's orthogonal space (q' = T q), scores and the value accumulator
// stay in that space, and the accumulator is rotated back once (T^T) after the
// split merge.  The context is split across workgroups by length and CU count
// (FreeToken v0.2.0 release notes, Kernels #729); a split whose chunk starts
// at -inf must not produce NaN (#654).
//
// Work decomposition (gfx950, wave64):
//   grid = (splits, kv heads, sequences), 256 threads = 4 waves.  A split is a
//   range of 64-token pages; wave w takes pages w, w+4, ... of its split and
//   keeps its own online-softmax state; the four states merge through LDS and
//   one partial (m, l, acc[128]) per query head is written to the workspace.
//   A second kernel merges the partials of all splits and applies T^T.
//
// Per page and wave, the G query heads of the group are the columns of 16x16
// matrix-core tiles (zero queries pad the group to 16 columns):
//   S^T[token][head] = K^[token][:] . Q'[head][:]   v_mfma_f32_16x16x32_f16, with
//       Q' split into an f16 high and low part (two MFMAs, ~2^-22 relative);
//       lane l's K operand is token l%16 and its coordinates come straight from
//       one 12-byte group of the token's record.
//   O'^T[dim][head] += V^T[dim][token] . P~^T[token][head]   (16x16x32); the V
//       pages are stored so that lane l's 48-byte region is exactly its V
//       operand for the page, so no transpose is needed.
// With G <= 8 the score MFMA's columns 8-15 carry the low part of Q' (one
// MFMA per k-step instead of two), and two 16-token score tiles then share
// one set of registers (columns 0-7 and 8-15, each the sum of a column and
// its partner eight lanes round), which halves the softmax work; the shared
// layout is also the B operand of the PV product after one row shift.
// 4-bit records (BITS = 4) use the same tiles: a record dword is eight
// coordinates of the score operand, and a V region dword eight tokens' nibbles
// of one coordinate pair (c, c + 16), i.e. accumulator tiles m and m + 4.
// Levels enter as alpha-scaled f16 (see iq_device.h); the key norm, 1/alpha,
// the softmax scale and log2(e) are one fp32 factor per score.  The value
// norm is folded into P~ relative to a per-page power-of-two frame so that P~
// stays inside the f16 range for any norm.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

struct DecodeArgs {
  uint8_t* k_codes;  // written only by a decode step (the appended token's record)
  uint16_t* k_norms;
  uint8_t* v_codes;
  uint16_t* v_norms;
  const uint8_t* k_new;  // decode step: the current token's K and V rows [B][Hkv][128]
  const uint8_t* v_new;
  int kv_dtype;
  int num_pages, hkv;
  int q_dtype;
  int hq, group;
  int max_pages;
  int pages_per_split, splits;
  float score_factor;  // softmax_scale * log2(e) / (128 * alpha)
  float out_factor;    // 1 / (sqrt(128) * alpha)
  Levels4 lv4;         // 4-bit records: thresholds and f16 level tables
  float* ws_acc;       // [B][Hq][splits][128]
  float* ws_ml;        // [B][Hq][splits][2]
  float* out;          // [B][Hq][128]
  // Balanced plan (several sequences): the plan's workgroup count, the batch,
  // and each sequence's split count, written for the merge.
  int plan_wgs, batch;
  int32_t* n_splits;
  // Merge workgroups in the split launch (host plan, the whole grid resident
  // at once): a flat grid of split_wgs split workgroups, then one merge
  // workgroup per query head.  A split workgroup counts itself in
  // arrive[b * hkv + g] once its partial rows are visible device-wide; the
  // merge workgroups of (b, g) wait for every non-empty split, merge, and the
  // last of them to finish counts itself in done[] and clears both counters.
  // Null: a merge kernel follows the split launch.
  uint32_t* arrive;
  uint32_t* done;
  int split_wgs;
  int deterministic;  // each wave takes pages w, w + W, ... of its split (no claiming)
};

// DPP controls (gfx9): shifts and rotation inside rows of 16 lanes.
constexpr int kRowShl8 = 0x108, kRowShr8 = 0x118, kRowRor8 = 0x128;

template <int CTRL, int BANK_MASK>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, BANK_MASK, false);
}
template <int CTRL, int BANK_MASK>
__device__ __forceinline__ float dpp_f(float old, float src) {
  return __builtin_bit_cast(float, dpp_u<CTRL, BANK_MASK>(__builtin_bit_cast(uint32_t, old),
                                                          __builtin_bit_cast(uint32_t, src)));
}

// Score tiles held by one lane: with PACK8 (G <= 8) tile t covers token block
// 2t + (lane%16 >= 8); otherwise tile t is token block t.
template <bool PACK8, int BITS>
struct PageRegs {
  static constexpr int NT = PACK8 ? 2 : 4;
  // K: the code bytes of coordinates 32*(lane/16) .. +31 of token 16*rb + lane%16
  // (12 of a 3-bit record, 16 of a 4-bit one)
  using KRec = typename std::conditional<BITS == 3, u3, u4>::type;
  KRec kc[4];
  u4 vr[BITS];    // V: the lane's 48- or 64-byte region
  u2 kn[NT], vn[NT];  // fp16 norms of the lane's four score tokens per tile
};

template <bool PACK8>
__device__ __forceinline__ int tile_block(int t, int col) {
  return PACK8 ? 2 * t + (col >> 3) : t;
}

// ---- LDS page ring -------------------------------------------------------
// Each wave streams its pages through two LDS slots, each the packed page of
// one kv head: K codes | V codes | K norms 128 | V norms 128 (3-bit: 6,400
// bytes, 4-bit: 8,448), filled by direct global->LDS loads of 1 KiB (K and V)
// and one of the norms.  Two pages are in flight while the wave computes a
// third from registers.
template <int BITS>
struct PageFmt {
  static constexpr int kRecBytes = BITS == 4 ? kRec4 : kRec;  // code bytes per vector
  static constexpr int kBlockBytes = kPage * kRecBytes;          // codes of one (page, kv head)
  static constexpr int kSlotBytes = 2 * kBlockBytes + 256;
  static constexpr int kDmaPerPage = 2 * kBlockBytes / 1024 + 1;
};
constexpr int kMaxPagesPerSplit = 512;   // the planner keeps splits within this (64 per wave)
#define IQ_MAX_GROUP_BYTES (16 * 128 * 4)  // up to 16 query heads of fp32

// The direct-to-LDS loads are issued from inline asm, so the compiler does
// not track them: it cannot tell which ring slot a load writes, and would put
// a wait for every outstanding load before each LDS read of a page (turning
// the two-slot ring into a one-slot one).  Every read of loaded LDS data is
// preceded by an explicit s_waitcnt on the counts of this kernel's issue
// order instead.  The asm has no register outputs: the address operands are
// read at issue, and the destination is LDS (m0 = wave-uniform LDS base).
typedef __attribute__((address_space(3))) void* lds_ptr;
__device__ __forceinline__ uint32_t lds_base(void* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)lds);
}
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_base(lds)) : "memory");
}
// N consecutive KiB from one address and one M0: the instruction's immediate
// offset moves the global and the LDS address alike, so the loads of a block
// need no address arithmetic each.
template <int N>
__device__ __forceinline__ void lds_dma16_kib(const void* g, void* lds) {
  static_assert(N >= 1 && N <= 4, "offsets stay within the 12-bit immediate");
  const uint32_t m0 = lds_base(lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
  if constexpr (N > 1) asm volatile("global_load_lds_dwordx4 %0, off offset:1024" ::"v"(g), "{m0}"(m0) : "memory");
  if constexpr (N > 2) asm volatile("global_load_lds_dwordx4 %0, off offset:2048" ::"v"(g), "{m0}"(m0) : "memory");
  if constexpr (N > 3) asm volatile("global_load_lds_dwordx4 %0, off offset:3072" ::"v"(g), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* g, void* lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_base(lds)) : "memory");
}
// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]); issued through the builtin so the compiler's own counter
// tracking knows which loads have landed.
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Issue the loads of one page into `slot` (wave-uniform pointer).
template <int BITS>
__device__ __forceinline__ void issue_page(const DecodeArgs& a, int page, int g, int lane,
                                           uint8_t* slot) {
  using F = PageFmt<BITS>;
  const size_t base = ((size_t)page * a.hkv + g) * kPage;  // record index of slot 0
  const uint8_t* kb = a.k_codes + base * F::kRecBytes + 16 * lane;
  const uint8_t* vb = a.v_codes + base * F::kRecBytes + 16 * lane;
  lds_dma16_kib<F::kBlockBytes / 1024>(kb, slot);
  lds_dma16_kib<F::kBlockBytes / 1024>(vb, slot + F::kBlockBytes);
  // lanes 0-31 bring the K norms (two per lane), lanes 32-63 the V norms
  const uint16_t* nb = (lane < 32 ? a.k_norms : a.v_norms) + base + 2 * (lane & 31);
  lds_dma4(nb, slot + 2 * F::kBlockBytes);
}

template <bool PACK8, int BITS>
__device__ __forceinline__ void read_page(const uint8_t* slot, int lane, PageRegs<PACK8, BITS>& r) {
  using F = PageFmt<BITS>;
  const int col = lane & 15, jq = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    r.kc[rb] = *reinterpret_cast<const typename PageRegs<PACK8, BITS>::KRec*>(
        slot + (16 * rb + col) * F::kRecBytes + (F::kRecBytes / 4) * jq);
  const u4* vreg = reinterpret_cast<const u4*>(slot + F::kBlockBytes + lane * F::kRecBytes);
#pragma unroll
  for (int i = 0; i < BITS; ++i) r.vr[i] = vreg[i];
  const uint16_t* kn = reinterpret_cast<const uint16_t*>(slot + 2 * F::kBlockBytes);
#pragma unroll
  for (int t = 0; t < PageRegs<PACK8, BITS>::NT; ++t) {
    const int tok = 16 * tile_block<PACK8>(t, col) + 4 * jq;
    r.kn[t] = *reinterpret_cast<const u2*>(kn + tok);
    r.vn[t] = *reinterpret_cast<const u2*>(kn + 64 + tok);
  }
}

__device__ __forceinline__ float norm_at(const u2& n, int r) {
  const uint32_t w = (r < 2) ? n[0] : n[1];
  return half_bits_to_float((r & 1) ? (w >> 16) : (w & 0xFFFFu));
}
// x * norm r of the pair, as one mixed-precision FMA (the fp16 norm is read
// from its half of the register, no separate conversion)
__device__ __forceinline__ float times_norm(float x, const u2& n, int r) {
  return __builtin_fmaf(x, norm_at(n, r), 0.0f);
}

struct PageState {
  float m_run, l_run;  // running max (log2 units) and partial sum (in units of the frame)
  int rho_e;           // value-norm frame 2^rho_e
  f4 acc[8];           // O'^T tiles: coordinates 32*(lane/16) + 4m + r, head lane%16
};

// Power-of-two frame for the value norms of a page: the exponent 15 - e of
// 2^(15 - e), e the biased exponent of the largest fp16 norm bits, so that
// vn * frame < 2.  A page without a nonzero norm keeps the current frame.
__device__ __forceinline__ int frame_exp(uint32_t max_bits, int current) {
  if (max_bits == 0) return current;
  return 15 - (int)((max_bits >> 10) & 0x1Fu);
}

template <bool PACK8>
__device__ __forceinline__ float column_max(float v) {
  // The column's values are scores or -inf, never NaN: a plain v_max_f32
  // (fmaxf would first quiet every operand that arrives through a lane
  // exchange, two extra instructions per step).
  auto vmax = [](float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
  };
  if (PACK8) v = vmax(v, dpp_f<kRowRor8, 0xF>(v, v));
  u2 p = pair_xor16(__builtin_bit_cast(uint32_t, v));
  v = vmax(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  p = pair_xor32(__builtin_bit_cast(uint32_t, v));
  return vmax(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}

// One page for one wave: scores on the matrix cores, online-softmax update,
// P~ V^ accumulation.  MASKED pages hold tokens at or beyond the length L.
template <bool PACK8, bool MASKED, int BITS>
__device__ __forceinline__ void process_page(const PageRegs<PACK8, BITS>& cur, PageState& st, int tok0,
                                             int L, int lane, float fac, const h8 qhi[4],
                                             const h8 qlo[4], const Levels4& lv) {
  constexpr int NT = PageRegs<PACK8, BITS>::NT;
  const int col = lane & 15, jq = lane >> 4;
  f4 s[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    // k-step kk takes coordinates 32 jq + 8 kk .. + 7 of the lane's token
    h8 av[4];
    if constexpr (BITS == 3) {
      uint32_t z[8];
      group_to_selectors(cur.kc[rb].x, cur.kc[rb].y, cur.kc[rb].z, z);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u2 d0 = selector_to_f16(z[2 * kk]), d1 = selector_to_f16(z[2 * kk + 1]);
        av[kk] = __builtin_bit_cast(h8, u4{d0[0], d0[1], d1[0], d1[1]});
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) av[kk] = dword4_to_h8(cur.kc[rb][kk], lv);
    }
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[kk], qhi[kk], acc, 0, 0, 0);
      // (PACK8: qhi carries both parts, columns 0-7 high and 8-15 low)
      if (!PACK8) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[kk], qlo[kk], acc, 0, 0, 0);
    }
    s[rb] = acc;
  }

  // Scores in column units: raw * key norm; the log2-scaled score is that
  // times the lane's column factor `fac` (> 0), applied inside the exponent.
  float sc[NT][4];
  float mp = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = tok0 + 16 * tile_block<PACK8>(t, col) + 4 * jq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // With PACK8 column c < 8 of a tile holds head c's high-part score and
      // column c + 8 its low part; the packed layout takes the even token
      // block in columns 0-7 and the odd one in 8-15, each the sum of its two
      // parts: the even tile plus itself shifted down eight lanes, the odd
      // one plus itself shifted up (each add takes its shift as a DPP
      // operand), and a per-lane select.
      float raw;
      if (PACK8) {
        const float e = s[2 * t][r], o = s[2 * t + 1][r];
        const float pe = e + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, e), kRowShl8, 0xF, 0xF, true));
        const float po = o + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, o), kRowShr8, 0xF, 0xF, true));
        raw = col < 8 ? pe : po;
      } else {
        raw = s[t][r];
      }
      const float v = times_norm(raw, cur.kn[t], r);
      sc[t][r] = (!MASKED || tok + r < L) ? v : -INFINITY;
      mp = fmaxf(mp, sc[t][r]);
    }
  }
  u2 vn[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    vn[t] = cur.vn[t];
    if (MASKED) {  // zero the norms of tokens at or beyond L
      const int t0 = tok0 + 16 * tile_block<PACK8>(t, col) + 4 * jq;
      vn[t][0] &= (t0 < L ? 0xFFFFu : 0u) | (t0 + 1 < L ? 0xFFFF0000u : 0u);
      vn[t][1] &= (t0 + 2 < L ? 0xFFFFu : 0u) | (t0 + 3 < L ? 0xFFFF0000u : 0u);
    }
  }
  uint32_t vbits = PACK8 ? max_half_bits(vn[0], vn[1])
                         : max(max_half_bits(vn[0], vn[1]), max_half_bits(vn[NT - 2], vn[NT - 1]));
  mp = column_max<PACK8>(mp) * fac;
  if (PACK8) vbits = max(vbits, dpp_u<kRowRor8, 0xF>(vbits, vbits));
  vbits = umax_xor32(umax_xor16(vbits));
  const float m_new = fmaxf(st.m_run, mp);        // finite: the page has a valid token
  const float corr = fast_exp2(st.m_run - m_new);  // 0 on the first page
  const int rho_new = frame_exp(vbits, st.rho_e);
  // the accumulator and the sum are both in units of the frame
  const float rescale = __builtin_amdgcn_ldexpf(corr, rho_new - st.rho_e);
  if (__any(rescale != 1.0f)) {
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] *= rescale;
    st.l_run *= rescale;
  }
  st.m_run = m_new;
  st.rho_e = rho_new;
  // p' = 2^(s - m + rho): the softmax weight times the frame
  const float m_shift = m_new - (float)rho_new;

  uint32_t pw[NT][2];  // P~ as f16 pairs: tokens r = 0,1 and r = 2,3 of each tile
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(__builtin_fmaf(sc[t][r], fac, -m_shift));  // masked tokens: 2^-inf = 0
      st.l_run += p[r];
      p[r] = times_norm(p[r], vn[t], r);  // p' * vn < 2: inside the f16 range
    }
    // round to nearest even (round-toward-zero would bias every weight down)
    typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
    pw[t][0] = __builtin_bit_cast(uint32_t, hh2{(_Float16)p[0], (_Float16)p[1]});
    pw[t][1] = __builtin_bit_cast(uint32_t, hh2{(_Float16)p[2], (_Float16)p[3]});
  }
  h8 pb[2];  // B operand of token blocks (2th, 2th+1)
#pragma unroll
  for (int th = 0; th < 2; ++th) {
    u4 w;
    if (PACK8) {
      w[0] = pw[th][0];
      w[1] = pw[th][1];
      // the odd block's weights (columns 8-15 of the score tile) move down
      // eight lanes; the product's columns 8-15 are never read (G <= 8),
      // so their lanes take zeros and no copy of the old value is needed
      w[2] = (uint32_t)__builtin_amdgcn_mov_dpp((int)pw[th][0], kRowShl8, 0xF, 0xF, true);
      w[3] = (uint32_t)__builtin_amdgcn_mov_dpp((int)pw[th][1], kRowShl8, 0xF, 0xF, true);
    } else {
      w[0] = pw[2 * th][0];
      w[1] = pw[2 * th][1];
      w[2] = pw[2 * th + 1][0];
      w[3] = pw[2 * th + 1][1];
    }
    pb[th] = __builtin_bit_cast(h8, w);
  }

  if constexpr (BITS == 3) {
    uint32_t zv[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 3 * c;
      group_to_selectors(cur.vr[d / 4][d % 4], cur.vr[(d + 1) / 4][(d + 1) % 4],
                         cur.vr[(d + 2) / 4][(d + 2) % 4], zv[c]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const u2 d0 = selector_to_f16(zv[2 * th][m]), d1 = selector_to_f16(zv[2 * th + 1][m]);
        const h8 av = __builtin_bit_cast(h8, u4{d0[0], d0[1], d1[0], d1[1]});
        st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[th], st.acc[m], 0, 0, 0);
      }
    }
  } else {
    // dword 4p + 2 th + q of the region: tokens 32 th + 16 q + 4 jq + r of
    // coordinates 32 (col / 4) + 4p + col % 4 (low nibbles, tile p) and
    // + 16 (high nibbles, tile p + 4)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const uint32_t w0 = cur.vr[m & 3][2 * th], w1 = cur.vr[m & 3][2 * th + 1];
        const int sh = m < 4 ? 0 : 4;
        const u2 d0 = nibbles_to_f16((w0 >> sh) & 0x0F0F0F0Fu, lv);
        const u2 d1 = nibbles_to_f16((w1 >> sh) & 0x0F0F0F0Fu, lv);
        const h8 av = __builtin_bit_cast(h8, u4{d0[0], d0[1], d1[0], d1[1]});
        st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[th], st.acc[m], 0, 0, 0);
      }
    }
  }
}

// Exchange with lane ^ 4 inside rows: two row shifts, each writing the banks
// (groups of four lanes) that read in its direction.
__device__ __forceinline__ float lane_xor4(float v) {
  const float t = dpp_f<0x104, 0x5>(v, v);  // row_shl:4 into banks 0 and 2
  return dpp_f<0x114, 0xA>(t, v);           // row_shr:4 into banks 1 and 3
}

// Q' for the heads of one pass: wave w rotates head hb + 2w + lane/32, lane
// r = lane % 32 holding coordinates 4r..4r+3 (SO(4) block r), and stores the
// f16 high and low parts in the B-operand layout of the score MFMA (head h,
// quarter j at lane h + 16j).  The Walsh-Hadamard butterflies at coordinate
// distance 1 and 2 are in-register, 4..64 are lane exchanges 1..16.
__device__ __forceinline__ void rotate_queries(int group, int q_dtype, const uint8_t* s_qraw,
                                               const float* s_rot, uint32_t* s_q, float* s_qinv,
                                               int hb, int wave, int lane) {
  const int r = lane & 31;
  const int h = hb + 2 * wave + (lane >> 5);
  float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
  if (h < group) {
    const int idx = h * kD + 4 * r;
    if (q_dtype == 0) {
      const f4 v = *reinterpret_cast<const f4*>(s_qraw + 4 * idx);
      x0 = v[0]; x1 = v[1]; x2 = v[2]; x3 = v[3];
    } else {
      const u2 v = *reinterpret_cast<const u2*>(s_qraw + 2 * idx);
      const uint32_t w0 = v[0], w1 = v[1];
      if (q_dtype == 1) {
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
  {
    const float a0 = x0 + x1, a1 = x0 - x1, a2 = x2 + x3, a3 = x2 - x3;
    x0 = a0 + a2; x2 = a0 - a2; x1 = a1 + a3; x3 = a1 - a3;
  }
  float s;
  s = (r & 1) ? -1.0f : 1.0f;
  x0 = fmaf(s, x0, quad_xor1(x0)); x1 = fmaf(s, x1, quad_xor1(x1));
  x2 = fmaf(s, x2, quad_xor1(x2)); x3 = fmaf(s, x3, quad_xor1(x3));
  s = (r & 2) ? -1.0f : 1.0f;
  x0 = fmaf(s, x0, quad_xor2(x0)); x1 = fmaf(s, x1, quad_xor2(x1));
  x2 = fmaf(s, x2, quad_xor2(x2)); x3 = fmaf(s, x3, quad_xor2(x3));
  s = (r & 4) ? -1.0f : 1.0f;
  x0 = fmaf(s, x0, lane_xor4(x0)); x1 = fmaf(s, x1, lane_xor4(x1));
  x2 = fmaf(s, x2, lane_xor4(x2)); x3 = fmaf(s, x3, lane_xor4(x3));
  s = (r & 8) ? -1.0f : 1.0f;
  x0 = fmaf(s, x0, dpp_f<kRowRor8, 0xF>(x0, x0)); x1 = fmaf(s, x1, dpp_f<kRowRor8, 0xF>(x1, x1));
  x2 = fmaf(s, x2, dpp_f<kRowRor8, 0xF>(x2, x2)); x3 = fmaf(s, x3, dpp_f<kRowRor8, 0xF>(x3, x3));
  {
    // swap pair (A, B) = (own, partner) on the lower row, (partner, own) on
    // the upper one: the butterfly is A + (+-1) B on both
    s = (r & 16) ? -1.0f : 1.0f;
    float* xs[4] = {&x0, &x1, &x2, &x3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u2 p = pair_xor16(__builtin_bit_cast(uint32_t, *xs[i]));
      *xs[i] = fmaf(s, __builtin_bit_cast(float, (uint32_t)p[1]), __builtin_bit_cast(float, (uint32_t)p[0]));
    }
  }
  // SO(4) block r
  const f4* m = reinterpret_cast<const f4*>(s_rot + 16 * r);
  float z[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f4 row = m[i];
    z[i] = row[0] * x0 + row[1] * x1 + row[2] * x2 + row[3] * x3;
  }
  // per-head power-of-two scale: max |z * sc| in [1, 2)
  float mx = fmaxf(fmaxf(fabsf(z[0]), fabsf(z[1])), fmaxf(fabsf(z[2]), fabsf(z[3])));
  mx = fmaxf(mx, quad_xor1(mx));
  mx = fmaxf(mx, quad_xor2(mx));
  mx = fmaxf(mx, lane_xor4(mx));
  mx = fmaxf(mx, dpp_f<kRowRor8, 0xF>(mx, mx));
  mx = max_xor16(mx);
  int e = 0;
  frexpf(mx, &e);
  const float sc = (mx > 0.f) ? ldexpf(1.0f, 1 - e) : 1.0f;
  if (h < 16) {
    const int j = r >> 3, kk = (r & 7) >> 1, d = 2 * (r & 1);
    const int dst = h + 16 * j;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float v0 = z[2 * t] * sc, v1 = z[2 * t + 1] * sc;
      const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
      const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
      s_q[(kk * 8 + d + t) * 64 + dst] =
          (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      s_q[(kk * 8 + 4 + d + t) * 64 + dst] =
          (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    if (r == 0) s_qinv[h] = 1.0f / sc;
  }
}

// A store performed at device scope (it completes at the point where every
// XCD sees it, not in this XCD's L2): partial rows read by merge workgroups
// that may run on another XCD.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- merge of split partials (one query head, 256 threads) ----
// Thread t keeps an online merge of coordinates 4*(t%32)..+3 over the splits
// s = t/32 (mod 8), with all of its loads issued before any result is used;
// the eight groups then combine through LDS, and the first wave normalises and
// rotates back: o = (H / sqrt(d)) B^T o'.
// The chunk (slots per thread whose loads go out together) is sized to the
// plan's slots, so that one chunk covers them and no load or exponential is
// spent on padding slots (4, 8 or 16 for up to 32, 64 or more slots).
constexpr int kMergeChunk = 16;

// The rows of SO(4) block (t % 64) / 2 of kv head g, which the first wave
// applies transposed (every thread loads one, so the load needs no branch).
__device__ __forceinline__ void merge_rot_block(const float* __restrict__ rot_all, int g, int tid,
                                                f4 mt[4]) {
  const f4* src = reinterpret_cast<const f4*>(rot_all + (size_t)g * kRotFloats + ((tid & 63) >> 1) * 16);
#pragma unroll
  for (int r = 0; r < 4; ++r) mt[r] = src[r];
}

// Rows row0 .. row0 + count - 1 of (m, l) and acc[128] (count >= 1) -> the
// 128 outputs of the head at `out`.  Must be called by all 256 threads.
template <bool ROTATE, int CHUNK = kMergeChunk>
__device__ __forceinline__ void merge_head(const f4 mt[4], const float* __restrict__ ws_acc,
                                           const float* __restrict__ ws_ml, size_t row0, int count,
                                           float* __restrict__ out, int tid) {
  const int quad = tid & 31, grp = tid >> 5;
  __shared__ float s_mm[8], s_ml[8];
  __shared__ f4 s_part[8][32];
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + row0;
  const f4* accp = reinterpret_cast<const f4*>(ws_acc + row0 * kD) + quad;
  float m_t = -INFINITY, l_t = 0.f;
  f4 acc_t = {0.f, 0.f, 0.f, 0.f};
  // splits s0, s0 + 8, ..., s0 + 8 (CHUNK - 1): loads first, then an
  // online merge into (m_t, l_t, acc_t)
  auto merge_chunk = [&](int s0) {
    float2 mv[CHUNK];
    f4 av[CHUNK];
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) {  // rows past the end repeat the last one
      const int sp = min(s0 + 8 * k, count - 1);
      mv[k] = ml[sp];
      av[k] = accp[(size_t)sp * (kD / 4)];
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any use
#pragma unroll
    for (int k = 0; k < CHUNK; ++k)
      if (s0 + 8 * k >= count) mv[k].x = -INFINITY;  // ... with zero weight
    float cm = m_t;
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) cm = fmaxf(cm, mv[k].x);
    // branch-free (a branch here would sink the loads behind it)
    const float keep = (m_t == -INFINITY) ? 0.f : fast_exp2(m_t - cm);
    acc_t *= keep;
    l_t *= keep;
#pragma unroll
    for (int k = 0; k < CHUNK; ++k) {
      // an empty row's accumulator is selected away, never multiplied
      const bool live = mv[k].x > -INFINITY;
      const float w = live ? fast_exp2(mv[k].x - cm) : 0.f;
      const f4 c = w * av[k];
      acc_t[0] += live ? c[0] : 0.f;
      acc_t[1] += live ? c[1] : 0.f;
      acc_t[2] += live ? c[2] : 0.f;
      acc_t[3] += live ? c[3] : 0.f;
      l_t += w * mv[k].y;
    }
    m_t = cm;
  };
  merge_chunk(grp);  // no loop before the first chunk: its loads follow the ones above
  for (int s0 = grp + 8 * CHUNK; s0 < count; s0 += 8 * CHUNK) merge_chunk(s0);
  s_part[grp][quad] = acc_t;
  if (quad == 0) {
    s_mm[grp] = m_t;
    s_ml[grp] = l_t;
  }
  __syncthreads();
  if (tid >= 64) return;
  // lane l owns coordinates 2l, 2l+1
  const int lane = tid;
  float M = -INFINITY;
#pragma unroll
  for (int gq = 0; gq < 8; ++gq) M = fmaxf(M, s_mm[gq]);
  float o0 = 0.f, o1 = 0.f, Ls = 0.f;
  if (M > -INFINITY) {
#pragma unroll
    for (int gq = 0; gq < 8; ++gq) {
      const float w = (s_mm[gq] == -INFINITY) ? 0.f : fast_exp2(s_mm[gq] - M);
      const f4 v = s_part[gq][lane >> 1];
      o0 += w * ((lane & 1) ? v[2] : v[0]);
      o1 += w * ((lane & 1) ? v[3] : v[1]);
      Ls += w * s_ml[gq];
    }
  }
  const float inv = (Ls > 0.f) ? 1.0f / Ls : 0.f;  // an empty sequence gives zeros
  o0 *= inv;
  o1 *= inv;
  if (!ROTATE) {
    *reinterpret_cast<float2*>(out + 2 * lane) = make_float2(o0, o1);
    return;
  }
  // B^T on block lane/2: this lane holds block coordinates c0 = 2*(lane&1), c0+1.
  const float n0 = quad_xor1(o0), n1 = quad_xor1(o1);
  const bool odd = lane & 1;
  const float v0 = odd ? n0 : o0, v1 = odd ? n1 : o1, v2 = odd ? o0 : n0, v3 = odd ? o1 : n1;
  const int c0 = odd ? 2 : 0;
  float y0 = mt[0][c0] * v0 + mt[1][c0] * v1 + mt[2][c0] * v2 + mt[3][c0] * v3;
  float y1 = mt[0][c0 + 1] * v0 + mt[1][c0 + 1] * v1 + mt[2][c0 + 1] * v2 + mt[3][c0 + 1] * v3;
  // Walsh-Hadamard: coordinate distance 1 in-lane, 2..64 across lanes (lane
  // distance 1..32): a butterfly keeps y + partner on the lower lane and
  // partner - y on the upper one.
  {
    const float t0 = y0 + y1, t1 = y0 - y1;
    y0 = t0;
    y1 = t1;
  }
  {
    const float sg = (lane & 1) ? -1.0f : 1.0f;
    y0 = fmaf(sg, y0, quad_xor1(y0));
    y1 = fmaf(sg, y1, quad_xor1(y1));
  }
  {
    const float sg = (lane & 2) ? -1.0f : 1.0f;
    y0 = fmaf(sg, y0, quad_xor2(y0));
    y1 = fmaf(sg, y1, quad_xor2(y1));
  }
  {
    const float sg = (lane & 4) ? -1.0f : 1.0f;
    y0 = fmaf(sg, y0, lane_xor4(y0));
    y1 = fmaf(sg, y1, lane_xor4(y1));
  }
  {
    const float sg = (lane & 8) ? -1.0f : 1.0f;
    y0 = fmaf(sg, y0, dpp_f<kRowRor8, 0xF>(y0, y0));
    y1 = fmaf(sg, y1, dpp_f<kRowRor8, 0xF>(y1, y1));
  }
  {
    // the swap pair (A, B): (own, partner) on the lower lanes, (partner, own)
    // on the upper ones, so both results are A + (+-1) B
    const float sg = (lane & 16) ? -1.0f : 1.0f;
    const u2 p0 = pair_xor16(__builtin_bit_cast(uint32_t, y0));
    const u2 p1 = pair_xor16(__builtin_bit_cast(uint32_t, y1));
    y0 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)p0[1]), __builtin_bit_cast(float, (uint32_t)p0[0]));
    y1 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)p1[1]), __builtin_bit_cast(float, (uint32_t)p1[0]));
  }
  {
    const float sg = (lane & 32) ? -1.0f : 1.0f;
    const u2 p0 = pair_xor32(__builtin_bit_cast(uint32_t, y0));
    const u2 p1 = pair_xor32(__builtin_bit_cast(uint32_t, y1));
    y0 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)p0[1]), __builtin_bit_cast(float, (uint32_t)p0[0]));
    y1 = fmaf(sg, __builtin_bit_cast(float, (uint32_t)p1[1]), __builtin_bit_cast(float, (uint32_t)p1[0]));
  }
  const float nrm = 0.08838834764831845f;  // 1/sqrt(128)
  *reinterpret_cast<float2*>(out + 2 * lane) = make_float2(y0 * nrm, y1 * nrm);
}

// A merge workgroup of the split launch (four waves): query head hh of the
// group of kv head g, sequence b.  The host enables this only when the whole
// grid can be resident at once, so the split workgroups it waits for are
// running or done; the wait is still bounded (2^20 polls, each a memory round
// trip: about a second), and a wait that runs out writes NaN rows instead of
// hanging.
constexpr uint32_t kMergeSpinLimit = 1u << 20;
__device__ __forceinline__ void merge_workgroup(const int32_t* __restrict__ seq_lens,
                                            const float* __restrict__ rot_all, int max_pages,
                                            int pages_per_split, int hq, int group, int splits,
                                            const DecodeArgs& a, int mid) {
  const int tid = threadIdx.x;
  const int hh = mid % group, g = (mid / group) % a.hkv, b = mid / (group * a.hkv);
  const int h = g * group + hh;
  float* out = a.out + ((size_t)b * hq + h) * kD;
  f4 mt[4];
  merge_rot_block(rot_all, g, tid, mt);  // before the wait: it does not depend on the splits
  const int L = seq_lens[b];
  const int n_pages = min((L + kPage - 1) / kPage, max_pages);
  const int n_used = (n_pages + pages_per_split - 1) / pages_per_split;  // the non-empty splits
  uint32_t* arrive = a.arrive + (size_t)b * a.hkv + g;
  __shared__ int s_timed_out;
  if (tid == 0) {
    uint32_t spins = 0;
    int timed_out = 0;
    while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)n_used) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins == kMergeSpinLimit) {
        timed_out = 1;
        break;
      }
    }
    // the split workgroups' partial rows, stored device-coherent before their
    // arrival: drop any older copies of them from this CU's and XCD's caches
    // (all waves of the workgroup share them)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_timed_out = timed_out;
  }
  __syncthreads();
  if (n_used == 0 || s_timed_out) {
    // an empty sequence gives zeros; a wait that ran out gives NaN rows
    if (tid < 32)
      reinterpret_cast<f4*>(out)[tid] = s_timed_out ? f4{NAN, NAN, NAN, NAN} : f4{0.f, 0.f, 0.f, 0.f};
  } else {
    merge_head<true>(mt, a.ws_acc, a.ws_ml, ((size_t)b * hq + h) * splits, n_used, out, tid);
  }
  // the last merge workgroup of (b, g) clears the counters for the next call
  // (every split has arrived and every merge workgroup has read the count)
  if (tid == 0) {
    uint32_t* done = a.done + (size_t)b * a.hkv + g;
    const uint32_t old = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (uint32_t)group) {
      __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// APPEND (a decode step): the current token of each sequence, at position
// L - 1, is quantised here instead of by a separate append: the wave that
// processes the sequence's last page quantises the token's K and V rows,
// patches the record into its LDS copy of the page before using it, and
// stores it into the cache.
// BALANCED (several sequences of unequal length): the split plan is made on
// the device from the lengths, so that every workgroup gets about the same
// number of pages: sequence b receives n_b = ceil(pages_b / P) splits per kv
// head, P the smallest budget for which these fit the plan's workgroups (a
// binary search from total pages / workgroups), and workgroup i (a flat grid)
// finds its (sequence, kv head, split) by a prefix sum over the sequences.
// Without it the host plans from the longest length alone, and the splits of
// short sequences idle while those of the longest run.
template <bool PACK8, int kDecWaves, bool APPEND, int BITS, bool BALANCED>
__global__ __launch_bounds__(64 * kDecWaves, kDecWaves == 4 ? 2 : 1) void decode_split_kernel(const int32_t* __restrict__ block_table,
                                                                      const int32_t* __restrict__ seq_lens,
                                                                      const uint8_t* __restrict__ q_bytes,
                                                                      const float* __restrict__ rot_all,
                                                                      int max_pages, int pps_arg,
                                                                      int hq, int group, int q_dtype,
                                                                      int splits, DecodeArgs a) {
  // The leading arguments are preloaded into SGPRs (14 dwords): everything
  // the first loads need.  The rest come from the argument struct.
  const int tid = threadIdx.x, lane = tid & 63;
  int split, g, b, pages_per_split;
  if constexpr (BALANCED) {
    // every wave computes the same plan; lane s holds sequence s (batch <= 64)
    int pages = 0;
    if (lane < a.batch) pages = min((seq_lens[lane] + kPage - 1) / kPage, max_pages);
    // sums over the lanes on the DPP / permlane path, in fp32 (exact: counts
    // stay far below 2^24)
    auto wave_sum = [](float v) {
      v += quad_xor1(v);
      v += quad_xor2(v);
      v = add_xor4(v);
      v += lane_xor8_f(v);
      return sum_xor32(sum_xor16(v));
    };
    const long long total = (long long)wave_sum((float)pages) * a.hkv;
    // the smallest per-workgroup budget P whose splits, rounded up per
    // sequence, fit the plan's workgroups (at most the staging cap)
    constexpr int kCap = 64 * kDecWaves;
    const int G = a.plan_wgs;
    const long long units = (long long)a.batch * a.hkv;
    auto fits = [&](int p) {  // the rounded-up split count fits the plan's workgroups
      const float n = wave_sum(lane < a.batch ? (float)max(1, (pages + p - 1) / p) : 0.f);
      return (long long)n * a.hkv <= G;
    };
    // bounds: total / G pages each is the least possible; total / (G - units)
    // always fits (rounding adds at most one split per kv head and sequence)
    int lo = (int)max(1LL, (total + G - 1) / G);
    int hi = G > units ? (int)max((long long)lo, (total + (G - units) - 1) / (G - units)) : max(lo, max_pages);
    hi = min(hi, max(lo, max_pages));
    if (fits(lo)) hi = lo;  // equal lengths: the even split
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (fits(mid)) hi = mid;
      else lo = mid + 1;
    }
    const int pbar = min(lo, kCap);
    const int nb = lane < a.batch ? max(1, (pages + pbar - 1) / pbar) : 0;  // an empty one gets 1
    int cum = nb * a.hkv;  // inclusive prefix sum over the sequences
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(cum, o);
      if (lane >= o) cum += t;
    }
    const int i = blockIdx.x;
    const int bb = __popcll(__ballot(lane < a.batch && cum <= i));
    if (bb >= a.batch) return;  // a workgroup beyond the plan (uniform)
    const int base = bb == 0 ? 0 : __shfl(cum, bb - 1);
    const int nbb = __shfl(nb, bb), pb = __shfl(pages, bb);
    const int off = i - base;
    b = __builtin_amdgcn_readfirstlane(bb);
    g = __builtin_amdgcn_readfirstlane(off / nbb);
    split = __builtin_amdgcn_readfirstlane(off - (off / nbb) * nbb);
    pages_per_split = __builtin_amdgcn_readfirstlane(max(1, (pb + nbb - 1) / nbb));
    if (tid == 0 && g == 0 && split == 0) a.n_splits[b] = nbb;
  } else {
    if (a.arrive) {  // flat grid: split workgroups, then merge workgroups
      const int id = blockIdx.x;
      if (id >= a.split_wgs) {
        if constexpr (kDecWaves == 4)
          merge_workgroup(seq_lens, rot_all, max_pages, pps_arg, hq, group, splits, a, id - a.split_wgs);
        return;
      }
      split = id % splits;
      g = (id / splits) % a.hkv;
      b = id / (splits * a.hkv);
    } else {
      split = blockIdx.x;
      g = blockIdx.y;
      b = blockIdx.z;
    }
    pages_per_split = pps_arg;
  }
  // wave-uniform: keeps the wave's page bookkeeping in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, jq = lane >> 4;
  constexpr int kLastWave = kDecWaves - 1;
  using F = PageFmt<BITS>;
  constexpr int kSlotBytes = F::kSlotBytes, kDmaPerPage = F::kDmaPerPage;

  // (eight waves: 102,400 B for 3-bit pages, 135,168 B for 4-bit ones)
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kDecWaves][2][kSlotBytes];
  // The sequence's partial last page, and before it the group's raw queries:
  // the queries are read only before the workgroup barrier that precedes the
  // first load into the tail slot.
  constexpr int kTailBytes = kSlotBytes > IQ_MAX_GROUP_BYTES ? kSlotBytes : IQ_MAX_GROUP_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t s_tail[kTailBytes];
  uint8_t* const s_qraw = s_tail;
  __shared__ __attribute__((aligned(16))) float s_rot[kRotFloats];     // 2,048 B
  __shared__ uint32_t s_q[32 * 64];  // Q' operands: [kstep*8 + dword][lane]
  __shared__ int s_pages[64 * kDecWaves];  // the split's page ids
  __shared__ float s_qinv[16];
  __shared__ float s_m[kDecWaves][16], s_l[kDecWaves][16], s_wt[kDecWaves][16];
  __shared__ int s_next;  // next unclaimed page of the split (waves claim pages as they go)
  __shared__ __attribute__((aligned(16))) uint8_t s_xraw[APPEND ? 1024 : 16];  // appended K | V rows

  // ---- prologue: every load that needs only the arguments goes out first ----
  // The split's page ids (an eighth per wave), the rotation blocks and the
  // group's queries arrive by direct-to-LDS loads; the length and the wave's
  // first two page ids are scalar loads.  The first two pages are requested
  // before the length is known: their block-table entries lie inside the table
  // and their ids are clamped into the cache, so the loads stay in bounds even
  // where the table holds no page yet, and a page beyond the length is never
  // used.
  const int pg_begin = split * pages_per_split;
  const int* bt = block_table + (size_t)b * max_pages;
  // scalar loads first: after the first direct-to-LDS load the compiler no
  // longer proves the table unmodified and would use vector loads + full waits
  const int L = seq_lens[b];
  const int last_entry = max_pages - 1;
  // the wave's first two pool pages, w and w + W; where the split is shorter
  // a slot repeats a page of the split (the same lines: no extra HBM traffic,
  // and every wave issues the same loads, so the waits below stay exact)
  const int first0 = pg_begin + min(wave, pages_per_split - 1);
  const int first1 = wave + kDecWaves < pages_per_split ? pg_begin + wave + kDecWaves : first0;
  const uint32_t bt0 = (uint32_t)bt[min(first0, last_entry)];
  const uint32_t bt1 = (uint32_t)bt[min(first1, last_entry)];
  const uint32_t last_page = (uint32_t)a.num_pages - 1u;
  const int n_alloc = min(pages_per_split, max_pages - pg_begin);  // readable table entries
  if (64 * wave < n_alloc && 64 * wave + lane < n_alloc)
    lds_dma4(bt + pg_begin + 64 * wave + lane, &s_pages[64 * wave]);
  // Each wave loads the rotation blocks (the same bytes into the same place)
  // and the rows of the query heads it rotates: 2w, 2w+1 (+ 2W, 2W+1 for
  // the second pass of a four-wave workgroup with a group above 8).
  const int esize = q_dtype == 0 ? 4 : 2;
  constexpr int kHeadsPerPass = 2 * kDecWaves;
  const int n_pass = (group + kHeadsPerPass - 1) / kHeadsPerPass;
  {
    const uint8_t* rg = reinterpret_cast<const uint8_t*>(rot_all + (size_t)g * kRotFloats) + 16 * lane;
    lds_dma16_kib<2>(rg, s_rot);
    const size_t row_bytes = (size_t)kD * esize;
    const uint8_t* qg = q_bytes + ((size_t)b * hq + (size_t)g * group) * row_bytes;
    for (int p = 0; p < n_pass; ++p) {
      const int h0 = kHeadsPerPass * p + 2 * wave;
      const int nbytes = max(0, min(2, group - h0)) * (int)row_bytes;
      if (16 * lane < nbytes) lds_dma16(qg + h0 * row_bytes + 16 * lane, s_qraw + h0 * row_bytes);
    }
    if (APPEND && wave == kLastWave) {
      // the current token's K and V rows of this kv head (quantised here if
      // the split holds the sequence's last page)
      const int vbytes = kD * (a.kv_dtype == 0 ? 4 : 2);
      const size_t off = ((size_t)b * a.hkv + g) * vbytes;
      if (16 * lane < vbytes) {
        lds_dma16(a.k_new + off + 16 * lane, s_xraw);
        lds_dma16(a.v_new + off + 16 * lane, s_xraw + 512);
      }
    }
  }
  // Four waves (one short pass over the chip): every wave's second page is
  // requested only once the prologue loads have landed, so that the first
  // pages of all waves stream in ahead of the second ones instead of beside
  // them.
  constexpr bool kLateSecond = kDecWaves == 4;
  issue_page<BITS>(a, (int)min(bt0, last_page), g, lane, s_ring[wave][0]);
  if constexpr (!kLateSecond) issue_page<BITS>(a, (int)min(bt1, last_page), g, lane, s_ring[wave][1]);

  // (a length beyond the block table breaks the contract; never read past it)
  const int n_pages = min((L + kPage - 1) / kPage, max_pages);
  if (pg_begin >= n_pages) {  // uniform for the workgroup
    // an empty split still leaves its mark: zero weight in the merge kernel
    // (merge workgroups read only the non-empty splits)
    if (!a.arrive && tid < group) {
      const size_t row = ((size_t)b * hq + (size_t)g * group + tid) * splits + split;
      a.ws_ml[2 * row] = -INFINITY;
      a.ws_ml[2 * row + 1] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // no load may still target this LDS
    return;
  }
  const int pg_end = min(n_pages, pg_begin + pages_per_split);
  // The partial last page of the sequence, if it falls in this split, is kept
  // out of the shared pool and handled (masked) by the last wave.
  // A decode step always treats the last page as the tail: its copy in LDS
  // gets the appended record before use.
  const bool append_here = APPEND && pg_end == n_pages && L <= max_pages * kPage;
  const bool has_tail =
      append_here || ((L % kPage) != 0 && n_pages * kPage > L && pg_end == n_pages);
  const int n_pool = (pg_end - pg_begin) - (has_tail ? 1 : 0);  // full pages to share
  if (tid == 0) s_next = 2 * kDecWaves;  // pool pages w and w + 8 are each wave's first two

  // Everything but the two pages (four waves: the first page) has landed once
  // at most their loads are outstanding (loads complete in issue order).  (One straight-line wait:
  // with waits on several paths the compiler would assume the worst and wait
  // for the pages before the LDS reads of the rotation below.)
  __builtin_amdgcn_s_waitcnt(wait_vm((kLateSecond ? 1 : 2) * kDmaPerPage));
  if constexpr (kLateSecond) issue_page<BITS>(a, (int)min(bt1, last_page), g, lane, s_ring[wave][1]);

  // Every wave rotates its query heads (rotate_queries: lane r of a half
  // wave holds coordinates 4r..4r+3).
  for (int p = 0; p < n_pass; ++p)
    rotate_queries(group, q_dtype, s_qraw, s_rot, s_q, s_qinv, kHeadsPerPass * p, wave, lane);
  // LDS writes visible to the workgroup; unlike __syncthreads this does not
  // wait for the page loads still in flight.
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();

  // With PACK8 (G <= 8) score columns 8-15 would multiply padding: they take
  // the low part of heads 0-7 instead (qhi of lane col >= 8 = low part of
  // head col - 8), so one MFMA per k-step yields both parts and qlo is unused.
  h8 qhi[4], qlo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u4 dh, dl;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (PACK8) {
        dh[d] = s_q[(kk * 8 + (col < 8 ? 0 : 4) + d) * 64 + (col < 8 ? lane : lane - 8)];
        dl[d] = 0u;
      } else {
        dh[d] = s_q[(kk * 8 + d) * 64 + lane];
        dl[d] = s_q[(kk * 8 + 4 + d) * 64 + lane];
      }
    }
    qhi[kk] = __builtin_bit_cast(h8, dh);
    qlo[kk] = __builtin_bit_cast(h8, dl);
  }
  // per-lane score factor of the lane's head column
  const float fac = a.score_factor * s_qinv[PACK8 ? (col & 7) : col];

  // the last wave brings the partial page now; it is used after its stream
  const bool tail_mine = has_tail && wave == kLastWave;
  // Where the wave's second prologue page is the tail page itself (pool page
  // w + W would be the first past the pool), that slot already holds it,
  // requested with the first pages: no second request, which would queue
  // behind the whole split's page traffic.  Otherwise the tail goes to its
  // own buffer now.
  const bool tail_in_ring = tail_mine && wave + kDecWaves == n_pool;
  uint8_t* const tail_buf = tail_in_ring ? s_ring[wave][1] : s_tail;
  const bool tail_load = tail_mine && !tail_in_ring;
  if (tail_load)
    issue_page<BITS>(a, (int)min((uint32_t)s_pages[n_pages - 1 - pg_begin], last_page), g, lane, s_tail);
  // ... and quantises the appended token (lanes 0-31 K, 32-63 V)
  float x_norm = 0.f;
  u3 x_rec = {0u, 0u, 0u};  // 3-bit: the group's three dwords; 4-bit: x_rec.x, this lane's dword
  if (append_here && wave == kLastWave) {
    const int r = lane & 31;
    const uint8_t* src = s_xraw + 512 * (lane >> 5);
    float x0, x1, x2, x3;
    if (a.kv_dtype == 0) {
      const f4 v = *reinterpret_cast<const f4*>(src + 16 * r);
      x0 = v[0]; x1 = v[1]; x2 = v[2]; x3 = v[3];
    } else {
      const u2 v = *reinterpret_cast<const u2*>(src + 8 * r);
      const uint32_t w0 = v[0], w1 = v[1];
      if (a.kv_dtype == 1) {
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
    const f4* m = reinterpret_cast<const f4*>(s_rot + 16 * r);
    if constexpr (BITS == 3)
      quantize_lanes32<true>(x0, x1, x2, x3, m[0], m[1], m[2], m[3], r, x_norm, x_rec);
    else
      x_rec.x = quantize_lanes32_4(x0, x1, x2, x3, m[0], m[1], m[2], m[3], r, lane >= 32, a.lv4, x_norm);
  }
  // The record goes into the cache (skipped for a bad page id) before the
  // wave's last pages are processed, so that the stores complete meanwhile
  // (stores issued after the last page's processing would hold up the end of
  // the workgroup).  The wave's memory counter completes in issue order, so
  // the stores wait for the pages requested before them: with four waves
  // (one or two pages each) they go out once the first page has landed; with
  // eight (long streams, where code in the page loop costs registers and
  // time on every page) right before the tail.  This split's copy of the
  // page in LDS is patched before use (the page load may have read the slot
  // before or after these stores).
  constexpr bool kRecordInLoop = kDecWaves == 4;
  bool record_pending = APPEND && kRecordInLoop && append_here && wave == kLastWave;
  auto store_record = [&]() {
    const uint32_t id = (uint32_t)s_pages[n_pages - 1 - pg_begin];
    if (id < (uint32_t)a.num_pages) {
      const size_t blk = (size_t)id * a.hkv + g;
      const bool is_v = lane >= 32;
      uint8_t* codes = (is_v ? a.v_codes : a.k_codes) + blk * F::kBlockBytes;
      uint16_t* norms = (is_v ? a.v_norms : a.k_norms) + blk * kPage;
      if constexpr (BITS == 3) place_record(is_v, lane & 31, x_rec, x_norm, codes, norms, (L - 1) & 63);
      else place_record4(is_v, lane & 31, x_rec.x, x_norm, codes, norms, (L - 1) & 63);
    }
    record_pending = false;
  };

  PageState st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.rho_e = 0;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.acc[m] = f4{0.f, 0.f, 0.f, 0.f};

  // The tail page: the appended record replaces slot L - 1 of its copy, then
  // it is processed (masked).
  // Eight waves (long streams) take it first, so that the waves' page claims
  // spread its cost over the workgroup; four waves (one or two pages each),
  // last.
  auto run_tail = [&]() {
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    if (append_here) {
      const bool is_v = lane >= 32;
      uint8_t* codes = tail_buf + (is_v ? F::kBlockBytes : 0);
      uint16_t* norms = reinterpret_cast<uint16_t*>(tail_buf + 2 * F::kBlockBytes + (is_v ? 128 : 0));
      if constexpr (BITS == 3) place_record(is_v, lane & 31, x_rec, x_norm, codes, norms, (L - 1) & 63);
      else place_record4(is_v, lane & 31, x_rec.x, x_norm, codes, norms, (L - 1) & 63);
      if (!kRecordInLoop || record_pending) store_record();  // (four waves: no pool page)
    }
    PageRegs<PACK8, BITS> cur;
    read_page<PACK8, BITS>(tail_buf, lane, cur);
    // Masked, also where the step completes the page (the mask then keeps
    // every token): a second, unmasked instance beside the loop's took the
    // four-wave step kernel from 156 to 219 registers (and an earlier
    // eight-wave one from 146 to 210) and measured no faster.
    process_page<PACK8, true, BITS>(cur, st, (n_pages - 1) * kPage, L, lane, fac, qhi, qlo, a.lv4);
  };
  constexpr bool kTailFirst = kDecWaves == 8;
  if constexpr (kTailFirst)
    if (tail_mine) run_tail();

  // ---- the wave's stream of full pages ----
  // Slots 0 and 1 start with pool pages w and w + W; each processed slot is
  // refilled with the next unclaimed pool page (an LDS counter), so the waves
  // of the workgroup finish within about a page of each other.  seq[] counts
  // page loads in issue order, to know how many may still be outstanding.
  bool have0 = wave < n_pool, have1 = wave + kDecWaves < n_pool;  // n_pool <= pages_per_split
  int pg0 = pg_begin + wave, pg1 = pg_begin + wave + kDecWaves;
  int seq0 = 0, seq1 = 1, issued = 2;
  int head = 0;
  bool pool_open = true;
  int next_fixed = wave + 2 * kDecWaves;  // deterministic: the wave's next page of the pool
  while (head == 0 ? have0 : have1) {
    uint8_t* slot = s_ring[wave][head];
    const int seq_h = head == 0 ? seq0 : seq1;
    // loads issued after this page's: the other slot (and the tail's, which
    // went out after the first pages)
    const int after = issued - 1 - seq_h + ((tail_load && seq_h < 2) ? 1 : 0);
    if (after <= 0) __builtin_amdgcn_s_waitcnt(wait_vm(0));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(wait_vm(kDmaPerPage));
    else __builtin_amdgcn_s_waitcnt(wait_vm(2 * kDmaPerPage));
    PageRegs<PACK8, BITS> cur;
    read_page<PACK8, BITS>(slot, lane, cur);
    if constexpr (APPEND && kRecordInLoop)
      if (record_pending) store_record();
    const int pg = head == 0 ? pg0 : pg1;
    // claim the next page and reuse this slot for it (claims only grow: a
    // failed claim ends the stream)
    int claim = n_pool;
    if (pool_open) {
      if (a.deterministic) {
        claim = next_fixed;
        next_fixed += kDecWaves;
      } else {
        int c = 0;
        if (lane == 0) c = atomicAdd(&s_next, 1);
        claim = __builtin_amdgcn_readfirstlane(c);
      }
    }
    const bool got = claim < n_pool;
    pool_open = got;
    if (got) {
      const uint32_t id = min((uint32_t)s_pages[claim], last_page);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // slot read before it is refilled
      issue_page<BITS>(a, (int)__builtin_amdgcn_readfirstlane(id), g, lane, slot);
    }
    if (head == 0) {
      have0 = got; pg0 = pg_begin + claim; seq0 = issued;
    } else {
      have1 = got; pg1 = pg_begin + claim; seq1 = issued;
    }
    issued += got ? 1 : 0;
    process_page<PACK8, false, BITS>(cur, st, pg * kPage, L, lane, fac, qhi, qlo, a.lv4);
    // the other slot's page is older than the refill, if it holds one
    if (head == 0 ? have1 : have0) head ^= 1;
  }
  if constexpr (!kTailFirst)
    if (tail_mine) run_tail();
  __builtin_amdgcn_s_waitcnt(wait_vm(0));  // a page requested but not used may still be landing

  // ---- merge the eight waves ----
  float l_col = __builtin_amdgcn_ldexpf(st.l_run, -st.rho_e);
  if (PACK8) l_col += dpp_f<kRowRor8, 0xF>(l_col, l_col);
  l_col = sum_xor32(sum_xor16(l_col));
  const float fin = __builtin_amdgcn_ldexpf(a.out_factor, -st.rho_e);
  // The wave's own two slots (contiguous) hold its accumulator now (all its
  // loads have landed and its reads of them are done), row-major [head]
  // [coordinate] with rows of kAccStride floats: padded so that the f4
  // writes of the 16 head columns fall on distinct banks.
  constexpr int kAccStride = 132;
  static_assert(2 * kSlotBytes >= 16 * kAccStride * 4, "two slots hold an accumulator");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  float* const acc_own = reinterpret_cast<float*>(s_ring[wave][0]);
#pragma unroll
  for (int m = 0; m < 8; ++m)
    *reinterpret_cast<f4*>(acc_own + col * kAccStride + 32 * jq + 4 * m) = st.acc[m] * fin;
  if (jq == 0) {
    s_m[wave][col] = st.m_run;
    s_l[wave][col] = l_col;
  }
  __syncthreads();
  const size_t row0 = ((size_t)b * hq + (size_t)g * group) * splits + split;  // head h: + h * splits
  // Head h's wave weights 2^(m_w - M), M the largest wave maximum; returns M.
  auto wave_weights = [&](int h, float (&wt)[kDecWaves]) {
    float mw[kDecWaves], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      mw[w] = s_m[w][h];
      M = fmaxf(M, mw[w]);
    }
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) wt[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
    return M;
  };
  if (!a.arrive) {
    // Each head's 32 threads compute its weights themselves (no second
    // barrier) and sum the waves' accumulators over four coordinates each:
    // one 512-byte row per head, and the (m, l) pair from its first thread.
    for (int h = tid >> 5; h < group; h += 2 * kDecWaves) {
      float wt[kDecWaves];
      const float M = wave_weights(h, wt);
      const int c = 4 * (tid & 31);
      f4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w)
        sum += wt[w] * *reinterpret_cast<const f4*>(reinterpret_cast<const float*>(s_ring[w][0]) +
                                                   h * kAccStride + c);
      *reinterpret_cast<f4*>(a.ws_acc + (row0 + (size_t)h * splits) * kD + c) = sum;
      if ((tid & 31) == 0) {
        float Ls = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) Ls += wt[w] * s_l[w][h];
        float* dst = a.ws_ml + 2 * (row0 + (size_t)h * splits);
        dst[0] = M;
        dst[1] = Ls;
      }
    }
    return;
  }
  // Merged in the same launch: the weights through LDS, and the rows as
  // device-coherent dword stores, 64 consecutive coordinates of one row per
  // wave instruction (whole lines).
  if (tid < group) {
    float wt[kDecWaves];
    const float M = wave_weights(tid, wt);
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      s_wt[w][tid] = wt[w];
      Ls += wt[w] * s_l[w][tid];
    }
    float* dst = a.ws_ml + 2 * (row0 + (size_t)tid * splits);
    store_agent(dst, M);
    store_agent(dst + 1, Ls);
  }
  __syncthreads();
  for (int v = tid; v < group * kD; v += 64 * kDecWaves) {
    const int h = v >> 7, c = v & (kD - 1);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w)
      sum += s_wt[w][h] * reinterpret_cast<const float*>(s_ring[w][0])[h * kAccStride + c];
    store_agent(a.ws_acc + (row0 + (size_t)h * splits) * kD + c, sum);
  }
  // Once every wave has its device-coherent stores acknowledged, count the
  // workgroup in.  (A release fence at device scope would also write back this
  // XCD's L2, which here took several microseconds per wave.)
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  __syncthreads();
  if (tid == 0)
    __hip_atomic_fetch_add(&a.arrive[(size_t)b * a.hkv + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per (query head, sequence): merge the split partials,
// normalise, and rotate back (merge_head).  ROTATE = false: the partials are
// already in the original space (the uncompressed baseline); the merge only
// normalises.
template <bool ROTATE, int CHUNK>
__global__ __launch_bounds__(256, 1) void decode_merge_kernel(const float* __restrict__ rot_all,
                                                           const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml,
                                                           int splits, int hq_n, int group,
                                                           const int32_t* __restrict__ n_splits,
                                                           float* __restrict__ out_all) {
  // All arguments arrive preloaded in SGPRs and every load is issued at once.
  // Each planned split has written its row (an empty one only m = -inf,
  // l = 0), so no length is needed here; zero-weight rows never touch the sums.
  // (A sequence's first merge chunk always exists: count >= 1.)
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row0 = ((size_t)b * hq_n + hq) * splits;
  // rows hold `splits` slots; a balanced plan used the first n_splits[b]
  const int count = n_splits ? n_splits[b] : splits;
  f4 mt[4];
  if (ROTATE) merge_rot_block(rot_all, hq / group, tid, mt);
  merge_head<ROTATE, CHUNK>(mt, ws_acc, ws_ml, row0, count, out_all + ((size_t)b * hq_n + hq) * kD, tid);
}

// Split planning: one workgroup per CU.  Few pages per kv head (short or
// single sequences, at most four pages per wave): four waves, one pass over
// the chip, the shortest critical path (at 64K x 4 kv heads, four pages per
// wave, 15.7 us per step against 16.9 us with eight waves).  Many pages: eight waves (two per SIMD;
// the LDS holds one such workgroup), a unit (sequence, kv head) getting
// ceil(CUs / units) splits of equal page ranges inside which the waves claim
// pages dynamically, so the waves of a CU finish together.  One workgroup
// per CU also keeps two workgroups from competing for the same SIMDs (the
// older would win the issue arbitration and the younger finish late).
// The caller may fix the waves, the pages per split of the host plan, the
// workgroups per CU planned for (more rounds of shorter splits, which the
// hardware dispatcher balances) and the plan kind.
DecodePlan plan_decode(int batch, int hkv, int max_seq_len, int num_cus, const DecodeOptions& o) {
  const int max_pages = max(1, (max_seq_len + kPage - 1) / kPage);
  const long long units = (long long)max(1, batch) * max(1, hkv);
  const long long cus = max(1, num_cus);
  DecodePlan p{};
  p.waves = (units * max_pages <= cus * 4 * 4) ? 4 : 8;
  if (o.waves == 4 || o.waves == 8) p.waves = o.waves;
  const long long rounds = o.rounds > 0 ? o.rounds : 1;
  long long splits = (rounds * cus + units - 1) / units;
  if (splits > max_pages) splits = max_pages;
  long long pps = (max_pages + splits - 1) / splits;
  if (o.pages_per_split > 0) pps = o.pages_per_split;
  const long long cap = 64LL * p.waves;  // page ids staged per split
  if (pps > cap) pps = cap;
  if (pps < 1) pps = 1;
  p.pages_per_split = (int)pps;
  p.splits = (int)((max_pages + pps - 1) / pps);
  p.balanced = 0;
  p.grid_x = p.splits;
  p.plan_wgs = 0;
  p.merge = o.merge;
  p.deterministic = o.deterministic ? 1 : 0;
  p.cus = (int)cus;
  // Several sequences: the device balances the pages (their lengths are known
  // only there).  The plan's G workgroups hold at most `cap` pages each; rows
  // of the workspace get ceil(G / Hkv) slots, the most one sequence can take
  // (its pages are at most total / Hkv), and the grid G + B Hkv workgroups
  // (rounding up every sequence's count adds at most one per kv head).
  bool balanced = batch > 1 && batch <= 64;
  if (o.plan == 1) balanced = false;
  if (balanced) {
    long long G = rounds * cus;
    const long long need = (units * max_pages + cap - 1) / cap;
    if (G < need) G = need;
    long long slots = (G + hkv - 1) / hkv;
    if (slots > max_pages) slots = max_pages;
    if (slots < 1) slots = 1;
    p.balanced = 1;
    p.plan_wgs = (int)G;
    p.grid_x = (int)(G + units);
    p.splits = (int)slots;
    p.pages_per_split = (int)cap;
  }
  return p;
}

size_t decode_workspace_bytes(int batch, int hq, const DecodePlan& plan) {
  const size_t rows = (size_t)batch * hq * plan.splits;
  // counters, the partial rows, and one split count per sequence for a
  // balanced plan
  return kWsCounterBytes + rows * kD * sizeof(float) + rows * 2 * sizeof(float) +
         (plan.balanced ? (size_t)batch * sizeof(int32_t) : 0);
}

namespace {

// Workgroups of one split-kernel instantiation that a CU holds at once (LDS,
// registers and waves), from the runtime's occupancy calculator; cached.
template <bool P8, int W, bool AP, int B, bool BAL>
int split_blocks_per_cu() {
  static std::atomic<int> cached{-1};
  int n = cached.load(std::memory_order_relaxed);
  if (n < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_kernel<P8, W, AP, B, BAL>, 64 * W, 0) !=
        hipSuccess)
      return 0;  // not cached: asked again next time
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

// split_blocks_per_cu of the instantiation a call launches.
int split_occupancy(bool pack8, int waves, bool append, int bits, bool balanced) {
#define IQ_OCC_B(P8, W, AP, B) (balanced ? split_blocks_per_cu<P8, W, AP, B, true>() : split_blocks_per_cu<P8, W, AP, B, false>())
#define IQ_OCC_W(P8, W, AP) (bits == 4 ? IQ_OCC_B(P8, W, AP, 4) : IQ_OCC_B(P8, W, AP, 3))
#define IQ_OCC_A(P8, W) (append ? IQ_OCC_W(P8, W, true) : IQ_OCC_W(P8, W, false))
#define IQ_OCC_P(W) (pack8 ? IQ_OCC_A(true, W) : IQ_OCC_A(false, W))
  return waves == 4 ? IQ_OCC_P(4) : IQ_OCC_P(8);
#undef IQ_OCC_P
#undef IQ_OCC_A
#undef IQ_OCC_W
#undef IQ_OCC_B
}

}  // namespace

// Merge workgroups join the split launch (host plan, four waves) when the
// caller asks for it and the runtime's occupancy calculator says every
// workgroup of the grid can be resident at once, so that a merge workgroup
// never waits for a split workgroup that has no CU.  It is not the default:
// the split workgroups then publish their partial rows with device-scope
// stores (the merge workgroups may sit on another XCD, whose L2 does not see
// this one's), and at the 32K single-sequence workload those stores took
// longer to complete than the launch gap before a merge kernel.
bool decode_fused_merge(const DecodePlan& plan, int batch, int hkv, int hq, int bits, bool append) {
  if (plan.merge != 1 || plan.balanced || plan.waves != 4 || (long long)batch * hkv > kMaxCounterUnits)
    return false;
  const long long split_wgs = (long long)plan.splits * hkv * batch;
  const long long merge_wgs = (long long)batch * hq;
  const int bpc = split_occupancy(hq / hkv <= 8, 4, append, bits, false);
  return bpc > 0 && split_wgs + merge_wgs <= (long long)bpc * plan.cus;
}

hipError_t launch_decode(const CacheView& c, const float* rot, const void* q, int q_dtype, int batch,
                         int hq, const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                         const DecodePlan& plan, float softmax_scale, float* out, void* workspace,
                         const void* k_new, const void* v_new, int kv_dtype, hipStream_t stream) {
  DecodeArgs a;
  const bool four = c.bits == 4;
  const double alpha = four ? (double)codebook4().alpha : (double)kLevelScale;
  a.lv4 = four ? codebook4().lv : Levels4{};
  a.k_codes = c.k_codes;
  a.k_norms = c.k_norms;
  a.v_codes = c.v_codes;
  a.v_norms = c.v_norms;
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.kv_dtype = kv_dtype;
  a.num_pages = c.num_pages;
  a.hkv = c.hkv;
  a.q_dtype = q_dtype;
  a.hq = hq;
  a.group = hq / c.hkv;
  a.max_pages = max_pages;
  a.pages_per_split = plan.pages_per_split;
  a.splits = plan.splits;
  const double log2e = 1.4426950408889634;
  a.score_factor = (float)((double)softmax_scale * log2e / (128.0 * alpha));
  a.out_factor = (float)(1.0 / (sqrt(128.0) * alpha));
  const size_t rows = (size_t)batch * hq * plan.splits;
  uint32_t* counters = reinterpret_cast<uint32_t*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kWsCounterBytes);
  a.ws_ml = a.ws_acc + rows * kD;
  a.out = out;
  a.plan_wgs = plan.plan_wgs;
  a.batch = batch;
  a.n_splits = plan.balanced ? reinterpret_cast<int32_t*>(a.ws_ml + rows * 2) : nullptr;
  a.deterministic = plan.deterministic;
  a.arrive = nullptr;
  a.done = nullptr;
  a.split_wgs = 0;
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  const bool append = k_new != nullptr;
  const long long split_wgs = (long long)plan.splits * c.hkv * batch;
  const long long merge_wgs = (long long)batch * hq;
  hipError_t e = hipSuccess;
  const bool fused = decode_fused_merge(plan, batch, c.hkv, hq, c.bits, append);
  if (fused) {
    a.arrive = counters;
    a.done = counters + kMaxCounterUnits;
    a.split_wgs = (int)split_wgs;
  }
  auto launch = [&](auto kernel, int waves) {
    const dim3 grid = plan.balanced ? dim3(plan.grid_x, 1, 1)
                      : fused       ? dim3((unsigned)(split_wgs + merge_wgs), 1, 1)
                                    : dim3(plan.splits, c.hkv, batch);
    hipLaunchKernelGGL(kernel, grid, dim3(64 * waves), 0, stream, block_table, seq_lens, qb, rot,
                       a.max_pages, a.pages_per_split, a.hq, a.group, a.q_dtype, a.splits, a);
    e = hipGetLastError();
  };
#define IQ_SPLIT_K(P8, W, AP, B, BAL) launch(decode_split_kernel<P8, W, AP, B, BAL>, W)
#define IQ_SPLIT(P8, W, AP, B)                    \
  if (plan.balanced) IQ_SPLIT_K(P8, W, AP, B, true); \
  else IQ_SPLIT_K(P8, W, AP, B, false)
#define IQ_SPLIT_B(P8, W, AP)               \
  if (four) { IQ_SPLIT(P8, W, AP, 4); }     \
  else { IQ_SPLIT(P8, W, AP, 3); }
#define IQ_SPLIT_W(P8, AP)              \
  if (plan.waves == 4) { IQ_SPLIT_B(P8, 4, AP); } \
  else { IQ_SPLIT_B(P8, 8, AP); }
  if (a.group <= 8) {
    if (append) { IQ_SPLIT_W(true, true); }
    else { IQ_SPLIT_W(true, false); }
  } else {
    if (append) { IQ_SPLIT_W(false, true); }
    else { IQ_SPLIT_W(false, false); }
  }
#undef IQ_SPLIT_W
#undef IQ_SPLIT_B
#undef IQ_SPLIT
#undef IQ_SPLIT_K
  if (e != hipSuccess || fused) return e;
  return launch_decode_merge(true, rot, a.ws_acc, a.ws_ml, plan.splits, batch, hq, a.group, a.n_splits,
                             out, stream);
}

hipError_t launch_decode_merge(bool rotate, const float* rot, const float* ws_acc, const float* ws_ml,
                               int splits, int batch, int hq, int group, const int32_t* n_splits,
                               float* out, hipStream_t stream) {
#define IQ_MERGE(R, C)                                                                         \
  hipLaunchKernelGGL((decode_merge_kernel<R, C>), dim3(hq, batch), dim3(256), 0, stream, rot, ws_acc, \
                     ws_ml, splits, hq, group, n_splits, out)
  // eight thread groups: one chunk of C slots each covers 8 C slots
  if (splits <= 32) {
    if (rotate) IQ_MERGE(true, 4); else IQ_MERGE(false, 4);
  } else if (splits <= 64) {
    if (rotate) IQ_MERGE(true, 8); else IQ_MERGE(false, 8);
  } else {
    if (rotate) IQ_MERGE(true, 16); else IQ_MERGE(false, 16);
  }
#undef IQ_MERGE
  return hipGetLastError();
}

}  // namespace iq
