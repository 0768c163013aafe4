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
// With G <= 8 two 16-token score tiles share one set of registers (columns
// 0-7 and 8-15), which halves the softmax work; the shared layout is also the
// B operand of the PV product after one row shift.
// Levels enter as alpha-scaled f16 (see iq_device.h); the key norm, 1/alpha,
// the softmax scale and log2(e) are one fp32 factor per score.  The value
// norm is folded into P~ relative to a per-page power-of-two frame so that P~
// stays inside the f16 range for any norm.
#include <math.h>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

struct DecodeArgs {
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  int hkv;
  const float* rot;
  const void* q;
  int q_dtype;
  int hq, group;
  const int32_t* block_table;
  int max_pages;
  const int32_t* seq_lens;
  int pages_per_split, splits;
  float score_factor;  // softmax_scale * log2(e) / (128 * alpha)
  float out_factor;    // 1 / (sqrt(128) * alpha)
  float* ws_acc;       // [B][Hq][splits][128]
  float* ws_ml;        // [B][Hq][splits][2]
  float* out;          // [B][Hq][128]
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
template <bool PACK8>
struct PageRegs {
  static constexpr int NT = PACK8 ? 2 : 4;
  u3 kc[4];       // K: 12 code bytes of token 16*rb + lane%16, group lane/16
  u4 vr[3];       // V: the lane's 48-byte region (chunks c = 0..3, dwords 3c..3c+2)
  u2 kn[NT], vn[NT];  // fp16 norms of the lane's four score tokens per tile
};

template <bool PACK8>
__device__ __forceinline__ int tile_block(int t, int col) {
  return PACK8 ? 2 * t + (col >> 3) : t;
}

// ---- LDS page ring -------------------------------------------------------
// Each wave streams its pages through two LDS slots of 6,400 bytes (the
// packed page of one kv head: K codes 3,072 | V codes 3,072 | K norms 128 |
// V norms 128), filled by direct global->LDS loads (7 per page).  Two pages are
// in flight while the wave computes a third from registers.
constexpr int kSlotBytes = 6400;
constexpr int kMaxPagesPerSplit = 256;  // the planner keeps splits within this
#define IQ_MAX_GROUP_BYTES (16 * 128 * 4)  // up to 16 query heads of fp32
constexpr int kDmaPerPage = 7;

typedef __attribute__((address_space(3))) void* lds_ptr;
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 4, 0, 0);
}
// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]); issued through the builtin so the compiler's own counter
// tracking knows which loads have landed.
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Issue the 7 loads of one page into `slot` (wave-uniform pointer).
__device__ __forceinline__ void issue_page(const DecodeArgs& a, int page, int g, int lane,
                                           uint8_t* slot) {
  const size_t base = ((size_t)page * a.hkv + g) * kPage;  // record index of slot 0
  const uint8_t* kb = a.k_codes + base * kRec + 16 * lane;
  const uint8_t* vb = a.v_codes + base * kRec + 16 * lane;
#pragma unroll
  for (int i = 0; i < 3; ++i) lds_dma16(kb + 1024 * i, slot + 1024 * i);
#pragma unroll
  for (int i = 0; i < 3; ++i) lds_dma16(vb + 1024 * i, slot + 3072 + 1024 * i);
  // lanes 0-31 bring the K norms (two per lane), lanes 32-63 the V norms
  const uint16_t* nb = (lane < 32 ? a.k_norms : a.v_norms) + base + 2 * (lane & 31);
  lds_dma4(nb, slot + 6144);
}

template <bool PACK8>
__device__ __forceinline__ void read_page(const uint8_t* slot, int lane, PageRegs<PACK8>& r) {
  const int col = lane & 15, jq = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    r.kc[rb] = *reinterpret_cast<const u3*>(slot + (16 * rb + col) * kRec + 12 * jq);
  const u4* vreg = reinterpret_cast<const u4*>(slot + 3072 + lane * kRec);
#pragma unroll
  for (int i = 0; i < 3; ++i) r.vr[i] = vreg[i];
  const uint16_t* kn = reinterpret_cast<const uint16_t*>(slot + 6144);
#pragma unroll
  for (int t = 0; t < PageRegs<PACK8>::NT; ++t) {
    const int tok = 16 * tile_block<PACK8>(t, col) + 4 * jq;
    r.kn[t] = *reinterpret_cast<const u2*>(kn + tok);
    r.vn[t] = *reinterpret_cast<const u2*>(kn + 64 + tok);
  }
}

__device__ __forceinline__ float norm_at(const u2& n, int r) {
  const uint32_t w = (r < 2) ? n[0] : n[1];
  return half_bits_to_float((r & 1) ? (w >> 16) : (w & 0xFFFFu));
}

struct PageState {
  float m_run, l_run, rho;  // running max (log2 units), partial sum, value-norm frame
  f4 acc[8];                // O'^T tiles: coordinates 32*(lane/16) + 4m + r, head lane%16
};

// Power-of-two frame for the value norms of a page: returns 2^(15 - e) for
// the largest fp16 norm bits with biased exponent e, so that vn * frame < 2.
__device__ __forceinline__ float norm_frame(uint32_t max_bits, float current) {
  if (max_bits == 0) return current;
  const int e16 = (int)((max_bits >> 10) & 0x1Fu);
  return __builtin_bit_cast(float, (uint32_t)(15 - e16 + 127) << 23);
}

template <bool PACK8>
__device__ __forceinline__ float column_max(float v) {
  if (PACK8) v = fmaxf(v, dpp_f<kRowRor8, 0xF>(v, v));
  return max_xor32(max_xor16(v));
}

// One page for one wave: scores on the matrix cores, online-softmax update,
// P~ V^ accumulation.  MASKED pages hold tokens at or beyond the length L.
template <bool PACK8, bool MASKED>
__device__ __forceinline__ void process_page(const PageRegs<PACK8>& cur, PageState& st, int tok0,
                                             int L, int lane, float fac, const h8 qhi[4],
                                             const h8 qlo[4]) {
  constexpr int NT = PageRegs<PACK8>::NT;
  const int col = lane & 15, jq = lane >> 4;
  f4 s[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    uint32_t z[8];
    group_to_selectors(cur.kc[rb].x, cur.kc[rb].y, cur.kc[rb].z, z);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u2 d0 = selector_to_f16(z[2 * kk]), d1 = selector_to_f16(z[2 * kk + 1]);
      const h8 av = __builtin_bit_cast(h8, u4{d0[0], d0[1], d1[0], d1[1]});
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qhi[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[kk], acc, 0, 0, 0);
    }
    s[rb] = acc;
  }

  float sc[NT][4];
  float mp = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tok = tok0 + 16 * tile_block<PACK8>(t, col) + 4 * jq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // with PACK8, columns 8-15 take the scores of the odd token block
      const float raw = PACK8 ? dpp_f<kRowShr8, 0xC>(s[2 * t][r], s[2 * t + 1][r]) : s[t][r];
      const float v = raw * (norm_at(cur.kn[t], r) * fac);
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
  mp = column_max<PACK8>(mp);
  if (PACK8) vbits = max(vbits, dpp_u<kRowRor8, 0xF>(vbits, vbits));
  vbits = umax_xor32(umax_xor16(vbits));
  const float m_new = fmaxf(st.m_run, mp);        // finite: the page has a valid token
  const float corr = fast_exp2(st.m_run - m_new);  // 0 on the first page
  const float rho_new = norm_frame(vbits, st.rho);
  const float rescale = corr * (rho_new / st.rho);
  if (__any(rescale != 1.0f)) {
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] *= rescale;
    st.l_run *= corr;
  }
  st.m_run = m_new;
  st.rho = rho_new;

  uint32_t pw[NT][2];  // P~ as f16 pairs: tokens r = 0,1 and r = 2,3 of each tile
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(sc[t][r] - m_new);  // masked tokens: 2^-inf = 0
      st.l_run += p[r];
      p[r] *= norm_at(vn[t], r) * rho_new;
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
      w[2] = dpp_u<kRowShl8, 0x3>(pw[th][0], pw[th][0]);
      w[3] = dpp_u<kRowShl8, 0x3>(pw[th][1], pw[th][1]);
    } else {
      w[0] = pw[2 * th][0];
      w[1] = pw[2 * th][1];
      w[2] = pw[2 * th + 1][0];
      w[3] = pw[2 * th + 1][1];
    }
    pb[th] = __builtin_bit_cast(h8, w);
  }

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
}

template <bool PACK8>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform: keeps the wave's page bookkeeping in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, jq = lane >> 4;
  const int pg_begin = split * a.pages_per_split;
  const int pg_first = pg_begin + wave;
  // Page ids of the wave's first two pages are fetched together with the length.
  const int* bt = a.block_table + (size_t)b * a.max_pages;
  const int page0 = (pg_first < a.max_pages) ? bt[pg_first] : 0;
  const int page1 = (pg_first + 4 < a.max_pages) ? bt[pg_first + 4] : 0;
  const int L = a.seq_lens[b];
  // (a length beyond the block table breaks the contract; never read past it)
  const int n_pages = min((L + kPage - 1) / kPage, a.max_pages);
  if (pg_begin >= n_pages) return;  // uniform for the workgroup
  const int pg_end = min(n_pages, pg_begin + a.pages_per_split);
  const int n_mine = pg_first < pg_end ? (pg_end - pg_first + 3) / 4 : 0;  // this wave's pages

  __shared__ __attribute__((aligned(16))) uint8_t s_ring[4][2][kSlotBytes];  // 51,200 B
  __shared__ __attribute__((aligned(16))) float s_rot[kRotFloats];           // 2,048 B
  __shared__ uint32_t s_q[32 * 64];  // Q' operands: [kstep*8 + dword][lane]
  __shared__ int s_pages[kMaxPagesPerSplit];  // the split's page ids
  __shared__ __attribute__((aligned(16))) uint8_t s_qraw[IQ_MAX_GROUP_BYTES];  // the group's queries
  __shared__ float s_qinv[16];
  __shared__ float s_m[4][16], s_l[4][16];

  // Everything the prologue needs arrives by direct-to-LDS loads issued before
  // the pages (lane-predicated): the split's page ids (a quarter per wave), and
  // in wave 0 the rotation blocks and the group's queries.  No load that the
  // compiler tracks in registers precedes the page loads, so no implicit wait
  // ever drains them.
  const int n_split = pg_end - pg_begin;
  int n_pre = 0;  // direct-to-LDS loads issued by this wave before its pages
  if (64 * wave < n_split) {
    if (64 * wave + lane < n_split) lds_dma4(bt + pg_begin + 64 * wave + lane, &s_pages[64 * wave]);
    ++n_pre;
  }
  const int qbytes = a.group * kD * (a.q_dtype == 0 ? 4 : 2);
  if (wave == 0) {
    const uint8_t* rg = reinterpret_cast<const uint8_t*>(a.rot + (size_t)g * kRotFloats) + 16 * lane;
    lds_dma16(rg, s_rot);
    lds_dma16(rg + 1024, reinterpret_cast<uint8_t*>(s_rot) + 1024);
    const uint8_t* qg = reinterpret_cast<const uint8_t*>(a.q) +
                        ((size_t)b * a.hq + (size_t)g * a.group) * kD * (a.q_dtype == 0 ? 4 : 2);
    for (int i = 0; 1024 * i < qbytes; ++i) {
      if (1024 * i + 16 * lane < qbytes) lds_dma16(qg + 1024 * i + 16 * lane, s_qraw + 1024 * i);
      ++n_pre;
    }
    n_pre += 2;
  }
  (void)n_pre;
  if (n_mine > 0) issue_page(a, page0, g, lane, s_ring[wave][0]);
  if (n_mine > 1) issue_page(a, page1, g, lane, s_ring[wave][1]);
  // The prologue loads have landed once at most the page loads are outstanding.
  if (n_mine > 1)
    __builtin_amdgcn_s_waitcnt(wait_vm(2 * kDmaPerPage));
  else if (n_mine == 1)
    __builtin_amdgcn_s_waitcnt(wait_vm(kDmaPerPage));
  else
    __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // Wave 0 rotates the queries with the four quarters of a head on adjacent
  // lanes (lane = 4h + j), so the cross-lane butterflies are DPP quad moves,
  // and writes Q' to LDS in the B-operand layout of the score MFMA: lane
  // h + 16j holds coordinates 32j..32j+31 of head h.
  if (wave == 0) {
    const int h = lane >> 2, j = lane & 3;
    float x[32];
    if (h < a.group) {
      lds_to_float32(s_qraw, h * kD + 32 * j, a.q_dtype, x);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.f;
    }
    wht128_quad(x, j);
    float z[32];
    so4_forward_quarter(s_rot, j, x, z);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(z[i]));
    mx = fmaxf(mx, quad_xor1(mx));
    mx = fmaxf(mx, quad_xor2(mx));
    int e = 0;
    frexpf(mx, &e);
    const float sc = (mx > 0.f) ? ldexpf(1.0f, 1 - e) : 1.0f;  // max |z*sc| in [1, 2)
    const int dst = h + 16 * j;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float v0 = z[8 * kk + 2 * d] * sc, v1 = z[8 * kk + 2 * d + 1] * sc;
        const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
        const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
        s_q[(kk * 8 + d) * 64 + dst] =
            (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        s_q[(kk * 8 + 4 + d) * 64 + dst] =
            (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
    }
    if (j == 0) s_qinv[h] = 1.0f / sc;
  }
  // LDS writes visible to the workgroup; unlike __syncthreads this does not
  // wait for the page loads still in flight.
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();

  h8 qhi[4], qlo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u4 dh, dl;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      dh[d] = s_q[(kk * 8 + d) * 64 + lane];
      dl[d] = s_q[(kk * 8 + 4 + d) * 64 + lane];
    }
    qhi[kk] = __builtin_bit_cast(h8, dh);
    qlo[kk] = __builtin_bit_cast(h8, dl);
  }
  // per-lane score factor of the lane's head column
  const float fac = a.score_factor * s_qinv[PACK8 ? (col & 7) : col];

  PageState st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.rho = 1.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.acc[m] = f4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < n_mine; ++i) {
    uint8_t* slot = s_ring[wave][i & 1];
    const int pg = pg_first + 4 * i;
    // page i has landed once at most the other slot's loads are outstanding
    if (i + 1 < n_mine)
      __builtin_amdgcn_s_waitcnt(wait_vm(kDmaPerPage));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
    PageRegs<PACK8> cur;
    read_page<PACK8>(slot, lane, cur);
    if (i + 2 < n_mine) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // slot read before it is refilled
      issue_page(a, s_pages[wave + 4 * (i + 2)], g, lane, slot);
    }
    if ((pg + 1) * kPage <= L)
      process_page<PACK8, false>(cur, st, pg * kPage, L, lane, fac, qhi, qlo);
    else
      process_page<PACK8, true>(cur, st, pg * kPage, L, lane, fac, qhi, qlo);
  }

  // ---- merge the four waves ----
  float l_col = st.l_run;
  if (PACK8) l_col += dpp_f<kRowRor8, 0xF>(l_col, l_col);
  l_col = sum_xor32(sum_xor16(l_col));
  const float fin = a.out_factor / st.rho;
  // The wave's own two slots hold its accumulator now (all its loads have
  // landed): values 0-15 in slot 0, 16-31 in slot 1.
  static_assert(kSlotBytes >= 16 * 64 * 4, "a slot holds half an accumulator");
  float* acc_lo = reinterpret_cast<float*>(s_ring[wave][0]);
  float* acc_hi = reinterpret_cast<float*>(s_ring[wave][1]);
#pragma unroll
  for (int k = 0; k < 32; ++k)
    (k < 16 ? acc_lo : acc_hi)[(k & 15) * 64 + lane] = st.acc[k >> 2][k & 3] * fin;
  if (jq == 0) {
    s_m[wave][col] = st.m_run;
    s_l[wave][col] = l_col;
  }
  __syncthreads();
  {
    const int part = wave;  // this thread merges values 8*part .. 8*part+7 of `lane`
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = s_m[w][col];
      M = fmaxf(M, mw[w]);
    }
    float wt[4], Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
      Ls += wt[w] * s_l[w][col];
    }
    if (col < a.group) {
      const size_t row = ((size_t)b * a.hq + (size_t)g * a.group + col) * a.splits + split;
      f4 o0, o1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // values 8*part + k and 8*part + 4 + k (slot 0 holds 0-15, slot 1 16-31)
          const float* wacc = reinterpret_cast<const float*>(s_ring[w][part < 2 ? 0 : 1]);
          s0 += wt[w] * wacc[((8 * part + k) & 15) * 64 + lane];
          s1 += wt[w] * wacc[((8 * part + 4 + k) & 15) * 64 + lane];
        }
        o0[k] = s0;
        o1[k] = s1;
      }
      f4* dst = reinterpret_cast<f4*>(a.ws_acc + row * kD + 32 * jq + 8 * part);
      dst[0] = o0;
      dst[1] = o1;
      if (jq == 0 && part == 0) {
        a.ws_ml[2 * row] = M;
        a.ws_ml[2 * row + 1] = Ls;
      }
    }
  }
}

// One workgroup per (query head, sequence): merge the split partials with all
// loads in flight at once, normalise, and rotate back: o = (H / sqrt(d)) B^T o'.
// Thread t adds coordinates 4*(t%32)..+3 over the splits s = t/32 (mod 8).
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  // A length above the planned maximum is outside the contract; never read
  // partials that the split kernel did not plan for.
  const int ns = min(a.splits, (n_pages + a.pages_per_split - 1) / a.pages_per_split);
  float* out = a.out + ((size_t)b * a.hq + hq) * kD;
  if (ns == 0) {
    if (tid < 32) reinterpret_cast<f4*>(out)[tid] = f4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  __shared__ float s_w[1024];
  __shared__ float s_red[8];
  __shared__ f4 s_part[8][32];
  const size_t row0 = ((size_t)b * a.hq + hq) * a.splits;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + row0;

  // maximum over splits
  float M = -INFINITY;
  for (int s = tid; s < ns; s += 256) M = fmaxf(M, ml[s].x);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) s_red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  // split weights and the normaliser
  float Ls = 0.f;
  for (int s = tid; s < ns; s += 256) {
    const float2 v = ml[s];
    const float w = fast_exp2(v.x - M);
    if (s < 1024) s_w[s] = w;
    Ls += w * v.y;
  }
  for (int o = 32; o > 0; o >>= 1) Ls += __shfl_xor(Ls, o);
  __syncthreads();
  if ((tid & 63) == 0) s_red[4 + (tid >> 6)] = Ls;
  __syncthreads();
  Ls = (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]);

  const int quad = tid & 31, grp = tid >> 5;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  const f4* src = reinterpret_cast<const f4*>(a.ws_acc + row0 * kD) + quad;
#pragma unroll 8
  for (int s = grp; s < ns; s += 8) {
    const float w = (s < 1024) ? s_w[s] : fast_exp2(ml[s].x - M);
    acc += w * src[(size_t)s * (kD / 4)];
  }
  s_part[grp][quad] = acc;
  __syncthreads();
  if (tid >= 64) return;
  // lane l owns coordinates 2l, 2l+1
  const int lane = tid;
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int gq = 0; gq < 8; ++gq) {
    const f4 v = s_part[gq][lane >> 1];
    o0 += (lane & 1) ? v[2] : v[0];
    o1 += (lane & 1) ? v[3] : v[1];
  }
  const float inv = 1.0f / Ls;
  o0 *= inv;
  o1 *= inv;
  // B^T on block lane/2: this lane holds block coordinates c0 = 2*(lane&1), c0+1.
  const float* mt = a.rot + (size_t)(hq / a.group) * kRotFloats + (lane >> 1) * 16;
  const float n0 = __shfl_xor(o0, 1), n1 = __shfl_xor(o1, 1);
  const bool odd = lane & 1;
  const float v0 = odd ? n0 : o0, v1 = odd ? n1 : o1, v2 = odd ? o0 : n0, v3 = odd ? o1 : n1;
  const int c0 = odd ? 2 : 0;
  float y0 = mt[c0] * v0 + mt[4 + c0] * v1 + mt[8 + c0] * v2 + mt[12 + c0] * v3;
  float y1 = mt[c0 + 1] * v0 + mt[5 + c0] * v1 + mt[9 + c0] * v2 + mt[13 + c0] * v3;
  // Walsh-Hadamard: coordinate distance 1 in-lane, 2..64 across lanes.
  {
    const float t0 = y0 + y1, t1 = y0 - y1;
    y0 = t0;
    y1 = t1;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float p0 = __shfl_xor(y0, m), p1 = __shfl_xor(y1, m);
    const float sgn = (lane & m) ? -1.0f : 1.0f;
    y0 = fmaf(sgn, y0, p0);
    y1 = fmaf(sgn, y1, p1);
  }
  const float nrm = 0.08838834764831845f;  // 1/sqrt(128)
  *reinterpret_cast<float2*>(out + 2 * lane) = make_float2(y0 * nrm, y1 * nrm);
}

DecodePlan plan_decode(int batch, int hkv, int max_seq_len, int num_cus) {
  const int max_pages = max(1, (max_seq_len + kPage - 1) / kPage);
  const long long units = (long long)max(1, batch) * max(1, hkv);
  long long target = 2LL * max(1, num_cus);
  if (const char* env = getenv("IQ_DECODE_TARGET_WGS")) {
    const long long v = atoll(env);
    if (v > 0) target = v;
  }
  long long splits = (target + units - 1) / units;
  splits = splits < 1 ? 1 : (splits > max_pages ? max_pages : splits);
  int pps = (int)((max_pages + splits - 1) / splits);
  if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
  DecodePlan p;
  p.pages_per_split = pps;
  p.splits = (max_pages + pps - 1) / pps;
  return p;
}

size_t decode_workspace_bytes(int batch, int hq, const DecodePlan& plan) {
  const size_t rows = (size_t)batch * hq * plan.splits;
  return rows * kD * sizeof(float) + rows * 2 * sizeof(float);
}

hipError_t launch_decode(const CacheView& c, const float* rot, const void* q, int q_dtype, int batch,
                         int hq, const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                         const DecodePlan& plan, float softmax_scale, float* out, void* workspace,
                         hipStream_t stream) {
  DecodeArgs a;
  a.k_codes = c.k_codes;
  a.k_norms = c.k_norms;
  a.v_codes = c.v_codes;
  a.v_norms = c.v_norms;
  a.hkv = c.hkv;
  a.rot = rot;
  a.q = q;
  a.q_dtype = q_dtype;
  a.hq = hq;
  a.group = hq / c.hkv;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.pages_per_split = plan.pages_per_split;
  a.splits = plan.splits;
  const double log2e = 1.4426950408889634;
  a.score_factor = (float)((double)softmax_scale * log2e / (128.0 * (double)kLevelScale));
  a.out_factor = (float)(1.0 / (sqrt(128.0) * (double)kLevelScale));
  const size_t rows = (size_t)batch * hq * plan.splits;
  a.ws_acc = reinterpret_cast<float*>(workspace);
  a.ws_ml = a.ws_acc + rows * kD;
  a.out = out;
  if (a.group <= 8)
    hipLaunchKernelGGL(decode_split_kernel<true>, dim3(plan.splits, c.hkv, batch), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, dim3(plan.splits, c.hkv, batch), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(hq, batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace iq
