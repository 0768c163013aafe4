// Chunked causal prefill attention on the packed 3-bit cache.
//
// "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention", abstract: attention directly on packed 3-bit
// K/V; FreeToken issue #141, Proposed Solution: GQA and faster prefill for
// the rotation-quantised family.  Query i of the chunk sits at position
// q_start + i and attends keys 0 .. q_start + i.
//
// The G query heads of a kv head share its keys, so the rows of one kv head
// (query x head-in-group) form a dense contraction against each 64-token page:
//   S^T[token][row] = K^[token] . Q'[row]     (v_mfma_f32_16x16x32_f16, Q' hi+lo)
//   O'^T[dim][row] += V^T[dim][token] P~[row][token]   (16x16x32)
//
// Work decomposition (gfx950): one workgroup of 4 waves per CU owns 128 rows
// of one kv head (32 rows = two row blocks per wave, so every K^ and V^
// fragment read from LDS feeds four matrix-core products; LDS read bandwidth,
// not the matrix cores, bounds a design with more, narrower waves) and walks
// the pages up to its causal limit.  Per page:
//   * raw pages arrive by direct-to-LDS loads three pages ahead (each wave
//     loads exactly the 12-byte groups it will unpack, so no wave waits for
//     another's loads);
//   * the unpacked page -- K^ token-major, V^ as [coordinate][token], both
//     alpha-scaled f16, and the fp16 norms -- is double-buffered in LDS, so a
//     page is unpacked while the previous one is multiplied and one barrier
//     per page suffices;
//   * only pages that reach past the smallest query position of the tile are
//     masked.
// The page ids of the whole causal range are staged in LDS once.
#include <math.h>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRowsPerTile = 32 * kPfWaves;  // 128 rows = queries x group heads
constexpr int kKStride = 136;   // halves per K^ row (128 + 8 pad)
constexpr int kVStride = 68;    // halves per V^T row (64 + 4 pad: 16 rows hit 16 distinct 8-byte bank slots)
constexpr int kRawWave = 2048;  // raw bytes per wave and page: K then V, 64 lanes x 16 B each
constexpr int kRawSlot = kPfWaves * kRawWave + 256;  // + the page's K and V norms
constexpr int kRawSlots = 3;

struct PrefillArgs {
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  int hkv, num_pages;
  const float* rot;
  const void* q;
  int q_dtype;
  int n_q, hq, group, q_start;
  const int32_t* block_table;
  float score_factor;  // softmax_scale * log2(e) / (128 * alpha)
  float out_factor;    // 1 / (sqrt(128) * alpha)
  float* out;
};

typedef __attribute__((address_space(3))) void* pf_lds_ptr;
__device__ __forceinline__ void pf_dma(const void* g, void* lds, int size) {
  if (size == 12)
    __builtin_amdgcn_global_load_lds(g, (pf_lds_ptr)lds, 12, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(g, (pf_lds_ptr)lds, 4, 0, 0);
}
// s_waitcnt vmcnt(n) (gfx9 encoding, other counters left alone)
#define IQ_PF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
constexpr int kPfWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

template <bool M>
struct PfMaskTag {
  static constexpr bool value = M;
};

__device__ __forceinline__ float norm_at2(const u2& n, int r) {
  const uint32_t w = (r < 2) ? n[0] : n[1];
  return half_bits_to_float((r & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// Raw loads of one page into a slot: wave w brings the K records of tokens
// 16w..16w+15 (lane l: token 16w + l/4, group l%4 -- 768 contiguous bytes)
// and chunk w of every V region (lane l: region l); wave 0 also the K norms
// (lanes 0-31) and V norms (lanes 32-63).
__device__ __forceinline__ void pf_issue(const PrefillArgs& a, int page_id, int g, int wave, int lane,
                                         uint8_t* slot) {
  // an id outside the cache (a table that breaks the contract) is clamped into
  // it, so a bad table gives wrong numbers, never an out-of-bounds read
  const uint32_t page = min((uint32_t)page_id, (uint32_t)a.num_pages - 1u);
  const size_t base = ((size_t)page * a.hkv + g) * kPage;
  uint8_t* dst = slot + wave * kRawWave;
  pf_dma(a.k_codes + base * kRec + 768 * wave + 12 * lane, dst, 12);
  pf_dma(a.v_codes + (base + lane) * kRec + 12 * wave, dst + 1024, 12);
  if (wave == 0) {
    const uint16_t* nb = (lane < 32 ? a.k_norms : a.v_norms) + base + 2 * (lane & 31);
    pf_dma(nb, slot + kPfWaves * kRawWave, 4);
  }
}

// Unpack this thread's two groups of a raw page (a K group and a V chunk)
// into the f16 buffers.
__device__ __forceinline__ void pf_unpack(const uint8_t* slot, int wave, int lane, _Float16* sk,
                                          _Float16* sv, uint16_t* snorm) {
  const uint8_t* raw = slot + wave * kRawWave + 16 * lane;
  const u3 ck = *reinterpret_cast<const u3*>(raw);
  const u3 cv = *reinterpret_cast<const u3*>(raw + 1024);
  uint32_t z[8];
  group_to_selectors(ck.x, ck.y, ck.z, z);
  {
    const int tok = 16 * wave + (lane >> 2), j = lane & 3;
    u4* dst = reinterpret_cast<u4*>(sk + tok * kKStride + 32 * j);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u2 d0 = selector_to_f16(z[2 * kk]), d1 = selector_to_f16(z[2 * kk + 1]);
      dst[kk] = u4{d0[0], d0[1], d1[0], d1[1]};
    }
  }
  group_to_selectors(cv.x, cv.y, cv.z, z);
  {
    // chunk c = wave of region (n, q): tokens 16c + 4q + r of coordinate row 16m + n
    const int n = lane & 15, q = lane >> 4;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *reinterpret_cast<u2*>(sv + (16 * m + n) * kVStride + 16 * wave + 4 * q) = selector_to_f16(z[m]);
  }
  if (wave == 0)
    reinterpret_cast<uint32_t*>(snorm)[lane] =
        reinterpret_cast<const uint32_t*>(slot + kPfWaves * kRawWave)[lane];
}

__global__ __launch_bounds__(kPfThreads, 1) void prefill_kernel(PrefillArgs a) {
  const int g = blockIdx.x, tile = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, jq = lane >> 4;
  const int qpt = kRowsPerTile / a.group;  // queries per tile
  const int q0 = tile * qpt;
  const int q_last = min(a.n_q, q0 + qpt) - 1;
  const int kv_end = a.q_start + q_last + 1;
  const int n_pages = (kv_end + kPage - 1) / kPage;
  // pages entirely at or before the smallest query position need no mask
  const int n_full = min(n_pages, (a.q_start + q0 + 1) / kPage);

  __shared__ __attribute__((aligned(16))) _Float16 s_k[2][kPage * kKStride];  // 34,816 B
  __shared__ __attribute__((aligned(16))) _Float16 s_v[2][kD * kVStride];     // 36,864 B
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kRawSlots][kRawSlot];  // 25,344 B
  __shared__ __attribute__((aligned(16))) uint16_t s_norm[2][2 * kPage];      // K | V norms
  __shared__ int s_pt[kPrefillMaxPages];                                       // 16,384 B

  // ---- page ids of the causal range (wave w: entries 1024w .. 1024w+1023) ----
  for (int i = 0; i < 16; ++i) {
    const int e0 = 1024 * wave + 64 * i;
    if (e0 < n_pages && e0 + lane < n_pages) pf_dma(a.block_table + e0 + lane, &s_pt[e0], 4);
  }

  // ---- this wave's 32 rows: Q' = T q (lane: row 16cb + col, quarter jq) ----
  h8 qhi[2][4], qlo[2][4];
  float fac[2];
  int qpos[2], qi_row[2], head_row[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = 32 * wave + 16 * cb + col;
    const int qi = q0 + row / a.group;
    const int h = row % a.group;
    qi_row[cb] = qi;
    head_row[cb] = h;
    qpos[cb] = (qi < a.n_q) ? a.q_start + qi : 0x7FFFFFFF;
    float x[32];
    if (qi < a.n_q) {
      load32(a.q, ((size_t)qi * a.hq + (size_t)g * a.group + h) * kD + 32 * jq, a.q_dtype, x);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.f;
    }
    wht128_spread<16, 32>(x, jq);
    float z[32];
    so4_forward_quarter(a.rot + (size_t)g * kRotFloats, jq, x, z);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(z[i]));
    mx = max_xor32(max_xor16(mx));
    int e = 0;
    frexpf(mx, &e);
    const float sc = (mx > 0.f) ? ldexpf(1.0f, 1 - e) : 1.0f;
    fac[cb] = a.score_factor / sc;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      h8 hi, lo;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float v = z[8 * kk + s] * sc;
        const _Float16 hv = (_Float16)v;
        hi[s] = hv;
        lo[s] = (_Float16)(v - (float)hv);
      }
      qhi[cb][kk] = hi;
      qlo[cb][kk] = lo;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // page-id loads landed (all counters)
  __syncthreads();

  const int per_page = (wave == 0) ? 3 : 2;  // raw loads this wave issues per page
  // first three pages in flight, the first unpacked
  for (int p = 0; p < 3 && p < n_pages; ++p) pf_issue(a, s_pt[p], g, wave, lane, s_raw[p]);
  {
    const int after = per_page * (min(n_pages, 3) - 1);
    if (after == 0) IQ_PF_WAIT_VM(0);
    else if (after == 2) IQ_PF_WAIT_VM(2);
    else if (after == 3) IQ_PF_WAIT_VM(3);
    else if (after == 4) IQ_PF_WAIT_VM(4);
    else IQ_PF_WAIT_VM(6);
    pf_unpack(s_raw[0], wave, lane, s_k[0], s_v[0], s_norm[0]);
  }
  __builtin_amdgcn_s_waitcnt(kPfWaitLgkm0);
  __builtin_amdgcn_s_barrier();

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  int rho_e = 0;
  f4 acc[2][8];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[cb][m] = f4{0.f, 0.f, 0.f, 0.f};

  // One page: products from the f16 buffers, online softmax, and the next
  // page's unpacking.  MASKED pages apply the causal and length masks.
  auto page_step = [&](int pg, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int f = pg & 1;
    if (pg + 3 < n_pages) pf_issue(a, s_pt[pg + 3], g, wave, lane, s_raw[pg % 3]);

    // ---- S^T tiles [token block tb][row block cb]: each K^ fragment feeds
    // both row blocks (hi and lo parts of Q') ----
    const _Float16* sk = s_k[f];
    f4 s[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      s[tb][0] = f4{0.f, 0.f, 0.f, 0.f};
      s[tb][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 av = *reinterpret_cast<const h8*>(sk + (16 * tb + col) * kKStride + 32 * jq + 8 * kk);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          s[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qhi[cb][kk], s[tb][cb], 0, 0, 0);
          s[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[cb][kk], s[tb][cb], 0, 0, 0);
        }
      }
    }
    // ---- unpack the next page into the other buffer while the products run
    // (independent of them: VALU and LDS work between matrix-core issues) ----
    if (pg + 1 < n_pages) {
      // loads of this wave still allowed in flight: those of pages pg+2, pg+3
      const int after = per_page * min(2, n_pages - 2 - pg);
      if (after == 0) IQ_PF_WAIT_VM(0);
      else if (after == 2) IQ_PF_WAIT_VM(2);
      else if (after == 3) IQ_PF_WAIT_VM(3);
      else if (after == 4) IQ_PF_WAIT_VM(4);
      else IQ_PF_WAIT_VM(6);
      pf_unpack(s_raw[(pg + 1) % 3], wave, lane, s_k[f ^ 1], s_v[f ^ 1], s_norm[f ^ 1]);
    }

    const uint16_t* nrm = s_norm[f];
    uint32_t vbits = 0;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const u2 vn = *reinterpret_cast<const u2*>(nrm + kPage + 16 * tb + 4 * jq);
      const us2 h0 = __builtin_bit_cast(us2, (uint32_t)vn[0]), h1 = __builtin_bit_cast(us2, (uint32_t)vn[1]);
      if (!MASKED) {
        const us2 m = __builtin_elementwise_max(h0, h1);
        vbits = max(vbits, (uint32_t)max(m[0], m[1]));
      } else {
        // tokens past the end of the chunk carry no norm
        const int t0 = pg * kPage + 16 * tb + 4 * jq;
        if (t0 < kv_end) vbits = max(vbits, (uint32_t)h0[0]);
        if (t0 + 1 < kv_end) vbits = max(vbits, (uint32_t)h0[1]);
        if (t0 + 2 < kv_end) vbits = max(vbits, (uint32_t)h1[0]);
        if (t0 + 3 < kv_end) vbits = max(vbits, (uint32_t)h1[1]);
      }
    }
    vbits = umax_xor32(umax_xor16(vbits));
    const int rho_new = (vbits == 0) ? rho_e : 15 - (int)((vbits >> 10) & 0x1Fu);
    const float frame = __builtin_amdgcn_ldexpf(1.0f, rho_new);
    const int tok_base = pg * kPage + 4 * jq;

    // ---- online softmax per row (column of S^T) ----
    h8 pb[2][2];  // [token pair tp][row block cb]
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float sv[4][4];
      float mp = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const u2 kn = *reinterpret_cast<const u2*>(nrm + 16 * tb + 4 * jq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = s[tb][cb][r] * (norm_at2(kn, r) * fac[cb]);
          if (MASKED) {
            const int tok = tok_base + 16 * tb + r;
            sv[tb][r] = (tok <= qpos[cb] && tok < kv_end) ? v : -INFINITY;
          } else {
            sv[tb][r] = v;
          }
          mp = fmaxf(mp, sv[tb][r]);
        }
      }
      mp = max_xor32(max_xor16(mp));
      const float m_new = fmaxf(m_run[cb], mp);
      // a row whose keys on this page are all masked keeps its state
      const bool live = !MASKED || m_new != -INFINITY;
      const float corr = live ? fast_exp2(m_run[cb] - m_new) : 1.0f;
      const float rescale = __builtin_amdgcn_ldexpf(corr, rho_new - rho_e);
      if (__any(rescale != 1.0f)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[cb][m] *= rescale;
      }
      l_run[cb] *= corr;
      m_run[cb] = m_new;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const u2 vn = *reinterpret_cast<const u2*>(nrm + kPage + 16 * tb + 4 * jq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // masked scores: 2^-inf = 0
          const float p = (!MASKED || live) ? fast_exp2(sv[tb][r] - m_new) : 0.f;
          l_run[cb] += p;
          pb[tb >> 1][cb][4 * (tb & 1) + r] = (_Float16)(p * (norm_at2(vn, r) * frame));
        }
      }
    }
    rho_e = rho_new;

    // ---- O'^T += V^T P~: each V^ fragment feeds both row blocks ----
    const _Float16* svp = s_v[f];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const _Float16* vr = svp + (16 * m + col) * kVStride + 32 * tp + 4 * jq;
        const h4 v0 = *reinterpret_cast<const h4*>(vr);
        const h4 v1 = *reinterpret_cast<const h4*>(vr + 16);
        const h8 av = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[tp][cb], acc[cb][m], 0, 0, 0);
      }
    }

    __builtin_amdgcn_s_waitcnt(kPfWaitLgkm0);
    __builtin_amdgcn_s_barrier();
  };
  int pg = 0;
  for (; pg < n_full; ++pg) page_step(pg, PfMaskTag<false>{});
  for (; pg < n_pages; ++pg) page_step(pg, PfMaskTag<true>{});

  // ---- epilogue: normalise, rotate back (B^T then H / sqrt(d)), store ----
  const float* rot = a.rot + (size_t)g * kRotFloats;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l = sum_xor32(sum_xor16(l_run[cb]));
    const float scale = (l > 0.f) ? __builtin_amdgcn_ldexpf(a.out_factor, -rho_e) / l : 0.f;
    float o[32], y[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) o[k] = acc[cb][k >> 2][k & 3] * scale;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const f4* mt = reinterpret_cast<const f4*>(rot + (8 * jq + bb) * 16);
      const f4 r0 = mt[0], r1 = mt[1], r2 = mt[2], r3 = mt[3];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        y[4 * bb + c] = r0[c] * o[4 * bb] + r1[c] * o[4 * bb + 1] + r2[c] * o[4 * bb + 2] +
                        r3[c] * o[4 * bb + 3];
    }
    wht128_spread<16, 32>(y, jq);
    if (qi_row[cb] < a.n_q) {
      f4* dst = reinterpret_cast<f4*>(a.out +
                                      ((size_t)qi_row[cb] * a.hq + (size_t)g * a.group + head_row[cb]) * kD +
                                      32 * jq);
      const float nrm = 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dst[i] = f4{y[4 * i] * nrm, y[4 * i + 1] * nrm, y[4 * i + 2] * nrm, y[4 * i + 3] * nrm};
    }
  }
}

PrefillPlan plan_prefill(int n_q, int hq, int hkv, int q_start, int num_cus) {
  (void)q_start;
  (void)num_cus;
  PrefillPlan p;
  const int group = hq / hkv;
  const int qpt = kRowsPerTile / group;
  p.row_tiles = (n_q + qpt - 1) / qpt;
  p.kv_splits = 1;
  return p;
}

size_t prefill_workspace_bytes(int n_q, int hq, const PrefillPlan& plan) {
  (void)n_q;
  (void)hq;
  (void)plan;
  return 0;
}

hipError_t launch_prefill(const CacheView& c, const float* rot, const void* q, int q_dtype, int n_q,
                          int hq, int q_start, const int32_t* block_table, int max_pages,
                          const PrefillPlan& plan, float softmax_scale, float* out, void* workspace,
                          hipStream_t stream) {
  (void)max_pages;
  (void)workspace;
  PrefillArgs a;
  a.k_codes = c.k_codes;
  a.k_norms = c.k_norms;
  a.v_codes = c.v_codes;
  a.v_norms = c.v_norms;
  a.hkv = c.hkv;
  a.num_pages = c.num_pages;
  a.rot = rot;
  a.q = q;
  a.q_dtype = q_dtype;
  a.n_q = n_q;
  a.hq = hq;
  a.group = hq / c.hkv;
  a.q_start = q_start;
  a.block_table = block_table;
  const double log2e = 1.4426950408889634;
  a.score_factor = (float)((double)softmax_scale * log2e / (128.0 * (double)kLevelScale));
  a.out_factor = (float)(1.0 / (sqrt(128.0) * (double)kLevelScale));
  a.out = out;
  hipLaunchKernelGGL(prefill_kernel, dim3(c.hkv, plan.row_tiles), dim3(kPfThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace iq
