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
// A workgroup (4 waves, 32 rows each) owns 128 rows of one kv head and walks
// the pages up to its causal limit.  Each page is unpacked once per workgroup
// into LDS as f16: K^ token-major (rows of 128 coordinates) and V^ as
// [coordinate][token], so every wave reads ready matrix-core operands.  V pages are stored in matrix-core order, so each
// thread converts one 12-byte chunk straight into four LDS rows.  Grid x is the kv head, so on an 8-XCD part the tiles
// of one kv head share an XCD's L2 when there are 8 kv heads.
#include <math.h>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

constexpr int kRowsPerTile = 128;
constexpr int kKStride = 136;   // halves per K^ row (128 + 8 pad)
constexpr int kVStride = 72;    // halves per V^T row (64 + 8 pad)

struct PrefillArgs {
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  int hkv;
  const float* rot;
  const void* q;
  int q_dtype;
  int n_q, hq, group, q_start;
  const int32_t* block_table;
  float score_factor;  // softmax_scale * log2(e) / (128 * alpha)
  float out_factor;    // 1 / (sqrt(128) * alpha)
  float* out;
};

__device__ __forceinline__ float norm_at2(const u2& n, int r) {
  const uint32_t w = (r < 2) ? n[0] : n[1];
  return half_bits_to_float((r & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__global__ __launch_bounds__(256, 1) void prefill_kernel(PrefillArgs a) {
  const int g = blockIdx.x, tile = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, jq = lane >> 4;
  const int qpt = kRowsPerTile / a.group;  // queries per tile
  const int q0 = tile * qpt;
  const int q_last = min(a.n_q, q0 + qpt) - 1;
  const int kv_end = a.q_start + q_last + 1;
  const int n_pages = (kv_end + kPage - 1) / kPage;

  __shared__ _Float16 s_k[kPage * kKStride];
  __shared__ _Float16 s_v[kD * kVStride];

  // ---- rotate this wave's 32 rows: lane (row col of block cb, quarter jq) ----
  h8 qhi[2][4], qlo[2][4];
  float fac[2];
  int qpos[2], qi_of[2], head_of[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int row = 32 * wave + 16 * cb + col;
    const int qi = q0 + row / a.group;
    const int h = row % a.group;
    qi_of[cb] = qi;
    head_of[cb] = h;
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

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f}, rho = 1.0f;
  f4 acc[2][8];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[cb][m] = f4{0.f, 0.f, 0.f, 0.f};

  // Per page, thread (lane, wave) loads K group jq of token 16*wave + col and
  // chunk `wave` of V region `lane` (V pages are stored in matrix-core order:
  // that chunk holds tokens 16*wave + 4*jq + r for coordinates 32*(col/4) +
  // 4m + col%4, m = 0..7).
  u3 kc, vc;
  auto load_codes = [&](int pg) {
    const int page = a.block_table[pg];
    const size_t base = ((size_t)page * a.hkv + g) * kPage;
    kc = *reinterpret_cast<const u3*>(a.k_codes + (base + 16 * wave + col) * kRec + 12 * jq);
    vc = *reinterpret_cast<const u3*>(a.v_codes + (base + lane) * kRec + 12 * wave);
  };
  if (n_pages > 0) load_codes(0);

  for (int pg = 0; pg < n_pages; ++pg) {
    // ---- unpack this page into LDS ----
    {
      uint32_t z[8];
      group_to_selectors(kc.x, kc.y, kc.z, z);
      u4* dst = reinterpret_cast<u4*>(s_k + (16 * wave + col) * kKStride + 32 * jq);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u2 d0 = selector_to_f16(z[2 * kk]), d1 = selector_to_f16(z[2 * kk + 1]);
        dst[kk] = u4{d0[0], d0[1], d1[0], d1[1]};
      }
      group_to_selectors(vc.x, vc.y, vc.z, z);
#pragma unroll
      for (int m = 0; m < 8; ++m)
        *reinterpret_cast<u2*>(s_v + (16 * m + col) * kVStride + 16 * wave + 4 * jq) = selector_to_f16(z[m]);
    }
    __syncthreads();
    if (pg + 1 < n_pages) load_codes(pg + 1);

    const int page = a.block_table[pg];
    const size_t nbase = ((size_t)page * a.hkv + g) * kPage;
    u2 kn[4], vn[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      kn[tb] = *reinterpret_cast<const u2*>(a.k_norms + nbase + 16 * tb + 4 * jq);
      vn[tb] = *reinterpret_cast<const u2*>(a.v_norms + nbase + 16 * tb + 4 * jq);
    }

    // ---- S^T tiles: [token block tb][row block cb] ----
    f4 s[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      s[tb][0] = f4{0.f, 0.f, 0.f, 0.f};
      s[tb][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 av = *reinterpret_cast<const h8*>(s_k + (16 * tb + col) * kKStride + 32 * jq + 8 * kk);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          s[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qhi[cb][kk], s[tb][cb], 0, 0, 0);
          s[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[cb][kk], s[tb][cb], 0, 0, 0);
        }
      }
    }

    // ---- online softmax per row (column of S^T) ----
    const int tok_base = pg * kPage + 4 * jq;
    float vmax = 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (tok_base + 16 * tb + r < kv_end) vmax = fmaxf(vmax, norm_at2(vn[tb], r));
    vmax = max_xor32(max_xor16(vmax));
    int e = 0;
    frexpf(vmax, &e);
    const float rho_new = (vmax > 0.f) ? ldexpf(1.0f, 1 - e) : rho;

    h8 pb[2][2];  // [token pair tp][row block cb]
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float sv[4][4];
      float mp = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = tok_base + 16 * tb + r;
          const float v = s[tb][cb][r] * norm_at2(kn[tb], r) * fac[cb];
          sv[tb][r] = (tok <= qpos[cb] && tok < kv_end) ? v : -INFINITY;
          mp = fmaxf(mp, sv[tb][r]);
        }
      mp = max_xor32(max_xor16(mp));
      const float m_new = fmaxf(m_run[cb], mp);
      // A row whose keys on this page are all masked keeps its state.
      const bool live = m_new != -INFINITY;
      const float corr = live ? exp2f(m_run[cb] - m_new) : 1.0f;
      const float rescale = corr * (rho_new / rho);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[cb][m] *= rescale;
      l_run[cb] *= corr;
      m_run[cb] = m_new;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = live ? exp2f(sv[tb][r] - m_new) : 0.f;
          l_run[cb] += p;
          const float pv = (sv[tb][r] == -INFINITY) ? 0.f : p * norm_at2(vn[tb], r) * rho_new;
          pb[tb >> 1][cb][4 * (tb & 1) + r] = (_Float16)pv;
        }
    }
    rho = rho_new;

    // ---- O'^T += V^T P~ ----
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const _Float16* vr = s_v + (16 * m + col) * kVStride + 32 * tp + 4 * jq;
        const h4 v0 = *reinterpret_cast<const h4*>(vr);
        const h4 v1 = *reinterpret_cast<const h4*>(vr + 16);
        const h8 av = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[tp][cb], acc[cb][m], 0, 0, 0);
      }
    }
    __syncthreads();  // LDS is rewritten by the next page
  }

  // ---- epilogue: normalise, rotate back (B^T then H / sqrt(d)), store ----
  const float* rot = a.rot + (size_t)g * kRotFloats;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l = sum_xor32(sum_xor16(l_run[cb]));
    const float scale = (l > 0.f) ? a.out_factor / (rho * l) : 0.f;
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
    if (qi_of[cb] < a.n_q) {
      f4* dst = reinterpret_cast<f4*>(a.out + ((size_t)qi_of[cb] * a.hq + (size_t)g * a.group + head_of[cb]) * kD + 32 * jq);
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
  hipLaunchKernelGGL(prefill_kernel, dim3(c.hkv, plan.row_tiles), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace iq
