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
// Per page and wave, the G query heads of the group are the 16 columns of
// 16x16 matrix-core tiles (padded with zero queries):
//   S^T[token][head] = K^[token][:] . Q'[head][:]   v_mfma_f32_16x16x32_f16, with
//       Q' split into an f16 high and low part (two MFMAs, ~2^-22 relative);
//       the K operand row of lane l is token l%16 and its 32 coordinates come
//       straight from one 12-byte group of the token's record.
//   V^ is transposed with an identity MFMA (exact) so that the contraction
//   index is the token, then O'^T[dim][head] += V^T . P~ (16x16x16).
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

struct PageRegs {
  u3 kc[4], vc[4];  // 12 code bytes of token 16*rb + (lane%16), group lane/16
  u2 kn[4], vn[4];  // fp16 norms of tokens 16*rb + 4*(lane/16) + 0..3
};

__device__ __forceinline__ void load_page(const DecodeArgs& a, int b, int g, int pg, int t, int jq,
                                          PageRegs& r) {
  const int page = a.block_table[(size_t)b * a.max_pages + pg];
  const size_t base = ((size_t)page * a.hkv + g) * kPage;  // record index of slot 0
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const size_t rec = base + 16 * rb + t;
    r.kc[rb] = *reinterpret_cast<const u3*>(a.k_codes + rec * kRec + 12 * jq);
    r.vc[rb] = *reinterpret_cast<const u3*>(a.v_codes + rec * kRec + 12 * jq);
    r.kn[rb] = *reinterpret_cast<const u2*>(a.k_norms + base + 16 * rb + 4 * jq);
    r.vn[rb] = *reinterpret_cast<const u2*>(a.v_norms + base + 16 * rb + 4 * jq);
  }
}

__device__ __forceinline__ float norm_at(const u2& n, int r) {
  const uint32_t w = (r < 2) ? n[0] : n[1];
  return half_bits_to_float((r & 1) ? (w >> 16) : (w & 0xFFFFu));
}

__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, jq = lane >> 4;
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const int pg_begin = split * a.pages_per_split;
  if (pg_begin >= n_pages) return;  // uniform for the workgroup
  const int pg_end = min(n_pages, pg_begin + a.pages_per_split);

  __shared__ uint32_t s_q[32 * 64];  // Q' operands: [kstep*8 + dword][lane]
  __shared__ float s_qinv[16];
  __shared__ float s_acc[4][32][64];
  __shared__ float s_m[4][16], s_l[4][16];

  // Issue the first page's loads before anything else.
  PageRegs cur;
  int pg = pg_begin + wave;
  if (pg < pg_end) load_page(a, b, g, pg, col, jq, cur);

  // Wave 0 rotates the group's queries: lane (head col, quarter jq) holds
  // coordinates 32jq..32jq+31, which is exactly the B-operand layout below.
  if (wave == 0) {
    float x[32];
    if (col < a.group) {
      load32(a.q, ((size_t)b * a.hq + (size_t)g * a.group + col) * kD + 32 * jq, a.q_dtype, x);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.f;
    }
    wht128_quad<16, 32>(x, jq);
    float z[32];
    so4_forward_quarter(a.rot + (size_t)g * kRotFloats, jq, x, z);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(z[i]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    int e = 0;
    frexpf(mx, &e);
    const float sc = (mx > 0.f) ? ldexpf(1.0f, 1 - e) : 1.0f;  // max |z*sc| in [1, 2)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float v0 = z[8 * kk + 2 * d] * sc, v1 = z[8 * kk + 2 * d + 1] * sc;
        const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
        const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
        s_q[(kk * 8 + d) * 64 + lane] =
            (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        s_q[(kk * 8 + 4 + d) * 64 + lane] =
            (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
    }
    if (jq == 0) s_qinv[col] = 1.0f / sc;
  }
  __syncthreads();

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
  const float fac = a.score_factor * s_qinv[col];
  h4 ident;
#pragma unroll
  for (int s = 0; s < 4; ++s) ident[s] = (4 * jq + s == col) ? (_Float16)1.0f : (_Float16)0.0f;

  float m_run = -INFINITY, l_run = 0.f, rho = 1.0f;
  f4 acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};

  for (; pg < pg_end; pg += 4) {
    PageRegs nxt;
    const bool more = pg + 4 < pg_end;
    if (more) load_page(a, b, g, pg + 4, col, jq, nxt);
    const int tok_base = pg * kPage + 4 * jq;

    // ---- scores (log2 units) ----
    float sc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      uint32_t z[8];
      group_to_selectors(cur.kc[rb].x, cur.kc[rb].y, cur.kc[rb].z, z);
      f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u2 d0 = selector_to_f16(z[2 * kk]), d1 = selector_to_f16(z[2 * kk + 1]);
        const h8 av = __builtin_bit_cast(h8, u4{d0[0], d0[1], d1[0], d1[1]});
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qhi[kk], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[kk], s, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tok_base + 16 * rb + r;
        const float v = s[r] * norm_at(cur.kn[rb], r) * fac;
        sc[rb][r] = (tok < L) ? v : -INFINITY;
      }
    }

    // ---- online softmax update ----
    float mp = -INFINITY, vmax = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mp = fmaxf(mp, sc[rb][r]);
        if (tok_base + 16 * rb + r < L) vmax = fmaxf(vmax, norm_at(cur.vn[rb], r));
      }
    mp = fmaxf(mp, __shfl_xor(mp, 16));
    mp = fmaxf(mp, __shfl_xor(mp, 32));
    vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
    vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
    const float m_new = fmaxf(m_run, mp);            // finite: the page has a valid token
    const float corr = exp2f(m_run - m_new);         // 0 on the first page
    int e = 0;
    frexpf(vmax, &e);
    const float rho_new = (vmax > 0.f) ? ldexpf(1.0f, 1 - e) : rho;
    const float rescale = corr * (rho_new / rho);
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] *= rescale;
    l_run *= corr;
    m_run = m_new;
    rho = rho_new;

    h4 pb[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(sc[rb][r] - m_new);  // masked tokens: exp2(-inf) = 0
        l_run += p;
        const bool valid = tok_base + 16 * rb + r < L;
        pb[rb][r] = (_Float16)(valid ? p * norm_at(cur.vn[rb], r) * rho : 0.f);
      }

    // ---- P~ V^ on the matrix cores ----
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      uint32_t z[8];
      group_to_selectors(cur.vc[rb].x, cur.vc[rb].y, cur.vc[rb].z, z);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const h4 av = __builtin_bit_cast(h4, selector_to_f16(z[m]));
        const f4 t = __builtin_amdgcn_mfma_f32_16x16x16f16(av, ident, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const h4 tv = {(_Float16)t[0], (_Float16)t[1], (_Float16)t[2], (_Float16)t[3]};
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(tv, pb[rb], acc[m], 0, 0, 0);
      }
    }
    if (more) cur = nxt;
  }

  // ---- merge the four waves ----
  float l_col = l_run + __shfl_xor(l_run, 16);
  l_col += __shfl_xor(l_col, 32);
  const float fin = a.out_factor / rho;
#pragma unroll
  for (int k = 0; k < 32; ++k) s_acc[wave][k][lane] = acc[k >> 2][k & 3] * fin;
  if (jq == 0) {
    s_m[wave][col] = m_run;
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
      wt[w] = (mw[w] == -INFINITY) ? 0.f : exp2f(mw[w] - M);
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
          s0 += wt[w] * s_acc[w][8 * part + k][lane];
          s1 += wt[w] * s_acc[w][8 * part + 4 + k][lane];
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

// One wave per (query head, sequence): merge the split partials, normalise,
// and rotate back: o = (H / sqrt(d)) B^T o'.  Lane l owns coordinates 2l, 2l+1.
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  // A length above the planned maximum is outside the contract; never read
  // partials that the split kernel did not plan for.
  const int ns = min(a.splits, (n_pages + a.pages_per_split - 1) / a.pages_per_split);
  float* out = a.out + ((size_t)b * a.hq + hq) * kD + 2 * lane;
  if (ns == 0) {
    out[0] = 0.f;
    out[1] = 0.f;
    return;
  }
  const size_t row0 = ((size_t)b * a.hq + hq) * a.splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_ml[2 * (row0 + s)]);
  float Ls = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float m = a.ws_ml[2 * (row0 + s)], l = a.ws_ml[2 * (row0 + s) + 1];
    const float w = exp2f(m - M);
    const float2 v = *reinterpret_cast<const float2*>(a.ws_acc + (row0 + s) * kD + 2 * lane);
    Ls += w * l;
    o0 += w * v.x;
    o1 += w * v.y;
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
  *reinterpret_cast<float2*>(out) = make_float2(y0 * nrm, y1 * nrm);
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
  const int pps = (int)((max_pages + splits - 1) / splits);
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
  hipLaunchKernelGGL(decode_split_kernel, dim3(plan.splits, c.hkv, batch), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(hq, batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace iq
