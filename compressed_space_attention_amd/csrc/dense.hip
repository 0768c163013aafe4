// Uncompressed bf16 paged decode: the baseline the packed path is measured
// against, on the same paging, planning and merge.
//
// "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention", abstract: the packed attention avoids
// materialising full-precision KV state.  This file is that full-precision
// state in a paged cache and a decode kernel for it, so that the byte
// reduction of the packed cache becomes a measured time on the same GPU.
//
// Cache (bf16): K token-major [pages][Hkv][64][128]; V coordinate-major
// [pages][Hkv][128][64], the value layout common in paged decode engines,
// because the P.V contraction runs over tokens and each matrix-core lane then
// reads eight tokens of one coordinate contiguously.
//
// Decode: grid (splits, Hkv, B), eight waves; the split's tokens are 32-token
// chunks taken round-robin by the waves, each loaded straight into registers
// (no LDS staging) one chunk ahead of its use.  Per chunk and wave:
//   S^T[token][head] = K[token][:] . Q[head][:]          v_mfma_f32_16x16x32_bf16
//   online softmax in log2 units per head column
//   O^T[coord][head] += V^T[coord][token] . P^T[token][head], with P in bf16
//   high + low parts (two products, ~2^-16 relative)
// and the same partial rows (m, l, acc[128]) and merge as the packed path.
//
// FP8 fallback (FreeToken issue #141, Proposed Solution: standard FP8 KV as
// the fallback format): the same layouts with one byte per value, OCP E4M3
// (bias 7, 3 mantissa bits, largest finite 448, no infinities) of x / scale
// with one scale per tensor and cache.  Every E4M3 value is exact in f16, so
// the kernel converts bytes to f16 with the gfx950 conversion instruction and
// runs the same products on v_mfma_f32_16x16x32_f16 (q converted from bf16 to
// f16, P as f16 high + low parts); K's scale joins the score factor, V's the
// partial accumulator.
#include <math.h>

#include <type_traits>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
typedef short ss2 __attribute__((ext_vector_type(2)));

// Cache formats (template parameter FMT).
constexpr int kFmtBf16 = 0, kFmtFp8 = 1;

// Four E4M3 bytes -> four f16 values (exact).
__device__ __forceinline__ u2 fp8x4_to_f16(uint32_t w) {
  const hh2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const hh2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return u2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
// Two floats -> two E4M3 bytes (round to nearest even), saturated at +-448,
// in the low 16 bits.
__device__ __forceinline__ uint32_t f32x2_to_fp8(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  const ss2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ss2{0, 0}, a, b, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r) & 0xFFFFu;
}

constexpr int kDenseChunk = 32;       // tokens per wave step (half a page)
constexpr int kDenseWaves = 8;
constexpr int kDenseMaxPagesPerSplit = 512;

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

// ---------------------------------------------------------------------------
// Append: one thread per (token, kv head, 8 coordinates) and tensor; K rows go
// to their slot as one 16-byte store, V values to eight coordinate rows.
// ---------------------------------------------------------------------------
template <int DT, int FMT>
__global__ __launch_bounds__(256) void dense_append_kernel(
    const void* __restrict__ k, const void* __restrict__ v, const int32_t* __restrict__ seq_idx,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_table, long long n_vec,
    int hkv, int max_pages, int num_pages, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
    float inv_k_scale, float inv_v_scale) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= 2 * n_vec * 16) return;
  const int part = (int)(gid & 15);  // coordinates 8 part .. 8 part + 7
  const long long gv = gid >> 4;
  const int which = gv >= n_vec;
  const long long vi = gv - (which ? n_vec : 0);
  const int tok = (int)(vi / hkv);
  const int head = (int)(vi - (long long)tok * hkv);
  const int p = pos[tok];
  const int si = seq_idx[tok];
  float x[8];
  {
    const size_t idx = (size_t)vi * kD + 8 * part;
    const void* src = which ? v : k;
    if (DT == 0) {
      const f4* a = reinterpret_cast<const f4*>(reinterpret_cast<const float*>(src) + idx);
      const f4 a0 = a[0], a1 = a[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[i] = a0[i]; x[4 + i] = a1[i]; }
    } else {
      const u4 a = *reinterpret_cast<const u4*>(reinterpret_cast<const uint16_t*>(src) + idx);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = a[i];
        if (DT == 1) {
          x[2 * i] = __builtin_bit_cast(float, w << 16);
          x[2 * i + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
        } else {
          x[2 * i] = half_bits_to_float(w & 0xFFFFu);
          x[2 * i + 1] = half_bits_to_float(w >> 16);
        }
      }
    }
  }
  const bool in_table = (unsigned)p < (unsigned)max_pages * kPage;
  const int page = in_table ? block_table[(size_t)si * max_pages + (p >> 6)] : -1;
  if ((unsigned)page >= (unsigned)num_pages) return;  // skipped, as the packed append
  const int slot = p & 63;
  const size_t blk = (size_t)page * hkv + head;
  if (FMT == kFmtBf16) {
    uint16_t* kh = reinterpret_cast<uint16_t*>(kc);
    uint16_t* vh = reinterpret_cast<uint16_t*>(vc);
    if (!which) {
      u4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)to_bf16_bits(x[2 * i]) | ((uint32_t)to_bf16_bits(x[2 * i + 1]) << 16);
      *reinterpret_cast<u4*>(kh + (blk * kPage + slot) * kD + 8 * part) = w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) vh[(blk * kD + 8 * part + i) * kPage + slot] = to_bf16_bits(x[i]);
    }
  } else {
    const float inv = which ? inv_v_scale : inv_k_scale;
    uint32_t b[4];  // bytes of coordinates 2i, 2i + 1
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = f32x2_to_fp8(x[2 * i] * inv, x[2 * i + 1] * inv);
    if (!which) {
      *reinterpret_cast<u2*>(kc + (blk * kPage + slot) * kD + 8 * part) =
          u2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vc[(blk * kD + 8 * part + i) * kPage + slot] = (uint8_t)(b[i >> 1] >> (8 * (i & 1)));
    }
  }
}

hipError_t launch_dense_append(const DenseCacheView& c, const void* k, const void* v, int dtype,
                               int n_tokens, const int32_t* seq_idx, const int32_t* pos,
                               const int32_t* block_table, int max_pages, hipStream_t stream) {
  const long long n_vec = (long long)n_tokens * c.hkv;
  const long long threads = 2 * n_vec * 16;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  const float ik = 1.0f / c.k_scale, iv = 1.0f / c.v_scale;
#define IQ_DAPP(DT, F)                                                                               \
  hipLaunchKernelGGL((dense_append_kernel<DT, F>), dim3(blocks), dim3(256), 0, stream, k, v, seq_idx, \
                     pos, block_table, n_vec, c.hkv, max_pages, c.num_pages, c.k, c.v, ik, iv)
#define IQ_DAPP_F(F)               \
  if (dtype == 0) IQ_DAPP(0, F);     \
  else if (dtype == 1) IQ_DAPP(1, F); \
  else IQ_DAPP(2, F)
  if (c.format == kFmtFp8) { IQ_DAPP_F(kFmtFp8); }
  else { IQ_DAPP_F(kFmtBf16); }
#undef IQ_DAPP_F
#undef IQ_DAPP
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode split kernel.
// ---------------------------------------------------------------------------
struct DenseArgs {
  const uint8_t* k;
  const uint8_t* v;
  int num_pages, hkv;
  float score_factor;  // softmax_scale * log2(e) (* K's scale for FP8)
  float v_scale;       // FP8: V's scale, applied to the partial accumulator
  float* ws_acc;       // [B][Hq][splits][128]
  float* ws_ml;        // [B][Hq][splits][2]
};

// One 32-token chunk of one kv head, in this lane's operand layout.
//   K: token 16t + lane%16, coordinates 32kk + 8(lane/16) .. +7
//   V: coordinate 16m + lane%16, tokens 4(lane/16) + 16h .. +3
template <int FMT> struct DenseChunk;
template <> struct DenseChunk<kFmtBf16> {
  u4 k[2][4];
  u2 v[8][2];
};
template <> struct DenseChunk<kFmtFp8> {
  u2 k[2][4];
  uint32_t v[8][2];
};

template <int FMT>
__device__ __forceinline__ void load_chunk(const DenseArgs& a, int page, int g, int half, int lane,
                                           DenseChunk<FMT>& c) {
  constexpr int E = FMT == kFmtFp8 ? 1 : 2;  // bytes per value
  using KT = decltype(c.k[0][0]);
  using VT = decltype(c.v[0][0]);
  const int col = lane & 15, jq = lane >> 4;
  const size_t blk = (size_t)page * a.hkv + g;
  const uint8_t* kb = a.k + ((blk * kPage + kDenseChunk * half + col) * kD + 8 * jq) * E;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      c.k[t][kk] = *reinterpret_cast<const typename std::remove_reference<KT>::type*>(
          kb + (16 * t * kD + 32 * kk) * E);
  const uint8_t* vb = a.v + ((blk * kD + col) * kPage + kDenseChunk * half + 4 * jq) * E;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      c.v[m][h] = *reinterpret_cast<const typename std::remove_reference<VT>::type*>(
          vb + (16 * m * kPage + 16 * h) * E);
}

struct DenseState {
  float m_run, l_run;
  f4 acc[8];  // O^T: coordinates 16m + 4(lane/16) + r, head lane%16
};

// One matrix-core product in the format's operand type.
template <int FMT>
__device__ __forceinline__ f4 dense_mfma(const u4& a, const u4& b, const f4& c) {
  if constexpr (FMT == kFmtFp8)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b),
                                                   c, 0, 0, 0);
}

// MASKED: the chunk holds tokens at or beyond L (their scores are -inf and
// their values are zeroed, so never-written slots cannot inject NaN).
// qb: the queries as the B operand (bf16, or f16 for the FP8 format).
template <bool MASKED, int FMT>
__device__ __forceinline__ void dense_chunk_step(DenseChunk<FMT> c, DenseState& st, int tok0, int L,
                                                 int lane, float fac, const u4 qb[4]) {
  const int jq = lane >> 4;
  f4 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u4 ka;
      if constexpr (FMT == kFmtFp8) {
        const u2 lo = fp8x4_to_f16(c.k[t][kk][0]), hi = fp8x4_to_f16(c.k[t][kk][1]);
        ka = u4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        ka = c.k[t][kk];
      }
      acc = dense_mfma<FMT>(ka, qb[kk], acc);
    }
    s[t] = acc;
  }
  float sc[2][4];
  float mp = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tok0 + 16 * t + 4 * jq + r;
      sc[t][r] = (!MASKED || tok < L) ? s[t][r] * fac : -INFINITY;
      mp = fmaxf(mp, sc[t][r]);
    }
  if (MASKED) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t0 = tok0 + 16 * h + 4 * jq;
      if constexpr (FMT == kFmtFp8) {
        const uint32_t mk = (t0 < L ? 0xFFu : 0u) | (t0 + 1 < L ? 0xFF00u : 0u) |
                            (t0 + 2 < L ? 0xFF0000u : 0u) | (t0 + 3 < L ? 0xFF000000u : 0u);
#pragma unroll
        for (int m = 0; m < 8; ++m) c.v[m][h] &= mk;
      } else {
        const uint32_t m0 = (t0 < L ? 0xFFFFu : 0u) | (t0 + 1 < L ? 0xFFFF0000u : 0u);
        const uint32_t m1 = (t0 + 2 < L ? 0xFFFFu : 0u) | (t0 + 3 < L ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          c.v[m][h][0] &= m0;
          c.v[m][h][1] &= m1;
        }
      }
    }
  }
  mp = max_xor32(max_xor16(mp));
  const float m_new = fmaxf(st.m_run, mp);  // finite: the chunk has a valid token
  const float corr = fast_exp2(st.m_run - m_new);
  if (__any(corr != 1.0f)) {
#pragma unroll
    for (int m = 0; m < 8; ++m) st.acc[m] *= corr;
    st.l_run *= corr;
  }
  st.m_run = m_new;
  // P^T operand: k index 8 jq + i holds token 4 jq + i (i < 4, first tile)
  // or 16 + 4 jq + i - 4 (second tile): exactly this lane's score rows.
  float p[8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[4 * t + r] = fast_exp2(sc[t][r] - m_new);
      st.l_run += p[4 * t + r];
    }
  u4 ph, pl;  // P as high + low parts in the operand type
  if constexpr (FMT == kFmtFp8) {
    h8 h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = (_Float16)p[i];
      l[i] = (_Float16)(p[i] - (float)h[i]);
    }
    ph = __builtin_bit_cast(u4, h);
    pl = __builtin_bit_cast(u4, l);
  } else {
    bf8 h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = (__bf16)p[i];
      l[i] = (__bf16)(p[i] - (float)h[i]);
    }
    ph = __builtin_bit_cast(u4, h);
    pl = __builtin_bit_cast(u4, l);
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    u4 va;
    if constexpr (FMT == kFmtFp8) {
      const u2 t0 = fp8x4_to_f16(c.v[m][0]), t1 = fp8x4_to_f16(c.v[m][1]);
      va = u4{t0[0], t0[1], t1[0], t1[1]};
    } else {
      va = u4{c.v[m][0][0], c.v[m][0][1], c.v[m][1][0], c.v[m][1][1]};
    }
    st.acc[m] = dense_mfma<FMT>(va, ph, st.acc[m]);
    st.acc[m] = dense_mfma<FMT>(va, pl, st.acc[m]);
  }
}

template <int FMT>
__global__ __launch_bounds__(64 * kDenseWaves, 1) void dense_decode_split_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, int max_pages, int pages_per_split, int hq, int group, int splits,
    DenseArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, jq = lane >> 4;
  __shared__ int s_pages[kDenseMaxPagesPerSplit];
  __shared__ float s_acc[kDenseWaves][32][64];  // 64 KB: the waves' accumulators
  __shared__ float s_m[kDenseWaves][16], s_l[kDenseWaves][16];

  const int L = seq_lens[b];
  const int n_pages = min((L + kPage - 1) / kPage, max_pages);
  const int pg_begin = split * pages_per_split;
  if (pg_begin >= n_pages) {  // empty split: zero weight in the merge
    if (tid < group) {
      const size_t row = ((size_t)b * hq + (size_t)g * group + tid) * splits + split;
      a.ws_ml[2 * row] = -INFINITY;
      a.ws_ml[2 * row + 1] = 0.f;
    }
    return;
  }
  const int pg_end = min(n_pages, pg_begin + pages_per_split);
  const int* bt = block_table + (size_t)b * max_pages;
  for (int i = tid; i < pg_end - pg_begin; i += 64 * kDenseWaves)
    s_pages[i] = min(max(bt[pg_begin + i], 0), a.num_pages - 1);
  // queries of the group as the B operand: head lane%16, coordinates 32kk + 8jq ..
  u4 qb[4];
  {
    const uint16_t* qh = q + ((size_t)b * hq + (size_t)g * group + col) * kD + 8 * jq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u4 w = col < group ? *reinterpret_cast<const u4*>(qh + 32 * kk) : u4{0u, 0u, 0u, 0u};
      if constexpr (FMT == kFmtFp8) {  // bf16 -> f16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const hh2 hv = {(_Float16)__builtin_bit_cast(float, w[i] << 16),
                          (_Float16)__builtin_bit_cast(float, w[i] & 0xFFFF0000u)};
          w[i] = __builtin_bit_cast(uint32_t, hv);
        }
      }
      qb[kk] = w;
    }
  }
  __syncthreads();

  const int tok_begin = pg_begin * kPage;
  const int tok_end = min(L, pg_end * kPage);
  const int n_chunks = (tok_end - tok_begin + kDenseChunk - 1) / kDenseChunk;
  const float fac = a.score_factor;
  DenseState st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) st.acc[m] = f4{0.f, 0.f, 0.f, 0.f};

  // Two register buffers in turn: while one chunk is computed the next one
  // of this wave is in flight.  Loads are unconditional (a prefetch past the
  // split's end repeats its last chunk: lines already in cache), so every
  // wait is a plain count of the loads issued since.
  const int last = n_chunks - 1;
  auto fetch = [&](int chunk, DenseChunk<FMT>& dst) {
    const int cc = min(chunk, last);
    load_chunk<FMT>(a, s_pages[cc >> 1], g, cc & 1, lane, dst);
  };
  auto step = [&](const DenseChunk<FMT>& src, int chunk) {
    const int tok0 = tok_begin + kDenseChunk * chunk;
    if (tok0 + kDenseChunk <= L) dense_chunk_step<false, FMT>(src, st, tok0, L, lane, fac, qb);
    else dense_chunk_step<true, FMT>(src, st, tok0, L, lane, fac, qb);
  };
  DenseChunk<FMT> b0, b1;
  fetch(wave, b0);
  fetch(wave + kDenseWaves, b1);
  for (int c = wave; c < n_chunks; c += 2 * kDenseWaves) {
    step(b0, c);
    fetch(c + 2 * kDenseWaves, b0);
    if (c + kDenseWaves >= n_chunks) break;
    step(b1, c + kDenseWaves);
    fetch(c + 3 * kDenseWaves, b1);
  }

  // ---- merge the waves through LDS ----
  float l_col = sum_xor32(sum_xor16(st.l_run));
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_acc[wave][4 * m + r][lane] = st.acc[m][r];
  if (jq == 0) {
    s_m[wave][col] = st.m_run;
    s_l[wave][col] = l_col;
  }
  __syncthreads();
  {
    // this thread merges values 4 wave .. 4 wave + 3 of `lane`: coordinates
    // 16 m + 4 jq + r with 4 m + r = 4 wave + r'
    float mw[kDenseWaves], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDenseWaves; ++w) {
      mw[w] = s_m[w][col];
      M = fmaxf(M, mw[w]);
    }
    float wt[kDenseWaves], Ls = 0.f;
#pragma unroll
    for (int w = 0; w < kDenseWaves; ++w) {
      wt[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
      Ls += wt[w] * s_l[w][col];
    }
    if (col < group) {
      const size_t row = ((size_t)b * hq + (size_t)g * group + col) * splits + split;
      const float vs = FMT == kFmtFp8 ? a.v_scale : 1.0f;
      f4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kDenseWaves; ++w) sum += wt[w] * s_acc[w][4 * wave + r][lane];
        o[r] = sum * vs;
      }
      // value index 4 wave + r = 4 m + r: coordinate 16 wave + 4 jq + r
      *reinterpret_cast<f4*>(a.ws_acc + row * kD + 16 * wave + 4 * jq) = o;
      if (jq == 0 && wave == 0) {
        a.ws_ml[2 * row] = M;
        a.ws_ml[2 * row + 1] = Ls;
      }
    }
  }
}

DecodePlan plan_dense_decode(int batch, int hkv, int max_seq_len, int num_cus) {
  const int max_pages = max(1, (max_seq_len + kPage - 1) / kPage);
  const long long units = (long long)max(1, batch) * max(1, hkv);
  const long long cus = max(1, num_cus);
  long long splits = (cus + units - 1) / units;
  if (splits > max_pages) splits = max_pages;
  long long pps = (max_pages + splits - 1) / splits;
  if (pps > kDenseMaxPagesPerSplit) pps = kDenseMaxPagesPerSplit;
  DecodePlan p{};
  p.waves = kDenseWaves;
  p.pages_per_split = (int)pps;
  p.splits = (int)((max_pages + pps - 1) / pps);
  return p;
}

hipError_t launch_dense_decode(const DenseCacheView& c, const void* q, int batch, int hq,
                               const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                               const DecodePlan& plan, float softmax_scale, float* out,
                               void* workspace, hipStream_t stream) {
  const bool fp8 = c.format == kFmtFp8;
  DenseArgs a;
  a.k = c.k;
  a.v = c.v;
  a.num_pages = c.num_pages;
  a.hkv = c.hkv;
  a.score_factor = (float)((double)softmax_scale * 1.4426950408889634 * (fp8 ? (double)c.k_scale : 1.0));
  a.v_scale = fp8 ? c.v_scale : 1.0f;
  const size_t rows = (size_t)batch * hq * plan.splits;
  // the partials follow the counter region every decode workspace starts with
  a.ws_acc = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kWsCounterBytes);
  a.ws_ml = a.ws_acc + rows * kD;
  const int group = hq / c.hkv;
  const dim3 grid(plan.splits, c.hkv, batch);
  const uint16_t* qh = static_cast<const uint16_t*>(q);
  if (fp8)
    hipLaunchKernelGGL(dense_decode_split_kernel<kFmtFp8>, grid, dim3(64 * kDenseWaves), 0, stream,
                       block_table, seq_lens, qh, max_pages, plan.pages_per_split, hq, group, plan.splits, a);
  else
    hipLaunchKernelGGL(dense_decode_split_kernel<kFmtBf16>, grid, dim3(64 * kDenseWaves), 0, stream,
                       block_table, seq_lens, qh, max_pages, plan.pages_per_split, hq, group, plan.splits, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_merge(false, nullptr, a.ws_acc, a.ws_ml, plan.splits, batch, hq, group, nullptr,
                             out, stream);
}

// ---------------------------------------------------------------------------
// HBM read probe: a fixed grid streams the buffer once with 16-byte loads,
// eight in flight per thread, and folds them into one word per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u4* __restrict__ buf,
                                                                   size_t n16, uint32_t* sink) {
  const size_t tid = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const size_t stride = (size_t)kProbeBlocks * kProbeThreads;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u4 v = buf[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = acc;
}

hipError_t launch_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace iq
