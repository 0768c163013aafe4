// Chunked causal prefill on the uncompressed bf16 / FP8 paged cache: the
// baseline of the packed prefill kernel, on the same paging, tiling and
// online softmax ("RotaryQuant: Fitting 120B MoE Models on Consumer Hardware
// via Fused Compressed-Space Attention", abstract: the packed attention avoids
// the full-precision KV state; FreeToken issue #141, Proposed Solution: FP8 as
// the fallback format).  Query i sits at position q_start + i and attends keys
// 0 .. q_start + i.
//
// Work decomposition (gfx950): as the packed prefill, one workgroup of eight
// waves owns 128 rows (query x head-in-group) of one kv head and walks its
// causal page range; wave w owns rows 16w .. 16w + 15.  Here a page needs no
// unpacking: its K tile (token-major) and V tile (coordinate-major) are loaded
// by direct-to-LDS loads straight into the layout the matrix cores read, three
// pages ahead, with one barrier per page.  Rows of a tile are stored with their
// 16-byte chunks XOR-permuted by row so that the sixteen rows one fragment read
// touches fall on distinct LDS banks (the per-lane global addresses of the
// loads apply the permutation; the LDS side of a load is always contiguous).
//   S^T[token][row] = K[token] . Q[row]        (bf16 or f16 products, fp32 sums)
//   O^T[dim][row] += V^T[dim][token] P^T[token][row]   (P as high + low parts)
// FP8 tiles hold E4M3 bytes and are converted to f16 (exactly) as fragments
// are read.
#include <math.h>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

namespace {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef _Float16 hh2v __attribute__((ext_vector_type(2)));
constexpr int kDpWaves = 8;
constexpr int kDpRows = 16 * kDpWaves;  // rows per workgroup
constexpr int kDpSlots = 3;

// Row bytes of the K and V tiles, and the XOR permutation of a row's 16-byte
// chunks: rows 256 / row_bytes apart share the same LDS banks, so the
// permutation varies with row / (256 / row_bytes).
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row) {
  constexpr int kChunks = ROW_BYTES / 16;
  constexpr int kPerBankSet = 256 / ROW_BYTES;  // rows per 256 bytes (all 64 banks)
  return (row / kPerBankSet) & (kChunks - 1);
}

template <int FMT>
struct DpFmt {
  static constexpr int E = FMT == 1 ? 1 : 2;            // bytes per value
  static constexpr int kKRow = 128 * E;                  // K tile: 64 rows (tokens)
  static constexpr int kVRow = 64 * E;                   // V tile: 128 rows (coordinates)
  static constexpr int kTile = 64 * kKRow;               // bytes of each tile
  static constexpr int kSlot = 2 * kTile;                // K tile | V tile
  static constexpr int kDmaPerTile = kTile / 1024;       // 1 KiB direct-to-LDS loads per tile
  static constexpr int kPerWave = 2 * kDmaPerTile / kDpWaves;  // loads per wave and page
};

typedef __attribute__((address_space(3))) void* dp_lds_ptr;
__device__ __forceinline__ void dp_dma16(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dp_lds_ptr)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dp_dma4(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dp_lds_ptr)lds);
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}
#define IQ_DP_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
constexpr int kDpWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

__device__ __forceinline__ void dp_wait_vm(int n) {  // n = 0..8
  switch (n) {
    case 0: IQ_DP_WAIT_VM(0); break;
    case 1: IQ_DP_WAIT_VM(1); break;
    case 2: IQ_DP_WAIT_VM(2); break;
    case 3: IQ_DP_WAIT_VM(3); break;
    case 4: IQ_DP_WAIT_VM(4); break;
    case 5: IQ_DP_WAIT_VM(5); break;
    case 6: IQ_DP_WAIT_VM(6); break;
    case 7: IQ_DP_WAIT_VM(7); break;
    default: IQ_DP_WAIT_VM(8); break;
  }
}

struct DpArgs {
  const uint8_t* k;
  const uint8_t* v;
  int hkv, num_pages;
  const uint16_t* q;  // bf16 [n_q][hq][128]
  int n_q, hq, group, q_start;
  const int32_t* block_table;
  int max_pages;
  float score_factor;  // softmax_scale * log2(e) (* K's scale for FP8)
  float v_scale;       // FP8: V's scale
  float* out;
};

// This wave's share of the loads of one page into `slot`: load j of a tile
// fills LDS bytes 1024 j .. of it; lane i's 16 bytes land at 1024 j + 16 i,
// which is row r, permuted chunk p, so it reads logical chunk p ^ swz(r).
template <int FMT>
__device__ __forceinline__ void dp_issue(const DpArgs& a, int page_id, int g, int wave, int lane,
                                         uint8_t* slot) {
  using F = DpFmt<FMT>;
  const uint32_t page = min((uint32_t)page_id, (uint32_t)a.num_pages - 1u);
  const size_t blk = ((size_t)page * a.hkv + g) * F::kTile;
#pragma unroll
  for (int t = 0; t < F::kDmaPerTile / kDpWaves; ++t) {
    const int j = wave + kDpWaves * t;
    const int byte = 1024 * j + 16 * lane;
    {
      const int r = byte / F::kKRow, p = (byte % F::kKRow) / 16;
      dp_dma16(a.k + blk + r * F::kKRow + 16 * (p ^ swz<F::kKRow>(r)), slot + 1024 * j);
    }
    {
      const int r = byte / F::kVRow, p = (byte % F::kVRow) / 16;
      dp_dma16(a.v + blk + r * F::kVRow + 16 * (p ^ swz<F::kVRow>(r)), slot + F::kTile + 1024 * j);
    }
  }
}

// 8 bytes (bf16: 4 values, FP8: 8 values) at logical byte offset `off` of row r.
template <int ROW_BYTES>
__device__ __forceinline__ const uint8_t* dp_at(const uint8_t* tile, int r, int off) {
  return tile + r * ROW_BYTES + 16 * ((off >> 4) ^ swz<ROW_BYTES>(r)) + (off & 15);
}

__device__ __forceinline__ u2 fp8x4_f16(uint32_t w) {
  const hh2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const hh2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return u2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

template <int FMT>
__device__ __forceinline__ f4 dp_mfma(const u4& a, const u4& b, const f4& c) {
  if constexpr (FMT == 1)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b),
                                                   c, 0, 0, 0);
}

template <bool M>
struct DpMaskTag {
  static constexpr bool value = M;
};

template <int FMT>
__global__ __launch_bounds__(64 * kDpWaves, 1) void dense_prefill_kernel(DpArgs a) {
  using F = DpFmt<FMT>;
  const int g = blockIdx.x, tile = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, jq = lane >> 4;
  const int qpt = kDpRows / a.group;  // queries per tile
  const int q0 = tile * qpt;
  if (q0 >= a.n_q) return;
  const int q_last = min(a.n_q, q0 + qpt) - 1;
  const int kv_end = a.q_start + q_last + 1;
  const int n_pages = min((kv_end + kPage - 1) / kPage, min(a.max_pages, kPrefillMaxPages));
  const int n_full = min(n_pages, (a.q_start + q0 + 1) / kPage);

  __shared__ __attribute__((aligned(16))) uint8_t s_slot[kDpSlots][F::kSlot];  // 96 KB bf16, 48 KB FP8
  __shared__ int s_pt[kPrefillMaxPages];                                         // 16 KB

  for (int i = 0; i < kPrefillMaxPages / (64 * kDpWaves); ++i) {
    const int e0 = (kPrefillMaxPages / kDpWaves) * wave + 64 * i;
    if (e0 < n_pages && e0 + lane < n_pages) dp_dma4(a.block_table + e0 + lane, &s_pt[e0]);
  }

  // this lane's row: 16 wave + col (query q0 + row / group, head row % group)
  const int row = 16 * wave + col;
  const int qi = q0 + row / a.group, h = row % a.group;
  const int qpos = qi < a.n_q ? a.q_start + qi : 0x7FFFFFFF;
  u4 qb[4];  // B operand: coordinates 32 kk + 8 jq .. + 7
  {
    const uint16_t* qr = a.q + ((size_t)qi * a.hq + (size_t)g * a.group + h) * kD + 8 * jq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u4 w = qi < a.n_q ? *reinterpret_cast<const u4*>(qr + 32 * kk) : u4{0u, 0u, 0u, 0u};
      if constexpr (FMT == 1) {  // bf16 -> f16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const hh2v hv = {(_Float16)__builtin_bit_cast(float, w[i] << 16),
                           (_Float16)__builtin_bit_cast(float, w[i] & 0xFFFF0000u)};
          w[i] = __builtin_bit_cast(uint32_t, hv);
        }
      }
      qb[kk] = w;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // page ids and queries landed (all counters)
  __syncthreads();

  for (int p = 0; p < kDpSlots && p < n_pages; ++p) dp_issue<FMT>(a, s_pt[p], g, wave, lane, s_slot[p]);

  const float fac = a.score_factor;
  float m_run = -INFINITY, l_run = 0.f;
  f4 acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};

  auto page_step = [&](int pg, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // this wave's loads of page pg have landed once those of the pages issued
    // after it are the only ones outstanding; the barrier makes every wave's
    // share visible and retires page pg - 1, whose slot takes page pg + 2
    const int after = pg == 0 ? min(kDpSlots - 1, n_pages - 1) : min(1, n_pages - 1 - pg);
    dp_wait_vm(F::kPerWave * after);
    __builtin_amdgcn_s_barrier();
    if (pg >= 1 && pg + 2 < n_pages) dp_issue<FMT>(a, s_pt[pg + 2], g, wave, lane, s_slot[(pg + 2) % kDpSlots]);
    const uint8_t* kt = s_slot[pg % kDpSlots];
    const uint8_t* vt = kt + F::kTile;

    // ---- S^T tiles: token block tb (rows of K), this wave's 16 rows ----
    f4 s[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      f4 c = {0.f, 0.f, 0.f, 0.f};
      const int r = 16 * tb + col;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u4 ka;
        if constexpr (FMT == 1) {
          const u2 w = *reinterpret_cast<const u2*>(dp_at<F::kKRow>(kt, r, 32 * kk + 8 * jq));
          const u2 lo = fp8x4_f16(w[0]), hi = fp8x4_f16(w[1]);
          ka = u4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          ka = *reinterpret_cast<const u4*>(dp_at<F::kKRow>(kt, r, 2 * (32 * kk + 8 * jq)));
        }
        c = dp_mfma<FMT>(ka, qb[kk], c);
      }
      s[tb] = c;
    }
    // ---- online softmax of the lane's row (column of S^T) ----
    const int tok_base = pg * kPage + 4 * jq;
    float sv[4][4];
    float mp = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tok_base + 16 * tb + r;
        sv[tb][r] = (!MASKED || (tok <= qpos && tok < kv_end)) ? s[tb][r] * fac : -INFINITY;
        mp = fmaxf(mp, sv[tb][r]);
      }
    mp = max_xor32(max_xor16(mp));
    const float m_new = fmaxf(m_run, mp);
    const bool live = !MASKED || m_new != -INFINITY;  // a row with no visible key yet keeps its state
    const float corr = live ? fast_exp2(m_run - m_new) : 1.0f;
    if (__any(corr != 1.0f)) {
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] *= corr;
      l_run *= corr;
    }
    m_run = m_new;
    // P^T operand of token pair tp: k index i holds token 32 tp + 16 (i / 4) +
    // 4 jq + i % 4, exactly this lane's score rows tb = 2 tp + i / 4
    u4 ph[2], pl[2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = live ? fast_exp2(sv[2 * tp + (i >> 2)][i & 3] - m_new) : 0.f;
        l_run += p[i];
      }
      if constexpr (FMT == 1) {
        h8 hv, lv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hv[i] = (_Float16)p[i];
          lv[i] = (_Float16)(p[i] - (float)hv[i]);
        }
        ph[tp] = __builtin_bit_cast(u4, hv);
        pl[tp] = __builtin_bit_cast(u4, lv);
      } else {
        bf8v hv, lv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hv[i] = (__bf16)p[i];
          lv[i] = (__bf16)(p[i] - (float)hv[i]);
        }
        ph[tp] = __builtin_bit_cast(u4, hv);
        pl[tp] = __builtin_bit_cast(u4, lv);
      }
    }
    // value masks of the two 4-token runs of each token pair: slots at or past
    // kv_end were never written (they may hold NaN patterns)
    uint32_t vmask[2][2] = {{~0u, ~0u}, {~0u, ~0u}};
    if (MASKED) {
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int t0 = tok_base + 32 * tp + 16 * hlf;
          vmask[tp][hlf] = (t0 < kv_end ? 0x000000FFu : 0u) | (t0 + 1 < kv_end ? 0x0000FF00u : 0u) |
                           (t0 + 2 < kv_end ? 0x00FF0000u : 0u) | (t0 + 3 < kv_end ? 0xFF000000u : 0u);
        }
    }
    // ---- O^T += V^T P^T: coordinate rows 16 m + col ----
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int d = 16 * m + col;
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        u4 va;
        if constexpr (FMT == 1) {
          uint32_t w0 = *reinterpret_cast<const uint32_t*>(dp_at<F::kVRow>(vt, d, 32 * tp + 4 * jq));
          uint32_t w1 = *reinterpret_cast<const uint32_t*>(dp_at<F::kVRow>(vt, d, 32 * tp + 16 + 4 * jq));
          if (MASKED) {
            w0 &= vmask[tp][0];
            w1 &= vmask[tp][1];
          }
          const u2 t0 = fp8x4_f16(w0), t1 = fp8x4_f16(w1);
          va = u4{t0[0], t0[1], t1[0], t1[1]};
        } else {
          u2 w0 = *reinterpret_cast<const u2*>(dp_at<F::kVRow>(vt, d, 2 * (32 * tp + 4 * jq)));
          u2 w1 = *reinterpret_cast<const u2*>(dp_at<F::kVRow>(vt, d, 2 * (32 * tp + 16 + 4 * jq)));
          if (MASKED) {  // byte masks -> 16-bit value masks
            const uint32_t m0 = vmask[tp][0], m1 = vmask[tp][1];
            w0[0] &= ((m0 & 1u) ? 0xFFFFu : 0u) | ((m0 & 0x100u) ? 0xFFFF0000u : 0u);
            w0[1] &= ((m0 & 0x10000u) ? 0xFFFFu : 0u) | ((m0 & 0x1000000u) ? 0xFFFF0000u : 0u);
            w1[0] &= ((m1 & 1u) ? 0xFFFFu : 0u) | ((m1 & 0x100u) ? 0xFFFF0000u : 0u);
            w1[1] &= ((m1 & 0x10000u) ? 0xFFFFu : 0u) | ((m1 & 0x1000000u) ? 0xFFFF0000u : 0u);
          }
          va = u4{w0[0], w0[1], w1[0], w1[1]};
        }
        acc[m] = dp_mfma<FMT>(va, ph[tp], acc[m]);
        acc[m] = dp_mfma<FMT>(va, pl[tp], acc[m]);
      }
    }
    __builtin_amdgcn_s_waitcnt(kDpWaitLgkm0);  // this wave's LDS reads of the page are done
  };
  int pg = 0;
  for (; pg < n_full; ++pg) page_step(pg, DpMaskTag<false>{});
  for (; pg < n_pages; ++pg) page_step(pg, DpMaskTag<true>{});
  IQ_DP_WAIT_VM(0);  // (no load is left in flight: every issued page was used)

  // ---- epilogue: normalise and store (coordinate 16 m + 4 jq + r) ----
  const float l = sum_xor32(sum_xor16(l_run));
  const float sc = (l > 0.f) ? (FMT == 1 ? a.v_scale : 1.0f) / l : 0.f;
  if (qi < a.n_q) {
    float* dst = a.out + ((size_t)qi * a.hq + (size_t)g * a.group + h) * kD + 4 * jq;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *reinterpret_cast<f4*>(dst + 16 * m) = f4{acc[m][0] * sc, acc[m][1] * sc, acc[m][2] * sc, acc[m][3] * sc};
  }
}

}  // namespace

hipError_t launch_dense_prefill(const DenseCacheView& c, const void* q, int n_q, int hq, int q_start,
                                const int32_t* block_table, int max_pages, float softmax_scale, float* out,
                                hipStream_t stream) {
  const bool fp8 = c.format == 1;
  DpArgs a;
  a.k = c.k;
  a.v = c.v;
  a.hkv = c.hkv;
  a.num_pages = c.num_pages;
  a.q = static_cast<const uint16_t*>(q);
  a.n_q = n_q;
  a.hq = hq;
  a.group = hq / c.hkv;
  a.q_start = q_start;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.score_factor = (float)((double)softmax_scale * 1.4426950408889634 * (fp8 ? (double)c.k_scale : 1.0));
  a.v_scale = fp8 ? c.v_scale : 1.0f;
  a.out = out;
  const int qpt = kDpRows / a.group;
  const dim3 grid(c.hkv, (n_q + qpt - 1) / qpt);
  if (fp8)
    hipLaunchKernelGGL(dense_prefill_kernel<1>, grid, dim3(64 * kDpWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(dense_prefill_kernel<0>, grid, dim3(64 * kDpWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace iq
