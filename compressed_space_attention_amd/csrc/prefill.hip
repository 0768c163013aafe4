// Chunked causal prefill attention on the packed 3-bit (or 4-bit) cache.
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
// Work decomposition (gfx950): one workgroup per CU owns 128 rows of one kv
// head and walks the pages up to its causal limit.  Two shapes (RB = row
// blocks of 16 per wave): RB = 2, four waves of 32 rows (every K^ and V^
// fragment read from LDS feeds four matrix-core products, one wave per SIMD);
// RB = 1, eight waves of 16 rows (two waves per SIMD).  The pages run as a
// software pipeline, one barrier per page:
//   * raw pages arrive by direct-to-LDS loads issued two steps before they
//     are unpacked (each wave loads exactly the code bytes it will unpack,
//     so no wave waits for another's loads);
//   * unpacked pages -- K^ token-major, V^ as [coordinate][token], both
//     alpha-scaled f16, and the fp16 norms -- sit in a ring of three LDS
//     buffers, stored chunk-major (see below): while page p's softmax and
//     P.V products run, page p + 1's scores are computed (into a second
//     register set) and page p + 2 is unpacked; the two waves of a SIMD take
//     these in opposite orders, so one's matrix-core products overlap the
//     other's vector work;
//   * only pages that reach past the smallest query position of the tile are
//     masked.
// The page ids of the whole causal range are staged in LDS once.
// 4-bit records (BITS = 4): a page's 8,192 code bytes fill the same raw slot
// (16-byte units: a quarter of a K record, or a quarter of a V region, per
// lane), and unpack into the same f16 buffers.
#include <math.h>
#include <stdlib.h>

#include <atomic>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {

constexpr int kRowsPerTile = 128;  // rows = queries x group heads
// The unpacked f16 tiles are stored chunk-major: 16-byte chunk c of every row
// forms a contiguous plane, so the 16 lanes of a matrix-core fragment read
// (16 consecutive rows, one chunk) read 256 contiguous bytes, which the LDS
// serves without bank conflicts (a padded row-major tile is served 2-way
// conflicted on this GPU).
//   K^:  plane c (coordinates 8c .. 8c+7) of the 64 tokens: byte 1024 c + 16 tok
//   V^T: plane c (token columns 8c .. 8c+7) of the 128 coordinate rows:
//        byte 2048 c + 16 row
constexpr int kKTileBytes = 16 * kPage * 16;  // 16 planes x 64 tokens x 16 B
constexpr int kVTileBytes = 8 * kD * 16;      // 8 planes x 128 rows x 16 B
// Within a V^T row the tokens of each 32-token half are in the matrix-core k
// order: column of token t (0..63): half tp = t / 32 holds, for lane group jq,
// tokens 4 jq .. +3 then 16 + 4 jq .. +3 at columns 32 tp + 8 jq ..
__host__ __device__ constexpr int vt_col(int t) {
  return 32 * (t >> 5) + 8 * ((t & 15) >> 2) + 4 * ((t & 31) >> 4) + (t & 3);
}
// byte offset of the 4-column (8-byte) run starting at column col (a multiple
// of 4) of V^T row `row`
__host__ __device__ constexpr int vt_at(int row, int col) {
  return 2048 * (col >> 3) + 16 * row + 2 * (col & 7);
}
constexpr int kRawPage = 8192;  // raw code bytes of a page in LDS: 512 groups of 12 B at a 16 B stride
constexpr int kRawSlot = kRawPage + 256;  // + the page's K and V norms
constexpr int kRawSlots = 3;
// The prefill kernel's LDS block: norms of the three unpacked pages, the
// wait flag, the raw page slots, the K^ and V^T tiles, the page ids.
constexpr int kPfLdsNorm = 0;
constexpr int kPfLdsFail = kPfLdsNorm + 3 * 2 * kPage * 2;
constexpr int kPfLdsRaw = kPfLdsFail + 16;
constexpr int kPfLdsK = kPfLdsRaw + kRawSlots * kRawSlot;
constexpr int kPfLdsV = kPfLdsK + 3 * kKTileBytes;
constexpr int kPfLdsPt = kPfLdsV + 3 * kVTileBytes;
constexpr int kPfLdsBytes = kPfLdsPt + 4 * kPrefillMaxPages;
static_assert(kPfLdsRaw % 16 == 0 && kPfLdsK % 16 == 0 && kPfLdsV % 16 == 0 && kPfLdsPt % 16 == 0,
              "16-byte aligned LDS arrays");
template <int RB> constexpr int pf_waves() { return 8 / RB; }

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
  // Batched variable-length form (null for one sequence): sequence b = blockIdx.z
  // owns query rows cu_q[b] .. cu_q[b+1]-1 of q and out, its first query sits at
  // q_starts[b], and its block-table row is block_table + b * max_pages.
  const int32_t* cu_q;
  const int32_t* q_starts;
  int max_pages;
  float score_factor;  // softmax_scale * log2(e) / (128 * alpha)
  float out_factor;    // 1 / (sqrt(128) * alpha)
  float* out;
  Levels4 lv4;         // 4-bit records: thresholds and f16 level tables
  // Fused quantise-append of the chunk (app_k null: none): tokens new_start ..
  // new_start + n_new - 1 of this sequence, rows [n_new][hkv][128] of
  // app_dtype, written into the cache by the workgroups of their kv head
  // before they read it.  The row tiles of kv head g share its (64-token
  // block, K|V) jobs; a workgroup adds the jobs it finished to app_arrive[g]
  // once their records are visible device-wide, and waits for all of them
  // before requesting the first page that holds appended tokens; the last
  // workgroup of kv head g to finish clears app_arrive[g] and app_done[g].
  const void* app_k;
  const void* app_v;
  int app_dtype, n_new, new_start, row_tiles;
  uint8_t* k_codes_w;
  uint16_t* k_norms_w;
  uint8_t* v_codes_w;
  uint16_t* v_norms_w;
  uint32_t* app_arrive;
  uint32_t* app_done;
};

// The wait for the appended pages is bounded (2^20 polls, each a memory round
// trip: about a second); a wait that runs out leaves NaN rows.
constexpr uint32_t kAppendSpinLimit = 1u << 20;

// The fused append's share of this workgroup (kv head g, row tile `tile`):
// K blocks first, then V blocks, 256 threads per block (a quad per token),
// every workgroup thread in every pass; each pass's rows are requested while
// the previous pass is coded.  lds: 2 KB for the head's rotation blocks + 4 KB
// per 256 threads for assembling whole V pages.  Returns the jobs done; their
// device-scope stores may still be in flight (the caller waits for them
// before counting the jobs in).
template <int BITS, int W>
__device__ __forceinline__ int prefill_append(const PrefillArgs& a, const int32_t* btab, int g, int tile,
                                              uint8_t* lds) {
  constexpr int kRecB = BITS == 4 ? kRec4 : kRec;
  constexpr int kPar = 64 * W / 256;  // blocks coded at once
  const int tid = threadIdx.x, half = tid >> 8, t = tid & 255, tl = t >> 2, j = t & 3;
  float* s_rot = reinterpret_cast<float*>(lds);
  uint8_t* s_vb = lds + 2048 + 4096 * half;
  if (tid < kRotFloats / 4)
    reinterpret_cast<f4*>(s_rot)[tid] = reinterpret_cast<const f4*>(a.rot + (size_t)g * kRotFloats)[tid];
  const int nb = (a.n_new + kPage - 1) / kPage;  // 64-token blocks of the chunk
  const int stride = a.row_tiles * kPar;
  const int per_kv = nb > tile * kPar ? (nb - tile * kPar + stride - 1) / stride : 0;  // passes per K | V
  const int passes = 2 * per_kv;
  // pass ps: K (ps < per_kv) or V, blocks b0 .. b0 + kPar - 1, this thread's block b0 + half
  auto pass_block = [&](int ps, int& which) {
    which = ps >= per_kv;
    return tile * kPar + (ps - which * per_kv) * stride + half;
  };
  auto request = [&](int ps, u4 (&r)[8]) {
    int which;
    const int blk = pass_block(ps, which);
    const int i = blk * kPage + tl;
    const bool valid = blk < nb && i < a.n_new;
    load32_raw(which ? a.app_v : a.app_k, ((size_t)(valid ? i : 0) * a.hkv + g) * kD + 32 * j, a.app_dtype, r);
  };
  u4 raw[8];
  if (passes > 0) request(0, raw);
  __syncthreads();  // the rotation blocks
  for (int ps = 0; ps < passes; ++ps) {
    float x[32];
    raw_to_f32(raw, a.app_dtype, x);
    if (ps + 1 < passes) request(ps + 1, raw);
    int which;
    const int blk = pass_block(ps, which);
    const bool job = blk < nb;
    const int i = blk * kPage + tl;  // token of the chunk
    const bool valid = job && i < a.n_new;
    const int p = a.new_start + i;
    // a position outside the table or a page id outside the cache is skipped
    const bool in_table = valid && (unsigned)p < (unsigned)a.max_pages * kPage;
    const int page = in_table ? btab[p >> 6] : -1;
    const bool stored = (unsigned)page < (unsigned)a.num_pages;
    // a whole page: the block's 64 tokens fill one page (uniform per block)
    const int p0 = a.new_start + blk * kPage;
    const bool whole = job && (p0 & 63) == 0 && blk * kPage + kPage <= a.n_new &&
                       (unsigned)p0 < (unsigned)a.max_pages * kPage &&
                       (unsigned)btab[min(p0 >> 6, a.max_pages - 1)] < (unsigned)a.num_pages;
    uint32_t sel[8];
    const float n = quad_codes<BITS>(x, j, s_rot, a.lv4, sel);
    const size_t pb = (size_t)(stored ? page : 0) * a.hkv + g;  // (page, kv head) block
    quad_store<BITS, DeviceStore, true>(which, stored, whole, j, p & 63, sel, n,
                                        (which ? a.v_codes_w : a.k_codes_w) + pb * (kPage * kRecB),
                                        (which ? a.v_norms_w : a.k_norms_w) + pb * kPage, s_vb, t);
    // the next pass assembles its V page in the same LDS bytes
    if (which) __syncthreads();
  }
  int jobs = 0;
  for (int b0 = tile * kPar; b0 < nb; b0 += stride) jobs += 2 * min(kPar, nb - b0);
  return jobs;
}

// Count this workgroup's append jobs in once every thread's record stores
// have completed (the stores are not tracked by the compiler: an explicit
// wait on all counters, then a barrier).
__device__ __forceinline__ void prefill_append_count(const PrefillArgs& a, int g, int jobs) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 && jobs > 0) {
    __hip_atomic_fetch_add(a.app_arrive + g, (uint32_t)jobs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // counted in before this workgroup can count itself done
  }
}

// Wait (thread 0, bounded) until every job of kv head g's appended chunk is
// visible, drop stale copies of the appended pages from this CU's and XCD's
// caches, then let the workgroup on.  *s_fail = 1 when the wait ran out.
__device__ __forceinline__ void prefill_wait_appended(const PrefillArgs& a, int g, int* s_fail) {
  if (threadIdx.x == 0) {
    const uint32_t target = 2u * (uint32_t)((a.n_new + kPage - 1) / kPage);
    uint32_t spins = 0;
    while (__hip_atomic_load(a.app_arrive + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins == kAppendSpinLimit) {
        *s_fail = 1;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __builtin_amdgcn_s_barrier();
}

// The last workgroup of kv head g to get here clears its counters for the
// next call (every workgroup has added its jobs and passed its wait).
__device__ __forceinline__ void prefill_append_finish(const PrefillArgs& a, int g) {
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.app_done + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == (uint32_t)a.row_tiles) {
      __hip_atomic_store(a.app_arrive + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.app_done + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Direct-to-LDS loads, issued from inline asm so that the compiler does not
// track them: it cannot tell which raw slot a load writes and would otherwise
// wait for every outstanding load (the two pages in flight) before each LDS
// read of a raw page.  Every read of loaded LDS data is preceded by an
// explicit s_waitcnt on this kernel's issue order instead.  No register
// outputs: the address is read at issue, the destination is LDS at m0.
typedef __attribute__((address_space(3))) void* pf_lds_ptr;
// LDS byte address of a shared-memory pointer (pointers into a kernel's
// __shared__ arrays only)
__device__ __forceinline__ uint32_t pf_lds_addr(const void* lds) {
  return (uint32_t)(uintptr_t)(pf_lds_ptr)lds;
}
__device__ __forceinline__ void pf_dma(const void* g, uint32_t lds, int size) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  if (size == 16)
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
  else if (size == 12)
    asm volatile("global_load_lds_dwordx3 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
  else
    asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}
// LDS reads at a 32-bit LDS address.  A page step's read groups each take one
// base address, computed once and kept opaque (so the compiler does not
// re-associate it into a vector add per read), plus constant offsets that
// the ds_read immediate field carries.
typedef __attribute__((address_space(3))) const h8* pf_lds_h8p;
typedef __attribute__((address_space(3))) const u2* pf_lds_u2p;
__device__ __forceinline__ uint32_t pf_opaque(uint32_t a) {
  asm volatile("" : "+v"(a));
  return a;
}
__device__ __forceinline__ h8 pf_ld_h8(uint32_t addr) { return *(pf_lds_h8p)(uintptr_t)addr; }
__device__ __forceinline__ u2 pf_ld_u2(uint32_t addr) { return *(pf_lds_u2p)(uintptr_t)addr; }

// s_waitcnt vmcnt(n) (gfx9 encoding, other counters left alone)
#define IQ_PF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
constexpr int kPfWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

template <bool M>
struct PfTag {
  static constexpr bool value = M;
};

// x * norm r of the pair as one mixed-precision FMA (fp16 operand in place)
__device__ __forceinline__ float times_norm2(float x, const u2& n, int r);
__device__ __forceinline__ float norm_at2(const u2& n, int r) {
  const uint32_t w = (r < 2) ? n[0] : n[1];
  return half_bits_to_float((r & 1) ? (w >> 16) : (w & 0xFFFFu));
}
__device__ __forceinline__ float times_norm2(float x, const u2& n, int r) {
  return __builtin_fmaf(x, norm_at2(n, r), 0.0f);
}

// What one wave loads and unpacks of every page: a quarter `part` of the K
// codes (DO_K) and/or of the V codes (DO_V), and with NORMS (wave 0) also the
// page's norms.  Four waves carry both quarters of their part; eight waves
// split them, waves 0-3 the K quarters and waves 4-7 the V quarters, so that
// every unpack runs on all 64 lanes.
// PRODUCTS_FIRST: the order of a page step.  true: the next page's scores,
// this page's softmax, the unpack of the page after next, this page's P.V
// products; false: softmax, scores, P.V, unpack.  Waves w and w + 4 share a
// SIMD; the K waves (0-3) take the first order and the V waves (4-7) the
// second, so that between two barriers one wave's matrix-core products run
// while the other does vector work.
template <bool DO_K, bool DO_V, bool NORMS, bool PRODUCTS_FIRST = true>
struct PfRole {
  static constexpr bool k = DO_K, v = DO_V, norms = NORMS, products_first = PRODUCTS_FIRST;
  static constexpr int loads = (DO_K ? 1 : 0) + (DO_V ? 1 : 0) + (NORMS ? 1 : 0);  // per page
};

// Raw loads of one page into a slot (each wave loads exactly the groups it
// unpacks).  Part p of a raw slot: K bytes at 2048 p, V bytes at 2048 p + 1024
// (64 lanes x 16 bytes each, lane l at 16 l).  The lanes are assigned so that
// the unpacked writes of 16 (or 32) consecutive lanes are contiguous:
//   3-bit K quarter p: lane l = group l / 16 (coordinates 32 (l / 16) ..) of
//     token 16 p + l % 16;
//   3-bit V quarter p: lane l = chunk 2 (l / 32) + (l / 16) % 2 of V region
//     16 p + l % 16;
//   4-bit K quarter p: lane l = quarter l / 16 (16 bytes) of token 16 p + l % 16;
//   4-bit V quarter p: lane l = dwords 4 (l / 16) .. + 3 of V region 16 p + l % 16.
// NORMS: the K norms (lanes 0-31) and V norms (lanes 32-63).
template <int BITS, class R>
__device__ __forceinline__ void pf_issue(const PrefillArgs& a, int page_id, int g, int part, int lane,
                                         uint32_t slot) {
  // an id outside the cache (a table that breaks the contract) is clamped into
  // it, so a bad table gives wrong numbers, never an out-of-bounds read
  const uint32_t page = min((uint32_t)page_id, (uint32_t)a.num_pages - 1u);
  const size_t base = ((size_t)page * a.hkv + g) * kPage;
  const uint32_t dst = slot + 2048 * part;
  const int row = 16 * part + (lane & 15);  // token (K) or V region of this lane
  if (BITS == 4) {
    if (R::k) pf_dma(a.k_codes + (base + row) * kRec4 + 16 * (lane >> 4), dst, 16);
    if (R::v) pf_dma(a.v_codes + base * kRec4 + row * 64 + 16 * (lane >> 4), dst + 1024, 16);
  } else {
    if (R::k) pf_dma(a.k_codes + (base + row) * kRec + 12 * (lane >> 4), dst, 12);
    if (R::v) {
      const int c = 2 * (lane >> 5) + ((lane >> 4) & 1);
      pf_dma(a.v_codes + (base + row) * kRec + 12 * c, dst + 1024, 12);
    }
  }
  if (R::norms) {
    const uint16_t* nb = (lane < 32 ? a.k_norms : a.v_norms) + base + 2 * (lane & 31);
    pf_dma(nb, slot + kRawPage, 4);
  }
}

// One K group (token tok, coordinates 32j..32j+31 = planes 4j .. 4j+3) into
// the f16 K^ tile.
typedef __attribute__((address_space(3))) u4* pf_lds_u4w;
typedef __attribute__((address_space(3))) u2* pf_lds_u2w;
__device__ __forceinline__ void pf_st_u4(uint32_t addr, const u4& v) { *(pf_lds_u4w)(uintptr_t)addr = v; }
__device__ __forceinline__ void pf_st_u2(uint32_t addr, const u2& v) { *(pf_lds_u2w)(uintptr_t)addr = v; }

// kd = LDS address of the K^ tile + 1024 * 4j + 16 * tok (token tok, quarter j)
__device__ __forceinline__ void pf_unpack_k(const u3& ck, uint32_t kd) {
  uint32_t z[8];
  group_to_selectors(ck.x, ck.y, ck.z, z);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const u2 d0 = selector_to_f16(z[2 * kk]), d1 = selector_to_f16(z[2 * kk + 1]);
    pf_st_u4(kd + 1024 * kk, u4{d0[0], d0[1], d1[0], d1[1]});
  }
}
// Chunk c of V region `region` = (n, q) = (region % 16, region / 16): tokens
// 16c + 4q + r, selector m, into row 16m + n of the f16 V^T tile (row 16m + n
// holds coordinate 32 (n / 4) + 4m + n % 4: accumulator order).  vd = LDS
// address of the tile + vt_at(n, vt_col(16c + 4q)): row 16m + n is 256 m
// further.
__device__ __forceinline__ int pf_v_lane_offset(int region, int c) {
  return vt_at(region & 15, vt_col(16 * c + 4 * (region >> 4)));  // the four tokens stay adjacent
}
__device__ __forceinline__ void pf_unpack_v(const u3& cv, uint32_t vd) {
  uint32_t z[8];
  group_to_selectors(cv.x, cv.y, cv.z, z);
#pragma unroll
  for (int m = 0; m < 8; ++m) pf_st_u2(vd + 256 * m, selector_to_f16(z[m]));
}

// 4-bit: quarter j of token tok's record (dword kk = coordinates 32j + 8kk
// .. + 7) into the f16 K^ tile; kd as for pf_unpack_k.
__device__ __forceinline__ void pf_unpack_k4(const u4& ck, uint32_t kd, const Levels4& lv) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pf_st_u4(kd + 1024 * kk, __builtin_bit_cast(u4, dword4_to_h8(ck[kk], lv)));
}
// 4-bit: dwords 4p .. 4p+3 of V region `region` = n + 16 jq: dword (th, q)
// holds tokens 32 th + 16 q + 4 jq + r of coordinate 32 (n / 4) + 4p + n % 4
// (low nibbles) and that + 16 (high nibbles).  The V^T tile is in
// accumulator order, as for 3-bit pages: row 16m + n holds coordinate
// 32 (n / 4) + 4m + n % 4, so the low nibbles go to row 16p + n and the high
// ones to row 16 (p + 4) + n.  Lanes of odd p take the dwords in the order
// 1 0 3 2, so that at every store the 32 lanes of a half-wave fill whole
// 16-byte chunks.
__device__ __forceinline__ void pf_unpack_v4(const u4& cv, int region, int p, uint8_t* sv,
                                             const Levels4& lv) {
  const int n = region & 15, jq = region >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = i ^ (p & 1);
    const int col = 32 * (d >> 1) + 8 * jq + 4 * (d & 1);  // vt_col(32 (d/2) + 16 (d%2) + 4 jq)
    const uint32_t w = (p & 1) ? cv[i ^ 1] : cv[i];
    *reinterpret_cast<u2*>(sv + vt_at(16 * p + n, col)) = nibbles_to_f16(w & 0x0F0F0F0Fu, lv);
    *reinterpret_cast<u2*>(sv + vt_at(16 * (p + 4) + n, col)) = nibbles_to_f16((w >> 4) & 0x0F0F0F0Fu, lv);
  }
}

// Unpack this wave's part of a raw page into the f16 tiles.
template <int BITS, class R>
__device__ __forceinline__ void pf_unpack(const uint8_t* slot, int part, int lane, uint8_t* sk,
                                          uint8_t* sv, uint16_t* snorm, const Levels4& lv) {
  // one opaque base per store group; the per-store offsets are immediates
  const uint8_t* raw = slot + 2048 * part + 16 * lane;
  const int row = 16 * part + (lane & 15);
  if (BITS == 4) {
    if (R::k)
      pf_unpack_k4(*reinterpret_cast<const u4*>(raw),
                   pf_opaque(pf_lds_addr(sk) + 1024 * 4 * (lane >> 4) + 16 * row), lv);
    if (R::v)
      pf_unpack_v4(*reinterpret_cast<const u4*>(raw + 1024), row, lane >> 4, sv, lv);
  } else {
    if (R::k)
      pf_unpack_k(*reinterpret_cast<const u3*>(raw),
                  pf_opaque(pf_lds_addr(sk) + 1024 * 4 * (lane >> 4) + 16 * row));
    if (R::v)
      pf_unpack_v(*reinterpret_cast<const u3*>(raw + 1024),
                  pf_opaque(pf_lds_addr(sv) + pf_v_lane_offset(row, 2 * (lane >> 5) + ((lane >> 4) & 1))));
  }
  if (R::norms)
    reinterpret_cast<uint32_t*>(snorm)[lane] = reinterpret_cast<const uint32_t*>(slot + kRawPage)[lane];
}

// APP: the launch also quantise-appends a chunk (PrefillArgs::app_k).
template <int RB, int BITS, bool APP>
__global__ __launch_bounds__(64 * pf_waves<RB>(), 1) void prefill_kernel(PrefillArgs a) {
  constexpr int W = pf_waves<RB>();
  const int g = blockIdx.x, tile = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, jq = lane >> 4;
  // this sequence's queries: rows row0 .. row0 + n_q - 1 of q and out
  int n_q = a.n_q, q_start = a.q_start, row0 = 0;
  const int32_t* btab = a.block_table;
  if (a.cu_q) {
    row0 = a.cu_q[b];
    n_q = a.cu_q[b + 1] - row0;
    q_start = a.q_starts[b];
    btab += (size_t)b * a.max_pages;
  }
  // One LDS block carved by hand, the arrays read every page first: the
  // norms sit within the 64 KiB that a ds_read's immediate offset reaches
  // from one base register (the compiler's own placement put them last, past
  // 136 KiB, and spent a vector add on every norm read).
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kPfLdsBytes];
  uint16_t (*s_norm)[2 * kPage] = reinterpret_cast<uint16_t (*)[2 * kPage]>(s_lds + kPfLdsNorm);  // K | V norms
  int& s_fail = *reinterpret_cast<int*>(s_lds + kPfLdsFail);
  uint8_t (*s_raw)[kRawSlot] = reinterpret_cast<uint8_t (*)[kRawSlot]>(s_lds + kPfLdsRaw);   // 25,344 B
  uint8_t (*s_k)[kKTileBytes] = reinterpret_cast<uint8_t (*)[kKTileBytes]>(s_lds + kPfLdsK);  // 49,152 B
  uint8_t (*s_v)[kVTileBytes] = reinterpret_cast<uint8_t (*)[kVTileBytes]>(s_lds + kPfLdsV);  // 49,152 B
  int* s_pt = reinterpret_cast<int*>(s_lds + kPfLdsPt);                                       // 16,384 B

  // ---- fused quantise-append: this workgroup's share of the chunk (the f16
  // tile buffers are free yet); its jobs are counted in once the records are
  // visible, after the query prologue below ----
  int app_jobs = 0;
  if constexpr (APP) {
    if (tid == 0) s_fail = 0;
    app_jobs = prefill_append<BITS, W>(a, btab, g, tile, s_k[0]);
  }

  const int qpt = kRowsPerTile / a.group;  // queries per tile
  const int q0 = tile * qpt;
  if (q0 >= n_q) {  // a tile past this sequence's queries (uniform)
    if constexpr (APP) {
      prefill_append_count(a, g, app_jobs);
      prefill_append_finish(a, g);
    }
    return;
  }
  const int q_last = min(n_q, q0 + qpt) - 1;
  const int kv_end = q_start + q_last + 1;
  // (a range beyond the table or the staging limit breaks the contract: never
  // read past either)
  const int n_pages = min((kv_end + kPage - 1) / kPage, min(a.max_pages, kPrefillMaxPages));
  // pages entirely at or before the smallest query position need no mask
  const int n_full = min(n_pages, (q_start + q0 + 1) / kPage);

  // ---- page ids of the causal range (wave w: a 1/W share of the entries) ----
  for (int i = 0; i < kPrefillMaxPages / (64 * W); ++i) {
    const int e0 = (kPrefillMaxPages / W) * wave + 64 * i;
    if (e0 < n_pages && e0 + lane < n_pages) pf_dma(btab + e0 + lane, pf_lds_addr(&s_pt[e0]), 4);
  }

  // ---- this wave's 16 RB rows: Q' = T q (lane: row 16cb + col, quarter jq) ----
  h8 qhi[RB][4], qlo[RB][4];
  float fac[RB];
  int qpos[RB], qi_row[RB], head_row[RB];
#pragma unroll
  for (int cb = 0; cb < RB; ++cb) {
    const int row = 16 * RB * wave + 16 * cb + col;
    const int qi = q0 + row / a.group;
    const int h = row % a.group;
    qi_row[cb] = qi;
    head_row[cb] = h;
    qpos[cb] = (qi < n_q) ? q_start + qi : 0x7FFFFFFF;
    float x[32];
    if (qi < n_q) {
      load32(a.q, ((size_t)(row0 + qi) * a.hq + (size_t)g * a.group + h) * kD + 32 * jq, a.q_dtype, x);
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
  if constexpr (APP) prefill_append_count(a, g, app_jobs);

  const uint32_t raw_base = pf_lds_addr(&s_raw[0][0]);
  float m_run[RB], l_run[RB];
  int rho_e = 0;
  f4 acc[RB][8];
#pragma unroll
  for (int cb = 0; cb < RB; ++cb) {
    m_run[cb] = -INFINITY;
    l_run[cb] = 0.f;
  }
#pragma unroll
  for (int cb = 0; cb < RB; ++cb)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[cb][m] = f4{0.f, 0.f, 0.f, 0.f};

  // ---- S^T tiles [token block tb][row block cb] of the page in f16 buffer
  // `buf`: each K^ fragment feeds every row block (hi and lo parts of Q') ----
  auto scores = [&](int buf, f4 (&s)[4][RB]) {
    const uint32_t kb = pf_opaque(pf_lds_addr(s_k[buf]) + 1024 * 4 * jq + 16 * col);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) s[tb][cb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 av = pf_ld_h8(kb + 1024 * kk + 256 * tb);
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) {
          s[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qhi[cb][kk], s[tb][cb], 0, 0, 0);
          s[tb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[cb][kk], s[tb][cb], 0, 0, 0);
        }
      }
    }
  };

  // Software pipeline over the pages.  Raw page p sits in raw slot p % 3 and
  // is unpacked into f16 buffer p % 3.  Step pg: request raw page pg + 4;
  // compute the scores of page pg + 1, page pg's softmax and P.V products,
  // and unpack page pg + 2, in the order of the wave's role (independent
  // work, so the matrix cores and the vector ALU of a SIMD both stay busy);
  // one barrier.  Every step issues the same loads -- past the last page it
  // requests the last page again, and the steps past the end compute and
  // unpack pages whose results are never used -- so the steady state holds
  // no branch and every wait is a constant count.
  const int part = wave & 3;
  auto run = [&](auto role) {
    using R = decltype(role);
    constexpr int per_page = R::loads;
    const int last = n_pages - 1;
    // a fused append's pages are requested only once all of them are written
    bool app_ready = !APP;
    const int app_first = APP ? a.new_start / kPage : 0;
    auto issue = [&](int p) {
      const int pp = min(p, last);
      if constexpr (APP) {
        if (!app_ready && pp >= app_first) {  // uniform: every wave issues the same pages
          prefill_wait_appended(a, g, &s_fail);
          app_ready = true;
        }
      }
      pf_issue<BITS, R>(a, s_pt[pp], g, part, lane, raw_base + (p % 3) * kRawSlot);
    };
    auto unpack = [&](int p) {
      const int u = p % 3;
      pf_unpack<BITS, R>(s_raw[u], part, lane, s_k[u], s_v[u], s_norm[u], a.lv4);
    };
    issue(0);
    issue(1);
    issue(2);
    IQ_PF_WAIT_VM(2 * per_page);
    unpack(0);
    IQ_PF_WAIT_VM(per_page);
    unpack(1);
    __builtin_amdgcn_s_waitcnt(kPfWaitLgkm0);  // slot 0 read out before it is refilled
    issue(3);
    __builtin_amdgcn_s_barrier();

    auto page_step = [&](int pg, f4 (&s)[4][RB], f4 (&s_next)[4][RB], auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int f = pg % 3;
      issue(pg + 4);  // into the slot page pg + 1 left (read out before the last barrier)
      if (R::products_first) scores((pg + 1) % 3, s_next);

      const uint32_t nb = pf_opaque(pf_lds_addr(s_norm[f]) + 8 * jq);  // norms of tokens 16 tb + 4 jq ..
      uint32_t vbits = 0;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const u2 vn = pf_ld_u2(nb + 2 * (kPage + 16 * tb));
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
      const int tok_base = pg * kPage + 4 * jq;

      // value norms of the page; on a masked page, slots at or past the end of
      // the appended chunk were never written and read as zero
      u2 vnp[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        vnp[tb] = pf_ld_u2(nb + 2 * (kPage + 16 * tb));
        if (MASKED) {
          const int t0 = tok_base + 16 * tb;
          vnp[tb][0] &= (t0 < kv_end ? 0xFFFFu : 0u) | (t0 + 1 < kv_end ? 0xFFFF0000u : 0u);
          vnp[tb][1] &= (t0 + 2 < kv_end ? 0xFFFFu : 0u) | (t0 + 3 < kv_end ? 0xFFFF0000u : 0u);
        }
      }

      // ---- online softmax per row (column of S^T) ----
      // Scores in row units (raw x key norm); the log2-scaled score is that
      // times the row factor fac[cb] > 0, applied inside the exponent.  The
      // accumulator and the sum are in units of the value-norm frame 2^rho.
      h8 pb[2][RB];  // [token pair tp][row block cb]
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        float sv[4][4];
        float mp = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const u2 kn = pf_ld_u2(nb + 2 * 16 * tb);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = times_norm2(s[tb][cb][r], kn, r);
            if (MASKED) {
              const int tok = tok_base + 16 * tb + r;
              sv[tb][r] = (tok <= qpos[cb] && tok < kv_end) ? v : -INFINITY;
            } else {
              sv[tb][r] = v;
            }
            mp = fmaxf(mp, sv[tb][r]);
          }
        }
        mp = max_xor32(max_xor16(mp)) * fac[cb];
        const float m_new = fmaxf(m_run[cb], mp);
        // a row whose keys on this page are all masked keeps its state
        const bool live = !MASKED || m_new != -INFINITY;
        const float corr = live ? fast_exp2(m_run[cb] - m_new) : 1.0f;
        const float rescale = __builtin_amdgcn_ldexpf(corr, rho_new - rho_e);
        if (__any(rescale != 1.0f)) {
#pragma unroll
          for (int m = 0; m < 8; ++m) acc[cb][m] *= rescale;
        }
        l_run[cb] *= rescale;
        m_run[cb] = m_new;
        const float m_shift = m_new - (float)rho_new;  // p' = 2^(s - m + rho)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // masked scores: 2^-inf = 0
            const float p = (!MASKED || live) ? fast_exp2(__builtin_fmaf(sv[tb][r], fac[cb], -m_shift)) : 0.f;
            l_run[cb] += p;
            pb[tb >> 1][cb][4 * (tb & 1) + r] = (_Float16)times_norm2(p, vnp[tb], r);  // p' vn < 2
          }
        }
      }
      rho_e = rho_new;
      if (!R::products_first) scores((pg + 1) % 3, s_next);

      // ---- unpack page pg + 2 into the buffer page pg - 1 used (every wave
      // has passed the barrier after its last read); loads still allowed in
      // flight: pages pg + 3 and pg + 4 ----
      if (R::products_first) {
        IQ_PF_WAIT_VM(2 * per_page);
        unpack(pg + 2);
      }

      // ---- O'^T += V^T P~: each V^ fragment feeds both row blocks ----
      const uint32_t vb = pf_opaque(pf_lds_addr(s_v[f]) + 2048 * jq + 16 * col);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          // k index 8 jq + i: token 32 tp + 4 jq + i (i < 4) or 32 tp + 16 + 4 jq + i - 4
          const h8 av = pf_ld_h8(vb + 8192 * tp + 256 * m);
#pragma unroll
          for (int cb = 0; cb < RB; ++cb)
            acc[cb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[tp][cb], acc[cb][m], 0, 0, 0);
        }
      }
      if (!R::products_first) {
        IQ_PF_WAIT_VM(2 * per_page);
        unpack(pg + 2);
      }

      __builtin_amdgcn_s_waitcnt(kPfWaitLgkm0);
      __builtin_amdgcn_s_barrier();
    };

    f4 s_cur[4][RB], s_nxt[4][RB];
    scores(0, s_cur);
    int pg = 0;
    // two pages per iteration, the score sets trading places (no copies)
    for (; pg + 1 < n_full; pg += 2) {
      page_step(pg, s_cur, s_nxt, PfTag<false>{});
      page_step(pg + 1, s_nxt, s_cur, PfTag<false>{});
    }
    if (pg < n_full) {
      page_step(pg, s_cur, s_nxt, PfTag<false>{});
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) s_cur[tb][cb] = s_nxt[tb][cb];
      ++pg;
    }
    for (; pg < n_pages; ++pg) {
      page_step(pg, s_cur, s_nxt, PfTag<true>{});
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) s_cur[tb][cb] = s_nxt[tb][cb];
    }
    // the last requests (repeats of the last page) land before the kernel ends
    IQ_PF_WAIT_VM(0);
  };
  if (W == 4) {
    if (wave == 0) run(PfRole<true, true, true>{});
    else run(PfRole<true, true, false>{});
  } else {
    if (wave == 0) run(PfRole<true, false, true>{});
    else if (wave < 4) run(PfRole<true, false, false>{});
    else run(PfRole<false, true, false, false>{});
  }

  // ---- epilogue: normalise, rotate back (B^T then H / sqrt(d)), store ----
  const float* rot = a.rot + (size_t)g * kRotFloats;
  const bool failed = APP && s_fail;  // the appended pages never all arrived
#pragma unroll
  for (int cb = 0; cb < RB; ++cb) {
    const float l = sum_xor32(sum_xor16(l_run[cb]));  // in units of the frame, as acc
    const float scale = (l > 0.f) ? a.out_factor / l : 0.f;
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
    if (qi_row[cb] < n_q) {
      f4* dst = reinterpret_cast<f4*>(a.out +
                                      ((size_t)(row0 + qi_row[cb]) * a.hq + (size_t)g * a.group + head_row[cb]) * kD +
                                      32 * jq);
      const float nrm = failed ? NAN : 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dst[i] = f4{y[4 * i] * nrm, y[4 * i + 1] * nrm, y[4 * i + 2] * nrm, y[4 * i + 3] * nrm};
    }
  }
  if constexpr (APP) prefill_append_finish(a, g);
}

PrefillPlan plan_prefill(int n_q, int hq, int hkv, int q_start, int num_cus) {
  (void)q_start;
  (void)num_cus;
  PrefillPlan p;
  const int group = hq / hkv;
  const int qpt = kRowsPerTile / group;
  p.row_tiles = (n_q + qpt - 1) / qpt;
  p.kv_splits = 1;
  p.waves = 8;
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
  return launch_prefill_varlen(c, rot, q, q_dtype, 1, n_q, hq, nullptr, q_start, nullptr, block_table,
                               max_pages, plan, softmax_scale, out, workspace, stream);
}

hipError_t launch_prefill_varlen(const CacheView& c, const float* rot, const void* q, int q_dtype,
                                 int batch, int n_q, int hq, const int32_t* cu_q, int q_start,
                                 const int32_t* q_starts, const int32_t* block_table, int max_pages,
                                 const PrefillPlan& plan, float softmax_scale, float* out,
                                 void* workspace, hipStream_t stream) {
  (void)workspace;
  return launch_prefill_args(c, rot, q, q_dtype, batch, n_q, hq, cu_q, q_start, q_starts, block_table,
                             max_pages, plan, softmax_scale, out, nullptr, stream);
}

namespace {

// Workgroups of one prefill instantiation that a CU holds at once; cached.
template <int RB, int BITS>
int prefill_blocks_per_cu() {
  static std::atomic<int> cached{-1};
  int n = cached.load(std::memory_order_relaxed);
  if (n < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_kernel<RB, BITS, true>, 64 * pf_waves<RB>(), 0) !=
        hipSuccess)
      return 0;  // not cached: asked again next time
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

bool prefill_append_fused(const PrefillPlan& plan, int hkv, int bits, int num_cus) {
  if (hkv > kMaxCounterUnits) return false;
  const int bpc = plan.waves == 4 ? (bits == 4 ? prefill_blocks_per_cu<2, 4>() : prefill_blocks_per_cu<2, 3>())
                                  : (bits == 4 ? prefill_blocks_per_cu<1, 4>() : prefill_blocks_per_cu<1, 3>());
  return bpc > 0 && (long long)hkv * plan.row_tiles <= (long long)bpc * num_cus;
}

hipError_t launch_prefill_args(const CacheView& c, const float* rot, const void* q, int q_dtype,
                               int batch, int n_q, int hq, const int32_t* cu_q, int q_start,
                               const int32_t* q_starts, const int32_t* block_table, int max_pages,
                               const PrefillPlan& plan, float softmax_scale, float* out,
                               const PrefillAppend* app, hipStream_t stream) {
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
  a.cu_q = cu_q;
  a.q_starts = q_starts;
  a.max_pages = max_pages;
  const bool four = c.bits == 4;
  const double alpha = four ? (double)codebook4().alpha : (double)kLevelScale;
  a.lv4 = four ? codebook4().lv : Levels4{};
  const double log2e = 1.4426950408889634;
  a.score_factor = (float)((double)softmax_scale * log2e / (128.0 * alpha));
  a.out_factor = (float)(1.0 / (sqrt(128.0) * alpha));
  a.out = out;
  a.app_k = a.app_v = nullptr;
  a.app_arrive = a.app_done = nullptr;
  a.k_codes_w = nullptr;
  a.k_norms_w = nullptr;
  a.v_codes_w = nullptr;
  a.v_norms_w = nullptr;
  a.app_dtype = a.n_new = a.new_start = 0;
  a.row_tiles = plan.row_tiles;
  if (app) {
    a.app_k = app->k;
    a.app_v = app->v;
    a.app_dtype = app->dtype;
    a.n_new = app->n_new;
    a.new_start = app->new_start;
    a.k_codes_w = c.k_codes;
    a.k_norms_w = c.k_norms;
    a.v_codes_w = c.v_codes;
    a.v_norms_w = c.v_norms;
    a.app_arrive = app->counters;
    a.app_done = app->counters + kMaxCounterUnits;
  }
  const int rb = plan.waves == 4 ? 2 : 1;  // 16-row blocks per wave
  const dim3 grid(c.hkv, plan.row_tiles, batch);
#define IQ_PREFILL(RB, B, APP) \
  hipLaunchKernelGGL((prefill_kernel<RB, B, APP>), grid, dim3(64 * pf_waves<RB>()), 0, stream, a)
  const int sel = (rb == 2 ? 4 : 0) + (four ? 2 : 0) + (app ? 1 : 0);
  switch (sel) {
    case 0: IQ_PREFILL(1, 3, false); break;
    case 1: IQ_PREFILL(1, 3, true); break;
    case 2: IQ_PREFILL(1, 4, false); break;
    case 3: IQ_PREFILL(1, 4, true); break;
    case 4: IQ_PREFILL(2, 3, false); break;
    case 5: IQ_PREFILL(2, 3, true); break;
    case 6: IQ_PREFILL(2, 4, false); break;
    default: IQ_PREFILL(2, 4, true); break;
  }
#undef IQ_PREFILL
  return hipGetLastError();
}

}  // namespace iq
