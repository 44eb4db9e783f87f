// HIP kernels for gfx950 (MI355X) and the device half of the C ABI.
//
// Kernels
//   split_kv_*   one wavefront per split-KV item: streams a kv range of one request's
//                paged K/V for one KV head and scores it against up to 16 query columns
//                (rows x query heads of the group) with 16x16 MFMA tiles; keeps a running
//                max and sum per column and writes a partial (m, 1/l, acc/l).
//   combine      merges the partials of each (row, head) output with the log-sum-exp
//                rule and writes the output row.
//   gather       copies K/V into logical order through the same page addressing (for
//                the bit-exact gather test).
//
// The softmax runs in the base-2 domain: scores are multiplied by scale*log2(e) once and
// exponentiated with v_exp_f32, so the running max m is in those units too.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <type_traits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "device_common.h"
#include "va_internal.h"

namespace va {

// ----------------------------------------------------------------- split-KV, bf16 --
// MFMA v_mfma_f32_16x16x32_bf16 operand layout: lane l holds row/column (l % 16) and
// k-elements 8*(l/16) .. 8*(l/16)+7; the 16x16 f32 result gives lane l column (l % 16),
// rows 4*(l/16) .. 4*(l/16)+3.
//
// Scores are computed transposed, S^T = K . Q^T (keys on M, query columns on N), so a
// lane's results all belong to its own query column.  The K rows of the four 16-key
// blocks of a 64-key step are permuted so that lane group grp ends up holding keys
// 32u + 8*grp .. +7 of sub-step u -- exactly the k-slice the P^T operand of the
// O^T += V^T . P^T MFMA needs -- so P never leaves registers.  V^T's 8-key slices are
// contiguous because V pages are stored transposed.
// One wavefront runs item `idx`.  NC = blocks of 16 query columns: with NC = 2 the item has
// up to 32 columns (multi-row decode with g * rows > 16) and every K/V load serves both
// blocks, so the kv range is read once instead of twice.
template <int D, int NC>
__device__ __forceinline__ void split_kv_bf16_wave(
    int idx, const SplitItem* __restrict__ items, const Column* __restrict__ cols,
    const bf16* __restrict__ q, const bf16* __restrict__ kpool, const bf16* __restrict__ vpool,
    const int32_t* __restrict__ bt, int bt_stride, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    bf16* __restrict__ out, int Hq, Paged pg, float scale_log2) {
  constexpr int KC = D / 32;
  constexpr int DB = D / 16;
  const int lane = threadIdx.x & 63;
  const SplitItem it = items[idx];
  const int n = lane & 15, grp = lane >> 4;
  bool cvalid[NC];
  Column c[NC];
  int limit[NC];
  bf16x8 qb[NC][KC];
  f32x4 acc[NC][DB];
  float m_run[NC], l_run[NC];
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    cvalid[cb] = 16 * cb + n < it.ncols;
    c[cb] = cols[it.col0 + (cvalid[cb] ? 16 * cb + n : 0)];
    limit[cb] = cvalid[cb] ? c[cb].limit : -1;
    const bf16* qp = q + (size_t(c[cb].q_row) * Hq + c[cb].q_head) * D + 8 * grp;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qb[cb][kc] = *reinterpret_cast<const bf16x8*>(qp + 32 * kc);
      if (!cvalid[cb]) qb[cb][kc] = bf16x8{};
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[cb] = kNegBig;
    l_run[cb] = 0.f;
  }
  const int32_t* btr = bt + size_t(it.req) * bt_stride;
  const int kvh = it.kvh;
  const int klast = it.k1 - 1;
  const bool masked_item = (it.flags & kItemMasked) != 0;

  // Page ids: lane i holds the page of the item's (pbase + i)-th page, fetched with one
  // vector load per 64 pages, and a lane finds its key's page with a cross-lane read, so
  // no K/V load waits for a block-table load of its own.
  const int last_page = klast >> pg.ps_shift;
  int pbase = it.k0 >> pg.ps_shift;
  int pids = btr[min(pbase + lane, last_page)];
  auto cover = [&](int k) {            // make the 64 keys from k addressable
    if (((min(k + kStepKeys, it.k1) - 1) >> pg.ps_shift) - pbase >= 64) {
      pbase = k >> pg.ps_shift;
      pids = btr[min(pbase + lane, last_page)];
    }
  };
  auto page_at = [&](int pos) -> int { return __shfl(pids, (pos >> pg.ps_shift) - pbase); };

  // K rows (4 blocks x KC chunks) and V^T slices (2 sub-steps x DB rows) of a 64-key step.
  // The loop is rotated: step k+64's K loads are issued as soon as step k's scores are
  // computed, its V loads once step k's P . V is issued, so a load is in flight while
  // the previous step computes.
  bf16x8 ka[4][KC], va[2][DB];
  auto load_k = [&](int k) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int key = k + 32 * (b >> 1) + 8 * (n >> 2) + 4 * (b & 1) + (n & 3);
      const int kk = min(key, klast);
      const bf16* kr = kpool + pg.k_row(page_at(kk), kvh, pg.slot_of(kk)) + 8 * grp;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) ka[b][kc] = *reinterpret_cast<const bf16x8*>(kr + 32 * kc);
    }
  };
  auto load_v = [&](int k) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int vk = min(k + 32 * u + 8 * grp, klast & ~7);
      const bf16* vr = vpool + pg.v_elem(page_at(vk), kvh, n, pg.slot_of(vk));
#pragma unroll
      for (int db = 0; db < DB; ++db)
        va[u][db] = *reinterpret_cast<const bf16x8*>(vr + (size_t(16 * db) << pg.ps_shift));
    }
  };
  cover(it.k0);
  load_k(it.k0);
  load_v(it.k0);
  for (int k = it.k0; k < it.k1; k += kStepKeys) {
    const bool tail = k + kStepKeys > it.k1;
    const bool more = k + kStepKeys < it.k1;
    // ---- scores S^T for 64 keys: lane holds v[cb][4b + r] = key k + 32(b>>1) + 8grp + 4(b&1) + r
    float v[NC][16];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x4 s[NC];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) s[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) s[cb] = mfma16_bf16(ka[b][kc], qb[cb][kc], s[cb]);
#pragma unroll
      for (int cb = 0; cb < NC; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[cb][4 * b + r] = s[cb][r] * scale_log2;
    }
    if (more) {
      cover(k + kStepKeys);
      load_k(k + kStepKeys);
    }
    if (masked_item || tail) {
#pragma unroll
      for (int cb = 0; cb < NC; ++cb)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k + 32 * (b >> 1) + 8 * grp + 4 * (b & 1) + r;
            if (key > klast || key > limit[cb]) v[cb][4 * b + r] = -INFINITY;
          }
    }
    if (tail) {
      // positions at or past k1 may lie past kv_len (unwritten slots): zero them so
      // 0 * garbage cannot reach the accumulator
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int valid = it.k1 - (k + 32 * u + 8 * grp);
        if (valid < 8) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= valid) va[u][db][e] = bf16(0.f);
        }
      }
    }
    // ---- online softmax per column block (max shared by the 4 lane groups of a column)
    bf16x8 pb[NC][2];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      float mx = v[cb][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, v[cb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[cb], mx);
      const float alpha = fast_exp2(m_run[cb] - m_new);
      m_run[cb] = m_new;
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bf16 pe = bf16(fast_exp2(v[cb][4 * (2 * u + (e >> 2)) + (e & 3)] - m_new));
          pb[cb][u][e] = pe;
          sum += float(pe);
        }
      l_run[cb] = l_run[cb] * alpha + sum;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[cb][db] *= alpha;
    }
    // ---- O^T += V^T . P^T
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) acc[cb][db] = mfma16_bf16(va[u][db], pb[cb][u], acc[cb][db]);
    if (more) load_v(k + kStepKeys);
  }
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    float l_tot = l_run[cb] + __shfl_xor(l_run[cb], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (cvalid[cb]) {
      if (it.flags & kItemDirect)
        store_output<D>(out, (size_t(c[cb].q_row) * Hq + c[cb].q_head) * D, grp, l_tot, acc[cb]);
      else
        store_partial<D>(ws_ml, ws_acc, c[cb].pbase + it.slot, grp, m_run[cb], l_tot, acc[cb]);
    }
  }
}

template <int D, int NC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3 - NC, 3 - NC))) void split_kv_bf16_kernel(
    const SplitItem* __restrict__ items, int nitems, const Column* __restrict__ cols,
    const bf16* __restrict__ q, const bf16* __restrict__ kpool, const bf16* __restrict__ vpool,
    const int32_t* __restrict__ bt, int bt_stride, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    bf16* __restrict__ out, int Hq, Paged pg, float scale_log2) {
  const int idx = blockIdx.x * kSplitWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (idx < nitems)
    split_kv_bf16_wave<D, NC>(idx, items, cols, q, kpool, vpool, bt, bt_stride, ws_ml, ws_acc, out, Hq, pg,
                              scale_log2);
}

// ------------------------------------------------------------------ split-KV, fp32 --
// Same structure with v_mfma_f32_16x16x4_f32 (one k-element per lane: k = l / 16) and
// 16-key steps: S^T rows are keys k + 4*grp + r, and the r-th PV MFMA contracts the keys
// {k + 4*grp + r : grp = 0..3}.
template <int D>
__global__ __launch_bounds__(256) void split_kv_f32_kernel(
    const SplitItem* __restrict__ items, int nitems, const Column* __restrict__ cols,
    const float* __restrict__ q, const float* __restrict__ kpool, const float* __restrict__ vpool,
    const int32_t* __restrict__ bt, int bt_stride, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    float* __restrict__ out, int Hq, Paged pg, float scale_log2) {
  constexpr int KC = D / 4;
  constexpr int DB = D / 16;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int idx = blockIdx.x * kSplitWaves + wv;
  if (idx >= nitems) return;
  const SplitItem it = items[idx];
  const int n = lane & 15, grp = lane >> 4;
  const bool cvalid = n < it.ncols;
  const Column c = cols[it.col0 + (cvalid ? n : 0)];
  const int limit = cvalid ? c.limit : -1;
  float qb[KC];
  {
    const float* qp = q + (size_t(c.q_row) * Hq + c.q_head) * D + grp;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qb[kc] = cvalid ? qp[4 * kc] : 0.f;
  }
  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;
  const int32_t* btr = bt + size_t(it.req) * bt_stride;
  const int kvh = it.kvh;
  const int klast = it.k1 - 1;
  for (int k = it.k0; k < it.k1; k += 16) {
    const int kk = min(k + n, klast);
    const float* kr = kpool + pg.k_row(pg.page_of(btr, kk), kvh, pg.slot_of(kk)) + grp;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) s = mfma16_f32(kr[4 * kc], qb[kc], s);
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k + 4 * grp + r;
      v[r] = (key > klast || key > limit) ? -INFINITY : s[r] * scale_log2;
    }
    float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float p[4], sum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(v[r] - m_new);
      sum += p[r];
    }
    l_run = l_run * alpha + sum;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int vkey = k + 4 * grp + r;
      const int vk = min(vkey, klast);
      const int page = pg.page_of(btr, vk), slot = pg.slot_of(vk);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float x = vpool[pg.v_elem(page, kvh, 16 * db + n, slot)];
        if (vkey > klast) x = 0.f;
        acc[db] = mfma16_f32(x, p[r], acc[db]);
      }
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (cvalid) {
    if (it.flags & kItemDirect) store_output<D>(out, (size_t(c.q_row) * Hq + c.q_head) * D, grp, l_tot, acc);
    else store_partial<D>(ws_ml, ws_acc, c.pbase + it.slot, grp, m_run, l_tot, acc);
  }
}

// ------------------------------------------------------------ MFMA prefill, bf16 --
// One workgroup = one PrefillTile of up to 128 query columns (new rows x query heads of one
// KV head, row-major), 4 wavefronts of 32 columns each.  KV tiles of 64 positions are
// copied by LDS-DMA loads (buffer_load ... lds: lane i's 16 bytes land at the
// instruction's LDS base + 16*i, from a per-lane source address) into double-buffered LDS
// shared by the 4 waves; no staging registers.  Wave w copies keys [16w, 16w+16) of each
// tile, which lie in one page (page_size >= 16), so its page lookup and source base are
// wave-uniform.
//
// LDS layouts (16-byte chunks):
//   K   [key][KCH+1]: rows padded by one chunk, so the 16 lanes of an MFMA operand read
//       (16 different keys, same d-chunk) hit 16 distinct bank groups and every read is a
//       per-lane base plus an immediate offset.  The pad chunk receives a duplicate.
//   V^T [slice w][d][2]: keys 16w .. 16w+15 of row d as two chunks, the chunk order
//       flipped when bit 3 of d is set so the 16 rows read at one key-chunk position fall
//       on 16 distinct bank groups.
//
// Per wave, v_mfma_f32_32x32x16_bf16 computes S^T = K . Q^T for two 32-key blocks (keys
// on M, the wave's 32 columns on N) and O^T += V^T . P^T.  32x32x16 layouts: A/B operands
// give lane l row/column (l % 32) and k-elements 8*(l/32) .. +7; the 32x32 f32 result
// gives lane l column (l % 32) and rows 8*i + 4*(l/32) + j at element 4*i + j.  A-operand
// row rho of an S^T block holds key kappa(rho) = rho with bits 2 and 3 swapped, which
// puts keys 16*t + 8*(l/32) .. +7 of the block in elements 8*t .. 8*t+7 of lane l: the
// k-slice the P^T operand of the t-th PV MFMA needs.  So P stays in registers.
//
// Software pipeline: iteration j issues the copies of K(j+2) and V(j+1), exponentiates
// tile j's scores while the MFMAs of tile j+1's scores run, accumulates P(j) . V(j), then
// waits for its copies and meets the other waves at the one barrier per tile.
//
// Online softmax in base 2 with lazy rescaling: the reference max of a column only moves
// when a tile's max exceeds it by more than 8 (p <= 2^8 otherwise); the final division
// by the running sum makes the result independent of the reference.
constexpr int kPTileKeys = 64;
constexpr int kPSliceKeys = kPTileKeys / kPrefillWaves;   // keys each wave copies per tile
constexpr float kRescaleSlack = 8.f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sum8_bf16(bf16x8 p) {
  const bf16x2 one = {bf16(1.f), bf16(1.f)};
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) s = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[e], p[e + 1]}, one, s, false);
  return s;
}

// value of the other half-wave (lane l <-> lane l ^ 32)
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(threadIdx.x & 32 ? r[0] : r[1]);
}

// Buffer resource over one page slice (wave-uniform base, raw addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
// 4 bytes per lane from rs + voff into LDS at dst + 4 * lane.
__device__ __forceinline__ void dma_b32(__amdgpu_buffer_rsrc_t rs, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, voff, 0, 0, 0);
}
// 16 bytes per lane from rs + voff + soff into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma_b128(__amdgpu_buffer_rsrc_t rs, bf16x8* dst, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D>
struct PrefillLds {
  static constexpr int KCH = D / 8;                    // 16-byte chunks per K row
  static constexpr int KROW = KCH + 1;                 // padded K row
  // a wave's 16-key K slice is 16 padded rows, copied by whole 64-lane DMA instructions
  // (the last one's spare lanes land in the slack after the rows, so no instruction needs
  // a lane mask)
  static constexpr int KSS = (kPSliceKeys * KROW + 63) / 64 * 64;
  static constexpr int KBUF = kPrefillWaves * KSS;     // chunks per K buffer
  static constexpr int VBUF = kPTileKeys / 8 * D;      // chunks per V^T buffer
  static constexpr int bytes = 2 * (KBUF + VBUF) * 16;
  // fp8, per key: the K and V scales as copied (two stages); the K scale times log2 e and
  // the softmax scale, log2 of the V scale and its inverse as a bf16 pair hi + lo (three
  // tiles: they are made two tiles ahead)
  static constexpr int scale_bytes = 2 * kPTileKeys * (4 + 4) + 3 * kPTileKeys * (4 + 4 + 2 + 2);
};

template <int D, bool F8>
constexpr int prefill_lds_bytes() {
  return PrefillLds<D>::bytes + (F8 ? PrefillLds<D>::scale_bytes : 0);
}

// A tile's columns are consecutive (row, head) pairs of one request.  A whole tile scores
// keys [0, kv_end) and normalises and writes the output rows; a key-chunk tile (one chunk
// of a cut tile) scores keys [kbeg, kv_end) and writes the partial (m, 1/l, acc/l)
// of column col to workspace slot pbase + col * pstride, for the combine pass.
// A column-list tile takes its columns from cols[c0 ..] (rows of one or several requests,
// each with its own causal limit), scores keys [kbeg, kv_end) of request req's block table
// and writes column col's partial to slot cols[c0 + col].pbase + q0: a shared-prefix group
// tile (pages every member shares, visible to every member row; "How To Scale Your Model
// 笔记(7-8)", section 3: one load of a common KV block serves several requests' queries,
// each keeping its own running max and sum) or the tile of a member's own keys after them.
//
// F8 = true: the pools hold fp8 e4m3fn codes with per-position float32 scales.  Each wave
// copies its 16-key slice of codes by LDS-DMA into the upper part of the same slice's bf16
// area (and, with the K codes, the slice's 16 K and 16 V scales into the scale area), then,
// once its copies have landed, widens the codes in place, exactly, in the layouts above, so
// the MFMA loop is the bf16 one.  A key's K scale multiplies its scores; log2 of its V scale
// is added to them, so its exponential is the weight P gives its V codes, and the row sum
// adds that bf16 weight divided by the V scale: numerator and row sum use the same weights
// (the rounding of P moves weights, as in the bf16 path, not the output's scale).
// The slice is the wave's own, and all its reads precede its writes, so no other wave is
// involved until the barrier that ends the iteration.
// kStageGather: no attention.  Workgroup b takes request b / Hkv, KV head b % Hkv, all of
// its keys, stages every 64-key tile into LDS through the same page lookup, DMA addressing,
// wait and tail handling as the attention tiles, and copies the staged K rows and V^T
// slices out in logical order (GatherOut), so the production address path can be checked
// bit for bit.
enum TileMode { kWholeTile, kAnyTile, kStageGather };

struct GatherOut {
  const int64_t* kv_offset;   // [num_reqs + 1] prefix sums of kv_len
  bf16* k_out;                // [sum kv_len][Hkv][D]
  bf16* v_out;                // same
};

// Instantiations: kWholeTile runs whole tiles only; kAnyTile runs every kind (whole tiles,
// key-chunk tiles and column-list tiles: a plan with any of the latter launches all its
// tiles on it, so all kinds share the GPU in one launch).  Both end in one epilogue that
// normalises every column and only chooses where the row goes: with a separate epilogue
// for partial results the compiler laid out the main loop differently and tiles ran 2-6 %
// slower.  The whole-tile kernel keeps the shorter set-up of consecutive columns.
template <int D, int MODE, bool F8>
__global__ __launch_bounds__(64 * kPrefillWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_bf16_kernel(
    const PrefillTile* __restrict__ tiles, const Column* __restrict__ cols, const bf16* __restrict__ q,
    const void* __restrict__ kpool, const void* __restrict__ vpool, const float* __restrict__ kscale,
    const float* __restrict__ vscale, const int32_t* __restrict__ bt, int bt_stride, bf16* __restrict__ out,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc, int Hq, int g, Paged pg, float scale_log2,
    GatherOut go) {
  using Lay = PrefillLds<D>;
  constexpr int KCH = Lay::KCH, KROW = Lay::KROW, KBUF = Lay::KBUF, VBUF = Lay::VBUF, KSS = Lay::KSS;
  constexpr int WK = kPSliceKeys;                      // 16 keys per wave slice
  static_assert(WK == 16, "slice layout assumes 16 keys per wave");
  constexpr int KSC = WK * KROW;                       // K slice chunks (with pad)
  constexpr int KNI = KSS / 64;                        // DMA instructions per K slice
  constexpr int KLAST = KSC - 64 * (KNI - 1);          // lanes of the last one that hold rows
  // whole tiles (prefill, MFMA-bound) issue their copies inside the loop's main block;
  // the other tiles (key chunks and column lists, mostly streaming KV from HBM) at the
  // top of each iteration, where the copies have the whole iteration to land
  constexpr bool kInBlockCopies = MODE == kWholeTile && !F8;
  constexpr int VSC = WK / 8 * D;                      // V^T slice chunks
  constexpr int VNI = VSC / 64;
  static_assert(VNI * 64 == VSC, "V^T slice must be whole instructions");
  extern __shared__ bf16x8 smem[];
  bf16x8* sK = smem;                                   // [2][KBUF]
  bf16x8* sV = smem + 2 * KBUF;                        // [2][VBUF]
  float* sKs = reinterpret_cast<float*>(smem + 2 * KBUF + 2 * VBUF);   // fp8: [2][64] K scales
  float* sVs = sKs + 2 * kPTileKeys;                                  // fp8: [2][64] V scales
  float* sKl = sVs + 2 * kPTileKeys;                                  // fp8: [3][64] K scale * log2 e * scale
  float* sLv = sKl + 3 * kPTileKeys;                                  // fp8: [3][64] log2 |V scale|
  bf16* sVh = reinterpret_cast<bf16*>(sLv + 3 * kPTileKeys);          // fp8: [3][64] 1 / |V scale|, hi
  bf16* sVl = sVh + 3 * kPTileKeys;                                   // fp8: [3][64] 1 / |V scale|, lo

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const PrefillTile T = [&] {
    if constexpr (MODE == kStageGather) {
      const int r = int(blockIdx.x) / pg.Hkv;
      const int L = int(go.kv_offset[r + 1] - go.kv_offset[r]);
      return PrefillTile{r, int(blockIdx.x) % pg.Hkv, 0, 0, 0, 0, L, 0, -1, 0, 0, 0};
    } else {
      return tiles[blockIdx.x];
    }
  }();
  const int h = lane >> 5;
  const int rho = lane & 31;
  const int kap = (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);   // swap bits 2 and 3
  const int col = wv * 32 + rho;
  const bool cvalid = col < T.ncols;
  const int c = T.c0 + (cvalid ? col : 0);
  int row, head, limit, w_min_limit, w_max_limit, kbeg, pslot;
  if constexpr (MODE == kAnyTile) {
    const int kl = T.kv_end - 1;
    kbeg = T.kbeg;
    if (T.flags & kTileColumnList) {
      // columns of a list, each with its own causal limit (clipped to the tile's keys)
      const Column cc = cols[c];
      row = cc.q_row;
      head = cc.q_head;
      pslot = cc.pbase + T.q0;
      limit = cvalid ? min(cc.limit, kl) : -1;
      int lo = cvalid ? limit : INT_MAX, hi = limit;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        lo = min(lo, __shfl_xor(lo, off));
        hi = max(hi, __shfl_xor(hi, off));
      }
      w_min_limit = __builtin_amdgcn_readfirstlane(lo);
      w_max_limit = __builtin_amdgcn_readfirstlane(hi);
    } else {
      const int i = c / g;
      row = T.q0 + i;
      head = T.kvh * g + c % g;
      pslot = T.pbase + col * T.pstride;
      // a key chunk before the last one ends before the diagonal: clip the limits to its
      // end (a no-op for whole tiles, which end one past their last row's last key)
      limit = cvalid ? min(T.S0 + i, kl) : -1;
      const int wcol_last = min(wv * 32 + 31, T.ncols - 1);
      w_min_limit = min(T.S0 + (T.c0 + wv * 32) / g, kl);
      w_max_limit = (wv * 32 < T.ncols) ? min(T.S0 + (T.c0 + wcol_last) / g, kl) : -1;
    }
  } else {
    const int i = c / g;
    row = T.q0 + i;
    head = T.kvh * g + c % g;
    pslot = 0;
    kbeg = 0;
    limit = cvalid ? T.S0 + i : -1;
    // the wave's first and last visible positions bound its causal work
    const int wcol_last = min(wv * 32 + 31, T.ncols - 1);
    w_min_limit = T.S0 + (T.c0 + wv * 32) / g;
    w_max_limit = (wv * 32 < T.ncols) ? T.S0 + (T.c0 + wcol_last) / g : -1;
  }

  bf16x8 qb[D / 16];
  if constexpr (MODE != kStageGather) {
    const bf16* qp = q + (size_t(row) * Hq + head) * D + 8 * h;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qb[kc] = *reinterpret_cast<const bf16x8*>(qp + 16 * kc);
      if (!cvalid) qb[kc] = bf16x8{};
    }
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  const int32_t* btr = bt + size_t(T.req) * bt_stride;
  const int kvh = T.kvh;
  const int kv_end = T.kv_end;
  const int ntiles = (kv_end - kbeg + kPTileKeys - 1) / kPTileKeys;   // tile t: keys kbeg + 64t ..
  const int ps_mask = (1 << pg.ps_shift) - 1;
  constexpr int EB = F8 ? 1 : 2;                       // bytes per stored element
  const size_t page_bytes = ((size_t(pg.Hkv) * D) << pg.ps_shift) * EB;
  const char* kbase = static_cast<const char*>(kpool) + pg.k_row(0, kvh, 0) * EB;
  const char* vbase = static_cast<const char*>(vpool) + pg.v_elem(0, kvh, 0, 0) * EB;
  // fp8: raw slice sizes (16-byte chunks) and where they sit inside the bf16 slices
  constexpr int KR = WK * D / 16;                      // K codes of the slice
  constexpr int VR = D;                                // V codes: one chunk (16 keys) per d
  constexpr int KRAW = KSS - KR;                       // raw K codes at the top of the slice
  constexpr int VRAW = VSC - VR;
  static_assert(KRAW >= 0 && VRAW >= 0, "raw fp8 slices must fit in the bf16 slices");

  // ---- per-lane DMA source offsets (bytes from the slice base)
  // K instruction r, lane -> slice chunk L = 64r + lane = (key L / KROW, d-chunk L % KROW);
  // the pad chunk copies d-chunk 0 again.
  uint32_t koff[KNI];
#pragma unroll
  for (int r = 0; r < KNI; ++r) {
    const int L = min(64 * r + lane, KSC - 1);
    koff[r] = uint32_t(((L / KROW) * D + 8 * min(L % KROW, KCH - 1)) * 2);
  }
  // V^T instruction r, lane -> slice chunk 64r + lane = (row d = 32r + lane/2, position
  // lane & 1), holding the slice's key-chunk (lane & 1) ^ bit 3 of d; r adds 32 rows.
  const int vd = lane >> 1;
  const int vkc = (lane & 1) ^ ((vd >> 3) & 1);
  const uint32_t voff = uint32_t(((vd << pg.ps_shift) + 8 * vkc) * 2);
  const int vrstep = (32 << pg.ps_shift) * 2;

  auto page_for = [&](int t) -> int {
    return pg.page_of(btr, min(kbeg + t * kPTileKeys + wv * WK, kv_end - 1));
  };
  // FULL: tile t is not the last one, so every slice holds 16 keys before the end
  auto issue_k = [&](int t, int page, int buf, bool full) {
    const int k0w = kbeg + t * kPTileKeys + wv * WK;
    if (!full && k0w >= kv_end) return;      // positions past the end: scores are masked
    const auto rs = slice_rsrc(kbase + size_t(page) * page_bytes + size_t(k0w & ps_mask) * D * EB);
    bf16x8* dst = sK + buf * KBUF + wv * KSS;
    if constexpr (F8) {
      // codes: lane -> raw chunk L = 64r + lane = (key L / (D/16), 16-byte piece L % (D/16))
#pragma unroll
      for (int r = 0; r < KR / 64; ++r) dma_b128(rs, dst + KRAW + 64 * r, uint32_t(16 * (64 * r + lane)), 0);
      // the key's K and V scales come with its K codes (the V scales are turned into log2
      // and inverse two tiles ahead, for the scores of the tile after next)
      const auto rsk = slice_rsrc(kscale + pg.scale_idx(page, kvh, k0w & ps_mask));
      const auto rsv = slice_rsrc(vscale + pg.scale_idx(page, kvh, k0w & ps_mask));
      if (lane < WK) {
        dma_b32(rsk, sKs + buf * kPTileKeys + wv * WK, uint32_t(4 * lane));
        dma_b32(rsv, sVs + buf * kPTileKeys + wv * WK, uint32_t(4 * lane));
      }
    } else {
#pragma unroll
      for (int r = 0; r < KNI; ++r)
        if (kInBlockCopies || r < KNI - 1 || lane < KLAST) dma_b128(rs, dst + 64 * r, koff[r], 0);
    }
  };
  auto issue_v = [&](int t, int page, int buf, bool full) {
    const int k0w = kbeg + t * kPTileKeys + wv * WK;
    bf16x8* dst = sV + buf * VBUF + wv * VSC;
    if (!full && k0w >= kv_end) {             // never read garbage into V: write zeros
#pragma unroll
      for (int r = 0; r < VNI; ++r) dst[64 * r + lane] = bf16x8{};
      return;
    }
    const auto rs = slice_rsrc(vbase + size_t(page) * page_bytes + (k0w & ps_mask) * EB);
    if constexpr (F8) {
      // codes: lane -> raw chunk d = 64r + lane, the 16 keys of V page row d
#pragma unroll
      for (int r = 0; r < VR / 64; ++r) dma_b128(rs, dst + VRAW + 64 * r, uint32_t((64 * r + lane) << pg.ps_shift), 0);
    } else {
#pragma unroll
      for (int r = 0; r < VNI; ++r) dma_b128(rs, dst + 64 * r, voff, r * vrstep);
    }
  };
  // fp8: widen the slice's codes in place, exactly (scale 1), once its copies have landed
  // (own slice only).  The scales act on the scores in base-2 units: a key's score is
  // (q . k_codes) * (s_K * log2 e * softmax scale) + log2 s_V, so its exponential is its
  // probability times s_V (the weight P gives its V codes), and the row sum adds that
  // rounded weight times 1 / s_V: numerator and row sum use the same weights.
  auto convert_k = [&](int t, int buf) {
    if constexpr (F8) {
      const int k0w = kbeg + t * kPTileKeys + wv * WK;
      if (lane < WK) {
        // key `lane` of the slice: K scale times log2 e and the softmax scale; log2 and
        // inverse of |V scale| into slot t % 3 (a V scale below the normal range, i.e. V
        // magnitudes under about 5e-36 or a zero scale, counts as 1 with the codes zeroed,
        // so 1 / s never overflows; positions past the end get zeros: finite, and masked)
        const int si = buf * kPTileKeys + wv * WK + lane, so = (t % 3) * kPTileKeys + wv * WK + lane;
        float kl = 0.f, ls = 0.f, inv = 0.f;
        if (k0w + lane < kv_end) {
          kl = sKs[si] * scale_log2;
          const float sv = fabsf(sVs[si]);
          const bool tiny = sv < FLT_MIN;
          // hardware log2 and reciprocal (about 1 ulp; s is normal here): the weights use
          // the same inverse in numerator and row sum, so only its f32 rounding remains
          ls = tiny ? 0.f : __builtin_amdgcn_logf(sv);
          inv = tiny ? 1.f : __builtin_amdgcn_rcpf(sv);
        }
        const bf16 hi = bf16(inv);
        sKl[so] = kl;
        sLv[so] = ls;
        sVh[so] = hi;
        sVl[so] = bf16(inv - float(hi));
      }
      if (k0w >= kv_end) return;
      bf16x8* sl = sK + buf * KBUF + wv * KSS;
      constexpr int PER = KR / 64;                      // raw chunks per lane
      bf16x8 raw[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) raw[i] = sl[KRAW + 64 * i + lane];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int L = 64 * i + lane, key = L / (D / 16), pc = L % (D / 16);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&raw[i]);
        sl[key * KROW + 2 * pc] = fp8x8_to_bf16(w[0], w[1]);
        sl[key * KROW + 2 * pc + 1] = fp8x8_to_bf16(w[2], w[3]);
      }
    }
  };
  auto convert_v = [&](int t, int buf) {
    if constexpr (F8) {
      const int k0w = kbeg + t * kPTileKeys + wv * WK;
      if (k0w >= kv_end) return;                        // zeros were written instead
      bf16x8* sl = sV + buf * VBUF + wv * VSC;
      constexpr int PER = VR / 64;
      bf16x8 raw[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) raw[i] = sl[VRAW + 64 * i + lane];
      const int valid = kv_end - k0w;                   // keys of the slice before the end
      // key `lane` of the slice (its V scale, copied with its K codes, is still in place):
      // positions at or past the end may be unwritten slots and a V scale below the normal
      // range counts as 1, so those keys' codes are zeroed (0 * NaN would still be NaN); a
      // negative V scale flips the key's codes (the weights use |s|)
      bool tiny = false, neg = false;
      if (lane < WK && lane < valid) {
        const float sv = sVs[buf * kPTileKeys + wv * WK + lane];
        tiny = fabsf(sv) < FLT_MIN;
        neg = sv < 0.f && !tiny;
      }
      const uint32_t zmask = uint32_t(__ballot(lane < WK && (lane >= valid || tiny)));   // keys to zero
      const uint32_t nmask = uint32_t(__ballot(neg));                                   // keys to negate
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int d = 64 * i + lane;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&raw[i]);
        bf16x8 o[2] = {fp8x8_to_bf16(w[0], w[1]), fp8x8_to_bf16(w[2], w[3])};
        if (zmask | nmask) {
#pragma unroll
          for (int k = 0; k < WK; ++k) {
            if ((nmask >> k) & 1) o[k >> 3][k & 7] = -o[k >> 3][k & 7];
            if ((zmask >> k) & 1) o[k >> 3][k & 7] = bf16(0.f);
          }
        }
        const int flip = (d >> 3) & 1;
        sl[2 * d + flip] = o[0];
        sl[2 * d + (flip ^ 1)] = o[1];
      }
    }
  };
  // after the copy of V(t) landed: zero the positions at or past the tile's end (they may
  // be unwritten slots; their scores are masked, but 0 * NaN would still be NaN)
  auto fix_v_tail = [&](int t, int buf) {
    if constexpr (F8) return;                 // the widening zeroes those positions
    const int k0w = kbeg + t * kPTileKeys + wv * WK;
    if (k0w >= kv_end || k0w + WK <= kv_end) return;
    bf16x8* dst = sV + buf * VBUF + wv * VSC;
    const int valid = kv_end - (k0w + 8 * vkc);
#pragma unroll
    for (int r = 0; r < VNI; ++r) {
      bf16x8 x = dst[64 * r + lane];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e >= valid) x[e] = bf16(0.f);
      dst[64 * r + lane] = x;
    }
  };

  // fp8, tiles tk (K codes and scales landed in K buffer bk) and tv (V codes in V buffer
  // bv) both whole (every key before the end): convert_k(tk) and convert_v(tv) without
  // branches, every LDS read first, so the wave waits on LDS once instead of once per step.
  // Lanes 16-63 repeat lane & 15's scale work and write the same values to the same slots.
  auto widen_full = [&](int tk, int bk, int tv, int bv) {
    if constexpr (F8) {
      const int key = lane & (WK - 1);
      bf16x8* kl = sK + bk * KBUF + wv * KSS;
      bf16x8* vl = sV + bv * VBUF + wv * VSC;
      constexpr int KP = KR / 64, VP = VR / 64;
      bf16x8 kraw[KP], vraw[VP];
#pragma unroll
      for (int i = 0; i < KP; ++i) kraw[i] = kl[KRAW + 64 * i + lane];
#pragma unroll
      for (int i = 0; i < VP; ++i) vraw[i] = vl[VRAW + 64 * i + lane];
      const float ks = sKs[bk * kPTileKeys + wv * WK + key];
      const float vs_k = sVs[bk * kPTileKeys + wv * WK + key];   // V scale of tile tk's key
      const float vs_v = sVs[bv * kPTileKeys + wv * WK + key];   // V scale of tile tv's key
      // tile tk's per-key terms (see convert_k)
      const float sv = fabsf(vs_k);
      const bool tiny_k = sv < FLT_MIN;
      const float ls = tiny_k ? 0.f : __builtin_amdgcn_logf(sv);
      const float inv = tiny_k ? 1.f : __builtin_amdgcn_rcpf(sv);
      const bf16 hi = bf16(inv);
      const int so = (tk % 3) * kPTileKeys + wv * WK + key;
      sKl[so] = ks * scale_log2;
      sLv[so] = ls;
      sVh[so] = hi;
      sVl[so] = bf16(inv - float(hi));
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const int L = 64 * i + lane, kk = L / (D / 16), pc = L % (D / 16);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&kraw[i]);
        kl[kk * KROW + 2 * pc] = fp8x8_to_bf16(w[0], w[1]);
        kl[kk * KROW + 2 * pc + 1] = fp8x8_to_bf16(w[2], w[3]);
      }
      // tile tv's V codes (see convert_v): zeroed where the scale is below the normal
      // range, negated where it is negative
      const bool tiny_v = fabsf(vs_v) < FLT_MIN;
      const uint32_t zmask = uint32_t(__ballot(lane < WK && tiny_v));
      const uint32_t nmask = uint32_t(__ballot(lane < WK && vs_v < 0.f && !tiny_v));
#pragma unroll
      for (int i = 0; i < VP; ++i) {
        const int d = 64 * i + lane;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&vraw[i]);
        bf16x8 o[2] = {fp8x8_to_bf16(w[0], w[1]), fp8x8_to_bf16(w[2], w[3])};
        if (zmask | nmask) {
#pragma unroll
          for (int k = 0; k < WK; ++k) {
            if ((nmask >> k) & 1) o[k >> 3][k & 7] = -o[k >> 3][k & 7];
            if ((zmask >> k) & 1) o[k >> 3][k & 7] = bf16(0.f);
          }
        }
        const int flip = (d >> 3) & 1;
        vl[2 * d + flip] = o[0];
        vl[2 * d + (flip ^ 1)] = o[1];
      }
    }
  };

  // ---- per-wave compute pieces
  const int kread = (kap >> 4) * KSS + (kap & 15) * KROW + h;       // + 2*b*KSS + 2*kc
  const int vread = rho * 2 + (h ^ ((rho >> 3) & 1));               // + (2b+t)*VSC + 64*db
  auto qk_block = [&](int buf, int b, f32x16& sn) {
    const bf16x8* kb = sK + buf * KBUF + kread + 2 * b * KSS;
#pragma unroll
    for (int e = 0; e < 16; ++e) sn[e] = 0.f;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) sn = mfma32_bf16(kb[2 * kc], qb[kc], sn);
  };
  // element 8t + x of a 32-key block's scores (and of its probabilities) is key
  // 32b + 16t + 8h + x of the 64-key tile
  // fp8 scores of tile t (scale slot t % 3) in base 2 with log2 |s_V| added
  auto k_scale_block = [&](int slot, int b, f32x16& sn) {
    if constexpr (F8) {
      const f32x4* ks = reinterpret_cast<const f32x4*>(sKl + slot * kPTileKeys + 32 * b + 8 * h);
      const f32x4* lv = reinterpret_cast<const f32x4*>(sLv + slot * kPTileKeys + 32 * b + 8 * h);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x4 f = ks[4 * t + u], l2 = lv[4 * t + u];
#pragma unroll
          for (int x = 0; x < 4; ++x) sn[8 * t + 4 * u + x] = fmaf(sn[8 * t + 4 * u + x], f[x], l2[x]);
        }
    }
  };
  // exponentials of a 32-key block's arguments (scores in base 2 less the running max)
  auto exp_block = [&](const f32x16& ex, int slot, int b, bf16x8 (&pb)[2]) {
    if constexpr (F8) {
      // the arguments include log2 |s_V|: the exponential is p * |s_V|, and the row sum
      // adds bf16(p * |s_V|) / |s_V|, the inverse taken as hi + lo bf16 parts
      const bf16x8* ih = reinterpret_cast<const bf16x8*>(sVh + slot * kPTileKeys + 32 * b + 8 * h);
      const bf16x8* il = reinterpret_cast<const bf16x8*>(sVl + slot * kPTileKeys + 32 * b + 8 * h);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[t][e] = bf16(fast_exp2(ex[8 * t + e]));
        const bf16x8 hi = ih[2 * t], lo = il[2 * t];
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 w = {pb[t][e], pb[t][e + 1]};
          ls[0] = __builtin_amdgcn_fdot2_f32_bf16(w, bf16x2{hi[e], hi[e + 1]}, ls[0], false);
          ls[1] = __builtin_amdgcn_fdot2_f32_bf16(w, bf16x2{lo[e], lo[e + 1]}, ls[1], false);
        }
        l_run += ls[0] + ls[1];
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[t][e] = bf16(fast_exp2(ex[8 * t + e]));
        l_run += sum8_bf16(pb[t]);
      }
    }
  };
  // the causal mask on tile t's scores (keys past a column's last visible position)
  auto mask_tile = [&](int t, f32x16 (&sn)[2]) {
    const int k0 = kbeg + t * kPTileKeys;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ii = e >> 2, jj = e & 3;
        const int key = k0 + 32 * b + 16 * (ii >> 1) + 8 * h + 4 * (ii & 1) + jj;
        if (key > limit) sn[b][e] = -INFINITY;
      }
  };
  // tile t's running max and exponent arguments ex (lazy rescaling: the reference max moves
  // only when the tile's max passes it by more than the slack; then the row sum, which holds
  // the tiles before t, is scaled by alpha here, and the accumulator before t's P.V)
  float alpha = 1.f;
  bool rescale = false;
  auto next_args = [&](const f32x16 (&sn)[2], f32x16 (&ex)[2]) {
    float mx = sn[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sn[b][e]);
    mx = fmaxf(mx, other_half(mx));
    const float m_tile = F8 ? mx : mx * scale_log2;    // fp8 scores are already in base 2
    const bool need = m_tile > m_run + kRescaleSlack;
    const float m_new = need ? m_tile : m_run;
    alpha = fast_exp2(m_run - m_new);
    rescale = __any(need);
    l_run *= alpha;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) ex[b][e] = F8 ? sn[b][e] - m_run : fmaf(sn[b][e], scale_log2, -m_run);
  };
  auto pv_tile = [&](int buf, const bf16x8 (&p)[2][2]) {
    const bf16x8* vb = sV + buf * VBUF + vread;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[db] = mfma32_bf16(vb[(2 * b + t) * VSC + 64 * db], p[b][t], acc[db]);
  };

  if constexpr (MODE == kStageGather) {
    // stage each 64-key tile as the attention tiles do, then copy it out in logical order:
    // K row kl of wave slice ws is chunks ws*KSS + kl*KROW + (0 .. KCH-1); element d of
    // key kl of V^T slice ws is element kl % 8 of chunk ws*VSC + 2d + ((kl / 8) ^ bit 3 of d)
    const int64_t obase = go.kv_offset[T.req];
    for (int t = 0; t < ntiles; ++t) {
      const int pt = page_for(t);
      issue_k(t, pt, 0, false);
      issue_v(t, pt, 0, false);
      wait_vmem();
      fix_v_tail(t, 0);
      __syncthreads();
      for (int e = tid; e < kPTileKeys * KCH; e += 64 * kPrefillWaves) {
        const int key = e / KCH, ch = e % KCH, pos = t * kPTileKeys + key;
        if (pos >= kv_end) continue;
        const int ws = key / WK, kl = key % WK;
        const size_t o = ((size_t(obase) + pos) * pg.Hkv + kvh) * D + 8 * ch;
        *reinterpret_cast<bf16x8*>(go.k_out + o) = sK[ws * KSS + kl * KROW + ch];
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = 8 * ch + i;
          v[i] = sV[ws * VSC + 2 * d + ((kl >> 3) ^ ((d >> 3) & 1))][kl & 7];
        }
        *reinterpret_cast<bf16x8*>(go.v_out + o) = v;
      }
      __syncthreads();
    }
    return;
  }

  // ---- prologue: K(0), K(1), V(0) in LDS; scores of tile 0 and their exponent arguments
  int p1 = ntiles > 1 ? page_for(1) : 0;
  {
    const int p0 = page_for(0);
    issue_k(0, p0, 0, false);
    issue_v(0, p0, 0, false);
    if (ntiles > 1) issue_k(1, p1, 1, false);
    wait_vmem();
    fix_v_tail(0, 0);
    convert_k(0, 0);
    convert_v(0, 0);
    if (ntiles > 1) convert_k(1, 1);
  }
  int p2 = ntiles > 2 ? page_for(2) : 0;
  int p3 = ntiles > 3 ? page_for(3) : 0;
  __syncthreads();
  // the last tile with keys this wave's columns see (-1: none), and the first whose keys pass
  // the first visible position of one of them (it and those after it need the mask); every
  // wave still copies its slice of every tile and meets the others at every barrier
  const int j_last = w_max_limit >= kbeg ? min(ntiles - 1, (w_max_limit - kbeg) / kPTileKeys) : -1;
  const int t_mask = w_min_limit - kbeg - (kPTileKeys - 1) < 0 ? 0 : (w_min_limit - kbeg - (kPTileKeys - 1)) / kPTileKeys + 1;
  f32x16 ex[2], sn[2];
  if (j_last >= 0) {
    qk_block(0, 0, sn[0]);
    qk_block(0, 1, sn[1]);
    k_scale_block(0, 0, sn[0]);
    k_scale_block(0, 1, sn[1]);
    if (t_mask == 0) mask_tile(0, sn);
    next_args(sn, ex);
    rescale = false;                          // the accumulator is still zero
  }
  __syncthreads();

  auto stage_in = [&](int j) {                // copies of K(j+2) and V(j+1)
    if (j + 2 < ntiles) issue_k(j + 2, p2, j & 1, false);
    if (j + 1 < ntiles) issue_v(j + 1, p1, (j + 1) & 1, false);
    p1 = p2;
    p2 = p3;
    if (j + 4 < ntiles) p3 = page_for(j + 4);
  };
  auto stage_done = [&](int j) {              // those copies landed (and widened): barrier
    wait_vmem();
    if (j + 1 < ntiles) fix_v_tail(j + 1, (j + 1) & 1);
    if (j + 2 < ntiles) convert_k(j + 2, j & 1);
    if (j + 1 < ntiles) convert_v(j + 1, (j + 1) & 1);
    __syncthreads();
  };
  // iteration j < j_last: tile j+1's scores (MFMA) under tile j's exponentials (VALU), then
  // tile j's P.V (MFMA) under tile j+1's max and exponent arguments (VALU).  MASKED: tile
  // j+1 needs the causal mask.  FAST (tiles j+1 and j+2 not the last: no tail to clear,
  // every copy whole, fp8 codes widened without branches): from the first MFMA to the
  // barrier one basic block, so the compiler keeps each VALU part beside the MFMAs it
  // overlaps.  IN_BLOCK (fast bf16 whole tiles): the copies are issued inside that block,
  // K(j+2) between the two score blocks and V(j+1) before the P.V, instead of all waves of
  // the workgroup issuing them at once after the barrier (the copy queue then holds each
  // wave for hundreds of cycles).  A rescale decided for tile j+1 is applied to the
  // accumulator at the top of the next iteration, after tile j's P.V and before tile j+1's.
  auto step = [&](int j, auto masked, auto fast) {
    constexpr bool FAST = decltype(fast)::value;
    if (rescale) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    }
    constexpr bool IN_BLOCK = FAST && kInBlockCopies;
    if constexpr (!FAST) {
      stage_in(j);
    } else if constexpr (!IN_BLOCK) {
      issue_k(j + 2, p2, j & 1, true);
      issue_v(j + 1, p1, (j + 1) & 1, true);
      p1 = p2;
      p2 = p3;
      p3 = page_for(j + 4);                   // clamped to the last key: always a valid entry
    }
    bf16x8 p[2][2];
    // LLVM's MFMA/LDS interleaving strategy 0 reads operands further ahead of their
    // MFMAs (whole tiles: chunk mix -2 %; the key-chunk and column-list tiles, which
    // wait on HBM, ran 1-9 % slower with it)
    if constexpr (IN_BLOCK) __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      qk_block((j + 1) & 1, b, sn[b]);
      exp_block(ex[b], j % 3, b, p[b]);
      if (IN_BLOCK && b == 0) issue_k(j + 2, p2, j & 1, true);
    }
    k_scale_block((j + 1) % 3, 0, sn[0]);
    k_scale_block((j + 1) % 3, 1, sn[1]);
    if constexpr (decltype(masked)::value) mask_tile(j + 1, sn);
    if constexpr (IN_BLOCK) {
      issue_v(j + 1, p1, (j + 1) & 1, true);
      p1 = p2;
      p2 = p3;
      p3 = page_for(j + 4);
    }
    pv_tile(j & 1, p);
    next_args(sn, ex);
    if constexpr (FAST) {
      __builtin_amdgcn_sched_barrier(0);      // the wait stays after all of the block's work
      wait_vmem();
      widen_full(j + 2, j & 1, j + 1, (j + 1) & 1);
      __syncthreads();
    } else {
      stage_done(j);
    }
  };
  using no = std::false_type;
  using yes = std::true_type;
  int j = 0;
  const int j_nm = min(j_last, max(0, t_mask - 1));   // j < j_nm: tile j+1 needs no mask
  const int j_f = min(j_last, ntiles - 3);             // j < j_f: fast
  for (; j < min(j_nm, j_f); ++j) step(j, no{}, yes{});
  for (; j < j_nm; ++j) step(j, no{}, no{});
  for (; j < j_f; ++j) step(j, yes{}, yes{});
  for (; j < j_last; ++j) step(j, yes{}, no{});
  if (j == j_last) {                          // the wave's last tile: exponentials and P.V
    if (rescale) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    }
    stage_in(j);
    bf16x8 p[2][2];
    exp_block(ex[0], j % 3, 0, p[0]);
    exp_block(ex[1], j % 3, 1, p[1]);
    pv_tile(j & 1, p);
    stage_done(j);
    ++j;
  }
  for (; j < ntiles; ++j) {
    stage_in(j);
    stage_done(j);
  }
  // ---- normalise and write: acc[db][4*ii + jj] is d = 32*db + 8*ii + 4*h + jj of this column
  const float l_tot = l_run + other_half(l_run);
  const bool part = MODE == kAnyTile && (T.pbase >= 0 || (T.flags & kTileColumnList));
  if (cvalid) {
    const float inv = MODE == kAnyTile ? (l_tot > 0.f ? 1.f / l_tot : 0.f) : 1.f / l_tot;
    if (part && h == 0) *reinterpret_cast<float2*>(ws_ml + 2 * size_t(pslot)) = float2{m_run, inv};
    float* wa = ws_acc + (part ? size_t(pslot) * D + 4 * h : 0);   // whole tiles have no slot
    bf16* op = out + (size_t(row) * Hq + head) * D + 4 * h;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        f32x4 o4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o4[jj] = acc[db][4 * ii + jj] * inv;
        if (part) {
          *reinterpret_cast<f32x4*>(wa + 32 * db + 8 * ii) = o4;
        } else {
          bf16x4 b4;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b4[jj] = bf16(o4[jj]);
          *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * ii) = b4;
        }
      }
  }
}


// ------------------------------------------------------------------------ combine --
// Partial s holds (m_s, 1/l_s, o_s = acc_s / l_s); with M = max_s m_s and weights
// w_s = 2^(m_s - M) l_s (0 for a part that saw no key, stored as 1/l = 0),
// out = sum_s w_s o_s / sum_s w_s, the same as sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const CombineRow* __restrict__ rows, int nrows,
                                                      const float* __restrict__ ws_ml,
                                                      const float* __restrict__ ws_acc, OutT* __restrict__ out,
                                                      int Hq) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (idx >= nrows) return;
  const CombineRow r = rows[idx];
  // lane s holds part s0 + s's (m, l), so the per-part scalars load in parallel; the
  // accumulator rows (lane d holds d, d + 64, ..) are loaded eight parts at a time
  float M = -INFINITY;
  for (int s0 = 0; s0 < r.nparts; s0 += 64)
    if (s0 + lane < r.nparts) M = fmaxf(M, ws_ml[2 * size_t(r.pbase + s0 + lane)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f;
  float o[D / 64];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) o[j] = 0.f;
  for (int s0 = 0; s0 < r.nparts; s0 += 64) {
    float w = 0.f;
    if (s0 + lane < r.nparts) {
      const size_t slot = size_t(r.pbase + s0 + lane);
      const float inv = ws_ml[2 * slot + 1];
      w = inv > 0.f ? fast_exp2(ws_ml[2 * slot] - M) / inv : 0.f;
      L += w;
    }
    const int n = min(64, r.nparts - s0);
    for (int t = 0; t < n; t += 8) {
      float a[8][D / 64], wt[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = t + u < n;
        wt[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), t + u)) : 0.f;
        const float* ap = ws_acc + size_t(r.pbase + s0 + (ok ? t + u : 0)) * D + lane;
#pragma unroll
        for (int j = 0; j < D / 64; ++j) a[u][j] = ap[64 * j];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < D / 64; ++j) o[j] += wt[u] * a[u][j];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
  const float inv = 1.f / L;
  OutT* op = out + (size_t(r.q_row) * Hq + r.q_head) * D + lane;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) op[64 * j] = OutT(o[j] * inv);
}

// --------------------------------------------------------------------- stream read --
// Reads n16 16-byte words once: each workgroup streams one contiguous span (so the DRAM
// pages it touches are read whole), its lanes reading consecutive words, eight loads in
// flight per lane.  The data decides whether a store to the sink happens (rarely), so the
// loads stay.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t span = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = int64_t(blockIdx.x) * span, hi = min(n16, lo + span);
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    uint4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = buf[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
  }
  for (; i < hi; i += 256) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// ------------------------------------------------------------------------- gather --
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const int64_t* __restrict__ kv_offset, int num_reqs,
                                                     int64_t total_elems, const int32_t* __restrict__ bt,
                                                     int bt_stride, const T* __restrict__ kpool,
                                                     const T* __restrict__ vpool, T* __restrict__ kout,
                                                     T* __restrict__ vout, Paged pg) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= total_elems) return;
  const int d = int(t % pg.D);
  const int kvh = int((t / pg.D) % pg.Hkv);
  const int64_t pos = t / (int64_t(pg.D) * pg.Hkv);
  int lo = 0, hi = num_reqs - 1;   // last request with kv_offset[r] <= pos
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kv_offset[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  const int j = int(pos - kv_offset[lo]);
  const int32_t* btr = bt + size_t(lo) * bt_stride;
  const int page = pg.page_of(btr, j), slot = pg.slot_of(j);
  kout[t] = kpool[pg.k_row(page, kvh, slot) + d];
  vout[t] = vpool[pg.v_elem(page, kvh, d, slot)];
}

// ------------------------------------------------------------------ host helpers --
static va_status hip_fail(const char* what, hipError_t e) {
  return fail(VA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool prefill_kernel_available(const va_params& p) {
  return (p.dtype == VA_DTYPE_BF16 || p.dtype == VA_DTYPE_FP8_E4M3) && (p.head_dim == 64 || p.head_dim == 128);
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static va_status prepare_kernels() {
  // the prefill kernel's dynamic LDS exceeds the 64 KiB default limit
  static hipError_t once = [] {
    const std::pair<const void*, int> kernels[] = {
#define VA_PREFILL_KERNEL(D, M, F) {reinterpret_cast<const void*>(&prefill_bf16_kernel<D, M, F>), prefill_lds_bytes<D, F>()}
        VA_PREFILL_KERNEL(128, kWholeTile, false), VA_PREFILL_KERNEL(64, kWholeTile, false),
        VA_PREFILL_KERNEL(128, kAnyTile, false), VA_PREFILL_KERNEL(64, kAnyTile, false),
        VA_PREFILL_KERNEL(128, kWholeTile, true),  VA_PREFILL_KERNEL(64, kWholeTile, true),
        VA_PREFILL_KERNEL(128, kAnyTile, true),  VA_PREFILL_KERNEL(64, kAnyTile, true),
        VA_PREFILL_KERNEL(128, kStageGather, false), VA_PREFILL_KERNEL(64, kStageGather, false)};
#undef VA_PREFILL_KERNEL
    for (const auto& k : kernels) {
      const hipError_t e = hipFuncSetAttribute(k.first, hipFuncAttributeMaxDynamicSharedMemorySize, k.second);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  return once == hipSuccess ? VA_OK : hip_fail("hipFuncSetAttribute(max dynamic LDS)", once);
}

int device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

va_status upload_plan(va_plan* plan) {
  if (va_status st = prepare_kernels(); st != VA_OK) return st;
  const size_t b_items = align256(plan->items.size() * sizeof(SplitItem));
  const size_t b_cols = align256(plan->cols.size() * sizeof(Column));
  const size_t b_comb = align256(plan->combine.size() * sizeof(CombineRow));
  const size_t b_tiles = align256(plan->tiles.size() * sizeof(PrefillTile));
  const size_t b_off = align256(plan->kv_offset.size() * sizeof(int64_t));
  const size_t total = b_items + b_cols + b_comb + b_tiles + b_off;
  std::vector<char> host(total, 0);
  size_t o = 0;
  auto put = [&](const void* src, size_t n, size_t span) {
    if (n) std::memcpy(host.data() + o, src, n);
    const size_t at = o;
    o += span;
    return at;
  };
  const size_t o_items = put(plan->items.data(), plan->items.size() * sizeof(SplitItem), b_items);
  const size_t o_cols = put(plan->cols.data(), plan->cols.size() * sizeof(Column), b_cols);
  const size_t o_comb = put(plan->combine.data(), plan->combine.size() * sizeof(CombineRow), b_comb);
  const size_t o_tiles = put(plan->tiles.data(), plan->tiles.size() * sizeof(PrefillTile), b_tiles);
  const size_t o_off = put(plan->kv_offset.data(), plan->kv_offset.size() * sizeof(int64_t), b_off);
  hipError_t e = hipGetDevice(&plan->device);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  e = hipMalloc(&plan->dev, total);
  if (e != hipSuccess) {
    plan->dev = nullptr;
    return fail(VA_ERR_OUT_OF_MEMORY, std::string("hipMalloc of the plan buffer: ") + hipGetErrorString(e));
  }
  plan->dev_bytes = total;
  e = hipMemcpy(plan->dev, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(plan->dev);
    plan->dev = nullptr;
    return hip_fail("hipMemcpy of the plan buffer", e);
  }
  char* base = static_cast<char*>(plan->dev);
  plan->d_items = reinterpret_cast<const SplitItem*>(base + o_items);
  plan->d_cols = reinterpret_cast<const Column*>(base + o_cols);
  plan->d_combine = reinterpret_cast<const CombineRow*>(base + o_comb);
  plan->d_tiles = reinterpret_cast<const PrefillTile*>(base + o_tiles);
  plan->d_kv_offset = reinterpret_cast<const int64_t*>(base + o_off);
  return VA_OK;
}

void free_plan_device(va_plan* plan) {
  if (plan->dev) (void)hipFree(plan->dev);
  plan->dev = nullptr;
}

static int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace va

using namespace va;

// k_scale / v_scale: the scale pools of an fp8 plan (NULL otherwise).
static va_status run_impl(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scale, const float* v_scale, const int32_t* block_table_dev, void* out,
                          void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  if (!plan) return fail(VA_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->dev) return fail(VA_ERR_INVALID_ARG, "plan has no device buffer (built with VA_FLAG_HOST_ONLY)");
  const bool fp8 = plan->p.dtype == VA_DTYPE_FP8_E4M3;
  const bool any = !plan->items.empty() || !plan->tiles.empty();
  if (!any && !events) return VA_OK;
  if (any && (!q || !k_pool || !v_pool || !block_table_dev || !out))
    return fail(VA_ERR_INVALID_ARG, "q, k_pool, v_pool, block_table_dev and out must be non-NULL");
  if (any && fp8) {
    if (!k_scale || !v_scale) return fail(VA_ERR_INVALID_ARG, "k_scale and v_scale must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale) |
         reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15)
      return fail(VA_ERR_INVALID_ARG, "fp8 pools and scale pools must be 16-byte aligned");
  }
  if (workspace_bytes < plan->ws_bytes)
    return fail(VA_ERR_WORKSPACE_TOO_SMALL, "workspace has " + std::to_string(workspace_bytes) + " bytes, plan needs " +
                                                std::to_string(plan->ws_bytes));
  if (plan->ws_bytes && !workspace) return fail(VA_ERR_INVALID_ARG, "workspace is NULL");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev != plan->device) return fail(VA_ERR_INVALID_ARG, "current HIP device is not the one the plan was built on");

  const va_params& p = plan->p;
  const int D = p.head_dim;
  const float scale = p.softmax_scale > 0.f ? p.softmax_scale : 1.f / std::sqrt(float(D));
  const float scale_log2 = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Paged pg{p.num_kv_heads, log2i(p.page_size), D};
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->ws_ml_off);
  float* ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->ws_acc_off);
  const int nitems = int(plan->items.size());
  const int ncomb = int(plan->combine.size());
  const int bt_stride = p.max_pages_per_req;
  const bool bf = p.dtype != VA_DTYPE_F32;     // bf16 Q and output (bf16 and fp8 plans)

  (void)hipGetLastError();   // clear a stale error left by earlier, unrelated calls
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : hipSuccess;
  };
  if ((e = mark(0)) != hipSuccess) return hip_fail("hipEventRecord", e);
  const int ntiles = int(plan->tiles.size());
  const int nwhole = plan->tiles_whole, nchunk = ntiles - nwhole;   // the rest run on kAnyTile
  auto launch_tiles = [&](auto mode, auto f8, const PrefillTile* tl, int n) {
    constexpr int M = decltype(mode)::value;
    constexpr bool F = decltype(f8)::value;
    const dim3 grid(n), block(64 * kPrefillWaves);
    auto* qq = static_cast<const bf16*>(q);
    auto* oo = static_cast<bf16*>(out);
    if (D == 128)
      prefill_bf16_kernel<128, M, F><<<grid, block, prefill_lds_bytes<128, F>(), s>>>(
          tl, plan->d_cols, qq, k_pool, v_pool, k_scale, v_scale, block_table_dev, bt_stride, oo, ws_ml, ws_acc,
          p.num_q_heads, plan->g, pg, scale_log2, GatherOut{});
    else
      prefill_bf16_kernel<64, M, F><<<grid, block, prefill_lds_bytes<64, F>(), s>>>(
          tl, plan->d_cols, qq, k_pool, v_pool, k_scale, v_scale, block_table_dev, bt_stride, oo, ws_ml, ws_acc,
          p.num_q_heads, plan->g, pg, scale_log2, GatherOut{});
    return hipGetLastError();
  };
  auto launch_kind = [&](auto mode, const PrefillTile* tl, int n) {
    return fp8 ? launch_tiles(mode, std::true_type{}, tl, n) : launch_tiles(mode, std::false_type{}, tl, n);
  };
  using Whole = std::integral_constant<int, kWholeTile>;
  using Any = std::integral_constant<int, kAnyTile>;
  if (nwhole && (e = launch_kind(Whole{}, plan->d_tiles, nwhole)) != hipSuccess)
    return hip_fail("prefill kernel launch", e);
  if (nchunk && (e = launch_kind(Any{}, plan->d_tiles + nwhole, nchunk)) != hipSuccess)
    return hip_fail("prefill kernel launch (any tile)", e);
  if ((e = mark(1)) != hipSuccess) return hip_fail("hipEventRecord", e);
  if (nitems) {
    const dim3 grid((nitems + kSplitWaves - 1) / kSplitWaves), block(64 * kSplitWaves);
    e = hipSuccess;
    if (fp8) {
      e = launch_split_kv_fp8(D, nitems, plan->items_wide, s, plan->d_items, plan->d_cols, q, k_pool, v_pool, k_scale, v_scale,
                          block_table_dev, bt_stride, ws_ml, ws_acc, out, p.num_q_heads, pg, scale_log2);
    } else if (bf) {
      auto* qq = static_cast<const bf16*>(q);
      auto* kk = static_cast<const bf16*>(k_pool);
      auto* vv = static_cast<const bf16*>(v_pool);
      // items of more than 16 columns (first in the list) on the two-block kernel
      const int nw = plan->items_wide, nn = nitems - nw;
      const dim3 gw((nw + kSplitWaves - 1) / kSplitWaves), gn((nn + kSplitWaves - 1) / kSplitWaves);
      const SplitItem* in = plan->d_items + nw;
      if (D == 128) {
        if (nw)
          split_kv_bf16_kernel<128, 2><<<gw, block, 0, s>>>(plan->d_items, nw, plan->d_cols, qq, kk, vv,
                                                            block_table_dev, bt_stride, ws_ml, ws_acc,
                                                            static_cast<bf16*>(out), p.num_q_heads, pg, scale_log2);
        if (nn)
          split_kv_bf16_kernel<128, 1><<<gn, block, 0, s>>>(in, nn, plan->d_cols, qq, kk, vv, block_table_dev,
                                                            bt_stride, ws_ml, ws_acc, static_cast<bf16*>(out),
                                                            p.num_q_heads, pg, scale_log2);
      } else {
        if (nw)
          split_kv_bf16_kernel<64, 2><<<gw, block, 0, s>>>(plan->d_items, nw, plan->d_cols, qq, kk, vv,
                                                           block_table_dev, bt_stride, ws_ml, ws_acc,
                                                           static_cast<bf16*>(out), p.num_q_heads, pg, scale_log2);
        if (nn)
          split_kv_bf16_kernel<64, 1><<<gn, block, 0, s>>>(in, nn, plan->d_cols, qq, kk, vv, block_table_dev,
                                                           bt_stride, ws_ml, ws_acc, static_cast<bf16*>(out),
                                                           p.num_q_heads, pg, scale_log2);
      }
    } else {
      auto* qq = static_cast<const float*>(q);
      auto* kk = static_cast<const float*>(k_pool);
      auto* vv = static_cast<const float*>(v_pool);
      if (D == 128)
        split_kv_f32_kernel<128><<<grid, block, 0, s>>>(plan->d_items, nitems, plan->d_cols, qq, kk, vv,
                                                        block_table_dev, bt_stride, ws_ml, ws_acc,
                                                        static_cast<float*>(out), p.num_q_heads, pg, scale_log2);
      else
        split_kv_f32_kernel<64><<<grid, block, 0, s>>>(plan->d_items, nitems, plan->d_cols, qq, kk, vv,
                                                       block_table_dev, bt_stride, ws_ml, ws_acc,
                                                       static_cast<float*>(out), p.num_q_heads, pg, scale_log2);
    }
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("split-KV kernel launch", e);
  }
  if ((e = mark(2)) != hipSuccess) return hip_fail("hipEventRecord", e);
  if (ncomb) {
    const dim3 grid((ncomb + 3) / 4), block(256);
    if (bf) {
      auto* o = static_cast<bf16*>(out);
      if (D == 128)
        combine_kernel<128, bf16><<<grid, block, 0, s>>>(plan->d_combine, ncomb, ws_ml, ws_acc, o, p.num_q_heads);
      else
        combine_kernel<64, bf16><<<grid, block, 0, s>>>(plan->d_combine, ncomb, ws_ml, ws_acc, o, p.num_q_heads);
    } else {
      auto* o = static_cast<float*>(out);
      if (D == 128)
        combine_kernel<128, float><<<grid, block, 0, s>>>(plan->d_combine, ncomb, ws_ml, ws_acc, o, p.num_q_heads);
      else
        combine_kernel<64, float><<<grid, block, 0, s>>>(plan->d_combine, ncomb, ws_ml, ws_acc, o, p.num_q_heads);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail("combine kernel launch", e);
  }
  if ((e = mark(3)) != hipSuccess) return hip_fail("hipEventRecord", e);
  return VA_OK;
}

extern "C" va_status varlen_attn_run(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table_dev, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (plan && plan->p.dtype == VA_DTYPE_FP8_E4M3)
    return fail(VA_ERR_INVALID_ARG, "an fp8 plan runs with varlen_attn_run_fp8 (it needs the scale pools)");
  return run_impl(plan, q, k_pool, v_pool, nullptr, nullptr, block_table_dev, out, workspace, workspace_bytes, stream,
                  nullptr);
}

extern "C" va_status varlen_attn_run_fp8(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_table_dev, void* out, void* workspace,
                                         size_t workspace_bytes, void* stream, void* const* events) {
  if (plan && plan->p.dtype != VA_DTYPE_FP8_E4M3)
    return fail(VA_ERR_INVALID_ARG, "varlen_attn_run_fp8 needs a plan built with dtype VA_DTYPE_FP8_E4M3");
  if (events)
    for (int i = 0; i < VA_RUN_EVENTS; ++i)
      if (!events[i]) return fail(VA_ERR_INVALID_ARG, "events[" + std::to_string(i) + "] is NULL");
  return run_impl(plan, q, k_pool, v_pool, k_scale, v_scale, block_table_dev, out, workspace, workspace_bytes, stream,
                  events);
}

// ------------------------------------------------------------- static scratch --
// The workspace of varlen_attn_run_noalloc: a file-scope device array (every GPU the
// library runs on holds its own copy until the process ends).  In host code `scratch` names
// a host-side stand-in, not device memory: its device address is looked up once per device
// with hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[VA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev` (the current device), looked up on the first
// call for that device.
va_status static_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return fail(VA_ERR_UNSUPPORTED, "device ordinal beyond the static scratch table");
  void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return hip_fail("hipGetSymbolAddress(static scratch)", e);
      g_scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return VA_OK;
}
}  // namespace

extern "C" va_status varlen_attn_run_noalloc(const va_plan* plan, const void* q, const void* k_pool,
                                             const void* v_pool, const int32_t* block_table_dev, void* out,
                                             void* stream) {
  if (!plan) return fail(VA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->p.dtype == VA_DTYPE_FP8_E4M3)
    return fail(VA_ERR_INVALID_ARG, "an fp8 plan runs with varlen_attn_run_fp8 (it needs the scale pools)");
  if (plan->ws_bytes > VA_STATIC_SCRATCH_BYTES)
    return fail(VA_ERR_WORKSPACE_TOO_SMALL, "plan needs " + std::to_string(plan->ws_bytes) +
                                                " bytes of workspace, the static scratch holds " +
                                                std::to_string(size_t(VA_STATIC_SCRATCH_BYTES)) +
                                                ": run it with varlen_attn_run and a workspace");
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  void* ws = nullptr;
  if (plan->ws_bytes) {
    if (va_status st = static_scratch(dev, &ws); st != VA_OK) return st;
  }
  return run_impl(plan, q, k_pool, v_pool, nullptr, nullptr, block_table_dev, out, ws, plan->ws_bytes, stream,
                  nullptr);
}

extern "C" va_status varlen_attn_run_events(const va_plan* plan, const void* q, const void* k_pool,
                                            const void* v_pool, const int32_t* block_table_dev, void* out,
                                            void* workspace, size_t workspace_bytes, void* stream,
                                            void* const* events) {
  if (!events) return fail(VA_ERR_INVALID_ARG, "events is NULL");
  for (int i = 0; i < VA_RUN_EVENTS; ++i)
    if (!events[i]) return fail(VA_ERR_INVALID_ARG, "events[" + std::to_string(i) + "] is NULL");
  if (plan && plan->p.dtype == VA_DTYPE_FP8_E4M3)
    return fail(VA_ERR_INVALID_ARG, "an fp8 plan runs with varlen_attn_run_fp8 (it needs the scale pools)");
  return run_impl(plan, q, k_pool, v_pool, nullptr, nullptr, block_table_dev, out, workspace, workspace_bytes, stream,
                  events);
}

extern "C" va_status varlen_attn_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return VA_OK;
  if (!buf || !sink) return fail(VA_ERR_INVALID_ARG, "buf and sink must be non-NULL");
  if ((bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return fail(VA_ERR_INVALID_ARG, "buf must be 16-byte aligned and bytes a multiple of 16");
  (void)hipGetLastError();
  stream_read_kernel<<<dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(buf), int64_t(bytes / 16), sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("stream read kernel launch", e);
  return VA_OK;
}

extern "C" va_status varlen_attn_debug_stage_gather(const va_plan* plan, const void* k_pool, const void* v_pool,
                                                    const int32_t* block_table_dev, void* k_out, void* v_out,
                                                    void* stream) {
  if (!plan) return fail(VA_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->dev) return fail(VA_ERR_INVALID_ARG, "plan has no device buffer (built with VA_FLAG_HOST_ONLY)");
  const va_params& p = plan->p;
  if (p.dtype != VA_DTYPE_BF16)
    return fail(VA_ERR_UNSUPPORTED, "the staged gather covers bf16 pools (the attention tiles' bf16 staging)");
  if (plan->num_reqs == 0 || plan->kv_offset.back() == 0) return VA_OK;
  if (!k_pool || !v_pool || !block_table_dev || !k_out || !v_out)
    return fail(VA_ERR_INVALID_ARG, "pointer argument is NULL");
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out) | reinterpret_cast<uintptr_t>(k_pool) |
       reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(VA_ERR_INVALID_ARG, "pools and outputs must be 16-byte aligned");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev != plan->device) return fail(VA_ERR_INVALID_ARG, "current HIP device is not the one the plan was built on");
  Paged pg{p.num_kv_heads, log2i(p.page_size), p.head_dim};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(int64_t(plan->num_reqs) * p.num_kv_heads)), block(64 * kPrefillWaves);
  const GatherOut go{plan->d_kv_offset, static_cast<bf16*>(k_out), static_cast<bf16*>(v_out)};
  (void)hipGetLastError();
  if (p.head_dim == 128)
    prefill_bf16_kernel<128, kStageGather, false><<<grid, block, prefill_lds_bytes<128, false>(), s>>>(
        nullptr, nullptr, nullptr, k_pool, v_pool, nullptr, nullptr, block_table_dev, p.max_pages_per_req, nullptr,
        nullptr, nullptr, p.num_q_heads, plan->g, pg, 0.f, go);
  else
    prefill_bf16_kernel<64, kStageGather, false><<<grid, block, prefill_lds_bytes<64, false>(), s>>>(
        nullptr, nullptr, nullptr, k_pool, v_pool, nullptr, nullptr, block_table_dev, p.max_pages_per_req, nullptr,
        nullptr, nullptr, p.num_q_heads, plan->g, pg, 0.f, go);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("staged gather kernel launch", e);
  return VA_OK;
}

extern "C" va_status varlen_attn_debug_gather(const va_plan* plan, const void* k_pool, const void* v_pool,
                                              const int32_t* block_table_dev, void* k_out, void* v_out,
                                              void* stream) {
  if (!plan) return fail(VA_ERR_INVALID_ARG, "plan is NULL");
  if (!plan->dev) return fail(VA_ERR_INVALID_ARG, "plan has no device buffer (built with VA_FLAG_HOST_ONLY)");
  const va_params& p = plan->p;
  const int64_t total = plan->kv_offset.back() * p.num_kv_heads * p.head_dim;
  if (total == 0 || plan->num_reqs == 0) return VA_OK;
  if (!k_pool || !v_pool || !block_table_dev || !k_out || !v_out)
    return fail(VA_ERR_INVALID_ARG, "pointer argument is NULL");
  Paged pg{p.num_kv_heads, log2i(p.page_size), p.head_dim};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  (void)hipGetLastError();
  if (p.dtype == VA_DTYPE_FP8_E4M3)
    gather_kernel<uint8_t><<<grid, block, 0, s>>>(plan->d_kv_offset, plan->num_reqs, total, block_table_dev,
                                                  p.max_pages_per_req, static_cast<const uint8_t*>(k_pool),
                                                  static_cast<const uint8_t*>(v_pool), static_cast<uint8_t*>(k_out),
                                                  static_cast<uint8_t*>(v_out), pg);
  else if (p.dtype == VA_DTYPE_BF16)
    gather_kernel<bf16><<<grid, block, 0, s>>>(plan->d_kv_offset, plan->num_reqs, total, block_table_dev,
                                               p.max_pages_per_req, static_cast<const bf16*>(k_pool),
                                               static_cast<const bf16*>(v_pool), static_cast<bf16*>(k_out),
                                               static_cast<bf16*>(v_out), pg);
  else
    gather_kernel<float><<<grid, block, 0, s>>>(plan->d_kv_offset, plan->num_reqs, total, block_table_dev,
                                                p.max_pages_per_req, static_cast<const float*>(k_pool),
                                                static_cast<const float*>(v_pool), static_cast<float*>(k_out),
                                                static_cast<float*>(v_out), pg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail("gather kernel launch", e);
  return VA_OK;
}
