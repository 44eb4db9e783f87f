// Split-KV attention over fp8 KV pools (gfx950).
//
// K and V are stored as OCP fp8 e4m3fn codes in the same page layouts as the bf16 pools
// (K [page][kv_head][slot][d], V [page][kv_head][d][slot]) plus one float32 scale per
// (page, kv_head, slot) for K and one for V: the stored value of a position's element d
// is code * scale.  The codes are widened to bf16 on chip (exactly: every e4m3fn value is
// a bf16 value) and the products run on the bf16 MFMA with fp32 accumulation, so the
// fp8 storage halves the bytes read and leaves the arithmetic as in the bf16 path.
// The scales are applied in fp32 outside the MFMAs: a K scale multiplies its key's scores
// before the softmax, a V scale multiplies its key's probability before P is rounded to
// bf16 for the P.V product, and the row sum adds the weight that product gives the key's
// values (the rounded product over the scale).
// The file also holds the append of new rows into fp8 pools (quantisation + scatter).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <string>
#include <type_traits>

#include "device_common.h"
#include "va_internal.h"

namespace va {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One wavefront runs item `idx` (same item / column records and partial layout as the
// bf16 split-KV kernel).
//
// Lane (n = lane % 16, grp = lane / 16).  The head dimension is split into four
// contiguous quarters, one per lane group: MFMA chunk kc of lane group grp contracts
// d = (D/4)*grp + 8*kc .. +7, for Q and K alike, so a lane's K bytes of one row are one
// contiguous run of D/4 bytes.  Key rows of the four 16-key blocks b of a 64-key step
// are key(b, i) = k + 16*(i/4) + 4*b + i%4, so after S^T = K . Q^T lane group grp holds
// the scores of the 16 consecutive keys k + 16*grp .. +15 (v[4b + r] is key
// k + 16*grp + 4b + r); those are also the keys of its V^T slice (16 contiguous bytes of
// a transposed V page row) and of its 16 scales, and P sub-step u element e is key
// k + 16*grp + 8*u + e.  Items start at multiples of 16 and pages hold >= 16 positions,
// so each 16-key run lies in one page.  NC = blocks of 16 query columns per item (2 for
// items of 17-32 columns): each widened K/V operand then feeds one MFMA per block.
template <int D, int NC>
__device__ __forceinline__ void split_kv_fp8_wave(
    int idx, const SplitItem* __restrict__ items, const Column* __restrict__ cols, const bf16* __restrict__ q,
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const float* __restrict__ kscale,
    const float* __restrict__ vscale, const int32_t* __restrict__ bt, int bt_stride, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, bf16* __restrict__ out, int Hq, Paged pg, float scale_log2) {
  constexpr int KC = D / 32;        // MFMA k-chunks of 8 per lane
  constexpr int NL = D / 64;        // 16-byte K loads per lane and key row
  constexpr int DB = D / 16;
  constexpr int QD = D / 4;         // head-dim quarter of a lane group
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
    const bf16* qp = q + (size_t(c[cb].q_row) * Hq + c[cb].q_head) * D + QD * grp;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qb[cb][kc] = *reinterpret_cast<const bf16x8*>(qp + 8 * kc);
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

  const int last_page = klast >> pg.ps_shift;
  int pbase = it.k0 >> pg.ps_shift;
  int pids = btr[min(pbase + lane, last_page)];
  auto cover = [&](int k) {
    if (((min(k + kStepKeys, it.k1) - 1) >> pg.ps_shift) - pbase >= 64) {
      pbase = k >> pg.ps_shift;
      pids = btr[min(pbase + lane, last_page)];
    }
  };
  auto page_at = [&](int pos) -> int { return __shfl(pids, (pos >> pg.ps_shift) - pbase); };

  // first key of the lane group's 16-key run, clamped to the run holding the last key
  auto run_start = [&](int k) { return min(k + 16 * grp, klast & ~15); };
  u32x4 ka[4][NL], va[DB];
  f32x4 ks[4], vs[4];
  auto load_k = [&](int k) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int key = min(k + 16 * (n >> 2) + 4 * b + (n & 3), klast);
      const uint8_t* kr = kpool + pg.k_row(page_at(key), kvh, pg.slot_of(key)) + QD * grp;
#pragma unroll
      for (int j = 0; j < NL; ++j) ka[b][j] = *reinterpret_cast<const u32x4*>(kr + 16 * j);
    }
    const int kb = run_start(k);
    const float* sp = kscale + pg.scale_idx(page_at(kb), kvh, pg.slot_of(kb));
#pragma unroll
    for (int i = 0; i < 4; ++i) ks[i] = *reinterpret_cast<const f32x4*>(sp + 4 * i);
  };
  auto load_v = [&](int k) {
    const int kb = run_start(k);
    const int page = page_at(kb), slot = pg.slot_of(kb);
    const uint8_t* vr = vpool + pg.v_elem(page, kvh, n, slot);
#pragma unroll
    for (int db = 0; db < DB; ++db) va[db] = *reinterpret_cast<const u32x4*>(vr + (size_t(16 * db) << pg.ps_shift));
    const float* sp = vscale + pg.scale_idx(page, kvh, slot);
#pragma unroll
    for (int i = 0; i < 4; ++i) vs[i] = *reinterpret_cast<const f32x4*>(sp + 4 * i);
  };
  cover(it.k0);
  load_k(it.k0);
  load_v(it.k0);
  for (int k = it.k0; k < it.k1; k += kStepKeys) {
    const bool tail = k + kStepKeys > it.k1;
    const bool more = k + kStepKeys < it.k1;
    // ---- scores S^T for 64 keys, times the keys' K scales
    float v[NC][16];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x4 s[NC];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) s[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const bf16x8 k0 = fp8x8_to_bf16(ka[b][j][0], ka[b][j][1]);
        const bf16x8 k1 = fp8x8_to_bf16(ka[b][j][2], ka[b][j][3]);
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
          s[cb] = mfma16_bf16(k0, qb[cb][2 * j], s[cb]);
          s[cb] = mfma16_bf16(k1, qb[cb][2 * j + 1], s[cb]);
        }
      }
#pragma unroll
      for (int cb = 0; cb < NC; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[cb][4 * b + r] = s[cb][r] * (ks[b][r] * scale_log2);
    }
    if (more) {
      cover(k + kStepKeys);
      load_k(k + kStepKeys);
    }
    // P carries each key's V scale s; the row sum adds the weights the MFMA applies to the
    // key's values, bf16(p * s) / s.  A scale below the normal range (V magnitudes under
    // about 5e-36, or zero) keeps p unscaled and zeroes the key's codes instead.
    float vsc[16], vin[16];
    uint32_t tiny = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float sv = vs[i >> 2][i & 3];
      const bool t = fabsf(sv) < FLT_MIN;
      tiny |= uint32_t(t) << i;
      vsc[i] = t ? 1.f : sv;
      vin[i] = t ? 1.f : __builtin_amdgcn_rcpf(sv);
    }
    if (masked_item || tail) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k + 16 * grp + i;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
          if (key > klast || key > limit[cb]) v[cb][i] = -INFINITY;
        // scales past the item's end may belong to unwritten slots: keep them out of P
        if (key > klast) vsc[i] = vin[i] = 0.f;
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
      for (int i = 0; i < 16; ++i) {
        const bf16 w = bf16(fast_exp2(v[cb][i] - m_new) * vsc[i]);
        pb[cb][i >> 3][i & 7] = w;
        sum = fmaf(float(w), vin[i], sum);
      }
      l_run[cb] = l_run[cb] * alpha + sum;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[cb][db] *= alpha;
    }
    // ---- O^T += V^T . P^T; codes at or past k1 may be unwritten slots: zeroed
    const int valid = it.k1 - (k + 16 * grp);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x8 v0 = fp8x8_to_bf16(va[db][0], va[db][1]);
      bf16x8 v1 = fp8x8_to_bf16(va[db][2], va[db][3]);
      if (tail && valid < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (e >= valid) v0[e] = bf16(0.f);
          if (8 + e >= valid) v1[e] = bf16(0.f);
        }
      }
      if (__any(tiny != 0)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if ((tiny >> e) & 1) v0[e] = bf16(0.f);
          if ((tiny >> (8 + e)) & 1) v1[e] = bf16(0.f);
        }
      }
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        acc[cb][db] = mfma16_bf16(v0, pb[cb][0], acc[cb][db]);
        acc[cb][db] = mfma16_bf16(v1, pb[cb][1], acc[cb][db]);
      }
    }
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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3 - NC, 3 - NC))) void split_kv_fp8_kernel(
    const SplitItem* __restrict__ items, int nitems, const Column* __restrict__ cols, const bf16* __restrict__ q,
    const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool, const float* __restrict__ kscale,
    const float* __restrict__ vscale, const int32_t* __restrict__ bt, int bt_stride, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, bf16* __restrict__ out, int Hq, Paged pg, float scale_log2) {
  const int idx = blockIdx.x * kSplitWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (idx < nitems)
    split_kv_fp8_wave<D, NC>(idx, items, cols, q, kpool, vpool, kscale, vscale, bt, bt_stride, ws_ml, ws_acc, out,
                             Hq, pg, scale_log2);
}

hipError_t launch_split_kv_fp8(int D, int nitems, int nwide, hipStream_t s, const SplitItem* items, const Column* cols,
                               const void* q, const void* kpool, const void* vpool, const float* kscale,
                               const float* vscale, const int32_t* bt, int bt_stride, float* ws_ml, float* ws_acc,
                               void* out, int Hq, Paged pg, float scale_log2) {
  const dim3 block(64 * kSplitWaves);
  auto* qq = static_cast<const bf16*>(q);
  auto* kk = static_cast<const uint8_t*>(kpool);
  auto* vv = static_cast<const uint8_t*>(vpool);
  auto* oo = static_cast<bf16*>(out);
  // items of more than 16 columns come first and run on the two-block kernel
  auto launch = [&](auto dim, auto ncb, const SplitItem* it, int n) {
    constexpr int DD = decltype(dim)::value, NC = decltype(ncb)::value;
    if (n)
      split_kv_fp8_kernel<DD, NC><<<dim3((n + kSplitWaves - 1) / kSplitWaves), block, 0, s>>>(
          it, n, cols, qq, kk, vv, kscale, vscale, bt, bt_stride, ws_ml, ws_acc, oo, Hq, pg, scale_log2);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (D == 128) {
    launch(std::integral_constant<int, 128>{}, I2{}, items, nwide);
    launch(std::integral_constant<int, 128>{}, I1{}, items + nwide, nitems - nwide);
  } else {
    launch(std::integral_constant<int, 64>{}, I2{}, items, nwide);
    launch(std::integral_constant<int, 64>{}, I1{}, items + nwide, nitems - nwide);
  }
  return hipGetLastError();
}

// Thread t widens codes 8t .. 8t+7 with the same converter the attention kernel uses.
__global__ __launch_bounds__(256) void fp8_to_bf16_kernel(const uint32_t* __restrict__ codes, int64_t groups,
                                                          bf16x8* __restrict__ out) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < groups) out[t] = fp8x8_to_bf16(codes[2 * t], codes[2 * t + 1]);
}

// ---------------------------------------------------------------- fp8 append --
// Storing new rows: per (token, KV head) vector, scale = max|x| / 448 in float32 (IEEE
// division; 1 for an all-zero vector), code = x / scale (IEEE division) rounded to the
// nearest e4m3fn value with ties to the even code by the hardware converter (checked bit
// for bit against the format's definition on every finite bf16 magnitude under sixteen
// row maxima, and on every midpoint between adjacent codes).

constexpr int kAppendFp8Tok = 16;

// One workgroup per (KV head, up to 16 consecutive tokens: more workgroups in flight, 36 us
// against 44 us with 64 for the ORCA iteration's 4098 rows).  Each wave quantises four rows
// at a time: lane group grp = lane / 16 takes token tt = 4*wave + 16*i + grp, lane
// s = lane % 16 its elements EPS*s .. +EPS-1 (one 16- or 8-byte load); the maximum is
// reduced over the 16 lanes of the group.  All of a wave's loads are issued before any
// row is quantised; threads 0..63 meanwhile turn each token's out_cache_loc into the offsets
// of its K code row, its scales and its V code column (page_size is a power of two).  K
// codes and both scales are written directly, V codes go through LDS and are written into
// the transposed V pages 16 tokens at a time -- one 16-byte store per d row -- where those
// tokens fill 16 consecutive slots of one page from a multiple of 16, else one byte per
// token.
template <int D>
__global__ __launch_bounds__(256) void append_kv_fp8_kernel(
    const bf16* __restrict__ k_new, const bf16* __restrict__ v_new, const int64_t* __restrict__ loc, int64_t ntok,
    int tpw_log2, int Hkv, int ps_shift, int64_t nslots, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale, int32_t* __restrict__ bad) {
  constexpr int EPS = D / 16;                    // elements per lane of a row group
  constexpr int IT = kAppendFp8Tok / 16;         // row groups per wave
  constexpr int VROW = D + 4;                    // padded code row: token-strided reads spread over banks
  typedef __bf16 row_t __attribute__((ext_vector_type(EPS)));
  constexpr int G = 16;                          // tokens per 16-byte V code store
  __shared__ __attribute__((aligned(16))) uint8_t vcode[kAppendFp8Tok * VROW];
  __shared__ int64_t srow_of[kAppendFp8Tok];     // (page * Hkv + kvh) * page_size + slot (-1: none)
  __shared__ int64_t vdst[kAppendFp8Tok];        // byte offset of V[page][kvh][0][slot] (-1: none)
  __shared__ int32_t vrun[kAppendFp8Tok / G];
  const int kvh = blockIdx.y;
  const int tpw = 1 << tpw_log2;
  const int64_t t0 = int64_t(blockIdx.x) << tpw_log2;
  const int n = int(min<int64_t>(tpw, ntok - t0));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, sub = lane & 15;
  row_t kx[IT], vx[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    if (4 * wave + 16 * i >= n) break;              // wave-uniform
    const int tt = min(4 * wave + 16 * i + grp, n - 1);   // rows past n: loaded, not stored
    const size_t src = size_t((t0 + tt) * Hkv + kvh) * D + EPS * sub;
    kx[i] = *reinterpret_cast<const row_t*>(k_new + src);
    vx[i] = *reinterpret_cast<const row_t*>(v_new + src);
  }
  if (tid < kAppendFp8Tok) {
    int64_t l = tid < n ? loc[t0 + tid] : -1;
    if (l >= nslots) {
      if (bad && kvh == 0) atomicAdd(bad, 1);
      l = -1;
    }
    const int64_t ph = (l >> ps_shift) * Hkv + kvh;
    const int64_t slot = l & ((int64_t(1) << ps_shift) - 1);
    srow_of[tid] = l < 0 ? -1 : (ph << ps_shift) + slot;
    vdst[tid] = l < 0 ? -1 : ((ph * D) << ps_shift) + slot;
  }
  __syncthreads();
  if (tid < kAppendFp8Tok / G) {
    const int t = tid * G;
    bool run = t + G <= n;
    const int64_t v0 = run ? vdst[t] : -1;
    run = run && v0 >= 0 && (v0 & (G - 1)) == 0;
    for (int i = 1; i < G && run; ++i) run = vdst[t + i] == v0 + i;
    vrun[tid] = run;
  }
  auto quant = [&](const row_t& row, uint32_t (&c)[EPS]) -> float {
    float x[EPS], amax = 0.f;
#pragma unroll
    for (int e = 0; e < EPS; ++e) {
      x[e] = float(row[e]);
      amax = fmaxf(amax, fabsf(x[e]));
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    // v_cvt_pk_fp8_f32: two quotients to e4m3fn codes, nearest even (|x / scale| <= 448 up to
    // the division's rounding, which still rounds to 448)
#pragma unroll
    for (int e = 0; e < EPS; e += 2) {
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[e] / scale, x[e + 1] / scale, 0, false);
      c[e] = uint32_t(pk) & 0xffu;
      c[e + 1] = (uint32_t(pk) >> 8) & 0xffu;
    }
    return scale;
  };
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int tt = 4 * wave + 16 * i + grp;
    if (4 * wave + 16 * i >= n) break;            // wave-uniform: no row of this group exists
    uint32_t kc[EPS], vc[EPS];
    const float ks = quant(kx[i], kc);
    const float vs = quant(vx[i], vc);
    if (tt >= n) continue;
#pragma unroll
    for (int e = 0; e < EPS; ++e) vcode[tt * VROW + EPS * sub + e] = uint8_t(vc[e]);
    const int64_t sr = srow_of[tt];
    if (sr < 0) continue;
    const size_t srow = size_t(sr);
    uint32_t w[EPS / 4];
#pragma unroll
    for (int j = 0; j < EPS / 4; ++j)
      w[j] = kc[4 * j] | (kc[4 * j + 1] << 8) | (kc[4 * j + 2] << 16) | (kc[4 * j + 3] << 24);
    uint8_t* kd = k_pool + srow * D + EPS * sub;
    if constexpr (EPS == 8)
      *reinterpret_cast<uint2*>(kd) = uint2{w[0], w[1]};
    else
      *reinterpret_cast<uint32_t*>(kd) = w[0];
    if (sub == 0) {
      k_scale[srow] = ks;
      v_scale[srow] = vs;
    }
  }
  __syncthreads();
  const int ng = (n + G - 1) / G;
  for (int task = tid; task < ng * D; task += blockDim.x) {
    const int gi = task % ng, d = task / ng, t = gi * G;
    if (vrun[gi]) {
      union {
        uint8_t b[G];
        uint4 v;
      } pk;
#pragma unroll
      for (int i = 0; i < G; ++i) pk.b[i] = vcode[(t + i) * VROW + d];
      *reinterpret_cast<uint4*>(v_pool + vdst[t] + (int64_t(d) << ps_shift)) = pk.v;
    } else {
      for (int i = 0; i < G && t + i < n; ++i) {
        const int64_t vd = vdst[t + i];
        if (vd >= 0) v_pool[vd + (int64_t(d) << ps_shift)] = vcode[(t + i) * VROW + d];
      }
    }
  }
}

}  // namespace va

using namespace va;

extern "C" va_status varlen_attn_append_kv_fp8(const va_params* params, int64_t num_tokens, const void* k_new,
                                               const void* v_new, const int64_t* out_cache_loc, void* k_pool,
                                               void* v_pool, float* k_scale, float* v_scale,
                                               int32_t* bad_loc_count, void* stream) {
  if (!params) return fail(VA_ERR_INVALID_ARG, "params is NULL");
  const va_params& p = *params;
  if (num_tokens < 0) return fail(VA_ERR_INVALID_ARG, "num_tokens < 0");
  if (p.num_kv_heads < 1 || p.num_pages < 1) return fail(VA_ERR_INVALID_ARG, "num_kv_heads and num_pages must be >= 1");
  if (p.dtype != VA_DTYPE_FP8_E4M3)
    return fail(VA_ERR_INVALID_ARG, "varlen_attn_append_kv_fp8 needs dtype VA_DTYPE_FP8_E4M3");
  if (p.head_dim != 64 && p.head_dim != 128) return fail(VA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int ps = p.page_size;
  if (ps != 16 && ps != 32 && ps != 64 && ps != 128 && ps != 256)
    return fail(VA_ERR_UNSUPPORTED, "page_size must be 16, 32, 64, 128 or 256");
  if (num_tokens == 0) return VA_OK;
  if (!k_new || !v_new || !out_cache_loc || !k_pool || !v_pool || !k_scale || !v_scale)
    return fail(VA_ERR_INVALID_ARG, "k_new, v_new, out_cache_loc, the pools and the scale pools must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_pool) |
       reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(VA_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must be 16-byte aligned");
  const int Hkv = p.num_kv_heads;
  const int64_t nslots = int64_t(p.num_pages) * ps;
  int ps_shift = 0;
  while ((1 << ps_shift) < ps) ++ps_shift;
  int tpw_log2 = 4;
  while (tpw_log2 > 0 && ((num_tokens * Hkv) >> tpw_log2) < 1024) --tpw_log2;
  const int tpw = 1 << tpw_log2;
  const dim3 block(256), grid(unsigned((num_tokens + tpw - 1) / tpw), unsigned(Hkv));
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* kn = static_cast<const bf16*>(k_new);
  auto* vn = static_cast<const bf16*>(v_new);
  auto* kp = static_cast<uint8_t*>(k_pool);
  auto* vp = static_cast<uint8_t*>(v_pool);
  (void)hipGetLastError();
  if (p.head_dim == 128)
    append_kv_fp8_kernel<128><<<grid, block, 0, s>>>(kn, vn, out_cache_loc, num_tokens, tpw_log2, Hkv, ps_shift, nslots, kp, vp,
                                                      k_scale, v_scale, bad_loc_count);
  else
    append_kv_fp8_kernel<64><<<grid, block, 0, s>>>(kn, vn, out_cache_loc, num_tokens, tpw_log2, Hkv, ps_shift, nslots, kp, vp,
                                                     k_scale, v_scale, bad_loc_count);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VA_ERR_HIP, std::string("fp8 append kernel launch: ") + hipGetErrorString(e));
  return VA_OK;
}

extern "C" va_status varlen_attn_debug_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, void* stream) {
  if (n < 0 || n % 8 != 0) return fail(VA_ERR_INVALID_ARG, "n must be a non-negative multiple of 8");
  if (n == 0) return VA_OK;
  if (!codes || !out) return fail(VA_ERR_INVALID_ARG, "codes and out must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(codes) & 7) || (reinterpret_cast<uintptr_t>(out) & 15))
    return fail(VA_ERR_INVALID_ARG, "codes must be 8-byte and out 16-byte aligned");
  const int64_t groups = n / 8;
  (void)hipGetLastError();
  fp8_to_bf16_kernel<<<dim3(unsigned((groups + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const uint32_t*>(codes), groups, reinterpret_cast<bf16x8*>(out));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VA_ERR_HIP, std::string("fp8 conversion kernel launch: ") + hipGetErrorString(e));
  return VA_OK;
}
