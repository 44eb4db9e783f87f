// Device-side pieces shared by the attention kernels (kernels.hip, kv_fp8.hip): vector
// types, page addressing, MFMA wrappers and the partial / output stores of a split-KV
// column.
#pragma once
#include <hip/hip_runtime.h>

#include "va_internal.h"

namespace va {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight fp8 e4m3fn codes (bytes 0..3 of w0, then of w1, low byte first) -> bf16x8 with
// the hardware converter at scale 1 (exact: every e4m3fn value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1e30f;   // running-max start: finite, so fully masked steps keep alpha = 1

// ---------------------------------------------------------------- page addressing --
// Pools: K [page][kv_head][slot][d], V [page][kv_head][d][slot] (transposed page).
// Logical position j of a request is slot j % page_size of page block_table[j / page_size].
struct Paged {
  int Hkv, ps_shift, D;
  __device__ __forceinline__ int ps() const { return 1 << ps_shift; }
  __device__ __forceinline__ int page_of(const int32_t* bt_row, int pos) const { return bt_row[pos >> ps_shift]; }
  __device__ __forceinline__ int slot_of(int pos) const { return pos & ((1 << ps_shift) - 1); }
  // element offset of K[page, kvh, slot, 0]
  __device__ __forceinline__ size_t k_row(int page, int kvh, int slot) const {
    return ((size_t(page) * Hkv + kvh) * (size_t(1) << ps_shift) + slot) * D;
  }
  // element offset of V[page, kvh, d, slot]
  __device__ __forceinline__ size_t v_elem(int page, int kvh, int d, int slot) const {
    return ((size_t(page) * Hkv + kvh) * D + d) * (size_t(1) << ps_shift) + slot;
  }
  // offset of the per-position scale of (page, kvh, slot) in a [page][kv_head][slot] pool
  __device__ __forceinline__ size_t scale_idx(int page, int kvh, int slot) const {
    return (size_t(page) * Hkv + kvh) * (size_t(1) << ps_shift) + slot;
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Write one column's partial result as (m, 1/l) and acc/l (1/l = 0 when no key was
// scored), so every partial has the same form as a finished row.  acc[db][r] holds
// d = 16*db + 4*grp + r.
template <int D>
__device__ __forceinline__ void store_partial(float* ws_ml, float* ws_acc, int slot, int grp, float m, float l,
                                              const f32x4* acc) {
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (grp == 0) *reinterpret_cast<float2*>(ws_ml + 2 * size_t(slot)) = float2{m, inv};
  float* wa = ws_acc + size_t(slot) * D + 4 * grp;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = acc[db][r] * inv;
    *reinterpret_cast<f32x4*>(wa + 16 * db) = o;
  }
}

// Write one column's finished output row (an item that covers the column's whole kv
// range): acc / l, rounded to the output type.
template <int D, typename OutT>
__device__ __forceinline__ void store_output(OutT* out, size_t row_off, int grp, float l, const f32x4* acc) {
  const float inv = 1.f / l;
  OutT* op = out + row_off + 4 * grp;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) op[16 * db + r] = OutT(acc[db][r] * inv);
}

// Split-KV kernels over fp8 e4m3fn K/V pools with per-position float32 scales
// (kv_fp8.hip); bf16 Q and output.  The first nwide items have more than 16 columns.
// Returns the launch status.
hipError_t launch_split_kv_fp8(int D, int nitems, int nwide, hipStream_t s, const SplitItem* items, const Column* cols,
                               const void* q, const void* kpool, const void* vpool, const float* kscale,
                               const float* vscale, const int32_t* bt, int bt_stride, float* ws_ml, float* ws_acc,
                               void* out, int Hq, Paged pg, float scale_log2);

}  // namespace va
