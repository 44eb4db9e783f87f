// Appending one iteration's new K/V to the paged pools: a bit-exact scatter through the
// slot mapping (out_cache_loc = page * page_size + slot for every new token).
//
// K pages are [page][kv_head][slot][d], V pages transposed [page][kv_head][d][slot].
#include <hip/hip_runtime.h>

#include <string>
#include <type_traits>

#include "va_internal.h"

namespace va {

// One workgroup per (KV head, tpw <= 16 consecutive tokens; fewer when there are few tokens,
// so the launch still has about a thousand workgroups; 16 measured faster than 64 -- 36 vs
// 42 us for the ORCA iteration's 4098 rows -- as more workgroups keep more rows in flight).  Every thread first issues its K and
// V row loads (16-byte chunks, consecutive threads -> consecutive chunks of a row); threads
// 0..tpw-1 turn their token's out_cache_loc into the offsets of its K row and of its V
// column (page_size is a power of two: shifts and masks).  K rows are stored straight from
// registers.  V rows go through LDS and are written into the transposed pages E = 16 /
// sizeof(T) tokens at a time -- one 16-byte store per d row -- where those E tokens fill E
// consecutive slots of one page starting at a multiple of E (a prefill's tokens do), else
// one element per token.
constexpr int kAppendTok = 16;

template <typename T, int D>
__global__ __launch_bounds__(256) void append_kv_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                        const int64_t* __restrict__ loc, int64_t ntok, int tpw_log2,
                                                        int Hkv, int ps_shift, int64_t nslots, T* __restrict__ k_pool,
                                                        T* __restrict__ v_pool, int32_t* __restrict__ bad) {
  constexpr int E = 16 / sizeof(T);                 // elements per 16-byte chunk; tokens per V store
  constexpr int CH = D / E;                         // chunks per row
  constexpr int ROW = D + E;                        // padded LDS row (elements)
  constexpr int NCH = kAppendTok * CH;              // chunks of a full workgroup
  constexpr int NC = (NCH + 255) / 256;             // chunks per thread
  constexpr int NG = kAppendTok / E;                // token groups of a full workgroup
  __shared__ __attribute__((aligned(16))) T tile[kAppendTok * ROW];
  __shared__ int64_t kdst[kAppendTok];              // element offset of the token's K row (-1: none)
  __shared__ int64_t vdst[kAppendTok];              // element offset of V[page][kvh][0][slot] (-1: none)
  __shared__ int32_t vrun[NG];                      // group stored with one 16-byte store per d row
  const int kvh = blockIdx.y;
  const int tpw = 1 << tpw_log2;
  const int64_t t0 = int64_t(blockIdx.x) << tpw_log2;
  const int n = int(min<int64_t>(tpw, ntok - t0));
  const int tid = threadIdx.x;
  int4 kr[NC], vr[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + 256 * i, tt = c / CH, ch = c % CH;
    if (c < NCH && tt < n) {
      const size_t src = size_t((t0 + tt) * Hkv + kvh) * D + ch * E;
      kr[i] = *reinterpret_cast<const int4*>(k_new + src);
      vr[i] = *reinterpret_cast<const int4*>(v_new + src);
    }
  }
  if (tid < kAppendTok) {
    int64_t l = tid < n ? loc[t0 + tid] : -1;
    if (l >= nslots) {
      if (bad && kvh == 0) atomicAdd(bad, 1);
      l = -1;
    }
    const int64_t ph = (l >> ps_shift) * Hkv + kvh;               // page * Hkv + kvh
    const int64_t slot = l & ((int64_t(1) << ps_shift) - 1);
    kdst[tid] = l < 0 ? -1 : ((ph << ps_shift) + slot) * D;
    vdst[tid] = l < 0 ? -1 : ((ph * D) << ps_shift) + slot;
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + 256 * i, tt = c / CH, ch = c % CH;
    if (c < NCH && tt < n) *reinterpret_cast<int4*>(tile + tt * ROW + ch * E) = vr[i];
  }
  __syncthreads();
  if (tid < NG) {
    // E tokens in consecutive slots of one page from a multiple of E: the V column offsets
    // then run v0, v0+1, .. (pages are page_size >= E apart in every V row)
    const int t = tid * E;
    bool run = t + E <= n;
    const int64_t v0 = run ? vdst[t] : -1;
    run = run && v0 >= 0 && (v0 & (E - 1)) == 0;
    for (int i = 1; i < E && run; ++i) run = vdst[t + i] == v0 + i;
    vrun[tid] = run;
  }
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + 256 * i, tt = c / CH, ch = c % CH;
    if (c < NCH && tt < n) {
      const int64_t kd = kdst[tt];
      if (kd >= 0) *reinterpret_cast<int4*>(k_pool + kd + ch * E) = kr[i];
    }
  }
  __syncthreads();
  const int ng = (n + E - 1) / E;
  for (int task = tid; task < ng * D; task += blockDim.x) {
    const int gi = task % ng, d = task / ng, t = gi * E;
    if (vrun[gi]) {
      union {
        T e[E];
        int4 v;
      } pk;
#pragma unroll
      for (int i = 0; i < E; ++i) pk.e[i] = tile[(t + i) * ROW + d];
      *reinterpret_cast<int4*>(v_pool + vdst[t] + (int64_t(d) << ps_shift)) = pk.v;
    } else {
      for (int i = 0; i < E && t + i < n; ++i) {
        const int64_t vd = vdst[t + i];
        if (vd >= 0) v_pool[vd + (int64_t(d) << ps_shift)] = tile[(t + i) * ROW + d];
      }
    }
  }
}

}  // namespace va

using namespace va;

extern "C" va_status varlen_attn_append_kv(const va_params* params, int64_t num_tokens, const void* k_new,
                                           const void* v_new, const int64_t* out_cache_loc, void* k_pool,
                                           void* v_pool, int32_t* bad_loc_count, void* stream) {
  if (!params) return fail(VA_ERR_INVALID_ARG, "params is NULL");
  const va_params& p = *params;
  if (num_tokens < 0) return fail(VA_ERR_INVALID_ARG, "num_tokens < 0");
  if (p.num_kv_heads < 1 || p.num_pages < 1) return fail(VA_ERR_INVALID_ARG, "num_kv_heads and num_pages must be >= 1");
  if (p.head_dim != 64 && p.head_dim != 128) return fail(VA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int ps = p.page_size;
  if (ps != 16 && ps != 32 && ps != 64 && ps != 128 && ps != 256)
    return fail(VA_ERR_UNSUPPORTED, "page_size must be 16, 32, 64, 128 or 256");
  if (p.dtype == VA_DTYPE_FP8_E4M3)
    return fail(VA_ERR_INVALID_ARG, "fp8 pools are written with varlen_attn_append_kv_fp8 (codes and scales)");
  if (p.dtype != VA_DTYPE_BF16 && p.dtype != VA_DTYPE_F32) return fail(VA_ERR_INVALID_ARG, "unknown dtype");
  if (num_tokens == 0) return VA_OK;
  if (!k_new || !v_new || !out_cache_loc || !k_pool || !v_pool)
    return fail(VA_ERR_INVALID_ARG, "k_new, v_new, out_cache_loc, k_pool and v_pool must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_pool) |
       reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(VA_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Hkv = p.num_kv_heads, D = p.head_dim;
  const int64_t nslots = int64_t(p.num_pages) * ps;
  const bool bf = p.dtype == VA_DTYPE_BF16;
  int ps_shift = 0;
  while ((1 << ps_shift) < ps) ++ps_shift;
  int tpw_log2 = 4;                       // kAppendTok = 16 tokens
  while (tpw_log2 > 0 && ((num_tokens * Hkv) >> tpw_log2) < 1024) --tpw_log2;
  const int tpw = 1 << tpw_log2;
  const dim3 block(256), grid(unsigned((num_tokens + tpw - 1) / tpw), unsigned(Hkv));
  (void)hipGetLastError();
  auto launch = [&](auto elem, auto dim) {
    using T = decltype(elem);
    constexpr int DD = decltype(dim)::value;
    append_kv_kernel<T, DD><<<grid, block, 0, s>>>(static_cast<const T*>(k_new), static_cast<const T*>(v_new),
                                                   out_cache_loc, num_tokens, tpw_log2, Hkv, ps_shift, nslots, static_cast<T*>(k_pool),
                                                   static_cast<T*>(v_pool), bad_loc_count);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  if (bf) {
    if (D == 128) launch(uint16_t{}, D128{}); else launch(uint16_t{}, D64{});
  } else {
    if (D == 128) launch(uint32_t{}, D128{}); else launch(uint32_t{}, D64{});
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VA_ERR_HIP, std::string("append kernel launch: ") + hipGetErrorString(e));
  return VA_OK;
}
