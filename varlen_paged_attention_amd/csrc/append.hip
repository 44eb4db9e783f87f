// Appending one iteration's new K/V to the paged pools: a bit-exact scatter through the
// slot mapping (out_cache_loc = page * page_size + slot for every new token).
//
// K pages are [page][kv_head][slot][d], V pages transposed [page][kv_head][d][slot].
#include <hip/hip_runtime.h>

#include <string>
#include <type_traits>

#include "va_internal.h"

namespace va {

// One workgroup per (KV head, tpw <= 64 consecutive tokens; fewer when there are few tokens,
// so the launch still has about a thousand workgroups).  K rows are copied with 16-byte
// loads and stores (consecutive threads -> consecutive chunks of a row).  V rows are read
// the same way into LDS, then written element by element with the token index fastest
// across lanes, so the writes of tokens that fill consecutive slots of a page land on
// consecutive addresses.
constexpr int kAppendTok = 64;

template <typename T, int D>
__global__ __launch_bounds__(256) void append_kv_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                        const int64_t* __restrict__ loc, int64_t ntok, int tpw_log2, int Hkv,
                                                        int ps, int64_t nslots, T* __restrict__ k_pool,
                                                        T* __restrict__ v_pool, int32_t* __restrict__ bad) {
  constexpr int E = 16 / sizeof(T);                 // elements per 16-byte chunk
  constexpr int CH = D / E;                         // chunks per row
  constexpr int ROW = D + E;                        // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) T tile[kAppendTok * ROW];
  __shared__ int64_t tloc[kAppendTok];
  const int kvh = blockIdx.y;
  const int tpw = 1 << tpw_log2;
  const int64_t t0 = int64_t(blockIdx.x) << tpw_log2;
  const int n = int(min<int64_t>(tpw, ntok - t0));
  const int tid = threadIdx.x;
  if (tid < kAppendTok) {
    int64_t l = tid < n ? loc[t0 + tid] : -1;
    if (l >= nslots) {
      if (bad && kvh == 0) atomicAdd(bad, 1);
      l = -1;
    }
    tloc[tid] = l;
  }
  for (int c = tid; c < n * CH; c += blockDim.x) {
    const int tt = c / CH, ch = c % CH;
    const size_t src = size_t((t0 + tt) * Hkv + kvh) * D + ch * E;
    *reinterpret_cast<int4*>(tile + tt * ROW + ch * E) = *reinterpret_cast<const int4*>(v_new + src);
  }
  __syncthreads();
  for (int c = tid; c < n * CH; c += blockDim.x) {
    const int tt = c / CH, ch = c % CH;
    const int64_t l = tloc[tt];
    if (l < 0) continue;
    const int64_t page = l / ps, slot = l % ps;
    *reinterpret_cast<int4*>(k_pool + ((page * Hkv + kvh) * ps + slot) * D + ch * E) =
        *reinterpret_cast<const int4*>(k_new + size_t((t0 + tt) * Hkv + kvh) * D + ch * E);
  }
  for (int e = tid; e < tpw * D; e += blockDim.x) {
    const int tt = e & (tpw - 1), d = e >> tpw_log2;
    if (tt >= n) continue;
    const int64_t l = tloc[tt];
    if (l < 0) continue;
    const int64_t page = l / ps, slot = l % ps;
    v_pool[((page * Hkv + kvh) * D + d) * ps + slot] = tile[tt * ROW + d];
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Hkv = p.num_kv_heads, D = p.head_dim;
  const int64_t nslots = int64_t(p.num_pages) * ps;
  const bool bf = p.dtype == VA_DTYPE_BF16;
  int tpw_log2 = 6;                       // kAppendTok = 64 tokens
  while (tpw_log2 > 0 && ((num_tokens * Hkv) >> tpw_log2) < 1024) --tpw_log2;
  const int tpw = 1 << tpw_log2;
  const dim3 block(256), grid(unsigned((num_tokens + tpw - 1) / tpw), unsigned(Hkv));
  (void)hipGetLastError();
  auto launch = [&](auto elem, auto dim) {
    using T = decltype(elem);
    constexpr int DD = decltype(dim)::value;
    append_kv_kernel<T, DD><<<grid, block, 0, s>>>(static_cast<const T*>(k_new), static_cast<const T*>(v_new),
                                                   out_cache_loc, num_tokens, tpw_log2, Hkv, ps, nslots, static_cast<T*>(k_pool),
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
