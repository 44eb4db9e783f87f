// Appending one iteration's new K/V to the paged pools: a bit-exact scatter through the
// slot mapping (out_cache_loc = page * page_size + slot for every new token).
//
// K pages are [page][kv_head][slot][d]: each thread copies one 16-byte chunk of one
// token's K row (consecutive threads -> consecutive chunks of a row).  V pages are stored
// transposed, [page][kv_head][d][slot]: each thread copies one element, with the token
// index fastest, so the tokens of a prefill chunk that fill consecutive slots of a page
// write consecutive addresses.
#include <hip/hip_runtime.h>

#include <string>

#include "va_internal.h"

namespace va {

template <typename T>
__global__ __launch_bounds__(256) void append_k_kernel(const T* __restrict__ k_new, const int64_t* __restrict__ loc,
                                                       int64_t ntok, int Hkv, int D, int ps, int64_t nslots,
                                                       T* __restrict__ k_pool, int32_t* __restrict__ bad) {
  constexpr int E = 16 / sizeof(T);                 // elements per 16-byte chunk
  const int chunks = D / E;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= ntok * Hkv * chunks) return;
  const int ch = int(i % chunks);
  const int kvh = int((i / chunks) % Hkv);
  const int64_t t = i / (int64_t(chunks) * Hkv);
  const int64_t l = loc[t];
  if (l < 0) return;
  if (l >= nslots) {
    if (bad && ch == 0 && kvh == 0) atomicAdd(bad, 1);
    return;
  }
  const int64_t page = l / ps, slot = l % ps;
  const int4* src = reinterpret_cast<const int4*>(k_new + (t * Hkv + kvh) * D) + ch;
  int4* dst = reinterpret_cast<int4*>(k_pool + ((page * Hkv + kvh) * ps + slot) * D) + ch;
  *dst = *src;
}

template <typename T>
__global__ __launch_bounds__(256) void append_v_kernel(const T* __restrict__ v_new, const int64_t* __restrict__ loc,
                                                       int64_t ntok, int Hkv, int D, int ps, int64_t nslots,
                                                       T* __restrict__ v_pool) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= ntok * Hkv * D) return;
  const int64_t t = i % ntok;
  const int d = int((i / ntok) % D);
  const int kvh = int(i / (ntok * D));
  const int64_t l = loc[t];
  if (l < 0 || l >= nslots) return;
  const int64_t page = l / ps, slot = l % ps;
  v_pool[((page * Hkv + kvh) * D + d) * ps + slot] = v_new[(t * Hkv + kvh) * D + d];
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
  if (p.dtype != VA_DTYPE_BF16 && p.dtype != VA_DTYPE_F32) return fail(VA_ERR_INVALID_ARG, "unknown dtype");
  if (num_tokens == 0) return VA_OK;
  if (!k_new || !v_new || !out_cache_loc || !k_pool || !v_pool)
    return fail(VA_ERR_INVALID_ARG, "k_new, v_new, out_cache_loc, k_pool and v_pool must be non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int Hkv = p.num_kv_heads, D = p.head_dim;
  const int64_t nslots = int64_t(p.num_pages) * ps;
  const bool bf = p.dtype == VA_DTYPE_BF16;
  const int64_t nk = num_tokens * Hkv * (D * (bf ? 2 : 4) / 16), nv = num_tokens * Hkv * D;
  const dim3 block(256), gk(unsigned((nk + 255) / 256)), gv(unsigned((nv + 255) / 256));
  (void)hipGetLastError();
  if (bf) {
    append_k_kernel<uint16_t><<<gk, block, 0, s>>>(static_cast<const uint16_t*>(k_new), out_cache_loc, num_tokens, Hkv, D,
                                                   ps, nslots, static_cast<uint16_t*>(k_pool), bad_loc_count);
    append_v_kernel<uint16_t><<<gv, block, 0, s>>>(static_cast<const uint16_t*>(v_new), out_cache_loc, num_tokens, Hkv, D,
                                                   ps, nslots, static_cast<uint16_t*>(v_pool));
  } else {
    append_k_kernel<uint32_t><<<gk, block, 0, s>>>(static_cast<const uint32_t*>(k_new), out_cache_loc, num_tokens, Hkv, D,
                                                   ps, nslots, static_cast<uint32_t*>(k_pool), bad_loc_count);
    append_v_kernel<uint32_t><<<gv, block, 0, s>>>(static_cast<const uint32_t*>(v_new), out_cache_loc, num_tokens, Hkv, D,
                                                   ps, nslots, static_cast<uint32_t*>(v_pool));
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VA_ERR_HIP, std::string("append kernel launch: ") + hipGetErrorString(e));
  return VA_OK;
}
