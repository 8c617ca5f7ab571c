// K/V cache materialisation for the base stream.
//
// Pages: "Orthros: Phase-Aware Heterogeneous Attention for Efficient
// Transformers", paper text §3.1 (keys and values of every base position
// form the layer-wise cache); reproduction note "Orthros：阶段异构注意力",
// background section (the output stream never writes K/V; the full cache
// grows with decoding).
//
// A pure copy: new rows [B, n, Hkv, D] -> cache [B, Hkv, cap, D] starting at
// row cache_len[b]. HBM-bound; each thread moves 16 bytes, reads and writes
// are coalesced along D. cache_len is advanced by a second, tiny kernel so
// that no copy thread can observe a half-updated length.
#include "common.h"

namespace orthros {

// Sticky capacity-fault flag, one per device (each device has its own copy
// of this variable); kernels receive its device address as an argument.
__device__ int g_device_flag;

hipError_t device_flag_ptr(int **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static int *cached[64] = {nullptr};
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!cached[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_flag));
    if (e != hipSuccess) return e;
    cached[dev] = static_cast<int *>(p);
  }
  *out = cached[dev];
  return hipSuccess;
}

// One thread per 16-byte chunk of a new row.
__global__ __launch_bounds__(256) void kv_append_kernel(
    uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache,
    const int32_t *__restrict__ cache_len, const uint4 *__restrict__ k_new,
    const uint4 *__restrict__ v_new, int B, int n, int Hkv, int chunks,
    int64_t cap, int64_t cap_stride, int *flag) {
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)B * n * Hkv * chunks;
  if (id >= total) return;
  int c = (int)(id % chunks);
  int64_t rest = id / chunks;
  int g = (int)(rest % Hkv);
  rest /= Hkv;
  int i = (int)(rest % n);
  int b = (int)(rest / n);
  int64_t len = cache_len[b];
  if (len < 0 || len + n > cap) {
    if (id == (((int64_t)b * n) * Hkv) * chunks) atomicOr(flag, 1);
    return;
  }
  int64_t src = id;  // [B, n, Hkv, chunks] is exactly the thread order
  int64_t dst = (((int64_t)b * Hkv + g) * cap_stride + len + i) * chunks + c;
  k_cache[dst] = k_new[src];
  v_cache[dst] = v_new[src];
}

// Same copy for rows whose byte size is not a multiple of 16 (4-byte units).
__global__ __launch_bounds__(256) void kv_append_kernel_u32(
    uint32_t *__restrict__ k_cache, uint32_t *__restrict__ v_cache,
    const int32_t *__restrict__ cache_len, const uint32_t *__restrict__ k_new,
    const uint32_t *__restrict__ v_new, int B, int n, int Hkv, int words,
    int64_t cap, int64_t cap_stride, int *flag) {
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)B * n * Hkv * words;
  if (id >= total) return;
  int c = (int)(id % words);
  int64_t rest = id / words;
  int g = (int)(rest % Hkv);
  rest /= Hkv;
  int i = (int)(rest % n);
  int b = (int)(rest / n);
  int64_t len = cache_len[b];
  if (len < 0 || len + n > cap) {
    if (id == (((int64_t)b * n) * Hkv) * words) atomicOr(flag, 1);
    return;
  }
  int64_t dst = (((int64_t)b * Hkv + g) * cap_stride + len + i) * words + c;
  k_cache[dst] = k_new[id];
  v_cache[dst] = v_new[id];
}

// Paged cache: one thread per 16-byte (or 4-byte) unit of a new row; the
// destination page comes from the block table. Rows whose block-table entry
// lies outside [0, n_pages), or all rows of a batch entry whose new length
// would need more than max_pages pages, are skipped and raise the flag (the
// length bump then leaves that entry's length unchanged).
template <typename U>
__global__ __launch_bounds__(256) void kv_append_paged_kernel(
    U *__restrict__ k_pool, U *__restrict__ v_pool,
    const int32_t *__restrict__ cache_len, const U *__restrict__ k_new,
    const U *__restrict__ v_new, int B, int n, int Hkv, int units,
    int64_t n_pages, int page_log2, const int32_t *__restrict__ block_table,
    int max_pages, int *flag) {
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)B * n * Hkv * units;
  if (id >= total) return;
  int c = (int)(id % units);
  int64_t rest = id / units;
  int g = (int)(rest % Hkv);
  rest /= Hkv;
  int i = (int)(rest % n);
  int b = (int)(rest / n);
  const int64_t len = cache_len[b];
  const int64_t page_size = (int64_t)1 << page_log2;
  if (len < 0 || len + n > (int64_t)max_pages * page_size) {
    if (id == (((int64_t)b * n) * Hkv) * units) atomicOr(flag, 1);
    return;
  }
  const int64_t pos = len + i;
  const int64_t page = block_table[(int64_t)b * max_pages + (pos >> page_log2)];
  if (page < 0 || page >= n_pages) {
    if (c == 0 && g == 0) atomicOr(flag, 1);
    return;
  }
  const int64_t row = pos & (page_size - 1);
  const int64_t dst = ((page * Hkv + g) * page_size + row) * units + c;
  k_pool[dst] = k_new[id];
  v_pool[dst] = v_new[id];
}

__global__ void len_bump_paged_kernel(int32_t *cache_len, int B, int n,
                                      int64_t cap, const int32_t *block_table,
                                      int max_pages, int page_log2,
                                      int64_t n_pages) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int64_t len = cache_len[b];
  bool ok = len >= 0 && len + n <= cap;
  if (ok) {
    const int64_t p0 = len >> page_log2, p1 = (len + n - 1) >> page_log2;
    for (int64_t p = p0; p <= p1 && ok; ++p) {
      const int32_t e = block_table[(int64_t)b * max_pages + p];
      ok = e >= 0 && e < n_pages;
    }
  }
  if (ok) cache_len[b] = (int32_t)(len + n);
}

__global__ void len_bump_kernel(int32_t *cache_len, int B, int n,
                                int64_t cap) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int64_t len = cache_len[b];
  if (len >= 0 && len + n <= cap) cache_len[b] = (int32_t)(len + n);
}

hipError_t launch_len_bump(int32_t *cache_len, int B, int n, int64_t cap,
                           hipStream_t stream) {
  hipLaunchKernelGGL(len_bump_kernel, dim3((B + 255) / 256), dim3(256), 0,
                     stream, cache_len, B, n, cap);
  return hipGetLastError();
}

hipError_t launch_kv_append(void *k_cache, void *v_cache, int32_t *cache_len,
                            const void *k_new, const void *v_new, int B,
                            int n_new, int Hkv, int row_bytes, int64_t cap,
                            int64_t cap_stride, int *flag, int bump,
                            hipStream_t stream) {
  const bool vec = (row_bytes % 16 == 0) &&
                   ((uintptr_t)k_cache % 16 == 0) &&
                   ((uintptr_t)v_cache % 16 == 0) &&
                   ((uintptr_t)k_new % 16 == 0) && ((uintptr_t)v_new % 16 == 0);
  if (vec) {
    int chunks = row_bytes / 16;
    int64_t total = (int64_t)B * n_new * Hkv * chunks;
    int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       stream, (uint4 *)k_cache, (uint4 *)v_cache, cache_len,
                       (const uint4 *)k_new, (const uint4 *)v_new, B, n_new,
                       Hkv, chunks, cap, cap_stride, flag);
  } else {
    int words = row_bytes / 4;
    int64_t total = (int64_t)B * n_new * Hkv * words;
    int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(kv_append_kernel_u32, dim3((unsigned)blocks), dim3(256),
                       0, stream, (uint32_t *)k_cache, (uint32_t *)v_cache,
                       cache_len, (const uint32_t *)k_new,
                       (const uint32_t *)v_new, B, n_new, Hkv, words, cap,
                       cap_stride, flag);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !bump) return e;
  return launch_len_bump(cache_len, B, n_new, cap, stream);
}

hipError_t launch_kv_append_paged(void *k_pool, void *v_pool,
                                  int32_t *cache_len, const void *k_new,
                                  const void *v_new, int B, int n_new,
                                  int Hkv, int row_bytes, int64_t n_pages,
                                  int page_log2, const int32_t *block_table,
                                  int max_pages, int *flag,
                                  hipStream_t stream) {
  const bool vec = (row_bytes % 16 == 0) && ((uintptr_t)k_pool % 16 == 0) &&
                   ((uintptr_t)v_pool % 16 == 0) &&
                   ((uintptr_t)k_new % 16 == 0) && ((uintptr_t)v_new % 16 == 0);
  const int units = vec ? row_bytes / 16 : row_bytes / 4;
  const int64_t total = (int64_t)B * n_new * Hkv * units;
  const int64_t blocks = (total + 255) / 256;
  if (vec)
    hipLaunchKernelGGL(kv_append_paged_kernel<uint4>, dim3((unsigned)blocks),
                       dim3(256), 0, stream, (uint4 *)k_pool, (uint4 *)v_pool,
                       cache_len, (const uint4 *)k_new, (const uint4 *)v_new,
                       B, n_new, Hkv, units, n_pages, page_log2, block_table,
                       max_pages, flag);
  else
    hipLaunchKernelGGL(kv_append_paged_kernel<uint32_t>,
                       dim3((unsigned)blocks), dim3(256), 0, stream,
                       (uint32_t *)k_pool, (uint32_t *)v_pool, cache_len,
                       (const uint32_t *)k_new, (const uint32_t *)v_new, B,
                       n_new, Hkv, units, n_pages, page_log2, block_table,
                       max_pages, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(len_bump_paged_kernel, dim3((B + 255) / 256), dim3(256),
                     0, stream, cache_len, B, n_new,
                     (int64_t)max_pages << page_log2, block_table, max_pages,
                     page_log2, n_pages);
  return hipGetLastError();
}

}  // namespace orthros
