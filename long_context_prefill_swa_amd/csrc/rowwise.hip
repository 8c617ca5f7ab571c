// Generic attention kernel: one wavefront per (query row, head, batch).
//
// Serves every case the MFMA kernels do not: fp32 inputs, head dimensions
// other than 128, and unaligned tensors. Same arithmetic as the pages'
// equations ("Orthros: Phase-Aware Heterogeneous Attention for Efficient
// Transformers", paper text §3.1: scale-offset on the query, softmax of
// q.k/sqrt(D) over [max(0,t-W+1), t] for the base stream and [0, t] for the
// output stream), evaluated as a streaming (online) softmax in fp32 over
// chunks of 64 keys: lane j scores key j of the chunk, the wave reduces the
// chunk maximum and sum, then every lane accumulates its own output channels.
#include "common.h"

namespace orthros {

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void st(T *p, int64_t i, float x);
template <>
__device__ __forceinline__ void st<float>(float *p, int64_t i, float x) {
  p[i] = x;
}
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t *p, int64_t i, float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  p[i] = __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename T>
__global__ __launch_bounds__(64) void rowwise_attn_kernel(
    const T *__restrict__ q, const float *__restrict__ alpha,
    const float *__restrict__ beta, const T *__restrict__ k_cache,
    const T *__restrict__ v_cache, T *__restrict__ o, int nrows, int Hq,
    int Hkv, int D, int64_t cap, int64_t t_limit, int64_t q_offset, int W,
    const int32_t *__restrict__ cache_len, HeadMap map) {
  __shared__ float q_s[256];
  __shared__ float p_s[64];
  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = map.kv_of_q[h];

  const int64_t t = (cache_len ? (int64_t)cache_len[b] : q_offset) + r;
  const int64_t orow = (((int64_t)b * nrows + r) * Hq + h) * D;
  if (t < 0 || t >= t_limit) {  // rejected length (flag already raised)
    for (int d = lane; d < D; d += 64) st<T>(o, orow + d, 0.0f);
    return;
  }
  const int64_t lo = (W > 0 && t - W + 1 > 0) ? t - W + 1 : 0;
  const int64_t hi = t;

  // Scale-offset affine on the query; 1/sqrt(D) folded in.
  const float scale = rsqrtf((float)D);
  for (int d = lane; d < D; d += 64)
    q_s[d] = (alpha[h * D + d] * ld<T>(q, orow + d) + beta[h * D + d]) * scale;
  __syncthreads();

  const T *kb = k_cache + ((int64_t)b * Hkv + g) * cap * D;
  const T *vb = v_cache + ((int64_t)b * Hkv + g) * cap * D;
  float m = -INFINITY, l = 0.0f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = lo; k0 <= hi; k0 += 64) {
    const int64_t j = k0 + lane;
    const bool valid = j <= hi;
    float s = -INFINITY;
    if (valid) {
      float dot = 0.0f;
      const T *kr = kb + j * D;
      for (int d = 0; d < D; ++d) dot += q_s[d] * ld<T>(kr, d);
      s = dot;
    }
    const float m_new = fmaxf(m, wave_max(s));  // finite: key hi >= k0 exists
    const float p = valid ? __expf(s - m_new) : 0.0f;
    const float corr = __expf(m - m_new);       // 0 on the first chunk
    l = l * corr + wave_sum(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= corr;
    p_s[lane] = p;
    __syncthreads();
    const int n = (int)((hi - k0 + 1) < 64 ? (hi - k0 + 1) : 64);
    for (int jj = 0; jj < n; ++jj) {
      const float pj = p_s[jj];
      const T *vr = vb + (k0 + jj) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) acc[i] += pj * ld<T>(vr, d);
      }
    }
    __syncthreads();
    m = m_new;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    if (d < D) st<T>(o, orow + d, acc[i] * inv);
  }
}

hipError_t launch_rowwise(const void *q, const float *alpha, const float *beta,
                          const void *k_cache, const void *v_cache, void *o,
                          int B, int nrows, int Hq, int Hkv, int D,
                          int64_t cap, int64_t t_limit, int64_t q_offset,
                          int W, const int32_t *cache_len, const HeadMap &map,
                          int is_bf16, hipStream_t stream) {
  dim3 grid(nrows, Hq, B);
  if (is_bf16) {
    hipLaunchKernelGGL(rowwise_attn_kernel<uint16_t>, grid, dim3(64), 0,
                       stream, (const uint16_t *)q, alpha, beta,
                       (const uint16_t *)k_cache, (const uint16_t *)v_cache,
                       (uint16_t *)o, nrows, Hq, Hkv, D, cap, t_limit, q_offset, W,
                       cache_len, map);
  } else {
    hipLaunchKernelGGL(rowwise_attn_kernel<float>, grid, dim3(64), 0, stream,
                       (const float *)q, alpha, beta, (const float *)k_cache,
                       (const float *)v_cache, (float *)o, nrows, Hq, Hkv, D,
                       cap, t_limit, q_offset, W, cache_len, map);
  }
  return hipGetLastError();
}

}  // namespace orthros
