// Probes for the benchmark's run record (not part of the attention library;
// built into its own small library, libclock_probe.so): the shader clock
// under MFMA load, and the HBM rate of plain streaming reads and copies.
//
// The MI355X's bf16 MFMA peak is quoted at 2.4 GHz, but under a sustained
// MFMA load the shader clock settles lower, and it varies from box to box.
// This kernel keeps every compute unit busy with independent MFMA chains
// (the load the sliding-window kernel puts on the chip) and reads two
// counters per workgroup at the start and the end of the chains: the shader
// cycle counter (clock64) and the constant-rate wall counter (wall_clock64,
// whose rate hipDeviceAttributeWallClockRate gives). Their ratio is the
// average shader clock under that load.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void clock_probe_kernel(uint64_t *out,
                                                          int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(lane + e));
    b[e] = (__bf16)(1e-3f * (float)(lane - e));
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  __syncthreads();
  const uint64_t c0 = clock64();
  const uint64_t w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  __syncthreads();
  const uint64_t c1 = clock64();
  const uint64_t w1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x + 0] = c1 - c0;
    out[3 * blockIdx.x + 1] = w1 - w0;
    // keeps the chains alive; the sum of tiny products is never this large
    out[3 * blockIdx.x + 2] = s > 1e30f ? 1u : 0u;
  }
}

// Streaming probes of the HBM rate this part reaches with plain loads and
// stores, the practical ceiling for the memory-bound kernels. Each
// workgroup (256 threads) walks its own contiguous region of `per_wg`
// bytes in iterations of 256 x NL x 16 bytes, with two iterations of loads
// in flight; buffer resources bound every access to the region.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;

template <int NL, bool COPY>
__global__ __launch_bounds__(256) void stream_probe_kernel(const char *src,
                                                           char *dst,
                                                           uint32_t per_wg,
                                                           u32x4 *sink) {
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * per_wg;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(src + base), 0, per_wg, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      COPY ? dst + base : const_cast<char *>(src + base), 0, COPY ? per_wg : 0,
      kBufferWord3);
  const uint32_t step = 256u * NL * 16u;
  const uint32_t n_it = per_wg / step;
  u32x4 acc = {0, 0, 0, 0};
  u32x4 cur[NL], nxt[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    cur[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (i * 256 + tid) * 16, 0, 0);
  for (uint32_t it = 0; it < n_it; ++it) {
    if (it + 1 < n_it) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        nxt[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rs, (it + 1) * step + (i * 256 + tid) * 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (COPY)
        __builtin_amdgcn_raw_buffer_store_b128(
            cur[i], rd, it * step + (i * 256 + tid) * 16, 0, 0);
      else
        acc ^= cur[i];
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) cur[i] = nxt[i];
  }
  if (!COPY) sink[(int64_t)blockIdx.x * 256 + tid] = acc;
}

}  // namespace

// Streaming read of `bytes` from src [dev] (n_blocks workgroups of 256
// threads, 8 x 16 bytes per thread per iteration); sink [dev] receives
// n_blocks x 256 x 16 bytes (keeps the loads alive). bytes must be a
// multiple of n_blocks x 32768. Returns a hipError_t value.
extern "C" int hbm_read_probe(const void *src, size_t bytes, int n_blocks,
                              void *sink, void *stream) {
  if (!src || !sink || n_blocks < 1 || bytes % ((size_t)n_blocks * 32768) ||
      bytes / n_blocks > 0xFFFFFFFFull)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL((stream_probe_kernel<8, false>), dim3(n_blocks), dim3(256),
                     0, reinterpret_cast<hipStream_t>(stream),
                     (const char *)src, (char *)nullptr,
                     (uint32_t)(bytes / n_blocks), (u32x4 *)sink);
  return (int)hipGetLastError();
}

// Copy of `bytes` from src to dst [dev] (n_blocks workgroups, 16 x 16 bytes
// per thread per iteration). bytes must be a multiple of n_blocks x 65536.
extern "C" int hbm_copy_probe(const void *src, void *dst, size_t bytes,
                              int n_blocks, void *stream) {
  if (!src || !dst || n_blocks < 1 || bytes % ((size_t)n_blocks * 65536) ||
      bytes / n_blocks > 0xFFFFFFFFull)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL((stream_probe_kernel<16, true>), dim3(n_blocks), dim3(256),
                     0, reinterpret_cast<hipStream_t>(stream),
                     (const char *)src, (char *)dst,
                     (uint32_t)(bytes / n_blocks), (u32x4 *)nullptr);
  return (int)hipGetLastError();
}

// Launches n_blocks workgroups of 256 threads, each running `iters` rounds of
// four independent MFMA chains; out [dev] receives 3 * n_blocks uint64
// values (shader cycles, wall ticks, 0) per workgroup. *wall_khz receives the
// wall counter's rate. Returns a hipError_t value (0 on success).
extern "C" int clock_probe(void *out, int n_blocks, int iters, int *wall_khz,
                           void *stream) {
  if (!out || n_blocks < 1 || iters < 1 || !wall_khz) return (int)hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(n_blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), (uint64_t *)out,
                     iters);
  return (int)hipGetLastError();
}
