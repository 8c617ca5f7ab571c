// Split-KV flash decode on gfx950 MFMA (bf16 in, fp32 accumulate), D = 128.
//
// Serves the two memory-bound parts of Orthros attention ("Orthros:
// Phase-Aware Heterogeneous Attention for Efficient Transformers"):
//  * the output stream's full cross-attention when only a few rows need it
//    (prefilling: one row at the last prompt position, paper text §3.2), and
//  * the decode pair step (paper text §3.1 and §3.2 Decoding): append the
//    base token's K/V, then the base query over its window and the output
//    query over the whole cache.
// Both stream every cache row once from HBM (§3.3: decoding is bound by
// memory I/O), so the design goal is coalesced, deep-in-flight reads with
// all query rows of a KV head sharing each read.
//
// Work split: grid (chunk, head group, batch). A workgroup (4 waves) owns
// `chunk` consecutive keys of one (batch, KV head) and every query row that
// reads that KV head (query heads of the group x streams x positions, at most
// 16). Each wave takes 32 keys per step:
//   S^T[key][row] = K Q^T        2 x 4 MFMA 16x16x32 (keys on M, rows on N)
//   online softmax per row       (one row per lane column; no cross-row work)
//   O^T[d][row] += V^T P^T        8 MFMA 16x16x32 (d on M, keys on K)
// K is read straight from global memory into MFMA operand registers; V rows
// are staged in LDS (a wave-private region) and gathered key-major for the
// transposed product. Waves then merge in LDS and the workgroup writes one
// (max, sum, unnormalised output) partial per row; a second kernel combines
// the partials of all chunks with log-sum-exp weights, normalises, writes
// the output rows and (decode) advances the cache length.
#include "common.h"

namespace orthros {
namespace {

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStep = 32;           // keys per wave step
constexpr int kMaxRows = 16;
constexpr int kVStride = D + 8;     // bf16 elements per staged V row (pad)

struct RowInfo {
  int64_t lo, hi;  // key range, lo > hi = inactive
};

__device__ __forceinline__ int64_t row_pos(const SplitKVArgs &a, int b,
                                           int j) {
  return (a.cache_len ? (int64_t)a.cache_len[b] : a.pos0) + j;
}

__device__ __forceinline__ int64_t ws_part_index(const SplitKVArgs &a,
                                                 int n_groups, int rows,
                                                 int b, int gi, int c,
                                                 int r) {
  return (((int64_t)b * n_groups + gi) * a.n_chunks + c) * rows + r;
}

__global__ __launch_bounds__(kThreads, 2) void splitkv_kernel(
    SplitKVArgs a, HeadGroups groups) {
  __shared__ __attribute__((aligned(16)))
      uint16_t v_s[kWaves][kStep][kVStride];        // 17 KB
  __shared__ float red_m[kWaves][kMaxRows];
  __shared__ float red_l[kWaves][kMaxRows];
  __shared__ float red_acc[kWaves][kMaxRows][D + 4];  // 33 KB

  const int c = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g4 = lane >> 4;
  const int gsize = groups.gsize;
  const int rows = a.n_streams * a.n_pos * gsize;
  const int kvh = groups.kv[gi];

  // ---- positions and validity (decode: lengths live on the device) -------
  int64_t n_old = 0;
  if (a.cache_len) {
    n_old = a.cache_len[b];
    const bool ok = n_old >= 0 && n_old + 1 <= a.max_len && n_old + 1 <= a.cap;
    if (c == 0 && gi == 0 && tid == 0) {
      a.ws_len[b] = ok ? (int32_t)n_old : -1;
      if (!ok) atomicOr(a.flag, 1);
    }
    if (!ok) return;
  }
  const int64_t hi_max = row_pos(a, b, a.n_pos - 1);
  const int64_t k_begin = (int64_t)c * a.chunk;
  if (k_begin > hi_max) return;
  const int64_t k_end = k_begin + a.chunk;  // exclusive

  // Per-row ranges (row = lane column `col` for this lane's softmax work).
  RowInfo ri;
  int row_h = -1, row_s = 0, row_j = 0;
  if (col < rows) {
    row_s = col / (a.n_pos * gsize);
    row_j = (col / gsize) % a.n_pos;
    row_h = groups.q[gi][col % gsize];
  }
  if (row_h >= 0) {
    const int64_t t = row_pos(a, b, row_j);
    const int Ws = a.W[row_s];
    ri.lo = (Ws > 0 && t - Ws + 1 > 0) ? t - Ws + 1 : 0;
    ri.hi = t;
  } else {
    ri.lo = 1;
    ri.hi = 0;
  }

  // cache pointers of this (batch, KV head)
  const int64_t head_off =
      ((int64_t)b * a.n_kv_heads + kvh) * a.cap * D;
  const uint16_t *kc = (const uint16_t *)a.k_cache + head_off;
  const uint16_t *vc = (const uint16_t *)a.v_cache + head_off;
  const uint16_t *kn = nullptr, *vn = nullptr;
  if (a.cache_len) {
    kn = (const uint16_t *)a.k_new + ((int64_t)b * a.n_kv_heads + kvh) * D;
    vn = (const uint16_t *)a.v_new + ((int64_t)b * a.n_kv_heads + kvh) * D;
    // The workgroup whose chunk holds the new row also stores it.
    if (n_old >= k_begin && n_old < k_end && w == 0 && lane < 32) {
      const int part = lane & 15;
      const uint4 *src = (const uint4 *)((lane < 16) ? kn : vn) + part;
      uint4 *dst = (uint4 *)(((lane < 16) ? (uint16_t *)a.k_cache
                                          : (uint16_t *)a.v_cache) +
                             head_off + n_old * D) + part;
      *dst = *src;
    }
  }

  // ---- query operand: Q^T (d on K, rows on N), affine + scale fused ------
  const float qscale = kLog2e * rsqrtf((float)D);
  bf16x8 qop[4];
  {
    const bool act = row_h >= 0;
    const uint16_t *qp = nullptr;
    const float *al = nullptr, *be = nullptr;
    if (act) {
      qp = (const uint16_t *)a.q[row_s] +
           (((int64_t)b * a.n_pos + row_j) * a.Hq + row_h) * D;
      al = a.alpha[row_s] + row_h * D;
      be = a.beta[row_s] + row_h * D;
    }
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int d0 = 32 * c4 + 8 * g4;
      uint4 raw = act ? *(const uint4 *)(qp + d0) : make_uint4(0, 0, 0, 0);
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = 0.0f;
        if (act) {
          const float qv = bf16_bits_to_f32((e & 1) ? (wv[e >> 1] >> 16)
                                                    : (wv[e >> 1] & 0xffffu));
          x = (al[d0 + e] * qv + be[d0 + e]) * qscale;
        }
        qop[c4][e] = (__bf16)x;
      }
    }
  }

  float m = -INFINITY, l = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_steps = a.chunk / (kWaves * kStep);
  for (int it = 0; it < n_steps; ++it) {
    const int64_t key0 = k_begin + (int64_t)(it * kWaves + w) * kStep;

    // K operand rows straight from global memory.
    bf16x8 kop[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int64_t key = key0 + 16 * kt + col;
      const uint16_t *src = (a.cache_len && key == n_old) ? kn : kc + key * D;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (key <= hi_max) raw = *(const uint4 *)(src + 32 * c4 + 8 * g4);
        kop[kt][c4] = __builtin_bit_cast(bf16x8, raw);
      }
    }
    // V rows into the wave's LDS region (16 lanes per 256-byte row).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kr = 4 * i + g4;
      const int64_t key = key0 + kr;
      const uint16_t *src = (a.cache_len && key == n_old) ? vn : vc + key * D;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (key <= hi_max) raw = *(const uint4 *)(src + 8 * col);
      *(uint4 *)&v_s[w][kr][8 * col] = raw;
    }

    // S^T tiles.
    f32x4 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kt][c4], qop[c4],
                                                        s[kt], 0, 0, 0);
    }

    // Mask to the row's key range, online softmax (base-2 domain).
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = key0 + 16 * kt + 4 * g4 + i;
        const bool ok = key >= ri.lo && key <= ri.hi;
        x[4 * kt + i] = ok ? s[kt][i] : -INFINITY;
        tmax = fmaxf(tmax, x[4 * kt + i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    float corr = 1.0f;
    bf16x8 pop;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pop[e] = (__bf16)0.0f;
    } else {
      corr = exp2f(m - m_new);
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pb = (__bf16)exp2f(x[e] - m_new);
        pop[e] = pb;
        ps += (float)pb;
      }
      l = l * corr + ps;
    }
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] *= corr;

    __syncthreads();  // V rows of every wave are in LDS
    // O^T += V^T P^T: the P^T operand holds keys {4g4..4g4+3} of the first
    // 16-key tile and the same of the second; V^T is gathered likewise.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + col;
      bf16x8 vop;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kr = (e < 4) ? (4 * g4 + e) : (16 + 4 * g4 + e - 4);
        vop[e] = __builtin_bit_cast(__bf16, v_s[w][kr][d]);
      }
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, acc[dt], 0,
                                                         0, 0);
    }
    __syncthreads();  // LDS region free for the next step
  }

  // ---- merge the 4 waves --------------------------------------------------
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (g4 == 0) {
    red_m[w][col] = m;
    red_l[w][col] = l;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_acc[w][col][16 * dt + 4 * g4 + i] = acc[dt][i];
  __syncthreads();

  const int r = tid >> 4;          // 16 rows x 16 threads
  const int d0 = (tid & 15) * 8;   // 8 channels each
  if (r < rows) {
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][r]);
    float L = 0.0f, o8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = red_m[ww][r];
        const float f = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
        L += f * red_l[ww][r];
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] += f * red_acc[ww][r][d0 + e];
      }
    }
    const int64_t pi = ws_part_index(a, groups.n_groups, rows, b, gi, c, r);
    float *ml = a.ws + pi * 2;
    float *pacc = a.ws + (int64_t)a.ws_acc_offset + pi * D + d0;
    if (d0 == 0) {
      ml[0] = M;
      ml[1] = L;
    }
    *(float4 *)pacc = make_float4(o8[0], o8[1], o8[2], o8[3]);
    *(float4 *)(pacc + 4) = make_float4(o8[4], o8[5], o8[6], o8[7]);
  }
}

// One block per (head group, batch); thread = (row, 8 channels).
__global__ __launch_bounds__(256) void splitkv_merge_kernel(SplitKVArgs a,
                                                            HeadGroups groups) {
  const int gi = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int gsize = groups.gsize;
  const int rows = a.n_streams * a.n_pos * gsize;
  int64_t n_old = 0;
  bool ok = true;
  if (a.cache_len) {
    n_old = a.ws_len[b];
    ok = n_old >= 0;
  }
  const int r = tid >> 4;
  const int d0 = (tid & 15) * 8;
  if (r < rows) {
    const int s = r / (a.n_pos * gsize);
    const int j = (r / gsize) % a.n_pos;
    const int h = groups.q[gi][r % gsize];
    if (h >= 0) {
      uint16_t *out = (uint16_t *)a.o[s] +
                      (((int64_t)b * a.n_pos + j) * a.Hq + h) * D + d0;
      float o8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (ok) {
        const int64_t t = (a.cache_len ? n_old : a.pos0) + j;
        const int Ws = a.W[s];
        const int64_t lo = (Ws > 0 && t - Ws + 1 > 0) ? t - Ws + 1 : 0;
        const int c_lo = (int)(lo / a.chunk), c_hi = (int)(t / a.chunk);
        float M = -INFINITY;
        for (int c = c_lo; c <= c_hi; ++c) {
          const int64_t pi = ws_part_index(a, groups.n_groups, rows, b, gi, c, r);
          M = fmaxf(M, a.ws[pi * 2]);
        }
        float L = 0.0f;
        for (int c = c_lo; c <= c_hi; ++c) {
          const int64_t pi = ws_part_index(a, groups.n_groups, rows, b, gi, c, r);
          const float mc = a.ws[pi * 2];
          if (mc == -INFINITY) continue;
          const float f = exp2f(mc - M);
          L += f * a.ws[pi * 2 + 1];
          const float *pacc = a.ws + (int64_t)a.ws_acc_offset + pi * D + d0;
          const float4 u = *(const float4 *)pacc;
          const float4 v = *(const float4 *)(pacc + 4);
          o8[0] += f * u.x; o8[1] += f * u.y; o8[2] += f * u.z; o8[3] += f * u.w;
          o8[4] += f * v.x; o8[5] += f * v.y; o8[6] += f * v.z; o8[7] += f * v.w;
        }
        const float inv = 1.0f / L;
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] *= inv;
      }
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo16 = __builtin_bit_cast(uint16_t, (__bf16)o8[2 * e]);
        const uint32_t hi16 = __builtin_bit_cast(uint16_t, (__bf16)o8[2 * e + 1]);
        pk[e] = lo16 | (hi16 << 16);
      }
      *(uint4 *)out = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
  }
  // Decode: the cache now holds n_old + 1 rows for this batch entry. Every
  // split workgroup has finished reading (kernel boundary), and the merge
  // reads the old length from the workspace, so this write races with none.
  if (a.cache_len && ok && gi == 0 && tid == 0)
    ((int32_t *)a.cache_len)[b] = (int32_t)(n_old + 1);
}

}  // namespace

int splitkv_rows(int n_streams, int n_pos, int gsize) {
  return n_streams * n_pos * gsize;
}

int splitkv_pick_chunk(int B, int n_groups, int64_t max_len) {
  int chunk = 512;
  while (chunk > 128 &&
         (int64_t)B * n_groups * ((max_len + chunk - 1) / chunk) < 2048)
    chunk /= 2;
  return chunk;
}

// Workspace layout: per-batch old lengths (int32, padded to 256 bytes), then
// (max, sum) float pairs of every partial, padded to 64 floats, then the
// unnormalised output rows. Must agree with the offsets set by the caller.
size_t splitkv_ws_bytes(int B, int n_groups, int rows, int n_chunks, int Dh) {
  const size_t parts = (size_t)B * n_groups * n_chunks * rows;
  const size_t len_bytes = ((size_t)B * 4 + 255) / 256 * 256;
  const size_t ml_floats = (parts * 2 + 63) / 64 * 64;
  return len_bytes + (ml_floats + parts * (size_t)Dh) * 4;
}

hipError_t launch_splitkv(const SplitKVArgs &a_in, const HeadGroups &groups,
                          hipStream_t stream) {
  SplitKVArgs a = a_in;
  dim3 grid(a.n_chunks, groups.n_groups, a.B);
  hipLaunchKernelGGL(splitkv_kernel, grid, dim3(kThreads), 0, stream, a,
                     groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(splitkv_merge_kernel, dim3(groups.n_groups, a.B),
                     dim3(256), 0, stream, a, groups);
  return hipGetLastError();
}

}  // namespace orthros
