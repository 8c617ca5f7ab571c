// Banded flash attention on gfx950 MFMA (bf16 in, fp32 accumulate), D = 128.
//
// Computes the base stream of Orthros attention ("Orthros: Phase-Aware
// Heterogeneous Attention for Efficient Transformers", paper text §3.1, the
// o_t equation: softmax of q_t.k_j/sqrt(D) over keys [t-W+1, t], with the
// base query's scale-offset alpha (.) q + beta) for every position, and with
// an unbounded window the output stream's full cross-attention when many
// output rows need it (§3.2 SFT / pre-training settings) and the full causal
// baseline. The paper-notes page of the same title (key design 3) runs both
// branches as flash-attention calls with window W and infinity; the
// reproduction note "Orthros：阶段异构注意力" (code mapping section) builds the
// window as a local view rather than a masked T x T matrix. Here: key tiles
// wholly outside a query tile's band are never loaded or multiplied.
//
// Tiling (one workgroup = 8 waves, 512 threads):
//  * the workgroup owns 32*P consecutive query rows of the `gsize` query
//    heads that share one KV head (P = 8 / gsize), so every K/V tile staged
//    in LDS feeds 8 waves x 32 rows;
//  * wave w owns 32 rows of one query head; lane (j, h) = (lane % 32,
//    lane / 32) holds query row j;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, rows on N, D on K):
//    each lane's 16 accumulators are 16 keys of its own row, so the row
//    maximum needs one cross-lane exchange (lane j with lane j + 32);
//  * O^T += V^T P^T on the same instruction (D on M, rows on N, keys on K):
//    P^T comes straight from the S^T accumulators (no LDS round trip); V is
//    written to LDS transposed, with the keys of every 16-key group permuted
//    so that each lane reads its 8 keys with one 16-byte load;
//  * the query is loaded once: affine in fp32, times log2(e)/sqrt(D), rounded
//    to bf16; softmax runs in base 2 with exp2;
//  * K/V tiles of 64 keys are double-buffered: the next tile's global loads
//    are in flight while the current tile is multiplied;
//  * workgroups are renumbered so that neighbouring query tiles of the same
//    KV head run on the same XCD (shared L2 for the overlapping bands), and
//    with an unbounded window the longest rows start first.
#include "common.h"

namespace orthros {
namespace {

constexpr int D = 128;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 32;          // query rows per wave
constexpr int kBN = 64;            // keys per LDS tile
constexpr int kKS = D + 8;         // K tile row stride (bf16)
constexpr int kVS = kBN + 8;       // V^T tile row stride (bf16)

struct Smem {
  uint16_t k[2][kBN][kKS];
  uint16_t vt[2][D][kVS];
};

// Position of key `e` (0..63) of a tile inside a V^T row: within every group
// of 16 keys the quads are stored in the order 0, 2, 1, 3, so that lane half
// h of the P^T operand (keys 4h..4h+3 and 8+4h..8+4h+3) reads 8 contiguous
// entries.
__device__ __forceinline__ int vt_slot(int e) {
  const int q = (e >> 2) & 3;
  const int perm = (q == 1) ? 2 : (q == 2) ? 1 : q;
  return (e & ~15) + perm * 4 + (e & 3);
}

__global__ __launch_bounds__(kThreads, 1) void band_mfma_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ alpha,
    const float *__restrict__ beta, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, uint16_t *__restrict__ o,
    int nrows, int Hq, int n_kv, int64_t cap, int64_t q_offset, int W,
    int n_qtiles, HeadGroups groups) {
  __shared__ __attribute__((aligned(16))) Smem sm;

  // ---- workgroup -> (query tile, head group, batch) ------------------------
  const int64_t n_blocks = (int64_t)gridDim.x;
  int64_t L = blockIdx.x;
  const int64_t n8 = n_blocks / 8 * 8;
  if (L < n8) L = (L % 8) * (n8 / 8) + L / 8;  // same-XCD neighbours
  int qt = (int)(L % n_qtiles);
  const int64_t rest = L / n_qtiles;
  const int gi = (int)(rest % groups.n_groups);
  const int b = (int)(rest / groups.n_groups);
  if (W <= 0) qt = n_qtiles - 1 - qt;  // unbounded: longest rows first

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int j = lane & 31, hh = lane >> 5;
  const int gsize = groups.gsize;
  const int P = kWaves / gsize;
  const int kvh = groups.kv[gi];
  const int head = groups.q[gi][w % gsize];
  const int ps = w / gsize;

  const int r0 = qt * kRows * P;
  const int r_end = min(r0 + kRows * P, nrows);       // exclusive
  const int64_t pos_lo = q_offset + r0;
  const int64_t pos_hi = q_offset + r_end - 1;
  const int64_t k_lo = (W > 0) ? max((int64_t)0, pos_lo - W + 1) : 0;
  const int64_t k_hi = pos_hi;
  const int64_t kt0 = k_lo / kBN;
  const int ntiles = (int)(k_hi / kBN - kt0 + 1);

  // This wave's rows and key band.
  const int wr0 = r0 + kRows * ps;
  const bool wave_on = head >= 0 && wr0 < nrows;
  const int64_t wpos_lo = q_offset + wr0;
  const int64_t wpos_hi = q_offset + min(wr0 + kRows, nrows) - 1;
  const int64_t wk_lo = (W > 0) ? max((int64_t)0, wpos_lo - W + 1) : 0;
  const int64_t wk_hi = wpos_hi;
  const int rq = wr0 + j;                      // this lane's query row
  const int64_t tq = q_offset + rq;
  const int64_t tq_lo = (W > 0) ? tq - W + 1 : INT64_MIN;

  const int64_t head_off = ((int64_t)b * n_kv + kvh) * cap * D;
  const uint16_t *kc = k_cache + head_off;
  const uint16_t *vc = v_cache + head_off;

  // ---- query operand (B of S^T): rows on N, D on K ------------------------
  bf16x8 qop[8];
  {
    const bool act = wave_on && rq < nrows;
    const float qs = kLog2e * rsqrtf((float)D);
    const uint16_t *qp = q + (((int64_t)b * nrows + rq) * Hq + head) * D;
    const float *al = alpha + head * D;
    const float *be = beta + head * D;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d0 = 16 * c + 8 * hh;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (act) raw = *(const uint4 *)(qp + d0);
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = 0.0f;
        if (act) {
          const float qv = bf16_bits_to_f32((e & 1) ? (wv[e >> 1] >> 16)
                                                    : (wv[e >> 1] & 0xffffu));
          x = (al[d0 + e] * qv + be[d0 + e]) * qs;
        }
        qop[c][e] = (__bf16)x;
      }
    }
  }

  // ---- tile staging: registers <-> LDS -------------------------------------
  // K: thread loads rows (tid/16) and (tid/16 + 32), 16 bytes at 8*(tid%16).
  // V: thread loads rows 2*(tid/16) and 2*(tid/16)+1 at the same channels and
  //    writes them transposed as 8 key pairs.
  const int st_row = tid >> 4, st_oct = tid & 15;
  uint4 kreg[2], vreg[2];
  auto load_tile = [&](int it) {
    const int64_t kb = (kt0 + it) * kBN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t key = kb + st_row + 32 * i;
      kreg[i] = (key <= k_hi) ? *(const uint4 *)(kc + key * D + 8 * st_oct)
                              : make_uint4(0, 0, 0, 0);
      const int64_t vkey = kb + 2 * st_row + i;
      vreg[i] = (vkey <= k_hi) ? *(const uint4 *)(vc + vkey * D + 8 * st_oct)
                               : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *(uint4 *)&sm.k[buf][st_row + 32 * i][8 * st_oct] = kreg[i];
    const uint32_t a0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
    const uint32_t a1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
    const int slot = vt_slot(2 * st_row);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // channel 8*oct + 2e: low halves; channel 8*oct + 2e + 1: high halves
      const uint32_t lo = __builtin_amdgcn_perm(a1[e], a0[e], 0x05040100u);
      const uint32_t hi = __builtin_amdgcn_perm(a1[e], a0[e], 0x07060302u);
      *(uint32_t *)&sm.vt[buf][8 * st_oct + 2 * e][slot] = lo;
      *(uint32_t *)&sm.vt[buf][8 * st_oct + 2 * e + 1][slot] = hi;
    }
  };

  float m = -INFINITY, l = 0.0f;
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int64_t kb = (kt0 + it) * kBN;
    if (it + 1 < ntiles) load_tile(it + 1);

    const bool touch = wave_on && kb <= wk_hi && kb + kBN - 1 >= wk_lo;
    if (touch) {
      // S^T for the two 32-key halves of the tile.
      f32x16 s[2];
#pragma unroll
      for (int sk = 0; sk < 2; ++sk) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[sk][v] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const bf16x8 kop =
              *(const bf16x8 *)&sm.k[buf][32 * sk + j][16 * c + 8 * hh];
          s[sk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[c], s[sk],
                                                          0, 0, 0);
        }
      }
      // Mask only tiles that cross a band edge of some row of this wave.
      const bool inside = (W <= 0 || kb >= wpos_hi - W + 1) &&
                          kb + kBN - 1 <= wpos_lo;
      float tmax = -INFINITY;
#pragma unroll
      for (int sk = 0; sk < 2; ++sk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (!inside) {
            const int64_t key =
                kb + 32 * sk + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (key > tq || key < tq_lo) s[sk][v] = -INFINITY;
          }
          tmax = fmaxf(tmax, s[sk][v]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m, tmax);
      float corr = 1.0f;
      bf16x8 pop[4];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
          for (int e = 0; e < 8; ++e) pop[kg][e] = (__bf16)0.0f;
      } else {
        corr = exp2f(m - m_new);
        float ps_sum = 0.0f;
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 pb = (__bf16)exp2f(s[kg >> 1][8 * (kg & 1) + e] - m_new);
            pop[kg][e] = pb;
            ps_sum += (float)pb;
          }
        l = l * corr + ps_sum;
      }
      m = m_new;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] *= corr;
      // O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) {
          const bf16x8 vop =
              *(const bf16x8 *)&sm.vt[buf][32 * dt + j][16 * kg + 8 * hh];
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[kg],
                                                            acc[dt], 0, 0, 0);
        }
    }

    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and store ---------------------------------------
  l += __shfl_xor(l, 32, 64);
  if (wave_on && rq < nrows) {
    const float inv = 1.0f / l;
    uint16_t *op = o + (((int64_t)b * nrows + rq) * Hq + head) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * dt + 8 * q4 + 4 * hh;
        uint32_t pk[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t lo =
              __builtin_bit_cast(uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e] * inv));
          const uint32_t hi = __builtin_bit_cast(
              uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e + 1] * inv));
          pk[e] = lo | (hi << 16);
        }
        *(uint2 *)(op + d0) = make_uint2(pk[0], pk[1]);
      }
  }
}

}  // namespace

hipError_t launch_band_mfma(const void *q, const float *alpha,
                            const float *beta, const void *k_cache,
                            const void *v_cache, void *o, int B, int nrows,
                            int Hq, int64_t cap, int64_t q_offset, int W,
                            const HeadGroups &groups, int n_kv,
                            hipStream_t stream) {
  const int P = kWaves / groups.gsize;
  const int n_qtiles = (nrows + kRows * P - 1) / (kRows * P);
  const int64_t n_blocks = (int64_t)n_qtiles * groups.n_groups * B;
  hipLaunchKernelGGL(band_mfma_kernel, dim3((unsigned)n_blocks),
                     dim3(kThreads), 0, stream, (const uint16_t *)q, alpha,
                     beta, (const uint16_t *)k_cache, (const uint16_t *)v_cache,
                     (uint16_t *)o, nrows, Hq, n_kv, cap, q_offset, W,
                     n_qtiles, groups);
  return hipGetLastError();
}

}  // namespace orthros
