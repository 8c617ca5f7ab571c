// Rolling-window attention for small windows on gfx950 MFMA (bf16, D = 128).
//
// The base stream of Orthros attention ("Orthros: Phase-Aware Heterogeneous
// Attention for Efficient Transformers", paper text §3.1, the o_t equation)
// with the small window the paper trains with (§4, W = 128). At such a
// window the work per query row is a few key tiles, so the pass is bound by
// streaming the queries and outputs from and to HBM, not by MFMA
// (§3.3: the window attention is linear in T; here its constant is small).
//
// Structure (one resident workgroup per compute unit, 8 waves, the 4 query
// heads of one KV head): a workgroup walks a contiguous segment of 64-row
// query tiles of one (batch, KV head). Query tile qt attends key tiles
// qt-NTB+1 .. qt (NTB = ceil((W-1)/64) + 1 = 3 for 65 < W <= 129; other
// windows run the banded kernel). Those tiles stay in an
// LDS ring of NTB+1 slots, so each query tile loads ONE new K/V tile (and
// its queries), which arrive in registers while the current tile is being
// computed; every byte of Q, K, V and O crosses HBM once.
//  * wave w owns 32 rows of query head w % 4 (row block w / 4); the MFMA
//    layouts are those of the banded kernel: S^T = K Q^T and O^T += V^T P^T
//    on v_mfma_f32_32x32x16_bf16, the V^T operand read with
//    ds_read_b64_tr_b16, each lane holding one query row;
//  * the softmax runs online over the NTB tiles (base 2, lazy rescaling of
//    the reference maximum, -m seeding the score accumulators), with band
//    masks only on tiles not inside every row's band;
//  * alpha (.) q + beta uses alpha, beta pre-scaled by log2(e)/sqrt(D) and
//    kept in LDS for the workgroup's heads.
#include "common.h"

namespace orthros {
namespace {

constexpr int D = 128;
constexpr int kRows = 32;          // query rows per wave
constexpr int kQT = 64;            // query rows per tile (2 row blocks)
constexpr int kBN = 64;            // keys per tile
constexpr int kKS = D + 8;         // K row stride (bf16): 272 bytes
constexpr int kVS = D + 32;        // V row stride (bf16): 320 bytes
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int kGsize = 4;          // query heads per KV head
constexpr float kTau = 8.0f;
constexpr int kBufferWord3 = 0x00020000;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

template <int NTB>
struct RollSmem {
  uint16_t k[NTB + 1][kBN][kKS];
  uint16_t v[NTB + 1][kBN][kVS];
  float ab[kGsize][2][D];  // alpha, beta of the group's heads, pre-scaled
};

template <int NTB>
__global__ __launch_bounds__(kNT, 2) void band_roll_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ alpha,
    const float *__restrict__ beta, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, uint16_t *__restrict__ o,
    int nrows, int Hq, int n_kv, int64_t cap, int W, int n_qtiles,
    int seg_len, int n_segs, HeadGroups groups) {
  constexpr int kSlots = NTB + 1;
  __shared__ __attribute__((aligned(16))) RollSmem<NTB> sm;

  const int seg = blockIdx.x % n_segs;
  const int rest = blockIdx.x / n_segs;
  const int gi = rest % groups.n_groups;
  const int b = rest / groups.n_groups;
  const int qt_begin = seg * seg_len;
  const int qt_end = min(qt_begin + seg_len, n_qtiles);
  if (qt_begin >= qt_end) return;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int j = lane & 31, hh = lane >> 5;
  const int kvh = groups.kv[gi];
  const int head = groups.q[gi][w % kGsize];
  const int ps = w / kGsize;
  const float qs = kLog2e * rsqrtf((float)D);

  // alpha / beta of the group's heads, scaled into the base-2 domain
  for (int i = tid; i < kGsize * 2 * D; i += kNT) {
    const int hs = i / (2 * D), which = (i / D) & 1, d = i % D;
    const int h = max((int)groups.q[gi][hs], 0);
    sm.ab[hs][which][d] = (which ? beta : alpha)[h * D + d] * qs;
  }

  // K/V slab of this (batch, KV head): rows past nrows read as zeros
  const int64_t head_off = ((int64_t)b * n_kv + kvh) * cap * D;
  const uint32_t slab_bytes = (uint32_t)nrows * (D * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(k_cache + head_off), 0, slab_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(v_cache + head_off), 0, slab_bytes, kBufferWord3);

  // staging of one K/V tile: 2 x 16 bytes per thread per tensor
  uint4 kst[2], vst[2];
  auto load_kv = [&](int kt) {  // kt >= 0
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off =
          (uint32_t)kt * (kBN * D * 2) + 16u * (uint32_t)(tid + kNT * i);
      kst[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      vst[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto store_kv = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + kNT * i;
      *(uint4 *)&sm.k[slot][idx >> 4][8 * (idx & 15)] = kst[i];
      *(uint4 *)&sm.v[slot][idx >> 4][8 * (idx & 15)] = vst[i];
    }
  };

  // raw query rows of a tile for this lane (row 64 qt + 32 ps + j, channels
  // 16 c + 8 hh .. + 7); rows past the end re-read the last row
  uint4 qraw[8];
  auto load_q = [&](int qt) {
    const int r = min(qt * kQT + kRows * ps + j, nrows - 1);
    const uint16_t *qp =
        q + (((int64_t)b * nrows + r) * Hq + max(head, 0)) * D + 8 * hh;
#pragma unroll
    for (int c = 0; c < 8; ++c) qraw[c] = *(const uint4 *)(qp + 16 * c);
  };
  bf16x8 qop[8];
  auto make_qop = [&](bool act) {
    const float *al = sm.ab[w % kGsize][0];
    const float *be = sm.ab[w % kGsize][1];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d0 = 16 * c + 8 * hh;
      const uint32_t wv[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = bf16_bits_to_f32((e & 1) ? (wv[e >> 1] >> 16)
                                                  : (wv[e >> 1] & 0xffffu));
        qop[c][e] = act ? (__bf16)(al[d0 + e] * qv + be[d0 + e])
                        : (__bf16)0.0f;
      }
    }
  };

  // V^T transposed-read addresses (see the banded kernel)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row0 = 4 * hh + (j16 >> 2);
  const int v_col0 = 16 * (g16 & 1) + 4 * (j16 & 3);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int Wm = W;

  // ---- prologue: key tiles qt_begin-NTB+1 .. qt_begin, queries of qt_begin
  for (int i = 0; i < NTB; ++i) {
    const int kt = qt_begin - NTB + 1 + i;
    if (kt < 0) continue;
    load_kv(kt);
    store_kv(kt % kSlots);
  }
  load_q(qt_begin);
  __syncthreads();  // ring tiles and alpha/beta visible
  {
    const int r = qt_begin * kQT + kRows * ps + j;
    make_qop(head >= 0 && r < nrows);
  }

  for (int qt = qt_begin; qt < qt_end; ++qt) {
    const bool has_next = qt + 1 < qt_end;
    if (has_next) {
      load_kv(qt + 1);
      load_q(qt + 1);
    }
    const int r_first = qt * kQT + kRows * ps;          // this wave's rows
    const int rq = r_first + j;
    const bool row_act = head >= 0 && rq < nrows;
    float m = -INFINITY, l = 0.0f;
    f32x16 acc[4], negm;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) negm[v] = 0.0f;

#pragma unroll
    for (int i = 0; i < NTB; ++i) {
      const int kt = qt - NTB + 1 + i;
      if (kt < 0) continue;  // before the sequence start (uniform)
      const int slot = kt % kSlots;
      // S^T - m
      f32x16 s[2];
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int sk = 0; sk < 2; ++sk) {
          const bf16x8 kop =
              *(const bf16x8 *)&sm.k[slot][32 * sk + j][16 * c + 8 * hh];
          s[sk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              kop, qop[c], c == 0 ? negm : s[sk], 0, 0, 0);
        }
      // band mask unless the tile lies inside every row's band (uniform per
      // wave): key offset d = key - t kept iff -W < d <= 0, i.e.
      // (unsigned)(d + W - 1) < W
      const bool inside = kt * kBN >= r_first + kRows - W &&
                          kt * kBN + kBN - 1 <= r_first;
      if (!inside) {
        const uint32_t u0 = (uint32_t)(kt * kBN - rq) + (uint32_t)(Wm - 1) +
                            4u * hh;
#pragma unroll
        for (int sk = 0; sk < 2; ++sk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t u =
                u0 + (uint32_t)(32 * sk + 8 * (v >> 2) + (v & 3));
            s[sk][v] = (u < (uint32_t)Wm) ? s[sk][v] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int sk = 0; sk < 2; ++sk)
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[sk][v]);
      tmax = max_xor32(tmax);
      const bool need = (m == -INFINITY) ? (tmax > -INFINITY) : (tmax > kTau);
      if (__any(need)) {
        const float shift = need ? tmax : 0.0f;
        const float corr =
            need ? ((m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(-shift))
                 : 1.0f;
        m = need ? ((m == -INFINITY) ? shift : m + shift) : m;
        l *= corr;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] *= corr;
#pragma unroll
        for (int sk = 0; sk < 2; ++sk) s[sk] -= shift;
        const float nm = (m == -INFINITY) ? 0.0f : -m;
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[v] = nm;
      }
      bf16x8 pop[4];
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pop[kg][e] = (__bf16)__builtin_amdgcn_exp2f(s[kg >> 1][8 * (kg & 1) + e]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pop[kg][e], pop[kg][e + 1]};
          l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        }
      }
#pragma unroll
      for (int kg = 0; kg < 4; ++kg)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int row = 16 * kg + v_row0;
          const int col = 32 * dt + v_col0;
          const bf16x4 lo4 = lds_read_tr(&sm.v[slot][row][col]);
          const bf16x4 hi4 = lds_read_tr(&sm.v[slot][row + 8][col]);
          const bf16x8 vop = {lo4[0], lo4[1], lo4[2], lo4[3],
                              hi4[0], hi4[1], hi4[2], hi4[3]};
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[kg],
                                                            acc[dt], 0, 0, 0);
        }
    }

    // ---- output rows of this tile ------------------------------------------
    l += __shfl_xor(l, 32, 64);
    if (row_act) {
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
            const uint32_t lo = __builtin_bit_cast(
                uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e] * inv));
            const uint32_t hi = __builtin_bit_cast(
                uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e + 1] * inv));
            pk[e] = lo | (hi << 16);
          }
          *(uint2 *)(op + d0) = make_uint2(pk[0], pk[1]);
        }
    }
    if (!has_next) break;
    // The new key tile goes to the slot of tile qt-NTB, which no wave reads
    // in this step; after the barrier every wave sees it.
    store_kv((qt + 1) % kSlots);
    {
      const int r = (qt + 1) * kQT + kRows * ps + j;
      make_qop(head >= 0 && r < nrows);
    }
    __syncthreads();
  }
}

}  // namespace

int band_roll_tiles(int W) { return (W - 1 + kBN - 1) / kBN + 1; }

hipError_t launch_band_roll(const void *q, const float *alpha,
                            const float *beta, const void *k_cache,
                            const void *v_cache, void *o, int B, int nrows,
                            int Hq, int64_t cap, int W,
                            const HeadGroups &groups, int n_kv,
                            hipStream_t stream) {
  const int n_qtiles = (nrows + kQT - 1) / kQT;
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount,
                              dev);
  if (e != hipSuccess) return e;
  // about one workgroup per compute unit, each on a contiguous segment
  const int64_t per = (int64_t)groups.n_groups * B;
  int64_t n_segs = (n_cu > 0 ? n_cu : 256) / per;
  if (n_segs < 1) n_segs = 1;
  if (n_segs > n_qtiles) n_segs = n_qtiles;
  const int seg_len = (int)((n_qtiles + n_segs - 1) / n_segs);
  n_segs = (n_qtiles + seg_len - 1) / seg_len;
  const dim3 grid((unsigned)(n_segs * per));
  const int ntb = band_roll_tiles(W);
#define ORTHROS_ROLL(N)                                                      \
  hipLaunchKernelGGL(band_roll_kernel<N>, grid, dim3(kNT), 0, stream,        \
                     (const uint16_t *)q, alpha, beta,                       \
                     (const uint16_t *)k_cache, (const uint16_t *)v_cache,   \
                     (uint16_t *)o, nrows, Hq, n_kv, cap, W, n_qtiles,       \
                     seg_len, (int)n_segs, groups)
  if (ntb == 3)
    ORTHROS_ROLL(3);
  else
    return hipErrorInvalidValue;
#undef ORTHROS_ROLL
  return hipGetLastError();
}

}  // namespace orthros
