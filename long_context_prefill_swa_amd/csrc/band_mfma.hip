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
// Tiling (one workgroup = NW waves):
//  * the workgroup owns 32*NW/gsize consecutive query rows of the `gsize`
//    query heads that share one KV head, so every K/V tile staged in LDS
//    feeds NW waves x 32 rows;
//  * wave w owns 32 rows of one query head; lane (j, h) = (lane % 32,
//    lane / 32) holds query row j;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, rows on N, D on K):
//    each lane's 16 accumulators are 16 keys of its own row, so the row
//    maximum needs one cross-lane exchange (lane j with lane j + 32);
//  * O^T += V^T P^T on the same instruction (D on M, rows on N, keys on K):
//    P^T comes straight from the S^T accumulators (no LDS round trip); V stays
//    in LDS in its natural [key][d] layout and the V^T operand is read with
//    the gfx950 transposing LDS load (ds_read_b64_tr_b16): within 16 lanes,
//    lane i receives element i%4 of the 8-byte rows addressed by lanes
//    4e + i/4 (e = 0..3), so pointing lane j at V[k0 + j/4][d0 + 4(j%4)]
//    hands lane i the four keys k0..k0+3 of channel d0 + i;
//  * the query is loaded once: affine in fp32, times log2(e)/sqrt(D), rounded
//    to bf16; the softmax runs in base 2;
//  * lazy rescaling: the running maximum m only moves when a tile's scores
//    exceed it by more than 2^8 (then the accumulators are rescaled); the
//    current -m is the accumulator input of the first S MFMA, so the scores
//    arrive already shifted; exp2 arguments stay <= 8;
//  * the row sum adds the same bf16 probabilities that feed the P V product
//    (v_dot2_f32_bf16 against ones);
//  * K/V tiles of 64 keys are double-buffered: the next tile's global loads
//    are in flight while the current tile is multiplied;
//  * workgroups are renumbered so that neighbouring query tiles of the same
//    KV head run on the same XCD (shared L2 for the overlapping bands), and
//    with an unbounded window the longest rows start first.

#include "common.h"

namespace orthros {
namespace {

constexpr int D = 128;
constexpr int kRows = 32;          // query rows per wave
constexpr int kBN = 64;            // keys per LDS tile
constexpr int kKS = D + 8;         // K tile row stride (bf16): 272 bytes
constexpr int kVS = D + 32;        // V tile row stride (bf16): 320 bytes
constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) buffer access
constexpr float kTau = 8.0f;       // lazy-rescale threshold (base-2 units)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct Smem {
  uint16_t k[2][kBN][kKS];
  uint16_t v[2][kBN][kVS];
};

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void band_mfma_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ alpha,
    const float *__restrict__ beta, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, uint16_t *__restrict__ o,
    int nrows, int Hq, int n_kv, int64_t cap, int64_t q_offset, int W,
    int n_qtiles, HeadGroups groups) {
  constexpr int NT = NW * 64;
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
  const int P = NW / gsize;
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
  const int rq = wr0 + j;                      // this lane's query row
  const int64_t tq = q_offset + rq;
  // Band of this lane's row in offsets d = key - tq: -Wm < d <= 0.
  const int Wm = (W > 0) ? W : INT32_MAX;

  // Cache slab of this (batch, KV head), read through buffer resources that
  // end after key k_hi: tile rows past it load as zeros.
  const int64_t head_off = ((int64_t)b * n_kv + kvh) * cap * D;
  const uint32_t slab_bytes = (uint32_t)((k_hi + 1) * D * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(k_cache + head_off), 0, slab_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(v_cache + head_off), 0, slab_bytes, kBufferWord3);

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
      float4 a0 = make_float4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
      if (act) {
        raw = *(const uint4 *)(qp + d0);
        a0 = *(const float4 *)(al + d0);
        a1 = *(const float4 *)(al + d0 + 4);
        b0 = *(const float4 *)(be + d0);
        b1 = *(const float4 *)(be + d0 + 4);
      }
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = bf16_bits_to_f32((e & 1) ? (wv[e >> 1] >> 16)
                                                  : (wv[e >> 1] & 0xffffu));
        qop[c][e] = (__bf16)((av[e] * qv + bv[e]) * qs);
      }
    }
  }

  // ---- tile staging: registers <-> LDS (16-byte chunks, natural layout) ----
  constexpr int kChunks = kBN * D / 8 / NT;   // per thread, per tensor
  // A staging set holds K of one tile and V of the tile before it.
  struct Stage {
    uint4 k[kChunks], v[kChunks];
  };
  auto load_tile = [&](Stage &r, int kt) {
    const uint32_t k_off = (uint32_t)((kt0 + kt) * kBN) * (D * 2);
    const uint32_t v_off = k_off - (uint32_t)(kBN * D * 2);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const uint32_t off = 16u * (uint32_t)(tid + NT * i);
      r.k[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + off, 0, 0));
      if (kt > 0)
        r.v[i] = __builtin_bit_cast(
            uint4,
            __builtin_amdgcn_raw_buffer_load_b128(rv, v_off + off, 0, 0));
    }
  };
  auto store_k = [&](const Stage &r, int buf) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int idx = tid + NT * i;
      *(uint4 *)&sm.k[buf][idx >> 4][8 * (idx & 15)] = r.k[i];
    }
  };
  auto store_v = [&](const Stage &r, int buf) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int idx = tid + NT * i;
      *(uint4 *)&sm.v[buf][idx >> 4][8 * (idx & 15)] = r.v[i];
    }
  };
  // Transposed-read addresses of the V^T operand: lane group g16 covers
  // channels 16*(g16 % 2) (+32 dt) and key half hh = g16 / 2.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row0 = 4 * hh + (j16 >> 2);          // + 16 kg (+ 8 second read)
  const int v_col0 = 16 * (g16 & 1) + 4 * (j16 & 3);  // + 32 dt

  float m = -INFINITY, l = 0.0f;
  f32x16 acc[4], negm;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) negm[v] = 0.0f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T - m of one tile: keys of K buffer `kbuf`, seeded with the current -m.
  auto scores = [&](f32x16 (&sn)[2], int kbuf) {
    sn[0] = negm;
    sn[1] = negm;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int sk = 0; sk < 2; ++sk) {
        const bf16x8 kop =
            *(const bf16x8 *)&sm.k[kbuf][32 * sk + j][16 * c + 8 * hh];
        sn[sk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[c], sn[sk],
                                                         0, 0, 0);
      }
  };
  // Band mask (only tiles crossing a band edge of some row of this wave),
  // row maximum, and the lazy move of the reference maximum.
  auto settle = [&](f32x16 (&sn)[2], int64_t kb) {
    const bool inside = (W <= 0 || kb >= wpos_hi - W + 1) &&
                        kb + kBN - 1 <= wpos_lo;
    if (!inside) {
      const int d0 = (int)(kb - tq);  // |kb - tq| < 2^31 (cap < 2^31)
#pragma unroll
      for (int sk = 0; sk < 2; ++sk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int d = d0 + 32 * sk + 8 * (v >> 2) + 4 * hh + (v & 3);
          sn[sk][v] = (d > 0 || d <= -Wm) ? -INFINITY : sn[sk][v];
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int sk = 0; sk < 2; ++sk)
#pragma unroll
      for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, sn[sk][v]);
    tmax = max_xor32(tmax);
    // Move the reference maximum only when needed (first keys of a row, or
    // scores more than kTau above it).
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
      for (int sk = 0; sk < 2; ++sk) sn[sk] -= shift;
      const float nm = (m == -INFINITY) ? 0.0f : -m;
#pragma unroll
      for (int v = 0; v < 16; ++v) negm[v] = nm;
    }
  };

  // Software pipeline, one 64-key tile per step. Entering step `it`:
  // scores of tile it are settled in registers, K of tile it+1 and V of tile
  // it are in LDS, and K of tile it+2 with V of tile it+1 are arriving in one
  // staging set (loaded during the previous step). The step starts the loads
  // of K of tile it+3 and V of tile it+2 into the other set, multiplies the
  // next tile's scores while it exponentiates this one (MFMA and VALU work of
  // one wave overlap), accumulates P V, settles the next scores and moves
  // the arrived set into LDS. Tiles past the last one load as zeros and are
  // masked, so the pipeline needs no tail branch.
  // Prologue: K of tiles 0 and 1 and V of tile 0 are loaded together, then
  // stored; K of tile 2 and V of tile 1 stay in flight through step 0.
  Stage ra, rb;
  load_tile(rb, 0);
  load_tile(ra, 1);
  store_k(rb, 0);
  store_k(ra, 1);
  store_v(ra, 0);
  load_tile(ra, 2);
  __syncthreads();
  f32x16 sa[2], sb[2];
  scores(sa, 0);
  settle(sa, kt0 * kBN);
  __syncthreads();  // K buffer 0 is refilled at the end of step 0

  auto step = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], Stage &r_in,
                  Stage &r_out, int it) {
    const int64_t kb = (kt0 + it) * kBN;
    load_tile(r_out, it + 3);  // stored at the end of the next step
    scores(sn, (it + 1) & 1);
    bf16x8 pop[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pop[kg][e] =
            (__bf16)__builtin_amdgcn_exp2f(sc[kg >> 1][8 * (kg & 1) + e]);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pop[kg][e], pop[kg][e + 1]};
        l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
      }
    }
    // O^T += V^T P^T
    const int vb = it & 1;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int row = 16 * kg + v_row0;
        const int col = 32 * dt + v_col0;
        const bf16x4 lo4 = lds_read_tr(&sm.v[vb][row][col]);
        const bf16x4 hi4 = lds_read_tr(&sm.v[vb][row + 8][col]);
        const bf16x8 vop = {lo4[0], lo4[1], lo4[2], lo4[3],
                            hi4[0], hi4[1], hi4[2], hi4[3]};
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[kg],
                                                          acc[dt], 0, 0, 0);
      }
    // Instruction order for the block above: the next tile's score MFMAs
    // interleaved with this tile's exponentials, conversions and row-sum
    // dots, then the P V MFMAs; LDS operand reads run two MFMAs ahead.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);    // K operand reads
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // score MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // K reads, then V^T
      __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);  // exp2
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // cvt, dot2
    }
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // V^T reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // P V MFMA
    }
    settle(sn, kb + kBN);
    store_k(r_in, it & 1);     // K of tile it+2
    store_v(r_in, vb ^ 1);     // V of tile it+1
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    step(sa, sb, ra, rb, it);
    step(sb, sa, rb, ra, it + 1);
  }
  if (it < ntiles) step(sa, sb, ra, rb, it);

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
  constexpr int NW = 8;  // one workgroup per compute unit
  const int P = NW / groups.gsize;
  const int n_qtiles = (nrows + kRows * P - 1) / (kRows * P);
  const int64_t n_blocks = (int64_t)n_qtiles * groups.n_groups * B;
  hipLaunchKernelGGL(band_mfma_kernel<NW>, dim3((unsigned)n_blocks),
                     dim3(NW * 64), 0, stream, (const uint16_t *)q, alpha,
                     beta, (const uint16_t *)k_cache,
                     (const uint16_t *)v_cache, (uint16_t *)o, nrows, Hq,
                     n_kv, cap, q_offset, W, n_qtiles, groups);
  return hipGetLastError();
}

}  // namespace orthros
