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
// query tiles of one (batch, KV head). Query tile qt needs key tiles qt-2 ..
// qt at most (W <= 129); those stay in an LDS ring of four slots, so each
// query tile loads ONE new K/V tile (and its queries), which arrive in
// registers while the current tile is being computed; every byte of Q, K, V
// and O crosses HBM once.
//  * wave w owns 32 rows of query head w % 4 (row block w / 4); the MFMA
//    layouts are those of the banded kernel: S^T = K Q^T and O^T += V^T P^T
//    on v_mfma_f32_32x32x16_bf16, the V^T operand read with
//    ds_read_b64_tr_b16, each lane holding one query row;
//  * the 32 rows of a wave need the keys of NSB = ceil((W-1)/32) + 1
//    sub-blocks of 32 keys; all their scores are formed first (independent
//    MFMA chains), so the softmax takes one exact row maximum and needs no
//    rescaling; band masks only on sub-blocks not inside every row's band;
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

constexpr int kSlots = 4;  // ring of key tiles: the band's three + the next
constexpr int kOutStride = 136;              // bytes per staged output row
constexpr int kOutRegion = kRows * kOutStride;  // per wave: 4352 bytes
static_assert(kGsize * kOutRegion <= kBN * kKS * 2, "output staging fits a K slot");

struct RollSmem {
  uint16_t k[kSlots][kBN][kKS];
  uint16_t v[kSlots][kBN][kVS];
  float ab[kGsize][2][D];  // alpha, beta of the group's heads, pre-scaled
};

template <int NSB>
__global__ __launch_bounds__(kNT, 2) void band_roll_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ alpha,
    const float *__restrict__ beta, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, uint16_t *__restrict__ o,
    int nrows, int Hq, int n_kv, int64_t cap, int W, int n_qtiles,
    int seg_len, int n_segs, HeadGroups groups) {
  static_assert(NSB >= 1 && NSB <= 5, "the ring holds three key tiles");
  __shared__ __attribute__((aligned(16))) RollSmem sm;

  const int seg = blockIdx.x % n_segs;
  const int rest = blockIdx.x / n_segs;
  const int gi = rest % groups.n_groups;
  const int b = rest / groups.n_groups;
  const int qt_begin = seg * seg_len;
  const int qt_end = min(qt_begin + seg_len, n_qtiles);
  if (qt_begin >= qt_end) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6;
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

  // Q and O rows of a query tile through a buffer resource based at the
  // tile's first row of this head: rows past nrows read as zeros and their
  // stores are dropped. This lane's row 32 ps + j of the tile, channels
  // 16 c + 8 hh .. + 7 (loads) / 32 dt + 8 q4 + 4 hh .. + 3 (stores).
  const uint32_t row_bytes = (uint32_t)Hq * (D * 2);
  const uint32_t lane_off = (uint32_t)(kRows * ps + j) * row_bytes;
  auto tile_rsrc = [&](const uint16_t *base, int qt) {
    const int rows_left = min(nrows - qt * kQT, kQT);
    const uint16_t *p =
        base + (((int64_t)b * nrows + (int64_t)qt * kQT) * Hq + max(head, 0)) * D;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p), 0,
        (uint32_t)(rows_left - 1) * row_bytes + D * 2, kBufferWord3);
  };
  uint4 qraw[8];
  auto load_q = [&](int qt) {
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(q, qt);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qraw[c] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     rq, lane_off + 16u * hh + 32u * c, 0, 0));
  };
  // Rows past the end (and padding heads) compute on valid clamped data;
  // their outputs are never stored.
  bf16x8 qop[8];
  auto make_qop = [&]() {
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
        qop[c][e] = (__bf16)(al[d0 + e] * qv + be[d0 + e]);
      }
    }
  };

  // V^T transposed-read addresses (see the banded kernel)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row0 = 4 * hh + (j16 >> 2);
  const int v_col0 = 16 * (g16 & 1) + 4 * (j16 & 3);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int Wm = W;

  // ---- prologue: key tiles qt_begin-2 .. qt_begin, queries of qt_begin;
  // tiles before the sequence start are zeros (finite, and masked out)
  for (int i = 0; i < kSlots - 1; ++i) {
    const int kt = qt_begin - (kSlots - 2) + i;
    if (kt >= 0) {
      load_kv(kt);
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) kst[u] = vst[u] = make_uint4(0, 0, 0, 0);
    }
    store_kv(kt & (kSlots - 1));
  }
  load_q(qt_begin);
  __syncthreads();  // ring tiles and alpha/beta visible
  make_qop();

  // Sub-blocks of 32 keys: this wave's rows r_first .. r_first+31 need keys
  // r_first-W+1 .. r_first+31, i.e. NSB sub-blocks ending with the one on the
  // diagonal (global sub-block index 2 qt + ps).
  f32x16 acc[4];
  auto step = [&](int qt, int qt_next) {
    const int r_first = qt * kQT + kRows * ps;
    const int rq = r_first + j;
    // keys lo .. rq of this lane's row
    const int lo = max(rq - Wm + 1, 0);
    const uint32_t span = (uint32_t)(rq - lo);
    const int sb_first = 2 * qt + ps - (NSB - 1);
    // S^T for every sub-block: independent MFMA chains
    f32x16 s[NSB];
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
      const int sbg = sb_first + i;
      const uint16_t *kp = &sm.k[(sbg >> 1) & (kSlots - 1)][32 * (sbg & 1) + j][8 * hh];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 kop = *(const bf16x8 *)(kp + 16 * c);
        s[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            kop, qop[c], c == 0 ? f32x16{} : s[i], 0, 0, 0);
      }
      // keep the operand reads of later sub-blocks from being hoisted
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next tile's queries arrive in the registers qop leaves free
    load_q(qt_next);
    // band mask on sub-blocks not inside every row's band (uniform per
    // wave): key kept iff lo <= key <= rq, i.e. (unsigned)(key - lo) <= span
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
      const int kb = 32 * (sb_first + i);
      if (kb >= 0 && kb >= r_first + kRows - Wm && kb + 31 <= r_first)
        continue;
      const uint32_t u0 = (uint32_t)(kb - lo) + 4u * hh;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t u = u0 + (uint32_t)(8 * (v >> 2) + (v & 3));
        s[i][v] = (u <= span) ? s[i][v] : -INFINITY;
      }
    }
    // one row maximum over the whole band (it always holds the diagonal)
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) m = fmaxf(m, s[i][v]);
    }
    m = max_xor32(m);
    // P = exp2(S - m), O^T += V^T P^T
    float l = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
#pragma unroll
    for (int i = 0; i < NSB; ++i) {
      const int sbg = sb_first + i;
      const int slot = (sbg >> 1) & (kSlots - 1);
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        bf16x8 pop;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pop[e] = (__bf16)__builtin_amdgcn_exp2f(s[i][8 * kg + e] - m);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pop[e], pop[e + 1]};
          l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        }
        const int row = 32 * (sbg & 1) + 16 * kg + v_row0;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int col = 32 * dt + v_col0;
          const bf16x4 lo4 = lds_read_tr(&sm.v[slot][row][col]);
          const bf16x4 hi4 = lds_read_tr(&sm.v[slot][row + 8][col]);
          const bf16x8 vop = {lo4[0], lo4[1], lo4[2], lo4[3],
                              hi4[0], hi4[1], hi4[2], hi4[3]};
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, acc[dt],
                                                            0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- output rows, staged through LDS ------------------------------------
    // Once every wave is past its PV products, the ring slot of tile qt-2
    // is free (the next step's band starts at qt-1). Each wave takes a
    // private 32 x 64-channel region of it (136-byte rows) and writes O in
    // two channel halves: fragments in, then whole 128-byte row pieces out
    // (8 lanes per row, 16 bytes each), so every store covers full lines.
    l += __shfl_xor(l, 32, 64);
    __syncthreads();
    if (head >= 0) {
      const float inv = 1.0f / l;
      const int fslot = (qt + 2) & (kSlots - 1);
      uint8_t *region =
          (ps == 0 ? (uint8_t *)&sm.k[fslot][0][0] : (uint8_t *)&sm.v[fslot][0][0]) +
          (w % kGsize) * kOutRegion;
      const __amdgpu_buffer_rsrc_t ro = tile_rsrc(o, qt);
      const int rr = lane >> 3, cc = lane & 7;  // read-back row / chunk
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) {
          const int dt = 2 * half + d2;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t pk[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const uint32_t lo = __builtin_bit_cast(
                  uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e] * inv));
              const uint32_t hi = __builtin_bit_cast(
                  uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e + 1] * inv));
              pk[e] = lo | (hi << 16);
            }
            *(uint2 *)(region + j * kOutStride + 64 * d2 + 16 * q4 + 8 * hh) =
                make_uint2(pk[0], pk[1]);
          }
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = rr + 8 * it;
          const uint8_t *src = region + r * kOutStride + 16 * cc;
          const uint2 a0 = *(const uint2 *)src;
          const uint2 a1 = *(const uint2 *)(src + 8);
          const u32x4 pk = {a0.x, a0.y, a1.x, a1.y};
          __builtin_amdgcn_raw_buffer_store_b128(
              pk, ro, (uint32_t)(kRows * ps + r) * row_bytes + 128u * half +
                          16u * cc, 0, 0);
        }
      }
    }
  };

  // The last step reloads its own tile into the unused slot (the loads are
  // unconditional so that the staging registers never live across steps).
  for (int qt = qt_begin; qt < qt_end; ++qt) {
    const int qt_next = min(qt + 1, qt_end - 1);
    load_kv(qt_next);
    step(qt, qt_next);
    if (qt + 1 == qt_end) break;
    // The new key tile goes to the slot of tile qt-3, which no wave reads in
    // this step; after the barrier every wave sees it.
    store_kv((qt + 1) & (kSlots - 1));
    make_qop();
    __syncthreads();
  }
}

}  // namespace

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
  if (W < 1 || W > kRollMaxWindow) return hipErrorInvalidValue;
  const int nsb = (W - 1 + 31) / 32 + 1;  // 32-key sub-blocks per row block
#define ORTHROS_ROLL(N)                                                      \
  hipLaunchKernelGGL(band_roll_kernel<N>, grid, dim3(kNT), 0, stream,        \
                     (const uint16_t *)q, alpha, beta,                       \
                     (const uint16_t *)k_cache, (const uint16_t *)v_cache,   \
                     (uint16_t *)o, nrows, Hq, n_kv, cap, W, n_qtiles,       \
                     seg_len, (int)n_segs, groups)
  switch (nsb) {
    case 1: ORTHROS_ROLL(1); break;
    case 2: ORTHROS_ROLL(2); break;
    case 3: ORTHROS_ROLL(3); break;
    case 4: ORTHROS_ROLL(4); break;
    default: ORTHROS_ROLL(5); break;
  }
#undef ORTHROS_ROLL
  return hipGetLastError();
}

}  // namespace orthros
