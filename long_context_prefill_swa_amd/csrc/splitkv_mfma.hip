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
// memory I/O), so the design goal is coalesced reads with many bytes in
// flight and all query rows of a KV head sharing each read.
//
// Work split: grid (chunk, head group, batch). A workgroup (4 waves) owns
// `chunk` consecutive keys of one (batch, KV head) and every query row that
// reads that KV head (query heads of the group x streams x positions, at most
// 16, one per MFMA column). The waves advance through the chunk 128 keys at a
// time, wave w taking keys 32w..32w+31 of each 128; they never synchronise
// inside the key loop. Per 32-key slice:
//   S^T[key][row] = K Q^T        2 x 4 MFMA 16x16x32 (keys on M, rows on N)
//   online softmax per row       (one row per lane column; no cross-row work)
//   O^T[d][row] += V^T P^T        8 MFMA 16x16x32 (d on M, keys on K)
// K goes from global memory straight into MFMA operand registers. V rows are
// written to a wave-private LDS region in their natural layout and the V^T
// operand is read with the transposing LDS load (ds_read_b64_tr_b16). The
// next slice's K and V are loaded into a second register set while the
// current one is multiplied (two-stage pipeline, unrolled by two so both
// sets stay in registers). All cache reads go through buffer resources whose
// range ends at the workgroup's last valid key: reads past it return zeros
// (never rows beyond the cache length), and the scores of those keys are
// masked, so the loop has no data-dependent branch.
//
// After the loop the 4 waves merge in LDS and the workgroup writes one
// (max, sum, unnormalised output) partial per row. The partials of all
// chunks are then combined with log-sum-exp weights, normalised and written
// as the output rows, in one of two ways:
//  * one launch (a grid that the chip holds at once, such as a long
//    prompt's output row): each workgroup counts itself in at its (batch,
//    head group) and the last to arrive combines the group's partials; in
//    a decode step the last workgroup of a batch entry to finish advances
//    its cache length. The arrival counters sit in the workspace, start at
//    zero and are left at zero.
//  * two launches (a grid of many rounds, such as a decode step over many
//    sequences): splitkv_merge_kernel combines after the split kernel, one
//    workgroup per (row, head group, batch), and advances the lengths from
//    the old ones the split kernel left in the workspace. Here the split
//    workgroups end as soon as their partials are issued; waiting for the
//    stores and counting in would hold each of the many workgroups' slots
//    a few microseconds longer (a B = 64 decode step measured 2-6% slower
//    in one launch).
#include "common.h"

namespace orthros {
namespace {

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSlice = 32;          // keys per wave per step
constexpr int kStepKeys = kWaves * kSlice;
constexpr int kMaxRows = 16;
constexpr int kVS = D + 16;         // staged V row stride (bf16): 288 bytes
constexpr int kAccS = D + 4;        // merge row stride (fp32)
constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) buffer access

struct VStage {
  uint16_t v[kWaves][kSlice][kVS];  // 36 KB
};
struct Merge {
  float acc[kWaves][kMaxRows][kAccS];  // 33 KB
  float m[kWaves][kMaxRows];
  float l[kWaves][kMaxRows];
};
// The last arriver's combination of the chunks' partials: the 8 half-wave
// slots' running results.
struct Combine {
  float m[8], l[8];
  float acc[8][D];
};
union SplitSmem {
  VStage st;
  Merge mg;
  Combine cb;
};

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

// Orders this wave's LDS stores before its later LDS loads (other lanes of
// the same wave read what a lane wrote). LDS operations of one wave execute
// in order, so only the compiler has to be kept from reordering.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int64_t ws_part_index(const SplitKVArgs &a,
                                                 int n_groups, int rows,
                                                 int b, int gi, int c,
                                                 int r) {
  return (((int64_t)b * n_groups + gi) * a.n_chunks + c) * rows + r;
}

// The partials cross workgroups, and so compute units and XCDs, within one
// launch. They are written and read with device-scope buffer stores and
// loads (cache policy SC1), which go to the level of the memory hierarchy
// all XCDs share; the writer waits for its stores to complete before it
// counts itself in. No cache-wide write-back or invalidation (what a
// device-scope fence does) is needed: those cost microseconds per
// workgroup. Every store and load instruction covers whole 128-byte lines
// (a half wave moves one 512-byte row of a partial): device-scope accesses
// are not combined in the L2, so partial lines would multiply the requests.
constexpr int kDeviceScope = 16;  // buffer cache policy: SC1
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The partials of (batch b, group gi): (max, sum) pairs and output rows of
// its n_chunks x rows partials, as two buffer resources (byte offsets
// (c rows + r) x 8 and x 512).
struct PartialView {
  __amdgpu_buffer_rsrc_t ml, acc;
};
__device__ __forceinline__ PartialView partial_view(const SplitKVArgs &a,
                                                    int n_groups, int rows,
                                                    int b, int gi) {
  const int64_t p0 = ((int64_t)b * n_groups + gi) * a.n_chunks * rows;
  const int n = a.n_chunks * rows;
  PartialView v;
  v.ml = __builtin_amdgcn_make_buffer_rsrc(a.ws + p0 * 2, 0, n * 8,
                                           kBufferWord3);
  v.acc = __builtin_amdgcn_make_buffer_rsrc(
      a.ws + a.ws_acc_offset + p0 * D, 0, n * D * 4, kBufferWord3);
  return v;
}

// The last arriver of (batch b, group gi): every output row of the group,
// from the partials of the chunks that hold keys of the row's range,
// combined with log-sum-exp weights, normalised and written in bf16. Rows go
// in passes of nr <= 8; in a pass the 8 half-wave slots split as spr =
// 8 / nr slots per row, slot g taking row r0 + g % nr and every spr-th chunk
// of its range from c_lo + g / nr. Lane f of a slot holds channels 4f ..
// 4f + 3 and a running (max, sum, output); loads go out kBatch chunks at a
// time, so a slot's chunks cost a few memory round trips. The slots of a row
// are then combined in LDS. Called by all threads of the workgroup.
__device__ __forceinline__ void combine_group(const SplitKVArgs &a,
                                              const HeadGroups &groups,
                                              Combine &cb, int b, int gi,
                                              int64_t pos_base) {
  constexpr int kBatch = 8;
  const int tid = threadIdx.x;
  const int gsize = groups.gsize;
  const int rows = a.n_streams * a.n_pos * gsize;
  const PartialView pv = partial_view(a, groups.n_groups, rows, b, gi);
  const int g = tid >> 5, f = tid & 31;
  for (int r0 = 0; r0 < rows; r0 += 8) {
    const int nr = min(rows - r0, 8), spr = 8 / nr;
    float M = -INFINITY, L = 0.0f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (g < nr * spr) {
      const int r = r0 + g % nr, sub = g / nr;
      const int s = r / (a.n_pos * gsize);
      const int64_t t = pos_base + (r / gsize) % a.n_pos;
      const int Ws = a.W[s];
      const int64_t lo = (Ws > 0 && t - Ws + 1 > 0) ? t - Ws + 1 : 0;
      const int c_lo = (int)(lo / a.chunk), c_hi = (int)(t / a.chunk);
      for (int c0 = c_lo + sub; c0 <= c_hi; c0 += kBatch * spr) {
        f32x2 mlv[kBatch];
        f32x4 u[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          // past the range: reload the last chunk, weight it out below
          const int cc = min(c0 + k * spr, c_hi);
          const int pi = cc * rows + r;
          mlv[k] = __builtin_bit_cast(
              f32x2, __builtin_amdgcn_raw_buffer_load_b64(pv.ml, pi * 8, 0,
                                                          kDeviceScope));
          u[k] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         pv.acc, pi * (D * 4) + f * 16, 0, kDeviceScope));
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const float mc = c0 + k * spr <= c_hi ? mlv[k].x : -INFINITY;
          if (mc != -INFINITY) {  // a chunk with keys in this row's range
            const float Mn = fmaxf(M, mc);
            const float fo = exp2f(M - Mn), fn = exp2f(mc - Mn);
            L = L * fo + mlv[k].y * fn;
            o = o * fo + u[k] * fn;
            M = Mn;
          }
        }
      }
    }
    __syncthreads();  // the previous pass's readers of cb are done
    if (f == 0) {
      cb.m[g] = M;
      cb.l[g] = L;
    }
    *(f32x4 *)&cb.acc[g][4 * f] = o;
    __syncthreads();
    const int j = tid >> 5;  // row r0 + j, channels 4f .. 4f + 3
    if (j < nr) {
      const int r = r0 + j;
      const int h = groups.q[gi][r % gsize];
      if (h >= 0) {  // a padded head slot has no output row
        float Mx = -INFINITY;
        for (int q = 0; q < spr; ++q) Mx = fmaxf(Mx, cb.m[j + q * nr]);
        float Lx = 0.0f;
        f32x4 out = {0.f, 0.f, 0.f, 0.f};
        if (Mx != -INFINITY) {
          for (int q = 0; q < spr; ++q) {
            const int gq = j + q * nr;
            const float w = exp2f(cb.m[gq] - Mx);  // 0 for an empty slot
            Lx += w * cb.l[gq];
            out += w * *(const f32x4 *)&cb.acc[gq][4 * f];
          }
        }
        const float inv = Lx > 0.0f ? 1.0f / Lx : 0.0f;
        const int s = r / (a.n_pos * gsize);
        const int jp = (r / gsize) % a.n_pos;
        uint16_t *dst = (uint16_t *)a.o[s] +
                        (((int64_t)b * a.n_pos + jp) * a.Hq + h) * D + 4 * f;
        uint32_t w2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t lo16 =
              __builtin_bit_cast(uint16_t, (__bf16)(out[2 * e] * inv));
          const uint32_t hi16 =
              __builtin_bit_cast(uint16_t, (__bf16)(out[2 * e + 1] * inv));
          w2[e] = lo16 | (hi16 << 16);
        }
        *(uint2 *)dst = make_uint2(w2[0], w2[1]);
      }
    }
  }
}

// Registers of one 32-key slice: K in MFMA operand layout (lane (col, g4)
// holds K[16 kt + col][32 c4 + 8 g4 ..]), V rows 4 i + g4 at channels 8 col.
struct Slice {
  uint4 k[2][4];
  uint4 v[8];
};

template <bool Paged>
__global__ __launch_bounds__(kThreads, 2) void splitkv_kernel(
    SplitKVArgs a, HeadGroups groups) {
  __shared__ __attribute__((aligned(16))) SplitSmem sm;

  // Chunk numbering rotated per sequence: workgroups are dealt to the XCDs
  // by flat id, so with a chunk count that is a multiple of 8 every XCD
  // would otherwise read the same chunk positions of every sequence's slab
  // (a 16-chunk decode step at B = 64 then streamed at 3.6 instead of
  // 5.7 TB/s). One sequence keeps the plain order.
  const int gi = blockIdx.y, b = blockIdx.z;
  const int c = (int)((blockIdx.x + (unsigned)b) % gridDim.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 15, g4 = lane >> 4;
  const int gsize = groups.gsize;
  const int rows = a.n_streams * a.n_pos * gsize;
  const int kvh = groups.kv[gi];

  // ---- positions and validity (decode: lengths live on the device) -------
  int64_t n_old = 0;
  if (a.cache_len) {
    n_old = a.cache_len[b];
    const bool ok = n_old >= 0 && n_old + 1 <= a.max_len && n_old + 1 <= a.cap;
    if (!ok) {
      // skipped (the length is left unchanged): chunk 0 of each group
      // writes the group's output rows as zeros
      if (c == 0) {
        if (gi == 0 && tid == 0) {
          atomicOr(a.flag, 1);
          if (!a.fused) a.ws_len[b] = -1;
        }
        const int r = tid >> 4, d0 = (tid & 15) * 8;
        if (r < rows) {
          const int hq = groups.q[gi][r % gsize];
          if (hq >= 0) {
            uint16_t *dst =
                (uint16_t *)a.o[r / (a.n_pos * gsize)] +
                (((int64_t)b * a.n_pos + (r / gsize) % a.n_pos) * a.Hq + hq) * D +
                d0;
            *(uint4 *)dst = make_uint4(0, 0, 0, 0);
          }
        }
      }
      return;
    }
  }
  // Decode: each workgroup of batch entry b counts itself out once it is
  // done with the entry's length; the last one out advances the length
  // (every other workgroup of the entry has read it by then).
  auto leave = [&]() {
    if (a.cache_len && tid == 0) {
      int32_t *bc = a.counters + (int64_t)a.B * groups.n_groups + b;
      if (atomicAdd(bc, 1) == (int)(gridDim.x * gridDim.y) - 1) {
        atomicExch(bc, 0);
        ((int32_t *)a.cache_len)[b] = (int32_t)(n_old + 1);
      }
    }
  };
  // two launches: the merge kernel reads the old length from the workspace
  if (!a.fused && a.cache_len && c == 0 && gi == 0 && tid == 0)
    a.ws_len[b] = (int32_t)n_old;
  const int64_t pos_base = a.cache_len ? n_old : a.pos0;  // row 0's position
  const int64_t hi_max = pos_base + a.n_pos - 1;
  const int64_t k_begin = (int64_t)c * a.chunk;
  if (k_begin > hi_max) {
    if (a.fused) leave();
    return;
  }
  // keys of this workgroup: [k_begin, k_stop)
  const int64_t k_stop = min(k_begin + (int64_t)a.chunk, hi_max + 1);
  const int n_steps = (int)((k_stop - k_begin + kStepKeys - 1) / kStepKeys);

  // This lane's softmax row (MFMA column `col`) and its key range.
  int row_h = -1, row_s = 0, row_j = 0;
  if (col < rows) {
    row_s = col / (a.n_pos * gsize);
    row_j = (col / gsize) % a.n_pos;
    row_h = groups.q[gi][col % gsize];
  }
  int64_t r_lo = 1, r_hi = 0;  // empty unless the row is active
  if (row_h >= 0) {
    const int64_t t = pos_base + row_j;
    const int Ws = row_s ? a.W[1] : a.W[0];
    r_lo = (Ws > 0 && t - Ws + 1 > 0) ? t - Ws + 1 : 0;
    r_hi = min(t, k_stop - 1);
  }

  // Contiguous cache: the slab of this (batch, KV head), rows [0, k_stop)
  // readable through buffer resources (reads past them return zeros).
  // Paged cache: each 32-key slice lies in one page (page_size >= 32); lane
  // l holds the block-table entry of the chunk's l-th page (a chunk spans at
  // most 64 pages), out-of-range entries are clamped and raise the flag.
  const int64_t head_off = ((int64_t)b * a.n_kv_heads + kvh) * a.cap * D;
  uint16_t *kc = (uint16_t *)a.k_cache + head_off;
  uint16_t *vc = (uint16_t *)a.v_cache + head_off;
  int my_page = 0, my_ok = 1;
  int64_t first_page = 0;
  int64_t page_elems = 0;  // elements of one KV head's part of a page
  if constexpr (Paged) {
    page_elems = (int64_t)D << a.page_log2;
    first_page = k_begin >> a.page_log2;
    const int64_t pi = first_page + lane;
    if (pi * (1 << a.page_log2) < k_stop && pi < a.max_pages) {
      const int32_t e = a.block_table[(int64_t)b * a.max_pages + pi];
      const bool ok = e >= 0 && e < a.n_pages;
      if (!ok) atomicOr(a.flag, 1);
      my_page = ok ? e : 0;
      my_ok = ok;
    }
  }
  // Base of key `key`'s page (paged) or of the slab, for this KV head.
  auto page_slot = [&](int64_t key) {
    return max(min((int)((key >> a.page_log2) - first_page), 63), 0);
  };
  auto page_base = [&](uint16_t *pool, int64_t key) -> uint16_t * {
    const int page = __builtin_amdgcn_readlane(my_page, page_slot(key));
    return pool + ((int64_t)page * a.n_kv_heads + kvh) * page_elems;
  };
  if (a.cache_len && n_old >= k_begin && n_old < k_stop) {
    // Decode: this workgroup's chunk holds the new row. Store it first; it
    // is the only workgroup that reads that row.
    uint16_t *kd = kc + n_old * D, *vd = vc + n_old * D;
    if constexpr (Paged) {
      const int64_t row = n_old & ((1 << a.page_log2) - 1);
      kd = page_base((uint16_t *)a.k_cache, n_old) + row * D;
      vd = page_base((uint16_t *)a.v_cache, n_old) + row * D;
    }
    bool store = true;
    if constexpr (Paged)  // an invalid page is not written (flag raised)
      store = __builtin_amdgcn_readlane(my_ok, page_slot(n_old)) != 0;
    if (store && w == 0 && lane < 32) {
      const int part = lane & 15;
      const int64_t src_off = ((int64_t)b * a.n_kv_heads + kvh) * D;
      const uint4 *src = (const uint4 *)((const uint16_t *)((lane < 16) ? a.k_new : a.v_new) +
                                         src_off) + part;
      uint4 *dst = (uint4 *)((lane < 16) ? kd : vd) + part;
      *dst = *src;
    }
    __syncthreads();  // workgroup scope: only this workgroup reads the row
  }
  const uint32_t slab_bytes = (uint32_t)(k_stop * D * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(kc, 0, slab_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(vc, 0, slab_bytes, kBufferWord3);

  // ---- query operand: Q^T (d on K, rows on N), affine + scale fused ------
  const float qscale = kLog2e * rsqrtf((float)D);
  bf16x8 qop[4];
  {
    const bool act = row_h >= 0;
    const uint16_t *qp = nullptr;
    const float *al = nullptr, *be = nullptr;
    if (act) {
      qp = (const uint16_t *)(row_s ? a.q[1] : a.q[0]) +
           (((int64_t)b * a.n_pos + row_j) * a.Hq + row_h) * D;
      al = (row_s ? a.alpha[1] : a.alpha[0]) + row_h * D;
      be = (row_s ? a.beta[1] : a.beta[0]) + row_h * D;
    }
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int d0 = 32 * c4 + 8 * g4;
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
        qop[c4][e] = (__bf16)((av[e] * qv + bv[e]) * qscale);
      }
    }
  }

  // ---- slice loads ---------------------------------------------------------
  // Slice `it` of this wave covers keys k_begin + 128 it + 32 w + [0, 32).
  const uint32_t k_lane = (uint32_t)col * (D * 2) + 16u * g4;
  const uint32_t v_lane = (uint32_t)g4 * (D * 2) + 16u * col;
  auto load = [&](Slice &sl, int it) {
    const int64_t key0 = k_begin + (int64_t)it * kStepKeys + kSlice * w;
    uint32_t base;
    __amdgpu_buffer_rsrc_t sk = rk, sv = rv;
    if constexpr (Paged) {
      // Resources over this slice's page, ending at the last valid key.
      const int64_t pkey0 = key0 & ~(int64_t)((1 << a.page_log2) - 1);
      const int64_t valid = min((int64_t)1 << a.page_log2, k_stop - pkey0);
      const uint32_t nbytes = valid > 0 ? (uint32_t)valid * (D * 2) : 0u;
      sk = __builtin_amdgcn_make_buffer_rsrc(
          page_base((uint16_t *)a.k_cache, key0), 0, nbytes, kBufferWord3);
      sv = __builtin_amdgcn_make_buffer_rsrc(
          page_base((uint16_t *)a.v_cache, key0), 0, nbytes, kBufferWord3);
      base = (uint32_t)(key0 - pkey0) * (D * 2);
    } else {
      base = (uint32_t)key0 * (D * 2);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        sl.k[kt][c4] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       sk, base + k_lane + 16u * (D * 2) * kt + 64u * c4, 0, 0));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      sl.v[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     sv, base + v_lane + 4u * (D * 2) * i, 0, 0));
  };

  // V^T transposed-read addresses: group g4 reads keys 4 g4.. (+16) and
  // channels 16 dt + (lane % 16).
  const int j16 = lane & 15;
  uint16_t(*vs)[kVS] = sm.st.v[w];
  const uint16_t *vtr0 = &vs[4 * g4 + (j16 >> 2)][4 * (j16 & 3)];

  float m = -INFINITY, l = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Slice &sl, int it) {
    // S^T tiles: lane holds keys 16 kt + 4 g4 + i of row `col`.
    f32x4 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, sl.k[kt][c4]), qop[c4], s[kt], 0, 0,
            0);
    }
    // V rows into this wave's LDS region.
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4 *)&vs[4 * i + g4][8 * col] = sl.v[i];

    // Mask to the row's key range, online softmax (base-2 domain).
    const int64_t kb = k_begin + (int64_t)it * kStepKeys + kSlice * w;
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = kb + 16 * kt + 4 * g4 + i;
        const bool ok = key >= r_lo && key <= r_hi;
        x[4 * kt + i] = ok ? s[kt][i] : -INFINITY;
        tmax = fmaxf(tmax, x[4 * kt + i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float ms = (m_new == -INFINITY) ? 0.0f : m_new;
    const float corr = __builtin_amdgcn_exp2f(m - ms);  // 0 while the row has seen no key
    bf16x8 pop;
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(x[e] - ms);
      pop[e] = pb;
      ps += (float)pb;
    }
    l = l * corr + ps;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] *= corr;

    wave_lds_fence();
    // O^T += V^T P^T: P^T holds keys {4g4..4g4+3} and {16+4g4..} of row col.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x4 lo4 = lds_read_tr(vtr0 + 16 * dt);
      const bf16x4 hi4 = lds_read_tr(vtr0 + 16 * kVS + 16 * dt);
      const bf16x8 vop = {lo4[0], lo4[1], lo4[2], lo4[3],
                          hi4[0], hi4[1], hi4[2], hi4[3]};
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, acc[dt], 0,
                                                         0, 0);
    }
    wave_lds_fence();  // the next slice's stores come after these reads
  };

  // The scheduling barriers keep each prefetch ahead of the wait for the
  // slice before it, so two slices are in flight while one is waited for.
  Slice s0, s1;
  load(s0, 0);
  for (int it = 0; it < n_steps; it += 2) {
    load(s1, it + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s0, it);
    load(s0, it + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < n_steps) compute(s1, it + 1);
  }

  // ---- merge the 4 waves --------------------------------------------------
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  __syncthreads();  // every wave is done with its V region (union below)
  if (g4 == 0) {
    sm.mg.m[w][col] = m;
    sm.mg.l[w][col] = l;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sm.mg.acc[w][col][16 * dt + 4 * g4 + i] = acc[dt][i];
  __syncthreads();

  // Rows r = tid / 32 (+ 8): lane tid % 32 of a half wave combines the 4
  // waves for channels 4 (tid % 32) .. + 3 and stores them (a whole 512-byte
  // row per half wave); lane 0 also stores the row's (max, sum).
  {
    const PartialView pv = partial_view(a, groups.n_groups, rows, b, gi);
    const int f = tid & 31;
    for (int r = tid >> 5; r < rows; r += 8) {
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.mg.m[ww][r]);
      float L = 0.0f;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float fw = exp2f(sm.mg.m[ww][r] - M);  // 0 for an empty wave
          L += fw * sm.mg.l[ww][r];
          o += fw * *(const f32x4 *)&sm.mg.acc[ww][r][4 * f];
        }
      }
      const int pi = c * rows + r;
      const u32x2 mlw = __builtin_bit_cast(u32x2, f32x2{M, L});
      const u32x4 ow = __builtin_bit_cast(u32x4, o);
      if (a.fused) {  // read back within this launch, by another XCD
        if (f == 0)
          __builtin_amdgcn_raw_buffer_store_b64(mlw, pv.ml, pi * 8, 0,
                                                kDeviceScope);
        __builtin_amdgcn_raw_buffer_store_b128(ow, pv.acc, pi * (D * 4) + f * 16,
                                               0, kDeviceScope);
      } else {  // read by the merge kernel, after the kernel boundary
        if (f == 0)
          __builtin_amdgcn_raw_buffer_store_b64(mlw, pv.ml, pi * 8, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(ow, pv.acc, pi * (D * 4) + f * 16,
                                               0, 0);
      }
    }
  }
  if (!a.fused) return;

  // ---- arrival; the last workgroup of (batch, group) merges ---------------
  // Chunks with work for this batch entry: those starting at or before its
  // last position (the others returned above and do not arrive). Every
  // thread's device-scope partial stores have completed before thread 0
  // counts the workgroup in, so the last arriver's device-scope loads see
  // every chunk's partials.
  const int used = (int)(hi_max / a.chunk) + 1;
  __shared__ int last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partials are out
  __syncthreads();
  if (tid == 0) {
    int32_t *cnt = a.counters + (int64_t)b * groups.n_groups + gi;
    last = atomicAdd(cnt, 1) == used - 1;
    if (last) atomicExch(cnt, 0);  // no other arrival is left in this call
  }
  __syncthreads();
  if (last) combine_group(a, groups, sm.cb, b, gi, pos_base);
  leave();
}

// Two-launch mode: one workgroup per (row, head group, batch), LANES chunk
// lanes of 256 / LANES threads. Thread (q, part): chunks c_lo + q,
// c_lo + q + LANES, ... and channels CH part .. CH part + CH - 1 (CH = D
// LANES / 256). Every load of a chunk is issued before its maximum is
// tested, so a row over up to LANES chunks costs one memory round trip; the
// lanes are then combined in LDS. 64 lanes serve rows over more than 32
// chunks; 16 lanes, with a quarter of the LDS and so more resident
// workgroups, serve a decode step's rows over a few.
template <int LANES>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(SplitKVArgs a,
                                                            HeadGroups groups) {
  constexpr int kParts = 256 / LANES, CH = D / kParts;
  __shared__ float sm_m[LANES], sm_l[LANES], sm_f[LANES];
  __shared__ float sm_sum;
  __shared__ float sm_acc[LANES][D + 4];
  const int r = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int gsize = groups.gsize;
  const int rows = a.n_streams * a.n_pos * gsize;
  const int s = r / (a.n_pos * gsize);
  const int j = (r / gsize) % a.n_pos;
  const int h = groups.q[gi][r % gsize];
  int64_t n_old = 0;
  if (a.cache_len) {
    n_old = a.ws_len[b];
    // a skipped entry: the split kernel wrote its zero rows
    if (n_old < 0) return;
  }
  // Decode: the cache now holds n_old + 1 rows for this batch entry. Every
  // split workgroup has finished reading (kernel boundary), and the merge
  // reads the old length from the workspace, so this write races with none.
  // Row 0 of group 0 always exists (its first query head).
  if (a.cache_len && r == 0 && gi == 0 && tid == 0)
    ((int32_t *)a.cache_len)[b] = (int32_t)(n_old + 1);
  if (h < 0) return;

  const int q = tid / kParts, part = tid % kParts, d0 = CH * part;
  float M = -INFINITY, L = 0.0f;
  f32x4 o[CH / 4];
#pragma unroll
  for (int k = 0; k < CH / 4; ++k) o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t t = (a.cache_len ? n_old : a.pos0) + j;
  const int Ws = a.W[s];
  const int64_t lo = (Ws > 0 && t - Ws + 1 > 0) ? t - Ws + 1 : 0;
  const int c_lo = (int)(lo / a.chunk), c_hi = (int)(t / a.chunk);
  for (int cc = c_lo + q; cc <= c_hi; cc += LANES) {
    const int64_t pi = ws_part_index(a, groups.n_groups, rows, b, gi, cc, r);
    const float mc = a.ws[pi * 2];
    const float lc = a.ws[pi * 2 + 1];
    const f32x4 *pacc =
        (const f32x4 *)(a.ws + (int64_t)a.ws_acc_offset + pi * D + d0);
    f32x4 u[CH / 4];
#pragma unroll
    for (int k = 0; k < CH / 4; ++k) u[k] = pacc[k];
    if (mc != -INFINITY) {  // a chunk with keys in this row's range
      const float Mn = fmaxf(M, mc);
      const float fo = exp2f(M - Mn), fn = exp2f(mc - Mn);
      L = L * fo + lc * fn;
#pragma unroll
      for (int k = 0; k < CH / 4; ++k) o[k] = o[k] * fo + u[k] * fn;
      M = Mn;
    }
  }
  if (part == 0) {
    sm_m[q] = M;
    sm_l[q] = L;
  }
#pragma unroll
  for (int k = 0; k < CH / 4; ++k) *(f32x4 *)&sm_acc[q][d0 + 4 * k] = o[k];
  __syncthreads();
  if (tid < LANES) {
    // the first LANES threads: the row maximum over the lanes, each lane's
    // weight, and the sum (xor shuffles within the LANES-wide group)
    const float mq = sm_m[tid];
    float Mx = mq;
#pragma unroll
    for (int sh = LANES / 2; sh >= 1; sh >>= 1)
      Mx = fmaxf(Mx, __shfl_xor(Mx, sh, 64));
    const float f = (mq == -INFINITY) ? 0.0f : exp2f(mq - Mx);
    sm_f[tid] = f;
    float lsum = f * sm_l[tid];
#pragma unroll
    for (int sh = LANES / 2; sh >= 1; sh >>= 1) lsum += __shfl_xor(lsum, sh, 64);
    if (tid == 0) sm_sum = lsum;
  }
  __syncthreads();
  if (tid < D / 2) {
    // thread tid: channels 2 tid, 2 tid + 1
    float out0 = 0.0f, out1 = 0.0f;
#pragma unroll 8
    for (int qq = 0; qq < LANES; ++qq) {
      const float f = sm_f[qq];
      const float2 v = *(const float2 *)&sm_acc[qq][2 * tid];
      out0 += f * v.x;
      out1 += f * v.y;
    }
    const float Lx = sm_sum;
    const float inv = Lx > 0.0f ? 1.0f / Lx : 0.0f;
    const uint32_t lo16 = __builtin_bit_cast(uint16_t, (__bf16)(out0 * inv));
    const uint32_t hi16 = __builtin_bit_cast(uint16_t, (__bf16)(out1 * inv));
    uint16_t *dst = (uint16_t *)a.o[s] +
                    (((int64_t)b * a.n_pos + j) * a.Hq + h) * D + 2 * tid;
    *(uint32_t *)dst = lo16 | (hi16 << 16);
  }
}

}  // namespace

hipError_t launch_splitkv(const SplitKVArgs &a, const HeadGroups &groups,
                          hipStream_t stream) {
  dim3 grid(a.n_chunks, groups.n_groups, a.B);
  if (a.block_table)
    hipLaunchKernelGGL(splitkv_kernel<true>, grid, dim3(kThreads), 0, stream,
                       a, groups);
  else
    hipLaunchKernelGGL(splitkv_kernel<false>, grid, dim3(kThreads), 0, stream,
                       a, groups);
  if (a.fused) return hipGetLastError();
  const int rows = a.n_streams * a.n_pos * groups.gsize;
  const dim3 mgrid(rows, groups.n_groups, a.B);
  if (a.n_chunks > 32)
    hipLaunchKernelGGL(splitkv_merge_kernel<64>, mgrid, dim3(256), 0, stream,
                       a, groups);
  else
    hipLaunchKernelGGL(splitkv_merge_kernel<16>, mgrid, dim3(256), 0, stream,
                       a, groups);
  return hipGetLastError();
}

}  // namespace orthros
