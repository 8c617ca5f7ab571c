// Persistent banded flash attention for the base stream (bf16, D = 128, 4
// query heads per KV head, bounded window).
//
// The same computation, MFMA layouts and per-tile step as the banded kernel
// (the o_t equation of "Orthros: Phase-Aware Heterogeneous Attention for
// Efficient Transformers", paper text §3.1; S^T = K Q^T and O^T += V^T P^T
// on v_mfma_f32_32x32x16_bf16, lazy base-2 softmax, K/V tiles of 64 keys
// double-buffered in LDS). What changes is the schedule around it. The
// banded kernel spends a fixed time per workgroup outside its tile loop: the
// launch of the next workgroup on the compute unit, the query load from
// HBM, the first tiles' round trip, and the output written as 8-byte pieces
// of 32 rows per instruction. Here a workgroup stays resident and walks 64-row
// query tiles ("items") of one (batch, KV head): tiles seg, seg + S, ...
// for S workgroups per (batch, KV head), all on one XCD, so that the S
// workgroups of a KV head work on neighbouring tiles whose bands share the
// XCD's L2. Per item:
//  * the query block (64 rows x 4 heads) was brought into LDS by direct
//    global-to-LDS loads (global_load_lds_dwordx4) issued early in the
//    previous item's tile loop;
//  * the first K/V tiles were requested before the previous item's output
//    was written;
//  * the tile loop is the banded kernel's;
//  * the output rows are normalised into LDS (over the free K/V buffers) and
//    written as whole 1 KB rows (four heads), one per store instruction.
#include "common.h"

namespace orthros {
namespace {

constexpr int D = 128;
constexpr int kRows = 32;          // query rows per wave
constexpr int kGs = 4;             // query heads per KV head
constexpr int kNW = 8;             // waves: 4 heads x 2 row blocks
constexpr int kNT = kNW * 64;
constexpr int kItemRows = kRows * kNW / kGs;   // 64 rows per item
constexpr int kBN = 64;            // keys per LDS tile
constexpr int kKS = D + 8;         // K tile row stride (bf16): 272 bytes
constexpr int kVS = D + 32;        // V tile row stride (bf16): 320 bytes
constexpr int kQS = kGs * D + 8;   // query / output block row stride (bf16)
constexpr int kBufferWord3 = 0x00020000;
constexpr float kTau = 8.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Tiles {
  uint16_t k[2][kBN][kKS];
  uint16_t v[2][kBN][kVS];
};
struct Smem {
  Tiles t;
  float ab[kGs][2][D];             // alpha, beta of the group's heads
};
// The next item's query block, and at the item's end its output block: a
// separate LDS object, so that the direct loads into it are not taken to
// alias the K/V tiles (no conservative waits before the tile reads).
struct QBlock {
  uint16_t qb[kItemRows][kQS];
};

// One direct global-to-LDS load of 16 bytes per lane: lane i's bytes land at
// LDS byte address lds_base + 16 i. Written as inline assembly so that the
// compiler's wait insertion does not treat every later LDS read as
// depending on it (the kernel waits for these loads itself, with vmcnt and
// a barrier, before reading the block). M0 is written here and read by
// nothing else in this kernel.
__device__ __forceinline__ void lds_dma16(const void *gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(gptr)
               : "memory");
}

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

// The lane id, recomputed where it is used: per-lane addresses needed only
// between items are rebuilt from it instead of being kept (or spilled)
// across the tile loop, which needs every VGPR.
__device__ __forceinline__ int fresh_lane() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0"
               : "=v"(ln));
  return ln;
}

__device__ __forceinline__ void wait_all_vm() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(kNT, 2) void band_persist_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ alpha,
    const float *__restrict__ beta, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, uint16_t *__restrict__ o,
    int nrows, int pos_off, int Hq, int n_kv, int64_t cap, int W, int n_qtiles,
    int n_segs, HeadGroups groups) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  __shared__ __attribute__((aligned(16))) QBlock qsm;
  typedef __attribute__((address_space(3))) void lds_void;

  // ---- workgroup -> (segment of items, head group, batch) -----------------
  // Workgroups are dealt to the 8 XCDs round-robin; when the number of
  // (batch, KV head) pairs is a multiple of 8, pair p runs on XCD p % 8.
  const int per = (int)(gridDim.x / n_segs);  // (batch, KV head) pairs
  int pair, seg;
  if (per % 8 == 0) {
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    seg = slot % n_segs;
    pair = xcd + 8 * (slot / n_segs);
  } else {
    seg = blockIdx.x % n_segs;
    pair = blockIdx.x / n_segs;
  }
  if (pair >= per || seg >= n_qtiles) return;
  const int gi = pair % groups.n_groups;
  const int b = pair / groups.n_groups;
  // items seg, seg + n_segs, ...: item number n is query tile seg + n n_segs
  const int n_last = (n_qtiles - 1 - seg) / n_segs;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hh = lane >> 5;
  const int kvh = groups.kv[gi];
  const int hs = w % kGs, ps = w / kGs;
  const int64_t head_off = ((int64_t)b * n_kv + kvh) * cap * D;

  // alpha / beta of the group's heads, times log2(e) / sqrt(D) (the
  // softmax runs in base 2)
  const float qs = kLog2e * rsqrtf((float)D);
  for (int i = tid; i < kGs * 2 * D; i += kNT) {
    const int s = i / (2 * D), which = (i / D) & 1, d = i % D;
    const int h = max((int)groups.q[gi][s], 0);
    sm.ab[s][which][d] = (which ? beta : alpha)[h * D + d] * qs;
  }

  // ---- query block in, output block out (LDS <-> HBM, whole rows) ---------
  // Wave w moves rows 8w .. 8w+7; lane i carries 16 bytes of head slot i/16
  // (a row of the four heads is 1 KB, contiguous when the heads are). Rows
  // past the end and padded head slots are loaded as copies of valid rows
  // (clamped) and never stored.
  const int gq0 = groups.q[gi][0], gq1 = groups.q[gi][1];
  const int gq2 = groups.q[gi][2], gq3 = groups.q[gi][3];
  auto slot_head_of = [&](int ln) __attribute__((always_inline)) {
    const int sl = ln >> 4;
    return sl == 0 ? gq0 : sl == 1 ? gq1 : sl == 2 ? gq2 : gq3;
  };
  auto load_qblock = [&](int qt) __attribute__((always_inline)) {
    const int ln = fresh_lane();
    const int hq = max(slot_head_of(ln), 0);
#pragma unroll
    for (int rr = 0; rr < kItemRows / kNW; ++rr) {
      const int row = (kItemRows / kNW) * w + rr;
      const int r = min(qt * kItemRows + row, nrows - 1);
      const uint16_t *src =
          q + (((int64_t)b * nrows + r) * Hq + hq) * D + 8 * (ln & 15);
      lds_dma16(src, __builtin_amdgcn_readfirstlane(
                         (uint32_t)(uintptr_t)(lds_void *)&qsm.qb[row][0]));
    }
  };
  // The output rows of item qt go through a buffer resource that covers just
  // the item's valid rows; padded head slots aim past its end. Out-of-range
  // stores are dropped by the hardware, so no lane branches, and all eight
  // rows are read from LDS before the first store (distinct registers: no
  // store waits on the one before it).
  auto store_oblock = [&](int qt) __attribute__((always_inline)) {
    const int ln = fresh_lane();
    const int sh = slot_head_of(ln);
    const uint32_t slot_off =
        sh >= 0 ? (uint32_t)(sh * D + 8 * (ln & 15)) * 2u : 0x80000000u;
    const int r0 = qt * kItemRows;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        o + ((int64_t)b * nrows + r0) * Hq * D, 0,
        (uint32_t)(min(kItemRows, nrows - r0) * Hq * D * 2), kBufferWord3);
    uint4 val[kItemRows / kNW];
#pragma unroll
    for (int rr = 0; rr < kItemRows / kNW; ++rr)
      val[rr] = *(const uint4 *)&qsm.qb[(kItemRows / kNW) * w + rr][8 * ln];
#pragma unroll
    for (int rr = 0; rr < kItemRows / kNW; ++rr) {
      const int row = (kItemRows / kNW) * w + rr;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, val[rr]), ro, slot_off,
          __builtin_amdgcn_readfirstlane(row * Hq * D * 2), 0);
    }
  };

  // ---- per-item geometry (uniform) ----------------------------------------
  struct Item {
    int qt, kt0, ntiles, wpos_lo, wpos_hi;
    __amdgpu_buffer_rsrc_t rk, rv;
  };
  auto item_of = [&](int n) __attribute__((always_inline)) {
    Item it;
    it.qt = seg + n * n_segs;
    // rows r0 .. r0 + 63 sit at positions pos_off + r0 ...
    const int r0 = it.qt * kItemRows;
    const int p0 = pos_off + r0;
    const int k_hi = pos_off + min(r0 + kItemRows, nrows) - 1;
    it.kt0 = max(0, p0 - W + 1) / kBN;
    it.ntiles = k_hi / kBN - it.kt0 + 1;
    it.wpos_lo = p0 + kRows * ps;
    it.wpos_hi = pos_off + min(r0 + kRows * ps + kRows, nrows) - 1;
    // Cache slab of this (batch, KV head), read through buffer resources
    // that end after key k_hi: tile rows past it load as zeros.
    const uint32_t slab_bytes = (uint32_t)(k_hi + 1) * (D * 2);
    it.rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(k_cache + head_off), 0, slab_bytes, kBufferWord3);
    it.rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(v_cache + head_off), 0, slab_bytes, kBufferWord3);
    return it;
  };

  // ---- tile staging: registers <-> LDS (16-byte chunks, natural layout) ----
  constexpr int kChunks = kBN * D / 8 / kNT;   // per thread, per tensor
  // A staging set holds K of one tile and V of the tile before it.
  struct Stage {
    uint4 k[kChunks], v[kChunks];
  };
  // (fresh: the lane's offsets rebuilt here, for the loads between items,
  // so that they are not kept or spilled across the tile loop)
  auto load_tile = [&](const Item &it, Stage &r, int kt, bool fresh = false)
      __attribute__((always_inline)) {
    const uint32_t k_off = (uint32_t)((it.kt0 + kt) * kBN) * (D * 2);
    const uint32_t v_off = k_off - (uint32_t)(kBN * D * 2);
    const int t_id = fresh ? 64 * w + fresh_lane() : tid;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const uint32_t off = 16u * (uint32_t)(t_id + kNT * i);
      r.k[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(it.rk, k_off + off, 0, 0));
      if (kt > 0)
        r.v[i] = __builtin_bit_cast(
            uint4,
            __builtin_amdgcn_raw_buffer_load_b128(it.rv, v_off + off, 0, 0));
    }
  };
  auto store_k = [&](const Stage &r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int idx = tid + kNT * i;
      *(uint4 *)&sm.t.k[buf][idx >> 4][8 * (idx & 15)] = r.k[i];
    }
  };
  auto store_v = [&](const Stage &r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int idx = tid + kNT * i;
      *(uint4 *)&sm.t.v[buf][idx >> 4][8 * (idx & 15)] = r.v[i];
    }
  };
  // Transposed-read addresses of the V^T operand: lane group g16 covers
  // channels 16*(g16 % 2) (+32 dt) and key half hh = g16 / 2.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row0 = 4 * hh + (j16 >> 2);          // + 16 kg (+ 8 second read)
  const int v_col0 = 16 * (g16 & 1) + 4 * (j16 & 3);  // + 32 dt

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // ---- query operand from the block in LDS (B of S^T) ----------------------
  bf16x8 qop[8];
  auto make_qop = [&]() __attribute__((always_inline)) {
      const int ln = fresh_lane();
      const uint16_t *qrow = &qsm.qb[kRows * ps + (ln & 31)][hs * D];
      const float *al = sm.ab[hs][0];
      const float *be = sm.ab[hs][1];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int d0 = 16 * c + 8 * (ln >> 5);
        const uint4 raw = *(const uint4 *)(qrow + d0);
        const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qv = bf16_bits_to_f32((e & 1) ? (wv[e >> 1] >> 16)
                                                    : (wv[e >> 1] & 0xffffu));
          qop[c][e] = (__bf16)(al[d0 + e] * qv + be[d0 + e]);
        }
      }
  };

  // Prologue: the first item's query block and operand.
  load_qblock(seg);
  wait_all_vm();
  __syncthreads();  // query block, alpha / beta
  make_qop();

  Item cur = item_of(0);
  Stage ra, rb;
  load_tile(cur, rb, 0);
  load_tile(cur, ra, 1);

  for (int n = 0; n <= n_last; ++n) {
    const int kt0 = cur.kt0;
    const int ntiles = cur.ntiles;
    const int wpos_lo = cur.wpos_lo, wpos_hi = cur.wpos_hi;
    const int tq = wpos_lo + (fresh_lane() & 31);  // this lane's position

    float m = -INFINITY;
    // the lazy-rescale threshold on the tile maximum (relative to m):
    // -inf while this row has seen no key, then kTau
    float thr = -INFINITY;
    // row-sum partials, one per 16-key group: four short dependency chains
    float l4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x16 acc[4], negm;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) negm[v] = 0.0f;

    // S^T - m of one tile: keys of K buffer `kbuf`, seeded with the current -m.
    auto scores = [&](f32x16 (&sn)[2], int kbuf) __attribute__((always_inline)) {
      sn[0] = negm;
      sn[1] = negm;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int sk = 0; sk < 2; ++sk) {
          const bf16x8 kop =
              *(const bf16x8 *)&sm.t.k[kbuf][32 * sk + j][16 * c + 8 * hh];
          sn[sk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[c], sn[sk],
                                                           0, 0, 0);
        }
    };
    // Row maximum of this lane's 32 scores (four independent chains), and
    // the maximum across the lane pair.
    auto tile_max = [&](const f32x16 (&sn)[2]) __attribute__((always_inline)) {
      float t4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t4[c] = -INFINITY;
#pragma unroll
        for (int v = 0; v < 8; ++v)
          t4[c] = fmaxf(t4[c], sn[c >> 1][8 * (c & 1) + v]);
      }
      return max_xor32(fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3])));
    };
    // Band mask (only tiles crossing a band edge of some row of this wave)
    // and the lazy move of the reference maximum. tmax is the tile's
    // maximum over all its keys, taken before the mask; a masked tile takes
    // it again. The tile offset is a 32-bit uniform value, so the band test
    // is scalar.
    // (first: the item's first tile; the accumulators and row sums are
    // still zero, so nothing is rescaled)
    auto settle = [&](f32x16 (&sn)[2], int kb, float tmax, bool first = false)
        __attribute__((always_inline)) {
      const bool inside = kb >= wpos_hi - W + 1 && kb + kBN - 1 <= wpos_lo;
      if (!inside) {
        const int d0 = (int)(kb - tq);
#pragma unroll
        for (int sk = 0; sk < 2; ++sk)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int d = d0 + 32 * sk + 8 * (v >> 2) + 4 * hh + (v & 3);
            sn[sk][v] = (d > 0 || d <= -W) ? -INFINITY : sn[sk][v];
          }
        tmax = tile_max(sn);  // the maximum over the keys in range
      }
      const bool need = tmax > thr;
      if (__any(need)) {
        const float shift = need ? tmax : 0.0f;
        const float corr =
            need ? ((m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(-shift))
                 : 1.0f;
        m = need ? ((m == -INFINITY) ? shift : m + shift) : m;
        if (!first) {
#pragma unroll
          for (int c = 0; c < 4; ++c) l4[c] *= corr;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) acc[dt] *= corr;
        }
#pragma unroll
        for (int sk = 0; sk < 2; ++sk) sn[sk] -= shift;
        const float nm = (m == -INFINITY) ? 0.0f : -m;
        thr = (m == -INFINITY) ? -INFINITY : kTau;
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[v] = nm;
      }
    };

    // Tiles 0 and 1 (K) and 0 (V) were requested already; K of tile 2 and V
    // of tile 1 stay in flight through step 0.
    store_k(rb, 0);
    store_k(ra, 1);
    store_v(ra, 0);
    load_tile(cur, ra, 2, true);
    __syncthreads();  // tiles in LDS; the last item's output block read
    // The next item's query block: issued at the start of the second loop
    // iteration when there is one (its address work then overlaps the
    // step's MFMAs, and it is older than that step's tile loads, whose wait
    // gives it a whole step), else here.
    const bool q_in_loop = ntiles >= 4;
    if (n < n_last && !q_in_loop) load_qblock(seg + (n + 1) * n_segs);
    f32x16 sa[2], sb[2];
    scores(sa, 0);
    settle(sa, kt0 * kBN, tile_max(sa), true);
    __syncthreads();  // K buffer 0 is refilled at the end of step 0

    // Software pipeline, one 64-key tile per step (the banded kernel's).
    auto step = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], Stage &r_in,
                    Stage &r_out, int it, bool fresh = false)
        __attribute__((always_inline)) {
      const int kb = (kt0 + it) * kBN;
      load_tile(cur, r_out, it + 3, fresh);  // stored at the end of the next step
      scores(sn, (it + 1) & 1);
      bf16x8 pop[4];
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pop[kg][e] =
              (__bf16)__builtin_amdgcn_exp2f(sc[kg >> 1][8 * (kg & 1) + e]);
        // row sum of the same bf16 probabilities, from the packed operand
        // words (through scalars: a bit cast of a vector element reads
        // element 0)
        const u32x4 pw = __builtin_bit_cast(u32x4, pop[kg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w2 = pw[e];
          l4[kg] = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2, w2), ones, l4[kg], false);
        }
      }
      const int vb = it & 1;
      // the next tile's maximum over all its keys, between the P V MFMAs
      // (edge tiles mask and take it again in the settle)
      const float tmax_next = tile_max(sn);
#pragma unroll
      for (int kg = 0; kg < 4; ++kg)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int row = 16 * kg + v_row0;
          const int col = 32 * dt + v_col0;
          const bf16x4 lo4 = lds_read_tr(&sm.t.v[vb][row][col]);
          const bf16x4 hi4 = lds_read_tr(&sm.t.v[vb][row + 8][col]);
          const bf16x8 vop = {lo4[0], lo4[1], lo4[2], lo4[3],
                              hi4[0], hi4[1], hi4[2], hi4[3]};
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[kg],
                                                            acc[dt], 0, 0, 0);
        }
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
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // the maximum
      }
      settle(sn, kb + kBN, tmax_next);
      store_k(r_in, it & 1);     // K of tile it+2
      store_v(r_in, vb ^ 1);     // V of tile it+1
      // All but this step's four tile loads are complete (the counter
      // retires in order): in particular the next item's query block, if it
      // was issued before them, so that after this barrier it is visible.
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
      __syncthreads();
    };
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
      if (it == 2 && q_in_loop && n < n_last)
        load_qblock(seg + (n + 1) * n_segs);
      step(sa, sb, ra, rb, it);
      step(sb, sa, rb, ra, it + 1);
    }
    if (it < ntiles) step(sa, sb, ra, rb, it, true);

    // ---- item end ----------------------------------------------------------
    // The next query block is complete and visible (issued before a step
    // whose wait covers it, and that step's barrier). Request the next
    // item's first tiles, take its query operand, then normalise this
    // item's rows into the query block over the slots this wave has just
    // read (no other wave reads them) and write the block out as whole
    // rows.
    const int qt = cur.qt;
    if (n < n_last) {
      cur = item_of(n + 1);
      load_tile(cur, rb, 0, true);
      load_tile(cur, ra, 1, true);
      make_qop();
    }
    {
      const float l = (l4[0] + l4[1]) + (l4[2] + l4[3]);
      // row sum: this lane's half plus its partner's (lane ^ 32)
      const auto lp = __builtin_amdgcn_permlane32_swap(
          __float_as_uint(l), __float_as_uint(l), false, false);
      const float inv =
          1.0f / (__uint_as_float(lp[0]) + __uint_as_float(lp[1]));
      const int ln = fresh_lane();
      uint16_t *orow = &qsm.qb[kRows * ps + (ln & 31)][hs * D];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * dt + 8 * q4 + 4 * (ln >> 5);
          uint32_t pk[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t lo = __builtin_bit_cast(
                uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e] * inv));
            const uint32_t hi = __builtin_bit_cast(
                uint16_t, (__bf16)(acc[dt][4 * q4 + 2 * e + 1] * inv));
            pk[e] = lo | (hi << 16);
          }
          *(uint2 *)(orow + d0) = make_uint2(pk[0], pk[1]);
        }
    }
    __syncthreads();  // output block complete
    store_oblock(qt);
  }
}

}  // namespace

// Workgroups of the persistent kernel: about one per compute unit, each on
// every n_segs-th query tile of one (batch, KV head). W <= 0: every key up
// to the row's position.
hipError_t launch_band_persist(const void *q, const float *alpha,
                               const float *beta, const void *k_cache,
                               const void *v_cache, void *o, int B, int nrows,
                               int pos_off, int Hq, int64_t cap, int W,
                               const HeadGroups &groups, int n_kv,
                               hipStream_t stream) {
  if (W <= 0) W = pos_off + nrows;
  const int n_qtiles = (nrows + kItemRows - 1) / kItemRows;
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t per = (int64_t)groups.n_groups * B;
  int64_t n_segs = (n_cu > 0 ? n_cu : 256) / per;
  if (n_segs < 1) n_segs = 1;
  if (n_segs > n_qtiles) n_segs = n_qtiles;
  hipLaunchKernelGGL(band_persist_kernel, dim3((unsigned)(n_segs * per)),
                     dim3(kNT), 0, stream, (const uint16_t *)q, alpha, beta,
                     (const uint16_t *)k_cache, (const uint16_t *)v_cache,
                     (uint16_t *)o, nrows, pos_off, Hq, n_kv, cap, W, n_qtiles,
                     (int)n_segs, groups);
  return hipGetLastError();
}

}  // namespace orthros
