// Training backward of Orthros attention on gfx950 MFMA (bf16, D = 128).
//
// Pages: "Orthros: Phase-Aware Heterogeneous Attention for Efficient
// Transformers", paper text §3.1 (the o_t and o'_t equations and the query
// scale-offset) and §3.2 (pre-training duplicates every position as an
// output row; SFT the response positions), which is where gradients of both
// streams are needed. The gradients follow the chain rule through one
// softmax row: with p = softmax(s), s_j = q.k_j / sqrt(D),
//   dp_j = dO . v_j,  ds_j = p_j (dp_j - dO . o),  dq = sum_j ds_j k_j / sqrt(D),
//   dk_j += ds_j q / sqrt(D),  dv_j += p_j dO,
// then dq_pre = alpha (.) dq, d alpha = sum dq (.) q_pre, d beta = sum dq.
//
// Three kernels, each in the layouts of v_mfma_f32_16x16x32_bf16 (lane
// (col = lane % 16, g4 = lane / 16); A rows and B columns on col, the
// 32-wide contraction split 8 per g4; C holds rows 4 g4 .. 4 g4 + 3 of
// column col):
//  * bwd_dq_kernel (per stream): 8 waves, each 32 query rows of one head.
//    One pass over the band's 64-key tiles forms S^T = K Q^T and
//    dP^T = V dO^T, dS^T against a reference row maximum, and
//    dQ^T += K^T dS^T (K^T read with ds_read_b64_tr_b16), rescaled when a
//    tile's maximum passes the reference by more than 2^8 (then the
//    reference moves) and divided by the row sum at the end. It writes
//    dq_pre, the row's log-sum-exp and dO . o, per 32-row block the
//    channel sums that make d alpha and d beta, and the query operand it
//    formed (bf16 of the scaled alpha q + beta) for the dK/dV kernel.
//  * bwd_dkv_kernel (both streams): 8 waves, each 16 keys of one KV head,
//    over every query head of that KV head and every 64-row block of either
//    stream that sees the keys (16-row quarters outside a wave's band are
//    skipped): S = Q K^T and dP = dO V^T with K, V held in
//    registers, then dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read
//    transposed from LDS. Q comes ready-made from the dQ kernels.
//  * bwd_reduce_kernel: the per-block channel sums, added in a fixed order.
// All softmax arithmetic is fp32 in base 2 (log2(e)/sqrt(D) folded into the
// query operand, as in the forward kernels); P and dS enter the MFMA as bf16.
#include "common.h"

namespace orthros {
namespace {

constexpr int D = 128;
constexpr int kS = D + 16;  // LDS row stride (bf16): 288 bytes
constexpr int kBufferWord3 = 0x00020000;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b,
                                        const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

// 16-byte row chunk `c4` for lane group g4 of row `row` (A/B operand rows).
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t (*t)[kS], int row,
                                           int c4, int g4) {
  return *(const bf16x8 *)&t[row][32 * c4 + 8 * g4];
}

// Transposed operand (16 channels x 32 rows of the tile, rows in the order
// the packed C fragments use): rows 4 g4 + (j16 / 4) (+16), channels
// 16 dt + 4 (j16 % 4).
__device__ __forceinline__ bf16x8 lds_tr8(const uint16_t (*t)[kS], int row0,
                                          int g4, int j16, int dt) {
  const uint16_t *p = &t[row0 + 4 * g4 + (j16 >> 2)][16 * dt + 4 * (j16 & 3)];
  const bf16x4 lo4 = lds_read_tr(p);
  const bf16x4 hi4 = lds_read_tr(p + 16 * kS);
  return bf16x8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return bf16_bits_to_f32(w & 0xffffu); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bf16_bits_to_f32(w >> 16); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// Sum over the 16 lanes of a row (lanes 16 k .. 16 k + 15), left in every
// one of them: four DPP adds (pairs, then quads, then the two halves by
// mirroring), no LDS permutes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

// Block -> (unit, (batch, head group) pair). Workgroups are dealt to the
// 8 XCDs by block id; when the pairs are a multiple of 8, pair p's units
// (row tiles or key blocks) all run on XCD p % 8, so the rows they share
// (K/V bands, Q/dO blocks) are re-read from that XCD's L2, not from HBM.
__device__ __forceinline__ void xcd_unit(int n_units, int &unit, int &pair) {
  const int n_pairs = (int)(gridDim.x / (unsigned)n_units);
  if (n_pairs % 8 == 0) {
    const int xcd = (int)(blockIdx.x % 8u), slot = (int)(blockIdx.x / 8u);
    unit = slot % n_units;
    pair = xcd + 8 * (slot / n_units);
  } else {
    unit = (int)(blockIdx.x % (unsigned)n_units);
    pair = (int)(blockIdx.x / (unsigned)n_units);
  }
}

// First key of row position p's range (W >= p + 1 means the whole prefix).
__device__ __forceinline__ int range_lo(int p, int W) {
  return p >= W ? p - W + 1 : 0;
}

// ============================================================================
// dQ (and the row statistics) of one stream
// ============================================================================
template <int GS>
struct DqSmem {
  uint16_t k[64][kS];
  uint16_t v[64][kS];
  float ab[GS][2][D];
};

template <int GS>
__global__ __launch_bounds__(512, 2) void bwd_dq_kernel(BwdStreamArgs a,
                                                        HeadGroups groups) {
  constexpr int kRowsWg = 32 * (8 / GS);
  __shared__ __attribute__((aligned(16))) DqSmem<GS> sm;
  const int n_wg_rows = (a.nrows + kRowsWg - 1) / kRowsWg;
  int wr, rest;
  xcd_unit(n_wg_rows, wr, rest);
  // a row tile's band never shrinks with its index (the window's start,
  // or the prefix of an unbounded window): the longest tiles start first
  wr = n_wg_rows - 1 - wr;
  const int gi = rest % groups.n_groups;
  const int b = rest / groups.n_groups;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4;
  const int hs = w % GS, rb = w / GS;
  const int head = groups.q[gi][hs];
  const int kvh = groups.kv[gi];
  const float qs = kLog2e * rsqrtf((float)D);

  for (int i = tid; i < GS * 2 * D; i += 512) {
    const int s = i / (2 * D), which = (i / D) & 1, d = i % D;
    const int h = max((int)groups.q[gi][s], 0);
    sm.ab[s][which][d] = (which ? a.beta : a.alpha)[h * D + d] * qs;
  }

  // rows of this wave: r0 + 16 h2 + col (h2 = 0, 1)
  const int r_wg = wr * kRowsWg;
  const int r0 = r_wg + 32 * rb;
  const int p_wg_first = a.q_offset + r_wg;
  const int p_wg_last = a.q_offset + min(r_wg + kRowsWg, a.nrows) - 1;
  const int lo_wg = range_lo(p_wg_first, a.W);
  const int hi_wg = min(p_wg_last, a.n_keys - 1);
  const int kt_lo = lo_wg / 64, kt_hi = hi_wg / 64;
  const bool wave_on = head >= 0 && r0 < a.nrows;
  const int p_w_first = a.q_offset + r0;
  const int p_w_last = a.q_offset + min(r0 + 32, a.nrows) - 1;
  const int lo_w = range_lo(p_w_first, a.W);

  // per-lane row operands (rows past the end re-read the last row)
  const int hq = max(head, 0);
  int prow[2];
  bool row_ok[2];
  bf16x8 qop[2][4], doop[2][4];
  float delta[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int r = r0 + 16 * h2 + col;
    row_ok[h2] = wave_on && r < a.nrows;
    prow[h2] = a.q_offset + r;
    const int rc = min(r, a.nrows - 1);
    const int64_t off = (((int64_t)b * a.nrows + rc) * a.Hq + hq) * D;
    float dsum = 0.0f;  // dO . o over this lane's 32 channels
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int d0 = 32 * c4 + 8 * g4;
      const uint4 oraw = *(const uint4 *)(a.o + off + d0);
      const uint4 graw = *(const uint4 *)(a.d_o + off + d0);
      doop[h2][c4] = as_bf16x8(graw);
      const uint32_t ow[4] = {oraw.x, oraw.y, oraw.z, oraw.w};
      const uint32_t gw[4] = {graw.x, graw.y, graw.z, graw.w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        dsum += bf16_lo(gw[e2]) * bf16_lo(ow[e2]) + bf16_hi(gw[e2]) * bf16_hi(ow[e2]);
    }
    dsum += __shfl_xor(dsum, 16, 64);
    dsum += __shfl_xor(dsum, 32, 64);
    delta[h2] = dsum;
  }

  // K/V tile staging: 2 x 16 bytes of K and of V per thread
  const int64_t slab = ((int64_t)b * a.n_kv + kvh) * a.cap * D;
  const uint32_t slab_bytes = (uint32_t)a.n_keys * (D * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.k_cache + slab), 0, slab_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(a.v_cache + slab), 0, slab_bytes, kBufferWord3);
  uint4 kst[2], vst[2];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = (uint32_t)kt * (64 * D * 2) + 16u * (uint32_t)(tid + 512 * i);
      kst[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      vst[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i;
      *(uint4 *)&sm.k[idx >> 4][8 * (idx & 15)] = kst[i];
      *(uint4 *)&sm.v[idx >> 4][8 * (idx & 15)] = vst[i];
    }
  };
  load(kt_lo);
  __syncthreads();  // alpha/beta table

  // query operand: bf16(alpha' q + beta') with the base-2 scale folded in
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int rc = min(r0 + 16 * h2 + col, a.nrows - 1);
    const int64_t off = (((int64_t)b * a.nrows + rc) * a.Hq + hq) * D;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int d0 = 32 * c4 + 8 * g4;
      const uint4 qraw = *(const uint4 *)(a.q + off + d0);
      const uint32_t qw[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = (e & 1) ? bf16_hi(qw[e >> 1]) : bf16_lo(qw[e >> 1]);
        qop[h2][c4][e] = (__bf16)(sm.ab[hs][0][d0 + e] * qv + sm.ab[hs][1][d0 + e]);
      }
      // the dK/dV kernel reads these operands rather than forming them again
      if (row_ok[h2])
        *(uint4 *)(a.qa + off + d0) = __builtin_bit_cast(uint4, qop[h2][c4]);
    }
  }

  // S^T block (16 keys of sub-block kb x 16 rows of half h2) minus the
  // row's reference maximum (the accumulator starts at -m)
  float negm[2] = {0.0f, 0.0f};
  auto scores_raw = [&](int kb, int h2) {
    f32x4 s = {negm[h2], negm[h2], negm[h2], negm[h2]};
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      s = mfma16(lds_row8(sm.k, 16 * kb + col, c4, g4), qop[h2][c4], s);
    return s;
  };
  // key kept iff lo <= key <= p, i.e. (unsigned)(key - lo) <= p - lo
  auto mask = [&](f32x4 &s, int kt, int kb, int h2) {
    const int lo = range_lo(prow[h2], a.W);
    const uint32_t u0 = (uint32_t)(kt * 64 + 16 * kb + 4 * g4 - lo);
    const uint32_t span = (uint32_t)(prow[h2] - lo);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (u0 + i <= span) ? s[i] : -INFINITY;
  };
  // tile inside every row's range of this wave (valid rows only): no mask
  const int p_w_valid_last = p_w_last;
  auto tile_inside = [&](int kt) {
    return kt * 64 >= range_lo(p_w_valid_last, a.W) && kt * 64 + 63 <= p_w_first &&
           r0 + 32 <= a.nrows;
  };

  // m: the reference maximum, moved only when a tile's maximum exceeds it
  // by more than kTau (then acc and l are rescaled); thr: -inf while the
  // row has seen no key, then kTau
  constexpr float kTau = 8.0f;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
  float thr[2] = {-INFINITY, -INFINITY};
  float lse[2] = {0.0f, 0.0f};
  f32x4 acc[2][8];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[h2][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int j16 = col;

  auto next_tile = [&](int kt) {
    __syncthreads();  // the previous tile's readers are done
    store();
    __syncthreads();
    (void)kt;
  };
  auto wave_needs = [&](int kt) {
    const int k_first = kt * 64, k_last = k_first + 63;
    return wave_on && k_last >= lo_w && k_first <= p_w_last;
  };

  // ---- one pass: S^T, dP^T, dS^T and dQ^T against a reference maximum ------
  // dQ = sum_j p_j (dp_j - delta) k_j with p_j = 2^(s_j - lse). With a
  // reference maximum m and the sum l of the keys seen so far, the pass
  // accumulates acc = sum_j 2^(s_j - m) (dp_j - delta) k_j and divides by l
  // at the end; lse = m + log2(l) comes out of the same pass. As in the
  // forward kernels m moves (and acc and l are rescaled) only when a tile's
  // maximum exceeds it by more than kTau, so the exponents stay <= kTau;
  // the score and dP accumulators start at -m and -delta, so neither
  // needs a subtraction per element.
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    next_tile(kt);
    if (kt < kt_hi) load(kt + 1);
    if (!wave_needs(kt)) continue;
    const bool inside = tile_inside(kt);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x4 sv[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sv[kb] = scores_raw(kb, h2);
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (!inside)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mask(sv[kb], kt, kb, h2);
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sv[kb][i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const bool need = tmax > thr[h2];
      if (__any(need)) {
        const float shift = need ? tmax : 0.0f;
        // 0 while the row has seen no key (acc and l are still zero)
        const float corr =
            need ? ((m[h2] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(-shift))
                 : 1.0f;
        m[h2] = need ? ((m[h2] == -INFINITY) ? shift : m[h2] + shift) : m[h2];
        l[h2] *= corr;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[h2][dt] *= corr;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sv[kb] -= shift;
        negm[h2] = (m[h2] == -INFINITY) ? 0.0f : -m[h2];
        thr[h2] = (m[h2] == -INFINITY) ? -INFINITY : kTau;
      }
      float ps = 0.0f;
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
        f32x4 dp[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kb = 2 * kp + half;
          // dP - delta: the accumulator starts at -delta (the row's dO . o)
          dp[half] = f32x4{-delta[h2], -delta[h2], -delta[h2], -delta[h2]};
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4)
            dp[half] = mfma16(lds_row8(sm.v, 16 * kb + col, c4, g4), doop[h2][c4], dp[half]);
        }
        bf16x8 dsop;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // masked keys give 2^(-inf) = 0
            const float pt = __builtin_amdgcn_exp2f(sv[2 * kp + half][i]);
            ps += pt;
            dsop[4 * half + i] = (__bf16)(pt * dp[half][i]);
          }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          acc[h2][dt] = mfma16(lds_tr8(sm.k, 32 * kp, g4, j16, dt), dsop, acc[h2][dt]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l[h2] += ps;
    }
  }
  // row sums over the four lane groups, log-sum-exp (base 2), 1 / l
  float inv_l[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    float lt = l[h2];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    lse[h2] = m[h2] + __log2f(lt);
    inv_l[h2] = lt > 0.0f ? 1.0f / lt : 0.0f;
  }

  // ---- outputs ---------------------------------------------------------------
  if (!wave_on) return;
  const float inv_sqrt_d = rsqrtf((float)D);
  float sa[8][4], sb[8][4];  // channel sums over this wave's rows
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[dt][i] = sb[dt][i] = 0.0f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int r = r0 + 16 * h2 + col;
    const int rc = min(r, a.nrows - 1);
    const int64_t off = (((int64_t)b * a.nrows + rc) * a.Hq + hq) * D;

#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d0 = 16 * dt + 4 * g4;
      const uint2 qraw = *(const uint2 *)(a.q + off + d0);
      const float qv[4] = {bf16_lo(qraw.x), bf16_hi(qraw.x), bf16_lo(qraw.y),
                           bf16_hi(qraw.y)};
      const float4 al = *(const float4 *)(a.alpha + hq * D + d0);
      const float alv[4] = {al.x, al.y, al.z, al.w};
      float g[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dq = row_ok[h2] ? acc[h2][dt][i] * (inv_l[h2] * inv_sqrt_d) : 0.0f;
        g[i] = alv[i] * dq;
        sa[dt][i] += dq * qv[i];
        sb[dt][i] += dq;
      }
      if (row_ok[h2])
        *(uint2 *)(a.dq + off + d0) = make_uint2(pack2(g[0], g[1]), pack2(g[2], g[3]));
    }
    if (g4 == 0 && row_ok[h2]) {
      const int64_t si = ((int64_t)b * a.Hq + head) * a.nrows + r;
      a.lse[si] = lse[h2];
      a.delta[si] = delta[h2];
    }
  }
  // sum over the 16 rows of a lane group (h2 already folded in)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[dt][i] = sum16(sa[dt][i]);
      sb[dt][i] = sum16(sb[dt][i]);
    }
  if (col == 0) {
    const int n_rb = (a.nrows + 31) / 32;
    const int rbg = r0 / 32;
    float *pa = a.part + ((((int64_t)b * n_rb + rbg) * a.Hq + head) * 2) * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d0 = 16 * dt + 4 * g4;
      *(float4 *)(pa + d0) = make_float4(sa[dt][0], sa[dt][1], sa[dt][2], sa[dt][3]);
      *(float4 *)(pa + D + d0) = make_float4(sb[dt][0], sb[dt][1], sb[dt][2], sb[dt][3]);
    }
  }
}

// ============================================================================
// dK, dV of one KV head and 64 keys, over both streams
// ============================================================================
template <int GS>
struct DkvSmem {
  uint16_t q[64][kS];
  uint16_t g[64][kS];
  float lse[64], delta[64];
};

constexpr int kKvWaves = 8;                 // 16 keys each
constexpr int kKvKeys = 16 * kKvWaves;      // keys per workgroup
constexpr int kKvThreads = 64 * kKvWaves;

template <int GS>
__global__ __launch_bounds__(kKvThreads, 2) void bwd_dkv_kernel(
    BwdKvArgs a, HeadGroups groups) {
  __shared__ __attribute__((aligned(16))) DkvSmem<GS> sm;
  const int n_kt = (a.T + kKvKeys - 1) / kKvKeys;
  int kt, rest;
  xcd_unit(n_kt, kt, rest);
  const int gi = rest % groups.n_groups;  // the one group of this KV head
  const int b = rest / groups.n_groups;
  const int kvh = groups.kv[gi];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4, j16 = col;
  const int k0 = kt * kKvKeys;
  const int kw = k0 + 16 * w;          // first key of this wave
  const int key = kw + col;            // this lane's key (B columns)

  // K and V rows of this wave's keys as B operands (channels 32 c4 + 8 g4)
  bf16x8 kop[4], vop[4];
  {
    const int kc = min(key, a.T - 1);
    const int64_t off = (((int64_t)b * a.n_kv + kvh) * a.cap + kc) * D;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      kop[c4] = as_bf16x8(*(const uint4 *)(a.k_cache + off + 32 * c4 + 8 * g4));
      vop[c4] = as_bf16x8(*(const uint4 *)(a.v_cache + off + 32 * c4 + 8 * g4));
    }
  }
  f32x4 dk[8], dv[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dk[dt] = dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Work list: (query head of this KV head) x (stream) x (64-row block).
  const int T_in = a.T - a.T_out;
  const int base_lo = k0 / 64;
  const int base_hi = min(a.T - 1, k0 + kKvKeys - 1 + a.W - 1) / 64;  // W <= T
  const int n_base = base_hi - base_lo + 1;
  int out_lo = 0, n_out = 0;
  if (a.T_out > 0) {
    out_lo = max(0, k0 - T_in) / 64;
    n_out = max(0, (a.T_out - 1) / 64 - out_lo + 1);
  }
  const int per_head = n_base + n_out;
  const GroupHeads gh = group_heads(groups, gi);
  int n_heads = 0;  // the group's slots up to the first empty one
  while (n_heads < GS && slot_head(gh, n_heads) >= 0) ++n_heads;
  const int n_it = n_heads * per_head;

  struct Item { int hi, s, qb; };
  // Work-list cursor (item index, head slot, index within the head's
  // items), advanced one item at a time and held at the last item, so that
  // no item number is ever divided.
  struct Cur { int it, hi, rr; };
  auto adv = [&](Cur c) {
    if (c.it + 1 < n_it) {
      ++c.it;
      if (++c.rr == per_head) {
        c.rr = 0;
        ++c.hi;
      }
    }
    return c;
  };
  auto decode = [&](Cur c) {
    const int s = c.rr >= n_base;
    return Item{c.hi, s, s ? out_lo + (c.rr - n_base) : base_lo + c.rr};
  };

  // staging: thread -> rows tid/16 + 32 u (u = 0, 1), one 16-byte chunk;
  // two register sets, so each block's loads are issued two blocks ahead
  const int srow = tid >> 4, sd0 = 8 * (tid & 15);
  struct Stage {
    uint4 q0, q1, g0, g1;
    float lse, delta;
  };
  auto load = [&](Stage &st, Cur cu) {
    const Item itm = decode(cu);
    const int h = slot_head(gh, itm.hi);
    const int nrows = itm.s ? a.T_out : a.T;
    const uint16_t *qsrc = itm.s ? a.qax : a.qa;
    const uint16_t *gsrc = itm.s ? a.d_ox : a.d_o;
    auto off = [&](int u) {
      const int r = min(itm.qb * 64 + srow + 16 * u, nrows - 1);
      return (((int64_t)b * nrows + r) * a.Hq + h) * D + sd0;
    };
    const int64_t o0 = off(0), o1 = off(2);
    st.q0 = *(const uint4 *)(qsrc + o0);
    st.q1 = *(const uint4 *)(qsrc + o1);
    st.g0 = *(const uint4 *)(gsrc + o0);
    st.g1 = *(const uint4 *)(gsrc + o1);
    // every thread loads (only the first 64 store): the same loads on
    // every path keep the waits before the LDS stores exact
    const int r = min(itm.qb * 64 + (tid & 63), nrows - 1);
    const int64_t si = ((int64_t)b * a.Hq + h) * nrows + r;
    st.lse = (itm.s ? a.lse_x : a.lse)[si];
    st.delta = (itm.s ? a.delta_x : a.delta)[si];
  };
  auto store = [&](const Stage &st) {
    // element-wise copies: a whole-struct copy made the compiler keep the
    // staging sets in scratch memory
    *(uint4 *)&sm.q[srow][sd0] = make_uint4(st.q0.x, st.q0.y, st.q0.z, st.q0.w);
    *(uint4 *)&sm.q[srow + 32][sd0] = make_uint4(st.q1.x, st.q1.y, st.q1.z, st.q1.w);
    *(uint4 *)&sm.g[srow][sd0] = st.g0;
    *(uint4 *)&sm.g[srow + 32][sd0] = st.g1;
    if (tid < 64) {
      sm.lse[tid] = st.lse;
      sm.delta[tid] = st.delta;
    }
  };
  auto block = [&](Cur cu) {
    const Item itm = decode(cu);
    const int nrows = itm.s ? a.T_out : a.T;
    const int pos0 = (itm.s ? T_in : 0) + itm.qb * 64;  // position of row 0
    const int Ws = itm.s ? a.T : a.W;
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // rows 32 half .. + 31
      bool none[2], all_in[2];
      float4 lse4[2], del4[2];
      f32x4 sc[2], dp[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int rq0 = 32 * half + 16 * h2;  // first row of this quarter
        const int p_lo = pos0 + rq0, p_hi = p_lo + 15;
        // quarter entirely outside every (row, key) range of the wave, or
        // entirely inside (no masking)
        none[h2] = itm.qb * 64 + rq0 >= nrows || kw > p_hi ||
                   kw + 15 < range_lo(p_lo, Ws) || kw >= a.T;
        all_in[h2] = itm.qb * 64 + rq0 + 15 < nrows && kw + 15 < a.T &&
                     kw + 15 <= p_lo && kw >= range_lo(p_hi, Ws);
        // row statistics of C rows rq0 + 4 g4 .. + 3, read up front
        lse4[h2] = *(const float4 *)&sm.lse[rq0 + 4 * g4];
        del4[h2] = *(const float4 *)&sm.delta[rq0 + 4 * g4];
        sc[h2] = dp[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (none[0] & none[1]) continue;  // no key of the wave in this half
      auto quarter = [&](int h2) {
        const int rq0 = 32 * half + 16 * h2;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          sc[h2] = mfma16(lds_row8(sm.q, rq0 + col, c4, g4), kop[c4], sc[h2]);
          dp[h2] = mfma16(lds_row8(sm.g, rq0 + col, c4, g4), vop[c4], dp[h2]);
        }
      };
      if (!none[0] && !none[1]) {
        quarter(0);
        quarter(1);
        // operand reads run ahead of the 16 MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      } else {
        if (!none[0]) quarter(0);
        if (!none[1]) quarter(1);
      }
      bf16x8 pop, dsop;
      if (all_in[0] & all_in[1]) {  // no masking in this half
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float lv[4] = {lse4[h2].x, lse4[h2].y, lse4[h2].z, lse4[h2].w};
          const float dv4[4] = {del4[h2].x, del4[h2].y, del4[h2].z, del4[h2].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(sc[h2][i] - lv[i]);
            pop[4 * h2 + i] = (__bf16)pr;
            dsop[4 * h2 + i] = (__bf16)(pr * (dp[h2][i] - dv4[i]));
          }
        }
      } else
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int rq0 = 32 * half + 16 * h2;
        const float lv[4] = {lse4[h2].x, lse4[h2].y, lse4[h2].z, lse4[h2].w};
        const float dv4[4] = {del4[h2].x, del4[h2].y, del4[h2].z, del4[h2].w};
        // C rows are query rows rq0 + 4 g4 + i, the column is this key
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = rq0 + 4 * g4 + i;
          const int p = pos0 + rl;
          // branch-free: exp2(-inf) = 0 outside the ranges
          const bool in = (itm.qb * 64 + rl < nrows) & (key < a.T) &
                          (key <= p) & (key >= range_lo(p, Ws));
          const bool ok = !none[h2] & (all_in[h2] | in);
          const float pr =
              __builtin_amdgcn_exp2f(ok ? sc[h2][i] - lv[i] : -INFINITY);
          pop[4 * h2 + i] = (__bf16)pr;
          dsop[4 * h2 + i] = (__bf16)(pr * (dp[h2][i] - dv4[i]));
        }
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        dv[dt] = mfma16(lds_tr8(sm.g, 32 * half, g4, j16, dt), pop, dv[dt]);
        dk[dt] = mfma16(lds_tr8(sm.q, 32 * half, g4, j16, dt), dsop, dk[dt]);
      }
      // transposed reads run two MFMAs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };

  // n_it >= 1: every group has a head and every key a base row. Loads
  // past the last block re-read it (unused), so that every block issues the
  // same loads; a counted loop of block pairs keeps one path through it.
  Stage sA = {}, sB = {};
  Cur c0 = {0, 0, 0};     // the block to compute
  Cur c2 = adv(c0);       // two cursors ahead: the next loads
  load(sA, c0);
  load(sB, c2);
  c2 = adv(c2);
  for (; c0.it + 1 < n_it;) {
    __syncthreads();  // readers of the previous block are done
    store(sA);
    __syncthreads();
    load(sA, c2);
    c2 = adv(c2);
    block(c0);
    c0 = adv(c0);
    __syncthreads();
    store(sB);
    __syncthreads();
    load(sB, c2);
    c2 = adv(c2);
    block(c0);
    c0 = adv(c0);
  }
  if ((n_it & 1) == 1) {
    __syncthreads();
    store(sA);
    __syncthreads();
    block(c0);
  }

  // dK = dS^T (c q) / (c sqrt(D)) with c sqrt(D) = log2(e); dV = P^T dO
  if (key >= a.T) return;
  const float kscale = 1.0f / kLog2e;
  const int64_t off = (((int64_t)b * a.T + key) * a.n_kv + kvh) * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int d0 = 16 * dt + 4 * g4;
    *(uint2 *)(a.dk + off + d0) =
        make_uint2(pack2(dk[dt][0] * kscale, dk[dt][1] * kscale),
                   pack2(dk[dt][2] * kscale, dk[dt][3] * kscale));
    *(uint2 *)(a.dv + off + d0) =
        make_uint2(pack2(dv[dt][0], dv[dt][1]), pack2(dv[dt][2], dv[dt][3]));
  }
}

// d alpha, d beta [Hq*D] from the per-block sums [B, n_rb, Hq, 2, D]: one
// workgroup per (head, alpha|beta), 8 slices of the (batch, block) range per
// channel, summed in a fixed order.
__global__ __launch_bounds__(1024) void bwd_reduce_kernel(
    const float *__restrict__ part, float *__restrict__ d_alpha,
    float *__restrict__ d_beta, int B, int n_rb, int Hq) {
  __shared__ float red[8][D];
  const int h = blockIdx.x >> 1, which = blockIdx.x & 1;
  const int d = threadIdx.x % D, sl = threadIdx.x / D;
  const int n = B * n_rb, per = (n + 7) / 8;
  const int i0 = sl * per, i1 = min(n, i0 + per);
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int i = i0;
  auto at = [&](int k) {
    return part[(((int64_t)k * Hq + h) * 2 + which) * D + d];  // k = b n_rb + r
  };
  for (; i + 4 <= i1; i += 4) {
    s0 += at(i);
    s1 += at(i + 1);
    s2 += at(i + 2);
    s3 += at(i + 3);
  }
  for (; i < i1; ++i) s0 += at(i);
  red[sl][d] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  if (sl == 0) {
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += red[k][d];
    (which ? d_beta : d_alpha)[h * D + d] = s;
  }
}

}  // namespace

hipError_t launch_bwd_dq(const BwdStreamArgs &a, const HeadGroups &groups,
                         int B, hipStream_t stream) {
  const int rows_wg = 32 * (8 / groups.gsize);
  const int n_wg_rows = (a.nrows + rows_wg - 1) / rows_wg;
  const dim3 grid((unsigned)(n_wg_rows * groups.n_groups * B));
  switch (groups.gsize) {
    case 1: hipLaunchKernelGGL(bwd_dq_kernel<1>, grid, dim3(512), 0, stream, a, groups); break;
    case 2: hipLaunchKernelGGL(bwd_dq_kernel<2>, grid, dim3(512), 0, stream, a, groups); break;
    case 4: hipLaunchKernelGGL(bwd_dq_kernel<4>, grid, dim3(512), 0, stream, a, groups); break;
    case 8: hipLaunchKernelGGL(bwd_dq_kernel<8>, grid, dim3(512), 0, stream, a, groups); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BwdKvArgs &a, const HeadGroups &groups,
                          int B, hipStream_t stream) {
  const int n_kt = (a.T + kKvKeys - 1) / kKvKeys;
  const dim3 grid((unsigned)(n_kt * groups.n_groups * B)), blk(kKvThreads);
  switch (groups.gsize) {
    case 1: hipLaunchKernelGGL(bwd_dkv_kernel<1>, grid, blk, 0, stream, a, groups); break;
    case 2: hipLaunchKernelGGL(bwd_dkv_kernel<2>, grid, blk, 0, stream, a, groups); break;
    case 4: hipLaunchKernelGGL(bwd_dkv_kernel<4>, grid, blk, 0, stream, a, groups); break;
    case 8: hipLaunchKernelGGL(bwd_dkv_kernel<8>, grid, blk, 0, stream, a, groups); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const float *part, float *d_alpha, float *d_beta,
                             int B, int n_rb, int Hq, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(2 * Hq), dim3(8 * D), 0, stream,
                     part, d_alpha, d_beta, B, n_rb, Hq);
  return hipGetLastError();
}

}  // namespace orthros
