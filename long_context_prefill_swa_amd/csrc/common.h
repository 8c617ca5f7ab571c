// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthros {

constexpr int kMaxHeads = 128;
constexpr int kMaxGroups = 128;
constexpr int kMaxGroupSize = 8;  // query heads packed with one KV head

// A query-head grouping passed by value to the kernels. Group i reads KV
// head kv[i] and serves up to `gsize` query heads q[i][0..gsize) (-1 marks
// an empty slot). Built on the host from the caller's head map.
struct HeadGroups {
  int n_groups;
  int gsize;  // 1, 2, 4 or 8
  uint8_t kv[kMaxGroups];
  int8_t q[kMaxGroups][kMaxGroupSize];
};

// The query heads of group gi packed in two dwords (slot s in bits
// 8 (s % 4) .. 8 (s % 4) + 7 of word s / 4). A kernel argument read one byte
// at a time is a vector load, and its wait also waits for every load in
// flight; the dwords are scalar loads.
struct GroupHeads {
  uint32_t w[2];
};
__device__ __forceinline__ GroupHeads group_heads(const HeadGroups &g, int gi) {
  const uint32_t *p = (const uint32_t *)&g.q[gi][0];
  return GroupHeads{{p[0], p[1]}};
}
// Query head of slot s (0 .. 7), or -1 for an empty slot.
__device__ __forceinline__ int slot_head(const GroupHeads &h, int s) {
  const uint32_t w = s < 4 ? h.w[0] : h.w[1];
  return (int)(int8_t)(w >> (8 * (s & 3)));
}

// Plain per-query-head map (generic kernels).
struct HeadMap {
  uint8_t kv_of_q[kMaxHeads];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// log2(e): scores are scaled into the base-2 domain once, at the query.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// max(v, v of lane ^ 32), one v_permlane32_swap (gfx950) instead of an LDS
// permute: swapping the upper half of one copy with the lower half of
// another leaves each lane holding both values of its pair.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                                  __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---- launchers (defined in the .hip files) --------------------------------

// Sticky device error flag (capacity faults); address on the current device.
hipError_t device_flag_ptr(int **out);

// Copies new rows into the cache at cache_len[b]; a batch entry whose new
// length would exceed `cap` is skipped and raises *flag. With bump != 0 the
// lengths are then advanced (a second kernel).
hipError_t launch_kv_append(void *k_cache, void *v_cache, int32_t *cache_len,
                            const void *k_new, const void *v_new, int B,
                            int n_new, int Hkv, int row_bytes, int64_t cap,
                            int64_t cap_stride, int *flag, int bump,
                            hipStream_t stream);

// Generic row-per-wave attention for any D <= 256, fp32 or bf16.
// Row r of batch b sits at position t = (cache_len ? cache_len[b] : q_offset)
// + r and attends keys [max(0, t-W+1), t] (W <= 0: [0, t]); rows with
// t >= t_limit (a rejected decode length) get zeros.
hipError_t launch_rowwise(const void *q, const float *alpha, const float *beta,
                          const void *k_cache, const void *v_cache, void *o,
                          int B, int nrows, int Hq, int Hkv, int D,
                          int64_t cap, int64_t t_limit, int64_t q_offset,
                          int W, const int32_t *cache_len, const HeadMap &map,
                          int is_bf16, hipStream_t stream);

// Paged variant: row len+i of batch entry b goes to page
// block_table[b * max_pages + (len + i) >> page_log2]; entries outside
// [0, n_pages) or lengths beyond max_pages pages skip the batch entry and
// raise *flag. Then the lengths are advanced.
hipError_t launch_kv_append_paged(void *k_pool, void *v_pool,
                                  int32_t *cache_len, const void *k_new,
                                  const void *v_new, int B, int n_new,
                                  int Hkv, int row_bytes, int64_t n_pages,
                                  int page_log2, const int32_t *block_table,
                                  int max_pages, int *flag,
                                  hipStream_t stream);

// Increments cache_len[b] by n where the result stays within [0, cap].
hipError_t launch_len_bump(int32_t *cache_len, int B, int n, int64_t cap,
                           hipStream_t stream);

// Banded flash attention, bf16, D = 128, MFMA. Rows r in [0, nrows) sit at
// positions q_offset + r; keys [max(0, t-W+1), t] (W <= 0: unbounded).
hipError_t launch_band_mfma(const void *q, const float *alpha,
                            const float *beta, const void *k_cache,
                            const void *v_cache, void *o, int B, int nrows,
                            int Hq, int64_t cap, int64_t q_offset, int W,
                            const HeadGroups &groups, int n_kv,
                            hipStream_t stream);

// ---- training backward (bf16, D = 128) -------------------------------------
// One stream's rows: positions q_offset + r, keys [max(0, p-W+1), p].
struct BwdStreamArgs {
  const uint16_t *q, *o, *d_o;          // [B, nrows, Hq, D]
  const uint16_t *k_cache, *v_cache;    // [B, n_kv, cap, D]
  const float *alpha, *beta;            // [Hq*D]
  uint16_t *dq;                         // [B, nrows, Hq, D] d q_pre
  uint16_t *qa;                         // [B, nrows, Hq, D] written: the
                                        // query operand bf16((alpha q_pre +
                                        // beta) log2(e) / sqrt(D))
  float *lse, *delta;                   // [B, Hq, nrows] base-2 lse, dO . o
  float *part;                          // [B, ceil(nrows/32), Hq, 2, D]
  int nrows, Hq, n_kv, n_keys, W, q_offset;  // W <= n_keys
  int64_t cap;
};
// Both streams, for dK and dV [B, T, n_kv, D].
struct BwdKvArgs {
  const uint16_t *qa, *qax;  // query operands the dQ kernels wrote
  const uint16_t *d_o, *d_ox, *k_cache, *v_cache;
  const float *lse, *delta, *lse_x, *delta_x;
  uint16_t *dk, *dv;
  int T, T_out, Hq, n_kv, W;  // W <= T
  int64_t cap;
};
hipError_t launch_bwd_dq(const BwdStreamArgs &a, const HeadGroups &groups,
                         int B, hipStream_t stream);
hipError_t launch_bwd_dkv(const BwdKvArgs &a, const HeadGroups &groups,
                          int B, hipStream_t stream);
hipError_t launch_bwd_reduce(const float *part, float *d_alpha, float *d_beta,
                             int B, int n_rb, int Hq, hipStream_t stream);

// Persistent banded attention (bf16, D = 128, 4 query heads per KV head):
// workgroups walk runs of 64-row query tiles. Row r sits at position
// pos_off + r and sees keys [max(0, pos - W + 1), pos]; W <= 0 means every
// key up to pos (pos_off + nrows <= cap < 2^31).
hipError_t launch_band_persist(const void *q, const float *alpha,
                               const float *beta, const void *k_cache,
                               const void *v_cache, void *o, int B, int nrows,
                               int pos_off, int Hq, int64_t cap, int W,
                               const HeadGroups &groups, int n_kv,
                               hipStream_t stream);

// Rolling-window attention for small windows, bf16, D = 128, 4 query heads
// per KV head, rows at positions 0 .. nrows-1, 1 <= W <= kRollMaxWindow.
constexpr int kRollMaxWindow = 129;
hipError_t launch_band_roll(const void *q, const float *alpha,
                            const float *beta, const void *k_cache,
                            const void *v_cache, void *o, int B, int nrows,
                            int Hq, int64_t cap, int W,
                            const HeadGroups &groups, int n_kv,
                            hipStream_t stream);

// Split-KV flash decode, bf16, D = 128, MFMA. See splitkv_mfma.hip.
struct SplitKVArgs {
  const void *q[2];          // [B, n_pos, Hq, D] per stream
  const float *alpha[2];
  const float *beta[2];
  void *o[2];                // [B, n_pos, Hq, D] per stream
  int W[2];                  // window per stream (<= 0: unbounded)
  int n_streams;             // 1 (global) or 2 (decode pair)
  int n_pos;                 // query positions per stream
  int B, Hq, n_kv_heads;
  int64_t cap;
  int64_t pos0;              // position of q row 0 (host known) ...
  const int32_t *cache_len;  // ... or, if non-null, cache_len[b] (decode)
  void *k_cache, *v_cache;
  const void *k_new, *v_new; // decode: appended row [B, Hkv, D]
  int64_t max_len;           // upper bound of keys per batch entry
  int chunk;                 // keys per split (multiple of 128)
  int n_chunks;
  float *ws;                 // partials: (max, sum) pairs, then outputs
  int64_t ws_acc_offset;     // float offset of the unnormalised outputs
  int fused;                 // 1: merge in the same launch; 0: merge kernel
  int32_t *counters;         // one launch: [B * n_groups] arrivals per
                             // (batch, group), then [B] (decode) per batch
                             // entry; zero at the start of a call, left zero
  int32_t *ws_len;           // two launches, decode: per-batch old length
                             // or -1 (skipped), for the merge kernel
  int *flag;
  // Paged cache (block_table != nullptr): k_cache / v_cache are pools of
  // n_pages pages [n_pages, n_kv_heads, page_size, D]; key i of batch entry
  // b sits in page block_table[b * max_pages + i / page_size], row
  // i % page_size. page_size is a power of two >= 32.
  const int32_t *block_table;
  int max_pages;
  int page_log2;
  int64_t n_pages;
};
int splitkv_rows(int n_streams, int n_pos, int gsize);
size_t splitkv_counter_bytes(int B, int n_groups);
size_t splitkv_len_bytes(int B);
bool splitkv_fused(int B, int n_groups, int n_chunks);
// Device address, on the current device, of the no-allocation decode pair's
// static scratch array (looked up on the first call on that device).
hipError_t noalloc_scratch_ptr(void **out);
size_t splitkv_ws_bytes(int B, int n_groups, int rows, int n_chunks, int D);
int splitkv_pick_chunk(int B, int n_groups, int64_t max_len, int max_chunk);
hipError_t launch_splitkv(const SplitKVArgs &a, const HeadGroups &groups,
                          hipStream_t stream);

}  // namespace orthros
