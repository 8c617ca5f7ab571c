// C ABI of the Orthros attention hot path: host-side validation, head
// grouping, workspace sizing and kernel selection. Every argument is checked
// before the first HIP call; a failing call launches nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "../../include/orthros.h"
#include "common.h"

using namespace orthros;

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(const char *what, hipError_t e) {
  return fail(ORTHROS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

void clear_error() { g_msg[0] = '\0'; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(int dtype) { return dtype == ORTHROS_F32 ? 4 : 2; }

int check_dtype_d(int dtype, int D) {
  if (dtype != ORTHROS_F32 && dtype != ORTHROS_BF16)
    return fail(ORTHROS_EUNSUPPORTED, "dtype %d is not ORTHROS_F32 or ORTHROS_BF16", dtype);
  if (D < 1 || D > ORTHROS_MAX_D)
    return fail(ORTHROS_EUNSUPPORTED, "head dimension D=%d outside [1, %d]", D,
                ORTHROS_MAX_D);
  if (dtype == ORTHROS_BF16 && (D % 2) != 0)
    return fail(ORTHROS_EUNSUPPORTED, "bf16 needs an even head dimension (D=%d)", D);
  return ORTHROS_OK;
}

int check_heads(int Hq, int Hkv) {
  if (Hq < 1 || Hkv < 1)
    return fail(ORTHROS_EINVAL, "head counts must be >= 1 (Hq=%d, Hkv=%d)", Hq, Hkv);
  if (Hq > ORTHROS_MAX_HEADS || Hkv > ORTHROS_MAX_HEADS)
    return fail(ORTHROS_EINVAL, "head counts above %d (Hq=%d, Hkv=%d)",
                ORTHROS_MAX_HEADS, Hq, Hkv);
  return ORTHROS_OK;
}

// Resolves the query-head -> KV-head map into both kernel forms.
int build_maps(const int32_t *head_map, int Hq, int Hkv, HeadMap *map,
               HeadGroups *groups) {
  int kv_of[kMaxHeads];
  if (!head_map) {
    if (Hq % Hkv != 0)
      return fail(ORTHROS_EINVAL,
                  "Hq=%d is not a multiple of Hkv=%d and no head map was given",
                  Hq, Hkv);
    for (int h = 0; h < Hq; ++h) kv_of[h] = h / (Hq / Hkv);
  } else {
    for (int h = 0; h < Hq; ++h) {
      if (head_map[h] < 0 || head_map[h] >= Hkv)
        return fail(ORTHROS_EINVAL, "head_map[%d]=%d outside [0, %d)", h,
                    head_map[h], Hkv);
      kv_of[h] = head_map[h];
    }
  }
  memset(map, 0, sizeof(*map));
  for (int h = 0; h < Hq; ++h) map->kv_of_q[h] = (uint8_t)kv_of[h];

  // Groups: the query heads of each KV head, in head order, packed `gsize`
  // at a time (gsize = the largest head count of a KV head, rounded up to a
  // power of two, at most 8).
  int count[kMaxHeads] = {0};
  int maxc = 0;
  for (int h = 0; h < Hq; ++h) maxc = std::max(maxc, ++count[kv_of[h]]);
  int gsize = 1;
  while (gsize < maxc && gsize < kMaxGroupSize) gsize *= 2;
  memset(groups, 0, sizeof(*groups));
  groups->gsize = gsize;
  int n = 0;
  for (int g = 0; g < Hkv; ++g) {
    int slot = gsize;  // forces a new group on the first head
    for (int h = 0; h < Hq; ++h) {
      if (kv_of[h] != g) continue;
      if (slot == gsize) {
        if (n >= kMaxGroups) return fail(ORTHROS_EINVAL, "too many head groups");
        groups->kv[n] = (uint8_t)g;
        for (int s = 0; s < kMaxGroupSize; ++s) groups->q[n][s] = -1;
        ++n;
        slot = 0;
      }
      groups->q[n - 1][slot++] = (int8_t)h;
    }
  }
  groups->n_groups = n;
  return ORTHROS_OK;
}

// Overflow-safe product of non-negative sizes.
bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool tensor_elems(int64_t *out, std::initializer_list<int64_t> dims) {
  int64_t n = 1;
  for (int64_t d : dims)
    if (!mul_ok(n, d, &n)) return false;
  *out = n;
  return true;
}

// MFMA kernels: bf16, D = 128, 16-byte aligned tensors, and key ranges whose
// byte offsets inside one (batch, KV head) slab fit 32 bits (n_keys rows of
// 256 bytes), as the kernels address the cache through buffer resources.
bool mfma_eligible(int dtype, int D, int64_t n_keys,
                   std::initializer_list<const void *> ptrs) {
  if (dtype != ORTHROS_BF16 || D != 128) return false;
  if (n_keys > (int64_t)(UINT32_MAX / 256)) return false;
  for (const void *p : ptrs)
    if (!aligned16(p)) return false;
  return true;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Split-KV plan shared by the workspace query and the launches.
struct SplitPlan {
  bool use = false;
  int rows = 0, chunk = 0, n_chunks = 0;
  bool fused = false;
  size_t ws_bytes = 0;
};

// Chunks of at most 4096 keys for output rows, 2048 for a decode step (its
// cache may be paged, and a chunk spans at most 64 pages).
constexpr int kChunkRows = 4096;
constexpr int kChunkDecode = 2048;

SplitPlan plan_split(int B, int n_streams, int n_pos, const HeadGroups &g,
                     int D, int64_t max_len, int max_chunk) {
  SplitPlan p;
  p.rows = splitkv_rows(n_streams, n_pos, g.gsize);
  // The split kernel addresses one (batch, KV head) slab of the cache with
  // 32-bit byte offsets: max_len rows of 256 bytes must stay below 4 GiB.
  if (D != 128 || p.rows > 16 || max_len > (int64_t)(UINT32_MAX / 256)) return p;
  p.use = true;
  p.chunk = splitkv_pick_chunk(B, g.n_groups, max_len, max_chunk);
  p.n_chunks = (int)((max_len + p.chunk - 1) / p.chunk);
  p.fused = splitkv_fused(B, g.n_groups, p.n_chunks);
  p.ws_bytes = splitkv_ws_bytes(B, g.n_groups, p.rows, p.n_chunks, D);
  return p;
}

// The counters take the first counter_region bytes of ws (at least
// splitkv_counter_bytes), the partials the rest.
void fill_ws(SplitKVArgs *a, void *ws, const SplitPlan &p, int B,
             int n_groups, size_t counter_region) {
  a->fused = p.fused ? 1 : 0;
  a->counters = (int32_t *)ws;
  a->ws_len = (int32_t *)((char *)ws + counter_region);
  a->ws = (float *)((char *)ws + counter_region + splitkv_len_bytes(B));
  const int64_t parts = (int64_t)B * n_groups * p.n_chunks * p.rows;
  a->ws_acc_offset = (parts * 2 + 63) / 64 * 64;
  a->chunk = p.chunk;
  a->n_chunks = p.n_chunks;
}

// The split plan of a workspace query; false when the call needs no
// workspace (unknown op, invalid sizes or map, or no split-KV launch).
// A pure query: the caller's last error message is left as it was.
bool query_plan(int op, int B, int Hq, int Hkv, int D, int T_out,
                int64_t max_len, const int32_t *head_map, SplitPlan *p,
                HeadGroups *g) {
  if (B < 1 || T_out < 1 || max_len < 1 || D < 1 || D > ORTHROS_MAX_D)
    return false;
  if (Hq < 1 || Hkv < 1 || Hq > ORTHROS_MAX_HEADS || Hkv > ORTHROS_MAX_HEADS)
    return false;
  // The same head grouping the calls build from (head_map, Hq, Hkv): the
  // number of groups and the group width size the partials.
  HeadMap map;
  char saved[sizeof(g_msg)];
  memcpy(saved, g_msg, sizeof(g_msg));
  const int rc = build_maps(head_map, Hq, Hkv, &map, g);
  memcpy(g_msg, saved, sizeof(g_msg));
  if (rc != ORTHROS_OK) return false;
  if (op == ORTHROS_OP_GLOBAL_XATTN)
    *p = plan_split(B, 1, T_out, *g, D, max_len, kChunkRows);
  else if (op == ORTHROS_OP_DECODE_PAIR)
    *p = plan_split(B, 2, 1, *g, D, max_len, kChunkDecode);
  else
    return false;
  return p->use;
}

}  // namespace

namespace orthros {
// Records a message for orthros_last_error (used by the layer entry point).
int api_error(int code, const char *msg) {
  snprintf(g_msg, sizeof(g_msg), "%s", msg);
  return code;
}
}  // namespace orthros

extern "C" {

int orthros_abi_version(void) { return ORTHROS_ABI_VERSION; }

const char *orthros_strerror(int code) {
  switch (code) {
    case ORTHROS_OK: return "ok";
    case ORTHROS_EINVAL: return "invalid argument";
    case ORTHROS_EUNSUPPORTED: return "unsupported dtype or head dimension";
    case ORTHROS_ECAPACITY: return "cache capacity exceeded";
    case ORTHROS_EWORKSPACE: return "workspace missing or too small";
    case ORTHROS_EHIP: return "HIP runtime error";
    default: return "unknown status code";
  }
}

const char *orthros_last_error(void) { return g_msg; }

size_t orthros_workspace_bytes(int op, int B, int Hq, int Hkv, int D,
                               int T_out, int64_t max_len,
                               const int32_t *head_map) {
  SplitPlan p;
  HeadGroups g;
  return query_plan(op, B, Hq, Hkv, D, T_out, max_len, head_map, &p, &g)
             ? p.ws_bytes
             : 0;
}

size_t orthros_workspace_counter_bytes(int op, int B, int Hq, int Hkv, int D,
                                       int T_out, int64_t max_len,
                                       const int32_t *head_map) {
  SplitPlan p;
  HeadGroups g;
  return query_plan(op, B, Hq, Hkv, D, T_out, max_len, head_map, &p, &g)
             ? splitkv_counter_bytes(B, g.n_groups)
             : 0;
}

int orthros_kv_append(void *k_cache, void *v_cache, int32_t *cache_len,
                      const void *k_new, const void *v_new, int B, int n_new,
                      int Hkv, int D, int64_t cap, int dtype, void *stream) {
  clear_error();
  int rc = check_dtype_d(dtype, D);
  if (rc) return rc;
  if (B < 0 || n_new < 0) return fail(ORTHROS_EINVAL, "negative size (B=%d, n_new=%d)", B, n_new);
  if (Hkv < 1 || Hkv > ORTHROS_MAX_HEADS) return fail(ORTHROS_EINVAL, "Hkv=%d outside [1, %d]", Hkv, ORTHROS_MAX_HEADS);
  if (cap < 1 || cap > INT32_MAX) return fail(ORTHROS_EINVAL, "cap=%lld outside [1, 2^31-1]", (long long)cap);
  if (n_new > cap) return fail(ORTHROS_ECAPACITY, "n_new=%d exceeds cap=%lld", n_new, (long long)cap);
  if (B == 0 || n_new == 0) return ORTHROS_OK;
  if (!k_cache || !v_cache || !cache_len || !k_new || !v_new)
    return fail(ORTHROS_EINVAL, "null pointer argument");
  int64_t n_elems;
  if (!tensor_elems(&n_elems, {B, Hkv, cap, D, (int64_t)esize(dtype)}))
    return fail(ORTHROS_EINVAL, "cache size overflows");
  const int row_bytes = D * (int)esize(dtype);
  int *flag = nullptr;
  hipError_t e = device_flag_ptr(&flag);
  if (e != hipSuccess) return hip_fail("device flag", e);
  e = launch_kv_append(k_cache, v_cache, cache_len, k_new, v_new, B, n_new,
                       Hkv, row_bytes, cap, cap, flag, 1, as_stream(stream));
  if (e != hipSuccess) return hip_fail("kv_append launch", e);
  return ORTHROS_OK;
}

int orthros_swa_prefill(const void *q_pre, const float *alpha,
                        const float *beta, const void *k_cache,
                        const void *v_cache, void *o, int B, int T, int Hq,
                        int Hkv, int D, int64_t cap, int W,
                        const int32_t *head_map, int dtype, void *stream) {
  clear_error();
  int rc = check_dtype_d(dtype, D);
  if (rc) return rc;
  if ((rc = check_heads(Hq, Hkv))) return rc;
  if (B < 0 || T < 0) return fail(ORTHROS_EINVAL, "negative size (B=%d, T=%d)", B, T);
  if (W < 1) return fail(ORTHROS_EINVAL, "window W=%d must be >= 1", W);
  if (cap < T || cap > INT32_MAX)
    return fail(ORTHROS_EINVAL, "cap=%lld must hold the T=%d rows", (long long)cap, T);
  HeadMap map;
  HeadGroups groups;
  if ((rc = build_maps(head_map, Hq, Hkv, &map, &groups))) return rc;
  if (B == 0 || T == 0) return ORTHROS_OK;
  if (!q_pre || !alpha || !beta || !k_cache || !v_cache || !o)
    return fail(ORTHROS_EINVAL, "null pointer argument");
  int64_t n_elems;
  if (!tensor_elems(&n_elems, {B, Hkv, cap, D, 2}) ||
      !tensor_elems(&n_elems, {B, T, Hq, D, 2}))
    return fail(ORTHROS_EINVAL, "tensor size overflows");
  hipError_t e;
  if (mfma_eligible(dtype, D, T, {q_pre, alpha, beta, k_cache, v_cache, o}) &&
      groups.gsize == 4 && W <= kRollMaxWindow) {
    // small window: the pass streams Q/O through HBM (rolling kernel)
    e = launch_band_roll(q_pre, alpha, beta, k_cache, v_cache, o, B, T, Hq,
                         cap, W, groups, Hkv, as_stream(stream));
  } else if (mfma_eligible(dtype, D, T,
                           {q_pre, alpha, beta, k_cache, v_cache, o}) &&
             groups.gsize == 4) {
    // larger windows (up to the whole prefix): resident workgroups walk
    // runs of query tiles (persistent kernel)
    e = launch_band_persist(q_pre, alpha, beta, k_cache, v_cache, o, B, T, 0,
                            Hq, cap, W, groups, Hkv, as_stream(stream));
  } else if (mfma_eligible(dtype, D, T,
                           {q_pre, alpha, beta, k_cache, v_cache, o})) {
    e = launch_band_mfma(q_pre, alpha, beta, k_cache, v_cache, o, B, T, Hq,
                         cap, 0, W, groups, Hkv, as_stream(stream));
  } else {
    e = launch_rowwise(q_pre, alpha, beta, k_cache, v_cache, o, B, T, Hq, Hkv,
                       D, cap, cap, 0, W, nullptr, map,
                       dtype == ORTHROS_BF16, as_stream(stream));
  }
  if (e != hipSuccess) return hip_fail("swa_prefill launch", e);
  return ORTHROS_OK;
}

int orthros_global_xattn(const void *qx_pre, const float *alpha_x,
                         const float *beta_x, const void *k_cache,
                         const void *v_cache, void *o_x, int B, int T_in,
                         int T_out, int Hq, int Hkv, int D, int64_t cap,
                         const int32_t *head_map, int dtype, void *ws,
                         size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_dtype_d(dtype, D);
  if (rc) return rc;
  if ((rc = check_heads(Hq, Hkv))) return rc;
  if (B < 0 || T_in < 0 || T_out < 0)
    return fail(ORTHROS_EINVAL, "negative size (B=%d, T_in=%d, T_out=%d)", B, T_in, T_out);
  const int64_t T = (int64_t)T_in + T_out;
  if (cap < T || cap > INT32_MAX)
    return fail(ORTHROS_EINVAL, "cap=%lld must hold T_in+T_out=%lld rows",
                (long long)cap, (long long)T);
  HeadMap map;
  HeadGroups groups;
  if ((rc = build_maps(head_map, Hq, Hkv, &map, &groups))) return rc;
  if (B == 0 || T_out == 0) return ORTHROS_OK;
  if (!qx_pre || !alpha_x || !beta_x || !k_cache || !v_cache || !o_x)
    return fail(ORTHROS_EINVAL, "null pointer argument");
  int64_t n_elems;
  if (!tensor_elems(&n_elems, {B, Hkv, cap, D, 2}) ||
      !tensor_elems(&n_elems, {B, T_out, Hq, D, 2}))
    return fail(ORTHROS_EINVAL, "tensor size overflows");

  hipError_t e;
  const bool mfma =
      mfma_eligible(dtype, D, T, {qx_pre, alpha_x, beta_x, k_cache, v_cache, o_x});
  const SplitPlan plan = plan_split(B, 1, T_out, groups, D, T, kChunkRows);
  if (mfma && plan.use) {
    if (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))
      return fail(ORTHROS_EWORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu",
                  plan.ws_bytes, ws ? ws_bytes : (size_t)0);
    SplitKVArgs a = {};
    a.q[0] = qx_pre;
    a.alpha[0] = alpha_x;
    a.beta[0] = beta_x;
    a.o[0] = o_x;
    a.W[0] = 0;
    a.n_streams = 1;
    a.n_pos = T_out;
    a.B = B;
    a.Hq = Hq;
    a.n_kv_heads = Hkv;
    a.cap = cap;
    a.pos0 = T_in;
    a.cache_len = nullptr;
    a.k_cache = const_cast<void *>(k_cache);
    a.v_cache = const_cast<void *>(v_cache);
    a.max_len = T;
    fill_ws(&a, ws, plan, B, groups.n_groups,
            splitkv_counter_bytes(B, groups.n_groups));
    e = device_flag_ptr(&a.flag);
    if (e != hipSuccess) return hip_fail("device flag", e);
    e = launch_splitkv(a, groups, as_stream(stream));
  } else if (mfma && groups.gsize == 4) {
    // many output rows, 4 query heads per KV head: the persistent kernel
    // with every key up to each row's position
    e = launch_band_persist(qx_pre, alpha_x, beta_x, k_cache, v_cache, o_x, B,
                            T_out, T_in, Hq, cap, 0, groups, Hkv,
                            as_stream(stream));
  } else if (mfma) {
    e = launch_band_mfma(qx_pre, alpha_x, beta_x, k_cache, v_cache, o_x, B,
                         T_out, Hq, cap, T_in, 0, groups, Hkv,
                         as_stream(stream));
  } else {
    e = launch_rowwise(qx_pre, alpha_x, beta_x, k_cache, v_cache, o_x, B, T_out,
                       Hq, Hkv, D, cap, cap, T_in, 0, nullptr, map,
                       dtype == ORTHROS_BF16, as_stream(stream));
  }
  if (e != hipSuccess) return hip_fail("global_xattn launch", e);
  return ORTHROS_OK;
}

}  // extern "C"

namespace {

constexpr size_t kScratchBytes = ORTHROS_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchCounterBytes = ORTHROS_NOALLOC_COUNTER_BYTES;

// The decode pair step. With from_scratch, the split-KV partials go to the
// static scratch array instead of the caller's ws (which is then ignored).
int decode_pair_impl(const void *q_pre, const void *qx_pre,
                     const float *alpha, const float *beta,
                     const float *alpha_x, const float *beta_x,
                     const void *k_new, const void *v_new, void *k_cache,
                     void *v_cache, int32_t *cache_len, void *o, void *o_x,
                     int B, int Hq, int Hkv, int D, int64_t cap,
                     int64_t max_len_after, int W, const int32_t *head_map,
                     int dtype, void *ws, size_t ws_bytes, bool from_scratch,
                     void *stream) {
  clear_error();
  int rc = check_dtype_d(dtype, D);
  if (rc) return rc;
  if ((rc = check_heads(Hq, Hkv))) return rc;
  if (B < 0) return fail(ORTHROS_EINVAL, "negative batch B=%d", B);
  if (W < 1) return fail(ORTHROS_EINVAL, "window W=%d must be >= 1", W);
  if (cap < 1 || cap > INT32_MAX) return fail(ORTHROS_EINVAL, "cap=%lld outside [1, 2^31-1]", (long long)cap);
  if (max_len_after < 1)
    return fail(ORTHROS_EINVAL, "max_len_after=%lld must be >= 1", (long long)max_len_after);
  if (max_len_after > cap)
    return fail(ORTHROS_ECAPACITY, "max_len_after=%lld exceeds cap=%lld",
                (long long)max_len_after, (long long)cap);
  HeadMap map;
  HeadGroups groups;
  if ((rc = build_maps(head_map, Hq, Hkv, &map, &groups))) return rc;
  if (B == 0) return ORTHROS_OK;
  if (!q_pre || !qx_pre || !alpha || !beta || !alpha_x || !beta_x || !k_new ||
      !v_new || !k_cache || !v_cache || !cache_len || !o || !o_x)
    return fail(ORTHROS_EINVAL, "null pointer argument");
  int64_t n_elems;
  if (!tensor_elems(&n_elems, {B, Hkv, cap, D, 2}))
    return fail(ORTHROS_EINVAL, "cache size overflows");

  hipStream_t st = as_stream(stream);
  const bool mfma = mfma_eligible(
      dtype, D, max_len_after, {q_pre, qx_pre, alpha, beta, alpha_x, beta_x, k_new, v_new,
                 k_cache, v_cache, o, o_x});
  const SplitPlan plan =
      plan_split(B, 2, 1, groups, D, max_len_after, kChunkDecode);
  const size_t ws_need = plan.ws_bytes;
  hipError_t e;
  size_t counter_region = splitkv_counter_bytes(B, groups.n_groups);
  if (mfma && plan.use && from_scratch) {
    // The scratch array keeps its counters in a fixed leading region, so
    // that no call's partials land where a later call with more (batch,
    // group) pairs expects zeroed counters.
    const size_t need = ws_need - counter_region + kScratchCounterBytes;
    if (counter_region > kScratchCounterBytes || need > kScratchBytes)
      return fail(ORTHROS_EWORKSPACE,
                  "these sizes need %zu bytes of scratch (%zu of counters); "
                  "the no-allocation decode pair holds %zu (%zu of counters; "
                  "use orthros_decode_pair with a workspace)",
                  ws_need, counter_region, kScratchBytes,
                  kScratchCounterBytes);
    e = noalloc_scratch_ptr(&ws);
    if (e != hipSuccess) return hip_fail("scratch symbol", e);
    ws_bytes = kScratchBytes;
    counter_region = kScratchCounterBytes;
  }
  if (mfma && plan.use && (!ws || ws_bytes < ws_need || !aligned16(ws)))
    return fail(ORTHROS_EWORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu",
                ws_need, ws ? ws_bytes : (size_t)0);
  int *flag = nullptr;
  e = device_flag_ptr(&flag);
  if (e != hipSuccess) return hip_fail("device flag", e);
  if (mfma && plan.use) {
    SplitKVArgs a = {};
    a.q[0] = q_pre;
    a.q[1] = qx_pre;
    a.alpha[0] = alpha;
    a.alpha[1] = alpha_x;
    a.beta[0] = beta;
    a.beta[1] = beta_x;
    a.o[0] = o;
    a.o[1] = o_x;
    a.W[0] = W;
    a.W[1] = 0;
    a.n_streams = 2;
    a.n_pos = 1;
    a.B = B;
    a.Hq = Hq;
    a.n_kv_heads = Hkv;
    a.cap = cap;
    a.pos0 = 0;
    a.cache_len = cache_len;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_new = k_new;
    a.v_new = v_new;
    a.max_len = max_len_after;
    a.flag = flag;
    fill_ws(&a, ws, plan, B, groups.n_groups, counter_region);
    e = launch_splitkv(a, groups, st);
    if (e != hipSuccess) return hip_fail("decode_pair launch", e);
    return ORTHROS_OK;
  }
  // Generic path: append (lengths unchanged), both attentions, then advance.
  const int row_bytes = D * (int)esize(dtype);
  e = launch_kv_append(k_cache, v_cache, cache_len, k_new, v_new, B, 1, Hkv,
                       row_bytes, max_len_after, cap, flag, 0, st);
  if (e == hipSuccess)
    e = launch_rowwise(q_pre, alpha, beta, k_cache, v_cache, o, B, 1, Hq, Hkv,
                       D, cap, max_len_after, 0, W, cache_len, map,
                       dtype == ORTHROS_BF16, st);
  if (e == hipSuccess)
    e = launch_rowwise(qx_pre, alpha_x, beta_x, k_cache, v_cache, o_x, B, 1,
                       Hq, Hkv, D, cap, max_len_after, 0, 0, cache_len, map,
                       dtype == ORTHROS_BF16, st);
  if (e == hipSuccess) e = launch_len_bump(cache_len, B, 1, max_len_after, st);
  if (e != hipSuccess) return hip_fail("decode_pair launch", e);
  return ORTHROS_OK;
}

}  // namespace

extern "C" {

int orthros_decode_pair(const void *q_pre, const void *qx_pre,
                        const float *alpha, const float *beta,
                        const float *alpha_x, const float *beta_x,
                        const void *k_new, const void *v_new, void *k_cache,
                        void *v_cache, int32_t *cache_len, void *o, void *o_x,
                        int B, int Hq, int Hkv, int D, int64_t cap,
                        int64_t max_len_after, int W, const int32_t *head_map,
                        int dtype, void *ws, size_t ws_bytes, void *stream) {
  return decode_pair_impl(q_pre, qx_pre, alpha, beta, alpha_x, beta_x, k_new,
                          v_new, k_cache, v_cache, cache_len, o, o_x, B, Hq,
                          Hkv, D, cap, max_len_after, W, head_map, dtype, ws,
                          ws_bytes, false, stream);
}

int orthros_decode_pair_noalloc(const void *q_pre, const void *qx_pre,
                                const float *alpha, const float *beta,
                                const float *alpha_x, const float *beta_x,
                                const void *k_new, const void *v_new,
                                void *k_cache, void *v_cache,
                                int32_t *cache_len, void *o, void *o_x, int B,
                                int Hq, int Hkv, int D, int64_t cap,
                                int64_t max_len_after, int W,
                                const int32_t *head_map, int dtype,
                                void *stream) {
  return decode_pair_impl(q_pre, qx_pre, alpha, beta, alpha_x, beta_x, k_new,
                          v_new, k_cache, v_cache, cache_len, o, o_x, B, Hq,
                          Hkv, D, cap, max_len_after, W, head_map, dtype,
                          nullptr, 0, true, stream);
}

// Shared checks of the paged-cache arguments; on success *log2 = log2 of
// page_size.
static int check_paged(void *k_pool, void *v_pool, int64_t n_pages,
                       int page_size, const int32_t *block_table,
                       int max_pages, int Hkv, int D, int dtype, int *log2) {
  if (page_size < 32 || page_size > 65536 || (page_size & (page_size - 1)))
    return fail(ORTHROS_EINVAL,
                "page_size=%d must be a power of two in [32, 65536]", page_size);
  if (n_pages < 1 || n_pages > INT32_MAX)
    return fail(ORTHROS_EINVAL, "n_pages=%lld outside [1, 2^31-1]",
                (long long)n_pages);
  if (max_pages < 1)
    return fail(ORTHROS_EINVAL, "max_pages=%d must be >= 1", max_pages);
  if (!k_pool || !v_pool || !block_table)
    return fail(ORTHROS_EINVAL, "null pointer argument");
  int64_t n_elems;
  if (!tensor_elems(&n_elems, {n_pages, Hkv, page_size, D, (int64_t)esize(dtype)}))
    return fail(ORTHROS_EINVAL, "page pool size overflows");
  if ((int64_t)max_pages * page_size > INT32_MAX)
    return fail(ORTHROS_EINVAL, "max_pages * page_size exceeds 2^31-1");
  int l = 0;
  while ((1 << l) < page_size) ++l;
  *log2 = l;
  return ORTHROS_OK;
}

int orthros_kv_append_paged(void *k_pool, void *v_pool, int64_t n_pages,
                            int page_size, const int32_t *block_table,
                            int max_pages, int32_t *cache_len,
                            const void *k_new, const void *v_new, int B,
                            int n_new, int Hkv, int D, int dtype,
                            void *stream) {
  clear_error();
  int rc = check_dtype_d(dtype, D);
  if (rc) return rc;
  if (B < 0 || n_new < 0) return fail(ORTHROS_EINVAL, "negative size (B=%d, n_new=%d)", B, n_new);
  if (Hkv < 1 || Hkv > ORTHROS_MAX_HEADS) return fail(ORTHROS_EINVAL, "Hkv=%d outside [1, %d]", Hkv, ORTHROS_MAX_HEADS);
  int log2 = 0;
  if ((rc = check_paged(k_pool, v_pool, n_pages, page_size, block_table,
                        max_pages, Hkv, D, dtype, &log2)))
    return rc;
  if ((int64_t)n_new > (int64_t)max_pages * page_size)
    return fail(ORTHROS_ECAPACITY, "n_new=%d exceeds max_pages * page_size", n_new);
  if (B == 0 || n_new == 0) return ORTHROS_OK;
  if (!cache_len || !k_new || !v_new) return fail(ORTHROS_EINVAL, "null pointer argument");
  int *flag = nullptr;
  hipError_t e = device_flag_ptr(&flag);
  if (e != hipSuccess) return hip_fail("device flag", e);
  e = launch_kv_append_paged(k_pool, v_pool, cache_len, k_new, v_new, B,
                             n_new, Hkv, D * (int)esize(dtype), n_pages, log2,
                             block_table, max_pages, flag, as_stream(stream));
  if (e != hipSuccess) return hip_fail("kv_append_paged launch", e);
  return ORTHROS_OK;
}

int orthros_decode_pair_paged(const void *q_pre, const void *qx_pre,
                              const float *alpha, const float *beta,
                              const float *alpha_x, const float *beta_x,
                              const void *k_new, const void *v_new,
                              void *k_pool, void *v_pool, int64_t n_pages,
                              int page_size, const int32_t *block_table,
                              int max_pages, int32_t *cache_len, void *o,
                              void *o_x, int B, int Hq, int Hkv, int D,
                              int64_t max_len_after, int W,
                              const int32_t *head_map, int dtype, void *ws,
                              size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_dtype_d(dtype, D);
  if (rc) return rc;
  if (dtype != ORTHROS_BF16 || D != 128)
    return fail(ORTHROS_EUNSUPPORTED,
                "the paged decode pair supports bf16 with D=128 (got dtype %d, D=%d)",
                dtype, D);
  if ((rc = check_heads(Hq, Hkv))) return rc;
  if (B < 0) return fail(ORTHROS_EINVAL, "negative batch B=%d", B);
  if (W < 1) return fail(ORTHROS_EINVAL, "window W=%d must be >= 1", W);
  int log2 = 0;
  if ((rc = check_paged(k_pool, v_pool, n_pages, page_size, block_table,
                        max_pages, Hkv, D, dtype, &log2)))
    return rc;
  if (max_len_after < 1)
    return fail(ORTHROS_EINVAL, "max_len_after=%lld must be >= 1", (long long)max_len_after);
  const int64_t cap = (int64_t)max_pages * page_size;
  if (max_len_after > cap)
    return fail(ORTHROS_ECAPACITY, "max_len_after=%lld exceeds max_pages * page_size = %lld",
                (long long)max_len_after, (long long)cap);
  HeadMap map;
  HeadGroups groups;
  if ((rc = build_maps(head_map, Hq, Hkv, &map, &groups))) return rc;
  if (B == 0) return ORTHROS_OK;
  if (!q_pre || !qx_pre || !alpha || !beta || !alpha_x || !beta_x || !k_new ||
      !v_new || !cache_len || !o || !o_x)
    return fail(ORTHROS_EINVAL, "null pointer argument");
  if (!mfma_eligible(dtype, D, max_len_after,
                     {q_pre, qx_pre, alpha, beta, alpha_x, beta_x, k_new,
                      v_new, k_pool, v_pool, o, o_x}))
    return fail(ORTHROS_EINVAL, "tensors must be 16-byte aligned");
  const SplitPlan plan =
      plan_split(B, 2, 1, groups, D, max_len_after, kChunkDecode);
  if (!plan.use)
    return fail(ORTHROS_EUNSUPPORTED, "no split plan for these sizes");
  if (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws))
    return fail(ORTHROS_EWORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu",
                plan.ws_bytes, ws ? ws_bytes : (size_t)0);
  int *flag = nullptr;
  hipError_t e = device_flag_ptr(&flag);
  if (e != hipSuccess) return hip_fail("device flag", e);
  SplitKVArgs a = {};
  a.q[0] = q_pre;
  a.q[1] = qx_pre;
  a.alpha[0] = alpha;
  a.alpha[1] = alpha_x;
  a.beta[0] = beta;
  a.beta[1] = beta_x;
  a.o[0] = o;
  a.o[1] = o_x;
  a.W[0] = W;
  a.W[1] = 0;
  a.n_streams = 2;
  a.n_pos = 1;
  a.B = B;
  a.Hq = Hq;
  a.n_kv_heads = Hkv;
  a.cap = cap;
  a.pos0 = 0;
  a.cache_len = cache_len;
  a.k_cache = k_pool;
  a.v_cache = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.max_len = max_len_after;
  a.flag = flag;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.page_log2 = log2;
  a.n_pages = n_pages;
  fill_ws(&a, ws, plan, B, groups.n_groups,
          splitkv_counter_bytes(B, groups.n_groups));
  e = launch_splitkv(a, groups, as_stream(stream));
  if (e != hipSuccess) return hip_fail("decode_pair_paged launch", e);
  return ORTHROS_OK;
}

int orthros_check_device_errors(void *stream) {
  clear_error();
  hipError_t e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail("stream synchronize", e);
  int *flag = nullptr;
  e = device_flag_ptr(&flag);
  if (e != hipSuccess) return hip_fail("device flag", e);
  int host = 0;
  e = hipMemcpy(&host, flag, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail("flag read", e);
  if (!host) return ORTHROS_OK;
  const int zero = 0;
  e = hipMemcpy(flag, &zero, sizeof(int), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail("flag clear", e);
  return fail(ORTHROS_ECAPACITY,
              "a cache append or decode step exceeded the cache capacity; "
              "the affected batch entries were skipped");
}

}  // extern "C"

// ---- training backward -------------------------------------------------------

namespace {

struct BwdWs {
  size_t lse, delta, lse_x, delta_x, part, part_x, qa, qa_x, total;
};

size_t al256(size_t n) { return (n + 255) & ~size_t(255); }

BwdWs bwd_ws(int B, int T, int T_out, int Hq, int D) {
  BwdWs w;
  size_t off = 0;
  const size_t rows = (size_t)B * Hq * 4;
  w.lse = off;
  off += al256(rows * T);
  w.delta = off;
  off += al256(rows * T);
  w.lse_x = off;
  off += al256(rows * T_out);
  w.delta_x = off;
  off += al256(rows * T_out);
  w.part = off;
  off += al256((size_t)B * ((T + 31) / 32) * Hq * 2 * D * 4);
  w.part_x = off;
  off += al256((size_t)B * ((T_out + 31) / 32) * Hq * 2 * D * 4);
  w.qa = off;  // the query operands (bf16) the dQ kernels pass on
  off += al256((size_t)B * T * Hq * D * 2);
  w.qa_x = off;
  off += al256((size_t)B * T_out * Hq * D * 2);
  w.total = off;
  return w;
}

}  // namespace

size_t orthros_backward_workspace_bytes(int B, int T, int T_out, int Hq,
                                        int Hkv, int D) {
  if (B < 1 || T < 1 || T_out < 0 || T_out > T || Hq < 1 || Hkv < 1 ||
      Hq > ORTHROS_MAX_HEADS || Hkv > ORTHROS_MAX_HEADS || D < 1 ||
      D > ORTHROS_MAX_D)
    return 0;
  return bwd_ws(B, T, T_out, Hq, D).total;
}

int orthros_attn_backward(
    const void *q_pre, const void *qx_pre, const float *alpha,
    const float *beta, const float *alpha_x, const float *beta_x,
    const void *k_cache, const void *v_cache, const void *o, const void *o_x,
    const void *d_o, const void *d_ox, void *dq_pre, void *dqx_pre, void *dk,
    void *dv, float *d_alpha, float *d_beta, float *d_alpha_x,
    float *d_beta_x, int B, int T, int T_out, int Hq, int Hkv, int D,
    int64_t cap, int W, const int32_t *head_map, int dtype, void *ws,
    size_t ws_bytes, void *stream) {
  clear_error();
  int rc = check_dtype_d(dtype, D);
  if (rc) return rc;
  if (dtype != ORTHROS_BF16 || D != 128)
    return fail(ORTHROS_EUNSUPPORTED, "the backward needs bf16 and D = 128 (D=%d)", D);
  if ((rc = check_heads(Hq, Hkv))) return rc;
  if (B < 0 || T < 0 || T_out < 0)
    return fail(ORTHROS_EINVAL, "negative size (B=%d, T=%d, T_out=%d)", B, T, T_out);
  if (T_out > T) return fail(ORTHROS_EINVAL, "T_out=%d exceeds T=%d", T_out, T);
  if (W < 1) return fail(ORTHROS_EINVAL, "window W=%d must be >= 1", W);
  if (cap < T || cap > INT32_MAX)
    return fail(ORTHROS_EINVAL, "cap=%lld must hold the T=%d rows", (long long)cap, T);
  HeadMap map;
  HeadGroups groups;
  if ((rc = build_maps(head_map, Hq, Hkv, &map, &groups))) return rc;
  {
    int seen[kMaxHeads] = {0};
    for (int g = 0; g < groups.n_groups; ++g) ++seen[groups.kv[g]];
    for (int g = 0; g < Hkv; ++g)
      if (seen[g] != 1)
        return fail(ORTHROS_EUNSUPPORTED,
                    "the backward needs 1..%d query heads on every KV head "
                    "(KV head %d has %s)", kMaxGroupSize, g,
                    seen[g] ? "more" : "none");
  }
  if (B == 0 || T == 0) return ORTHROS_OK;
  if (!q_pre || !alpha || !beta || !k_cache || !v_cache || !o || !d_o ||
      !dq_pre || !dk || !dv || !d_alpha || !d_beta)
    return fail(ORTHROS_EINVAL, "null pointer argument");
  if (T_out > 0 && (!qx_pre || !alpha_x || !beta_x || !o_x || !d_ox || !dqx_pre ||
                    !d_alpha_x || !d_beta_x))
    return fail(ORTHROS_EINVAL, "null pointer argument (output stream)");
  int64_t n_elems;
  if (!tensor_elems(&n_elems, {B, Hkv, cap, D, 2}) ||
      !tensor_elems(&n_elems, {B, T, Hq, D, 2}))
    return fail(ORTHROS_EINVAL, "tensor size overflows");
  if (!mfma_eligible(dtype, D, T, {q_pre, k_cache, v_cache, o, d_o, dq_pre, dk, dv,
                                   alpha, beta, d_alpha, d_beta}) ||
      (T_out > 0 && !mfma_eligible(dtype, D, T, {qx_pre, o_x, d_ox, dqx_pre,
                                                 alpha_x, beta_x})))
    return fail(ORTHROS_EUNSUPPORTED,
                "the backward needs 16-byte aligned tensors and T <= 2^24");
  const BwdWs w = bwd_ws(B, T, T_out, Hq, D);
  if (!ws || ws_bytes < w.total)
    return fail(ORTHROS_EWORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, w.total);
  char *base = static_cast<char *>(ws);
  const int Wb = W < T ? W : T;
  const hipStream_t st = as_stream(stream);

  BwdStreamArgs sa;
  sa.q = (const uint16_t *)q_pre;
  sa.o = (const uint16_t *)o;
  sa.d_o = (const uint16_t *)d_o;
  sa.k_cache = (const uint16_t *)k_cache;
  sa.v_cache = (const uint16_t *)v_cache;
  sa.alpha = alpha;
  sa.beta = beta;
  sa.dq = (uint16_t *)dq_pre;
  sa.lse = (float *)(base + w.lse);
  sa.delta = (float *)(base + w.delta);
  sa.part = (float *)(base + w.part);
  sa.qa = (uint16_t *)(base + w.qa);
  sa.nrows = T;
  sa.Hq = Hq;
  sa.n_kv = Hkv;
  sa.n_keys = T;
  sa.W = Wb;
  sa.q_offset = 0;
  sa.cap = cap;
  hipError_t e = launch_bwd_dq(sa, groups, B, st);
  if (e != hipSuccess) return hip_fail("backward dq launch", e);
  if (T_out > 0) {
    BwdStreamArgs sx = sa;
    sx.q = (const uint16_t *)qx_pre;
    sx.o = (const uint16_t *)o_x;
    sx.d_o = (const uint16_t *)d_ox;
    sx.alpha = alpha_x;
    sx.beta = beta_x;
    sx.dq = (uint16_t *)dqx_pre;
    sx.lse = (float *)(base + w.lse_x);
    sx.delta = (float *)(base + w.delta_x);
    sx.part = (float *)(base + w.part_x);
    sx.qa = (uint16_t *)(base + w.qa_x);
    sx.nrows = T_out;
    sx.W = T;
    sx.q_offset = T - T_out;
    e = launch_bwd_dq(sx, groups, B, st);
    if (e != hipSuccess) return hip_fail("backward dq launch (output stream)", e);
  }
  BwdKvArgs ka;
  ka.qa = (const uint16_t *)(base + w.qa);
  ka.qax = (const uint16_t *)(base + w.qa_x);
  ka.d_o = (const uint16_t *)d_o;
  ka.d_ox = (const uint16_t *)d_ox;
  ka.k_cache = (const uint16_t *)k_cache;
  ka.v_cache = (const uint16_t *)v_cache;
  ka.lse = sa.lse;
  ka.delta = sa.delta;
  ka.lse_x = (float *)(base + w.lse_x);
  ka.delta_x = (float *)(base + w.delta_x);
  ka.dk = (uint16_t *)dk;
  ka.dv = (uint16_t *)dv;
  ka.T = T;
  ka.T_out = T_out;
  ka.Hq = Hq;
  ka.n_kv = Hkv;
  ka.W = Wb;
  ka.cap = cap;
  e = launch_bwd_dkv(ka, groups, B, st);
  if (e != hipSuccess) return hip_fail("backward dk/dv launch", e);
  e = launch_bwd_reduce(sa.part, d_alpha, d_beta, B, (T + 31) / 32, Hq, st);
  if (e == hipSuccess && d_alpha_x && d_beta_x)
    e = launch_bwd_reduce((float *)(base + w.part_x), d_alpha_x, d_beta_x, B,
                          (T_out + 31) / 32, Hq, st);
  if (e != hipSuccess) return hip_fail("backward reduce launch", e);
  return ORTHROS_OK;
}
