// Forward pass of one Orthros attention layer (pages: "Orthros: Phase-Aware
// Heterogeneous Attention for Efficient Transformers", paper text §3.1, the
// layer description around Algorithm 1 and Figure 1(b)).
//
// The input holds the T base tokens followed by the T_out output-specific
// tokens of each sequence. Every row is projected with the shared W_Q; the
// base rows alone are projected with W_K and W_V and fill the cache; the base
// queries run the sliding window, the output queries the global
// cross-attention over that cache; the two outputs, in the same row order
// as the input, go through W_O. The projections are hipBLASLt GEMMs, the
// attention is this library's kernels, and the row order of the input is
// kept in every intermediate, so no concatenation is ever copied.
#include <stdio.h>

#include "../../include/orthros.h"
#include "common.h"

namespace orthros {
// C[M, N] = A[M, K] Wt[N, K]^T, row-major bf16 (weights stored out x in).
int gemm_bf16(const void *A, const void *Wt, void *C, int64_t M, int64_t N,
              int64_t K, void *ws, size_t ws_bytes, hipStream_t stream,
              char *msg, size_t msg_len);
int api_error(int code, const char *msg);
}  // namespace orthros

using namespace orthros;

namespace {

constexpr size_t kGemmWorkspace = size_t(64) << 20;

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct LayerWs {
  size_t q_all, k, v, o_cat, xattn_ws, xattn_bytes, xattn_counter_bytes,
      gemm_ws, total;
};

// Workspace layout, reused by the batch entries one after the other.
bool layer_ws(int T, int T_out, int Hq, int Hkv, int D, LayerWs *w) {
  const size_t M = (size_t)T + T_out;
  size_t off = 0;
  w->q_all = off;
  off += align256(M * Hq * D * 2);
  w->k = off;
  off += align256((size_t)T * Hkv * D * 2);
  w->v = off;
  off += align256((size_t)T * Hkv * D * 2);
  w->o_cat = off;
  off += align256(M * Hq * D * 2);
  w->xattn_bytes = T_out > 0 ? orthros_workspace_bytes(ORTHROS_OP_GLOBAL_XATTN, 1, Hq,
                                                       Hkv, D, T_out, T, nullptr)
                             : 0;
  w->xattn_counter_bytes = T_out > 0 ? orthros_workspace_counter_bytes(
                                           ORTHROS_OP_GLOBAL_XATTN, 1, Hq, Hkv,
                                           D, T_out, T, nullptr)
                                     : 0;
  w->xattn_ws = off;
  off += align256(w->xattn_bytes);
  w->gemm_ws = off;
  off += kGemmWorkspace;
  w->total = off;
  return true;
}

// Sets one cache length and zeroes the n int32 arrival counters at the start
// of the cross-attention workspace (the split-KV kernel expects them zero;
// the layer workspace may hold anything on entry). One block of 64 threads.
__global__ void set_len_kernel(int32_t *len, int32_t v, int32_t *counters,
                               int n) {
  if (threadIdx.x == 0) *len = v;
  for (int i = threadIdx.x; i < n; i += 64) counters[i] = 0;
}

int fail_msg(int code, const char *fmt, long long a = 0, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, a, b);
  return api_error(code, buf);
}

}  // namespace

extern "C" size_t orthros_layer_workspace_bytes(int B, int T, int T_out,
                                                int d_model, int Hq, int Hkv,
                                                int D) {
  (void)B;
  (void)d_model;
  if (T < 1 || T_out < 0 || T_out > T || Hq < 1 || Hkv < 1 || D < 1) return 0;
  LayerWs w;
  layer_ws(T, T_out, Hq, Hkv, D, &w);
  return w.total;
}

extern "C" int orthros_layer_forward(
    const void *x, const void *w_q, const void *w_k, const void *w_v,
    const void *w_o, const float *alpha, const float *beta,
    const float *alpha_x, const float *beta_x, void *k_cache, void *v_cache,
    int32_t *cache_len, void *y, int B, int T, int T_out, int d_model, int Hq,
    int Hkv, int D, int64_t cap, int W, void *ws, size_t ws_bytes,
    void *stream) {
  api_error(ORTHROS_OK, "");
  if (B < 0) return fail_msg(ORTHROS_EINVAL, "negative batch B=%lld", B);
  if (T < 1 || T_out < 0 || T_out > T)
    return fail_msg(ORTHROS_EINVAL, "need 1 <= T and 0 <= T_out <= T (T=%lld, T_out=%lld)",
                    T, T_out);
  if (d_model < 1) return fail_msg(ORTHROS_EINVAL, "d_model=%lld must be >= 1", d_model);
  if (Hq < 1 || Hkv < 1 || Hq > ORTHROS_MAX_HEADS || Hkv > ORTHROS_MAX_HEADS ||
      Hq % Hkv != 0)
    return fail_msg(ORTHROS_EINVAL, "heads Hq=%lld, Hkv=%lld: need Hkv | Hq, both <= 128",
                    Hq, Hkv);
  if (D < 2 || D > ORTHROS_MAX_D || D % 2)
    return fail_msg(ORTHROS_EUNSUPPORTED, "head dimension D=%lld", D);
  if (W < 1) return fail_msg(ORTHROS_EINVAL, "window W=%lld must be >= 1", W);
  if (cap < T || cap > INT32_MAX)
    return fail_msg(ORTHROS_EINVAL, "cap=%lld must hold the T=%lld rows", cap, T);
  if (B == 0) return ORTHROS_OK;
  if (!x || !w_q || !w_k || !w_v || !w_o || !alpha || !beta || !k_cache ||
      !v_cache || !cache_len || !y || (T_out > 0 && (!alpha_x || !beta_x)))
    return fail_msg(ORTHROS_EINVAL, "null pointer argument");
  LayerWs lw;
  layer_ws(T, T_out, Hq, Hkv, D, &lw);
  if (!ws || ws_bytes < lw.total)
    return fail_msg(ORTHROS_EWORKSPACE, "workspace of %lld bytes, need %lld",
                    (long long)ws_bytes, (long long)lw.total);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char *base = static_cast<char *>(ws);
  char *q_all = base + lw.q_all, *kp = base + lw.k, *vp = base + lw.v;
  char *o_cat = base + lw.o_cat;
  const int64_t M = (int64_t)T + T_out;
  const int64_t HqD = (int64_t)Hq * D, HkvD = (int64_t)Hkv * D;
  char msg[256];
  for (int b = 0; b < B; ++b) {
    const char *xb = static_cast<const char *>(x) + (size_t)b * M * d_model * 2;
    char *yb = static_cast<char *>(y) + (size_t)b * M * d_model * 2;
    const size_t slab = (size_t)Hkv * cap * D * 2;
    char *kc = static_cast<char *>(k_cache) + (size_t)b * slab;
    char *vc = static_cast<char *>(v_cache) + (size_t)b * slab;
    // projections: q of every row, k and v of the base rows
    if (gemm_bf16(xb, w_q, q_all, M, HqD, d_model, base + lw.gemm_ws,
                  kGemmWorkspace, st, msg, sizeof(msg)) ||
        gemm_bf16(xb, w_k, kp, T, HkvD, d_model, base + lw.gemm_ws,
                  kGemmWorkspace, st, msg, sizeof(msg)) ||
        gemm_bf16(xb, w_v, vp, T, HkvD, d_model, base + lw.gemm_ws,
                  kGemmWorkspace, st, msg, sizeof(msg)))
      return api_error(ORTHROS_EHIP, msg);
    // the cache of this sequence is filled from row 0
    hipLaunchKernelGGL(set_len_kernel, dim3(1), dim3(64), 0, st, cache_len + b,
                       0, (int32_t *)(base + lw.xattn_ws),
                       (int)(lw.xattn_counter_bytes / 4));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail_msg(ORTHROS_EHIP, "length reset launch failed");
    int rc = orthros_kv_append(kc, vc, cache_len + b, kp, vp, 1, T, Hkv, D, cap,
                               ORTHROS_BF16, stream);
    if (rc) return rc;
    rc = orthros_swa_prefill(q_all, alpha, beta, kc, vc, o_cat, 1, T, Hq, Hkv, D,
                             cap, W, nullptr, ORTHROS_BF16, stream);
    if (rc) return rc;
    if (T_out > 0) {
      rc = orthros_global_xattn(q_all + (size_t)T * HqD * 2, alpha_x, beta_x, kc,
                                vc, o_cat + (size_t)T * HqD * 2, 1, T - T_out,
                                T_out, Hq, Hkv, D, cap, nullptr, ORTHROS_BF16,
                                base + lw.xattn_ws, lw.xattn_bytes, stream);
      if (rc) return rc;
    }
    if (gemm_bf16(o_cat, w_o, yb, M, d_model, HqD, base + lw.gemm_ws,
                  kGemmWorkspace, st, msg, sizeof(msg)))
      return api_error(ORTHROS_EHIP, msg);
  }
  return ORTHROS_OK;
}
