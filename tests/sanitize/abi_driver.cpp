// Host sanitizer driver for the C ABI (test infrastructure): argument
// validation and split-KV workspace sizing of include/orthros.h, linked
// against host-only launcher stand-ins (abi_stubs.cpp) and run under
// AddressSanitizer and UndefinedBehaviorSanitizer. Checks:
//  * rejected calls return the documented code and launch nothing;
//  * a workspace of exactly orthros_workspace_bytes(...) bytes, for default
//    and uneven head maps, is accepted, and every region the split-KV
//    kernels use lies inside it (the stand-in writes all of it); one byte
//    less is rejected.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/orthros.h"

extern "C" int stub_launches;
extern "C" int stub_splitkv_launches;

static int failures = 0;
#define CHECK(c, ...) do { if (!(c)) { ++failures; \
    fprintf(stderr, "FAIL line %d: ", __LINE__); fprintf(stderr, __VA_ARGS__); \
    fprintf(stderr, " [%s]\n", orthros_last_error()); } } while (0)

static void *const F = (void *)0x100000;   // aligned, never dereferenced

static void sizing(int op, int B, int Hq, int Hkv, int T_out, int64_t len,
                   const int32_t *map) {
  const size_t need = orthros_workspace_bytes(op, B, Hq, Hkv, 128, T_out, len,
                                              map);
  CHECK(need > 0, "op %d B=%d Hq=%d Hkv=%d: no workspace size", op, B, Hq, Hkv);
  const size_t cb = orthros_workspace_counter_bytes(op, B, Hq, Hkv, 128, T_out,
                                                    len, map);
  CHECK(cb >= (size_t)B * 8 && cb % 256 == 0 && cb < need,
        "op %d B=%d: counter bytes %zu of %zu", op, B, cb, need);
  for (int exact = 0; exact < 2; ++exact) {
    const size_t nb = exact ? need : need - 1;
    void *ws = calloc(nb, 1);  // zero counters, as the calls require
    const int before = stub_splitkv_launches;
    int rc;
    if (op == ORTHROS_OP_GLOBAL_XATTN)
      rc = orthros_global_xattn(F, (float *)F, (float *)F, F, F, F, B,
                                (int)len - T_out, T_out, Hq, Hkv, 128, len, map,
                                ORTHROS_BF16, ws, nb, NULL);
    else
      rc = orthros_decode_pair(F, F, (float *)F, (float *)F, (float *)F,
                               (float *)F, F, F, F, F, (int32_t *)F, F, F, B,
                               Hq, Hkv, 128, len + 7, len, 16, map,
                               ORTHROS_BF16, ws, nb, NULL);
    if (exact) {
      CHECK(rc == ORTHROS_OK, "exact workspace rejected (rc %d)", rc);
      CHECK(stub_splitkv_launches == before + 1, "no split-KV launch");
    } else {
      CHECK(rc == ORTHROS_EWORKSPACE, "short workspace accepted (rc %d)", rc);
      CHECK(stub_splitkv_launches == before, "launch on a short workspace");
    }
    free(ws);
  }
}

#define REJECT(call, code) do { const int n0 = stub_launches; \
    const int rc_ = (call); \
    CHECK(rc_ == (code), #call " returned %d", rc_); \
    CHECK(stub_launches == n0, #call " launched"); } while (0)

int main() {
  const int32_t uneven[6] = {0, 0, 0, 1, 2, 2};
  const int32_t five[5] = {0, 1, 1, 0, 1};
  const int32_t seven[8] = {1, 1, 1, 1, 1, 1, 1, 0};
  const int32_t bad[4] = {0, 1, 2, 0};
  for (int op = 1; op <= 2; ++op) {
    sizing(op, 1, 32, 8, 1, 131072, NULL);
    sizing(op, 64, 32, 8, 1, 33024, NULL);
    sizing(op, 3, 6, 3, 1, 999, uneven);
    sizing(op, 2, 5, 2, 1, 300, five);
    sizing(op, 2, 8, 2, 1, 5000, seven);
  }
  sizing(ORTHROS_OP_GLOBAL_XATTN, 2, 8, 2, 4, 3000, NULL);   // 16 rows
  CHECK(orthros_workspace_bytes(1, 1, 4, 2, 128, 1, 100, bad) == 0, "bad map");

  REJECT(orthros_swa_prefill(F, (float *)F, (float *)F, F, F, F, 1, 64, 4, 2,
                             128, 64, 0, NULL, ORTHROS_BF16, NULL),
         ORTHROS_EINVAL);                                        // W = 0
  REJECT(orthros_swa_prefill(F, (float *)F, (float *)F, F, F, F, 1, 64, 4, 2,
                             128, 63, 16, NULL, ORTHROS_BF16, NULL),
         ORTHROS_EINVAL);                                        // cap < T
  REJECT(orthros_swa_prefill(F, (float *)F, (float *)F, F, F, F, 1, 64, 4, 3,
                             128, 64, 16, NULL, ORTHROS_BF16, NULL),
         ORTHROS_EINVAL);                                        // 4 % 3
  REJECT(orthros_swa_prefill(F, (float *)F, (float *)F, F, F, F, 1, 64, 4, 2,
                             128, 64, 16, bad, ORTHROS_BF16, NULL),
         ORTHROS_EINVAL);                                        // map entry
  REJECT(orthros_swa_prefill(F, (float *)F, (float *)F, F, F, F, 1, 64, 4, 2,
                             257, 64, 16, NULL, ORTHROS_F32, NULL),
         ORTHROS_EUNSUPPORTED);                                  // D
  REJECT(orthros_swa_prefill(NULL, (float *)F, (float *)F, F, F, F, 1, 64, 4,
                             2, 128, 64, 16, NULL, ORTHROS_BF16, NULL),
         ORTHROS_EINVAL);                                        // null
  REJECT(orthros_kv_append(F, F, (int32_t *)F, F, F, 1, 65, 2, 128, 64,
                           ORTHROS_BF16, NULL), ORTHROS_ECAPACITY);
  REJECT(orthros_global_xattn(F, (float *)F, (float *)F, F, F, F, 1, 100, 1, 4,
                              2, 128, 100, NULL, ORTHROS_BF16, NULL, 0, NULL),
         ORTHROS_EINVAL);                                        // cap < T
  REJECT(orthros_global_xattn(F, (float *)F, (float *)F, F, F, F, 1, 100, 1, 4,
                              2, 128, 101, NULL, ORTHROS_BF16, NULL, 0, NULL),
         ORTHROS_EWORKSPACE);
  REJECT(orthros_decode_pair(F, F, (float *)F, (float *)F, (float *)F,
                             (float *)F, F, F, F, F, (int32_t *)F, F, F, 2, 4,
                             2, 128, 100, 101, 16, NULL, ORTHROS_BF16, NULL, 0,
                             NULL), ORTHROS_ECAPACITY);
  REJECT(orthros_decode_pair_paged(F, F, (float *)F, (float *)F, (float *)F,
                                   (float *)F, F, F, F, F, 16, 48,
                                   (int32_t *)F, 4, (int32_t *)F, F, F, 2, 4, 2,
                                   128, 100, 16, NULL, ORTHROS_BF16, NULL, 0,
                                   NULL), ORTHROS_EINVAL);       // page size
  REJECT(orthros_attn_backward(F, F, (float *)F, (float *)F, (float *)F,
                               (float *)F, F, F, F, F, F, F, F, F, F, F,
                               (float *)F, (float *)F, (float *)F, (float *)F,
                               1, 64, 65, 4, 2, 128, 64, 16, NULL,
                               ORTHROS_BF16, NULL, 0, NULL),
         ORTHROS_EINVAL);                                        // T_out > T
  // zero-sized calls succeed and launch nothing
  REJECT(orthros_swa_prefill(F, (float *)F, (float *)F, F, F, F, 0, 64, 4, 2,
                             128, 64, 16, NULL, ORTHROS_BF16, NULL), ORTHROS_OK);
  // an accepted window call launches exactly one kernel
  {
    const int n0 = stub_launches;
    CHECK(orthros_swa_prefill(F, (float *)F, (float *)F, F, F, F, 2, 300, 8, 2,
                              128, 300, 100, NULL, ORTHROS_BF16, NULL) == 0,
          "valid window call");
    CHECK(stub_launches == n0 + 1, "window launches");
  }
  // the no-allocation decode pair near its limit: the partials follow the
  // fixed counter region inside the static array (here the stand-in's host
  // array, every byte of the partials written)
  {
    const int n0 = stub_splitkv_launches;
    CHECK(orthros_decode_pair_noalloc(F, F, (float *)F, (float *)F, (float *)F,
                                      (float *)F, F, F, F, F, (int32_t *)F, F,
                                      F, 64, 32, 8, 128, 60007, 60000, 16, NULL,
                                      ORTHROS_BF16, NULL) == ORTHROS_OK,
          "no-allocation decode pair");
    CHECK(stub_splitkv_launches == n0 + 1, "no-allocation launch");
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("C-ABI sanitizer driver: ok\n");
  return 0;
}
