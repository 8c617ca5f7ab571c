// Host-only stand-ins for the kernel launchers (test infrastructure): the
// C-ABI layer (orthros_api.cpp) and the split-KV sizing (splitkv_plan.cpp)
// are linked against these instead of the HIP kernels, so that the host
// validation and the workspace layout can be run under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.
//
// Every launcher counts its calls (a rejected call must launch nothing).
// The split-KV launcher also writes every byte of the workspace regions the
// kernels use (counters, partial maxima and sums, partial outputs), computed
// from the arguments it receives: with a workspace allocated at exactly the
// size orthros_workspace_bytes returned, any region past its end is a heap
// overflow that the sanitizer reports.
#include <string.h>

#include "../../include/orthros.h"
#include "../../long_context_prefill_swa_amd/csrc/common.h"

extern "C" int stub_launches = 0;
extern "C" int stub_splitkv_launches = 0;

namespace orthros {

static int g_flag = 0;

hipError_t device_flag_ptr(int **out) {
  *out = &g_flag;
  return hipSuccess;
}

hipError_t launch_kv_append(void *, void *, int32_t *, const void *,
                            const void *, int, int, int, int, int64_t, int64_t,
                            int *, int, hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_rowwise(const void *, const float *, const float *,
                          const void *, const void *, void *, int, int, int,
                          int, int, int64_t, int64_t, int64_t, int,
                          const int32_t *, const HeadMap &, int, hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_kv_append_paged(void *, void *, int32_t *, const void *,
                                  const void *, int, int, int, int, int64_t,
                                  int, const int32_t *, int, int *,
                                  hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_len_bump(int32_t *, int, int, int64_t, hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_band_mfma(const void *, const float *, const float *,
                            const void *, const void *, void *, int, int, int,
                            int64_t, int64_t, int, const HeadGroups &, int,
                            hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_bwd_dq(const BwdStreamArgs &, const HeadGroups &, int,
                         hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_bwd_dkv(const BwdKvArgs &, const HeadGroups &, int,
                          hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_bwd_reduce(const float *, float *, float *, int, int, int,
                             hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_band_persist(const void *, const float *, const float *,
                               const void *, const void *, void *, int, int,
                               int, int, int64_t, int, const HeadGroups &, int,
                               hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_band_roll(const void *, const float *, const float *,
                            const void *, const void *, void *, int, int, int,
                            int64_t, int, const HeadGroups &, int,
                            hipStream_t) {
  ++stub_launches;
  return hipSuccess;
}

hipError_t launch_splitkv(const SplitKVArgs &a, const HeadGroups &groups,
                          hipStream_t) {
  ++stub_launches;
  ++stub_splitkv_launches;
  const int rows = splitkv_rows(a.n_streams, a.n_pos, groups.gsize);
  const int64_t parts = (int64_t)a.B * groups.n_groups * a.n_chunks * rows;
  if (a.ws_acc_offset < 2 * parts) return hipErrorInvalidValue;  // overlap
  const int64_t n_counters = (int64_t)a.B * (groups.n_groups + 1);
  if ((char *)a.ws_len < (char *)(a.counters + n_counters) ||
      (char *)a.ws < (char *)(a.ws_len + a.B))
    return hipErrorInvalidValue;
  // the kernel's counters are read-modify-write and left as they were
  for (int64_t i = 0; i < n_counters; ++i) a.counters[i] += 0;
  memset(a.ws_len, 0x5a, sizeof(int32_t) * (size_t)a.B);
  memset(a.ws, 0x5a, sizeof(float) * 2 * (size_t)parts);
  memset(a.ws + a.ws_acc_offset, 0x5a, sizeof(float) * 128 * (size_t)parts);
  return hipSuccess;
}

// The no-allocation scratch array: a host array of the same size, zero at
// load like the device one.
static unsigned char host_scratch[ORTHROS_NOALLOC_SCRATCH_BYTES]
    __attribute__((aligned(256)));

hipError_t noalloc_scratch_ptr(void **out) {
  *out = host_scratch;
  return hipSuccess;
}

}  // namespace orthros
