// Host-side sizing of the split-KV calls: rows per workgroup, keys per
// chunk and the workspace layout. Pure host code (no device, no HIP calls),
// shared by the workspace query and the launches, so that the size a caller
// is told to allocate is the size the kernels use.
#include "common.h"

namespace orthros {

int splitkv_rows(int n_streams, int n_pos, int gsize) {
  return n_streams * n_pos * gsize;
}

// Keys per workgroup: a power of two from 256 to 2048, the largest that still
// gives every compute unit its two resident workgroups. The compute-unit
// count is fixed at 256 (every gfx950 part this library targets has 256)
// rather than queried, so that the chunk, and with it the workspace size,
// depends on the sizes only: orthros_workspace_bytes is a pure host function
// and its answer is the same on every device. At most 2048 keys, so a chunk
// of a paged cache spans at most 64 pages (one block-table entry per lane).
// Long caches then run in whole rounds of long-lived workgroups; short ones
// still spread over the whole chip.
int splitkv_pick_chunk(int B, int n_groups, int64_t max_len) {
  constexpr int64_t kAssumedCUs = 256;
  constexpr int64_t kResidentSlots = 2 * kAssumedCUs;
  int chunk = 2048;
  while (chunk > 256 &&
         (int64_t)B * n_groups * ((max_len + chunk - 1) / chunk) < kResidentSlots)
    chunk /= 2;
  return chunk;
}

// Workspace layout: per-batch old lengths (int32, padded to 256 bytes), then
// (max, sum) float pairs of every partial, padded to 64 floats, then the
// unnormalised output rows. Must agree with the offsets set by the caller.
size_t splitkv_ws_bytes(int B, int n_groups, int rows, int n_chunks, int Dh) {
  const size_t parts = (size_t)B * n_groups * n_chunks * rows;
  const size_t len_bytes = ((size_t)B * 4 + 255) / 256 * 256;
  const size_t ml_floats = (parts * 2 + 63) / 64 * 64;
  return len_bytes + (ml_floats + parts * (size_t)Dh) * 4;
}

}  // namespace orthros
