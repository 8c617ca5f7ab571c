// Host-side sizing of the split-KV calls: rows per workgroup, keys per
// chunk and the workspace layout. Pure host code (no device, no HIP calls),
// shared by the workspace query and the launches, so that the size a caller
// is told to allocate is the size the kernels use.
#include "common.h"

namespace orthros {

int splitkv_rows(int n_streams, int n_pos, int gsize) {
  return n_streams * n_pos * gsize;
}

// Keys per workgroup: a power of two from 256 to max_chunk, the largest that
// still gives every compute unit a workgroup. The compute-unit count is
// fixed at 256 (every gfx950 part this library targets has 256) rather than
// queried, so that the chunk, and with it the workspace size, depends on the
// sizes only: orthros_workspace_bytes is a pure host function and its answer
// is the same on every device. One long-lived workgroup per compute unit
// streams as fast as two (a measured pure-read kernel over the 512 MiB of a
// 128K cache ran at the same rate with 256 workgroups of 4096 keys as with
// 512 of 2048, and faster than with more, smaller ones), and the fewer the
// chunks, the less the last workgroup has to combine. Decode steps cap the
// chunk at 2048 keys, so that a chunk of a paged cache spans at most 64
// pages (one block-table entry per lane).
int splitkv_pick_chunk(int B, int n_groups, int64_t max_len, int max_chunk) {
  constexpr int64_t kAssumedCUs = 256;
  int chunk = max_chunk;
  while (chunk > 256 &&
         (int64_t)B * n_groups * ((max_len + chunk - 1) / chunk) < kAssumedCUs)
    chunk /= 2;
  return chunk;
}

// Workspace layout: the arrival counters (int32, one per (batch, head group)
// and one per batch entry, padded to 256 bytes; they depend on B and the
// head grouping only), the old lengths of a two-launch decode step (int32
// per batch entry, padded to 256 bytes), then (max, sum) float pairs of
// every partial, padded to 64 floats, then the unnormalised output rows.
// Must agree with the offsets set by the caller.
size_t splitkv_counter_bytes(int B, int n_groups) {
  return ((size_t)B * (n_groups + 1) * 4 + 255) / 256 * 256;
}

size_t splitkv_len_bytes(int B) { return ((size_t)B * 4 + 255) / 256 * 256; }

size_t splitkv_ws_bytes(int B, int n_groups, int rows, int n_chunks, int Dh) {
  const size_t parts = (size_t)B * n_groups * n_chunks * rows;
  const size_t ml_floats = (parts * 2 + 63) / 64 * 64;
  return splitkv_counter_bytes(B, n_groups) + splitkv_len_bytes(B) +
         (ml_floats + parts * (size_t)Dh) * 4;
}

// One launch when the chip holds the whole grid at once (two workgroups
// per compute unit, 256 compute units): the last workgroup of each group
// then merges while no other work waits for its slot.
bool splitkv_fused(int B, int n_groups, int n_chunks) {
  return (int64_t)B * n_groups * n_chunks <= 512;
}

}  // namespace orthros
