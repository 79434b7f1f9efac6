// mla_plan.hpp -- host-side work plan of one mla_decode call: head padding,
// split-T chunking and the workspace layout.  A pure function of the
// parameters, so mla_decode_workspace_size() never touches the device.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// MI355X: 256 compute units in 8 XCDs.  The split count targets a few
// workgroups per CU; it is a design constant so the plan stays host-only.
constexpr int kTargetCUs = 256;
constexpr int kTileRows = 32;      // cache rows per LDS tile of the attention kernel
constexpr int kMinChunkRows = 64;  // smallest split-T chunk

struct DecodePlan {
  int heads_padded;  // H rounded up to a multiple of 32 (one 32-head block per wave)
  int head_blocks;   // heads_padded / 32
  int chunk_rows;    // rows of the selection handled by one split (multiple of 32)
  int num_splits;    // splits per sequence (upper bound; the kernels skip empty ones)
  size_t off_qt, off_part_o, off_part_ml, off_olat, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline DecodePlan make_decode_plan(const mla_params& p) {
  DecodePlan d{};
  const int B = p.batch, H = p.num_heads;
  d.heads_padded = (H + 31) / 32 * 32;
  d.head_blocks = d.heads_padded / 32;
  const long long n_max = p.topk > 0 ? p.topk : p.max_seq_len;
  const long long rows_total = (long long)B * n_max;
  const long long target_groups = 2LL * kTargetCUs;
  long long chunk = (rows_total + target_groups - 1) / target_groups;
  chunk = (chunk + kTileRows - 1) / kTileRows * kTileRows;
  if (chunk < kMinChunkRows) chunk = kMinChunkRows;
  const long long n_cap = (n_max + kTileRows - 1) / kTileRows * kTileRows;
  if (chunk > n_cap) chunk = n_cap > 0 ? n_cap : kTileRows;
  d.chunk_rows = (int)chunk;
  d.num_splits = n_max > 0 ? (int)((n_max + chunk - 1) / chunk) : 1;
  size_t off = 0;
  d.off_qt = off;
  off = align256(off + (size_t)B * d.heads_padded * 576 * 2);
  d.off_part_o = off;  // bf16 [B][H][num_splits][512]
  off = align256(off + (size_t)B * d.num_splits * H * 512 * 2);
  d.off_part_ml = off;  // fp32 [B][H][num_splits][2]
  off = align256(off + (size_t)B * d.num_splits * H * 2 * 4);
  d.off_olat = off;
  off = align256(off + (size_t)B * H * 512 * 2);
  d.bytes = off;
  return d;
}

}  // namespace mla
