// mla_plan.hpp -- host-side work plan of one mla_decode call: head padding,
// split-T chunking and the workspace layout.  A pure function of the
// parameters, so mla_decode_workspace_size() never touches the device.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// MI355X: 256 compute units in 8 XCDs.  The attention kernel runs at most one
// workgroup per CU (its LDS ring takes most of the 160 KB) and the plan aims
// for one round of them; a design constant so the plan stays host-only.
constexpr int kTargetCUs = 256;
constexpr int kTileRows = 32;           // cache rows per LDS tile of the attention kernel
constexpr int kMaxTopkGroupTiles = 32;  // top-k: tiles per workgroup (index staging bound)

// Work split of the attention kernel.  Work item b has t_b tiles of 32
// selected entries.  For a tile budget S, item b gets k_b = ceil(t_b / S)
// workgroups, and workgroup i = w_b + p (w_b = k_0 + ... + k_{b-1}) takes its
// tiles [floor(p t_b / k_b), floor((p+1) t_b / k_b)) and writes its partial
// (O, m, l) into slot i.  S is the smallest budget with sum k_b <= 256 (one
// round), at least min_group_tiles (2: a workgroup's fixed costs, the query
// load and the 128 KB partial, then cover at least two tiles; 4 with a top-k
// selection, whose gathered tiles are cheap next to the partial), and at most
// 32 with a top-k selection.
// The lengths live on the device, so w_b and S are computed there; the sizes
// here are upper bounds.
struct DecodePlan {
  // Work items.  Normally each query token (batch x seqlen_q of them) is an item
  // with H query rows.  With s > 1 query tokens, a dense selection and s x H <=
  // 128, the s tokens of a sequence share one item instead: its rows are the
  // packed (token i, head h) pairs, row i H + h, so every tile of the sequence
  // is read and scored once for all of them (each row masked at its token's
  // own limit).
  long long items;      // work items: batch (packed) or batch x seqlen_q
  int pack_s;           // tokens per item: seqlen_q when packed, else 1
  int rows;             // query rows per item: pack_s x H
  int heads_padded;     // rows rounded up to a multiple of 32 (one 32-row block per wave)
  int head_blocks;      // heads_padded / 32
  int head_split;       // attention workgroups per plan workgroup (1, 2 or 4), each
                        // with head_blocks / head_split of the head blocks
  long long max_groups; // plan workgroups (upper bound of sum k_b; the attention grid is
                        // max_groups x head_split)
  int min_group_tiles;  // lower bound of S
  long long max_tiles;  // tiles of the longest possible selection
  size_t off_qt, off_part_o, off_part_ml, off_olat, off_wcum, off_rec, off_slot, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline DecodePlan make_decode_plan(const mla_params& p) {
  DecodePlan d{};
  // B: work items (each planned as a sequence of its own over the rows its
  // last token sees), batch x seqlen_q or, with packed tokens, batch
  // (64-bit: the product is formed before the caller's limit on it is known
  // to hold; mla_decode rejects batch x seqlen_q > 65535)
  const int sq = p.seqlen_q > 0 ? p.seqlen_q : 1;
  const int H = p.num_heads;
  const bool pack = sq > 1 && p.topk == 0 && (long long)sq * H <= 128;
  d.pack_s = pack ? sq : 1;
  d.items = pack ? (long long)p.batch : (long long)p.batch * sq;
  d.rows = d.pack_s * H;
  const long long B = d.items;
  d.heads_padded = (d.rows + 31) / 32 * 32;
  d.head_blocks = d.heads_padded / 32;
  const long long n_max = p.topk > 0 ? p.topk : p.max_seq_len;
  d.max_tiles = (n_max + kTileRows - 1) / kTileRows;
  d.min_group_tiles = p.topk > 0 ? 4 : 2;
  long long G = B > kTargetCUs ? B : (long long)kTargetCUs;
  if (p.topk > 0) {
    const long long capped = B * ((d.max_tiles + kMaxTopkGroupTiles - 1) / kMaxTopkGroupTiles);
    if (G < capped) G = capped;
  }
  // no sequence takes more than ceil(max_tiles / min_group_tiles) workgroups
  const long long bound = B * ((d.max_tiles + d.min_group_tiles - 1) / d.min_group_tiles);
  if (G > bound) G = bound;
  G = (G + 7) / 8 * 8;  // whole rows of the XCD placement
  d.max_groups = G;
  // Few workgroups (a short batch): split each one's heads over up to four
  // workgroups, so that more CUs load the query and share the tile loads.
  // Each CU keeps only a limited amount of loads in flight, and every
  // workgroup of a token loads the whole absorbed query (144 KB at 128 heads).
  d.head_split = 1;
  while (d.head_split < 4 && d.head_blocks % (2 * d.head_split) == 0 &&
         G * 2 * d.head_split <= kTargetCUs)
    d.head_split *= 2;
  size_t off = 0;
  d.off_qt = off;  // bf16 [items][heads_padded][576], in the attention kernel's fragment order
  off = align256(off + (size_t)B * d.heads_padded * 576 * 2);
  d.off_part_o = off;  // bf16 [max_groups][heads_padded][512], in fragment order
  off = align256(off + (size_t)G * d.heads_padded * 512 * 2);
  d.off_part_ml = off;  // fp32 [max_groups][rows][2]
  off = align256(off + (size_t)G * d.rows * 2 * 4);
  d.off_olat = off;  // bf16 [items][rows][512] = [batch x seqlen_q tokens][H][512]
  off = align256(off + (size_t)B * d.rows * 512 * 2);
  d.off_wcum = off;  // int32 [items + 1]: w_b, w_B = workgroups in use
  off = align256(off + ((size_t)B + 1) * 4);
  d.off_rec = off;  // int32 [max_groups][4]: sequence (-1: unused), first tile, end tile, length
  off = align256(off + (size_t)G * 16);
  d.off_slot = off;  // int32 [max_groups]: plan slot (partial index) run by each workgroup
  off = align256(off + (size_t)G * 4);
  d.bytes = off;
  return d;
}

}  // namespace mla
