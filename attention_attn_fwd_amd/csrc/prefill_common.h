// Tile schedule of the prefill kernels: which (batch, kv-head) group, rows and
// key-range piece a workgroup takes, and the positions its rows span.
#pragma once

#include "attn_internal.h"

namespace attn {

// A tile: rows [r0, r0 + 128) of the row list of one (batch, kv-head) group
// (n_rows rows, row r = query row r % Q of head h_base + r / Q), and the
// piece `split` of its key range.  `part` numbers (group, split, tile)
// triples; it indexes the partial states of a split pass.
struct PrefillTile {
  int b, kh, h_base, r0, n_rows, split, part, dv_part;
};

// Tile `rem` of group `grp` (rank order: heaviest causal tile first, heads
// fastest among per-head tiles).
__device__ __forceinline__ PrefillTile prefill_tile_of(const Params& p, int grp, int rem) {
  PrefillTile t;
  t.b = grp / p.Hkv;
  t.kh = grp - t.b * p.Hkv;
  if (prefill_packed(p.Q, p.group)) {
    t.h_base = t.kh * p.group;
    t.n_rows = p.group * p.Q;
    t.r0 = (prefill_group_tiles(p.Q, p.group) - 1 - rem) * kPrefillBM;
  } else {
    const int n_qt = (p.Q + kPrefillBM - 1) / kPrefillBM;
    const int qrank = rem / p.group;
    t.h_base = t.kh * p.group + (rem - qrank * p.group);
    t.n_rows = p.Q;
    t.r0 = (n_qt - 1 - qrank) * kPrefillBM;
  }
  t.split = 0;
  t.part = 0;
  t.dv_part = 0;
  return t;
}

// Block index -> tile.  A virtual group is a (piece, group) pair.  When the
// virtual groups divide evenly over the device's XCDs (workgroup i of a
// launch runs on XCD i % n_xcd), each XCD gets whole virtual groups and
// finishes one (all its tiles, heaviest first, and both output-channel parts
// of a tile next to each other) before the next, so the workgroups resident
// on an XCD stream the same K/V through its L2; otherwise the order is
// heaviest tile first with virtual groups fastest.
__device__ __forceinline__ PrefillTile prefill_tile(const Params& p) {
  const int x = blockIdx.x;
  const int vgroups = p.B * p.Hkv * p.n_split;
  const int per_grp = prefill_group_tiles(p.Q, p.group);
  const int per_vg = per_grp * p.dv_parts;  // workgroups per virtual group
  int vg, remx;
  const int nx = p.n_xcd;
  if (nx > 1 && vgroups % nx == 0) {
    const int slot = x / nx, xcd = x - slot * nx;
    const int gi = slot / per_vg;
    remx = slot - gi * per_vg;
    vg = gi * nx + xcd;
  } else {
    remx = x / vgroups;
    vg = x - remx * vgroups;
  }
  const int rem = remx / p.dv_parts, dv_part = remx - rem * p.dv_parts;
  // Split-major: virtual group vg is piece vg / groups of group vg % groups,
  // so an XCD gets every piece of its groups (pieces late in a range are
  // often empty; dealing pieces to XCDs would leave the XCDs that got the
  // first pieces with most of the work).
  const int groups = p.B * p.Hkv;
  const int split = vg / groups, grp = vg - split * groups;
  PrefillTile t = prefill_tile_of(p, grp, rem);
  t.split = split;
  t.dv_part = dv_part;
  t.part = (grp * p.n_split + split) * per_grp + rem;  // a row's pieces lie 128 rows apart
  return t;
}

// Query rows r0 .. r1 of a row list (r0 <= r1) lie at positions q + delta with
// q in [qlo, qhi]: the exact range when the rows belong to one head, else the
// whole head.
__device__ __forceinline__ void row_q_range(int r0, int r1, int Q, int* qlo, int* qhi) {
  if (r0 / Q == r1 / Q) {
    *qlo = r0 % Q;
    *qhi = r1 % Q;
  } else {
    *qlo = 0;
    *qhi = Q - 1;
  }
}

}  // namespace attn
