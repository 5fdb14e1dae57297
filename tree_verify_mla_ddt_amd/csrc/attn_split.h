// attn_split.h -- the work split of the verify-attention kernels, as plain
// integer arithmetic usable on the host and the device.
//
// The attention kernels cut the (request, 128-row tile, 32-key tile) work into
// contiguous ranges, one per workgroup; row tiles whose key range is cut are
// written as partial results to workspace slots and combined by the merge
// kernels.  Everything that decides which workgroup takes which tiles, which
// slot a partial result lands in and which slots the merge reads is here, so
// that a host program (the split checker) runs exactly the code the kernels
// run.
//
// The work is one stream of positions.  Each row tile with work occupies a
// segment of nkb + c positions: c positions that stand for the cost of
// starting the tile in a workgroup (query load, pipeline fill, partial output;
// a few key tiles' worth), then its nkb key tiles.  Ranges are equal cuts of
// the stream, so a range that crosses into a second row tile takes that many
// fewer key tiles.  c is 0 when every range lies inside one row tile anyway.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ddt {

constexpr int kTileKeys = 32;     // keys per tile
constexpr int kRowsPerWG = 128;   // rows per tile
constexpr int kMaxBatch = 512;    // requests the attention kernels take
constexpr int kXcds = 8;          // XCDs the workgroups are dealt to
constexpr int kMaxGrid = 1024;    // upper bound of the attention grid
constexpr int kUnitCost = 6;      // stream positions charged for starting a row tile

#define DDT_HD __host__ __device__ __forceinline__

DDT_HD int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Per-request quantities shared by the attention and merge kernels.
struct ReqInfo {
  int L;      // prefix length
  int nb;     // tree entries
  int nkb;    // key tiles
  int vt;     // row tiles holding at least one live row
};

// From the clamped prefix length and tree size.
DDT_HD ReqInfo req_info_ln(int L, int nb, int H, int RT) {
  ReqInfo r;
  r.L = L;
  r.nb = nb;
  r.nkb = (r.L + r.nb + kTileKeys - 1) / kTileKeys;
  const long long live_rows = (long long)r.nb * H;
  long long vt = (live_rows + kRowsPerWG - 1) / kRowsPerWG;
  r.vt = (int)(vt > RT ? RT : vt);
  return r;
}

// Prefix length clamped to [0, max_kv], tree size to [0, min(Q, max_kv - L)].
DDT_HD void clamp_request(int prefix_len, int n_nodes, int Q, int max_kv, int& L, int& nb) {
  L = clampi(prefix_len, 0, max_kv);
  const int cap = Q < max_kv - L ? Q : max_kv - L;
  nb = clampi(n_nodes, 0, cap);
}

DDT_HD ReqInfo req_info(const int32_t* prefix_len, const int32_t* n_nodes, int b, int Q, int H,
                        int max_kv, int RT) {
  int L, nb;
  clamp_request(prefix_len[b], n_nodes[b], Q, max_kv, L, nb);
  return req_info_ln(L, nb, H, RT);
}

// Start of range g when W tiles are cut into G contiguous ranges.
DDT_HD long long range_start(long long g, long long W, long long G) { return (g * W) / G; }
// The range holding tile t (0 <= t < W).
DDT_HD long long range_owner(long long t, long long W, long long G) { return ((t + 1) * G - 1) / W; }

// Logical id of workgroup bl (0 <= bl < G): workgroups are dealt to the XCDs
// round-robin (bl % 8), so XCD x gets the consecutive logical ids
// [start_x, start_x + count_x) and consecutive ranges share an L2.
DDT_HD long long logical_gid(long long bl, long long G) {
  const long long xcd = bl % kXcds;
  return xcd * (G / kXcds) + (xcd < G % kXcds ? xcd : G % kXcds) + bl / kXcds;
}

// The split mode: U = B * vt row tiles with work when every request has the
// same row-tile and key-tile counts (`same`) and U >= G (the aligned split,
// launched with 2G workgroups), else -1 (one stream over all work, cut into G
// ranges).
DDT_HD long long split_mode(bool same, int vt0, int B, long long G) {
  const long long U = (long long)B * vt0;
  return (same && vt0 > 0 && U >= G) ? U : -1;
}

// Start cost c of a row tile in the stream (see the top of this file): 0 when
// the ranges never cross a row tile, that is when every row tile has the same
// key-tile count (`same`) and the number of row tiles in the cut stream
// divides G; else kUnitCost.  Under the aligned split (mode >= 0) only the
// leftover units r = mode mod G form a cut stream.
DDT_HD int unit_cost(long long mode, bool same, long long units, long long G) {
  if (mode >= 0) {
    const long long r = mode % G;
    return (r == 0 || G % r == 0) ? 0 : kUnitCost;
  }
  return (same && units > 0 && G % units == 0) ? 0 : kUnitCost;
}

// Range [start, end) of the stream taken by the workgroup with logical id gid
// in the first (second = false) or second half of an aligned-split launch.
// Under the aligned split every unit is a segment of seg = nkb + c positions,
// unit u covering [u*seg, (u+1)*seg): the first G workgroups take q = U / G
// whole units each, the second G the r = U - q*G leftover units as one stream
// cut into G ranges.  Otherwise the whole stream Wtot is cut into G ranges
// (first half only).
DDT_HD void workgroup_range(long long mode, bool second, long long gid, long long Wtot, int seg,
                            long long G, long long& start, long long& end) {
  if (mode < 0) {
    start = range_start(gid, Wtot, G);
    end = range_start(gid + 1, Wtot, G);
    if (second) end = start;
    return;
  }
  const long long q = mode / G, r = mode - q * G;
  if (!second) {
    start = gid * q * seg;
    end = start + q * seg;
  } else {
    start = q * G * seg + range_start(gid, r * seg, G);
    end = q * G * seg + range_start(gid + 1, r * seg, G);
  }
}

// For a row tile with work, its place in the stream that holds it: S (start of
// its segment) and W (stream length); false for a whole unit of the aligned
// split (written directly).  pref: exclusive stream prefix over requests, with
// pref[B] the total; c: the start cost.
DDT_HD bool stream_place(long long mode, const long long* pref, int B, int b, int rt,
                         const ReqInfo& ri, long long G, int c, long long& S, long long& W) {
  const long long seg = (long long)ri.nkb + c;
  if (mode >= 0) {
    const long long q = mode / G, r = mode - q * G;
    const long long u = (long long)b * ri.vt + rt;
    if (u < q * G) return false;
    S = (u - q * G) * seg;
    W = r * seg;
    return true;
  }
  S = pref[b] + (long long)rt * seg;
  W = pref[B];
  return true;
}

// The ranges that hold a key tile of the row tile whose segment starts at S:
// g_first .. g_last (equal when one range holds them all).
DDT_HD void tile_owners(long long S, long long W, long long G, int nkb, int c, long long& g_first,
                        long long& g_last) {
  g_first = range_owner(S + c, W, G);
  g_last = range_owner(S + c + nkb - 1, W, G);
}

// Workspace slot a workgroup writes a partial result of a cut row tile to:
// 2g for the tile holding the start of its range (its head), 2g + 1 for the
// one holding its end (a range cuts at most two row tiles).
DDT_HD long long partial_slot(long long gid, bool head) { return 2 * gid + (head ? 0 : 1); }

// The merge's rule: contributor gg (g_first <= gg <= g_last, the ranges
// holding key tiles of a row tile whose segment starts at S_u) wrote slot
// 2gg (its range starts inside the segment) or 2gg + 1, or nothing (empty
// range).
DDT_HD long long contributor_slot(long long gg, long long S_u, long long W, long long G) {
  const long long s0 = range_start(gg, W, G);
  const long long s1 = range_start(gg + 1, W, G);
  if (s0 == s1) return -1;
  return partial_slot(gg, s0 >= S_u);
}

// The narrow form runs four workgroups per range, one per 32-row quarter of
// its row tiles.  Workgroup bid serves range 8 * (bid / 32) + bid % 8 and
// quarter (bid / 8) % 4, so the four quarters of a range are dealt to the same
// XCD (bid % 8) and share its L2; the ranges are padded to a multiple of 8.
constexpr int kQuarters = kRowsPerWG / 32;
DDT_HD long long narrow_blocks(long long ranges) {
  return (long long)kQuarters * kXcds * ((ranges + kXcds - 1) / kXcds);
}
DDT_HD void narrow_place(long long bid, long long& range, int& quarter) {
  range = kXcds * (bid / (kXcds * kQuarters)) + bid % kXcds;
  quarter = (int)((bid / kXcds) % kQuarters);
}

// One unit (a row tile over a key range) of a workgroup's range: the unit
// whose segment holds stream position pos, inside request b (pref[b] <= pos <
// pref[b + 1]), with start cost c.  Key tiles [kb0, kb1) (empty when the
// range ends inside the start cost); adv: the positions of the range it
// takes, so that the next unit starts at pos + adv.
struct UnitPos {
  int rt, kb0, kb1;
  long long adv;
  bool complete;
};
DDT_HD UnitPos unit_at(long long pos, long long end, long long pref_b, const ReqInfo& ri, int c) {
  UnitPos u;
  const long long seg = (long long)ri.nkb + c;
  const long long off = pos - pref_b;
  u.rt = (int)(off / seg);
  const long long in = off % seg;                              // position inside the segment
  const long long stop = seg - in < end - pos ? seg : in + (end - pos);
  u.kb0 = in > c ? (int)(in - c) : 0;
  u.kb1 = stop > c ? (int)(stop - c) : 0;
  u.adv = stop - in;
  u.complete = u.kb0 == 0 && u.kb1 == ri.nkb;
  return u;
}

#undef DDT_HD

// The attention launch: grid (workgroups per half), row tiles per request and
// the workspace it needs.
struct AttnPlan {
  int grid;          // work ranges (attention workgroups per half of the wide form)
  int row_tiles;     // ceil(Q*H / 128)
  int num_cu;        // compute units the plan was made for
  bool narrow;       // four 32-row workgroups per range instead of one 128-row one
  size_t ws_bytes;   // workspace bytes needed
};

constexpr int kMinTilesPerWG = 3;    // key tiles per workgroup before splitting further
constexpr int kMinTilesNarrow = 4;   // ... per range of the narrow form

inline AttnPlan plan_verify_attn(int B, int Q, int H, int max_kv, int d_lat, int num_cu) {
  AttnPlan p;
  const long long rows = (long long)Q * H;
  p.row_tiles = (int)((rows + kRowsPerWG - 1) / kRowsPerWG);
  const long long nkb = ((long long)max_kv + kTileKeys - 1) / kTileKeys;
  const long long work = (long long)B * p.row_tiles * nkb;
  // One resident workgroup per CU (LDS-bound), but at least min_tiles key
  // tiles each so that query loads and partial outputs stay a small share.
  long long cap = num_cu > 0 ? num_cu : 256;
  if (cap > kMaxGrid) cap = kMaxGrid;
  const long long units = (long long)B * p.row_tiles;
  // Very few row tiles (the 512-wide latent form only, at most a sixteenth of
  // the CUs, as at batch 1): a range's row tiles are taken by four workgroups
  // of 32 rows each, so that each row tile is cut into a quarter as many
  // ranges for the same number of busy CUs, which quarters the partial rows
  // written and merged.  Each of the four loads the key tiles itself, so with
  // more row tiles the 128-row form is faster.
  p.narrow = d_lat == 512 && units * 16 <= cap;
  const int min_tiles = p.narrow ? kMinTilesNarrow : kMinTilesPerWG;
  if (p.narrow) cap /= 4;
  const long long per_unit = (nkb + min_tiles - 1) / min_tiles;
  long long g;
  if (units * per_unit <= cap) {
    // Few row tiles: cut each into ranges of at most min_tiles tiles, so
    // that every workgroup's range lies inside one row tile (one query load,
    // one partial output) and none is longer than that.
    g = units * per_unit;
  } else {
    g = cap;
    const long long by_work = (work + min_tiles - 1) / min_tiles;
    if (by_work < g) g = by_work;
    // When a multiple of the row-tile count comes within 10% of that, take it
    // (requests of equal length then give ranges inside one row tile).
    if (units <= g && units * (g / units) * 10 >= g * 9) g = units * (g / units);
  }
  if (g < 1) g = 1;
  p.grid = (int)g;
  p.num_cu = num_cu > 0 ? num_cu : 256;
  // Partial outputs and log-sum-exps (two slots per workgroup), then the
  // stream prefix over requests, the split mode and the start cost that the
  // merge kernels read.
  p.ws_bytes = (size_t)2 * p.grid * kRowsPerWG * ((size_t)d_lat + 1) * sizeof(float) +
               ((size_t)B + 3) * sizeof(long long);
  return p;
}

}  // namespace ddt
