// split_check.hip -- a host-side checker of the verify-attention work split.
//
// It runs the split arithmetic of attn_split.h (the same functions the
// attention and merge kernels call) for every workgroup of a launch and
// checks, for one set of request sizes:
//  * every (request, row tile, key tile) with work is taken by exactly one
//    workgroup, and no range walks into a row tile without work;
//  * the stream (row-tile segments of start cost c plus key tiles) is cut as
//    the kernels cut it, and ranges that end inside a start cost run nothing;
//  * a workgroup writes at most one partial result per slot, its slots lie in
//    [0, 2G) (the workspace holds 2G), and no slot is written by two units;
//  * for every row tile, the merge's contributor rule names exactly the slots
//    the attention kernel wrote for it (none for a tile written directly);
//  * the grid, the batch and the contributor counts fit the kernels' limits;
//  * in the narrow form, the launch's workgroups take every (range, quarter)
//    exactly once and the padding workgroups none.
// Host code only (no kernels); built into its own library for the CPU tests.
#include <stdio.h>

#include <map>
#include <set>
#include <vector>

#include "attn_split.h"

namespace {

int fail(char* msg, int len, const char* what, long long a, long long b, long long c) {
  if (msg && len > 0) snprintf(msg, (size_t)len, "%s (%lld, %lld, %lld)", what, a, b, c);
  return 1;
}

}  // namespace

// plant != 0 plants a mistake in the merge's view (1: head and tail slots
// swapped, 2: the last contributor dropped), to show the check catches it.
// stats (may be NULL) receives: [0] the start cost c, [1] ranges that end
// inside a start cost, [2] ranges holding key tiles of two or more row tiles,
// [3] the largest (key tiles + c per row tile begun) over ranges, [4] the
// stream length per range rounded up.
extern "C" int ddt_split_check(int B, int Q, int H, int max_kv, const int32_t* prefix_len,
                               const int32_t* n_nodes, int num_cu, int d_lat, int plant,
                               char* msg, int msg_len, long long* stats) {
  using namespace ddt;
  if (msg && msg_len > 0) msg[0] = '\0';
  if (B < 1 || B > kMaxBatch || Q < 1 || H < 1 || max_kv < 1) return fail(msg, msg_len, "bad args", B, Q, H);
  const AttnPlan plan = plan_verify_attn(B, Q, H, max_kv, d_lat, num_cu);
  const long long G = plan.grid;
  const int RT = plan.row_tiles;
  if (G < 1 || G > kMaxGrid) return fail(msg, msg_len, "grid out of range", G, 0, 0);
  const size_t need = (size_t)2 * G * kRowsPerWG * ((size_t)d_lat + 1) * sizeof(float) +
                      ((size_t)B + 3) * sizeof(long long);
  if (plan.ws_bytes < need) return fail(msg, msg_len, "workspace too small", (long long)plan.ws_bytes, (long long)need, 0);

  if (plan.narrow) {
    if (d_lat != 512) return fail(msg, msg_len, "narrow form for another width", d_lat, 0, 0);
    const long long ranges = ((long long)B * RT >= G ? 2 : 1) * G;
    const long long blocks = narrow_blocks(ranges);
    std::vector<int> seen((size_t)(ranges * kQuarters), 0);
    for (long long bid = 0; bid < blocks; ++bid) {
      long long r;
      int q;
      narrow_place(bid, r, q);
      if (q < 0 || q >= kQuarters || r < 0) return fail(msg, msg_len, "narrow place", bid, r, q);
      if (r < ranges) ++seen[(size_t)(r * kQuarters + q)];
    }
    for (size_t i = 0; i < seen.size(); ++i)
      if (seen[i] != 1) return fail(msg, msg_len, "narrow (range, quarter) taken", (long long)i, seen[i], blocks);
  }

  std::vector<ReqInfo> ri(B);
  std::vector<long long> tiles(B + 1, 0);  // key tiles with work before request b
  long long units = 0;
  bool same = true;
  for (int b = 0; b < B; ++b) {
    ri[b] = req_info(prefix_len, n_nodes, b, Q, H, max_kv, RT);
    tiles[b + 1] = tiles[b] + (long long)ri[b].vt * ri[b].nkb;
    units += ri[b].vt;
    if (ri[b].nkb != ri[0].nkb || ri[b].vt != ri[0].vt) same = false;
  }
  const bool split2 = (long long)B * RT >= G;
  const long long mode = split2 ? split_mode(same, ri[0].vt, B, G) : -1;
  const int c = unit_cost(mode, same, units, G);
  if (c < 0 || c > kUnitCost) return fail(msg, msg_len, "start cost", c, mode, units);
  std::vector<long long> pref(B + 1, 0);  // the stream prefix
  for (int b = 0; b < B; ++b) pref[b + 1] = pref[b] + (long long)ri[b].vt * (ri[b].nkb + c);
  const long long Wtot = pref[B];

  long long n_empty = 0, n_multi = 0, max_load = 0;
  std::vector<int> cover((size_t)tiles[B], 0);
  std::map<long long, std::set<long long>> written;  // unit (b * RT + rt) -> slots
  std::map<long long, long long> slot_owner;         // slot -> unit
  std::set<long long> direct;                        // units written whole
  for (int half = 0; half < (split2 ? 2 : 1); ++half) {
    for (long long bl = 0; bl < G; ++bl) {
      const long long gid = logical_gid(bl, G);
      if (gid < 0 || gid >= G) return fail(msg, msg_len, "logical id out of range", bl, gid, G);
      long long start, end;
      workgroup_range(mode, half == 1, gid, Wtot, ri[0].nkb + c, G, start, end);
      if (start >= end) continue;
      if (start < 0 || end > Wtot) return fail(msg, msg_len, "range outside the work", start, end, Wtot);
      int b = 0;
      while (b + 1 < B && pref[b + 1] <= start) ++b;
      long long pos = start;
      int tails = 0, n_units = 0;
      long long load = 0;
      while (pos < end) {
        while (pref[b + 1] <= pos) ++b;
        if (b >= B || ri[b].vt == 0) return fail(msg, msg_len, "walked into a request without work", b, pos, gid);
        const UnitPos up = unit_at(pos, end, pref[b], ri[b], c);
        if (up.adv < 1 || pos + up.adv > end)
          return fail(msg, msg_len, "unit advance", pos, up.adv, end);
        const bool head = pos == start;
        pos += up.adv;
        if (up.kb1 <= up.kb0) {
          // Only a range's last unit may be empty, and only by ending inside
          // the start cost of its row tile.
          if (pos != end || up.kb0 != 0 || up.kb1 != 0)
            return fail(msg, msg_len, "empty unit not at a range's end", b, up.rt, up.kb0);
          ++n_empty;
          continue;
        }
        ++n_units;
        load += (up.kb1 - up.kb0) + (up.kb0 == 0 ? c : 0);
        if (up.rt < 0 || up.rt >= ri[b].vt || up.kb0 < 0 || up.kb1 > ri[b].nkb)
          return fail(msg, msg_len, "unit outside its request", b, up.rt, up.kb0);
        for (int kb = up.kb0; kb < up.kb1; ++kb)
          ++cover[(size_t)(tiles[b] + (long long)up.rt * ri[b].nkb + kb)];
        const long long unit = (long long)b * RT + up.rt;
        if (up.complete) {
          direct.insert(unit);
        } else {
          if (!head && ++tails > 1) return fail(msg, msg_len, "two cut tails in one range", gid, b, up.rt);
          const long long slot = partial_slot(gid, head);
          if (slot < 0 || slot >= 2 * G) return fail(msg, msg_len, "slot out of range", slot, gid, G);
          auto it = slot_owner.find(slot);
          if (it != slot_owner.end()) return fail(msg, msg_len, "slot written twice", slot, it->second, unit);
          slot_owner[slot] = unit;
          written[unit].insert(slot);
        }
      }
      if (n_units > 1) ++n_multi;
      if (load > max_load) max_load = load;
    }
  }
  for (long long t = 0; t < tiles[B]; ++t)
    if (cover[(size_t)t] != 1) return fail(msg, msg_len, "tile covered", t, cover[(size_t)t], tiles[B]);

  // The merge's view of every row tile with work.
  for (int b = 0; b < B; ++b) {
    for (int rt = 0; rt < ri[b].vt; ++rt) {
      const long long unit = (long long)b * RT + rt;
      const auto wit = written.find(unit);
      const size_t nw = wit == written.end() ? 0 : wit->second.size();
      long long S, W;
      if (!stream_place(mode, pref.data(), B, b, rt, ri[b], G, c, S, W)) {
        if (nw != 0 || !direct.count(unit)) return fail(msg, msg_len, "whole unit not written whole", b, rt, (long long)nw);
        continue;
      }
      long long gf, gl;
      tile_owners(S, W, G, ri[b].nkb, c, gf, gl);
      if (gf == gl) {
        if (nw != 0 || !direct.count(unit)) return fail(msg, msg_len, "uncut tile not written directly", b, rt, (long long)nw);
        continue;
      }
      if (gl - gf + 1 > kMaxGrid) return fail(msg, msg_len, "too many contributors", b, rt, gl - gf + 1);
      std::set<long long> contrib;
      for (long long gg = gf; gg <= gl - (plant == 2 ? 1 : 0); ++gg) {
        const long long src = contributor_slot(gg, S, W, G);
        if (src >= 0) contrib.insert(plant == 1 ? (src ^ 1) : src);
      }
      if (nw == 0 || contrib != wit->second)
        return fail(msg, msg_len, "merge contributors differ from written slots", b, rt, (long long)contrib.size() - (long long)nw);
      if (direct.count(unit)) return fail(msg, msg_len, "cut tile also written whole", b, rt, 0);
    }
  }
  if (stats) {
    stats[0] = c;
    stats[1] = n_empty;
    stats[2] = n_multi;
    stats[3] = max_load;
    stats[4] = (Wtot + G - 1) / G;
  }
  return 0;
}

// The plan itself, for tests that check which form a shape takes.
extern "C" int ddt_split_plan(int B, int Q, int H, int max_kv, int d_lat, int num_cu, int* grid,
                              int* narrow, int* row_tiles, unsigned long long* ws_bytes) {
  const ddt::AttnPlan p = ddt::plan_verify_attn(B, Q, H, max_kv, d_lat, num_cu);
  *grid = p.grid;
  *narrow = p.narrow ? 1 : 0;
  *row_tiles = p.row_tiles;
  *ws_bytes = p.ws_bytes;
  return 0;
}
