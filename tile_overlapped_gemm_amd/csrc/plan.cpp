// plan.cpp -- production orders, tile numbering and reduction wait tables.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs" (paperpeel.com/paper/2609.11562).
//  * Sec. 3.1 "Interleaved production" with Equation (1): the logical block
//    order cycles through the output partitions, so blocks whose output stays
//    local are spread among blocks whose output goes to peers.  The worked
//    example of Figure 4 (four GPUs) fixes the cycle: GPU 1's partition is
//    visited at positions 1, 5, 9, ..., the same on every rank.  We read
//    Equation (1) as partition = p mod P, block within partition = p div P.
//  * Sec. 2.2 ("Insight 1"): a traversal grouped by partition runs through the
//    rank's own partition as one contiguous stretch (partition-major order;
//    we put the local run last so it differs from the global raster).
//  * Sec. 5.3.1: the GEMM's default M-major traversal, the ablation baseline.
//  * Sec. 3.1 "Matching task order": the Q tiles of a partition are numbered
//    in the producer's traversal order, N-major inside a partition, so
//    consumer j's sequence j, j+x, ... follows production.
//  * Sec. 5.3.2: a release group of g tiles becomes visible when its last
//    tile finishes.
#include "plan.h"

#include <algorithm>
#include <numeric>

#include "entwine.h"

namespace entwine {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int make_geometry(int64_t M, int64_t N, int P, int bm, int bn, int tm, int tn, Geometry* g) {
  if (M <= 0 || N <= 0 || P < 1 || M % P != 0) return ENTWINE_ERR_INVALID_ARGUMENT;
  if (P > 8) return ENTWINE_ERR_UNSUPPORTED;
  if (!((bm == 128 || bm == 256) && (bn == 128 || bn == 256)) && !(bm == 128 && bn == 384))
    return ENTWINE_ERR_UNSUPPORTED;
  if (!((tm == 64 || tm == 128) && (tn == 64 || tn == 128)))
    return ENTWINE_ERR_UNSUPPORTED;
  if (bm % tm != 0 || bn % tn != 0) return ENTWINE_ERR_INVALID_ARGUMENT;
  Geometry r;
  r.M = M;
  r.N = N;
  r.P = P;
  r.R = M / P;
  r.bm = bm;
  r.bn = bn;
  r.tm = tm;
  r.tn = tn;
  r.sub_m = bm / tm;
  r.sub_n = bn / tn;
  r.Rb = ceil_div(r.R, bm);
  r.Cb = ceil_div(N, bn);
  r.Bd = r.Rb * r.Cb;
  r.NB = r.Bd * P;
  r.Rt = ceil_div(r.R, tm);
  r.Ct = ceil_div(N, tn);
  r.Q = r.Rt * r.Ct;
  if (r.NB > INT32_MAX || r.Q * P > INT32_MAX) return ENTWINE_ERR_UNSUPPORTED;
  *g = r;
  return ENTWINE_OK;
}

void block_at(const Geometry& g, int rank, int order, int64_t p, int* d, int64_t* i) {
  const int P = g.P;
  switch (order) {
    case ENTWINE_ORDER_INTERLEAVED:
      *d = (int)(p % P);
      *i = p / P;
      return;
    case ENTWINE_ORDER_PARTITION_MAJOR: {
      const int64_t k = p / g.Bd;
      *d = (int)((rank + 1 + k) % P);
      *i = p % g.Bd;
      return;
    }
    case ENTWINE_ORDER_COL_MAJOR: {
      // Column-major over the global grid of P*Rb block rows and Cb columns.
      const int64_t rows = (int64_t)P * g.Rb;
      const int64_t grow = p % rows, bc = p / rows;
      *d = (int)(grow / g.Rb);
      *i = (grow % g.Rb) * g.Cb + bc;
      return;
    }
    case ENTWINE_ORDER_ROW_MAJOR:
    default:
      *d = (int)(p / g.Bd);
      *i = p % g.Bd;
      return;
  }
}

int64_t position_of(const Geometry& g, int rank, int order, int d, int64_t i) {
  const int P = g.P;
  switch (order) {
    case ENTWINE_ORDER_INTERLEAVED:
      return i * P + d;
    case ENTWINE_ORDER_PARTITION_MAJOR: {
      const int64_t k = ((int64_t)d - rank - 1 + 2 * (int64_t)P) % P;
      return k * g.Bd + i;
    }
    case ENTWINE_ORDER_COL_MAJOR: {
      const int64_t br = i / g.Cb, bc = i % g.Cb;
      return bc * ((int64_t)P * g.Rb) + (int64_t)d * g.Rb + br;
    }
    case ENTWINE_ORDER_ROW_MAJOR:
    default:
      return (int64_t)d * g.Bd + i;
  }
}

void block_valid_tiles(const Geometry& g, int64_t i, int* vm, int* vn) {
  const int64_t br = i / g.Cb, bc = i % g.Cb;
  *vm = (int)std::min<int64_t>(g.sub_m, g.Rt - br * g.sub_m);
  *vn = (int)std::min<int64_t>(g.sub_n, g.Ct - bc * g.sub_n);
}

int build_plan(const Geometry& g, int rank, int order, int peer_ready, int release_group,
               Plan* out) {
  if (rank < 0 || rank >= g.P) return ENTWINE_ERR_INVALID_ARGUMENT;
  if (order < ENTWINE_ORDER_ROW_MAJOR || order > ENTWINE_ORDER_COL_MAJOR)
    return ENTWINE_ERR_INVALID_ARGUMENT;
  if (peer_ready != ENTWINE_PEERS_PRESEEDED && peer_ready != ENTWINE_PEERS_SYMMETRIC)
    return ENTWINE_ERR_INVALID_ARGUMENT;
  if (release_group < ENTWINE_RELEASE_OUTPUT) return ENTWINE_ERR_INVALID_ARGUMENT;

  Plan pl;
  pl.g = g;
  pl.rank = rank;
  pl.order = order;
  pl.peer_ready = peer_ready;
  pl.release_group = release_group;

  // Tile numbering inside a partition: blocks in N-major order, the block's
  // valid tiles row-major.  Identical for every partition and every order.
  pl.first_tile.resize(g.Bd);
  std::vector<int32_t> tile_block(g.Q);  // block index of each tile
  pl.tiles.resize(2 * g.Q);
  int64_t t = 0;
  for (int64_t i = 0; i < g.Bd; ++i) {
    pl.first_tile[i] = (int32_t)t;
    int vm, vn;
    block_valid_tiles(g, i, &vm, &vn);
    const int64_t br = i / g.Cb, bc = i % g.Cb;
    for (int sm = 0; sm < vm; ++sm)
      for (int sn = 0; sn < vn; ++sn) {
        pl.tiles[2 * t] = (int32_t)(br * g.sub_m + sm);
        pl.tiles[2 * t + 1] = (int32_t)(bc * g.sub_n + sn);
        tile_block[t] = (int32_t)i;
        ++t;
      }
  }
  if (t != g.Q) return ENTWINE_ERR_INVALID_ARGUMENT;  // geometry inconsistent

  pl.blocks.resize(4 * g.NB);
  for (int64_t p = 0; p < g.NB; ++p) {
    int d;
    int64_t i;
    block_at(g, rank, order, p, &d, &i);
    pl.blocks[4 * p + 0] = d;
    pl.blocks[4 * p + 1] = (int32_t)(i / g.Cb);
    pl.blocks[4 * p + 2] = (int32_t)(i % g.Cb);
    pl.blocks[4 * p + 3] = pl.first_tile[i];
  }

  // Which block position releases tile t's group, as seen by source rank r:
  // the latest-produced block among the group's tiles under r's order.
  auto release_position = [&](int src, int64_t tt) -> int64_t {
    if (release_group == ENTWINE_RELEASE_OUTPUT) return g.NB - 1;
    int64_t lo, hi;
    if (release_group == ENTWINE_RELEASE_PARTITION) {
      lo = 0;
      hi = g.Q;
    } else {
      lo = tt / release_group * release_group;
      hi = std::min<int64_t>(lo + release_group, g.Q);
    }
    int64_t best = -1;
    for (int64_t u = lo; u < hi; ++u)
      best = std::max(best, position_of(g, src, order, rank, tile_block[u]));
    return best;
  };
  // The local flag of the block at logical position p (any of its tiles:
  // a block publishes all of its tiles' flags together, after all stores).
  auto flag_at_position = [&](int64_t p, int64_t tt_same_block) -> int32_t {
    int d;
    int64_t i;
    block_at(g, rank, order, p, &d, &i);
    int64_t tt = tt_same_block;
    if (tt < pl.first_tile[i] ||
        tt >= (i + 1 < g.Bd ? pl.first_tile[i + 1] : g.Q))
      tt = pl.first_tile[i];
    return (int32_t)(d * g.Q + tt);
  };

  // Wait slots per tile: one per source rank, then one for the release
  // group.  The local slot is always the tile's own flag: it is what makes the
  // tile's data safe to read.  A release group (Sec. 5.3.2) additionally holds
  // the tile back until the block at the group's last logical position is
  // done, i.e. the group is released when its last tile is produced.
  const int slots = g.P + 1;
  pl.wait_slots = slots;
  pl.waits.assign((size_t)g.Q * slots, -1);
  for (int64_t tt = 0; tt < g.Q; ++tt) {
    int32_t* w = &pl.waits[tt * slots];
    for (int r = 0; r < g.P; ++r) {
      if (r == rank) {
        w[r] = (int32_t)(rank * g.Q + tt);
      } else if (peer_ready == ENTWINE_PEERS_SYMMETRIC) {
        // Peer r produces tile tt (block tile_block[tt] of partition `rank`)
        // at its own logical position; this GPU's block at that position
        // stands in for it.
        const int64_t p = release_group == ENTWINE_RELEASE_TILE
                              ? position_of(g, r, order, rank, tile_block[tt])
                              : release_position(r, tt);
        w[r] = flag_at_position(p, tt);
      }
    }
    if (release_group != ENTWINE_RELEASE_TILE)
      w[g.P] = flag_at_position(release_position(rank, tt), tt);
  }
  *out = std::move(pl);
  return ENTWINE_OK;
}

// Distinct X row panels plus W column panels touched by a set of blocks.
static int64_t panels(const std::vector<std::pair<int64_t, int64_t>>& rc, size_t lo, size_t hi) {
  std::vector<int64_t> rows, cols;
  for (size_t k = lo; k < hi; ++k) {
    rows.push_back(rc[k].first);
    cols.push_back(rc[k].second);
  }
  std::sort(rows.begin(), rows.end());
  std::sort(cols.begin(), cols.end());
  return (int64_t)(std::unique(rows.begin(), rows.end()) - rows.begin()) +
         (int64_t)(std::unique(cols.begin(), cols.end()) - cols.begin());
}

void assign_dispatch(Plan* plan, int64_t window) {
  const Geometry& g = plan->g;
  const int64_t NB = g.NB;
  plan->dispatch.resize(NB);
  std::iota(plan->dispatch.begin(), plan->dispatch.end(), 0);
  if (window >= kXcds) {
    window -= window % kXcds;
    for (int64_t w0 = 0; w0 < NB; w0 += window) {
      const int64_t w1 = std::min(NB, w0 + window), n = w1 - w0;
      // Global block coordinates of the window's positions.
      std::vector<std::pair<int64_t, int64_t>> rc(n);
      for (int64_t k = 0; k < n; ++k) {
        const int32_t* b = &plan->blocks[4 * (w0 + k)];
        rc[k] = {(int64_t)b[0] * g.Rb + b[1], (int64_t)b[2]};
      }
      std::vector<int64_t> urows, ucols;
      for (auto& v : rc) {
        urows.push_back(v.first);
        ucols.push_back(v.second);
      }
      std::sort(urows.begin(), urows.end());
      urows.erase(std::unique(urows.begin(), urows.end()), urows.end());
      std::sort(ucols.begin(), ucols.end());
      ucols.erase(std::unique(ucols.begin(), ucols.end()), ucols.end());
      // Slots of each XCD inside the window: workgroups b in [w0, w1) with
      // b % kXcds == x, in order (w0 is a multiple of kXcds).
      std::vector<int64_t> slots(kXcds, 0);
      for (int64_t b = w0; b < w1; ++b) ++slots[b % kXcds];
      // The identity deal (XCD x takes positions w0 + x + kXcds*k) as written
      // in deal order, then splits of the window's rows into a groups and its
      // columns into kXcds / a groups; keep the deal whose busiest XCD touches
      // the fewest panels.
      std::vector<int64_t> best_order;
      int64_t best_cost = -1;
      {
        std::vector<int64_t> order;
        std::vector<std::pair<int64_t, int64_t>> sorted;
        for (int x = 0; x < kXcds; ++x)
          for (int64_t k = x; k < n; k += kXcds) {
            order.push_back(k);
            sorted.push_back(rc[k]);
          }
        size_t lo = 0;
        best_cost = 0;
        for (int x = 0; x < kXcds; ++x) {
          best_cost = std::max(best_cost, panels(sorted, lo, lo + slots[x]));
          lo += slots[x];
        }
        best_order = order;
      }
      for (int a = 1; a <= kXcds; a *= 2) {
        const int bgrp = kXcds / a;
        std::vector<int64_t> order(n);
        std::iota(order.begin(), order.end(), 0);
        auto key = [&](int64_t k) {
          const int64_t ri = std::lower_bound(urows.begin(), urows.end(), rc[k].first) - urows.begin();
          const int64_t ci = std::lower_bound(ucols.begin(), ucols.end(), rc[k].second) - ucols.begin();
          const int64_t grp = (ri * a / (int64_t)urows.size()) * bgrp + ci * bgrp / (int64_t)ucols.size();
          return std::make_tuple(grp, rc[k].first, rc[k].second);
        };
        std::stable_sort(order.begin(), order.end(),
                         [&](int64_t u, int64_t v) { return key(u) < key(v); });
        std::vector<std::pair<int64_t, int64_t>> sorted(n);
        for (int64_t k = 0; k < n; ++k) sorted[k] = rc[order[k]];
        int64_t cost = 0;
        size_t lo = 0;
        for (int x = 0; x < kXcds; ++x) {
          cost = std::max(cost, panels(sorted, lo, lo + slots[x]));
          lo += slots[x];
        }
        if (cost < best_cost) {
          best_cost = cost;
          best_order = order;
        }
      }
      // XCD x takes the next slots[x] positions of the chosen order; its
      // k-th workgroup in the window is b = w0 + x + kXcds * k.
      int64_t lo = 0;
      for (int x = 0; x < kXcds; ++x) {
        for (int64_t k = 0; k < slots[x]; ++k)
          plan->dispatch[w0 + x + kXcds * k] = (int32_t)(w0 + best_order[lo + k]);
        lo += slots[x];
      }
    }
  }
  plan->launch.resize(4 * NB);
  for (int64_t b = 0; b < NB; ++b)
    for (int f = 0; f < 4; ++f) plan->launch[4 * b + f] = plan->blocks[4 * plan->dispatch[b] + f];
}

std::vector<int32_t> task_list(const Plan& plan, int slabs, bool push) {
  const Geometry& g = plan.g;
  // Dispatch index of each logical position, and of each flag's block.
  std::vector<int64_t> at(g.NB);
  for (int64_t b = 0; b < g.NB; ++b) at[plan.dispatch[b]] = b;
  auto block_of_tile = [&](int64_t tt) {
    return (int64_t)(std::upper_bound(plan.first_tile.begin(), plan.first_tile.end(),
                                      (int32_t)tt) - plan.first_tile.begin()) - 1;
  };
  auto flag_dispatch = [&](int64_t flag) -> int64_t {
    const int d = (int)(flag / g.Q);
    const int64_t tt = flag % g.Q;
    return at[position_of(g, plan.rank, plan.order, d, block_of_tile(tt))];
  };
  struct Key {
    int64_t ready;
    int d;
    int64_t t;
    bool operator<(const Key& o) const {
      return ready != o.ready ? ready < o.ready : d != o.d ? d < o.d : t < o.t;
    }
  };
  std::vector<Key> keys;
  for (int d = 0; d < g.P; ++d) {
    if (d != plan.rank && !push) continue;
    for (int64_t tt = 0; tt < g.Q; ++tt) {
      int64_t last = -1;
      if (d == plan.rank) {
        for (int s = 0; s < plan.wait_slots; ++s) {
          const int32_t f = plan.waits[tt * plan.wait_slots + s];
          if (f >= 0) last = std::max(last, flag_dispatch(f));
        }
      } else {
        last = flag_dispatch((int64_t)d * g.Q + tt);
      }
      keys.push_back(Key{last, d, tt});
    }
  }
  std::sort(keys.begin(), keys.end());
  std::vector<int32_t> order;
  order.reserve(keys.size() * slabs);
  for (const auto& k : keys)
    for (int s = 0; s < slabs; ++s) order.push_back((int32_t)((k.d * g.Q + k.t) * slabs + s));
  return order;
}

}  // namespace entwine
