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

#include "entwine.h"

namespace entwine {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int make_geometry(int64_t M, int64_t N, int P, int bm, int bn, int tm, int tn, Geometry* g) {
  if (M <= 0 || N <= 0 || P < 1 || M % P != 0) return ENTWINE_ERR_INVALID_ARGUMENT;
  if (P > 8) return ENTWINE_ERR_UNSUPPORTED;
  if (!((bm == 128 || bm == 256) && (bn == 128 || bn == 256)))
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

}  // namespace entwine
