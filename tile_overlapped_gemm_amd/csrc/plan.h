// plan.h -- host-side schedule of the tile-overlapped GEMM-ReduceScatter:
// block geometry, production orders, tile numbering and reduction waits.
//
// Method: "Entwine: Coordinating Tiled Computation and Fine-Grained
// Communication across GPUs", Sec. 3.1 (interleaved production, Equation (1),
// independent tile communication, matching task order) and Sec. 5.3.2
// (release granularity).  Pure C++; no HIP calls.
#pragma once

#include <cstdint>
#include <vector>

namespace entwine {

// Blocks and tiles are aligned to partitions: a partition of R = M/P rows is
// covered by Rb = ceil(R/BM) block rows and Cb = ceil(N/BN) block columns, and
// rows or columns beyond the partition's end are masked, never handed to the
// next partition.
struct Geometry {
  int64_t M = 0, N = 0, R = 0;  // R = rows per partition
  int P = 0;
  int bm = 0, bn = 0, tm = 0, tn = 0;
  int sub_m = 0, sub_n = 0;     // reduction tiles per block along rows / cols
  int64_t Rb = 0, Cb = 0;       // block rows / cols per partition
  int64_t Bd = 0;               // blocks per partition
  int64_t NB = 0;               // blocks in total (P * Bd)
  int64_t Rt = 0, Ct = 0;       // tile rows / cols per partition
  int64_t Q = 0;                // tiles per partition
};

// Returns 0 on success or an entwine_status.
int make_geometry(int64_t M, int64_t N, int P, int bm, int bn, int tm, int tn, Geometry* g);

// Partition and in-partition block index produced at logical position p by
// `rank` under `order` (ENTWINE_ORDER_*).
void block_at(const Geometry& g, int rank, int order, int64_t p, int* d, int64_t* i);

// Logical position at which `rank` produces block i of partition d.
int64_t position_of(const Geometry& g, int rank, int order, int d, int64_t i);

// Valid reduction tiles (rows, cols) inside block i of any partition.
void block_valid_tiles(const Geometry& g, int64_t i, int* vm, int* vn);

struct Plan {
  Geometry g;
  int rank = 0, order = 0, peer_ready = 0, release_group = 1;
  std::vector<int32_t> blocks;   // [NB][4]: d, br, bc, first tile, by logical position
  std::vector<int32_t> dispatch; // [NB]: logical position computed by workgroup b
  std::vector<int32_t> launch;   // [NB][4]: blocks[dispatch[b]], what the GEMM reads
  std::vector<int32_t> tiles;    // [Q][2]: tile row, tile col
  int wait_slots = 0;            // P + 1
  std::vector<int32_t> waits;    // [Q][wait_slots]: flag index or -1
  std::vector<int32_t> first_tile;  // [Bd]: number of block i's first tile
};

int build_plan(const Geometry& g, int rank, int order, int peer_ready, int release_group,
               Plan* out);

// The devices this is built for dispatch workgroup b of a grid to XCD
// b % kXcds, each XCD's workgroups in order.  Blocks resident at the same
// time (a window of `window` consecutive logical positions) run concurrently,
// so within each window the positions are dealt to XCDs such that every XCD
// gets a compact rectangle of the global block grid: its L2 then holds few X
// row panels and W column panels.  Across windows the production order is
// unchanged.  window = 0 (or 1) keeps the identity (workgroup b computes
// position b).  Fills plan->dispatch and plan->launch.
constexpr int kXcds = 8;
void assign_dispatch(Plan* plan, int64_t window);

// Tasks in production order (Sec. 3.1 "Matching task order") as global ids
// (d * Q + t) * slabs + s: the reductions of the rank's tiles and, with
// `push`, the send tasks of every other partition's tiles.  Tiles are sorted
// by the dispatch index of the last block they wait for (a reduction: any of
// its wait slots; a send task: the tile's own block), ties by partition, then
// tile.  Needs plan->dispatch (assign_dispatch).
std::vector<int32_t> task_list(const Plan& plan, int slabs, bool push);

}  // namespace entwine
