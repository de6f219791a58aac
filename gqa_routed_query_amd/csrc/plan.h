// Host-side planning of causal prefill grids: the dispatch order of row-tile
// bands and the key splits of routed launches. Plain C++ (no HIP), so it can be
// built and checked on its own.
//
// Dispatch order of the row-tile bands of a causal grid. The hardware hands
// blocks to CUs in index order as CUs free up; a band is one row tile of every
// problem. Heaviest first leaves the last round short of work: at B=4, h=32,
// g=8, T=2048 two rounds end together and 192 light jobs remain for 256 CUs.
// The order is searched on a model of that dispatch: a job costs its key tiles
// plus a fixed cost, goes to the CU that frees first, and pairwise swaps of
// bands are kept while they shorten the simulated end. The per-job fixed cost
// (prologue and epilogue) was fitted by measurement: about 4 tiles of 32 keys.
// Cached per shape; shapes with more bands keep heaviest first.
//
// Key splitting (routed launches given a workspace): when the grid holds less
// than two blocks per CU, the heaviest row tiles of the upper half of the
// sequence are split at a key tile into two parts that run as separate jobs;
// the second part merges the first part's partial result into its own. The split key tile is
// never past the tile's first token, so every row sees keys in both parts.
// A split is kept when it shortens the modelled end.
#pragma once

#include <stdint.h>

#include <tuple>
#include <vector>

namespace gqa {

constexpr int kMaxOrder = 48;  // row-tile bands (plus split parts) with a planned dispatch order

// A causal grid: n_bands row tiles of `rows` attention rows per problem, R rows
// per token, T tokens, key tiles of kBN keys; BG_main (batch, group) problems
// plus B_sh shared-head problems (one row per token); n_cu compute units; at
// most max_split row tiles split.
struct OrderShape {
  int n_bands, rows, R, T, kBN, BG_main, B_sh, n_cu, max_split;
  bool operator<(const OrderShape& o) const {
    return std::tie(n_bands, rows, R, T, kBN, BG_main, B_sh, n_cu, max_split) <
           std::tie(o.n_bands, o.rows, o.R, o.T, o.kBN, o.BG_main, o.B_sh, o.n_cu, o.max_split);
  }
};

// One dispatch band: row tile `tile`, whole (part 0) or the keys before
// (part 1) or from (part 2) key tile `split`; sbi numbers the split tiles.
struct Slot {
  uint16_t tile, split;
  uint8_t part, sbi;
};

struct BandKeys {
  int n_tiles, split;
};
// Key tiles of row tile i of a problem with T*R rows (R per token) in row
// tiles of `rows`, with key tiles of kBN keys, and the key tile at which it may
// be split (0: none).
BandKeys band_keys(int i, int rows, int R, int T, int kBN);

// Row tiles that may be split in one launch (0 when the grid has two or more
// blocks per CU): those of the upper half with a split point inside, and fewer
// than n_cu / BG, so that the second parts (which wait for the first) never
// hold every CU.
int split_cap(int n_bands, int rows, int R, int T, int kBN, int BG, int n_cu);

// The planned dispatch order: one slot per band (a whole row tile, or one part
// of a split one), at most kMaxOrder slots.
std::vector<Slot> plan_order(const OrderShape& s);

}  // namespace gqa
