// jf_tile_order.h -- which output tile a GEMM workgroup computes.
//
// Workgroups are dealt to the eight XCDs round-robin (XCD = workgroup id % 8),
// and each XCD has its own L2.  The id is renumbered so that every XCD owns
// one contiguous range of tiles, and that range is walked in groups of eight
// tile rows (column by column inside a group), so workgroups that run at the
// same time on one XCD share A row panels and B column panels.
//
// The map is a bijection from workgroup ids 0..ntiles-1 onto the tiles of a
// tilesM x tilesN grid (ntiles = tilesM * tilesN) for every grid shape; a CPU
// test checks this exhaustively over small grids.  constexpr, so the same
// function serves the kernel and host-side checks.
#pragma once

namespace jf {

struct TileCoord {
    int tm, tn;   // tile row, tile column
};

constexpr int kXcds = 8;
constexpr int kTileGroupRows = 8;

constexpr TileCoord tile_of(int bid, int ntiles, int tilesN) {
    const int tilesM = ntiles / tilesN;
    // renumber: XCD x = bid % 8 owns tiles [x * per + min(x, rem), ...)
    const int x = bid % kXcds, j = bid / kXcds;
    const int per = ntiles / kXcds, rem = ntiles % kXcds;
    const int t = x * per + (x < rem ? x : rem) + j;
    // walk: groups of kTileGroupRows tile rows, column-major inside a group
    const int in_group = kTileGroupRows * tilesN;
    const int first_m = (t / in_group) * kTileGroupRows;
    const int left = tilesM - first_m;
    const int gsize = left < kTileGroupRows ? left : kTileGroupRows;
    return TileCoord{first_m + (t % in_group) % gsize, (t % in_group) / gsize};
}

}  // namespace jf
