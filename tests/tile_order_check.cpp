// Exhaustive host check of the GEMM's workgroup -> tile map (jf_tile_order.h):
// for every grid of tilesM x tilesN tiles with both sides up to LIMIT, every
// workgroup id maps into the grid and every tile is computed by exactly one
// workgroup.
// Prints "ok <grids checked>" or the first failing grid.
#include <cstdio>
#include <vector>

#include "../int8_block_quantized_amd/csrc/jf_tile_order.h"

int main() {
    const int LIMIT = 160;
    long grids = 0;
    std::vector<int> hit;
    for (int tm = 1; tm <= LIMIT; ++tm)
        for (int tn = 1; tn <= LIMIT; ++tn) {
            const int n = tm * tn;
            hit.assign(n, 0);
            for (int bid = 0; bid < n; ++bid) {
                const jf::TileCoord c = jf::tile_of(bid, n, tn);
                if (c.tm < 0 || c.tm >= tm || c.tn < 0 || c.tn >= tn) {
                    std::printf("out of range: grid %dx%d bid %d -> (%d, %d)\n", tm, tn, bid, c.tm, c.tn);
                    return 1;
                }
                ++hit[c.tm * tn + c.tn];
            }
            for (int i = 0; i < n; ++i)
                if (hit[i] != 1) {
                    std::printf("tile (%d, %d) of grid %dx%d computed %d times\n", i / tn, i % tn, tm, tn, hit[i]);
                    return 1;
                }
            ++grids;
        }
    std::printf("ok %ld\n", grids);
    return 0;
}
