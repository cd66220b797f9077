// Host-side check of the quantizers' block walks (block_walk.hpp): for every
// shape below, the walk the launchers pick visits each 128x128 block exactly
// once, and the XCD-tiled walk is the one picked for the wide activations.
#include "block_walk.hpp"

#include <cstdio>
#include <cstdlib>
#include <vector>

using puro::BlockRC;
using puro::BlockWalk;

static int check(const BlockWalk& w, int64_t nrb, int64_t ncb, const char* what)
{
    std::vector<unsigned char> seen((size_t)(nrb * ncb), 0);
    for (int64_t bid = 0; bid < nrb * ncb; ++bid) {
        const BlockRC b = puro::block_of(bid, nrb, ncb, w);
        if (b.rb < 0 || b.rb >= nrb || b.cb < 0 || b.cb >= ncb || seen[(size_t)(b.rb * ncb + b.cb)]++) {
            std::printf("FAIL %s nrb=%lld ncb=%lld walk=(%d,%d,%d,%d) bid=%lld -> (%lld,%lld)\n", what,
                        (long long)nrb, (long long)ncb, w.group_rows, w.tile_rows, w.tile_cols,
                        w.xcd_rows, (long long)bid, (long long)b.rb, (long long)b.cb);
            return 1;
        }
    }
    return 0;
}

int main()
{
    int fails = 0, shapes = 0, xcd = 0;
    // the activation shapes of the linear layers (tokens x features), ragged
    // token counts and small ones
    const int64_t rows[] = {128, 256, 384, 1024, 3000, 4096, 16384, 16383, 32768, 32700};
    const int64_t cols[] = {128, 512, 2048, 2176, 4096, 6144, 8192, 12288, 16384};
    for (int64_t r : rows)
        for (int64_t c : cols) {
            const int64_t nrb = (r + 127) / 128, ncb = c / 128;
            const BlockWalk w = puro::act_walk(puro::quant_group_rows(false, c), nrb, ncb);
            xcd += w.tile_rows > 0;
            fails += check(w, nrb, ncb, "act");
            fails += check(puro::grouped_walk(puro::quant_group_rows(true, c)), nrb, ncb, "weight");
            ++shapes;
        }
    // every XCD-tile arrangement on a few divisible shapes
    for (int xr : {1, 2, 4, 8})
        for (int tr : {1, 2, 4})
            for (int tc : {1, 4, 8}) {
                const int64_t nrb = 8 * tr * xr, ncb = 2 * tc * (8 / xr);
                fails += check(BlockWalk{8, tr, tc, xr}, nrb, ncb, "tiles");
                ++shapes;
            }
    // the wide activations of the block take the XCD walk
    const BlockWalk w16k = puro::act_walk(8, 256, 128), w6k = puro::act_walk(8, 256, 48),
                    w2k = puro::act_walk(16, 256, 16);
    if (w16k.tile_rows != 4 || w16k.xcd_rows != 1 || w6k.tile_rows != 4 || w6k.xcd_rows != 2 ||
        w2k.tile_rows != 0) {
        std::printf("FAIL walk choice\n");
        ++fails;
    }
    std::printf("%s: %d shapes, %d on the XCD walk\n", fails ? "FAILED" : "ok", shapes, xcd);
    return fails ? 1 : 0;
}
