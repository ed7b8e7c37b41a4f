// Host check of the workgroup -> (head, tile rank) mapping that every
// matrix-core launch uses (tile_order and tile_group in fa_device.h): for each
// head count and tile count below, and every head-group size the launches
// can take, the grid's workgroup ids must map one to one onto all
// (head, rank) pairs.  Runs on the CPU; prints "ok" or the first failure.
#include <cstdio>
#include <vector>

#include "../../flashattention_online_softmax_fa_amd/csrc/fa_device.h"

static int check(uint32_t heads, uint32_t tiles, uint32_t group) {
    std::vector<unsigned char> seen((size_t)heads * tiles, 0);
    for (uint32_t bid = 0; bid < heads * tiles; ++bid) {
        const fa::TileId t = fa::tile_order(bid, heads, tiles, group);
        if (t.head >= heads || t.rank >= tiles) {
            std::printf("heads %u tiles %u group %u: bid %u -> (%u, %u) out of range\n", heads,
                        tiles, group, bid, t.head, t.rank);
            return 1;
        }
        unsigned char &s = seen[(size_t)t.head * tiles + t.rank];
        if (s) {
            std::printf("heads %u tiles %u group %u: (%u, %u) taken twice\n", heads, tiles,
                        group, t.head, t.rank);
            return 1;
        }
        s = 1;
        // workgroups are dealt round-robin over the 8 XCDs: when the heads
        // split evenly, every tile of a head must land on one XCD
        if (heads % 8 == 0 && t.head / (heads / 8) != bid % 8) {
            std::printf("heads %u tiles %u group %u: bid %u (XCD %u) -> head %u of XCD %u\n",
                        heads, tiles, group, bid, bid % 8, t.head, t.head / (heads / 8));
            return 1;
        }
    }
    return 0;
}

int main() {
    const uint32_t heads_list[] = {1, 2, 3, 7, 8, 12, 16, 24, 32, 40, 64, 96, 2048};
    const uint32_t tiles_list[] = {1, 2, 3, 5, 16, 17, 32, 64, 128};
    int bad = 0, cases = 0;
    for (uint32_t h : heads_list)
        for (uint32_t n : tiles_list) {
            const uint32_t per_xcd = h % 8 == 0 ? h / 8 : h;
            std::vector<uint32_t> groups = {fa::tile_group(h)};
            for (uint32_t g = 1; g <= per_xcd; ++g)  // every divisor (FA_TILE_GROUP builds)
                if (per_xcd % g == 0 && g <= 16) groups.push_back(g);
            for (uint32_t g : groups) {
                ++cases;
                bad |= check(h, n, g);
            }
        }
    if (bad) return 1;
    std::printf("ok %d cases\n", cases);
    return 0;
}
