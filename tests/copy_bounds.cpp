// Host check of the prefill and wide-group decode kernels' whole-tile HBM -> LDS
// copies (global_load_lds_dwordx4 with an SGPR tile base and a 32-bit lane offset):
// for every supported (d, Bc), wave count and sequence length, every lane of
// every copy of every tile is enumerated through the offset functions the
// kernels themselves call (csrc/tile_copy.h), and
//   * the 16 bytes it reads lie inside the sequence's rows [0, T) of the
//     tensor slab (rows at the tile's own offset, clamped to T - 1 past the end),
//   * the LDS bytes it writes lie inside the tile's LDS buffer,
//   * every (row, chunk) of the tile's rows below T is loaded, and a full tile
//     loads each exactly once, into the LDS position the kernels read it from.
// Exit status 0 and one summary line when every check holds.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "tile_copy.h"

using namespace blasst;

static long g_checked = 0;
static int g_fail = 0;

#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            if (g_fail < 20) {                             \
                printf("FAIL %s:%d: ", __FILE__, __LINE__); \
                printf(__VA_ARGS__);                       \
                printf("\n");                              \
            }                                              \
            ++g_fail;                                      \
        }                                                  \
    } while (0)

template <int D, int BC>
void check_config(int NW, const std::vector<int>& lengths) {
    constexpr int CPR = D / 8, ROWB = 2 * D, TILE = BC * ROWB;
    if (TILE % (1024 * NW) != 0) return;
    const int CPW = TILE / (1024 * NW);
    for (int T : lengths) {
        const int nk = (T + BC - 1) / BC;
        for (int j = 0; j < nk; ++j) {
            std::vector<int> hits((size_t)BC * CPR, 0);
            const bool ragged = tile_is_ragged<BC>(j, T);
            for (int wave = 0; wave < NW; ++wave)
                for (int f = 0; f < CPW; ++f)
                    for (int lane = 0; lane < 64; ++lane) {
                        const uint32_t off0 = tile_copy_offset<CPR>(wave, CPW, f, lane);
                        const uint32_t off = ragged ? tile_copy_clamp<CPR, BC>(off0, j, T) : off0;
                        ++g_checked;
                        CHECK(off % 16 == 0, "misaligned offset %u", off);
                        CHECK(off < (uint32_t)TILE && off <= off0, "offset %u outside the tile (from %u)", off, off0);
                        const long byte = (long)j * BC * ROWB + off;  // from the slab's row 0
                        const long row = byte / ROWB;
                        CHECK(byte >= 0 && row <= T - 1 && byte + 16 <= (long)T * ROWB,
                              "D=%d BC=%d NW=%d T=%d j=%d wave=%d f=%d lane=%d reads bytes [%ld, %ld) of %ld", D, BC,
                              NW, T, j, wave, f, lane, byte, byte + 16, (long)T * ROWB);
                        const int lds = (wave * CPW + f) * 1024 + 16 * lane;
                        CHECK(lds >= 0 && lds + 16 <= TILE, "LDS bytes [%d, %d) outside the %d-byte tile", lds,
                              lds + 16, TILE);
                        // the LDS position the kernels read logical chunk c of tile row r from
                        const int r = (int)(off0 / ROWB), c = (int)((off0 % ROWB) / 16);
                        CHECK(lds == r * ROWB + ((c ^ chunk_swizzle<CPR>(r)) << 4),
                              "tile row %d chunk %d lands at LDS %d", r, c, lds);
                        if (row - (long)j * BC == r) hits[(size_t)r * CPR + c] += 1;
                        else CHECK(ragged && row == T - 1, "row %ld re-read outside a ragged tile", row);
                    }
            const int rows = T - j * BC < BC ? T - j * BC : BC;
            for (int r = 0; r < rows; ++r)
                for (int c = 0; c < CPR; ++c)
                    CHECK(hits[(size_t)r * CPR + c] == 1, "D=%d BC=%d NW=%d T=%d j=%d: row %d chunk %d loaded %d times",
                          D, BC, NW, T, j, r, c, hits[(size_t)r * CPR + c]);
        }
    }
}

int main() {
    std::vector<int> lengths = {1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 513, 1000, 1024, 4097,
                                9000, 32768, 32769};
    // issuing waves: Bc/32 (one head per workgroup; or, with two heads, the group in phase X,
    // which issues each phase's whole tile), or 2 Bc/32 (both heads' waves: the first K and V tiles)
    for (int hpw = 1; hpw <= 2; ++hpw) {
        check_config<64, 64>(2 * hpw, lengths);
        check_config<64, 128>(4 * hpw, lengths);
        check_config<128, 64>(2 * hpw, lengths);
        check_config<128, 128>(4 * hpw, lengths);
    }
    // the wide-group decode kernel: eight waves, d = 128, K and V blocks of Bc = 64 or 128 keys
    check_config<128, 64>(8, lengths);
    check_config<128, 128>(8, lengths);
    printf("%s: %ld lane copies checked, %d failures\n", g_fail ? "FAILED" : "OK", g_checked, g_fail);
    return g_fail ? 1 : 0;
}
