// Address arithmetic of the whole-tile HBM -> LDS copies of the prefill and
// wide-group decode kernels (global_load_lds_dwordx4 with a wave-uniform tile base in SGPRs and
// a 32-bit byte offset per lane), kept host-callable so that every lane's
// address range can be enumerated and checked on the CPU.
//
// A tile is BC rows of a [.., T, d] bf16 tensor (rows of ROWB = 2 d bytes =
// CPR 16-byte chunks) starting at row j * BC.  Copy f of wave w moves 1 KiB:
// lane l writes LDS position pp = (w * CPW + f) * 64 + l, which holds tile row
// pp / CPR and, in its physical chunk pp % CPR, the logical chunk
// (pp % CPR) ^ chunk_swizzle(row).  A last tile that runs past the sequence's
// T rows re-reads row T - 1 in place of the missing rows.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define BLASST_HD __host__ __device__
#else
#define BLASST_HD
#endif

namespace blasst {

// XOR mask applied to the 16-byte chunk index of row r of a K/V tile in LDS.
// With 16 chunks per row (256-byte rows) it is the GF(2)-linear map sending the
// row's bits 0..3 to 4, 10, 1, 2; with 8 chunks per row, bits 0..2 to 2, 4, 1.
// An exhaustive search over such maps found these conflict-free (256-byte
// rows) or least-conflicting (128-byte rows) for both access patterns used on
// the tiles -- 32 consecutive rows x one chunk (ds_read_b128, MFMA A rows) and
// 4 consecutive rows x two chunks per 16 lanes (ds_read_b64_tr_b16) -- whether
// the LDS serves 32 or 64 banks per cycle.
template <int CPR>
BLASST_HD inline constexpr int chunk_swizzle(int r) {
    if constexpr (CPR == 16)
        return ((r & 1) * 4) ^ (((r >> 1) & 1) * 10) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) * 2);
    else
        return ((r & 1) * 2) ^ (((r >> 1) & 1) * 4) ^ ((r >> 2) & 1);
}

// Byte offset, inside a tile, of the 16 bytes lane `lane` copies in copy f of
// wave `wave` (CPW copies per wave per tile).
template <int CPR>
BLASST_HD inline constexpr uint32_t tile_copy_offset(int wave, int cpw, int f, int lane) {
    const int pp = (wave * cpw + f) * 64 + lane;
    return (uint32_t)((pp / CPR) * (16 * CPR) + (((pp % CPR) ^ chunk_swizzle<CPR>(pp / CPR)) << 4));
}

// Tile j of a sequence of T rows runs past its end.
template <int BC>
BLASST_HD inline constexpr bool tile_is_ragged(int j, int T) {
    return (j + 1) * BC > T;
}

// The offset of a ragged tile's copy with the tile row clamped to T - 1 (the
// tile's first row j * BC is at most T - 1, so the result never underflows).
template <int CPR, int BC>
BLASST_HD inline constexpr uint32_t tile_copy_clamp(uint32_t off, int j, int T) {
    constexpr int ROWB = 16 * CPR;
    const int over = j * BC + (int)(off / ROWB) - (T - 1);
    return off - (uint32_t)((over > 0 ? over : 0) * ROWB);
}

}  // namespace blasst
