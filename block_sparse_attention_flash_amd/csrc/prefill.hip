// Causal GQA prefill with the skip-softmax rule.
//
// BLASST blog, section on the prefill kernel: prefill is compute bound, so a
// skipped tile saves the exp, the row sum and the P V product; S = Q K^T is
// always formed (its row max is what the test reads) and V tiles are fetched
// unconditionally, which keeps the copy pipeline regular.  The tile is skipped
// only when every one of the query block's Bc rows votes to skip (the AND over
// the query block; section on the lambda = a/L rule and on the decision cost).
//
// Work decomposition: one workgroup per (query block i of Br = Bc rows, group
// of HPW query heads that share a kv head, batch).  Bc/32 waves per head, wave
// owning 32 query rows.  The HPW heads share every K/V tile staged in LDS, so
// one tile copy feeds HPW times the MFMA work.  Workgroups are issued heaviest
// first (the last query block has the most KV tiles under the causal mask), and
// the workgroups of one query block are spread so that those sharing a kv head
// land on the same XCD (its L2 then serves their common K/V tiles).
//
// Per KV tile (all on MFMA 32x32x16 bf16, fp32 accumulate):
//   S^T = K Q^T      A = K rows from LDS (ds_read_b128), B = Q^T in registers.
//                    In S^T's accumulator layout each lane holds 16 scores of
//                    one query row, so row max, exp and row sum are mostly
//                    in-lane (plus one exchange with lane l^32).
//   vote             per row (mt - max(m, mt)) * scale < ln(lambda) in log2
//                    units, then an AND over the wave (ballot) and over the
//                    head's waves (an LDS word per wave).
//   O^T += V^T P^T   only for kept tiles.  P^T is the S^T accumulator after
//                    2^(s*scale - m*scale) rounded to bf16 (no data movement);
//                    V^T comes from the V tile in LDS through ds_read_b64_tr_b16.
// K and V tiles are copied HBM -> LDS directly (global_load_lds_dwordx4), two
// stages deep, XOR-swizzled by 16-byte chunk so both the row reads and the
// transposed reads are bank-conflict free.  Only the diagonal tile (and a ragged
// last tile) pays for causal / tail masking.
#include "device_common.h"
#include "kernels.h"

namespace blasst {

namespace {

template <int D, int BC, int HPW>
__global__ __launch_bounds__(2 * BC * HPW) void prefill_kernel(PrefillArgs a) {
    constexpr int NWH = BC / 32;           // waves per head
    constexpr int NW = NWH * HPW;          // waves per workgroup
    constexpr int KT = BC / 32;            // 32-key tiles of S^T
    constexpr int DS = D / 16;             // MFMA k-steps over d
    constexpr int DT = D / 32;             // 32-wide d tiles of O^T
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int ROWB = 2 * D;            // bytes per K/V row
    constexpr int TILE = BC * ROWB;        // bytes per K or V tile
    constexpr int CPW = TILE / (1024 * NW);  // 1 KiB copies per wave per tile
    static_assert(TILE % (1024 * NW) == 0, "tile copies must split evenly over the waves");

    __shared__ __attribute__((aligned(16))) char lds_k[2][TILE];
    __shared__ __attribute__((aligned(16))) char lds_v[2][TILE];
    __shared__ int lds_vote[NW];

    // ---- workgroup -> (query block, head group, batch)
    const int hg_count = a.Hq / HPW;
    const int bh_count = a.B * hg_count;
    const int L = blockIdx.x;
    const int i = a.nq - 1 - L / bh_count;
    int bh = L % bh_count;
    if (bh_count % 8 == 0) bh = (bh % 8) * (bh_count / 8) + bh / 8;
    const int hgrp = bh % hg_count, b = bh / hg_count;
    const int T = a.T;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int hsub = wave / NWH, wrow = wave % NWH;
    const int hq = hgrp * HPW + hsub;
    const int hkv = hq / a.G;
    const int col = lane & 31, half = lane >> 5;   // query column of S^T / O^T, and lane half
    const int qidx = i * BC + 32 * wrow + col;     // this lane's query row
    const bool row_ok = qidx < T;

    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    const float c = a.score_scale;

    // Q^T as the B operand: lane holds q[qidx][16s + 8*half .. +8].
    bf16x8 qf[DS];
    {
        const uint16_t* qrow = a.q + (((size_t)b * a.Hq + hq) * T + min(qidx, T - 1)) * D;
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[s] = as_bf16x8(load16(qrow + 16 * s + 8 * half));
    }

    const int last_row = min(T, (i + 1) * BC) - 1;
    const int jend = a.causal ? last_row / BC + 1 : a.nk;

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
    float m = kNegInf, l = 0.f;  // m in raw (unscaled) score units

    // ---- tile copy: this wave's 1 KiB pieces, LDS position p -> row p / CPR,
    //      physical chunk p % CPR holding logical chunk (p % CPR) ^ swizzle(row)
    auto issue_tile = [&](int j, int stage) {
#pragma unroll
        for (int f = 0; f < CPW; ++f) {
            const int piece = wave * CPW + f;
            const int p = piece * 64 + lane;
            const int row = p / CPR, cc = (p % CPR) ^ chunk_swizzle<CPR>(row);
            const size_t off = (size_t)min(j * BC + row, T - 1) * D + cc * 8;
            global_to_lds16(kbase + off, lds_addr(&lds_k[stage][piece * 1024]));
            global_to_lds16(vbase + off, lds_addr(&lds_v[stage][piece * 1024]));
        }
    };
    // Per-lane byte offsets inside a tile.  The swizzle depends on row & 15 only,
    // which is the same for every 32-key sub-tile, so sub-tile and stage offsets
    // are compile-time constants added to these.
    //   K (S^T A operand): row 32kt + col, chunk 2s + half
    //   V (transposed, PV A operand): row 32kt + 16p + 4(g16 >> 1) + (jj >> 2) (+ 8 for
    //   the second half), chunk 4dt + 2(g16 & 1) + ((jj & 3) >> 1), 8-byte half (jj & 1)
    int koff[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) koff[s] = col * ROWB + (((2 * s + half) ^ chunk_swizzle<CPR>(col)) << 4);
    int voff[2][DT];
    {
        const int g16 = lane >> 4, jj = lane & 15;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            const int r = 4 * (g16 >> 1) + (jj >> 2) + 8 * h8;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int chunk = 4 * dt + 2 * (g16 & 1) + ((jj & 3) >> 1);
                voff[h8][dt] = r * ROWB + ((chunk ^ chunk_swizzle<CPR>(r)) << 4) + (jj & 1) * 8;
            }
        }
    }

    uint8_t* mask_row = a.mask ? a.mask + (((size_t)b * a.Hq + hq) * a.nq + i) * a.nk : nullptr;

    issue_tile(0, 0);
    for (int j = 0; j < jend; ++j) {
        const int st = j & 1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's pieces of tile j
        __syncthreads();                                   // every piece of tile j; stage st^1 free
        if (j + 1 < jend) issue_tile(j + 1, st ^ 1);

        // ---- S^T = K Q^T for this wave's 32 query columns, all BC keys
        f32x16 sacc[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            sacc[kt] = f32x16{};
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const u32x4 kf = *(const u32x4*)(&lds_k[st][32 * kt * ROWB + koff[s]]);
                sacc[kt] = mfma32x32x16(as_bf16x8(kf), qf[s], sacc[kt]);
            }
        }

        // ---- causal / tail mask (diagonal or ragged tile only), row max over the tile
        const bool need_mask = (a.causal && j == i) || (j + 1) * BC > T;
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int kidx = j * BC + 32 * kt + 8 * (e >> 2) + 4 * half + (e & 3);
                    if (kidx >= T || (a.causal && kidx > qidx)) sacc[kt][e] = kNegInf;
                }
        }
        float mt = kNegInf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kt][e]);
        mt = fmaxf(mt, wave_shfl_xor(mt, 32));

        // ---- Eq. 1 then the log-space test; AND over every row of the head's query block
        const float m_new = fmaxf(m, mt);
        const bool vote_skip = !row_ok || mt == kNegInf || (mt - m_new) * c < a.thr;
        const bool wave_skip = __all(vote_skip);
        if (lane == 0) lds_vote[wave] = wave_skip;
        __syncthreads();
        bool skip = true;
#pragma unroll
        for (int w = 0; w < NWH; ++w) skip = skip && lds_vote[hsub * NWH + w];
        if (wrow == 0 && lane == 0 && mask_row) mask_row[j] = (uint8_t)skip;
        if (skip) continue;

        // ---- kept tile: rescale (only if some row's max moved), P, row sum, O^T += V^T P^T
        if (!__all(m_new == m)) {
            const float alpha = exp2_fast((m - m_new) * c);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        }
        m = m_new;
        const float mc = m * c;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = exp2_fast(__builtin_fmaf(sacc[kt][8 * p + e], c, -mc));
                    l += pv[e];
                }
                const bf16x8 pb = as_bf16x8(u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});
                // keys of these 8 slots: 32kt + 16p + 4*half + {0..3} and the same + 8
                const char* vsub = &lds_v[st][(32 * kt + 16 * p) * ROWB];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 av = lds_read_tr16_pair((const lds_char*)(vsub + voff[0][dt]),
                                                         (const lds_char*)(vsub + voff[1][dt]));
                    oacc[dt] = mfma32x32x16(av, pb, oacc[dt]);
                }
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: O / l and LSE for this lane's row
    l += wave_shfl_xor(l, 32);
    if (row_ok) {
        const float inv = 1.f / l;
        float* orow = a.o + (((size_t)b * a.Hq + hq) * T + qidx) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int eg = 0; eg < 4; ++eg)
                *(f32x4*)(orow + 32 * dt + 8 * eg + 4 * half) =
                    f32x4{oacc[dt][4 * eg] * inv, oacc[dt][4 * eg + 1] * inv, oacc[dt][4 * eg + 2] * inv,
                          oacc[dt][4 * eg + 3] * inv};
        if (half == 0 && a.lse) a.lse[((size_t)b * a.Hq + hq) * T + qidx] = m * c * kLn2 + logf(l);
    }
    if (mask_row && wrow == 0)
        for (int j = jend + lane; j < a.nk; j += 64) mask_row[j] = 2;
}

template <int D, int BC, int HPW>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.nq * a.B * (a.Hq / HPW));
    hipLaunchKernelGGL((prefill_kernel<D, BC, HPW>), grid, dim3(2 * BC * HPW), 0, stream, a);
    return hipGetLastError();
}

// Two heads of a kv group per workgroup when the group has an even number of
// heads (they share the staged K/V tiles); otherwise one head.
template <int D, int BC>
hipError_t launch_hpw(const PrefillArgs& a, hipStream_t stream) {
    if (a.G % 2 == 0) return launch<D, BC, 2>(a, stream);
    return launch<D, BC, 1>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int d, int Bc, hipStream_t stream) {
    if (d == 128) return Bc == 128 ? launch_hpw<128, 128>(a, stream) : launch_hpw<128, 64>(a, stream);
    return Bc == 128 ? launch_hpw<64, 128>(a, stream) : launch_hpw<64, 64>(a, stream);
}

}  // namespace blasst
