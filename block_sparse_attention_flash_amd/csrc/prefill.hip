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
// land on the same XCD (its L2 then serves their common K/V tiles); which kv
// heads an XCD serves turns every few query blocks, so that heads that skip
// less than the others do not keep one XCD busy after the rest.
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
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace blasst {

namespace {

#ifndef BLASST_PREFILL_PRIO_Y
#define BLASST_PREFILL_PRIO_Y 1
#endif
constexpr int PRIO_Y = BLASST_PREFILL_PRIO_Y;
#ifndef BLASST_PREFILL_PFV
#define BLASST_PREFILL_PFV 2
#endif
constexpr int PFV = BLASST_PREFILL_PFV;  // V^T prefetch distance in 16-key sub-tiles
constexpr float kLagLog2 = 8.f;          // how far (log2 units) the softmax reference may trail the max

// SKIP = false builds the same kernel without the skip test (every tile kept,
// no vote): the dense reference the test's cost is measured against.
template <int D, int BC, int HPW, bool SKIP = true>
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
    __shared__ __attribute__((aligned(16))) uint32_t lds_vote[NW];

    // ---- workgroup -> (query block, head group, batch)
    const int hg_count = a.Hq / HPW;
    const int bh_count = a.B * hg_count;
    const int L = blockIdx.x;
    int i, hgrp, b;
    if (a.lens != nullptr && a.B <= 64) {
        // Ragged batch: the workgroups take the batch's work heaviest first -- query
        // block i of every sequence that has one (i from the last down; a block's
        // causal work depends on i only), then the blocks past each sequence's end
        // (padded rows, no tiles) at the very end.  Interleaving those cheap
        // workgroups with the heavy ones cost a 16K sequence among three empty ones
        // 3.6 ms against 2.0 ms alone.  Lane b of every wave holds sequence b.
        const int ln = threadIdx.x % 64;
        const int nqb = ln < a.B ? (min(max(a.lens[ln], 0), a.T) + BC - 1) / BC : 0;
        auto items_from = [&](int i0) {  // active items of rows i0 .. nq - 1
            int v = max(nqb - i0, 0);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            return hg_count * v;
        };
        const int active = items_from(0);
        if (L < active) {
            int lo = 0, hi = a.nq - 1;  // the last row i with items_from(i) > L
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (items_from(mid) > L) lo = mid;
                else hi = mid - 1;
            }
            i = lo;
            const int r = L - items_from(i + 1);
            hgrp = r % hg_count;
            if (hg_count % 8 == 0) {
                // XCD r % 8 serves head groups of one residue mod 8; the residue turns
                // every xcd_rot query blocks, as for a plain batch (below)
                const int turn = (a.nq - 1 - i) / a.xcd_rot;
                hgrp = (hgrp % 8 + turn) % 8 + 8 * (hgrp / 8);
            }
            uint64_t has = __ballot(nqb > i);
            for (int k = r / hg_count; k > 0; --k) has &= has - 1;
            b = min(__builtin_ctzll(has), a.B - 1);
        } else {
            int e = L - active;
            b = 0;
            for (; b < a.B - 1; ++b) {
                const int c = (a.nq - __shfl(nqb, b)) * hg_count;
                if (e < c) break;
                e -= c;
            }
            i = __shfl(nqb, b) + e / hg_count;
            hgrp = e % hg_count;
        }
        i = __builtin_amdgcn_readfirstlane(i);
        hgrp = __builtin_amdgcn_readfirstlane(hgrp);
        b = __builtin_amdgcn_readfirstlane(b);
    } else {
        i = a.nq - 1 - L / bh_count;
        int bh = L % bh_count;
        // Workgroups go round-robin over the 8 XCDs; the head groups of a kv group
        // are kept on one XCD, whose L2 then serves their common K/V tiles.  A plain
        // batch gives each XCD one eighth of the (sequence, head group) pairs, and
        // which eighth turns every xcd_rot query blocks (about the query blocks one
        // XCD holds at once): heads skip at very different rates, and with a fixed
        // eighth the XCD holding the least-skipping heads set the launch time (up to
        // 1.16x the mean XCD's work at 50% sparsity on the 32K length sweep).  A
        // ragged batch (more than 64 sequences, with a multiple of 8 kv groups) gives
        // XCD x kv groups x, x + 8, ..., so every sequence's work is spread over all
        // eight XCDs (whole sequences per XCD ran a 16K sequence among three empty ones
        // on a quarter of the chip).
        const int hgpk = a.G / HPW;            // head groups per kv group
        const int nkvg = bh_count / hgpk;      // kv groups in the batch
        if (a.lens && nkvg % 8 == 0) {
            const int x = bh % 8, s = bh / 8;
            bh = (x + 8 * (s / hgpk)) * hgpk + s % hgpk;
        } else if (bh_count % 8 == 0) {
            const int turn = (L / bh_count) / a.xcd_rot;
            bh = ((bh % 8 + turn) % 8) * (bh_count / 8) + bh / 8;
        }
        hgrp = bh % hg_count;
        b = bh / hg_count;
    }
    // Row stride Tcap; this sequence holds its first T rows (a ragged batch
    // gives every sequence its own length, a plain one T = Tcap).
    const int Tcap = a.T;
    const int T = a.lens ? __builtin_amdgcn_readfirstlane(min(max(a.lens[b], 0), Tcap)) : Tcap;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int hsub = wave / NWH, wrow = wave % NWH;
    const int hq = hgrp * HPW + hsub;
    const int hkv = hq / a.G;
    const int col = lane & 31, half = lane >> 5;   // query column of S^T / O^T, and lane half
    const int qidx = i * BC + 32 * wrow + col;     // this lane's query row
    const bool row_ok = qidx < T;
    uint8_t* mask_row = a.mask ? a.mask + (((size_t)b * a.Hq + hq) * a.nq + i) * a.nk : nullptr;

    if (i * BC >= T) {
        // a query block past the end of its sequence: padded rows hold O = 0 and
        // LSE = -inf, and no tile of the row is visited
        if (qidx < Tcap) {
            float* orow = a.o + (((size_t)b * a.Hq + hq) * Tcap + qidx) * D;
#pragma unroll
            for (int e = 0; e < D / 2; e += 4) *(f32x4*)(orow + e + (D / 2) * half) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (half == 0 && a.lse) a.lse[((size_t)b * a.Hq + hq) * Tcap + qidx] = kNegInf;
        }
        if (mask_row && wrow == 0)
            for (int j = lane; j < a.nk; j += 64) mask_row[j] = 2;
        return;
    }

    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)Tcap * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)Tcap * D;
    const float c = a.score_scale;

    // Q^T as the B operand: lane holds q[qidx][16s + 8*half .. +8].
    bf16x8 qf[DS];
    {
        const uint16_t* qrow = a.q + (((size_t)b * a.Hq + hq) * Tcap + min(qidx, T - 1)) * D;
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[s] = as_bf16x8(load16(qrow + 16 * s + 8 * half));
    }

    const int last_row = min(T, (i + 1) * BC) - 1;
    const int jend = a.causal ? last_row / BC + 1 : (T + BC - 1) / BC;

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
    // m: the row's running max (raw, unscaled score units), which the skip test reads;
    // mref: the max the exponentials and (O, l) are currently taken against.  mref trails m by
    // at most kLagLog2 in log2 units, so O and l are rescaled only when some row's max has
    // moved that far (P = 2^(s c - mref c) then stays below 2^kLagLog2, exact in range for
    // bf16 and fp32); the result O / l and the LSE mref c ln 2 + ln l do not depend on mref.
    float m = kNegInf, mref = kNegInf, l = 0.f;

    // ---- tile copies: this wave's 1 KiB pieces, LDS position pp -> row pp / CPR,
    //      physical chunk pp % CPR holding logical chunk (pp % CPR) ^ swizzle(row).
    //      The byte offset inside a tile is fixed per lane; the tile base is
    //      wave-uniform.  Only a ragged last tile clamps its rows to T - 1.
    uint32_t toff[CPW];
#pragma unroll
    for (int f = 0; f < CPW; ++f) toff[f] = tile_copy_offset<CPR>(wave, CPW, f, lane);
    auto issue = [&](const uint16_t* base, char* lds_tile, int j) {
        const uint16_t* tbase = base + (size_t)j * BC * D;
        if (__builtin_expect(tile_is_ragged<BC>(j, T), 0)) {
            // only a last tile running past the sequence clamps its rows (a wave-uniform branch)
#pragma unroll
            for (int f = 0; f < CPW; ++f)
                global_to_lds16_sbase(tbase, tile_copy_clamp<CPR, BC>(toff[f], j, T),
                                      lds_addr(lds_tile + (wave * CPW + f) * 1024));
        } else {
#pragma unroll
            for (int f = 0; f < CPW; ++f)
                global_to_lds16_sbase(tbase, toff[f], lds_addr(lds_tile + (wave * CPW + f) * 1024));
        }
    };
    auto issue_k = [&](int j, int stage) { issue(kbase, &lds_k[stage][0], j); };
    auto issue_v = [&](int j, int stage) { issue(vbase, &lds_v[stage][0], j); };
    // Per-lane byte offsets inside a tile.  The swizzle depends on row & 15 only,
    // which is the same for every 32-key sub-tile, so sub-tile and stage offsets
    // are compile-time constants added to these.
    //   K (S^T A operand): row 32kt + col, chunk 2s + half.  2s only touches
    //   chunk bits 1..3, so the offset for step s is kofs ^ (32 s).
    //   V (transposed, PV A operand): row 16p + r (+ 8 for the second half) with
    //   r = 4(g16 >> 1) + (jj >> 2), chunk 4dt + 2(g16 & 1) + ((jj & 3) >> 1),
    //   8-byte half (jj & 1).  4dt only touches chunk bits 2..3, so dt gives
    //   vofs ^ (64 dt).  Row r + 8 flips swizzle bit 1 with 16 chunks per row
    //   (+ 8 rows and ^ 32) and leaves the 8-chunk swizzle unchanged (+ 8 rows).
    const int kofs = col * ROWB + ((half ^ chunk_swizzle<CPR>(col)) << 4);
    int vofs;
    {
        const int g16 = lane >> 4, jj = lane & 15;
        const int r = 4 * (g16 >> 1) + (jj >> 2);
        const int chunk = 2 * (g16 & 1) + ((jj & 3) >> 1);
        vofs = r * ROWB + ((chunk ^ chunk_swizzle<CPR>(r)) << 4) + (jj & 1) * 8;
    }
    static_assert(CPR == 8 || CPR == 16, "swizzle offsets assume 8 or 16 chunks per row");
    constexpr int VH8 = (chunk_swizzle<CPR>(8) ^ chunk_swizzle<CPR>(0)) << 4;

    // ---- phase X_j: S^T(j) = K(j) Q^T, row max, this wave's vote (state kept for Y_j)
    f32x16 sacc[KT];
    float m_new = kNegInf;
    auto phase_x = [&](int j) {
        const char* kt_base = &lds_k[j & 1][0];
        // K fragments n = d-step-major (s = n / KT, kt = n % KT), so consecutive
        // MFMAs feed the KT independent accumulators; PFK reads kept in flight
        // ahead of the MFMA that consumes them (LDS latency >> one MFMA)
        constexpr int NF = KT * DS, PFK = 8;
        auto kread = [&](int n) -> u32x4 {
            return *(const u32x4*)(kt_base + 32 * (n % KT) * ROWB + (kofs ^ (32 * (n / KT))));
        };
        u32x4 kf[PFK];
#pragma unroll
        for (int n = 0; n < PFK; ++n) kf[n] = kread(n);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) sacc[kt] = f32x16{};
#pragma unroll
        for (int n = 0; n < NF; ++n) {
            const u32x4 cur = kf[n % PFK];
            if (n + PFK < NF) kf[n % PFK] = kread(n + PFK);
            sacc[n % KT] = mfma32x32x16(as_bf16x8(cur), qf[n / KT], sacc[n % KT]);
        }
        // order: PFK reads, then (MFMA n, read n + PFK) pairs, then the last MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, PFK, 0);
#pragma unroll
        for (int n = 0; n < NF; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (n + PFK < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        // causal / tail mask (diagonal or ragged tile only)
        const bool need_mask = (a.causal && j == i) || (j + 1) * BC > T;
        if (need_mask) {
            // key j*BC + 4*half + o is allowed iff o <= lim; branch-free select
            // (sign of lim - o as a bit mask) keeps the compares out of SGPRs
            const int lim = min(T - 1, a.causal ? qidx : T - 1) - j * BC - 4 * half;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int o = 32 * kt + 8 * (e >> 2) + (e & 3);
                    const uint32_t drop = (uint32_t)((lim - o) >> 31);
                    // read the element into a scalar first: bit_cast of a vector
                    // element lvalue reads element 0 with this compiler
                    const float sv = sacc[kt][e];
                    const uint32_t sb = __float_as_uint(sv);
                    sacc[kt][e] = __uint_as_float((sb & ~drop) | (0xff800000u & drop));
                }
        }
        float mt = kNegInf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kt][e]);
        mt = wave_max_xor32(mt);
        // Eq. 1 then the log-space test (log2 units)
        m_new = fmaxf(m, mt);
        if constexpr (SKIP) {
            const bool vote_skip = !row_ok || mt == kNegInf || (mt - m_new) * c < a.thr;
            const bool wave_skip = __all(vote_skip);
            if (lane == 0) lds_vote[wave] = wave_skip ? 1u : 0u;
        }
    };

    // ---- phase Y_j: AND over the head's waves; kept tile -> rescale, P, row sum, O^T += V^T P^T
    auto phase_y = [&](int j) {
        bool skip = SKIP;
        if constexpr (SKIP) {
            // the head's NWH votes are adjacent words: one LDS read for all of them (an
            // AND written with && waited for each word in turn before the next read)
            static_assert(NWH == 2 || NWH == 4, "votes read as one 8- or 16-byte word");
            uint32_t all;
            if constexpr (NWH == 4) {
                const u32x4 v = *(const u32x4*)&lds_vote[hsub * 4];
                all = v[0] & v[1] & v[2] & v[3];
            } else {
                const u32x2 v = *(const u32x2*)&lds_vote[hsub * 2];
                all = v[0] & v[1];
            }
            skip = __builtin_amdgcn_readfirstlane(all) != 0;
        }
        if (wrow == 0 && lane == 0 && mask_row) mask_row[j] = (uint8_t)skip;
        if (skip) return;
        if (!__all(m_new == mref || (m_new - mref) * c <= kLagLog2)) {
            // some row's max moved more than kLagLog2 past its reference: every row moves its
            // reference to its running max (a row still at -inf keeps factor 1)
            const float alpha = m_new == mref ? 1.f : exp2_fast((mref - m_new) * c);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            mref = m_new;
        }
        m = m_new;
        const float mc = mref * c;
        const char* vt_base = &lds_v[j & 1][0];
        // Software-pipelined over the 2*KT sub-tiles of 16 keys: P of sub-tile
        // u + 1 (exp, row sum, bf16 pack) is formed between the four PV MFMAs of
        // sub-tile u, so this wave keeps the VALU busy while its MFMAs run.
        auto make_p = [&](int u) -> bf16x8 {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = exp2_fast(__builtin_fmaf(sacc[u >> 1][8 * (u & 1) + e], c, -mc));
                l += pv[e];
            }
            return as_bf16x8(u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                   pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});
        };
        auto vread = [&](int u, bf16x8* av) {
            // keys of sub-tile u's 8 slots: 16u + 4*half + {0..3} and the same + 8
            const char* vsub = vt_base + 16 * u * ROWB;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int vo = vofs ^ (64 * dt);
                av[dt] = lds_read_tr16_pair((const lds_char*)(vsub + vo), (const lds_char*)(vsub + 8 * ROWB + (vo ^ VH8)));
            }
        };
        // V^T fragments of sub-tile u + PFV are read before the MFMAs of u
        constexpr int NU = 2 * KT, NB = PFV + 1;
        bf16x8 av[NB][DT];
#pragma unroll
        for (int u = 0; u < PFV; ++u) vread(u, av[u]);
        bf16x8 pb = make_p(0);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (u + PFV < NU) vread(u + PFV, av[(u + PFV) % NB]);
            const bf16x8 pcur = pb;
            if (u + 1 < NU) pb = make_p(u + 1);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma32x32x16(av[u % NB][dt], pcur, oacc[dt]);
            if (u + 1 < NU) {
                if (u + PFV < NU) __builtin_amdgcn_sched_group_barrier(0x100, 2 * DT, 0);  // V^T reads first
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);  // two exp
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // fma, add, pack
                }
            }
        }
    };

    // ---- phase schedule.  Head group g runs phase q = p - g of its own sequence
    //      X_0, Y_0, X_1, Y_1, ...: with two groups, in every phase one group forms
    //      S (MFMA-heavy) while the other does softmax + P V (VALU-heavy), and each
    //      SIMD holds one wave of each.  K(j) is read in phases 2j and 2j+1, V(j) in
    //      2j+1 and 2j+2; both are double-buffered.  Every wave issues its pieces of
    //      one tile copy per phase (K(p/2 + 1) in even phases, V((p+1)/2) in odd
    //      ones) into the buffer freed by the previous barrier, and the barrier
    //      closing the phase waits for every copy but the one just issued.  Each
    //      group runs its own straight-line loop; both pass the same barriers.
    auto open_phase = [&](int p) -> bool {
        const int jn = (p & 1) ? (p + 1) / 2 : p / 2 + 1;
        if (jn >= jend) return false;
        if (p & 1) issue_v(jn, jn & 1);
        else issue_k(jn, jn & 1);
        return true;
    };
    auto close_phase = [&](bool issued) {
        if (issued) asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(CPW) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // Two head groups: the phase's whole tile copy is issued by the group in phase X, CPX
    // pieces per wave, and the group in phase Y issues none.  Issuing a share of every copy
    // at its head cost the phase-Y wave -- the longer of each SIMD's two -- 7-14% of its
    // phase, while the phase-X wave waited 17-24% of its phase at the closing barrier.  A
    // copy issued in phase p is waited for when its waves close phase p + 1 (in phase Y
    // then, with nothing of their own in flight).
    constexpr int CPX = 2 * CPW;
    auto open_phase_x = [&](int p) -> bool {
        const int jn = (p & 1) ? (p + 1) / 2 : p / 2 + 1;
        if (jn >= jend) return false;
        const uint16_t* tbase = ((p & 1) ? vbase : kbase) + (size_t)jn * BC * D;
        char* tile = (p & 1) ? &lds_v[jn & 1][0] : &lds_k[jn & 1][0];
        if (__builtin_expect(tile_is_ragged<BC>(jn, T), 0)) {
#pragma unroll
            for (int f = 0; f < CPX; ++f)
                global_to_lds16_sbase(tbase, tile_copy_clamp<CPR, BC>(tile_copy_offset<CPR>(wrow, CPX, f, lane), jn, T),
                                      lds_addr(tile + (wrow * CPX + f) * 1024));
        } else {
#pragma unroll
            for (int f = 0; f < CPX; ++f)
                global_to_lds16_sbase(tbase, tile_copy_offset<CPR>(wrow, CPX, f, lane),
                                      lds_addr(tile + (wrow * CPX + f) * 1024));
        }
        return true;
    };
    auto close_phase_x = [&](bool issued) {
        if (issued) asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(CPX) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // The wave in phase Y gets the higher issue priority: its PV MFMAs then take
    // the matrix unit as soon as they are ready (between the S MFMAs of the wave
    // in phase X) instead of stalling its in-order VALU stream behind them.
    auto raise_prio = [&] { if (HPW == 2) __builtin_amdgcn_s_setprio(PRIO_Y); };
    auto lower_prio = [&] { if (HPW == 2) __builtin_amdgcn_s_setprio(0); };
    issue_k(0, 0);
    issue_v(0, 0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");  // K(0)
    __syncthreads();
    if (HPW == 1) {
        for (int j = 0; j < jend; ++j) {
            bool is = open_phase(2 * j);
            phase_x(j);
            close_phase(is);
            is = open_phase(2 * j + 1);
            phase_y(j);
            close_phase(is);
        }
    } else if (hsub == 0) {
        for (int j = 0; j < jend; ++j) {
            const bool is = open_phase_x(2 * j);
            phase_x(j);
            close_phase_x(is);
            raise_prio();
            phase_y(j);
            lower_prio();
            close_phase_x(false);
        }
        close_phase_x(false);  // phase 2 jend: the other group's last phase Y; no copy
    } else {
        close_phase_x(false);  // phase 0: the other group's X(0), which issues its copy
        for (int j = 0; j < jend; ++j) {
            const bool is = open_phase_x(2 * j + 1);
            phase_x(j);
            close_phase_x(is);
            raise_prio();
            phase_y(j);
            lower_prio();
            close_phase_x(false);
        }
    }

    // ---- epilogue: O / l and LSE for this lane's row
    l = wave_sum_xor32(l);
    if (qidx < Tcap) {
        // rows past a ragged sequence's end (inside its last block) hold O = 0, LSE = -inf
        const float inv = row_ok ? 1.f / l : 0.f;
        float* orow = a.o + (((size_t)b * a.Hq + hq) * Tcap + qidx) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int eg = 0; eg < 4; ++eg)
                *(f32x4*)(orow + 32 * dt + 8 * eg + 4 * half) =
                    f32x4{oacc[dt][4 * eg] * inv, oacc[dt][4 * eg + 1] * inv, oacc[dt][4 * eg + 2] * inv,
                          oacc[dt][4 * eg + 3] * inv};
        if (half == 0 && a.lse) a.lse[((size_t)b * a.Hq + hq) * Tcap + qidx] = row_ok ? mref * c * kLn2 + logf(l) : kNegInf;
    }
    if (mask_row && wrow == 0)
        for (int j = jend + lane; j < a.nk; j += 64) mask_row[j] = 2;
}

// Workgroups of prefill_kernel<D, BC, HPW> resident on the whole device at once
// (compute units x workgroups per unit), queried once per device.
template <int D, int BC, int HPW>
hipError_t resident_workgroups(int* out) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_kernel<D, BC, HPW, true>, 2 * BC * HPW, 0);
        if (e != hipSuccess) return e;
        n = std::max(1, cus) * std::max(1, per_cu);
        cache[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return hipSuccess;
}

template <int D, int BC, int HPW>
hipError_t launch(const PrefillArgs& a_in, hipStream_t stream) {
    PrefillArgs a = a_in;
    int resident = 0;
    hipError_t e = resident_workgroups<D, BC, HPW>(&resident);
    if (e != hipSuccess) return e;
    // one turn of the kv-group -> XCD rotation per batch of resident workgroups
    a.xcd_rot = std::max(1, resident / std::max(1, a.B * (a.Hq / HPW)));
    const dim3 grid((unsigned)a.nq * a.B * (a.Hq / HPW));
    if (a.dense)
        hipLaunchKernelGGL((prefill_kernel<D, BC, HPW, false>), grid, dim3(2 * BC * HPW), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_kernel<D, BC, HPW, true>), grid, dim3(2 * BC * HPW), 0, stream, a);
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

// ---------------------------------------------------------------------------
// Decision margins of causal / full prefill, for every lambda at once.
//
// BLASST blog, section on the decision rule (Eq. 5) and section on the
// one-pass calibration (Algorithm 2): the test of tile (i, j) for query row r
// compares m~_r - m_r (block max minus the updated running max) with ln(lambda),
// and the tile is skipped iff every row of the query block votes to skip.  A
// skipped tile never moves the running max, so m_r is the prefix max of the
// block maxima whatever lambda is; the tile's margin
//     M(i, j) = max over the rows r of the query block of (m~_r - m_r) / sqrt(d)
// (natural-log units) decides it for every lambda: skipped iff M < ln(lambda).
// This pass forms S = Q K^T only (no softmax, no V) and writes M for visited
// tiles, NaN for tiles above the diagonal.
namespace blasst {
namespace {

template <int D, int BC>
__global__ __launch_bounds__(2 * BC) void prefill_margin_kernel(PrefillArgs a) {
    constexpr int NW = BC / 32;            // waves, 32 query rows each
    constexpr int KT = BC / 32;
    constexpr int DS = D / 16;
    constexpr int CPR = D / 8;
    constexpr int ROWB = 2 * D;
    constexpr int TILE = BC * ROWB;
    constexpr int CPW = TILE / (1024 * NW);
    static_assert(TILE % (1024 * NW) == 0, "tile copies must split evenly over the waves");

    __shared__ __attribute__((aligned(16))) char lds_k[2][TILE];
    __shared__ float lds_m[2][NW];

    const int bh_count = a.B * a.Hq;
    const int L = blockIdx.x;
    const int i = a.nq - 1 - L / bh_count;
    const int bh = L % bh_count;
    const int hq = bh % a.Hq, b = bh / a.Hq;
    const int hkv = hq / a.G;
    const int T = a.T;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;
    const int qidx = i * BC + 32 * wave + col;
    const bool row_ok = qidx < T;
    const float inv_sqrt_d = a.score_scale * 0.69314718055994531f;  // (log2 e / sqrt d) * ln 2

    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    bf16x8 qf[DS];
    {
        const uint16_t* qrow = a.q + (((size_t)b * a.Hq + hq) * T + min(qidx, T - 1)) * D;
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[s] = as_bf16x8(load16(qrow + 16 * s + 8 * half));
    }
    const int last_row = min(T, (i + 1) * BC) - 1;
    const int jend = a.causal ? last_row / BC + 1 : a.nk;

    uint32_t toff[CPW];
#pragma unroll
    for (int f = 0; f < CPW; ++f) toff[f] = tile_copy_offset<CPR>(wave, CPW, f, lane);
    auto issue_k = [&](int j) {
        const uint16_t* tbase = kbase + (size_t)j * BC * D;
        const bool ragged = tile_is_ragged<BC>(j, T);
#pragma unroll
        for (int f = 0; f < CPW; ++f) {
            const uint32_t off = ragged ? tile_copy_clamp<CPR, BC>(toff[f], j, T) : toff[f];
            global_to_lds16_sbase(tbase, off, lds_addr(&lds_k[j & 1][(wave * CPW + f) * 1024]));
        }
    };
    const int kofs = col * ROWB + ((half ^ chunk_swizzle<CPR>(col)) << 4);

    float* mrow = a.margin + (((size_t)b * a.Hq + hq) * a.nq + i) * a.nk;
    float m = kNegInf;  // running (prefix) max of this lane's row, raw score units
    issue_k(0);
    for (int j = 0; j < jend; ++j) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's pieces of K(j)
        __syncthreads();                                   // all of K(j); stage (j+1)&1 and lds_m[(j+1)&1] free
        if (j + 1 < jend) issue_k(j + 1);
        // the previous tile's margin: every wave's vote has landed
        if (j > 0 && tid == 0) {
            float x = kNegInf;
#pragma unroll
            for (int w = 0; w < NW; ++w) x = fmaxf(x, lds_m[(j - 1) & 1][w]);
            mrow[j - 1] = x;
        }
        f32x16 sacc[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            sacc[kt] = f32x16{};
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const u32x4 kf = *(const u32x4*)(&lds_k[j & 1][0] + 32 * kt * ROWB + (kofs ^ (32 * s)));
                sacc[kt] = mfma32x32x16(as_bf16x8(kf), qf[s], sacc[kt]);
            }
        }
        if ((a.causal && j == i) || (j + 1) * BC > T) {
            const int lim = min(T - 1, a.causal ? qidx : T - 1) - j * BC - 4 * half;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int o = 32 * kt + 8 * (e >> 2) + (e & 3);
                    const uint32_t drop = (uint32_t)((lim - o) >> 31);
                    const float sv = sacc[kt][e];  // scalar first (see the main kernel)
                    sacc[kt][e] = __uint_as_float((__float_as_uint(sv) & ~drop) | (0xff800000u & drop));
                }
        }
        float mt = kNegInf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kt][e]);
        mt = wave_max_xor32(mt);
        const float m_new = fmaxf(m, mt);
        // a row that sees no key of the tile, or a row past T, votes skip with no effect
        float dr = (row_ok && mt != kNegInf) ? (mt - m_new) * inv_sqrt_d : kNegInf;
        m = m_new;
        dr = wave_max_xor32(wave_max_xor16(row16_max(dr)));
        if (lane == 0) lds_m[j & 1][wave] = dr;
    }
    __syncthreads();
    if (tid == 0 && jend > 0) {
        float x = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) x = fmaxf(x, lds_m[(jend - 1) & 1][w]);
        mrow[jend - 1] = x;
    }
    for (int j = jend + tid; j < a.nk; j += blockDim.x) mrow[j] = __builtin_nanf("");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D, int BC>
hipError_t launch_margins(const PrefillArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.nq * a.B * a.Hq);
    hipLaunchKernelGGL((prefill_margin_kernel<D, BC>), grid, dim3(2 * BC), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_margins(const PrefillArgs& a, int d, int Bc, hipStream_t stream) {
    if (d == 128) return Bc == 128 ? launch_margins<128, 128>(a, stream) : launch_margins<128, 64>(a, stream);
    return Bc == 128 ? launch_margins<64, 128>(a, stream) : launch_margins<64, 64>(a, stream);
}

}  // namespace blasst
