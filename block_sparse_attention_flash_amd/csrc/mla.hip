// Split-KV MLA decode with the skip-softmax rule.
//
// Multi-head latent attention in its absorbed decode form: every query head
// of a sequence reads the same cache row per token, 576 bf16 = a 512-wide
// latent part followed by a 64-wide rotary part, and the value of a token is
// its latent part.  BLASST blog, section on the decode kernel: with the KV
// state compressed into the latent space, MLA decode can be compute bound, so
// besides the V load (here V is part of the K row and is read anyway) a skip
// must also save the softmax work -- the exp, the row sum and the P V product.
// A head skips a block when its block max trails the running max by more than
// ln(lambda) (Eq. 5); a skipping head's P is zero, and the P V product of a
// 16-head tile runs only if some head of the tile keeps the block.
//
// Two kernels, both over split-KV work units (split, group of heads, sequence):
//
// mla_pipe_kernel (groups of 64 heads; blocks of 32 or 64 tokens): a two-role
// pipeline over 32-token sub-blocks, described above the kernel.  It is what
// every head count that is a multiple of 64 runs.
//
// mla_split_kernel (groups of 32 heads, 64-token blocks): 8 waves; per block
//   copy     the block's cache rows go HBM -> LDS (global_load_lds_dwordx4,
//            whole rows per instruction) through two 72 KiB stages.  Latent
//            rows (1 KiB) are XOR-swizzled by 16-byte chunk within groups of 16
//            chunks, rotary rows (128 B) within their 8 chunks (both kernels).
//   S^T      K Q^T on MFMA 16x16x32 bf16 (16 keys x 16 heads per tile, 18
//            k-steps over the 576 columns); wave w owns head tile w / (8/NT)
//            and 16-key tiles, q^T stays in registers.  Block max per head
//            through LDS, then every lane takes the decisions of its heads
//            (prefix max: no cascade inside a block).
//   P        2^(t - m) for kept heads, 0 otherwise, rounded to bf16 and stored
//            head-major in LDS; each S wave keeps its heads' row-sum partials.
//   O^T      += V^T P^T: wave w owns latent columns [64w, 64w + 64) of every
//            head of the group, V^T read from the latent tile with
//            ds_read_b64_tr_b16, P^T from LDS.  No cross-wave reduction of O.
// Scores are in log2 units (t = s * scale * log2 e); the test reads
// t~ - m < ln(lambda) * log2 e.
#include "device_common.h"
#include "kernels.h"

namespace blasst {

namespace {

constexpr int MLA_DN = 512;  // latent columns (the value)
constexpr int MLA_DR = 64;   // rotary columns
constexpr int MLA_DQK = MLA_DN + MLA_DR;

// Physical 16-byte chunk of logical chunk c in latent row r: an XOR within each
// group of 16 chunks (256 B) by a GF(2)-linear image of the row's low four bits
// (bits 0..3 -> masks 3, 6, 9, 8).  Measured (SQ_LDS_BANK_CONFLICT on an
// in-bounds probe of both read patterns) to leave the S K reads (ds_read_b128,
// lane (n, g): row 16 kt + n, chunk 4 st + g) and the P V transposed reads
// (ds_read_b64_tr_b16, lane (n, g): rows 4 g + n / 4 and + 16, chunk
// 2 dt + (n & 3) / 2) free of bank conflicts; the plain XOR by the row costs the
// transposed reads a 2-way conflict.
__device__ __forceinline__ int nope_chunk(int c, int r) {
    const int f = ((r & 1) * 3) ^ (((r >> 1) & 1) * 6) ^ (((r >> 2) & 1) * 9) ^ (((r >> 3) & 1) * 8);
    return (c & ~15) | ((c & 15) ^ f);
}

// BCM tokens per block; NSTAGE blocks staged in LDS (NSTAGE - 1 in flight
// while one is computed): 2 x 72 KiB at BCM = 64, 4 x 36 KiB at BCM = 32.
template <int NT, int BCM>
__global__ __launch_bounds__(512) void mla_split_kernel(MlaArgs a) {
    constexpr int W = 8;
    constexpr int MLA_BC = BCM;
    constexpr int KTB = BCM / 16;                // 16-key tiles per block
    constexpr int WPH = W / NT;                  // S waves per head tile
    constexpr int KPW = KTB / WPH;               // 16-key tiles per S wave
    constexpr int HG = 16 * NT;                  // heads per workgroup
    constexpr int NOPE_ROW = 2 * MLA_DN;         // 1024 B
    constexpr int ROPE_ROW = 2 * MLA_DR;         // 128 B
    constexpr int NOPE_TILE = MLA_BC * NOPE_ROW;
    constexpr int STAGE = NOPE_TILE + MLA_BC * ROPE_ROW;
    constexpr int NSTAGE = BCM == 32 ? 4 : 2;
    constexpr int PROW = 2 * MLA_BC + 16;        // one head's P^T row: BCM bf16 + 16 B pad
    constexpr int KSTEPS = MLA_DQK / 32;         // 18
    constexpr int NOPE_PER_WAVE = BCM / W;       // latent rows (1 KiB copies) per wave per block
    constexpr int ROPE_WAVES = BCM / 8;          // waves with one rotary copy (8 rows) per block
    static_assert(NT == 2 || NT == 4, "16*NT heads per workgroup, NT in {2, 4}");
    static_assert(BCM == 64 || (BCM == 32 && NT == 4), "32-token blocks need 64 heads per workgroup");
    static_assert(KPW >= 1, "every S wave owns at least one key tile");

    __shared__ __attribute__((aligned(16))) char lds_kv[NSTAGE][STAGE];
    __shared__ __attribute__((aligned(16))) char lds_p[HG * PROW];
    __shared__ float lds_pmax[WPH][HG];
    __shared__ float lds_l[WPH][HG];

    const int split = blockIdx.x, hgrp = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int N = a.N, nk = a.nk;
    const int j0 = (int)((int64_t)split * nk / a.S);
    const int j1 = (int)((int64_t)(split + 1) * nk / a.S);
    const int h0 = hgrp * HG;
    const uint16_t* kvb = a.kv + (size_t)b * N * MLA_DQK;

    // S role: head tile sht, key tiles kt0 .. kt0 + KPW - 1
    const int sht = wave / WPH, kt0 = (wave % WPH) * KPW;
    bf16x8 qf[KSTEPS];
    {
        const uint16_t* qrow = a.q + ((size_t)b * a.Hq + h0 + 16 * sht + n) * MLA_DQK;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(load16(qrow + 32 * s + 8 * g));
    }

    f32x4 oacc[NT][4];
    float m_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = kNegInf;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) oacc[nt][dd] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float l_part = 0.f;  // S role: row-sum partial of head 16*sht + n over this lane's keys

    // Wave w copies latent rows w, w + 8, ... of a block (one 1 KiB instruction
    // per row, lane l landing at physical chunk l) and, for w < BCM/8, the 8
    // rotary rows 8w .. 8w + 7 (lane l -> row 8w + l/8, physical chunk l % 8).
    // Rows past the context re-read its last row.
    const bool rope_wave = wave < ROPE_WAVES;
    auto issue = [&](int j, int stage) {
        char* base = &lds_kv[stage][0];
#pragma unroll
        for (int i = 0; i < NOPE_PER_WAVE; ++i) {
            const int r = wave + W * i;
            const int key = min(j * MLA_BC + r, N - 1);
            const int c = nope_chunk(lane, r);
            global_to_lds16(kvb + (size_t)key * MLA_DQK + 8 * c, lds_addr(base + r * NOPE_ROW));
        }
        if (rope_wave) {
            const int r = 8 * wave + (lane >> 3);
            const int key = min(j * MLA_BC + r, N - 1);
            const int c = (lane & 7) ^ (r & 7);
            global_to_lds16(kvb + (size_t)key * MLA_DQK + MLA_DN + 8 * c,
                            lds_addr(base + NOPE_TILE + 8 * wave * ROPE_ROW));
        }
    };
    // block j's copies are complete once only those of the nb blocks issued after it are outstanding
    auto wait_blocks_after = [&](int nb) {
        if (nb <= 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else if (nb == 1) {
            if (rope_wave) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NOPE_PER_WAVE + 1) : "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NOPE_PER_WAVE) : "memory");
        } else {
            if (rope_wave) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (NOPE_PER_WAVE + 1)) : "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NOPE_PER_WAVE) : "memory");
        }
    };
    static_assert(NSTAGE - 2 <= 2, "wait_blocks_after covers up to two blocks in flight");

#pragma unroll
    for (int q = 0; q < NSTAGE - 1; ++q)
        if (j0 + q < j1) issue(j0 + q, q);
    for (int j = j0; j < j1; ++j) {
        const int st = (j - j0) % NSTAGE;
        // this block's rows have landed (every wave's copies) and the stage the
        // next copy goes to (block j - 1's) and the P buffer are no longer read
        wait_blocks_after(min(NSTAGE - 2, j1 - 1 - j));
        __syncthreads();
        if (j + NSTAGE - 1 < j1) issue(j + NSTAGE - 1, (j + NSTAGE - 1 - j0) % NSTAGE);
        const char* kvt = &lds_kv[st][0];

        // ---- S^T tiles of this wave: fragment f = (k-step f / KPW, key tile f % KPW),
        //      PFK fragments read ahead of the MFMA that consumes them
        f32x4 sacc[KPW];
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk) sacc[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            constexpr int NF = KSTEPS * KPW, PFK = 8;
            auto kread = [&](int f) -> u32x4 {
                const int st_ = f / KPW, kk = f % KPW;
                const int r = 16 * (kt0 + kk) + n;
                const int c = 4 * (st_ < 16 ? st_ : st_ - 16) + g;
                const int off = st_ < 16 ? r * NOPE_ROW + (nope_chunk(c, r) << 4)
                                         : NOPE_TILE + r * ROPE_ROW + ((c ^ (r & 7)) << 4);
                return *(const u32x4*)(kvt + off);
            };
            u32x4 kf[PFK];
#pragma unroll
            for (int f = 0; f < PFK; ++f) kf[f] = kread(f);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const u32x4 cur = kf[f % PFK];
                if (f + PFK < NF) kf[f % PFK] = kread(f + PFK);
                sacc[f % KPW] = mfma16x16x32(as_bf16x8(cur), qf[f / KPW], sacc[f % KPW]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, PFK, 0);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (f + PFK < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        float pm = kNegInf;
#pragma unroll
        for (int kk = 0; kk < KPW; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = j * MLA_BC + 16 * (kt0 + kk) + 4 * g + i;
                float x = sacc[kk][i] * a.score_scale;
                x = key < N ? x : kNegInf;
                sacc[kk][i] = x;
                pm = fmaxf(pm, x);
            }
        pm = wave_max_xor32(wave_max_xor16(pm));
        if (g == 0) lds_pmax[wave % WPH][16 * sht + n] = pm;
        __syncthreads();

        // ---- decisions for head n of every head tile (Eq. 1, then Eq. 5)
        bool keep[NT];
        float alpha[NT];
        bool any_keep = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float bm = kNegInf;
#pragma unroll
            for (int w = 0; w < WPH; ++w) bm = fmaxf(bm, lds_pmax[w][16 * nt + n]);
            const float m_new = fmaxf(m_run[nt], bm);
            keep[nt] = !((bm - m_new) < a.thr);
            alpha[nt] = exp2_fast(m_run[nt] - m_new);
            m_run[nt] = m_new;
            any_keep = any_keep || keep[nt];
        }
        if (a.skip != nullptr && wave == 0 && g == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                a.skip[((size_t)b * a.Hq + h0 + 16 * nt + n) * nk + j] = (uint8_t)!keep[nt];
        }
        // the P V step runs iff some head of the group keeps the block
        const bool vkeep = __builtin_amdgcn_readfirstlane((int)(__ballot(any_keep) != 0)) != 0;

        // ---- P of this wave's tiles (0 for a skipping head), row-sum partials
        {
            bool kp = keep[0];
            float mm = m_run[0], al = alpha[0];
#pragma unroll
            for (int nt = 1; nt < NT; ++nt)
                if (sht == nt) { kp = keep[nt]; mm = m_run[nt]; al = alpha[nt]; }
            l_part *= al;
            if (vkeep) {
#pragma unroll
                for (int kk = 0; kk < KPW; ++kk) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = exp2_fast(sacc[kk][i] - mm);
                        p[i] = kp ? e : 0.f;
                    }
                    l_part += (p[0] + p[1]) + (p[2] + p[3]);
                    const u32x2 w2 = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
                    *(u32x2*)(lds_p + (16 * sht + n) * PROW + 2 * (16 * (kt0 + kk) + 4 * g)) = w2;
                }
            }
        }
        __syncthreads();

        // ---- O^T += V^T P^T for latent columns [64 wave, 64 wave + 64)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) oacc[nt][dd] *= alpha[nt];
        if (vkeep) {
#pragma unroll
            for (int ks = 0; ks < MLA_BC / 32; ++ks) {
                // B = P^T: k-slots 0..3 = keys 32ks + 4g + i, 4..7 = keys 32ks + 16 + 4g + i
                bf16x8 pf[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const char* prow = lds_p + (16 * nt + n) * PROW + 2 * (32 * ks + 4 * g);
                    const u32x2 lo = *(const u32x2*)prow;
                    const u32x2 hi = *(const u32x2*)(prow + 32);
                    pf[nt] = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
                }
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    const int dt = 4 * wave + dd;
                    const int cc = 2 * dt + ((n & 3) >> 1);
                    const int r0 = 32 * ks + 4 * g + (n >> 2), r1 = r0 + 16;
                    const u32x2 lo = lds_read_tr16((const lds_char*)(kvt + r0 * NOPE_ROW + (nope_chunk(cc, r0) << 4) + (n & 1) * 8));
                    const u32x2 hi = lds_read_tr16((const lds_char*)(kvt + r1 * NOPE_ROW + (nope_chunk(cc, r1) << 4) + (n & 1) * 8));
                    const bf16x8 av = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) oacc[nt][dd] = mfma16x16x32(av, pf[nt], oacc[nt][dd]);
                }
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: l per head from the S waves' partials, O / l and LSE
    {
        const float lw = wave_sum_xor32(wave_sum_xor16(l_part));
        if (g == 0) lds_l[wave % WPH][16 * sht + n] = lw;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < WPH; ++w) l += lds_l[w][16 * nt + n];
        const float inv = l > 0.f ? 1.f / l : 0.f;  // 0: a split with no block
        const size_t orow = ((size_t)b * a.Hq + h0 + 16 * nt + n) * a.S + split;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
            const f32x4 o = oacc[nt][dd] * inv;
            *(f32x4*)(a.o_part + orow * MLA_DN + 16 * (4 * wave + dd) + 4 * g) = o;
        }
        if (wave == 0 && g == 0) a.lse_part[orow] = l > 0.f ? m_run[nt] * kLn2 + logf(l) : kNegInf;
    }
}

// 64 heads per workgroup as a two-role pipeline over 32-token sub-blocks.
// Waves 0-3 ("S waves", one 16-head tile each) form S^T of sub-block t, and at
// the end of each BCM-token block take their heads' decisions and write P^T
// (bf16, head-major) plus each head's rescale factor to LDS.  Waves 4-7 ("P V
// waves", 128 latent columns of all 64 heads each) copy the V^T fragments of
// sub-block t out of its stage into registers while the S waves read it, and
// run O^T += V^T P^T for the block whose P was written one step before.  So a
// sub-block's stage is free after one step, three sub-blocks are in flight, and
// one barrier per step orders everything: the sub-block's copies have landed,
// P and the factors of the finished block are visible, and the stage the next
// copy overwrites is no longer read.  Each SIMD holds one wave of each role, so
// the S MFMAs of one block overlap the P V MFMAs of the previous one.
template <int BCM>
__global__ __launch_bounds__(512) void mla_pipe_kernel(MlaArgs a) {
    constexpr int W = 8;                         // waves: four of each role
    static_assert(64 * W == 512, "the launch bounds hold eight waves");
    constexpr int SB = 32;                       // tokens per sub-block (one pipeline step)
    constexpr int HPB = BCM / SB;                // sub-blocks per decision block
    constexpr int HG = 64;                       // heads per workgroup
    constexpr int NOPE_ROW = 2 * MLA_DN;         // 1024 B
    constexpr int ROPE_ROW = 2 * MLA_DR;         // 128 B
    constexpr int NOPE_TILE = SB * NOPE_ROW;
    constexpr int STAGE = NOPE_TILE + SB * ROPE_ROW;  // 36 KiB
    constexpr int NSTAGE = 4;
    constexpr int KSTEPS = MLA_DQK / 32;         // 18
    constexpr int CW = MLA_DN / 4;               // latent columns per P V wave (128)
    constexpr int DTW = CW / 16;                 // 16-column tiles per P V wave (8)
    // P^T of a sub-block (32 keys per head) lives in buffer u % NPH from the end
    // of its block's decision step until its P V step u + HPB
    constexpr int NPH = HPB == 1 ? 2 : 3;
    // One head's P^T row of a sub-block: 32 bf16 in k-slot order (bytes 16 g .. 16 g + 15 hold
    // keys 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, the B fragment of lane group g), written
    // and read 16 bytes per lane.  Row strides measured bank-conflict free for that pattern
    // (96 B) or, where three buffers must fit (64-token blocks), the one with the fewest (64 B).
    constexpr int PROW = HPB == 1 ? 96 : 64;
    static_assert(BCM == 32 || BCM == 64, "32- or 64-token blocks");
    static_assert(NSTAGE * STAGE + NPH * HG * PROW + 2 * HG * 4 * 2 + 2 * 4 * 4 <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) char lds_kv[NSTAGE][STAGE];
    __shared__ __attribute__((aligned(16))) char lds_p[NPH][HG * PROW];
    __shared__ float lds_alpha[2][HG];           // per block parity: each head's rescale factor
    __shared__ int lds_tkeep[2][4];              // per block parity: does some head of tile w keep
    __shared__ float lds_ml[2][HG];              // final m and l per head

    const int split = blockIdx.x, hgrp = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool s_wave = wave < 4;
    const int g = lane >> 4, n = lane & 15;
    const int N = a.N, nk = a.nk;
    const int j0 = (int)((int64_t)split * nk / a.S);
    const int j1 = (int)((int64_t)(split + 1) * nk / a.S);
    const int nsub = (j1 - j0) * HPB;            // sub-blocks of this split
    const int nsteps = nsub + HPB;               // sub-block u's P V runs in step u + HPB
    const int key_base = j0 * BCM;               // first key of the split
    const int h0 = hgrp * HG;
    const uint16_t* kvb = a.kv + (size_t)b * N * MLA_DQK;

    // The sub-block copies are issued by one role's four waves: latent rows iw + 4 i (i < 8;
    // one 1 KiB instruction each, lane l at physical chunk l) and one rotary copy of 8 rows
    // (lane l -> row 8 iw + l / 8, chunk l % 8), iw being the wave's index in its role.  A
    // wave that issues a copy waits for the CU's address unit to take it, and every wave
    // issuing its share right after the step's barrier held all of them back: the role with
    // slack issues them all -- the S waves with 64-token blocks (107.9 -> 105.6 us on
    // decode_mla_32k), the P V waves with 32-token blocks (107.1 -> 101.3 us); the other
    // choice was 10-13% slower than all waves issuing.
    constexpr bool S_ISSUES = BCM == 64;
    constexpr int NIW = 4;                       // issuing waves
    const int iw = S_ISSUES ? wave : wave - 4;
    const bool issuer = S_ISSUES ? wave < 4 : wave >= 4;
    const bool rope_wave = issuer;               // SB / 8 = 4 rotary copies: one per issuing wave
    static_assert(SB / 8 == NIW, "one rotary copy per issuing wave");
    constexpr int NPC = SB / NIW;                // latent copies per issuing wave per sub-block
    auto issue = [&](int t) {
        if (!issuer) return;
        char* base = &lds_kv[t % NSTAGE][0];
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int r = iw + NIW * i;
            const int key = min(key_base + t * SB + r, N - 1);
            global_to_lds16(kvb + (size_t)key * MLA_DQK + 8 * nope_chunk(lane, r), lds_addr(base + r * NOPE_ROW));
        }
        if (rope_wave) {
            const int r = 8 * iw + (lane >> 3);
            const int key = min(key_base + t * SB + r, N - 1);
            const int c = (lane & 7) ^ (r & 7);
            global_to_lds16(kvb + (size_t)key * MLA_DQK + MLA_DN + 8 * c, lds_addr(base + NOPE_TILE + 8 * iw * ROPE_ROW));
        }
    };
    // sub-block t's copies are complete once only those of the nb sub-blocks issued after it are outstanding
    auto wait_after = [&](int nb) {
        if (nb <= 0 || !issuer) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else if (nb == 1) {
            if (rope_wave) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NPC + 1) : "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NPC) : "memory");
        } else {
            if (rope_wave) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (NPC + 1)) : "memory");
            else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NPC) : "memory");
        }
    };

#pragma unroll
    for (int q = 0; q < NSTAGE - 1; ++q)
        if (q < nsub) issue(q);

    // Step t forms S^T of sub-block t (t < nsub), and the P V of sub-block
    // t - HPB, whose block was decided at the end of step t - HPB + (HPB - 1 -
    // its half) <= t - 1.  The two roles run separate loops (their register
    // state is disjoint) that pass the same barriers.
    if (s_wave) {
        // ---- S role: q^T of head tile `wave`, the block's S^T tiles, m and l of head n
        bf16x8 qf[KSTEPS];
        {
            const uint16_t* qrow = a.q + ((size_t)b * a.Hq + h0 + 16 * wave + n) * MLA_DQK;
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(load16(qrow + 32 * s + 8 * g));
        }
        f32x4 sacc[2 * HPB];
        float m_run = kNegInf, l_part = 0.f;
        for (int t = 0; t < nsteps; ++t) {
            if (t < nsub) wait_after(min(2, nsub - 1 - t));
            // this wave's LDS reads of the stage the next copy overwrites, and its
            // P / factor writes, are complete before the barrier
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            if (t + NSTAGE - 1 < nsub) issue(t + NSTAGE - 1);
            if (t >= nsub) continue;
            const char* kvt = &lds_kv[t % NSTAGE][0];
            // S^T of sub-block t: fragment f = (k-step f / 2, key tile f % 2); the two
            // tiles become the block's tiles 2 hs and 2 hs + 1
            const int hs = t % HPB;
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            {
                constexpr int NF = KSTEPS * 2, PFK = 8;
                auto kread = [&](int f) -> u32x4 {
                    const int st_ = f / 2, kt = f % 2;
                    const int r = 16 * kt + n;
                    const int c = 4 * (st_ < 16 ? st_ : st_ - 16) + g;
                    const int off = st_ < 16 ? r * NOPE_ROW + (nope_chunk(c, r) << 4)
                                             : NOPE_TILE + r * ROPE_ROW + ((c ^ (r & 7)) << 4);
                    return *(const u32x4*)(kvt + off);
                };
                u32x4 kf[PFK];
#pragma unroll
                for (int f = 0; f < PFK; ++f) kf[f] = kread(f);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const u32x4 cur = kf[f % PFK];
                    if (f + PFK < NF) kf[f % PFK] = kread(f + PFK);
                    if (f % 2 == 0) s0 = mfma16x16x32(as_bf16x8(cur), qf[f / 2], s0);
                    else s1 = mfma16x16x32(as_bf16x8(cur), qf[f / 2], s1);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, PFK, 0);
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (f + PFK < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
#pragma unroll
            for (int x = 0; x < HPB; ++x)
                if (x == hs) {
                    sacc[2 * x] = s0;
                    sacc[2 * x + 1] = s1;
                }
            if (hs != HPB - 1) continue;
            // ---- end of block jb: decisions of head n (Eq. 1, then Eq. 5), P^T, factors
            const int jb = j0 + t / HPB;
            float bm = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 2 * HPB; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = jb * BCM + 16 * kt + 4 * g + i;
                    float x = sacc[kt][i] * a.score_scale;
                    x = key < N ? x : kNegInf;
                    sacc[kt][i] = x;
                    bm = fmaxf(bm, x);
                }
            bm = wave_max_xor32(wave_max_xor16(bm));
            const float m_new = fmaxf(m_run, bm);
            const bool keep = !((bm - m_new) < a.thr);
            const float alpha = exp2_fast(m_run - m_new);
            m_run = m_new;
            l_part *= alpha;
            if (a.skip != nullptr && g == 0) a.skip[((size_t)b * a.Hq + h0 + 16 * wave + n) * nk + jb] = (uint8_t)!keep;
            const int u0 = t - (HPB - 1);  // the block's first sub-block
#pragma unroll
            for (int sb = 0; sb < HPB; ++sb) {
                float p[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float e = exp2_fast(sacc[2 * sb + i / 4][i % 4] - m_run);
                    p[i] = keep ? e : 0.f;
                }
                l_part += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                char* prow = &lds_p[(u0 + sb) % NPH][0] + (16 * wave + n) * PROW + 16 * g;
                *(u32x4*)prow = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                      pack_bf16x2(p[6], p[7])};
            }
            const int par = (t / HPB) & 1;
            if (g == 0) lds_alpha[par][16 * wave + n] = alpha;
            const bool tk = __ballot(keep) != 0;
            if (lane == 0) lds_tkeep[par][wave] = tk;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // ---- epilogue: l and m of head n for the P V waves; LSE
        const float l = wave_sum_xor32(wave_sum_xor16(l_part));
        if (g == 0) {
            lds_ml[0][16 * wave + n] = m_run;
            lds_ml[1][16 * wave + n] = l;
            const size_t orow = ((size_t)b * a.Hq + h0 + 16 * wave + n) * a.S + split;
            a.lse_part[orow] = l > 0.f ? m_run * kLn2 + logf(l) : kNegInf;
        }
        __syncthreads();
    } else {
        // ---- P V role: O^T of column tiles 8 cw + dt for the 4 head tiles, V^T sets
        const int cw = wave - 4;
        f32x4 oacc[4][DTW];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt) oacc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // V^T of the last two sub-blocks: vb the newer, va the older (register moves, no indexing)
        bf16x8 va[DTW], vb[DTW];
        for (int t = 0; t < nsteps; ++t) {
            if (t < nsub) wait_after(min(2, nsub - 1 - t));
            // this wave's LDS reads of the stage the next copy overwrites, and its
            // P / factor writes, are complete before the barrier
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            if (t + NSTAGE - 1 < nsub) issue(t + NSTAGE - 1);
            // ---- V^T of sub-block t for columns [128 cw, 128 cw + 128)
            auto read_vt = [&](bf16x8* dst) {
                const char* kvt = &lds_kv[t % NSTAGE][0];
                const int r0 = 4 * g + (n >> 2), r1 = r0 + 16;
#pragma unroll
                for (int dt = 0; dt < DTW; ++dt) {
                    const int cc = 2 * (DTW * cw + dt) + ((n & 3) >> 1);
                    const u32x2 lo = lds_read_tr16((const lds_char*)(kvt + r0 * NOPE_ROW + (nope_chunk(cc, r0) << 4) + (n & 1) * 8));
                    const u32x2 hi = lds_read_tr16((const lds_char*)(kvt + r1 * NOPE_ROW + (nope_chunk(cc, r1) << 4) + (n & 1) * 8));
                    dst[dt] = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
                }
            };
            // ---- O^T += V^T P^T for sub-block u = t - HPB (half u % HPB of block kb):
            //      the block's rescale once, then the MFMAs of the head tiles that keep it
            const int u = t - HPB;
            const int kb = u / HPB;
            const int par = kb & 1;
            const char* pbuf = &lds_p[(u + NPH) % NPH][0];
            auto p_frag = [&](int nt) -> bf16x8 {
                // B = P^T: k-slots 0..3 = keys 4 g + i, 4..7 = keys 16 + 4 g + i of the sub-block
                return as_bf16x8(*(const u32x4*)(pbuf + (16 * nt + n) * PROW + 16 * g));
            };
            if constexpr (HPB == 1) {
                // 32-token blocks: every LDS read of the step (V^T of sub-block t, the
                // factors, P) goes out before the MFMAs of sub-block t - 1 (in vb)
                bf16x8 nv[DTW];
                if (t < nsub) read_vt(nv);
                if (t >= HPB) {
                    float al[4];
                    int tk[4];
                    bf16x8 pf[4];
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        al[nt] = lds_alpha[par][16 * nt + n];
                        tk[nt] = lds_tkeep[par][nt];
                        pf[nt] = p_frag(nt);
                    }
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        if (!__all(al[nt] == 1.f)) {
#pragma unroll
                            for (int dt = 0; dt < DTW; ++dt) oacc[nt][dt] *= al[nt];
                        }
                        if (__builtin_amdgcn_readfirstlane(tk[nt]) == 0) continue;
#pragma unroll
                        for (int dt = 0; dt < DTW; ++dt) oacc[nt][dt] = mfma16x16x32(vb[dt], pf[nt], oacc[nt][dt]);
                    }
                }
                if (t < nsub) {
#pragma unroll
                    for (int dt = 0; dt < DTW; ++dt) vb[dt] = nv[dt];
                }
            } else {
                // 64-token blocks: sub-block t - 2 is va (the registers do not allow the
                // read-ahead); the ring moves on every step, after the last sub-block too
                if (t >= HPB) {
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        if (u % HPB == 0) {
                            const float al = lds_alpha[par][16 * nt + n];
                            if (!__all(al == 1.f)) {
#pragma unroll
                                for (int dt = 0; dt < DTW; ++dt) oacc[nt][dt] *= al;
                            }
                        }
                        if (__builtin_amdgcn_readfirstlane(lds_tkeep[par][nt]) == 0) continue;
                        const bf16x8 pf = p_frag(nt);
#pragma unroll
                        for (int dt = 0; dt < DTW; ++dt) oacc[nt][dt] = mfma16x16x32(va[dt], pf, oacc[nt][dt]);
                    }
                }
#pragma unroll
                for (int dt = 0; dt < DTW; ++dt) va[dt] = vb[dt];
                if (t < nsub) read_vt(vb);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // ---- epilogue: O / l
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const float l = lds_ml[1][16 * nt + n];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const size_t orow = ((size_t)b * a.Hq + h0 + 16 * nt + n) * a.S + split;
#pragma unroll
            for (int dt = 0; dt < DTW; ++dt)
                *(f32x4*)(a.o_part + orow * MLA_DN + 16 * (DTW * cw + dt) + 4 * g) = oacc[nt][dt] * inv;
        }
    }
}

}  // namespace

hipError_t launch_decode_mla(const MlaArgs& a, int Bc, hipStream_t stream) {
    // 64 heads per workgroup: the two-role pipeline (either block size)
    if (a.Hq % 64 == 0) {
        const dim3 grid(a.S, a.Hq / 64, a.B);
        if (Bc == 32) hipLaunchKernelGGL((mla_pipe_kernel<32>), grid, dim3(512), 0, stream, a);
        else hipLaunchKernelGGL((mla_pipe_kernel<64>), grid, dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    // 32 heads per workgroup (64-token blocks; the caller checked Hq % 32 == 0)
    hipLaunchKernelGGL((mla_split_kernel<2, 64>), dim3(a.S, a.Hq / 32, a.B), dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace blasst
