// Split-KV decode with the skip-softmax rule, and the log-sum-exp merge of splits.
//
// BLASST blog, section on the decode kernel: decode is bound by reading the KV
// cache, so what a skip must save there is the V load.  The decision needs the
// block max, which needs S = q K^T; deciding block by block would serialise
// "decide -> load V".  The blog's answer is batched load scheduling: form the
// S blocks of a batch first, decide them together, then issue V loads only for
// kept blocks.  Here a batch ("phase") is as large as the registers allow
// (for 4-head groups at Bc = 128: 16 blocks, a whole 32K/16-way split).
//
// One workgroup = W waves per (batch b, kv head, split), or two per split
// (DSPLIT = 2, each forming O for half of the d columns) when one per split
// would leave CUs idle.  Each block is cut into 32-key units; wave w owns units
// w, w+W, w+2W, ... of the phase.
//
//  K pass   every unit's 32 K rows go HBM -> LDS (global_load_lds_dwordx4,
//           whole rows per instruction, XOR-swizzled by 16-byte chunk) through
//           a ring of NSLOT slots per wave, so copies for later units are in
//           flight while earlier ones are multiplied; they are read back in the
//           MFMA A layout (ds_read_b128).  S^T = K q^T runs on MFMA 16x16x32
//           bf16 with the 32 keys as two 16-row tiles and the G query heads of
//           the group as 16-wide column tiles (heads beyond G are zero columns
//           that never vote).  q^T sits in registers, or for four head tiles
//           in LDS, read per unit (its registers then hold S^T tiles).  The
//           S^T tiles stay in registers; each unit's per-head partial max goes
//           to LDS.
//  decide   a barrier; every lane then walks the phase's blocks in order.
//           Because a skipped block never moves the running max
//           (mt < m + ln(lambda) < m), the running max before block j is the
//           prefix max of the block maxima: all decisions of the phase are
//           taken at once with no cascade.  V is needed for a block iff some
//           head of the group keeps it.  With paired workgroups the blocks
//           every wave has finished before its last two K units arrive are
//           decided first, and their V copies start in the slots those two
//           units free (early V).
//  V pass   only kept units: V rows (or half rows) go HBM -> LDS through the
//           same slots and are read back transposed (ds_read_b64_tr_b16) as
//           the A operand of O^T += V^T P^T.  P^T is the S^T accumulator (same
//           lane layout) after 2^(t - m), rounded to bf16.
// Cache policy of the copies: V non-temporal; K non-temporal except where the
// other workgroup of a pair, or another head part, reads it again from L2 (the
// K pass says where).
// Scores are kept in log2 units (t = s * log2(e)), so P uses v_exp_f32 directly
// and the test reads t~ - m < ln(lambda) * log2(e).
#include "device_common.h"
#include "kernels.h"

#include <type_traits>
#include <climits>
#include <mutex>

namespace blasst {

namespace {

constexpr float LAZY_LAG = 8.f;  // how far (log2 units) a head's softmax reference may trail its max

// s_waitcnt vmcnt(F * n) for a wave-uniform n in 0..3 (the count is an immediate)
template <int F>
__device__ __forceinline__ void wait_vm(int n) {
    if (n <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(F) : "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * F) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * F) : "memory");
}

// MARGINS: the margin pass (BLASST blog, section on the one-pass calibration):
// the K pass and the decisions' prefix max only, writing for every (head,
// block) D = (m~ - m_new) in natural-log units and for every block the max of D
// over the group's heads (skipped / V not loaded at lambda iff below ln lambda);
// no V pass, no partial outputs.
// DSPLIT = 2: two workgroups per split, each forming the V pass for one half
// of the d columns; both run the same K pass and decisions (the second one's
// K reads hit the L2 the first one filled: the pair sits on one XCD), so each
// CU streams K plus half of V instead of K plus all of V.
// HS > 1: HS workgroups per split, each the whole pass for HT = 16 NT of the
// group's heads (a group wider than one workgroup's registers hold); they sit
// on one XCD, so the K and V blocks they share come from HBM once.  The V skip
// mask is then an OR of the parts' "loaded" votes: the launcher sets it to
// "not loaded" first and each part clears the bytes of the blocks it loads.
// ONEPHASE: every split spans at most one phase (the launcher checks), so K
// is non-temporal throughout (see the K pass) with no per-unit branch.
template <int D, int BC, int NT, int UW, int W, int NSLOT, bool MARGINS = false, int DSPLIT = 1, int HS = 1,
          bool ONEPHASE = false>
__global__ __launch_bounds__(64 * W) void decode_split_kernel(DecodeArgs a) {
    constexpr int KG = BC / 32;           // 32-key units per block
    constexpr int UPP = W * UW;           // units per phase
    constexpr int BPP = UPP / KG;         // blocks per phase
    constexpr int DS = D / 32;            // MFMA k-steps over d for S
    constexpr int FR = D / 16;            // 16-byte fragments per lane per unit
    constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
    constexpr int HT = 16 * NT;           // head columns per workgroup
    constexpr int VSLOT = 32 * D * 2;     // bytes of one 32-row K (or V) slice
    constexpr int DV = D / DSPLIT;        // V columns this workgroup forms O for
    constexpr int DTV = DV / 16;          // 16-wide d tiles of O^T
    constexpr int FRV = DV / 16;          // 16-byte fragments per lane per V unit
    constexpr int CPRV = DV / 8;          // 16-byte chunks per staged V row
    static_assert(DSPLIT == 1 || DSPLIT == 2, "one or two workgroups per split");
    static_assert(HS == 1 || DSPLIT == 1, "head parts run the full-width V pass");
    static_assert(UPP % KG == 0, "units must tile the phase");
    static_assert(BPP <= 32, "decision masks are 32-bit");
    static_assert(W * DTV * 4 * 64 * 4 <= NSLOT * W * VSLOT, "O reduction must fit the staging area");
    static_assert(NSLOT >= 2 && NSLOT <= 4, "staging ring depth");
    // Early V (pairs with a two-slot ring): the blocks whose units every wave has
    // finished before its last two K units arrive are decided at that point, and
    // the V copies of the wave's first VD units go into the slots those two K
    // units free, so the V stream is already running when the K pass ends.
    constexpr int VD = NSLOT * DSPLIT;    // V units in the ring (a V unit fills 1/DSPLIT slot)
    constexpr bool EARLYV = !MARGINS && DSPLIT == 2 && NSLOT == 2 && UW >= 4;
    constexpr int UE = UW - 2;            // K units consumed before the early decisions
    constexpr int BE = EARLYV ? W * UE / KG : 0;  // blocks decided early
    constexpr int BG = BPP < 4 ? BPP : 4;  // blocks per group of LDS reads in the decisions
    static_assert(!EARLYV || (UE % NSLOT == 0 && W * UE % KG == 0 && BE % BG == 0 && W * VD <= KG * BE),
                  "the ring's first V units must lie in blocks decided early");

    __shared__ __attribute__((aligned(16))) char lds_v[NSLOT * W * VSLOT];
    __shared__ float lds_pmax[2][UPP * HT];
    __shared__ float lds_l[W][64];
    // Four head tiles: q^T is read from LDS per unit (its registers hold S^T tiles instead)
    constexpr bool QL = NT >= 4;
    __shared__ __attribute__((aligned(16))) char lds_q[QL ? HT * D * 2 : 16];

    int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z, half = 0, part = 0;
    if constexpr (DSPLIT * HS > 1) {
        // 1-D grid: workgroups L, L + 8, ... form a unit's DSPLIT * HS parts, so
        // that they land on the same XCD (workgroups go round-robin over 8)
        constexpr int NP = DSPLIT * HS;
        const int L = blockIdx.x;
        const int unit = (L / (8 * NP)) * 8 + (L % 8);
        part = (L / 8) % NP;
        half = DSPLIT == 2 ? part : 0;
        if (unit >= a.S * a.Hkv * a.B) return;
        split = unit % a.S;
        hkv = (unit / a.S) % a.Hkv;
        b = unit / (a.S * a.Hkv);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    // Row stride a.N (capacity); this sequence's context is its first N keys, nk
    // blocks (a ragged batch gives every sequence its own length).  Splits
    // partition the sequence's own blocks; a split left without one (S > nk)
    // writes the merge identity, O = 0 and LSE = -inf.
    const int G = a.G;
    const int h0 = HS > 1 ? part * HT : 0;  // this workgroup's first head of the group
    const int N = a.lens ? __builtin_amdgcn_readfirstlane(min(max(a.lens[b], 0), a.N)) : a.N;
    const int nk = a.lens ? (N + BC - 1) / BC : a.nk;
    const int j0 = (int)((int64_t)split * nk / a.S);
    const int j1 = (int)((int64_t)(split + 1) * nk / a.S);

    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.N * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.N * D;
    if (a.lens && split == a.S - 1 && nk < a.nk && part == 0) {
        // blocks past the sequence's end are not visited (2)
        for (int x = threadIdx.x; x < (G + 1) * (a.nk - nk); x += 64 * W) {
            const int r = x / (a.nk - nk), j = nk + x % (a.nk - nk);
            uint8_t* row = r < G ? a.skip : a.vskip;
            if (row != nullptr)
                row[(r < G ? ((size_t)b * a.Hq + (size_t)hkv * G + r) : ((size_t)b * a.Hkv + hkv)) * a.nk + j] = 2;
        }
    }

    // Each unit's 32 K rows go HBM -> LDS (global_load_lds_dwordx4, whole rows per
    // instruction, XOR-swizzled by 16-byte chunk) into the wave's staging slots;
    // unit u of the wave (in the phase starting at block p0) uses slot u % NSLOT.
    // Units past the split re-read its last block (cached), so the wait counts are
    // fixed.  Cache policy: non-temporal where no other workgroup reads the rows,
    // and in a split's first phase, where the two workgroups of a pair start
    // together and the second one's reads still find the first one's lines in L2.
    // Later phases of a pair keep the default policy: the pair drifts apart, and
    // non-temporal lines left L2 before the second read (a 32K-key split ran 1.36x
    // slower).  Head parts (HS > 1) share K and V for the whole pass: default policy.
    auto slot_of = [&](int u) { return lds_v + (NSLOT * wave + (u % NSLOT)) * VSLOT; };
    auto issue_k_as = [&](int p0, int u, auto stream) {
        const int U = wave + W * u;
        const int key0 = min(p0 + U / KG, j1 - 1) * BC + (U % KG) * 32;
        const char* slot = slot_of(u);
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            const int p = 64 * f + lane;
            const int row = p / CPR, cc = (p % CPR) ^ (row & (CPR - 1));
            const int key = min(key0 + row, N - 1);
            global_to_lds16<decltype(stream)::value>(kbase + (size_t)key * D + cc * 8, lds_addr(slot + 1024 * f));
        }
    };
    // The first phase's first units go out before q is read: the compiler waits for
    // the q loads before the phase loop, which would otherwise hold these copies back
    // by a whole memory round trip (decode_32k: 24.14 -> 23.75 us).  The 8-wave launch
    // with one workgroup per split keeps the old order: at d = 128, Bc = 64 the early
    // copies would need one register more than its 256.
    constexpr bool EARLY_K = !(DSPLIT == 1 && W == 8);
    if (EARLY_K && j0 < j1) {
#pragma unroll
        for (int u = 0; u < (NSLOT < UW ? NSLOT : UW); ++u) {
            if constexpr (HS == 1) issue_k_as(j0, u, std::true_type{});
            else issue_k_as(j0, u, std::false_type{});
        }
    }

    // q^T as the B operand: lane (g, n) holds q[head n][32s + 8g .. +8].
    bf16x8 qf[QL ? 1 : NT][DS];
    bool head_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int h = h0 + nt * 16 + n;
        head_ok[nt] = h < G;
        if constexpr (!QL) {
            const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)hkv * G + (head_ok[nt] ? h : 0)) * D;
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                u32x4 z = {0u, 0u, 0u, 0u};
                qf[nt][s] = as_bf16x8(head_ok[nt] ? load16(qrow + 32 * s + 8 * g) : z);
            }
        }
    }
    // QL: the group's q rows (zero beyond G), chunk c of row r at chunk c ^ (r mod CPR)
    constexpr int QCH = QL ? HT * CPR / (64 * W) : 1;  // 16-byte chunks per thread
    static_assert(!QL || HT * CPR % (64 * W) == 0, "q chunks must split evenly over the threads");
    u32x4 qst[QCH];
    if constexpr (QL) {
#pragma unroll
        for (int x = 0; x < QCH; ++x) {
            const int e = x * 64 * W + threadIdx.x, r = e / CPR, c = e % CPR;
            const int h = h0 + r;
            qst[x] = h < G ? load16(a.q + ((size_t)b * a.Hq + (size_t)hkv * G + h) * D + 8 * c) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    bool q_staged = !QL;

    f32x4 oacc[NT][DTV];
    // m_run: the head's running max (log2 units), which the decisions continue;
    // mref: the max P and (O, l) are currently taken against.  mref trails m_run by
    // at most LAZY_LAG, so the phase's rescale of O and l (VALU work on the
    // accumulators, which live partly in AGPRs) runs only when some head's max has
    // moved that far; P = 2^(t - mref) then stays below 2^LAZY_LAG, exact in range
    // for bf16 and fp32, and O / l and the LSE mref ln 2 + ln l do not depend on mref.
    float m_run[NT], mref[NT], l_part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = kNegInf;
        mref[nt] = kNegInf;
        l_part[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DTV; ++dt) oacc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int parity = 0;
    for (int p0 = j0; p0 < j1; p0 += BPP, parity ^= 1) {
        const int nb = min(BPP, j1 - p0);
        int ukey0[UW];
        bool uok[UW];
#pragma unroll
        for (int u = 0; u < UW; ++u) {
            const int U = wave + W * u;
            ukey0[u] = (p0 + U / KG) * BC + (U % KG) * 32;
            uok[u] = U / KG < nb;
        }

        // ================= K pass =================
        // K units (issue_k_as above) in the wave's staging slots -- the same slots
        // and copy pattern as the V pass -- read back in the MFMA A layout
        // (ds_read_b128).  With EARLY_K the first phase's first units are already
        // in flight.
        const bool k_stream = HS == 1 && (DSPLIT == 1 || ONEPHASE || p0 == j0);
        auto issue_k = [&](int u) {  // one uniform branch per unit, not per copy
            if (k_stream) issue_k_as(p0, u, std::true_type{});
            else issue_k_as(p0, u, std::false_type{});
        };
        if (!EARLY_K || p0 != j0) {
#pragma unroll
            for (int u = 0; u < (NSLOT < UW ? NSLOT : UW); ++u) issue_k(u);
        }
        if constexpr (QL) {
            if (!q_staged) {  // first phase: q goes to LDS while the first K copies are in flight
#pragma unroll
                for (int x = 0; x < QCH; ++x) {
                    const int e = x * 64 * W + threadIdx.x, r = e / CPR, c = e % CPR;
                    *(u32x4*)(lds_q + r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4)) = qst[x];
                }
                __syncthreads();
                q_staged = true;
            }
        }

        // ---- decisions (prefix max of the block maxima; no cascade): blocks
        //      [lo, hi) of the phase, continuing the running max m_dec
        float m_dec[NT];
        uint32_t keep[NT];
        float vmax_blk[MARGINS ? BPP : 1];
#pragma unroll
        for (int bi = 0; bi < (MARGINS ? BPP : 1); ++bi) vmax_blk[bi] = kNegInf;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            m_dec[nt] = m_run[nt];
            keep[nt] = 0u;
        }
        auto decide = [&](int lo, int hi) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                // block maxima four blocks at a time: each group's LDS reads go out together
                float m = m_dec[nt];
                uint32_t kb = keep[nt];
#pragma unroll
                for (int b0 = lo; b0 < hi; b0 += BG) {
                    float bmv[BG];
#pragma unroll
                    for (int bb = 0; bb < BG; ++bb) {
                        float bm = kNegInf;
#pragma unroll
                        for (int kg = 0; kg < KG; ++kg)
                            bm = fmaxf(bm, lds_pmax[parity][((b0 + bb) * KG + kg) * HT + nt * 16 + n]);
                        bmv[bb] = bm;
                    }
#pragma unroll
                    for (int bb = 0; bb < BG; ++bb) {
                        const int bi = b0 + bb;
                        if (bi < nb) {
                            const float bm = bmv[bb];
                            m = fmaxf(m, bm);
                            kb |= (uint32_t)(!((bm - m) < a.thr)) << bi;
                            if constexpr (MARGINS) {
                                const float dm = head_ok[nt] ? (bm - m) * kLn2 : kNegInf;
                                if (wave == 0 && g == 0 && head_ok[nt])
                                    a.margin[((size_t)b * a.Hq + (size_t)hkv * G + h0 + nt * 16 + n) * a.nk + p0 + bi] = dm;
                                if (HS == 1 && a.vmargin != nullptr) vmax_blk[bi] = fmaxf(vmax_blk[bi], row16_max(dm));
                            }
                        }
                    }
                }
                m_dec[nt] = m;
                keep[nt] = head_ok[nt] ? kb : 0u;
            }
        };
        auto vslot_of = [&](int u) { return lds_v + NSLOT * wave * VSLOT + (u % VD) * (VSLOT / DSPLIT); };
        auto issue_v = [&](int u) {
            const char* slot = vslot_of(u);
#pragma unroll
            for (int f = 0; f < FRV; ++f) {
                const int p = 64 * f + lane;
                const int row = p / CPRV, cc = (p % CPRV) ^ (row & (CPRV - 1));
                const int key = min(ukey0[u] + row, N - 1);
                global_to_lds16<HS == 1>(vbase + (size_t)key * D + half * DV + cc * 8, lds_addr(slot + 1024 * f));
            }
        };
        // this wave's kept units among the first VD (known after the early decisions)
        uint32_t km_early = 0;

        f32x4 t[UW][2][NT];
#pragma unroll
        for (int u = 0; u < UW; ++u) {
            if constexpr (EARLYV) {
                if (u == UE) {
                    // every wave has published the maxima of its units 0 .. UE - 1,
                    // which cover blocks 0 .. BE - 1
                    __syncthreads();
                    decide(0, BE);
                    uint32_t vk = 0;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) vk |= keep[nt];
                    vk = row16_or(vk);
#pragma unroll
                    for (int v = 0; v < VD; ++v)
                        km_early |= (uint32_t)(uok[v] && ((vk >> ((wave + W * v) / KG)) & 1u)) << v;
                    km_early = (uint32_t)__builtin_amdgcn_readfirstlane((int)km_early);
                }
            }
            // K(u) is complete once only the copies issued after it are outstanding:
            // the K units u + 1 .. u + NSLOT - 1, and (early V) the V units issued
            // into the slot K(UE) freed
            if (EARLYV && u == UE + 1) wait_vm<FRV>(__builtin_popcount(km_early & ((1u << DSPLIT) - 1u)));
            else wait_vm<FR>(min(NSLOT - 1, UW - 1 - u));
            const char* kslot = slot_of(u);
            u32x4 kf[2][DS];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int s = 0; s < DS; ++s) {
                    const int r = 16 * kt + n, c = 4 * s + g;
                    kf[kt][s] = *(const u32x4*)(kslot + r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4));
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this slot has been read
            if (u + NSLOT < UW) issue_k(u + NSLOT);
            if constexpr (EARLYV) {
                // the slot K(u) used holds V units (u % NSLOT) * DSPLIT .. + DSPLIT - 1 of the ring
                if (u >= UE) {
#pragma unroll
                    for (int v = 0; v < VD; ++v)
                        if (v / DSPLIT == u % NSLOT && ((km_early >> v) & 1u)) issue_v(v);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float pm = kNegInf;
                bf16x8 qv[DS];
#pragma unroll
                for (int s = 0; s < DS; ++s) {
                    if constexpr (QL) {
                        const int r = nt * 16 + n, c = 4 * s + g;
                        qv[s] = as_bf16x8(*(const u32x4*)(lds_q + r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4)));
                    } else {
                        qv[s] = qf[nt][s];
                    }
                }
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < DS; ++s) acc = mfma16x16x32(as_bf16x8(kf[kt][s]), qv[s], acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = ukey0[u] + 16 * kt + 4 * g + i;
                        float x = acc[i] * a.score_scale;
                        x = key < N ? x : kNegInf;
                        acc[i] = x;
                        pm = fmaxf(pm, x);
                    }
                    t[u][kt][nt] = acc;
                }
                // over the 4 lane groups g (the 16 key rows of each): the permlane
                // form is faster but takes two registers, which one head tile's
                // ring-fed K pass cannot spare
                if constexpr (NT == 1) {
                    pm = fmaxf(pm, wave_shfl_xor(pm, 16));
                    pm = fmaxf(pm, wave_shfl_xor(pm, 32));
                } else {
                    pm = wave_max_xor32(wave_max_xor16(pm));
                }
                if (uok[u] && g == 0) lds_pmax[parity][(wave + W * u) * HT + nt * 16 + n] = pm;
            }
        }
        __syncthreads();

        // ================= decide (the blocks not decided early) =================
        decide(BE, BPP);
        uint32_t vkeep = 0;
        bool lag = false;  // some head's max ran more than LAZY_LAG past its reference
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            vkeep |= keep[nt];
            m_run[nt] = head_ok[nt] ? m_dec[nt] : m_run[nt];
            lag |= !(m_run[nt] == mref[nt] || m_run[nt] - mref[nt] <= LAZY_LAG);
        }
        vkeep = row16_or(vkeep);
        if constexpr (MARGINS) {
            // (head parts: the launcher forms the group's max from the per-head margins)
            if (HS == 1 && a.vmargin != nullptr && wave == 0 && lane == 0) {
                float* vrow = a.vmargin + ((size_t)b * a.Hkv + hkv) * a.nk + p0;
                for (int bi = 0; bi < nb; ++bi) vrow[bi] = vmax_blk[bi];
            }
            __syncthreads();  // lds_pmax[parity] is rewritten two phases on
            continue;         // the margin pass stops here: no V pass
        }

        // decision bytes: one lane per (head, block)
        if (a.skip != nullptr && half == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int h = h0 + nt * 16 + n;
                if (!head_ok[nt]) continue;
                uint8_t* row = a.skip + ((size_t)b * a.Hq + (size_t)hkv * G + h) * a.nk + p0;
                for (int bi = wave * 4 + g; bi < nb; bi += 4 * W) row[bi] = (uint8_t)(((keep[nt] >> bi) & 1u) ^ 1u);
            }
        }
        if (a.vskip != nullptr && half == 0) {
            uint8_t* row = a.vskip + ((size_t)b * a.Hkv + hkv) * a.nk + p0;
            for (int bi = threadIdx.x; bi < nb; bi += 64 * W) {
                const uint8_t skipped = (uint8_t)(((vkeep >> bi) & 1u) ^ 1u);
                if (HS == 1) row[bi] = skipped;
                else if (!skipped) row[bi] = 0;  // parts that load the block all store the same 0
            }
        }

        // ================= V pass (kept units only) =================
        bool kept[UW];
#pragma unroll
        for (int u = 0; u < UW; ++u) kept[u] = uok[u] && ((vkeep >> ((wave + W * u) / KG)) & 1u);

        uint32_t km = 0;  // kept units of this wave (the same in every lane)
#pragma unroll
        for (int u = 0; u < UW; ++u) km |= (uint32_t)kept[u] << u;
        km = (uint32_t)__builtin_amdgcn_readfirstlane((int)km);
        // A V unit of DV columns fills 1/DSPLIT of a slot: the V ring holds VD =
        // NSLOT * DSPLIT units per wave (more V copies in flight when each is smaller).
        // With early V the ring's first VD units are already on their way.
        if constexpr (!EARLYV) {
#pragma unroll
            for (int u = 0; u < (VD < UW ? VD : UW); ++u)
                if ((km >> u) & 1u) issue_v(u);
        }

        // move every head's reference to its running max when one has run too far
        // ahead (overlaps the V loads).  Each wave holds every head in the same
        // lanes and the same m_run, mref, so all waves take the branch together and
        // keep one reference per head: their partial O and l are summed at the end.
        if (__any(lag)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float alpha = m_run[nt] == mref[nt] ? 1.f : exp2_fast(mref[nt] - m_run[nt]);
                l_part[nt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DTV; ++dt) oacc[nt][dt] *= alpha;
                mref[nt] = m_run[nt];
            }
        }

#pragma unroll
        for (int u = 0; u < UW; ++u) {
            if ((km >> u) & 1u) {
                // V(u) is complete once only the kept units issued after it
                // (among u + 1 .. u + VD - 1) are outstanding
                wait_vm<FRV>(__builtin_popcount((km >> (u + 1)) & ((1u << (VD - 1)) - 1u)));
                const lds_char* vslot = (const lds_char*)vslot_of(u);
                const int blk_bit = (wave + W * u) / KG;
                bf16x8 pf[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bool kp = (keep[nt] >> blk_bit) & 1u;
                    float p[8];
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float e = exp2_fast(t[u][kt][nt][i] - mref[nt]);
                            p[4 * kt + i] = kp ? e : 0.f;
                        }
                    l_part[nt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                    u32x4 w4 = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
                    pf[nt] = as_bf16x8(w4);
                }
#pragma unroll
                for (int dt = 0; dt < DTV; ++dt) {
                    const int cc = 2 * dt + ((n & 3) >> 1);
                    const int r0 = 4 * g + (n >> 2), r1 = 16 + 4 * g + (n >> 2);
                    const u32x2 lo = lds_read_tr16(vslot + r0 * (2 * DV) + ((cc ^ (r0 & (CPRV - 1))) << 4) + (n & 1) * 8);
                    const u32x2 hi = lds_read_tr16(vslot + r1 * (2 * DV) + ((cc ^ (r1 & (CPRV - 1))) << 4) + (n & 1) * 8);
                    const bf16x8 av = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) oacc[nt][dt] = mfma16x16x32(av, pf[nt], oacc[nt][dt]);
                }
            }
            if (u + VD < UW && ((km >> (u + VD < UW ? u + VD : 0)) & 1u)) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // unit u's place in the ring has been read
                issue_v(u + VD);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    if constexpr (MARGINS) return;
    // ---- reduce the waves' partial O^T and l; write the split's result
    __syncthreads();
    float* red = (float*)lds_v;  // [W waves][DT][4][64]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const float l = wave_sum_xor32(wave_sum_xor16(l_part[nt]));
#pragma unroll
        for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[((wave * DTV + dt) * 4 + i) * 64 + lane] = oacc[nt][dt][i];
        lds_l[wave][lane] = l;
        __syncthreads();
        float lt = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) lt += lds_l[w][lane];
        const int h = h0 + nt * 16 + n;
        if (h < G) {
            const size_t orow = ((size_t)b * a.Hq + (size_t)hkv * G + h) * a.S + split;
            const float inv = lt > 0.f ? 1.f / lt : 0.f;  // 0: a split with no block
            for (int dt = wave; dt < DTV; dt += W) {
                float o4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = 0.f;
#pragma unroll
                    for (int w = 0; w < W; ++w) x += red[((w * DTV + dt) * 4 + i) * 64 + lane];
                    o4[i] = x * inv;
                }
                *(f32x4*)(a.o_part + orow * D + half * DV + 16 * dt + 4 * g) = f32x4{o4[0], o4[1], o4[2], o4[3]};
            }
            if (wave == 0 && g == 0 && half == 0) a.lse_part[orow] = mref[nt] * kLn2 + logf(lt);
        }
        __syncthreads();
    }
}

// Wide-group decode: one kv head shared by 33..64 query heads (MQA and wide
// GQA), d = 128.  The decisions and the skip rule are those of
// decode_split_kernel (Eq. 5 of the BLASST blog on the prefix max of the block
// maxima, no cascade; V copied only for blocks some head keeps); the work is
// laid out differently, because 64 heads' worth of O^T per wave (128 fp32 per
// lane) leaves one wave per SIMD and forces the accumulators through the AGPR
// file.  A block of BC keys is split over the eight waves two ways:
//   S^T = K q^T    wave w forms the scores of 32-key unit us and 16-head tiles
//                  st0 .. st0 + SNT - 1 of the block (q^T in registers), and
//                  publishes each (unit, head) maximum in LDS;
//   decisions      every wave reads the block maxima of all 64 heads and runs
//                  the same prefix max, so the V copy (issued only when some
//                  head keeps the block) and the rescale branch are uniform;
//   P              the wave's exponentials go to LDS in the MFMA B-operand
//                  layout (bf16, 16-byte chunks XOR-swizzled by head);
//   O^T += V^T P^T wave w owns d rows 16 w .. 16 w + 15 of O^T for every head,
//                  over all of the block's units (V^T read back transposed).
// So each lane holds 16 O^T values, and two waves share each SIMD.
// Software pipeline: step jj forms S and the decisions of block jj and issues
// K(jj + 2), forms P of block jj, then forms O for block jj - 1 while issuing
// V(jj) between its MFMAs (a V copy can only start once its block is decided);
// the next step waits for V(jj) before its second barrier.  K runs two blocks
// ahead through a two-slot ring, V through two slots, and P of block jj waits
// in registers until step jj + 1, when every wave is done with P of block jj - 1.  A rescale from block jj's decisions is applied to O only
// after O has taken block jj - 1 (whose P used the previous reference).
template <int BC>
__global__ __launch_bounds__(512) void decode_wide_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int W = 8;                   // waves; wave w forms O^T rows 16 w .. 16 w + 15
    constexpr int KG = BC / 32;            // 32-key units per block
    constexpr int NT = 4;                  // 16-head tiles (64 heads)
    constexpr int SNT = NT * KG / W;       // S head tiles per wave
    constexpr int DS = D / 32;             // MFMA k-steps over d for S
    constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
    constexpr int ROWB = 2 * D;            // bytes per K/V row
    constexpr int TILE = BC * ROWB;        // bytes of a K or V block
    constexpr int CPW = TILE / (1024 * W); // 1 KiB copies per wave per block
    static_assert(SNT >= 1 && (NT * KG) % W == 0 && TILE % (1024 * W) == 0, "work must split evenly");
    static_assert(W * 16 == D, "one 16-row O^T tile per wave");

    __shared__ __attribute__((aligned(16))) char lds_k[2][TILE];
    __shared__ __attribute__((aligned(16))) char lds_v[2][TILE];
    __shared__ __attribute__((aligned(16))) char lds_p[KG * 64 * 64];  // [unit][head][32 keys] bf16
    __shared__ float lds_pmax[KG][64];
    // decision bytes of up to 32 blocks, written to HBM a chunk at a time with consecutive lanes
    // on consecutive bytes of a head's row (one byte store per decision would cost a memory
    // transaction each)
    constexpr int MCH = 32;
    __shared__ uint8_t lds_mask[MCH][64];
    __shared__ uint8_t lds_vmask[MCH];
    float(*lds_l)[64] = (float(*)[64])lds_p;  // [W][64] after the last step

    const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int G = a.G, N = a.N, nk = a.nk;
    const int j0 = (int)((int64_t)split * nk / a.S);
    const int j1 = (int)((int64_t)(split + 1) * nk / a.S);
    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)N * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)N * D;

    // this wave's S items: unit us of the block, head tiles st0 .. st0 + SNT - 1
    const int us = wave / (NT / SNT);
    const int st0 = (wave % (NT / SNT)) * SNT;
    bool head_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) head_ok[nt] = nt * 16 + n < G;

    // q^T as the S B operand: lane (g, n) holds q[head][32 s + 8 g .. + 8] (zero past G)
    bf16x8 qf[SNT][DS];
#pragma unroll
    for (int i = 0; i < SNT; ++i) {
        const int h = (st0 + i) * 16 + n;
        const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)hkv * G + (h < G ? h : 0)) * D;
#pragma unroll
        for (int s = 0; s < DS; ++s)
            qf[i][s] = as_bf16x8(h < G ? load16(qrow + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u});
    }

    // m_run: each head's running max (log2 units); mref: the max P and (O, l) are
    // taken against, trailing m_run by at most LAZY_LAG (as in decode_split_kernel);
    // l_own: the row sums of this wave's S items
    f32x4 oacc[NT];
    float m_run[NT], mref[NT], l_own[SNT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[nt] = kNegInf;
        mref[nt] = kNegInf;
    }
#pragma unroll
    for (int i = 0; i < SNT; ++i) l_own[i] = 0.f;

    // block j of K or V -> a tile: copy f of this wave moves 16 bytes per lane (a
    // fixed byte offset inside the block, chunk x of tile row r landing at
    // x ^ chunk_swizzle(r), the prefill tiles' map: free of bank conflicts for the
    // K row reads (16 rows x one chunk per 16 lanes) and the transposed V reads
    // (4 rows x two chunks per 16 lanes)) from a wave-uniform block base in SGPRs;
    // only a last block running past the context re-reads key N - 1 in place of
    // the missing rows (their scores are masked)
    uint32_t toff[CPW];
#pragma unroll
    for (int f = 0; f < CPW; ++f) toff[f] = tile_copy_offset<CPR>(wave, CPW, f, lane);
    auto issue = [&](const uint16_t* base, char* tile, int j) {
        const uint16_t* tbase = base + (size_t)j * BC * D;
        if (__builtin_expect(tile_is_ragged<BC>(j, N), 0)) {
#pragma unroll
            for (int f = 0; f < CPW; ++f)
                global_to_lds16_sbase<true>(tbase, tile_copy_clamp<CPR, BC>(toff[f], j, N),
                                      lds_addr(tile + (wave * CPW + f) * 1024));
        } else {
#pragma unroll
            for (int f = 0; f < CPW; ++f)
                global_to_lds16_sbase<true>(tbase, toff[f], lds_addr(tile + (wave * CPW + f) * 1024));
        }
    };
    if (j0 < j1) issue(kbase, lds_k[0], j0);
    if (j0 + 1 < j1) issue(kbase, lds_k[1], j0 + 1);
    wait_vm<CPW>(j0 + 1 < j1 ? 1 : 0);  // this wave's K(j0) copies
    __syncthreads();

    u32x4 pr[SNT];             // P of the block formed last step, for the LDS
    bool vkeep_prev = false;   // the block formed last step is kept by some head
    for (int jj = j0; jj <= j1; ++jj) {
        const bool front = jj < j1;  // block jj: S, decisions, P, V copy
        const int x = (jj - j0) & 1;  // ring slot of block jj
        float t[SNT][2][4];           // raw scores of keys 16 kt + 4 g + e of unit us, head (st0 + i) * 16 + n
        if (front) {
            // ---- S^T = K q^T: A = K rows 16 kt + n of unit us (chunk 4 s + g), B = q^T
            const char* kt_base = lds_k[x] + us * 32 * ROWB;
            u32x4 kf[2][DS];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int s = 0; s < DS; ++s) {
                    const int r = 16 * kt + n, c = 4 * s + g;
                    kf[kt][s] = *(const u32x4*)(kt_base + r * ROWB + ((c ^ chunk_swizzle<CPR>(r)) << 4));
                }
            const bool tail = tile_is_ragged<BC>(jj, N);  // keys past the context are masked
#pragma unroll
            for (int i = 0; i < SNT; ++i) {
                float pm = kNegInf;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < DS; ++s) acc = mfma16x16x32(as_bf16x8(kf[kt][s]), qf[i][s], acc);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float v = acc[e];
                        if (tail) v = jj * BC + 32 * us + 16 * kt + 4 * g + e < N ? v : kNegInf;
                        t[i][kt][e] = v;
                        pm = fmaxf(pm, v);
                    }
                }
                // over the four lane groups g; published in log2 units (the scale is positive)
                pm = wave_max_xor32(wave_max_xor16(pm)) * a.score_scale;
                if (g == 0) lds_pmax[us][(st0 + i) * 16 + n] = pm;
            }
        }
        // block maxima published; every wave is done with K(jj)'s slot, with V(jj - 2)'s
        // slot and with P of block jj - 2
        __syncthreads();

        if (vkeep_prev) {  // P of block jj - 1 (lane (g, n): chunk g of head n's row)
#pragma unroll
            for (int i = 0; i < SNT; ++i) {
                const int h = (st0 + i) * 16 + n;
                *(u32x4*)(lds_p + (us * 64 + h) * 64 + ((g ^ ((h >> 2) & 3)) << 4)) = pr[i];
            }
        }
        bool vkeep = false, lag = false;
        float alpha[NT];
        if (front) {
            // ---- decisions for all 64 heads (every wave the same): Eq. 5 on the block max
            uint32_t keepm = 0;  // bit nt: head nt * 16 + n keeps block jj
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float bm = kNegInf;
#pragma unroll
                for (int u = 0; u < KG; ++u) bm = fmaxf(bm, lds_pmax[u][nt * 16 + n]);
                const float mn = fmaxf(m_run[nt], bm);
                keepm |= (uint32_t)(head_ok[nt] && !((bm - mn) < a.thr)) << nt;
                m_run[nt] = head_ok[nt] ? mn : m_run[nt];
                lag |= !(m_run[nt] == mref[nt] || m_run[nt] - mref[nt] <= LAZY_LAG);
            }
            vkeep = __any(keepm != 0u);
            lag = __any(lag);  // the same in every wave: the same lanes hold the same maxima
            // K(jj + 2) into the slot K(jj) used (V(jj) follows, between the P V MFMAs)
            if (jj + 2 < j1) issue(kbase, lds_k[x], jj + 2);
            if (wave == 0 && g == 0) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) lds_mask[(jj - j0) % MCH][nt * 16 + n] = (uint8_t)(((keepm >> nt) & 1u) ^ 1u);
                if (n == 0) lds_vmask[(jj - j0) % MCH] = (uint8_t)!vkeep;
            }
            // ---- lazy rescale: l now, O after it has taken block jj - 1
            if (lag) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    alpha[nt] = m_run[nt] == mref[nt] ? 1.f : exp2_fast(mref[nt] - m_run[nt]);
                    mref[nt] = m_run[nt];
                }
#pragma unroll
                for (int i = 0; i < SNT; ++i) {
                    float al = alpha[0];
#pragma unroll
                    for (int nt = 1; nt < NT; ++nt) al = st0 + i == nt ? alpha[nt] : al;
                    l_own[i] *= al;
                }
            }
            // ---- P of this wave's S items (held in registers until next step)
            if (vkeep) {
#pragma unroll
                for (int i = 0; i < SNT; ++i) {
                    const int nts = st0 + i;
                    float mr = mref[0];
#pragma unroll
                    for (int nt = 1; nt < NT; ++nt) mr = nts == nt ? mref[nt] : mr;
                    const bool kp = (keepm >> nts) & 1u;
                    const float sc = a.score_scale;
                    float p[8];
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            p[4 * kt + e] = kp ? exp2_fast(__builtin_fmaf(t[i][kt][e], sc, -mr)) : 0.f;
                    l_own[i] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                    pr[i] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                  pack_bf16x2(p[6], p[7])};
                }
            }
        }
        // V(jj - 1), issued during last step's P V, and K(jj + 1) have landed; only K(jj + 2),
        // issued this step, may be in flight
        wait_vm<CPW>(front && jj + 2 < j1 ? 1 : 0);
        __syncthreads();  // P and V of block jj - 1 and K(jj + 1) visible to every wave

        // ---- a full chunk of decision bytes (or the split's last) to HBM; the chunk's bytes are
        //      rewritten only after the next step's first barrier, when every wave has read them
        if (front && ((jj - j0) % MCH == MCH - 1 || jj == j1 - 1)) {
            const int base = jj - (jj - j0) % MCH, cnt = (jj - j0) % MCH + 1;
            if (a.skip != nullptr) {
                for (int t = threadIdx.x; t < G * MCH; t += 64 * W) {
                    const int h = t / MCH, c = t % MCH;
                    if (c < cnt) a.skip[((size_t)b * a.Hq + (size_t)hkv * G + h) * nk + base + c] = lds_mask[c][h];
                }
            }
            if (a.vskip != nullptr && (int)threadIdx.x < cnt)
                a.vskip[((size_t)b * a.Hkv + hkv) * nk + base + threadIdx.x] = lds_vmask[threadIdx.x];
        }

        // ---- O^T rows 16 wave .. + 15 += V^T P^T over block jj - 1's units, with V(jj) (kept
        //      blocks only; into the slot V(jj - 2) used, free since the step's first barrier)
        //      issued between the MFMAs.  Issued with the decisions, V's pieces stalled each
        //      wave on the CU's address unit inside the barrier-to-barrier section every wave
        //      waits for: decode_mqa_16k ran 7% slower.
        const bool cpv = front && vkeep;
        auto copy_piece = [&](int f) {  // piece f of V(jj)
            if (!cpv) return;
            const uint16_t* tbase = vbase + (size_t)jj * BC * D;
            const uint32_t off = tile_is_ragged<BC>(jj, N) ? tile_copy_clamp<CPR, BC>(toff[f], jj, N) : toff[f];
            global_to_lds16_sbase<true>(tbase, off, lds_addr(lds_v[x] + (wave * CPW + f) * 1024));
        };
        if (!vkeep_prev) {
#pragma unroll
            for (int f = 0; f < CPW; ++f) copy_piece(f);
        }
        if (vkeep_prev) {
            const char* vt = lds_v[x ^ 1];
#pragma unroll
            for (int u = 0; u < KG; ++u) {
                const char* vs = vt + u * 32 * ROWB;
                const int cc = 2 * wave + ((n & 3) >> 1);
                const int r0 = 4 * g + (n >> 2), r1 = 16 + 4 * g + (n >> 2);
                const int sw = chunk_swizzle<CPR>(r0) << 4;  // rows r0 and r0 + 16 share it
                const u32x2 lo = lds_read_tr16((const lds_char*)(vs + r0 * ROWB + ((cc << 4) ^ sw) + (n & 1) * 8));
                const u32x2 hi = lds_read_tr16((const lds_char*)(vs + r1 * ROWB + ((cc << 4) ^ sw) + (n & 1) * 8));
                const bf16x8 av = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int h = nt * 16 + n;
                    const u32x4 pf = *(const u32x4*)(lds_p + (u * 64 + h) * 64 + ((g ^ ((h >> 2) & 3)) << 4));
                    oacc[nt] = mfma16x16x32(av, as_bf16x8(pf), oacc[nt]);
                    // CPW pieces over the KG * NT MFMAs
                    constexpr int NM = KG * NT, NQ = CPW;
                    const int mi = u * NT + nt;
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
                        if ((q * NM) / NQ == mi) copy_piece(q);
                }
            }
        }
        if (lag) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) oacc[nt] *= alpha[nt];
        }
        vkeep_prev = vkeep;
    }

    // ---- l per head: the waves' sums over their S items' keys; O / l and the LSE
    __syncthreads();  // every wave is done with P of the last block (lds_l shares its bytes)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float ls = 0.f;  // head tiles outside this wave's S items hold 0
#pragma unroll
        for (int i = 0; i < SNT; ++i) ls = st0 + i == nt ? l_own[i] : ls;
        ls = wave_sum_xor32(wave_sum_xor16(ls));
        if (g == 0) lds_l[wave][nt * 16 + n] = ls;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float lt = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) lt += lds_l[w][nt * 16 + n];
        const int h = nt * 16 + n;
        if (h < G) {
            const size_t orow = ((size_t)b * a.Hq + (size_t)hkv * G + h) * a.S + split;
            const float inv = lt > 0.f ? 1.f / lt : 0.f;  // 0: a split with no block
            *(f32x4*)(a.o_part + orow * D + 16 * wave + 4 * g) = oacc[nt] * inv;
            if (wave == 0 && g == 0) a.lse_part[orow] = mref[nt] * kLn2 + logf(lt);
        }
    }
}

// s_waitcnt vmcnt(F * n) for a wave-uniform n in 0..7
template <int F>
__device__ __forceinline__ void wait_vm8(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(F) : "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * F) : "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * F) : "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * F) : "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * F) : "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * F) : "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(7 * F) : "memory"); break;
    }
}

// Dense split-KV decode (FlashDecoding): the reference every skip is measured
// against.  No decision, so nothing ties the waves together until the end: K
// and V of each 32-key unit are copied HBM -> LDS together, one after the
// other, through NSLOT (K, V) slot pairs per wave (a pair is read into
// registers as soon as it lands and refilled at once), and each wave runs its
// own online softmax (Eqs. 1-4 of the BLASST blog's section on FlashAttention,
// with no Eq. 5) over its units w, w + W, w + 2W, ... of the split.  The waves'
// (m, l, O) are merged by their maxima at the end.  DSPLIT = 2: two workgroups
// per split, 8 apart in a 1-D grid (one XCD), both forming S from all of K and
// each O for half of the d columns from half of every V row -- the layout of
// decode_split_kernel's pairs.  The copies, swizzles and MFMA layouts are those
// of decode_split_kernel: S^T = K q^T on MFMA 16x16x32 (keys x heads), then
// O^T += V^T P^T with V^T read back transposed (ds_read_b64_tr_b16).  Up to 32
// heads per kv group (NT <= 2).
template <int D, int BC, int NT, int W, int NSLOT, int DSPLIT>
__global__ __launch_bounds__(64 * W) void decode_dense_kernel(DecodeArgs a) {
    constexpr int DS = D / 32;            // MFMA k-steps over d for S
    constexpr int FR = D / 16;            // 16-byte copies per lane per 32-row K slice
    constexpr int CPR = D / 8;            // 16-byte chunks per K row
    constexpr int DV = D / DSPLIT;        // V columns this workgroup forms O for
    constexpr int DTV = DV / 16;          // 16-wide d tiles of O^T
    constexpr int FRV = DV / 16;          // 16-byte copies per lane per 32-row V slice
    constexpr int CPRV = DV / 8;          // 16-byte chunks per staged V row
    constexpr int HT = 16 * NT;           // head columns per workgroup
    constexpr int KSLOT = 32 * D * 2;     // bytes of one 32-row K slice
    constexpr int VSLOT = 32 * DV * 2;    // bytes of one 32-row V slice (half rows with DSPLIT = 2)
    constexpr int PAIR = KSLOT + VSLOT;
    static_assert(NT == 1 || NT == 2, "up to 32 heads");
    static_assert(DSPLIT == 1 || DSPLIT == 2, "one or two workgroups per split");
    static_assert(W * DTV * 4 * 64 * 4 <= NSLOT * W * PAIR, "O reduction must fit the staging area");
    static_assert((FR + FRV) * (NSLOT - 1) <= 63, "wait counts fit vmcnt");

    __shared__ __attribute__((aligned(16))) char lds_kv[NSLOT * W * PAIR];
    __shared__ float lds_m[W][HT];
    __shared__ float lds_l[W][64];

    int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z, half = 0;
    if constexpr (DSPLIT == 2) {
        // workgroups L and L + 8 form a unit's two halves (workgroups go round-robin over 8 XCDs)
        const int L = blockIdx.x;
        const int unit = (L / 16) * 8 + (L % 8);
        half = (L / 8) % 2;
        if (unit >= a.S * a.Hkv * a.B) return;
        split = unit % a.S;
        hkv = (unit / a.S) % a.Hkv;
        b = unit / (a.S * a.Hkv);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int G = a.G, N = a.N;
    const int j0 = (int)((int64_t)split * a.nk / a.S);
    const int j1 = (int)((int64_t)(split + 1) * a.nk / a.S);
    // 32-key units of the split that hold at least one key; this wave's share
    const int nunits = max(0, min((j1 - j0) * (BC / 32), (N - j0 * BC + 31) / 32));
    const int nu = nunits > wave ? (nunits - wave + W - 1) / W : 0;
    const int key_base = j0 * BC;

    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)N * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)N * D + half * DV;

    // q^T as the B operand: lane (g, n) holds q[head n][32s + 8g .. +8]
    bf16x8 qf[NT][DS];
    bool head_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int h = nt * 16 + n;
        head_ok[nt] = h < G;
        const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)hkv * G + (head_ok[nt] ? h : 0)) * D;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qf[nt][s] = as_bf16x8(head_ok[nt] ? load16(qrow + 32 * s + 8 * g) : z);
        }
    }

    // unit u of this wave: keys key_base + 32 (wave + W u) ..; slot pair u % NSLOT
    auto pair_of = [&](int u) { return lds_kv + (NSLOT * wave + u % NSLOT) * PAIR; };
    // V non-temporal as in the split kernel; K on the default cache policy, with
    // which this kernel ran 4% faster (the split kernel, unlike this one, runs
    // faster with K non-temporal)
    auto issue = [&](int u) {
        const int key0 = key_base + 32 * (wave + W * u);
        const char* slot = pair_of(u);
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            const int p = 64 * f + lane;
            const int row = p / CPR, cc = (p % CPR) ^ (row & (CPR - 1));
            const int key = min(key0 + row, N - 1);
            global_to_lds16(kbase + (size_t)key * D + cc * 8, lds_addr(slot + 1024 * f));
        }
#pragma unroll
        for (int f = 0; f < FRV; ++f) {
            const int p = 64 * f + lane;
            const int row = p / CPRV, cc = (p % CPRV) ^ (row & (CPRV - 1));
            const int key = min(key0 + row, N - 1);
            global_to_lds16<true>(vbase + (size_t)key * D + cc * 8, lds_addr(slot + KSLOT + 1024 * f));
        }
    };
    for (int u = 0; u < min(NSLOT, nu); ++u) issue(u);

    f32x4 oacc[NT][DTV];
    float m_w[NT], l_part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_w[nt] = kNegInf;
        l_part[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DTV; ++dt) oacc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int u = 0; u < nu; ++u) {
        const int later = min(NSLOT - 1, nu - 1 - u);  // units issued after this one
        const int key0 = key_base + 32 * (wave + W * u);
        // K(u) and V(u) have landed once only the later units' copies are outstanding;
        // both slices are read into registers at once, so the slot pair is refilled
        // before any arithmetic on this unit
        wait_vm8<FR + FRV>(later);
        const char* kslot = pair_of(u);
        const lds_char* vslot = (const lds_char*)(kslot + KSLOT);
        u32x4 kf[2][DS];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const int r = 16 * kt + n, c = 4 * s + g;
                kf[kt][s] = *(const u32x4*)(kslot + r * (2 * D) + ((c ^ (r & (CPR - 1))) << 4));
            }
        bf16x8 vf[DTV];
#pragma unroll
        for (int dt = 0; dt < DTV; ++dt) {
            const int cc = 2 * dt + ((n & 3) >> 1);
            const int r0 = 4 * g + (n >> 2), r1 = 16 + 4 * g + (n >> 2);
            const u32x2 lo = lds_read_tr16(vslot + r0 * (2 * DV) + ((cc ^ (r0 & (CPRV - 1))) << 4) + (n & 1) * 8);
            const u32x2 hi = lds_read_tr16(vslot + r1 * (2 * DV) + ((cc ^ (r1 & (CPRV - 1))) << 4) + (n & 1) * 8);
            vf[dt] = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot pair has been read
        if (u + NSLOT < nu) issue(u + NSLOT);

        bf16x8 pf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 t[2];
            float um = kNegInf;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < DS; ++s) acc = mfma16x16x32(as_bf16x8(kf[kt][s]), qf[nt][s], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key0 + 16 * kt + 4 * g + i;
                    float x = acc[i] * a.score_scale;
                    x = key < N ? x : kNegInf;
                    acc[i] = x;
                    um = fmaxf(um, x);
                }
                t[kt] = acc;
            }
            um = wave_max_xor32(wave_max_xor16(um));  // over the unit's 32 keys (every unit holds one)
            const float m_new = fmaxf(m_w[nt], um);
            const float alpha = exp2_fast(m_w[nt] - m_new);  // 0 on the first unit
            m_w[nt] = m_new;
            if (!__all(alpha == 1.f)) {
                l_part[nt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DTV; ++dt) oacc[nt][dt] *= alpha;
            }
            float p[8];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[4 * kt + i] = exp2_fast(t[kt][i] - m_new);
            l_part[nt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            pf[nt] = as_bf16x8(u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
        }
#pragma unroll
        for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) oacc[nt][dt] = mfma16x16x32(vf[dt], pf[nt], oacc[nt][dt]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- merge the waves' (m, l, O) by their maxima; write the split's result
    __syncthreads();
    float* red = (float*)lds_kv;  // [W waves][DTV][4][64]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (g == 0) lds_m[wave][nt * 16 + n] = m_w[nt];
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, lds_m[w][nt * 16 + n]);
        // a wave with no unit has m = -inf and weight 0; a split with no key has M = -inf
        const float sc = M == kNegInf ? 0.f : exp2_fast(m_w[nt] - M);
        const float l = wave_sum_xor32(wave_sum_xor16(l_part[nt])) * sc;
#pragma unroll
        for (int dt = 0; dt < DTV; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[((wave * DTV + dt) * 4 + i) * 64 + lane] = oacc[nt][dt][i] * sc;
        lds_l[wave][lane] = l;
        __syncthreads();
        float lt = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) lt += lds_l[w][lane];
        const int h = nt * 16 + n;
        if (h < G) {
            const size_t orow = ((size_t)b * a.Hq + (size_t)hkv * G + h) * a.S + split;
            const float inv = lt > 0.f ? 1.f / lt : 0.f;  // 0: a split with no key
            for (int dt = wave; dt < DTV; dt += W) {
                float o4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = 0.f;
#pragma unroll
                    for (int w = 0; w < W; ++w) x += red[((w * DTV + dt) * 4 + i) * 64 + lane];
                    o4[i] = x * inv;
                }
                *(f32x4*)(a.o_part + orow * D + half * DV + 16 * dt + 4 * g) = f32x4{o4[0], o4[1], o4[2], o4[3]};
            }
            if (wave == 0 && g == 0 && half == 0) a.lse_part[orow] = lt > 0.f ? M * kLn2 + logf(lt) : kNegInf;
        }
        __syncthreads();
    }
}

// The split kernel's loads alone: a measurement kernel, not part of any result.
// It issues the HBM -> LDS copies decode_split_kernel issues for two workgroups
// per split at lambda = 0 -- every 32-key K unit of the split by both
// workgroups of the pair, then each workgroup half of every V row -- through
// the same rings (eight waves, two 8 KiB slots each), with no arithmetic and
// no barrier, and with the same cache policies (K non-temporal in the split's
// first phase of 64 units, V non-temporal).  Its time is the floor those bytes
// and that access pattern set for the decode kernel on this part.
template <int D, int BC>
__global__ __launch_bounds__(512) void decode_load_only_kernel(DecodeArgs a) {
    constexpr int W = 8, NSLOT = 2;
    constexpr int FR = D / 16, CPR = D / 8;
    constexpr int DV = D / 2, FRV = DV / 16, CPRV = DV / 8;
    constexpr int SLOT = 32 * D * 2;
    __shared__ __attribute__((aligned(16))) char lds[NSLOT * W * SLOT];
    const int L = blockIdx.x;
    const int unit = (L / 16) * 8 + (L % 8);
    const int half = (L / 8) % 2;
    if (unit >= a.S * a.Hkv * a.B) return;
    const int split = unit % a.S, hkv = (unit / a.S) % a.Hkv, b = unit / (a.S * a.Hkv);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int N = a.N;
    const int j0 = (int)((int64_t)split * a.nk / a.S), j1 = (int)((int64_t)(split + 1) * a.nk / a.S);
    const int key_base = j0 * BC;
    const int nunits = max(0, min((j1 - j0) * (BC / 32), (N - key_base + 31) / 32));
    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)N * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)N * D + half * DV;
    int i = 0;
    for (int U = wave; U < nunits; U += W, ++i) {
        if (i >= NSLOT) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(FR) : "memory");
        const char* slot = lds + (NSLOT * wave + (i % NSLOT)) * SLOT;
#pragma unroll
        for (int f = 0; f < FR; ++f) {
            const int p = 64 * f + lane, row = p / CPR, cc = (p % CPR) ^ (row & (CPR - 1));
            const int key = min(key_base + 32 * U + row, N - 1);
            if (U < 64) global_to_lds16<true>(kbase + (size_t)key * D + cc * 8, lds_addr(slot + 1024 * f));
            else global_to_lds16<false>(kbase + (size_t)key * D + cc * 8, lds_addr(slot + 1024 * f));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    i = 0;
    for (int U = wave; U < nunits; U += W, ++i) {
        if (i >= 2 * NSLOT) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((2 * NSLOT - 1) * FRV) : "memory");
        const char* slot = lds + NSLOT * wave * SLOT + (i % (2 * NSLOT)) * (SLOT / 2);
#pragma unroll
        for (int f = 0; f < FRV; ++f) {
            const int p = 64 * f + lane, row = p / CPRV, cc = (p % CPRV) ^ (row & (CPRV - 1));
            const int key = min(key_base + 32 * U + row, N - 1);
            global_to_lds16<true>(vbase + (size_t)key * D + cc * 8, lds_addr(slot + 1024 * f));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Merge of S split results per (b, head) row.  One workgroup per row, one
// thread per d column.  Up to 32 splits every load is issued at once (one
// memory round trip); beyond that the splits are walked in a loop.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ o_part,
                                                            const float* __restrict__ lse_part,
                                                            float* __restrict__ o, float* __restrict__ lse,
                                                            int S) {
    constexpr int SMAX = 32;
    const size_t row = blockIdx.x;
    const int e = threadIdx.x;
    const float* L = lse_part + row * S;
    const float* op = o_part + row * S * D + e;
    float acc = 0.f, total;
    if (S <= SMAX) {
        float lv[SMAX], xv[SMAX];
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            lv[s] = s < S ? L[s] : kNegInf;
            xv[s] = s < S ? op[(size_t)s * D] : 0.f;
        }
        float top = kNegInf;
#pragma unroll
        for (int s = 0; s < SMAX; ++s) top = fmaxf(top, lv[s]);
        // every split empty (no key at all): O = 0, LSE = -inf
        const float ref = top == kNegInf ? 0.f : top;
        float z = 0.f;
#pragma unroll
        for (int s = 0; s < SMAX; ++s) z += exp2_fast((lv[s] - ref) * kLog2e);
        total = ref + logf(z);
#pragma unroll
        for (int s = 0; s < SMAX; ++s) acc += exp2_fast((lv[s] - total) * kLog2e) * xv[s];
        acc = top == kNegInf ? 0.f : acc;
    } else {
        float top = kNegInf;
        for (int s = 0; s < S; ++s) top = fmaxf(top, L[s]);
        const float ref = top == kNegInf ? 0.f : top;
        float z = 0.f;
        for (int s = 0; s < S; ++s) z += exp2_fast((L[s] - ref) * kLog2e);
        total = ref + logf(z);
        for (int s = 0; s < S; ++s) acc += exp2_fast((L[s] - total) * kLog2e) * op[(size_t)s * D];
        acc = top == kNegInf ? 0.f : acc;
    }
    o[row * D + e] = acc;
    if (e == 0 && lse != nullptr) lse[row] = total;
}

// The same merge with four columns per thread (16-byte loads and stores) and
// 256 / (D / 4) rows per workgroup, for 16-byte aligned partials and outputs.
template <int D>
__global__ __launch_bounds__(256) void decode_combine4_kernel(const float* __restrict__ o_part,
                                                              const float* __restrict__ lse_part,
                                                              float* __restrict__ o, float* __restrict__ lse,
                                                              int S, int rows) {
    constexpr int TPR = D / 4;          // threads per row
    constexpr int RPW = 256 / TPR;      // rows per workgroup
    constexpr int SMAX = 32;
    const int r = blockIdx.x * RPW + (int)threadIdx.x / TPR;
    if (r >= rows) return;
    const size_t row = (size_t)r;
    const int e = threadIdx.x % TPR;
    const float* L = lse_part + row * S;
    const f32x4* op = (const f32x4*)(o_part + row * S * D) + e;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float top = kNegInf, total;
    if (S <= SMAX) {
        float lv[SMAX];
        f32x4 xv[SMAX];
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            lv[s] = s < S ? L[s] : kNegInf;
            xv[s] = s < S ? op[(size_t)s * TPR] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < SMAX; ++s) top = fmaxf(top, lv[s]);
        // every split empty (no key at all): O = 0, LSE = -inf
        const float ref = top == kNegInf ? 0.f : top;
        float z = 0.f;
#pragma unroll
        for (int s = 0; s < SMAX; ++s) z += exp2_fast((lv[s] - ref) * kLog2e);
        total = ref + logf(z);
#pragma unroll
        for (int s = 0; s < SMAX; ++s) acc += exp2_fast((lv[s] - total) * kLog2e) * xv[s];
    } else {
        for (int s = 0; s < S; ++s) top = fmaxf(top, L[s]);
        const float ref = top == kNegInf ? 0.f : top;
        float z = 0.f;
        for (int s = 0; s < S; ++s) z += exp2_fast((L[s] - ref) * kLog2e);
        total = ref + logf(z);
        for (int s = 0; s < S; ++s) acc += exp2_fast((L[s] - total) * kLog2e) * op[(size_t)s * TPR];
    }
    if (top == kNegInf) acc = f32x4{0.f, 0.f, 0.f, 0.f};
    *((f32x4*)(o + row * D) + e) = acc;
    if (e == 0 && lse != nullptr) lse[row] = total;
}

template <int D, int BC, int NT, int UW, int W, int NSLOT, bool MARGINS = false>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid(a.S, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_split_kernel<D, BC, NT, UW, W, NSLOT, MARGINS>), grid, dim3(64 * W), 0, stream, a);
    return hipGetLastError();
}

// Two workgroups per split (each half of the V columns), pairs 8 apart in a 1-D grid.
template <int D, int BC, int NT, int UW, int W, int NSLOT>
hipError_t launch_split_pairs(const DecodeArgs& a, hipStream_t stream) {
    const int64_t units = (int64_t)a.S * a.Hkv * a.B;
    const dim3 grid((unsigned)(2 * ((units + 7) / 8) * 8));
    constexpr int BPP = W * UW / (BC / 32);  // blocks per phase
    if ((a.nk + a.S - 1) / a.S <= BPP)       // every split (of any ragged length too) in one phase
        hipLaunchKernelGGL((decode_split_kernel<D, BC, NT, UW, W, NSLOT, false, 2, 1, true>), grid, dim3(64 * W), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, BC, NT, UW, W, NSLOT, false, 2>), grid, dim3(64 * W), 0, stream, a);
    return hipGetLastError();
}

// Sets n bytes to v.
__global__ __launch_bounds__(256) void fill_u8_kernel(uint8_t* __restrict__ p, size_t n, uint8_t v) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// HS workgroups per split, each HT = 16 NT heads of the group, 8 apart in a 1-D
// grid.  The V skip mask starts as all "not loaded"; the parts clear the bytes
// of the blocks they load.
// The margin pass with head parts: each group's max of D over its heads, per
// block, from the per-head margins the parts wrote (rows (b, hkv) * G + h).
__global__ __launch_bounds__(256) void group_margin_kernel(const float* __restrict__ margin,
                                                           float* __restrict__ vmargin, int G, int nk, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const size_t bh = i / nk, j = i % nk;
    const float* m = margin + bh * G * nk + j;
    float v = kNegInf;
    for (int h = 0; h < G; ++h) v = fmaxf(v, m[(size_t)h * nk]);
    vmargin[i] = v;
}

template <int D, int BC, int NT, int UW, int W, int NSLOT, int HS, bool MARGINS = false>
hipError_t launch_split_heads(const DecodeArgs& a, hipStream_t stream) {
    if (!MARGINS && a.vskip != nullptr) {
        const size_t n = (size_t)a.B * a.Hkv * a.nk;
        hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.vskip, n,
                           (uint8_t)1);
    }
    const int64_t units = (int64_t)a.S * a.Hkv * a.B;
    if (HS * ((units + 7) / 8) * 8 > INT_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(HS * ((units + 7) / 8) * 8));
    hipLaunchKernelGGL((decode_split_kernel<D, BC, NT, UW, W, NSLOT, MARGINS, 1, HS>), grid, dim3(64 * W), 0, stream, a);
    if (MARGINS && a.vmargin != nullptr) {
        const size_t n = (size_t)a.B * a.Hkv * a.nk;
        hipLaunchKernelGGL(group_margin_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.margin,
                           a.vmargin, a.G, a.nk, n);
    }
    return hipGetLastError();
}

// The margin pass reads K only; the four-wave shape keeps 128 KiB in flight.
template <int D, int BC>
hipError_t launch_margins_nt(const DecodeArgs& a, hipStream_t stream) {
    if (a.G <= 16) return launch_split<D, BC, 1, 16, 4, 4, true>(a, stream);
    if (a.G <= 32) return launch_split<D, BC, 2, 8, 4, 4, true>(a, stream);
    if (a.G <= 64) return launch_split<D, BC, 4, 2, 4, 2, true>(a, stream);
    return launch_split_heads<D, BC, 4, 2, 4, 2, 2, true>(a, stream);
}

template <int BC>
hipError_t launch_wide(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid(a.S, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_wide_kernel<BC>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

template <int D, int BC>
hipError_t launch_split_nt(const DecodeArgs& a, hipStream_t stream) {
    // Up to 16 heads: 128 KiB of copies in flight per workgroup either way.  With
    // few workgroups (one per CU) eight waves x two slots measured faster; with
    // many, one wave per SIMD x four slots (the SIMD's second wave lags otherwise).
    if (a.G <= 16) {
        // at most half a workgroup per CU: two workgroups per split, each the V pass of half the columns
        if ((int64_t)a.S * a.Hkv * a.B <= 128) return launch_split_pairs<D, BC, 1, 8, 8, 2>(a, stream);
        if ((int64_t)a.S * a.Hkv * a.B <= 256) return launch_split<D, BC, 1, 8, 8, 2>(a, stream);
        return launch_split<D, BC, 1, 16, 4, 4>(a, stream);
    }
    if (a.G <= 32) return launch_split<D, BC, 2, 8, 4, 4>(a, stream);
    if constexpr (D == 128) {
        if (a.G <= 64 && a.lens == nullptr) return launch_wide<BC>(a, stream);
    }
    if (a.G <= 64) {
        // few units: pairs, each with four slots per wave (46 -> 37 us at 2 x 64 heads x 32K, 16 splits);
        // many: one workgroup per unit (128 vs 173 us for pairs at 64 x 64 heads x 16K, 8 splits)
        if ((int64_t)a.S * a.Hkv * a.B <= 128) return launch_split_pairs<D, BC, 4, 4, 4, 4>(a, stream);
        return launch_split<D, BC, 4, 2, 4, 2>(a, stream);
    }
    return launch_split_heads<D, BC, 4, 2, 4, 2, 2>(a, stream);
}

}  // namespace

// Scratch of the allocation-free decode step: the split partials (o_part, then
// lse_part) of blasst_decode_step_noalloc, one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress, looked up once
// per device (with that device current) and kept in scratch_ptr.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int d, int Bc, hipStream_t stream) {
    if (d == 128) return Bc == 128 ? launch_split_nt<128, 128>(a, stream) : launch_split_nt<128, 64>(a, stream);
    return Bc == 128 ? launch_split_nt<64, 128>(a, stream) : launch_split_nt<64, 64>(a, stream);
}

namespace {
template <int D, int BC, int NT>
hipError_t launch_dense_shape(const DecodeArgs& a, hipStream_t stream) {
    // eight waves, one (K, V) slot pair each (two at d = 64): 128 KiB in flight per workgroup;
    // at most 128 (b, kv head, split) units: two workgroups per split, each half of V's columns
    constexpr int NSLOT = D == 128 ? 1 : 2;
    const int64_t units = (int64_t)a.S * a.Hkv * a.B;
    if (units <= 128) {
        const dim3 grid((unsigned)(2 * ((units + 7) / 8) * 8));
        hipLaunchKernelGGL((decode_dense_kernel<D, BC, NT, 8, NSLOT, 2>), grid, dim3(512), 0, stream, a);
    } else {
        hipLaunchKernelGGL((decode_dense_kernel<D, BC, NT, 8, NSLOT, 1>), dim3(a.S, a.Hkv, a.B), dim3(512), 0, stream, a);
    }
    return hipGetLastError();
}

template <int D, int BC>
hipError_t launch_dense_nt(const DecodeArgs& a, hipStream_t stream) {
    return a.G <= 16 ? launch_dense_shape<D, BC, 1>(a, stream) : launch_dense_shape<D, BC, 2>(a, stream);
}
}  // namespace

hipError_t launch_decode_dense(const DecodeArgs& a, int d, int Bc, hipStream_t stream) {
    if (a.G > 32 || a.lens != nullptr) return hipErrorInvalidValue;
    if (d == 128) return Bc == 128 ? launch_dense_nt<128, 128>(a, stream) : launch_dense_nt<128, 64>(a, stream);
    return Bc == 128 ? launch_dense_nt<64, 128>(a, stream) : launch_dense_nt<64, 64>(a, stream);
}

hipError_t launch_decode_load_only(const DecodeArgs& a, int d, int Bc, hipStream_t stream) {
    const int64_t units = (int64_t)a.S * a.Hkv * a.B;
    if (units > (int64_t)INT_MAX / 16) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(2 * ((units + 7) / 8) * 8));
    if (d == 128 && Bc == 128) hipLaunchKernelGGL((decode_load_only_kernel<128, 128>), grid, dim3(512), 0, stream, a);
    else if (d == 128) hipLaunchKernelGGL((decode_load_only_kernel<128, 64>), grid, dim3(512), 0, stream, a);
    else if (Bc == 128) hipLaunchKernelGGL((decode_load_only_kernel<64, 128>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((decode_load_only_kernel<64, 64>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_margins(const DecodeArgs& a, int d, int Bc, hipStream_t stream) {
    if (d == 128) return Bc == 128 ? launch_margins_nt<128, 128>(a, stream) : launch_margins_nt<128, 64>(a, stream);
    return Bc == 128 ? launch_margins_nt<64, 128>(a, stream) : launch_margins_nt<64, 64>(a, stream);
}

hipError_t launch_decode_combine(const float* o_part, const float* lse_part, float* o, float* lse, int rows,
                                 int d, int S, hipStream_t stream) {
    if ((((uintptr_t)o_part | (uintptr_t)o) & 15u) == 0) {
        // 16-byte aligned: four columns per thread, several rows per workgroup
        const int rpw = 256 / (d / 4);
        const dim3 grid((unsigned)((rows + rpw - 1) / rpw));
        if (d == 512)
            hipLaunchKernelGGL(decode_combine4_kernel<512>, grid, dim3(256), 0, stream, o_part, lse_part, o, lse, S, rows);
        else if (d == 128)
            hipLaunchKernelGGL(decode_combine4_kernel<128>, grid, dim3(256), 0, stream, o_part, lse_part, o, lse, S, rows);
        else
            hipLaunchKernelGGL(decode_combine4_kernel<64>, grid, dim3(256), 0, stream, o_part, lse_part, o, lse, S, rows);
        return hipGetLastError();
    }
    if (d == 512)
        hipLaunchKernelGGL(decode_combine_kernel<512>, dim3(rows), dim3(512), 0, stream, o_part, lse_part, o, lse, S);
    else if (d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(rows), dim3(128), 0, stream, o_part, lse_part, o, lse, S);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(rows), dim3(64), 0, stream, o_part, lse_part, o, lse, S);
    return hipGetLastError();
}

}  // namespace blasst
