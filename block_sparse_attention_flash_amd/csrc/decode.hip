// Split-KV decode with the skip-softmax rule, and the log-sum-exp merge of splits.
//
// BLASST blog, section on the decode kernel: decode is bound by reading the KV
// cache, so what a skip must save there is the V load.  The decision needs the
// block max, which needs S = q K^T; deciding block by block would serialise
// "decide -> load V".  The blog's answer is batched load scheduling: form the
// S blocks of a batch first, decide them together, then issue V loads only for
// kept blocks.  That is the structure here.
//
// Work decomposition (one workgroup = 4 waves per (batch b, kv head, split)):
//  * The split's KV blocks are walked in batches.  Every block is cut into
//    32-key units; a wave owns NB units per batch.  For Bc = 128 wave w takes
//    keys [32w, 32w+32) of each of NB consecutive blocks.
//  * S^T = K q^T for a unit runs on MFMA 16x16x32 bf16 with the 32 keys as two
//    16-row tiles and the G query heads of the group as the 16-wide column
//    tiles (NT tiles of 16; heads beyond G are zero columns that never vote).
//    K fragments are loaded straight from HBM into the MFMA A-operand layout
//    (16 bytes per lane, each row of 16 lanes a contiguous 64-byte run).
//  * Each unit's per-head partial max goes through LDS; after one barrier every
//    lane knows the block maxima of the whole batch.  Because a skipped block
//    never moves the running max (mt < m + ln(lambda) < m), the running max
//    before block j is the prefix max of the block maxima, so all decisions of
//    the batch are taken at once, in block order, with no cascade.
//  * V rows are loaded only for blocks some head of the group keeps, staged
//    through a wave-private LDS slot and read back transposed
//    (ds_read_b64_tr_b16) as the A operand of O^T += V^T P^T.  P^T comes
//    straight from the S^T accumulators (same lane layout), rounded to bf16.
//  * Scores are kept in log2 units (t = s * log2(e)), so P = 2^(t - m) uses
//    v_exp_f32 directly and the test reads t~ - m < ln(lambda) * log2(e).
#include "device_common.h"
#include "kernels.h"

namespace blasst {

namespace {

constexpr int kDecodeThreads = 256;  // 4 waves

template <int D, int BC, int NT, int NB>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(DecodeArgs a) {
    constexpr int KG = BC / 32;           // 32-key units per block
    constexpr int NBB = 4 * NB / KG;      // blocks per batch
    constexpr int DS = D / 32;            // MFMA k-steps over d for S
    constexpr int DT = D / 16;            // 16-wide d tiles of O^T
    constexpr int FR = D / 16;            // 16-byte fragments per lane per unit
    constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
    constexpr int HT = 16 * NT;           // head columns per workgroup
    constexpr int VSLOT = 32 * D * 2;     // bytes of one staged 32-row V slice
    static_assert(NBB * KG == 4 * NB, "units must tile the batch");
    static_assert(4 * DT * 4 * 64 * 4 <= 4 * VSLOT, "O reduction must fit the V staging area");

    __shared__ __attribute__((aligned(16))) char lds_v[4 * VSLOT];
    __shared__ float lds_pmax[2][NBB * KG * HT];
    __shared__ float lds_l[4][64];

    const int split = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int N = a.N, nk = a.nk, G = a.G;
    const int j0 = (int)((int64_t)split * nk / a.S);
    const int j1 = (int)((int64_t)(split + 1) * nk / a.S);

    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)N * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)N * D;
    lds_char* vslot = (lds_char*)(lds_v + wave * VSLOT);

    // q^T as the B operand: lane (g, n) holds q[head n][32s + 8g .. +8].
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

    f32x4 oacc[NT][DT];
    float m_run[NT], l_part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m_run[nt] = kNegInf;
        l_part[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int parity = 0;
    for (int jb0 = j0; jb0 < j1; jb0 += NBB, parity ^= 1) {
        // ---- units of this wave in the batch
        int ublk[NB], ukey0[NB];
        bool uok[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int U = wave + 4 * u;
            ublk[u] = jb0 + U / KG;
            ukey0[u] = ublk[u] * BC + (U % KG) * 32;
            uok[u] = ublk[u] < j1;
        }

        // ---- K fragments straight into the MFMA A layout
        u32x4 kv[NB][FR];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int key = min(ukey0[u] + 16 * kt + n, N - 1);
#pragma unroll
                for (int s = 0; s < DS; ++s) {
                    if (uok[u]) kv[u][kt * DS + s] = load16(kbase + (size_t)key * D + 32 * s + 8 * g);
                    else kv[u][kt * DS + s] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }

        // ---- S^T = K q^T, scaled to log2 units, tail keys masked; partial maxima
        f32x4 t[NB][2][NT];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                float pm = kNegInf;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < DS; ++s) acc = mfma16x16x32(as_bf16x8(kv[u][kt * DS + s]), qf[nt][s], acc);
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
                pm = fmaxf(pm, wave_shfl_xor(pm, 16));
                pm = fmaxf(pm, wave_shfl_xor(pm, 32));
                if (uok[u] && g == 0) lds_pmax[parity][(wave + 4 * u) * HT + nt * 16 + n] = pm;
            }
        }
        __syncthreads();

        // ---- decisions for the whole batch (prefix max; no cascade)
        const int nblk = min(NBB, j1 - jb0);
        uint32_t keep[NT];
        uint32_t vkeep = 0;
        float alpha[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float m = m_run[nt];
            uint32_t kb = 0;
            for (int bi = 0; bi < nblk; ++bi) {
                float bm = kNegInf;
#pragma unroll
                for (int kg = 0; kg < KG; ++kg) bm = fmaxf(bm, lds_pmax[parity][(bi * KG + kg) * HT + nt * 16 + n]);
                m = fmaxf(m, bm);
                const bool skip = (bm - m) < a.thr;
                kb |= (uint32_t)(!skip) << bi;
            }
            kb = head_ok[nt] ? kb : 0u;
            keep[nt] = kb;
            vkeep |= kb;
            alpha[nt] = head_ok[nt] ? exp2_fast(m_run[nt] - m) : 1.f;
            m_run[nt] = head_ok[nt] ? m : m_run[nt];
        }
        vkeep |= __shfl_xor(vkeep, 1, 64);
        vkeep |= __shfl_xor(vkeep, 2, 64);
        vkeep |= __shfl_xor(vkeep, 4, 64);
        vkeep |= __shfl_xor(vkeep, 8, 64);

        // ---- decision bytes
        if (wave == 0 && g == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (!head_ok[nt] || a.skip == nullptr) continue;
                uint8_t* row = a.skip + ((size_t)b * a.Hq + (size_t)hkv * G + nt * 16 + n) * nk + jb0;
                for (int bi = 0; bi < nblk; ++bi) row[bi] = (uint8_t)(((keep[nt] >> bi) & 1u) ^ 1u);
            }
            if (n == 0 && a.vskip != nullptr) {
                uint8_t* row = a.vskip + ((size_t)b * a.Hkv + hkv) * nk + jb0;
                for (int bi = 0; bi < nblk; ++bi) row[bi] = (uint8_t)(((vkeep >> bi) & 1u) ^ 1u);
            }
        }

        // ---- rescale the running state to the batch's new max
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            l_part[nt] *= alpha[nt];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[nt][dt] *= alpha[nt];
        }

        // ---- V loads, kept blocks only (coalesced rows; reuse the K registers)
        bool uv[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            uv[u] = uok[u] && ((vkeep >> ((wave + 4 * u) / KG)) & 1u);
            if (uv[u]) {
#pragma unroll
                for (int f = 0; f < FR; ++f) {
                    const int c = lane + 64 * f;
                    const int key = min(ukey0[u] + c / CPR, N - 1);
                    kv[u][f] = load16(vbase + (size_t)key * D + (c % CPR) * 8);
                }
            }
        }

        // ---- P V for kept units: stage V through LDS, read it back transposed
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (!uv[u]) continue;
#pragma unroll
            for (int f = 0; f < FR; ++f) {
                const int c = lane + 64 * f;
                const int row = c / CPR, cc = c % CPR;
                *(u32x4*)(lds_v + wave * VSLOT + row * (2 * D) + ((cc ^ (row & (CPR - 1))) << 4)) = kv[u][f];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

            bf16x8 pf[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bool kp = (keep[nt] >> ((wave + 4 * u) / KG)) & 1u;
                float p[8];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = exp2_fast(t[u][kt][nt][i] - m_run[nt]);
                        p[4 * kt + i] = kp ? e : 0.f;
                    }
                float ps = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ps += p[i];
                l_part[nt] += ps;
                u32x4 w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                           pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
                pf[nt] = as_bf16x8(w);
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                u32x2 lo, hi;
                {
                    const int r = 4 * g + (n >> 2), cc = 2 * dt + ((n & 3) >> 1);
                    lo = lds_read_tr16(vslot + r * (2 * D) + ((cc ^ (r & (CPR - 1))) << 4) + (n & 1) * 8);
                }
                {
                    const int r = 16 + 4 * g + (n >> 2), cc = 2 * dt + ((n & 3) >> 1);
                    hi = lds_read_tr16(vslot + r * (2 * D) + ((cc ^ (r & (CPR - 1))) << 4) + (n & 1) * 8);
                }
                const bf16x8 av = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) oacc[nt][dt] = mfma16x16x32(av, pf[nt], oacc[nt][dt]);
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    }

    // ---- reduce the four waves' partial O^T and l; write the split's result
    __syncthreads();
    float* red = (float*)lds_v;  // [4 waves][DT][4][64]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float l = l_part[nt];
        l += wave_shfl_xor(l, 16);
        l += wave_shfl_xor(l, 32);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[((wave * DT + dt) * 4 + i) * 64 + lane] = oacc[nt][dt][i];
        lds_l[wave][lane] = l;
        __syncthreads();
        const float lt = lds_l[0][lane] + lds_l[1][lane] + lds_l[2][lane] + lds_l[3][lane];
        const int h = nt * 16 + n;
        if (h < G) {
            const size_t orow = ((size_t)b * a.Hq + (size_t)hkv * G + h) * a.S + split;
            const float inv = 1.f / lt;
            for (int dt = wave; dt < DT; dt += 4) {
                float o4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = 0.f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) x += red[((w * DT + dt) * 4 + i) * 64 + lane];
                    o4[i] = x * inv;
                }
                *(f32x4*)(a.o_part + orow * D + 16 * dt + 4 * g) = f32x4{o4[0], o4[1], o4[2], o4[3]};
            }
            if (wave == 0 && g == 0) a.lse_part[orow] = m_run[nt] * kLn2 + logf(lt);
        }
        __syncthreads();
    }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ o_part,
                                                            const float* __restrict__ lse_part,
                                                            float* __restrict__ o, float* __restrict__ lse,
                                                            int S) {
    const size_t row = blockIdx.x;
    const int e = threadIdx.x;
    const float* L = lse_part + row * S;
    float top = kNegInf;
    for (int s = 0; s < S; ++s) top = fmaxf(top, L[s]);
    float z = 0.f;
    for (int s = 0; s < S; ++s) z += exp2_fast((L[s] - top) * kLog2e);
    const float total = top + logf(z);
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc += exp2_fast((L[s] - total) * kLog2e) * o_part[(row * S + s) * D + e];
    o[row * D + e] = acc;
    if (e == 0 && lse != nullptr) lse[row] = total;
}

template <int D, int BC, int NT, int NB>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid(a.S, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_split_kernel<D, BC, NT, NB>), grid, dim3(kDecodeThreads), 0, stream, a);
    return hipGetLastError();
}

template <int D, int BC>
hipError_t launch_split_nt(const DecodeArgs& a, hipStream_t stream) {
    if (a.G <= 16) return launch_split<D, BC, 1, 4>(a, stream);
    if (a.G <= 32) return launch_split<D, BC, 2, 2>(a, stream);
    return launch_split<D, BC, 4, 2>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int d, int Bc, hipStream_t stream) {
    if (d == 128) return Bc == 128 ? launch_split_nt<128, 128>(a, stream) : launch_split_nt<128, 64>(a, stream);
    return Bc == 128 ? launch_split_nt<64, 128>(a, stream) : launch_split_nt<64, 64>(a, stream);
}

hipError_t launch_decode_combine(const float* o_part, const float* lse_part, float* o, float* lse, int rows,
                                 int d, int S, hipStream_t stream) {
    if (d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(rows), dim3(128), 0, stream, o_part, lse_part, o, lse, S);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(rows), dim3(64), 0, stream, o_part, lse_part, o, lse, S);
    return hipGetLastError();
}

}  // namespace blasst
