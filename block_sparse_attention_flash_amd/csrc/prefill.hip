// Causal GQA prefill with the skip-softmax rule.
//
// BLASST blog, section on the prefill kernel: prefill is compute bound, so a
// skipped tile saves the exp, the row sum and the P V product; S = Q K^T is
// always formed (its row max is what the test reads) and V tiles are fetched
// unconditionally, which keeps the copy pipeline regular.  The tile is skipped
// only when every one of the query block's Bc rows votes to skip (the AND over
// the query block; section on the lambda = a/L rule and on the decision cost).
//
// Work decomposition: one workgroup per (query block i of Br = Bc rows, query
// head, batch), Bc/32 waves, wave w owning query rows [32w, 32w+32) of the block.
// Workgroups are issued heaviest first (the last query block has the most KV
// tiles under the causal mask), and the query heads of one kv group are laid
// on the same XCD so the group's K/V tiles are shared through that XCD's L2.
//
// Per KV tile (all on MFMA 32x32x16 bf16, fp32 accumulate):
//   S^T = K Q^T      A = K rows from LDS (ds_read_b128), B = Q^T in registers.
//                    In S^T's accumulator layout each lane holds 16 scores of
//                    one query row, so row max, exp and row sum are mostly
//                    in-lane (plus one exchange with lane l^32).
//   vote             per row mt - max(m, mt) < ln(lambda) (log2 units), then an
//                    AND over the wave (ballot) and over the waves (LDS word).
//   O^T += V^T P^T   only for kept tiles.  P^T is the S^T accumulator rounded
//                    to bf16 (no data movement); V^T comes from the V tile in
//                    LDS through ds_read_b64_tr_b16.
// K and V tiles are XOR-swizzled in LDS by 16-byte chunk so both the row reads
// and the transposed reads are bank-conflict free; the next tile's global
// loads are issued before the current tile is computed.
#include "device_common.h"
#include "kernels.h"

namespace blasst {

namespace {

template <int D, int BC>
__global__ __launch_bounds__(2 * BC) void prefill_kernel(PrefillArgs a) {
    constexpr int NW = BC / 32;            // waves; 32 query rows each
    constexpr int NTH = 64 * NW;           // threads
    constexpr int KT = BC / 32;            // 32-key tiles of S^T
    constexpr int DS = D / 16;             // MFMA k-steps over d
    constexpr int DT = D / 32;             // 32-wide d tiles of O^T
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int CH = BC * CPR / NTH;     // chunks per thread per tile
    constexpr int ROWB = 2 * D;            // bytes per K/V row

    __shared__ __attribute__((aligned(16))) char lds_k[BC * ROWB];
    __shared__ __attribute__((aligned(16))) char lds_v[BC * ROWB];
    __shared__ int lds_vote[NW];

    // ---- workgroup -> (query block, head, batch): heaviest query blocks first;
    //      within one query block, heads of a kv group land on one XCD.
    const int bh_count = a.B * a.Hq;
    const int L = blockIdx.x;
    const int i = a.nq - 1 - L / bh_count;
    int bh = L % bh_count;
    if (bh_count % 8 == 0) bh = (bh % 8) * (bh_count / 8) + bh / 8;
    const int hq = bh % a.Hq, b = bh / a.Hq;
    const int hkv = hq / a.G;
    const int T = a.T;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;   // query column of S^T / O^T, and lane half
    const int qidx = i * BC + 32 * wave + col;     // this lane's query row
    const bool row_ok = qidx < T;

    const uint16_t* kbase = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;
    const uint16_t* vbase = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)T * D;

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
    float m = kNegInf, l = 0.f;

    // ---- tile copy: thread chunk c = tid + NTH*f -> row c / CPR, chunk c % CPR
    u32x4 kreg[CH], vreg[CH];
    auto fetch = [&](int j) {
#pragma unroll
        for (int f = 0; f < CH; ++f) {
            const int c = tid + NTH * f;
            const int key = min(j * BC + c / CPR, T - 1);
            kreg[f] = load16(kbase + (size_t)key * D + (c % CPR) * 8);
            vreg[f] = load16(vbase + (size_t)key * D + (c % CPR) * 8);
        }
    };
    auto swz = [](int row, int chunk) { return row * ROWB + ((chunk ^ (row & (CPR - 1))) << 4); };

    uint8_t* mask_row = a.mask ? a.mask + (((size_t)b * a.Hq + hq) * a.nq + i) * a.nk : nullptr;

    fetch(0);
    for (int j = 0; j < jend; ++j) {
        __syncthreads();  // every wave is done with the previous tile
#pragma unroll
        for (int f = 0; f < CH; ++f) {
            const int c = tid + NTH * f;
            *(u32x4*)(lds_k + swz(c / CPR, c % CPR)) = kreg[f];
            *(u32x4*)(lds_v + swz(c / CPR, c % CPR)) = vreg[f];
        }
        if (j + 1 < jend) fetch(j + 1);
        __syncthreads();

        // ---- S^T = K Q^T for this wave's 32 query columns, all BC keys
        f32x16 sacc[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            sacc[kt] = f32x16{};
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const u32x4 kf = *(const u32x4*)(lds_k + swz(32 * kt + col, 2 * s + half));
                sacc[kt] = mfma32x32x16(as_bf16x8(kf), qf[s], sacc[kt]);
            }
        }

        // ---- scale to log2 units, causal / tail mask, row max over the tile
        float mt = kNegInf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int kidx = j * BC + 32 * kt + 8 * (e >> 2) + 4 * half + (e & 3);
                const bool hidden = kidx >= T || (a.causal && kidx > qidx);
                const float x = hidden ? kNegInf : sacc[kt][e] * a.score_scale;
                sacc[kt][e] = x;
                mt = fmaxf(mt, x);
            }
        mt = fmaxf(mt, wave_shfl_xor(mt, 32));

        // ---- Eq. 1 then the log-space test; AND over every row of the query block
        const float m_new = fmaxf(m, mt);
        const bool vote_skip = !row_ok || mt == kNegInf || (mt - m_new) < a.thr;
        const bool wave_skip = __all(vote_skip);
        if (lane == 0) lds_vote[wave] = wave_skip;
        __syncthreads();
        bool skip = true;
#pragma unroll
        for (int w = 0; w < NW; ++w) skip = skip && lds_vote[w];
        if (tid == 0 && mask_row) mask_row[j] = (uint8_t)skip;
        if (skip) continue;

        // ---- kept tile: rescale, P = 2^(t - m), row sum, O^T += V^T P^T
        const float alpha = exp2_fast(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = exp2_fast(sacc[kt][8 * p + e] - m);
                    l += pv[e];
                }
                const bf16x8 pb = as_bf16x8(u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                                  pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});
                // keys of these 8 slots: 32kt + 16p + 4*half + {0..3} and the same + 8
                const int g16 = lane >> 4, jj = lane & 15;
                const int r0 = 32 * kt + 16 * p + 4 * (g16 >> 1) + (jj >> 2);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int chunk = 4 * dt + 2 * (g16 & 1) + ((jj & 3) >> 1);
                    const int byte = (jj & 1) * 8;
                    const u32x2 lo = lds_read_tr16((const lds_char*)(lds_v + swz(r0, chunk) + byte));
                    const u32x2 hi = lds_read_tr16((const lds_char*)(lds_v + swz(r0 + 8, chunk) + byte));
                    oacc[dt] = mfma32x32x16(as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}), pb, oacc[dt]);
                }
            }
        }
    }

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
        if (half == 0 && a.lse) a.lse[((size_t)b * a.Hq + hq) * T + qidx] = m * kLn2 + logf(l);
    }
    if (mask_row)
        for (int j = jend + tid; j < a.nk; j += NTH) mask_row[j] = 2;
}

template <int D, int BC>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.nq * a.B * a.Hq);
    hipLaunchKernelGGL((prefill_kernel<D, BC>), grid, dim3(2 * BC), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int d, int Bc, hipStream_t stream) {
    if (d == 128) return Bc == 128 ? launch<128, 128>(a, stream) : launch<128, 64>(a, stream);
    return Bc == 128 ? launch<64, 128>(a, stream) : launch<64, 64>(a, stream);
}

}  // namespace blasst
