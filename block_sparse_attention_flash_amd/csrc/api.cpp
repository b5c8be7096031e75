// C ABI of libblasst.so (declared in include/blasst.h): host-side argument
// validation, threshold set-up and kernel dispatch.  Nothing here allocates.
#include "blasst.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"

#define BLASST_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr double kLog2e = 1.4426950408889634;

bool supported_dim(int x) { return x == 64 || x == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ln(lambda) in log2 units; lambda = 0 never skips.
float log2_threshold(double lambda) {
    return lambda > 0.0 ? static_cast<float>(std::log(lambda) * kLog2e) : -INFINITY;
}

bool lambda_ok(double lambda) { return lambda >= 0.0 && lambda < 1.0; }  // NaN fails both

blasst_status from_hip(hipError_t e) { return e == hipSuccess ? BLASST_OK : BLASST_ERR_HIP; }

}  // namespace

namespace {

blasst_status prefill_impl(const void* q, const void* k, const void* v, float* o, float* lse, uint8_t* skip_mask,
                           const int32_t* seq_lens, int B, int Hq, int T, int d, int gqa_ratio, int Bc,
                           double lambda, int causal, blasst_stream_t stream, bool dense = false) {
    try {
        if (B < 0 || Hq < 0 || T < 0 || d <= 0 || Bc <= 0 || gqa_ratio < 1) return BLASST_ERR_INVALID_ARG;
        if (Hq % gqa_ratio != 0 || !lambda_ok(lambda) || (causal != 0 && causal != 1))
            return BLASST_ERR_INVALID_ARG;
        if (!supported_dim(d) || !supported_dim(Bc)) return BLASST_ERR_UNSUPPORTED;
        if ((int64_t)B * Hq * T == 0) return BLASST_OK;  // nothing to do; pointers are not read
        if (!q || !k || !v || !o) return BLASST_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return BLASST_ERR_INVALID_ARG;
        const int64_t nq = (T + Bc - 1) / Bc;
        if (nq * B * Hq > INT32_MAX) return BLASST_ERR_UNSUPPORTED;

        blasst::PrefillArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        a.o = o;
        a.lse = lse;
        a.mask = skip_mask;
        a.B = B;
        a.Hq = Hq;
        a.G = gqa_ratio;
        a.Hkv = Hq / gqa_ratio;
        a.T = T;
        a.nq = (int)nq;
        a.nk = (int)nq;
        a.causal = causal;
        a.score_scale = static_cast<float>(kLog2e / std::sqrt((double)d));
        a.thr = log2_threshold(lambda);
        a.lens = seq_lens;
        a.dense = dense;
        return from_hip(blasst::launch_prefill(a, d, Bc, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}

blasst_status decode_impl(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                          uint8_t* skip_mask, uint8_t* vskip_mask, const int32_t* seq_lens, int B, int Hq, int N,
                          int d, int gqa_ratio, int Bc, double lambda, int causal, int num_splits,
                          blasst_stream_t stream, bool dense = false, bool validate_only = false) {
    try {
        if (B < 0 || Hq < 0 || N <= 0 || d <= 0 || Bc <= 0 || gqa_ratio < 1) return BLASST_ERR_INVALID_ARG;
        if (Hq % gqa_ratio != 0 || !lambda_ok(lambda) || (causal != 0 && causal != 1))
            return BLASST_ERR_INVALID_ARG;
        const int64_t nk = ((int64_t)N + Bc - 1) / Bc;
        if (num_splits < 1 || num_splits > nk) return BLASST_ERR_INVALID_ARG;
        if (!supported_dim(d) || !supported_dim(Bc)) return BLASST_ERR_UNSUPPORTED;
        if (gqa_ratio > 128) return BLASST_ERR_UNSUPPORTED;  // at most two 64-head workgroups per split
        if ((int64_t)B * Hq == 0) return BLASST_OK;  // nothing to do; pointers are not read
        if (!q || !k || !v || (!validate_only && (!o_part || !lse_part))) return BLASST_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part)) return BLASST_ERR_INVALID_ARG;
        if (B > 65535 || Hq / gqa_ratio > 65535) return BLASST_ERR_UNSUPPORTED;
        if (validate_only) return BLASST_OK;

        blasst::DecodeArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        a.o_part = o_part;
        a.lse_part = lse_part;
        a.skip = skip_mask;
        a.vskip = vskip_mask;
        a.B = B;
        a.Hq = Hq;
        a.G = gqa_ratio;
        a.Hkv = Hq / gqa_ratio;
        a.N = N;
        a.nk = (int)nk;
        a.S = num_splits;
        a.score_scale = static_cast<float>(kLog2e / std::sqrt((double)d));
        a.thr = log2_threshold(lambda);
        a.lens = seq_lens;
        if (dense && gqa_ratio <= 32 && seq_lens == nullptr)
            return from_hip(blasst::launch_decode_dense(a, d, Bc, reinterpret_cast<hipStream_t>(stream)));
        return from_hip(blasst::launch_decode(a, d, Bc, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}

bool lens_ok(const int32_t* seq_lens) { return seq_lens != nullptr && (reinterpret_cast<uintptr_t>(seq_lens) & 3u) == 0; }

}  // namespace

BLASST_EXPORT blasst_status blasst_prefill(const void* q, const void* k, const void* v, float* o, float* lse,
                                           uint8_t* skip_mask, int B, int Hq, int T, int d, int gqa_ratio,
                                           int Bc, double lambda, int causal, blasst_stream_t stream) {
    return prefill_impl(q, k, v, o, lse, skip_mask, nullptr, B, Hq, T, d, gqa_ratio, Bc, lambda, causal, stream);
}

BLASST_EXPORT blasst_status blasst_prefill_ragged(const void* q, const void* k, const void* v, float* o, float* lse,
                                                  uint8_t* skip_mask, const int32_t* seq_lens, int B, int Hq, int T,
                                                  int d, int gqa_ratio, int Bc, double lambda, int causal,
                                                  blasst_stream_t stream) {
    if ((int64_t)B * Hq * T != 0 && !lens_ok(seq_lens)) return BLASST_ERR_INVALID_ARG;
    return prefill_impl(q, k, v, o, lse, skip_mask, seq_lens, B, Hq, T, d, gqa_ratio, Bc, lambda, causal, stream);
}

BLASST_EXPORT blasst_status blasst_prefill_dense(const void* q, const void* k, const void* v, float* o, float* lse,
                                                 int B, int Hq, int T, int d, int gqa_ratio, int Bc, int causal,
                                                 blasst_stream_t stream) {
    return prefill_impl(q, k, v, o, lse, nullptr, nullptr, B, Hq, T, d, gqa_ratio, Bc, 0.0, causal, stream, true);
}

BLASST_EXPORT blasst_status blasst_decode_dense(const void* q, const void* k, const void* v, float* o_part,
                                                float* lse_part, int B, int Hq, int N, int d, int gqa_ratio, int Bc,
                                                int num_splits, blasst_stream_t stream) {
    // Up to 32 heads per kv group: the single-pass dense kernel (K and V of each unit copied
    // together, no decision).  Wider groups run the skip kernel with the threshold at -inf
    // (the compare never fires) and no decision bytes.
    return decode_impl(q, k, v, o_part, lse_part, nullptr, nullptr, nullptr, B, Hq, N, d, gqa_ratio, Bc, 0.0, 1,
                       num_splits, stream, true);
}

BLASST_EXPORT blasst_status blasst_decode_load_ceiling(const void* k, const void* v, int B, int Hkv, int N, int d,
                                                       int Bc, int num_splits, blasst_stream_t stream) {
    try {
        if (B < 0 || Hkv < 0 || N <= 0 || d <= 0 || Bc <= 0) return BLASST_ERR_INVALID_ARG;
        const int64_t nk = ((int64_t)N + Bc - 1) / Bc;
        if (num_splits < 1 || num_splits > nk) return BLASST_ERR_INVALID_ARG;
        if (!supported_dim(d) || !supported_dim(Bc)) return BLASST_ERR_UNSUPPORTED;
        if ((int64_t)B * Hkv == 0) return BLASST_OK;
        if (!k || !v || !aligned16(k) || !aligned16(v)) return BLASST_ERR_INVALID_ARG;
        blasst::DecodeArgs a{};
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        a.B = B;
        a.Hkv = Hkv;
        a.N = N;
        a.nk = (int)nk;
        a.S = num_splits;
        return from_hip(blasst::launch_decode_load_only(a, d, Bc, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}

BLASST_EXPORT blasst_status blasst_decode(const void* q, const void* k, const void* v, float* o_part,
                                          float* lse_part, uint8_t* skip_mask, uint8_t* vskip_mask, int B,
                                          int Hq, int N, int d, int gqa_ratio, int Bc, double lambda, int causal,
                                          int num_splits, blasst_stream_t stream) {
    return decode_impl(q, k, v, o_part, lse_part, skip_mask, vskip_mask, nullptr, B, Hq, N, d, gqa_ratio, Bc, lambda,
                       causal, num_splits, stream);
}

BLASST_EXPORT blasst_status blasst_decode_ragged(const void* q, const void* k, const void* v, float* o_part,
                                                 float* lse_part, uint8_t* skip_mask, uint8_t* vskip_mask,
                                                 const int32_t* seq_lens, int B, int Hq, int N, int d, int gqa_ratio,
                                                 int Bc, double lambda, int num_splits, blasst_stream_t stream) {
    if ((int64_t)B * Hq != 0 && !lens_ok(seq_lens)) return BLASST_ERR_INVALID_ARG;
    return decode_impl(q, k, v, o_part, lse_part, skip_mask, vskip_mask, seq_lens, B, Hq, N, d, gqa_ratio, Bc,
                       lambda, 1, num_splits, stream);
}

namespace {

// Bytes of the split partials of one decode step: o_part [B,Hq,S,d] then lse_part [B,Hq,S] (fp32).
size_t step_workspace_bytes(int B, int Hq, int d, int num_splits) {
    return (size_t)B * Hq * num_splits * ((size_t)d + 1) * sizeof(float);
}

// blasst_decode into the partials at `ws`, then the merge into o / lse.
blasst_status decode_step_impl(const void* q, const void* k, const void* v, float* o, float* lse, uint8_t* skip_mask,
                               uint8_t* vskip_mask, void* ws, int B, int Hq, int N, int d, int gqa_ratio, int Bc,
                               double lambda, int causal, int num_splits, blasst_stream_t stream) {
    float* o_part = static_cast<float*>(ws);
    float* lse_part = o_part + (size_t)B * Hq * num_splits * d;
    blasst_status st = decode_impl(q, k, v, o_part, lse_part, skip_mask, vskip_mask, nullptr, B, Hq, N, d, gqa_ratio,
                                   Bc, lambda, causal, num_splits, stream);
    if (st != BLASST_OK) return st;
    try {
        return from_hip(blasst::launch_decode_combine(o_part, lse_part, o, lse, B * Hq, d, num_splits,
                                                      reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}

// Arguments of a decode step that blasst_decode does not check: the output and its size.
blasst_status step_args_ok(float* o, int B, int Hq, int d, int num_splits) {
    if (B < 0 || Hq < 0 || d <= 0 || num_splits < 1) return BLASST_ERR_INVALID_ARG;
    if ((int64_t)B * Hq == 0) return BLASST_OK;
    if (!o) return BLASST_ERR_INVALID_ARG;
    if ((int64_t)B * Hq > INT32_MAX) return BLASST_ERR_UNSUPPORTED;
    return BLASST_OK;
}

}  // namespace

BLASST_EXPORT size_t blasst_decode_step_workspace_size(int B, int Hq, int d, int num_splits) {
    if (B < 0 || Hq < 0 || d <= 0 || num_splits < 1) return 0;
    return step_workspace_bytes(B, Hq, d, num_splits);
}

BLASST_EXPORT blasst_status blasst_decode_step(const void* q, const void* k, const void* v, float* o, float* lse,
                                               uint8_t* skip_mask, uint8_t* vskip_mask, void* workspace,
                                               size_t workspace_bytes, int B, int Hq, int N, int d, int gqa_ratio,
                                               int Bc, double lambda, int causal, int num_splits,
                                               blasst_stream_t stream) {
    blasst_status st = step_args_ok(o, B, Hq, d, num_splits);
    if (st == BLASST_OK)
        st = decode_impl(q, k, v, nullptr, nullptr, skip_mask, vskip_mask, nullptr, B, Hq, N, d, gqa_ratio, Bc, lambda,
                         causal, num_splits, stream, false, true);
    if (st != BLASST_OK || (int64_t)B * Hq == 0) return st;
    if (!workspace || !aligned16(workspace) || workspace_bytes < step_workspace_bytes(B, Hq, d, num_splits))
        return BLASST_ERR_INVALID_ARG;
    return decode_step_impl(q, k, v, o, lse, skip_mask, vskip_mask, workspace, B, Hq, N, d, gqa_ratio, Bc, lambda,
                            causal, num_splits, stream);
}

BLASST_EXPORT size_t blasst_decode_step_noalloc_max_bytes(void) { return blasst::kDecodeScratchBytes; }

BLASST_EXPORT blasst_status blasst_decode_step_noalloc(const void* q, const void* k, const void* v, float* o,
                                                       float* lse, uint8_t* skip_mask, uint8_t* vskip_mask, int B,
                                                       int Hq, int N, int d, int gqa_ratio, int Bc, double lambda,
                                                       int causal, int num_splits, blasst_stream_t stream) {
    blasst_status st = step_args_ok(o, B, Hq, d, num_splits);
    if (st == BLASST_OK)
        st = decode_impl(q, k, v, nullptr, nullptr, skip_mask, vskip_mask, nullptr, B, Hq, N, d, gqa_ratio, Bc, lambda,
                         causal, num_splits, stream, false, true);
    if (st != BLASST_OK || (int64_t)B * Hq == 0) return st;
    if (step_workspace_bytes(B, Hq, d, num_splits) > blasst::kDecodeScratchBytes) return BLASST_ERR_UNSUPPORTED;
    void* ws = nullptr;
    try {
        if (blasst::decode_scratch(&ws) != hipSuccess) return BLASST_ERR_HIP;
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
    return decode_step_impl(q, k, v, o, lse, skip_mask, vskip_mask, ws, B, Hq, N, d, gqa_ratio, Bc, lambda, causal,
                            num_splits, stream);
}

BLASST_EXPORT blasst_status blasst_decode_combine(const float* o_part, const float* lse_part, float* o, float* lse,
                                                  int B, int Hq, int d, int num_splits, blasst_stream_t stream) {
    try {
        if (B < 0 || Hq < 0 || d <= 0 || num_splits < 1) return BLASST_ERR_INVALID_ARG;
        if (!supported_dim(d) && d != 512) return BLASST_ERR_UNSUPPORTED;
        const int64_t rows = (int64_t)B * Hq;
        if (rows == 0) return BLASST_OK;  // nothing to do; pointers are not read
        if (!o_part || !lse_part || !o) return BLASST_ERR_INVALID_ARG;
        if (rows > INT32_MAX) return BLASST_ERR_UNSUPPORTED;
        return from_hip(blasst::launch_decode_combine(o_part, lse_part, o, lse, (int)rows, d, num_splits,
                                                      reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}

BLASST_EXPORT blasst_status blasst_prefill_margins(const void* q, const void* k, float* margin, int B, int Hq, int T,
                                                   int d, int gqa_ratio, int Bc, int causal, blasst_stream_t stream) {
    try {
        if (B < 0 || Hq < 0 || T < 0 || d <= 0 || Bc <= 0 || gqa_ratio < 1) return BLASST_ERR_INVALID_ARG;
        if (Hq % gqa_ratio != 0 || (causal != 0 && causal != 1)) return BLASST_ERR_INVALID_ARG;
        if (!supported_dim(d) || !supported_dim(Bc)) return BLASST_ERR_UNSUPPORTED;
        if ((int64_t)B * Hq * T == 0) return BLASST_OK;  // nothing to do; pointers are not read
        if (!q || !k || !margin) return BLASST_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k)) return BLASST_ERR_INVALID_ARG;
        const int64_t nq = (T + Bc - 1) / Bc;
        if (nq * B * Hq > INT32_MAX) return BLASST_ERR_UNSUPPORTED;

        blasst::PrefillArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = nullptr;
        a.o = nullptr;
        a.lse = nullptr;
        a.mask = nullptr;
        a.margin = margin;
        a.B = B;
        a.Hq = Hq;
        a.G = gqa_ratio;
        a.Hkv = Hq / gqa_ratio;
        a.T = T;
        a.nq = (int)nq;
        a.nk = (int)nq;
        a.causal = causal;
        a.score_scale = static_cast<float>(kLog2e / std::sqrt((double)d));
        a.thr = -INFINITY;
        return from_hip(blasst::launch_prefill_margins(a, d, Bc, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}

BLASST_EXPORT blasst_status blasst_decode_margins(const void* q, const void* k, float* margin, float* vmargin, int B,
                                                  int Hq, int N, int d, int gqa_ratio, int Bc, int num_splits,
                                                  blasst_stream_t stream) {
    try {
        if (B < 0 || Hq < 0 || N <= 0 || d <= 0 || Bc <= 0 || gqa_ratio < 1) return BLASST_ERR_INVALID_ARG;
        if (Hq % gqa_ratio != 0) return BLASST_ERR_INVALID_ARG;
        const int64_t nk = ((int64_t)N + Bc - 1) / Bc;
        if (num_splits < 1 || num_splits > nk) return BLASST_ERR_INVALID_ARG;
        if (!supported_dim(d) || !supported_dim(Bc)) return BLASST_ERR_UNSUPPORTED;
        if (gqa_ratio > 128) return BLASST_ERR_UNSUPPORTED;  // at most two 64-head workgroups per split
        if ((int64_t)B * Hq == 0) return BLASST_OK;  // nothing to do; pointers are not read
        if (!q || !k || !margin) return BLASST_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k)) return BLASST_ERR_INVALID_ARG;
        if (B > 65535 || Hq / gqa_ratio > 65535) return BLASST_ERR_UNSUPPORTED;

        blasst::DecodeArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = nullptr;
        a.o_part = nullptr;
        a.lse_part = nullptr;
        a.skip = nullptr;
        a.vskip = nullptr;
        a.margin = margin;
        a.vmargin = vmargin;
        a.B = B;
        a.Hq = Hq;
        a.G = gqa_ratio;
        a.Hkv = Hq / gqa_ratio;
        a.N = N;
        a.nk = (int)nk;
        a.S = num_splits;
        a.score_scale = static_cast<float>(kLog2e / std::sqrt((double)d));
        a.thr = -INFINITY;
        return from_hip(blasst::launch_decode_margins(a, d, Bc, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}

BLASST_EXPORT const char* blasst_status_string(blasst_status status) {
    switch (status) {
        case BLASST_OK: return "ok";
        case BLASST_ERR_INVALID_ARG: return "invalid argument";
        case BLASST_ERR_UNSUPPORTED: return "unsupported configuration";
        case BLASST_ERR_HIP: return "HIP launch or runtime error";
        case BLASST_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

BLASST_EXPORT blasst_status blasst_decode_mla(const void* q, const void* kv, float* o_part, float* lse_part,
                                              uint8_t* skip_mask, int B, int Hq, int N, int d_qk, int d_v, int Bc,
                                              double softmax_scale, double lambda, int num_splits,
                                              blasst_stream_t stream) {
    try {
        if (B < 0 || Hq < 0 || N <= 0 || d_qk <= 0 || d_v <= 0 || d_v > d_qk || Bc <= 0) return BLASST_ERR_INVALID_ARG;
        if (!lambda_ok(lambda) || !(softmax_scale > 0.0) || !std::isfinite(softmax_scale))
            return BLASST_ERR_INVALID_ARG;
        const int64_t nk = ((int64_t)N + Bc - 1) / Bc;
        if (num_splits < 1 || num_splits > nk) return BLASST_ERR_INVALID_ARG;
        if (d_qk != 576 || d_v != 512 || (Bc != 64 && Bc != 32) || Hq % (Bc == 32 ? 64 : 32) != 0)
            return BLASST_ERR_UNSUPPORTED;
        if ((int64_t)B * Hq == 0) return BLASST_OK;  // nothing to do; pointers are not read
        if (!q || !kv || !o_part || !lse_part) return BLASST_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(kv) || !aligned16(o_part)) return BLASST_ERR_INVALID_ARG;
        if (B > 65535 || (int64_t)N * 576 * B > ((int64_t)1 << 40)) return BLASST_ERR_UNSUPPORTED;

        blasst::MlaArgs a;
        a.q = static_cast<const uint16_t*>(q);
        a.kv = static_cast<const uint16_t*>(kv);
        a.o_part = o_part;
        a.lse_part = lse_part;
        a.skip = skip_mask;
        a.B = B;
        a.Hq = Hq;
        a.N = N;
        a.nk = (int)nk;
        a.S = num_splits;
        a.score_scale = static_cast<float>(softmax_scale * kLog2e);
        a.thr = log2_threshold(lambda);
        return from_hip(blasst::launch_decode_mla(a, Bc, reinterpret_cast<hipStream_t>(stream)));
    } catch (...) {
        return BLASST_ERR_INTERNAL;
    }
}
