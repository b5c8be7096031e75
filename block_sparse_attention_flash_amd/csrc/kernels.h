// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blasst {

// Split-KV decode launch.  Pointers and sizes already validated by the caller.
struct DecodeArgs {
    const uint16_t* q;  // bf16 [B, Hq, 1, d]
    const uint16_t* k;  // bf16 [B, Hkv, N, d]
    const uint16_t* v;  // bf16 [B, Hkv, N, d]
    float* o_part;      // [B, Hq, S, d]
    float* lse_part;    // [B, Hq, S]
    uint8_t* skip;      // [B, Hq, nk] or null
    uint8_t* vskip;     // [B, Hkv, nk] or null
    int B, Hq, Hkv, G, N, nk, S;
    float score_scale;  // log2(e) / sqrt(d): scores are handled in log2 units
    float thr;          // ln(lambda) * log2(e); -inf when lambda == 0
    float* margin = nullptr;   // margin pass only: [B, Hq, nk]
    float* vmargin = nullptr;  // margin pass only: [B, Hkv, nk] or null
    const int* lens = nullptr;  // ragged batch: [B] context lengths (device), clamped to [0, N]; N, nk = capacity
};

// Causal / full prefill launch.
struct PrefillArgs {
    const uint16_t* q;  // bf16 [B, Hq, T, d]
    const uint16_t* k;  // bf16 [B, Hkv, T, d]
    const uint16_t* v;  // bf16 [B, Hkv, T, d]
    float* o;           // [B, Hq, T, d]
    float* lse;         // [B, Hq, T] or null
    uint8_t* mask;      // [B, Hq, nq, nk] or null
    int B, Hq, Hkv, G, T, nq, nk, causal;
    float score_scale;
    float thr;
    float* margin = nullptr;  // margin pass only: [B, Hq, nq, nk]
    const int* lens = nullptr;  // ragged batch: [B] sequence lengths (device), clamped to [0, T]; T, nq = capacity
    bool dense = false;         // the kernel built without the skip test (every tile kept)
    int xcd_rot = 1 << 30;      // query blocks per turn of the kv-group -> XCD rotation (set at launch)
};

// MLA decode (absorbed latent form): 576-wide cache rows, value = the first 512 columns, Bc in {32, 64}.
struct MlaArgs {
    const uint16_t* q;   // bf16 [B, Hq, 576]
    const uint16_t* kv;  // bf16 [B, N, 576]
    float* o_part;       // [B, Hq, S, 512]
    float* lse_part;     // [B, Hq, S]
    uint8_t* skip;       // [B, Hq, nk] or null
    int B, Hq, N, nk, S;
    float score_scale;   // softmax scale * log2(e)
    float thr;           // ln(lambda) * log2(e); -inf when lambda == 0
};

hipError_t launch_decode(const DecodeArgs& a, int d, int Bc, hipStream_t stream);
// Bytes of the per-device scratch of the allocation-free decode step.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
// The current device's scratch (device address, 256-byte aligned, kDecodeScratchBytes long).
hipError_t decode_scratch(void** ptr);
// Dense split-KV decode, K and V streamed together (no skip test); G <= 32, plain batches.
hipError_t launch_decode_dense(const DecodeArgs& a, int d, int Bc, hipStream_t stream);
// Measurement only: the loads of the split kernel's two-workgroups-per-split layout at lambda = 0, nothing else.
hipError_t launch_decode_load_only(const DecodeArgs& a, int d, int Bc, hipStream_t stream);
hipError_t launch_decode_mla(const MlaArgs& a, int Bc, hipStream_t stream);
hipError_t launch_decode_combine(const float* o_part, const float* lse_part, float* o, float* lse, int rows,
                                 int d, int S, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int d, int Bc, hipStream_t stream);
hipError_t launch_prefill_margins(const PrefillArgs& a, int d, int Bc, hipStream_t stream);
hipError_t launch_decode_margins(const DecodeArgs& a, int d, int Bc, hipStream_t stream);

}  // namespace blasst
