/*
 * blasst.h — C ABI of libblasst.so: skip-softmax ("BLASST") block-sparse
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The method (BLASST blog, "BLASST: Dynamic BLocked Attention Sparsity via
 * Softmax Thresholding", MLSys 2026 notes):
 *   Blockwise online-softmax attention (section on FlashAttention's online
 *   softmax, Eqs. 1-4) with one extra test (section on the decision rule,
 *   Eq. 5): for KV block j the kernel forms S = Q K_j^T / sqrt(d), takes the
 *   block row max mt, updates the running max m_new = max(m, mt), and skips
 *   the block when mt - m_new < ln(lambda).  A skipped block does no exp, no
 *   P V product and (in decode) no V load; S itself is always formed (section
 *   on what a skip saves).  In prefill a block is skipped only if every row of
 *   the query block votes to skip; in decode each query head decides alone
 *   (Table 12 discussion under the lambda = a/L section).
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous, row-major, innermost dimension last, in device
 *     memory owned by the caller.  q/k/v are bfloat16 (passed as const void*).
 *     Every pointer must be 16-byte aligned.
 *   - Query head h reads kv head h / gqa_ratio (Hkv = Hq / gqa_ratio):
 *     gqa_ratio = 1 is MHA, 1 < gqa_ratio < Hq is GQA, gqa_ratio = Hq is MQA.
 *   - lambda in [0, 1).  lambda = 0 never skips (dense attention).
 *   - Scores are scaled by 1/sqrt(d) before the max and the test.
 *   - Supported: d in {64, 128}, Bc in {64, 128}.  Sequence lengths need not
 *     be multiples of Bc: the last block is shorter.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and return once the kernels are enqueued.  Buffers must stay
 *     alive until the stream passes that point.  The library allocates no
 *     memory and keeps no state between calls; concurrent calls on different
 *     streams are safe.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     rejected call enqueues nothing.  A launch failure returns BLASST_ERR_HIP.
 *     No C++ exception crosses this interface.
 *   - Mask bytes: 0 = block kept, 1 = block skipped, 2 = block not visited
 *     (prefill, above the causal diagonal; ragged batches, past a sequence's
 *     end).
 */
#ifndef BLASST_H
#define BLASST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t. */
typedef struct ihipStream_t* blasst_stream_t;

typedef enum {
    BLASST_OK = 0,
    BLASST_ERR_INVALID_ARG = 1, /* null required pointer, bad size, lambda outside [0,1), ... */
    BLASST_ERR_UNSUPPORTED = 2, /* valid but not built: d or Bc outside {64,128}, ... */
    BLASST_ERR_HIP = 3,         /* a HIP launch or runtime call failed */
    BLASST_ERR_INTERNAL = 4
} blasst_status;

/*
 * Causal (or full) GQA prefill.  The blog's prefill kernel: every KV tile's
 * S = Q K^T is computed; a tile whose Bc query rows all vote to skip does no
 * exp, row sum or P V (section on the prefill kernel; query block height
 * Br = Bc).
 *
 *   q          bf16 [B, Hq,  T, d]
 *   k, v       bf16 [B, Hkv, T, d]       Hkv = Hq / gqa_ratio
 *   o          fp32 [B, Hq,  T, d]       output rows O / l
 *   lse        fp32 [B, Hq,  T] or NULL  natural-log m + ln(l) per row
 *   skip_mask  u8   [B, Hq, ceil(T/Bc), ceil(T/Bc)] or NULL; entry (i, j) is the
 *              decision for query block i and KV block j (0/1), or 2 when
 *              causal and j > i.  Every entry is written.
 *   causal     1: row t sees keys <= t.  0: every row sees every key.
 * Errors: INVALID_ARG for a null q/k/v/o, B/Hq/T < 0, d/Bc <= 0, gqa_ratio < 1
 * or not dividing Hq, lambda outside [0,1) or NaN, causal not 0/1;
 * UNSUPPORTED for d or Bc outside {64, 128}.  Scalar arguments are checked
 * first; then B*Hq*T == 0 returns OK and does nothing (the pointers may then be
 * NULL and are not read).
 */
blasst_status blasst_prefill(const void* q, const void* k, const void* v, float* o, float* lse,
                             uint8_t* skip_mask, int B, int Hq, int T, int d, int gqa_ratio,
                             int Bc, double lambda, int causal, blasst_stream_t stream);

/*
 * Split-KV decode step, one query token per (batch, query head).  The KV
 * blocks [0, ceil(N/Bc)) are cut into num_splits contiguous ranges, split s
 * covering [floor(s*nk/S), floor((s+1)*nk/S)); each split runs the online
 * softmax from a fresh state (running max -inf) and writes its normalised
 * partial output and log-sum-exp (split-KV tiles as in the SANTA notes'
 * FlashDecoding pattern).  Within a split, the blog's decode kernel is
 * followed: the S blocks of a batch are formed first, all their decisions
 * are taken together, and V is loaded only for blocks that some head of the
 * kv group keeps (section on the decode kernel, batched load scheduling).
 *
 *   q          bf16 [B, Hq, 1, d]
 *   k, v       bf16 [B, Hkv, N, d]       Hkv = Hq / gqa_ratio
 *   o_part     fp32 [B, Hq, num_splits, d]
 *   lse_part   fp32 [B, Hq, num_splits]  natural log
 *   skip_mask  u8   [B, Hq,  ceil(N/Bc)] or NULL   per-head decision
 *   vskip_mask u8   [B, Hkv, ceil(N/Bc)] or NULL   1 = V block not loaded
 *   causal     accepted for symmetry; one decode query sees all N keys.
 *   num_splits 1 <= num_splits <= ceil(N/Bc)
 * Errors: INVALID_ARG for a null q/k/v/o_part/lse_part, B/Hq < 0, N <= 0,
 * gqa_ratio < 1 or not dividing Hq, lambda outside [0,1), bad num_splits;
 * UNSUPPORTED for d or Bc outside {64, 128}, or gqa_ratio > 128.  Scalar
 * arguments are checked first; then B*Hq == 0 returns OK and does nothing (the
 * pointers may then be NULL and are not read).
 */
blasst_status blasst_decode(const void* q, const void* k, const void* v, float* o_part,
                            float* lse_part, uint8_t* skip_mask, uint8_t* vskip_mask, int B,
                            int Hq, int N, int d, int gqa_ratio, int Bc, double lambda,
                            int causal, int num_splits, blasst_stream_t stream);

/*
 * Dense references (plain softmax attention, nothing ever skipped, no decision
 * bytes; same arguments minus lambda and the masks; results equal the
 * lambda = 0 calls up to rounding order).  They are what the blog measures its
 * kernels against (dense FlashAttention; sections on kernel speed and on the
 * decision cost, 0.96-1.00x at 0% sparsity), and serve callers that want
 * plain attention.
 *
 * blasst_prefill_dense: blasst_prefill built without the skip test (no row
 * votes, no vote exchange between waves, every tile kept).
 *
 * blasst_decode_dense: split-KV decode in one pass (FlashDecoding).  For
 * gqa_ratio <= 32 a kernel of its own copies K and V of every 32-key unit
 * together and runs an online softmax per wave, with no decision and no
 * barrier before the merge of the waves -- the dense decode the skip kernel's
 * V savings are measured against.  Wider groups run blasst_decode's kernel
 * with the threshold at -inf.  o_part and lse_part are as blasst_decode's, so
 * blasst_decode_combine merges them; num_splits is the caller's choice (a
 * dense decode picks the split count that fills the GPU).
 * Errors as blasst_prefill / blasst_decode.
 */
blasst_status blasst_prefill_dense(const void* q, const void* k, const void* v, float* o, float* lse,
                                   int B, int Hq, int T, int d, int gqa_ratio, int Bc, int causal,
                                   blasst_stream_t stream);
blasst_status blasst_decode_dense(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                                  int B, int Hq, int N, int d, int gqa_ratio, int Bc, int num_splits,
                                  blasst_stream_t stream);

/*
 * blasst_decode_step: one whole split-KV decode step in one call -- blasst_decode
 * followed by blasst_decode_combine (the split-KV merge by log-sum-exp, SANTA
 * notes, method details), for callers that want O and not the split partials.
 * The partials live in a caller-provided workspace of
 * blasst_decode_step_workspace_size(B, Hq, d, num_splits) =
 * B*Hq*num_splits*(d+1)*4 bytes (o_part [B,Hq,S,d] fp32 then lse_part
 * [B,Hq,S] fp32), 16-byte aligned, which the call overwrites and the caller
 * owns; its contents after the call are unspecified.
 *   o          fp32 [B, Hq, d]: the merged output (the query's attention row)
 *   lse        fp32 [B, Hq] or NULL: the merged log-sum-exp
 *   skip_mask, vskip_mask, and every other argument: as blasst_decode.
 * Errors: as blasst_decode, plus INVALID_ARG for a NULL o, or a NULL,
 * misaligned or too small workspace (when B*Hq != 0).  Asynchronous on stream.
 * blasst_decode_step_workspace_size returns 0 for invalid sizes.
 */
size_t blasst_decode_step_workspace_size(int B, int Hq, int d, int num_splits);
blasst_status blasst_decode_step(const void* q, const void* k, const void* v, float* o, float* lse,
                                 uint8_t* skip_mask, uint8_t* vskip_mask, void* workspace, size_t workspace_bytes,
                                 int B, int Hq, int N, int d, int gqa_ratio, int Bc, double lambda, int causal,
                                 int num_splits, blasst_stream_t stream);

/*
 * blasst_decode_step_noalloc: blasst_decode_step for callers that cannot
 * allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing (no hipMalloc,
 * no hipFree, no allocating library call): the split partials live in a
 * static device array of the library, one per GPU, of
 * blasst_decode_step_noalloc_max_bytes() = 32 MiB, held until the process
 * ends.  Arguments as blasst_decode_step without the workspace; the current
 * device's array is used, so `stream` must belong to the current device.
 * Errors: as blasst_decode_step, plus UNSUPPORTED when the partials,
 * B*Hq*num_splits*(d+1)*4 bytes, exceed the array; HIP if the array's device
 * address cannot be looked up.
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's partials (every call writes all of the partials it reads, so nothing
 * must start at zero): calls that overlap on one GPU (on different streams, or
 * from several host threads) race and must be ordered by the caller.
 */
size_t blasst_decode_step_noalloc_max_bytes(void);
blasst_status blasst_decode_step_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                                         uint8_t* skip_mask, uint8_t* vskip_mask, int B, int Hq, int N, int d,
                                         int gqa_ratio, int Bc, double lambda, int causal, int num_splits,
                                         blasst_stream_t stream);

/*
 * blasst_decode_load_ceiling -- a measurement call, not part of any result.
 * Issues exactly the HBM reads blasst_decode's kernel issues at lambda = 0 in
 * its two-workgroups-per-split layout (every K row of a split read by both
 * workgroups of the pair, which share one L2; each workgroup then half of
 * every V row), through the same LDS rings, and nothing else: no arithmetic,
 * no barrier, no output.  Its time is the floor that the bytes of
 * K + V = 2 * B * Hkv * N * d * 2 and that access pattern set for the decode
 * split kernel (the memory-bound decode kernel of the BLASST blog's section
 * on the decode kernel), so a bench can state how far the kernel is from its
 * own data movement.  k, v as blasst_decode; same validation (d, Bc in
 * {64, 128}, 1 <= num_splits <= ceil(N / Bc)).  Asynchronous on stream.
 */
blasst_status blasst_decode_load_ceiling(const void* k, const void* v, int B, int Hkv, int N, int d, int Bc,
                                         int num_splits, blasst_stream_t stream);

/*
 * Ragged batches: one length per sequence (the serving-shaped form of the same
 * two calls).  The tensors keep their padded layout -- T (prefill) or N
 * (decode) is the capacity, the row stride of every sequence -- and sequence b
 * uses only its first seq_lens[b] rows, each sequence being exactly the
 * plain call at its own length.
 *
 *   seq_lens  int32 [B], device memory, 4-byte aligned; values are clamped to
 *             [0, T] or [0, N] on the device (they are never read on the host).
 *
 * blasst_prefill_ragged: arguments as blasst_prefill.  Sequence b is a causal
 * (or full) prefill of its first L_b = seq_lens[b] query rows over its first L_b
 * keys.  Rows t >= L_b hold O = 0 and LSE = -inf; skip_mask entries of query
 * blocks i >= ceil(L_b/Bc) and of KV blocks j >= ceil(L_b/Bc) are 2 (not visited).
 * Errors as blasst_prefill, plus INVALID_ARG for a null or misaligned seq_lens
 * when B*Hq*T != 0.
 */
blasst_status blasst_prefill_ragged(const void* q, const void* k, const void* v, float* o, float* lse,
                                    uint8_t* skip_mask, const int32_t* seq_lens, int B, int Hq, int T, int d,
                                    int gqa_ratio, int Bc, double lambda, int causal, blasst_stream_t stream);

/*
 * blasst_decode_ragged: arguments as blasst_decode (without `causal`).
 * Sequence b attends to its first N_b = seq_lens[b] keys; its nk_b =
 * ceil(N_b/Bc) blocks are cut into the num_splits ranges of blasst_decode.  A
 * split left with no block (num_splits > nk_b, or N_b = 0) writes O = 0 and
 * LSE = -inf, the identity of the merge.  Mask entries of blocks j >= nk_b are
 * 2 (not visited).  num_splits is checked against the capacity:
 * 1 <= num_splits <= ceil(N/Bc).  Errors as blasst_decode, plus INVALID_ARG for
 * a null or misaligned seq_lens when B*Hq != 0.
 */
blasst_status blasst_decode_ragged(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                                   uint8_t* skip_mask, uint8_t* vskip_mask, const int32_t* seq_lens, int B, int Hq,
                                   int N, int d, int gqa_ratio, int Bc, double lambda, int num_splits,
                                   blasst_stream_t stream);

/*
 * MLA decode: multi-head latent attention in its absorbed decode form (the
 * variant named in the BLASST blog's section on the decode kernel: MLA decode
 * can be compute bound, so a skip also saves the softmax -- the exp, the row
 * sum and the P V product -- not only a V load).  Every query head of sequence
 * b reads the same cache row per token, [latent (d_v) | rotary (d_qk - d_v)];
 * the value of token t is its latent part kv[b, t, 0 .. d_v).  Scores are
 * (q . kv_t) * softmax_scale.  Blocks of Bc tokens, num_splits contiguous
 * splits each restarting the running max, and per-head decisions exactly as in
 * blasst_decode (each head decides alone); the P V product of a block is
 * formed only for heads that keep it.  Merge the splits with
 * blasst_decode_combine (d = d_v).
 *
 *   q          bf16 [B, Hq, d_qk]          (absorbed queries)
 *   kv         bf16 [B, N, d_qk]           (latent cache rows)
 *   o_part     fp32 [B, Hq, num_splits, d_v]
 *   lse_part   fp32 [B, Hq, num_splits]    natural log
 *   skip_mask  u8   [B, Hq, ceil(N/Bc)] or NULL   per-head decision
 *   softmax_scale  the model's scale (e.g. 1/sqrt(192) for 128 + 64 query
 *              columns before absorption); finite and > 0
 *   num_splits 1 <= num_splits <= ceil(N/Bc)
 * Built for d_qk = 576, d_v = 512, and Bc = 64 with Hq a multiple of 32, or
 * Bc = 32 with Hq a multiple of 64 (smaller blocks let the kernel keep three
 * blocks of cache rows in flight instead of one).
 * Errors: INVALID_ARG for a null q/kv/o_part/lse_part, B/Hq < 0, N <= 0,
 * d_v > d_qk, a bad scale or lambda, bad num_splits, a misaligned pointer;
 * UNSUPPORTED for other d_qk/d_v/Bc or head counts.  Scalar
 * arguments are checked first; then B*Hq == 0 returns OK and does nothing.
 */
blasst_status blasst_decode_mla(const void* q, const void* kv, float* o_part, float* lse_part,
                                uint8_t* skip_mask, int B, int Hq, int N, int d_qk, int d_v, int Bc,
                                double softmax_scale, double lambda, int num_splits,
                                blasst_stream_t stream);

/*
 * Merge of the splits by their true normalisers (SANTA notes, merge of
 * FlashDecoding tiles): LSE = ln sum_s exp(lse_s), O = sum_s exp(lse_s - LSE) O_s.
 * A split with lse_s = -inf contributes nothing; when every split has
 * lse_s = -inf (no key at all) the row gets O = 0 and LSE = -inf.
 *
 *   o_part     fp32 [B, Hq, num_splits, d]
 *   lse_part   fp32 [B, Hq, num_splits]
 *   o          fp32 [B, Hq, d]
 *   lse        fp32 [B, Hq] or NULL
 * Errors: INVALID_ARG for a null o_part/lse_part/o, B/Hq < 0, num_splits < 1,
 * d <= 0; UNSUPPORTED for d outside {64, 128, 512} (512: MLA's latent width).  B*Hq == 0 returns OK without
 * reading the pointers.
 */
blasst_status blasst_decode_combine(const float* o_part, const float* lse_part, float* o,
                                    float* lse, int B, int Hq, int d, int num_splits,
                                    blasst_stream_t stream);

/*
 * Decision margins for every lambda at once: the one-pass calibration tool
 * (BLASST blog, section on the lambda = a/L policy and Algorithm 2, and section
 * on the decision rule, Eq. 5).  A block's skip test compares D = m~ - m_new
 * (block max minus the updated running max, scaled scores) with ln(lambda);
 * since a skipped block never moves the running max, m_new is the prefix max
 * of the block maxima and D does not depend on lambda.  So one pass gives the
 * decision -- and the block sparsity -- at any lambda: skipped iff D < ln(lambda).
 * These passes form S = Q K^T only: no softmax, no V, no outputs besides the
 * margins.  Margins are fp32, natural-log units.
 *
 * blasst_prefill_margins: q, k as in blasst_prefill (v is not read).
 *   margin  fp32 [B, Hq, ceil(T/Bc), ceil(T/Bc)]: for query block i and KV block
 *           j, the max over the block's rows of D (the AND over rows becomes
 *           a max: skipped iff every row's D < ln(lambda)); NaN for blocks the
 *           causal mask leaves unvisited (j > i).
 * Errors and argument rules as blasst_prefill (lambda absent); a null margin is
 * INVALID_ARG.
 */
blasst_status blasst_prefill_margins(const void* q, const void* k, float* margin, int B, int Hq, int T, int d,
                                     int gqa_ratio, int Bc, int causal, blasst_stream_t stream);

/*
 * blasst_decode_margins: q, k as in blasst_decode (v is not read).
 *   margin   fp32 [B, Hq, ceil(N/Bc)]: D per query head and block, the running
 *            max restarting at each of the num_splits splits.
 *   vmargin  fp32 [B, Hkv, ceil(N/Bc)] or NULL: the max of D over the kv
 *            group's heads (the V block is not loaded iff it is < ln(lambda)).
 * Errors and argument rules as blasst_decode (lambda absent); a null margin
 * is INVALID_ARG.  Above 64 heads per kv head, vmargin is formed by a second
 * kernel from margin after the pass.
 */
blasst_status blasst_decode_margins(const void* q, const void* k, float* margin, float* vmargin, int B, int Hq,
                                    int N, int d, int gqa_ratio, int Bc, int num_splits, blasst_stream_t stream);

/* Static, human-readable name of a status code. */
const char* blasst_status_string(blasst_status status);

#ifdef __cplusplus
}
#endif

#endif /* BLASST_H */
