/*
 * ffpa_attn.h - C ABI of the large-head-dimension fused attention library
 * (libffpa_attn.so, hand-written HIP kernels for AMD MI355X / gfx950).
 *
 * Operation. The forward computes, for every batch b and query head h,
 *     O[b,h] = softmax(scale * Q[b,h] K[b,hk]^T + mask) V[b,hk],   hk = h / (Hq / Hkv)
 * and the natural-log log-sum-exp of each row of the scaled, masked scores.
 *  - The definition is the materialised attention listed as "naive_math" in
 *    section "3. Attention Variants" of the attention-kernel-profiler design
 *    document (scores = Q K^T / sqrt(d_head), mask, softmax, attn V); the
 *    scale is an argument here (callers normally pass 1/sqrt(D)).
 *  - The additive mask is the one of "FFPA Attention Benchmark"
 *    (ffpa-attn.readthedocs.io), section "Quick Start": a compact key-position
 *    bias of shape [1,1,1,Nkv] (mask_rows = 1), or a per-query bias
 *    [1,1,Nq,Nkv] (mask_rows = Nq). It is added to the scaled scores.
 *  - Grouped-query attention maps query head h to K/V head h / (Hq/Hkv), the
 *    repeat_interleave convention of "gqa_4kv" in the same section 3.
 *  - The cases served are those of the benchmark tables in section "More
 *    Benchmark" of "FFPA Attention Benchmark": self-attn, cross-attn
 *    (Nq != Nkv), decode-attn (Nq = 1), gqa, causal, attn-mask and
 *    non-aligned lengths, at head dimensions well above 256 (D = 320 ... 1024,
 *    "FFPA-Attn Performance Benchmarks on Lambda.ai", sections 1-3).
 *  - The backward returns dQ, dK, dV: the "standard 5 GEMMs" backward named in
 *    "More Benchmark" (P recomputed from Q, K and the forward's lse).
 *
 * Readings taken where the pages say nothing:
 *  - causal masking is top-left aligned: query i sees keys j <= i, also when
 *    Nq != Nkv (so a lone decode query sees key 0 only);
 *  - a query row whose every score is -inf gets O = 0 and lse = -inf;
 *  - lse is natural-log and includes scale and mask;
 *  - "fp16 accumulation" (FFPA_ACC_F16): gfx950 has no MFMA with an fp16
 *    result, so scores and every MFMA partial (one key tile's P V product)
 *    stay fp32; the running output accumulator is held in fp16, kept
 *    normalised (|O| <= max |V|), and each tile's product is rounded to fp16
 *    when folded into it. For bf16 inputs the accumulator is fp16 as well:
 *    V entries must then lie inside fp16's range (|v| < 65520); an element
 *    whose product reaches fp16 infinity makes that output element
 *    non-finite (use FFPA_ACC_F32 for such data).
 *
 * Layout. All tensors are dense, row-major and contiguous:
 *   q, o, dout, dq : [B, Hq,  Nq,  D]  (element type = dtype)
 *   k, v, dk, dv   : [B, Hkv, Nkv, D]  (element type = dtype)
 *   lse            : [B, Hq,  Nq]      float32
 *   mask           : [mask_rows, Nkv]  (element type = dtype, -inf allowed)
 * Element type: FFPA_F16 = IEEE binary16, FFPA_BF16 = bfloat16.
 * Outputs are rounded to nearest even.
 *
 * Ownership and memory. Every tensor pointer is a DEVICE pointer owned by the
 * caller; the library never allocates or frees device memory. Pointers must
 * be 16-byte aligned. Scratch space, when an entry point needs it, is passed
 * by the caller as (workspace, workspace_bytes); its size comes from the
 * matching *_workspace_size query. It need not be initialised.
 *
 * Execution. Entry points validate their arguments, then only enqueue kernels
 * on `stream` (a hipStream_t; NULL = the default stream) and return. FFPA_OK
 * means "launched"; faults on the device surface at the caller's next
 * synchronisation. Calls that share a workspace must be ordered on one stream.
 *
 * Errors. On any non-OK status nothing has been enqueued and no output has
 * been written; ffpa_last_error() returns a thread-local message. Arguments
 * are checked in this order: null required pointer, sizes < 1,
 * Hq % Hkv != 0, causal not 0/1, mask_rows not in {1, Nq} with a mask present
 * (FFPA_ERR_INVALID_ARG); dtype, accumulator or D not supported
 * (FFPA_ERR_UNSUPPORTED); a pointer not 16-byte aligned or a NaN scale
 * (FFPA_ERR_INVALID_ARG); workspace too small (FFPA_ERR_WORKSPACE); a shape
 * the built kernels do not cover (FFPA_ERR_UNSUPPORTED); a HIP launch error
 * (FFPA_ERR_HIP).
 *
 * Threading. The library holds no mutable global state besides the
 * thread-local error message, the table of tuned variants (mutex-guarded;
 * see ffpa_attn_fwd_tune) and, for ffpa_attn_fwd_noalloc, its per-GPU
 * scratch array (see there); all other entry points are reentrant.
 */
#ifndef FFPA_ATTN_H_
#define FFPA_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FFPA_F16 = 0, FFPA_BF16 = 1 } ffpa_dtype_t;
typedef enum { FFPA_ACC_F32 = 0, FFPA_ACC_F16 = 1 } ffpa_accum_t;
typedef enum {
  FFPA_OK = 0,
  FFPA_ERR_INVALID_ARG = 1,
  FFPA_ERR_UNSUPPORTED = 2,
  FFPA_ERR_WORKSPACE = 3,
  FFPA_ERR_HIP = 4
} ffpa_status_t;

/* Largest supported head dimension; D must be a multiple of 32 in [32, 1024]. */
#define FFPA_MAX_HEAD_DIM 1024

/*
 * Forward attention.
 *   q, k, v   : inputs (layout above).
 *   o         : output [B, Hq, Nq, D], written in full.
 *   lse       : output [B, Hq, Nq] float32, or NULL to skip it.
 *   scale     : multiplies Q K^T before the mask is added (usually 1/sqrt(D)).
 *   causal    : 0 or 1 (top-left aligned).
 *   mask      : NULL, or an additive mask [mask_rows, Nkv] with mask_rows 1 or Nq.
 *   accum_dtype : FFPA_ACC_F32 or FFPA_ACC_F16 (see the reading above).
 *   dtype     : FFPA_F16 or FFPA_BF16, for q, k, v, mask and o.
 *   workspace : device scratch of at least ffpa_attn_fwd_workspace_size(...)
 *               bytes, 16-byte aligned (NULL allowed when that size is 0).
 *               Nq = 1 takes the split-KV decode path, which keeps
 *               per-key-range partial outputs (fp32 o and log-sum-exp) there.
 *               For Nq > 1 with D > 512, or D <= 512 and Nq * Hq >=
 *               3072 * Hkv (many queries per key), the call first writes a
 *               transposed copy of V there, dtype, zero past Nkv, the size
 *               of V with the keys padded to P = Nkv rounded up to 64:
 *               [B, Hkv, D, P] for D <= 512, and in blocks of 32 keys
 *               [B, Hkv, P / 32, D, 32] for D > 512. The attention kernel
 *               reads its V operand from it; otherwise the call needs none.
 *               The call owns the workspace until the work it enqueued has
 *               finished.
 *   stream    : hipStream_t to enqueue on.
 * Built today: every D (multiple of 32, <= 1024) for Nq = 1; for Nq > 1, D a
 * multiple of 64 up to 1024. Both mask shapes are built on every path. Other
 * valid shapes (Nq > 1 with D not a multiple of 64) return
 * FFPA_ERR_UNSUPPORTED before any launch. The accumulator, by path:
 *  - Nq > 1, D <= 512: fp32 or fp16 as accum_dtype asks (one kernel each);
 *  - Nq > 1, D > 512: FFPA_ACC_F32 runs a kernel that splits D across wave
 *    pairs with an fp32 accumulator (64 query rows per workgroup);
 *    FFPA_ACC_F16 runs one with the fp16 accumulator (128 rows per
 *    workgroup up to D = 768, where a wave holds all of D; 64 above);
 *  - Nq = 1 (decode, bound by memory bandwidth): fp32 whatever accum_dtype
 *    asks for (at least as accurate as asked).
 */
int ffpa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                  const void* mask, int mask_rows, int accum_dtype, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace ffpa_attn_fwd needs for these sizes (0 if none). */
size_t ffpa_attn_fwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype);

/*
 * Forward attention that allocates nothing and takes no workspace: for
 * callers that cannot allocate device memory (work captured into a HIP graph,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * results and error order as ffpa_attn_fwd without (workspace,
 * workspace_bytes); it calls no allocating routine.
 *  - Scratch: a 32 MiB array in each GPU's memory that the library holds from
 *    its load until the process ends (one per GPU it runs on). When
 *    ffpa_attn_fwd_workspace_size(...) <= 32 MiB the call runs exactly the
 *    path of ffpa_attn_fwd with that array as its workspace (same bits).
 *  - Larger needs: for Nq > 1 and D <= 512 the call stages V as is instead of
 *    writing its transposed copy (no scratch; same results up to rounding
 *    order); otherwise it returns FFPA_ERR_WORKSPACE before any launch.
 *  - Every call on one GPU shares that GPU's array: calls that overlap on one
 *    GPU (several streams, or host threads) race on it; order them. The array
 *    keeps whatever the last call left; every call writes what it reads.
 *  - The stream's device is the one whose array is used; its address is looked
 *    up (hipGetSymbolAddress) on the first call there, and a failure of that
 *    lookup returns FFPA_ERR_HIP.
 */
int ffpa_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                          const void* mask, int mask_rows, int accum_dtype, int dtype, void* stream);

/*
 * Backward attention: given dout = dL/dO, writes dq, dk, dv (same dtype and
 * layout as q, k, v). o and lse must be the forward's outputs for the same
 * q, k, v, scale, causal and mask. dk and dv of a K/V head sum the
 * contributions of all query heads that share it. accum_dtype must be
 * FFPA_ACC_F32. workspace: 16-byte aligned, at least
 * ffpa_attn_bwd_workspace_size_min(...) bytes (delta_i = sum_d dO_id O_id
 * and lse_i log2(e) per query row, rows padded to a multiple of 64). The
 * path is chosen by the workspace size alone:
 *  - with room beyond the minimum for a transposed copy of K (the size of K,
 *    keys padded to 64) and the dS blocks of at least one kv head's query
 *    heads (g * ceil(Nq/32) * ceil(Nkv/32) * 2 KiB, g = Hq / Hkv), the dK/dV
 *    pass stores dS (bf16/fp16, per 32 x 32 block) and the dQ pass reads it
 *    back (one product instead of three). Both passes run over chunks of as
 *    many kv heads as the dS room holds, reusing it chunk after chunk;
 *  - otherwise, for one query row (Nq = 1) without dropout and a group of
 *    g = 1, 2 or 4 query heads per kv head (4 only up to D = 512), with at
 *    least max(minimum, B * Hq * S * D * 4) bytes: the decode backward, a
 *    stream over K and V on the vector ALUs that writes dK and dV once per
 *    key and fp32 dQ partials of S key ranges per head (S: about 2048 waves
 *    over the B * Hkv kv heads, ranges of at least 256 keys, at most 64),
 *    which a second kernel adds in range order;
 *  - with less, dQ recomputes S and dP.
 * ffpa_attn_bwd_workspace_size(...) gives the stored-dS path a dS buffer of at
 * most 1 GiB, or more where needed for one kv head's group or for a chunk
 * whose dQ pass has at least 512 workgroups, in equal chunks: at B = 1,
 * Hq = Hkv = 32, D = 512 that is 8 heads of 128 MiB at N = 8192 (1 GiB) and
 * 4 heads of 512 MiB at N = 16384 (2 GiB) (ffpa_attn_bwd_workspace_size_stored).
 * For Nq = 1 ffpa_attn_bwd_workspace_size returns the decode backward's
 * size where that path is built, and for other Nq <= 64 the minimum: one dQ
 * workgroup per head then reads K and V once, which costs less than the
 * transposed copy of K.
 * Every path and chunk size gives the same gradients up to rounding order;
 * a given workspace size always gives the same bits. Kernels enqueued: the
 * delta pass, then [the K transpose, then per chunk: dK/dV, dQ] or
 * [dK/dV, dQ]; or the decode backward and its dQ sum. Built for D a multiple of 64 up to 1024, with either mask
 * shape; other valid shapes (D not a multiple of 64) return
 * FFPA_ERR_UNSUPPORTED.
 * The gradients are those of sum(dout * O) ("FFPA Attention Benchmark",
 * "More Benchmark": the backward counted as 5 GEMMs).
 */
int ffpa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv,
                  int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                  const void* mask, int mask_rows, int accum_dtype, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace the backward takes by default: that of the stored-dS
 * path with its default, bounded dS buffer (ffpa_attn_bwd_workspace_size_stored);
 * for Nq = 1 that of the decode backward where it is built; for other
 * Nq <= 64 the minimum. */
size_t ffpa_attn_bwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype);

/* Bytes of workspace of the stored-dS path with its default, bounded dS
 * buffer, whatever Nq. */
size_t ffpa_attn_bwd_workspace_size_stored(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype);

/* The least workspace ffpa_attn_bwd accepts (dQ then recomputes S and dP). */
size_t ffpa_attn_bwd_workspace_size_min(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype);

/*
 * Forward variants and tuning: the pages' benchmark tunes its kernels per
 * problem ("FFPA Attention Benchmark", "Quick Start": --tune fast / --tune
 * max; the H20 tables of "More Benchmark" are taken with autotuning). Here
 * every problem has a few built variants (tile shape or staging layout), all
 * computing the same attention:
 *   Nq > 1, D <= 512: 1 = V staged in LDS as is (transposed by the LDS
 *                     reads), 2 = V read from a transposed copy that the call
 *                     first writes to the workspace;
 *   Nq > 1, D > 512:  1 = fp32 output accumulator, 64 query rows per
 *                     workgroup, D split across wave pairs; with
 *                     accum_dtype = FFPA_ACC_F16 also 2 = fp16 accumulator,
 *                     a wave holds all of D, 128 rows per workgroup (D <= 768;
 *                     64-key tiles at D = 576 and 640, 32-key tiles above)
 *                     and 3 = fp16 accumulator, D split across wave pairs, 64
 *                     rows per workgroup;
 *   Nq = 1:           1, 2, 3 = the default number of key ranges per head
 *                     (split-KV) divided by 1, 2, 4.
 * Variant 0 is the library's default choice (the one ffpa_attn_fwd runs
 * untuned). Results of different variants agree within the accuracy of the
 * accumulator; a given variant always gives the same bits.
 *
 * ffpa_attn_fwd_variant: ffpa_attn_fwd as `variant` (0 .. 3); a variant that
 * does not exist for the problem returns FFPA_ERR_INVALID_ARG (checked after
 * the argument checks of ffpa_attn_fwd, before the workspace check). Its
 * workspace is ffpa_attn_fwd_variant_workspace_size(...) bytes.
 *
 * ffpa_attn_fwd_tune: times every variant that exists for the problem and
 * fits the workspace given (level 1 = "fast": 1 warm-up and 3 timed calls
 * each; level 2 = "max": 3 and 10), on the caller's buffers and stream with
 * HIP events, and records the fastest for this problem (sizes, causal, mask
 * shape, accum_dtype, dtype) in a table of the process. Later ffpa_attn_fwd
 * and ffpa_attn_fwd_noalloc calls of that problem run the recorded variant
 * when their workspace holds what it needs (else the default). It writes o
 * and lse (last with the chosen variant), and blocks the calling thread until
 * the timing runs finish. chosen (nullable) receives the variant; ms
 * (nullable, 3 floats) the mean milliseconds per call of variants 1 .. 3, -1
 * for those not run. Returns FFPA_ERR_WORKSPACE if no variant fits the
 * workspace; the table is guarded by a mutex. ffpa_attn_tune_reset empties it.
 */
int ffpa_attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                          const void* mask, int mask_rows, int accum_dtype, int dtype, int variant,
                          void* workspace, size_t workspace_bytes, void* stream);

size_t ffpa_attn_fwd_variant_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype,
                                            int causal, int variant);

int ffpa_attn_fwd_tune(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                       const void* mask, int mask_rows, int accum_dtype, int dtype,
                       void* workspace, size_t workspace_bytes, int level, int* chosen, float* ms,
                       void* stream);

void ffpa_attn_tune_reset(void);

/*
 * FP8 forward: S = Q K^T and O = P V on the fp8 (OCP e4m3) matrix cores of
 * gfx950, fp32 accumulation. The pages list fp8 attention kernels next to the
 * 16-bit ones ("FFPA Attention Benchmark", "FP8 and FP4") without stating
 * their quantisation; the reading taken here:
 *  - each head's Q, each kv head's K and V: one scale per head and tensor,
 *    x8 = e4m3(x * (448 / amax)) with amax = max |x| over that head, the
 *    product in fp32, rounded to nearest even (448 is e4m3's largest finite
 *    value; an all-zero head gets codes 0);
 *  - scores S = scale * (Q8 K8^T) * (amax_Q / 448) * (amax_K / 448), online
 *    softmax in fp32 against a running reference m per row: over the keys in
 *    tiles of 64 (in order), m rises to the tile's largest score when that
 *    exceeds m by more than 2.5 ln(2), and only then; P = exp(S - m) of the
 *    tile (at most 2^2.5) is quantised as e4m3(64 P); the row sum takes the
 *    unquantised P;
 *  - O = (sum_j P8_j V8_j) (amax_V / 448) / (64 l), rounded to the output
 *    type; lse = m + ln l (natural log, of the scores above).
 * q, k, v, o, lse, sizes, scale, causal (top-left), dtype: as ffpa_attn_fwd
 * (no mask; FFPA_ACC_F32 implied). Built for D a multiple of 64 in
 * [128, 512] (else FFPA_ERR_UNSUPPORTED, checked after the argument checks of
 * ffpa_attn_fwd). workspace: at least ffpa_attn_fwd_fp8_workspace_size(...)
 * bytes, 16-byte aligned; the call writes there the per-head amax values, Q8,
 * K8 and V8 transposed per tile of 64 keys. Kernels enqueued: amax clear,
 * amax, quantisation of Q and K, of V, the attention.
 */
int ffpa_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

size_t ffpa_attn_fwd_fp8_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D);

/*
 * Attention with dropout on the attention probabilities: the "dropout" case
 * of the forward and backward tables of "FFPA Attention Benchmark", section
 * "More Benchmark", which run it beside PyTorch SDPA. The pages fix neither
 * the random numbers nor p; the reading taken here is SDPA's dropout_p:
 *     O = (softmax(scale Q K^T + mask) o Z / (1 - p')) V,
 * Z a 0/1 keep mask, dropped after the softmax; lse is that of the undropped
 * scores. The keep mask is counter-based, so that the backward (and any
 * checker) regenerates it from (seed, head, query, key) alone:
 *  - generator: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 *    numbers: as easy as 1, 2, 3", SC 2011), key = (seed low 32 bits, seed
 *    high 32 bits);
 *  - one call per block of 4 queries x 4 keys of a head: counter
 *    (key / 4, query / 4, b * Hq + h, 0); of its four 32-bit output words,
 *    word query % 4 belongs to the query and byte key % 4 of that word (bits
 *    8 (key % 4) .. +7) to the element;
 *  - the element is kept when that byte is >= t, t = round(256 dropout_p)
 *    computed in float32 (at most 255); kept elements are scaled by
 *    256 / (256 - t). So p' = t / 256 exactly; dropout_p = 0 (t = 0) is the
 *    plain attention, bit for bit the same as ffpa_attn_fwd / _bwd.
 * dropout_p must lie in [0, 1): else FFPA_ERR_INVALID_ARG, checked after the
 * pointer alignment (and, in the forward, scale) checks and before the
 * workspace check. The dropout kernels accumulate in fp32: in the forward,
 * t > 0 with accum_dtype = FFPA_ACC_F16 returns FFPA_ERR_UNSUPPORTED (before
 * the workspace check). Workspace, layout, paths and errors otherwise as
 * ffpa_attn_fwd and ffpa_attn_bwd (same workspace sizes). The backward must
 * get the forward's seed and dropout_p.
 */
int ffpa_attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                          const void* mask, int mask_rows, int accum_dtype, int dtype,
                          float dropout_p, uint64_t seed,
                          void* workspace, size_t workspace_bytes, void* stream);

int ffpa_attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                          const void* mask, int mask_rows, int accum_dtype, int dtype,
                          float dropout_p, uint64_t seed,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Thread-local message describing the last non-OK status ("" if none). */
const char* ffpa_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int ffpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFPA_ATTN_H_ */
