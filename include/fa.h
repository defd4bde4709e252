/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (forward,
 * split-KV forward, backward).
 *
 * The operation is the attention of "FlashAttention算子优化" section 2 and
 * of "FlashAttention 与显存" plates 04, 07 and 08: for every batch b and head
 * h,
 *     S = scale * Q K^T            ([N_q, N_kv] scores; never stored)
 *     P = softmax(S) row by row    (with the causal mask, if requested)
 *     O = P V                      ([N_q, d])
 *     LSE_i = ln(sum_j exp(S_ij))  (the per-row statistic that plate 09 keeps
 *                                   for the backward pass, in one number)
 * computed tile by tile with the online softmax, so S and P never reach HBM.
 * The result equals the definition up to floating-point rounding.
 *
 * Very long key ranges.  The single-pass forward (fa_fwd, fa_fwd_ex) adds
 * each key tile's share to float32 running sums per row (the row sum once
 * per tile, the output accumulator once per 16 to 64 keys).  Each addition
 * can round away up to half an ulp of the running sum, so when much of a
 * row's softmax mass is spread thinly over a long key range the error grows
 * with the number of additions: with 2^24 keys of which the low-score
 * majority carries 2-12 % of the mass, O is off by about 1e-2 and LSE by
 * about 6e-3, against bars of 5e-3 and 1e-3.  The single-pass entry points
 * therefore accept at most FA_MAX_NKV_SINGLE_PASS = 2^20 keys per row, where
 * the same worst case stays at ordinary rounding, and return FA_ERR_LONG_KV
 * beyond it.  fa_fwd_splitkv sums chunks of at most 2^20 keys and merges
 * them, and handles any N_kv up to 2^30 (O relative L2 2e-3, LSE 2e-5
 * measured at 2^24 keys).  Byte offsets are 64-bit throughout: tensors
 * larger than 4 GiB are supported.
 *
 * Layout.  Q is [B, H, N_q, d]; K and V are [B, H, N_kv, d]; O is
 * [B, H, N_q, d]; LSE is [B, H, N_q].  All are dense row-major with d the
 * fastest dimension (the per-(batch, head) [N, d] slices of the section-2
 * pseudocode of "FlashAttention算子优化", stacked).
 *
 * Element types.  FA_F32, FA_F16 and FA_BF16 inputs produce O of the same
 * type.  FA_FP8_E4M3 inputs (OCP E4M3, per-tensor descales, see
 * fa_fwd_args) produce O in bfloat16.  LSE is always float32, natural log,
 * of the scaled (and masked) scores.
 *
 * Causal mask.  When causal != 0, key j is visible to query i iff j <= i
 * (top-left alignment, also when N_q != N_kv); no row is ever fully masked.
 *
 * Memory.  Q, K, V, O and LSE are device pointers on the current HIP device,
 * owned by the caller.  Q, K, V are read-only; O and LSE are written in
 * full.  The library allocates nothing and keeps no mutable global state, so
 * calls on different streams may run concurrently.  Calls are asynchronous
 * with respect to the host; errors raised while a kernel runs surface at the
 * caller's next synchronisation.
 *
 * Errors.  Every entry point returns 0 (FA_OK) or an fa_status code;
 * fa_strerror() names it.  Arguments are validated on the host, before any
 * HIP call; no C++ exception crosses this interface.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_F32 = 0,
    FA_F16 = 1,
    FA_BF16 = 2,
    FA_FP8_E4M3 = 3
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer (Q, K, V, O, args) is NULL */
    FA_ERR_SHAPE = 2,     /* B, H or N_q < 0, N_kv < 1, or a size overflows */
    FA_ERR_HEAD_DIM = 3,  /* d not in {64, 128, 256} */
    FA_ERR_DTYPE = 4,     /* dtype not an fa_dtype value */
    FA_ERR_ALIGN = 5,     /* Q, K, V or O not 16-byte aligned, LSE not 4-byte aligned */
    FA_ERR_SCALE = 6,     /* scale or a descale is not finite */
    FA_ERR_ALIAS = 7,     /* O or LSE overlaps Q, K, V, or each other */
    FA_ERR_DEVICE = 8,    /* no usable gfx950 device / HIP runtime error before launch */
    FA_ERR_LAUNCH = 9,    /* the kernel launch failed */
    FA_ERR_VARIANT = 10,  /* no compiled variant for this problem / tile_override out of range */
    FA_ERR_WORKSPACE = 11, /* split-KV or backward workspace NULL, misaligned or too small */
    FA_ERR_DROPOUT = 12,   /* dropout_p outside [0, 1), or dropout where it is not supported */
    FA_ERR_LONG_KV = 13,   /* N_kv above FA_MAX_NKV_SINGLE_PASS for fa_fwd / fa_fwd_ex */
    FA_ERR_SCRATCH = 14    /* fa_fwd_splitkv_noalloc: partials exceed FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Longest key range per row the single-pass forward accepts (see "Very
 * long key ranges"); also the longest chunk fa_fwd_splitkv forms. */
#define FA_MAX_NKV_SINGLE_PASS (1 << 20)

/*
 * fa_fwd -- attention forward on the null stream.
 *
 * Q, K, V: device inputs (see Layout); O: device output; LSE: device
 * float32 output, or NULL to skip it.  B, H >= 0 batches and heads;
 * N_q >= 0 query rows and 1 <= N_kv <= FA_MAX_NKV_SINGLE_PASS key rows per
 * head (FA_ERR_LONG_KV above it); d in {64, 128, 256}.
 * B, H or N_q equal to 0 is a successful no-op.  scale multiplies QK^T
 * before the softmax (1/sqrt(d) in the pages); any finite value is valid,
 * including 0 and negative values.  causal: 0 or non-zero (see Causal
 * mask).  dtype: an fa_dtype; FA_FP8_E4M3 needs fa_fwd_ex for descales
 * other than 1.
 */
int fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE,
           int64_t B, int64_t H, int64_t N_q, int64_t N_kv, int64_t d,
           float scale, int causal, int dtype);

/*
 * Full argument set.  descale_q/k/v multiply the decoded E4M3 values of Q,
 * K and V (only read for FA_FP8_E4M3; must be finite).  stream is a
 * hipStream_t (NULL = null stream).  tile_override selects a compiled tile
 * variant (0 = the library's choice; 1..fa_num_variants() for tuning and
 * cross-checks).
 *
 * Dropout ("FlashAttention 与显存" plates 07 and 09 list it among the
 * operations the fused kernel absorbs; the pages give no generator).
 * dropout_p in [0, 1) is quantised to p8 / 256 with p8 = floor(256 p + 1/2)
 * clamped to 255; p8 = 0 means no dropout.  Otherwise
 *     O_i = 256 / (256 - p8) * sum_j P_ij keep_ij v_j
 * (LSE stays that of the scores), where keep_ij = 1 iff byte
 * 4 (i mod 4) + (j mod 4) of Philox4x32-10 (Salmon et al., SC 2011) with
 * counter (j / 4, i / 4, b H + h, dropout_offset mod 2^32) and key
 * (dropout_seed mod 2^32, dropout_seed / 2^32) is >= p8; byte k of the four
 * output words w0..w3 is bits 8 (k mod 4) .. +7 of word k / 4.  i and j are
 * the row and key indices within the (batch, head).  Supported for FA_F16
 * and FA_BF16 (every d and tile variant); FA_ERR_DROPOUT for other dtypes
 * and from fa_fwd_splitkv.  fa_bwd with the
 * same dropout_p, dropout_seed and dropout_offset replays the same mask.
 * fa_dropout_mask writes the mask itself.
 */
typedef struct {
    const void *Q;
    const void *K;
    const void *V;
    void *O;
    float *LSE;
    int64_t B, H, N_q, N_kv, d;
    float scale;
    int causal;
    int dtype;
    float descale_q, descale_k, descale_v;
    void *stream;
    int tile_override;
    float dropout_p;         /* 0 = no dropout */
    uint64_t dropout_seed;
    uint64_t dropout_offset;
} fa_fwd_args;

/* Attention forward with the full argument set (see fa_fwd_args). */
int fa_fwd_ex(const fa_fwd_args *args);

/*
 * Validates args exactly as fa_fwd_ex does, without any HIP call (usable
 * on a machine without a GPU).  Returns FA_OK or the status fa_fwd_ex would
 * return before launching.
 */
int fa_validate(const fa_fwd_args *args);

/*
 * Split-KV forward (the decode-time scheme of "Flash Attention 原理与实践"
 * section 5.1, Flash-Decoding): the key range of every (batch, head) is cut
 * into num_splits contiguous chunks that separate workgroups process in
 * parallel, each writing a float32 partial output O_s and LSE_s for its chunk
 * into the caller's workspace; a second kernel then merges the chunks with
 * the rule of "FlashAttention 与显存" plate 08 applied to whole chunks,
 * L = ln sum_s exp(L_s), O = sum_s exp(L_s - L) O_s, and writes O and LSE as
 * fa_fwd_ex does.  The result equals fa_fwd_ex's up to rounding; it pays off
 * when fa_fwd_ex's workgroups (B * H * ceil(N_q / 256) at d = 128) cannot fill
 * the GPU (few query rows, long key ranges).
 *
 * args: as for fa_fwd_ex, except that N_kv may exceed
 * FA_MAX_NKV_SINGLE_PASS (up to 2^30); dtype FA_BF16 or FA_F16 with d in
 * {64, 128, 256}, or FA_FP8_E4M3 with d = 128 (descales as for fa_fwd_ex,
 * bf16 O) (otherwise FA_ERR_VARIANT); tile_override 0 or 1.  num_splits:
 * 0 lets the library choose, otherwise an upper bound (every chunk is
 * non-empty, so fewer may be used), except that no chunk is made longer
 * than FA_MAX_NKV_SINGLE_PASS keys: more chunks are used where needed.
 * FA_ERR_SHAPE if num_splits < 0 or the grid (chunks x B x H x query
 * blocks of 128 rows) exceeds 2^31 - 1 workgroups.  workspace: device memory owned by the caller, 256-byte
 * aligned, at least fa_splitkv_workspace_bytes(args, num_splits) bytes, not
 * overlapping Q, K, V, O or LSE (FA_ERR_WORKSPACE / FA_ERR_ALIAS otherwise);
 * its contents are overwritten.  Both kernels run on args->stream, in order.
 */
int fa_fwd_splitkv(const fa_fwd_args *args, int num_splits, void *workspace,
                   int64_t workspace_bytes);

/* Size of the static device buffer behind fa_fwd_splitkv_noalloc. */
#define FA_NOALLOC_SCRATCH_BYTES (64 << 20)

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, result and kernels as
 * fa_fwd_splitkv, but the float32 partials go to a static device buffer of
 * FA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every device
 * it runs on until the process ends; the call allocates nothing.  The
 * caller still passes Q, K, V, O and LSE.  FA_ERR_SCRATCH (before any HIP
 * call) when fa_splitkv_workspace_bytes(args, num_splits) exceeds the
 * buffer: decode shapes need far less (one query row, 256 heads, d = 128: 0.5
 * MiB).  Every call on one device shares that device's buffer: calls on one
 * stream are ordered, but calls that may overlap (other streams, other host
 * threads) race on it and must be serialised by the caller.
 */
int fa_fwd_splitkv_noalloc(const fa_fwd_args *args, int num_splits);

/*
 * Workspace bytes fa_fwd_splitkv needs for these arguments and num_splits
 * (the same choice of chunks); 0 for an empty problem, -1 for arguments
 * fa_fwd_splitkv would reject.  Host-only, no HIP call.
 */
int64_t fa_splitkv_workspace_bytes(const fa_fwd_args *args, int num_splits);

/*
 * Attention backward.  "FlashAttention 与显存" plate 09 keeps only O and the
 * per-row statistic from the forward pass and recomputes S and P tile by tile
 * when the gradients are needed; this entry point does that.  For every
 * (batch, head), with S, P the forward's scores and probabilities (masked as
 * in the forward) and dO the gradient of a loss with respect to O:
 *     dV = P^T dO
 *     dP = dO V^T,   D_i = sum_c dO_ic O_ic  (= sum_j P_ij dP_ij)
 *     dS = P * (dP - D)     (elementwise; D_i broadcast along row i)
 *     dQ = scale dS K,      dK = scale dS^T Q
 * (the pages give no derivative formulas; these are the textbook gradients of
 * softmax(scale Q K^T) V).  P is recomputed from Q, K and the forward's LSE
 * as exp(scale q_i . k_j - LSE_i).
 *
 * Q, K, V, O, dO: device inputs; O and LSE must be the forward's outputs for
 * these Q, K, V, scale and causal (fa_fwd / fa_fwd_ex), dO has O's shape and
 * type.  dQ, dK, dV: device outputs with the type and layout of Q, K and V,
 * written in full; they must not overlap each other, the inputs or the
 * workspace (FA_ERR_ALIAS).  dtype: FA_BF16 or FA_F16 (else FA_ERR_DTYPE); d
 * in {64, 128, 256} (else FA_ERR_HEAD_DIM); dropout as in the forward.
 * Other rules as for fa_fwd_ex (shapes,
 * 16-byte alignment, finite scale, top-left causal mask).  B or H equal to 0
 * is a no-op; N_q = 0 writes dK = dV = 0.
 */
typedef struct {
    const void *Q;
    const void *K;
    const void *V;
    const void *O;
    const void *dO;
    const float *LSE;
    void *dQ;
    void *dK;
    void *dV;
    int64_t B, H, N_q, N_kv, d;
    float scale;
    int causal;
    int dtype;
    void *stream;   /* hipStream_t; NULL = null stream */
    float dropout_p;         /* as in fa_fwd_args; must match the forward */
    uint64_t dropout_seed;
    uint64_t dropout_offset;
} fa_bwd_args;

/*
 * Validates args exactly as fa_bwd does (without the workspace checks),
 * without any HIP call.  Returns FA_OK or the status fa_bwd would return.
 */
int fa_bwd_validate(const fa_bwd_args *args);

/*
 * Workspace bytes fa_bwd needs (float32 D and LSE log2(e), one value each
 * per query row, each array rounded up to 256 bytes); -1 for arguments
 * fa_bwd_validate rejects.  Host-only.
 */
int64_t fa_bwd_workspace_bytes(const fa_bwd_args *args);

/*
 * Attention backward (see fa_bwd_args).  workspace: device memory owned by
 * the caller, 256-byte aligned, at least fa_bwd_workspace_bytes(args) bytes,
 * not overlapping any argument buffer (FA_ERR_WORKSPACE / FA_ERR_ALIAS
 * otherwise); its contents are overwritten.  Three kernels run on
 * args->stream, in order: D from dO and O (and LSE log2(e) from LSE), then dQ
 * (one workgroup per query block), then dK and dV (one workgroup per key
 * block; at d = 256 as two kernels, dV then dK, each recomputing the scores,
 * because both accumulators do not fit one wave's registers).  No atomics: every
 * output element is written by exactly one lane, so results are bitwise
 * repeatable.
 */
int fa_bwd(const fa_bwd_args *args, void *workspace, int64_t workspace_bytes);

/*
 * The dropout keep mask of fa_fwd_args (see Dropout above) for BH = B * H
 * (batch, head) slices of N_q x N_kv: mask[(bh * N_q + i) * N_kv + j] = 1 if
 * element (i, j) of slice bh is kept, else 0 (all 1 when p8 = 0).  mask:
 * device memory of BH * N_q * N_kv bytes owned by the caller; runs on
 * stream (hipStream_t, NULL = null stream).  For tests and for callers that
 * replay the mask elsewhere.  FA_ERR_SHAPE for negative sizes,
 * FA_ERR_DROPOUT for dropout_p outside [0, 1), FA_ERR_NULL for a NULL mask
 * with a non-empty size.
 */
int fa_dropout_mask(float dropout_p, uint64_t dropout_seed, uint64_t dropout_offset, int64_t BH,
                    int64_t N_q, int64_t N_kv, uint8_t *mask, void *stream);

/* Static, never-NULL description of a status code. */
const char *fa_strerror(int status);

/*
 * Number of compiled tile variants for (dtype, d, causal), 0 if the
 * combination is unsupported.  Host-only, no HIP call.
 */
int fa_num_variants(int dtype, int64_t d, int causal);

/*
 * Static description of variant v (1-based) for (dtype, d, causal), e.g.
 * "br8x32_bc64" (8 waves of 32 query rows, 64-key tiles); "" if v is out of
 * range.  Host-only, no HIP call.
 */
const char *fa_variant_name(int dtype, int64_t d, int causal, int v);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
