/*
 * fa_probe.h -- measurement probes of libfa.so (not part of the attention
 * operation).
 *
 * The attention kernels are bound by the matrix cores, with the softmax
 * exponentials on the vector unit beside them ("FlashAttention算子优化"
 * section 3 and "FlashAttention 与显存" plate 11 put the time of the fused
 * kernel in its two matrix products and in its exponentials).  To state how
 * close a kernel gets, these probes measure on the device itself what the
 * published peaks only assume: the sustained MFMA rate of each input type,
 * the rate of v_exp_f32 and of a plain fp32 FMA, and the shader clock while
 * they run.  Each kind of fa_probe is one kernel of register-only loops with
 * many independent dependency chains per wave.  The split-KV decode is bound
 * by HBM instead; fa_probe_hbm_read measures the read rate it is held
 * against.
 *
 * Memory.  sink and clocks are device buffers owned by the caller:
 * sink holds n_wg * 256 floats (one result per thread, written so that the
 * compiler keeps the loop), clocks holds n_wg * 4 * 2 uint64 values (per wave
 * w of workgroup g, clocks[2 (4 g + w)] = shader-clock cycles and
 * clocks[2 (4 g + w) + 1] = constant-rate wall-clock ticks spent in the loop;
 * clocks may be NULL).  Workgroups have 256 threads (4 waves).  The call is
 * asynchronous on stream (hipStream_t, NULL = null stream).
 *
 * fa_probe_hbm_read measures the other bound, HBM: a streaming read of the
 * caller's device buffer buf (bytes, a multiple of 16, 16-byte aligned;
 * read only).  Its n_wg workgroups of 256 threads read the buffer's 16-byte
 * chunks grid-stride, eight loads in flight per thread, and each thread
 * stores the low 16 bits of the xor of the 32-bit words it read (as an exact
 * float) into sink[n_wg * 256].  bytes / (time of the call) is the read rate
 * that a kernel bound by HBM reads is compared with.
 *
 * Errors.  0 (FA_OK); FA_ERR_SHAPE for n_wg outside [1, 2^20] or iters outside
 * [1, 2^30] (fa_probe_hbm_read: bytes not a positive multiple of 16); FA_ERR_NULL
 * for a NULL sink or buf; FA_ERR_ALIGN for a sink not 4-byte, clocks not
 * 8-byte or buf not 16-byte aligned; FA_ERR_DTYPE for an unknown kind;
 * FA_ERR_DEVICE without a gfx950 device; FA_ERR_LAUNCH if the launch fails.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_PROBE_MFMA_BF16 = 0,  /* v_mfma_f32_32x32x16_bf16 */
    FA_PROBE_MFMA_F16 = 1,   /* v_mfma_f32_32x32x16_f16 */
    FA_PROBE_MFMA_FP8 = 2,   /* v_mfma_f32_32x32x64_f8f6f4 (E4M3 operands) */
    FA_PROBE_MFMA_F32 = 3,   /* v_mfma_f32_32x32x2_f32 */
    FA_PROBE_EXP = 4,        /* v_exp_f32 */
    FA_PROBE_FMA = 5         /* v_fma_f32 */
} fa_probe_kind;

/* Runs probe `kind` on n_wg workgroups, each wave looping iters times. */
int fa_probe(int kind, int64_t n_wg, int64_t iters, float *sink, uint64_t *clocks, void *stream);

/* Streaming read of bytes of buf by n_wg workgroups (see above). */
int fa_probe_hbm_read(const void *buf, int64_t bytes, int64_t n_wg, float *sink, void *stream);

/*
 * Work of one loop iteration of one wave: FLOPs for the MFMA probes (2 per
 * multiply-add), lane operations for FA_PROBE_EXP and FA_PROBE_FMA (64 lanes x
 * the instructions issued); 0 for an unknown kind.  Host-only.
 */
double fa_probe_work_per_iter(int kind);

/*
 * Rate of the constant wall clock that clocks[] counts, in kHz, for the
 * current device; 0 if it cannot be read.
 */
int64_t fa_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
