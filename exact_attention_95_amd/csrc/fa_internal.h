// Internal interface between the host dispatcher (fa_api.cpp) and the kernel
// translation units (fa_fwd*.hip).  Not part of the C ABI.
#pragma once
#include <stdint.h>

namespace fa {

// Kernel arguments shared by every forward kernel.  Byte pointers; each
// (batch, head) slice is contiguous, [n_q, d] for Q/O and [n_kv, d] for K/V.
struct KParams {
    const char *q;
    const char *k;
    const char *v;
    char *o;
    float *lse;        // may be null
    int n_bh;          // B * H
    int n_q;
    int n_kv;
    int n_qblk;        // ceil(n_q / BR)
    int n_wg;          // n_bh * n_qblk
    float c;           // |scale| * log2(e) (times descale_q * descale_k for E4M3)
    float o_mul;       // factor applied to O at the end (descale_v for E4M3, else 1)
    int neg;           // 1 if scale < 0: Q is negated on load and c = |scale|*log2(e)
    // split-KV (Flash-Decoding) only: the key range of every head is cut into
    // n_split chunks of kv_split keys (the last one shorter, none empty); split
    // s writes its normalised partial output and LSE (float32) to
    // part_o[((s * n_bh + bh) * n_q + i) * d ...] and part_lse[(s * n_bh + bh) * n_q + i].
    int n_split;
    int kv_split;
    float *part_o;
    float *part_lse;
    // dropout: p8 = 0 means none; o_mul already includes 256 / (256 - p8)
    unsigned p8;
    unsigned seed_lo, seed_hi, drop_off;
};

// A compiled kernel instance and the query-block height it uses.
typedef int (*launch_fn)(const KParams &p, void *stream);

struct Variant {
    int dtype;         // fa_dtype
    int d;             // head dimension
    int causal;        // 0 or 1
    int split;         // 1: split-KV partial kernel (writes part_o / part_lse)
    int br;            // query rows per workgroup
    const char *name;
    launch_fn launch;
};

// Every compiled variant, grouped by (dtype, d, causal, split); within a
// group the first entry is the default.
const Variant *variants(int *count);

// Merge of split-KV partials into O (output dtype) and LSE; 0 on success.
int launch_merge(int dtype, int d, const KParams &p, void *stream);

// Arguments of the backward kernels.  Byte pointers; each (batch, head)
// slice is contiguous ([n_q, d] for Q, O, dO, dQ; [n_kv, d] for K, V, dK, dV).
struct BwdParams {
    const char *q;
    const char *k;
    const char *v;
    const char *o;
    const char *dout;
    const float *lse;  // forward LSE, natural log
    char *dq;
    char *dk;
    char *dv;
    float *delta;      // workspace: D_i = sum_c dO_ic O_ic, [n_bh * n_q]
    float *lse2;       // workspace: LSE_i log2(e), [n_bh * n_q]
    int n_bh;
    int n_q;
    int n_kv;
    float c;           // scale * log2(e) (signed)
    float scale;       // signed
    // dropout: p8 = 0 means none; drop_scale = 256 / (256 - p8)
    unsigned p8;
    unsigned seed_lo, seed_hi, drop_off;
    float drop_scale;
};

// The three backward launches (D, dQ, dK/dV) for one (dtype, d, causal).
typedef int (*bwd_launch_fn)(const BwdParams &p, void *stream);

struct BwdVariant {
    int dtype;
    int d;
    int causal;
    const char *name;
    bwd_launch_fn launch;
};

const BwdVariant *bwd_variants(int *count);

// Writes the dropout keep mask (bytes) of n_bh slices of n_q x n_kv; 0 on success.
int launch_dropout_mask(unsigned p8, unsigned seed_lo, unsigned seed_hi, unsigned off, int64_t n_bh,
                        int64_t n_q, int64_t n_kv, unsigned char *mask, void *stream);

}  // namespace fa
