// Host side of the C ABI declared in include/fa.h: argument validation
// (pure host code, no HIP call), variant selection and kernel launch.
#include <hip/hip_runtime_api.h>

#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {
const Variant *variants16(int *count);
const Variant *variants32(int *count);
const Variant *variants8(int *count);

const Variant *variants(int *count) {
    static std::vector<Variant> all = [] {
        std::vector<Variant> v;
        const Variant *(*parts[])(int *) = {variants32, variants16, variants8};
        for (auto part : parts) {
            int n = 0;
            const Variant *t = part(&n);
            v.insert(v.end(), t, t + n);
        }
        return v;
    }();
    *count = (int)all.size();
    return all.data();
}
}  // namespace fa

namespace {

const fa::Variant *find_variant(int dtype, int64_t d, int causal, int which, int split = 0) {
    int n = 0;
    const fa::Variant *t = fa::variants(&n);
    int seen = 0;
    for (int i = 0; i < n; ++i) {
        if (t[i].dtype == dtype && t[i].d == d && t[i].causal == (causal ? 1 : 0) &&
            t[i].split == split) {
            ++seen;
            if (seen == (which <= 0 ? 1 : which)) return &t[i];
        }
    }
    return nullptr;
}

int in_size(int dtype) { return dtype == FA_F32 ? 4 : dtype == FA_FP8_E4M3 ? 1 : 2; }
int out_size(int dtype) { return dtype == FA_F32 ? 4 : 2; }

bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
    if (na <= 0 || nb <= 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// float32 value of |scale| * log2(e) [* descale_q * descale_k], rounded once.
double score_factor(const fa_fwd_args *a) {
    double c = fabs((double)a->scale) * 1.4426950408889634;
    if (a->dtype == FA_FP8_E4M3) c *= (double)a->descale_q * (double)a->descale_k;
    return c;
}

const int64_t kMaxRows = (int64_t)1 << 30;

// Dropout probability quantised to p8 / 256 (0 = no dropout); -1 if p is not
// in [0, 1).
int dropout_p8(float p) {
    if (!(p >= 0.0f && p < 1.0f)) return -1;
    double x = floor((double)p * 256.0 + 0.5);
    return (int)(x > 255.0 ? 255.0 : x);
}

}  // namespace

namespace {
// Checks shared by the single-pass and split-KV forwards (everything but the
// single-pass key-range limit).
int validate_fwd_common(const fa_fwd_args *a) {
    if (!a) return FA_ERR_NULL;
    if (a->dtype < FA_F32 || a->dtype > FA_FP8_E4M3) return FA_ERR_DTYPE;
    if (a->d != 64 && a->d != 128 && a->d != 256) return FA_ERR_HEAD_DIM;
    if (a->B < 0 || a->H < 0 || a->N_q < 0 || a->N_kv < 1) return FA_ERR_SHAPE;
    if (a->N_q > kMaxRows || a->N_kv > kMaxRows) return FA_ERR_SHAPE;
    if (a->B > 0 && a->H > INT32_MAX / a->B) return FA_ERR_SHAPE;
    const int64_t bh = a->B * a->H;
    // every tensor byte count must fit int64 and the grid must fit 2^31 workgroups
    if (bh > 0 && (a->N_q > INT64_MAX / 4 / a->d / bh || a->N_kv > INT64_MAX / 4 / a->d / bh))
        return FA_ERR_SHAPE;
    if (bh > 0 && (a->N_q + 31) / 32 > INT32_MAX / bh) return FA_ERR_SHAPE;
    if (!isfinite(a->scale)) return FA_ERR_SCALE;
    if (a->dtype == FA_FP8_E4M3 &&
        (!isfinite(a->descale_q) || !isfinite(a->descale_k) || !isfinite(a->descale_v)))
        return FA_ERR_SCALE;
    if (!isfinite((float)score_factor(a))) return FA_ERR_SCALE;
    const int p8 = dropout_p8(a->dropout_p);
    if (p8 < 0) return FA_ERR_DROPOUT;
    if (p8 > 0 && a->dtype != FA_BF16 && a->dtype != FA_F16) return FA_ERR_DROPOUT;
    if (fa_num_variants(a->dtype, a->d, a->causal) == 0) return FA_ERR_HEAD_DIM;
    if (a->tile_override < 0 || a->tile_override > fa_num_variants(a->dtype, a->d, a->causal))
        return FA_ERR_VARIANT;
    if (bh == 0 || a->N_q == 0) return FA_OK;  // nothing to read or write
    if (!a->Q || !a->K || !a->V || !a->O) return FA_ERR_NULL;
    if (((uintptr_t)a->Q | (uintptr_t)a->K | (uintptr_t)a->V | (uintptr_t)a->O) & 15)
        return FA_ERR_ALIGN;
    if ((uintptr_t)a->LSE & 3) return FA_ERR_ALIGN;
    const int64_t qb = bh * a->N_q * a->d * in_size(a->dtype);
    const int64_t kb = bh * a->N_kv * a->d * in_size(a->dtype);
    const int64_t ob = bh * a->N_q * a->d * out_size(a->dtype);
    const int64_t lb = a->LSE ? bh * a->N_q * 4 : 0;
    if (overlap(a->O, ob, a->Q, qb) || overlap(a->O, ob, a->K, kb) || overlap(a->O, ob, a->V, kb))
        return FA_ERR_ALIAS;
    if (lb && (overlap(a->LSE, lb, a->Q, qb) || overlap(a->LSE, lb, a->K, kb) ||
               overlap(a->LSE, lb, a->V, kb) || overlap(a->LSE, lb, a->O, ob)))
        return FA_ERR_ALIAS;
    return FA_OK;
}
}  // namespace

extern "C" int fa_validate(const fa_fwd_args *a) {
    const int st = validate_fwd_common(a);
    if (st != FA_OK) return st;
    // the float32 running sums of one pass hold ordinary rounding up to this
    // many keys per row (include/fa.h, "Very long key ranges")
    if (a->N_kv > FA_MAX_NKV_SINGLE_PASS) return FA_ERR_LONG_KV;
    return FA_OK;
}

namespace {
int count_variants(int dtype, int64_t d, int causal, int split) {
    int n = 0, count = 0;
    const fa::Variant *t = fa::variants(&n);
    for (int i = 0; i < n; ++i)
        if (t[i].dtype == dtype && t[i].d == d && t[i].causal == (causal ? 1 : 0) && t[i].split == split)
            ++count;
    return count;
}
}  // namespace

extern "C" int fa_num_variants(int dtype, int64_t d, int causal) {
    return count_variants(dtype, d, causal, 0);
}

extern "C" const char *fa_variant_name(int dtype, int64_t d, int causal, int v) {
    if (v < 1) return "";
    const fa::Variant *x = find_variant(dtype, d, causal, v);
    return x ? x->name : "";
}

extern "C" const char *fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (B, H, N_q < 0, N_kv < 1, or size overflow)";
        case FA_ERR_HEAD_DIM: return "unsupported head dimension for this dtype";
        case FA_ERR_DTYPE: return "unknown dtype";
        case FA_ERR_ALIGN: return "misaligned pointer (Q, K, V, O need 16 bytes, LSE 4)";
        case FA_ERR_SCALE: return "scale or descale not finite (also scale*log2(e)*descales in float32)";
        case FA_ERR_ALIAS: return "output overlaps an input or the other output";
        case FA_ERR_DEVICE: return "no usable gfx950 device";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_VARIANT: return "no compiled variant for this problem (or tile_override out of range)";
        case FA_ERR_WORKSPACE: return "workspace NULL, misaligned or too small";
        case FA_ERR_DROPOUT: return "dropout_p outside [0, 1), or dropout not supported here (fp16/bf16 only, not split-KV)";
        case FA_ERR_LONG_KV: return "N_kv above the single-pass limit of 2^20 keys per row; use fa_fwd_splitkv";
        case FA_ERR_SCRATCH: return "split-KV partials exceed the 64 MiB static scratch buffer of fa_fwd_splitkv_noalloc; use fa_fwd_splitkv with a workspace";
        default: return "unknown status";
    }
}

namespace {

// 1 if the current device is a gfx950, cached per device ordinal.
int device_ok() {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1, -1);
    if (cache[dev] < 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
        cache[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    }
    return cache[dev];
}

}  // namespace

extern "C" int fa_fwd_ex(const fa_fwd_args *a) {
    const int st = fa_validate(a);
    if (st != FA_OK) return st;
    if (a->B * a->H == 0 || a->N_q == 0) return FA_OK;
    if (!device_ok()) return FA_ERR_DEVICE;
    const fa::Variant *v = find_variant(a->dtype, a->d, a->causal, a->tile_override);
    if (!v) return FA_ERR_VARIANT;
    fa::KParams p;
    p.q = (const char *)a->Q;
    p.k = (const char *)a->K;
    p.v = (const char *)a->V;
    p.o = (char *)a->O;
    p.lse = a->LSE;
    p.n_bh = (int)(a->B * a->H);
    p.n_q = (int)a->N_q;
    p.n_kv = (int)a->N_kv;
    p.n_qblk = (int)((a->N_q + v->br - 1) / v->br);
    p.n_wg = p.n_bh * p.n_qblk;
    // c >= FLT_MIN keeps c > 0, so a masked score (-inf) always gives P = 0; for
    // |scale * log2 e| below FLT_MIN every exp2 argument rounds to the same
    // value as with the exact c (|s c| < 2^-25 gives exp2 = 1).
    p.c = fmaxf((float)score_factor(a), FLT_MIN);
    p.o_mul = a->dtype == FA_FP8_E4M3 ? a->descale_v : 1.0f;
    p.neg = a->scale < 0 ? 1 : 0;
    p.n_split = 1;
    p.kv_split = (int)a->N_kv;
    p.part_o = nullptr;
    p.part_lse = nullptr;
    p.p8 = (unsigned)dropout_p8(a->dropout_p);
    p.seed_lo = (unsigned)a->dropout_seed;
    p.seed_hi = (unsigned)(a->dropout_seed >> 32);
    p.drop_off = (unsigned)a->dropout_offset;
    if (p.p8 != 0) p.o_mul = (float)(256.0 / (256.0 - p.p8));
    (void)hipGetLastError();  // clear a stale error so it is not reported as ours
    return v->launch(p, a->stream) == 0 ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE, int64_t B,
                      int64_t H, int64_t N_q, int64_t N_kv, int64_t d, float scale, int causal,
                      int dtype) {
    fa_fwd_args a;
    memset(&a, 0, sizeof a);
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.O = O;
    a.LSE = LSE;
    a.B = B;
    a.H = H;
    a.N_q = N_q;
    a.N_kv = N_kv;
    a.d = d;
    a.scale = scale;
    a.causal = causal;
    a.dtype = dtype;
    a.descale_q = a.descale_k = a.descale_v = 1.0f;
    a.stream = nullptr;
    a.tile_override = 0;
    return fa_fwd_ex(&a);
}

namespace {

// Chunking of the key range for split-KV: chunks of a whole number of 64-key
// tiles, none empty.  Returns the number of chunks and sets *kv_split.
const int kSplitTile = 64, kSplitRows = 128;  // key tile and query block of the split kernels
const int64_t kMaxChunkTiles = FA_MAX_NKV_SINGLE_PASS / kSplitTile;

int plan_splits(const fa_fwd_args *a, int num_splits, int *kv_split) {
    const int64_t tiles = (a->N_kv + kSplitTile - 1) / kSplitTile;
    const int64_t blocks = a->B * a->H * ((a->N_q + kSplitRows - 1) / kSplitRows);
    int64_t want = num_splits;
    if (want == 0) {
        // about 1024 workgroups in flight (4 per CU), at least 4 tiles per chunk
        want = (1024 + blocks - 1) / blocks;
        const int64_t cap = tiles / 4 > 0 ? tiles / 4 : 1;
        want = want < cap ? want : cap;
    }
    if (want > tiles) want = tiles;
    if (want > 4096) want = 4096;
    // no chunk longer than the single-pass limit (float32 running sums)
    const int64_t min_chunks = (tiles + kMaxChunkTiles - 1) / kMaxChunkTiles;
    if (want < min_chunks) want = min_chunks;
    if (want < 1) want = 1;
    const int64_t per = (tiles + want - 1) / want;
    *kv_split = (int)(per * kSplitTile);
    return (int)((a->N_kv + *kv_split - 1) / *kv_split);
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Status of the split-KV arguments before the workspace is looked at.
int validate_split(const fa_fwd_args *a, int num_splits) {
    const int st = validate_fwd_common(a);
    if (st != FA_OK) return st;
    if (num_splits < 0) return FA_ERR_SHAPE;
    if (dropout_p8(a->dropout_p) != 0) return FA_ERR_DROPOUT;
    const int nv = count_variants(a->dtype, a->d, a->causal, 1);
    if (nv == 0) return FA_ERR_VARIANT;
    if (a->tile_override > nv) return FA_ERR_VARIANT;
    if (a->B * a->H == 0 || a->N_q == 0) return FA_OK;
    // the grid (chunks x heads x query blocks) must fit 2^31 - 1 workgroups,
    // and the float32 partials (chunks x rows x (d + 1) x 4 bytes) int64
    int kv_split = 0;
    const int64_t n = plan_splits(a, num_splits, &kv_split);
    const int64_t blocks = a->B * a->H * ((a->N_q + kSplitRows - 1) / kSplitRows);
    if (blocks > INT32_MAX / n) return FA_ERR_SHAPE;
    const int64_t rows = a->B * a->H * a->N_q;
    if (rows > INT64_MAX / 8 / n / (a->d + 1)) return FA_ERR_SHAPE;
    return FA_OK;
}

}  // namespace

extern "C" int64_t fa_splitkv_workspace_bytes(const fa_fwd_args *a, int num_splits) {
    if (validate_split(a, num_splits) != FA_OK) return -1;
    if (a->B * a->H == 0 || a->N_q == 0) return 0;
    int kv_split = 0;
    const int64_t n = plan_splits(a, num_splits, &kv_split);
    const int64_t rows = a->B * a->H * a->N_q;
    return align256(n * rows * a->d * 4) + align256(n * rows * 4);
}

extern "C" int fa_fwd_splitkv(const fa_fwd_args *a, int num_splits, void *workspace,
                              int64_t workspace_bytes) {
    const int st = validate_split(a, num_splits);
    if (st != FA_OK) return st;
    if (a->B * a->H == 0 || a->N_q == 0) return FA_OK;
    const int64_t need = fa_splitkv_workspace_bytes(a, num_splits);
    if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < need) return FA_ERR_WORKSPACE;
    const int64_t bh = a->B * a->H;
    const int64_t qb = bh * a->N_q * a->d * in_size(a->dtype);
    const int64_t kb = bh * a->N_kv * a->d * in_size(a->dtype);
    const int64_t ob = bh * a->N_q * a->d * out_size(a->dtype);
    const int64_t lb = a->LSE ? bh * a->N_q * 4 : 0;
    if (overlap(workspace, need, a->Q, qb) || overlap(workspace, need, a->K, kb) ||
        overlap(workspace, need, a->V, kb) || overlap(workspace, need, a->O, ob) ||
        (lb && overlap(workspace, need, a->LSE, lb)))
        return FA_ERR_ALIAS;
    if (!device_ok()) return FA_ERR_DEVICE;
    const fa::Variant *v = find_variant(a->dtype, a->d, a->causal, a->tile_override, 1);
    if (!v) return FA_ERR_VARIANT;
    int kv_split = 0;
    const int n_split = plan_splits(a, num_splits, &kv_split);
    const int64_t rows = bh * a->N_q;
    fa::KParams p;
    p.q = (const char *)a->Q;
    p.k = (const char *)a->K;
    p.v = (const char *)a->V;
    p.o = (char *)a->O;
    p.lse = a->LSE;
    p.n_bh = (int)bh;
    p.n_q = (int)a->N_q;
    p.n_kv = (int)a->N_kv;
    p.n_qblk = (int)((a->N_q + v->br - 1) / v->br);
    p.n_wg = n_split * p.n_bh * p.n_qblk;
    p.c = fmaxf((float)score_factor(a), FLT_MIN);
    p.o_mul = a->dtype == FA_FP8_E4M3 ? a->descale_v : 1.0f;  // applied by the merge
    p.neg = a->scale < 0 ? 1 : 0;
    p.n_split = n_split;
    p.kv_split = kv_split;
    p.p8 = 0;
    p.seed_lo = p.seed_hi = p.drop_off = 0;
    p.part_o = (float *)workspace;
    p.part_lse = (float *)((char *)workspace + align256((int64_t)n_split * rows * a->d * 4));
    (void)hipGetLastError();
    if (v->launch(p, a->stream) != 0) return FA_ERR_LAUNCH;
    return fa::launch_merge(a->dtype, (int)a->d, p, a->stream) == 0 ? FA_OK : FA_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Backward.

namespace {

const fa::BwdVariant *find_bwd(int dtype, int64_t d, int causal) {
    int n = 0;
    const fa::BwdVariant *t = fa::bwd_variants(&n);
    for (int i = 0; i < n; ++i)
        if (t[i].dtype == dtype && t[i].d == d && t[i].causal == (causal ? 1 : 0)) return &t[i];
    return nullptr;
}

const int kBwdKeyBlock = 128;  // keys per workgroup of the dK/dV kernel

}  // namespace

extern "C" int fa_bwd_validate(const fa_bwd_args *a) {
    if (!a) return FA_ERR_NULL;
    if (a->dtype != FA_BF16 && a->dtype != FA_F16) return FA_ERR_DTYPE;
    if (a->d != 64 && a->d != 128 && a->d != 256) return FA_ERR_HEAD_DIM;
    if (a->B < 0 || a->H < 0 || a->N_q < 0 || a->N_kv < 1) return FA_ERR_SHAPE;
    if (a->N_q > kMaxRows || a->N_kv > kMaxRows) return FA_ERR_SHAPE;
    if (a->B > 0 && a->H > INT32_MAX / a->B) return FA_ERR_SHAPE;
    const int64_t bh = a->B * a->H;
    if (bh > 0 && (a->N_q > INT64_MAX / 4 / a->d / bh || a->N_kv > INT64_MAX / 4 / a->d / bh))
        return FA_ERR_SHAPE;
    if (bh > 0 && ((a->N_q + 31) / 32 > INT32_MAX / bh || (a->N_kv + kBwdKeyBlock - 1) / kBwdKeyBlock > INT32_MAX / bh))
        return FA_ERR_SHAPE;
    if (!isfinite(a->scale) || !isfinite((float)((double)a->scale * 1.4426950408889634)))
        return FA_ERR_SCALE;
    const int p8 = dropout_p8(a->dropout_p);
    if (p8 < 0) return FA_ERR_DROPOUT;
    if (!find_bwd(a->dtype, a->d, a->causal)) return FA_ERR_HEAD_DIM;
    if (bh == 0) return FA_OK;  // nothing to read or write
    if (!a->K || !a->V || !a->dK || !a->dV) return FA_ERR_NULL;
    const bool rows = a->N_q > 0;
    if (rows && (!a->Q || !a->O || !a->dO || !a->LSE || !a->dQ)) return FA_ERR_NULL;
    uintptr_t al = (uintptr_t)a->K | (uintptr_t)a->V | (uintptr_t)a->dK | (uintptr_t)a->dV;
    if (rows) al |= (uintptr_t)a->Q | (uintptr_t)a->O | (uintptr_t)a->dO | (uintptr_t)a->dQ;
    if (al & 15) return FA_ERR_ALIGN;
    if (rows && ((uintptr_t)a->LSE & 3)) return FA_ERR_ALIGN;
    const int64_t qb = rows ? bh * a->N_q * a->d * 2 : 0;
    const int64_t kb = bh * a->N_kv * a->d * 2;
    const int64_t lb = rows ? bh * a->N_q * 4 : 0;
    const void *outs[3] = {a->dQ, a->dK, a->dV};
    const int64_t osz[3] = {qb, kb, kb};
    const void *ins[6] = {a->Q, a->K, a->V, a->O, a->dO, a->LSE};
    const int64_t isz[6] = {qb, kb, kb, qb, qb, lb};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], osz[i], ins[j], isz[j])) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], osz[i], outs[j], osz[j])) return FA_ERR_ALIAS;
    }
    return FA_OK;
}

extern "C" int64_t fa_bwd_workspace_bytes(const fa_bwd_args *a) {
    if (fa_bwd_validate(a) != FA_OK) return -1;
    return 2 * align256(a->B * a->H * a->N_q * 4);  // D, then LSE log2(e)
}

extern "C" int fa_bwd(const fa_bwd_args *a, void *workspace, int64_t workspace_bytes) {
    const int st = fa_bwd_validate(a);
    if (st != FA_OK) return st;
    const int64_t bh = a->B * a->H;
    if (bh == 0) return FA_OK;
    const int64_t need = fa_bwd_workspace_bytes(a);
    if (need > 0) {
        if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < need) return FA_ERR_WORKSPACE;
        const int64_t qb = bh * a->N_q * a->d * 2;
        const int64_t kb = bh * a->N_kv * a->d * 2;
        const void *bufs[9] = {a->Q, a->K, a->V, a->O, a->dO, a->LSE, a->dQ, a->dK, a->dV};
        const int64_t sz[9] = {qb, kb, kb, qb, qb, bh * a->N_q * 4, qb, kb, kb};
        for (int i = 0; i < 9; ++i)
            if (overlap(workspace, need, bufs[i], sz[i])) return FA_ERR_ALIAS;
    }
    if (!device_ok()) return FA_ERR_DEVICE;
    const fa::BwdVariant *v = find_bwd(a->dtype, a->d, a->causal);
    if (!v) return FA_ERR_HEAD_DIM;
    fa::BwdParams p;
    p.q = (const char *)a->Q;
    p.k = (const char *)a->K;
    p.v = (const char *)a->V;
    p.o = (const char *)a->O;
    p.dout = (const char *)a->dO;
    p.lse = a->LSE;
    p.dq = (char *)a->dQ;
    p.dk = (char *)a->dK;
    p.dv = (char *)a->dV;
    p.delta = (float *)workspace;
    p.lse2 = (float *)((char *)workspace + need / 2);
    p.n_bh = (int)bh;
    p.n_q = (int)a->N_q;
    p.n_kv = (int)a->N_kv;
    p.c = (float)((double)a->scale * 1.4426950408889634);
    p.scale = a->scale;
    p.p8 = (unsigned)dropout_p8(a->dropout_p);
    p.seed_lo = (unsigned)a->dropout_seed;
    p.seed_hi = (unsigned)(a->dropout_seed >> 32);
    p.drop_off = (unsigned)a->dropout_offset;
    p.drop_scale = p.p8 ? (float)(256.0 / (256.0 - p.p8)) : 1.0f;
    (void)hipGetLastError();
    return v->launch(p, a->stream) == 0 ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" int fa_dropout_mask(float dropout_p, uint64_t dropout_seed, uint64_t dropout_offset, int64_t BH,
                               int64_t N_q, int64_t N_kv, uint8_t *mask, void *stream) {
    if (BH < 0 || N_q < 0 || N_kv < 0) return FA_ERR_SHAPE;
    if (BH > INT32_MAX || N_q > kMaxRows || N_kv > kMaxRows) return FA_ERR_SHAPE;
    if (BH > 0 && N_q > 0 && N_kv > INT64_MAX / BH / N_q) return FA_ERR_SHAPE;
    const int p8 = dropout_p8(dropout_p);
    if (p8 < 0) return FA_ERR_DROPOUT;
    if (BH * N_q * N_kv == 0) return FA_OK;
    if (!mask) return FA_ERR_NULL;
    if (!device_ok()) return FA_ERR_DEVICE;
    (void)hipGetLastError();
    return fa::launch_dropout_mask((unsigned)p8, (unsigned)dropout_seed, (unsigned)(dropout_seed >> 32),
                                   (unsigned)dropout_offset, BH, N_q, N_kv, mask, stream) == 0
               ? FA_OK
               : FA_ERR_LAUNCH;
}
