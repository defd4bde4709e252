// Attention forward for float32 inputs on gfx950.
//
// Same decomposition and online-softmax merge as the 16-bit kernel (one
// workgroup per block of 32*NW query rows, one wave per 32 rows, key tiles
// of 32 rows, S^T = K Q^T so that each lane owns one query row), with every
// product in float32 on v_mfma_f32_32x32x2_f32: nothing is narrowed, so the
// result keeps float32 accuracy.  K and V tiles go through registers into
// padded LDS rows (row stride d+1 floats keeps the 32 rows of a K column in
// 32 different banks).
#include "fa_device.h"
#include "../../include/fa.h"

namespace fa {
namespace {

template <int D_, int NW_, bool CAUSAL_>
struct Cfg32 {
    static constexpr int D = D_, NW = NW_, NT = NW * 64, BR = 32 * NW, BC = 32;
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr int LD = D + 1;              // padded LDS row, floats
    static constexpr int KS = D / 2;              // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;
    static constexpr float TAU = 8.0f;
};

template <class C>
__global__ __launch_bounds__(C::NT) void fwd32_kernel(KParams p) {
    __shared__ float ks_lds[C::BC * C::LD];
    __shared__ float vs_lds[C::BC * C::LD];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = wave_id();
    const int h = lane >> 5;
    const int l32 = lane & 31;

    const int bid = xcd_remap(blockIdx.x, p.n_wg);
    const int bh = bid / p.n_qblk;
    int qb = bid - bh * p.n_qblk;
    if (C::CAUSAL) qb = p.n_qblk - 1 - qb;
    const int q0 = qb * C::BR;
    const int wq0 = q0 + w * 32;
    const int qi = wq0 + l32;
    const int n_q = p.n_q, n_kv = p.n_kv;
    const float *qh = (const float *)p.q + (int64_t)bh * n_q * C::D;
    const float *kh = (const float *)p.k + (int64_t)bh * n_kv * C::D;
    const float *vh = (const float *)p.v + (int64_t)bh * n_kv * C::D;

    int ntile = (n_kv + C::BC - 1) / C::BC;
    if (C::CAUSAL) ntile = min(ntile, min(q0 + C::BR - 1, n_q - 1) / C::BC + 1);
    const int wq_last = min(wq0 + 31, n_q - 1);
    const bool wave_has_rows = wq0 < n_q;

    // Q^T operand: lane holds Q[qi][2ks + h] for every k-step.
    float qf[C::KS];
    {
        const float *qrow = qh + (int64_t)(qi < n_q ? qi : n_q - 1) * C::D;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[ks] = p.neg ? -qrow[2 * ks + h] : qrow[2 * ks + h];
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = (f32x16){};
    float m_use = kNegInf, l_acc = 0.f;
    const float c = p.c;

    for (int t = 0; t < ntile; ++t) {
        const int t0 = t * C::BC;
        __syncthreads();  // previous tile fully consumed
        for (int idx = tid; idx < C::BC * (C::D / 4); idx += C::NT) {
            const int r = idx / (C::D / 4), c4 = idx % (C::D / 4);
            int gr = t0 + r;
            gr = gr < n_kv ? gr : n_kv - 1;
            const f32x4 kv = *(const f32x4 *)(kh + (int64_t)gr * C::D + 4 * c4);
            const f32x4 vv = *(const f32x4 *)(vh + (int64_t)gr * C::D + 4 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks_lds[r * C::LD + 4 * c4 + e] = kv[e];
                vs_lds[r * C::LD + 4 * c4 + e] = vv[e];
            }
        }
        __syncthreads();
        if (!wave_has_rows || (C::CAUSAL && t0 > wq_last)) continue;

        // S^T = K Q^T
        f32x16 s = (f32x16){};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_lds[l32 * C::LD + 2 * ks + h], qf[ks], s, 0, 0, 0);

        const bool need_mask = (t0 + C::BC > n_kv) || (C::CAUSAL && t0 + C::BC - 1 > wq0);
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = t0 + 8 * (r >> 2) + 4 * h + (r & 3);
                const bool vis = key < n_kv && (!C::CAUSAL || key <= qi);
                s[r] = vis ? s[r] : kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = (mx == kNegInf) ? kNegInf : mx * c;
        if (__any(mt > m_use + C::TAU)) {
            const float m_new = fmaxf(m_use, mt);
            const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_use - m_new);
            l_acc *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
            m_use = m_new;
        }
        const float mref = (m_use == kNegInf) ? 0.f : m_use;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mref));
            if (need_mask) e = (s[r] == kNegInf) ? 0.f : e;
            s[r] = e;
            l_acc += e;
        }
        // O^T += V^T P^T; register r of S^T holds key 8(r/4) + 4h + r%4.
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * h + (r & 3);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_lds[key * C::LD + 32 * db + l32], s[r], o[db], 0, 0, 0);
            }
    }

    if (qi >= n_q) return;
    const float l_tot = l_acc + __shfl_xor(l_acc, 32);
    const float inv = p.o_mul / l_tot;
    float *orow = (float *)p.o + ((int64_t)bh * n_q + qi) * C::D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            f32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = o[db][4 * jj + e] * inv;
            *(f32x4 *)(orow + 32 * db + 8 * jj + 4 * h) = out;
        }
    if (p.lse && h == 0) p.lse[(int64_t)bh * n_q + qi] = (m_use + __log2f(l_tot)) * kLn2;
}

template <class C>
int launch32(const KParams &p, void *stream) {
    hipLaunchKernelGGL(fwd32_kernel<C>, dim3(p.n_wg), dim3(C::NT), 0, (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

#define FA_V32(D, NW, CAUSAL) Variant{FA_F32, D, CAUSAL, 0, 32 * NW, "br" #NW "x32_bc32", &launch32<Cfg32<D, NW, CAUSAL>>}

// Host-side table of the compiled float32 variants.
const Variant *variants32(int *count) {
    static const Variant table[] = {
        FA_V32(64, 4, 0),  FA_V32(64, 4, 1),  FA_V32(128, 4, 0),
        FA_V32(128, 4, 1), FA_V32(256, 4, 0), FA_V32(256, 4, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
