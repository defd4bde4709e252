// Attention forward for 16-bit inputs (bf16, fp16) on gfx950.
//
// Work decomposition ("FlashAttention算子优化" section 2, v2 loop order;
// "FlashAttention 与显存" plates 07 and 11): one workgroup per (batch*head,
// block of BR = 32*NW query rows); the workgroup streams the key/value rows
// in tiles of BC through LDS; each of its NW waves owns 32 query rows and
// carries their running max m, running sum l and output accumulator in
// registers.  Per tile and wave:
//
//   S^T = K_tile Q^T             v_mfma_f32_32x32x16_{bf16,f16}; the
//                                accumulator holds one query per lane, so
//                                the row max/sum are in-lane reductions plus
//                                one exchange between the two half-waves
//   m, l, O rescale              online softmax merge (plate 08); the stored
//                                reference max is only raised when the tile
//                                max exceeds it by more than 2^TAU, which
//                                keeps P <= 2^TAU and changes nothing but
//                                rounding
//   P = exp2(S*c - m)            c = scale*log2(e); v_exp_f32
//   O^T += V_tile^T P^T          V^T operand read with ds_read_b64_tr_b16
//
// and after the last tile O = O_acc / l, LSE = (m + log2 l) ln 2 (v2 defers
// the division to the end).  K/V tiles are double-buffered in LDS and filled
// with direct global->LDS copies (global_load_lds_dwordx4) one tile ahead.
// The causal variant stops at the diagonal tile (plate 07: the mask is fused
// into the kernel) and masks only the tiles that straddle it.
#include "fa_device.h"
#include "../../include/fa.h"

namespace fa {
namespace {

template <typename T> struct Mma16;
template <> struct Mma16<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma16<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <typename T_, int D_, int NW_, int BC_, bool CAUSAL_>
struct Cfg {
    typedef T_ T;
    static constexpr int D = D_, NW = NW_, BC = BC_, NT = NW * 64, BR = 32 * NW;
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr int RB = D * 2;                      // LDS / global row bytes
    static constexpr int NC = RB / 16;                    // 16-byte chunks per row
    static constexpr int RPB = RB >= 256 ? 1 : 256 / RB;  // rows per 256-byte bank window
    static constexpr int KX = (NC < 16 ? NC : 16) - 1;    // K chunk swizzle mask
    static constexpr int VX = (NC / 4 < 4 ? NC / 4 : 4) - 1;  // V swizzle mask (4-chunk units)
    static constexpr int TILE = BC * RB;                  // bytes of one K or V tile
    static constexpr int STAGE = 2 * TILE;
    static constexpr int LDS = 2 * STAGE;
    static constexpr int KS = D / 16;                     // k-steps of S^T = K Q^T
    static constexpr int KB = BC / 32;                    // 32-key blocks per tile
    static constexpr int DB = D / 32;                     // 32-row blocks of O^T
    static constexpr int LDI = TILE / (1024 * NW);        // copy instructions per wave per tensor
    static constexpr float TAU = 8.0f;
    static_assert(TILE % (1024 * NW) == 0, "tile must split into whole wave copies");
    static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// K rows: chunk c of row r is stored at chunk c ^ kswz(r).  With this XOR,
// 16 lanes reading the same logical chunk of 16 consecutive rows touch 16
// different 16-byte bank groups.
template <class C> __device__ __forceinline__ int kswz(int r) { return (r / C::RPB) & C::KX; }
// V rows: chunk c of row r is stored at chunk c ^ vswz(r); the transposed
// reads cover 4 consecutive rows x 4 chunks per half-wave, which this XOR
// spreads over 16 different bank groups.
template <class C> __device__ __forceinline__ int vswz(int r) { return 4 * ((r / C::RPB) & C::VX); }

// Issues the direct-to-LDS copies of key/value rows [t0, t0 + BC) of one
// head into one LDS stage.  Rows past n_kv are clamped to the last row (their
// scores are masked, their P entries are zero).
template <class C>
__device__ __forceinline__ void load_tile(const char *kh, const char *vh, int t0, int n_kv,
                                          char *stage, int w, int lane) {
#pragma unroll
    for (int i = 0; i < C::LDI; ++i) {
        const int cb = (i * C::NW + w) * 64;       // first chunk of this wave's copy
        const int chunk = cb + lane;
        const int r = chunk / C::NC;
        const int pc = chunk % C::NC;               // physical chunk in the LDS row
        int gr = t0 + r;
        gr = gr < n_kv ? gr : n_kv - 1;
        const int64_t rowoff = (int64_t)gr * C::RB;
        copy16_to_lds(kh + rowoff + 16 * (pc ^ kswz<C>(r)), stage + cb * 16);
        copy16_to_lds(vh + rowoff + 16 * (pc ^ vswz<C>(r)), stage + C::TILE + cb * 16);
    }
}

template <class C>
__global__ __launch_bounds__(C::NT) void fwd16_kernel(KParams p) {
    typedef typename C::T T;
    typedef Mma16<T> M;
    typedef typename M::v8 v8;
    typedef typename M::v4 v4;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

    const int lane = lane_id();
    const int w = wave_id();
    const int h = lane >> 5;     // half-wave
    const int l32 = lane & 31;

    // ---- which (head, query block) ----
    const int bid = xcd_remap(blockIdx.x, p.n_wg);
    const int bh = bid / p.n_qblk;
    int qb = bid - bh * p.n_qblk;
    if (C::CAUSAL) qb = p.n_qblk - 1 - qb;  // longest rows first
    const int q0 = qb * C::BR;
    const int wq0 = q0 + w * 32;             // first query row of this wave
    const int qi = wq0 + l32;                 // this lane's query row
    const int n_q = p.n_q, n_kv = p.n_kv;

    const char *qh = p.q + (int64_t)bh * n_q * C::RB;
    const char *kh = p.k + (int64_t)bh * n_kv * C::RB;
    const char *vh = p.v + (int64_t)bh * n_kv * C::RB;

    const int ntile_all = (n_kv + C::BC - 1) / C::BC;
    int ntile = ntile_all;
    if (C::CAUSAL) {
        const int qlast = min(q0 + C::BR - 1, n_q - 1);
        ntile = min(ntile_all, qlast / C::BC + 1);
    }
    const int wq_last = min(wq0 + 31, n_q - 1);
    const bool wave_has_rows = wq0 < n_q;

    // Start streaming tile 0 while Q is loaded.
    load_tile<C>(kh, vh, 0, n_kv, smem, w, lane);

    // ---- Q^T operand: lane holds Q[qi][ks*16 + 8h .. +7] for every k-step ----
    v8 qf[C::KS];
    {
        const int qr = qi < n_q ? qi : n_q - 1;
        const char *qrow = qh + (int64_t)qr * C::RB + 16 * h;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            u32x4 raw = *(const u32x4 *)(qrow + 32 * ks);
            if (p.neg) raw ^= 0x80008000u;  // scale < 0: fold the sign into Q (exact)
            qf[ks] = __builtin_bit_cast(v8, raw);
        }
    }

    // ---- per-lane LDS offsets (tile-independent parts) ----
    // K operand of k-step ks: row l32 of the 32-key block, logical chunk 2ks+h.
    int koff[C::KS < 8 ? C::KS : 8];
    {
        const int sw = kswz<C>(l32);
#pragma unroll
        for (int ks = 0; ks < (C::KS < 8 ? C::KS : 8); ++ks)
            koff[ks] = l32 * C::RB + 16 * ((2 * ks + h) ^ sw);
    }
    // V^T operand via transposed reads: the 16-lane group g = lane/16 covers
    // rows kbase + (lane%16)/4 and columns 32*dblk + 16*(g%2) + 4*(lane%4).
    int voff[C::DB < 4 ? C::DB : 4];
    {
        const int j = lane & 15;
        const int rsub = 4 * h + (j >> 2);               // row within a group of 8
        const int x = vswz<C>(j >> 2) >> 2;              // swizzle of that row, in 4-chunk units
        const int y = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
#pragma unroll
        for (int db = 0; db < (C::DB < 4 ? C::DB : 4); ++db)
            voff[db] = rsub * C::RB + 16 * (4 * (db ^ x) + y) + 8 * (j & 1);
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = (f32x16){};
    float m_use = kNegInf;   // reference max (log2 units) of this lane's query row
    float l_acc = 0.f;       // this half-wave's share of the row sum
    const float c = p.c;

    for (int t = 0; t < ntile; ++t) {
        wait_vm();
        __syncthreads();
        char *stage = smem + (t & 1) * C::STAGE;
        if (t + 1 < ntile)
            load_tile<C>(kh, vh, (t + 1) * C::BC, n_kv, smem + ((t + 1) & 1) * C::STAGE, w, lane);
        const int t0 = t * C::BC;
        if (!wave_has_rows || (C::CAUSAL && t0 > wq_last)) continue;

        const char *Ks = stage;
        const char *Vs = stage + C::TILE;

        // ---- S^T = K Q^T ----
        f32x16 s[C::KB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            s[kb] = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const v8 a = *(const v8 *)(Ks + kb * 32 * C::RB + koff[ks & 7] + 256 * (ks >> 3));
                s[kb] = M::mma(a, qf[ks], s[kb]);
            }
        }

        // ---- mask (only tiles past n_kv or straddling the diagonal) ----
        const bool need_mask = (t0 + C::BC > n_kv) || (C::CAUSAL && t0 + C::BC - 1 > wq0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    const bool vis = key < n_kv && (!C::CAUSAL || key <= qi);
                    s[kb][r] = vis ? s[kb][r] : kNegInf;
                }
        }

        // ---- row max over the tile (in-lane, then across half-waves) ----
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = (mx == kNegInf) ? kNegInf : mx * c;

        // ---- online-softmax merge: raise the reference only when needed ----
        if (__any(mt > m_use + C::TAU)) {
            const float m_new = fmaxf(m_use, mt);
            const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_use - m_new);
            l_acc *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
            m_use = m_new;
        }
        const float mref = (m_use == kNegInf) ? 0.f : m_use;

        // ---- P = exp2(S c - m), row sum, convert to the MFMA type ----
        v8 pb[C::KB][2];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mref));
                if (need_mask) e = (s[kb][r] == kNegInf) ? 0.f : e;
                s[kb][r] = e;
                l_acc += e;
            }
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                v8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (T)s[kb][8 * k2 + e];
                pb[kb][k2] = x;
            }
        }

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const char *base = Vs + (kb * 32 + 16 * k2) * C::RB + voff[db & 3] + 256 * (db >> 2);
                    const i16x4 lo = lds_read_tr16(base);
                    const i16x4 hi = lds_read_tr16(base + 8 * C::RB);
                    const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[db] = M::mma(a, pb[kb][k2], o[db]);
                }
            }
        }
    }

    // ---- epilogue: O = O_acc / l, LSE = m + ln l ----
    if (qi >= n_q) return;
    const float l_tot = l_acc + __shfl_xor(l_acc, 32);
    const float inv = p.o_mul / l_tot;
    char *orow = p.o + ((int64_t)bh * n_q + qi) * C::RB;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            v4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (T)(o[db][4 * jj + e] * inv);
            *(v4 *)(orow + 2 * (32 * db + 8 * jj + 4 * h)) = out;
        }
    if (p.lse && h == 0) p.lse[(int64_t)bh * n_q + qi] = (m_use + __log2f(l_tot)) * kLn2;
}

template <class C>
int launch(const KParams &p, void *stream) {
    hipLaunchKernelGGL(fwd16_kernel<C>, dim3(p.n_wg), dim3(C::NT), 0, (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

#define FA_V16(T, DT, D, NW, BC, CAUSAL)                                                   \
    Variant{DT, D, CAUSAL, 32 * NW, "br" #NW "x32_bc" #BC, &launch<Cfg<T, D, NW, BC, CAUSAL>>}

// Host-side table of the compiled 16-bit variants.
const Variant *variants16(int *count) {
    static const Variant table[] = {
        FA_V16(__bf16, FA_BF16, 64, 8, 64, 0),
        FA_V16(__bf16, FA_BF16, 64, 8, 64, 1),
        FA_V16(__bf16, FA_BF16, 128, 8, 64, 0),
        FA_V16(__bf16, FA_BF16, 128, 8, 64, 1),
        FA_V16(__bf16, FA_BF16, 256, 4, 64, 0),
        FA_V16(__bf16, FA_BF16, 256, 4, 64, 1),
        FA_V16(_Float16, FA_F16, 64, 8, 64, 0),
        FA_V16(_Float16, FA_F16, 64, 8, 64, 1),
        FA_V16(_Float16, FA_F16, 128, 8, 64, 0),
        FA_V16(_Float16, FA_F16, 128, 8, 64, 1),
        FA_V16(_Float16, FA_F16, 256, 4, 64, 0),
        FA_V16(_Float16, FA_F16, 256, 4, 64, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
