// Attention forward for OCP E4M3 (8-bit float) inputs on gfx950; O in bfloat16.
//
// Same decomposition, online softmax and one-tile software pipeline as the
// 16-bit kernel (one workgroup per (batch*head, 256 query rows), one wave per
// 32 rows, S^T = K Q^T so each lane owns a query row, K and V double-buffered
// in LDS by direct global->LDS copies), with both products on the 8-bit
// matrix instruction v_mfma_f32_32x32x64_f8f6f4:
//
//   S^T = K Q^T        E4M3 codes; the descales of Q and K are folded into
//                      the exponent factor c = |scale| dq dk log2(e)
//   P' = exp2(S c - m + 6) = 64 P   float32; the reference max m is raised
//                      only when the tile max exceeds it by more than 2 (log2
//                      units), so P <= 4 and P' <= 256 < 448 (E4M3's largest
//                      value); the factor 2^6 scales P into E4M3's normal
//                      range and is folded into the exponent; the row sum l
//                      accumulates the float32 P'
//   O^T += V^T P'^T    P' rounded to E4M3; V read with ds_read_b64_tr_b8
//   O = O_acc dv / l   stored as bfloat16 (the 2^6 cancels);
//   LSE = (m - 6 + log2 l) ln 2
//
// The softmax of each tile is split at its 32-key block boundary: block 0
// runs under the PV MFMAs of the previous tile, block 1 under the S MFMAs of
// the next, so the VALU work (here larger than the MFMA time of a wave) is
// spread over both halves of the loop.
//
// Key order inside a 32-key block: row rho of the S^T MFMA is key
// pi(rho) = 16 ((rho/4) % 2) + 4 (rho/8) + rho % 4, which makes the S^T
// registers of each half-wave hold 16 consecutive keys, so the V^T operand
// of the P V product is four transposed reads of 8 consecutive rows.
#include <type_traits>

#include "fa_device.h"
#include "../../include/fa.h"

namespace fa {
namespace {

// SPLIT: the workgroup covers one chunk of the key range (split-KV, with
// 4 waves) and writes a float32 partial output and LSE instead of O.
template <bool CAUSAL_, bool SPLIT_ = false, int NW_ = 8>
struct Cfg8 {
    static constexpr int D = 128, NW = NW_, BC = 64, NT = NW * 64, BR = 32 * NW;
    static constexpr bool CAUSAL = CAUSAL_, SPLIT = SPLIT_;
    static constexpr int RB = D;            // bytes per row
    static constexpr int TILE = BC * RB;    // 8 KB
    static constexpr int LDI = TILE / (1024 * NW);  // copy instructions per wave per tile
    // waves per SIMD the register budget must allow: two workgroups of 4
    // waves per CU for the split kernels (bound by HBM, they want copies in
    // flight), one of 8 waves otherwise
    static constexpr int MIN_WAVES = NW_ == 4 ? 2 : 1;
    static constexpr int LDS = 4 * TILE;    // K0, K1, V0, V1
    static constexpr int KS = D / 64;       // k-steps of S^T = K Q^T
    static constexpr int KB = BC / 32;
    static constexpr int DB = D / 32;
    // reference max raised only past TAU (log2 units), so P <= 2^TAU; P is
    // stored as 2^PSHIFT P, at most 2^(TAU + PSHIFT) = 256 < 448 (E4M3's max)
    static constexpr float TAU = 2.0f, PSHIFT = 6.0f;
    static_assert(TAU + PSHIFT <= 8.0f, "scaled P must stay below E4M3's largest value");
    static_assert(TILE % (1024 * NW) == 0, "whole copy instructions per wave per tile");
};

// Key row of S^T MFMA row rho (within a 32-key block).
__device__ __forceinline__ int key_of_row(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// LDS swizzles (XOR on the 16-byte chunk index of a 128-byte row).
// K: the 16 rows one half-wave reads together are {0..7, 16..23} (+8, +32k);
// this XOR gives each of the 8 rows of one parity its own chunk.
__device__ __forceinline__ int kswz8(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
// V: a half-wave's transposed reads cover 8 consecutive rows x 2 chunks.
__device__ __forceinline__ int vswz8(int r) { return 2 * ((r >> 1) & 3); }

// Issues the direct-to-LDS copy of rows [t0, t0 + BC) of one head (one 16-byte
// chunk per lane, LDI instructions per wave); rows past n_kv are clamped.
template <class C, bool IS_V>
__device__ __forceinline__ void copy_tile(const char *src, int t0, int n_kv, char *buf, int w, int lane) {
#pragma unroll
    for (int i = 0; i < C::LDI; ++i) {
        const int chunk = (i * C::NW + w) * 64 + lane;
        const int r = chunk >> 3;
        const int pc = chunk & 7;
        const int gr = min(t0 + r, n_kv - 1);
        const int lc = pc ^ (IS_V ? vswz8(r) : kswz8(r));
        copy16_to_lds(src + (int64_t)gr * C::RB + 16 * lc, buf + (i * C::NW + w) * 1024);
    }
}

__device__ __forceinline__ void both_halves8(float x, float &lo, float &hi) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    unsigned v;
    asm("v_mov_b32 %0, %1" : "=v"(v) : "v"(u));
    const auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// S^T = K_tile Q^T for the 2 x 32-key blocks of a tile.
template <class C>
__device__ __forceinline__ void qk8(f32x16 (&s)[C::KB], const char *Ks, const int (&koff)[C::KS][2],
                                    const i32x8 (&qf)[C::KS]) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) s[kb] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            const u32x4 lo = *(const u32x4 *)(Ks + kb * 32 * C::RB + koff[ks][0]);
            const u32x4 hi = *(const u32x4 *)(Ks + kb * 32 * C::RB + koff[ks][1]);
            const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            s[kb] = mma8(a, qf[ks], s[kb]);
        }
}

// O^T += V^T P^T.  k-slot e (0..31) of half-wave h carries key
// 32 (e/16) + 16 h + e % 16; four transposed reads of 8 rows give V^T.
template <class C>
__device__ __forceinline__ void pv8(f32x16 (&o)[C::DB], const char *Vs, const int (&voff)[C::DB],
                                    const i32x8 &pb) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        i32x2v r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = lds_read_tr8(Vs + (8 * (u & 1) + 32 * (u >> 1)) * C::RB + voff[db]);
        const i32x8 a = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
        o[db] = mma8(a, pb, o[db]);
    }
}

// Keys past n_kv and (causal) keys after qi become -inf.
template <class C>
__device__ __forceinline__ void mask8(f32x16 (&s)[C::KB], int t0, int qi, int n_kv, int h) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = t0 + 32 * kb + 16 * h + r;
            const bool vis = key < n_kv && (!C::CAUSAL || key <= qi);
            s[kb][r] = vis ? s[kb][r] : kNegInf;
        }
}

// Online-softmax step (plate 08 merge) for one tile, in two parts at the
// 32-key block boundary.  The reference max is raised when the tile's row max
// exceeds it by more than TAU (wave-uniform decision), so P = exp2(S c - m) <=
// 2^TAU; the kernel computes P' = 2^PSHIFT P = exp2(S c - m + PSHIFT)
// directly, sums the float32 P' into l_acc and rounds P' to E4M3 into the P^T
// operand; `raised` and alpha tell the caller to rescale O before
// accumulating this tile.  Each pair of codes is written over the operand
// word's previous contents, whose last reader was the P V product of the
// tile before, so the half-word conversions need no zeroed register.  softmax8_head takes the row max, the decision and
// block 0 of P' (words 0-3 of the operand); softmax8_tail block 1 (words 4-7)
// with the same bias.  The loop runs the head under the PV MFMAs of the
// previous tile and the tail under the S MFMAs of the next, so both halves of
// the loop carry VALU work (one max per tile, no extra instructions).
template <class C>
__device__ __forceinline__ void softmax8_head(f32x16 (&s)[C::KB], i32x8 &pb, float &m_use, float &l_acc,
                                              float &alpha, bool &raised, float c, float &bias) {
    float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
    float lo, hi;
    both_halves8(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])), lo, hi);
    const float mt = fmaxf(lo, hi) * c;
    raised = __any(mt > m_use + C::TAU);
    const float m_new = raised ? fmaxf(m_use, mt) : m_use;
    alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_use - m_new);
    l_acc *= alpha;
    m_use = m_new;
    bias = C::PSHIFT - ((m_use == kNegInf) ? 0.f : m_use);
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[0][4 * w4 + e], c, bias));
            l4[e] += v[e];
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], pb[w4], false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
        pb[w4] = word;
    }
    l_acc += (l4[0] + l4[1]) + (l4[2] + l4[3]);
}
template <class C>
__device__ __forceinline__ void softmax8_tail(const f32x16 &s1, i32x8 &pb, float &l_acc, float c, float bias) {
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[4 * w4 + e], c, bias));
            l4[e] += v[e];
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], pb[4 + w4], false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
        pb[4 + w4] = word;
    }
    l_acc += (l4[0] + l4[1]) + (l4[2] + l4[3]);
}

template <class C>
__global__ __launch_bounds__(C::NT, C::MIN_WAVES) void fwd8_kernel(KParams p) {
    // K and V buffers as four LDS objects: a read of one is not held up by a
    // copy in flight into another
    __shared__ __attribute__((aligned(1024))) char sk0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sk1[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sv0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sv1[C::TILE];
    auto kbuf = [&](int i) { return i ? sk1 : sk0; };
    auto vbuf = [&](int i) { return i ? sv1 : sv0; };

    const int lane = lane_id();
    const int w = wave_id();
    const int h = lane >> 5;
    const int l32 = lane & 31;

    int bid = xcd_remap(blockIdx.x, p.n_wg);
    int split = 0;
    if (C::SPLIT) {
        const int per = p.n_bh * p.n_qblk;
        split = bid / per;
        bid -= split * per;
    }
    const int bh = bid / p.n_qblk;
    int qb = bid - bh * p.n_qblk;
    if (C::CAUSAL) qb = p.n_qblk - 1 - qb;
    const int q0 = qb * C::BR;
    const int wq0 = q0 + w * 32;
    const int qi = wq0 + l32;
    const int n_q = p.n_q;
    // Keys [kofs, kofs + n_kv) of the head; the causal comparisons below use
    // query indices shifted by -kofs so that they stay relative to this range.
    const int kofs = C::SPLIT ? split * p.kv_split : 0;
    const int n_kv = C::SPLIT ? min(p.kv_split, p.n_kv - kofs) : p.n_kv;
    const int rwq0 = wq0 - kofs, rqi = qi - kofs;
    const char *qh = p.q + (int64_t)bh * n_q * C::RB;
    const char *kh = p.k + ((int64_t)bh * p.n_kv + kofs) * C::RB;
    const char *vh = p.v + ((int64_t)bh * p.n_kv + kofs) * C::RB;

    int ntile = (n_kv + C::BC - 1) / C::BC;
    if (C::CAUSAL) {
        const int last = min(q0 + C::BR - 1, n_q - 1) - kofs;  // last row, relative
        ntile = last < 0 ? 0 : min(ntile, last / C::BC + 1);
    }
    int wn = 0;
    if (wq0 < n_q) {
        const int last = min(wq0 + 31, n_q - 1) - kofs;
        wn = !C::CAUSAL ? ntile : (last < 0 ? 0 : min(ntile, last / C::BC + 1));
    }
    auto need_mask = [&](int t) {
        return (t + 1) * C::BC > n_kv || (C::CAUSAL && (t + 1) * C::BC - 1 > rwq0);
    };

    copy_tile<C, false>(kh, 0, n_kv, kbuf(0), w, lane);
    copy_tile<C, true>(vh, 0, n_kv, vbuf(0), w, lane);
    if (ntile > 1) copy_tile<C, false>(kh, C::BC, n_kv, kbuf(1), w, lane);

    // Q^T operand: lane holds Q[qi][64 ks + 32 h .. +31] for each k-step.
    i32x8 qf[C::KS];
    {
        const char *qrow = qh + (int64_t)min(qi, n_q - 1) * C::RB + 32 * h;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            u32x4 lo = *(const u32x4 *)(qrow + 64 * ks);
            u32x4 hi = *(const u32x4 *)(qrow + 64 * ks + 16);
            if (p.neg) {  // scale < 0: flip the sign bit of every code (exact)
                lo ^= 0x80808080u;
                hi ^= 0x80808080u;
            }
            qf[ks] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
    // K operand: row key_of_row(l32) of each 32-key block, chunks 4ks + 2h and +1.
    int koff[C::KS][2];
    {
        const int r = key_of_row(l32);
        const int sw = kswz8(r);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) koff[ks][s2] = r * C::RB + 16 * ((4 * ks + 2 * h + s2) ^ sw);
    }
    // V^T operand: in group g = lane/16, lane j addresses row 16h + j/2 (+ the
    // read's base row) and columns 32 db + 16 (g % 2) + 8 (j % 2).
    int voff[C::DB];
    {
        const int j = lane & 15;
        const int row = 16 * h + (j >> 1);
        const int x = vswz8(row) >> 1;
        const int g2 = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) voff[db] = row * C::RB + 16 * (2 * (db ^ x) + g2) + 8 * (j & 1);
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = (f32x16){};
    float m_use = kNegInf, l_acc = 0.f, alpha = 1.f;
    bool raised = false;
    const float c = p.c;
    i32x8 p0 = (i32x8){}, p1 = (i32x8){};

    wait_vm();
    __syncthreads();
    f32x16 s_tail = (f32x16){};  // block 1 of the last tile's scores
    float bias_tail = 0.f;        // and the exponent bias of its P'
    if (wn > 0) {
        f32x16 s[C::KB];
        qk8<C>(s, kbuf(0), koff, qf);
        if (need_mask(0)) mask8<C>(s, 0, rqi, n_kv, h);
        softmax8_head<C>(s, p0, m_use, l_acc, alpha, raised, c, bias_tail);
        s_tail = s[1];
        raised = false;
    }

    auto iteration = [&](auto par, int t, i32x8 &pc, i32x8 &pn) {
        constexpr int PAR = decltype(par)::value;
        wait_vm();
        __syncthreads();
        if (t + 2 < ntile) copy_tile<C, false>(kh, (t + 2) * C::BC, n_kv, kbuf(PAR), w, lane);
        if (t + 1 < ntile) copy_tile<C, true>(vh, (t + 1) * C::BC, n_kv, vbuf(1 - PAR), w, lane);
        if (t >= wn) return;
        if (raised) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
        }
        if (t + 1 < wn) {
            f32x16 s[C::KB];
            const bool masked = need_mask(t + 1);
            qk8<C>(s, kbuf(1 - PAR), koff, qf);
            softmax8_tail<C>(s_tail, pc, l_acc, c, bias_tail);
            // keep the tail under the S MFMAs: without this the compiler
            // sinks it past the masking branch, next to the PV MFMAs
            asm volatile("" : "+v"(pc), "+v"(l_acc));
            if (masked) mask8<C>(s, (t + 1) * C::BC, rqi, n_kv, h);
            pv8<C>(o, vbuf(PAR), voff, pc);
            softmax8_head<C>(s, pn, m_use, l_acc, alpha, raised, c, bias_tail);
            s_tail = s[1];
        } else {
            softmax8_tail<C>(s_tail, pc, l_acc, c, bias_tail);
            pv8<C>(o, vbuf(PAR), voff, pc);
        }
    };
    for (int t = 0; t < ntile; t += 2) {
        iteration(std::integral_constant<int, 0>(), t, p0, p1);
        if (t + 1 >= ntile) break;
        iteration(std::integral_constant<int, 1>(), t + 1, p1, p0);
    }

    // O (bf16, 256-byte rows) leaves through LDS so that each store
    // instruction writes 128-byte row segments instead of 8-byte pieces of
    // 32 rows (the accumulator layout).  The tile buffers hold 4 KB per wave
    // once every wave is past its last K/V read: 32 rows of 128 bytes, so
    // each wave stages its rows in two column halves.  Staging rows of 128
    // bytes use the swizzle (r / 2) % 8 of their 16-byte chunks, which keeps
    // the 8-byte writes by column and the 16-byte reads by row free of bank
    // conflicts.
    float lo, hi;
    both_halves8(l_acc, lo, hi);
    const float l_tot = lo + hi;
    if (C::SPLIT) {
        // partial of this key chunk, float32 and not yet multiplied by the V
        // descale (the merge applies it); a row that sees no key of the chunk
        // (causal) gets O = 0 and LSE = -inf, i.e. weight 0 in the merge
        if (qi >= n_q) return;
        const int64_t row = ((int64_t)split * p.n_bh + bh) * n_q + qi;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *orow = p.part_o + row * C::D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = o[db][4 * jj + e] * inv;
                *(f32x4 *)(orow + 32 * db + 8 * jj + 4 * h) = out;
            }
        if (h == 0) p.part_lse[row] = l_tot > 0.f ? (m_use - C::PSHIFT + __log2f(l_tot)) * kLn2 : kNegInf;
        return;
    }
    static_assert(C::SPLIT || (C::TILE == 2 * 4096 && C::NW == 8), "two waves' staging per tile buffer");
    __syncthreads();
    if (wq0 >= n_q) return;
    const float inv = p.o_mul / l_tot;
    char *stage = (w < 2 ? sk0 : w < 4 ? sk1 : w < 6 ? sv0 : sv1) + 4096 * (w & 1);
    const int rr = lane >> 3, cc = lane & 7;
    char *obase = p.o + ((int64_t)bh * n_q + wq0) * (2 * C::D);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                bf16x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = (__bf16)(o[2 * half + d2][4 * jj + e] * inv);
                *(bf16x4 *)(stage + 128 * l32 + 16 * ((4 * d2 + jj) ^ ((l32 >> 1) & 7)) + 8 * h) = out;
            }
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int r = 8 * s4 + rr;
            const u32x4 val = *(const u32x4 *)(stage + 128 * r + 16 * (cc ^ ((r >> 1) & 7)));
            if (wq0 + r < n_q) *(u32x4 *)(obase + (int64_t)r * (2 * C::D) + 128 * half + 16 * cc) = val;
        }
    }
    if (p.lse && h == 0 && qi < n_q) p.lse[(int64_t)bh * n_q + qi] = (m_use - C::PSHIFT + __log2f(l_tot)) * kLn2;
}

template <class C>
int launch8(const KParams &p, void *stream) {
    hipLaunchKernelGGL(fwd8_kernel<C>, dim3(p.n_wg), dim3(C::NT), 0, (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

// Host-side table of the compiled E4M3 variants.
const Variant *variants8(int *count) {
    static const Variant table[] = {
        Variant{FA_FP8_E4M3, 128, 0, 0, 256, "br8x32_bc64", &launch8<Cfg8<false>>},
        Variant{FA_FP8_E4M3, 128, 1, 0, 256, "br8x32_bc64", &launch8<Cfg8<true>>},
        Variant{FA_FP8_E4M3, 128, 0, 1, 128, "split_br4x32_bc64", &launch8<Cfg8<false, true, 4>>},
        Variant{FA_FP8_E4M3, 128, 1, 1, 128, "split_br4x32_bc64", &launch8<Cfg8<true, true, 4>>},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
