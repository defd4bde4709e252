// Attention backward for 16-bit inputs (bf16, fp16) on gfx950.
//
// "FlashAttention 与显存" plate 09: the backward pass keeps only O and the
// per-row statistic (here the LSE) from the forward and recomputes the
// scores and probabilities tile by tile.  With P_ij = exp(scale q_i.k_j -
// LSE_i) and the textbook gradients of softmax(scale Q K^T) V,
//
//   D_i   = sum_c dO_ic O_ic                      bwd_dq_kernel, per row first
//   dQ_i  = scale sum_j P_ij (dP_ij - D_i) k_j     bwd_dq_kernel (query blocks)
//   dV_j  = sum_i P_ij dO_i                         bwd_dkdv_kernel (key blocks)
//   dK_j  = scale sum_i P_ij (dP_ij - D_i) q_i
//
// with dP_ij = dO_i . v_j.  dQ and dK/dV are computed by separate kernels so
// that every output element has exactly one writer (no atomics; results are
// bitwise repeatable); the price is computing S and dP twice.  At d = 256 the
// dK and dV accumulators of a wave (128 registers each) do not fit together
// beside this wave's K and V rows, so the dK/dV kernel runs as two passes,
// one accumulating dV (S and P only) and one dK (S, dP and dS).
//
// Both kernels use the 32x32x16 MFMA layouts of the forward kernel (the
// tile helpers of fa_tile16.h).  In the dQ kernel a wave owns 32 query rows,
// as in the forward: S^T = K Q^T and dP^T = V dO^T have one query per lane,
// and dQ^T += K^T dS^T reads K transposed from LDS.  In the dK/dV kernel a
// wave owns 32 keys and the roles of queries and keys swap: S = Q K^T and
// dP = dO V^T have one key per lane (Q and dO tiles streamed through LDS,
// this wave's K and V rows in registers), and dV^T += dO^T P, dK^T += Q^T dS
// read dO and Q transposed.  LSE_i and D_i vary along the accumulator's rows
// there, so they are staged through LDS with the tiles.
#include <utility>

#include "fa_device.h"
#include "fa_tile16.h"
#include "../../include/fa.h"

namespace fa {
namespace {

constexpr int kBwdTile = 64;  // rows per streamed tile (keys for dQ, queries for dK/dV)

// f(integral_constant<int, I>) for I = 0 .. N-1 in order, each with a
// compile-time index (a long #pragma unroll loop is not always unrolled)
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

// DROP: the dropout keep mask of the forward is replayed.  PART: in the
// dK/dV kernel 0 accumulates dK and dV, 1 dV only, 2 dK only; in the dQ
// kernel 0 accumulates all of dQ, 1 its first half of columns, 2 the second.
template <typename T_, int D_, int NW_, bool CAUSAL_, bool DROP_ = false, int PART_ = 0>
struct CfgB {
    typedef T_ T;
    static constexpr int D = D_, NW = NW_, BC = kBwdTile, NT = NW * 64, BR = 32 * NW;
    static constexpr bool CAUSAL = CAUSAL_, DROP = DROP_;
    static constexpr int PART = PART_;
    static constexpr bool WANT_DV = PART_ != 2, WANT_DK = PART_ != 1;
    static constexpr int RB = D * 2, NC = RB / 16, RPB = RB >= 256 ? 1 : 256 / RB;
    static constexpr int KX = (NC < 16 ? NC : 16) - 1, VX = (NC / 4 < 4 ? NC / 4 : 4) - 1;
    static constexpr int TILE = BC * RB;
    static constexpr int KS = D / 16, KB = BC / 32, DB = D / 32, LDI = TILE / (1024 * NW);
    static constexpr int NVO = DB < 4 ? DB : 4;
    // dQ column blocks of this pass (dQ kernel)
    static constexpr int QDB = PART_ == 0 ? DB : DB / 2, QDB0 = PART_ == 2 ? DB / 2 : 0;
    static constexpr int LDS = 4 * TILE + 2 * 512;  // two streams x two buffers, + LSE/D tiles
    // waves per SIMD the register budget must allow: at d = 64 the dK/dV
    // kernel fits two (two workgroups of 4 waves per CU); at d = 128 its
    // accumulators alone take 128 registers and it runs one
    static constexpr int MIN_WAVES = D <= 64 ? 2 : 1;
    static_assert(TILE % (1024 * NW) == 0, "tile must split into whole wave copies");
};

// Per-lane LDS offsets of the two operand reads of a tile in the layout read
// both ways (bswz): row reads (k-step 0 of qk_tile; k-step ks is koff ^ 32
// ks) and transposed reads (pv_tile).
template <class C>
__device__ __forceinline__ int row_offset_b(int lane) {
    const int l32 = lane & 31, h = lane >> 5;
    return l32 * C::RB + 16 * (h ^ bswz<C>(l32));
}
// A transposed operand is two reads, rows rsub and rsub + 8 of a 16-row
// slice (slices start at multiples of 16 rows).  Row rsub + 8 has the
// swizzle of row rsub with bit 1 flipped, so its offset is the first one
// XOR 32, plus 8 rows.  tr_hi keeps the second offsets in registers up to
// d = 128 and recomputes them at d = 256, where the dK pass has no
// registers to spare.
struct TrOffsets {
    int lo[4], hi[4];
};
template <class C>
__device__ __forceinline__ int tr_hi(const TrOffsets &vo, int i) {
    return C::D >= 256 ? (vo.lo[i] ^ 32) + 8 * C::RB : vo.hi[i];
}
template <class C>
__device__ __forceinline__ TrOffsets tr_offsets(int lane) {
    const int h = lane >> 5;
    const int j = lane & 15;
    const int rsub = 4 * h + (j >> 2);
    const int g = bswz<C>(rsub);
    const int y = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
    TrOffsets t;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        t.lo[db] = rsub * C::RB + 16 * (4 * (db ^ (g >> 2)) + (y ^ (g & 3))) + 8 * (j & 1);
        t.hi[db] = C::D >= 256 ? 0 : (t.lo[db] ^ 32) + 8 * C::RB;
    }
    return t;
}

// This lane's row of a [n, d] slice as the 32x32x16 B operand (row r of the
// wave's 32-row block, k-steps ks: elements ks*16 + 8h .. +7).
template <class C>
__device__ __forceinline__ void load_rows(const char *base, int row, int n,
                                          typename Mma16<typename C::T>::v8 (&f)[C::KS], int h) {
    typedef typename Mma16<typename C::T>::v8 v8;
    const int r = row < n ? row : n - 1;
    const char *p = base + (int64_t)r * C::RB + 16 * h;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) f[ks] = __builtin_bit_cast(v8, *(const u32x4 *)(p + 32 * ks));
}

// Stores rows of an O^T-layout accumulator (one row per lane, d columns)
// times mul, converted to T.
template <class C, int NDB = C::DB, int DB0 = 0>
__device__ __forceinline__ void store_rows(char *rowp, const f32x16 (&acc)[NDB], float mul, int h) {
    typedef typename Mma16<typename C::T>::v4 v4;
    typedef typename C::T T;
    rowp += 64 * DB0;  // column 32 DB0
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            v4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (T)(acc[db][4 * jj + e] * mul);
            *(v4 *)(rowp + 2 * (32 * db + 8 * jj + 4 * h)) = out;
        }
}

// Two products of one 32-row block: s = A f and dp = G g, with A and G the
// block's rows of two LDS tiles (row reads from koff0) and f, g this lane's
// register rows.  Every operand read is issued before the first MFMA, in a
// scheduling region of its own: left to itself the scheduler places each read
// right before its MFMA and reuses one register set, which exposes the LDS
// latency on every MFMA.  The two accumulation chains alternate.
template <class C>
__device__ __forceinline__ void qk_rows2(f32x16 &s, f32x16 &dp, const char *ablk, const char *gblk, int koff0,
                                         const typename Mma16<typename C::T>::v8 (&f)[C::KS],
                                         const typename Mma16<typename C::T>::v8 (&g)[C::KS]) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    asm volatile("" : "+v"(koff0));
    auto off = [&](int ks) { return (koff0 ^ (32 * (ks & 7))) + 256 * (ks >> 3); };
    s = (f32x16){};
    dp = (f32x16){};
    if constexpr (C::D <= 128) {
        v8 a[C::KS], b[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            a[ks] = *(const v8 *)(ablk + off(ks));
            b[ks] = *(const v8 *)(gblk + off(ks));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            s = M::mma(a[ks], f[ks], s);
            dp = M::mma(b[ks], g[ks], dp);
        }
    } else {
        // d = 256: all 32 operand reads up front would take 128 registers;
        // a rolling window of L k-steps ahead instead, each step a
        // scheduling region of its own
        constexpr int L = 4;
        v8 a[L], b[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            a[j] = *(const v8 *)(ablk + off(j));
            b[j] = *(const v8 *)(gblk + off(j));
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            s = M::mma(a[ks % L], f[ks], s);
            dp = M::mma(b[ks % L], g[ks], dp);
            if (ks + L < C::KS) {
                a[ks % L] = *(const v8 *)(ablk + off(ks + L));
                b[ks % L] = *(const v8 *)(gblk + off(ks + L));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Two products of one 32-row block of pv_tile: o1^T += A1^T p1 and
// o2^T += A2^T p2, with A1, A2 the block's rows of two LDS tiles (transposed
// reads) and p1, p2 the block's packed operands (k2 = 0, 1).  Reads first, in
// their own scheduling region, as in qk_rows2.
template <class C>
__device__ __forceinline__ void pv_rows2(f32x16 (&o1)[C::DB], const char *blk1,
                                         const typename Mma16<typename C::T>::v8 (&p1)[2], f32x16 (&o2)[C::DB],
                                         const char *blk2, const typename Mma16<typename C::T>::v8 (&p2)[2],
                                         const TrOffsets &vo) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    v8 a1[2][C::DB], a2[2][C::DB];
    auto rd = [&](const char *blk, int k2, int db) {
        const int base = 16 * k2 * C::RB + 256 * (db >> 2);
        const i16x4 lo = lds_read_tr16(blk + base + vo.lo[db & 3]);
        const i16x4 hi = lds_read_tr16(blk + base + tr_hi<C>(vo, db & 3));
        return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            a1[k2][db] = rd(blk1, k2, db);
            a2[k2][db] = rd(blk2, k2, db);
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            o1[db] = M::mma(a1[k2][db], p1[k2], o1[db]);
            o2[db] = M::mma(a2[k2][db], p2[k2], o2[db]);
        }
}

// One product of one 32-row block, s = A f, as qk_rows2 (reads first).
template <class C>
__device__ __forceinline__ void qk_rows1(f32x16 &s, const char *ablk, int koff0,
                                         const typename Mma16<typename C::T>::v8 (&f)[C::KS]) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    asm volatile("" : "+v"(koff0));
    v8 a[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) a[ks] = *(const v8 *)(ablk + (koff0 ^ (32 * (ks & 7))) + 256 * (ks >> 3));
    __builtin_amdgcn_sched_barrier(0);
    s = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s = M::mma(a[ks], f[ks], s);
}

// One product of one 32-row block of pv_tile, o^T += A^T p, as pv_rows2.
template <class C>
__device__ __forceinline__ void pv_rows1(f32x16 (&o)[C::DB], const char *blk,
                                         const typename Mma16<typename C::T>::v8 (&pv)[2],
                                         const TrOffsets &vo) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    v8 a[2][C::DB];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const char *base = blk + 16 * k2 * C::RB + 256 * (db >> 2);
            const i16x4 lo = lds_read_tr16(base + vo.lo[db & 3]);
            const i16x4 hi = lds_read_tr16(base + tr_hi<C>(vo, db & 3));
            a[k2][db] = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] = M::mma(a[k2][db], pv[k2], o[db]);
}

// S = K-tile rows x qf and dP = V-tile rows x gf for both 32-key blocks, with
// a rolling window of L operand reads ahead of the MFMAs.  Each step (MFMA i,
// then the read for MFMA i + L) is a scheduling region of its own, so the
// scheduler cannot pull the reads back next to their MFMAs.
template <class C, int L>
__device__ __forceinline__ void qk_dq_rolling(f32x16 (&s)[C::KB], f32x16 (&dp)[C::KB], const char *Ks,
                                              const char *Vs, int koffk, int koffv,
                                              const typename Mma16<typename C::T>::v8 (&qf)[C::KS],
                                              const typename Mma16<typename C::T>::v8 (&gf)[C::KS]) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    constexpr int N = 2 * C::KB * C::KS;
    asm volatile("" : "+v"(koffk), "+v"(koffv));
    auto rd = [&](int i) {
        const int ks = i / (2 * C::KB), kb = (i >> 1) % C::KB, wh = i & 1;
        const char *base = (wh ? Vs : Ks) + kb * 32 * C::RB;
        return *(const v8 *)(base + (((wh ? koffv : koffk) ^ (32 * (ks & 7))) + 256 * (ks >> 3)));
    };
    v8 buf[L];
#pragma unroll
    for (int j = 0; j < L; ++j) buf[j] = rd(j);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
        s[kb] = (f32x16){};
        dp[kb] = (f32x16){};
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int ks = i / (2 * C::KB), kb = (i >> 1) % C::KB, wh = i & 1;
        const v8 a = buf[i % L];
        if (wh)
            dp[kb] = M::mma(a, gf[ks], dp[kb]);
        else
            s[kb] = M::mma(a, qf[ks], s[kb]);
        if (i + L < N) buf[i % L] = rd(i + L);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// o^T += V_tile^T P^T as pv_tile, with a rolling window of L MFMAs' operand
// reads (two transposed reads each) ahead.
template <class C, int L>
__device__ __forceinline__ void pv_dq_rolling(f32x16 (&o)[C::QDB], const char *Vs, const TrOffsets &vo,
                                              const typename Mma16<typename C::T>::v8 (&pb)[C::KB][2]) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    constexpr int NB = C::QDB;  // column blocks C::QDB0 .. + NB of this pass
    constexpr int N = C::KB * 2 * NB;
    auto rd = [&](int i) {
        const int kb = i / (2 * NB), k2 = (i / NB) & 1, db = C::QDB0 + i % NB;
        const char *base = Vs + (kb * 32 + 16 * k2) * C::RB + 256 * (db >> 2);
        const i16x4 lo = lds_read_tr16(base + vo.lo[db & 3]);
        const i16x4 hi = lds_read_tr16(base + tr_hi<C>(vo, db & 3));
        return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    v8 buf[L];
#pragma unroll
    for (int j = 0; j < L; ++j) buf[j] = rd(j);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int kb = i / (2 * NB), k2 = (i / NB) & 1, db = i % NB;
        o[db] = M::mma(buf[i % L], pb[kb][k2], o[db]);
        if (i + L < N) buf[i % L] = rd(i + L);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (batch*head, block of 32*NW query rows), streaming
// K and V tiles of 64 keys.  K is stored in the layout read both ways (by
// rows and transposed), V in the K-style layout (read by rows only).
template <class C>
__global__ __launch_bounds__(C::NT, C::MIN_WAVES) void bwd_dq_kernel(BwdParams p) {
    typedef typename C::T T;
    typedef Mma16<T> M;
    typedef typename M::v8 v8;
    // four LDS objects (K, V x two buffers): a read of one is then not held
    // up by a copy in flight into another
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
    const int n_qblk = (p.n_q + C::BR - 1) / C::BR;
    const int bid = xcd_remap(blockIdx.x, p.n_bh * n_qblk);
    const int bh = bid / n_qblk;
    int qb = bid - bh * n_qblk;
    if (C::CAUSAL) qb = n_qblk - 1 - qb;  // longest rows first
    const int q0 = qb * C::BR;
    const int wq0 = q0 + 32 * w;
    const int qi = wq0 + l32;
    const int n_q = p.n_q, n_kv = p.n_kv;

    const char *qh = p.q + (int64_t)bh * n_q * C::RB;
    const char *gh = p.dout + (int64_t)bh * n_q * C::RB;
    const char *kh = p.k + (int64_t)bh * n_kv * C::RB;
    const char *vh = p.v + (int64_t)bh * n_kv * C::RB;

    int ntile = (n_kv + C::BC - 1) / C::BC;
    if (C::CAUSAL) ntile = min(ntile, min(q0 + C::BR - 1, n_q - 1) / C::BC + 1);
    int wn = 0;
    if (wq0 < n_q) wn = !C::CAUSAL ? ntile : min(ntile, min(wq0 + 31, n_q - 1) / C::BC + 1);

    const CopyPlan<C, kLayoutBoth> kplan(w, lane);
    const CopyPlan<C, kLayoutK> vplan(w, lane);
    if (ntile > 0) {
        kplan.issue(kh, 0, n_kv, kbuf(0), w, lane);
        vplan.issue(vh, 0, n_kv, vbuf(0), w, lane);
    }

    v8 qf[C::KS], gf[C::KS];
    load_rows<C>(qh, qi, n_q, qf, h);
    load_rows<C>(gh, qi, n_q, gf, h);
    const int64_t row = (int64_t)bh * n_q + (qi < n_q ? qi : n_q - 1);
    // D_i = sum_c dO_ic O_ic (float32) and LSE_i log2 e of this lane's row,
    // for this kernel and, through the workspace, for the dK/dV kernel that
    // runs after it: each lane reads the half of O's row that matches its dO
    // operand, and the two half-waves' sums are added
    float dlt;
    {
        typedef typename M::v8 v8o;
        const char *orow = p.o + (row * C::RB) + 16 * h;
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const v8o ov = __builtin_bit_cast(v8o, *(const u32x4 *)(orow + 32 * ks));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (float)ov[e] * (float)gf[ks][e];
        }
        dlt = sum_halves(acc);
    }
    const float lse2 = p.lse[row] * kLog2e;
    if (C::PART != 2 && h == 0 && qi < n_q) {  // the second dQ pass finds them stored
        p.delta[row] = dlt;
        p.lse2[row] = lse2;
    }
    const float c = p.c;
    DropQuad dr{};
    if (C::DROP) dr = make_drop_quad(p.p8, (unsigned)qi >> 2, (unsigned)bh, p.drop_off, p.seed_lo, p.seed_hi);

    const int koff_k = row_offset_b<C>(lane);
    const int koff_v = l32 * C::RB + 16 * (h ^ kswz<C>(l32));
    const TrOffsets voff = tr_offsets<C>(lane);

    f32x16 dq[C::QDB];
#pragma unroll
    for (int db = 0; db < C::QDB; ++db) dq[db] = (f32x16){};

    // MASKED: the tile holds keys past n_kv or (causal) keys after some row
    // of this wave; only such tiles carry the compare and select per element
    auto tile = [&](auto par, auto msk, int t) {
        constexpr int PAR = decltype(par)::value;
        constexpr bool MASKED = decltype(msk)::value;
        wait_vm();
        __syncthreads();
        if (t + 1 < ntile) {
            kplan.issue(kh, (t + 1) * C::BC, n_kv, kbuf(1 - PAR), w, lane);
            vplan.issue(vh, (t + 1) * C::BC, n_kv, vbuf(1 - PAR), w, lane);
        }
        if (t >= wn) return;
        f32x16 s[C::KB], dp[C::KB];
        // reads ahead: as many as the register budget of two waves per SIMD allows
        constexpr int LQ = C::DROP && C::D >= 128 ? 4 : 6;
        // the wave issuing S and dP takes issue priority over the other wave
        // of its SIMD, which is then in its VALU or dQ part (measured +2 %
        // at d = 128; no effect with one wave per SIMD)
        __builtin_amdgcn_s_setprio(1);
        qk_dq_rolling<C, LQ>(s, dp, kbuf(PAR), vbuf(PAR), koff_k, koff_v, qf, gf);
        __builtin_amdgcn_s_setprio(0);
        // keys past n_kv, and (causal) keys after qi, have P = 0
        const int lim = C::CAUSAL ? min(n_kv, qi + 1) : n_kv;
        v8 ds[C::KB][2];
        // dropout keep bits: keys t BC + 32 kb + 16 k2 + 8 half + 4 h + (0..3)
        // are block t BC/4 + h + 2 (4 kb + 2 k2 + half)
        unsigned kq[C::KB] = {};
        if (C::DROP) {
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
                kq[kb] = drop_group_bits<false>(dr, (unsigned)(t * C::BC >> 2) + h, kb);
        }
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                // dropout: dP of a dropped element is 0, a kept one is scaled
                const unsigned keep = C::DROP ? (kq[kb] >> (8 * k2)) & 0xFFu : 0xFFu;
                v8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 8 * k2 + e;
                    float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -lse2));
                    if constexpr (MASKED) {
                        const int key = t * C::BC + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        pr = key < lim ? pr : 0.f;
                    }
                    const float dpz = C::DROP ? (((keep >> e) & 1u) ? dp[kb][r] * p.drop_scale : 0.f) : dp[kb][r];
                    x[e] = (T)(pr * (dpz - dlt));
                }
                ds[kb][k2] = x;
            }
        pv_dq_rolling<C, 4>(dq, kbuf(PAR), voff, ds);
    };
    // Tiles [0, tu) need no mask for any row of this wave (all keys below n_kv
    // and, causal, at most the wave's first row); they run in pairs with
    // compile-time buffers and no per-element compare.  The rest run with the
    // mask.  Every wave passes one barrier per tile either way.  With dropout
    // every tile takes the masked body (a second body would spill).
    const std::integral_constant<int, 0> p0;
    const std::integral_constant<int, 1> p1;
    const std::false_type full;
    const std::true_type part;
    int tu = C::DROP ? 0 : n_kv / C::BC;
    if (C::CAUSAL) tu = min(tu, (wq0 + 1) / C::BC);
    int t = 0;
    if constexpr (!C::DROP) {
        for (; t + 2 <= tu; t += 2) {
            tile(p0, full, t);
            tile(p1, full, t + 1);
        }
    }
    for (; t < ntile; ++t) {
        if (t & 1)
            tile(p1, part, t);
        else
            tile(p0, part, t);
    }
    if constexpr (C::D <= 128) {
        // dQ leaves through LDS as whole rows (store_rows_staged), in the
        // tile buffers once every wave is past its last read of K and V
        static_assert(C::BR <= 4 * C::BC, "dQ staging must fit the four tile buffers");
        __syncthreads();
        if (wq0 >= n_q) return;
        constexpr int WPB = C::BC / 32;  // waves per tile buffer
        const int b = w / WPB;
        char *stage = (b == 0 ? sk0 : b == 1 ? sk1 : b == 2 ? sv0 : sv1) + (w % WPB) * 32 * C::RB;
        store_rows_staged<C>(stage, p.dq + ((int64_t)bh * n_q + wq0) * C::RB, n_q - wq0, dq, p.scale, lane);
    } else {
        if (qi < n_q) store_rows<C, C::QDB, C::QDB0>(p.dq + ((int64_t)bh * n_q + qi) * C::RB, dq, p.scale, h);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (batch*head, block of 32*NW keys), streaming Q
// and dO tiles of 64 query rows (both in the layout read both ways: by rows
// and transposed) with the tiles' LSE_i log2(e) and D_i (LDS, after the
// four tile buffers: [0, 256) LSE, [256, 512) D per buffer).
template <class C>
__global__ __launch_bounds__(C::NT, C::MIN_WAVES) void bwd_dkdv_kernel(BwdParams p) {
    typedef typename C::T T;
    typedef Mma16<T> M;
    typedef typename M::v8 v8;
    // separate LDS objects per stream and buffer, so that reads of one buffer
    // are not held up by the copies in flight into the other (the unmasked
    // loop below picks every buffer at compile time)
    __shared__ __attribute__((aligned(1024))) char sq0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sq1[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sg0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sg1[C::TILE];
    __shared__ __attribute__((aligned(16))) char ss0[512];
    __shared__ __attribute__((aligned(16))) char ss1[512];
    auto qbuf = [&](int i) { return i ? sq1 : sq0; };
    auto gbuf = [&](int i) { return i ? sg1 : sg0; };
    auto sbuf = [&](int i) { return i ? ss1 : ss0; };

    const int lane = lane_id();
    const int w = wave_id();
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int n_kblk = (p.n_kv + C::BR - 1) / C::BR;
    const int bid = xcd_remap(blockIdx.x, p.n_bh * n_kblk);
    const int bh = bid / n_kblk;
    const int kb0 = bid - bh * n_kblk;
    const int k0 = kb0 * C::BR;
    const int wk0 = k0 + 32 * w;   // first key of this wave
    const int kj = wk0 + l32;       // this lane's key
    const int n_q = p.n_q, n_kv = p.n_kv;

    const char *qh = p.q + (int64_t)bh * n_q * C::RB;
    const char *gh = p.dout + (int64_t)bh * n_q * C::RB;
    const float *lh = p.lse2 + (int64_t)bh * n_q;
    const float *dh = p.delta + (int64_t)bh * n_q;

    // query tiles [t0, ntile): causal rows before the block's first key see none of it
    const int ntile = (n_q + C::BC - 1) / C::BC;
    const int t0 = C::CAUSAL ? min(k0 / C::BC, ntile) : 0;
    const int wt0 = C::CAUSAL ? min(wk0 / C::BC, ntile) : 0;  // this wave's first tile

    const CopyPlan<C, kLayoutBoth> plan(w, lane);
    // LSE and D of tile t (wave 0: lanes 0-15 fetch LSE rows 4i..4i+3, lanes
    // 16-31 the same rows of D); rows past n_q read as 0 through the buffer
    // descriptors' bounds (their P is forced to 0 below)
    auto issue_stats = [&](int t, char *dst) {
        if (w == 0) {
            const int rows = min(C::BC, n_q - t * C::BC);
            if (lane < 16)
                copy16_to_lds(make_rsrc(lh + t * C::BC, rows * 4), 16 * lane, dst);
            else if (lane < 32)
                copy16_to_lds(make_rsrc(dh + t * C::BC, rows * 4), 16 * (lane - 16), dst);
        }
    };
    auto issue = [&](int t, int b) {
        plan.issue(qh, t * C::BC, n_q, qbuf(b), w, lane);
        plan.issue(gh, t * C::BC, n_q, gbuf(b), w, lane);
        issue_stats(t, sbuf(b));
    };
    if (t0 < ntile) issue(t0, t0 & 1);

    v8 kf[C::KS], vf[C::KS];
    load_rows<C>(p.k + (int64_t)bh * n_kv * C::RB, kj, n_kv, kf, h);
    if (C::WANT_DK) load_rows<C>(p.v + (int64_t)bh * n_kv * C::RB, kj, n_kv, vf, h);
    const float c = p.c;
    DropQuad dc{};
    if (C::DROP) dc = make_drop_quad(p.p8, (unsigned)kj >> 2, (unsigned)bh, p.drop_off, p.seed_lo, p.seed_hi);
    const int koff = row_offset_b<C>(lane);
    const TrOffsets voff = tr_offsets<C>(lane);

    f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
        dk[db] = (f32x16){};
        dv[db] = (f32x16){};
    }

    // P and dS of one 32-row block kb of the tile (VALU), from its S and dP
    auto elementwise = [&](auto mk, int t, const float *st, int kb, const f32x16 &s, const f32x16 &dp,
                           v8 (&pb)[2], v8 (&ds)[2]) {
        constexpr bool MK = decltype(mk)::value;
        // dropout keep bits: rows t BC + 32 kb + 16 k2 + 8 half + 4 h + (0..3)
        // are block t BC/4 + h + 2 (4 kb + 2 k2 + half)
        const unsigned kq = C::DROP ? drop_group_bits<true>(dc, (unsigned)(t * C::BC >> 2) + h, kb) : 0u;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            // rows 32 kb + 16 k2 + 8 (e/4) + 4 h + e%4 of the tile
            const unsigned keep = C::DROP ? (kq >> (8 * k2)) & 0xFFu : 0xFFu;
            const f32x4 l_lo = *(const f32x4 *)(st + 32 * kb + 16 * k2 + 4 * h);
            const f32x4 l_hi = *(const f32x4 *)(st + 32 * kb + 16 * k2 + 8 + 4 * h);
            const f32x4 d_lo = *(const f32x4 *)(st + 64 + 32 * kb + 16 * k2 + 4 * h);
            const f32x4 d_hi = *(const f32x4 *)(st + 64 + 32 * kb + 16 * k2 + 8 + 4 * h);
            v8 xp, xs;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 8 * k2 + e;
                const float l2 = e < 4 ? l_lo[e & 3] : l_hi[e & 3];
                const float dl = e < 4 ? d_lo[e & 3] : d_hi[e & 3];
                float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l2));
                if (MK) {
                    // rows past n_q, and (causal) rows before this lane's key, have P = 0
                    const int q = t * C::BC + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                    pr = (q < n_q && (!C::CAUSAL || kj <= q)) ? pr : 0.f;
                }
                // dropout: P o keep for dV (the 1/(1-p) goes into the dV store),
                // dP of a dropped element 0 and of a kept one scaled
                const bool kept = !C::DROP || ((keep >> e) & 1u);
                if (C::WANT_DV) xp[e] = (T)(kept ? pr : 0.f);
                if (C::WANT_DK) xs[e] = (T)(pr * ((C::DROP ? (kept ? dp[r] * p.drop_scale : 0.f) : dp[r]) - dl));
            }
            if (C::WANT_DV) pb[k2] = xp;
            if (C::WANT_DK) ds[k2] = xs;
        }
    };
    // One tile, software-pipelined over its two 32-row blocks in four
    // scheduling segments: S, dP of block 0; S, dP of block 1 under the VALU
    // of block 0; dV, dK of block 0 under the VALU of block 1; dV, dK of
    // block 1.
    auto body = [&](auto mk, int t, const char *qt, const char *gt, const char *sb) {
        const float *st = (const float *)sb;
        f32x16 s[2], dp[2];
        v8 pb[2][2], ds[2][2];
        constexpr int NPROD = C::PART == 0 ? 2 : 1;
        constexpr int NQK = (C::WANT_DK ? 2 : 1) * C::KS, NPV = 2 * NPROD * C::DB;  // MFMAs per block
        auto qk = [&](int blk) {
            if (C::WANT_DK)
                qk_rows2<C>(s[blk], dp[blk], qt + 32 * blk * C::RB, gt + 32 * blk * C::RB, koff, kf, vf);
            else
                qk_rows1<C>(s[blk], qt + 32 * blk * C::RB, koff, kf);
        };
        auto pv = [&](int blk) {
            if (C::PART == 0)
                pv_rows2<C>(dv, gt + 32 * blk * C::RB, pb[blk], dk, qt + 32 * blk * C::RB, ds[blk], voff);
            else if (C::WANT_DV)
                pv_rows1<C>(dv, gt + 32 * blk * C::RB, pb[blk], voff);
            else
                pv_rows1<C>(dk, qt + 32 * blk * C::RB, ds[blk], voff);
        };
        // segment A: S, dP of block 0
        qk(0);
        __builtin_amdgcn_sched_barrier(0);
        // segment B: S, dP of block 1 under the VALU of block 0
        qk(1);
        elementwise(mk, t, st, 0, s[0], dp[0], pb[0], ds[0]);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // segment C: dV, dK of block 0 under the VALU of block 1
        pv(0);
        elementwise(mk, t, st, 1, s[1], dp[1], pb[1], ds[1]);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        // segment D: dV, dK of block 1
        pv(1);
    };
    // The same tile (both products, no dropout, d = 128) as one stream of
    // MFMAs with every operand read issued RL steps ahead of its MFMA, across
    // the segment boundaries, so that no segment starts by waiting for its
    // reads.  Steps [0, NQ): S and dP of block 0; [NQ, 2 NQ): those of block
    // 1; [2 NQ, 2 NQ + NP): dV and dK of block 0; then those of block 1.  The
    // VALU of block 0 runs one element (d = 64: two) per step over steps
    // NQ + 1 .. 2 NQ, after the last dP MFMA of block 0 has had a step to
    // finish; that of block 1 over steps 2 NQ + 1 .. 3 NQ.  Each block's
    // first 8 elements (k2 = 0) are complete before its first dV/dK MFMA,
    // the other 8 before the first MFMA that reads them (k2 = 1).
    auto body_roll = [&](auto mk, int t, const char *qt, const char *gt, const char *sb) {
        constexpr bool MK = decltype(mk)::value;
        constexpr int NQ = 2 * C::KS, NP = 4 * C::DB, N = 2 * (NQ + NP), RL = 4;
        constexpr int EPS = 16 / NQ;  // elements per step
        static_assert(NQ == NP && 16 % NQ == 0, "one VALU window per product segment");
        const float *st = (const float *)sb;
        f32x16 s[2], dp[2];
        v8 pb[2][2], ds[2][2];
        f32x4 stt[2][4];  // LSE and D of the block whose VALU runs: [k2][l_lo, l_hi, d_lo, d_hi]
        auto rd = [&](int i) -> v8 {
            if (i < 2 * NQ) {
                const int blk = i / NQ, j = i % NQ, ks = j >> 1;
                const char *base = ((j & 1) ? gt : qt) + 32 * blk * C::RB;
                return *(const v8 *)(base + ((koff ^ (32 * (ks & 7))) + 256 * (ks >> 3)));
            }
            const int i2 = i - 2 * NQ, blk = i2 / NP, j = i2 % NP;
            const int k2 = j / (2 * C::DB), db = (j >> 1) % C::DB;
            const char *base = ((j & 1) ? qt : gt) + (32 * blk + 16 * k2) * C::RB + 256 * (db >> 2);
            const i16x4 lo = lds_read_tr16(base + voff.lo[db & 3]);
            const i16x4 hi = lds_read_tr16(base + tr_hi<C>(voff, db & 3));
            return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        auto load_stats = [&](int kb) {
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                stt[k2][0] = *(const f32x4 *)(st + 32 * kb + 16 * k2 + 4 * h);
                stt[k2][1] = *(const f32x4 *)(st + 32 * kb + 16 * k2 + 8 + 4 * h);
                stt[k2][2] = *(const f32x4 *)(st + 64 + 32 * kb + 16 * k2 + 4 * h);
                stt[k2][3] = *(const f32x4 *)(st + 64 + 32 * kb + 16 * k2 + 8 + 4 * h);
            }
        };
        // element x (k2 = x / 8, e = x % 8) of P and dS of block kb
        auto elem = [&](int kb, int x) {
            const int k2 = x >> 3, e = x & 7, r = 8 * k2 + e;
            const float l2 = e < 4 ? stt[k2][0][e & 3] : stt[k2][1][e & 3];
            const float dl = e < 4 ? stt[k2][2][e & 3] : stt[k2][3][e & 3];
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -l2));
            if (MK) {
                const int q = t * C::BC + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                pr = (q < n_q && (!C::CAUSAL || kj <= q)) ? pr : 0.f;
            }
            pb[kb][k2][e] = (T)pr;
            ds[kb][k2][e] = (T)(pr * (dp[kb][r] - dl));
        };
        v8 buf[RL];
#pragma unroll
        for (int j = 0; j < RL; ++j) buf[j] = rd(j);
        static_for<N>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const v8 a = buf[i % RL];
            if (i < 2 * NQ) {
                const int blk = i / NQ, j = i % NQ, ks = j >> 1;
                if (j & 1)
                    dp[blk] = M::mma(a, vf[ks], ks == 0 ? (f32x16){} : dp[blk]);
                else
                    s[blk] = M::mma(a, kf[ks], ks == 0 ? (f32x16){} : s[blk]);
            } else {
                const int i2 = i - 2 * NQ, blk = i2 / NP, j = i2 % NP;
                const int k2 = j / (2 * C::DB), db = (j >> 1) % C::DB;
                if (j & 1)
                    dk[db] = M::mma(a, ds[blk][k2], dk[db]);
                else
                    dv[db] = M::mma(a, pb[blk][k2], dv[db]);
            }
            if (i + RL < N) buf[i % RL] = rd(i + RL);
            if (i == NQ) load_stats(0);
            if (i > NQ && i <= 2 * NQ) {
#pragma unroll
                for (int u = 0; u < EPS; ++u) elem(0, (i - NQ - 1) * EPS + u);
            }
            // after block 0's last element, which runs in this same step
            if (i == 2 * NQ) load_stats(1);
            if (i > 2 * NQ && i <= 3 * NQ) {
#pragma unroll
                for (int u = 0; u < EPS; ++u) elem(1, (i - 2 * NQ - 1) * EPS + u);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // (at d = 64 the two waves per SIMD leave no room for the read window)
    constexpr bool ROLL = !C::DROP && C::PART == 0 && C::D == 128;
    auto run_body = [&](auto mk, int t, const char *qt, const char *gt, const char *sb) {
        if constexpr (ROLL)
            body_roll(mk, t, qt, gt, sb);
        else
            body(mk, t, qt, gt, sb);
    };
    auto sync_issue = [&](int t) {
        wait_vm();
        __syncthreads();
        if (t + 1 < ntile) issue(t + 1, 1 - (t & 1));
    };
    static_assert(C::KB == 2, "two 32-row blocks per tile");
    // Tiles in order, each loop with one body (a branch between a masked and
    // an unmasked body inside one loop makes the compiler move the dK, dV
    // accumulators between AGPRs and VGPRs on every tile):
    //   [t0, wt0)        rows before this wave's keys: barriers and copies only
    //   [wt0, tm)        causal: tiles below some key of this wave, masked
    //   [tm, tf)         full tiles, unmasked
    //   [tf, ntile)      the ragged last tile, masked
    const int tm = C::CAUSAL ? max(wt0, min(ntile, (wk0 + 31) / C::BC + 1)) : wt0;
    const int tf = max(tm, min(ntile, n_q / C::BC));
    auto pin = [&]() {
        // keeps the accumulators in AGPRs across iterations
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            if (C::WANT_DK) asm volatile("" : "+a"(dk[db]));
            if (C::WANT_DV) asm volatile("" : "+a"(dv[db]));
        }
    };
    // tile t with its buffers chosen at run time
    auto tile_rt = [&](auto mk, int t) {
        sync_issue(t);
        const int b = t & 1;
        run_body(mk, t, qbuf(b), gbuf(b), sbuf(b));
        pin();
    };
    // tile t of parity PAR, buffers fixed
    auto tile_ct = [&](auto par, int t) {
        constexpr int PAR = decltype(par)::value;
        wait_vm();
        __syncthreads();
        if (t + 1 < ntile) {
            plan.issue(qh, (t + 1) * C::BC, n_q, PAR ? sq0 : sq1, w, lane);
            plan.issue(gh, (t + 1) * C::BC, n_q, PAR ? sg0 : sg1, w, lane);
            issue_stats(t + 1, PAR ? ss0 : ss1);
        }
        run_body(std::integral_constant<bool, false>(), t, PAR ? sq1 : sq0, PAR ? sg1 : sg0, PAR ? ss1 : ss0);
        pin();
    };
    int t = t0;
    for (; t < wt0; ++t) sync_issue(t);
    for (; t < tm; ++t) tile_rt(std::integral_constant<bool, true>(), t);
    if constexpr (C::DROP) {
        // (one body: the dropout bodies do not fit four copies in registers)
        for (; t < tf; ++t) tile_rt(std::integral_constant<bool, false>(), t);
    } else {
        if (t < tf && (t & 1)) tile_rt(std::integral_constant<bool, false>(), t++);
        for (; t + 1 < tf; t += 2) {
            tile_ct(std::integral_constant<int, 0>(), t);
            tile_ct(std::integral_constant<int, 1>(), t + 1);
        }
        if (t < tf) tile_rt(std::integral_constant<bool, false>(), t++);
    }
    for (; t < ntile; ++t) tile_rt(std::integral_constant<bool, true>(), t);
    if constexpr (C::D <= 128) {
        // dK and dV leave through LDS as whole rows (store_rows_staged), one
        // after the other in the same staging rows of the tile buffers, once
        // every wave is past its last read of Q and dO
        static_assert(C::BR <= 4 * C::BC, "dK/dV staging must fit the four tile buffers");
        __syncthreads();
        if (wk0 >= n_kv) return;
        constexpr int WPB = C::BC / 32;  // waves per tile buffer
        const int b = w / WPB;
        char *stage = (b == 0 ? sq0 : b == 1 ? sq1 : b == 2 ? sg0 : sg1) + (w % WPB) * 32 * C::RB;
        const int64_t row0 = (int64_t)bh * n_kv + wk0;
        if (C::WANT_DK) store_rows_staged<C>(stage, p.dk + row0 * C::RB, n_kv - wk0, dk, p.scale, lane);
        if (C::WANT_DV)
            store_rows_staged<C>(stage, p.dv + row0 * C::RB, n_kv - wk0, dv, C::DROP ? p.drop_scale : 1.f, lane);
    } else if (kj < n_kv) {
        const int64_t row = (int64_t)bh * n_kv + kj;
        if (C::WANT_DK) store_rows<C>(p.dk + row * C::RB, dk, p.scale, h);
        if (C::WANT_DV) store_rows<C>(p.dv + row * C::RB, dv, C::DROP ? p.drop_scale : 1.f, h);
    }
}

template <typename T, int D, int NWQ, int NWK, bool CAUSAL, bool DROP>
int launch_bwd_t(const BwdParams &p, void *stream) {
    // d = 256 with dropout: the dQ kernel as two passes over the two halves
    // of dQ's columns (each recomputes S and dP).  In one pass, the Philox
    // state on top of the full dQ accumulator exceeds the 512 registers of a
    // wave and spilled about 100 of them (3.2 times the time of the
    // dropout-free kernel).
    constexpr bool QSPLIT = D >= 256 && DROP;
    typedef CfgB<T, D, NWQ, CAUSAL, DROP, (QSPLIT ? 1 : 0)> CQ;
    typedef CfgB<T, D, NWQ, CAUSAL, DROP, 2> CQ2;
    // d = 256: the dK/dV kernel as two passes (dV, then dK), see above
    typedef CfgB<T, D, NWK, CAUSAL, DROP, (D >= 256 ? 1 : 0)> CK;
    typedef CfgB<T, D, NWK, CAUSAL, DROP, 2> CK2;
    hipStream_t st = (hipStream_t)stream;
    const int64_t rows = (int64_t)p.n_bh * p.n_q;
    if (rows > 0) {
        const int nq = (p.n_q + CQ::BR - 1) / CQ::BR;
        hipLaunchKernelGGL(bwd_dq_kernel<CQ>, dim3(p.n_bh * nq), dim3(CQ::NT), 0, st, p);
        if constexpr (QSPLIT) hipLaunchKernelGGL(bwd_dq_kernel<CQ2>, dim3(p.n_bh * nq), dim3(CQ2::NT), 0, st, p);
    }
    const int nk = (p.n_kv + CK::BR - 1) / CK::BR;
    hipLaunchKernelGGL(bwd_dkdv_kernel<CK>, dim3(p.n_bh * nk), dim3(CK::NT), 0, st, p);
    if constexpr (D >= 256) hipLaunchKernelGGL(bwd_dkdv_kernel<CK2>, dim3(p.n_bh * nk), dim3(CK2::NT), 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <typename T, int D, int NWQ, int NWK, bool CAUSAL>
int launch_bwd(const BwdParams &p, void *stream) {
    return p.p8 != 0 ? launch_bwd_t<T, D, NWQ, NWK, CAUSAL, true>(p, stream)
                     : launch_bwd_t<T, D, NWQ, NWK, CAUSAL, false>(p, stream);
}

// The dropout keep mask as bytes, one 4 x 4 block of one slice per thread
// (one Philox call).
__global__ __launch_bounds__(256) void dropout_mask_kernel(unsigned p8, unsigned k0, unsigned k1, unsigned off,
                                                           int64_t n_bh, int64_t n_q, int64_t n_kv,
                                                           unsigned char *mask) {
    const int64_t qb = (n_q + 3) / 4, kb = (n_kv + 3) / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_bh * qb * kb) return;
    const int64_t bh = idx / (qb * kb);
    const int64_t rest = idx - bh * qb * kb;
    const int64_t i4 = rest / kb, j4 = rest - (rest / kb) * kb;
    unsigned out[4];
    philox4x32_10((unsigned)j4, (unsigned)i4, (unsigned)bh, off, k0, k1, out);
    for (int a = 0; a < 4; ++a) {
        const int64_t i = 4 * i4 + a;
        if (i >= n_q) break;
        for (int b = 0; b < 4; ++b) {
            const int64_t j = 4 * j4 + b;
            if (j >= n_kv) break;
            const unsigned byte = (out[a] >> (8 * b)) & 0xFFu;
            mask[(bh * n_q + i) * n_kv + j] = (p8 == 0 || byte >= p8) ? 1 : 0;
        }
    }
}

}  // namespace

int launch_dropout_mask(unsigned p8, unsigned seed_lo, unsigned seed_hi, unsigned off, int64_t n_bh,
                        int64_t n_q, int64_t n_kv, unsigned char *mask, void *stream) {
    const int64_t n = n_bh * ((n_q + 3) / 4) * ((n_kv + 3) / 4);
    if (n == 0) return 0;
    hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, p8, seed_lo, seed_hi, off, n_bh, n_q, n_kv, mask);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

#define FA_B16(T, DT, D, NWQ, NWK, CAUSAL)                                                  \
    BwdVariant{DT, D, CAUSAL, "dq_w" #NWQ "_dkdv_w" #NWK, &launch_bwd<T, D, NWQ, NWK, CAUSAL>}

// Host-side table of the compiled backward variants.
const BwdVariant *bwd_variants(int *count) {
    static const BwdVariant table[] = {
        FA_B16(__bf16, FA_BF16, 64, 8, 4, 0),   FA_B16(__bf16, FA_BF16, 64, 8, 4, 1),
        FA_B16(__bf16, FA_BF16, 128, 8, 4, 0),  FA_B16(__bf16, FA_BF16, 128, 8, 4, 1),
        FA_B16(_Float16, FA_F16, 64, 8, 4, 0),  FA_B16(_Float16, FA_F16, 64, 8, 4, 1),
        FA_B16(_Float16, FA_F16, 128, 8, 4, 0), FA_B16(_Float16, FA_F16, 128, 8, 4, 1),
        FA_B16(__bf16, FA_BF16, 256, 4, 4, 0),  FA_B16(__bf16, FA_BF16, 256, 4, 4, 1),
        FA_B16(_Float16, FA_F16, 256, 4, 4, 0), FA_B16(_Float16, FA_F16, 256, 4, 4, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
