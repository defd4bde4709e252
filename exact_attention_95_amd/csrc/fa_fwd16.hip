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
// the division to the end).
//
// The loop is software-pipelined by one tile: iteration j issues the MFMAs
// of S_{j+1} = K_{j+1} Q^T, then the MFMAs of O += V_j^T P_j^T together with
// the softmax (VALU) of S_{j+1}, so the exponentials of one tile overlap the
// matrix products of the previous one.  A rescale of O decided by the
// softmax of tile j+1 is applied at the start of iteration j+1, before P_{j+1}
// is accumulated.  K and V tiles have two LDS buffers each and are filled by
// direct copies to LDS (buffer_load_dwordx4 ... lds): K two tiles ahead, V
// one tile ahead.  The causal variant stops at the diagonal tile (plate 07:
// the mask is fused into the kernel) and masks only the tiles that straddle
// it.
#include <type_traits>

#include "fa_device.h"
#include "fa_tile16.h"
#include "../../include/fa.h"

namespace fa {
namespace {

// SPLIT: the workgroup covers one chunk of the key range (split-KV) and
// writes a float32 partial output and LSE instead of O.
// DROP: P is multiplied by the dropout keep mask before the PV product.
template <typename T_, int D_, int NW_, int BC_, bool CAUSAL_, bool SPLIT_ = false, bool DROP_ = false>
struct Cfg {
    typedef T_ T;
    static constexpr int D = D_, NW = NW_, BC = BC_, NT = NW * 64, BR = 32 * NW;
    static constexpr bool SPLIT = SPLIT_, DROP = DROP_;
    typedef Cfg<T_, D_, NW_, BC_, CAUSAL_, SPLIT_, true> WithDrop;
    // waves per SIMD the register budget must allow: workgroups of 4 waves
    // with d <= 128 run two per CU (the split kernels are bound by HBM and
    // want them in flight; at d = 64 the two workgroups' waves on a SIMD
    // are not tied by one barrier and overlap each other's softmax).  At
    // d = 256 every kernel, split or not, needs one SIMD's registers per wave.
    static constexpr int MIN_WAVES = ((SPLIT_ || NW_ == 4) && D_ <= 128) ? 2 : 1;
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr int RB = D * 2;                      // LDS / global row bytes
    static constexpr int NC = RB / 16;                    // 16-byte chunks per row
    static constexpr int RPB = RB >= 256 ? 1 : 256 / RB;  // rows per 256-byte bank window
    static constexpr int KX = (NC < 16 ? NC : 16) - 1;    // K chunk swizzle mask
    static constexpr int VX = (NC / 4 < 4 ? NC / 4 : 4) - 1;  // V swizzle mask (4-chunk units)
    static constexpr int TILE = BC * RB;                  // bytes of one K or V tile
    static constexpr int LDS = 4 * TILE;                  // K0, K1, V0, V1
    static constexpr int KS = D / 16;                     // k-steps of S^T = K Q^T
    static constexpr int KB = BC / 32;                    // 32-key blocks per tile
    static constexpr int DB = D / 32;                     // 32-row blocks of O^T
    static constexpr int LDI = TILE / (1024 * NW);        // copy instructions per wave per tile
    static constexpr int NVO = DB < 4 ? DB : 4;           // distinct V read offsets per lane
    static constexpr float TAU = 8.0f;
    // d = 256 runs one wave per SIMD and needs more than the 256 arch VGPRs:
    // the read-only Q operand (64 registers) is kept in AGPRs, which the
    // MFMAs read directly, and O, S and P stay in arch VGPRs
    static constexpr bool Q_IN_AGPR = D_ >= 256;
    static_assert(TILE % (1024 * NW) == 0, "tile must split into whole wave copies");
    static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Masks the scores of one S^T tile for this lane's query row qi: keys past
// n_kv, and (causal) keys after qi, become -inf.
template <class C>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[C::KB], int t0, int qi, int n_kv, int h) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = t0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool vis = key < n_kv && (!C::CAUSAL || key <= qi);
            s[kb][r] = vis ? s[kb][r] : kNegInf;
        }
}

// Online-softmax step for one tile of S^T (this lane's query row): takes
// the row max, raises the reference max m_use if the tile max exceeds it by
// more than TAU (wave-uniform decision, returned in `raised` with the factor
// alpha that O must still be multiplied by), and writes P = exp2(S c - m_use)
// as the MFMA operand type into pb while accumulating this half-wave's share
// of the row sum (of the float32 P, before rounding) into l_acc.  c > 0, so
// masked scores (-inf) give P = 0.
template <class C>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[C::KB],
                                             typename Mma16<typename C::T>::v8 (&pb)[C::KB][2],
                                             float &m_use, float &l_acc, float &alpha, bool &raised,
                                             float c, const DropQuad &dq = DropQuad{}, int t0 = 0) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    typedef typename C::T T;
    float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], s[kb][r]);
    const float mt = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * c;
    raised = __any(mt > m_use + C::TAU);
    const float m_new = raised ? fmaxf(m_use, mt) : m_use;
    alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_use - m_new);
    l_acc *= alpha;
    m_use = m_new;
    const float mref = (m_use == kNegInf) ? 0.f : m_use;
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
    const int h = lane_id() >> 5;
    // keys t0 + 32 kb + 16 k2 + 8 half + 4 h + (0..3) are block t0/4 + h + 2 (4 kb + 2 k2 + half)
    unsigned kq[C::KB] = {};
    if (C::DROP) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) kq[kb] = drop_group_bits<false>(dq, (unsigned)(t0 >> 2) + h, kb);
    }
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            // register 8 k2 + e holds key t0 + 32 kb + 8 (2 k2 + e/4) + 4 h + e%4
            unsigned keep = 0xFFu;
            if (C::DROP) keep = (kq[kb] >> (8 * k2)) & 0xFFu;
            v8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * k2 + e], c, -mref));
                l4[e & 3] += v;  // the row sum is that of the scores, before dropout
                x[e] = (T)(((keep >> e) & 1u) ? v : 0.f);
            }
            pb[kb][k2] = x;
        }
    }
    l_acc += (l4[0] + l4[1]) + (l4[2] + l4[3]);
}

// Instruction order for the compiler's scheduler.  S^T MFMAs: each K read
// one MFMA ahead.  PV MFMAs: each preceded by the two transposed V reads it
// needs and followed by a share of the softmax VALU work, so that the
// exponentials issue while the matrix core is busy and only a few operands
// are in flight at a time.
template <class C>
__device__ __forceinline__ void schedule_qk() {
    constexpr int N = C::KB * C::KS;
    constexpr int AHEAD = N < 4 ? N : 4;
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS read
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}
template <class C>
__device__ __forceinline__ void schedule_pv_softmax() {
    constexpr int NPV = C::DB * C::KB * 2;
    constexpr int VALU = 120 * C::KB / 2;  // softmax VALU instructions, about
    constexpr int VPM = (VALU + NPV - 1) / NPV;
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // VALU
    }
}

template <class C>
__global__ __launch_bounds__(C::NT, C::MIN_WAVES) void fwd16_kernel(KParams p) {
    typedef typename C::T T;
    typedef Mma16<T> M;
    typedef typename M::v8 v8;
    typedef typename M::v4 v4;
    // LDS: K buffers 0 and 1, V buffers 0 and 1, as four separate objects so
    // that the compiler can tell a read of one buffer from a copy in flight
    // into another (with one array it waits for every outstanding copy before
    // each LDS read)
    __shared__ __attribute__((aligned(1024))) char sk0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sk1[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sv0[C::TILE];
    __shared__ __attribute__((aligned(1024))) char sv1[C::TILE];
    // Single pass, d <= 128: O leaves through LDS, so that global memory
    // sees whole rows, 1 KB per store instruction, instead of 8-byte pieces
    // of 32 rows (the MFMA accumulator layout).  At d = 64, Q arrives the
    // same way, by direct-to-LDS copies of whole rows, into a buffer of its
    // own (each wave owning 32 rows) that O reuses.  At d = 128 that buffer
    // (64 KB) would leave LDS room for one workgroup per CU, and the
    // compiler then schedules for that occupancy and spills; there O is
    // staged in the tile buffers once every wave is done with them.  Rows
    // use the K swizzle, which keeps the row-wise copies and reads and the
    // column-wise operand reads and accumulator writes free of bank
    // conflicts.  At d = 256 staging O measured slower.
    constexpr bool STAGE_O = !C::SPLIT && C::D <= 128;
    constexpr bool STAGE = STAGE_O && C::D <= 64;
    __shared__ __attribute__((aligned(1024))) char sq[STAGE ? C::BR * C::RB : 16];
    auto kbuf = [&](int i) { return i ? sk1 : sk0; };
    auto vbuf = [&](int i) { return i ? sv1 : sv0; };

    const int lane = lane_id();
    const int w = wave_id();
    const int h = lane >> 5;     // half-wave
    const int l32 = lane & 31;

    // ---- which (head, query block) ----
    int bid = xcd_remap(blockIdx.x, p.n_wg);
    int split = 0;
    if (C::SPLIT) {
        const int per = p.n_bh * p.n_qblk;
        split = bid / per;
        bid -= split * per;
    }
    const int bh = bid / p.n_qblk;
    int qb = bid - bh * p.n_qblk;
    if (C::CAUSAL) qb = p.n_qblk - 1 - qb;  // longest rows first
    const int q0 = qb * C::BR;
    const int wq0 = q0 + w * 32;             // first query row of this wave
    const int qi = wq0 + l32;                 // this lane's query row
    const int n_q = p.n_q;
    // Keys [kofs, kofs + n_kv) of the head; the causal comparisons below use
    // query indices shifted by -kofs so that they stay relative to this range.
    const int kofs = C::SPLIT ? split * p.kv_split : 0;
    const int n_kv = C::SPLIT ? min(p.kv_split, p.n_kv - kofs) : p.n_kv;
    const int rq0 = q0 - kofs, rwq0 = wq0 - kofs, rqi = qi - kofs;

    const char *qh = p.q + (int64_t)bh * n_q * C::RB;
    const char *kh = p.k + ((int64_t)bh * p.n_kv + kofs) * C::RB;
    const char *vh = p.v + ((int64_t)bh * p.n_kv + kofs) * C::RB;

    // tiles streamed by the workgroup, and tiles this wave computes
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
    (void)rq0;
    // tile t needs masking past n_kv, or when it reaches above this wave's first row
    auto need_mask = [&](int t) {
        return (t + 1) * C::BC > n_kv || (C::CAUSAL && (t + 1) * C::BC - 1 > rwq0);
    };

    const CopyPlan<C, kLayoutK> kplan(w, lane);
    const CopyPlan<C, kLayoutV> vplan(w, lane);
    char *qst = sq + (STAGE ? w * 32 * C::RB : 0);  // this wave's rows of Q, then of O
    if constexpr (STAGE) {
        // rows past n_q (a ragged last block) repeat the last row
        const int qr0 = min(wq0, n_q - 1);
        const int avail = min(n_q - qr0, 32);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(qh + (int64_t)qr0 * C::RB, avail * C::RB);
#pragma unroll
        for (int i = 0; i < C::RB / 32; ++i) {
            const int r = (64 * i + lane) / C::NC, pc = lane % C::NC;
            const int gr = min(r, avail - 1);
            copy16_to_lds(rs, (unsigned)(gr * C::RB + 16 * (pc ^ kswz<C>(r))), qst + 1024 * i);
        }
    }
    if (ntile > 0) {
        kplan.issue(kh, 0, n_kv, kbuf(0), w, lane);
        vplan.issue(vh, 0, n_kv, vbuf(0), w, lane);
    }
    if (ntile > 1) kplan.issue(kh, C::BC, n_kv, kbuf(1), w, lane);

    // ---- Q^T operand: lane holds Q[qi][ks*16 + 8h .. +7] for every k-step ----
    v8 qf[C::KS];
    if constexpr (!STAGE) {
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
    const int koff = l32 * C::RB + 16 * (h ^ kswz<C>(l32));
    // V^T operand via transposed reads: the 16-lane group g = lane/16 covers
    // rows kbase + 4h + (lane%16)/4 and columns 32*dblk + 16*(g%2) + 4*(lane%4).
    int voff[C::NVO];
    {
        const int j = lane & 15;
        const int rsub = 4 * h + (j >> 2);               // row within a group of 8
        const int x = vswz<C>(j >> 2) >> 2;              // swizzle of that row, in 4-chunk units
        const int y = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
#pragma unroll
        for (int db = 0; db < C::NVO; ++db)
            voff[db] = rsub * C::RB + 16 * (4 * (db ^ x) + y) + 8 * (j & 1);
    }

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = (f32x16){};
    float m_use = kNegInf;   // reference max (log2 units) of this lane's query row
    float l_acc = 0.f;       // this half-wave's share of the row sum
    float alpha = 1.f;       // pending rescale of O
    bool raised = false;
    const float c = p.c;
    DropQuad dr{};
    if (C::DROP) dr = make_drop_quad(p.p8, (unsigned)qi >> 2, (unsigned)bh, p.drop_off, p.seed_lo, p.seed_hi);
    v8 p0[C::KB][2], p1[C::KB][2];  // P of even / odd tiles

    wait_vm();
    __syncthreads();
    if constexpr (STAGE) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            u32x4 raw = *(const u32x4 *)(qst + l32 * C::RB + 16 * ((2 * ks + h) ^ kswz<C>(l32)));
            if (p.neg) raw ^= 0x80008000u;
            qf[ks] = __builtin_bit_cast(v8, raw);
        }
    }
    if (wn > 0) {
        f32x16 s[C::KB];
        qk_tile<C>(s, kbuf(0), koff, qf);
        if (need_mask(0)) mask_tile<C>(s, 0, rqi, n_kv, h);
        softmax_tile<C>(s, p0, m_use, l_acc, alpha, raised, c, dr, 0);
        raised = false;  // O is still zero
    }

    auto pin = [&]() {
        if constexpr (C::Q_IN_AGPR) {
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) asm volatile("" : "+a"(qf[ks]));
        }
    };
    pin();

    // One pipelined iteration for tile t (t % 2 == PAR): S_{t+1} and the
    // softmax of tile t+1 (into pn), PV of tile t (from pc).
    auto iteration = [&](auto par, int t, v8 (&pc)[C::KB][2], v8 (&pn)[C::KB][2]) {
        constexpr int PAR = decltype(par)::value;
        wait_vm();
        __syncthreads();
        if (t + 2 < ntile) kplan.issue(kh, (t + 2) * C::BC, n_kv, kbuf(PAR), w, lane);
        if (t + 1 < ntile) vplan.issue(vh, (t + 1) * C::BC, n_kv, vbuf(1 - PAR), w, lane);
        if (t >= wn) return;
        if (raised) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
        }
        if (t + 1 < wn) {
            f32x16 s[C::KB];
            const bool masked = need_mask(t + 1);
            qk_tile<C>(s, kbuf(1 - PAR), koff, qf);
            schedule_qk<C>();
            if (masked) mask_tile<C>(s, (t + 1) * C::BC, rqi, n_kv, h);
            // d = 64 (three waves per SIMD, bound by the softmax VALU): the
            // wave in its PV + softmax section takes issue priority over the
            // waves issuing S, so the exponentials of one wave keep flowing
            // while another's S MFMAs fill the matrix core
            if constexpr (C::D <= 64) __builtin_amdgcn_s_setprio(1);
            pv_tile<C>(o, vbuf(PAR), voff, pc);
            softmax_tile<C>(s, pn, m_use, l_acc, alpha, raised, c, dr, (t + 1) * C::BC);
            schedule_pv_softmax<C>();
            if constexpr (C::D <= 64) __builtin_amdgcn_s_setprio(0);
        } else {
            pv_tile<C>(o, vbuf(PAR), voff, pc);
        }
        pin();
    };
    for (int t = 0; t < ntile; t += 2) {
        iteration(std::integral_constant<int, 0>(), t, p0, p1);
        if (t + 1 >= ntile) break;
        iteration(std::integral_constant<int, 1>(), t + 1, p1, p0);
    }

    // ---- epilogue: O = O_acc / l, LSE = m + ln l ----
    if (C::SPLIT) {
        if (qi >= n_q) return;
        const float l_tot = sum_halves(l_acc);
        // partial of this key chunk, float32; a row that sees no key of the
        // chunk (causal) gets O = 0 and LSE = -inf, i.e. weight 0 in the merge
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
        if (h == 0) p.part_lse[row] = l_tot > 0.f ? (m_use + __log2f(l_tot)) * kLn2 : kNegInf;
        return;
    }
    if (!STAGE_O) {
        if (qi >= n_q) return;
        const float l_tot = sum_halves(l_acc);
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
        return;
    }
    // O leaves through 32 staging rows of this wave.  Without a buffer of
    // its own the wave uses part of the tile buffers, after a barrier that
    // lets the slowest wave finish its last reads of K and V.
    static_assert(STAGE || C::SPLIT || C::BR <= 4 * C::BC, "O staging must fit the four tile buffers");
    char *stage = qst;
    if constexpr (!STAGE) {
        __syncthreads();
        constexpr int WPB = C::BC / 32;  // waves per tile buffer
        const int b = w / WPB;
        stage = (b == 0 ? sk0 : b == 1 ? sk1 : b == 2 ? sv0 : sv1) + (w % WPB) * 32 * C::RB;
    }
    if (wq0 >= n_q) return;
    const float l_tot = sum_halves(l_acc);
    store_rows_staged<C>(stage, p.o + ((int64_t)bh * n_q + wq0) * C::RB, n_q - wq0, o, p.o_mul / l_tot, lane);
    if (p.lse && h == 0 && qi < n_q) p.lse[(int64_t)bh * n_q + qi] = (m_use + __log2f(l_tot)) * kLn2;
}

template <class C>
int launch(const KParams &p, void *stream) {
    if (p.p8 != 0) {
        // dropout instances exist for the single-pass kernels
        if constexpr (!C::SPLIT) {
            hipLaunchKernelGGL(fwd16_kernel<typename C::WithDrop>, dim3(p.n_wg), dim3(C::NT), 0,
                               (hipStream_t)stream, p);
            return hipGetLastError() == hipSuccess ? 0 : 1;
        }
        return 1;
    }
    hipLaunchKernelGGL(fwd16_kernel<C>, dim3(p.n_wg), dim3(C::NT), 0, (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

#define FA_V16(T, DT, D, NW, BC, CAUSAL)                                                   \
    Variant{DT, D, CAUSAL, 0, 32 * NW, "br" #NW "x32_bc" #BC, &launch<Cfg<T, D, NW, BC, CAUSAL>>}
#define FA_V16S(T, DT, D, NW, BC, CAUSAL)                                                  \
    Variant{DT, D, CAUSAL, 1, 32 * NW, "split_br" #NW "x32_bc" #BC,                        \
            &launch<Cfg<T, D, NW, BC, CAUSAL, true>>}
// Merge of split-KV partials (Flash-Decoding's final step, "Flash Attention
// 原理与实践" section 5.1), with the merge rule of "FlashAttention 与显存"
// plate 08 applied to whole chunks: for each row, L = log sum_s exp(L_s) and
// O = sum_s exp(L_s - L) O_s.  D/4 threads per row, four columns each.
template <typename TO, int D>
__global__ __launch_bounds__(256) void merge_kernel(KParams p) {
    constexpr int TPR = D / 4;
    const int64_t n_rows = (int64_t)p.n_bh * p.n_q;
    const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    if (row >= n_rows) return;
    const int col = (threadIdx.x % TPR) * 4;
    float mx = kNegInf;
    for (int s = 0; s < p.n_split; ++s) mx = fmaxf(mx, p.part_lse[s * n_rows + row]);
    float den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.n_split; ++s) {
        const float ls = p.part_lse[s * n_rows + row];
        const float wgt = ls == kNegInf ? 0.f : expf(ls - mx);
        den += wgt;
        acc += wgt * *(const f32x4 *)(p.part_o + (s * n_rows + row) * D + col);
    }
    const float inv = p.o_mul / den;
    TO *orow = (TO *)p.o + row * D + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = (TO)(acc[e] * inv);
    if (p.lse && col == 0) p.lse[row] = mx + logf(den);
}

template <typename TO, int D>
int launch_merge_t(const KParams &p, void *stream) {
    constexpr int RPB = 256 / (D / 4);
    const int64_t n_rows = (int64_t)p.n_bh * p.n_q;
    hipLaunchKernelGGL((merge_kernel<TO, D>), dim3((unsigned)((n_rows + RPB - 1) / RPB)), dim3(256), 0,
                       (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int launch_merge(int dtype, int d, const KParams &p, void *stream) {
    if (dtype == FA_BF16 && d == 64) return launch_merge_t<__bf16, 64>(p, stream);
    if (dtype == FA_BF16 && d == 128) return launch_merge_t<__bf16, 128>(p, stream);
    if (dtype == FA_F16 && d == 64) return launch_merge_t<_Float16, 64>(p, stream);
    if (dtype == FA_F16 && d == 128) return launch_merge_t<_Float16, 128>(p, stream);
    if (dtype == FA_BF16 && d == 256) return launch_merge_t<__bf16, 256>(p, stream);
    if (dtype == FA_FP8_E4M3 && d == 128) return launch_merge_t<__bf16, 128>(p, stream);  // bf16 O
    if (dtype == FA_F16 && d == 256) return launch_merge_t<_Float16, 256>(p, stream);
    return 1;
}

// Host-side table of the compiled 16-bit variants.
const Variant *variants16(int *count) {
    static const Variant table[] = {
        // default first: d = 64 runs 4-wave workgroups, three per CU
        // (measured 7-13 % faster than 8-wave workgroups on B=64 H=16
        // N=1024 and on causal N from 4096 to 65536)
        FA_V16(__bf16, FA_BF16, 64, 4, 64, 0),
        FA_V16(__bf16, FA_BF16, 64, 8, 128, 0),
        FA_V16(__bf16, FA_BF16, 64, 8, 64, 0),
        FA_V16(__bf16, FA_BF16, 64, 4, 64, 1),
        FA_V16(__bf16, FA_BF16, 64, 8, 128, 1),
        FA_V16(__bf16, FA_BF16, 64, 8, 64, 1),
        FA_V16(__bf16, FA_BF16, 128, 8, 64, 0),
        FA_V16(__bf16, FA_BF16, 128, 8, 64, 1),
        FA_V16(__bf16, FA_BF16, 256, 4, 32, 0),
        FA_V16(__bf16, FA_BF16, 256, 4, 32, 1),
        FA_V16(_Float16, FA_F16, 64, 4, 64, 0),
        FA_V16(_Float16, FA_F16, 64, 8, 128, 0),
        FA_V16(_Float16, FA_F16, 64, 8, 64, 0),
        FA_V16(_Float16, FA_F16, 64, 4, 64, 1),
        FA_V16(_Float16, FA_F16, 64, 8, 128, 1),
        FA_V16(_Float16, FA_F16, 64, 8, 64, 1),
        FA_V16(_Float16, FA_F16, 128, 8, 64, 0),
        FA_V16(_Float16, FA_F16, 128, 8, 64, 1),
        FA_V16(_Float16, FA_F16, 256, 4, 32, 0),
        FA_V16(_Float16, FA_F16, 256, 4, 32, 1),
        // split-KV partial kernels (decode: few query rows, long key ranges)
        FA_V16S(__bf16, FA_BF16, 64, 4, 64, 0),
        FA_V16S(__bf16, FA_BF16, 64, 4, 64, 1),
        FA_V16S(__bf16, FA_BF16, 128, 4, 64, 0),
        FA_V16S(__bf16, FA_BF16, 128, 4, 64, 1),
        FA_V16S(_Float16, FA_F16, 64, 4, 64, 0),
        FA_V16S(_Float16, FA_F16, 64, 4, 64, 1),
        FA_V16S(_Float16, FA_F16, 128, 4, 64, 0),
        FA_V16S(_Float16, FA_F16, 128, 4, 64, 1),
        FA_V16S(__bf16, FA_BF16, 256, 4, 32, 0),
        FA_V16S(__bf16, FA_BF16, 256, 4, 32, 1),
        FA_V16S(_Float16, FA_F16, 256, 4, 32, 0),
        FA_V16S(_Float16, FA_F16, 256, 4, 32, 1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
