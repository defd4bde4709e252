// Tile building blocks shared by the 16-bit attention kernels (forward and
// backward) on gfx950: the 32x32x16 MFMA, the LDS swizzles, the
// direct-to-LDS tile copies, half-wave reductions, and the two tile products
// whose operand layouts the kernels are built around.
//
// A kernel configuration C provides: T (element type), D (head dim), NW
// (waves), BC (rows per streamed tile), RB = 2 D (row bytes), NC = RB / 16,
// RPB, KX, VX (swizzle parameters), TILE = BC RB, KS = D / 16, KB = BC / 32,
// DB = D / 32, LDI = TILE / (1024 NW), NVO = min(DB, 4).
#pragma once
#include "fa_device.h"

namespace fa {

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

// K rows: chunk c of row r is stored at chunk c ^ kswz(r).  With this XOR,
// 16 lanes reading the same logical chunk of 16 consecutive rows touch 16
// different 16-byte bank groups.
template <class C> __device__ __forceinline__ int kswz(int r) { return (r / C::RPB) & C::KX; }
// V rows: chunk c of row r is stored at chunk c ^ vswz(r); the transposed
// reads cover 4 consecutive rows x 4 chunks per half-wave, which this XOR
// spreads over 16 different bank groups.
template <class C> __device__ __forceinline__ int vswz(int r) { return 4 * ((r / C::RPB) & C::VX); }
// Rows read both ways (by rows and transposed): chunk c of row r is stored at
// chunk c ^ bswz(r).  The bits of vswz keep the four rows of a half-wave's
// transposed read in four different 64-byte bank ranges; the two low bits,
// taken from bits 2-3 of the row, make the 16 rows of a row read land on 16
// different bank groups (with vswz alone they share four).
template <class C> __device__ __forceinline__ int bswz(int r) { return vswz<C>(r) | ((r >> 2) & 3); }

// Tile layouts: K-style (row reads only), V-style (transposed reads only),
// or both.
enum { kLayoutK = 0, kLayoutV = 1, kLayoutBoth = 2 };

// Per-lane part of the direct-to-LDS copies of one tile in layout LAYOUT:
// copy instruction i of wave w moves chunks cb..cb+63 (cb = (i*NW + w)*64)
// of the tile's LDS image; this lane's chunk is row r, physical chunk pc, so
// it fetches logical chunk pc ^ swizzle(r) of row r.
template <class C, int LAYOUT>
struct CopyPlan {
    // Offsets are kept in registers only when there are few of them; wide
    // heads (many copies per wave, many live accumulators) recompute them.
    static constexpr bool KEEP = C::LDI <= 2;
    unsigned off[KEEP ? C::LDI : 1];  // byte offset of the fetched chunk within a full tile
    __device__ __forceinline__ static unsigned offset(int i, int w, int lane, int *row) {
        const int chunk = (i * C::NW + w) * 64 + lane;
        const int r = chunk / C::NC;
        const int pc = chunk % C::NC;
        const int sw = LAYOUT == kLayoutBoth ? bswz<C>(r) : LAYOUT == kLayoutV ? vswz<C>(r) : kswz<C>(r);
        *row = r;
        return (unsigned)(r * C::RB + 16 * (pc ^ sw));
    }
    __device__ __forceinline__ CopyPlan(int w, int lane) {
        int r;
        if (KEEP) {
#pragma unroll
            for (int i = 0; i < C::LDI; ++i) off[i] = offset(i, w, lane, &r);
        }
    }
    // Issues the copies of rows [t0, t0 + BC) of one head into an LDS buffer,
    // through a buffer resource that covers the head's rows [t0, n_kv).  Rows
    // past n_kv (only in the last, ragged tile) are clamped to the last row:
    // their scores are masked and their P entries are zero.
    __device__ __forceinline__ void issue(const char *src, int t0, int n_kv, char *buf, int w,
                                          int lane) const {
        const int rows = min(C::BC, n_kv - t0);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (int64_t)t0 * C::RB, rows * C::RB);
        if (rows == C::BC) {
#pragma unroll
            for (int i = 0; i < C::LDI; ++i) {
                int r;
                const unsigned o = KEEP ? off[KEEP ? i : 0] : offset(i, w, lane, &r);
                copy16_to_lds(rs, o, buf + (i * C::NW + w) * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::LDI; ++i) {
                int r;
                const unsigned o = offset(i, w, lane, &r);
                const int gr = min(r, rows - 1);
                copy16_to_lds(rs, o - (unsigned)((r - gr) * C::RB), buf + (i * C::NW + w) * 1024);
            }
        }
    }
};

// Stores the 32 rows of an O^T-layout accumulator (one row per lane, d
// columns), times mul and converted to T, through 32 staging rows of LDS
// that belong to this wave: written by column in the K swizzle, read back by
// row, so that every store instruction writes 64 / NC consecutive whole rows
// (one kilobyte) instead of 8-byte pieces of 32 rows.  The K swizzle keeps
// the 8-byte writes and the 16-byte reads free of bank conflicts.  Rows at or
// past `valid` are not stored.
template <class C>
__device__ __forceinline__ void store_rows_staged(char *stage, char *dst, int valid, const f32x16 (&acc)[C::DB],
                                                  float mul, int lane) {
    typedef typename Mma16<typename C::T>::v4 v4;
    typedef typename C::T T;
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            v4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (T)(acc[db][4 * jj + e] * mul);
            *(v4 *)(stage + l32 * C::RB + 16 * ((4 * db + jj) ^ kswz<C>(l32)) + 8 * h) = out;
        }
    constexpr int RPS = 64 / C::NC;  // rows per store instruction
    const int rr = lane / C::NC, cc = lane % C::NC;
#pragma unroll
    for (int s = 0; s < 32 / RPS; ++s) {
        const int r = s * RPS + rr;
        const u32x4 val = *(const u32x4 *)(stage + r * C::RB + 16 * (cc ^ kswz<C>(r)));
        if (r < valid) *(u32x4 *)(dst + (int64_t)r * C::RB + 16 * cc) = val;
    }
}

// v_permlane32_swap(a, b) returns ([a_lo, b_lo], [a_hi, b_hi]) (lo = lanes
// 0-31, hi = lanes 32-63).  With a = b = x every lane thus receives the lower
// half's x in the first result and the upper half's x in the second.  The
// second operand is an opaque copy of x: the compiler would otherwise treat
// the two results of a swap of identical operands as interchangeable.
__device__ __forceinline__ void both_halves(float x, float &lo, float &hi) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    unsigned v;
    asm("v_mov_b32 %0, %1" : "=v"(v) : "v"(u));
    const auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Maximum / sum over the two half-waves (lanes l and l ^ 32), in every lane.
__device__ __forceinline__ float max_halves(float x) {
    float lo, hi;
    both_halves(x, lo, hi);
    return fmaxf(lo, hi);
}

__device__ __forceinline__ float sum_halves(float x) {
    float lo, hi;
    both_halves(x, lo, hi);
    return lo + hi;
}

// S^T (32 keys x 32 queries per block) = K_tile Q^T.  The KB accumulation
// chains are interleaved so that consecutive MFMAs are independent.  koff0
// is this lane's LDS offset of k-step 0; k-step ks (< 8) is at koff0 ^ 32 ks
// (the swizzled chunk index is (2 ks + h) ^ kswz, and 2 ks occupies bits the
// row offset and the half-wave bit leave free), plus 256 per further 8 steps.
// The offsets are recomputed per tile (the empty asm keeps the compiler from
// hoisting them into registers that live across the whole loop).
template <class C>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[C::KB], const char *Ks, int koff0,
                                        const typename Mma16<typename C::T>::v8 (&qf)[C::KS]) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
    asm volatile("" : "+v"(koff0));
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) s[kb] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            const int ko = (koff0 ^ (32 * (ks & 7))) + 256 * (ks >> 3);
            const v8 a = *(const v8 *)(Ks + kb * 32 * C::RB + ko);
            s[kb] = M::mma(a, qf[ks], s[kb]);
        }
}

// O^T += V_tile^T P^T.  Register r of S^T block kb holds key
// 32 kb + 8 (r/4) + 4 h + r%4, so the B operand of k-step (kb, k2) carries
// keys 32 kb + 16 k2 + {0..3, 8..11} (+4 in the upper half-wave), and the
// matching V^T operand is two transposed reads of 4 consecutive rows each.
template <class C>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[C::DB], const char *Vs, const int (&voff)[C::NVO],
                                        const typename Mma16<typename C::T>::v8 (&pb)[C::KB][2]) {
    typedef Mma16<typename C::T> M;
    typedef typename M::v8 v8;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const char *base = Vs + (kb * 32 + 16 * k2) * C::RB + voff[db & 3] + 256 * (db >> 2);
                const i16x4 lo = lds_read_tr16(base);
                const i16x4 hi = lds_read_tr16(base + 8 * C::RB);
                const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = M::mma(a, pb[kb][k2], o[db]);
            }
}

// Dropout mask bits, shared across the four lanes of a quad.  The mask of
// element (row i, key j) is byte 4 (i mod 4) + (j mod 4) of the Philox4x32-10
// output for counter (j / 4, i / 4, batch-head index, offset), compared with
// p8; one call therefore covers a 4 x 4 block of rows and keys.  In both
// register layouts the four lanes of a quad hold four consecutive indices of
// the same block (four rows in the query-per-lane layout, four keys in the
// key-per-lane layout) and need the same blocks, so each lane computes one
// block of every four and the quad exchanges the resulting 16 keep bits with
// DPP moves.
struct DropQuad {
    unsigned pp, plo;         // p8 in every byte, and its low 7 bits in every byte
    unsigned fixed, c2, c3;   // the quad's own block index (row or key), batch-head, offset
    unsigned k0, k1;          // Philox key (seed)
    unsigned r;               // lane & 3: the lane's row or key within the block
};

__device__ __forceinline__ DropQuad make_drop_quad(unsigned p8, unsigned fixed, unsigned bh, unsigned off,
                                                   unsigned seed_lo, unsigned seed_hi) {
    DropQuad q;
    q.pp = p8 * 0x01010101u;
    q.plo = q.pp & 0x7F7F7F7Fu;
    q.fixed = fixed;
    q.c2 = bh;
    q.c3 = off;
    q.k0 = seed_lo;
    q.k1 = seed_hi;
    q.r = lane_id() & 3u;
    return q;
}

// Keep bits of one 4 x 4 block: bit 4 w + c is set iff byte c of word w is
// >= p8.  The four byte comparisons of a word run in one register: with h the
// high bit of each byte, (x | h) - (p & ~h) leaves in each byte's high bit
// whether x's low 7 bits are >= p's, which decides when the high bits agree;
// otherwise x's own high bit does.  Multiplying the four high bits by
// 2^0 + 2^7 + 2^14 + 2^21 lands bit c of the word at bit 28 + c with no
// other term at or above bit 28.
__device__ __forceinline__ unsigned drop_block_bits(const unsigned (&out)[4], const DropQuad &q) {
    unsigned b = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const unsigned x = out[w];
        const unsigned t = (x | 0x80808080u) - q.plo;
        const unsigned m = x ^ q.pp;
        const unsigned ge = ((m & x) | (~m & t)) & 0x80808080u;
        b |= ((ge * 0x00204081u) >> 28) << (4 * w);
    }
    return b;
}

// Keep bits of the lane for the 4 blocks base + 2 (4 g + i), i = 0 .. 3, along
// the varying index (keys for COL = false, rows for COL = true): bits
// 4 i .. 4 i + 3 hold the 4 elements of block i in increasing order of the
// varying index.  Lane r of the quad computes block i = r.
template <bool COL>
__device__ __forceinline__ unsigned drop_group_bits(const DropQuad &q, unsigned base, unsigned g) {
    const unsigned blk = base + 2u * (4u * g + q.r);
    unsigned out[4];
    if (COL)
        philox4x32_10(q.fixed, blk, q.c2, q.c3, q.k0, q.k1, out);
    else
        philox4x32_10(blk, q.fixed, q.c2, q.c3, q.k0, q.k1, out);
    const unsigned b16 = drop_block_bits(out, q);
    unsigned v[4];
    v[0] = b16;
    // quad_perm patterns of lane xor 1, 2, 3
    v[1] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)b16, 0xB1, 0xF, 0xF, true);
    v[2] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)b16, 0x4E, 0xF, 0xF, true);
    v[3] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)b16, 0x1B, 0xF, 0xF, true);
    unsigned keep = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // v[k] came from lane r ^ k, which computed block r ^ k of the group
        unsigned nib;
        if (COL)  // the lane's key is byte r: bits r, 4 + r, 8 + r, 12 + r
            nib = ((((v[k] >> q.r) & 0x1111u) * 0x1248u) >> 12) & 0xFu;
        else      // the lane's row is word r: bits 4 r .. 4 r + 3
            nib = (v[k] >> (4u * q.r)) & 0xFu;
        keep |= nib << (4u * (q.r ^ (unsigned)k));
    }
    return keep;
}

}  // namespace fa
