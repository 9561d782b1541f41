// gq_mmv.hip -- decode product y[b][n] = sum_k w[n][k] x[b][k] for a batch of
// up to 16 vectors on the matrix cores (gfx950), against packed Q4_0 / Q4_K /
// Q5_K / Q6_K rows.
//
// Small batches are what a speculative-decoding verify step or a few
// concurrent sequences present: the Gemma 4 26B-A4B Show HN page (sections
// "How it works" and "Architecture") checks blocks of up to 16 draft tokens
// and runs a matrix-unit kernel for 5 to 16 tokens.  Each extra vector costs
// the dot-product path a full pass of VALU work per weight; here the weights
// are expanded once and the products for all vectors run on the matrix cores.
//
// Tile: a wavefront computes R output tiles of 16 (rows) x 16 (vectors) with
// v_mfma_f32_16x16x32_bf16 (Q4_0, Q4_K, Q5_K: one MFMA per 32-weight
// sub-block) or v_mfma_f32_16x16x16_bf16 (Q6_K: one per 16-weight sub-block):
//   A (16 x K) = the activations, vector t in row t (rows >= batch read zeros),
//   B (K x 16) = the weights of a tile's 16 rows as the exact bf16 values of
//                c (q - z), z the format's zero point and c a power of two
//                (16 for Q4_0 and Q4_K's high nibbles, 4 for Q6_K, else 1):
//                the quant bits are placed in the bytes of a register (with
//                the zero point removed by flipping the sign bit of c q where
//                z = 128 / c), each byte converted to fp32 (unsigned, or
//                sign-extended) and two fp32 packed into a bf16 pair -- every
//                step exact,
//   C lane l, register r = output (vector 4 (l/16) + r, row l % 16).
// A sub-block adds (s / c) acc to the output, s = d * sc its scale; Q4_K /
// Q5_K also subtract dmin m sum(x), with sum(x) from one MFMA against ones
// that the R tiles of a wavefront share.  Every product in the MFMAs is exact
// (8-bit by 8-bit significands) and the sums are fp32, so the error is
// relative to sum |w x|; a sub-block whose quants all equal the zero point
// contributes exactly zero.
// fp32 activations enter as x = hi + lo with hi the bf16 truncation of x and
// lo the bf16 rounding of the exact remainder (|x - hi - lo| <= 2^-17 |x|),
// two MFMAs each.
//
// Loads.  Lane l = 16 g + n (row n of a tile, lane group g) reads 16
// contiguous bytes of its row per load, the four groups together one 64-byte
// run, so that every load instruction fetches whole 64-byte lines: the L1
// tag lookups, not the bytes, are what limits a load pattern that scatters
// small pieces over many lines.  The bytes then move between lane groups
// with the gfx950 lane-swap instructions (v_permlane32_swap: groups 2, 3 <->
// 0, 1; v_permlane16_swap: groups 1, 3 <-> 0, 2) into the k-slot order of
// the MFMA operand, and the activations are read in that same order.
//
// Workgroup: its W wavefronts share 16 R rows and split the K range, wavefront
// w taking steps w, w + W, w + 2 W, ..., so that the wavefronts of a
// workgroup stream neighbouring parts of the same rows (against contiguous
// runs of steps per wavefront: the hidden-5120 layer's q|k and o at 8 and 16
// bf16 vectors 14-17% faster, v 8-9%, down 4-5%, the hidden-2560 layer's
// q|k|v at 4 fp32 vectors 17%); their partial tiles are summed in LDS in
// wavefront order (deterministic), and wavefront 0 stores.  R and W depend on
// N and K only, so every output column is the same whatever the batch.
#include "gq_gemv_core.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int WMAX = 8;                   // wavefronts per workgroup
constexpr uint32_t BONE = 0x3F803F80u;    // bf16 pair (1, 1)
constexpr uint32_t LO4 = 0x0F0F0F0Fu, HI4 = 0xF0F0F0F0u, SIGN8 = 0x80808080u;

__device__ __forceinline__ f32x4 mma32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const u32x2& a, const u32x2& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// The four bytes of w as exact bf16 values, in two pairs (bytes 0, 1 and 2,
// 3): unsigned (v_cvt_f32_ubyteN) or sign-extended (SDWA byte select).
__device__ __forceinline__ u32x2 bytes_u(uint32_t w) {
    return u32x2{pk_bf16((float)(w & 0xffu), (float)((w >> 8) & 0xffu)),
                 pk_bf16((float)((w >> 16) & 0xffu), (float)(w >> 24))};
}
__device__ __forceinline__ u32x2 bytes_s(uint32_t w) {
    return u32x2{pk_bf16((float)(int8_t)w, (float)(int8_t)(w >> 8)),
                 pk_bf16((float)(int8_t)(w >> 16), (float)(int8_t)(w >> 24))};
}
__device__ __forceinline__ u32x4 cat(u32x2 a, u32x2 b) { return u32x4{a.x, a.y, b.x, b.y}; }

// Two fp32 (bit patterns) -> bf16 pairs hi = truncation, lo = RN of x - hi.
__device__ __forceinline__ uint32_t split_hi(uint32_t e0, uint32_t e1) {
    return __builtin_amdgcn_perm(e1, e0, 0x07060302u);
}
__device__ __forceinline__ uint32_t split_lo(uint32_t e0, uint32_t e1) {
    const float r0 = __builtin_bit_cast(float, e0) - __builtin_bit_cast(float, e0 & 0xFFFF0000u);
    const float r1 = __builtin_bit_cast(float, e1) - __builtin_bit_cast(float, e1 & 0xFFFF0000u);
    return pk_bf16(r0, r1);
}

// ------------------------------------------------------ lane exchanges ----
// a of groups 2, 3 <-> b of groups 0, 1 (lane l <-> lane l - 32)
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
// a of groups 1, 3 <-> b of groups 0, 2 (lane l <-> lane l - 16)
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

// Group g holds the 16-byte piece g of a 64-byte run (bytes 16 g .. 16 g + 15).
// After: (x, y) = bytes off(g) .. off(g) + 7 of the run's first 32 bytes and
// (z, w) = the same bytes of its last 32, off = 0, 16, 8, 24 for g = 0..3.
__device__ __forceinline__ void pair_swap(u32x4& v) {
    uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    swap32(a, c);
    swap32(b, d);
    v = u32x4{a, b, c, d};
}
__device__ __forceinline__ uint32_t pair_off(int g) { return (uint32_t)(((g & 1) << 4) | ((g >> 1) << 3)); }

// Group g holds dwords 0..3 of a 16-byte piece P_g.  After: dword j = dword g
// of piece P_j (a 4 x 4 transpose of (group, dword)).
__device__ __forceinline__ void transpose4(u32x4& v) {
    uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    swap32(a, c);  // groups 0,1: (P_g.0, P_g.1, P_g+2.0, P_g+2.1); 2,3: (P_g-2.2, P_g-2.3, P_g.2, P_g.3)
    swap32(b, d);
    swap16(a, b);
    swap16(c, d);
    v = u32x4{a, b, c, d};
}

// The value v_g of group g, for every g, in every lane: out[j] = v_j.
__device__ __forceinline__ void gather4(uint32_t v, uint32_t out[4]) {
    uint32_t a = v, b = v;
    swap32(a, b);  // a = v_(g&1), b = v_(2+(g&1))
    uint32_t a1 = a, b1 = b;
    swap16(a, a1);  // a = v_0, a1 = v_1
    swap16(b, b1);  // b = v_2, b1 = v_3
    out[0] = a;
    out[1] = a1;
    out[2] = b;
    out[3] = b1;
}

// -------------------------------------------------- activation operands ----
// The A operand of one K=32 MFMA (8 k-slots per lane) as loaded, and prepared
// (bf16 as given; fp32 as the hi / lo pair).
template <int XT>
struct XA8;

template <>
struct XA8<1> {
    u32x4 v;
    __device__ void load8(Rsrc xs, uint32_t o) { v = bld16(xs, o); }
    __device__ void load44(Rsrc xs, uint32_t o0, uint32_t o1) {
        const u32x2 a = bld8(xs, o0), b = bld8(xs, o1);
        v = u32x4{a.x, a.y, b.x, b.y};
    }
};

template <>
struct XA8<0> {
    u32x4 v0, v1;
    __device__ void load8(Rsrc xs, uint32_t o) {
        v0 = bld16(xs, o);
        v1 = bld16(xs, o + 16);
    }
    __device__ void load44(Rsrc xs, uint32_t o0, uint32_t o1) {
        v0 = bld16(xs, o0);
        v1 = bld16(xs, o1);
    }
};

template <int XT>
struct AO8;

template <>
struct AO8<1> {
    u32x4 hi;
    __device__ explicit AO8(const XA8<1>& a) : hi(a.v) {}
    __device__ f32x4 mm(const u32x4& b) const { return mma32(hi, b, f32x4{0.f, 0.f, 0.f, 0.f}); }
};

template <>
struct AO8<0> {
    u32x4 hi, lo;
    __device__ explicit AO8(const XA8<0>& a) {
        hi = u32x4{split_hi(a.v0.x, a.v0.y), split_hi(a.v0.z, a.v0.w), split_hi(a.v1.x, a.v1.y),
                   split_hi(a.v1.z, a.v1.w)};
        lo = u32x4{split_lo(a.v0.x, a.v0.y), split_lo(a.v0.z, a.v0.w), split_lo(a.v1.x, a.v1.y),
                   split_lo(a.v1.z, a.v1.w)};
    }
    __device__ f32x4 mm(const u32x4& b) const { return mma32(lo, b, mma32(hi, b, f32x4{0.f, 0.f, 0.f, 0.f})); }
};

// The same for a K=16 MFMA (4 k-slots per lane).
template <int XT>
struct XA4;

template <>
struct XA4<1> {
    u32x2 v;
    __device__ void load4(Rsrc xs, uint32_t o) { v = bld8(xs, o); }
};

template <>
struct XA4<0> {
    u32x4 v;
    __device__ void load4(Rsrc xs, uint32_t o) { v = bld16(xs, o); }
};

template <int XT>
struct AO4;

template <>
struct AO4<1> {
    u32x2 hi;
    __device__ explicit AO4(const XA4<1>& a) : hi(a.v) {}
    __device__ f32x4 mm(const u32x2& b) const { return mma16(hi, b, f32x4{0.f, 0.f, 0.f, 0.f}); }
};

template <>
struct AO4<0> {
    u32x2 hi, lo;
    __device__ explicit AO4(const XA4<0>& a) {
        hi = u32x2{split_hi(a.v.x, a.v.y), split_hi(a.v.z, a.v.w)};
        lo = u32x2{split_lo(a.v.x, a.v.y), split_lo(a.v.z, a.v.w)};
    }
    __device__ f32x4 mm(const u32x2& b) const { return mma16(lo, b, mma16(hi, b, f32x4{0.f, 0.f, 0.f, 0.f})); }
};

// y += s acc
__device__ __forceinline__ void add_sub_block(f32x4& y, float s, const f32x4& acc) {
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = __builtin_fmaf(s, acc[r], y[r]);
}
// y += s acc - m sx   (sx = sum of the sub-block's activations, m = dmin * min)
__device__ __forceinline__ void add_sub_block_min(f32x4& y, float s, float m, const f32x4& acc, const f32x4& sx) {
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = __builtin_fmaf(-m, sx[r], __builtin_fmaf(s, acc[r], y[r]));
}

// ------------------------------------------------------------- formats ----
// A step is the K range one iteration covers: one super-block (Q4_K, Q5_K,
// Q6_K) or four 32-weight blocks (Q4_0).  load_w() gets the byte offset of
// the row's step (OOB for rows past N or steps past the wavefront's range);
// load_x() the offset of the lane's vector (OOB for vectors past the batch)
// and the step's first weight index k0.

// Q4_K: header (d, dmin, 12 scale bytes) then 128 quant bytes; quant byte j of
// chunk c = bytes 32c..32c+31 holds weight 64c + j (low nibble, sub-block 2c)
// and 64c + 32 + j (high nibble, sub-block 2c + 1).  Group g loads quant bytes
// 16g.. of chunks (0, 1) and (2, 3); after pair_swap its k-slots j = 0..7 of
// sub-block s are weights 32 s + off(g) + j.  w = d sc q - dmin m: the low
// nibbles enter as q (c = 1), the high ones in place as 16 q (c = 16), and the
// min term is dmin m sum x.
template <int TYPE>
struct MF;

template <>
struct MF<T_Q4_K> {
    static constexpr int QK = 256, BB = 144, BPS = 1, QOFF = 16;
    struct W {
        u32x4 h, qa, qb;
    };
    template <int XT>
    struct X {
        XA8<XT> a[8];
    };
    __device__ static void load_w(Rsrc ws, uint32_t bo, int g, W& w) {
        w.h = bld16(ws, bo);
        w.qa = bld16(ws, bo + QOFF + 16 * g);
        w.qb = bld16(ws, bo + QOFF + 64 + 16 * g);
    }
    template <int XT>
    __device__ static void load_x(Rsrc xs, uint32_t xo, uint32_t k0, int g, X<XT>& x) {
        constexpr uint32_t ESZ = XT == 0 ? 4 : 2;
        const uint32_t base = xo + ESZ * (k0 + pair_off(g));
#pragma unroll
        for (int s = 0; s < 8; ++s) x.a[s].load8(xs, base + ESZ * 32 * s);
    }
    // 6-bit (scale, min) of the eight sub-blocks, as bytes [s0..s3], [s4..s7]
    // (b[0..11] = h.y, h.z, h.w):
    //   s < 4:  sc = b[s] & 63,                          m = b[s+4] & 63
    //   s >= 4: sc = (b[s+4] & 15) | (b[s-4] >> 6) << 4, m = (b[s+4] >> 4) | (b[s] >> 6) << 4
    struct Scl {
        float d, dm;
        uint32_t sc0, sc1, m0, m1;
        __device__ explicit Scl(const u32x4& h) {
            d = h2f(h.x & 0xffffu);
            dm = h2f(h.x >> 16);
            sc0 = h.y & 0x3F3F3F3Fu;
            m0 = h.z & 0x3F3F3F3Fu;
            sc1 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
            m1 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
        }
        __device__ float s(int sb) const {
            const uint32_t v = sb < 4 ? sc0 : sc1;
            return d * (float)((v >> (8 * (sb & 3))) & 0xffu);
        }
        __device__ float m(int sb) const {
            const uint32_t v = sb < 4 ? m0 : m1;
            return dm * (float)((v >> (8 * (sb & 3))) & 0xffu);
        }
    };
    // weight operands of chunk c from the swapped quant registers: k-slot j of
    // sub-block 2c is the low nibble of byte j of (q0, q1), of 2c + 1 the high
    // nibble.  Q4_K: bl = q, bh = 16 q.  Q5_K (FIFTH): bit 2c (2c + 1) of plane
    // byte j is bit 4 of the low (high) quant, bl = q, bh = q.
    template <bool FIFTH>
    __device__ static void chunk_ops(const W& w, int c, const u32x2& f, u32x4& bl, u32x4& bh) {
        const uint32_t q0 = c == 0 ? w.qa.x : c == 1 ? w.qa.z : c == 2 ? w.qb.x : w.qb.z;
        const uint32_t q1 = c == 0 ? w.qa.y : c == 1 ? w.qa.w : c == 2 ? w.qb.y : w.qb.w;
        uint32_t l0 = q0 & LO4, l1 = q1 & LO4, h0, h1;
        if constexpr (FIFTH) {
            const uint32_t sl = 2u * (uint32_t)c, sh = sl + 1u;
            l0 |= ((f.x >> sl) & 0x01010101u) << 4;
            l1 |= ((f.y >> sl) & 0x01010101u) << 4;
            h0 = ((q0 >> 4) & LO4) | (((f.x >> sh) & 0x01010101u) << 4);
            h1 = ((q1 >> 4) & LO4) | (((f.y >> sh) & 0x01010101u) << 4);
        } else {
            h0 = q0 & HI4;
            h1 = q1 & HI4;
        }
        bl = cat(bytes_u(l0), bytes_u(l1));
        bh = cat(bytes_u(h0), bytes_u(h1));
    }
    template <int XT, int R, bool FIFTH = false>
    __device__ static void compute_k(W (&w)[R], const X<XT>& x, const u32x2 (&f)[R], f32x4 (&y)[R]) {
#pragma unroll
        for (int t = 0; t < R; ++t) {
            pair_swap(w[t].qa);
            pair_swap(w[t].qb);
        }
        const u32x4 ones = {BONE, BONE, BONE, BONE};
        constexpr float hs = FIFTH ? 1.0f : 0.0625f;  // 1 / c of the high nibbles
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const AO8<XT> al(x.a[2 * c]), ah(x.a[2 * c + 1]);
            const f32x4 sxl = al.mm(ones), sxh = ah.mm(ones);
#pragma unroll
            for (int t = 0; t < R; ++t) {
                u32x4 bl, bh;
                chunk_ops<FIFTH>(w[t], c, f[t], bl, bh);
                const Scl sc(w[t].h);
                add_sub_block_min(y[t], sc.s(2 * c), sc.m(2 * c), al.mm(bl), sxl);
                add_sub_block_min(y[t], hs * sc.s(2 * c + 1), sc.m(2 * c + 1), ah.mm(bh), sxh);
            }
        }
    }
    template <int XT, int R>
    __device__ static void compute(W (&w)[R], const X<XT>& x, int, f32x4 (&y)[R]) {
        u32x2 f[R];
#pragma unroll
        for (int t = 0; t < R; ++t) f[t] = u32x2{0u, 0u};
        compute_k<XT, R, false>(w, x, f, y);
    }
};

// Q5_K: the Q4_K header, a 32-byte plane of fifth bits at 16 (bit s of byte
// j: weight 32 s + j), the quants at 48.  Operands q <= 31, exact in bf16.
template <>
struct MF<T_Q5_K> : MF<T_Q4_K> {
    static constexpr int BB = 176, QOFF = 48;
    struct W : MF<T_Q4_K>::W {
        u32x2 f;
    };
    __device__ static void load_w(Rsrc ws, uint32_t bo, int g, W& w) {
        w.h = bld16(ws, bo);
        w.qa = bld16(ws, bo + QOFF + 16 * g);
        w.qb = bld16(ws, bo + QOFF + 64 + 16 * g);
        w.f = bld8(ws, bo + 16 + pair_off(g));
    }
    template <int XT, int R>
    __device__ static void compute(W (&w)[R], const X<XT>& x, int, f32x4 (&y)[R]) {
        MF<T_Q4_K>::W b[R];
        u32x2 f[R];
#pragma unroll
        for (int t = 0; t < R; ++t) {
            b[t] = w[t];
            f[t] = w[t].f;
        }
        compute_k<XT, R, true>(b, x, f, y);
    }
};

// Q4_0: a step is four 18-byte blocks (d, then 16 quant bytes: byte j holds
// weight j in its low nibble and 16 + j in its high one).  Group g loads block
// g's quants; after transpose4 its dword j holds bytes 4g..4g+3 of block j:
// k-slots 0..3 = weights 4g..4g+3, 4..7 = weights 16 + 4g..16 + 4g + 3.
// w = d (q - 8): the operand is 16 (q - 8), the byte 16 q with its sign bit
// flipped, read sign-extended (c = 16).
template <>
struct MF<T_Q4_0> {
    static constexpr int QK = 32, BB = 18, BPS = 4;
    struct W {
        u32x4 q;
        uint32_t d;
    };
    template <int XT>
    struct X {
        XA8<XT> a[4];
    };
    // bo: offset of the step's first block (the lane loads block g, or a zero
    // block past the row's last one)
    __device__ static void load_w(Rsrc ws, uint32_t bo, int g, W& w, bool blk_ok) {
        const uint32_t o = blk_ok ? bo + (uint32_t)(18 * g) : OOB;
        w.d = bld2(ws, o);
        w.q = bld16(ws, o + 2);
    }
    template <int XT>
    __device__ static void load_x(Rsrc xs, uint32_t xo, uint32_t k0, int g, int nvalid, X<XT>& x) {
        constexpr uint32_t ESZ = XT == 0 ? 4 : 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t base = j < nvalid ? xo + ESZ * (k0 + 32 * j + 4 * g) : OOB;
            x.a[j].load44(xs, base, base + ESZ * 16);
        }
    }
    template <int XT, int R>
    __device__ static void compute(W (&w)[R], const X<XT>& x, int, f32x4 (&y)[R]) {
        uint32_t d[R][4];
#pragma unroll
        for (int t = 0; t < R; ++t) {
            transpose4(w[t].q);
            gather4(w[t].d, d[t]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const AO8<XT> a(x.a[j]);
#pragma unroll
            for (int t = 0; t < R; ++t) {
                const uint32_t q = w[t].q[j];
                // 16 (low nibble - 8), then 16 (high nibble - 8)
                const u32x4 b = cat(bytes_s(((q << 4) & HI4) ^ SIGN8), bytes_s((q & HI4) ^ SIGN8));
                add_sub_block(y[t], h2f(d[t][j]) * 0.0625f, a.mm(b));
            }
        }
    }
};

// Q6_K: ql (128 B) at 0, qh (64 B) at 128, 16 int8 scales at 192, d at 208.
// Weight i = 128 h + 32 q4 + l (l < 32): low 4 bits = nibble q4 >> 1 of
// ql[64 h + 32 (q4 & 1) + l], high 2 bits = bits 2 q4, 2 q4 + 1 of
// qh[32 h + l]; sub-block (16 weights) 8 h + 2 q4 + l / 16.  Group g loads
// 16-byte piece g of ql[0..63], ql[64..127] and qh; after transpose4 its dword
// j of each holds bytes 16 j + 4 p(g) .. 16 j + 4 p(g) + 3, so for sub-block
// (h, q4, a = l / 16) its k-slots i = 0..3 are l = 16 a + 4 p(g) + i: ql
// dword 2 (q4 & 1) + a of half h, qh dword 2 h + a.  p(g) = g for fp32
// activations.  bf16 activations are loaded 16 bytes at a time, group g the
// inputs 8 g .. 8 g + 7 of a sub-block pair, then v_permlane32_swap gives
// group g the inputs 4 p(g) .. 4 p(g) + 3 of each sub-block of the pair with
// p = (0, 2, 1, 3) (half the load instructions of 8-byte loads, which limited
// this path); the weight pieces' dwords 1 and 2 are exchanged before the
// transpose to match (the product sums over each sub-block's k, so any order
// common to both operands gives the same sums).  w = d sc (q - 32): the
// operand is 4 (q - 32), the byte 4 q with its sign bit flipped, read
// sign-extended (c = 4).
template <>
struct MF<T_Q6_K> {
    static constexpr int QK = 256, BB = 210, BPS = 1;
    struct W {
        u32x4 l0, l1, qh, sc;
        uint32_t d;
    };
    // fp32: sub-block sb's four inputs per lane; bf16: sub-block pair pp's
    // eight inputs 8 g.. per lane as loaded
    template <int XT>
    struct X {
        XA4<XT> a[16];  // sub-block index 8 h + 2 q4 + a
    };
    __device__ static void load_w(Rsrc ws, uint32_t bo, int g, W& w) {
        w.l0 = bld16(ws, bo + 16 * g);
        w.l1 = bld16(ws, bo + 64 + 16 * g);
        w.qh = bld16(ws, bo + 128 + 16 * g);
        w.sc = bld16(ws, bo + 192);
        w.d = bld2(ws, bo + 208);
    }
    template <int XT>
    __device__ static void load_x(Rsrc xs, uint32_t xo, uint32_t k0, int g, X<XT>& x) {
        if constexpr (XT == 0) {
            const uint32_t base = xo + 4 * (k0 + 4 * g);
#pragma unroll
            for (int sb = 0; sb < 16; ++sb) x.a[sb].load4(xs, base + 4 * 16 * sb);
        } else {
            const uint32_t base = xo + 2 * (k0 + 8 * g);
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) {
                const u32x4 v = bld16(xs, base + 2 * 32 * pp);
                x.a[2 * pp].v = u32x2{v.x, v.y};
                x.a[2 * pp + 1].v = u32x2{v.z, v.w};
            }
        }
    }
    template <int XT, int R>
    __device__ static void compute(W (&w)[R], const X<XT>& xin, int, f32x4 (&y)[R]) {
        X<XT> x = xin;
        if constexpr (XT == 1) {
            // groups 0, 1 keep inputs 0..3 of their eight and take 0..3 of
            // groups 2, 3 (the pair's second sub-block); groups 2, 3 keep
            // 4..7 and take 4..7 of groups 0, 1 (the first sub-block)
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) {
                uint32_t a0 = x.a[2 * pp].v.x, a1 = x.a[2 * pp].v.y;
                uint32_t b0 = x.a[2 * pp + 1].v.x, b1 = x.a[2 * pp + 1].v.y;
                swap32(a0, b0);
                swap32(a1, b1);
                x.a[2 * pp].v = u32x2{a0, a1};
                x.a[2 * pp + 1].v = u32x2{b0, b1};
            }
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
            if constexpr (XT == 1) {
                w[t].l0 = u32x4{w[t].l0.x, w[t].l0.z, w[t].l0.y, w[t].l0.w};
                w[t].l1 = u32x4{w[t].l1.x, w[t].l1.z, w[t].l1.y, w[t].l1.w};
                w[t].qh = u32x4{w[t].qh.x, w[t].qh.z, w[t].qh.y, w[t].qh.w};
            }
            transpose4(w[t].l0);
            transpose4(w[t].l1);
            transpose4(w[t].qh);
        }
#pragma unroll
        for (int sb = 0; sb < 16; ++sb) {
            const int h = sb >> 3, q4 = (sb >> 1) & 3, a = sb & 1;
            const AO4<XT> ao(x.a[sb]);
#pragma unroll
            for (int t = 0; t < R; ++t) {
                const uint32_t L = (h ? w[t].l1 : w[t].l0)[2 * (q4 & 1) + a];
                const uint32_t H = w[t].qh[2 * h + a];
                const int ns = 4 * (q4 >> 1), hs = 2 * q4;
                // byte i = 4 q of k-slot i with its sign bit flipped: 4 (q - 32)
                const uint32_t q = ((L >> ns) & LO4) | (((H >> hs) & 0x03030303u) << 4);
                const u32x2 b = bytes_s((q << 2) ^ SIGN8);
                const float s = h2f(w[t].d) * (float)(int)(int8_t)(w[t].sc[sb >> 2] >> (8 * (sb & 3)));
                add_sub_block(y[t], s * 0.25f, ao.mm(b));
            }
        }
    }
};

// Uniform load interface over the formats (Q4_0 needs the block count to
// zero the blocks past the row's end).
template <int TYPE, int XT>
struct Step {
    using F = MF<TYPE>;
    __device__ static void load(Rsrc ws, uint32_t ro, int step, int nblk, int g, typename F::W& w) {
        if constexpr (TYPE == T_Q4_0) {
            const bool ok = ro != OOB && 4 * step + g < nblk;
            F::load_w(ws, ro + (uint32_t)step * (4 * F::BB), g, w, ok);
        } else {
            F::load_w(ws, ro == OOB ? OOB : ro + (uint32_t)step * F::BB, g, w);
        }
    }
    __device__ static void load_x(Rsrc xs, uint32_t xo, int step, int nblk, int g, typename F::template X<XT>& x) {
        if constexpr (TYPE == T_Q4_0) {
            const int nvalid = xo == OOB ? 0 : nblk - 4 * step;
            F::template load_x<XT>(xs, xo, (uint32_t)step * 128u, g, nvalid, x);
        } else {
            F::template load_x<XT>(xs, xo, (uint32_t)step * F::QK, g, x);
        }
    }
};

// --------------------------------------------------------------- kernel ----

// R row tiles per wavefront, P steps in flight per lane.
template <int TYPE, int XT, int R, int P>
__global__ __launch_bounds__(64 * WMAX) void k_mmv(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                   const uint8_t* __restrict__ x, int batch, float* __restrict__ y) {
    using F = MF<TYPE>;
    using S = Step<TYPE, XT>;
    constexpr int ESZ = XT == 0 ? 4 : 2;
    __shared__ f32x4 red[WMAX - 1][R][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nw = (int)(blockDim.x >> 6);
    const int nl = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * R);
    const int rows = (int)(N - n0 < 16 * R ? N - n0 : 16 * R);
    const uint32_t row_bytes = (uint32_t)(K / F::QK) * F::BB;
    const Rsrc ws = make_rsrc(W + n0 * (int64_t)row_bytes, (uint32_t)rows * row_bytes);
    const Rsrc xs = make_rsrc(x, (uint32_t)((int64_t)batch * K * ESZ));
    uint32_t roff[R];
#pragma unroll
    for (int t = 0; t < R; ++t) roff[t] = 16 * t + nl < rows ? (uint32_t)(16 * t + nl) * row_bytes : OOB;
    const uint32_t xoff = nl < batch ? (uint32_t)((int64_t)nl * K * ESZ) : OOB;

    const int nblk = (int)(K / F::QK);
    const int steps = (nblk + F::BPS - 1) / F::BPS;
    // wavefront w takes steps w, w + nw, ...: at any moment the wavefronts
    // of a workgroup read neighbouring steps of the same rows
    const int s0 = wave;
    const int n = steps > wave ? (steps - wave + nw - 1) / nw : 0;

    f32x4 acc[R];
#pragma unroll
    for (int t = 0; t < R; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    typename F::W wr[P][R];
    typename F::template X<XT> xr[P];
    auto issue = [&](int j, int i) {
        const bool ok = i < n;
        const int st = s0 + nw * (ok ? i : 0);
#pragma unroll
        for (int t = 0; t < R; ++t) S::load(ws, ok ? roff[t] : OOB, st, nblk, g, wr[j][t]);
        S::load_x(xs, ok ? xoff : OOB, st, nblk, g, xr[j]);
    };
#pragma unroll
    for (int j = 0; j < P; ++j) issue(j, j);
    // Whole rounds of P steps in straight-line code, so that the wait before
    // each slot is exact (a conditional slot in the loop body merges load
    // counts from several paths into a wait for all loads), then the last
    // partial round.  The refill of slot j goes out right after slot j is
    // consumed (left to itself the scheduler sinks it behind the next slot's
    // work, and the wait for that slot would then cover it too).
    int i = 0;
    for (; i + P <= n; i += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            F::template compute<XT, R>(wr[j], xr[j], g, acc);
            __builtin_amdgcn_sched_barrier(0);
            issue(j, i + j + P);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < P - 1; ++j)
        if (i + j < n) F::template compute<XT, R>(wr[j], xr[j], g, acc);

    if (nw > 1) {
        if (wave > 0)
#pragma unroll
            for (int t = 0; t < R; ++t) red[wave - 1][t][lane] = acc[t];
        __syncthreads();
        if (wave != 0) return;
        for (int w = 0; w < nw - 1; ++w)
#pragma unroll
            for (int t = 0; t < R; ++t) acc[t] += red[w][t][lane];
    }
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int row = 16 * t + nl;
        if (row < rows) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = 4 * g + r;
                if (v < batch) y[(int64_t)v * N + n0 + row] = acc[t][r];
            }
        }
    }
}

template <int TYPE, int XT, int R>
hipError_t launch_r(const uint8_t* W, int64_t N, int64_t K, const uint8_t* x, int batch, float* y, int nw,
                    hipStream_t s) {
    // steps in flight per wavefront: 1, which leaves room for 3-5
    // wavefronts per SIMD whose interleaving hides the memory latency
    // (measured against 2-3 in flight: 2-13% faster on Q4_K / Q5_K / Q6_K,
    // fp32 and bf16, 4-16 vectors); bf16 Q4_0 keeps 2 (2% faster there)
    constexpr int P = TYPE == T_Q4_0 && XT == 1 ? 2 : 1;
    const int64_t groups = (N + 16 * R - 1) / (16 * R);
    if (groups > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_mmv<TYPE, XT, R, P>), dim3((unsigned)groups), dim3(64 * nw), 0, s, W, N, K, x, batch, y);
    return hipGetLastError();
}

template <int TYPE, int XT>
hipError_t launch(const uint8_t* W, int64_t N, int64_t K, const uint8_t* x, int batch, float* y, hipStream_t s) {
    using F = MF<TYPE>;
    const int64_t tiles = (N + 15) / 16;
    const int64_t steps = (K / F::QK + F::BPS - 1) / F::BPS;
    // Row tiles per wavefront R (each activation fragment serves R tiles) and
    // wavefronts per workgroup (splitting K): R = 2 if its launch still holds
    // >= 1024 wavefronts, else 1, each workgroup doubling its wavefronts while
    // the launch holds < 2048 and each keeps >= 1 step, or while it holds
    // < 4096 and each keeps >= 4 steps (>= 2 steps below 2048 measured up to
    // 7% slower on short-K matrices; going on to 4096 is 1-2% faster on the
    // large matrices but 47% slower on 19456 x 2560 at 8 fp32 vectors, where
    // each wavefront would keep 1-2 of its 10 steps; 8192 no faster).  (Four tiles per
    // wavefront, which bf16 Q4_0 / Q4_K activations fit in two wavefronts'
    // registers per SIMD, measured 5-33% slower from 5 to 12 vectors -- half
    // the wavefronts where rows are few -- and at most 1% faster at 16; one
    // tile, 0-40% slower.)
    auto waves = [&](int R, int& nw) {
        const int64_t groups = (tiles + R - 1) / R;
        nw = 1;
        while (nw < WMAX && ((groups * nw < 2048 && steps >= 2 * nw) || (groups * nw < 4096 && steps >= 8 * nw)))
            nw *= 2;
        return groups * nw;
    };
    int nw;
    if (waves(2, nw) >= 1024) return launch_r<TYPE, XT, 2>(W, N, K, x, batch, y, nw, s);
    waves(1, nw);
    return launch_r<TYPE, XT, 1>(W, N, K, x, batch, y, nw, s);
}

template <int TYPE>
hipError_t launch_x(const uint8_t* W, int64_t N, int64_t K, const uint8_t* x, int x_dtype, int batch, float* y,
                    hipStream_t s) {
    if (x_dtype == DT_F32) return launch<TYPE, 0>(W, N, K, x, batch, y, s);
    return launch<TYPE, 1>(W, N, K, x, batch, y, s);
}

}  // namespace

hipError_t gqk_mmv(int type, const void* W, int64_t N, int64_t K, const void* x, int x_dtype, int batch, float* y,
                   hipStream_t s) {
    if (N == 0) return hipSuccess;
    const uint8_t* w = static_cast<const uint8_t*>(W);
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    if (type == T_Q4_0) return launch_x<T_Q4_0>(w, N, K, xb, x_dtype, batch, y, s);
    if (type == T_Q4_K) return launch_x<T_Q4_K>(w, N, K, xb, x_dtype, batch, y, s);
    if (type == T_Q5_K) return launch_x<T_Q5_K>(w, N, K, xb, x_dtype, batch, y, s);
    return launch_x<T_Q6_K>(w, N, K, xb, x_dtype, batch, y, s);
}
