// gq_mmv.hip -- decode product y[b][n] = sum_k w[n][k] x[b][k] for a batch of
// up to 16 vectors on the matrix cores (gfx950), against packed Q4_0 / Q4_K /
// Q6_K rows.
//
// Small batches are what a speculative-decoding verify step or a few
// concurrent sequences present: the Gemma 4 26B-A4B Show HN page (sections
// "How it works" and "Architecture") checks blocks of up to 16 draft tokens
// and runs a matrix-unit kernel for 5 to 16 tokens.  Each extra vector costs
// the dot-product path a full pass of VALU work per weight; here the weights
// are expanded once and the products for all vectors run on the matrix cores.
//
// Tile: one wavefront computes a 16 (rows) x 16 (vectors) output tile with
// v_mfma_f32_16x16x32_bf16 (Q4_0, Q4_K: one MFMA per 32-weight sub-block) or
// v_mfma_f32_16x16x16_bf16 (Q6_K: one per 16-weight sub-block):
//   A (16 x K) = the activations, vector t in row t (rows >= batch read zeros),
//   B (K x 16) = the weights of the tile's 16 rows, expanded in registers to
//                the exact bf16 values 128 + q (OR-ing q into bf16 128.0),
//   C lane l, register r = output (vector 4 (l/16) + r, row l % 16).
// With acc = A B and az = A Z (the same MFMA against the constant Z = 128 +
// the format's zero point, i.e. the operand of a sub-block whose quants all sit
// on the zero point), a sub-block adds s (acc - az) to the output, s = d * sc
// its scale; Q4_K also subtracts dmin m (az / 128).  Every product in the MFMAs
// is exact (8-bit by 8-bit significands) and the sums are fp32; a sub-block
// whose quants all equal the zero point gives acc == az bit for bit and so
// contributes exactly zero.
// fp32 activations enter as x = hi + lo with hi the bf16 truncation of x and
// lo the bf16 rounding of the exact remainder (|x - hi - lo| <= 2^-17 |x|),
// two MFMAs each.
//
// Lane l of a tile holds row l % 16 and reads the quants of k-slot group
// g = l / 16; the weight bytes are spread with byte permutes so that k-slots
// follow the activation order and activations load as they lie in memory.
//
// Workgroup: the W wavefronts of a workgroup share one 16-row tile and split
// its K range into contiguous runs of units; their partial tiles are summed
// in LDS in wavefront order (deterministic), and wavefront 0 stores.
#include "gq_gemv_core.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int WMAX = 16;                 // wavefronts per workgroup
constexpr uint32_t BMAG = 0x43004300u;    // bf16 pair (128, 128)
constexpr uint32_t M4 = 0x000F000Fu;
// byte permutes [b0, 0, b1, 0] and [b2, 0, b3, 0] of one dword
constexpr uint32_t SEL01 = 0x0C010C00u, SEL23 = 0x0C030C02u;

__device__ __forceinline__ f32x4 mma32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const u32x2& a, const u32x2& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}

__device__ __forceinline__ uint32_t perm(uint32_t w, uint32_t sel) { return __builtin_amdgcn_perm(w, w, sel); }

// bf16 pair (128 + low nibble of byte 0, 128 + low nibble of byte 2)
__device__ __forceinline__ uint32_t nib_lo(uint32_t t) { return (t & M4) | BMAG; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t t) { return ((t >> 4) & M4) | BMAG; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 (bit patterns) -> bf16 pairs hi = truncation, lo = RN of x - hi.
__device__ __forceinline__ uint32_t split_hi(uint32_t e0, uint32_t e1) {
    return __builtin_amdgcn_perm(e1, e0, 0x07060302u);
}
__device__ __forceinline__ uint32_t split_lo(uint32_t e0, uint32_t e1) {
    const float r0 = __builtin_bit_cast(float, e0) - __builtin_bit_cast(float, e0 & 0xFFFF0000u);
    const float r1 = __builtin_bit_cast(float, e1) - __builtin_bit_cast(float, e1 & 0xFFFF0000u);
    return pk_bf16(r0, r1);
}

// -------------------------------------------------- activation fragments ----
// Eight activations of one vector for one K=32 MFMA (two runs of four for
// Q4_0, one run of eight otherwise), kept as loaded.
template <int XT>
struct X8;

template <>
struct X8<0> {
    u32x4 v0, v1;
    __device__ void load8(Rsrc xs, uint32_t xo, uint32_t k) {
        v0 = bld16(xs, xo + 4 * k);
        v1 = bld16(xs, xo + 4 * k + 16);
    }
    __device__ void load44(Rsrc xs, uint32_t xo, uint32_t k0, uint32_t k1) {
        v0 = bld16(xs, xo + 4 * k0);
        v1 = bld16(xs, xo + 4 * k1);
    }
    // acc += A B, az += A Z for the weight operand b and the zero operand z
    __device__ void mma(const u32x4& b, uint32_t z, f32x4& acc, f32x4& az) const {
        const u32x4 zz = {z, z, z, z};
        const u32x4 hi = {split_hi(v0.x, v0.y), split_hi(v0.z, v0.w), split_hi(v1.x, v1.y), split_hi(v1.z, v1.w)};
        const u32x4 lo = {split_lo(v0.x, v0.y), split_lo(v0.z, v0.w), split_lo(v1.x, v1.y), split_lo(v1.z, v1.w)};
        acc = mma32(hi, b, acc);
        acc = mma32(lo, b, acc);
        az = mma32(hi, zz, az);
        az = mma32(lo, zz, az);
    }
};

template <>
struct X8<1> {
    u32x4 v;
    __device__ void load8(Rsrc xs, uint32_t xo, uint32_t k) { v = bld16(xs, xo + 2 * k); }
    __device__ void load44(Rsrc xs, uint32_t xo, uint32_t k0, uint32_t k1) {
        const u32x2 a = bld8(xs, xo + 2 * k0), b = bld8(xs, xo + 2 * k1);
        v = u32x4{a.x, a.y, b.x, b.y};
    }
    __device__ void mma(const u32x4& b, uint32_t z, f32x4& acc, f32x4& az) const {
        const u32x4 zz = {z, z, z, z};
        acc = mma32(v, b, acc);
        az = mma32(v, zz, az);
    }
};

// Four activations of one vector for one K=16 MFMA.
template <int XT>
struct X4;

template <>
struct X4<0> {
    u32x4 v;
    __device__ void load4(Rsrc xs, uint32_t xo, uint32_t k) { v = bld16(xs, xo + 4 * k); }
    __device__ void mma(const u32x2& b, uint32_t z, f32x4& acc, f32x4& az) const {
        const u32x2 zz = {z, z};
        const u32x2 hi = {split_hi(v.x, v.y), split_hi(v.z, v.w)};
        const u32x2 lo = {split_lo(v.x, v.y), split_lo(v.z, v.w)};
        acc = mma16(hi, b, acc);
        acc = mma16(lo, b, acc);
        az = mma16(hi, zz, az);
        az = mma16(lo, zz, az);
    }
};

template <>
struct X4<1> {
    u32x2 v;
    __device__ void load4(Rsrc xs, uint32_t xo, uint32_t k) { v = bld8(xs, xo + 2 * k); }
    __device__ void mma(const u32x2& b, uint32_t z, f32x4& acc, f32x4& az) const {
        const u32x2 zz = {z, z};
        acc = mma16(v, b, acc);
        az = mma16(v, zz, az);
    }
};

// y += s (acc - az)
__device__ __forceinline__ void add_sub_block(f32x4& y, float s, const f32x4& acc, const f32x4& az) {
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = __builtin_fmaf(s, acc[r] - az[r], y[r]);
}
// y += s (acc - az) - m az   (m = dmin * min / 128)
__device__ __forceinline__ void add_sub_block_min(f32x4& y, float s, float m, const f32x4& acc, const f32x4& az) {
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = __builtin_fmaf(-m, az[r], __builtin_fmaf(s, acc[r] - az[r], y[r]));
}

// ------------------------------------------------------------- formats ----
// A unit is the K range one lane loads and reduces in one step.  load() gets
// the weight offset of the unit's block (bo, OOB for rows past N or units past
// the wavefront's range), the lane's k-slot group g, the activation offset of
// the lane's vector (xo, OOB for vectors past the batch) and the unit's first
// weight index k.

template <int TYPE, int XT>
struct MU;

// Q4_0: unit = one 18-byte block of 32 weights.  Group g holds quant bytes
// 4g..4g+3: k-slots 0..3 = weights 4g..4g+3 (low nibbles), 4..7 = weights
// 16+4g..16+4g+3 (high nibbles).  w = d (q - 8): s = d, Z = 128 + 8.
template <int XT>
struct MU<T_Q4_0, XT> {
    static constexpr int QK = 32, BB = 18, UW = 32;
    uint32_t d, q;
    X8<XT> x;
    __device__ void load(Rsrc ws, uint32_t bo, int g, Rsrc xs, uint32_t xo, uint32_t k, int) {
        d = bld2(ws, bo);
        q = __builtin_amdgcn_raw_buffer_load_b32(ws, (int)(bo + 2 + 4 * g), 0, 0);
        x.load44(xs, xo, k + 4 * g, k + 16 + 4 * g);
    }
    __device__ void compute(int, f32x4& y) const {
        const uint32_t t0 = perm(q, SEL01), t1 = perm(q, SEL23);
        const u32x4 b = {nib_lo(t0), nib_lo(t1), nib_hi(t0), nib_hi(t1)};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, az = acc;
        x.mma(b, 0x43084308u, acc, az);
        add_sub_block(y, h2f(d), acc, az);
    }
};

// Q4_K: unit c (0..3) of a super-block = quant bytes 32c..32c+31 (sub-blocks
// 2c: low nibbles, 2c+1: high nibbles) and the 16-byte header.  Group g holds
// bytes 32c+8g..32c+8g+7: k-slot j = weight 8g + j of either sub-block.
// w = d sc q - dmin m: s = d sc, Z = 128, and the min term dmin m sum x with
// sum x = az / 128.
template <int XT>
struct MU<T_Q4_K, XT> {
    static constexpr int QK = 256, BB = 144, UW = 64;
    u32x4 h;
    u32x2 q;
    X8<XT> xa, xb;
    __device__ void load(Rsrc ws, uint32_t bo, int g, Rsrc xs, uint32_t xo, uint32_t k, int c) {
        h = bld16(ws, bo);
        q = bld8(ws, bo + 16 + 32 * c + 8 * g);
        xa.load8(xs, xo, k + 8 * g);
        xb.load8(xs, xo, k + 32 + 8 * g);
    }
    // (scale, min) 6-bit pairs of sub-blocks 2c, 2c+1 from the 12 scale bytes
    // b[0..11] = h.y, h.z, h.w, j = 2 (c & 1):
    //   c < 2:  sc = b[j] & 63,                        m = b[j+4] & 63
    //   c >= 2: sc = (b[j+8] & 15) | (b[j] >> 6) << 4, m = (b[j+8] >> 4) | (b[j+4] >> 6) << 4
    // both built as bytes [scL, scH, mL, mH] with permutes.  With FIFTH, f
    // holds the fifth bits of the lane's eight weights (Q5_K): bit 2c for
    // sub-block 2c and 2c+1 for 2c+1.
    template <bool FIFTH>
    __device__ void compute_q(int c, const u32x2& f, f32x4& y) const {
        const uint32_t j = 2u * (uint32_t)(c & 1);
        const uint32_t C = __builtin_amdgcn_perm(h.z, h.y, j | (j + 1) << 8 | (j + 4) << 16 | (j + 5) << 24);
        const uint32_t A = __builtin_amdgcn_perm(h.w, h.w, j | (j + 1) << 8 | j << 16 | (j + 1) << 24);
        const uint32_t v = c < 2 ? (C & 0x3F3F3F3Fu)
                                 : (((C >> 2) & 0x30303030u) | (A & 0x00000F0Fu) | ((A >> 4) & 0x0F0F0000u));
        const float d = h2f(h.x & 0xffffu), dmin = h2f(h.x >> 16);
        const float sL = d * (float)(v & 0xffu), sH = d * (float)((v >> 8) & 0xffu);
        const float mL = (dmin * (float)((v >> 16) & 0xffu)) * 0.0078125f;
        const float mH = (dmin * (float)(v >> 24)) * 0.0078125f;
        const uint32_t t0 = perm(q.x, SEL01), t1 = perm(q.x, SEL23), t2 = perm(q.y, SEL01), t3 = perm(q.y, SEL23);
        u32x4 bl = {nib_lo(t0), nib_lo(t1), nib_lo(t2), nib_lo(t3)};
        u32x4 bh = {nib_hi(t0), nib_hi(t1), nib_hi(t2), nib_hi(t3)};
        if constexpr (FIFTH) {
            const uint32_t u[4] = {perm(f.x, SEL01), perm(f.x, SEL23), perm(f.y, SEL01), perm(f.y, SEL23)};
            const uint32_t sl = 2u * (uint32_t)c, sh = sl + 1u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bl[i] |= ((u[i] >> sl) & 0x00010001u) << 4;
                bh[i] |= ((u[i] >> sh) & 0x00010001u) << 4;
            }
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, az = acc;
        xa.mma(bl, BMAG, acc, az);
        add_sub_block_min(y, sL, mL, acc, az);
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        az = acc;
        xb.mma(bh, BMAG, acc, az);
        add_sub_block_min(y, sH, mH, acc, az);
    }
    __device__ void compute(int c, f32x4& y) const { compute_q<false>(c, u32x2{0u, 0u}, y); }
};

// Q5_K: Q4_K with a 32-byte plane of fifth bits at 16 (quants at 48).  Group g
// also loads plane bytes 8g..8g+7: bit 2c of byte 8g + j is the fifth bit of
// k-slot j in sub-block 2c, bit 2c+1 in sub-block 2c+1.  Operands 128 + q,
// q <= 31, stay exact in bf16.
template <int XT>
struct MU<T_Q5_K, XT> : MU<T_Q4_K, XT> {
    static constexpr int BB = 176;
    u32x2 f;
    __device__ void load(Rsrc ws, uint32_t bo, int g, Rsrc xs, uint32_t xo, uint32_t k, int c) {
        this->h = bld16(ws, bo);
        this->q = bld8(ws, bo + 48 + 32 * c + 8 * g);
        f = bld8(ws, bo + 16 + 8 * g);
        this->xa.load8(xs, xo, k + 8 * g);
        this->xb.load8(xs, xo, k + 32 + 8 * g);
    }
    __device__ void compute(int c, f32x4& y) const { this->template compute_q<true>(c, f, y); }
};

// Q6_K: unit u % 4 = 2h + a of a super-block: half h, quarters jq = a (low
// nibbles of ql, qh bits 2a..2a+1) and jq = a + 2 (high nibbles, bits
// 2a+4..2a+5), each as two 16-weight sub-blocks sh = 0, 1 (sub-block index
// 8h + 2jq + sh, weights 128h + 32jq + 16sh + 0..15).  Group g holds the
// bytes 16sh+4g..16sh+4g+3 of the quarter's ql and qh runs: k-slot i = weight
// 16sh + 4g + i.  w = d sc (q - 32): s = d sc, Z = 128 + 32.
template <int XT>
struct MU<T_Q6_K, XT> {
    static constexpr int QK = 256, BB = 210, UW = 64;
    uint32_t l0, l1, h0, h1, d;
    u32x2 sc;
    X4<XT> x[4];  // [jq = a, sh 0], [a, 1], [a + 2, 0], [a + 2, 1]
    __device__ void load(Rsrc ws, uint32_t bo, int g, Rsrc xs, uint32_t xo, uint32_t k, int p) {
        const int hh = p >> 1, a = p & 1;
        const uint32_t ql = bo + 64 * hh + 32 * a + 4 * g, qh = bo + 128 + 32 * hh + 4 * g;
        l0 = __builtin_amdgcn_raw_buffer_load_b32(ws, (int)ql, 0, 0);
        l1 = __builtin_amdgcn_raw_buffer_load_b32(ws, (int)(ql + 16), 0, 0);
        h0 = __builtin_amdgcn_raw_buffer_load_b32(ws, (int)qh, 0, 0);
        h1 = __builtin_amdgcn_raw_buffer_load_b32(ws, (int)(qh + 16), 0, 0);
        sc = bld8(ws, bo + 192 + 8 * hh);
        d = bld2(ws, bo + 208);
        // k is the unit's first weight 256 b + 128 h; quarter jq starts 32 jq later
        const uint32_t k0 = k - 64 * (uint32_t)a;  // 256 b + 128 h
        x[0].load4(xs, xo, k0 + 32 * a + 4 * g);
        x[1].load4(xs, xo, k0 + 32 * a + 16 + 4 * g);
        x[2].load4(xs, xo, k0 + 32 * (a + 2) + 4 * g);
        x[3].load4(xs, xo, k0 + 32 * (a + 2) + 16 + 4 * g);
    }
    __device__ void compute(int p, f32x4& y) const {
        const int a = p & 1;
        const float dd = h2f(d);
        // scale bytes 2jq + sh of the half: a: 2a, 2a+1; a+2: 2a+4, 2a+5
        const uint32_t s01 = a ? (sc.x >> 16) : sc.x, s23 = a ? (sc.y >> 16) : sc.y;
        const float s[4] = {dd * (float)(int)(int8_t)(s01 & 0xffu), dd * (float)(int)(int8_t)((s01 >> 8) & 0xffu),
                            dd * (float)(int)(int8_t)(s23 & 0xffu), dd * (float)(int)(int8_t)((s23 >> 8) & 0xffu)};
        const uint32_t L[2] = {l0, l1}, H[2] = {h0, h1};
        const uint32_t shl = 4u - 2u * (uint32_t)a, shr = 2u * (uint32_t)a;
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
            const uint32_t t0 = perm(L[sh], SEL01), t1 = perm(L[sh], SEL23);
            const uint32_t u0 = perm(H[sh], SEL01), u1 = perm(H[sh], SEL23);
            // quarter a: q = low nibble | qh bits (2a, 2a+1) << 4
            const u32x2 bl = {(t0 & M4) | ((u0 << shl) & 0x00300030u) | BMAG,
                              (t1 & M4) | ((u1 << shl) & 0x00300030u) | BMAG};
            // quarter a + 2: q = high nibble | qh bits (2a+4, 2a+5) << 4
            const u32x2 bh = {((t0 >> 4) & M4) | ((u0 >> shr) & 0x00300030u) | BMAG,
                              ((t1 >> 4) & M4) | ((u1 >> shr) & 0x00300030u) | BMAG};
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, az = acc;
            x[sh].mma(bl, 0x43204320u, acc, az);
            add_sub_block(y, s[sh], acc, az);
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            az = acc;
            x[2 + sh].mma(bh, 0x43204320u, acc, az);
            add_sub_block(y, s[2 + sh], acc, az);
        }
    }
};

// --------------------------------------------------------------- kernel ----

// Units in flight per lane: P.  Unit u of a row: block u / UPB, position
// u % UPB inside it (UPB = QK / UW).
template <int TYPE, int XT, int P>
__global__ __launch_bounds__(64 * WMAX) void k_mmv(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                   const uint8_t* __restrict__ x, int batch, float* __restrict__ y) {
    using U = MU<TYPE, XT>;
    constexpr int UPB = U::QK / U::UW;
    constexpr int ESZ = XT == 0 ? 4 : 2;
    __shared__ f32x4 red[WMAX - 1][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nw = (int)(blockDim.x >> 6);
    const int nl = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int rows = (int)(N - n0 < 16 ? N - n0 : 16);
    const uint32_t row_bytes = (uint32_t)(K / U::QK) * U::BB;
    const Rsrc ws = make_rsrc(W + n0 * (int64_t)row_bytes, (uint32_t)rows * row_bytes);
    const Rsrc xs = make_rsrc(x, (uint32_t)((int64_t)batch * K * ESZ));
    const uint32_t roff = nl < rows ? (uint32_t)nl * row_bytes : OOB;
    const uint32_t xoff = nl < batch ? (uint32_t)((int64_t)nl * K * ESZ) : OOB;

    const int nu = (int)(K / U::UW);
    const int u0 = (int)((int64_t)wave * nu / nw), u1 = (int)((int64_t)(wave + 1) * nu / nw);
    const int n = u1 - u0;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    U ring[P];
    auto issue = [&](U& r, int i) {
        const bool ok = i < n;
        const int u = ok ? u0 + i : u0;
        const int blk = u / UPB, pos = u % UPB;
        r.load(ws, ok ? roff + (uint32_t)blk * U::BB : OOB, g, xs, ok ? xoff : OOB, (uint32_t)u * U::UW, pos);
    };
#pragma unroll
    for (int j = 0; j < P; ++j) issue(ring[j], j);
    for (int i = 0; i < n; i += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            if (i + j < n) ring[j].compute((u0 + i + j) % UPB, acc);
            issue(ring[j], i + j + P);
        }
    }

    if (nw > 1) {
        if (wave > 0) red[wave - 1][lane] = acc;
        __syncthreads();
        if (wave != 0) return;
        for (int w = 0; w < nw - 1; ++w) acc += red[w][lane];
    }
    const int64_t nn = n0 + nl;
    if (nl < rows) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            if (t < batch) y[(int64_t)t * N + nn] = acc[r];
        }
    }
}

template <int TYPE, int XT, int P>
hipError_t launch(const uint8_t* W, int64_t N, int64_t K, const uint8_t* x, int batch, float* y, hipStream_t s) {
    using U = MU<TYPE, XT>;
    const int64_t tiles = (N + 15) / 16;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    // wavefronts per workgroup: enough to put about four per SIMD on the chip
    // (2 x 2048 wavefronts), each with at least three units of K
    const int64_t nu = K / U::UW;
    int nw = 1;
    while (nw < WMAX && tiles * nw < 4096 && nu >= 3 * (2 * nw)) nw *= 2;
    hipLaunchKernelGGL((k_mmv<TYPE, XT, P>), dim3((unsigned)tiles), dim3(64 * nw), 0, s, W, N, K, x, batch, y);
    return hipGetLastError();
}

template <int TYPE>
hipError_t launch_x(const uint8_t* W, int64_t N, int64_t K, const uint8_t* x, int x_dtype, int batch, float* y,
                    hipStream_t s) {
    if (x_dtype == DT_F32) return launch<TYPE, 0, 3>(W, N, K, x, batch, y, s);
    return launch<TYPE, 1, 4>(W, N, K, x, batch, y, s);
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
