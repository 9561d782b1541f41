// gq_gemv_core.h -- the decode product core shared by gq_matvec and
// gq_matvec_id (gfx950, wave64).
//
// Work split.  A workgroup (256 threads, 4 wavefronts) owns a tile of output
// rows and a small batch of activation vectors.  Each wavefront covers
// 64 / LPR rows: its 64 lanes form 64/LPR groups of LPR lanes, one group per
// row, and inside a group lane v takes the row's "units" v, v+LPR, ... (a unit
// is 32 or 64 consecutive weights).  Every lane streams its own 16-byte pieces
// of the row with buffer loads, unpacks them in registers and keeps fp32
// partial sums; one shuffle reduction per output ends the kernel.
//
// Loads.  The weights of a workgroup are addressed through one buffer
// resource that spans exactly its rows.  A lane whose unit lies past the end
// of its row (or whose row lies past N) loads at an offset beyond that span:
// the hardware returns zeros for it without a memory access.  So the number of
// load instructions is fixed at compile time (the load counter waits stay
// exact) while no byte is fetched twice or needlessly.
//
// Arithmetic.  Every weight reaches the fp16 dot instructions as the exact
// fp16 value of q - z (z = the format's zero point), so every product is exact
// and the fp32 sums carry nothing that only cancels later:
//   Q4_0, Q6_K:  q is OR-ed into the mantissa of 1024 (1024 + q, or 1024 + 16 q
//                for a high nibble) and 1024 + z (1024 + 16 z) is subtracted
//                with one packed fp16 add per two weights -- exact, the
//                result is a small integer;
//   Q4_K, Q5_K:  z = 0 and the masked quant bits are used as they are: the fp16
//                subnormal q * 2^-24 (16 q * 2^-24 for a high nibble), exact,
//                with the 2^24 folded into the block scale.
// Activations are staged once per workgroup in LDS as fp16 pairs that match
// the register order of the weights, each group of 32 inputs scaled by a power
// of two 2^e so that its largest magnitude lies in [2^14, 2^15) (the scaling is
// exact; only the fp16 rounding of the scaled value, at most 2^-11 relative, is
// inexact).  One v_dot2_f32_f16 then adds two weight-activation products into
// an fp32 accumulator.  Per sub-block the format's scale (and min) are applied
// once:
//   Q4_0:  d * 2^-e * ( S_lo + S_hi / 16 )
//   Q4_K:  d*2^24*sc * 2^-e * S - dmin*m * sum(x)
//   Q6_K:  d*sc * 2^-e * S          (S / 16 for the high-nibble groups)
// where S is the dot product of the integers q - z with the staged values.
// A sub-block whose quants all equal the zero point has S == 0 exactly.
#pragma once

#include "gq_device.h"

namespace gqd {

constexpr int NTHREADS = 256;

// ------------------------------------------------------ buffer loads ----

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Offset that is past every buffer's span: such a load returns zeros and
// touches no memory.  Spans are kept below 2^31 bytes.
constexpr uint32_t OOB = 0x80000000u;

// Raw (unformatted, stride 0) buffer over [base, base + bytes).
__device__ __forceinline__ Rsrc make_rsrc(const uint8_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}
// Loads at any byte offset (gfx9 buffer loads accept unaligned addresses).
__device__ __forceinline__ u32x4 bld16(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x2 bld8(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t bld2(Rsrc r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

template <int TYPE>
struct Fmt;

// Every format describes a unit by (block, position inside the block): the
// block offset is b * BB and the lane-constant part (`pos`, from unit % UPB,
// with UPB units per block) is fixed per lane because LPR is a multiple of 4.

// ---------------------------------------------------------------- Q4_0 ----
// Unit = one 18-byte block (32 weights).  Accumulator 0 = low nibbles
// (weights 0..15), accumulator 1 = high nibbles (weights 16..31).
template <>
struct Fmt<T_Q4_0> {
    static constexpr int QK = 32, BB = 18, UW = 32, UPB = 1, NA = 2, NP = 8, NF = 1, NQ = NA * NP / 4;
    static constexpr int KIND = 0;  // staged factors: {2^-e, -, -, -}
    struct Raw {
        uint32_t d;
        u32x4 q;
    };
    struct Lane {
        __device__ explicit Lane(int) {}
    };
    struct Scl {
        float d;
    };
    __device__ static uint32_t zero_pattern(int a) { return a == 0 ? 0x64086408u : 0x64806480u; }
    __device__ static Raw load(Rsrc rs, uint32_t boff, const Lane&) {
        Raw r;
        r.d = bld2(rs, boff);
        r.q = bld16(rs, boff + 2);
        return r;
    }
    // the runs of 32-input group g: run r covers group elements 16r..16r+15
    static constexpr int RPG = 2;
    __device__ static void group_run(int g, int r, int& unit, int& a) {
        unit = g;
        a = r;
    }
    // q - 8 (16 (q - 8) for the high nibbles) as exact fp16 pairs
    __device__ static void pairs(const Raw& r, int a, uint32_t magic, uint32_t P[NP]) {
        const uint32_t mask = a == 0 ? 0x000F000Fu : 0x00F000F0u;
        const uint32_t z = zero_pattern(a);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t w = r.q[k];
            P[2 * k] = sub_h2((w & mask) | magic, z);
            P[2 * k + 1] = sub_h2(((w >> 8) & mask) | magic, z);
        }
    }
    __device__ static Scl scales(const Raw& r, const Lane&) { return Scl{h2f(r.d)}; }
    // dacc[a] = dot product of run a; f[0] = {2^-e, -, -, -}
    __device__ static float contrib(const Scl& s, const float dacc[NA], const f32x4 f[NF]) {
        return (s.d * f[0].x) * __builtin_fmaf(0.0625f, dacc[1], dacc[0]);
    }
};

// ---------------------------------------------------------------- Q4_K ----
// Unit c (0..3) of a super-block = a 32-byte slice of the quants (64 weights:
// sub-blocks 2c and 2c+1) plus the block's 16-byte header.
template <>
struct Fmt<T_Q4_K> {
    static constexpr int QK = 256, BB = 144, UW = 64, UPB = 4, NA = 2, NP = 16, NF = 1, NQ = NA * NP / 4;
    static constexpr int KIND = 1;  // staged factors: {2^-eL, 2^-eH, sum xL, sum xH}
    struct Raw {
        u32x4 h, q0, q1;
    };
    // Per-lane constants of the scale decode for slice c: byte selectors of
    // the 6-bit (sc, m) fields of sub-blocks 2c, 2c+1 (see scales()).
    struct Lane {
        uint32_t qoff, sel_lo, sel_hi;
        bool low;
        __device__ explicit Lane(int c) {
            qoff = 16 + 32 * c;
            const uint32_t j = 2 * (c & 1);
            // bytes j, j+1 of scale words 0 (h.y) and 1 (h.z): [y_j, y_j+1, z_j, z_j+1]
            sel_lo = j | (j + 1) << 8 | (j + 4) << 16 | (j + 5) << 24;
            // bytes j, j+1 of scale word 2 (h.w), twice: [w_j, w_j+1, w_j, w_j+1]
            sel_hi = j | (j + 1) << 8 | j << 16 | (j + 1) << 24;
            low = c < 2;
        }
    };
    struct Scl {
        float dsL, dsH, dmL, dmH;
    };
    __device__ static Raw load(Rsrc rs, uint32_t boff, const Lane& ln) {
        Raw r;
        r.h = bld16(rs, boff);
        r.q0 = bld16(rs, boff + ln.qoff);
        r.q1 = bld16(rs, boff + ln.qoff + 16);
        return r;
    }
    static constexpr int RPG = 1;
    __device__ static void group_run(int g, int, int& unit, int& a) {
        unit = g >> 1;
        a = g & 1;
    }
    // q (16 q for the high nibbles) as exact fp16 subnormals, times 2^-24
    __device__ static void pairs(const Raw& r, int a, uint32_t, uint32_t P[NP]) {
        const uint32_t mask = a == 0 ? 0x000F000Fu : 0x00F000F0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t w = k < 4 ? r.q0[k] : r.q1[k - 4];
            P[2 * k] = w & mask;
            P[2 * k + 1] = (w >> 8) & mask;
        }
    }
    // 6-bit (scale, min) of sub-blocks s = 2c, 2c+1 (j = s & 3 over the 12
    // scale bytes b[0..11] = h.y, h.z, h.w):
    //   s < 4:  sc = b[j] & 63,                        m = b[j+4] & 63
    //   s >= 4: sc = (b[j+8] & 15) | (b[j] >> 6) << 4, m = (b[j+8] >> 4) | (b[j+4] >> 6) << 4
    // Both forms are built with byte permutes as [scL, scH, mL, mH] and the
    // lane's slice picks one -- no divergent branch.
    __device__ static Scl scales(const Raw& r, const Lane& ln) {
        const uint32_t C = __builtin_amdgcn_perm(r.h.z, r.h.y, ln.sel_lo);
        const uint32_t A = __builtin_amdgcn_perm(r.h.w, r.h.w, ln.sel_hi);
        const uint32_t lo = C & 0x3F3F3F3Fu;
        const uint32_t hi = ((C >> 2) & 0x30303030u) | (A & 0x00000F0Fu) | ((A >> 4) & 0x0F0F0000u);
        const uint32_t v = ln.low ? lo : hi;
        // d * 2^24 undoes the subnormal encoding of the quants (exact)
        const float d = h2f(r.h.x & 0xffffu) * 16777216.0f, dmin = h2f(r.h.x >> 16);
        Scl s;
        s.dsL = d * (float)(v & 0xffu);
        s.dsH = (d * 0.0625f) * (float)((v >> 8) & 0xffu);
        s.dmL = dmin * (float)((v >> 16) & 0xffu);
        s.dmH = dmin * (float)(v >> 24);
        return s;
    }
    // f[0] = {2^-eL, 2^-eH, sum xL, sum xH}
    __device__ static float contrib(const Scl& s, const float dacc[NA], const f32x4 f[NF]) {
        float v = (s.dsL * f[0].x) * dacc[0];
        v = __builtin_fmaf(s.dsH * f[0].y, dacc[1], v);
        v = __builtin_fmaf(-s.dmL, f[0].z, v);
        return __builtin_fmaf(-s.dmH, f[0].w, v);
    }
};

// ---------------------------------------------------------------- Q5_K ----
// Q4_K with a plane of fifth bits (32 bytes at 16; the quants move to 48).
// Unit c as for Q4_K; the pair of sub-block 2c (low nibbles, subnormal q)
// takes bit 2c of the plane byte as its bit 4, the pair of 2c+1 (high nibbles
// in place, 16 q) takes bit 2c+1 as its bit 8: one rotate and one and-or per
// pair.
template <>
struct Fmt<T_Q5_K> : Fmt<T_Q4_K> {
    static constexpr int BB = 176;
    struct Raw : Fmt<T_Q4_K>::Raw {
        u32x4 f0, f1;
        uint32_t rlo, rhi;
    };
    struct Lane : Fmt<T_Q4_K>::Lane {
        uint32_t rlo, rhi;  // right rotations: plane bit 2c -> bit 4, bit 2c+1 -> bit 8
        __device__ explicit Lane(int c) : Fmt<T_Q4_K>::Lane(c) {
            qoff = 48 + 32 * c;
            rlo = (uint32_t)(2 * c - 4) & 31u;
            rhi = (uint32_t)(2 * c + 1 - 8) & 31u;
        }
    };
    __device__ static Raw load(Rsrc rs, uint32_t boff, const Lane& ln) {
        Raw r;
        r.h = bld16(rs, boff);
        r.q0 = bld16(rs, boff + ln.qoff);
        r.q1 = bld16(rs, boff + ln.qoff + 16);
        r.f0 = bld16(rs, boff + 16);
        r.f1 = bld16(rs, boff + 32);
        r.rlo = ln.rlo;
        r.rhi = ln.rhi;
        return r;
    }
    __device__ static void pairs(const Raw& r, int a, uint32_t, uint32_t P[NP]) {
        const uint32_t mask = a == 0 ? 0x000F000Fu : 0x00F000F0u;
        const uint32_t fm = a == 0 ? 0x00100010u : 0x01000100u;
        const uint32_t rot = a == 0 ? r.rlo : r.rhi;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t w = k < 4 ? r.q0[k] : r.q1[k - 4];
            const uint32_t f = k < 4 ? r.f0[k] : r.f1[k - 4];
            P[2 * k] = (w & mask) | (__builtin_amdgcn_alignbit(f, f, rot) & fm);
            P[2 * k + 1] = ((w >> 8) & mask) | (__builtin_amdgcn_alignbit(f, f, rot + 8u) & fm);
        }
    }
};

// ---------------------------------------------------------------- Q6_K ----
// Unit (h, lh) of a super-block, unit % 4 = 2h + lh: lanes l = 16 lh .. 16 lh
// + 15 of the four 32-weight groups g of half h (64 weights, four 16-weight
// sub-blocks).  Accumulator g.
template <>
struct Fmt<T_Q6_K> {
    static constexpr int QK = 256, BB = 210, UW = 64, UPB = 4, NA = 4, NP = 8, NF = 1, NQ = NA * NP / 4;
    static constexpr int KIND = 2;  // staged factors: {2^-e of groups 0..3}
    struct Raw {
        u32x4 la, lb, qh;
        u32x2 sc;
        uint32_t d;
    };
    struct Lane {
        uint32_t ql, qh, sc;
        int sh;
        __device__ explicit Lane(int p) {
            const int h = p >> 1, lh = p & 1;
            ql = 64 * h + 16 * lh;
            qh = 128 + 32 * h + 16 * lh;
            sc = 192 + 8 * h;
            sh = 8 * lh;
        }
    };
    struct Scl {
        float ds[4];
    };
    // zero point q = 32: 1024 + 32 for groups 0,1 and 1024 + 16*32 for 2,3
    __device__ static uint32_t zero_pattern(int a) { return a < 2 ? 0x64206420u : 0x66006600u; }
    __device__ static Raw load(Rsrc rs, uint32_t boff, const Lane& ln) {
        Raw r;
        r.la = bld16(rs, boff + ln.ql);
        r.lb = bld16(rs, boff + ln.ql + 32);
        r.qh = bld16(rs, boff + ln.qh);
        r.sc = bld8(rs, boff + ln.sc);
        r.d = bld2(rs, boff + 208);
        return r;
    }
    // group g = (block g/8, half h, group gg): lane halves 0 and 1 are units
    // 4*block + 2h and 4*block + 2h + 1, accumulator gg
    static constexpr int RPG = 2;
    __device__ static void group_run(int g, int r, int& unit, int& a) {
        unit = 4 * (g >> 3) + 2 * ((g >> 2) & 1) + r;
        a = g & 3;
    }
    __device__ static void pairs(const Raw& r, int g, uint32_t magic, uint32_t P[NP]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t A = r.la[k] >> (8 * j), Bq = r.lb[k] >> (8 * j), H = r.qh[k] >> (8 * j);
                uint32_t v;
                if (g == 0) v = ((H << 4) & 0x00300030u) | (A & 0x000F000Fu);
                else if (g == 1) v = ((H << 2) & 0x00300030u) | (Bq & 0x000F000Fu);
                else if (g == 2) v = ((H << 4) & 0x03000300u) | (A & 0x00F000F0u);
                else v = ((H << 2) & 0x03000300u) | (Bq & 0x00F000F0u);
                P[2 * k + j] = sub_h2(v | magic, zero_pattern(g));
            }
        }
    }
    __device__ static Scl scales(const Raw& r, const Lane& ln) {
        const int sh = ln.sh;
        const float d = h2f(r.d), d16 = d * 0.0625f;
        Scl s;
        s.ds[0] = d * (float)(int)(int8_t)(r.sc.x >> sh);
        s.ds[1] = d * (float)(int)(int8_t)(r.sc.x >> (sh + 16));
        s.ds[2] = d16 * (float)(int)(int8_t)(r.sc.y >> sh);
        s.ds[3] = d16 * (float)(int)(int8_t)(r.sc.y >> (sh + 16));
        return s;
    }
    // f[0] = 2^-e of groups 0..3
    __device__ static float contrib(const Scl& s, const float dacc[NA], const f32x4 f[NF]) {
        float v = (s.ds[0] * f[0].x) * dacc[0];
        v = __builtin_fmaf(s.ds[1] * f[0].y, dacc[1], v);
        v = __builtin_fmaf(s.ds[2] * f[0].z, dacc[2], v);
        return __builtin_fmaf(s.ds[3] * f[0].w, dacc[3], v);
    }
};

// ----------------------------------------------------------- staging ----

// Where the activation vectors of this workgroup live: p[b] points at element
// 0 of vector b.  The element type is a template parameter XT of the kernels
// (0 = fp32, 1 = bf16).  Only ever indexed with a wave-uniform b.
struct XSrc {
    const uint8_t* p[8];
    // p[b] for a wave-uniform b without indexing the array by a variable
    // (which would put a local copy of it in scratch memory)
    __device__ __forceinline__ const uint8_t* at(int b) const {
        const uint8_t* r = p[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) r = b == i ? p[i] : r;
        return r;
    }
};

// One 32-input group of raw activation bits (fp32: 8 x 16 B, bf16: 4 x 16 B),
// kept as loaded so that no arithmetic waits on the load before the weight
// loads are issued.
template <int XT>
struct XRaw {
    u32x4 q[XT == 0 ? 8 : 4];
};

template <int XT>
__device__ __forceinline__ void load_group(const uint8_t* xb, int64_t k, XRaw<XT>& r) {
    const u32x4* p = reinterpret_cast<const u32x4*>(xb + (XT == 0 ? 4 : 2) * k);
#pragma unroll
    for (int i = 0; i < (XT == 0 ? 8 : 4); ++i) r.q[i] = p[i];
}

// Bits of element i as an fp32 pattern.  (Element copied to a scalar first:
// __builtin_bit_cast of a vector-element lvalue reads element 0 with this
// compiler.)
template <int XT>
__device__ __forceinline__ uint32_t group_bits(const XRaw<XT>& r, int i) {
    if (XT == 0) {
        uint32_t w = r.q[i >> 2][i & 3];
        return w;
    }
    uint32_t w = r.q[i >> 3][(i >> 1) & 3];
    return (i & 1) ? (w & 0xffff0000u) : (w << 16);
}

// Wait until every vector memory load of this wavefront has returned
// (s_waitcnt vmcnt(0), the other counters left alone).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Exponent e that puts the largest magnitude of a 32-group into
// [2^14, 2^15), from the largest |x| bit pattern (non-negative floats order
// like their bit patterns); 0 for an all-zero group or one holding Inf/NaN
// (which then propagate).
__device__ __forceinline__ int group_exp(uint32_t mbits) {
    if (mbits == 0 || mbits >= 0x7f800000u) return 0;
    return 15 - __builtin_amdgcn_frexp_expf(__builtin_bit_cast(float, mbits));
}

// Staged activations of one K tile, unit-major: the record of (unit u,
// vector b) is NQ fp16-pair quads followed by NF (= 1) factor vector, 16 B each, at
// 16-byte slot (u * RS + b * (NQ + NF)).  The unit stride RS is odd (in 16-B
// slots), so the lanes of a wave, which read consecutive units, hit distinct
// LDS banks; all reads of one record share a base address.
template <class F>
struct TileLds {
    u32x4* base;
    int U, nb, RS;
    static constexpr int NREC = F::NQ + F::NF;
    __host__ __device__ static int unit_stride(int nb_) { return (NREC * nb_) | 1; }
    __device__ void carve(uint8_t* p, int U_, int nb_) {
        base = reinterpret_cast<u32x4*>(p);
        U = U_;
        nb = nb_;
        RS = unit_stride(nb_);
    }
    __device__ u32x4* rec(int u, int b) const { return base + u * RS + b * NREC; }
};

// One run (16 or 32 consecutive inputs) of an already-scaled group -> fp16
// pairs in unpack order, and the run's factors.
template <class F>
__device__ __forceinline__ void stage_write_run(const TileLds<F>& L, int b, int u, int a, const float* r, int e) {
    uint32_t P[F::NP];
#pragma unroll
    for (int n = 0; n < F::NP; ++n) {
        int t = 4 * (n >> 1) + (n & 1);
        P[n] = pack_h2(r[t], r[t + 2]);
    }
    u32x4* rp = L.rec(u, b);
#pragma unroll
    for (int qd = 0; qd < F::NP / 4; ++qd)
        rp[a * (F::NP / 4) + qd] = u32x4{P[4 * qd], P[4 * qd + 1], P[4 * qd + 2], P[4 * qd + 3]};
    float sc = __builtin_ldexpf(1.0f, -e);
    float* f0 = reinterpret_cast<float*>(rp + F::NQ);
    if constexpr (F::KIND == 0) {  // Q4_0: {2^-e, 0, 0, 0} (both runs share e)
        if (a == 0) *reinterpret_cast<f32x4*>(f0) = f32x4{sc, 0.f, 0.f, 0.f};
    } else if constexpr (F::KIND == 1) {  // Q4_K: {sL, sH, sum xL, sum xH}
        // sum of the run's fp16 values (dot2 against ones), times 2^-e
        float sx = 0.f;
#pragma unroll
        for (int n = 0; n < F::NP; ++n) sx = dot2(0x3C003C00u, P[n], sx);
        f0[a] = sc;
        f0[2 + a] = sx * sc;
    } else {  // Q6_K: {s0..3}
        f0[a] = sc;
    }
}

// A whole 32-input group of vector b: exponent, scaling, and every run in it.
template <class F, int XT>
__device__ __forceinline__ void stage_group(const TileLds<F>& L, int b, int g, const XRaw<XT>& in) {
    uint32_t bits[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) bits[i] = group_bits<XT>(in, i);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        uint32_t a0 = bits[i] & 0x7fffffffu, a1 = bits[i + 1] & 0x7fffffffu;
        m = a0 > m ? a0 : m;
        m = a1 > m ? a1 : m;
    }
    const int e = group_exp(m);
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_ldexpf(__builtin_bit_cast(float, bits[i]), e);
#pragma unroll
    for (int r = 0; r < F::RPG; ++r) {
        int u, a;
        F::group_run(g, r, u, a);
        stage_write_run<F>(L, b, u, a, v + 16 * r, e);
    }
}

// stage_issue loads this thread's first group (vector 0); the caller then
// issues the weight loads, so the in-order load counter lets staging start as
// soon as the activations arrive.  stage_finish does the arithmetic, the
// remaining groups one at a time (loop over vectors is wave-uniform, so the
// vector pointer stays a scalar) and ends with an LDS barrier.  Loading the
// next group while staging one held a second group's registers (32 for fp32
// activations) through the whole kernel: without it the batch-1 products
// drop from 143-146 to 114-116 registers and the routed ones from 142 to 115
// (4 wavefronts per SIMD instead of 3); measured 0-3% faster (dense layer at
// 4 vectors 55.6 -> 54.0 us, fused MoE layer 1.8%), nowhere slower beyond
// the noise.
template <class F, int XT>
__device__ __forceinline__ void stage_issue(const XSrc& xs, int64_t k0, const TileLds<F>& L, XRaw<XT>& in) {
    // every thread loads (threads past the groups reload group 0): an
    // unconditional load keeps the load-counter waits exact
    const int G = L.U * F::UW / 32;
    const int g = (int)threadIdx.x < G ? (int)threadIdx.x : 0;
    load_group<XT>(xs.p[0], k0 + 32 * g, in);
}

template <class F, int XT, int NT>
__device__ __forceinline__ void stage_finish(const XSrc& xs, int64_t k0, const TileLds<F>& L,
                                             const XRaw<XT>& first) {
    const int G = L.U * F::UW / 32;
    const int tid = (int)threadIdx.x;
    constexpr int nthreads = NT;
    // work items: (vector b, round r) -> group tid + nthreads r of vector b
    const int rounds = (G + nthreads - 1) / nthreads;
    const int items = L.nb * rounds;
    if (tid < G) stage_group<F, XT>(L, 0, tid, first);
    // the later items' loads are unconditional (threads past the groups
    // reload group 0) so that the load-counter waits stay exact
#pragma unroll 1
    for (int i = 1; i < items; ++i) {
        const int g = tid + nthreads * (i % rounds);
        XRaw<XT> cur;
        load_group<XT>(xs.at(i / rounds), k0 + 32 * (g < G ? g : 0), cur);
        if (g < G) stage_group<F, XT>(L, i / rounds, g, cur);
    }
    lds_barrier();
}

// ----------------------------------------------------------- compute ----

// One unit of a row against nb staged vectors (record uc of the tile).
template <class F, int BMAX>
__device__ __forceinline__ void unit_math(const TileLds<F>& L, const typename F::Raw& raw,
                                          const typename F::Lane& ln, int uc, bool valid, uint32_t magic,
                                          float acc[BMAX]) {
    const int nb = L.nb;
    const typename F::Scl sc = F::scales(raw, ln);
    uint32_t P[F::NA][F::NP];
#pragma unroll
    for (int a = 0; a < F::NA; ++a) F::pairs(raw, a, magic, P[a]);
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        if (b >= nb) break;
        const u32x4* rp = L.rec(uc, b);
        f32x4 f[F::NF];
#pragma unroll
        for (int j = 0; j < F::NF; ++j) f[j] = __builtin_bit_cast(f32x4, rp[F::NQ + j]);
        float dacc[F::NA];
#pragma unroll
        for (int a = 0; a < F::NA; ++a) {
            u32x4 xq[F::NP / 4];
#pragma unroll
            for (int qd = 0; qd < F::NP / 4; ++qd) xq[qd] = rp[a * (F::NP / 4) + qd];
            float s = 0.f;
#pragma unroll
            for (int qd = 0; qd < F::NP / 4; ++qd)
#pragma unroll
                for (int n4 = 0; n4 < 4; ++n4) s = dot2(P[a][4 * qd + n4], xq[qd][n4], s);
            dacc[a] = s;
        }
        const float c = F::contrib(sc, dacc, f);
        acc[b] += valid ? c : 0.f;
    }
}

// Sum acc over the LPR lanes of each group (lanes differ only in the low bits).
template <int BMAX>
__device__ __forceinline__ void reduce_group(float acc[BMAX], int LPR) {
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
        for (int off = LPR >> 1; off > 0; off >>= 1) acc[b] += __shfl_xor(acc[b], off);
}

// Output rows of the vectors: y_b[n] = p[b][n].  Wave-uniform.
struct YDst {
    float* p[8];
};

// Most units per lane in one straight-line pass (larger K tiles use the ring,
// whose depth each launcher picks), and the default number of them in flight
// before the first is taken (PF; the plain product takes 1, measured 3-9%
// faster on its own launches, while the routed and gated kernels lose 1-1.5%
// with fewer than 3).
constexpr int D_MAX = 6;
constexpr int PREFETCH = 3;

// The whole decode product for one workgroup: rows [rowA, rowA + wcount * SR)
// of the packed matrix W (N rows, K inputs) against nb <= BMAX staged vectors;
// this wavefront is number wslot of the wcount that share those rows (all
// wavefronts of the workgroup stage the activations together, so wavefronts
// of one workgroup may work on different matrices with the same K).
//
// Each K tile of U units gives every lane T = ceil(U / LPR) units.  Without
// RING, T <= D: the loads of the first min(D, PF) units are issued
// around the activation staging and each later one as an earlier unit is
// taken, all in straight-line code (units past the tile load as zeros).  With
// RING a ring keeps D units per lane in flight over any number of units.
template <int TYPE, int XT, int BMAX, int D, bool RING, int NT = NTHREADS, int PF = PREFETCH>
__device__ __forceinline__ void gemv_workgroup(const uint8_t* __restrict__ W, int64_t N, int64_t K, int64_t rowA,
                                               const XSrc& xs, int nb, const YDst& yd, int LPR, int tile_units,
                                               uint8_t* lds, int wslot, int wcount) {
    using F = Fmt<TYPE>;
    using Raw = typename F::Raw;
    const int lane = threadIdx.x & 63;
    const int SR = 64 / LPR;
    const int s = lane / LPR, v = lane - s * LPR;
    const uint32_t row_bytes = (uint32_t)((K / F::QK) * F::BB);
    const int64_t wg_rows = (int64_t)wcount * SR;
    const int64_t rows_here = N - rowA < wg_rows ? N - rowA : wg_rows;
    const Rsrc rs = make_rsrc(W + rowA * (int64_t)row_bytes, (uint32_t)rows_here * row_bytes);
    const int rloc = wslot * SR + s;
    const bool row_ok = rloc < rows_here;
    const typename F::Lane ln(v % F::UPB);
    // byte offset of the block of unit (u0 + v + LPR t) is blk0 + t * step
    const uint32_t row_off = (uint32_t)rloc * row_bytes;
    const uint32_t step = (uint32_t)(LPR / F::UPB) * F::BB;
    const uint32_t magic = magic_vgpr();

    float acc[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) acc[b] = 0.f;

    const int64_t units = K / F::UW;
    for (int64_t u0 = 0; u0 < units; u0 += tile_units) {
        const int U = (int)((units - u0) < tile_units ? (units - u0) : tile_units);
        const int T = (U + LPR - 1) / LPR;
        const uint32_t blk0 = row_off + (uint32_t)((u0 + v) / F::UPB) * F::BB;
        auto off_of = [&](int t) -> uint32_t {
            return (row_ok && v + LPR * t < U) ? blk0 + (uint32_t)t * step : OOB;
        };
        TileLds<F> L;
        L.carve(lds, U, nb);
        // activation loads first, then the weights, so the staging arithmetic
        // overlaps the weight stream
        XRaw<XT> xin;
        stage_issue<F, XT>(xs, u0 * F::UW, L, xin);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int P = RING ? D : (D < PF ? D : PF);
        // one unit's loads go out before the staging waits for the
        // activations (later loads would only queue ahead of them), the rest
        // of the prefetch right after
        Raw ring[D];
        ring[0] = F::load(rs, off_of(0), ln);
        __builtin_amdgcn_sched_barrier(0);
        stage_finish<F, XT, NT>(xs, u0 * F::UW, L, xin);
#pragma unroll
        for (int t = 1; t < P; ++t) ring[t] = F::load(rs, off_of(t), ln);
        if constexpr (!RING) {
#pragma unroll
            for (int t = 0; t < D; ++t) {
                if (t + P < D) ring[t + P] = F::load(rs, off_of(t + P), ln);
                if (t < T) {
                    const int u = v + LPR * t;
                    unit_math<F, BMAX>(L, ring[t], ln, u < U ? u : U - 1, u < U, magic, acc);
                }
            }
        } else {
            for (int t0 = 0; t0 < T; t0 += D) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    const int t = t0 + j;
                    const Raw cur = ring[j];
                    // unconditional refill (zeros past the tile): straight-line
                    // loads keep the load-counter waits exact
                    ring[j] = F::load(rs, off_of(t + D), ln);
                    if (t < T) {
                        const int u = v + LPR * t;
                        unit_math<F, BMAX>(L, cur, ln, u < U ? u : U - 1, u < U, magic, acc);
                    }
                }
            }
            // the last D refills were zero loads past the tile: drain them so
            // that no load is pending into these registers at the next tile
            wait_loads();
        }
        lds_barrier();
    }
    reduce_group<BMAX>(acc, LPR);
    if (v == 0 && row_ok) {
        const int64_t r = rowA + rloc;
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
            if (b < nb) yd.p[b][r] = acc[b];
    }
}

// LDS budget per workgroup for staged activations.
constexpr int LDS_BUDGET = 48 * 1024;

// ------------------------------------------------------ launch plan ----

struct Plan {
    int LPR, D, tile_units;
    bool ring;
    int64_t grid;
    size_t lds;
};

// Lanes per row (LPR) depends only on N and K, and every K tile holds a
// multiple of LPR units, so lane v of a row group always sums units v, v+LPR,
// v+2LPR, ... in the same order whatever the batch size: each batch column is
// bit-identical to a batch-1 product of the same vector.
//
// The choice: the fewest lanes per row (most rows per workgroup, so the
// activation staging is shared by more rows) that still gives at least ~2048
// wavefronts (8 per CU) and keeps >= 80% of the lanes busy; small matrices
// take more lanes per row to spread their bytes over more wavefronts.
template <class F>
inline int lanes_per_row(int64_t N, int64_t units, int min_lpr = 8) {
    int best = 0;
    double best_u = -1.0;
    for (int lpr = min_lpr; lpr <= 32; lpr <<= 1) {
        const int64_t slots = ((units + lpr - 1) / lpr) * lpr;
        const double util = units ? (double)units / (double)slots : 1.0;
        if (util >= 0.8 && N * lpr / 64 >= 2048) return lpr;
        if (util >= 0.8) {  // the widest well-used choice so far
            best = lpr;
            best_u = 2.0;
        } else if (best_u < 0.8 && util > best_u) {
            best = lpr;
            best_u = util;
        }
    }
    return best;
}

template <class F>
inline Plan plan_for(int64_t N, int64_t K, int nb, int64_t rows_in_flight = -1, int min_lpr = 8) {
    // rows_in_flight: rows of all products sharing the launch (several
    // experts' matrices in a routed product), which decides the lanes per row;
    // min_lpr 4 lets such a launch give a workgroup 64 rows, which spreads its
    // fixed costs (the grouping, the activation staging) over more rows
    Plan p;
    const int64_t units = K / F::UW;
    p.LPR = lanes_per_row<F>(rows_in_flight > 0 ? rows_in_flight : N, units, min_lpr);
    // K tile: as many units as the LDS budget allows for nb vectors, rounded
    // down to a multiple of LPR (a multiple of 4 units = whole super-blocks)
    const size_t per_unit = (size_t)16 * TileLds<F>::unit_stride(nb);
    const int64_t step = p.LPR;
    int64_t max_units = (int64_t)(LDS_BUDGET / per_unit) / step * step;
    if (max_units < step) max_units = step;
    if (units <= max_units) {
        p.tile_units = (int)(units > 0 ? units : 1);
    } else {
        const int64_t n_tiles = (units + max_units - 1) / max_units;
        const int64_t tu = (units + n_tiles - 1) / n_tiles;
        p.tile_units = (int)((tu + step - 1) / step * step);
    }
    const int T = (p.tile_units + p.LPR - 1) / p.LPR;
    p.ring = T > D_MAX;
    p.D = p.ring ? 0 : T;  // ring depth: chosen by the launcher
    const int SR = 64 / p.LPR;
    p.grid = (N + 4 * (int64_t)SR - 1) / (4 * (int64_t)SR);
    p.lds = per_unit * p.tile_units;
    return p;
}

}  // namespace gqd
