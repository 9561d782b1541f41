// gq_gemv_core.h -- the decode product core shared by gq_matvec and
// gq_matvec_id (gfx950, wave64).
//
// Work split.  A workgroup (256 threads, 4 wavefronts) owns a tile of output
// rows and a small batch of activation vectors.  Each wavefront covers
// R * (64 / LPR) rows: its 64 lanes form 64/LPR groups of LPR lanes, one group
// per row, and inside a group lane v walks the row's "units" v, v+LPR, ...
// (a unit is 32 or 64 consecutive weights).  Every lane therefore streams its
// own 16-byte pieces of R rows with vector loads, unpacks them in registers and
// keeps fp32 partial sums; one shuffle reduction per output ends the kernel.
//
// Arithmetic.  A weight quant q (4 or 6 bits) is turned into the fp16 value
// 1024 + q (or 1024 + 16 q for a high nibble) by OR-ing it into the mantissa of
// 1024 -- two weights per 32-bit register with one AND-OR.  Activations are
// staged once per workgroup in LDS as fp16 pairs that match that register
// order, each group of 32 inputs scaled by a power of two 2^e so that its
// largest magnitude lies in [2^14, 2^15) (the scaling is exact; only the fp16
// rounding of the scaled value, at most 2^-11 relative, is inexact).  One
// v_dot2_f32_f16 then adds two weight-activation products into an fp32
// accumulator.  Per sub-block the format's scale (and min) are applied once:
//   Q4_0:  d * 2^-e * ( S_lo + S_hi / 16 )
//   Q4_K:  d*sc * 2^-e * S - dmin*m * sum(x)
//   Q6_K:  d*sc * 2^-e * S          (S / 16 for the high-nibble groups)
// where S is the integer-weighted dot product.  The constant 1024 (and the
// format's zero point 8 or 32) is removed by subtracting a correction that the
// staging step computes with exactly the same dot2 sequence applied to the
// zero-point's fp16 pattern, so a sub-block whose quants all equal the zero
// point contributes exactly zero.
#pragma once

#include "gq_device.h"

namespace gqd {

constexpr int NTHREADS = 256;

template <int TYPE>
struct Fmt;

// ---------------------------------------------------------------- Q4_0 ----
// Unit = one 18-byte block (32 weights).  Accumulator 0 = low nibbles
// (weights 0..15), accumulator 1 = high nibbles (weights 16..31).
template <>
struct Fmt<T_Q4_0> {
    static constexpr int QK = 32, BB = 18, UW = 32, NA = 2, NP = 8, NF = 1, NQ = NA * NP / 4;
    struct Raw {
        uint32_t d;
        u32x4 q;
    };
    struct Scl {
        float d;
    };
    __device__ static uint32_t zero_pattern(int a) { return a == 0 ? 0x64086408u : 0x64806480u; }
    __device__ static Raw load(const uint8_t* row, int unit) {
        const uint8_t* bp = row + (int64_t)unit * BB;
        Raw r;
        r.d = ld2(bp);
        r.q = ld16u(bp + 2);
        return r;
    }
    // first weight (relative to the unit's block row position) of accumulator a
    __device__ static int run_base(int unit, int a) { return 32 * unit + 16 * a; }
    // the runs of 32-input group g: run r covers group elements 16r..16r+15
    static constexpr int RPG = 2;
    __device__ static void group_run(int g, int r, int& unit, int& a) {
        unit = g;
        a = r;
    }
    __device__ static void pairs(const Raw& r, int a, uint32_t magic, uint32_t P[NP]) {
        const uint32_t mask = a == 0 ? 0x000F000Fu : 0x00F000F0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t w = r.q[k];
            P[2 * k] = (w & mask) | magic;
            P[2 * k + 1] = ((w >> 8) & mask) | magic;
        }
    }
    __device__ static Scl scales(const Raw& r, int) { return Scl{h2f(r.d)}; }
    // dacc[a] = accumulator - correction; f[0] = {corr0, corr1, 2^-e, 0}
    __device__ static float contrib(const Scl& s, const float dacc[NA], const f32x4 f[NF]) {
        return (s.d * f[0].z) * (dacc[0] + 0.0625f * dacc[1]);
    }
};

// ---------------------------------------------------------------- Q4_K ----
// Unit = a 32-byte slice of the quants (64 weights = sub-blocks 2c and 2c+1 of
// one super-block, c = unit % 4) plus the block's 16-byte header.
template <>
struct Fmt<T_Q4_K> {
    static constexpr int QK = 256, BB = 144, UW = 64, NA = 2, NP = 16, NF = 2, NQ = NA * NP / 4;
    struct Raw {
        u32x4 h, q0, q1;
    };
    struct Scl {
        float dsL, dsH, dmL, dmH;
    };
    __device__ static uint32_t zero_pattern(int) { return MAGIC; }
    __device__ static Raw load(const uint8_t* row, int unit) {
        const uint8_t* bp = row + (int64_t)(unit >> 2) * BB;
        int c = unit & 3;
        Raw r;
        r.h = ld16a(bp);
        r.q0 = ld16a(bp + 16 + 32 * c);
        r.q1 = ld16a(bp + 32 + 32 * c);
        return r;
    }
    __device__ static int run_base(int unit, int a) { return 256 * (unit >> 2) + 64 * (unit & 3) + 32 * a; }
    static constexpr int RPG = 1;
    __device__ static void group_run(int g, int, int& unit, int& a) {
        unit = g >> 1;
        a = g & 1;
    }
    __device__ static void pairs(const Raw& r, int a, uint32_t magic, uint32_t P[NP]) {
        const uint32_t mask = a == 0 ? 0x000F000Fu : 0x00F000F0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t w = k < 4 ? r.q0[k] : r.q1[k - 4];
            P[2 * k] = (w & mask) | magic;
            P[2 * k + 1] = ((w >> 8) & mask) | magic;
        }
    }
    // 6-bit (scale, min) of sub-blocks 2c and 2c+1: for c < 2 they are the low 6
    // bits of scale bytes s and s+4; for c >= 2 a low/high nibble of byte s+4
    // plus the top two bits of bytes s-4 and s.
    __device__ static Scl scales(const Raw& r, int unit) {
        int c = unit & 3;
        float d = h2f(r.h.x & 0xffffu), dmin = h2f(r.h.x >> 16);
        int sh = 16 * (c & 1);  // byte (2c) & 3 and (2c+1) & 3 -> shifts sh, sh+8
        uint32_t b0 = r.h.y >> sh, b1 = r.h.z >> sh, b2 = r.h.w >> sh;
        uint32_t scL, mL, scH, mH;
        if (c < 2) {
            scL = b0 & 63u;
            mL = b1 & 63u;
            scH = (b0 >> 8) & 63u;
            mH = (b1 >> 8) & 63u;
        } else {
            scL = (b2 & 15u) | (((b0 >> 6) & 3u) << 4);
            mL = ((b2 >> 4) & 15u) | (((b1 >> 6) & 3u) << 4);
            scH = ((b2 >> 8) & 15u) | (((b0 >> 14) & 3u) << 4);
            mH = ((b2 >> 12) & 15u) | (((b1 >> 14) & 3u) << 4);
        }
        Scl s;
        s.dsL = d * (float)scL;
        s.dsH = d * (float)scH * 0.0625f;
        s.dmL = dmin * (float)mL;
        s.dmH = dmin * (float)mH;
        return s;
    }
    // f[0] = {corrL, corrH, 2^-eL, 2^-eH}; f[1] = {sum xL, sum xH, 0, 0}
    __device__ static float contrib(const Scl& s, const float dacc[NA], const f32x4 f[NF]) {
        float v = (s.dsL * f[0].z) * dacc[0];
        v = __builtin_fmaf(s.dsH * f[0].w, dacc[1], v);
        v = __builtin_fmaf(-s.dmL, f[1].x, v);
        return __builtin_fmaf(-s.dmH, f[1].y, v);
    }
};

// ---------------------------------------------------------------- Q6_K ----
// Unit = (half h, lane half lh) of a super-block: lanes l = 16 lh .. 16 lh + 15
// of the four 32-weight groups g of half h (64 weights, four 16-weight
// sub-blocks).  Accumulator g.
template <>
struct Fmt<T_Q6_K> {
    static constexpr int QK = 256, BB = 210, UW = 64, NA = 4, NP = 8, NF = 2, NQ = NA * NP / 4;
    struct Raw {
        u32x4 la, lb, qh;
        u32x2 sc;
        uint32_t d;
    };
    struct Scl {
        float ds[4];
    };
    // zero point q = 32: 1024 + 32 for groups 0,1 and 1024 + 16*32 for 2,3
    __device__ static uint32_t zero_pattern(int a) { return a < 2 ? 0x64206420u : 0x66006600u; }
    __device__ static Raw load(const uint8_t* row, int unit) {
        const uint8_t* bp = row + (int64_t)(unit >> 2) * BB;
        int h = (unit >> 1) & 1, lh = unit & 1;
        Raw r;
        r.la = ld16u(bp + 64 * h + 16 * lh);
        r.lb = ld16u(bp + 64 * h + 32 + 16 * lh);
        r.qh = ld16u(bp + 128 + 32 * h + 16 * lh);
        r.sc = ld8u(bp + 192 + 8 * h);
        r.d = ld2(bp + 208);
        return r;
    }
    __device__ static int run_base(int unit, int a) {
        return 256 * (unit >> 2) + 128 * ((unit >> 1) & 1) + 32 * a + 16 * (unit & 1);
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
                P[2 * k + j] = v | magic;
            }
        }
    }
    __device__ static Scl scales(const Raw& r, int unit) {
        int sh = 8 * (unit & 1);
        float d = h2f(r.d);
        Scl s;
        s.ds[0] = d * (float)(int)(int8_t)(r.sc.x >> sh);
        s.ds[1] = d * (float)(int)(int8_t)(r.sc.x >> (sh + 16));
        s.ds[2] = d * (float)(int)(int8_t)(r.sc.y >> sh) * 0.0625f;
        s.ds[3] = d * (float)(int)(int8_t)(r.sc.y >> (sh + 16)) * 0.0625f;
        return s;
    }
    // f[0] = corrections of groups 0..3; f[1] = 2^-e of groups 0..3
    __device__ static float contrib(const Scl& s, const float dacc[NA], const f32x4 f[NF]) {
        float v = (s.ds[0] * f[1].x) * dacc[0];
        v = __builtin_fmaf(s.ds[1] * f[1].y, dacc[1], v);
        v = __builtin_fmaf(s.ds[2] * f[1].z, dacc[2], v);
        return __builtin_fmaf(s.ds[3] * f[1].w, dacc[3], v);
    }
};

// ----------------------------------------------------------- staging ----

// Where the activation vectors of this workgroup live: p[b] points at element
// 0 of vector b.  The element type is a template parameter XT of the kernels
// (0 = fp32, 1 = bf16).  Only ever indexed with a wave-uniform b.
struct XSrc {
    const uint8_t* p[8];
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

template <int XT>
__device__ __forceinline__ float group_elem(const XRaw<XT>& r, int i) {
    // (element copied to a scalar first: __builtin_bit_cast of a vector-element
    // lvalue reads element 0 with this compiler)
    if (XT == 0) {
        uint32_t w = r.q[i >> 2][i & 3];
        return __builtin_bit_cast(float, w);
    }
    uint32_t w = r.q[i >> 3][(i >> 1) & 3];
    return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Exponent e that puts max|x| of a 32-group into [2^14, 2^15); 0 for a group
// that is all zero or holds Inf/NaN (which then propagate).
__device__ __forceinline__ int group_exp(float m) {
    if (!(m > 0.f) || !(m < __builtin_inff())) return 0;
    return 15 - __builtin_amdgcn_frexp_expf(m);
}

// Staged activations of one K tile, unit-major: the record of (unit u,
// vector b) is NQ fp16-pair quads followed by NF factor vectors, 16 B each, at
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

// Barrier for LDS traffic only.  __syncthreads() is a full workgroup fence,
// which on gfx950 also waits for every outstanding global load (vmcnt(0)) --
// here that would stall on the weight loads already in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Staging of the activations of inputs [k0, k0 + U*UW) for nb vectors, in one
// pass: a thread takes one accumulator run (16 or 32 consecutive inputs); it
// reads the whole 32-input group the run lies in, finds the group's exponent,
// rounds the scaled run to fp16 pairs in unpack order, and computes the
// zero-point correction with the same dot2 chain the main loop will run.
// Every run lies inside one 32-group in all three formats.
//
// stage_issue loads the group of the thread's first run; the caller then
// issues the weight loads, so the (in-order) load counter lets staging proceed
// as soon as the activations arrive.  stage_finish does the arithmetic, any
// further runs, and ends with an LDS barrier.
// One run (16 or 32 consecutive inputs starting at group element `off`) of an
// already-scaled group -> fp16 pairs in unpack order, its zero-point
// correction, and its factors.
template <class F>
__device__ __forceinline__ void stage_write_run(const TileLds<F>& L, int b, int u, int a, const float* r, int e) {
    constexpr int RUN = 2 * F::NP;
    uint32_t P[F::NP];
    float sx = 0.f;
#pragma unroll
    for (int n = 0; n < F::NP; ++n) {
        int t = 4 * (n >> 1) + (n & 1);
        P[n] = pack_h2(r[t], r[t + 2]);
    }
#pragma unroll
    for (int t = 0; t < RUN; ++t) sx += (float)(_Float16)r[t];
    u32x4* rp = L.rec(u, b);
#pragma unroll
    for (int qd = 0; qd < F::NP / 4; ++qd)
        rp[a * (F::NP / 4) + qd] = u32x4{P[4 * qd], P[4 * qd + 1], P[4 * qd + 2], P[4 * qd + 3]};
    const uint32_t z = F::zero_pattern(a);
    float corr = 0.f;
#pragma unroll
    for (int n = 0; n < F::NP; ++n) corr = dot2(z, P[n], corr);
    float sc = __builtin_ldexpf(1.0f, -e);
    float* f0 = reinterpret_cast<float*>(rp + F::NQ);
    float* f1 = reinterpret_cast<float*>(rp + F::NQ + F::NF - 1);
    if (F::NA == 2 && F::NF == 1) {  // Q4_0: {corr0, corr1, 2^-e, 0}
        f0[a] = corr;
        if (a == 0) f0[2] = sc;
        else f0[3] = 0.f;
    } else if (F::NA == 2) {         // Q4_K: {corrL, corrH, sL, sH}, {sum xL, sum xH, 0, 0}
        f0[a] = corr;
        f0[2 + a] = sc;
        f1[a] = sx * sc;
        f1[2 + a] = 0.f;
    } else {                         // Q6_K: {corr0..3}, {s0..3}
        f0[a] = corr;
        f1[a] = sc;
    }
}

// A whole 32-input group of vector b: exponent, scaling, and every run in it.
template <class F, int XT>
__device__ __forceinline__ void stage_group(const TileLds<F>& L, int b, int g, const XRaw<XT>& in) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = group_elem<XT>(in, i);
    float m = 0.f;
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
        nan |= v[i] != v[i];
    }
    int e = group_exp(nan ? __builtin_nanf("") : m);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = __builtin_ldexpf(v[i], e);
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
// remaining groups (loop over vectors is wave-uniform, so the vector pointer
// stays a scalar) and ends with an LDS barrier.
template <class F, int XT>
__device__ __forceinline__ void stage_issue(const XSrc& xs, int64_t k0, const TileLds<F>& L, XRaw<XT>& in) {
    const int G = L.U * F::UW / 32;
    if ((int)threadIdx.x < G) load_group<XT>(xs.p[0], k0 + 32 * threadIdx.x, in);
}

template <class F, int XT>
__device__ __forceinline__ void stage_finish(const XSrc& xs, int64_t k0, const TileLds<F>& L,
                                             const XRaw<XT>& first) {
    const int G = L.U * F::UW / 32;
    if ((int)threadIdx.x < G) stage_group<F, XT>(L, 0, threadIdx.x, first);
    for (int g = threadIdx.x + blockDim.x; g < G; g += blockDim.x) {
        XRaw<XT> in;
        load_group<XT>(xs.p[0], k0 + 32 * g, in);
        stage_group<F, XT>(L, 0, g, in);
    }
    for (int b = 1; b < L.nb; ++b) {
        const uint8_t* xb = xs.p[b];
        for (int g = threadIdx.x; g < G; g += blockDim.x) {
            XRaw<XT> in;
            load_group<XT>(xb, k0 + 32 * g, in);
            stage_group<F, XT>(L, b, g, in);
        }
    }
    lds_barrier();
}

// ----------------------------------------------------------- compute ----

// Load the R rows' unit (unit0 + min(u, U-1)) -- clamped so the last, partly
// idle iteration never reads outside the tile.
template <class F, int R>
__device__ __forceinline__ void load_units(const uint8_t* const rowp[R], int unit0, int u, int U,
                                           typename F::Raw raw[R]) {
    int uc = u < U ? u : U - 1;
#pragma unroll
    for (int i = 0; i < R; ++i) raw[i] = F::load(rowp[i], unit0 + uc);
}

// One unit of R rows against nb staged vectors.  All LDS reads of a vector's
// record are issued before its dot products, so one LDS latency is paid per
// unit and vector.
template <class F, int BMAX, int R>
__device__ __forceinline__ void unit_math(const TileLds<F>& L, const typename F::Raw raw[R], int unit, int uc,
                                          bool valid, uint32_t magic, float acc[R][BMAX]) {
    const int nb = L.nb;
    typename F::Scl sc[R];
#pragma unroll
    for (int i = 0; i < R; ++i) sc[i] = F::scales(raw[i], unit);
    uint32_t P[R][F::NA][F::NP];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int a = 0; a < F::NA; ++a) F::pairs(raw[i], a, magic, P[i][a]);
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        if (b >= nb) break;
        const u32x4* rp = L.rec(uc, b);
        u32x4 xq[F::NQ];
        f32x4 f[F::NF];
#pragma unroll
        for (int q = 0; q < F::NQ; ++q) xq[q] = rp[q];
#pragma unroll
        for (int j = 0; j < F::NF; ++j) f[j] = __builtin_bit_cast(f32x4, rp[F::NQ + j]);
        float dacc[R][F::NA];
#pragma unroll
        for (int a = 0; a < F::NA; ++a) {
            float s[R];
#pragma unroll
            for (int i = 0; i < R; ++i) s[i] = 0.f;
#pragma unroll
            for (int qd = 0; qd < F::NP / 4; ++qd) {
                const u32x4 xv = xq[a * (F::NP / 4) + qd];
#pragma unroll
                for (int n4 = 0; n4 < 4; ++n4) {
                    const uint32_t xe = xv[n4];
#pragma unroll
                    for (int i = 0; i < R; ++i) s[i] = dot2(P[i][a][4 * qd + n4], xe, s[i]);
                }
            }
            const float corr = f[0][a];
#pragma unroll
            for (int i = 0; i < R; ++i) dacc[i][a] = s[i] - corr;
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float c = F::contrib(sc[i], dacc[i], f);
            acc[i][b] += valid ? c : 0.f;
        }
    }
}

// Accumulate the tile [unit0, unit0 + U) of R rows (pointers rowp[i]) for
// nb <= BMAX vectors into acc[R][BMAX].  Lane v of an LPR-lane group handles
// units v, v + LPR, ...  `ring` holds the loads of the lane's first D units on
// entry (issued before the activations were staged); the loads of unit t + D
// are issued right after unit t's registers are consumed, so D units per row
// are always in flight.
template <class F, int BMAX, int R, int D>
__device__ __forceinline__ void compute_tile(const TileLds<F>& L, const uint8_t* const rowp[R], int unit0, int v,
                                             int LPR, typename F::Raw ring[D][R], float acc[R][BMAX]) {
    const int U = L.U;
    const int T = (U + LPR - 1) / LPR;
    const uint32_t magic = magic_vgpr();
    for (int t0 = 0; t0 < T; t0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            int t = t0 + j;
            int u = v + LPR * t;
            bool valid = u < U;
            int uc = valid ? u : U - 1;
            typename F::Raw cur[R];
#pragma unroll
            for (int i = 0; i < R; ++i) cur[i] = ring[j][i];
            // unconditional (clamped) refill: straight-line loads keep the
            // load-counter waits exact
            load_units<F, R>(rowp, unit0, u + LPR * D, U, ring[j]);
            if (t < T) unit_math<F, BMAX, R>(L, cur, unit0 + uc, uc, valid, magic, acc);
        }
    }
}

template <class F, int R, int D>
__device__ __forceinline__ void prefetch_ring(const uint8_t* const rowp[R], int unit0, int v, int LPR, int U,
                                              typename F::Raw ring[D][R]) {
#pragma unroll
    for (int j = 0; j < D; ++j) load_units<F, R>(rowp, unit0, v + LPR * j, U, ring[j]);
}

// Sum acc over the LPR lanes of each group (lanes differ only in the low bits).
template <int BMAX, int R>
__device__ __forceinline__ void reduce_group(float acc[R][BMAX], int LPR) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
            for (int off = LPR >> 1; off > 0; off >>= 1) acc[i][b] += __shfl_xor(acc[i][b], off);
}

// Output rows of the vectors: y_b[n] = p[b][n].  Wave-uniform.
struct YDst {
    float* p[8];
};

// The whole decode product for one workgroup: rows [rowA, rowA + waves*R*SR)
// of the packed matrix W (N rows, K inputs) against nb <= BMAX staged vectors.
template <int TYPE, int XT, int BMAX, int R, int D>
__device__ __forceinline__ void gemv_workgroup(const uint8_t* __restrict__ W, int64_t N, int64_t K, int64_t rowA,
                                               const XSrc& xs, int nb, const YDst& yd, int LPR, int tile_units,
                                               uint8_t* lds) {
    using F = Fmt<TYPE>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int SR = 64 / LPR;
    const int s = lane / LPR, v = lane - s * LPR;
    const int64_t row_bytes = (K / F::QK) * F::BB;
    const int64_t row0 = rowA + (int64_t)wave * R * SR + s;

    const uint8_t* rowp[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        int64_t r = row0 + (int64_t)i * SR;
        rowp[i] = W + (r < N ? r : N - 1) * row_bytes;
    }
    float acc[R][BMAX];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int b = 0; b < BMAX; ++b) acc[i][b] = 0.f;

    const int64_t units = K / F::UW;
    for (int64_t u0 = 0; u0 < units; u0 += tile_units) {
        int U = (int)((units - u0) < tile_units ? (units - u0) : tile_units);
        TileLds<F> L;
        L.carve(lds, U, nb);
        // activation loads first, then the first D units of weights, so the
        // staging arithmetic overlaps the weight stream
        XRaw<XT> xin;
        stage_issue<F, XT>(xs, u0 * F::UW, L, xin);
        __builtin_amdgcn_sched_barrier(0);
        typename F::Raw ring[D][R];
        prefetch_ring<F, R, D>(rowp, (int)u0, v, LPR, U, ring);
        __builtin_amdgcn_sched_barrier(0);
        stage_finish<F, XT>(xs, u0 * F::UW, L, xin);
        compute_tile<F, BMAX, R, D>(L, rowp, (int)u0, v, LPR, ring, acc);
        lds_barrier();
    }
    reduce_group<BMAX, R>(acc, LPR);
    if (v == 0) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            int64_t r = row0 + (int64_t)i * SR;
            if (r < N) {
#pragma unroll
                for (int b = 0; b < BMAX; ++b)
                    if (b < nb) yd.p[b][r] = acc[i][b];
            }
        }
    }
}

// LDS budget per workgroup for staged activations.
constexpr int LDS_BUDGET = 48 * 1024;

// ------------------------------------------------------ launch plan ----

struct Plan {
    int LPR, R, WPW, tile_units;
    int64_t grid;
    size_t lds;
};

// Lanes per row (LPR) depends only on K, and every K tile holds a multiple of
// LPR units, so lane v of a row group always sums units v, v+LPR, v+2LPR, ...
// in the same order whatever the batch size: each batch column is
// bit-identical to a batch-1 product of the same vector.  (Rows per lane R and
// waves per workgroup only decide which lane group owns a row.)
template <class F>
inline int lanes_per_row(int64_t units) {
    // 32 at most: a tile of 32 units for 8 vectors still fits the LDS budget
    int best = 32;
    double best_u = -1;
    for (int lpr = 32; lpr >= 8; lpr >>= 1) {
        int64_t slots = ((units + lpr - 1) / lpr) * lpr;
        double util = units ? (double)units / (double)slots : 1.0;
        if (util >= 0.9) return lpr;
        if (util > best_u + 1e-9) {
            best_u = util;
            best = lpr;
        }
    }
    return best;
}

template <class F>
inline Plan plan_for(int64_t N, int64_t K, int nb) {
    Plan p;
    int64_t units = K / F::UW;
    p.LPR = lanes_per_row<F>(units);
    const int SR = 64 / p.LPR;
    // K tile: as many units as the LDS budget allows for nb vectors, rounded
    // down to a multiple of LPR (a multiple of 4 units = whole super-blocks)
    size_t per_unit = (size_t)16 * TileLds<F>::unit_stride(nb);
    int64_t step = p.LPR;
    int64_t max_units = (int64_t)(LDS_BUDGET / per_unit) / step * step;
    if (max_units < step) max_units = step;
    if (units <= max_units) {
        p.tile_units = (int)(units > 0 ? units : 1);
    } else {
        int64_t n_tiles = (units + max_units - 1) / max_units;
        int64_t tu = (units + n_tiles - 1) / n_tiles;
        p.tile_units = (int)((tu + step - 1) / step * step);
    }
    // rows per lane group (R = 2 would let one LDS read of an activation serve
    // two rows, but costs too many registers at present)
    p.R = 1;
    // waves per workgroup: the most (least staging per row) that still gives
    // >= 512 workgroups (two per CU); for small N fewer rows per lane group
    p.WPW = 1;
    for (int w = 4; w >= 1; w >>= 1) {
        if ((N + (int64_t)w * p.R * SR - 1) / ((int64_t)w * p.R * SR) >= 512) {
            p.WPW = w;
            break;
        }
    }
    p.grid = (N + (int64_t)p.WPW * p.R * SR - 1) / ((int64_t)p.WPW * p.R * SR);
    p.lds = per_unit * p.tile_units;
    return p;
}

}  // namespace gqd
