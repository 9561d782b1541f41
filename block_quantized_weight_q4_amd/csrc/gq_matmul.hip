// gq_matmul.hip -- prefill product Y[m][n] = sum_k X[m][k] w[n][k] with Q4_0,
// Q4_K, Q5_K or Q6_K weights and bf16 activations on the CDNA4 matrix cores (gfx950).
//
// The dequantise-then-matrix-engine step follows the prefill design of "Show
// HN: Gemma 4 26B-A4B at up to 100+ tokens/s on a 16 GB Mac" (Architecture
// section: the GPU expands the 4-bit experts to a dense 16-bit format which a
// matrix engine then multiplies); here both happen in one kernel, the weight
// tile being expanded to bf16 in LDS right before the MFMAs read it.  A
// Q4_K_M checkpoint ("GGUF in transformers", section on the GGUF format) mixes
// Q4_K with Q6_K tensors, so a layer's prefill needs both.
//
// Tiling.  A workgroup of 8 wavefronts (two per SIMD) owns a BM x BN =
// 256 x 256 tile of Y; wavefront (wm, wn) owns a 128 x 64 eighth as 8 x 4
// blocks of v_mfma_f32_16x16x32_bf16 (128 fp32 accumulators), so one
// wavefront's MFMAs run while the other expands weights or waits on LDS.  K
// advances in stages of BK = 64 inputs: one 32-byte slice of quants of a Q4_K
// super-block, two Q4_0 blocks, or the two 32-input quarters of a Q6_K
// super-block half whose low bits share 32 ql bytes (inputs 0-31 with 64-95,
// or 32-63 with 96-127, of the half; X's columns are taken in the same
// order).  Each thread expands its W row's slices of a stage and loads only
// the half of the stage's quant bytes those slices use.
//
// Pipeline.  LDS holds two stage buffers.  While the MFMAs of stage s read
// buffer s & 1, the wavefronts fill the other buffer with stage s+1: its W
// rows expanded to bf16 (the format's fp32 weight, one rounding to nearest
// even) in slices placed among or after a k step's MFMAs (per format:
// WF<>::IL), from global loads issued two
// stages ahead into two alternating register sets, and its X rows copied by
// the global-to-LDS form of the buffer load, issued at the start of stage s
// and waited for before its end (no registers and no LDS stores for X).  One
// LDS-only barrier per stage.  Measured against the earlier form of this
// kernel (32x32x16 MFMAs, X through registers, whole slices loaded; Q6_K on a
// 4-wavefront 128 x 128 variant): Q4_K 3015x17408x5120 3.0% faster, Q4_0
// 2.2%, Q6_K 3015x5120x17408 6.4%.
//
// Rows of X past M and of W past N, and inputs past K, are read as zeros
// (buffer loads beyond the resource's span); their outputs are never stored.
#include <atomic>

#include "gq_device.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDX = BK + 8;                   // bf16 per LDS row (+16 B pad: conflict-free b128 reads)
constexpr int ROWB = LDX * 2;                 // bytes per LDS row
// a stage buffer: X rows unpadded (128 B, 16-byte chunks XOR-swizzled), then
// W rows padded (conflict-free b128 reads)
constexpr int XROWS_BYTES = BM * 128;
constexpr int LDS8_BYTES = 2 * (XROWS_BYTES + BN * ROWB);  // 139,264 B

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) void* LdsPtr;

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Eight weights w_i = fmaf(s, q_i, -c) (q_i the bytes of two dwords whose
// every byte is below 256) packed to bf16.
__device__ __forceinline__ u32x4 expand_bytes(uint32_t w0, uint32_t w1, float s, float c) {
    // hide the known-zero bits: otherwise each byte is first extracted with a
    // bit-field instruction instead of being converted by v_cvt_f32_ubyteN
    __asm__("" : "+v"(w0), "+v"(w1));
    float a[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = (float)((w0 >> (8 * i)) & 0xffu);
        a[4 + i] = (float)((w1 >> (8 * i)) & 0xffu);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(s, a[i], -c);
    return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])};
}

// Weight formats.  For one W row and stage s a format loads the bytes that
// slices 2 part and 2 part + 1 need (load_part into Regs, from the row's
// buffer offset woff, NLOADS load instructions; ok == false loads zeros),
// decodes the stage's scales (Scl) and expands slice j (0..3) of them
// (expand_part): lo = stage inputs 8j..8j+7, hi = 32+8j..32+8j+7, as bf16.
template <int TYPE>
struct WF;

// Q4_K: stage s = slice c = s % 4 of super-block s / 4: quant bytes
// 32c..32c+31 (low nibbles: sub-block 2c = inputs 0..31 of the stage, high
// nibbles: 2c+1 = inputs 32..63) and the header.  w = (d sc) q - dmin m.
template <>
struct WF<T_Q4_K> {
    // input index of the stage's 8-input chunk c (c = 0..7): contiguous
    __device__ static uint32_t xin(int s, int c) { return (uint32_t)s * 64u + 8u * (uint32_t)c; }
    static constexpr int QK = 256, BB = 144;
    static constexpr int NLOADS = 2;  // load instructions per stage of load_part
    // where the W slices are expanded (measured, A-B-B-A): -1 after both
    // halves of a k step's MFMAs, 0 among the second half's, n > 0 there with
    // n VALU instructions placed after each MFMA
    static constexpr int IL = 3;
    struct Regs {
        u32x4 h, q0, q1;
    };
    struct Scl {
        float dsL, dmL, dsH, dmH;
    };
    // Selects rather than branches: the decode sits in the same scheduling
    // region as the MFMAs it is interleaved with.
    __device__ static Scl scales(const Regs& r, int s) {
        const int c = s & 3;
        const float d = h2f(r.h.x & 0xffffu), dmin = h2f(r.h.x >> 16);
        const int sh = 16 * (c & 1);
        const uint32_t b0 = r.h.y >> sh, b1 = r.h.z >> sh, b2 = r.h.w >> sh;
        const bool low = c < 2;
        const uint32_t scL = low ? (b0 & 63u) : ((b2 & 15u) | (((b0 >> 6) & 3u) << 4));
        const uint32_t mL = low ? (b1 & 63u) : (((b2 >> 4) & 15u) | (((b1 >> 6) & 3u) << 4));
        const uint32_t scH = low ? ((b0 >> 8) & 63u) : (((b2 >> 8) & 15u) | (((b0 >> 14) & 3u) << 4));
        const uint32_t mH = low ? ((b1 >> 8) & 63u) : (((b2 >> 12) & 15u) | (((b1 >> 14) & 3u) << 4));
        return Scl{d * (float)scL, dmin * (float)mL, d * (float)scH, dmin * (float)mH};
    }
    // quant bytes 8j..8j+7: low nibbles are inputs 8j.., high nibbles 32+8j..
    // w = (d*sc) * q - dmin*m: both products exact in fp32, one rounding
    __device__ static void expand(const Regs& r, const Scl& sc, int, int j, u32x4& lo, u32x4& hi) {
        const u32x4 q = j < 2 ? r.q0 : r.q1;
        const uint32_t w0 = q[2 * (j & 1)], w1 = q[2 * (j & 1) + 1];
        lo = expand_bytes(w0 & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, sc.dsL, sc.dmL);
        hi = expand_bytes((w0 >> 4) & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu, sc.dsH, sc.dmH);
    }
    // a thread that expands only slices 2 part, 2 part + 1 loads only their
    // 16 quant bytes (into q0)
    __device__ static void load_part(Rsrc wr, uint32_t woff, int s, bool ok, bool, int part, Regs& r) {
        const uint32_t bo = ok ? woff + (uint32_t)(s >> 2) * BB : 0x80000000u;
        r.h = bld16(wr, bo);
        r.q0 = bld16(wr, bo + 16 + 32 * (s & 3) + 16 * part);
    }
    __device__ static void expand_part(const Regs& r, const Scl& sc, int s, int j, u32x4& lo, u32x4& hi) {
        Regs t = r;
        t.q1 = r.q0;
        expand(t, sc, s, j, lo, hi);
    }
};

// Q5_K: Q4_K with a 32-byte plane of fifth bits at 16 (quants at 48): input
// 8j + i of slice j (low nibble, sub-block 2c) takes bit 2c of plane byte
// 8j + i as its bit 4, input 32 + 8j + i (high nibble) bit 2c + 1.
template <>
struct WF<T_Q5_K> {
    // input index of the stage's 8-input chunk c (c = 0..7): contiguous
    __device__ static uint32_t xin(int s, int c) { return (uint32_t)s * 64u + 8u * (uint32_t)c; }
    static constexpr int QK = 256, BB = 176;
    static constexpr int NLOADS = 3;
    static constexpr int IL = -1;  // among the MFMAs it spills
    struct Regs {
        u32x4 h, q0, q1, f0, f1;
    };
    using Scl = WF<T_Q4_K>::Scl;
    __device__ static Scl scales(const Regs& r, int s) {
        WF<T_Q4_K>::Regs h4;
        h4.h = r.h;
        return WF<T_Q4_K>::scales(h4, s);
    }
    __device__ static void load_part(Rsrc wr, uint32_t woff, int s, bool ok, bool, int part, Regs& r) {
        const uint32_t bo = ok ? woff + (uint32_t)(s >> 2) * BB : 0x80000000u;
        r.h = bld16(wr, bo);
        r.q0 = bld16(wr, bo + 48 + 32 * (s & 3) + 16 * part);
        r.f0 = bld16(wr, bo + 16 + 16 * part);
    }
    __device__ static void expand_part(const Regs& r, const Scl& sc, int s, int j, u32x4& lo, u32x4& hi) {
        Regs t = r;
        t.q1 = r.q0;
        t.f1 = r.f0;
        expand(t, sc, s, j, lo, hi);
    }
    __device__ static void expand(const Regs& r, const Scl& sc, int s, int j, u32x4& lo, u32x4& hi) {
        const u32x4 q = j < 2 ? r.q0 : r.q1, f = j < 2 ? r.f0 : r.f1;
        const int k = 2 * (j & 1);
        const uint32_t sl = 2u * (uint32_t)(s & 3), sh = sl + 1u;
        const uint32_t w0 = q[k], w1 = q[k + 1], f0 = f[k], f1 = f[k + 1];
        lo = expand_bytes((w0 & 0x0F0F0F0Fu) | (((f0 >> sl) & 0x01010101u) << 4),
                          (w1 & 0x0F0F0F0Fu) | (((f1 >> sl) & 0x01010101u) << 4), sc.dsL, sc.dmL);
        hi = expand_bytes(((w0 >> 4) & 0x0F0F0F0Fu) | (((f0 >> sh) & 0x01010101u) << 4),
                          ((w1 >> 4) & 0x0F0F0F0Fu) | (((f1 >> sh) & 0x01010101u) << 4), sc.dsH, sc.dmH);
    }
};

// Q4_0: stage s = blocks 2s (inputs 0..31) and 2s+1 (32..63), 36 bytes from
// row offset 36 s: block A = bytes 0..17 (d, then quants 2..17), block B =
// bytes 18..35.  Input i < 16 of a block is the low nibble of its quant byte
// i, input i >= 16 the high nibble of byte i-16.  w = d (q - 8), exact in fp32.
template <>
struct WF<T_Q4_0> {
    // input index of the stage's 8-input chunk c (c = 0..7): contiguous
    __device__ static uint32_t xin(int s, int c) { return (uint32_t)s * 64u + 8u * (uint32_t)c; }
    static constexpr int QK = 32, BB = 18;
    // (3 loads, the last one's address chosen by full, removes the 8-byte
    // spill but measured 1.3% slower)
    static constexpr int NLOADS = 4;
    static constexpr int IL = -1;  // 0 / 2 / 3: 6.5% / 6.5% / 4.5% slower
    struct Regs {
        u32x4 a, b;
        uint32_t c;
    };
    struct Scl {
        float dA, dB;
    };
    // full == false: the row ends after block A, and block B's bytes belong
    // to the next row or lie past the buffer (where a load that straddles the
    // end returns zeros as a whole) -- block A's last two quant bytes come
    // from a dword that ends with them, the rest is zero (d_B = 0)
    __device__ static void load(Rsrc wr, uint32_t woff, int s, bool ok, bool full, Regs& r) {
        const uint32_t bo = ok ? woff + (uint32_t)s * (2 * BB) : 0x80000000u;
        r.a = bld16(wr, bo);
        r.b = bld16(wr, bo + 16);
        r.c = __builtin_amdgcn_raw_buffer_load_b32(wr, (int)(bo + 32), 0, 0);
        const uint32_t tail = __builtin_amdgcn_raw_buffer_load_b32(wr, (int)(bo + 14), 0, 0);
        r.b = full ? r.b : u32x4{tail >> 16, 0u, 0u, 0u};
        r.c = full ? r.c : 0u;
    }
    __device__ static Scl scales(const Regs& r, int) { return Scl{h2f(r.a.x & 0xffffu), h2f(r.b.x >> 16)}; }
    __device__ static void expand(const Regs& r, const Scl& sc, int, int j, u32x4& lo, u32x4& hi) {
        // quant dwords: A = bytes 2..17 (straddling dwords), B = bytes 20..35
        const uint32_t qa[4] = {__builtin_amdgcn_alignbyte(r.a.y, r.a.x, 2), __builtin_amdgcn_alignbyte(r.a.z, r.a.y, 2),
                                __builtin_amdgcn_alignbyte(r.a.w, r.a.z, 2), __builtin_amdgcn_alignbyte(r.b.x, r.a.w, 2)};
        const uint32_t qb[4] = {r.b.y, r.b.z, r.b.w, r.c};
        const int k = 2 * (j & 1), sh = j < 2 ? 0 : 4;
        lo = expand_bytes((qa[k] >> sh) & 0x0F0F0F0Fu, (qa[k + 1] >> sh) & 0x0F0F0F0Fu, sc.dA, 8.0f * sc.dA);
        hi = expand_bytes((qb[k] >> sh) & 0x0F0F0F0Fu, (qb[k + 1] >> sh) & 0x0F0F0F0Fu, sc.dB, 8.0f * sc.dB);
    }
    // every slice needs both blocks' quant bytes: part loads load everything
    __device__ static void load_part(Rsrc wr, uint32_t woff, int s, bool ok, bool full, int, Regs& r) {
        load(wr, woff, s, ok, full, r);
    }
    __device__ static void expand_part(const Regs& r, const Scl& sc, int s, int j, u32x4& lo, u32x4& hi) {
        expand(r, sc, s, j, lo, hi);
    }
};

// Q6_K: stage s = quarter pair c = s % 4 of super-block s / 4: half h = c / 2,
// quarters jq = 2 (c & 1) (inputs 0..31 of the stage) and jq + 1 (32..63).
// Input l of quarter jq: q = nibble of ql[64h + 32 (jq & 1) + l] (low for
// jq < 2) | bits 2jq, 2jq+1 of qh[32h + l] << 4; sub-block 8h + 2jq + l/16.
// w = (d sc) (q - 32), one rounding.
template <>
struct WF<T_Q6_K> {
    static constexpr int QK = 256, BB = 210;
    // Stage s = (half h, part p) = ((s % 4) / 2, s % 2) of super-block s / 4:
    // the quarters p and p + 2 of half h, whose low 4 bits are the low and
    // high nibbles of the same 32 ql bytes 64h + 32p.. and whose high 2 bits
    // are bits 2p.. and 2p+4.. of the 32 qh bytes 128 + 32h...  Stage input
    // k < 32 is input 128h + 32p + k of the super-block, k >= 32 is input
    // 128h + 64 + 32p + (k - 32): the product sums over k, so X's columns
    // follow the same order (xin).
    struct Regs {
        u32x4 l0, l1, h0, h1;
        uint32_t sc, d;
    };
    struct Scl {
        float s[4];  // the stage's four 16-input scales: quarter p (two), quarter p + 2 (two)
    };
    __device__ static uint32_t xin(int s, int c) {
        const uint32_t c4 = (uint32_t)(s & 3);
        return (uint32_t)(s >> 2) * 256u + 128u * (c4 >> 1) + 32u * (c4 & 1u) + 8u * (uint32_t)c + (c >= 4 ? 32u : 0u);
    }
    __device__ static Scl scales(const Regs& r, int) {
        const float d = h2f(r.d);
        Scl o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o.s[i] = d * (float)(int)(int8_t)((r.sc >> (8 * i)) & 0xffu);
        return o;
    }
    // slice j: ql / qh bytes 8j..8j+7 of the stage's 32; lo = their low
    // nibbles with qh bits 2p (quarter p), hi = high nibbles with qh bits
    // 2p + 4 (quarter p + 2); w = (d sc) q - 32 (d sc)
    __device__ static void expand(const Regs& r, const Scl& sc, int s, int j, u32x4& lo, u32x4& hi) {
        const uint32_t sh = 2u * (uint32_t)(s & 1);
        const u32x4 lq = j < 2 ? r.l0 : r.l1, hq = j < 2 ? r.h0 : r.h1;
        const int k = 2 * (j & 1), i = j >> 1;  // bytes 8j.. lie in 16-input sub-block i of each quarter
        const uint32_t a0 = (lq[k] & 0x0F0F0F0Fu) | (((hq[k] >> sh) & 0x03030303u) << 4);
        const uint32_t a1 = (lq[k + 1] & 0x0F0F0F0Fu) | (((hq[k + 1] >> sh) & 0x03030303u) << 4);
        const uint32_t b0 = ((lq[k] >> 4) & 0x0F0F0F0Fu) | (((hq[k] >> (sh + 4)) & 0x03030303u) << 4);
        const uint32_t b1 = ((lq[k + 1] >> 4) & 0x0F0F0F0Fu) | (((hq[k + 1] >> (sh + 4)) & 0x03030303u) << 4);
        // selects, not an indexed array: j may be a runtime value, and an
        // indexed private array would live in scratch memory
        const float s_lo = i ? sc.s[1] : sc.s[0], s_hi = i ? sc.s[3] : sc.s[2];
        lo = expand_bytes(a0, a1, s_lo, 32.0f * s_lo);
        hi = expand_bytes(b0, b1, s_hi, 32.0f * s_hi);
    }
    // slices 2 part, 2 part + 1 use ql / qh bytes 16 part..16 part + 15 of
    // the stage's 32 (into l0 / h0), the scales and d
    static constexpr int NLOADS = 4;  // one scale load instead of two: 0.986-0.988 (A-B-B-A, twice)
    static constexpr int IL = 0;      // 3.8% faster than -1 (2: 2.8%)
    __device__ static void load_part(Rsrc wr, uint32_t woff, int s, bool ok, bool, int part, Regs& r) {
        const uint32_t c4 = (uint32_t)(s & 3), h = c4 >> 1, p = c4 & 1u;
        const uint32_t bo = ok ? woff + (uint32_t)(s >> 2) * BB : 0x80000000u;
        r.l0 = bld16(wr, bo + 64 * h + 32 * p + 16 * part);
        r.h0 = bld16(wr, bo + 128 + 32 * h + 16 * part);
        // the 8 scale bytes of half h in one load; the stage's four are
        // bytes 2p, 2p + 1 (quarter p) and 4 + 2p, 5 + 2p (quarter p + 2)
        const auto sv = __builtin_amdgcn_raw_buffer_load_b64(wr, (int)(bo + 192 + 8 * h), 0, 0);
        r.sc = __builtin_amdgcn_perm(sv[1], sv[0], p ? 0x07060302u : 0x05040100u);
        r.d = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(wr, (int)(bo + 208), 0, 0);
    }
    __device__ static void expand_part(const Regs& r, const Scl& sc, int s, int j, u32x4& lo, u32x4& hi) {
        Regs t = r;
        t.l1 = r.l0;
        t.h1 = r.h0;
        expand(t, sc, s, j, lo, hi);
    }
};

// Grid: one workgroup per output tile, tiles numbered n-tile fastest (gn of
// them per row of tiles).  Wavefront (wm, wn) = (wave / 4, wave % 4) owns a
// 128 x (NT / 4) part of the 256 x NT tile (8 x NT/64 blocks of 16x16x32
// MFMAs), so two wavefronts share each SIMD.  NT = 256 for whole tiles; when
// the last round would fill only part of the GPU and four workgroups per tile
// do not fit in it, its tiles (those from n_full on) are split in two K
// halves -- stages [0, s_split) and [s_split, S) -- added into Y.
// NT = 128 runs the tiles of a last, partial round as quarters: workgroup
// n_full + q takes N half (q / 2) % 2 and K half q % 2 of tile n_full + q / 4
// and adds its partial tile into Y (zeroed there beforehand), so that round
// takes about a quarter of a whole tile's time instead of half.  Both kinds
// of workgroup are one launch, so the quarters start on the CUs that the
// whole tiles free.
template <int TYPE, int NT>
__device__ __forceinline__ void matmul8_tile(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                             const uint16_t* __restrict__ X, int64_t M, int64_t ldx,
                                             float* __restrict__ Y, int64_t ldy, int gn, int n_full, int s_split,
                                             int wg) {
    using F = WF<TYPE>;
    using SR8 = typename F::Regs;                 // one stage's bytes of this thread's W row
    constexpr int JB = NT / 64;                   // 16-column blocks per wavefront
    constexpr int TBUF = XROWS_BYTES + NT * ROWB; // one stage buffer: X rows (swizzled) then W rows
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int S = (int)((K + BK - 1) / BK);
    bool split;
    int tile, s0, s1;
    int64_t n0;
    if constexpr (NT == 256) {
        split = wg >= n_full;
        tile = split ? n_full + ((wg - n_full) >> 1) : wg;
        s0 = split && ((wg - n_full) & 1) ? s_split : 0;
        s1 = split && !((wg - n_full) & 1) ? s_split : S;
        n0 = (int64_t)(tile % gn) * BN;
    } else {
        const int q = wg - n_full;
        split = true;
        tile = n_full + (q >> 2);
        s0 = (q & 1) ? s_split : 0;
        s1 = (q & 1) ? S : s_split;
        n0 = (int64_t)(tile % gn) * BN + NT * ((q >> 1) & 1);
        if (n0 >= N) return;  // the second half of a last, narrow column of tiles: nothing to compute
    }
    const int64_t m0 = (int64_t)(tile / gn) * BM;
    const uint32_t row_bytes = (uint32_t)((K / F::QK) * F::BB);

    const int64_t rows_x = M - m0 < BM ? M - m0 : BM, rows_w = N - n0 < NT ? N - n0 : NT;
    const Rsrc xr = make_rsrc(X + m0 * ldx, (uint32_t)(rows_x * ldx * 2));
    const Rsrc wr = make_rsrc(W + n0 * (int64_t)row_bytes, (uint32_t)rows_w * row_bytes);
    // X: wavefront w moves rows 32 w + 8 t + lane / 8 (t = 0..3) straight into
    // LDS; lane's 16 bytes land at position lane % 8 of its row, which holds
    // the row's 8-input chunk (lane % 8) ^ (row % 8)
    const int drow = 32 * wave + (lane >> 3), dchunk = (lane & 7) ^ (drow & 7);
    const uint32_t dsrc = (uint32_t)drow * (uint32_t)(ldx * 2), dstep = (uint32_t)(8 * ldx * 2);
    // W: thread tid expands row tid % NT; with NT = 256 wavefronts 0-3 take
    // slices 0, 1 and 4-7 slices 2, 3; with NT = 128 slice tid / 128
    const int wrow = tid & (NT - 1), wpart = NT == 256 ? wave >> 2 : tid >> 7;
    const uint32_t woff = (uint32_t)wrow * row_bytes;

    // inputs past K (the second half of a Q4_0 row's last stage) read as zeros
    auto dma_x = [&](int s, int buf) {
        const bool ok = s < s1 && (TYPE != T_Q4_0 || (int64_t)s * BK + 8 * dchunk < K);
        const uint32_t base = ok ? dsrc + 2u * F::xin(s, dchunk) : 0x80000000u;
#pragma unroll
        for (int t = 0; t < 4; ++t)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (LdsPtr)(lds + buf * TBUF + (32 * wave + 8 * t) * 128), 16,
                                                     ok ? base + (uint32_t)t * dstep : base, 0, 0, 0);
    };
    // the half of each stage's quant bytes this thread expands (slices
    // 2 part, 2 part + 1)
    const int part = NT == 256 ? wpart : wpart >> 1;
    auto load_stage = [&](int s, SR8& r) { F::load_part(wr, woff, s, s < s1, (int64_t)s * BK + 32 < K, part, r); };
    auto store_w = [&](int s, const SR8& r, const typename F::Scl& sc, int buf, int j) {
        uint8_t* ws = lds + buf * TBUF + XROWS_BYTES + wrow * ROWB;
        u32x4 lo, hi;
        F::expand_part(r, sc, s, j, lo, hi);
        reinterpret_cast<u32x4*>(ws)[j] = lo;
        reinterpret_cast<u32x4*>(ws + 64)[j] = hi;
    };
    // the stage's W slices this thread writes while k step ks runs
    auto store_w_at = [&](int ks, int s, const SR8& r, const typename F::Scl& sc, int buf) {
        if constexpr (NT == 256) {
            if ((ks & 1) == 0) store_w(s, r, sc, buf, 2 * wpart + (ks >> 1));
        } else {
            if (ks == 0) store_w(s, r, sc, buf, wpart);
        }
    };

    f32x4 acc[8][JB];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[i][j] = f32x4{};

    // fragment addresses (v_mfma_f32_16x16x32_bf16): A (X rows) lane l -> row
    // 16 i + l%16, inputs 8 (l/16)..+7 of the 32-deep k step; B (W rows) the
    // same with row 16 j + l%16 of the wavefront's columns
    const int fr = lane & 15, fk = 8 * (lane >> 4);
    const uint32_t a_base = (uint32_t)((wm * 128 + fr) * 128);
    uint32_t a_sw[2];  // the chunk 4 kk + lane / 16 of X row (16 i + fr): row % 8 = fr % 8
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) a_sw[kk] = (uint32_t)(((4 * kk + (lane >> 4)) ^ (fr & 7)) << 4);
    const uint32_t b_base = (uint32_t)(XROWS_BYTES + (wn * 16 * JB + fr) * ROWB + fk * 2);

    auto stage_body = [&](int s, SR8& nxt) {
        const int cur = (s - s0) & 1;
        const uint8_t* buf = lds + cur * TBUF;
        // stage s+1's X rows go straight into the other buffer, free since
        // the barrier that ended stage s-1
        dma_x(s + 1, cur ^ 1);
        const typename F::Scl sc = F::scales(nxt, s + 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 b[JB];
#pragma unroll
            for (int j = 0; j < JB; ++j) b[j] = *reinterpret_cast<const bf16x8*>(buf + b_base + j * 16 * ROWB + kk * 64);
            // the X fragments in two halves of four row blocks: fewer live
            // registers than all eight at once
#pragma unroll
            for (int ih = 0; ih < 2; ++ih) {
                bf16x8 a[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = *reinterpret_cast<const bf16x8*>(buf + a_base + (4 * ih + i) * 16 * 128 + a_sw[kk]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < JB; ++j)
                        acc[4 * ih + i][j] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[4 * ih + i][j], 0, 0, 0);
                if (F::IL >= 0 && ih == 1) {
                    // the next stage's W slices in the same scheduling region
                    // as the second half's MFMAs, IL VALU instructions after
                    // each MFMA when IL > 0
#pragma unroll
                    for (int h = 0; h < 2; ++h) store_w_at(2 * kk + h, s + 1, nxt, sc, cur ^ 1);
                    if constexpr (F::IL > 0) {
#pragma unroll
                        for (int q = 0; q < 4 * JB; ++q) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
                            __builtin_amdgcn_sched_group_barrier(0x002, F::IL, 0); // VALU
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (F::IL < 0) {
#pragma unroll
                for (int h = 0; h < 2; ++h) store_w_at(2 * kk + h, s + 1, nxt, sc, cur ^ 1);
            }
        }
        load_stage(s + 3, nxt);
        // the X rows of stage s+1 have landed: only the W loads of stage s+3,
        // issued after them, may still be in flight
        wait_vm<F::NLOADS>();
        lds_barrier();
    };

    SR8 r0, r1;
    if (s1 > s0) {
        dma_x(s0, 0);
        load_stage(s0, r0);
        load_stage(s0 + 1, r1);
        const typename F::Scl sc0 = F::scales(r0, s0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) store_w_at(ks, s0, r0, sc0, 0);
        load_stage(s0 + 2, r0);
        // stage s0's X rows and W loads have landed; those of s0+1 and s0+2
        // may be in flight
        wait_vm<2 * F::NLOADS>();
        lds_barrier();
    }
    for (int s = s0; s < s1; s += 2) {
        stage_body(s, r1);
        stage_body(s + 1, r0);
    }
    // C block (i, j): lane holds W row 16 j + lane%16 (column of Y) and X rows
    // 16 i + 4 (lane/16) + r for register r
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int64_t n = n0 + wn * 16 * JB + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 128 + 16 * i + 4 * (lane >> 4) + r;
                if (m < M && n < N) {
                    if (split) unsafeAtomicAdd(&Y[m * ldy + n], acc[i][j][r]);
                    else Y[m * ldy + n] = acc[i][j][r];
                }
            }
        }
    }
}

template <int TYPE>
__global__ __launch_bounds__(512, 1) void k_matmul8(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                    const uint16_t* __restrict__ X, int64_t M, int64_t ldx,
                                                    float* __restrict__ Y, int64_t ldy, int gn, int n_full,
                                                    int s_split, int quarters) {
    const int wg = (int)blockIdx.x;
    if (quarters && wg >= n_full)
        matmul8_tile<TYPE, 128>(W, N, K, X, M, ldx, Y, ldy, gn, n_full, s_split, wg);
    else
        matmul8_tile<TYPE, 256>(W, N, K, X, M, ldx, Y, ldy, gn, n_full, s_split, wg);
}

// Zeroes the output tiles from n_full on (clipped to M x N) before their two
// K halves are added in.
// Workgroup (r, t): rows 4r..4r+3 of split tile t, 64 threads per row, four
// columns per thread (16-byte stores: rows of Y are 16-byte aligned and the
// tile starts at a multiple of 256 columns).
__global__ __launch_bounds__(256) void k_zero_tiles(float* __restrict__ Y, int64_t ldy, int64_t M, int64_t N, int gn,
                                                    int n_full) {
    const int tile = n_full + (int)blockIdx.y;
    const int64_t n0 = (int64_t)(tile % gn) * BN, m0 = (int64_t)(tile / gn) * BM;
    const int64_t m = m0 + 4 * (int64_t)blockIdx.x + (threadIdx.x >> 6);
    if (m >= M) return;
    const int64_t n = n0 + 4 * (int64_t)(threadIdx.x & 63);
    float* y = Y + m * ldy + n;
    if (n + 4 <= N) {
        *reinterpret_cast<f32x4*>(y) = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        for (int i = 0; n + i < N; ++i) y[i] = 0.f;
    }
}

template <int TYPE>
hipError_t launch(const void* W, int64_t N, int64_t K, const void* X, int64_t M, int64_t ldx, float* Y, int64_t ldy,
                  hipStream_t s) {
    const int64_t gn = (N + BN - 1) / BN, gm = (M + BM - 1) / BM;
    const int64_t tiles = gn * gm;
    if (tiles > 0x3fffffff) return hipErrorInvalidValue;
    // one workgroup per CU (the LDS holds one).  A last round that would
    // fill only part of the GPU runs its tiles as N and K quarters when four
    // workgroups per tile fit in one round, else as K halves.
    const int cus = gqk_cu_count();
    const int64_t tail = tiles % cus;
    const int S = (int)((K + BK - 1) / BK);
    const bool part = tiles > cus && tail > 0 && S >= 4;
    const bool quarters = part && 4 * tail <= cus;
    const bool halves = !quarters && part && tail <= cus / 2;
    const int n_full = (int)(part && (quarters || halves) ? tiles - tail : tiles);
    if (n_full < tiles) {
        hipLaunchKernelGGL(k_zero_tiles, dim3(BM / 4, (unsigned)tail), dim3(256), 0, s, Y, ldy, M, N, (int)gn, n_full);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
    }
    // LDS above the default per-workgroup size (gfx950 allows 160 KB)
    const int64_t grid = halves ? n_full + 2 * tail : quarters ? n_full + 4 * tail : tiles;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_matmul8<TYPE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS8_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_matmul8<TYPE>, dim3((unsigned)grid), dim3(512), LDS8_BYTES, s,
                       static_cast<const uint8_t*>(W), N, K, static_cast<const uint16_t*>(X), M, ldx, Y, ldy,
                       (int)gn, n_full, S / 2, quarters ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

int gqk_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t gqk_matmul(int type, const void* W, int64_t N, int64_t K, const void* X, int x_dtype, int64_t M,
                      int64_t ldx, float* Y, int64_t ldy, hipStream_t s) {
    (void)x_dtype;  // validated by the ABI: bf16 activations
    if (type == T_Q4_0) return launch<T_Q4_0>(W, N, K, X, M, ldx, Y, ldy, s);
    if (type == T_Q6_K) return launch<T_Q6_K>(W, N, K, X, M, ldx, Y, ldy, s);
    if (type == T_Q5_K) return launch<T_Q5_K>(W, N, K, X, M, ldx, Y, ldy, s);
    return launch<T_Q4_K>(W, N, K, X, M, ldx, Y, ldy, s);
}
