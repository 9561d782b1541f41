// gq_matmul.hip -- prefill product Y[m][n] = sum_k X[m][k] w[n][k] with Q4_K
// weights and bf16 activations on the CDNA4 matrix cores (gfx950).
//
// The dequantise-then-matrix-engine step follows the prefill design of "Show
// HN: Gemma 4 26B-A4B at up to 100+ tokens/s on a 16 GB Mac" (Architecture
// section: the GPU expands the 4-bit experts to a dense 16-bit format which a
// matrix engine then multiplies); here both happen in one kernel, the weight
// tile being expanded to bf16 in LDS right before the MFMAs read it.
//
// Tiling.  A workgroup (4 wavefronts, one per SIMD) owns a BM x BN = 256 x 256
// tile of Y; wavefront (wm, wn) owns the 128 x 128 quarter, as 4 x 4 blocks
// of v_mfma_f32_32x32x16_bf16 (fp32 accumulators in the AGPRs).  K advances in
// stages of BK = 64 inputs = one 32-byte slice of quants of every Q4_K
// super-block row (sub-blocks 2c and 2c+1).
//
// Pipeline.  LDS holds two stage buffers.  While the MFMAs of stage s read
// buffer s & 1, the same wavefronts write stage s+1 -- its X rows as loaded and
// its W rows expanded to bf16 with w = (d * sc) * q - dmin * m in fp32, one
// rounding to nearest even -- into the other buffer, in four slices placed
// between the four 16-deep k steps; then they issue the global loads of stage
// s+3 into the registers just freed (two register sets alternate, so a load
// has more than a stage of MFMA work to arrive).  One LDS-only barrier per
// stage.
//
// Rows of X past M and of W past N are read as zeros (buffer loads beyond
// the resource's span); their outputs are never stored.
#include "gq_device.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDX = BK + 8;                   // bf16 per LDS row (+16 B pad: conflict-free b128 reads)
constexpr int ROWB = LDX * 2;                 // bytes per LDS row
constexpr int BUF = (BM + BN) * ROWB;         // one stage buffer: X rows then W rows
constexpr int LDS_BYTES = 2 * BUF;            // 147,456 B

typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Global data of one stage for this thread: eight 16-byte chunks of X (one
// from each of eight rows 32 apart), the 16-byte header and the 32-byte
// quant slice of its W row.
struct StageRegs {
    u32x4 x[8];
    u32x4 h, q0, q1;
};

// The (d*sc, dmin*m) pairs of sub-blocks 2c and 2c+1 (c uniform).
struct Scales {
    float dsL, dmL, dsH, dmH;
};

// Selects rather than branches: the decode sits in the same scheduling region
// as the MFMAs it is interleaved with.
__device__ __forceinline__ Scales q4k_scales(u32x4 hdr, int c) {
    const float d = h2f(hdr.x & 0xffffu), dmin = h2f(hdr.x >> 16);
    const int sh = 16 * (c & 1);
    const uint32_t b0 = hdr.y >> sh, b1 = hdr.z >> sh, b2 = hdr.w >> sh;
    const bool low = c < 2;
    const uint32_t scL = low ? (b0 & 63u) : ((b2 & 15u) | (((b0 >> 6) & 3u) << 4));
    const uint32_t mL = low ? (b1 & 63u) : (((b2 >> 4) & 15u) | (((b1 >> 6) & 3u) << 4));
    const uint32_t scH = low ? ((b0 >> 8) & 63u) : (((b2 >> 8) & 15u) | (((b0 >> 14) & 3u) << 4));
    const uint32_t mH = low ? ((b1 >> 8) & 63u) : (((b2 >> 12) & 15u) | (((b1 >> 14) & 3u) << 4));
    return Scales{d * (float)scL, dmin * (float)mL, d * (float)scH, dmin * (float)mH};
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Expand quant bytes 8j..8j+7 of the slice (dwords w0, w1): low nibbles are
// k = 8j..8j+7, high nibbles k = 32+8j..32+8j+7 -> two 16-byte rows of bf16.
__device__ __forceinline__ void expand8(uint32_t w0, uint32_t w1, const Scales& s, u32x4& lo, u32x4& hi) {
    uint32_t l0 = w0 & 0x0F0F0F0Fu, l1 = w1 & 0x0F0F0F0Fu;
    uint32_t h0 = (w0 >> 4) & 0x0F0F0F0Fu, h1 = (w1 >> 4) & 0x0F0F0F0Fu;
    // hide the known-zero bits: otherwise each byte is first extracted with a
    // bit-field instruction instead of being converted by v_cvt_f32_ubyteN
    __asm__("" : "+v"(l0), "+v"(l1), "+v"(h0), "+v"(h1));
    float a[8], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = (float)((l0 >> (8 * i)) & 0xffu);
        a[4 + i] = (float)((l1 >> (8 * i)) & 0xffu);
        b[i] = (float)((h0 >> (8 * i)) & 0xffu);
        b[4 + i] = (float)((h1 >> (8 * i)) & 0xffu);
    }
    // w = (d*sc) * q - dmin*m: both products exact in fp32, one rounding
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = __builtin_fmaf(s.dsL, a[i], -s.dmL);
        b[i] = __builtin_fmaf(s.dsH, b[i], -s.dmH);
    }
    lo = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])};
    hi = u32x4{pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]), pack_bf16x2(b[4], b[5]), pack_bf16x2(b[6], b[7])};
}

__global__ __launch_bounds__(256, 1) void k_matmul_q4k(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                       const uint16_t* __restrict__ X, int64_t M, int64_t ldx,
                                                       float* __restrict__ Y, int64_t ldy) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
    const uint32_t row_bytes = (uint32_t)((K / 256) * 144);
    const int S = (int)(K / BK);

    // X: thread tid stages 16-byte chunk tid % 8 of rows tid / 8 + 32 i
    // (i = 0..7): eight lanes cover one row's 128 bytes, so every load
    // instruction reads whole cache lines.  W: thread tid stages row n0 + tid.
    const int64_t rows_x = M - m0 < BM ? M - m0 : BM, rows_w = N - n0 < BN ? N - n0 : BN;
    const Rsrc xr = make_rsrc(X + m0 * ldx, (uint32_t)(rows_x * ldx * 2));
    const Rsrc wr = make_rsrc(W + n0 * (int64_t)row_bytes, (uint32_t)rows_w * row_bytes);
    const int xrow = tid >> 3, xchunk = tid & 7;
    const uint32_t xstride = (uint32_t)(32 * ldx * 2);
    const uint32_t xoff = (uint32_t)xrow * (uint32_t)(ldx * 2) + 16 * xchunk, woff = (uint32_t)tid * row_bytes;

    // a stage past the last loads zeros without touching memory (offset past
    // the buffers), so every load is unconditional and the load-counter waits
    // stay exact
    auto load_stage = [&](int s, StageRegs& r) {
        const bool ok = s < S;
        const uint32_t xo = ok ? xoff + (uint32_t)s * (BK * 2) : 0x80000000u;
#pragma unroll
        for (int i = 0; i < 8; ++i) r.x[i] = bld16(xr, ok ? xo + (uint32_t)i * xstride : xo);
        const uint32_t bo = ok ? woff + (uint32_t)(s >> 2) * 144 : 0x80000000u;
        r.h = bld16(wr, bo);
        r.q0 = bld16(wr, bo + 16 + 32 * (s & 3));
        r.q1 = bld16(wr, bo + 32 + 32 * (s & 3));
    };
    // slice j (0..3) of the stage's LDS writes: X chunks 2j, 2j+1 and W quant
    // bytes 8j..8j+7 expanded to k = 8j..8j+7 and 32+8j..32+8j+7
    auto store_slice = [&](int s, const StageRegs& r, const Scales& sc, int buf, int j) {
        uint8_t* xs = lds + buf * BUF + xrow * ROWB + 16 * xchunk;
        uint8_t* ws = lds + buf * BUF + BM * ROWB + tid * ROWB;
        *reinterpret_cast<u32x4*>(xs + (2 * j) * 32 * ROWB) = r.x[2 * j];
        *reinterpret_cast<u32x4*>(xs + (2 * j + 1) * 32 * ROWB) = r.x[2 * j + 1];
        const u32x4 q = j < 2 ? r.q0 : r.q1;
        u32x4 lo, hi;
        expand8(q[2 * (j & 1)], q[2 * (j & 1) + 1], sc, lo, hi);
        reinterpret_cast<u32x4*>(ws)[j] = lo;
        reinterpret_cast<u32x4*>(ws + 64)[j] = hi;
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // fragment addresses: A (X rows) lane l -> row 32*mi + l%32, k 8*(l/32);
    // B (W rows) lane l -> row 32*ni + l%32, same k
    const int fr = lane & 31, fk = 8 * (lane >> 5);
    const uint32_t a_base = (uint32_t)((wm * 128 + fr) * ROWB + fk * 2);
    const uint32_t b_base = (uint32_t)(BM * ROWB + (wn * 128 + fr) * ROWB + fk * 2);

    // stage s's global data lives in register set s & 1; it is loaded two
    // stages before its LDS writes, which happen during stage s-1's MFMAs
    auto stage_body = [&](int s, StageRegs& nxt) {
        const int cur = s & 1;
        const uint8_t* buf = lds + cur * BUF;
        // stage s+1's data arrived during the previous stage; past the last
        // stage it is zeros, written to a buffer nobody reads
        const Scales sc = q4k_scales(nxt.h, (s + 1) & 3);
        bf16x8 a[2][4], b[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[0][i] = *reinterpret_cast<const bf16x8*>(buf + a_base + i * 32 * ROWB);
            b[0][i] = *reinterpret_cast<const bf16x8*>(buf + b_base + i * 32 * ROWB);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int p = ks & 1;
            if (ks < 3) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[p ^ 1][i] = *reinterpret_cast<const bf16x8*>(buf + a_base + i * 32 * ROWB + (ks + 1) * 32);
                    b[p ^ 1][i] = *reinterpret_cast<const bf16x8*>(buf + b_base + i * 32 * ROWB + (ks + 1) * 32);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[p][i], b[p][j], acc[i][j], 0, 0, 0);
            store_slice(s + 1, nxt, sc, cur ^ 1, ks);
            // one k step = one scheduling region: each MFMA is followed by a
            // few VALU instructions of the expansion and the LDS traffic, so
            // they issue while the matrix core is busy
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if (ks < 3 && i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
                if ((i & 3) == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        load_stage(s + 3, nxt);
        lds_barrier();
    };

    // S is a multiple of 4 (K is whole super-blocks)
    StageRegs r0, r1;
    if (S > 0) {
        load_stage(0, r0);
        load_stage(1, r1);
        const Scales sc0 = q4k_scales(r0.h, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) store_slice(0, r0, sc0, 0, j);
        load_stage(2, r0);
        lds_barrier();
    }
    for (int s = 0; s < S; s += 2) {
        stage_body(s, r1);      // writes stage s+1 (set 1), then loads s+3 into set 1
        stage_body(s + 1, r0);  // writes stage s+2 (set 0), then loads s+4 into set 0
    }

    // C block (i, j): lane holds W row 32*j + lane%32 (column of Y) and X rows
    // 32*i + 8*(r/4) + 4*(lane/32) + r%4 for register r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 128 + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) Y[m * ldy + n] = acc[i][j][r];
            }
        }
    }
}

}  // namespace

hipError_t gqk_matmul(int type, const void* W, int64_t N, int64_t K, const void* X, int x_dtype, int64_t M,
                      int64_t ldx, float* Y, int64_t ldy, hipStream_t s) {
    (void)type;
    (void)x_dtype;  // validated by the ABI: Q4_K weights, bf16 activations
    const int64_t gn = (N + BN - 1) / BN, gm = (M + BM - 1) / BM;
    if (gn > 0x7fffffff || gm > 65535) return hipErrorInvalidValue;
    // LDS above the default per-workgroup size (gfx950 allows 160 KB)
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_matmul_q4k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_matmul_q4k, dim3((unsigned)gn, (unsigned)gm), dim3(256), LDS_BYTES, s,
                       static_cast<const uint8_t*>(W), N, K, static_cast<const uint16_t*>(X), M, ldx, Y, ldy);
    return hipGetLastError();
}
