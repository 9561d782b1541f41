// gq_matmul.hip -- prefill product Y[m][n] = sum_k X[m][k] w[n][k] with Q4_K
// weights and bf16 activations on the CDNA4 matrix cores (gfx950).
//
// The dequantise-then-matrix-engine step follows the prefill design of "Show
// HN: Gemma 4 26B-A4B at up to 100+ tokens/s on a 16 GB Mac" (Architecture
// section: the GPU expands the 4-bit experts to a dense 16-bit format which a
// matrix engine then multiplies); here both happen in one kernel, the weight
// tile being expanded to bf16 in LDS right before the MFMAs read it.
//
// Tiling.  A workgroup (4 wavefronts) owns a BM x BN = 256 x 128 tile of Y; a
// wavefront owns 128 x 64 of it as 8 x 4 blocks of v_mfma_f32_16x16x32_bf16
// (fp32 accumulators).  K advances in stages of BK = 64 inputs = one 32-byte
// slice of quants of every Q4_K super-block row (sub-blocks 2c and 2c+1).  Per
// stage each thread
//   * loads 128 bytes of one X row (bf16) and 16 quant bytes + the 16-byte
//     header of one W row, for the NEXT stage, into registers, while
//   * the MFMAs consume the current stage from LDS;
// then the registers are written to LDS -- X as is, W expanded to bf16 with
// w = (d * sc) * q - dmin * m in fp32, rounded to nearest even.
// Rows of X past M are zero; W rows past N are clamped to row N-1 and their
// outputs are never stored.
#include "gq_device.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LDX = BK + 8;  // bf16 per LDS row (+16 B pad: conflict-free b128 reads)
constexpr int LDS_X = BM * LDX * 2, LDS_W = BN * LDX * 2;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// (scale, min) of sub-block s from the 12 scale bytes (hdr.y, hdr.z, hdr.w)
__device__ __forceinline__ void q4k_sm(u32x4 hdr, int s, float d, float dmin, float& ds, float& dm) {
    int j = s & 3;
    uint32_t b0 = (hdr.y >> (8 * j)) & 0xffu, b1 = (hdr.z >> (8 * j)) & 0xffu, b2 = (hdr.w >> (8 * j)) & 0xffu;
    uint32_t sc, m;
    if (s < 4) {
        sc = b0 & 63u;
        m = b1 & 63u;
    } else {
        sc = (b2 & 15u) | ((b0 >> 6) << 4);
        m = (b2 >> 4) | ((b1 >> 6) << 4);
    }
    ds = d * (float)sc;
    dm = dmin * (float)m;
}

struct StageRegs {
    u32x4 x[8];     // 128 B of one X row (64 bf16)
    u32x4 q, hdr;   // 16 quant bytes and the header of one W row
};

__global__ __launch_bounds__(256) void k_matmul_q4k(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                    const uint16_t* __restrict__ X, int64_t M, int64_t ldx,
                                                    float* __restrict__ Y, int64_t ldy) {
    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t* Xs = reinterpret_cast<uint16_t*>(lds);
    uint16_t* Ws = reinterpret_cast<uint16_t*>(lds + LDS_X);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t row_bytes = (K / 256) * 144;

    // this thread's X row (one of 256) and W row / half (128 rows x 2 halves)
    const int64_t xm = m0 + tid;
    const bool x_ok = xm < M;
    const uint16_t* xrow = X + (x_ok ? xm : 0) * ldx;
    const int wr = tid >> 1, wh = tid & 1;
    const int64_t wnr = n0 + wr < N ? n0 + wr : N - 1;
    const uint8_t* wrow = W + wnr * row_bytes;

    auto load_stage = [&](int st, StageRegs& r) {
        const int64_t k0 = (int64_t)st * BK;
        const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + k0);
#pragma unroll
        for (int i = 0; i < 8; ++i) r.x[i] = x_ok ? xp[i] : u32x4{0, 0, 0, 0};
        const uint8_t* bp = wrow + (k0 >> 8) * 144;
        const int c = (int)((k0 >> 6) & 3);
        r.hdr = ld16a(bp);
        r.q = ld16a(bp + 16 + 32 * c + 16 * wh);
    };
    auto store_stage = [&](int st, const StageRegs& r) {
        u32x4* xd = reinterpret_cast<u32x4*>(Xs + tid * LDX);
#pragma unroll
        for (int i = 0; i < 8; ++i) xd[i] = r.x[i];
        // expand 32 weights: low nibbles -> sub-block 2c (k 16*wh + t),
        // high nibbles -> sub-block 2c+1 (k 32 + 16*wh + t)
        const int c = (int)((((int64_t)st * BK) >> 6) & 3);
        float d = h2f(r.hdr.x & 0xffffu), dmin = h2f(r.hdr.x >> 16);
        float dsL, dmL, dsH, dmH;
        q4k_sm(r.hdr, 2 * c, d, dmin, dsL, dmL);
        q4k_sm(r.hdr, 2 * c + 1, d, dmin, dsH, dmH);
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w = r.q[i];
            float ql[4], qh[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint32_t byte = (w >> (8 * b)) & 0xffu;
                ql[b] = (float)(byte & 15u);
                qh[b] = (float)(byte >> 4);
            }
            // w = (d*sc)*q - dmin*m: both products exact, one rounding
            lo[2 * i] = pack_bf16x2(__builtin_fmaf(dsL, ql[0], -dmL), __builtin_fmaf(dsL, ql[1], -dmL));
            lo[2 * i + 1] = pack_bf16x2(__builtin_fmaf(dsL, ql[2], -dmL), __builtin_fmaf(dsL, ql[3], -dmL));
            hi[2 * i] = pack_bf16x2(__builtin_fmaf(dsH, qh[0], -dmH), __builtin_fmaf(dsH, qh[1], -dmH));
            hi[2 * i + 1] = pack_bf16x2(__builtin_fmaf(dsH, qh[2], -dmH), __builtin_fmaf(dsH, qh[3], -dmH));
        }
        uint16_t* wd = Ws + wr * LDX + 16 * wh;
        reinterpret_cast<u32x4*>(wd)[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        reinterpret_cast<u32x4*>(wd)[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
        reinterpret_cast<u32x4*>(wd + 32)[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        reinterpret_cast<u32x4*>(wd + 32)[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
    };

    f32x4v acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

    const int n_stages = (int)(K / BK);
    StageRegs cur;
    if (n_stages > 0) load_stage(0, cur);
    for (int st = 0; st < n_stages; ++st) {
        store_stage(st, cur);
        lds_barrier();
        if (st + 1 < n_stages) load_stage(st + 1, cur);
        const int r16 = lane & 15, kq = 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 a[8], b[4];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(Xs + (wm * 128 + 16 * i + r16) * LDX + kk + kq);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(Ws + (wn * 64 + 16 * j + r16) * LDX + kk + kq);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        lds_barrier();
    }

    // C block (i, j): lane holds rows 4*(lane/16) + v (X rows), column lane%16 (W row)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 64 + 16 * j + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = m0 + wm * 128 + 16 * i + 4 * (lane >> 4) + v;
                if (m < M && n < N) Y[m * ldy + n] = acc[i][j][v];
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
    const size_t lds = (size_t)LDS_X + LDS_W;
    hipLaunchKernelGGL(k_matmul_q4k, dim3((unsigned)gn, (unsigned)gm), dim3(256), lds, s,
                       static_cast<const uint8_t*>(W), N, K, static_cast<const uint16_t*>(X), M, ldx, Y, ldy);
    return hipGetLastError();
}
