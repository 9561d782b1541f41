// gq_dequant.hip -- packed blocks -> fp32 / bf16 / fp16 weights (gfx950).
//
// The dequantising fallback of "GGUF in transformers" (sections "Load GGUF
// with transformers" and "transformers and llama.cpp": expanding the packed
// weights, e.g. to bf16 for fine-tuning).  Each weight is evaluated with fp32
// factors, left to right, exactly as the format defines it:
//   Q4_0  w = d * (q - 8)
//   Q4_K  w = (d * sc) * q - dmin * m
//   Q6_K  w = (d * sc) * (q - 32)
//   Q5_K  w = (d * sc) * q - dmin * m   (Q4_K's, with 5-bit q)
// Every product is exact in fp32 (fp16 d has 11 significant bits, the integer
// factors at most 12), so the fp32 result is unique; bf16/fp16 outputs are that
// fp32 value rounded to nearest even.
//
// One thread produces 8 consecutive weights (two 16-byte stores for fp32, one
// for 16-bit outputs); consecutive threads cover consecutive weights so the
// stores are fully coalesced.  Block loads are 8- or 16-byte vector loads that
// neighbouring threads share through the cache.
#include "gq_device.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

#pragma clang fp contract(off)

__device__ __forceinline__ void dq_q4_0(const uint8_t* blk, int part, float w[8]) {
    // part 0,1: low nibbles of quant bytes 8*part..; part 2,3: high nibbles of
    // bytes 8*(part-2)..  (weights 16..31)
    float d = h2f(ld2(blk));
    u32x2 q = ld8u(blk + 2 + 8 * (part & 1));
    int sh = (part >> 1) * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t byte = (q[i >> 2] >> (8 * (i & 3))) & 0xffu;
        int qq = (int)((byte >> sh) & 15u);
        w[i] = d * (float)(qq - 8);
    }
}

__device__ __forceinline__ void q4k_scale_min(u32x4 hdr, int s, int& sc, int& m) {
    // hdr.y = scale bytes 0..3, hdr.z = bytes 4..7, hdr.w = bytes 8..11
    int j = s & 3;
    uint32_t b0 = byte_of(hdr.y, j), b1 = byte_of(hdr.z, j), b2 = byte_of(hdr.w, j);
    if (s < 4) {
        sc = (int)(b0 & 63u);
        m = (int)(b1 & 63u);
    } else {
        sc = (int)((b2 & 15u) | ((b0 >> 6) << 4));
        m = (int)((b2 >> 4) | ((b1 >> 6) << 4));
    }
}

__device__ __forceinline__ void dq_q4_k(const uint8_t* blk, int part, float w[8]) {
    // part p: weights 8p..8p+7.  chunk c = p/8, j0 = 8*(p%8) within the chunk.
    u32x4 hdr = ld16a(blk);
    int c = part >> 3, j0 = 8 * (part & 7);
    int hi = j0 >= 32;
    int sub = 2 * c + hi;
    const uint8_t* qp = blk + 16 + 32 * c + (j0 & 31);
    u32x2 q = *reinterpret_cast<const u32x2*>(qp);
    int sc, m;
    q4k_scale_min(hdr, sub, sc, m);
    float d = h2f(hdr.x & 0xffffu), dmin = h2f(hdr.x >> 16);
    float a = d * (float)sc;
    float mm = dmin * (float)m;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t byte = (q[i >> 2] >> (8 * (i & 3))) & 0xffu;
        int qq = (int)(hi ? (byte >> 4) : (byte & 15u));
        float p = a * (float)qq;
        w[i] = p - mm;
    }
}

__device__ __forceinline__ void dq_q5_k(const uint8_t* blk, int part, float w[8]) {
    // as Q4_K with the quants 32 bytes further (after the fifth-bit plane);
    // weight 8p + i takes its fifth bit from bit `sub` of plane byte (j0 & 31) + i
    u32x4 hdr = ld16a(blk);
    int c = part >> 3, j0 = 8 * (part & 7);
    int hi = j0 >= 32;
    int sub = 2 * c + hi;
    u32x2 q = *reinterpret_cast<const u32x2*>(blk + 48 + 32 * c + (j0 & 31));
    u32x2 qh = *reinterpret_cast<const u32x2*>(blk + 16 + (j0 & 31));
    int sc, m;
    q4k_scale_min(hdr, sub, sc, m);
    float d = h2f(hdr.x & 0xffffu), dmin = h2f(hdr.x >> 16);
    float a = d * (float)sc;
    float mm = dmin * (float)m;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t byte = (q[i >> 2] >> (8 * (i & 3))) & 0xffu;
        uint32_t hb = (qh[i >> 2] >> (8 * (i & 3))) & 0xffu;
        int qq = (int)((hi ? (byte >> 4) : (byte & 15u)) | (((hb >> sub) & 1u) << 4));
        float p = a * (float)qq;
        w[i] = p - mm;
    }
}

__device__ __forceinline__ void dq_q6_k(const uint8_t* blk, int part, float w[8]) {
    // part p: weights 8p..8p+7 -> half h = p/16, r0 = 8*(p%16), group g = r0/32,
    // lane l0 = r0%32.
    int h = part >> 4, r0 = 8 * (part & 15), g = r0 >> 5, l0 = r0 & 31;
    u32x2 ql = ld8u(blk + 64 * h + l0 + 32 * (g & 1));
    u32x2 qh = ld8u(blk + 128 + 32 * h + l0);
    int sc = (int)(int8_t)blk[192 + 8 * h + (r0 >> 4)];
    float d = h2f(ld2(blk + 208));
    float a = d * (float)sc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t lb = (ql[i >> 2] >> (8 * (i & 3))) & 0xffu;
        uint32_t hb = (qh[i >> 2] >> (8 * (i & 3))) & 0xffu;
        uint32_t lo = g < 2 ? (lb & 15u) : (lb >> 4);
        uint32_t hi2 = (hb >> (2 * g)) & 3u;
        int qq = (int)(lo | (hi2 << 4));
        w[i] = a * (float)(qq - 32);
    }
}

template <int TYPE, int OUT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ blocks, int64_t n_parts,
                                                 void* __restrict__ out) {
    constexpr int QK = TYPE == T_Q4_0 ? 32 : 256;
    constexpr int BB = TYPE == T_Q4_0 ? 18 : (TYPE == T_Q4_K ? 144 : (TYPE == T_Q5_K ? 176 : 210));
    constexpr int PPB = QK / 8;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_parts) return;
    int64_t blk = gid / PPB;
    int part = (int)(gid - blk * PPB);
    const uint8_t* bp = blocks + blk * BB;
    float w[8];
    if (TYPE == T_Q4_0) dq_q4_0(bp, part, w);
    else if (TYPE == T_Q4_K) dq_q4_k(bp, part, w);
    else if (TYPE == T_Q5_K) dq_q5_k(bp, part, w);
    else dq_q6_k(bp, part, w);
    if (OUT == DT_F32) {
        f32x4* o = reinterpret_cast<f32x4*>(out) + 2 * gid;
        o[0] = f32x4{w[0], w[1], w[2], w[3]};
        o[1] = f32x4{w[4], w[5], w[6], w[7]};
    } else {
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo = OUT == DT_BF16 ? f2bf(w[2 * i]) : f2h(w[2 * i]);
            uint32_t hi = OUT == DT_BF16 ? f2bf(w[2 * i + 1]) : f2h(w[2 * i + 1]);
            p[i] = lo | (hi << 16);
        }
        reinterpret_cast<u32x4*>(out)[gid] = u32x4{p[0], p[1], p[2], p[3]};
    }
}

template <int TYPE>
hipError_t launch_t(const void* blocks, int64_t n_blocks, void* out, int out_dtype, hipStream_t s) {
    constexpr int QK = TYPE == T_Q4_0 ? 32 : 256;
    int64_t n_parts = n_blocks * (QK / 8);
    int64_t grid = (n_parts + 255) / 256;
    const uint8_t* b = static_cast<const uint8_t*>(blocks);
    if (out_dtype == DT_F32) hipLaunchKernelGGL((k_dequant<TYPE, DT_F32>), dim3((unsigned)grid), dim3(256), 0, s, b, n_parts, out);
    else if (out_dtype == DT_BF16) hipLaunchKernelGGL((k_dequant<TYPE, DT_BF16>), dim3((unsigned)grid), dim3(256), 0, s, b, n_parts, out);
    else hipLaunchKernelGGL((k_dequant<TYPE, DT_F16>), dim3((unsigned)grid), dim3(256), 0, s, b, n_parts, out);
    return hipGetLastError();
}

}  // namespace

hipError_t gqk_dequant(int type, const void* blocks, int64_t n_blocks, void* out, int out_dtype,
                       hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    if (type == T_Q4_0) return launch_t<T_Q4_0>(blocks, n_blocks, out, out_dtype, s);
    if (type == T_Q4_K) return launch_t<T_Q4_K>(blocks, n_blocks, out, out_dtype, s);
    if (type == T_Q5_K) return launch_t<T_Q5_K>(blocks, n_blocks, out, out_dtype, s);
    return launch_t<T_Q6_K>(blocks, n_blocks, out, out_dtype, s);
}
