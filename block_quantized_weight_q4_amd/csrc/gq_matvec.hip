// gq_matvec.hip -- decode product y[b][n] = sum_k w[n][k] x[b][k] against
// packed Q4_0 / Q4_K / Q6_K rows (gfx950).  The per-lane work is in
// gq_gemv_core.h; this file maps workgroups to row tiles and picks the kernel
// variant (vectors per workgroup, units per lane in flight).
//
// Grid: one 4-wavefront workgroup per tile of 4 * (64 / LPR) consecutive rows.
// The activations are staged tile by tile along K (each tile fits the LDS
// budget; at batch 1 all of K is one tile), and the lane partial sums stay in
// registers across K tiles, so every packed byte is read exactly once.
#include "gq_gemv_core.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

// WGW wavefronts per workgroup: 4, or 8 for products whose 8-wave grid holds
// 150..256 workgroups -- twice the rows then share each staged activation
// tile and the staging has twice the threads, while every workgroup still
// gets a CU of its own (measured: the 2560-row projections of the hidden-2560
// layer gain 10-20% at 1 vector and 9-11% at 2; grids of 64-128 workgroups
// lose, since fewer CUs then pull the weights).
template <int TYPE, int XT, int BMAX, int D, bool RING, int WGW>
__global__ __launch_bounds__(64 * WGW) void k_matvec(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                     XSrc xs, int nb, YDst yd, int LPR, int tile_units) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int64_t rpw = (int64_t)WGW * (64 / LPR);
    gemv_workgroup<TYPE, XT, BMAX, D, RING, 64 * WGW, 1>(W, N, K, (int64_t)blockIdx.x * rpw, xs, nb, yd, LPR, tile_units, lds,
                                            (int)(threadIdx.x >> 6), WGW);
}

template <int TYPE, int XT, int BMAX, int WGW, int D, bool RING = false>
hipError_t launch_d(const Plan& p, const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y,
                    hipStream_t s) {
    YDst yd;
    for (int b = 0; b < 8; ++b) yd.p[b] = y + (int64_t)(b < nb ? b : 0) * N;
    const int64_t rows = (int64_t)WGW * (64 / p.LPR);
    const int64_t grid = (N + rows - 1) / rows;
    hipLaunchKernelGGL((k_matvec<TYPE, XT, BMAX, D, RING, WGW>), dim3((unsigned)grid), dim3(64 * WGW), p.lds, s, W,
                       N, K, xs, nb, yd, p.LPR, p.tile_units);
    return hipGetLastError();
}

template <int TYPE, int XT, int BMAX, int WGW>
hipError_t launch_w(const Plan& p, const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y,
                    hipStream_t s) {
    if (p.ring) {
        // units in flight per lane: 1 while the launch gives each CU at most
        // 12 wavefronts (the occupancy then hides the latency, and the short
        // ring keeps more wavefronts resident), 2 above that (measured on
        // Q4_0 / Q4_K / Q5_K at 17408-34816 x 5120, 1 and 2 vectors: up to
        // 22% faster than 4 in flight, at most 2% slower)
        const int64_t waves = (N + (int64_t)WGW * (64 / p.LPR) - 1) / ((int64_t)WGW * (64 / p.LPR)) * WGW;
        if (waves <= 12 * (int64_t)gqk_cu_count()) return launch_d<TYPE, XT, BMAX, WGW, 1, true>(p, W, N, K, xs, nb, y, s);
        return launch_d<TYPE, XT, BMAX, WGW, 2, true>(p, W, N, K, xs, nb, y, s);
    }
    switch (p.D) {
    case 1: return launch_d<TYPE, XT, BMAX, WGW, 1>(p, W, N, K, xs, nb, y, s);
    case 2: return launch_d<TYPE, XT, BMAX, WGW, 2>(p, W, N, K, xs, nb, y, s);
    case 3: return launch_d<TYPE, XT, BMAX, WGW, 3>(p, W, N, K, xs, nb, y, s);
    case 4: return launch_d<TYPE, XT, BMAX, WGW, 4>(p, W, N, K, xs, nb, y, s);
    case 5: return launch_d<TYPE, XT, BMAX, WGW, 5>(p, W, N, K, xs, nb, y, s);
    case 6: return launch_d<TYPE, XT, BMAX, WGW, 6>(p, W, N, K, xs, nb, y, s);
    default: return hipErrorInvalidValue;
    }
}

template <int TYPE, int XT, int BMAX>
hipError_t launch_b(const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y, hipStream_t s) {
    using F = Fmt<TYPE>;
    const Plan p = plan_for<F>(N, K, nb);
    if (p.grid > 0x7fffffff) return hipErrorInvalidValue;
    {
        const int64_t rows8 = 8 * (int64_t)(64 / p.LPR);
        const int64_t g8 = (N + rows8 - 1) / rows8;
        if (g8 >= 150 && g8 <= 256) return launch_w<TYPE, XT, BMAX, 8>(p, W, N, K, xs, nb, y, s);
    }
    return launch_w<TYPE, XT, BMAX, 4>(p, W, N, K, xs, nb, y, s);
}

template <int TYPE, int XT>
hipError_t launch_t(const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y, hipStream_t s) {
    // (3..8 vectors share one variant: a 4-vector one needs no fewer registers)
    if (nb == 1) return launch_b<TYPE, XT, 1>(W, N, K, xs, nb, y, s);
    if (nb == 2) return launch_b<TYPE, XT, 2>(W, N, K, xs, nb, y, s);
    return launch_b<TYPE, XT, 8>(W, N, K, xs, nb, y, s);
}

template <int TYPE>
hipError_t launch_x(const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int x_dtype, int nb, float* y,
                    hipStream_t s) {
    if (x_dtype == DT_F32) return launch_t<TYPE, 0>(W, N, K, xs, nb, y, s);
    return launch_t<TYPE, 1>(W, N, K, xs, nb, y, s);
}

// ------------------------------------------------ gated-unit epilogue ----
// h[b][n] = act(gate[b][n]) * up[b][n] with gate = W_gate x_b, up = W_up x_b:
// the two products of a gated feed-forward block and the elementwise step
// between them in one launch.  Wavefronts 0, 1 of a workgroup compute rows
// [n0, n0 + 2 SR) of the gate matrix, wavefronts 2, 3 the same rows of the up
// matrix (each pair through its own buffer resource), all four staging the
// activations together; the two partial tiles meet in LDS, where wavefronts
// 0, 1 apply the activation and store h.

template <int TYPE, int XT, int BMAX, int D, bool RING>
__global__ __launch_bounds__(NTHREADS) void k_glu(const uint8_t* __restrict__ Wg, const uint8_t* __restrict__ Wu,
                                                  int64_t N, int64_t K, XSrc xs, int nb, int act, void* __restrict__ h,
                                                  int h_bf16, int LPR, int tile_units) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float part[2][BMAX][16];  // [gate | up][vector][row in tile]; 2 SR <= 16 rows (LPR >= 8)
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), half = wave >> 1;
    const int SR = 64 / LPR, rows = 2 * SR;
    const int64_t n0 = (int64_t)blockIdx.x * rows;
    const int64_t row_bytes = (K / Fmt<TYPE>::QK) * Fmt<TYPE>::BB;
    YDst yd;
#pragma unroll
    for (int b = 0; b < 8; ++b) yd.p[b] = &part[half][b < BMAX ? b : 0][0];
    gemv_workgroup<TYPE, XT, BMAX, D, RING>((half ? Wu : Wg) + n0 * row_bytes, N - n0, K, 0, xs, nb, yd, LPR,
                                            tile_units, lds, wave & 1, 2);
    __syncthreads();
    const int64_t nr = N - n0 < rows ? N - n0 : rows;
    for (int i = (int)threadIdx.x; i < nb * rows; i += NTHREADS) {
        const int b = i / rows, r = i - b * rows;
        if (r >= nr) continue;
        const float v = act_fn(act, part[0][b][r]) * part[1][b][r];
        const int64_t o = (int64_t)b * N + n0 + r;
        if (h_bf16) static_cast<uint16_t*>(h)[o] = f2bf(v);
        else static_cast<float*>(h)[o] = v;
    }
}

template <int TYPE, int XT, int BMAX, int D, bool RING = false>
hipError_t launch_glu_d(const Plan& p, const uint8_t* Wg, const uint8_t* Wu, int64_t N, int64_t K, const XSrc& xs,
                        int nb, int act, void* h, int h_bf16, hipStream_t s) {
    const int64_t grid = (N + 2 * (64 / p.LPR) - 1) / (2 * (64 / p.LPR));
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_glu<TYPE, XT, BMAX, D, RING>), dim3((unsigned)grid), dim3(NTHREADS), p.lds, s, Wg, Wu, N,
                       K, xs, nb, act, h, h_bf16, p.LPR, p.tile_units);
    return hipGetLastError();
}

template <int TYPE, int XT, int BMAX>
hipError_t launch_glu_b(const uint8_t* Wg, const uint8_t* Wu, int64_t N, int64_t K, const XSrc& xs, int nb, int act,
                        void* h, int h_bf16, hipStream_t s) {
    using F = Fmt<TYPE>;
    // lanes per row chosen for the 2N rows of the launch
    const Plan p = plan_for<F>(N, K, nb, 2 * N);
    // two units per lane in flight (measured against 1 and 4: bf16 17408 x
    // 5120 8% faster than with 4, the fp32 hidden-2560 shapes equal)
    if (p.ring) return launch_glu_d<TYPE, XT, BMAX, 2, true>(p, Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    switch (p.D) {
    case 1: return launch_glu_d<TYPE, XT, BMAX, 1>(p, Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    case 2: return launch_glu_d<TYPE, XT, BMAX, 2>(p, Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    case 3: return launch_glu_d<TYPE, XT, BMAX, 3>(p, Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    case 4: return launch_glu_d<TYPE, XT, BMAX, 4>(p, Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    case 5: return launch_glu_d<TYPE, XT, BMAX, 5>(p, Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    case 6: return launch_glu_d<TYPE, XT, BMAX, 6>(p, Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    default: return hipErrorInvalidValue;
    }
}

template <int TYPE, int XT>
hipError_t launch_glu_t(const uint8_t* Wg, const uint8_t* Wu, int64_t N, int64_t K, const XSrc& xs, int nb, int act,
                        void* h, int h_bf16, hipStream_t s) {
    if (nb == 1) return launch_glu_b<TYPE, XT, 1>(Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    if (nb == 2) return launch_glu_b<TYPE, XT, 2>(Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    return launch_glu_b<TYPE, XT, 8>(Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
}

template <int TYPE>
hipError_t launch_glu_x(const uint8_t* Wg, const uint8_t* Wu, int64_t N, int64_t K, const XSrc& xs, int x_dtype,
                        int nb, int act, void* h, int h_bf16, hipStream_t s) {
    if (x_dtype == DT_F32) return launch_glu_t<TYPE, 0>(Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
    return launch_glu_t<TYPE, 1>(Wg, Wu, N, K, xs, nb, act, h, h_bf16, s);
}

}  // namespace

hipError_t gqk_matvec_glu(int type, const void* Wg, const void* Wu, int64_t N, int64_t K, const void* x, int x_dtype,
                          int batch, int act, void* h, int h_dtype, hipStream_t s) {
    if (N == 0) return hipSuccess;
    XSrc xs;
    const int esz = x_dtype == DT_F32 ? 4 : 2;
    for (int b = 0; b < 8; ++b)
        xs.p[b] = static_cast<const uint8_t*>(x) + (int64_t)(b < batch ? b : 0) * K * esz;
    const uint8_t* g = static_cast<const uint8_t*>(Wg);
    const uint8_t* u = static_cast<const uint8_t*>(Wu);
    const int hb = h_dtype == DT_BF16 ? 1 : 0;
    if (type == T_Q4_0) return launch_glu_x<T_Q4_0>(g, u, N, K, xs, x_dtype, batch, act, h, hb, s);
    if (type == T_Q4_K) return launch_glu_x<T_Q4_K>(g, u, N, K, xs, x_dtype, batch, act, h, hb, s);
    if (type == T_Q5_K) return launch_glu_x<T_Q5_K>(g, u, N, K, xs, x_dtype, batch, act, h, hb, s);
    return launch_glu_x<T_Q6_K>(g, u, N, K, xs, x_dtype, batch, act, h, hb, s);
}

hipError_t gqk_matvec(int type, const void* W, int64_t N, int64_t K, const void* x, int x_dtype, int batch,
                      float* y, hipStream_t s) {
    if (N == 0) return hipSuccess;
    XSrc xs;
    const int esz = x_dtype == DT_F32 ? 4 : 2;
    for (int b = 0; b < 8; ++b)
        xs.p[b] = static_cast<const uint8_t*>(x) + (int64_t)(b < batch ? b : 0) * K * esz;
    const uint8_t* w = static_cast<const uint8_t*>(W);
    if (type == T_Q4_0) return launch_x<T_Q4_0>(w, N, K, xs, x_dtype, batch, y, s);
    if (type == T_Q4_K) return launch_x<T_Q4_K>(w, N, K, xs, x_dtype, batch, y, s);
    if (type == T_Q5_K) return launch_x<T_Q5_K>(w, N, K, xs, x_dtype, batch, y, s);
    return launch_x<T_Q6_K>(w, N, K, xs, x_dtype, batch, y, s);
}
