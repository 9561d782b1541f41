// gq_matvec.hip -- decode product y[b][n] = sum_k w[n][k] x[b][k] against
// packed Q4_0 / Q4_K / Q6_K rows (gfx950).  The per-lane work is in
// gq_gemv_core.h; this file maps workgroups to row tiles and K tiles.
//
// Grid: one workgroup (1, 2 or 4 wavefronts) per tile of WPW * R * (64 / LPR)
// consecutive rows.
// The activations are staged tile by tile along K (each tile fits the LDS
// budget; usually all of K is one tile), and the lane partial sums stay in
// registers across K tiles, so every packed byte is read exactly once.
#include "gq_gemv_core.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

template <int TYPE, int XT, int BMAX, int R, int D>
__global__ __launch_bounds__(NTHREADS) void k_matvec(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                     XSrc xs, int nb, YDst yd, int LPR, int tile_units) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int SR = 64 / LPR;
    const int64_t rpw = (int64_t)(blockDim.x >> 6) * R * SR;
    gemv_workgroup<TYPE, XT, BMAX, R, D>(W, N, K, (int64_t)blockIdx.x * rpw, xs, nb, yd, LPR, tile_units, lds);
}

template <int TYPE, int XT, int BMAX, int R>
hipError_t launch_r(const Plan& p, const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y,
                    hipStream_t s) {
    constexpr int D = 4 / R;
    YDst yd;
    for (int b = 0; b < 8; ++b) yd.p[b] = y + (int64_t)(b < nb ? b : 0) * N;
    hipLaunchKernelGGL((k_matvec<TYPE, XT, BMAX, R, D>), dim3((unsigned)p.grid), dim3(64 * p.WPW), p.lds, s, W, N, K, xs,
                       nb, yd, p.LPR, p.tile_units);
    return hipGetLastError();
}

template <int TYPE, int XT, int BMAX>
hipError_t launch_b(const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y, hipStream_t s) {
    using F = Fmt<TYPE>;
    Plan p = plan_for<F>(N, K, nb);
    if (p.grid > 0x7fffffff) return hipErrorInvalidValue;
    return launch_r<TYPE, XT, BMAX, 1>(p, W, N, K, xs, nb, y, s);
}

template <int TYPE, int XT>
hipError_t launch_t(const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y, hipStream_t s) {
    if (nb == 1) return launch_b<TYPE, XT, 1>(W, N, K, xs, nb, y, s);
    if (nb == 2) return launch_b<TYPE, XT, 2>(W, N, K, xs, nb, y, s);
    if (nb <= 4) return launch_b<TYPE, XT, 4>(W, N, K, xs, nb, y, s);
    return launch_b<TYPE, XT, 8>(W, N, K, xs, nb, y, s);
}

template <int TYPE>
hipError_t launch_x(const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int x_dtype, int nb, float* y,
                    hipStream_t s) {
    if (x_dtype == DT_F32) return launch_t<TYPE, 0>(W, N, K, xs, nb, y, s);
    return launch_t<TYPE, 1>(W, N, K, xs, nb, y, s);
}

}  // namespace

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
    return launch_x<T_Q6_K>(w, N, K, xs, x_dtype, batch, y, s);
}
