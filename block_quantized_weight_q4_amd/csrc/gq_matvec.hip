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

template <int TYPE, int XT, int BMAX, int D, bool RING>
__global__ __launch_bounds__(NTHREADS) void k_matvec(const uint8_t* __restrict__ W, int64_t N, int64_t K,
                                                     XSrc xs, int nb, YDst yd, int LPR, int tile_units) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int64_t rpw = (int64_t)(NTHREADS >> 6) * (64 / LPR);
    gemv_workgroup<TYPE, XT, BMAX, D, RING>(W, N, K, (int64_t)blockIdx.x * rpw, xs, nb, yd, LPR, tile_units, lds);
}

template <int TYPE, int XT, int BMAX, int D, bool RING = false>
hipError_t launch_d(const Plan& p, const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y,
                    hipStream_t s) {
    YDst yd;
    for (int b = 0; b < 8; ++b) yd.p[b] = y + (int64_t)(b < nb ? b : 0) * N;
    hipLaunchKernelGGL((k_matvec<TYPE, XT, BMAX, D, RING>), dim3((unsigned)p.grid), dim3(NTHREADS), p.lds, s, W, N, K,
                       xs, nb, yd, p.LPR, p.tile_units);
    return hipGetLastError();
}

template <int TYPE, int XT, int BMAX>
hipError_t launch_b(const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y, hipStream_t s) {
    using F = Fmt<TYPE>;
    const Plan p = plan_for<F>(N, K, nb);
    if (p.grid > 0x7fffffff) return hipErrorInvalidValue;
    if (p.ring) return launch_d<TYPE, XT, BMAX, D_RING, true>(p, W, N, K, xs, nb, y, s);
    switch (p.D) {
    case 1: return launch_d<TYPE, XT, BMAX, 1>(p, W, N, K, xs, nb, y, s);
    case 2: return launch_d<TYPE, XT, BMAX, 2>(p, W, N, K, xs, nb, y, s);
    case 3: return launch_d<TYPE, XT, BMAX, 3>(p, W, N, K, xs, nb, y, s);
    case 4: return launch_d<TYPE, XT, BMAX, 4>(p, W, N, K, xs, nb, y, s);
    case 5: return launch_d<TYPE, XT, BMAX, 5>(p, W, N, K, xs, nb, y, s);
    case 6: return launch_d<TYPE, XT, BMAX, 6>(p, W, N, K, xs, nb, y, s);
    default: return hipErrorInvalidValue;
    }
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
    if (type == T_Q5_K) return launch_x<T_Q5_K>(w, N, K, xs, x_dtype, batch, y, s);
    return launch_x<T_Q6_K>(w, N, K, xs, x_dtype, batch, y, s);
}
