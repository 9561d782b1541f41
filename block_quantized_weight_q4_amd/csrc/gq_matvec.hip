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
                                                     XSrc xs, int nb, float* __restrict__ y, int LPR,
                                                     int tile_units) {
    using F = Fmt<TYPE>;
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
    const int SR = 64 / LPR;
    const int s = lane / LPR, v = lane - s * LPR;
    const int64_t row_bytes = (K / F::QK) * F::BB;
    const int64_t rpw = (int64_t)waves * R * SR;
    const int64_t row0 = (int64_t)blockIdx.x * rpw + (int64_t)wave * R * SR + s;

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
                    if (b < nb) y[(int64_t)b * N + r] = acc[i][b];
            }
        }
    }
}

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
int lanes_per_row(int64_t units) {
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
Plan plan_for(int64_t N, int64_t K, int nb) {
    Plan p;
    int64_t units = K / F::UW;
    p.LPR = lanes_per_row<F>(units);
    const int SR = 64 / p.LPR;
    // K tile: as many units as the LDS budget allows for nb vectors, rounded
    // down to a multiple of LPR (a multiple of 4 units = whole super-blocks)
    size_t per_unit = (size_t)16 * (F::NQ + F::NF) * nb;
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

template <int TYPE, int XT, int BMAX, int R>
hipError_t launch_r(const Plan& p, const uint8_t* W, int64_t N, int64_t K, const XSrc& xs, int nb, float* y,
                    hipStream_t s) {
    constexpr int D = 4 / R;
    hipLaunchKernelGGL((k_matvec<TYPE, XT, BMAX, R, D>), dim3((unsigned)p.grid), dim3(64 * p.WPW), p.lds, s, W, N, K, xs,
                       nb, y, p.LPR, p.tile_units);
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
