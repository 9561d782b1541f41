// gq_matvec_id.hip -- routed-expert product (gfx950): only the experts the
// router chose are read, each once for all the (token, slot) pairs sent to it
// (the ggml-quantization row of the kernel table in "GGUF in transformers";
// the routed 4-bit experts of the Architecture section of "Show HN: Gemma 4
// 26B-A4B at up to 100+ tokens/s on a 16 GB Mac").
//
// Three launches on the caller's stream, no host synchronisation:
//  1. k_group (one workgroup): rank-sorts the slots s = t*top_k + j by
//     (expert id, s) on the device and cuts each expert's run of slots into
//     groups of at most CH; ids outside [0, n_experts) are counted and left out.
//  2. k_experts: one workgroup per (group, row tile) runs the shared decode
//     product on that expert's rows with the group's activation vectors
//     (gathered by slot), writing one output row per slot.  Workgroups whose
//     group index is past the number of groups exit at once (the grid is sized
//     for the worst case, because the host never reads the ids).
//  3. k_combine (route_w given): y[t][n] = sum_j route_w[t][j] * slot[t][j][n],
//     j in increasing order; or k_zero_bad (no route_w): zero the output rows of
//     out-of-range slots.
#include "gq_gemv_core.h"
#include "gq_internal.h"

using namespace gqd;

namespace {

constexpr int CH = 4;           // slots per group = vectors per product workgroup
constexpr int MAX_SLOTS = 1024; // n_tokens * top_k handled by k_group

struct WsLayout {
    int S, Gmax;
    size_t off_groups, off_sorted, off_out, total;
};

WsLayout layout(int n_experts, int n_tokens, int top_k, int64_t N) {
    WsLayout L;
    L.S = n_tokens * top_k;
    int distinct = L.S < n_experts ? L.S : n_experts;
    L.Gmax = distinct + L.S / CH + 1;
    L.off_groups = 16;
    L.off_sorted = (L.off_groups + 16 * (size_t)L.Gmax + 15) & ~size_t(15);
    L.off_out = (L.off_sorted + 4 * (size_t)L.S + 255) & ~size_t(255);
    L.total = L.off_out + 4 * (size_t)L.S * (size_t)N;
    return L;
}

struct Group {
    int expert, start, count, pad;
};

// ---------------------------------------------------------------- group ----
__global__ __launch_bounds__(256) void k_group(const int32_t* __restrict__ ids, int S, int n_experts,
                                               uint8_t* __restrict__ ws, int off_groups, int off_sorted) {
    __shared__ int key[MAX_SLOTS];      // expert id, or INT_MAX for an invalid id
    __shared__ int head[MAX_SLOTS];     // 1 where a group starts (by sorted position)
    __shared__ int head_e[MAX_SLOTS];   // expert of the slot at that sorted position
    __shared__ int head_cnt[MAX_SLOTS]; // group size if it starts there
    __shared__ int part[256];
    __shared__ int bad_total;
    const int tid = threadIdx.x;
    int* sorted = reinterpret_cast<int*>(ws + off_sorted);
    Group* groups = reinterpret_cast<Group*>(ws + off_groups);
    if (tid == 0) bad_total = 0;
    __syncthreads();
    int bad = 0;
    for (int i = tid; i < S; i += 256) {
        int e = ids[i];
        bool ok = e >= 0 && e < n_experts;
        key[i] = ok ? e : 0x7fffffff;
        bad += ok ? 0 : 1;
        head[i] = 0;
    }
    if (bad) atomicAdd(&bad_total, bad);
    __syncthreads();
    // rank of slot i in (expert, slot) order; first = rank of the expert's
    // first slot; cnt = slots routed to the same expert
    for (int i = tid; i < S; i += 256) {
        int ki = key[i];
        int less = 0, same_before = 0, same = 0;
        for (int j = 0; j < S; ++j) {
            int kj = key[j];
            less += kj < ki;
            same += kj == ki;
            same_before += (kj == ki) & (j < i);
        }
        int pos = less + same_before;
        sorted[pos] = i;
        if (ki != 0x7fffffff && same_before % CH == 0) {
            head[pos] = 1;
            head_e[pos] = ki;
            int left = same - same_before;
            head_cnt[pos] = left < CH ? left : CH;
        }
    }
    __syncthreads();
    // exclusive scan of the head flags over sorted positions: group numbers
    const int per = (S + 255) / 256;
    int lo = tid * per, hi = lo + per < S ? lo + per : S;
    int c = 0;
    for (int p = lo; p < hi; ++p) c += head[p];
    part[tid] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int g = part[tid] - c;
    for (int p = lo; p < hi; ++p) {
        if (head[p]) {
            groups[g] = Group{head_e[p], p, head_cnt[p], 0};
            ++g;
        }
    }
    if (tid == 255) {
        int* hdr = reinterpret_cast<int*>(ws);
        hdr[0] = bad_total;
        hdr[1] = part[255];
    }
}

// ------------------------------------------------------------- product ----
template <int TYPE, int XT, int D, bool RING>
__global__ __launch_bounds__(NTHREADS) void k_experts(const uint8_t* __restrict__ experts, int64_t expert_bytes,
                                                      int64_t N, int64_t K, const uint8_t* __restrict__ x,
                                                      int x_per_slot, int top_k, const uint8_t* __restrict__ ws,
                                                      int off_groups, int off_sorted, float* __restrict__ out,
                                                      int LPR, int tile_units) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int* hdr = reinterpret_cast<const int*>(ws);
    const int gi = blockIdx.x;
    if (gi >= hdr[1]) return;
    const Group grp = reinterpret_cast<const Group*>(ws + off_groups)[gi];
    const int* sorted = reinterpret_cast<const int*>(ws + off_sorted);
    const int esz = XT == 0 ? 4 : 2;
    XSrc xs;
    YDst yd;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        int slot = sorted[grp.start + (b < grp.count ? b : 0)];
        int64_t xrow = x_per_slot ? slot : slot / top_k;
        xs.p[b] = x + xrow * K * esz;
        yd.p[b] = out + (int64_t)slot * N;
    }
    const int64_t rpw = (int64_t)(NTHREADS >> 6) * (64 / LPR);
    gemv_workgroup<TYPE, XT, CH, D, RING>(experts + (int64_t)grp.expert * expert_bytes, N, K,
                                       (int64_t)blockIdx.y * rpw, xs, grp.count, yd, LPR, tile_units, lds);
}

// ------------------------------------------------------------- combine ----
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ slot_out, const int32_t* __restrict__ ids,
                                                 const float* __restrict__ route_w, int n_experts, int top_k,
                                                 int64_t N, float* __restrict__ y) {
    const int t = blockIdx.y;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float acc = 0.f;
    for (int j = 0; j < top_k; ++j) {
        int e = ids[t * top_k + j];
        if (e < 0 || e >= n_experts) continue;
        acc = __builtin_fmaf(route_w[t * top_k + j], slot_out[((int64_t)t * top_k + j) * N + n], acc);
    }
    y[(int64_t)t * N + n] = acc;
}

__global__ __launch_bounds__(256) void k_zero_bad(const int32_t* __restrict__ ids, int n_experts, int64_t N,
                                                  float* __restrict__ y) {
    const int s = blockIdx.y;
    const int e = ids[s];
    if (e >= 0 && e < n_experts) return;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n < N) y[(int64_t)s * N + n] = 0.f;
}

template <int TYPE, int XT, int D, bool RING = false>
hipError_t launch_experts_d(const Plan& p, const WsLayout& L, const uint8_t* experts, int64_t N, int64_t K,
                            const uint8_t* x, int x_per_slot, int top_k, const uint8_t* ws, float* out,
                            hipStream_t s) {
    using F = Fmt<TYPE>;
    const int64_t expert_bytes = N * (K / F::QK) * F::BB;
    hipLaunchKernelGGL((k_experts<TYPE, XT, D, RING>), dim3((unsigned)L.Gmax, (unsigned)p.grid), dim3(NTHREADS),
                       p.lds, s, experts, expert_bytes, N, K, x, x_per_slot, top_k, ws, (int)L.off_groups,
                       (int)L.off_sorted, out, p.LPR, p.tile_units);
    return hipGetLastError();
}

template <int TYPE, int XT>
hipError_t launch_experts(const WsLayout& L, const uint8_t* experts, int64_t N, int64_t K, const uint8_t* x,
                          int x_per_slot, int top_k, const uint8_t* ws, float* out, hipStream_t s) {
    using F = Fmt<TYPE>;
    const Plan p = plan_for<F>(N, K, CH);
    if (p.grid > 65535) return hipErrorInvalidValue;
    if (p.ring) return launch_experts_d<TYPE, XT, D_RING, true>(p, L, experts, N, K, x, x_per_slot, top_k, ws, out, s);
    switch (p.D) {
    case 1: return launch_experts_d<TYPE, XT, 1>(p, L, experts, N, K, x, x_per_slot, top_k, ws, out, s);
    case 2: return launch_experts_d<TYPE, XT, 2>(p, L, experts, N, K, x, x_per_slot, top_k, ws, out, s);
    case 3: return launch_experts_d<TYPE, XT, 3>(p, L, experts, N, K, x, x_per_slot, top_k, ws, out, s);
    case 4: return launch_experts_d<TYPE, XT, 4>(p, L, experts, N, K, x, x_per_slot, top_k, ws, out, s);
    case 5: return launch_experts_d<TYPE, XT, 5>(p, L, experts, N, K, x, x_per_slot, top_k, ws, out, s);
    case 6: return launch_experts_d<TYPE, XT, 6>(p, L, experts, N, K, x, x_per_slot, top_k, ws, out, s);
    default: return hipErrorInvalidValue;
    }
}

template <int TYPE>
hipError_t launch_experts_x(const WsLayout& L, const uint8_t* experts, int64_t N, int64_t K, const void* x,
                            int x_dtype, int x_per_slot, int top_k, const uint8_t* ws, float* out, hipStream_t s) {
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    if (x_dtype == DT_F32) return launch_experts<TYPE, 0>(L, experts, N, K, xb, x_per_slot, top_k, ws, out, s);
    return launch_experts<TYPE, 1>(L, experts, N, K, xb, x_per_slot, top_k, ws, out, s);
}

}  // namespace

size_t gqk_matvec_id_ws_bytes(int n_experts, int n_tokens, int top_k, int64_t N) {
    return layout(n_experts, n_tokens, top_k, N).total;
}

hipError_t gqk_matvec_id(int type, const void* experts, int n_experts, int64_t N, int64_t K, const int32_t* ids,
                         int n_tokens, int top_k, const void* x, int x_dtype, int x_per_slot, const float* route_w,
                         float* y, void* ws, hipStream_t s) {
    WsLayout L = layout(n_experts, n_tokens, top_k, N);
    if (L.S > MAX_SLOTS) return hipErrorInvalidValue;
    uint8_t* w = static_cast<uint8_t*>(ws);
    hipLaunchKernelGGL(k_group, dim3(1), dim3(256), 0, s, ids, L.S, n_experts, w, (int)L.off_groups,
                       (int)L.off_sorted);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // per-slot outputs: straight into y when there is no routing combine
    float* out = route_w ? reinterpret_cast<float*>(w + L.off_out) : y;
    const uint8_t* ex = static_cast<const uint8_t*>(experts);
    if (type == T_Q4_0) e = launch_experts_x<T_Q4_0>(L, ex, N, K, x, x_dtype, x_per_slot, top_k, w, out, s);
    else if (type == T_Q4_K) e = launch_experts_x<T_Q4_K>(L, ex, N, K, x, x_dtype, x_per_slot, top_k, w, out, s);
    else e = launch_experts_x<T_Q6_K>(L, ex, N, K, x, x_dtype, x_per_slot, top_k, w, out, s);
    if (e != hipSuccess) return e;
    const unsigned nx = (unsigned)((N + 255) / 256);
    if (route_w) {
        hipLaunchKernelGGL(k_combine, dim3(nx, (unsigned)n_tokens), dim3(256), 0, s, out, ids, route_w, n_experts,
                           top_k, N, y);
    } else {
        hipLaunchKernelGGL(k_zero_bad, dim3(nx, (unsigned)L.S), dim3(256), 0, s, ids, n_experts, N, y);
    }
    return hipGetLastError();
}

hipError_t gqk_matvec_id_bad_count(const void* ws, hipStream_t s, int32_t* n_bad) {
    hipError_t e = hipMemcpyAsync(n_bad, ws, sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);
}
