// gq_route.hip -- per-token expert routing: top-k selection over the router
// logits and a softmax over the selected ones, in one launch.
//
// The operation is the "topk" row of the kernel table in "GGUF in
// transformers" (section "Reusing ggml's Metal kernels"), which combines the
// softmax with the top-k choice of experts; the Show HN page on Gemma 4
// 26B-A4B (section "How it works") routes each token to 8 of 128 experts this
// way before the routed 4-bit expert products.
//
// The per-token step (top-k by order-preserving keys, softmax over the
// selection) is in gq_route_core.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gq_internal.h"
#include "gq_route_core.h"

namespace {

constexpr int WAVES = 4;  // tokens per workgroup

template <int NI>
__global__ __launch_bounds__(64 * WAVES) void k_route(const float* __restrict__ logits, int n_tokens, int n_experts,
                                                      int top_k, int32_t* __restrict__ ids,
                                                      float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (t >= n_tokens) return;  // t is the same for the whole wave
    int id;
    float w;
    gqr::route_token<NI>(logits + (int64_t)t * n_experts, n_experts, top_k, lane, id, w);
    if (lane < top_k) {
        ids[(int64_t)t * top_k + lane] = id;
        weights[(int64_t)t * top_k + lane] = w;
    }
}

template <int NI>
hipError_t launch(const float* logits, int n_tokens, int n_experts, int top_k, int32_t* ids, float* w,
                  hipStream_t s) {
    const unsigned grid = (unsigned)((n_tokens + WAVES - 1) / WAVES);
    hipLaunchKernelGGL(k_route<NI>, dim3(grid), dim3(64 * WAVES), 0, s, logits, n_tokens, n_experts, top_k, ids, w);
    return hipGetLastError();
}

}  // namespace

hipError_t gqk_route_topk(const float* logits, int n_tokens, int n_experts, int top_k, int32_t* ids, float* w,
                          hipStream_t s) {
    const int ni = (n_experts + 63) / 64;
    if (ni <= 1) return launch<1>(logits, n_tokens, n_experts, top_k, ids, w, s);
    if (ni <= 2) return launch<2>(logits, n_tokens, n_experts, top_k, ids, w, s);
    if (ni <= 4) return launch<4>(logits, n_tokens, n_experts, top_k, ids, w, s);
    if (ni <= 8) return launch<8>(logits, n_tokens, n_experts, top_k, ids, w, s);
    if (ni <= 16) return launch<16>(logits, n_tokens, n_experts, top_k, ids, w, s);
    if (ni <= 32) return launch<32>(logits, n_tokens, n_experts, top_k, ids, w, s);
    return launch<64>(logits, n_tokens, n_experts, top_k, ids, w, s);
}
