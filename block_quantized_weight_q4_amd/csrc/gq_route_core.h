// gq_route_core.h -- the per-token top-k + softmax step shared by the router
// kernels (gfx950, wave64).
//
// One wave per token.  Lane l holds the logits of experts l, l + 64, ...
// (NI of them, coalesced loads) as 64-bit keys: an order-preserving integer
// image of the fp32 logit in the high half and the complement of the expert
// id in the low half, so the largest key is the largest logit and, among
// equal logits, the lowest id.  Each of the top_k rounds takes the lane-local
// largest key, reduces it over the wave with xor shuffles, and clears the
// winner in its owner lane; lane j keeps the j-th winner.  The softmax then
// runs across lanes 0..top_k-1 in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqr {

// fp32 logit -> 32-bit key with the same order (IEEE total order on non-NaN
// values); -0 is taken as +0 so that the two compare equal, as they do in fp32.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __builtin_bit_cast(uint32_t, v);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Route one token (the whole wave takes part): lane j < top_k gets the j-th
// chosen expert and its softmax weight.
template <int NI>
__device__ __forceinline__ void route_token(const float* __restrict__ l, int n_experts, int top_k, int lane,
                                            int& id, float& weight) {
    // key 0 marks an empty or already chosen position: every real key is
    // larger, since its low half (the complemented id) is never zero.
    uint64_t key[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < n_experts ? ((uint64_t)order_key(l[e]) << 32) | (uint32_t)~(uint32_t)e : 0ull;
    }
    int my_id = 0;
    float my_logit = 0.f;
    for (int j = 0; j < top_k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NI; ++i) best = key[i] > best ? key[i] : best;
        const uint64_t win = wave_max_u64(best);
        const int e = (int)~(uint32_t)win;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (e == lane + 64 * i) key[i] = 0ull;
        if (lane == j) {
            my_id = e;
            my_logit = key_value((uint32_t)(win >> 32));
        }
    }
    // softmax over the selected logits, shifted by the largest (lane 0's)
    const float l0 = __shfl(my_logit, 0, 64);
    const float ex = lane < top_k ? expf(my_logit - l0) : 0.f;
    const float sum = wave_sum(ex);
    id = my_id;
    weight = ex / sum;
}

}  // namespace gqr
