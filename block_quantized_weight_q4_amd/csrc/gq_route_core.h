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

// One step of the wave maximum: each lane takes the larger of its key and
// the key that the DPP pattern CTRL brings from another lane (rows outside
// ROWS, and lanes whose source lies outside their row, keep their own).
template <int CTRL, int ROWS>
__device__ __forceinline__ void max_step(uint32_t& hi, uint32_t& lo) {
    const uint32_t th = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROWS, 0xF, false);
    const uint32_t tl = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROWS, 0xF, false);
    const bool gt = th > hi || (th == hi && tl > lo);
    hi = gt ? th : hi;
    lo = gt ? tl : lo;
}

// Largest 64-bit key of the wave, in every lane.  Cross-lane moves by DPP
// instead of LDS permutes: row shifts right by 1, 2, 4, 8 leave each 16-lane
// row's maximum in its lane 15; row_bcast15 and row_bcast31 carry those into
// lane 63, which is then read as a scalar.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
    max_step<0x111, 0xF>(hi, lo);  // row_shr:1
    max_step<0x112, 0xF>(hi, lo);  // row_shr:2
    max_step<0x114, 0xF>(hi, lo);  // row_shr:4
    max_step<0x118, 0xF>(hi, lo);  // row_shr:8
    max_step<0x142, 0xA>(hi, lo);  // row_bcast15 into rows 1 and 3
    max_step<0x143, 0xC>(hi, lo);  // row_bcast31 into rows 2 and 3
    const uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
    const uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
    return ((uint64_t)h << 32) | l;
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
    // (each load is unconditional, from a clamped index, and masked
    // afterwards: as a conditional load each would wait for the one before)
    uint64_t key[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int e = lane + 64 * i;
        const float v = l[e < n_experts ? e : n_experts - 1];
        const uint64_t keep = 0ull - (uint64_t)(e < n_experts);
        key[i] = (((uint64_t)order_key(v) << 32) | (uint32_t)~(uint32_t)e) & keep;
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
