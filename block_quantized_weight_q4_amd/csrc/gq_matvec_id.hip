// gq_matvec_id.hip -- routed-expert product (gfx950): only the experts the
// router chose are read, each once for all the (token, slot) pairs sent to it
// (the ggml-quantization row of the kernel table in "GGUF in transformers";
// the routed 4-bit experts of the Architecture section of "Show HN: Gemma 4
// 26B-A4B at up to 100+ tokens/s on a 16 GB Mac").
//
// Up to three launches on the caller's stream, no host synchronisation:
//  1. k_plan (one workgroup): the slots s = t*top_k + j are ordered by expert
//     id and each expert's slots are cut into groups of at most CH; the group
//     table (expert, slot count, slots) goes to the workspace, with the group
//     and invalid-id counts in its header and each slot's expert (-1 for an
//     invalid id).  Ids outside [0, n_experts) are left out, counted, and
//     their output rows zeroed.  A weighted product called without ids reuses
//     the table an earlier call left in the workspace (the gated unit and the
//     down projection of one layer route the same ids) and skips this launch.
//  2. k_experts: one workgroup per (group, row tile) reads its table entry
//     and runs the shared decode product on that expert's rows with the
//     group's activation vectors (gathered by slot), writing one output row
//     per slot.  Workgroups past the number of groups exit at once (the grid
//     is sized for the worst case, because the host never reads the ids).
//     The row tiles are the grid's x dimension and the groups its y, so the
//     workgroups are dispatched group by group, an expert's row tiles one
//     after another and the unused entries last (64 tokens x top 8:
//     A-B-B-A 0.961 against the transposed grid; 8 tokens: 0.995).
//     The K tile is chosen by each workgroup from its group's slot count, so a
//     group of one or two slots stages as many inputs at a time as the LDS
//     budget allows for that count.
//  3. k_combine (route_w given): y[t][n] = sum_j route_w[t][j] * slot[t][j][n],
//     j in increasing order.
// The gated unit of a routed feed-forward block (gate and up stacks, the
// activation between them) is the same k_experts launch in its GLU form: one
// launch writes h[t][j][n] = act(gate_e[n] . x_t) * (up_e[n] . x_t), e =
// ids[t][j], which the down projection then takes as its per-slot vectors.
#include <mutex>

#include "gq_gemv_core.h"
#include "gq_internal.h"
#include "gq_route_core.h"

using namespace gqd;

// Workspace of gq_matvec_id_noalloc: one per device, held until the process
// ends.  Host code never uses this name as an address (on the host it is only
// a stand-in for the symbol); the device address of each GPU's copy comes
// from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[GQK_NOALLOC_WS_BYTES];

namespace {

constexpr int CH = 8;           // slots per group = vectors per product workgroup
constexpr int MAX_SLOTS = 1024; // n_tokens * top_k

// One group of the table: expert e, nb <= CH slots in slot order.  Kernels
// read an entry through a pointer (a private copy indexed by a runtime slot
// number would live in scratch memory).
struct alignas(64) Entry {
    int e, nb, sel[CH];
};

// Workspace: header (int [0] = invalid ids, [1] = groups), each slot's expert
// (-1 for an invalid id), the group table, the per-slot outputs of a weighted
// product.  Everything before the outputs depends on n_experts and the slot
// count only, so calls with different N find the same table.
struct WsLayout {
    int S, Gmax;
    size_t off_slot, off_plan, off_out, total;
};

WsLayout layout(int n_experts, int n_tokens, int top_k, int64_t N) {
    WsLayout L;
    L.S = n_tokens * top_k;
    const int distinct = L.S < n_experts ? L.S : n_experts;
    L.Gmax = distinct + L.S / CH + 1;
    L.off_slot = 256;
    L.off_plan = L.off_slot + ((size_t)L.S * 4 + 255) / 256 * 256;
    L.off_out = L.off_plan + ((size_t)L.Gmax * sizeof(Entry) + 255) / 256 * 256;
    L.total = L.off_out + 4 * (size_t)L.S * (size_t)N;
    return L;
}

// ---------------------------------------------------------------- plan ----
// rank = position of a slot among the slots of its expert in slot order;
// slot s belongs to group first[e_s] + rank_s / CH, where first[e] counts the
// groups of the experts below e (an LDS histogram of the slots per expert and
// a scan of ceil(count / CH) over the experts; with more than
// MAX_EXPERTS_LDS experts, the group heads -- rank % CH == 0 -- with a smaller
// expert id, counted directly).  out (if given): the [S][N] outputs whose rows
// of invalid slots are zeroed (fp32, or bf16 when out_bf16).  The barriers
// order LDS traffic only: no thread reads what another wrote to global memory
// before the kernel ends, and a full barrier would wait for every store to be
// acknowledged (together about 3 of the router kernel's 8 us).
constexpr int MAX_EXPERTS_LDS = 1024;

template <int NT>
__device__ __forceinline__ void plan_body(const int32_t* ids, int S, int n_experts, int* __restrict__ hdr,
                                          int* __restrict__ slot_e, Entry* __restrict__ plan, void* __restrict__ out,
                                          int64_t N, int out_bf16) {
    __shared__ int4 key4[MAX_SLOTS / 4];
    __shared__ int4 head4[MAX_SLOTS / 4];  // expert id of a group head, INT_MAX otherwise
    __shared__ int rank[MAX_SLOTS];
    __shared__ int cnt[MAX_EXPERTS_LDS];   // slots per expert, then groups before it
    __shared__ int n_bad, n_grp;
    int* key = reinterpret_cast<int*>(key4);
    int* head = reinterpret_cast<int*>(head4);
    const int tid = threadIdx.x;
    const int S4 = (S + 3) >> 2;
    const bool small_e = n_experts <= MAX_EXPERTS_LDS;
    if (tid == 0) {
        n_bad = 0;
        n_grp = 0;
    }
    if (small_e)
        for (int e = tid; e < n_experts; e += NT) cnt[e] = 0;
    for (int s = tid; s < 4 * S4; s += NT) {
        const int e = s < S ? ids[s] : -2;
        key[s] = s >= S ? -2 : ((e >= 0 && e < n_experts) ? e : -1);  // -2: padding
        head[s] = 0x7fffffff;
    }
    lds_barrier();
    int bad = 0;
    for (int s = tid; s < S; s += NT) {
        const int e = key[s];
        slot_e[s] = e;
        int r = 0;
#pragma unroll 4
        for (int j4 = 0; 4 * j4 < s; ++j4) {
            const int4 k = key4[j4];
            const int j = 4 * j4;
            r += (k.x == e) + ((k.y == e) & (j + 1 < s)) + ((k.z == e) & (j + 2 < s)) + ((k.w == e) & (j + 3 < s));
        }
        rank[s] = r;
        if (e < 0) ++bad;
        else {
            if (small_e) atomicAdd(&cnt[e], 1);
            if (r % CH == 0) head[s] = e;
        }
    }
    if (bad) atomicAdd(&n_bad, bad);
    lds_barrier();
    if (small_e) {
        // exclusive scan of ceil(cnt / CH) over the experts by wavefront 0:
        // each lane a contiguous run of experts, then a shuffle scan of the
        // 64 run totals (no barrier inside)
        if (tid < 64) {
            const int per = (n_experts + 63) / 64;
            const int lo = tid * per, hi = lo + per < n_experts ? lo + per : n_experts;
            int sum = 0;
            for (int e = lo; e < hi; ++e) sum += (cnt[e] + CH - 1) / CH;
            int incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(incl, off, 64);
                if (tid >= off) incl += v;
            }
            int run = incl - sum;
            for (int e = lo; e < hi; ++e) {
                const int c = cnt[e];
                cnt[e] = run | (c << 16);  // groups before e (low half), slot count (high half)
                run += (c + CH - 1) / CH;
            }
            if (tid == 63) n_grp = incl;  // the group count: the scan's total
        }
        lds_barrier();
    }
    int heads = 0;
    for (int s = tid; s < S; s += NT) {
        const int e = key[s];
        if (e < 0) continue;
        int before, count;
        if (small_e) {
            before = cnt[e] & 0xffff;
            count = cnt[e] >> 16;
        } else {
            before = 0;
            count = 0;
            for (int j4 = 0; j4 < S4; ++j4) {
                const int4 h = head4[j4], k = key4[j4];
                before += (h.x < e) + (h.y < e) + (h.z < e) + (h.w < e);
                count += (k.x == e) + (k.y == e) + (k.z == e) + (k.w == e);
            }
        }
        const int r = rank[s];
        Entry& en = plan[before + r / CH];
        en.sel[r % CH] = s;
        if (r % CH == 0) {
            en.e = e;
            en.nb = count - r < CH ? count - r : CH;
            ++heads;
        }
    }
    // (an LDS atomic that every lane of a wavefront takes part in costs a
    // scalar loop over the lanes, about 2 us for 64: the scan counts the
    // groups when the experts fit in LDS)
    if (!small_e && heads) atomicAdd(&n_grp, heads);
    lds_barrier();
    if (tid == 0) {
        hdr[0] = n_bad;
        hdr[1] = n_grp;
    }
    if (out && n_bad)
        for (int s = 0; s < S; ++s)
            if (key[s] < 0)
                for (int64_t n = tid; n < N; n += NT) {
                    const int64_t o = (int64_t)s * N + n;
                    if (out_bf16) static_cast<uint16_t*>(out)[o] = 0;
                    else static_cast<float*>(out)[o] = 0.f;
                }
}

__global__ __launch_bounds__(NTHREADS) void k_plan(const int32_t* __restrict__ ids, int S, int n_experts,
                                                   int* __restrict__ hdr, int* __restrict__ slot_e,
                                                   Entry* __restrict__ plan, void* __restrict__ out, int64_t N,
                                                   int out_bf16) {
    plan_body<NTHREADS>(ids, S, n_experts, hdr, slot_e, plan, out, N, out_bf16);
}

// Routing and the table in one launch (one workgroup): wave w routes tokens
// w, w + RW, ... (the step of gq_route_topk), writing ids and weights and the
// ids into LDS; the table is then built from those.
constexpr int RW = 16;  // waves of the routing workgroup

template <int NI>
__global__ __launch_bounds__(64 * RW) void k_route_plan(const float* __restrict__ logits, int n_tokens, int n_experts,
                                                       int top_k, int32_t* __restrict__ ids,
                                                       float* __restrict__ weights, int* __restrict__ hdr,
                                                       int* __restrict__ slot_e, Entry* __restrict__ plan) {
    __shared__ int lids[MAX_SLOTS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int t = wave; t < n_tokens; t += RW) {
        int id;
        float w;
        gqr::route_token<NI>(logits + (int64_t)t * n_experts, n_experts, top_k, lane, id, w);
        if (lane < top_k) {
            ids[(int64_t)t * top_k + lane] = id;
            weights[(int64_t)t * top_k + lane] = w;
            lids[t * top_k + lane] = id;
        }
    }
    lds_barrier();
    plan_body<64 * RW>(lids, n_tokens * top_k, n_experts, hdr, slot_e, plan, nullptr, 0, 0);
}

// ------------------------------------------------------------- product ----
// K tile (units) of a workgroup whose group has nb slots: as many units as
// the LDS budget allows for nb vectors, a multiple of LPR, balanced over the
// tiles -- the same rule as the dense product's launch plan, so the lanes sum
// their units in the same order whatever the tile (tiles hold whole multiples
// of LPR units).
template <class F>
__host__ __device__ inline int tile_for(int64_t units, int nb, int LPR) {
    const int64_t per_unit = (int64_t)16 * TileLds<F>::unit_stride(nb);
    int64_t max_units = (int64_t)(LDS_BUDGET / per_unit) / LPR * LPR;
    if (max_units < LPR) max_units = LPR;
    if (units <= max_units) return (int)(units > 0 ? units : 1);
    const int64_t n_tiles = (units + max_units - 1) / max_units;
    const int64_t tu = (units + n_tiles - 1) / n_tiles;
    return (int)((tu + LPR - 1) / LPR * LPR);
}

// GLU: the gated unit of the routed feed-forward block instead of one
// product.  experts is then the gate stack and experts_up the up stack; a
// workgroup covers 2 SR rows, wavefronts 0, 1 computing the gate rows and
// wavefronts 2, 3 the same rows of the up matrix (on the activations they
// stage together), and out[slot][n] = act(gate) * up, fp32 or bf16 (out_bf16).
// Row tile blockIdx.x of the product of one group: entry en (expert e, nb >= 1
// slots; en may point to global or LDS memory).
template <int TYPE, int XT, int D, bool RING, bool GLU>
__device__ __forceinline__ void experts_tile(const uint8_t* __restrict__ experts,
                                             const uint8_t* __restrict__ experts_up, int64_t expert_bytes, int64_t N,
                                             int64_t K, const uint8_t* __restrict__ x, int x_per_slot, int top_k,
                                             int S, const Entry* en, int nb, int e, void* __restrict__ out,
                                             int out_bf16, int act, int LPR, uint8_t* lds) {
    const int tid = threadIdx.x;
    const int tile_units = tile_for<Fmt<TYPE>>(K / Fmt<TYPE>::UW, nb, LPR);
    const int64_t rpw = (int64_t)(GLU ? 2 : NTHREADS >> 6) * (64 / LPR);
    const int64_t rowA = (int64_t)blockIdx.x * rpw;
    // the group's vector and output pointers live in LDS: the staging picks
    // them by a loop index, which a private copy would turn into scratch
    // memory accesses
    __shared__ XSrc xs;
    __shared__ YDst yd;
    if (tid < 8) {
        const int esz = XT == 0 ? 4 : 2;
        const int slot = min(max(en->sel[tid < nb ? tid : 0], 0), S - 1);
        const int64_t xrow = x_per_slot ? slot : slot / top_k;
        xs.p[tid] = x + xrow * K * esz;
        yd.p[tid] = static_cast<float*>(out) + (int64_t)slot * N;
    }
    __syncthreads();
    if constexpr (!GLU) {
        gemv_workgroup<TYPE, XT, 8, D, RING>(experts + (int64_t)e * expert_bytes, N, K, rowA, xs, nb, yd, LPR,
                                              tile_units, lds, (int)(threadIdx.x >> 6), NTHREADS >> 6);
    } else {
        // [gate | up][vector][row in tile]; 2 SR <= 32 rows (LPR >= 4)
        __shared__ float gu[2][CH][32];
        const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), half = wave >> 1;
        const int64_t row_bytes = (K / Fmt<TYPE>::QK) * Fmt<TYPE>::BB;
        YDst yp;
#pragma unroll
        for (int b = 0; b < 8; ++b) yp.p[b] = &gu[half][b < CH ? b : 0][0];
        const uint8_t* W = (half ? experts_up : experts) + (int64_t)e * expert_bytes + rowA * row_bytes;
        gemv_workgroup<TYPE, XT, 8, D, RING>(W, N - rowA, K, 0, xs, nb, yp, LPR, tile_units, lds, wave & 1, 2);
        __syncthreads();
        const int rows = (int)rpw;
        const int64_t nr = N - rowA < rpw ? N - rowA : rpw;
        for (int i = tid; i < nb * rows; i += NTHREADS) {
            const int b = i / rows, r = i - b * rows;
            if (r >= nr) continue;
            const float v = act_fn(act, gu[0][b][r]) * gu[1][b][r];
            const int64_t o = (int64_t)min(max(en->sel[b], 0), S - 1) * N + rowA + r;
            if (out_bf16) static_cast<uint16_t*>(out)[o] = f2bf(v);
            else static_cast<float*>(out)[o] = v;
        }
    }
}

template <int TYPE, int XT, int D, bool RING, bool GLU>
__global__ __launch_bounds__(NTHREADS) void k_experts(const uint8_t* __restrict__ experts,
                                                      const uint8_t* __restrict__ experts_up, int64_t expert_bytes,
                                                      int64_t N, int64_t K, const uint8_t* __restrict__ x,
                                                      int x_per_slot, int top_k, int n_experts, int S,
                                                      const int* __restrict__ ws_hdr, const Entry* __restrict__ plan,
                                                      void* __restrict__ out, int out_bf16, int act, int LPR) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int g = blockIdx.y;
    // the group count and this workgroup's entry, loaded together (the grid
    // has one row per table entry, so plan[g] exists even when unused)
    const int n_groups = ws_hdr[1];
    const Entry* en = plan + g;
    // fields clamped to their ranges: a workspace that holds no table (a
    // caller's mistake when ids are not given) then gives wrong numbers but
    // no access outside the experts, the activations or the outputs.  An
    // entry of no slots is a slot that heads no group in a table indexed by
    // slot (k_experts_routed's).
    const int nb = min(max(en->nb, 0), CH), e = min(max(en->e, 0), n_experts - 1);
    if (g >= n_groups || nb == 0) return;
    experts_tile<TYPE, XT, D, RING, GLU>(experts, experts_up, expert_bytes, N, K, x, x_per_slot, top_k, S, en, nb, e,
                                         out, out_bf16, act, LPR, lds);
}

// The gated unit with the routing in the same launch, for at most 8 tokens,
// 64 slots and 128 experts.  Row blockIdx.y of the grid stands for slot
// s = t * top_k + j, and each workgroup finds the group that s heads, if any,
// without a table: the expert e of s is the key of rank j among token t's
// (the 64-bit keys of gq_route_topk: the logit's order-preserving image above
// the complemented id), found bit by bit from the top -- the largest v with
// more than j keys >= v -- by wavefront ballots; the slots of e are then, for
// each token u, slot u * top_k + r when the rank r of e's key among token u's
// keys is below top_k.  s heads a group when its rank among the slots of e
// (slot order) is a multiple of CH, and the group is s and the next slots of
// e, at most CH: the groups k_plan forms, each computed in the same order, so
// h is identical to routing and a k_experts launch.  Workgroups of the other
// slots exit.  For the later products of the layer, the workgroups of row
// tile 0 leave a table indexed by slot in the workspace (entry s: the group
// that s heads, or no slots), the slots' experts, the header (no invalid ids,
// S entries), and slot s's id and weight, which they take from the router's
// own step (gq_route_topk's top_k rounds and softmax) so that both are
// bit-identical to gq_route_topk's.
constexpr int ROUTE_NI = 2;    // keys per lane: up to 128 experts
constexpr int ROUTE_TMAX = 8;  // tokens

// (the load is unconditional, from a clamped index, so that the loads of all
// the keys are issued before the first wait)
__device__ __forceinline__ uint64_t route_key(const float* __restrict__ l, int ex, int n_experts, bool valid) {
    const float v = l[ex < n_experts ? ex : n_experts - 1];
    const uint64_t keep = 0ull - (uint64_t)(valid && ex < n_experts);  // all ones or zero
    return (((uint64_t)gqr::order_key(v) << 32) | (uint32_t)~(uint32_t)ex) & keep;
}

// number of the wavefront's keys (ROUTE_NI per lane) >= v, or > v (GT)
template <bool GT>
__device__ __forceinline__ int keys_above(const uint64_t (&k)[ROUTE_NI], uint64_t v) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < ROUTE_NI; ++i) c += __popcll(__ballot(GT ? k[i] > v : k[i] >= v));
    return c;
}

template <int TYPE, int XT, int D, bool RING>
__global__ __launch_bounds__(NTHREADS) void k_experts_routed(
    const uint8_t* __restrict__ gate, const uint8_t* __restrict__ up, int64_t expert_bytes, int64_t N, int64_t K,
    const uint8_t* __restrict__ x, const float* __restrict__ logits, int n_tokens, int top_k, int n_experts,
    int32_t* __restrict__ ids, float* __restrict__ weights, int* __restrict__ hdr, int* __restrict__ slot_e,
    Entry* __restrict__ plan, void* __restrict__ out, int out_bf16, int act, int LPR) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ Entry le;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int S = n_tokens * top_k, s = blockIdx.y, t = s / top_k, j = s - t * top_k;
    const bool writer = blockIdx.x == 0;
    // wavefront 0 finds the group (the others wait at the barrier, leaving
    // their SIMDs' issue slots to the other workgroups there); in row tile 0
    // wavefront 1 meanwhile routes token t for slot s's id and weight
    if (wave == 0) {
        // every token's keys, token t's apart; the empty asm statements take
        // every loaded value before the first use, so that all the loads are
        // in flight together (left to itself the compiler issues the later
        // tokens' loads one round trip after the search)
        uint64_t key[ROUTE_TMAX][ROUTE_NI], kt[ROUTE_NI];
#pragma unroll
        for (int u = 0; u < ROUTE_TMAX; ++u)
#pragma unroll
            for (int i = 0; i < ROUTE_NI; ++i)
                key[u][i] = route_key(logits + (int64_t)min(u, n_tokens - 1) * n_experts, lane + 64 * i, n_experts,
                                      u < n_tokens);
#pragma unroll
        for (int i = 0; i < ROUTE_NI; ++i)
            kt[i] = route_key(logits + (int64_t)t * n_experts, lane + 64 * i, n_experts, true);
#pragma unroll
        for (int u = 0; u < ROUTE_TMAX; ++u)
#pragma unroll
            for (int i = 0; i < ROUTE_NI; ++i) asm volatile("" : : "v"(key[u][i]));
        // the key of rank j: its high half bit by bit (32-bit compares), then
        // the id bits among the keys of that high half (every real key's low
        // half is ~id with id < 128, so its 25 upper bits are set)
        uint32_t kh[ROUTE_NI], kl[ROUTE_NI];
#pragma unroll
        for (int i = 0; i < ROUTE_NI; ++i) {
            kh[i] = (uint32_t)(kt[i] >> 32);
            kl[i] = (uint32_t)kt[i];
        }
        uint32_t vh = 0;
        for (int b = 31; b >= 0; --b) {
            const uint32_t c = vh | (1u << b);
            int n = 0;
#pragma unroll
            for (int i = 0; i < ROUTE_NI; ++i) n += __popcll(__ballot(kh[i] >= c));
            if (n > j) vh = c;
        }
        int above = 0;
        uint64_t eq[ROUTE_NI];
#pragma unroll
        for (int i = 0; i < ROUTE_NI; ++i) {
            above += __popcll(__ballot(kh[i] > vh));
            eq[i] = __ballot(kh[i] == vh);
        }
        uint32_t vl = 0xFFFFFF80u;
        for (int b = 6; b >= 0; --b) {
            const uint32_t c = vl | (1u << b);
            int n = above;
#pragma unroll
            for (int i = 0; i < ROUTE_NI; ++i) n += __popcll(__ballot(kl[i] >= c) & eq[i]);
            if (n > j) vl = c;
        }
        const int e = min(max((int)~vl, 0), n_experts - 1);  // (in range by construction)
        // the slots of e: token u holds e at rank r < top_k as slot u * top_k + r
        uint64_t same = 0;
#pragma unroll
        for (int u = 0; u < ROUTE_TMAX; ++u) {
            const uint64_t kx = ROUTE_NI == 1 || e < 64 ? key[u][0] : key[u][ROUTE_NI - 1];
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(kx >> 32), e & 63);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kx, e & 63);
            const int r = keys_above<true>(key[u], ((uint64_t)hi << 32) | lo);
            if (u < n_tokens && r < top_k) same |= 1ull << (u * top_k + r);
        }
        const uint64_t below = same & ((1ull << s) - 1ull);  // s < S <= 64
        const uint64_t from = same & ~below;                 // s and the later slots of e
        const int nb = __popcll(below) % CH ? 0 : min(CH, __popcll(from));
        int sel = s;  // lane i < nb: the i-th slot of the group
        uint64_t m = from;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int b = __ffsll((unsigned long long)m) - 1;
            if (lane == i && i < nb) sel = b;
            m &= m - 1ull;
        }
        if (lane < CH) le.sel[lane] = sel;
        if (lane == 0) {
            le.e = e;
            le.nb = nb;
        }
        if (writer) {
            if (lane < CH) plan[s].sel[lane] = sel;
            if (lane == 0) {
                plan[s].e = e;
                plan[s].nb = nb;
                slot_e[s] = e;
                if (s == 0) {
                    hdr[0] = 0;
                    hdr[1] = S;
                }
            }
        }
    } else if (wave == 1 && writer) {
        int id;
        float w;
        gqr::route_token<ROUTE_NI>(logits + (int64_t)t * n_experts, n_experts, top_k, lane, id, w);
        if (lane == j) {
            ids[s] = id;
            weights[s] = w;
        }
    }
    lds_barrier();
    const int nb = __builtin_amdgcn_readfirstlane(le.nb), e = __builtin_amdgcn_readfirstlane(le.e);
    if (nb == 0) return;
    experts_tile<TYPE, XT, D, RING, true>(gate, up, expert_bytes, N, K, x, 0, top_k, S, &le, nb, e, out, out_bf16,
                                          act, LPR, lds);
}

// ------------------------------------------------------------- combine ----
// y[t][n] = sum_j route_w[t][j] * slot[t][j][n] over the valid slots, j in
// increasing order (slot_e: each slot's expert from the table, -1 if invalid).
// The slots are read eight at a time, every load issued before the first sum
// (an invalid slot's row is read and then skipped), so that a token's slots
// cost one round trip per eight instead of one each.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ slot_out, const int* __restrict__ slot_e,
                                                 const float* __restrict__ route_w, int top_k, int64_t N,
                                                 float* __restrict__ y) {
    const int t = blockIdx.y;
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float acc = 0.f;
    for (int j0 = 0; j0 < top_k; j0 += 8) {
        float v[8], w[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u < top_k ? j0 + u : top_k - 1;
            ok[u] = j0 + u < top_k && slot_e[t * top_k + j] >= 0;
            w[u] = route_w[t * top_k + j];
            v[u] = slot_out[((int64_t)t * top_k + j) * N + n];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (ok[u]) acc = __builtin_fmaf(w[u], v[u], acc);
    }
    y[(int64_t)t * N + n] = acc;
}

// What one launch computes: a plain routed product (up == nullptr, fp32 out)
// or the gated unit (gate stack in experts, up stack in up).
struct Job {
    const uint8_t* experts;
    const uint8_t* up;
    int64_t N, K;
    const uint8_t* x;
    int x_per_slot, top_k, n_experts;
    const int32_t* ids;  // nullptr: the table in the workspace is reused
    int* ws_hdr;
    int* slot_e;
    Entry* plan;
    void* out;
    int out_bf16, act;
    bool zero_bad;  // invalid slots' output rows are the caller's (zero them)
    // the gated unit routing its tokens itself (k_experts_routed): logits in,
    // ids and weights out
    const float* logits = nullptr;
    int n_tokens = 0;
    int32_t* ids_out = nullptr;
    float* w_out = nullptr;
};

template <int TYPE, int XT, int D, bool RING = false>
hipError_t launch_experts_d(const Plan& p, const WsLayout& L, const Job& j, hipStream_t s) {
    using F = Fmt<TYPE>;
    const int64_t expert_bytes = j.N * (j.K / F::QK) * F::BB;
    const bool glu = j.up != nullptr;
    const int64_t rpw = (int64_t)(glu ? 2 : NTHREADS >> 6) * (64 / p.LPR);
    const int64_t gy = (j.N + rpw - 1) / rpw;
    if (L.Gmax > 65535 || gy > 0x7fffffff) return hipErrorInvalidValue;
    if (j.logits) {
        hipLaunchKernelGGL((k_experts_routed<TYPE, XT, D, RING>), dim3((unsigned)gy, (unsigned)L.S), dim3(NTHREADS),
                           p.lds, s, j.experts, j.up, expert_bytes, j.N, j.K, j.x, j.logits, j.n_tokens, j.top_k,
                           j.n_experts, j.ids_out, j.w_out, j.ws_hdr, j.slot_e, j.plan, j.out, j.out_bf16, j.act,
                           p.LPR);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)gy, (unsigned)L.Gmax);
    if (glu)
        hipLaunchKernelGGL((k_experts<TYPE, XT, D, RING, true>), grid, dim3(NTHREADS), p.lds, s, j.experts, j.up,
                           expert_bytes, j.N, j.K, j.x, j.x_per_slot, j.top_k, j.n_experts, L.S, j.ws_hdr, j.plan,
                           j.out, j.out_bf16, j.act, p.LPR);
    else
        hipLaunchKernelGGL((k_experts<TYPE, XT, D, RING, false>), grid, dim3(NTHREADS), p.lds, s, j.experts, j.up,
                           expert_bytes, j.N, j.K, j.x, j.x_per_slot, j.top_k, j.n_experts, L.S, j.ws_hdr, j.plan,
                           j.out, 0, 0, p.LPR);
    return hipGetLastError();
}

template <int TYPE, int XT>
hipError_t launch_experts(const WsLayout& L, const Job& j, hipStream_t s) {
    using F = Fmt<TYPE>;
    // the launch covers the rows of up to min(S, n_experts) experts (twice
    // as many for the gated unit)
    const int64_t distinct = L.S < j.n_experts ? L.S : j.n_experts;
    Plan p = plan_for<F>(j.N, j.K, CH, (j.up ? 2 : 1) * j.N * distinct, 4);
    // each workgroup picks its K tile from its slot count (tile_for): the
    // LDS is sized for the largest of those tiles, and the units per lane of
    // the largest tile (one slot) decide between the straight-line form and
    // the ring
    const int64_t units = j.K / F::UW;
    p.lds = 0;
    for (int nb = 1; nb <= CH; ++nb) {
        const size_t b = (size_t)16 * TileLds<F>::unit_stride(nb) * (size_t)tile_for<F>(units, nb, p.LPR);
        p.lds = b > p.lds ? b : p.lds;
    }
    const int T1 = (tile_for<F>(units, 1, p.LPR) + p.LPR - 1) / p.LPR;
    p.ring = T1 > D_MAX;
    p.D = p.ring ? 0 : T1;
#define GQ_LAUNCH(DD, RR) launch_experts_d<TYPE, XT, DD, RR>(p, L, j, s)
    // two units per lane in flight (measured against 1 and 4: the gated MoE
    // product 2.5% faster than with 4, the rest equal)
    if (p.ring) return GQ_LAUNCH(2, true);
    switch (p.D) {
    case 1: return GQ_LAUNCH(1, false);
    case 2: return GQ_LAUNCH(2, false);
    case 3: return GQ_LAUNCH(3, false);
    case 4: return GQ_LAUNCH(4, false);
    case 5: return GQ_LAUNCH(5, false);
    case 6: return GQ_LAUNCH(6, false);
    default: return hipErrorInvalidValue;
    }
#undef GQ_LAUNCH
}

template <int TYPE>
hipError_t launch_experts_x(const WsLayout& L, const Job& j, int x_dtype, hipStream_t s) {
    if (x_dtype == DT_F32) return launch_experts<TYPE, 0>(L, j, s);
    return launch_experts<TYPE, 1>(L, j, s);
}

hipError_t launch_type(int type, const WsLayout& L, const Job& j, int x_dtype, hipStream_t s) {
    // the group table first; zeroed rows for invalid ids where the product
    // writes its outputs straight to the caller's buffer
    if (j.ids) {
        void* zero_out = j.zero_bad ? j.out : nullptr;
        hipLaunchKernelGGL(k_plan, dim3(1), dim3(NTHREADS), 0, s, j.ids, L.S, j.n_experts, j.ws_hdr, j.slot_e, j.plan,
                           zero_out, j.N, j.out_bf16);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (type == T_Q4_0) return launch_experts_x<T_Q4_0>(L, j, x_dtype, s);
    if (type == T_Q4_K) return launch_experts_x<T_Q4_K>(L, j, x_dtype, s);
    if (type == T_Q5_K) return launch_experts_x<T_Q5_K>(L, j, x_dtype, s);
    return launch_experts_x<T_Q6_K>(L, j, x_dtype, s);
}

template <int NI>
hipError_t launch_route_plan(const float* logits, int n_tokens, int n_experts, int top_k, int32_t* ids, float* w,
                             void* ws, hipStream_t s) {
    const WsLayout L = layout(n_experts, n_tokens, top_k, 0);
    uint8_t* b = static_cast<uint8_t*>(ws);
    hipLaunchKernelGGL(k_route_plan<NI>, dim3(1), dim3(64 * RW), 0, s, logits, n_tokens, n_experts, top_k, ids, w,
                       reinterpret_cast<int*>(b), reinterpret_cast<int*>(b + L.off_slot),
                       reinterpret_cast<Entry*>(b + L.off_plan));
    return hipGetLastError();
}

}  // namespace

hipError_t gqk_route_topk_plan(const float* logits, int n_tokens, int n_experts, int top_k, int32_t* ids, float* w,
                               void* ws, hipStream_t s) {
    if (n_tokens * top_k > MAX_SLOTS) return hipErrorInvalidValue;
    const int ni = (n_experts + 63) / 64;
    if (ni <= 1) return launch_route_plan<1>(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
    if (ni <= 2) return launch_route_plan<2>(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
    if (ni <= 4) return launch_route_plan<4>(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
    if (ni <= 8) return launch_route_plan<8>(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
    if (ni <= 16) return launch_route_plan<16>(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
    if (ni <= 32) return launch_route_plan<32>(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
    return launch_route_plan<64>(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
}

size_t gqk_matvec_id_ws_bytes(int n_experts, int n_tokens, int top_k, int64_t N) {
    return layout(n_experts, n_tokens, top_k, N).total;
}

hipError_t gqk_matvec_id(int type, const void* experts, int n_experts, int64_t N, int64_t K, const int32_t* ids,
                         int n_tokens, int top_k, const void* x, int x_dtype, int x_per_slot, const float* route_w,
                         float* y, void* ws, hipStream_t s) {
    const WsLayout L = layout(n_experts, n_tokens, top_k, N);
    if (L.S > MAX_SLOTS) return hipErrorInvalidValue;
    uint8_t* w = static_cast<uint8_t*>(ws);
    int* hdr = reinterpret_cast<int*>(w);
    // per-slot outputs: straight into y when there is no routing combine
    float* out = route_w ? reinterpret_cast<float*>(w + L.off_out) : y;
    Entry* plan = reinterpret_cast<Entry*>(w + L.off_plan);
    int* slot_e = reinterpret_cast<int*>(w + L.off_slot);
    const Job j{static_cast<const uint8_t*>(experts), nullptr, N, K, static_cast<const uint8_t*>(x), x_per_slot,
                top_k, n_experts, ids, hdr, slot_e, plan, out, 0, 0, route_w == nullptr};
    const hipError_t e = launch_type(type, L, j, x_dtype, s);
    if (e != hipSuccess || !route_w) return e;
    const unsigned nx = (unsigned)((N + 255) / 256);
    hipLaunchKernelGGL(k_combine, dim3(nx, (unsigned)n_tokens), dim3(256), 0, s, out, slot_e, route_w, top_k, N, y);
    return hipGetLastError();
}

hipError_t gqk_matvec_id_glu(int type, const void* experts_gate, const void* experts_up, int n_experts, int64_t N,
                             int64_t K, const int32_t* ids, int n_tokens, int top_k, const void* x, int x_dtype,
                             int act, void* h, int h_dtype, void* ws, hipStream_t s) {
    const WsLayout L = layout(n_experts, n_tokens, top_k, N);
    if (L.S > MAX_SLOTS) return hipErrorInvalidValue;
    uint8_t* w = static_cast<uint8_t*>(ws);
    const Job j{static_cast<const uint8_t*>(experts_gate), static_cast<const uint8_t*>(experts_up), N, K,
                static_cast<const uint8_t*>(x), 0, top_k, n_experts, ids, reinterpret_cast<int*>(w),
                reinterpret_cast<int*>(w + L.off_slot), reinterpret_cast<Entry*>(w + L.off_plan), h,
                h_dtype == DT_BF16 ? 1 : 0, act, true};
    return launch_type(type, L, j, x_dtype, s);
}

hipError_t gqk_route_matvec_id_glu(int type, const void* experts_gate, const void* experts_up, int n_experts,
                                   int64_t N, int64_t K, const float* logits, int n_tokens, int top_k, int32_t* ids,
                                   float* w, const void* x, int x_dtype, int act, void* h, int h_dtype, void* ws,
                                   hipStream_t s) {
    const WsLayout L = layout(n_experts, n_tokens, top_k, N);
    if (L.S > MAX_SLOTS) return hipErrorInvalidValue;
    // the one-launch form needs the slots in one wavefront's lanes, the
    // logits in ROUTE_NI per lane, and a table slot for every slot (the later
    // products' grids have Gmax rows); otherwise the router with the table,
    // then the gated unit on it
    if (n_tokens > ROUTE_TMAX || L.S > 64 || n_experts > 64 * ROUTE_NI || L.S > L.Gmax || N == 0 || K == 0) {
        const hipError_t e = gqk_route_topk_plan(logits, n_tokens, n_experts, top_k, ids, w, ws, s);
        if (e != hipSuccess || N == 0) return e;
        return gqk_matvec_id_glu(type, experts_gate, experts_up, n_experts, N, K, nullptr, n_tokens, top_k, x,
                                 x_dtype, act, h, h_dtype, ws, s);
    }
    uint8_t* b = static_cast<uint8_t*>(ws);
    Job j{static_cast<const uint8_t*>(experts_gate), static_cast<const uint8_t*>(experts_up), N, K,
          static_cast<const uint8_t*>(x), 0, top_k, n_experts, nullptr, reinterpret_cast<int*>(b),
          reinterpret_cast<int*>(b + L.off_slot), reinterpret_cast<Entry*>(b + L.off_plan), h,
          h_dtype == DT_BF16 ? 1 : 0, act, true};
    j.logits = logits;
    j.n_tokens = n_tokens;
    j.ids_out = ids;
    j.w_out = w;
    return launch_type(type, L, j, x_dtype, s);
}

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];  // device address of `scratch` on each device

hipError_t scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t gqk_matvec_id_noalloc(int type, const void* experts, int n_experts, int64_t N, int64_t K,
                                 const int32_t* ids, int n_tokens, int top_k, const void* x, int x_dtype,
                                 int x_per_slot, const float* route_w, float* y, hipStream_t s) {
    if (gqk_matvec_id_ws_bytes(n_experts, n_tokens, top_k, N) > GQK_NOALLOC_WS_BYTES) return hipErrorInvalidValue;
    void* ws = nullptr;
    const hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess) return e;
    // the table, its header and the per-slot outputs are all written by the
    // call itself: nothing in the array has to start at zero
    return gqk_matvec_id(type, experts, n_experts, N, K, ids, n_tokens, top_k, x, x_dtype, x_per_slot, route_w, y,
                         ws, s);
}

hipError_t gqk_matvec_id_bad_count(const void* ws, hipStream_t s, int32_t* n_bad) {
    hipError_t e = hipMemcpyAsync(n_bad, ws, sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);
}
