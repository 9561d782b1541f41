// gq_abi.cpp -- the extern "C" boundary: argument validation (before any HIP
// call), dispatch to the kernel launchers, status codes.  See include/gq.h.
#include "../../include/gq.h"

#include <hip/hip_runtime.h>

#include "gq_internal.h"

namespace {

bool known_type(int t) { return t == GQ_Q4_0 || t == GQ_Q4_K || t == GQ_Q6_K || t == GQ_Q5_K; }

int qk_of(int t) { return t == GQ_Q4_0 ? 32 : 256; }
int bytes_of(int t) { return t == GQ_Q4_0 ? 18 : (t == GQ_Q4_K ? 144 : (t == GQ_Q5_K ? 176 : 210)); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gq_status from_hip(hipError_t e) { return e == hipSuccess ? GQ_OK : GQ_ERR_LAUNCH; }

// Largest element count any single launch handles (keeps 32-bit grid sizes
// and 64-bit byte offsets far from overflow).
constexpr int64_t MAX_ELEMS = (int64_t)1 << 40;
// Longest row the decode products take: a workgroup addresses its (at most 64)
// rows through one buffer resource whose span must stay below 2^31 bytes.
constexpr int64_t MAX_K_DECODE = (int64_t)1 << 22;

// Which decode path: the dot-product path's work grows with every vector, the
// matrix-core path's per-weight work does not, but it carries more fixed cost
// per row tile.  Measured crossovers (MI355X, Q4_0 / Q4_K / Q5_K / Q6_K at
// hidden 2560..5120 and the routed-expert shapes): from 5 vectors the matrix
// cores win for every type and shape; at 4 they win for the 4/5-bit types
// unless N > 4 K (many short rows, where the dot path stages few activations
// per row), at 3 only for N <= 1.25 K; at 1..2 and for Q6_K below 5 the dot
// path wins.
bool use_matrix_cores(int batch, int type, int64_t N, int64_t K) {
    if (batch >= 5) return true;
    if (type == GQ_Q6_K || batch < 3) return false;
    return batch == 4 ? N <= 4 * K : 4 * N <= 5 * K;
}

}  // namespace

extern "C" {

int gq_abi_version(void) { return GQ_ABI_VERSION; }

const char* gq_status_str(gq_status s) {
    switch (s) {
    case GQ_OK: return "ok";
    case GQ_ERR_TYPE: return "unknown block type";
    case GQ_ERR_DTYPE: return "unsupported element type";
    case GQ_ERR_SHAPE: return "invalid shape";
    case GQ_ERR_NULL: return "null pointer";
    case GQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GQ_ERR_UNSUPPORTED: return "unsupported combination";
    case GQ_ERR_WORKSPACE: return "workspace missing or too small";
    case GQ_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

gq_status gq_block_info(gq_type t, int32_t* elems, int32_t* bytes) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (!elems || !bytes) return GQ_ERR_NULL;
    *elems = qk_of(t);
    *bytes = bytes_of(t);
    return GQ_OK;
}

gq_status gq_dequant(gq_type t, const void* blocks, int64_t n_blocks, void* out, gq_dtype out_dtype,
                     hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (out_dtype != GQ_F32 && out_dtype != GQ_BF16 && out_dtype != GQ_F16) return GQ_ERR_DTYPE;
    if (n_blocks < 0 || n_blocks * qk_of(t) > MAX_ELEMS) return GQ_ERR_SHAPE;
    if (n_blocks == 0) return GQ_OK;
    if (!blocks || !out) return GQ_ERR_NULL;
    if (!aligned16(blocks) || !aligned16(out)) return GQ_ERR_ALIGN;
    try {
        return from_hip(gqk_dequant(t, blocks, n_blocks, out, out_dtype, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_matvec(gq_type t, const void* W, int64_t N, int64_t K, const void* x, gq_dtype x_dtype,
                    int32_t batch, float* y, hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (N < 0 || K < 0 || K % qk_of(t) != 0 || batch < 1) return GQ_ERR_SHAPE;
    if (N > MAX_ELEMS || K > MAX_K_DECODE || (K > 0 && N > MAX_ELEMS / K)) return GQ_ERR_SHAPE;
    if (batch > 16) return GQ_ERR_UNSUPPORTED;
    if (N == 0) return GQ_OK;
    if (!y || (K > 0 && (!W || !x))) return GQ_ERR_NULL;
    if (!aligned16(y) || (K > 0 && (!aligned16(W) || !aligned16(x)))) return GQ_ERR_ALIGN;
    try {
        if (use_matrix_cores(batch, t, N, K)) return from_hip(gqk_mmv(t, W, N, K, x, x_dtype, batch, y, stream));
        return from_hip(gqk_matvec(t, W, N, K, x, x_dtype, batch, y, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_matvec_glu(gq_type t, const void* W_gate, const void* W_up, int64_t N, int64_t K, const void* x,
                        gq_dtype x_dtype, int32_t batch, gq_act act, void* h, gq_dtype h_dtype, hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (h_dtype != GQ_F32 && h_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (N < 0 || K < 0 || K % qk_of(t) != 0 || batch < 1) return GQ_ERR_SHAPE;
    if (N > MAX_ELEMS || K > MAX_K_DECODE || (K > 0 && N > MAX_ELEMS / K)) return GQ_ERR_SHAPE;
    if (batch > 8 || (act != GQ_ACT_SILU && act != GQ_ACT_GELU_TANH)) return GQ_ERR_UNSUPPORTED;
    if (N == 0) return GQ_OK;
    if (!h || (K > 0 && (!W_gate || !W_up || !x))) return GQ_ERR_NULL;
    if (!aligned16(h) || (K > 0 && (!aligned16(W_gate) || !aligned16(W_up) || !aligned16(x)))) return GQ_ERR_ALIGN;
    try {
        return from_hip(gqk_matvec_glu(t, W_gate, W_up, N, K, x, x_dtype, batch, act, h, h_dtype, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_matvec_id_workspace(int32_t n_experts, int32_t n_tokens, int32_t top_k, int64_t N, size_t* bytes) {
    if (!bytes) return GQ_ERR_NULL;
    if (n_experts < 1 || n_tokens < 0 || top_k < 1 || top_k > n_experts || N < 0 ||
        (int64_t)n_tokens * top_k > 1024)
        return GQ_ERR_SHAPE;
    *bytes = gqk_matvec_id_ws_bytes(n_experts, n_tokens, top_k, N);
    return GQ_OK;
}

gq_status gq_matvec_id(gq_type t, const void* experts, int32_t n_experts, int64_t N, int64_t K,
                       const int32_t* ids, int32_t n_tokens, int32_t top_k, const void* x, gq_dtype x_dtype,
                       int32_t x_per_slot, const float* route_w, float* y, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (n_experts < 1 || n_tokens < 0 || top_k < 1 || top_k > n_experts || N < 0 || K < 0 ||
        K % qk_of(t) != 0 || (x_per_slot != 0 && x_per_slot != 1) || (int64_t)n_tokens * top_k > 1024)
        return GQ_ERR_SHAPE;
    if (N > MAX_ELEMS || K > MAX_K_DECODE || (K > 0 && N > MAX_ELEMS / K) ||
        (K > 0 && N > 0 && (int64_t)n_experts > MAX_ELEMS / (N * K)))
        return GQ_ERR_SHAPE;
    if (n_tokens == 0 || N == 0) return GQ_OK;
    // ids may be NULL: the group table already in ws is then used
    if (!y || !ws || (K > 0 && (!experts || !x))) return GQ_ERR_NULL;
    if ((ids && !aligned16(ids)) || !aligned16(y) || !aligned16(ws) || (route_w && !aligned16(route_w)) ||
        (K > 0 && (!aligned16(experts) || !aligned16(x))))
        return GQ_ERR_ALIGN;
    if (ws_bytes < gqk_matvec_id_ws_bytes(n_experts, n_tokens, top_k, N)) return GQ_ERR_WORKSPACE;
    try {
        return from_hip(gqk_matvec_id(t, experts, n_experts, N, K, ids, n_tokens, top_k, x, x_dtype, x_per_slot,
                                      route_w, y, ws, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_matvec_id_noalloc(gq_type t, const void* experts, int32_t n_experts, int64_t N, int64_t K,
                               const int32_t* ids, int32_t n_tokens, int32_t top_k, const void* x,
                               gq_dtype x_dtype, int32_t x_per_slot, const float* route_w, float* y,
                               hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (n_experts < 1 || n_tokens < 0 || top_k < 1 || top_k > n_experts || N < 0 || K < 0 ||
        K % qk_of(t) != 0 || (x_per_slot != 0 && x_per_slot != 1) || (int64_t)n_tokens * top_k > 1024)
        return GQ_ERR_SHAPE;
    if (N > MAX_ELEMS || K > MAX_K_DECODE || (K > 0 && N > MAX_ELEMS / K) ||
        (K > 0 && N > 0 && (int64_t)n_experts > MAX_ELEMS / (N * K)))
        return GQ_ERR_SHAPE;
    if (n_tokens == 0 || N == 0) return GQ_OK;
    if (!y || (K > 0 && (!experts || !x))) return GQ_ERR_NULL;
    if ((ids && !aligned16(ids)) || !aligned16(y) || (route_w && !aligned16(route_w)) ||
        (K > 0 && (!aligned16(experts) || !aligned16(x))))
        return GQ_ERR_ALIGN;
    if (gqk_matvec_id_ws_bytes(n_experts, n_tokens, top_k, N) > GQK_NOALLOC_WS_BYTES) return GQ_ERR_WORKSPACE;
    try {
        return from_hip(gqk_matvec_id_noalloc(t, experts, n_experts, N, K, ids, n_tokens, top_k, x, x_dtype,
                                              x_per_slot, route_w, y, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_matvec_id_glu(gq_type t, const void* experts_gate, const void* experts_up, int32_t n_experts, int64_t N,
                           int64_t K, const int32_t* ids, int32_t n_tokens, int32_t top_k, const void* x,
                           gq_dtype x_dtype, gq_act act, void* h, gq_dtype h_dtype, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (h_dtype != GQ_F32 && h_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (n_experts < 1 || n_tokens < 0 || top_k < 1 || top_k > n_experts || N < 0 || K < 0 ||
        K % qk_of(t) != 0 || (int64_t)n_tokens * top_k > 1024)
        return GQ_ERR_SHAPE;
    if (N > MAX_ELEMS || K > MAX_K_DECODE || (K > 0 && N > MAX_ELEMS / K) ||
        (K > 0 && N > 0 && (int64_t)n_experts > MAX_ELEMS / (N * K)))
        return GQ_ERR_SHAPE;
    if (act != GQ_ACT_SILU && act != GQ_ACT_GELU_TANH) return GQ_ERR_UNSUPPORTED;
    if (n_tokens == 0 || N == 0) return GQ_OK;
    if (!h || !ws || (K > 0 && (!experts_gate || !experts_up || !x))) return GQ_ERR_NULL;
    if ((ids && !aligned16(ids)) || !aligned16(h) || !aligned16(ws) ||
        (K > 0 && (!aligned16(experts_gate) || !aligned16(experts_up) || !aligned16(x))))
        return GQ_ERR_ALIGN;
    if (ws_bytes < gqk_matvec_id_ws_bytes(n_experts, n_tokens, top_k, N)) return GQ_ERR_WORKSPACE;
    try {
        return from_hip(gqk_matvec_id_glu(t, experts_gate, experts_up, n_experts, N, K, ids, n_tokens, top_k, x,
                                          x_dtype, act, h, h_dtype, ws, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_matvec_id_check(const void* ws, hipStream_t stream, int32_t* n_bad_ids) {
    if (!ws || !n_bad_ids) return GQ_ERR_NULL;
    if (!aligned16(ws)) return GQ_ERR_ALIGN;
    try {
        return from_hip(gqk_matvec_id_bad_count(ws, stream, n_bad_ids));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_route_topk_plan(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t top_k, int32_t* ids,
                             float* weights, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts || (int64_t)n_tokens * top_k > 1024)
        return GQ_ERR_SHAPE;
    if ((int64_t)n_tokens * n_experts > MAX_ELEMS) return GQ_ERR_SHAPE;
    if (n_experts > 4096 || top_k > 64) return GQ_ERR_UNSUPPORTED;
    if (n_tokens == 0) return GQ_OK;
    if (!logits || !ids || !weights || !ws) return GQ_ERR_NULL;
    if (!aligned16(logits) || !aligned16(ids) || !aligned16(weights) || !aligned16(ws)) return GQ_ERR_ALIGN;
    if (ws_bytes < gqk_matvec_id_ws_bytes(n_experts, n_tokens, top_k, 0)) return GQ_ERR_WORKSPACE;
    try {
        return from_hip(gqk_route_topk_plan(logits, n_tokens, n_experts, top_k, ids, weights, ws, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_route_matvec_id_glu(gq_type t, const void* experts_gate, const void* experts_up, int32_t n_experts,
                                 int64_t N, int64_t K, const float* logits, int32_t n_tokens, int32_t top_k,
                                 int32_t* ids, float* weights, const void* x, gq_dtype x_dtype, gq_act act, void* h,
                                 gq_dtype h_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (h_dtype != GQ_F32 && h_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (n_experts < 1 || n_tokens < 0 || top_k < 1 || top_k > n_experts || N < 0 || K < 0 ||
        K % qk_of(t) != 0 || (int64_t)n_tokens * top_k > 1024)
        return GQ_ERR_SHAPE;
    if ((int64_t)n_tokens * n_experts > MAX_ELEMS) return GQ_ERR_SHAPE;
    if (N > MAX_ELEMS || K > MAX_K_DECODE || (K > 0 && N > MAX_ELEMS / K) ||
        (K > 0 && N > 0 && (int64_t)n_experts > MAX_ELEMS / (N * K)))
        return GQ_ERR_SHAPE;
    if (n_experts > 4096 || top_k > 64) return GQ_ERR_UNSUPPORTED;
    if (act != GQ_ACT_SILU && act != GQ_ACT_GELU_TANH) return GQ_ERR_UNSUPPORTED;
    if (n_tokens == 0) return GQ_OK;
    if (!logits || !ids || !weights || !ws || (N > 0 && !h) || (N > 0 && K > 0 && (!experts_gate || !experts_up || !x)))
        return GQ_ERR_NULL;
    if (!aligned16(logits) || !aligned16(ids) || !aligned16(weights) || !aligned16(ws) || (N > 0 && !aligned16(h)) ||
        (N > 0 && K > 0 && (!aligned16(experts_gate) || !aligned16(experts_up) || !aligned16(x))))
        return GQ_ERR_ALIGN;
    if (ws_bytes < gqk_matvec_id_ws_bytes(n_experts, n_tokens, top_k, N)) return GQ_ERR_WORKSPACE;
    try {
        return from_hip(gqk_route_matvec_id_glu(t, experts_gate, experts_up, n_experts, N, K, logits, n_tokens, top_k,
                                                ids, weights, x, x_dtype, act, h, h_dtype, ws, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t top_k, int32_t* ids,
                        float* weights, hipStream_t stream) {
    if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return GQ_ERR_SHAPE;
    if ((int64_t)n_tokens * n_experts > MAX_ELEMS) return GQ_ERR_SHAPE;
    if (n_experts > 4096 || top_k > 64) return GQ_ERR_UNSUPPORTED;
    if (n_tokens == 0) return GQ_OK;
    if (!logits || !ids || !weights) return GQ_ERR_NULL;
    if (!aligned16(logits) || !aligned16(ids) || !aligned16(weights)) return GQ_ERR_ALIGN;
    try {
        return from_hip(gqk_route_topk(logits, n_tokens, n_experts, top_k, ids, weights, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

gq_status gq_matmul(gq_type t, const void* W, int64_t N, int64_t K, const void* X, gq_dtype x_dtype, int64_t M,
                    int64_t ldx, float* Y, int64_t ldy, hipStream_t stream) {
    if (!known_type(t)) return GQ_ERR_TYPE;
    if (x_dtype != GQ_F32 && x_dtype != GQ_BF16) return GQ_ERR_DTYPE;
    if (N < 0 || K < 0 || M < 0 || K % qk_of(t) != 0 || ldx < K || ldy < N) return GQ_ERR_SHAPE;
    if (N > MAX_ELEMS || K > MAX_ELEMS || M > MAX_ELEMS || (M > 0 && ldx > MAX_ELEMS / M) ||
        (M > 0 && ldy > MAX_ELEMS / M) || (K > 0 && N > MAX_ELEMS / K))
        return GQ_ERR_SHAPE;
    // the prefill kernel addresses 256 rows of X or W through one buffer
    // resource whose span must stay below 2^31 bytes
    if (K > MAX_K_DECODE || ldx >= MAX_K_DECODE) return GQ_ERR_SHAPE;
    if (x_dtype != GQ_BF16) return GQ_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GQ_OK;
    if (!Y || (K > 0 && (!W || !X))) return GQ_ERR_NULL;
    if (!aligned16(Y) || (K > 0 && (!aligned16(W) || !aligned16(X)))) return GQ_ERR_ALIGN;
    if ((ldx * 2) % 16 != 0 || (ldy * 4) % 16 != 0) return GQ_ERR_ALIGN;
    try {
        return from_hip(gqk_matmul(t, W, N, K, X, x_dtype, M, ldx, Y, ldy, stream));
    } catch (...) {
        return GQ_ERR_LAUNCH;
    }
}

}  // extern "C"
