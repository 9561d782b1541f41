// gq_internal.h -- launchers behind the C ABI (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Compute units of the current device (queried once per device).
int gqk_cu_count();

// All launchers assume their arguments were validated by the ABI layer.
hipError_t gqk_dequant(int type, const void* blocks, int64_t n_blocks, void* out, int out_dtype,
                       hipStream_t s);

hipError_t gqk_matvec(int type, const void* W, int64_t N, int64_t K, const void* x, int x_dtype,
                      int batch, float* y, hipStream_t s);
// Gated unit: h = act(W_gate x) * (W_up x), batch 1..8 (gq_matvec.hip).
hipError_t gqk_matvec_glu(int type, const void* Wg, const void* Wu, int64_t N, int64_t K, const void* x, int x_dtype,
                          int batch, int act, void* h, int h_dtype, hipStream_t s);
// The same product on the matrix cores, batch 1..16 (gq_mmv.hip).
hipError_t gqk_mmv(int type, const void* W, int64_t N, int64_t K, const void* x, int x_dtype, int batch,
                   float* y, hipStream_t s);

// Routed experts.  Workspace layout is private to gq_matvec_id.hip.
size_t gqk_matvec_id_ws_bytes(int n_experts, int n_tokens, int top_k, int64_t N);
hipError_t gqk_matvec_id(int type, const void* experts, int n_experts, int64_t N, int64_t K,
                         const int32_t* ids, int n_tokens, int top_k, const void* x, int x_dtype,
                         int x_per_slot, const float* route_w, float* y, void* ws, hipStream_t s);
// Routed gated unit: h[t][j][n] = act(gate_e[n] . x_t) * (up_e[n] . x_t), e = ids[t][j];
// ws has the layout of gqk_matvec_id_ws_bytes (header and group table; the
// per-slot output area is not used).
hipError_t gqk_matvec_id_glu(int type, const void* experts_gate, const void* experts_up, int n_experts, int64_t N,
                             int64_t K, const int32_t* ids, int n_tokens, int top_k, const void* x, int x_dtype,
                             int act, void* h, int h_dtype, void* ws, hipStream_t s);
hipError_t gqk_matvec_id_bad_count(const void* ws, hipStream_t s, int32_t* n_bad);
// gqk_matvec_id with the workspace in a per-device array of the library
// (GQK_NOALLOC_WS_BYTES; larger requests fail with hipErrorInvalidValue).
constexpr size_t GQK_NOALLOC_WS_BYTES = (size_t)8 << 20;
hipError_t gqk_matvec_id_noalloc(int type, const void* experts, int n_experts, int64_t N, int64_t K,
                                 const int32_t* ids, int n_tokens, int top_k, const void* x, int x_dtype,
                                 int x_per_slot, const float* route_w, float* y, hipStream_t s);

hipError_t gqk_matmul(int type, const void* W, int64_t N, int64_t K, const void* X, int x_dtype,
                      int64_t M, int64_t ldx, float* Y, int64_t ldy, hipStream_t s);

hipError_t gqk_route_topk(const float* logits, int n_tokens, int n_experts, int top_k, int32_t* ids, float* w,
                          hipStream_t s);
// Routing and the routed gated unit (gq_matvec_id.hip): ids, weights, h and
// the group table in ws, as gqk_route_topk_plan then gqk_matvec_id_glu with
// no ids.
hipError_t gqk_route_matvec_id_glu(int type, const void* experts_gate, const void* experts_up, int n_experts,
                                   int64_t N, int64_t K, const float* logits, int n_tokens, int top_k, int32_t* ids,
                                   float* w, const void* x, int x_dtype, int act, void* h, int h_dtype, void* ws,
                                   hipStream_t s);
// Routing plus the routed products' group table in ws (gq_matvec_id.hip).
hipError_t gqk_route_topk_plan(const float* logits, int n_tokens, int n_experts, int top_k, int32_t* ids, float* w,
                               void* ws, hipStream_t s);
