/*
 * gq.h -- C ABI of the block-quantized weight product library (gfx950).
 *
 * The library computes products against weights kept in their packed ggml
 * block form, the operation that "GGUF in transformers" (Hugging Face blog)
 * describes in section "Reusing ggml's Metal kernels", kernel table, row
 * "ggml-quantization": matrix operations that read the packed quantized
 * weights directly -- including only the selected experts of an MoE model --
 * instead of expanding the whole weight matrix before each decode step.  The
 * same section notes that such a kernel works on tensors and does not need the
 * model to come from a GGUF file; this ABI therefore takes plain device
 * pointers.  The section "What is the GGUF file format?" names the block
 * formats (Q4_K_M mixes Q4_K with Q6_K tensors); the page "Show HN: Gemma 4
 * 26B-A4B at up to 100+ tokens/s on a 16 GB Mac" (Architecture section) uses
 * the same product for routed 4-bit experts, and its prefill step, where the
 * GPU expands 4-bit experts to fp16 for a matrix engine, motivates the
 * dequantise-then-matrix-core prefill path.
 *
 * Block formats (public ggml layout; byte offsets inside one block):
 *   GQ_Q4_0:  32 weights, 18 B.  fp16 d @0; 16 quant bytes @2.  Weight j < 16 is
 *             the low nibble of quant byte j, weight j >= 16 the high nibble of
 *             byte j-16.  w = d * (q - 8).
 *   GQ_Q4_K: 256 weights, 144 B.  fp16 d @0, fp16 dmin @2, 12 bytes of eight
 *             6-bit (scale, min) pairs @4, 128 quant bytes @16.  Weight i:
 *             chunk c = i/64 uses quant bytes 32c..32c+31; i%64 < 32 is the low
 *             nibble (sub-block 2c), otherwise the high nibble (sub-block 2c+1).
 *             w = (d * sc) * q - dmin * m.
 *   GQ_Q6_K: 256 weights, 210 B.  128 B low 4-bit parts @0, 64 B high 2-bit
 *             parts @128, 16 int8 scales @192 (one per 16 weights), fp16 d @208.
 *             w = (d * sc) * (q - 32), q in 0..63.
 *   GQ_Q5_K: 256 weights, 176 B.  Q4_K's 16-byte header @0, 32 bytes of fifth
 *             bits @16, Q4_K's 128 quant bytes @48.  Weight i (chunk c = i/64,
 *             j = i%64) has Q4_K's low four bits and, as bit 4, bit 2c + (j >=
 *             32) of fifth-bit byte j % 32.  w = (d * sc) * q - dmin * m, q in
 *             0..31.  (The pages list the Q5_K_M variant in the size table of
 *             "GGUF in transformers" but print no layout; this is ggml's.)
 *
 * Matrix layout: a matrix with N output rows and K inputs is N rows of K/QK
 * consecutive blocks each (QK = 32 or 256), rows back to back with no padding.
 * Activations are row-major [batch][K] (fp32 or bf16); outputs row-major fp32.
 *
 * Conventions shared by every call:
 *  - Every pointer argument except host out-parameters is a DEVICE pointer owned
 *    by the caller; the library never frees or retains it.  Device pointers must
 *    be 16-byte aligned (rows inside a matrix need not be).
 *  - Calls are asynchronous: they enqueue work on `stream` (0 = the default
 *    stream) and return.  Only gq_matvec_id_check waits for the device.
 *  - All arguments are validated on the host before any HIP call.  On an error
 *    nothing is launched and no output is written.
 *  - No C++ exception crosses this boundary.  Launch failures return
 *    GQ_ERR_LAUNCH.
 *  - Calls are re-entrant; the library keeps no mutable global state.
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQ_ABI_VERSION 1

typedef enum { GQ_Q4_0 = 1, GQ_Q4_K = 2, GQ_Q6_K = 3, GQ_Q5_K = 4 } gq_type;

typedef enum { GQ_F32 = 0, GQ_BF16 = 1, GQ_F16 = 2 } gq_dtype;

/* Activations of a gated feed-forward unit (gq_matvec_glu). */
typedef enum { GQ_ACT_SILU = 0, GQ_ACT_GELU_TANH = 1 } gq_act;

typedef enum {
    GQ_OK = 0,
    GQ_ERR_TYPE = 1,        /* unknown block type */
    GQ_ERR_DTYPE = 2,       /* unsupported activation / output element type */
    GQ_ERR_SHAPE = 3,       /* negative size, K not a whole number of blocks, batch/top_k out of range */
    GQ_ERR_NULL = 4,        /* required pointer is NULL */
    GQ_ERR_ALIGN = 5,       /* device pointer not 16-byte aligned */
    GQ_ERR_UNSUPPORTED = 6, /* valid request this build does not implement */
    GQ_ERR_WORKSPACE = 7,   /* workspace missing or too small */
    GQ_ERR_LAUNCH = 8       /* the HIP runtime refused a launch */
} gq_status;

/* ABI version of the loaded library (GQ_ABI_VERSION at build time). */
int gq_abi_version(void);

/* Static, human-readable name of a status code. */
const char* gq_status_str(gq_status s);

/* Host only.  Weights per block and bytes per block of type t
 * (32/18, 256/144, 256/210).  GQ_ERR_TYPE for an unknown t, GQ_ERR_NULL for a
 * NULL out-parameter. */
gq_status gq_block_info(gq_type t, int32_t* elems, int32_t* bytes);

/* Dequantise n_blocks consecutive blocks of type t into out[0 .. n_blocks*QK).
 * The operation is the dequantising fallback that "GGUF in transformers"
 * mentions twice: when no packed kernel is available, and as
 * GgufConfig(dequantize=True) for fine-tuning (section "transformers and
 * llama.cpp").
 *   out_dtype GQ_F32: bit-exact fp32 weights, each formula evaluated with fp32
 *     factors left to right (the only rounding is Q4_K's final subtraction).
 *   GQ_BF16 / GQ_F16: that fp32 value rounded to nearest even.
 * n_blocks == 0 is a no-op.  blocks and out must be 16-byte aligned. */
gq_status gq_dequant(gq_type t, const void* blocks, int64_t n_blocks, void* out,
                     gq_dtype out_dtype, hipStream_t stream);

/* Decode matrix-vector product for a small batch:
 *   y[b][n] = sum_k w[n][k] * x[b][k],  0 <= b < batch, 0 <= n < N.
 * W: packed [N][K/QK] blocks of type t.  x: [batch][K] of x_dtype (GQ_F32 or
 * GQ_BF16).  y: [batch][N] fp32.  1 <= batch <= 16 (GQ_ERR_UNSUPPORTED above;
 * the Gemma 4 26B-A4B Show HN page verifies blocks of up to 16 draft tokens).
 * K must be a multiple of QK and at most 4,194,304 (GQ_ERR_SHAPE otherwise).
 * N == 0 is a no-op; K == 0 writes zeros.
 * Two paths compute it: batch >= 5, Q4_0 / Q4_K / Q5_K at batch 4 with
 * N <= 4 K and at batch 3 with 4 N <= 5 K run on the matrix cores (the
 * measured crossovers); the rest on the packed fp16 dot instructions.
 * Accuracy.  Every weight enters the arithmetic as the exact value of q - z
 * (z its format's zero point) times a power of two, so every product is exact
 * and nothing in the fp32 sums cancels later.  Dot path: activations enter as
 * fp16 after an exact power-of-two scaling per 32 inputs (relative rounding
 * <= 2^-11).  Matrix-core path: bf16 activations enter exactly, fp32 ones as a
 * bf16 pair hi + lo (relative error <= 2^-17).  Sums are fp32.  The result is
 * within 1e-3 * sum_k |w[n][k] * x[b][k]| of the exact product, and a
 * sub-block whose quants all equal the zero point contributes exactly zero.
 * For Q4_K / Q5_K the min term dmin * m * sum(x) is taken once per 32-weight
 * sub-block, so there the same bound holds with sum |w x| replaced by
 * d * sc * sum q |x| + dmin * m * sum |x| over each sub-block -- the same
 * quantity unless d * sc * q and dmin * m nearly cancel for most weights of a
 * sub-block.  On the dot path, a group of 32 activations whose magnitudes
 * span more than 2^28 loses its smallest elements to fp16 subnormals.  Each
 * vector's result depends on that vector and on N, K alone (bit for bit)
 * within one path. */
gq_status gq_matvec(gq_type t, const void* W, int64_t N, int64_t K, const void* x,
                    gq_dtype x_dtype, int32_t batch, float* y, hipStream_t stream);

/* Gated feed-forward unit in one launch: for 0 <= b < batch, 0 <= n < N,
 *   h[b][n] = act(g) * u,  g = sum_k w_gate[n][k] x[b][k],  u = sum_k w_up[n][k] x[b][k].
 * "GGUF in transformers" (section "Reusing ggml's Metal kernels") notes that a
 * specialised kernel can merge several operations; this one merges the gate
 * and up projections with the activation and product between them, so that h
 * can feed the down projection directly.  The two products share the staged
 * activations and each weight byte is read once.
 *   act GQ_ACT_SILU:      act(g) = g / (1 + e^-g)  (SwiGLU, Qwen-style blocks)
 *   act GQ_ACT_GELU_TANH: act(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3)))
 *                         (GeGLU, Gemma-style blocks)
 * W_gate, W_up: packed [N][K/QK] blocks of type t (separate matrices, or the
 * two halves of one [2N] gate|up matrix).  x: [batch][K] of x_dtype (GQ_F32 or
 * GQ_BF16).  h: [batch][N] of h_dtype (GQ_F32, or GQ_BF16 rounded to nearest
 * even).  1 <= batch <= 8 (GQ_ERR_UNSUPPORTED above, and for an unknown act).
 * K limited as for gq_matvec; N == 0 is a no-op; K == 0 writes zeros.
 * Accuracy: g and u as gq_matvec's dot-product path; act in fp32 (expf,
 * tanhf), then one fp32 product (and the bf16 rounding). */
gq_status gq_matvec_glu(gq_type t, const void* W_gate, const void* W_up, int64_t N, int64_t K, const void* x,
                        gq_dtype x_dtype, int32_t batch, gq_act act, void* h, gq_dtype h_dtype,
                        hipStream_t stream);

/* Workspace bytes needed by gq_matvec_id and gq_matvec_id_glu for these sizes
 * (host only): a header, the table of expert groups and, for a weighted
 * product, the per-slot outputs. */
gq_status gq_matvec_id_workspace(int32_t n_experts, int32_t n_tokens, int32_t top_k, int64_t N,
                                 size_t* bytes);

/* Routed-expert product: only the experts chosen for each token are read
 * (ggml-quantization row of the kernel table in "GGUF in transformers").
 * experts: packed [n_experts][N][K/QK] blocks; ids: [n_tokens][top_k] int32
 * expert ids (device).  x: [n_tokens][K] when x_per_slot == 0 (all slots of a
 * token read the token's vector, as gate/up projections do), or
 * [n_tokens][top_k][K] when x_per_slot == 1 (each slot its own vector, as for
 * a down projection).
 *   route_w == NULL: y is [n_tokens][top_k][N],
 *       y[t][j][n] = sum_k w_{ids[t][j]}[n][k] * x_{t,j}[k].
 *   route_w != NULL (fp32 [n_tokens][top_k], device): y is [n_tokens][N],
 *       y[t][n] = sum_j route_w[t][j] * (sum_k w_{ids[t][j]}[n][k] * x_{t,j}[k]),
 *       summed over j in increasing order.
 * The (token, slot) pairs routed to one expert are taken in groups of up to
 * 8, and each group reads the expert's rows once: an expert that receives at
 * most 8 of the call's slots (every expert of an 8-token top-8 step; an
 * 8-token block reads about 29 experts per layer in the Show HN page's
 * "Speculative decoding" section) is read once for all of them.
 * ws: device workspace of at least gq_matvec_id_workspace bytes; its contents
 * need no initialisation.  Each call given ids leaves in ws the table of
 * groups it built from them.  ids may be NULL: the call then uses the table
 * already in ws -- left by gq_route_topk_plan, gq_route_matvec_id_glu or the
 * previous routed call (gq_matvec_id or gq_matvec_id_glu) made with the same ws, n_experts,
 * n_tokens, top_k and ids -- and builds none, so that the products of one
 * layer share one table; ws must still be large enough for this call's N.
 * (Table fields are clamped to their ranges, so a workspace that holds no
 * table gives wrong values but no access out of bounds.)  An id outside
 * [0, n_experts) makes its slot contribute zero and is counted in ws (see
 * gq_matvec_id_check); with ids == NULL, the output rows of such slots are
 * left as they were (a weighted product still leaves them out).  1 <= top_k <= n_experts, n_tokens * top_k <=
 * 1024, x_dtype GQ_F32 or GQ_BF16, K limited as for gq_matvec.  Accuracy as
 * gq_matvec (for route_w != NULL the bound is 1e-3 * sum_j |route_w[t][j]| *
 * sum_k |w * x|). */
gq_status gq_matvec_id(gq_type t, const void* experts, int32_t n_experts, int64_t N, int64_t K,
                       const int32_t* ids, int32_t n_tokens, int32_t top_k, const void* x,
                       gq_dtype x_dtype, int32_t x_per_slot, const float* route_w, float* y,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* gq_matvec_id without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The call allocates nothing: its workspace is an
 * array inside the library, one per GPU, of GQ_NOALLOC_WS_BYTES (8 MiB), held
 * from the first call on that GPU until the process ends.  Arguments,
 * results, limits and accuracy are those of gq_matvec_id with
 * ws = that array; a call whose gq_matvec_id_workspace(n_experts, n_tokens,
 * top_k, N) exceeds GQ_NOALLOC_WS_BYTES returns GQ_ERR_WORKSPACE and launches
 * nothing (e.g. 64 slots allow N up to about 32,000).  Every call on a GPU
 * uses that GPU's one array, which keeps the last call's contents: ids may
 * be NULL (with route_w) to reuse the group table of the previous call of
 * this function on the same GPU, and calls that overlap on one GPU (other
 * streams, other threads) race with each other -- serialise them.  Invalid
 * ids are handled as by gq_matvec_id but their count cannot be read back. */
#define GQ_NOALLOC_WS_BYTES ((size_t)8 << 20)
gq_status gq_matvec_id_noalloc(gq_type t, const void* experts, int32_t n_experts, int64_t N, int64_t K,
                               const int32_t* ids, int32_t n_tokens, int32_t top_k, const void* x,
                               gq_dtype x_dtype, int32_t x_per_slot, const float* route_w, float* y,
                               hipStream_t stream);

/* Routed gated unit: the gate and up products of a routed feed-forward block
 * and the activation between them, in one launch (the routed 4-bit experts of
 * the Architecture section of the Gemma 4 26B-A4B Show HN page; the
 * ggml-quantization row of the kernel table in "GGUF in transformers").
 * experts_gate, experts_up: packed [n_experts][N][K/QK] blocks of type t;
 * ids: [n_tokens][top_k] int32 (device); x: [n_tokens][K] of x_dtype (GQ_F32
 * or GQ_BF16), read by every slot of its token.  For each slot (t, j) with
 * e = ids[t][j]:
 *   h[t][j][n] = act(sum_k gate_e[n][k] x_t[k]) * (sum_k up_e[n][k] x_t[k]),
 * h: [n_tokens][top_k][N] of h_dtype (GQ_F32 or GQ_BF16) -- the per-slot
 * vectors a down projection takes as gq_matvec_id's x with x_per_slot == 1.
 * Each expert's rows of both stacks are read once per group of up to 8 of its
 * slots (so once for all of them when it receives at most 8).
 * act as for gq_matvec_glu.  ws: device workspace of at least
 * gq_matvec_id_workspace bytes for (n_experts, n_tokens, top_k, N), no
 * initialisation needed; an id outside
 * [0, n_experts) gives its slot a zero row of h and is counted in ws (see
 * gq_matvec_id_check).  ids may be NULL to use the table already in ws, as
 * for gq_matvec_id.  Shapes and limits as gq_matvec_id; n_tokens == 0 or
 * N == 0 is a no-op.  Accuracy: g and u as gq_matvec_id, act and the product
 * as gq_matvec_glu. */
gq_status gq_matvec_id_glu(gq_type t, const void* experts_gate, const void* experts_up, int32_t n_experts,
                           int64_t N, int64_t K, const int32_t* ids, int32_t n_tokens, int32_t top_k,
                           const void* x, gq_dtype x_dtype, gq_act act, void* h, gq_dtype h_dtype, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Waits for `stream`, then reports how many ids of the last gq_matvec_id or
 * gq_matvec_id_glu call that used `ws` were outside [0, n_experts). */
gq_status gq_matvec_id_check(const void* ws, hipStream_t stream, int32_t* n_bad_ids);

/* Expert routing ("GGUF in transformers", section "Reusing ggml's Metal
 * kernels", kernel table row "topk": the softmax and the top-k choice in one
 * kernel; the Gemma 4 26B-A4B Show HN page routes 8 of 128 experts per token).
 * logits: fp32 [n_tokens][n_experts] (device).  For each token t:
 *   ids[t][0..top_k-1]: the experts of the top_k largest logits, in
 *     decreasing logit order; among equal logits the lower id comes first
 *     (-0 and +0 are equal).  Bit-exact: the choice compares the fp32 logits.
 *   weights[t][j] = exp(l[ids[t][j]] - l[ids[t][0]]) / sum_i exp(l[ids[t][i]] - l[ids[t][0]]),
 *     the softmax over the selected logits (equal to the softmax over all
 *     experts renormalised over the selected ones), in fp32: within
 *     (top_k + 8) * 2^-24 of the exact value.
 * ids: int32 [n_tokens][top_k], weights: fp32 [n_tokens][top_k] (device),
 * ready to be passed to gq_matvec_id as ids and route_w.
 * 1 <= top_k <= n_experts; n_experts <= 4096 and top_k <= 64
 * (GQ_ERR_UNSUPPORTED beyond).  n_tokens == 0 is a no-op.  NaN logits leave
 * ids distinct and in range but their order unspecified; weights are NaN when
 * the largest selected logit is infinite. */
gq_status gq_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                        int32_t* ids, float* weights, hipStream_t stream);

/* gq_route_topk and the routed products' table of expert groups in one
 * launch: ids and weights exactly as gq_route_topk computes them, and in ws
 * the table that gq_matvec_id / gq_matvec_id_glu would build from those ids,
 * so that the products of the layer can all be called with ids == NULL (the
 * topk kernel row of "GGUF in transformers" feeding its routed-expert
 * product).  ws: at least gq_matvec_id_workspace(n_experts, n_tokens, top_k,
 * N) bytes for the largest N of the products that will use it (0 for the
 * table alone).  n_tokens * top_k <= 1024; other limits as gq_route_topk. */
gq_status gq_route_topk_plan(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                             int32_t* ids, float* weights, void* ws, size_t ws_bytes, hipStream_t stream);

/* gq_route_topk_plan followed by gq_matvec_id_glu with ids == NULL, in one
 * launch where it fits: the router of a routed feed-forward block (kernel
 * table row "topk" of "GGUF in transformers", section "Reusing ggml's Metal
 * kernels") and its gated unit (the routed 4-bit experts of the Architecture
 * section of the Gemma 4 26B-A4B Show HN page).  logits: fp32
 * [n_tokens][n_experts]; ids, weights: [n_tokens][top_k] as gq_route_topk
 * writes them (bit-identical); h: [n_tokens][top_k][N] as gq_matvec_id_glu
 * computes it from those ids (bit-identical); ws: at least
 * gq_matvec_id_workspace(n_experts, n_tokens, top_k, N') bytes, N' the
 * largest N of this call and the products that follow, which may then be
 * called with ids == NULL (a down projection by gq_matvec_id with
 * x_per_slot == 1 and route_w = weights).  The one-launch form needs
 * n_tokens * top_k <= 64, n_experts <= 128 and n_tokens * top_k <= n_experts
 * (one top-8 step of up to 8 tokens over 128 experts); every workgroup of it
 * routes all the tokens itself.  Other sizes take the two launches.  Limits,
 * x_dtype, h_dtype and act as gq_route_topk and gq_matvec_id_glu; N == 0
 * routes only; n_tokens == 0 is a no-op. */
gq_status gq_route_matvec_id_glu(gq_type t, const void* experts_gate, const void* experts_up, int32_t n_experts,
                                 int64_t N, int64_t K, const float* logits, int32_t n_tokens, int32_t top_k,
                                 int32_t* ids, float* weights, const void* x, gq_dtype x_dtype, gq_act act, void* h,
                                 gq_dtype h_dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/* Prefill product Y[m][n] = sum_k X[m][k] * w[n][k] for 0 <= m < M, 0 <= n < N.
 * X: [M][ldx] of x_dtype (row stride ldx >= K elements); Y: [M][ldy] fp32
 * (ldy >= N).  Weight tiles are dequantised to bf16 in LDS and multiplied on
 * the matrix cores with fp32 accumulation.  Every block type is accepted (a
 * Q4_K_M layer mixes Q4_K and Q6_K tensors); x_dtype must be GQ_BF16
 * (GQ_ERR_UNSUPPORTED otherwise).  K must be a multiple of the type's QK and
 * at most 4,194,304, and ldx below 4,194,304 (GQ_ERR_SHAPE otherwise: 256 rows
 * of X are addressed through one buffer resource whose span stays below 2^31
 * bytes); ldx * 2 and ldy * 4 must be multiples of 16 (GQ_ERR_ALIGN).
 * M == 0 or N == 0 is a no-op. */
gq_status gq_matmul(gq_type t, const void* W, int64_t N, int64_t K, const void* X,
                    gq_dtype x_dtype, int64_t M, int64_t ldx, float* Y, int64_t ldy,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
