/*
 * nf4moe.h -- C ABI of libnf4moe.so: the routed Mixture-of-Experts expert layer
 * computed directly on 4-bit packed weights, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one described on the page "How do I run a grouped GEMM
 * directly on NF4 packed MoE expert weights, without dequantizing to bf16
 * first?" (sections "Why it happens", "Smallest correct example", "Supported
 * scope") and in the grouped-nf4-gemm PKG-INFO (intro, "Try it on CPU right
 * now", "The MXFP4 native-byte lane"): one grouped GEMM over an expert-major
 * stack of 4-bit codes, each code decoded through a 16-entry codebook in
 * registers, block-scaled, accumulated in fp32, with no bf16 copy of any expert
 * written to memory. This library also does the routing (router logits, top-k,
 * grouping) and the router-weighted combine, so one call runs a whole layer.
 *
 * Conventions for every entry point
 *  - Pointers marked "device" are HIP device memory owned by the caller. The
 *    library allocates no device memory and keeps no state between calls; the
 *    scratch an operation needs is a caller-provided workspace.
 *  - stream: a hipStream_t (NULL = the null stream). All device work is
 *    enqueued asynchronously on it; no call synchronises the host, so the
 *    forward pass can be captured in a HIP graph.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    an error nothing is enqueued, the status is returned and
 *    nf4moe_last_error() (thread-local) describes it.
 *  - Element offsets are computed in 64 bits everywhere, so expert stacks may
 *    exceed 2 GiB (the pages' "Limitations": every expert-base offset int64).
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Device faults surface as NF4MOE_ERR_HIP at the caller's next stream
 *    synchronisation; nothing is retried or recovered.
 *
 * Formats (the pages' layouts, "Supported scope" and "The MXFP4 native-byte lane")
 *  NF4_B64   codes uint8 [.., N, K/2], two codes per byte, HIGH nibble = even k;
 *            scales float32 absmax [.., N, K/64]; value = codebook[code] * absmax
 *            rounded once to fp32. K % 64 == 0. The 16 codebook values are the
 *            NormalFloat construction (see nf4moe_codebook).
 *  MXFP4_B32 codes uint8 [.., N, K/2], LOW nibble = even k, OCP e2m1 values;
 *            scales uint8 e8m0 [.., N, K/32]; value = e2m1(code) * 2^(e8m0-127),
 *            e8m0 = 255 is NaN. K % 32 == 0.
 *  NF4_B64_BF16ABS  as NF4_B64 with the absmax stored as bf16 bits, uint16
 *            [.., N, K/64]; the decode widens it to fp32 first.
 */
#ifndef NF4MOE_H
#define NF4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NF4MOE_OK = 0,
  NF4MOE_ERR_INVALID_ARG = 1, /* bad size, null or misaligned pointer, bad enum */
  NF4MOE_ERR_UNSUPPORTED = 2, /* valid request outside what this library supports */
  NF4MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required     */
  NF4MOE_ERR_HIP = 4          /* a HIP runtime call failed (launch, device query) */
} nf4moe_status_t;

/* Weight formats. NF4_B64_BF16ABS is NF4_B64 with each block's absmax stored
 * as bf16 (2 bytes instead of 4, 5.6 % fewer bytes per weight row): the
 * experts4bit-qlora page's bf16 absmax, lossless for bf16-source weights
 * because a block maximum of bf16 values is a bf16 value ("The one ordering
 * trap" paragraph before it: --absmax-dtype bf16). Codes, nibble order and the
 * decode c[code] * absmax (one fp32 product) are those of NF4_B64. */
typedef enum {
  NF4MOE_FMT_NF4_B64 = 0,
  NF4MOE_FMT_MXFP4_B32 = 1,
  NF4MOE_FMT_NF4_B64_BF16ABS = 2
} nf4moe_format_t;
typedef enum { NF4MOE_DT_F32 = 0, NF4MOE_DT_BF16 = 1 } nf4moe_dtype_t;

/* Which grouped-GEMM kernel family runs. AUTO picks from the routed row count
 * known on the host (R = T * top_k): R <= 64 for NF4 and R <= 48 for MXFP4
 * (with H, I <= 4096) runs the bandwidth-bound decode kernels, larger R the
 * MFMA kernels (tiles of up to 64 rows of one expert when the groups average
 * at most 48 rows, else up to 128; each tile runs a 128-, 64- or 32-row body
 * by its row count). The other values force one family (for A/B measurement
 * and tests); the result must satisfy the same tolerance. */
typedef enum { NF4MOE_PATH_AUTO = 0, NF4MOE_PATH_SMALL_M = 1, NF4MOE_PATH_MFMA = 2 } nf4moe_path_t;

/* nf4moe_auto_path -- the family AUTO runs for a grouped GEMM of R routed rows
 * whose K (for a forward: max(H, I)) is K_max, in format fmt: NF4MOE_PATH_SMALL_M
 * or NF4MOE_PATH_MFMA. Host only; no errors. */
int32_t nf4moe_auto_path(nf4moe_format_t fmt, int64_t R, int64_t K_max);

/* The gate_up epilogue. SWIGLU: h = silu(g) * u, silu(g) = g / (1 + exp(-g)).
 * CLAMPED: the gpt-oss expert form the experts4bit-qlora page names without
 * defining it ("Scope": MXFP4 experts with per-expert biases and a clamped-GLU
 * epilogue); read here as g' = min(g, limit), u' = clamp(u, -limit, limit),
 * h = (u' + 1) * g' / (1 + exp(-alpha * g')), alpha and limit given by the
 * caller (gpt-oss publishes alpha = 1.702, limit = 7). */
typedef enum { NF4MOE_GLU_SWIGLU = 0, NF4MOE_GLU_CLAMPED = 1 } nf4moe_glu_t;

/* One MoE layer. All pointers are device memory owned by the caller.
 * The fused gate_up stack is [E, 2I, H] (rows [0, I) gate, [I, 2I) up, or with
 * glu_interleaved rows 2c gate and 2c + 1 up) and the down stack [E, H, I] --
 * the experts4bit-qlora README's fused expert-stack convention ("Quickstart")
 * -- each stored in `fmt`. Optional per-expert biases (the gpt-oss form):
 * b13 [E, 2I] fp32 added to the gate_up product row by row (same row order as
 * w13) before the epilogue, b2 [E, H] fp32 added to each expert's down output
 * before its routing weight. A zero-filled struct tail (glu 0, biases NULL)
 * is the plain SwiGLU layer. */
typedef struct {
  nf4moe_format_t fmt;
  int32_t E;           /* experts, 1..1024                                   */
  int32_t H;           /* hidden size (K of gate_up, N of down)              */
  int32_t I;           /* intermediate size (K of down)                      */
  int32_t top_k;       /* experts per token, 1..min(E, 32)                   */
  int32_t renormalize; /* 1: softmax over the k selected logits; 0: full softmax at the ids */
  int32_t path;        /* nf4moe_path_t                                      */
  const uint8_t *w13;  /* [E, 2I, H/2] codes                                  */
  const void *w13_scale; /* NF4: float [E, 2I, H/64]; MXFP4: uint8 [E, 2I, H/32] */
  const uint8_t *w2;   /* [E, H, I/2] codes                                   */
  const void *w2_scale;  /* NF4: float [E, H, I/64];  MXFP4: uint8 [E, H, I/32]  */
  const float *router_w; /* [E, H] fp32                                        */
  const float *router_b; /* [E] fp32 added to the logits, or NULL              */
  int32_t glu;           /* nf4moe_glu_t                                        */
  float glu_alpha;       /* CLAMPED only: > 0, finite                           */
  float glu_limit;       /* CLAMPED only: > 0, finite                           */
  int32_t glu_interleaved; /* 0: gate rows [0, I), up [I, 2I); 1: gate 2c, up 2c + 1 */
  const float *b13;      /* [E, 2I] fp32 or NULL                                */
  const float *b2;       /* [E, H] fp32 or NULL                                 */
} nf4moe_layer_t;

/* ---------------------------------------------------------------------------
 * nf4moe_quantize -- fp32 weights [rows, K] (device, row-major) -> packed codes
 * [rows, K/2] + scales (device). Off the timed path.
 * NF4 (grouped-nf4-gemm PKG-INFO, "Try it on CPU right now", block 1): absmax =
 *   max |w| over each 64-block, stored fp32; code = the exact nearest codebook
 *   value to w/absmax (decided by fp64 midpoint comparisons), ties to the lower
 *   code; an all-zero block stores absmax 0 and code 7 (0.0).
 * MXFP4 (same section, block 2; OCP MX v1.0): X = floor(log2 amax) - 2 clamped
 *   to [-127, 127], e8m0 = X + 127; code = nearest e2m1 of w / 2^X, ties to the
 *   even code, saturating at 6; code bit 3 = the input's sign bit.
 * NF4_B64_BF16ABS: the NF4 rule with the block absmax rounded up to the nearest
 *   bf16 value before the codes are chosen (no change when it is one, as for
 *   bf16-source weights: then codes and decoded values equal NF4_B64's); scales
 *   uint16 bf16 bits [rows, K/64].
 * Errors: INVALID_ARG for null pointers, rows < 0, K not a multiple of the block,
 * packed not 4-byte aligned. rows == 0 is a no-op. Non-finite inputs give
 * unspecified codes.
 * ------------------------------------------------------------------------- */
nf4moe_status_t nf4moe_quantize(nf4moe_format_t fmt, const float *w, int64_t rows, int64_t K,
                                uint8_t *packed, void *scale, void *stream);

/* nf4moe_dequantize -- packed codes + scales (device) -> fp32 [rows, K] (device).
 * A test export of the decode the GEMM kernels perform in registers: every
 * element equals the reference decode bit for bit ("Expected result": the
 * per-element decode is identical). Errors as for nf4moe_quantize. */
nf4moe_status_t nf4moe_dequantize(nf4moe_format_t fmt, const uint8_t *packed, const void *scale,
                                  int64_t rows, int64_t K, float *w_out, void *stream);

/* nf4moe_absmax_to_bf16 -- the bf16 absmax cast of an existing NF4_B64 scale
 * array (experts4bit-qlora page, the --absmax-dtype bf16 paragraph: the cast is
 * taken only where it is exact and is refused otherwise). absmax fp32 [n] ->
 * out uint16 bf16 bits [n], each rounded up to the nearest bf16 value when it
 * is not one; *n_inexact (device int32, zeroed by the caller) receives the
 * number of such entries: a caller refuses the cast unless it reads 0, and the
 * codes stay valid only then. Asynchronous on `stream`. Errors: INVALID_ARG for
 * n < 0, NULL or misaligned pointers; n == 0 is a no-op. */
nf4moe_status_t nf4moe_absmax_to_bf16(const float *absmax, int64_t n, uint16_t *out, int32_t *n_inexact,
                                      void *stream);

/* nf4moe_router_workspace_bytes -- workspace that lets nf4moe_router_logits use
 * the matrix cores for T tokens (the partial sums over 8 chunks of H: 4 * S * T
 * * E bytes, S = min(8, H / 16)); 0 for T < 1, E < 1, or H not a positive
 * multiple of 16 (the vector path needs none). */
size_t nf4moe_router_workspace_bytes(int32_t T, int32_t E, int32_t H);

/* nf4moe_router_logits -- logits[t, e] = sum_h x[t, h] * router_w[e, h] (+ router_b[e]),
 * x bf16 [T, H], router_w fp32 [E, H], optional router_b fp32 [E], logits fp32
 * [T, E] (all device); fp32-accurate accumulation. The first step of the routed
 * layer (the router, outside the kernel on the pages' "Why it happens" dataflow,
 * inside this library). ws (device, caller-owned, 256-byte aligned) may be NULL.
 * With ws and H % 16 == 0 the product runs on the matrix cores: x exact in
 * bf16, each weight as the exact sum of three bf16 parts (weights of normal
 * range), fp32 partial sums over S chunks of H added in chunk order, then the
 * bias; these are the bits nf4moe_moe_forward routes on when it takes the MFMA
 * path. Without ws: the vector ALUs (one workgroup per expert, a token's sum in
 * the same order for every T, up to 256 tokens; a tiled kernel above). Either
 * way a token's logits carry the same bits whatever the other tokens.
 * Errors: INVALID_ARG for T < 0, E outside 1..1024, H <= 0 or H % 8, null or
 * misaligned pointers; WORKSPACE for a non-NULL ws (H % 16 == 0) smaller than
 * nf4moe_router_workspace_bytes(T, E, H). */
nf4moe_status_t nf4moe_router_logits(const uint16_t *x, int32_t T, int32_t H,
                                     const float *router_w, const float *router_b, int32_t E,
                                     float *logits, void *ws, size_t ws_bytes, void *stream);

/* nf4moe_route_workspace_bytes -- workspace nf4moe_route_permute needs. */
size_t nf4moe_route_workspace_bytes(int32_t T, int32_t E, int32_t top_k);

/* nf4moe_route_permute -- top-k + softmax and grouping by expert, from given fp32
 * logits [T, E] (device). Outputs (device):
 *   topk_ids [T, k] int32: the k largest logits per token, ordered by (logit
 *     descending, expert id ascending);
 *   topk_w [T, k] fp32: renormalize=1 -> exp(L_j - L_0) / sum_j' exp(L_j' - L_0);
 *     renormalize=0 -> softmax over all E at the selected ids;
 *   expert_offsets [E+1] int32: rows of expert e are [off[e], off[e+1]);
 *   sorted_slots [T*k] int32: slots s = t*k + j grouped by expert, ascending s
 *     within an expert (a stable counting sort).
 * This is the pages' "a_cat sorted by expert, sizes + expert_ids" grouping
 * ("Why it happens" dataflow), done on the device with no host sync.
 * ids, offsets and slots are exact integers (bit-identical to a stable sort of
 * the same fp32 logits). Non-finite logits: the order compares IEEE total-order
 * keys with -0 taken as +0 (+inf and -inf in place, a positive NaN above +inf,
 * a negative NaN below -inf; ties still go to the lower id), so every token
 * always gets k distinct experts and every index stays in range; the weights
 * of a token with a NaN or infinite logit are unspecified (NaN in practice).
 * Errors: INVALID_ARG (T < 0, E outside 1..1024, top_k outside 1..min(E, 32),
 * null pointers), WORKSPACE (ws_bytes too small). */
nf4moe_status_t nf4moe_route_permute(const float *logits, int32_t T, int32_t E, int32_t top_k,
                                     int32_t renormalize, int32_t *topk_ids, float *topk_w,
                                     int32_t *expert_offsets, int32_t *sorted_slots,
                                     void *ws, size_t ws_bytes, void *stream);

/* nf4moe_gemm_workspace_bytes -- workspace nf4moe_grouped_gemm needs. */
size_t nf4moe_gemm_workspace_bytes(int32_t G, int32_t R);

/* nf4moe_grouped_gemm -- the pages' gemm_4bit_grouped ("Smallest correct example",
 * "Supported scope"): c[r, :] = a[row(r), :] . W[e(r)]^T over routed groups,
 * W decoded from 4-bit codes in registers, fp32 accumulation.
 *   a        bf16 [a_rows, K] (device, 16-byte aligned rows: K % 8 == 0)
 *   a_row_of int32 [R] (device) or NULL: row r reads a[a_row_of[r]] (gather),
 *            NULL means a[r] (then a_rows >= R). Indices outside [0, a_rows)
 *            are a caller error; the kernels clamp them into that range, so
 *            such a row's output is unspecified but no read leaves a
 *   B, B_scale  expert stack [E, N, K/2] + scales in `fmt` (device)
 *   G, group_offsets int32 [G+1] (device): group g = rows [off[g], off[g+1]),
 *            off[0] = 0, non-decreasing, off[G] = R (the caller guarantees this;
 *            kernels clamp to R so a violation cannot write out of bounds)
 *   group_experts int32 [G] (device) or NULL (group g uses expert g); values in [0, E)
 *   c        [R, N] fp32 or bf16 (RNE) in group order (device)
 *   path     nf4moe_path_t
 * Empty groups are allowed. Errors: INVALID_ARG (K or N not a multiple of the
 * format block / of 64, null pointers, R < 0, G outside 1..65536), WORKSPACE. */
nf4moe_status_t nf4moe_grouped_gemm(nf4moe_format_t fmt, const uint16_t *a, const int32_t *a_row_of,
                                    int32_t a_rows, const uint8_t *B, const void *B_scale, int32_t E,
                                    int64_t N, int64_t K, int32_t G, const int32_t *group_offsets,
                                    const int32_t *group_experts, int32_t R, void *c,
                                    nf4moe_dtype_t c_dtype, int32_t path, void *ws, size_t ws_bytes,
                                    void *stream);

/* nf4moe_grouped_dgrad -- the pages' dgrad_4bit_grouped (grouped-nf4-gemm page,
 * "Training: the backward is a kernel too"): the input gradient of
 * nf4moe_grouped_gemm, da[r, :] = dc[r, :] . W[e(r)] over routed groups, W the
 * [N, K] weights decoded from 4-bit codes exactly as the forward decodes them
 * (never written out), fp32 accumulation.
 *   dc       bf16 [R, N] gradient of the GEMM output, rows in group order (device,
 *            16-byte aligned)
 *   B, B_scale  expert stack [E, N, K/2] + scales in `fmt` (device)
 *   G, group_offsets, group_experts  as nf4moe_grouped_gemm (empty groups allowed)
 *   da       [R, K] fp32 or bf16 (RNE), same row order (device)
 *   ws       nf4moe_gemm_workspace_bytes(G, R) bytes, 256-byte aligned (device)
 * Matrix-core kernel for every R (tiles of 128 rows x 128 columns).
 * Errors: INVALID_ARG (K not a multiple of the format block, bad sizes, null or
 * misaligned pointers), UNSUPPORTED (N % 64 != 0), WORKSPACE. */
nf4moe_status_t nf4moe_grouped_dgrad(nf4moe_format_t fmt, const uint16_t *dc, const uint8_t *B,
                                     const void *B_scale, int32_t E, int64_t N, int64_t K, int32_t G,
                                     const int32_t *group_offsets, const int32_t *group_experts,
                                     int32_t R, void *da, nf4moe_dtype_t da_dtype, void *ws,
                                     size_t ws_bytes, void *stream);

/* nf4moe_workspace_bytes -- workspace nf4moe_moe_forward needs for T <= T_max. */
size_t nf4moe_workspace_bytes(const nf4moe_layer_t *layer, int32_t T_max);

/* nf4moe_moe_forward -- one routed MoE layer: router logits, top-k + softmax,
 * grouping by expert, grouped gate_up GEMM with in-register decode, SwiGLU
 * (silu(gate) * up), grouped down GEMM, and the router-weighted combine
 * out[t] = bf16_RNE( sum_j w[t, j] * y[t*k + j] ) summed in fp32. The pages'
 * moe_layer_forward "gate -> GLU -> down" (grouped-nf4-gemm PKG-INFO, "The NVMe
 * tier") plus the routing and combine the pages leave upstream.
 *   x   bf16 [T, H] (device, 16-byte aligned, H % 64 == 0)
 *   out bf16 [T, H] (device)
 *   topk_ids_out [T, k] int32 / topk_w_out [T, k] fp32: optional copies of the
 *   routing decision (device, may be NULL).
 * The gate_up epilogue is SwiGLU, or with layer->glu the clamped GLU with the
 * layer's biases (see nf4moe_glu_t). Intermediates (h, partial products) stay
 * fp32; no bf16 expert weight is written anywhere.
 * Non-finite input (NaN or inf in x, the weights or the router): routing keeps
 * the order of nf4moe_route_permute (k distinct in-range experts per token,
 * whichever kernel routes), so no index leaves its buffer; the outputs of the
 * affected tokens are then unspecified.
 * Row-count invariance (the pages' STATUS page, kernel section): on the small-M
 * path (AUTO picks it for T * top_k <= 64, 48 for MXFP4) a token's outputs and routing carry
 * the same bits whatever the other tokens of the call, for every T; on the
 * MFMA path, among calls of up to 16 tokens (routed on the vector router's
 * logits) and among calls of more than 16 (the matrix-core router's); across
 * these they differ in summation order.
 * Errors: INVALID_ARG (layer fields, sizes, pointers), WORKSPACE (ws_bytes <
 * nf4moe_workspace_bytes(layer, T)). T == 0 is a no-op. */
nf4moe_status_t nf4moe_moe_forward(const nf4moe_layer_t *layer, const uint16_t *x, int32_t T,
                                   uint16_t *out, int32_t *topk_ids_out, float *topk_w_out,
                                   void *ws, size_t ws_bytes, void *stream);

/* nf4moe_moe_forward_noalloc -- nf4moe_moe_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument; the scratch is a
 * library-owned device array of NF4MOE_NOALLOC_SCRATCH_BYTES (32 MiB) that each
 * GPU the library runs on holds until the process ends, looked up on the
 * first call on that device. The call allocates nothing and uses the scratch
 * of the device current on the calling thread (the stream must belong to it).
 * Same kernels and the same results, bit for bit, as nf4moe_moe_forward with a
 * workspace; nothing in the scratch has to start at zero.
 * Limit: layers and token counts with nf4moe_workspace_bytes(layer, T) <=
 * NF4MOE_NOALLOC_SCRATCH_BYTES (an OLMoE-1B-7B-shaped layer, E=64, top_k=8,
 * H=2048, I=1024, up to 333 tokens); larger calls return WORKSPACE and enqueue
 * nothing.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents: calls on one stream are ordered, but calls that can overlap on one
 * GPU (several streams or threads) race and must be serialised by the caller.
 * The scratch address lookup is a runtime query, not a stream operation; a
 * caller that captures this call into a graph can make one eager call on each
 * device first so that the capture holds kernel launches only.
 * Errors as for nf4moe_moe_forward. */
#define NF4MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
nf4moe_status_t nf4moe_moe_forward_noalloc(const nf4moe_layer_t *layer, const uint16_t *x, int32_t T,
                                           uint16_t *out, int32_t *topk_ids_out, float *topk_w_out,
                                           void *stream);

/* nf4moe_moe_forward_profiled -- nf4moe_moe_forward (same kernels, same result,
 * no topk copies) that also uses six caller-created timing HIP events
 * (hipEvent_t, hipEventDefault flags) on `stream`: events[0] is recorded before
 * the router, events[1] after routing + grouping, events[2] after the gate_up +
 * SwiGLU kernel, events[3] after the down projection and combine; events[4] and
 * events[5] are handed to the gate_up kernel's launch (hipExtLaunchKernelGGL)
 * and so carry that kernel's own start and end times. For measurement. Errors
 * as for nf4moe_moe_forward, plus INVALID_ARG for a NULL events array. */
nf4moe_status_t nf4moe_moe_forward_profiled(const nf4moe_layer_t *layer, const uint16_t *x,
                                            int32_t T, uint16_t *out, void *ws, size_t ws_bytes,
                                            void *stream, void *const *events);

/* nf4moe_stream_read -- a measurement aid, not part of the layer: one launch
 * that reads `bytes` bytes of `buf` (device, 16-byte aligned, bytes a positive
 * multiple of 16) once with 16-byte loads, loads_per_thread (1, 2, 4, 8 or 16)
 * of them per thread of 256-thread workgroups, and writes one 32-bit XOR per
 * workgroup to sink (device, nf4moe_stream_read_sink_words(bytes,
 * loads_per_thread) words). Its duration gives the plain HBM read rate of a
 * single launch of that size, the measured ceiling the decode kernels are set
 * beside. Errors: INVALID_ARG for a bad size or loads_per_thread, NULL or
 * misaligned pointers; UNSUPPORTED past 2^31 workgroups. */
int64_t nf4moe_stream_read_sink_words(int64_t bytes, int32_t loads_per_thread);
nf4moe_status_t nf4moe_stream_read(const void *buf, int64_t bytes, int32_t loads_per_thread, uint32_t *sink,
                                   void *stream);

/* nf4moe_mfma_peak -- a measurement aid, not part of the layer: one launch of
 * `workgroups` 512-thread workgroups in which every wave runs `iters` rounds of
 * 8 independent bf16 MFMAs (32x32x16) on pseudo-random finite register
 * operands, with no memory traffic; each thread writes one float to sink
 * (device, workgroups * 512 floats). nf4moe_mfma_peak_flops(workgroups,
 * iters) gives the launch's flops (0 for invalid arguments); flops over the
 * launch's duration is the bf16 matrix-core rate the GPU sustains under full
 * load, the measured ceiling beside the published dense peak. Errors:
 * INVALID_ARG for workgroups outside 1..2^20, iters <= 0, a NULL or misaligned
 * sink. */
int64_t nf4moe_mfma_peak_flops(int32_t workgroups, int32_t iters);
nf4moe_status_t nf4moe_mfma_peak(int32_t workgroups, int32_t iters, float *sink, void *stream);

/* nf4moe_codebook -- host copy of the 16 fp32 decode values the kernels use for
 * `fmt` (index = 4-bit code). No device access. Returns INVALID_ARG for a bad fmt
 * or NULL out. */
nf4moe_status_t nf4moe_codebook(nf4moe_format_t fmt, float out[16]);

/* Human-readable name of a status; never NULL. */
const char *nf4moe_status_string(nf4moe_status_t st);

/* Thread-local description of this thread's last non-OK status ("" if none). */
const char *nf4moe_last_error(void);

/* Library version string. */
const char *nf4moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NF4MOE_H */
