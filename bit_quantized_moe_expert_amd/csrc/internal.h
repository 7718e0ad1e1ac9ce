// Host-side declarations shared by the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace nf4moe {

constexpr int kChunk = 256;        // routed slots per grouping workgroup
constexpr int kMfmaBM = 128;       // rows (tokens) per MFMA tile
constexpr int kMaxTopK = 32;
constexpr int kMaxE = 1024;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

// Routing results and grouping scratch, all device memory.
struct RouteBufs {
  int32_t *topk_ids = nullptr;   // [T, k]
  float *topk_w = nullptr;       // [T, k]
  int32_t *expert_offsets = nullptr;  // [E + 1]
  int32_t *sorted_slots = nullptr;    // [R]
  int32_t *slot_pos = nullptr;        // [R] inverse of sorted_slots
  int32_t *chunk_hist = nullptr;      // [E, nchunks] expert-major
  int32_t *grp_expert = nullptr;      // [max groups] compacted non-empty groups
  int32_t *grp_row0 = nullptr;
  int32_t *grp_rows = nullptr;
  int32_t *counters = nullptr;        // [0] groups, [1] tiles, [2] / [3] class 0 / 1 tiles
  int4 *tiles = nullptr;              // [2][max tiles] (expert, row0, rows, group rows): by group, by class
};

hipError_t launch_quantize(int fmt, const float *w, int64_t rows, int64_t K, uint8_t *packed,
                           void *scale, hipStream_t s);
hipError_t launch_dequantize(int fmt, const uint8_t *packed, const void *scale, int64_t rows,
                             int64_t K, float *out, hipStream_t s);
hipError_t launch_absmax_bf16(const float *a, int64_t n, uint16_t *out, int32_t *inexact, hipStream_t s);

// Router logits. launch_router_rows: one workgroup per expert (and 32-token
// chunk), each token's sum in the same order for every T (the small-M path's
// router). launch_router_partials: the matrix-core router, H split into
// router_split(H) chunks of router_chunk(H) (H % 16 == 0), writing the partial
// sums P[s][t][e] (router_partials_bytes); a token's partials depend on its
// own row only. launch_router_logits: logits [T, E] from the partials
// (summed in chunk order, then the bias) when `partials` is given, else from
// the rows kernel up to kRowsLogitsMaxT tokens and an fp32 tiled kernel above.
constexpr int kRouterSplit = 8;
// The MFMA path routes up to this many tokens on the rows kernel (router +
// one-workgroup top-k and grouping: two launches; measured at 16 Qwen3-shaped
// tokens, 17 us of routing against 23 us for the matrix-core router, its
// partial sums and the same grouping); above it, on the matrix-core router.
constexpr int kMfmaRowsRouterMaxT = 16;
constexpr int kRowsLogitsMaxT = 256;
int router_split(int H);
int router_chunk(int H);
size_t router_partials_bytes(int T, int E, int H);
hipError_t launch_router_rows(const uint16_t *x, int T, int H, const float *W, const float *b, int E,
                              float *logits, hipStream_t s);
hipError_t launch_router_partials(const uint16_t *x, int T, int H, const float *W, int E, float *P,
                                  hipStream_t s);
hipError_t launch_router_logits(const uint16_t *x, int T, int H, const float *W, const float *b,
                                int E, float *logits, float *partials, hipStream_t s);
// top-k + softmax, then grouping. Fills every RouteBufs field. From given
// logits [T, E], or from router partials (S of them, T * E apart, summed in
// order, then + bias).
hipError_t launch_route(const float *logits, int T, int E, int k, int renorm, const RouteBufs &rb,
                        int bm, hipStream_t s);
hipError_t launch_route_partials(const float *partials, int S, const float *bias, int T, int E, int k,
                                 int renorm, const RouteBufs &rb, int bm, hipStream_t s);
// Fill n int32 with v (a kernel, so the sequence stays graph-capturable).
hipError_t launch_fill_i32(int32_t *p, int n, int v, hipStream_t s);
// Groups and tiles from caller-given group offsets / experts.
hipError_t launch_groups_from_offsets(const int32_t *goff, const int32_t *gexp, int G, int R,
                                      int E, const RouteBufs &rb, int bm, hipStream_t s);

// Small-M (bandwidth-bound) kernels.
enum Epi { EPI_SWIGLU = 0, EPI_PLAIN_F32 = 1, EPI_PLAIN_BF16 = 2, EPI_SLOT = 3 };
struct GemmArgs {
  int fmt;
  const void *a;            // bf16 [*, K] (a_is_f32 = 0), fp32 [*, K] (1), 32-bit
  int a_is_f32;             //   (bf16 hi, bf16 lo) pairs [*, K] (2: MFMA path only), or
                            //   the e4m3 split of launch_e4m3_split (3: MXFP4 MFMA SwiGLU only)
  const int32_t *a_row_of;  // row r reads a[a_row_of[r]] or, with a_div > 1, a[a_row_of[r] / a_div]
  int a_div;
  int a_rows;               // rows of a: a gathered row index is clamped into [0, a_rows)
  const uint8_t *B;         // [E, N, K/2]
  const void *B_scale;
  int64_t N, K;             // N = weight rows (2I for SwiGLU), K
  int R;                    // rows of the routed problem
  const int32_t *grp_expert, *grp_row0, *grp_rows, *n_grp;  // device group list
  int max_grp;
  const int4 *tiles;        // MFMA path: (expert, row0, rows, rows of the whole group)
  const int32_t *n_tiles;
  int max_tiles;
  int epi;
  void *c;                  // SwiGLU: fp32 [R, N/2]; plain: [R, N]; slot: fp32 [R_slots, N]
  int c_split;              // MFMA SwiGLU: write h as 32-bit (bf16 hi, bf16 lo) pairs
  const int32_t *slot_of;   // EPI_SLOT: row r -> slot
  const float *slot_w;      // EPI_SLOT: weight of slot
  // One-token routing folded into the gate_up kernel: when route_logits is set
  // (T = 1, E <= 128), every workgroup ranks the E logits itself and takes the
  // blockIdx.y-th selected expert (ascending id); workgroup (0, 0) also writes
  // the routing results into route_out for the kernels that follow.
  const float *route_logits;
  int route_E, route_k, route_renorm;
  RouteBufs route_out;
  // Optional timing: when set, the kernel is launched with these two HIP
  // events, which take the kernel's own start and end timestamps.
  void *ev_start, *ev_stop;
  // EPI_SWIGLU: glu 0 = silu(g) * u, 1 = clamped GLU (glu_alpha, glu_limit);
  // glu_inter: gate / up weight rows 2c, 2c + 1 instead of c, c + N/2.
  int glu;
  float glu_alpha, glu_limit;
  int glu_inter;
  // Per-expert bias [E, N] added to the product (by weight row) before the
  // epilogue: SwiGLU before the activation, slot before the routing weight.
  const float *bias;
  // MFMA path: rows per tile of the tile table (128, or 64 for routed batches
  // with few rows per expert; 0 means 128). Each workgroup runs a 64-row body
  // for a tile of at most 64 rows.
  int tile_rows;
};

// Rows per MFMA tile for R routed rows over at most G groups: 64-row tiles
// when the groups average at most 48 rows, else 128. More, shorter tiles put
// more workgroups on the chip when a batch has few rows per expert (measured:
// Qwen3-shaped T = 128 / 512 172 / 306 us against 205 / 323 us with 128-row
// tables); with many rows per expert, 128-row tiles decode each weight tile
// half as often. Each tile runs the 128-, 64- or 32-row body by its own row
// count.
inline int mfma_tile_rows(int64_t R, int64_t G) {
  const int64_t groups = R < G ? R : G;
  return (groups > 0 && R <= 48 * groups) ? 64 : 128;
}

// Launch through hipExtLaunchKernelGGL when the arguments carry events.
#define NF4MOE_LAUNCH(G, KERNEL, GRID, BLOCK, STREAM, ...)                                          \
  do {                                                                                            \
    if ((G).ev_start)                                                                             \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, (hipEvent_t)(G).ev_start,             \
                            (hipEvent_t)(G).ev_stop, 0, __VA_ARGS__);                             \
    else                                                                                          \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__);                            \
  } while (0)
hipError_t launch_gemv_grouped(const GemmArgs &g, int ms_hint, hipStream_t s);
// bf16 [rows, K] (K % 32 == 0) -> the block-scaled operand of the MXFP4 MFMA
// kernels: e4m3 planes a1, a2 [rows, K] and e8m0 scales [rows, K / 32], with
// x = 2^(scale - 127) * (a1 + a2).
size_t e4m3_split_bytes(int64_t rows, int K);
hipError_t launch_e4m3_split(const uint16_t *x, int64_t rows, int K, uint8_t *q, hipStream_t s);
hipError_t launch_mfma_grouped(const GemmArgs &g, hipStream_t s);

// Token-centric down projection + combine for a handful of tokens; the same
// bits as the grouped GEMV's slot output followed by launch_combine. Shapes:
// down_combine_supported(I, k).
bool down_combine_supported(int I, int k);
hipError_t launch_gemv_down_combine(int fmt, const float *h, const int32_t *slot_pos,
                                    const int32_t *topk_ids, const float *topk_w, int T, int k,
                                    const uint8_t *w2, const void *w2_scale, const float *b2, int H,
                                    int I, uint16_t *out, hipStream_t s);
// out[t] = bf16(sum_j slotbuf[t*k + j]) in j order.
hipError_t launch_combine(const float *slotbuf, int T, int k, int H, uint16_t *out, hipStream_t s);

// Plain streaming read of `bytes` (a multiple of 16), `loads` 16-byte loads
// per thread, with one XOR word per workgroup written to
// sink[stream_read_grid(bytes, loads)]: a measurement aid.
bool stream_read_loads_ok(int loads);
int64_t stream_read_grid(int64_t bytes, int loads);
hipError_t launch_stream_read(const void *src, int64_t bytes, int loads, uint32_t *sink, hipStream_t s);

}  // namespace nf4moe
