// C ABI of libnf4moe.so (declared in include/nf4moe.h): host-side validation,
// workspace carving and launch sequencing. Every check runs before anything is
// enqueued; on a non-OK status nothing was launched.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/nf4moe.h"
#include "common.h"
#include "dgrad.h"
#include "internal.h"
#include "probe.h"

using namespace nf4moe;

// Scratch of the allocation-free forward (nf4moe_moe_forward_noalloc): a
// file-scope device array that every GPU the library runs on holds until the
// process ends. Host code never uses its name as an address; it uses the
// per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[NF4MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

nf4moe_status_t fail(nf4moe_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

nf4moe_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return NF4MOE_OK;
  return fail(NF4MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool fmt_nf4(nf4moe_format_t f) { return f == NF4MOE_FMT_NF4_B64 || f == NF4MOE_FMT_NF4_B64_BF16ABS; }
int fmt_block(nf4moe_format_t f) { return fmt_nf4(f) ? 64 : 32; }
bool fmt_ok(nf4moe_format_t f) { return fmt_nf4(f) || f == NF4MOE_FMT_MXFP4_B32; }
int scale_align(nf4moe_format_t f) { return f == NF4MOE_FMT_NF4_B64 ? 4 : f == NF4MOE_FMT_NF4_B64_BF16ABS ? 2 : 1; }

// Routed rows up to which AUTO picks the small-M kernels: 64 for NF4, 48 for
// MXFP4, whose MFMA path makes one product per weight instead of two and
// overtakes sooner (same box: gpt-oss-shaped T = 12 / 16 small-M 340 / 420 us,
// MFMA 351 / 380 us). The crossover follows the rows per active expert, which
// the host cannot see: Qwen3-shaped Zipf batches want the MFMA path from
// 12 tokens (96 rows), OLMoE-shaped uniform ones the small-M path up to 16
// (128 rows); 64 serves the skewed case.
constexpr int kSmallR = 64;
constexpr int kSmallRMxfp4 = 48;
static int auto_small_rows(int fmt) { return fmt == NF4MOE_FMT_MXFP4_B32 ? kSmallRMxfp4 : kSmallR; }
// Tokens up to which the small-M path's down projection is token-centric (fused
// with the combine: no slot buffer, no combine launch). Each token re-reads the
// weights of its experts, which pays at these sizes: same box, against the
// grouped GEMV + combine, OLMoE-shaped T = 4 / 8 48.5 / 70.6 -> 44.9 / 67.1 us,
// Qwen3-shaped T = 8 64.0 -> 58.2 us, gpt-oss-shaped T = 16 423.6 -> 419.2 us.
constexpr int kTokenCentricT = 32;

// Activation rows the grouped GEMV applies per weight pass, from the average
// rows per group: 1 up to 2 (the usual decode batch: one or two rows per
// expert; more would hold idle rows' registers), 2 up to 4, else 4. Same box,
// OLMoE-shaped T = 4 / 8 layers: 81.1 / 116.8 us with 4, 48.5 / 70.5 us with 1.
// A row's arithmetic does not depend on it.
static int gemv_rows_per_pass(int64_t R, int64_t groups) {
  if (groups <= 0 || R <= 2 * groups) return 1;
  return R <= 4 * groups ? 2 : 4;
}
constexpr int64_t kSmallMaxK = 4096;

// Bump allocator over the caller's workspace.
struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *b) : base((char *)b) {}
  template <class T>
  T *take(size_t count) {
    off = align_up(off);
    T *p = base ? (T *)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

struct RoutePlan {
  int R, nchunks, max_grp, max_tiles, tile_rows;
};

RoutePlan route_plan(int T, int E, int k) {
  RoutePlan rp;
  rp.R = T * k;
  rp.nchunks = (int)cdiv(rp.R, kChunk);
  rp.max_grp = rp.R < E ? rp.R : E;
  rp.tile_rows = mfma_tile_rows(rp.R, E);
  rp.max_tiles = (int)cdiv(rp.R, rp.tile_rows) + rp.max_grp;
  return rp;
}

// Route scratch (everything RouteBufs needs except the caller-visible outputs).
void carve_route_scratch(Carve &cv, const RoutePlan &rp, int E, RouteBufs &rb) {
  rb.chunk_hist = cv.take<int32_t>((size_t)E * (rp.nchunks > 0 ? rp.nchunks : 1));
  rb.slot_pos = cv.take<int32_t>(rp.R > 0 ? rp.R : 1);
  rb.grp_expert = cv.take<int32_t>(E);
  rb.grp_row0 = cv.take<int32_t>(E);
  rb.grp_rows = cv.take<int32_t>(E);
  rb.counters = cv.take<int32_t>(16);
  // room for 64-row tiles whatever the plan, so the size only grows with R;
  // the table in two orders (by group, then by tile class) at tiles and
  // tiles + max_tiles
  rb.tiles = cv.take<int4>(2 * ((size_t)cdiv(rp.R, 64) + rp.max_grp + 1));
}

struct ForwardCarve {
  float *logits;     // [T, E] logits (small-M path), or the first of the router's
  float *partials;   //   partial sums [S][T][E] (MFMA path): the same memory
  RouteBufs rb;
  float *h;
  float *slotbuf;
  uint8_t *xq;  // MXFP4: x as the block-scaled MFMA operand (launch_e4m3_split), else null
  size_t bytes;
};

ForwardCarve carve_forward(void *ws, const nf4moe_layer_t &L, int T) {
  ForwardCarve fc;
  const RoutePlan rp = route_plan(T, L.E, L.top_k);
  Carve cv(ws);
  fc.partials = cv.take<float>(router_partials_bytes(T, L.E, L.H) / sizeof(float));
  fc.logits = fc.partials;
  fc.rb.topk_ids = cv.take<int32_t>(rp.R > 0 ? rp.R : 1);
  fc.rb.topk_w = cv.take<float>(rp.R > 0 ? rp.R : 1);
  fc.rb.expert_offsets = cv.take<int32_t>(L.E + 1);
  fc.rb.sorted_slots = cv.take<int32_t>(rp.R > 0 ? rp.R : 1);
  carve_route_scratch(cv, rp, L.E, fc.rb);
  fc.h = cv.take<float>((size_t)(rp.R > 0 ? rp.R : 1) * L.I);
  fc.slotbuf = cv.take<float>((size_t)(rp.R > 0 ? rp.R : 1) * L.H);
  fc.xq = L.fmt == NF4MOE_FMT_MXFP4_B32 ? cv.take<uint8_t>(e4m3_split_bytes(T > 0 ? T : 1, L.H)) : nullptr;
  fc.bytes = align_up(cv.off);
  return fc;
}

nf4moe_status_t check_layer(const nf4moe_layer_t *L) {
  if (!L) return fail(NF4MOE_ERR_INVALID_ARG, "layer is NULL");
  if (!fmt_ok(L->fmt)) return fail(NF4MOE_ERR_INVALID_ARG, "unknown format %d", (int)L->fmt);
  if (L->E < 1 || L->E > kMaxE) return fail(NF4MOE_ERR_INVALID_ARG, "E=%d outside 1..%d", L->E, kMaxE);
  const int kmax = L->E < kMaxTopK ? L->E : kMaxTopK;
  if (L->top_k < 1 || L->top_k > kmax)
    return fail(NF4MOE_ERR_INVALID_ARG, "top_k=%d outside 1..%d", L->top_k, kmax);
  if (L->H <= 0 || L->H % 64)
    return fail(NF4MOE_ERR_INVALID_ARG, "H=%d must be a positive multiple of 64", L->H);
  const int blk = fmt_block(L->fmt);
  if (L->I <= 0 || L->I % blk)
    return fail(NF4MOE_ERR_INVALID_ARG, "I=%d must be a positive multiple of %d", L->I, blk);
  if (L->renormalize != 0 && L->renormalize != 1)
    return fail(NF4MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
  if (L->path < NF4MOE_PATH_AUTO || L->path > NF4MOE_PATH_MFMA)
    return fail(NF4MOE_ERR_INVALID_ARG, "unknown path %d", L->path);
  if (!L->w13 || !L->w13_scale || !L->w2 || !L->w2_scale || !L->router_w)
    return fail(NF4MOE_ERR_INVALID_ARG, "layer weight pointer is NULL");
  if (!aligned(L->w13, 16) || !aligned(L->w2, 16) || !aligned(L->router_w, 16))
    return fail(NF4MOE_ERR_INVALID_ARG, "layer weights must be 16-byte aligned");
  if (!aligned(L->w13_scale, scale_align(L->fmt)) || !aligned(L->w2_scale, scale_align(L->fmt)))
    return fail(NF4MOE_ERR_INVALID_ARG, "scales must be aligned to their element size");
  if (L->router_b && !aligned(L->router_b, 4))
    return fail(NF4MOE_ERR_INVALID_ARG, "router_b must be 4-byte aligned");
  if (L->glu != NF4MOE_GLU_SWIGLU && L->glu != NF4MOE_GLU_CLAMPED)
    return fail(NF4MOE_ERR_INVALID_ARG, "unknown glu %d", L->glu);
  if (L->glu == NF4MOE_GLU_CLAMPED &&
      !(L->glu_alpha > 0.0f && L->glu_alpha < 1e30f && L->glu_limit > 0.0f && L->glu_limit < 1e30f))
    return fail(NF4MOE_ERR_INVALID_ARG, "clamped GLU needs finite alpha > 0 and limit > 0");
  if (L->glu_interleaved != 0 && L->glu_interleaved != 1)
    return fail(NF4MOE_ERR_INVALID_ARG, "glu_interleaved must be 0 or 1");
  if ((L->b13 && !aligned(L->b13, 4)) || (L->b2 && !aligned(L->b2, 4)))
    return fail(NF4MOE_ERR_INVALID_ARG, "b13/b2 must be 4-byte aligned");
  return NF4MOE_OK;
}

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

nf4moe_status_t noalloc_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(NF4MOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(NF4MOE_ERR_HIP, "scratch address %p not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return NF4MOE_OK;
}

GemmArgs base_args(nf4moe_format_t fmt) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.fmt = (int)fmt;
  g.a_div = 1;
  return g;
}

}  // namespace

extern "C" {

const char *nf4moe_version(void) { return "nf4moe 0.1.0 (gfx950)"; }

int32_t nf4moe_auto_path(nf4moe_format_t fmt, int64_t R, int64_t K_max) {
  return (R <= auto_small_rows((int)fmt) && K_max <= kSmallMaxK) ? NF4MOE_PATH_SMALL_M : NF4MOE_PATH_MFMA;
}

const char *nf4moe_status_string(nf4moe_status_t st) {
  switch (st) {
    case NF4MOE_OK: return "NF4MOE_OK";
    case NF4MOE_ERR_INVALID_ARG: return "NF4MOE_ERR_INVALID_ARG";
    case NF4MOE_ERR_UNSUPPORTED: return "NF4MOE_ERR_UNSUPPORTED";
    case NF4MOE_ERR_WORKSPACE: return "NF4MOE_ERR_WORKSPACE";
    case NF4MOE_ERR_HIP: return "NF4MOE_ERR_HIP";
  }
  return "NF4MOE_ERR_UNKNOWN";
}

const char *nf4moe_last_error(void) { return g_err; }

nf4moe_status_t nf4moe_codebook(nf4moe_format_t fmt, float out[16]) {
  if (!fmt_ok(fmt)) return fail(NF4MOE_ERR_INVALID_ARG, "unknown format %d", (int)fmt);
  if (!out) return fail(NF4MOE_ERR_INVALID_ARG, "out is NULL");
  for (int i = 0; i < 16; ++i) out[i] = fmt_nf4(fmt) ? nf4_value(i) : e2m1_value(i);
  return NF4MOE_OK;
}

static nf4moe_status_t check_quant_args(nf4moe_format_t fmt, const void *dense, int64_t rows,
                                        int64_t K, const void *packed, const void *scale) {
  if (!fmt_ok(fmt)) return fail(NF4MOE_ERR_INVALID_ARG, "unknown format %d", (int)fmt);
  if (rows < 0) return fail(NF4MOE_ERR_INVALID_ARG, "rows=%lld < 0", (long long)rows);
  const int blk = fmt_block(fmt);
  if (K <= 0 || K % blk) return fail(NF4MOE_ERR_INVALID_ARG, "K=%lld must be a positive multiple of %d", (long long)K, blk);
  if (rows == 0) return NF4MOE_OK;
  if (!dense || !packed || !scale) return fail(NF4MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(dense, 8) || !aligned(packed, 4) || !aligned(scale, scale_align(fmt)))
    return fail(NF4MOE_ERR_INVALID_ARG, "misaligned pointer");
  return NF4MOE_OK;
}

nf4moe_status_t nf4moe_quantize(nf4moe_format_t fmt, const float *w, int64_t rows, int64_t K,
                                uint8_t *packed, void *scale, void *stream) {
  nf4moe_status_t st = check_quant_args(fmt, w, rows, K, packed, scale);
  if (st != NF4MOE_OK || rows == 0) return st;
  return hip_status(launch_quantize((int)fmt, w, rows, K, packed, scale, (hipStream_t)stream),
                    "quantize launch");
}

nf4moe_status_t nf4moe_absmax_to_bf16(const float *absmax, int64_t n, uint16_t *out, int32_t *n_inexact,
                                      void *stream) {
  if (n < 0) return fail(NF4MOE_ERR_INVALID_ARG, "n=%lld < 0", (long long)n);
  if (n == 0) return NF4MOE_OK;
  if (!absmax || !out || !n_inexact) return fail(NF4MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(absmax, 4) || !aligned(out, 2) || !aligned(n_inexact, 4))
    return fail(NF4MOE_ERR_INVALID_ARG, "misaligned pointer");
  return hip_status(launch_absmax_bf16(absmax, n, out, n_inexact, (hipStream_t)stream), "absmax cast launch");
}

nf4moe_status_t nf4moe_dequantize(nf4moe_format_t fmt, const uint8_t *packed, const void *scale,
                                  int64_t rows, int64_t K, float *w_out, void *stream) {
  nf4moe_status_t st = check_quant_args(fmt, w_out, rows, K, packed, scale);
  if (st != NF4MOE_OK || rows == 0) return st;
  return hip_status(launch_dequantize((int)fmt, packed, scale, rows, K, w_out, (hipStream_t)stream),
                    "dequantize launch");
}

size_t nf4moe_router_workspace_bytes(int32_t T, int32_t E, int32_t H) {
  if (T < 1 || E < 1 || H <= 0 || H % 16) return 0;
  return align_up(router_partials_bytes(T, E, H));
}

nf4moe_status_t nf4moe_router_logits(const uint16_t *x, int32_t T, int32_t H,
                                     const float *router_w, const float *router_b, int32_t E,
                                     float *logits, void *ws, size_t ws_bytes, void *stream) {
  if (T < 0) return fail(NF4MOE_ERR_INVALID_ARG, "T=%d < 0", T);
  if (E < 1 || E > kMaxE) return fail(NF4MOE_ERR_INVALID_ARG, "E=%d outside 1..%d", E, kMaxE);
  if (H <= 0 || H % 8) return fail(NF4MOE_ERR_INVALID_ARG, "H=%d must be a positive multiple of 8", H);
  if (T == 0) return NF4MOE_OK;
  if (!x || !router_w || !logits) return fail(NF4MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(logits, 4))
    return fail(NF4MOE_ERR_INVALID_ARG, "misaligned pointer");
  float *partials = nullptr;
  if (ws && H % 16 == 0) {
    const size_t need = router_partials_bytes(T, E, H);
    if (ws_bytes < need) return fail(NF4MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(NF4MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    partials = static_cast<float *>(ws);
  }
  return hip_status(launch_router_logits(x, T, H, router_w, router_b, E, logits, partials, (hipStream_t)stream),
                    "router launch");
}

size_t nf4moe_route_workspace_bytes(int32_t T, int32_t E, int32_t top_k) {
  if (T < 0 || E < 1 || top_k < 1) return 0;
  const RoutePlan rp = route_plan(T, E, top_k);
  Carve cv(nullptr);
  RouteBufs rb;
  carve_route_scratch(cv, rp, E, rb);
  return align_up(cv.off);
}

nf4moe_status_t nf4moe_route_permute(const float *logits, int32_t T, int32_t E, int32_t top_k,
                                     int32_t renormalize, int32_t *topk_ids, float *topk_w,
                                     int32_t *expert_offsets, int32_t *sorted_slots, void *ws,
                                     size_t ws_bytes, void *stream) {
  if (T < 0) return fail(NF4MOE_ERR_INVALID_ARG, "T=%d < 0", T);
  if (E < 1 || E > kMaxE) return fail(NF4MOE_ERR_INVALID_ARG, "E=%d outside 1..%d", E, kMaxE);
  const int kmax = E < kMaxTopK ? E : kMaxTopK;
  if (top_k < 1 || top_k > kmax) return fail(NF4MOE_ERR_INVALID_ARG, "top_k=%d outside 1..%d", top_k, kmax);
  if (renormalize != 0 && renormalize != 1) return fail(NF4MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
  if (!expert_offsets) return fail(NF4MOE_ERR_INVALID_ARG, "expert_offsets is NULL");
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_slots))
    return fail(NF4MOE_ERR_INVALID_ARG, "NULL pointer");
  const size_t need = nf4moe_route_workspace_bytes(T, E, top_k);
  if (!ws || ws_bytes < need)
    return fail(NF4MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(NF4MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {
    // every expert is empty
    return hip_status(launch_fill_i32(expert_offsets, E + 1, 0, s), "fill");
  }
  const RoutePlan rp = route_plan(T, E, top_k);
  Carve cv(ws);
  RouteBufs rb;
  carve_route_scratch(cv, rp, E, rb);
  rb.topk_ids = topk_ids;
  rb.topk_w = topk_w;
  rb.expert_offsets = expert_offsets;
  rb.sorted_slots = sorted_slots;
  return hip_status(launch_route(logits, T, E, top_k, renormalize, rb, kMfmaBM, s), "route launch");
}

size_t nf4moe_gemm_workspace_bytes(int32_t G, int32_t R) {
  if (G < 1 || R < 0) return 0;
  Carve cv(nullptr);
  cv.take<int32_t>(G);
  cv.take<int32_t>(G);
  cv.take<int32_t>(G);
  cv.take<int32_t>(16);
  cv.take<int4>(2 * ((size_t)cdiv(R, 64) + G));  // 64-row tiles, both orders
  return align_up(cv.off);
}

nf4moe_status_t nf4moe_grouped_gemm(nf4moe_format_t fmt, const uint16_t *a, const int32_t *a_row_of,
                                    int32_t a_rows, const uint8_t *B, const void *B_scale, int32_t E,
                                    int64_t N, int64_t K, int32_t G, const int32_t *group_offsets,
                                    const int32_t *group_experts, int32_t R, void *c,
                                    nf4moe_dtype_t c_dtype, int32_t path, void *ws, size_t ws_bytes,
                                    void *stream) {
  if (!fmt_ok(fmt)) return fail(NF4MOE_ERR_INVALID_ARG, "unknown format %d", (int)fmt);
  const int blk = fmt_block(fmt);
  if (K <= 0 || K % blk) return fail(NF4MOE_ERR_INVALID_ARG, "K=%lld must be a positive multiple of %d", (long long)K, blk);
  if (N <= 0) return fail(NF4MOE_ERR_INVALID_ARG, "N=%lld must be positive", (long long)N);
  if (E < 1) return fail(NF4MOE_ERR_INVALID_ARG, "E=%d must be positive", E);
  if (G < 1 || G > 65536) return fail(NF4MOE_ERR_INVALID_ARG, "G=%d outside 1..65536", G);
  if (R < 0) return fail(NF4MOE_ERR_INVALID_ARG, "R=%d < 0", R);
  if (a_rows < 0 || (!a_row_of && a_rows < R) || (R > 0 && a_rows < 1))
    return fail(NF4MOE_ERR_INVALID_ARG, "a_rows=%d too small for R=%d%s", a_rows, R,
                a_row_of ? "" : " without a gather");
  if (c_dtype != NF4MOE_DT_F32 && c_dtype != NF4MOE_DT_BF16)
    return fail(NF4MOE_ERR_INVALID_ARG, "unknown output dtype %d", (int)c_dtype);
  if (path < NF4MOE_PATH_AUTO || path > NF4MOE_PATH_MFMA)
    return fail(NF4MOE_ERR_INVALID_ARG, "unknown path %d", path);
  if (!group_offsets) return fail(NF4MOE_ERR_INVALID_ARG, "group_offsets is NULL");
  if (R > 0 && (!a || !B || !B_scale || !c)) return fail(NF4MOE_ERR_INVALID_ARG, "NULL pointer");
  if (R > 0 && (!aligned(a, 16) || !aligned(B, 16) || !aligned(c, 4) ||
                !aligned(B_scale, scale_align(fmt))))
    return fail(NF4MOE_ERR_INVALID_ARG, "misaligned pointer");
  const size_t need = nf4moe_gemm_workspace_bytes(G, R);
  if (!ws || ws_bytes < need)
    return fail(NF4MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(NF4MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int use = path;
  if (use == NF4MOE_PATH_AUTO) use = nf4moe_auto_path(fmt, R, K);
  if (use == NF4MOE_PATH_SMALL_M && K > kSmallMaxK)
    return fail(NF4MOE_ERR_UNSUPPORTED, "small-M path needs K <= %lld", (long long)kSmallMaxK);
  if (R == 0) return NF4MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  Carve cv(ws);
  RouteBufs rb;
  rb.grp_expert = cv.take<int32_t>(G);
  rb.grp_row0 = cv.take<int32_t>(G);
  rb.grp_rows = cv.take<int32_t>(G);
  rb.counters = cv.take<int32_t>(16);
  rb.tiles = cv.take<int4>(2 * ((size_t)cdiv(R, 64) + G));
  const int bm = mfma_tile_rows(R, G);
  hipError_t e = launch_groups_from_offsets(group_offsets, group_experts, G, R, E, rb, bm, s);
  if (e != hipSuccess) return hip_status(e, "group table launch");
  GemmArgs g = base_args(fmt);
  g.a = a;
  g.a_is_f32 = 0;
  g.a_row_of = a_row_of;
  g.a_rows = a_rows;
  g.B = B;
  g.B_scale = B_scale;
  g.N = N;
  g.K = K;
  g.R = R;
  g.grp_expert = rb.grp_expert;
  g.grp_row0 = rb.grp_row0;
  g.grp_rows = rb.grp_rows;
  g.n_grp = rb.counters;
  g.max_grp = G;
  g.tiles = rb.tiles;
  g.n_tiles = rb.counters + 1;
  g.max_tiles = (int)(cdiv(R, bm) + G);
  g.tile_rows = bm;
  g.epi = c_dtype == NF4MOE_DT_F32 ? EPI_PLAIN_F32 : EPI_PLAIN_BF16;
  g.c = c;
  if (use == NF4MOE_PATH_SMALL_M)
    e = launch_gemv_grouped(g, gemv_rows_per_pass(R, G), s);
  else
    e = launch_mfma_grouped(g, s);
  return hip_status(e, "grouped GEMM launch");
}

nf4moe_status_t nf4moe_grouped_dgrad(nf4moe_format_t fmt, const uint16_t *dc, const uint8_t *B,
                                     const void *B_scale, int32_t E, int64_t N, int64_t K, int32_t G,
                                     const int32_t *group_offsets, const int32_t *group_experts,
                                     int32_t R, void *da, nf4moe_dtype_t da_dtype, void *ws,
                                     size_t ws_bytes, void *stream) {
  if (!fmt_ok(fmt)) return fail(NF4MOE_ERR_INVALID_ARG, "unknown format %d", (int)fmt);
  const int blk = fmt_block(fmt);
  if (K <= 0 || K % blk) return fail(NF4MOE_ERR_INVALID_ARG, "K=%lld must be a positive multiple of %d", (long long)K, blk);
  if (N <= 0) return fail(NF4MOE_ERR_INVALID_ARG, "N=%lld must be positive", (long long)N);
  if (N % 64) return fail(NF4MOE_ERR_UNSUPPORTED, "dgrad needs N %% 64 == 0 (N=%lld)", (long long)N);
  if (E < 1) return fail(NF4MOE_ERR_INVALID_ARG, "E=%d must be positive", E);
  if (G < 1 || G > 65536) return fail(NF4MOE_ERR_INVALID_ARG, "G=%d outside 1..65536", G);
  if (R < 0) return fail(NF4MOE_ERR_INVALID_ARG, "R=%d < 0", R);
  if (da_dtype != NF4MOE_DT_F32 && da_dtype != NF4MOE_DT_BF16)
    return fail(NF4MOE_ERR_INVALID_ARG, "unknown output dtype %d", (int)da_dtype);
  if (!group_offsets) return fail(NF4MOE_ERR_INVALID_ARG, "group_offsets is NULL");
  if (R > 0 && (!dc || !B || !B_scale || !da)) return fail(NF4MOE_ERR_INVALID_ARG, "NULL pointer");
  if (R > 0 && (!aligned(dc, 16) || !aligned(da, 4) || !aligned(B_scale, scale_align(fmt))))
    return fail(NF4MOE_ERR_INVALID_ARG, "misaligned pointer");
  const size_t need = nf4moe_gemm_workspace_bytes(G, R);
  if (!ws || ws_bytes < need)
    return fail(NF4MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(NF4MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (R == 0) return NF4MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  Carve cv(ws);
  RouteBufs rb;
  rb.grp_expert = cv.take<int32_t>(G);
  rb.grp_row0 = cv.take<int32_t>(G);
  rb.grp_rows = cv.take<int32_t>(G);
  rb.counters = cv.take<int32_t>(16);
  rb.tiles = cv.take<int4>(2 * ((size_t)cdiv(R, kMfmaBM) + G));
  hipError_t e = launch_groups_from_offsets(group_offsets, group_experts, G, R, E, rb, kMfmaBM, s);
  if (e != hipSuccess) return hip_status(e, "group table launch");
  DgradArgs a;
  a.fmt = (int)fmt;
  a.dc = dc;
  a.B = B;
  a.B_scale = B_scale;
  a.N = N;
  a.K = K;
  a.tiles = rb.tiles;
  a.n_tiles = rb.counters + 1;
  a.max_tiles = (int)(cdiv(R, kMfmaBM) + G);
  a.da = da;
  a.da_bf16 = da_dtype == NF4MOE_DT_BF16;
  return hip_status(launch_dgrad(a, s), "dgrad launch");
}

size_t nf4moe_workspace_bytes(const nf4moe_layer_t *layer, int32_t T_max) {
  if (!layer || T_max < 0 || layer->E < 1 || layer->top_k < 1) return 0;
  return carve_forward(nullptr, *layer, T_max).bytes;
}

static nf4moe_status_t forward_impl(const nf4moe_layer_t *layer, const uint16_t *x, int32_t T,
                                    uint16_t *out, int32_t *topk_ids_out, float *topk_w_out,
                                    void *ws, size_t ws_bytes, void *stream,
                                    void *const *events) {
  nf4moe_status_t st = check_layer(layer);
  if (st != NF4MOE_OK) return st;
  const nf4moe_layer_t &L = *layer;
  if (T < 0) return fail(NF4MOE_ERR_INVALID_ARG, "T=%d < 0", T);
  if (T == 0) return NF4MOE_OK;
  if (!x || !out) return fail(NF4MOE_ERR_INVALID_ARG, "x/out is NULL");
  if (!aligned(x, 16) || !aligned(out, 8)) return fail(NF4MOE_ERR_INVALID_ARG, "x must be 16-byte and out 8-byte aligned");
  if ((int64_t)T * L.top_k > (int64_t)1 << 30) return fail(NF4MOE_ERR_UNSUPPORTED, "T*top_k too large");
  const ForwardCarve need = carve_forward(nullptr, L, T);
  if (!ws || ws_bytes < need.bytes)
    return fail(NF4MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need.bytes);
  if (!aligned(ws, 256)) return fail(NF4MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const RoutePlan rp = route_plan(T, L.E, L.top_k);
  int use = L.path;
  const int64_t maxK = L.H > L.I ? L.H : L.I;
  if (use == NF4MOE_PATH_AUTO) use = nf4moe_auto_path(L.fmt, rp.R, maxK);
  if (use == NF4MOE_PATH_SMALL_M && maxK > kSmallMaxK)
    return fail(NF4MOE_ERR_UNSUPPORTED, "small-M path needs H, I <= %lld", (long long)kSmallMaxK);

  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  auto mark = [&](int i) -> hipError_t {
    return events ? hipEventRecord((hipEvent_t)events[i], s) : hipSuccess;
  };
  ForwardCarve fc = carve_forward(ws, L, T);
  if ((e = mark(0)) != hipSuccess) return hip_status(e, "event record");
  // The small-M path keeps each token's bits independent of T: per-token
  // router logits for every T, and kernels whose per-row order is fixed.
  // Routing logits: the rows kernel on the small-M path and for few tokens on
  // the MFMA path, else the matrix-core router; each has a fixed per-token
  // order (the latter sums fixed chunks of H in order), so a token's bits do
  // not depend on T within each of them.
  const bool small = use == NF4MOE_PATH_SMALL_M;
  const bool rows_router = small || T <= kMfmaRowsRouterMaxT;
  e = rows_router ? launch_router_rows(x, T, L.H, L.router_w, L.router_b, L.E, fc.logits, s)
                  : launch_router_partials(x, T, L.H, L.router_w, L.E, fc.partials, s);
  if (e != hipSuccess) return hip_status(e, "router launch");
  // One decode token on the small-M path: top-k and grouping happen inside the
  // gate_up kernel; otherwise they are their own launches.
  const bool fused_route = use == NF4MOE_PATH_SMALL_M && T == 1 && L.E <= 128;
  if (!fused_route) {
    e = rows_router ? launch_route(fc.logits, T, L.E, L.top_k, L.renormalize, fc.rb, rp.tile_rows, s)
                    : launch_route_partials(fc.partials, router_split(L.H), L.router_b, T, L.E, L.top_k,
                                            L.renormalize, fc.rb, rp.tile_rows, s);
    if (e != hipSuccess) return hip_status(e, "route launch");
  }
  if ((e = mark(1)) != hipSuccess) return hip_status(e, "event record");

  // gate_up + SwiGLU -> h [R, I] in expert-sorted order (fp32; on the MFMA
  // path 32-bit (bf16 hi, bf16 lo) pairs)
  GemmArgs g = base_args(L.fmt);
  g.a = x;
  g.a_is_f32 = 0;
  if (use == NF4MOE_PATH_MFMA && fc.xq) {  // MXFP4: block-scaled MFMAs on an e4m3 split of x
    if ((e = launch_e4m3_split(x, T, L.H, fc.xq, s)) != hipSuccess) return hip_status(e, "split launch");
    g.a = fc.xq;
    g.a_is_f32 = 3;
  }
  g.a_row_of = fc.rb.sorted_slots;
  g.a_div = L.top_k;
  g.a_rows = T;
  g.B = L.w13;
  g.B_scale = L.w13_scale;
  g.N = 2 * (int64_t)L.I;
  g.K = L.H;
  g.R = rp.R;
  g.grp_expert = fc.rb.grp_expert;
  g.grp_row0 = fc.rb.grp_row0;
  g.grp_rows = fc.rb.grp_rows;
  g.n_grp = fc.rb.counters;
  g.max_grp = rp.max_grp;
  g.tiles = fc.rb.tiles;
  g.n_tiles = fc.rb.counters + 1;
  g.max_tiles = rp.max_tiles;
  g.tile_rows = rp.tile_rows;
  g.epi = EPI_SWIGLU;
  g.glu = L.glu;
  g.glu_alpha = L.glu_alpha;
  g.glu_limit = L.glu_limit;
  g.glu_inter = L.glu_interleaved;
  g.bias = L.b13;
  g.c = fc.h;
  if (use == NF4MOE_PATH_MFMA) g.c_split = 1;  // h as (bf16 hi, lo) pairs for the down MFMAs
  if (fused_route) {
    g.route_logits = fc.logits;
    g.route_E = L.E;
    g.route_k = L.top_k;
    g.route_renorm = L.renormalize;
    g.route_out = fc.rb;
  }
  const int ms = gemv_rows_per_pass(rp.R, rp.max_grp);
  if (events) {  // the gate_up kernel's own start / end timestamps
    g.ev_start = events[4];
    g.ev_stop = events[5];
  }
  e = use == NF4MOE_PATH_SMALL_M ? launch_gemv_grouped(g, ms, s) : launch_mfma_grouped(g, s);
  if (e != hipSuccess) return hip_status(e, "gate_up launch");
  if ((e = mark(2)) != hipSuccess) return hip_status(e, "event record");

  // down projection + router-weighted combine
  if (small && T <= kTokenCentricT && down_combine_supported(L.I, L.top_k)) {
    e = launch_gemv_down_combine((int)L.fmt, fc.h, fc.rb.slot_pos, fc.rb.topk_ids, fc.rb.topk_w, T,
                                 L.top_k, L.w2, L.w2_scale, L.b2, L.H, L.I, out, s);
    if (e != hipSuccess) return hip_status(e, "down launch");
  } else {
    GemmArgs d = g;
    d.route_logits = nullptr;
    d.ev_start = d.ev_stop = nullptr;
    d.a = fc.h;
    d.a_is_f32 = use == NF4MOE_PATH_MFMA ? 2 : 1;
    d.c_split = 0;
    d.a_row_of = nullptr;
    d.a_div = 1;
    d.a_rows = rp.R;
    d.B = L.w2;
    d.B_scale = L.w2_scale;
    d.N = L.H;
    d.K = L.I;
    d.epi = EPI_SLOT;
    d.glu_inter = 0;
    d.bias = L.b2;
    d.c = fc.slotbuf;
    d.slot_of = fc.rb.sorted_slots;
    d.slot_w = fc.rb.topk_w;
    e = use == NF4MOE_PATH_SMALL_M ? launch_gemv_grouped(d, ms, s) : launch_mfma_grouped(d, s);
    if (e != hipSuccess) return hip_status(e, "down launch");
    e = launch_combine(fc.slotbuf, T, L.top_k, L.H, out, s);
    if (e != hipSuccess) return hip_status(e, "combine launch");
  }
  if ((e = mark(3)) != hipSuccess) return hip_status(e, "event record");
  if (topk_ids_out) {
    e = hipMemcpyAsync(topk_ids_out, fc.rb.topk_ids, sizeof(int32_t) * rp.R, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, "copy topk_ids");
  }
  if (topk_w_out) {
    e = hipMemcpyAsync(topk_w_out, fc.rb.topk_w, sizeof(float) * rp.R, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_status(e, "copy topk_w");
  }
  return NF4MOE_OK;
}

nf4moe_status_t nf4moe_moe_forward(const nf4moe_layer_t *layer, const uint16_t *x, int32_t T,
                                   uint16_t *out, int32_t *topk_ids_out, float *topk_w_out,
                                   void *ws, size_t ws_bytes, void *stream) {
  return forward_impl(layer, x, T, out, topk_ids_out, topk_w_out, ws, ws_bytes, stream, nullptr);
}

nf4moe_status_t nf4moe_moe_forward_noalloc(const nf4moe_layer_t *layer, const uint16_t *x, int32_t T,
                                           uint16_t *out, int32_t *topk_ids_out, float *topk_w_out,
                                           void *stream) {
  nf4moe_status_t st = check_layer(layer);
  if (st != NF4MOE_OK) return st;
  if (T < 0) return fail(NF4MOE_ERR_INVALID_ARG, "T=%d < 0", T);
  if (T == 0) return NF4MOE_OK;
  if ((int64_t)T * layer->top_k > (int64_t)1 << 30) return fail(NF4MOE_ERR_UNSUPPORTED, "T*top_k too large");
  const size_t need = carve_forward(nullptr, *layer, T).bytes;
  if (need > (size_t)NF4MOE_NOALLOC_SCRATCH_BYTES)
    return fail(NF4MOE_ERR_WORKSPACE,
                "this layer at T=%d needs %zu bytes of scratch; the allocation-free forward holds %zu "
                "(call nf4moe_moe_forward with a workspace instead)",
                T, need, (size_t)NF4MOE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != NF4MOE_OK) return st;
  // Nothing in the scratch needs to start at zero: within one call every
  // kernel writes what it later reads.
  return forward_impl(layer, x, T, out, topk_ids_out, topk_w_out, ws, NF4MOE_NOALLOC_SCRATCH_BYTES, stream,
                      nullptr);
}

nf4moe_status_t nf4moe_moe_forward_profiled(const nf4moe_layer_t *layer, const uint16_t *x,
                                            int32_t T, uint16_t *out, void *ws, size_t ws_bytes,
                                            void *stream, void *const *events) {
  if (!events) return fail(NF4MOE_ERR_INVALID_ARG, "events is NULL");
  return forward_impl(layer, x, T, out, nullptr, nullptr, ws, ws_bytes, stream, events);
}

int64_t nf4moe_stream_read_sink_words(int64_t bytes, int32_t loads_per_thread) {
  return bytes > 0 && bytes % 16 == 0 && stream_read_loads_ok(loads_per_thread)
             ? stream_read_grid(bytes, loads_per_thread) : 0;
}

nf4moe_status_t nf4moe_stream_read(const void *buf, int64_t bytes, int32_t loads_per_thread, uint32_t *sink,
                                   void *stream) {
  if (bytes <= 0 || bytes % 16) return fail(NF4MOE_ERR_INVALID_ARG, "bytes=%lld must be a positive multiple of 16", (long long)bytes);
  if (!stream_read_loads_ok(loads_per_thread))
    return fail(NF4MOE_ERR_INVALID_ARG, "loads_per_thread=%d must be 1, 2, 4, 8 or 16", loads_per_thread);
  if (stream_read_grid(bytes, loads_per_thread) > 0x7fffffff) return fail(NF4MOE_ERR_UNSUPPORTED, "bytes=%lld too large", (long long)bytes);
  if (!buf || !sink) return fail(NF4MOE_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(NF4MOE_ERR_INVALID_ARG, "misaligned pointer");
  return hip_status(launch_stream_read(buf, bytes, loads_per_thread, sink, (hipStream_t)stream), "stream read launch");
}

int64_t nf4moe_mfma_peak_flops(int32_t workgroups, int32_t iters) {
  return workgroups > 0 && iters > 0 && workgroups <= (1 << 20) ? mfma_peak_flops(workgroups, iters) : 0;
}

nf4moe_status_t nf4moe_mfma_peak(int32_t workgroups, int32_t iters, float *sink, void *stream) {
  if (workgroups <= 0 || workgroups > (1 << 20))
    return fail(NF4MOE_ERR_INVALID_ARG, "workgroups=%d outside 1..%d", workgroups, 1 << 20);
  if (iters <= 0) return fail(NF4MOE_ERR_INVALID_ARG, "iters=%d must be positive", iters);
  if (!sink) return fail(NF4MOE_ERR_INVALID_ARG, "NULL sink");
  if (!aligned(sink, 4)) return fail(NF4MOE_ERR_INVALID_ARG, "misaligned sink");
  return hip_status(launch_mfma_peak(workgroups, iters, sink, (hipStream_t)stream), "mfma peak launch");
}

}  // extern "C"
