// Routing on the device: router logits, top-k + softmax, and the stable
// grouping of routed slots by expert (histogram, one flat scan, scatter), plus
// the group and tile tables the grouped GEMMs read. No host synchronisation.
//
// The pages keep this upstream of the kernel (page "How do I run a grouped GEMM
// directly on NF4 packed MoE expert weights ...", section "Why it happens":
// tokens are sorted by expert and scattered back outside the kernel; the
// kernel takes a_cat sorted by expert with sizes + expert_ids). Here it is the
// library's own first stage. Integer results are exact: a slot's position is
// the number of slots routed to lower experts plus the number of earlier slots
// routed to its own expert.
#include <limits.h>

#include "common.h"
#include "internal.h"

namespace nf4moe {

// ---------------------------------------------------------------------------
// Router logits, few tokens: one workgroup per (expert, chunk of TMAX tokens),
// threads stride over H. A token's logit is summed in the same order whatever
// TMAX, the chunk it falls in and the other tokens of the call.
// ---------------------------------------------------------------------------
template <int TMAX>
__global__ __launch_bounds__(256) void k_logits_rows(const uint16_t *__restrict__ x, int T, int H,
                                                     const float *__restrict__ W,
                                                     const float *__restrict__ b, int E,
                                                     float *__restrict__ L) {
  const int e = blockIdx.x;
  const int64_t t0 = (int64_t)blockIdx.y * TMAX;
  x += t0 * H;
  L += t0 * E;
  T = (int)((int64_t)T - t0 < TMAX ? (int64_t)T - t0 : TMAX);
  const float *w = W + (int64_t)e * H;
  float acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0f;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    const float4 w0 = *reinterpret_cast<const float4 *>(w + h);
    const float4 w1 = *reinterpret_cast<const float4 *>(w + h + 4);
    // Tokens in batches of up to 8: the batch's loads (clamped to a valid row,
    // no branch) are all issued before the first is used.
    constexpr int BT = TMAX < 8 ? TMAX : 8;
#pragma unroll
    for (int t0 = 0; t0 < TMAX; t0 += BT) {
      if (t0 >= T) break;  // uniform
      uint4 xv[BT];
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        const int t = t0 + i < T ? t0 + i : 0;
        xv[i] = *reinterpret_cast<const uint4 *>(x + (int64_t)t * H + h);
      }
#pragma unroll
      for (int i = 0; i < BT; ++i) {
        float a = acc[t0 + i];
        a = fmaf(bf16lo_to_f32(xv[i].x), w0.x, a);
        a = fmaf(bf16hi_to_f32(xv[i].x), w0.y, a);
        a = fmaf(bf16lo_to_f32(xv[i].y), w0.z, a);
        a = fmaf(bf16hi_to_f32(xv[i].y), w0.w, a);
        a = fmaf(bf16lo_to_f32(xv[i].z), w1.x, a);
        a = fmaf(bf16hi_to_f32(xv[i].z), w1.y, a);
        a = fmaf(bf16lo_to_f32(xv[i].w), w1.z, a);
        a = fmaf(bf16hi_to_f32(xv[i].w), w1.w, a);
        acc[t0 + i] = a;   // rows past T are computed from row 0 and never stored
      }
    }
  }
  __shared__ float red[4][TMAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    float v = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    if (b) v += b[e];
    L[(int64_t)t * E + e] = v;
  }
}

// ---------------------------------------------------------------------------
// Router logits, many tokens, on the matrix cores. x is bf16, an exact MFMA
// operand. Each fp32 router weight is split exactly into three bf16 parts
// w = w1 + w2 + w3 (w1 = w truncated to bf16, w2 = the remainder truncated,
// w3 = what is left, at most 8 significant bits), so three bf16 products
// accumulated in fp32 give the fp32 dot product.
// k_split3: the three planes [3][E][H] (bf16 bits) from router_w.
// k_logits_mfma: 32 tokens x 32 experts per workgroup, eight waves taking one
// eighth of H each, loads issued eight k-steps ahead (their partial sums meet
// in LDS, in a fixed order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_split3(const float *__restrict__ W, int64_t n,
                                                uint16_t *__restrict__ planes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = __float_as_uint(W[i]);
  const uint32_t p1 = w >> 16;
  const float r1 = __uint_as_float(w) - __uint_as_float(p1 << 16);
  const uint32_t p2 = __float_as_uint(r1) >> 16;
  const float r2 = r1 - __uint_as_float(p2 << 16);
  planes[i] = (uint16_t)p1;
  planes[n + i] = (uint16_t)p2;
  planes[2 * n + i] = (uint16_t)(__float_as_uint(r2) >> 16);
}

typedef __bf16 lg_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float lg_f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void k_logits_mfma(const uint16_t *__restrict__ x, int T, int H,
                                                     const uint16_t *__restrict__ planes,
                                                     const float *__restrict__ b, int E,
                                                     float *__restrict__ L) {
  constexpr int NW = 8, BATCH = 8;
  __shared__ float red[NW - 1][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int t = blockIdx.x * 32 + l32, e = blockIdx.y * 32 + l32;
  const int64_t xrow = t < T ? t : 0, wrow = e < E ? e : 0;
  const int64_t n = (int64_t)E * H;
  // wave w takes k-steps [s0, s1) of 16 (H % 32 == 0)
  const int nsteps = H / 16;
  const int s0 = wave * nsteps / NW, s1 = (wave + 1) * nsteps / NW;
  const uint16_t *xa = x + xrow * H + 8 * g;
  const uint16_t *wa = planes + wrow * H + 8 * g;
  lg_f32x16_t acc = {};
  for (int sb = s0; sb < s1; sb += BATCH) {
    uint4 a[BATCH], b1[BATCH], b2[BATCH], b3[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {      // the batch's loads first (clamped to the range)
      const int st = sb + i < s1 ? sb + i : s1 - 1;
      a[i] = *reinterpret_cast<const uint4 *>(xa + 16 * st);
      b1[i] = *reinterpret_cast<const uint4 *>(wa + 16 * st);
      b2[i] = *reinterpret_cast<const uint4 *>(wa + n + 16 * st);
      b3[i] = *reinterpret_cast<const uint4 *>(wa + 2 * n + 16 * st);
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      if (sb + i < s1) {
        const lg_bf16x8_t av = __builtin_bit_cast(lg_bf16x8_t, a[i]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(lg_bf16x8_t, b1[i]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(lg_bf16x8_t, b2[i]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(lg_bf16x8_t, b3[i]), acc, 0, 0, 0);
      }
    }
  }
  // 32x32 accumulator: lane holds expert column l32, token rows
  // 8 * (v / 4) + 4 * g + (v % 4). Partial sums meet in wave order.
  if (wave > 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave - 1][v][lane] = acc[v];
  }
  __syncthreads();
  if (wave > 0 || e >= E) return;
  const float bias = b ? b[e] : 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float sum = acc[v];
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) sum += red[w][v][lane];
    const int tt = blockIdx.x * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
    if (tt < T) L[(int64_t)tt * E + e] = sum + bias;
  }
}

size_t router_split_bytes(int E, int H) { return (size_t)3 * E * H * sizeof(uint16_t); }

// ---------------------------------------------------------------------------
// Router logits, many tokens: 32 tokens x 64 experts per workgroup, H in
// steps of 64 through LDS; each thread owns 2 tokens x 4 experts.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_logits_tiled(const uint16_t *__restrict__ x, int T, int H,
                                                      const float *__restrict__ W,
                                                      const float *__restrict__ b, int E,
                                                      float *__restrict__ L) {
  __shared__ float xs[64][33];
  __shared__ float ws[64][65];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 64;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[2][4] = {};
  for (int h0 = 0; h0 < H; h0 += 64) {
    {  // x: 32 tokens x 64 h, 8 bf16 per thread
      const int tt = tid >> 3, hh = (tid & 7) * 8;
      const int t = t0 + tt, h = h0 + hh;
      uint4 xv = make_uint4(0, 0, 0, 0);
      if (t < T && h < H) xv = *reinterpret_cast<const uint4 *>(x + (int64_t)t * H + h);
      xs[hh + 0][tt] = bf16lo_to_f32(xv.x);
      xs[hh + 1][tt] = bf16hi_to_f32(xv.x);
      xs[hh + 2][tt] = bf16lo_to_f32(xv.y);
      xs[hh + 3][tt] = bf16hi_to_f32(xv.y);
      xs[hh + 4][tt] = bf16lo_to_f32(xv.z);
      xs[hh + 5][tt] = bf16hi_to_f32(xv.z);
      xs[hh + 6][tt] = bf16lo_to_f32(xv.w);
      xs[hh + 7][tt] = bf16hi_to_f32(xv.w);
    }
    {  // W: 64 experts x 64 h, 16 fp32 per thread
      const int ee = tid >> 2, hh = (tid & 3) * 16;
      const int e = e0 + ee;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int h = h0 + hh + 4 * q;
        float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < E && h < H) wv = *reinterpret_cast<const float4 *>(W + (int64_t)e * H + h);
        ws[hh + 4 * q + 0][ee] = wv.x;
        ws[hh + 4 * q + 1][ee] = wv.y;
        ws[hh + 4 * q + 2][ee] = wv.z;
        ws[hh + 4 * q + 3][ee] = wv.w;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int hh = 0; hh < 64; ++hh) {
      const float xa0 = xs[hh][ty * 2], xa1 = xs[hh][ty * 2 + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float wv = ws[hh][tx * 4 + q];
        acc[0][q] = fmaf(xa0, wv, acc[0][q]);
        acc[1][q] = fmaf(xa1, wv, acc[1][q]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + ty * 2 + i;
    if (t >= T) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + tx * 4 + q;
      if (e < E) L[(int64_t)t * E + e] = acc[i][q] + (b ? b[e] : 0.0f);
    }
  }
}

hipError_t launch_router_logits(const uint16_t *x, int T, int H, const float *W, const float *b,
                                int E, float *logits, void *split_ws, hipStream_t s, bool rows_only) {
  if (T <= 0) return hipSuccess;
  if (T == 1) {  // one token: no idle token slots (the same per-token order)
    hipLaunchKernelGGL(k_logits_rows<1>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  } else if (rows_only) {  // the per-token order of k_logits_rows for every T
    if (T <= 2)
      hipLaunchKernelGGL(k_logits_rows<2>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
    else if (T <= 4)
      hipLaunchKernelGGL(k_logits_rows<4>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
    else if (T <= 8)
      hipLaunchKernelGGL(k_logits_rows<8>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
    else
      hipLaunchKernelGGL(k_logits_rows<32>, dim3(E, (unsigned)cdiv(T, 32)), dim3(256), 0, s, x, T, H, W,
                         b, E, logits);
  } else if (split_ws && T >= kMfmaLogitsT && H % 32 == 0) {
    uint16_t *planes = reinterpret_cast<uint16_t *>(split_ws);
    const int64_t n = (int64_t)E * H;
    hipLaunchKernelGGL(k_split3, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, W, n, planes);
    hipLaunchKernelGGL(k_logits_mfma, dim3((unsigned)cdiv(T, 32), (unsigned)cdiv(E, 32)), dim3(512), 0, s,
                       x, T, H, planes, b, E, logits);
  } else if (T <= 8) {
    hipLaunchKernelGGL(k_logits_rows<8>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  } else if (T <= 32) {
    hipLaunchKernelGGL(k_logits_rows<32>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  } else {
    hipLaunchKernelGGL(k_logits_tiled, dim3((unsigned)cdiv(T, 32), (unsigned)cdiv(E, 64)),
                       dim3(256), 0, s, x, T, H, W, b, E, logits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// top-k + softmax: one wave per token. Lane l holds the logits of experts
// l, l + 64, ...; k rounds of a wave-wide argmax under the order (logit
// descending, id ascending); lane j keeps the j-th pick.
//
// The argmax runs on order-preserving 32-bit keys of the logits: the wave
// maximum of the keys comes from DPP row shifts and row broadcasts (no LDS
// round trips), and the lowest expert id holding it from one ballot per
// logit slot, so ties go to the lower id as the compare order requires.
// ---------------------------------------------------------------------------
// Larger float -> larger key; -0 is folded onto +0 first, so floats that
// compare equal get equal keys.
__device__ inline uint32_t float_order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Maximum of v over the 64 lanes: within each row of 16 lanes by right
// shifts (1, 2, 3, then 4 and 8 on the upper banks), then across rows by the
// row-15 and row-31 broadcasts; lane 63 ends with the maximum.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x113, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xf, 0xe, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xf, 0xc, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

template <int EPL>
__device__ inline void wave_topk(const float *Lrow, int E, int k, int renorm, int &my_id, float &wgt) {
  const int lane = threadIdx.x & 63;
  float v[EPL];
  uint32_t key[EPL];  // 0: no expert, or already picked (below every logit's key)
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? Lrow[e] : -__builtin_inff();
    key[j] = e < E ? float_order_key(v[j]) : 0u;
  }
  float my_v = 0.0f;
  my_id = 0;
  for (int i = 0; i < k; ++i) {
    uint32_t lm = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) lm = max(lm, key[j]);
    const uint32_t wm = wave_max_u32(lm);
    int win = -1;  // lowest id holding the maximum (uniform)
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const uint64_t m = __ballot(key[j] == wm);
      if (win < 0 && m != 0) win = 64 * j + (int)__builtin_ctzll(m);
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (win == lane + 64 * j) key[j] = 0u;
    float wv = 0.0f;  // the pick's logit, read from its lane
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if ((win >> 6) == j) wv = lane_value(v[j], win & 63);
    if (lane == i) {
      my_id = win;
      my_v = wv;
    }
  }
  const float v0 = lane_value(my_v, 0);  // the largest logit
  // Denominator summed in one fixed order (selected experts by rank, or all
  // experts by id), the order every routing kernel here uses.
  float den = 0.0f;
  if (renorm) {
    const float ex = lane < k ? expf(my_v - v0) : 0.0f;
    for (int q = 0; q < k; ++q) den += lane_value(ex, q);
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const float ex = lane + 64 * j < E ? expf(v[j] - v0) : 0.0f;
      for (int l = 0; l < 64 && 64 * j + l < E; ++l) den += lane_value(ex, l);
    }
  }
  wgt = expf(my_v - v0) / den;
}

template <int EPL>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ L, int T, int E, int k,
                                              int renorm, int32_t *__restrict__ ids,
                                              float *__restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int my_id;
  float wgt;
  wave_topk<EPL>(L + (int64_t)t * E, E, k, renorm, my_id, wgt);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    wts[(int64_t)t * k + lane] = wgt;
  }
}

// ---------------------------------------------------------------------------
// Grouping, stage 1: per-chunk expert histogram, stored expert-major
// hist[e * nchunks + c], so one flat exclusive scan of hist gives, at (e, c),
// the first sorted position of chunk c's slots routed to expert e.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_group_hist(const int32_t *__restrict__ ids, int R, int E,
                                                    int nchunks, int32_t *__restrict__ hist) {
  __shared__ int cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int s = blockIdx.x * kChunk + threadIdx.x;
  if (s < R) atomicAdd(&cnt[ids[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(int64_t)e * nchunks + blockIdx.x] = cnt[e];
}

// Exclusive scan of one value per thread across a 1024-thread block; *total
// (shared memory) receives the block total. Every thread must call it.
__device__ inline int block_scan_1024(int v, int *total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? wsum[lane] : 0;
    int wi = w;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int o = __shfl_up(wi, d, kWave);
      if (lane >= d) wi += o;
    }
    if (lane < 16) wsum[lane] = wi - w;  // exclusive offset of each wave
    if (lane == 15) *total = wi;
  }
  __syncthreads();
  const int ex = wsum[wave] + inc - v;
  __syncthreads();  // wsum is reused by the next call
  return ex;
}

// Tiles of at most bm rows for every group; single workgroup of 1024 threads.
__device__ void build_tiles(const int32_t *grp_expert, const int32_t *grp_row0,
                            const int32_t *grp_rows, int n_grp, int bm, int max_tiles, int4 *tiles,
                            int32_t *n_tiles_out) {
  __shared__ int s_total;
  __shared__ int s_carry;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int g0 = 0; g0 < n_grp; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    const int rows = g < n_grp ? grp_rows[g] : 0;
    const int nt = (rows + bm - 1) / bm;
    const int ex = block_scan_1024(nt, &s_total);
    const int base = s_carry + ex;
    for (int i = 0; i < nt && base + i < max_tiles; ++i) {
      const int r0 = i * bm;
      tiles[base + i] = make_int4(grp_expert[g], grp_row0[g] + r0, min(bm, rows - r0), rows);
    }
    __syncthreads();
    if (threadIdx.x == 0) s_carry += s_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_tiles_out = min(s_carry, max_tiles);
}

// Grouping, stage 2 (single workgroup): flat exclusive scan of the histogram,
// expert offsets, the compacted list of non-empty experts, and the MFMA tiles.
__global__ __launch_bounds__(1024) void k_group_scan(int32_t *__restrict__ hist, int E, int nchunks,
                                                     int R, int bm, int max_tiles,
                                                     int32_t *__restrict__ off,
                                                     int32_t *__restrict__ grp_expert,
                                                     int32_t *__restrict__ grp_row0,
                                                     int32_t *__restrict__ grp_rows,
                                                     int32_t *__restrict__ counters,
                                                     int4 *__restrict__ tiles) {
  __shared__ int s_total;
  const int64_t n = (int64_t)E * nchunks;
  const int64_t per = (n + 1023) / 1024;
  const int64_t i0 = per * threadIdx.x, i1 = min(n, i0 + per);
  int sum = 0;
  for (int64_t i = i0; i < i1; ++i) sum += hist[i];
  int run = block_scan_1024(sum, &s_total);
  for (int64_t i = i0; i < i1; ++i) {
    const int v = hist[i];
    hist[i] = run;
    run += v;
  }
  __syncthreads();
  // expert offsets and the compacted non-empty experts (ascending id)
  int cnt_total = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    int o = 0, c = 0;
    if (e < E) {
      o = hist[(int64_t)e * nchunks];
      c = (e + 1 < E ? hist[(int64_t)(e + 1) * nchunks] : R) - o;
      off[e] = o;
    }
    const int slot = block_scan_1024(c > 0 ? 1 : 0, &s_total);
    if (c > 0 && cnt_total + slot < E) {
      grp_expert[cnt_total + slot] = e;
      grp_row0[cnt_total + slot] = o;
      grp_rows[cnt_total + slot] = c;
    }
    cnt_total += s_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    off[E] = R;
    counters[0] = cnt_total;
  }
  __syncthreads();
  build_tiles(grp_expert, grp_row0, grp_rows, cnt_total, bm, max_tiles, tiles, counters + 1);
}

// Grouping, stage 3: stable scatter. Within a chunk, a slot's rank among equal
// experts comes from a wave-wide match (one ballot per id bit) plus the counts
// of the earlier waves of the chunk.
__global__ __launch_bounds__(256) void k_group_scatter(const int32_t *__restrict__ ids, int R, int E,
                                                       int nchunks,
                                                       const int32_t *__restrict__ base,
                                                       int32_t *__restrict__ sorted_slots,
                                                       int32_t *__restrict__ slot_pos) {
  __shared__ int cnt[4][kMaxE];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) cnt[i / E][i % E] = 0;
  __syncthreads();
  const int s = blockIdx.x * kChunk + threadIdx.x;
  const bool valid = s < R;
  const int e = valid ? ids[s] : E;  // E: sentinel shared by the idle lanes
  const int nbits = 32 - __clz(E);
  uint64_t m = ~0ull;
  for (int bit = 0; bit < nbits; ++bit) {
    const int on = (e >> bit) & 1;
    const uint64_t bal = __ballot(on);
    m &= on ? bal : ~bal;
  }
  const int rank = __popcll(m & lanemask_lt());
  if (valid && rank == 0) cnt[wave][e] = __popcll(m);
  __syncthreads();
  if (valid) {
    int pos = base[(int64_t)e * nchunks + blockIdx.x] + rank;
    for (int w = 0; w < wave; ++w) pos += cnt[w][e];
    if (pos >= 0 && pos < R) {  // always true for a consistent histogram
      sorted_slots[pos] = s;
      slot_pos[s] = pos;
    }
  }
}

// ---------------------------------------------------------------------------
// Small-batch routing tail (T <= kSmallT tokens, E <= kSmallE experts,
// T * E <= kSmallTE, T * k <= 1024) in one workgroup of 1024 threads: the
// token's logits copied to LDS, top-k + softmax by wave_topk (one wave per
// token, as k_topk), then one block scan for the expert offsets, the
// non-empty expert list and the MFMA tiles, and stable ranks by ballots.
// ---------------------------------------------------------------------------
constexpr int kSmallT = 32;
constexpr int kSmallE = 256;
constexpr int kSmallTE = 4096;  // bounds the LDS copy of the logits

__global__ __launch_bounds__(1024) void k_route_tail_small(const float *__restrict__ L, int T, int E,
                                                           int k, int renorm, int bm, int max_tiles,
                                                           RouteBufs o) {
  __shared__ __attribute__((aligned(16))) float Ls[kSmallTE];
  __shared__ int sel_id[kSmallT * kMaxTopK];
  __shared__ float sel_w[kSmallT * kMaxTopK];
  __shared__ int cnt[kSmallE];
  __shared__ int offs[kSmallE];
  __shared__ int wcnt[16][kSmallE];  // per wave: slots routed to each expert
  __shared__ int s_total;
  const int tid = threadIdx.x;
  const int R = T * k;
  const int Ep = (E + 3) & ~3;  // LDS row stride: 16-byte rows, padded with -inf
  for (int i = tid; i < T * Ep; i += 1024) {
    const int t = i / Ep, f = i - t * Ep;
    Ls[i] = f < E ? L[(int64_t)t * E + f] : -__builtin_inff();
  }
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  // top k of each token: one wave per token (wave_topk), weights included
  {
    const int wave = tid >> 6, lane = tid & 63;
    for (int t = wave; t < T; t += 16) {
      int my_id;
      float wgt;
      if (E <= 64)
        wave_topk<1>(Ls + t * Ep, E, k, renorm, my_id, wgt);
      else if (E <= 128)
        wave_topk<2>(Ls + t * Ep, E, k, renorm, my_id, wgt);
      else
        wave_topk<4>(Ls + t * Ep, E, k, renorm, my_id, wgt);
      if (lane < k) {
        sel_id[t * k + lane] = my_id;
        sel_w[t * k + lane] = wgt;
      }
    }
  }
  __syncthreads();
  if (tid < R) {
    o.topk_ids[tid] = sel_id[tid];
    o.topk_w[tid] = sel_w[tid];
    atomicAdd(&cnt[sel_id[tid]], 1);
  }
  // zero the per-wave expert counts of the stable ranking below
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
  __syncthreads();
  // One scan gives each expert its first sorted row (11 bits: R <= 1024), its
  // slot in the non-empty expert list (9 bits: E <= 256) and its first tile
  // (11 bits: at most R + E tiles).
  const int c = tid < E ? cnt[tid] : 0;
  const int nt = (c + bm - 1) / bm;
  const int ex = block_scan_1024(c | ((c > 0 ? 1 : 0) << 11) | (nt << 20), &s_total);
  const int off = ex & 0x7ff, slot = (ex >> 11) & 0x1ff, tile0 = ex >> 20;
  if (tid < E) {
    offs[tid] = off;
    o.expert_offsets[tid] = off;
  }
  if (tid == 0) {
    o.expert_offsets[E] = R;
    o.counters[0] = (s_total >> 11) & 0x1ff;
    o.counters[1] = min(s_total >> 20, max_tiles);
  }
  if (c > 0) {
    o.grp_expert[slot] = tid;
    o.grp_row0[slot] = off;
    o.grp_rows[slot] = c;
    for (int i = 0; i < nt && tile0 + i < max_tiles; ++i)
      o.tiles[tile0 + i] = make_int4(tid, off + i * bm, min(bm, c - i * bm), c);
  }
  // Stable position of slot s among the slots routed to its expert: its rank
  // among equal ids in its wave (one ballot per id bit) plus the counts of
  // the earlier waves.
  const int wave = tid >> 6;
  const bool valid = tid < R;
  const int e = valid ? sel_id[tid] : E;  // E: sentinel shared by the idle lanes
  uint64_t m = ~0ull;
  for (int bit = 0; bit < 9; ++bit) {
    const int on = (e >> bit) & 1;
    const uint64_t bal = __ballot(on);
    m &= on ? bal : ~bal;
  }
  const int rank = __popcll(m & lanemask_lt());
  if (valid && rank == 0) wcnt[wave][e] = __popcll(m);
  __syncthreads();
  if (valid) {
    int pos = offs[e] + rank;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
    o.sorted_slots[pos] = tid;
    o.slot_pos[tid] = pos;
  }
}

hipError_t launch_route(const float *logits, int T, int E, int k, int renorm, const RouteBufs &rb,
                        int bm, hipStream_t s) {
  const int R = T * k;
  if (T <= kSmallT && E <= kSmallE && T * ((E + 3) & ~3) <= kSmallTE && R <= 1024) {
    const int max_tiles = (int)cdiv(R, bm) + (R < E ? R : E);
    hipLaunchKernelGGL(k_route_tail_small, dim3(1), dim3(1024), 0, s, logits, T, E, k, renorm, bm,
                       max_tiles, rb);
    return hipGetLastError();
  }
  const dim3 tk((unsigned)cdiv(T, 4));
  if (E <= 64)
    hipLaunchKernelGGL(k_topk<1>, tk, dim3(256), 0, s, logits, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else if (E <= 128)
    hipLaunchKernelGGL(k_topk<2>, tk, dim3(256), 0, s, logits, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk<4>, tk, dim3(256), 0, s, logits, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_topk<8>, tk, dim3(256), 0, s, logits, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else
    hipLaunchKernelGGL(k_topk<16>, tk, dim3(256), 0, s, logits, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  const int nchunks = (int)cdiv(R, kChunk);
  hipLaunchKernelGGL(k_group_hist, dim3(nchunks), dim3(256), 0, s, rb.topk_ids, R, E, nchunks,
                     rb.chunk_hist);
  const int max_tiles = (int)cdiv(R, bm) + (R < E ? R : E);
  hipLaunchKernelGGL(k_group_scan, dim3(1), dim3(1024), 0, s, rb.chunk_hist, E, nchunks, R, bm,
                     max_tiles, rb.expert_offsets, rb.grp_expert, rb.grp_row0, rb.grp_rows, rb.counters,
                     rb.tiles);
  hipLaunchKernelGGL(k_group_scatter, dim3(nchunks), dim3(256), 0, s, rb.topk_ids, R, E, nchunks,
                     rb.chunk_hist, rb.sorted_slots, rb.slot_pos);
  return hipGetLastError();
}

// Caller-given groups (the grouped GEMM entry point): group g = rows
// [off[g], off[g+1]) with expert gexp[g] (or g). Offsets are clamped to [0, R]
// and groups naming an expert outside [0, E) are treated as empty, so a bad
// table cannot make a kernel read or write out of bounds.
__global__ __launch_bounds__(1024) void k_groups_from_offsets(const int32_t *__restrict__ goff,
                                                              const int32_t *__restrict__ gexp,
                                                              int G, int R, int E, int bm,
                                                              int max_tiles,
                                                              int32_t *__restrict__ grp_expert,
                                                              int32_t *__restrict__ grp_row0,
                                                              int32_t *__restrict__ grp_rows,
                                                              int32_t *__restrict__ counters,
                                                              int4 *__restrict__ tiles) {
  for (int g = threadIdx.x; g < G; g += 1024) {
    int a = goff[g], b = goff[g + 1];
    a = min(max(a, 0), R);
    b = min(max(b, a), R);
    const int e = gexp ? gexp[g] : g;
    const bool ok = e >= 0 && e < E;
    grp_expert[g] = ok ? e : 0;
    grp_row0[g] = a;
    grp_rows[g] = ok ? b - a : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) counters[0] = G;
  build_tiles(grp_expert, grp_row0, grp_rows, G, bm, max_tiles, tiles, counters + 1);
}

__global__ void k_fill_i32(int32_t *p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t *p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_groups_from_offsets(const int32_t *goff, const int32_t *gexp, int G, int R,
                                      int E, const RouteBufs &rb, int bm, hipStream_t s) {
  const int max_tiles = (int)cdiv(R, bm) + G;
  hipLaunchKernelGGL(k_groups_from_offsets, dim3(1), dim3(1024), 0, s, goff, gexp, G, R, E, bm,
                     max_tiles, rb.grp_expert, rb.grp_row0, rb.grp_rows, rb.counters, rb.tiles);
  return hipGetLastError();
}

}  // namespace nf4moe
