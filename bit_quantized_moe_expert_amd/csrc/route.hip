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
    // Tokens in batches of up to 16: the batch's loads (clamped to a valid row,
    // no branch) are all issued before the first is used.
    constexpr int BT = TMAX < 16 ? TMAX : 16;
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
// Router logits on the matrix cores, H split into S chunks. Each wave takes
// one unit (32 tokens, 32 experts, one chunk) and writes the chunk's partial
// sums P[s][t][e]; a consumer adds the S partials in chunk order (then the
// bias), so a token's logit depends on its own row only: the same bits for
// every T and every tile position. x is bf16, an exact MFMA operand; each fp32
// router weight is split in registers into three bf16 parts w = w1 + w2 + w3
// (w1 = w truncated to bf16, w2 = the remainder truncated, w3 = what is left,
// at most 8 significant bits: exact for weights of normal range), and the
// three products accumulate in fp32 in three accumulators, added at the end.
// The four waves of a workgroup are consecutive units (expert tile fastest),
// so with E <= 128 they share one x chunk through L1.
// ---------------------------------------------------------------------------
typedef __bf16 lg_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float lg_f32x16_t __attribute__((ext_vector_type(16)));

int router_split(int H) {
  const int steps = H / 16;                       // H % 16 == 0
  const int s = steps < kRouterSplit ? steps : kRouterSplit;
  const int chunk = (int)cdiv(steps, s) * 16;
  return (int)cdiv(H, chunk);
}
int router_chunk(int H) {
  const int steps = H / 16;
  const int s = steps < kRouterSplit ? steps : kRouterSplit;
  return (int)cdiv(steps, s) * 16;
}

// (hi halves of a and b) as one word: the truncated bf16 of two floats
__device__ inline uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int MB, int B>
__global__ __launch_bounds__(256) void k_logits_ks(const uint16_t *__restrict__ x, int T, int H,
                                                   const float *__restrict__ W, int E, int chunk,
                                                   int S, float *__restrict__ P) {
  // MB: 32-token blocks per wave (each weight split once for all of them);
  // B: k-steps of 16 whose loads are issued together.
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ET = (E + 31) >> 5;
  const int64_t u = (int64_t)blockIdx.x * 4 + wave;
  const int et = (int)(u % ET);
  const int64_t r = u / ET;
  const int s = (int)(r % S);
  const int64_t tt = r / S;
  if (tt * 32 * MB >= T) return;  // uniform over the wave
  const int g = lane >> 5, l32 = lane & 31;
  const int e = et * 32 + l32;
  const int64_t wrow = e < E ? e : E - 1;
  const int kb = s * chunk, ke = kb + chunk < H ? kb + chunk : H;
  const uint16_t *xa[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t t = (tt * MB + mb) * 32 + l32;
    xa[mb] = x + (t < T ? t : T - 1) * H + 8 * g;  // rows past the end compute on a valid row, never stored
  }
  const float *wa = W + wrow * H + 8 * g;
  lg_f32x16_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = lg_f32x16_t{};
  for (int k0 = kb; k0 < ke; k0 += 16 * B) {
    uint4 av[B][MB];
    float4 w0[B], w1[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {  // clamped to the chunk's last step: always in bounds
      const int k = k0 + 16 * i < ke ? k0 + 16 * i : ke - 16;
      w0[i] = *reinterpret_cast<const float4 *>(wa + k);
      w1[i] = *reinterpret_cast<const float4 *>(wa + k + 4);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[i][mb] = *reinterpret_cast<const uint4 *>(xa[mb] + k);
    }
    // Every step of the batch is computed; a step past the chunk (the last
    // batch of a chunk that is not a multiple of 16 * B) has its weight
    // operands zeroed. The mask is opaque to the compiler: with a branch per
    // step instead, it sinks each step's loads into the branch, and the
    // steps become one memory round trip each.
#pragma unroll
    for (int i = 0; i < B; ++i) {
      uint32_t keep = k0 + 16 * i < ke ? 0xffffffffu : 0u;
      asm volatile("" : "+v"(keep));
      const float wf[8] = {w0[i].x, w0[i].y, w0[i].z, w0[i].w, w1[i].x, w1[i].y, w1[i].z, w1[i].w};
      uint32_t q1[8], q2[8], q3[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t b0 = __float_as_uint(wf[j]) & keep;
        const float r1 = __uint_as_float(b0) - __uint_as_float(b0 & 0xffff0000u);
        const uint32_t b1 = __float_as_uint(r1);
        const float r2 = r1 - __uint_as_float(b1 & 0xffff0000u);
        q1[j] = b0;
        q2[j] = b1;
        q3[j] = __float_as_uint(r2);
      }
      uint4 p1, p2, p3;
      p1.x = pack_hi16(q1[0], q1[1]); p1.y = pack_hi16(q1[2], q1[3]);
      p1.z = pack_hi16(q1[4], q1[5]); p1.w = pack_hi16(q1[6], q1[7]);
      p2.x = pack_hi16(q2[0], q2[1]); p2.y = pack_hi16(q2[2], q2[3]);
      p2.z = pack_hi16(q2[4], q2[5]); p2.w = pack_hi16(q2[6], q2[7]);
      p3.x = pack_hi16(q3[0], q3[1]); p3.y = pack_hi16(q3[2], q3[3]);
      p3.z = pack_hi16(q3[4], q3[5]); p3.w = pack_hi16(q3[6], q3[7]);
      const lg_bf16x8_t b1v = __builtin_bit_cast(lg_bf16x8_t, p1);
      const lg_bf16x8_t b2v = __builtin_bit_cast(lg_bf16x8_t, p2);
      const lg_bf16x8_t b3v = __builtin_bit_cast(lg_bf16x8_t, p3);
      // a row's sum: per k-step w1, w2, w3 in that order into one accumulator
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(lg_bf16x8_t, av[i][mb]), b1v, acc[mb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(lg_bf16x8_t, av[i][mb]), b2v, acc[mb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(lg_bf16x8_t, av[i][mb]), b3v, acc[mb], 0, 0, 0);
    }
  }
  // 32x32 accumulator: lane holds expert column l32, token rows
  // 8 * (v / 4) + 4 * g + (v % 4) of each 32-token block.
  if (e >= E) return;
  float *Ps = P + (int64_t)s * T * E;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t tr = (tt * MB + mb) * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (tr < T) Ps[tr * E + e] = acc[mb][v];
    }
  }
}

// L[t][e] = (sum over s of P[s][t][e], in s order) + b[e]: the same bits as
// the top-k kernels' own sum of the partials.
__global__ __launch_bounds__(256) void k_logits_sum(const float *__restrict__ P, int S, int64_t n, int E,
                                                    const float *__restrict__ b, float *__restrict__ L) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = P[i];
  for (int s = 1; s < S; ++s) v += P[(int64_t)s * n + i];
  if (b) v += b[i % E];
  L[i] = v;
}

size_t router_partials_bytes(int T, int E, int H) {
  return (size_t)router_split(H) * (size_t)(T > 0 ? T : 1) * (size_t)E * sizeof(float);
}

hipError_t launch_router_partials(const uint16_t *x, int T, int H, const float *W, int E, float *P,
                                  hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int S = router_split(H), chunk = router_chunk(H);
  // 128 or 64 tokens per wave from 1024 tokens on (each weight split and read
  // once per 128 or 64 tokens; gpt-oss-shaped T = 2048: 27.5 against 38 us
  // with 32), the taller wave while it still gives a workgroup per CU, 32
  // below (more waves for the latency-bound smaller calls; Qwen3-shaped
  // T = 256 / 512: 9 us less routing than with 128). A row's arithmetic is the
  // same either way.
  const int64_t per128 = cdiv(T, 128) * (int64_t)S * cdiv(E, 32);
  if (T >= 1024 && cdiv(per128, 4) >= 256) {
    hipLaunchKernelGGL((k_logits_ks<4, 4>), dim3((unsigned)cdiv(per128, 4)), dim3(256), 0, s, x, T, H, W, E,
                       chunk, S, P);
  } else if (T >= 1024) {
    const int64_t units = cdiv(T, 64) * (int64_t)S * cdiv(E, 32);
    hipLaunchKernelGGL((k_logits_ks<2, 4>), dim3((unsigned)cdiv(units, 4)), dim3(256), 0, s, x, T, H, W, E,
                       chunk, S, P);
  } else {
    const int64_t units = cdiv(T, 32) * (int64_t)S * cdiv(E, 32);
    hipLaunchKernelGGL((k_logits_ks<1, 8>), dim3((unsigned)cdiv(units, 4)), dim3(256), 0, s, x, T, H, W, E,
                       chunk, S, P);
  }
  return hipGetLastError();
}

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

hipError_t launch_router_rows(const uint16_t *x, int T, int H, const float *W, const float *b, int E,
                              float *logits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (T == 1)  // one token: no idle token slots (the same per-token order)
    hipLaunchKernelGGL(k_logits_rows<1>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  else if (T <= 2)
    hipLaunchKernelGGL(k_logits_rows<2>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  else if (T <= 4)
    hipLaunchKernelGGL(k_logits_rows<4>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  else if (T <= 8)
    hipLaunchKernelGGL(k_logits_rows<8>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  else if (T <= 16)
    hipLaunchKernelGGL(k_logits_rows<16>, dim3(E), dim3(256), 0, s, x, T, H, W, b, E, logits);
  else
    hipLaunchKernelGGL(k_logits_rows<32>, dim3(E, (unsigned)cdiv(T, 32)), dim3(256), 0, s, x, T, H, W, b,
                       E, logits);
  return hipGetLastError();
}

hipError_t launch_router_logits(const uint16_t *x, int T, int H, const float *W, const float *b,
                                int E, float *logits, float *partials, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (partials) {
    hipError_t e = launch_router_partials(x, T, H, W, E, partials, s);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)T * E;
    hipLaunchKernelGGL(k_logits_sum, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, partials,
                       router_split(H), n, E, b, logits);
    return hipGetLastError();
  }
  if (T <= kRowsLogitsMaxT) return launch_router_rows(x, T, H, W, b, E, logits, s);
  hipLaunchKernelGGL(k_logits_tiled, dim3((unsigned)cdiv(T, 32), (unsigned)cdiv(E, 64)), dim3(256), 0, s,
                     x, T, H, W, b, E, logits);
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
// float_order_key (common.h) gives the keys.

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

// Where a token's logits come from: P[t * E + e] summed with the partials
// P[s * stride + t * E + e], s = 1 .. S-1, in s order, then + bias[e] (S = 1
// and no bias: given logits).
struct LogitSrc {
  const float *P;
  int64_t stride;
  int S;
  const float *bias;
};

__device__ inline float logit_at(const LogitSrc &L, int64_t i, int e) {
  float v = L.P[i];
  for (int s = 1; s < L.S; ++s) v += L.P[(int64_t)s * L.stride + i];
  if (L.bias) v += L.bias[e];
  return v;
}

// get(e): logit of expert e (e < E) of this wave's token.
template <int EPL, class Get>
__device__ inline void wave_topk(Get get, int E, int k, int renorm, int &my_id, float &wgt) {
  const int lane = threadIdx.x & 63;
  float v[EPL];
  uint32_t key[EPL];  // 0: no expert, or already picked (below every logit's key)
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? get(e) : -__builtin_inff();
    // key 0 belongs to one NaN bit pattern only; it ties with key 1 (another
    // NaN) instead, so that 0 stays the marker
    key[j] = e < E ? max(float_order_key(v[j]), 1u) : 0u;
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
__global__ __launch_bounds__(256) void k_topk(LogitSrc L, int T, int E, int k, int renorm,
                                              int32_t *__restrict__ ids, float *__restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  int my_id;
  float wgt;
  const int64_t row = (int64_t)t * E;
  wave_topk<EPL>([&](int e) { return logit_at(L, row + e, e); }, E, k, renorm, my_id, wgt);
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

// Exclusive scan of a pair of 32-bit counts (low, high word) per thread
// across a 1024-thread block; *total receives the block totals.
__device__ inline uint64_t block_scan_1024_u64(uint64_t v, uint64_t *total) {
  __shared__ uint64_t wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const uint64_t w = lane < 16 ? wsum[lane] : 0;
    uint64_t wi = w;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const uint64_t o = __shfl_up(wi, d, kWave);
      if (lane >= d) wi += o;
    }
    if (lane < 16) wsum[lane] = wi - w;
    if (lane == 15) *total = wi;
  }
  __syncthreads();
  const uint64_t ex = wsum[wave] + inc - v;
  __syncthreads();
  return ex;
}

// The MFMA tile table comes in two orders, each of n_tiles entries:
//  - tiles[0, max_tiles): by group, within a group by rows (the n-tile-major
//    kernels and dgrad: consecutive tiles of an expert share its weights);
//  - tiles[max_tiles, 2 max_tiles): by class, the body a tile runs (0: more
//    than 64 rows, 1: 33 to 64, 2: at most 32), then as above, so that the
//    tile-major kernels start their longest tiles first and the short ones
//    fill the end of the launch instead of trailing alone.
// counters[1] = tiles, [2] = class 0 tiles, [3] = class 1 tiles.
__device__ inline int tile_class(int rows) { return rows > 64 ? 0 : (rows > 32 ? 1 : 2); }

// tiles of each class in a group of `rows` rows cut into tiles of bm rows
__device__ inline void group_tile_counts(int rows, int bm, int &c0, int &c1, int &c2) {
  const int full = rows / bm, rem = rows - full * bm;
  const int fc = tile_class(bm);
  c0 = fc == 0 ? full : 0;
  c1 = fc == 1 ? full : 0;
  c2 = fc == 2 ? full : 0;
  if (rem > 0) {
    const int rc = tile_class(rem);
    c0 += rc == 0;
    c1 += rc == 1;
    c2 += rc == 2;
  }
}

// the tiles of one group: first at pe in group order, first of each class at
// b0 / b1 / b2 in class order
__device__ inline void write_group_tiles(int e, int row0, int rows, int bm, int pe, int b0, int b1, int b2,
                                         int max_tiles, int4 *tiles) {
  const int full = rows / bm, rem = rows - full * bm;
  const int fc = tile_class(bm);
  const int fb = fc == 0 ? b0 : (fc == 1 ? b1 : b2);
  for (int i = 0; i < full; ++i) {
    const int4 t = make_int4(e, row0 + i * bm, bm, rows);
    if (pe + i < max_tiles) tiles[pe + i] = t;
    if (fb + i < max_tiles) tiles[max_tiles + fb + i] = t;
  }
  if (rem > 0) {
    const int4 t = make_int4(e, row0 + full * bm, rem, rows);
    const int rc = tile_class(rem);
    const int pos = (rc == 0 ? b0 : (rc == 1 ? b1 : b2)) + (rc == fc ? full : 0);
    if (pe + full < max_tiles) tiles[pe + full] = t;
    if (pos < max_tiles) tiles[max_tiles + pos] = t;
  }
}

// Tiles of at most bm rows for every group, in both orders; single workgroup
// of 1024 threads. n_tiles_out[0] = tiles, [1] / [2] = class 0 / 1 tiles.
__device__ void build_tiles(const int32_t *grp_expert, const int32_t *grp_row0,
                            const int32_t *grp_rows, int n_grp, int bm, int max_tiles, int4 *tiles,
                            int32_t *n_tiles_out) {
  __shared__ uint64_t s_t01;
  __shared__ int s_t2;
  int T0 = 0, T1 = 0, T2 = 0;
  if (n_grp > 1024) {  // class totals first: class 1 tiles start after every class 0 tile
    int a0 = 0, a1 = 0, a2 = 0;
    for (int g = threadIdx.x; g < n_grp; g += 1024) {
      int c0, c1, c2;
      group_tile_counts(grp_rows[g], bm, c0, c1, c2);
      a0 += c0;
      a1 += c1;
      a2 += c2;
    }
    block_scan_1024_u64((uint64_t)a0 | ((uint64_t)a1 << 32), &s_t01);
    block_scan_1024(a2, &s_t2);
    T0 = (int)(s_t01 & 0xffffffffu);
    T1 = (int)(s_t01 >> 32);
    T2 = s_t2;
  }
  int k0 = 0, k1 = 0, k2 = 0;  // tiles of each class before this round of groups
  for (int g0 = 0; g0 < n_grp; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    const int rows = g < n_grp ? grp_rows[g] : 0;
    int c0, c1, c2;
    group_tile_counts(rows, bm, c0, c1, c2);
    const uint64_t e01 = block_scan_1024_u64((uint64_t)c0 | ((uint64_t)c1 << 32), &s_t01);
    const int e2 = block_scan_1024(c2, &s_t2);
    const int t0 = (int)(s_t01 & 0xffffffffu), t1 = (int)(s_t01 >> 32), t2 = s_t2;
    if (n_grp <= 1024) {  // one round: its totals are the table's
      T0 = t0;
      T1 = t1;
      T2 = t2;
    }
    const int e0 = k0 + (int)(e01 & 0xffffffffu), e1 = k1 + (int)(e01 >> 32), ee2 = k2 + e2;
    if (rows > 0)
      write_group_tiles(grp_expert[g], grp_row0[g], rows, bm, e0 + e1 + ee2, e0, T0 + e1, T0 + T1 + ee2,
                        max_tiles, tiles);
    k0 += t0;
    k1 += t1;
    k2 += t2;
    __syncthreads();  // every thread has read the totals before the next scans
  }
  if (threadIdx.x == 0) {
    n_tiles_out[0] = min(T0 + T1 + T2, max_tiles);
    n_tiles_out[1] = T0;
    n_tiles_out[2] = T1;
  }
}

// Grouping, stage 2 (single workgroup): flat exclusive scan of the histogram,
// expert offsets, the compacted list of non-empty experts, and the MFMA tiles.
// A histogram of up to kScanLdsN entries is scanned in LDS (one round of
// coalesced loads; the group list also stays in LDS for the tiles), a larger
// one in place in global memory.
constexpr int kScanLdsN = 16384;

__global__ __launch_bounds__(1024) void k_group_scan(int32_t *__restrict__ hist, int E, int nchunks,
                                                     int R, int bm, int max_tiles,
                                                     int32_t *__restrict__ off,
                                                     int32_t *__restrict__ grp_expert,
                                                     int32_t *__restrict__ grp_row0,
                                                     int32_t *__restrict__ grp_rows,
                                                     int32_t *__restrict__ counters,
                                                     int4 *__restrict__ tiles) {
  __shared__ int sh[kScanLdsN];
  __shared__ int g_e[kMaxE], g_r0[kMaxE], g_n[kMaxE];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)E * nchunks;
  const bool in_lds = n <= kScanLdsN;  // uniform
  int *h = in_lds ? sh : hist;
  if (in_lds) {
    for (int i = tid; i < n; i += 1024) sh[i] = hist[i];
    __syncthreads();
  }
  // each thread scans a contiguous slice; the slice totals are block-scanned
  const int64_t per = (n + 1023) / 1024;
  const int64_t i0 = per * tid, i1 = min(n, i0 + per);
  int sum = 0;
  for (int64_t i = i0; i < i1; ++i) sum += h[i];
  int run = block_scan_1024(sum, &s_total);
  for (int64_t i = i0; i < i1; ++i) {
    const int v = h[i];
    h[i] = run;
    run += v;
  }
  __syncthreads();
  if (in_lds) {
    for (int i = tid; i < n; i += 1024) hist[i] = sh[i];
  }
  // expert offsets and the compacted non-empty experts (ascending id)
  int cnt_total = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + tid;
    int o = 0, c = 0;
    if (e < E) {
      o = h[(int64_t)e * nchunks];
      c = (e + 1 < E ? h[(int64_t)(e + 1) * nchunks] : R) - o;
      off[e] = o;
    }
    const int slot = block_scan_1024(c > 0 ? 1 : 0, &s_total);
    if (c > 0 && cnt_total + slot < E) {
      const int gi = cnt_total + slot;
      grp_expert[gi] = e;
      grp_row0[gi] = o;
      grp_rows[gi] = c;
      g_e[gi] = e;
      g_r0[gi] = o;
      g_n[gi] = c;
    }
    cnt_total += s_total;
    __syncthreads();
  }
  if (tid == 0) {
    off[E] = R;
    counters[0] = cnt_total;
  }
  __syncthreads();
  build_tiles(g_e, g_r0, g_n, cnt_total, bm, max_tiles, tiles, counters + 1);
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
// Routing in one workgroup of 1024 threads for up to kTailR routed slots and
// E <= kSmallE experts. TOPK (up to 1024 slots): the tokens' logits are copied
// to LDS when they fit (T * E <= kSmallTE, else read from L2) and ranked by
// wave_topk (one wave per token, as k_topk), weights included; otherwise the
// ids come from topk_ids, written by k_topk before. Then one block scan gives
// the expert offsets, the non-empty expert list and the MFMA tiles, and
// ballots give the stable ranks, 1024 slots per pass with the per-expert
// counts of the earlier passes carried in LDS.
// ---------------------------------------------------------------------------
constexpr int kSmallR = 1024;   // routed slots ranked in one pass (one per thread)
// Routed slots grouped by the one-workgroup tail; above it the three-launch
// grouping. Measured against it: routing stage 32.1 -> 28.6 us at 2048 slots
// (Qwen3-shaped T = 256), even at 4096, 5 us slower at 8192.
constexpr int kTailR = 4096;
constexpr int kSmallE = 256;
constexpr int kSmallTE = 4096;  // bounds the LDS copy of the logits (else read from L2)
// Up to this many tokens the one-workgroup kernel also ranks the experts;
// above it the ranking runs in parallel (k_topk, one wave per token) first:
// a single workgroup ranking 128 tokens took 27 us against ~5 us.
constexpr int kTailTopkMaxT = 16;

template <bool TOPK>
__global__ __launch_bounds__(1024) void k_route_tail_small(LogitSrc L, int T, int E, int k, int renorm,
                                                           int bm, int max_tiles, RouteBufs o) {
  constexpr int kR = TOPK ? kSmallR : kTailR;
  __shared__ __attribute__((aligned(16))) float Ls[TOPK ? kSmallTE : 4];
  __shared__ int sel_id[kR];
  __shared__ float sel_w[TOPK ? kSmallR : 4];
  __shared__ int cnt[kSmallE];
  __shared__ int offs[kSmallE];   // first sorted row of each expert, plus the earlier passes' slots
  __shared__ int wcnt[16][kSmallE];  // per wave of a pass: slots routed to each expert
  __shared__ uint64_t s_total64;
  const int tid = threadIdx.x;
  const int R = T * k;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  if constexpr (TOPK) {
    const int Ep = (E + 3) & ~3;  // LDS row stride: 16-byte rows, padded with -inf
    const bool in_lds = T * Ep <= kSmallTE;  // uniform
    if (in_lds) {  // every load issued before the first LDS store
      float v[kSmallTE / 1024];
#pragma unroll
      for (int r = 0; r < kSmallTE / 1024; ++r) {
        const int i = tid + r * 1024, t = i / Ep, f = i - t * Ep;
        v[r] = i < T * Ep && f < E ? logit_at(L, (int64_t)t * E + f, f) : -__builtin_inff();
      }
#pragma unroll
      for (int r = 0; r < kSmallTE / 1024; ++r)
        if (tid + r * 1024 < T * Ep) Ls[tid + r * 1024] = v[r];
    }
    __syncthreads();
    // top k of each token: one wave per token (wave_topk), weights included
    const int wave = tid >> 6, lane = tid & 63;
    for (int t = wave; t < T; t += 16) {
      int my_id;
      float wgt;
      const float *lrow = Ls + t * Ep;
      const int64_t grow = (int64_t)t * E;
      auto get = [&](int e) { return in_lds ? lrow[e] : logit_at(L, grow + e, e); };
      if (E <= 64)
        wave_topk<1>(get, E, k, renorm, my_id, wgt);
      else if (E <= 128)
        wave_topk<2>(get, E, k, renorm, my_id, wgt);
      else
        wave_topk<4>(get, E, k, renorm, my_id, wgt);
      if (lane < k) {
        sel_id[t * k + lane] = my_id;
        sel_w[t * k + lane] = wgt;
      }
    }
  }
  __syncthreads();
  for (int s0 = 0; s0 < R; s0 += 1024) {
    const int sl = s0 + tid;
    if (sl < R) {
      int id;
      if constexpr (TOPK) {
        id = sel_id[sl];
        o.topk_ids[sl] = id;
        o.topk_w[sl] = sel_w[sl];
      } else {
        id = o.topk_ids[sl];  // from k_topk: always in [0, E)
        sel_id[sl] = id;
      }
      atomicAdd(&cnt[id], 1);
    }
  }
  __syncthreads();
  // One scan gives each expert its first sorted row (14 bits: R <= kTailR) and
  // its slot in the non-empty expert list (9 bits: E <= 256), and in the high
  // word its first tile of each class (10 bits each: at most R / 65 + 64 tiles
  // of class 0, R / 33 + 128 of class 1, E of class 2).
  const int c = tid < E ? cnt[tid] : 0;
  int c0, c1, c2;
  group_tile_counts(c, bm, c0, c1, c2);
  const uint64_t ex64 = block_scan_1024_u64(
      (uint64_t)(c | ((c > 0 ? 1 : 0) << 14)) | ((uint64_t)(c0 | (c1 << 10) | (c2 << 20)) << 32), &s_total64);
  const int ex = (int)(ex64 & 0xffffffffu), exc = (int)(ex64 >> 32);
  const int tot = (int)(s_total64 & 0xffffffffu), totc = (int)(s_total64 >> 32);
  const int off = ex & 0x3fff, slot = (ex >> 14) & 0x1ff;
  const int n_grp = (tot >> 14) & 0x1ff;
  const int T0 = totc & 0x3ff, T1 = (totc >> 10) & 0x3ff, T2 = totc >> 20;
  if (tid < E) {
    offs[tid] = off;
    o.expert_offsets[tid] = off;
  }
  if (tid == 0) {
    o.expert_offsets[E] = R;
    o.counters[0] = n_grp;
    o.counters[1] = min(T0 + T1 + T2, max_tiles);
    o.counters[2] = T0;
    o.counters[3] = T1;
  }
  if (c > 0) {
    o.grp_expert[slot] = tid;
    o.grp_row0[slot] = off;
    o.grp_rows[slot] = c;
    const int e0 = exc & 0x3ff, e1 = (exc >> 10) & 0x3ff, e2 = exc >> 20;
    write_group_tiles(tid, off, c, bm, e0 + e1 + e2, e0, T0 + e1, T0 + T1 + e2, max_tiles, o.tiles);
  }
  // Stable position of slot s among the slots routed to its expert: the
  // expert's first row plus the slots of earlier passes (carried in offs),
  // the counts of the earlier waves of this pass, and its rank among equal
  // ids in its wave (one ballot per id bit).
  const int wave = tid >> 6;
  for (int s0 = 0; s0 < R; s0 += 1024) {
    for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int sl = s0 + tid;
    const bool valid = sl < R;
    const int e = valid ? sel_id[sl] : E;  // E: sentinel shared by the idle lanes
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
      o.sorted_slots[pos] = sl;
      o.slot_pos[sl] = pos;
    }
    __syncthreads();
    if (tid < E) {  // this pass's slots of each expert come before the next pass's
      int n = 0;
      for (int w = 0; w < 16; ++w) n += wcnt[w][tid];
      offs[tid] += n;
    }
    __syncthreads();  // wcnt and offs are read before the next pass rewrites them
  }
}

static hipError_t launch_topk(const LogitSrc &L, int T, int E, int k, int renorm, const RouteBufs &rb,
                              hipStream_t s) {
  const dim3 tk((unsigned)cdiv(T, 4));
  if (E <= 64)
    hipLaunchKernelGGL(k_topk<1>, tk, dim3(256), 0, s, L, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else if (E <= 128)
    hipLaunchKernelGGL(k_topk<2>, tk, dim3(256), 0, s, L, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk<4>, tk, dim3(256), 0, s, L, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_topk<8>, tk, dim3(256), 0, s, L, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  else
    hipLaunchKernelGGL(k_topk<16>, tk, dim3(256), 0, s, L, T, E, k, renorm, rb.topk_ids, rb.topk_w);
  return hipGetLastError();
}

static hipError_t launch_route_src(const LogitSrc &L, int T, int E, int k, int renorm, const RouteBufs &rb,
                                   int bm, hipStream_t s) {
  const int R = T * k;
  const bool one_wg = E <= kSmallE && R <= kTailR;
  const int max_tiles = (int)cdiv(R, bm) + (R < E ? R : E);
  if (one_wg && T <= kTailTopkMaxT && R <= kSmallR) {
    hipLaunchKernelGGL(k_route_tail_small<true>, dim3(1), dim3(1024), 0, s, L, T, E, k, renorm, bm,
                       max_tiles, rb);
    return hipGetLastError();
  }
  hipError_t e = launch_topk(L, T, E, k, renorm, rb, s);
  if (e != hipSuccess) return e;
  if (one_wg) {
    hipLaunchKernelGGL(k_route_tail_small<false>, dim3(1), dim3(1024), 0, s, L, T, E, k, renorm, bm,
                       max_tiles, rb);
    return hipGetLastError();
  }
  const int nchunks = (int)cdiv(R, kChunk);
  hipLaunchKernelGGL(k_group_hist, dim3(nchunks), dim3(256), 0, s, rb.topk_ids, R, E, nchunks,
                     rb.chunk_hist);
  hipLaunchKernelGGL(k_group_scan, dim3(1), dim3(1024), 0, s, rb.chunk_hist, E, nchunks, R, bm,
                     max_tiles, rb.expert_offsets, rb.grp_expert, rb.grp_row0, rb.grp_rows, rb.counters,
                     rb.tiles);
  hipLaunchKernelGGL(k_group_scatter, dim3(nchunks), dim3(256), 0, s, rb.topk_ids, R, E, nchunks,
                     rb.chunk_hist, rb.sorted_slots, rb.slot_pos);
  return hipGetLastError();
}

hipError_t launch_route(const float *logits, int T, int E, int k, int renorm, const RouteBufs &rb,
                        int bm, hipStream_t s) {
  return launch_route_src(LogitSrc{logits, (int64_t)T * E, 1, nullptr}, T, E, k, renorm, rb, bm, s);
}

hipError_t launch_route_partials(const float *partials, int S, const float *bias, int T, int E, int k,
                                 int renorm, const RouteBufs &rb, int bm, hipStream_t s) {
  return launch_route_src(LogitSrc{partials, (int64_t)T * E, S, bias}, T, E, k, renorm, rb, bm, s);
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
