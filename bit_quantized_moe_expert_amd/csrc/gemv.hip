// Small-M grouped GEMM on 4-bit packed weights: the bandwidth-bound path for
// decode-sized routed batches.
//
// What it computes is the pages' gemm_4bit_grouped (page "How do I run a
// grouped GEMM directly on NF4 packed MoE expert weights ...", sections "Why it
// happens" and "Supported scope": nibble -> codebook decode in registers,
// block scale, fp32 accumulation, one launch for every active expert; "One-token
// groups take the GEMV path"). The design is ours, for gfx950:
//  - a lane owns fixed 32-element K chunks of a weight row and streams them with
//    16-byte loads, so a wave reads whole rows coalesced; the activations of
//    those K positions stay in registers as fp32 for every row the wave visits;
//  - a packed byte is decoded by one LDS lookup into a 256-entry table of
//    (even-k value, odd-k value) fp32 pairs, replicated 32 times so the lanes
//    of an access hit distinct banks; the block scale multiplies the per-chunk
//    partial sum, so each weight costs one lookup per two codes and one FMA;
//  - partial sums meet in a wave reduction; SwiGLU (gate row n with up row
//    n + I) or the routing weight is applied before the store.
#include "common.h"
#include "internal.h"

namespace nf4moe {

constexpr int kGemvRep = 32;  // LDS table replicas

// Sum over aligned groups of LPR lanes (LPR a power of two <= 64).
template <int LPR>
__device__ inline float seg_sum(float v) {
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int FMT>
__device__ inline float block_scale(const void *scale, int64_t idx) {
  if (FMT == 0) return reinterpret_cast<const float *>(scale)[idx];
  return e8m0_to_f32(reinterpret_cast<const uint8_t *>(scale)[idx]);
}

// Load 32 activations (one 16-byte weight chunk's K range) as fp32.
template <int AF32>
__device__ inline void load_act32(const void *a, int64_t off, float *xr) {
  if (AF32) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = p[i];
      xr[4 * i + 0] = v.x;
      xr[4 * i + 1] = v.y;
      xr[4 * i + 2] = v.z;
      xr[4 * i + 3] = v.w;
    }
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = p[i];
      xr[8 * i + 0] = bf16lo_to_f32(v.x);
      xr[8 * i + 1] = bf16hi_to_f32(v.x);
      xr[8 * i + 2] = bf16lo_to_f32(v.y);
      xr[8 * i + 3] = bf16hi_to_f32(v.y);
      xr[8 * i + 4] = bf16lo_to_f32(v.z);
      xr[8 * i + 5] = bf16hi_to_f32(v.z);
      xr[8 * i + 6] = bf16lo_to_f32(v.w);
      xr[8 * i + 7] = bf16hi_to_f32(v.w);
    }
  }
}

// Dot product of one 16-byte chunk of codes (32 weights) with 32 activations
// for MS activation rows at once; each byte is looked up once.
template <int MS>
__device__ inline void chunk_dot(const float2 *tab, uint4 q, const float (*xr)[32], float *dot) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int bsel = 0; bsel < 4; ++bsel) {
      const uint32_t byte = (w[d] >> (8 * bsel)) & 0xffu;
      const float2 p = tab[byte * kGemvRep];
      const int k = 8 * d + 2 * bsel;
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        dot[m] = fmaf(xr[m][k], p.x, dot[m]);
        dot[m] = fmaf(xr[m][k + 1], p.y, dot[m]);
      }
    }
  }
}

// One workgroup = 4 waves; blockIdx.y = group, blockIdx.x = block of output
// columns. Each wave reads NL wave-loads of weight rows (RPL rows per
// wave-load when a row is shorter than 64 chunks; at most 16 rows and 8
// 16-byte loads in flight per lane) and applies them to the group's rows MS at
// a time.
template <int FMT, int EPI, int AF32, int LPR, int NJ, int MS>
__global__ __launch_bounds__(256) void k_gemv(GemmArgs p) {
  constexpr int RPL = 64 / LPR;
  constexpr int NL = (8 / NJ) < (16 / RPL) ? (8 / NJ) : (16 / RPL);
  constexpr int WR = NL * RPL;                       // weight rows per wave (<= 16)
  constexpr int RPU = (EPI == EPI_SWIGLU) ? 2 : 1;   // weight rows per output column
  constexpr int UPW = WR / RPU;                      // output columns per wave
  static_assert(MS * UPW <= 64, "one lane per output");
  __shared__ float2 tab_all[256 * kGemvRep];

  const int gi = blockIdx.y;
  const int ngrp = p.n_grp ? *p.n_grp : p.max_grp;
  if (gi >= ngrp) return;                            // uniform over the workgroup
  const int rows = p.grp_rows[gi];
  if (rows <= 0) return;
  build_pair_table<FMT, kGemvRep>(tab_all);
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = p.grp_expert[gi], row0 = p.grp_row0[gi];
  const int64_t ncol = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
  const int64_t u0 = ((int64_t)blockIdx.x * 4 + wave) * UPW;
  if (u0 >= ncol) return;                            // no barrier follows
  const float2 *tab = tab_all + (lane & (kGemvRep - 1));
  const int sr = lane / LPR, li = lane % LPR;
  const int64_t nch = p.K / 32;                      // 16-byte chunks per row
  const int64_t rowbytes = p.K / 2;
  const uint8_t *Be = p.B + (int64_t)e * p.N * rowbytes;
  const int64_t sc_per_row = p.K / Fmt<FMT>::kBlock;
  const int64_t sc_base = (int64_t)e * p.N * sc_per_row;

  // Issue every weight load of this wave first.
  uint4 wq[NL][NJ];
  float sc[NL][NJ];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = i * RPL + sr;                      // position in the wave's row list
    int64_t col, wrow;
    if (EPI == EPI_SWIGLU) {
      col = u0 + (q >> 1);
      wrow = (q & 1) ? col + ncol : col;
    } else {
      col = u0 + q;
      wrow = col;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t c = li + (int64_t)LPR * j;
      if (col < ncol && c < nch) {
        wq[i][j] = *reinterpret_cast<const uint4 *>(Be + wrow * rowbytes + c * 16);
        const int64_t sidx = FMT == 0 ? (c >> 1) : c;
        sc[i][j] = block_scale<FMT>(p.B_scale, sc_base + wrow * sc_per_row + sidx);
      } else {
        wq[i][j] = make_uint4(0, 0, 0, 0);
        sc[i][j] = 0.0f;
      }
    }
  }

  const int my_m = lane / UPW, my_u = lane % UPW;
  for (int m0 = 0; m0 < rows; m0 += MS) {
    float xr[MS][NJ][32];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const int r = row0 + m0 + m;
      const bool live = (m0 + m) < rows;
      int64_t arow = r;
      if (live && p.a_row_of) arow = p.a_row_of[r] / p.a_div;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t c = li + (int64_t)LPR * j;
        if (live && c < nch) {
          load_act32<AF32>(p.a, arow * p.K + c * 32, xr[m][j]);
        } else {
#pragma unroll
          for (int t = 0; t < 32; ++t) xr[m][j][t] = 0.0f;
        }
      }
    }
    float acc[MS][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
#pragma unroll
      for (int m = 0; m < MS; ++m) acc[m][i] = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float xj[MS][32];
#pragma unroll
        for (int m = 0; m < MS; ++m)
#pragma unroll
          for (int t = 0; t < 32; ++t) xj[m][t] = xr[m][j][t];
        float dot[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) dot[m] = 0.0f;
        chunk_dot<MS>(tab, wq[i][j], xj, dot);
#pragma unroll
        for (int m = 0; m < MS; ++m) acc[m][i] = fmaf(sc[i][j], dot[m], acc[m][i]);
      }
#pragma unroll
      for (int m = 0; m < MS; ++m) acc[m][i] = seg_sum<LPR>(acc[m][i]);
    }
    // Route each finished row value to the lane that stores it.
    float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int q = 0; q < WR; ++q) {
        const float v = RPL == 1 ? acc[m][q] : __shfl(acc[m][q / RPL], (q % RPL) * LPR, kWave);
        if (my_m == m) {
          if (EPI == EPI_SWIGLU) {
            if (q == 2 * my_u) v0 = v;
            if (q == 2 * my_u + 1) v1 = v;
          } else if (q == my_u) {
            v0 = v;
          }
        }
      }
    }
    if (lane < MS * UPW) {
      const int64_t col = u0 + my_u;
      const int mm = m0 + my_m;
      if (mm < rows && col < ncol) {
        const int64_t r = row0 + mm;
        if (EPI == EPI_SWIGLU) {
          const float hval = v0 / (1.0f + expf(-v0)) * v1;
          reinterpret_cast<float *>(p.c)[r * ncol + col] = hval;
        } else if (EPI == EPI_PLAIN_F32) {
          reinterpret_cast<float *>(p.c)[r * ncol + col] = v0;
        } else if (EPI == EPI_PLAIN_BF16) {
          reinterpret_cast<uint16_t *>(p.c)[r * ncol + col] = (uint16_t)f32_to_bf16_rne(v0);
        } else {
          const int64_t slot = p.slot_of[r];
          reinterpret_cast<float *>(p.c)[slot * ncol + col] = p.slot_w[slot] * v0;
        }
      }
    }
  }
}

template <int FMT, int EPI, int AF32, int LPR, int NJ, int MS>
static void launch_gemv_t(const GemmArgs &g, hipStream_t s) {
  constexpr int RPL = 64 / LPR;
  constexpr int NL = (8 / NJ) < (16 / RPL) ? (8 / NJ) : (16 / RPL);
  constexpr int WR = NL * RPL;
  constexpr int UPW = WR / ((EPI == EPI_SWIGLU) ? 2 : 1);
  const int64_t ncol = (EPI == EPI_SWIGLU) ? g.N / 2 : g.N;
  const dim3 grid((unsigned)cdiv(ncol, 4 * UPW), (unsigned)g.max_grp);
  hipLaunchKernelGGL((k_gemv<FMT, EPI, AF32, LPR, NJ, MS>), grid, dim3(256), 0, s, g);
}

template <int FMT, int EPI, int AF32, int LPR, int NJ>
static hipError_t pick_ms(const GemmArgs &g, int ms, hipStream_t s) {
  if constexpr (NJ == 2) {
    launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 1>(g, s);  // two chunks per lane: one row at a time
  } else {
    if (ms <= 1)
      launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 1>(g, s);
    else if (ms == 2)
      launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 2>(g, s);
    else
      launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 4>(g, s);
  }
  return hipGetLastError();
}

template <int FMT, int EPI, int AF32>
static hipError_t pick_shape(const GemmArgs &g, int ms, hipStream_t s) {
  const int64_t nch = g.K / 32;
  if (nch > 64) {
    if (nch > 128) return hipErrorInvalidValue;
    return pick_ms<FMT, EPI, AF32, 64, 2>(g, ms, s);
  }
  if (nch > 32) return pick_ms<FMT, EPI, AF32, 64, 1>(g, ms, s);
  if (nch > 16) return pick_ms<FMT, EPI, AF32, 32, 1>(g, ms, s);
  return pick_ms<FMT, EPI, AF32, 16, 1>(g, ms, s);
}

template <int FMT>
static hipError_t pick_epi(const GemmArgs &g, int ms, hipStream_t s) {
  switch (g.epi) {
    case EPI_SWIGLU:
      return g.a_is_f32 ? pick_shape<FMT, EPI_SWIGLU, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_SWIGLU, 0>(g, ms, s);
    case EPI_PLAIN_F32:
      return g.a_is_f32 ? pick_shape<FMT, EPI_PLAIN_F32, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_PLAIN_F32, 0>(g, ms, s);
    case EPI_PLAIN_BF16:
      return g.a_is_f32 ? pick_shape<FMT, EPI_PLAIN_BF16, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_PLAIN_BF16, 0>(g, ms, s);
    default:
      return g.a_is_f32 ? pick_shape<FMT, EPI_SLOT, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_SLOT, 0>(g, ms, s);
  }
}

hipError_t launch_gemv_grouped(const GemmArgs &g, int ms_hint, hipStream_t s) {
  if (g.max_grp <= 0) return hipSuccess;
  return g.fmt == 0 ? pick_epi<0>(g, ms_hint, s) : pick_epi<1>(g, ms_hint, s);
}

// ---------------------------------------------------------------------------
// Token-centric down projection fused with the router-weighted combine, for a
// handful of tokens: out[t, n] = bf16( sum_j w[t,j] * h[pos(t,j)] . W2[e_j][n] ).
// A workgroup owns RB output rows of one token; the k (slot, chunk) pairs of a
// row are spread over the 4 waves, each lane keeping its slot's activations
// (already multiplied by the routing weight) in registers; the four wave
// partials of a row are added in wave order, so the result is deterministic.
// ---------------------------------------------------------------------------
template <int FMT, int NQ, int RB>
__global__ __launch_bounds__(256) void k_down_combine(const float *__restrict__ h,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const int32_t *__restrict__ topk_ids,
                                                      const float *__restrict__ topk_w, int T,
                                                      int k, const uint8_t *__restrict__ w2,
                                                      const void *__restrict__ w2s, int H, int I,
                                                      uint16_t *__restrict__ out) {
  __shared__ float2 tab_all[256 * kGemvRep];
  __shared__ float red[4][RB];
  build_pair_table<FMT, kGemvRep>(tab_all);
  __syncthreads();
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * RB;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float2 *tab = tab_all + (lane & (kGemvRep - 1));
  const int nch = I / 32;
  const int Q = k * nch;
  const int QW = (Q + 3) / 4;
  const int64_t rowbytes = I / 2;
  const int64_t sc_per_row = I / Fmt<FMT>::kBlock;

  float hv[NQ][32];
  const uint8_t *wbase[NQ];
  int64_t sbase[NQ];
  bool live[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const int ql = qi * 64 + lane;
    const int q = wave * QW + ql;
    live[qi] = ql < QW && q < Q;
    const int j = live[qi] ? q / nch : 0;
    const int c = live[qi] ? q % nch : 0;
    const int slot = t * k + j;
    const int e = topk_ids[slot];
    const float wj = topk_w[slot];
    const int64_t r = slot_pos[slot];
    if (live[qi]) {
      load_act32<1>(h, r * I + (int64_t)c * 32, hv[qi]);
#pragma unroll
      for (int i = 0; i < 32; ++i) hv[qi][i] *= wj;
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) hv[qi][i] = 0.0f;
    }
    wbase[qi] = w2 + (int64_t)e * H * rowbytes + (int64_t)c * 16;
    sbase[qi] = (int64_t)e * H * sc_per_row + (FMT == 0 ? (c >> 1) : c);
  }
  uint4 wq[RB][NQ];
  float sc[RB][NQ];
#pragma unroll
  for (int n = 0; n < RB; ++n) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int row = n0 + n;
      if (live[qi] && row < H) {
        wq[n][qi] = *reinterpret_cast<const uint4 *>(wbase[qi] + (int64_t)row * rowbytes);
        sc[n][qi] = block_scale<FMT>(w2s, sbase[qi] + (int64_t)row * sc_per_row);
      } else {
        wq[n][qi] = make_uint4(0, 0, 0, 0);
        sc[n][qi] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int n = 0; n < RB; ++n) {
    float acc = 0.0f;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      float dot = 0.0f;
      float xj[1][32];
#pragma unroll
      for (int i = 0; i < 32; ++i) xj[0][i] = hv[qi][i];
      chunk_dot<1>(tab, wq[n][qi], xj, &dot);
      acc = fmaf(sc[n][qi], dot, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) red[wave][n] = acc;
  }
  __syncthreads();
  if (threadIdx.x < RB && n0 + (int)threadIdx.x < H) {
    const int n = threadIdx.x;
    const float v = ((red[0][n] + red[1][n]) + red[2][n]) + red[3][n];
    out[(int64_t)t * H + n0 + n] = (uint16_t)f32_to_bf16_rne(v);
  }
}

hipError_t launch_gemv_down_combine(int fmt, const float *h, const int32_t *slot_pos,
                                    const int32_t *topk_ids, const float *topk_w, int T, int k,
                                    const uint8_t *w2, const void *w2_scale, int H, int I,
                                    uint16_t *out, hipStream_t s) {
  constexpr int RB = 8;
  const int Q = k * (I / 32);
  const int QW = (Q + 3) / 4;
  const dim3 grid((unsigned)cdiv(H, RB), (unsigned)T);
  if (QW > 128) return hipErrorInvalidValue;
  if (QW > 64) {
    if (fmt == 0)
      hipLaunchKernelGGL((k_down_combine<0, 2, RB>), grid, dim3(256), 0, s, h, slot_pos, topk_ids,
                         topk_w, T, k, w2, w2_scale, H, I, out);
    else
      hipLaunchKernelGGL((k_down_combine<1, 2, RB>), grid, dim3(256), 0, s, h, slot_pos, topk_ids,
                         topk_w, T, k, w2, w2_scale, H, I, out);
  } else {
    if (fmt == 0)
      hipLaunchKernelGGL((k_down_combine<0, 1, RB>), grid, dim3(256), 0, s, h, slot_pos, topk_ids,
                         topk_w, T, k, w2, w2_scale, H, I, out);
    else
      hipLaunchKernelGGL((k_down_combine<1, 1, RB>), grid, dim3(256), 0, s, h, slot_pos, topk_ids,
                         topk_w, T, k, w2, w2_scale, H, I, out);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: out[t, n] = bf16( sum_{j ascending} slotbuf[t*k + j, n] ), fp32 sum.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ slotbuf, int T, int k,
                                                 int H, uint16_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one float4 of one token
  const int64_t per_tok = H / 4;
  if (i >= (int64_t)T * per_tok) return;
  const int64_t t = i / per_tok, n4 = i % per_tok;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float4 v = reinterpret_cast<const float4 *>(slotbuf + (t * k + j) * H)[n4];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const uint32_t lo = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
  const uint32_t hi = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
  reinterpret_cast<uint2 *>(out + t * H)[n4] = make_uint2(lo, hi);
}

hipError_t launch_combine(const float *slotbuf, int T, int k, int H, uint16_t *out, hipStream_t s) {
  const int64_t n = (int64_t)T * (H / 4);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, slotbuf, T, k, H, out);
  return hipGetLastError();
}

}  // namespace nf4moe
