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

// Expert weights are read once per call: non-temporal 16-byte loads, so the
// stream of codes does not push out of the caches the small operands that the
// next kernels and the next call read again (router weights, logits,
// activations, h).
__device__ inline uint4 load_stream16(const uint8_t *p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int FMT>
__device__ inline float block_scale(const void *scale, int64_t idx) {
  return Fmt<FMT>::value(Fmt<FMT>::raw(scale, idx));
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
// for MS activation rows at once; each byte is one v_perm (table address) and
// one 8-byte LDS read, then two FMAs per activation row.
template <int MS>
__device__ inline void chunk_dot(const char *tab, uint32_t lanebyte, uint4 q, const float (*xr)[32],
                                 float *dot) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int bsel = 0; bsel < 4; ++bsel) {
      const float2 p = *reinterpret_cast<const float2 *>(tab + tab_offset(w[d], lanebyte, bsel));
      const int k = 8 * d + 2 * bsel;
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        dot[m] = fmaf(xr[m][k], p.x, dot[m]);
        dot[m] = fmaf(xr[m][k + 1], p.y, dot[m]);
      }
    }
  }
}

// One workgroup = kGemvWaves waves; blockIdx.y = group, blockIdx.x = block of
// output columns. Each wave reads NL wave-loads of weight rows (RPL rows per
// wave-load when a row is shorter than 64 chunks; at most 16 rows and 8
// 16-byte loads in flight per lane) and applies them to the group's rows MS at
// a time. Weight and first activation loads are issued before the LDS table is
// built, so the table build overlaps their latency.
constexpr int kGemvWaves = 8;
constexpr int kGemvWavesRoute = kGemvWaves;  // waves sharing the one-token ranking
// Grouped launches (many groups, several rounds of workgroups) use 4-wave
// workgroups so two fit on a CU next to each other's 64 KB table.
template <int ROUTE>
constexpr int gemv_waves() { return ROUTE > 0 ? kGemvWaves : 4; }

// Wave-loads (16 bytes per lane each) a wave keeps in flight: 8 / NJ, at most
// 16 rows per wave, and 4 when four activation rows are held in registers.
template <int LPR, int NJ, int MS>
constexpr int gemv_loads() {
  constexpr int a = 8 / NJ, b = 16 / (64 / LPR), c = MS >= 4 ? (LPR == 16 ? 2 : 4) : 8;
  return a < b ? (a < c ? a : c) : (b < c ? b : c);
}
// One token (ROUTE > 0): at most 4, so the few routed experts' rows spread
// over twice the workgroups (an OLMoE-shaped token: 512 of 8 waves, 2 per CU; against 8 wave-
// loads, the gate_up kernel 9.25 -> 8.86 us). Rows of two chunks per lane
// (2048 < K <= 4096) take 6 rows per wave: a gpt-oss-shaped token's 4 x 5760
// gate_up rows at 4 rows per wave need 5760 waves, more than the 4096 that
// are resident at once, so the launch ran in 1.4 rounds; at 6 it is 480
// workgroups, one round (the chunk-major loop below keeps the registers under
// the 128 that 16 waves per CU allow).
template <int LPR, int NJ, int MS, int ROUTE>
constexpr int gemv_wave_loads() {
  constexpr int n = gemv_loads<LPR, NJ, MS>();
  return ROUTE > 0 ? (NJ == 2 && MS == 1 ? 6 : (n > 4 ? 4 : n)) : n;
}

// Routing of a single token inside the gate_up kernel, spread over the
// kGemvWaves waves of a workgroup. Rank of expert e under (logit descending,
// id ascending), compared on float_order_key so that the order is total for
// any logits (NaN included) and the ranks of the E experts are a permutation
// of 0..E-1 = number of experts f ordered before it; wave w counts the f in
// its slice of E / kGemvWaves ids (route_partial), the partial counts meet in
// LDS across the workgroup barrier, and route_finish sums them, selects the k
// experts, and returns the expert of group `gi` (the gi-th selected id in
// ascending order). With publish set, wave 0 also writes every routing output
// (ids, weights, offsets, permutation, group list, tiles) for the kernels that
// follow.
template <int EPL>
struct RouteToken {
  float v[EPL];      // logit of expert lane + 64 j (-inf past E)
  int rank[EPL];     // its rank (set by route_finish)
  uint64_t sel[EPL]; // ballot of the selected experts (set by route_finish)
};

template <int EPL>
__device__ inline RouteToken<EPL> route_load(const GemmArgs &p) {
  RouteToken<EPL> r;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    r.v[j] = e < p.route_E ? p.route_logits[e] : -__builtin_inff();
  }
  return r;
}

template <int EPL>
__device__ inline void route_partial(const GemmArgs &p, const RouteToken<EPL> &r, int wave,
                                     int (*s_rank)[64 * EPL]) {
  constexpr int S = 64 * EPL / kGemvWavesRoute;   // ids per wave slice
  const int lane = threadIdx.x & 63;
  const int E = p.route_E;
  int cnt[EPL];
  uint32_t kv[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) cnt[j] = 0;
  float uu[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {                     // all loads first, clamped, no branches
    const int f = wave * S + i;                     // wave-uniform
    uu[i] = p.route_logits[f < E ? f : E - 1];
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) kv[j] = max(float_order_key(r.v[j]), 1u);  // as wave_topk
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int f = wave * S + i;
    if (f >= E) continue;                           // wave-uniform: ids past E count for no one
    const uint32_t ku = max(float_order_key(uu[i]), 1u);
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      cnt[j] += (ku > kv[j] || (ku == kv[j] && f < e)) ? 1 : 0;
    }
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) s_rank[wave][lane + 64 * j] = cnt[j];
}

template <int EPL>
__device__ inline int route_finish(const GemmArgs &p, RouteToken<EPL> &r, int gi,
                                   const int (*s_rank)[64 * EPL]) {
  const int lane = threadIdx.x & 63;
  const int E = p.route_E, k = p.route_k;
  int *rank = r.rank;
  uint64_t *sel = r.sel;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    rank[j] = 0;
#pragma unroll
    for (int w = 0; w < kGemvWavesRoute; ++w) rank[j] += s_rank[w][lane + 64 * j];
    sel[j] = __ballot(lane + 64 * j < E && rank[j] < k);
  }
  // expert of group gi: the selected id with gi selected ids below it
  int e_gi = 0, below = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const bool chosen = (sel[j] >> lane) & 1;
    const uint64_t hit = __ballot(chosen && below + __popcll(sel[j] & lanemask_lt()) == gi);
    if (hit) e_gi = 64 * j + __builtin_ctzll(hit);
    below += __popcll(sel[j]);
  }
  return e_gi;
}

// Routing outputs of the token for the kernels that follow (one wave of one
// workgroup calls it, after its own weight loads are in flight).
template <int EPL>
__device__ inline void route_publish(const GemmArgs &p, const RouteToken<EPL> &r) {
  const int lane = threadIdx.x & 63;
  const int E = p.route_E, k = p.route_k;
  const int *rank = r.rank;
  const uint64_t *sel = r.sel;
  {
    float vmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j < E && rank[j] == 0) vmax = r.v[j];
    vmax = wave_max(vmax);
    // The denominator in the routing kernels' one order: selected experts by
    // rank, or every expert by id.
    float ex[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) ex[j] = lane + 64 * j < E ? expf(r.v[j] - vmax) : 0.0f;
    float denom = 0.0f;
    if (p.route_renorm) {
      for (int q = 0; q < k; ++q) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const uint64_t hit = __ballot(lane + 64 * j < E && rank[j] == q);
          if (hit) denom += __shfl(ex[j], (int)__builtin_ctzll(hit), kWave);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        for (int l = 0; l < 64 && 64 * j + l < E; ++l) denom += __shfl(ex[j], l, kWave);
    }
    const RouteBufs &o = p.route_out;
    int bl = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      const int pos_e = bl + __popcll(sel[j] & lanemask_lt());  // selected ids < e
      const bool chosen = (sel[j] >> lane) & 1;
      if (e < E) o.expert_offsets[e] = pos_e;
      if (chosen) {
        const int rk = rank[j];
        o.topk_ids[rk] = e;
        o.topk_w[rk] = expf(r.v[j] - vmax) / denom;
        o.slot_pos[rk] = pos_e;
        o.sorted_slots[pos_e] = rk;
        o.grp_expert[pos_e] = e;
        o.grp_row0[pos_e] = pos_e;
        o.grp_rows[pos_e] = 1;
        o.tiles[pos_e] = make_int4(e, pos_e, 1, 1);
      }
      bl += __popcll(sel[j]);
    }
    if (lane == 0) {
      o.expert_offsets[E] = k;
      o.counters[0] = k;
      o.counters[1] = k;  // one-row tiles: all of class 2
      o.counters[2] = 0;
      o.counters[3] = 0;
    }
  }
}

// One workgroup = kGemvWaves waves; blockIdx.y = group, blockIdx.x = block of
// output columns. Grouped (ROUTE = 0): the group's activation and weight loads
// are issued first and the LDS table is built while they fly; the barrier
// after it orders LDS only. One token (ROUTE > 0): the logits load, table build
// and partial ranks come first, and the weight stream starts right after the
// barrier, once every wave knows its expert.
// XF: the extended gate_up / down epilogue (clamped GLU, interleaved gate and
// up rows, per-expert biases); XF = 0 instantiates the plain SwiGLU kernel.
template <int FMT, int EPI, int AF32, int LPR, int NJ, int MS, int ROUTE, int XF>
__global__ __launch_bounds__(gemv_waves<ROUTE>() * 64) void k_gemv(GemmArgs p) {
  constexpr int NWV = gemv_waves<ROUTE>();
  constexpr int RPL = 64 / LPR;
  constexpr int NL = gemv_wave_loads<LPR, NJ, MS, ROUTE>();
  constexpr int WR = NL * RPL;                       // weight rows per wave (<= 16)
  constexpr int RPU = (EPI == EPI_SWIGLU) ? 2 : 1;   // weight rows per output column
  constexpr int UPW = WR / RPU;                      // output columns per wave
  static_assert(MS * UPW <= 64, "one lane per output");
  __shared__ float2 tab_all[256 * kGemvRep];
  __shared__ int s_rank[(ROUTE > 0 ? kGemvWavesRoute : 1)][64 * (ROUTE > 0 ? ROUTE : 1)];

  const int gi = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  int e, row0, rows;
  RouteToken<(ROUTE > 0 ? ROUTE : 1)> rt;
  if constexpr (ROUTE > 0) {
    if (gi >= p.route_k) return;                     // uniform over the workgroup
    rt = route_load<ROUTE>(p);                        // in flight during the table build
    e = 0;
    row0 = gi;
    rows = 1;
  } else {
    const int ngrp = p.n_grp ? *p.n_grp : p.max_grp;
    if (gi >= ngrp) return;                          // uniform over the workgroup
    rows = p.grp_rows[gi];
    if (rows <= 0) return;
    e = p.grp_expert[gi];
    row0 = p.grp_row0[gi];
  }
  const int64_t ncol = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
  const int64_t u0 = ((int64_t)blockIdx.x * NWV + wave) * UPW;
  const bool wave_live = u0 < ncol;                  // uniform per wave
  if constexpr (ROUTE > 0) {
    // Table build and partial ranks while the logits load; one barrier; then
    // every wave knows its expert and starts the weight stream.
    build_pair_table<FMT, kGemvRep>(tab_all, 0, NWV);
    route_partial<ROUTE>(p, rt, wave, s_rank);
    lds_barrier();
    e = route_finish<ROUTE>(p, rt, gi, s_rank);
  }
  const int sr = lane / LPR, li = lane % LPR;
  const int64_t nch = p.K / 32;                      // 16-byte chunks per row
  const int64_t rowbytes = p.K / 2;
  const uint8_t *Be = p.B + (int64_t)e * p.N * rowbytes;
  const int64_t sc_per_row = p.K / Fmt<FMT>::kBlock;
  const int64_t sc_base = (int64_t)e * p.N * sc_per_row;

  // Activations: raw loads first (bf16 bits or fp32), converted only once the
  // weight loads below are in flight.
  constexpr int XW = AF32 ? 8 : 4;                   // 16-byte words per 32 activations
  uint4 xraw[MS][NJ][XW];
  auto issue_x = [&](int m0) {
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const bool live = (m0 + m) < rows;
      const int r = row0 + (live ? m0 + m : 0);
      int64_t arow = ROUTE > 0 ? 0 : r;
      if (ROUTE == 0 && p.a_row_of) {                // a bad index cannot read past a
        arow = p.a_row_of[r] / p.a_div;
        arow = arow < 0 ? 0 : (arow < p.a_rows ? arow : p.a_rows - 1);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t c = li + (int64_t)LPR * j;
        const int64_t off = arow * p.K + (c < nch ? c : 0) * 32;
        const uint4 *src = AF32 ? reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(p.a) + off)
                                : reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.a) + off);
#pragma unroll
        for (int w = 0; w < XW; ++w) xraw[m][j][w] = src[w];
      }
    }
  };
  // Values in lanes past the row end or rows past the group are finite (the
  // addresses are clamped) and never reach an output: their chunks carry a zero
  // scale and their rows are not stored.
  float xr[MS][NJ][32];
  auto convert_x = [&]() {
#pragma unroll
    for (int m = 0; m < MS; ++m) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int w = 0; w < XW; ++w) {
          const uint4 v = xraw[m][j][w];
          if (AF32) {
            xr[m][j][4 * w + 0] = __uint_as_float(v.x);
            xr[m][j][4 * w + 1] = __uint_as_float(v.y);
            xr[m][j][4 * w + 2] = __uint_as_float(v.z);
            xr[m][j][4 * w + 3] = __uint_as_float(v.w);
          } else {
            xr[m][j][8 * w + 0] = bf16lo_to_f32(v.x);
            xr[m][j][8 * w + 1] = bf16hi_to_f32(v.x);
            xr[m][j][8 * w + 2] = bf16lo_to_f32(v.y);
            xr[m][j][8 * w + 3] = bf16hi_to_f32(v.y);
            xr[m][j][8 * w + 4] = bf16lo_to_f32(v.z);
            xr[m][j][8 * w + 5] = bf16hi_to_f32(v.z);
            xr[m][j][8 * w + 6] = bf16lo_to_f32(v.w);
            xr[m][j][8 * w + 7] = bf16hi_to_f32(v.w);
          }
        }
      }
    }
  };
  issue_x(0);
  if constexpr (MS > 1) convert_x();  // several rows: convert now, fewer live registers
  __builtin_amdgcn_sched_barrier(0);  // keep the activation loads first

  // Weight loads of this wave, after the activations and in row order (code,
  // then scale), so that row i waits only for its own data: vector loads
  // retire in issue order. Addresses are clamped into the expert's rows so
  // every load is unconditional; an out-of-range row or chunk gets scale 0.
  uint4 wq[NL][NJ];
  float sc[NL][NJ];
  bool sok[NL][NJ];
  int64_t wrow_of[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = i * RPL + sr;                      // position in the wave's row list
    int64_t col, wrow;
    if (EPI == EPI_SWIGLU) {
      col = u0 + (q >> 1);
      wrow = (XF && p.glu_inter) ? 2 * col + (q & 1) : ((q & 1) ? col + ncol : col);
    } else {
      col = u0 + q;
      wrow = col;
    }
    const bool rok = col < ncol;
    wrow_of[i] = rok ? wrow : 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) sok[i][j] = rok && li + (int64_t)LPR * j < nch;
  }
  // Scales of every row first (a few bytes each), then the code chunks in row
  // order. All unconditional: no branch may split the in-order accounting.
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t c = li + (int64_t)LPR * j;
      const int64_t cc = c < nch ? c : 0;
      const int64_t sidx = Fmt<FMT>::kBlock == 64 ? (cc >> 1) : cc;
      sc[i][j] = block_scale<FMT>(p.B_scale, sc_base + wrow_of[i] * sc_per_row + sidx);
    }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t c = li + (int64_t)LPR * j;
      const int64_t cc = c < nch ? c : 0;
      wq[i][j] = load_stream16(Be + wrow_of[i] * rowbytes + cc * 16);
      __builtin_amdgcn_sched_barrier(0);  // keep row order
    }
  __builtin_amdgcn_sched_barrier(0);  // every load is in flight before any wait
  if constexpr (ROUTE > 0) {
    if (blockIdx.x == 0 && gi == 0 && wave == 0) route_publish<ROUTE>(p, rt);
  }
  if constexpr (ROUTE == 0) {
    // The table build overlaps the loads' latency; the barrier orders LDS
    // only, so the loads stay in flight through it.
    build_pair_table<FMT, kGemvRep>(tab_all, 0, NWV);
    lds_barrier();
  }
  if (!wave_live) return;                            // no barrier follows

  const char *tab = reinterpret_cast<const char *>(tab_all);
  const uint32_t lanebyte = (uint32_t)(lane & (kGemvRep - 1)) * 8u;
  const int my_m = lane / UPW, my_u = lane % UPW;
  // One token with two chunks per lane: chunk-major, each chunk's activations
  // converted to fp32 just before its rows use them, so only one chunk is held
  // as fp32 (a row's arithmetic and order are those of the loop below: per
  // chunk j ascending, acc = fma(scale, dot, acc) from 0).
  constexpr bool kChunkMajor = ROUTE > 0 && NJ == 2 && MS == 1 && !AF32;
  for (int m0 = 0; m0 < rows; m0 += MS) {
    if constexpr (!kChunkMajor) {
      if (m0 > 0) {
        issue_x(m0);
        convert_x();
      } else if constexpr (MS == 1) {
        convert_x();
      }
    }
    float acc[MS][NL];
    if constexpr (kChunkMajor) {
#pragma unroll
      for (int i = 0; i < NL; ++i) acc[0][i] = 0.0f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float xj[1][32];
#pragma unroll
        for (int w = 0; w < XW; ++w) {
          const uint4 v = xraw[0][j][w];
          xj[0][8 * w + 0] = bf16lo_to_f32(v.x);
          xj[0][8 * w + 1] = bf16hi_to_f32(v.x);
          xj[0][8 * w + 2] = bf16lo_to_f32(v.y);
          xj[0][8 * w + 3] = bf16hi_to_f32(v.y);
          xj[0][8 * w + 4] = bf16lo_to_f32(v.z);
          xj[0][8 * w + 5] = bf16hi_to_f32(v.z);
          xj[0][8 * w + 6] = bf16lo_to_f32(v.w);
          xj[0][8 * w + 7] = bf16hi_to_f32(v.w);
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float dot = 0.0f;
          chunk_dot<1>(tab, lanebyte, wq[i][j], xj, &dot);
          acc[0][i] = fmaf(sok[i][j] ? sc[i][j] : 0.0f, dot, acc[0][i]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
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
        chunk_dot<MS>(tab, lanebyte, wq[i][j], xj, dot);
#pragma unroll
        for (int m = 0; m < MS; ++m) acc[m][i] = fmaf(sok[i][j] ? sc[i][j] : 0.0f, dot[m], acc[m][i]);
      }
      // keep the scheduler from hoisting every row's LDS lookups at once
      __builtin_amdgcn_sched_barrier(0);
    }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int m = 0; m < MS; ++m) acc[m][i] = seg_sum<LPR>(acc[m][i]);
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
          float hval;
          if constexpr (XF) {
            float gv = v0, uv = v1;
            if (p.bias) {
              const float *bb = p.bias + (int64_t)e * p.N;
              gv += bb[p.glu_inter ? 2 * col : col];
              uv += bb[p.glu_inter ? 2 * col + 1 : col + ncol];
            }
            hval = glu_value(p.glu, p.glu_alpha, p.glu_limit, gv, uv);
          } else {
            hval = sig_gate(v0, 1.0f) * v1;
          }
          reinterpret_cast<float *>(p.c)[r * ncol + col] = hval;
        } else if (EPI == EPI_PLAIN_F32) {
          reinterpret_cast<float *>(p.c)[r * ncol + col] = v0;
        } else if (EPI == EPI_PLAIN_BF16) {
          reinterpret_cast<uint16_t *>(p.c)[r * ncol + col] = (uint16_t)f32_to_bf16_rne(v0);
        } else {
          const int64_t slot = p.slot_of[r];
          const float y = (XF && p.bias) ? v0 + p.bias[(int64_t)e * p.N + col] : v0;
          reinterpret_cast<float *>(p.c)[slot * ncol + col] = p.slot_w[slot] * y;
        }
      }
    }
  }
}

template <int FMT, int EPI, int AF32, int LPR, int NJ, int MS, int ROUTE = 0, int XF = 0>
static void launch_gemv_t(const GemmArgs &g, hipStream_t s) {
  constexpr int RPL = 64 / LPR;
  constexpr int NL = gemv_wave_loads<LPR, NJ, MS, ROUTE>();
  constexpr int WR = NL * RPL;
  constexpr int UPW = WR / ((EPI == EPI_SWIGLU) ? 2 : 1);
  const int64_t ncol = (EPI == EPI_SWIGLU) ? g.N / 2 : g.N;
  constexpr int NWV = gemv_waves<ROUTE>();
  const dim3 grid((unsigned)cdiv(ncol, NWV * UPW), (unsigned)(ROUTE > 0 ? g.route_k : g.max_grp));
  NF4MOE_LAUNCH(g, (k_gemv<FMT, EPI, AF32, LPR, NJ, MS, ROUTE, XF>), grid, dim3(NWV * 64), s, g);
}

template <int FMT, int EPI, int AF32, int LPR, int NJ, int XF>
static hipError_t pick_ms(const GemmArgs &g, int ms, hipStream_t s) {
  if constexpr (NJ == 2) {
    launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 1, 0, XF>(g, s);  // two chunks per lane: one row at a time
  } else {
    if (ms <= 1)
      launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 1, 0, XF>(g, s);
    else if (ms == 2)
      launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 2, 0, XF>(g, s);
    else
      launch_gemv_t<FMT, EPI, AF32, LPR, NJ, 4, 0, XF>(g, s);
  }
  return hipGetLastError();
}

template <int FMT, int EPI, int AF32, int XF = 0>
static hipError_t pick_shape(const GemmArgs &g, int ms, hipStream_t s) {
  const int64_t nch = g.K / 32;
  if (nch > 64) {
    if (nch > 128) return hipErrorInvalidValue;
    return pick_ms<FMT, EPI, AF32, 64, 2, XF>(g, ms, s);
  }
  if (nch > 32) return pick_ms<FMT, EPI, AF32, 64, 1, XF>(g, ms, s);
  if (nch > 16) return pick_ms<FMT, EPI, AF32, 32, 1, XF>(g, ms, s);
  return pick_ms<FMT, EPI, AF32, 16, 1, XF>(g, ms, s);
}

// The extended epilogue is instantiated where the forward uses it: SwiGLU on
// bf16 activations (gate_up) and the slot output on fp32 ones (down).
inline bool extended_epilogue(const GemmArgs &g) { return g.glu != 0 || g.glu_inter != 0 || g.bias != nullptr; }

template <int FMT>
static hipError_t pick_epi(const GemmArgs &g, int ms, hipStream_t s) {
  const bool xf = extended_epilogue(g);
  switch (g.epi) {
    case EPI_SWIGLU:
      if (xf) return g.a_is_f32 ? hipErrorInvalidValue : pick_shape<FMT, EPI_SWIGLU, 0, 1>(g, ms, s);
      return g.a_is_f32 ? pick_shape<FMT, EPI_SWIGLU, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_SWIGLU, 0>(g, ms, s);
    case EPI_PLAIN_F32:
      if (xf) return hipErrorInvalidValue;
      return g.a_is_f32 ? pick_shape<FMT, EPI_PLAIN_F32, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_PLAIN_F32, 0>(g, ms, s);
    case EPI_PLAIN_BF16:
      if (xf) return hipErrorInvalidValue;
      return g.a_is_f32 ? pick_shape<FMT, EPI_PLAIN_BF16, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_PLAIN_BF16, 0>(g, ms, s);
    default:
      if (xf) return g.a_is_f32 ? pick_shape<FMT, EPI_SLOT, 1, 1>(g, ms, s) : hipErrorInvalidValue;
      return g.a_is_f32 ? pick_shape<FMT, EPI_SLOT, 1>(g, ms, s)
                        : pick_shape<FMT, EPI_SLOT, 0>(g, ms, s);
  }
}

template <int FMT, int XF>
static hipError_t launch_routed(const GemmArgs &g, hipStream_t s) {
  const int64_t nch = g.K / 32;
  const bool two = g.route_E > 64;
  if (nch > 128) return hipErrorInvalidValue;
  if (nch > 64) {
    if (two) launch_gemv_t<FMT, EPI_SWIGLU, 0, 64, 2, 1, 2, XF>(g, s);
    else launch_gemv_t<FMT, EPI_SWIGLU, 0, 64, 2, 1, 1, XF>(g, s);
  } else if (nch > 32) {
    if (two) launch_gemv_t<FMT, EPI_SWIGLU, 0, 64, 1, 1, 2, XF>(g, s);
    else launch_gemv_t<FMT, EPI_SWIGLU, 0, 64, 1, 1, 1, XF>(g, s);
  } else if (nch > 16) {
    if (two) launch_gemv_t<FMT, EPI_SWIGLU, 0, 32, 1, 1, 2, XF>(g, s);
    else launch_gemv_t<FMT, EPI_SWIGLU, 0, 32, 1, 1, 1, XF>(g, s);
  } else {
    if (two) launch_gemv_t<FMT, EPI_SWIGLU, 0, 16, 1, 1, 2, XF>(g, s);
    else launch_gemv_t<FMT, EPI_SWIGLU, 0, 16, 1, 1, 1, XF>(g, s);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const GemmArgs &g, int ms_hint, hipStream_t s) {
  if (g.route_logits) {
    if (g.epi != EPI_SWIGLU || g.a_is_f32 || g.route_E > 128 || g.route_k > kMaxTopK)
      return hipErrorInvalidValue;
    if (extended_epilogue(g))
      return g.fmt == 0 ? launch_routed<0, 1>(g, s) : g.fmt == 2 ? launch_routed<2, 1>(g, s) : launch_routed<1, 1>(g, s);
    return g.fmt == 0 ? launch_routed<0, 0>(g, s) : g.fmt == 2 ? launch_routed<2, 0>(g, s) : launch_routed<1, 0>(g, s);
  }
  if (g.max_grp <= 0) return hipSuccess;
  return g.fmt == 0 ? pick_epi<0>(g, ms_hint, s) : g.fmt == 2 ? pick_epi<2>(g, ms_hint, s) : pick_epi<1>(g, ms_hint, s);
}

// ---------------------------------------------------------------------------
// Token-centric down projection fused with the router-weighted combine, for a
// handful of tokens: out[t, n] = bf16( sum_j w[t,j] * h[pos(t,j)] . W2[e_j][n] ).
// It takes the same arithmetic steps, in the same order, as the grouped GEMV
// (slot output) followed by k_combine, so a token gets the same bits from
// either pair of kernels: per slot j, each of LPR lanes sums its chunks
// c = li + LPR * jj (jj < NJ; a chunk's 32-term dot times its block scale), the
// lanes meet in seg_sum<LPR>, s_j = w_j * y_j, and out = bf16 of the fp32 sum
// of s_0, s_1, ... from 0. A workgroup owns RB output rows of one token; its 4
// waves hold 4 * 64 / LPR lane segments, one slot each per pass (NP passes).
// ---------------------------------------------------------------------------
// NT: the weight loads are non-temporal (one token: every weight row is read
// once; with several tokens the tokens that share an expert read its rows
// again, and keeping them cached measured faster). RS: 4 * RS waves, the RB
// rows split between RS groups of 4 (each wave the same lane segments and
// slots, over RB / RS rows), for one token with two chunks per lane, whose
// 4 waves otherwise each decode 8 rows of 2 chunks in sequence, at 158
// VGPRs, with few waves per CU.
template <int FMT, int LPR, int NJ, int NP, int RB, int XF, int NT, int RS>
__global__ __launch_bounds__(256 * RS) void k_down_combine(const float *__restrict__ h,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const int32_t *__restrict__ topk_ids,
                                                      const float *__restrict__ topk_w, int T,
                                                      int k, const uint8_t *__restrict__ w2,
                                                      const void *__restrict__ w2s, int H, int I,
                                                      uint16_t *__restrict__ out,
                                                      const float *__restrict__ b2) {
  constexpr int SPW = 64 / LPR;      // lane segments per wave
  constexpr int NSEG = 4 * SPW;      // slots per pass
  __shared__ float2 tab_all[256 * kGemvRep];
  __shared__ float red[kMaxTopK][RB];
  const int t = blockIdx.y;
  const int n0 = blockIdx.x * RB;
  static_assert(RS >= 1 && RS <= 4 && RB % RS == 0, "row split");
  constexpr int RW = RB / RS;        // rows per wave
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wave = wave_all & 3, rg = wave_all >> 2;  // slot wave, row group
  const int seg = wave * SPW + lane / LPR, li = lane % LPR;
  const int nr0 = rg * RW;           // this wave's first row within the workgroup's RB
  const int nch = I / 32;
  const int64_t rowbytes = I / 2;
  const int64_t sc_per_row = I / Fmt<FMT>::kBlock;

  // Routing metadata first (written by the previous kernel), the LDS table
  // built while it arrives, then addresses.
  bool live[NP];
  int eraw[NP], praw[NP];
  float wj[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int j = q * NSEG + seg;
    live[q] = j < k;
    const int slot = t * k + (live[q] ? j : 0);
    eraw[q] = topk_ids[slot];
    wj[q] = topk_w[slot];
    praw[q] = slot_pos[slot];
  }
  __builtin_amdgcn_sched_barrier(0);
  build_pair_table<FMT, kGemvRep>(tab_all, 0, 4 * RS);
  __builtin_amdgcn_sched_barrier(0);
  // Chunks past the row end read chunk 0 and get scale 0, as in the GEMV.
  bool cok[NJ];
  int64_t cc[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int c = li + LPR * jj;
    cok[jj] = c < nch;
    cc[jj] = cok[jj] ? c : 0;
  }
  // Loads: activations first, then weights in row order (vector loads retire
  // in issue order, so row n waits only for its own data); all unconditional
  // from clamped addresses.
  uint4 hraw[NP][NJ][8];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const uint4 *src = reinterpret_cast<const uint4 *>(h + (int64_t)praw[q] * I + cc[jj] * 32);
#pragma unroll
      for (int w = 0; w < 8; ++w) hraw[q][jj][w] = src[w];
    }
  uint4 wq[RW][NP][NJ];
  float sc[RW][NP][NJ];
#pragma unroll
  for (int n = 0; n < RW; ++n) {
    const int row = n0 + nr0 + n;
    const int64_t rc = row < H ? row : H - 1;
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int64_t eb = (int64_t)eraw[q] * H;
        const uint8_t *wp = w2 + (eb + rc) * rowbytes + cc[jj] * 16;
        if constexpr (NT)
          wq[n][q][jj] = load_stream16(wp);
        else
          wq[n][q][jj] = *reinterpret_cast<const uint4 *>(wp);
        sc[n][q][jj] = block_scale<FMT>(w2s, (eb + rc) * sc_per_row + (Fmt<FMT>::kBlock == 64 ? (cc[jj] >> 1) : cc[jj]));
      }
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is in flight before any wait
  lds_barrier();                      // the table is complete; the loads stay in flight
  const char *tab = reinterpret_cast<const char *>(tab_all);
  const uint32_t lanebyte = (uint32_t)(lane & (kGemvRep - 1)) * 8u;
#pragma unroll
  for (int n = 0; n < RW; ++n) {
    const int nn = nr0 + n;          // row within the workgroup
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      float acc = 0.0f;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        float xj[1][32];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          xj[0][4 * w + 0] = __uint_as_float(hraw[q][jj][w].x);
          xj[0][4 * w + 1] = __uint_as_float(hraw[q][jj][w].y);
          xj[0][4 * w + 2] = __uint_as_float(hraw[q][jj][w].z);
          xj[0][4 * w + 3] = __uint_as_float(hraw[q][jj][w].w);
        }
        float dot = 0.0f;
        chunk_dot<1>(tab, lanebyte, wq[n][q][jj], xj, &dot);
        acc = fmaf((cok[jj] && n0 + nn < H) ? sc[n][q][jj] : 0.0f, dot, acc);
      }
      acc = seg_sum<LPR>(acc);
      if constexpr (XF) acc += b2[(int64_t)eraw[q] * H + (n0 + nn < H ? n0 + nn : H - 1)];
      if (li == 0 && live[q]) red[q * NSEG + seg][nn] = wj[q] * acc;
    }
  }
  lds_barrier();
  if (threadIdx.x < RB && n0 + (int)threadIdx.x < H) {
    const int n = threadIdx.x;
    float v = 0.0f;
    for (int j = 0; j < k; ++j) v += red[j][n];
    out[(int64_t)t * H + n0 + n] = (uint16_t)f32_to_bf16_rne(v);
  }
}

template <int FMT, int LPR, int NJ, int NP, int RB, int NT = 0, int RS = 1>
static void launch_down_combine_rb(const float *h, const int32_t *slot_pos, const int32_t *topk_ids,
                                   const float *topk_w, int T, int k, const uint8_t *w2,
                                   const void *w2_scale, const float *b2, int H, int I, uint16_t *out,
                                   hipStream_t s) {
  const dim3 grid((unsigned)cdiv(H, RB), (unsigned)T);
  if (b2)
    hipLaunchKernelGGL((k_down_combine<FMT, LPR, NJ, NP, RB, 1, NT, RS>), grid, dim3(256 * RS), 0, s, h,
                       slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, H, I, out, b2);
  else
    hipLaunchKernelGGL((k_down_combine<FMT, LPR, NJ, NP, RB, 0, NT, RS>), grid, dim3(256 * RS), 0, s, h,
                       slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, H, I, out, b2);
}

// Output rows per workgroup: the smallest of 4, 8, 12 that keeps the grid
// within two workgroups per CU (T * H / RB <= 512), else 16: a one-token
// OLMoE- or Qwen3-shaped layer (H = 2048) runs 512 workgroups of 4 rows, a
// gpt-oss-shaped one (H = 2880) 360 of 8, two tokens 512 of 8 or 480 of 12,
// more tokens rows of 16 (same box, T = 4 / 8 against 12: OLMoE-shaped
// 44.7 / 66.6 -> 43.2 / 64.3 us; 24 was slower). A row's arithmetic does not
// depend on how many rows share its workgroup.
template <int FMT, int LPR, int NJ, int NP>
static void launch_down_combine_t(const float *h, const int32_t *slot_pos, const int32_t *topk_ids,
                                  const float *topk_w, int T, int k, const uint8_t *w2,
                                  const void *w2_scale, const float *b2, int H, int I, uint16_t *out,
                                  hipStream_t s) {
  constexpr int64_t kMaxWG = 512;
  // one token: non-temporal weight loads (OLMoE-shaped layer 17.64 -> 16.9 us,
  // Qwen3-shaped 17.77 -> 16.77, gpt-oss-shaped 43.0 -> 41.3, same box, the
  // gate_up loads non-temporal too); T = 1 takes 4 or 8 rows for H <= 4096
  // One token with two chunks per lane (I > 2048): 12 rows per workgroup over
  // three groups of 4 waves (4 rows per wave), 240 workgroups, one per CU at
  // the gpt-oss shape (against 8 rows over 8 waves, 360 workgroups of which
  // 104 CUs ran two: gpt-oss-shaped T = 1 layer 35.7 -> 34.05 us, down +
  // combine 17.5 -> 15.8 us; 6 rows over 8 waves, 480 workgroups: 34.1 us).
  if constexpr (NJ == 2) {
    if (T == 1) {
      launch_down_combine_rb<FMT, LPR, NJ, NP, 12, 1, 3>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
      return;
    }
  }
  if ((int64_t)T * cdiv(H, 4) <= kMaxWG) {
    if (T == 1)
      launch_down_combine_rb<FMT, LPR, NJ, NP, 4, 1>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
    else
      launch_down_combine_rb<FMT, LPR, NJ, NP, 4>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  } else if ((int64_t)T * cdiv(H, 8) <= kMaxWG) {
    if (T == 1)
      launch_down_combine_rb<FMT, LPR, NJ, NP, 8, 1>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
    else
      launch_down_combine_rb<FMT, LPR, NJ, NP, 8>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  }
  else if ((int64_t)T * cdiv(H, 12) <= kMaxWG)
    launch_down_combine_rb<FMT, LPR, NJ, NP, 12>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  else
    launch_down_combine_rb<FMT, LPR, NJ, NP, 16>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
}

// Lane-segment shape of the grouped GEMV for K = I (pick_shape's rule): LPR
// lanes per row, NJ chunks per lane.
static void gemv_segment_shape(int64_t nch, int *lpr, int *nj) {
  *nj = nch > 64 ? 2 : 1;
  *lpr = nch > 32 ? 64 : (nch > 16 ? 32 : 16);
}

bool down_combine_supported(int I, int k) {
  const int64_t nch = I / 32;
  if (nch > 128 || k > kMaxTopK) return false;
  int lpr, nj;
  gemv_segment_shape(nch, &lpr, &nj);
  const int np = (k + 4 * (64 / lpr) - 1) / (4 * (64 / lpr));
  return np * nj <= 2;  // activation and weight registers of at most two chunk passes
}

template <int FMT, int LPR, int NJ>
static void down_combine_passes(const float *h, const int32_t *slot_pos, const int32_t *topk_ids,
                                const float *topk_w, int T, int k, const uint8_t *w2,
                                const void *w2_scale, const float *b2, int H, int I, uint16_t *out,
                                hipStream_t s) {
  constexpr int NSEG = 4 * (64 / LPR);
  if (NJ == 1 && k > NSEG)
    launch_down_combine_t<FMT, LPR, 1, 2>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  else
    launch_down_combine_t<FMT, LPR, NJ, 1>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
}

template <int FMT>
static void down_combine_shape(const float *h, const int32_t *slot_pos, const int32_t *topk_ids,
                               const float *topk_w, int T, int k, const uint8_t *w2,
                               const void *w2_scale, const float *b2, int H, int I, uint16_t *out,
                               hipStream_t s) {
  int lpr, nj;
  gemv_segment_shape(I / 32, &lpr, &nj);
  if (nj == 2)
    down_combine_passes<FMT, 64, 2>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  else if (lpr == 64)
    down_combine_passes<FMT, 64, 1>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  else if (lpr == 32)
    down_combine_passes<FMT, 32, 1>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  else
    down_combine_passes<FMT, 16, 1>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
}

hipError_t launch_gemv_down_combine(int fmt, const float *h, const int32_t *slot_pos,
                                    const int32_t *topk_ids, const float *topk_w, int T, int k,
                                    const uint8_t *w2, const void *w2_scale, const float *b2, int H,
                                    int I, uint16_t *out, hipStream_t s) {
  if (!down_combine_supported(I, k)) return hipErrorInvalidValue;
  if (fmt == 0)
    down_combine_shape<0>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  else if (fmt == 2)
    down_combine_shape<2>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
  else
    down_combine_shape<1>(h, slot_pos, topk_ids, topk_w, T, k, w2, w2_scale, b2, H, I, out, s);
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
