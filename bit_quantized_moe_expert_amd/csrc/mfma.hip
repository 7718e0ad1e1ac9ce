// Large-M grouped GEMM on 4-bit packed weights with gfx950 matrix cores.
//
// Same operation as the small-M path (the pages' gemm_4bit_grouped: decode in
// registers, block scale, fp32 accumulation; "larger groups the M-tile path",
// page "How do I run a grouped GEMM directly on NF4 packed MoE expert weights
// ...", section "Supported scope"), used once per-expert row counts make it a
// dense contraction. Design for gfx950:
//  - tiles of up to 128 routed rows of one expert (from the device tile
//    table) by 128 weight rows, K in steps of 64 (one NF4 absmax block);
//    4 waves, each 64 x 64 as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16;
//  - A rows are gathered (token of each routed slot) into LDS as bf16; fp32
//    activations (h of the down projection) are split into bf16 hi + lo;
//  - each lane's B operand is 8 consecutive k of one weight row; the K order
//    inside a 64-block is permuted the same way for A and B so that a lane's
//    operands for all 4 K-steps come from one 16-byte load of codes;
//  - NF4 codes become bf16 hi + lo pairs (hi + lo carries 16 significant bits
//    of the fp32 codebook value) through an LDS byte table; the per-(row,
//    block) absmax multiplies the block's accumulator in fp32. MXFP4 values
//    times their power-of-two scale are exact in bf16, so one product suffices
//    and the scale is folded into B;
//  - SwiGLU pairs gate column n and up column n + I inside one wave.
// Workgroups are remapped so consecutive tiles sharing a weight tile land on
// the same XCD (its L2), with tiles of one expert adjacent.
#include "common.h"
#include "internal.h"

namespace nf4moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = kMfmaBM;  // 128
constexpr int kBK = 64;
constexpr int kApad = 72;     // bf16 per LDS row of A (64 + 8 padding)
constexpr int kMRep = 16;     // LDS table replicas

__device__ inline bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, v);
}

// NF4: byte -> (bf16 hi of even, bf16 hi of odd | bf16 lo of even, lo of odd).
__device__ inline void build_nf4_bf16_table(uint2 *tab) {
  for (int i = threadIdx.x; i < 256 * kMRep; i += blockDim.x) {
    const uint32_t b = (uint32_t)i / kMRep;
    const float2 pv = pair_value<0>(b);
    const float ve = pv.x, vo = pv.y;
    const uint32_t he = f32_to_bf16_rne(ve), ho = f32_to_bf16_rne(vo);
    const uint32_t le = f32_to_bf16_rne(ve - bf16_to_f32(he));
    const uint32_t lo = f32_to_bf16_rne(vo - bf16_to_f32(ho));
    tab[i] = make_uint2(he | (ho << 16), le | (lo << 16));
  }
}

// MXFP4: byte -> (even value, odd value) as fp32.
__device__ inline void build_e2m1_f32_table(uint2 *tab) {
  for (int i = threadIdx.x; i < 256 * kMRep; i += blockDim.x) {
    const uint32_t b = (uint32_t)i / kMRep;
    const float2 pv = pair_value<1>(b);
    tab[i] = make_uint2(__float_as_uint(pv.x), __float_as_uint(pv.y));
  }
}

template <int FMT, int EPI, int AF32>
__global__ __launch_bounds__(256, 2) void k_mfma(GemmArgs p, int ntn, int per) {
  __shared__ __attribute__((aligned(16))) uint16_t Ahi[kBM * kApad];
  __shared__ __attribute__((aligned(16))) uint16_t Alo[AF32 ? kBM * kApad : 8];
  __shared__ uint2 tab_all[256 * kMRep];

  // XCD-aware order: hardware XCD = blockIdx.x % 8; give each XCD a contiguous
  // run of (n-tile major, tile minor) work.
  const int L = blockIdx.x;
  const int Lp = (L & 7) * per + (L >> 3);
  if (Lp >= p.max_tiles * ntn) return;
  const int nt = Lp / p.max_tiles, ti = Lp % p.max_tiles;
  if (ti >= *p.n_tiles) return;
  const int4 tile = p.tiles[ti];  // expert, row0, rows
  const int e = tile.x, trow0 = tile.y, trows = tile.z;

  if (FMT == 0)
    build_nf4_bf16_table(tab_all);
  else
    build_e2m1_f32_table(tab_all);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 5, l32 = lane & 31;
  const uint2 *tab = tab_all + (lane & (kMRep - 1));

  const int64_t N = p.N, K = p.K;
  const int64_t ncol = (EPI == EPI_SWIGLU) ? N / 2 : N;
  int64_t colbase, nrow[2];
  if (EPI == EPI_SWIGLU) {
    colbase = (int64_t)nt * 64 + wn * 32;
    nrow[0] = colbase + l32;          // gate row
    nrow[1] = ncol + colbase + l32;   // up row
  } else {
    colbase = (int64_t)nt * 128 + wn * 64;
    nrow[0] = colbase + l32;
    nrow[1] = colbase + 32 + l32;
  }
  bool nvalid[2];
  nvalid[0] = (EPI == EPI_SWIGLU) ? (colbase + l32 < ncol) : (nrow[0] < N);
  nvalid[1] = (EPI == EPI_SWIGLU) ? (colbase + l32 < ncol) : (nrow[1] < N);

  const int64_t rowbytes = K / 2;
  const uint8_t *Be = p.B + (int64_t)e * N * rowbytes;
  const int64_t sc_per_row = K / Fmt<FMT>::kBlock;
  const int64_t sc_base = (int64_t)e * N * sc_per_row;

  // A-tile row owned by this thread for the LDS fill
  const int am = tid >> 1, ahf = tid & 1;
  const bool arow_ok = am < trows;
  int64_t arow = 0;
  if (arow_ok) {
    const int r = trow0 + am;
    arow = p.a_row_of ? (int64_t)(p.a_row_of[r] / p.a_div) : (int64_t)r;
  }

  f32x16_t C[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) C[i][j][v] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    // ---- A tile -> LDS: this thread fills row am, k in [k0 + 32 ahf, +32)
    {
      const int64_t kk = k0 + 32 * ahf;
      const bool ok = arow_ok && kk < K;
      uint16_t *dh = Ahi + am * kApad + 32 * ahf;
      if (AF32) {
        uint16_t *dl = Alo + am * kApad + 32 * ahf;
        const float4 *src = reinterpret_cast<const float4 *>(
            reinterpret_cast<const float *>(p.a) + arow * K + kk);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float4 v = ok ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
          const float f[4] = {v.x, v.y, v.z, v.w};
          uint32_t hb[4], lb[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t hi = __float_as_uint(f[q]) & 0xffff0000u;  // truncated hi
            hb[q] = hi >> 16;
            lb[q] = f32_to_bf16_rne(f[q] - __uint_as_float(hi));
          }
          *reinterpret_cast<uint2 *>(dh + 4 * i) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
          *reinterpret_cast<uint2 *>(dl + 4 * i) = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
        }
      } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint16_t *>(p.a) + arow * K + kk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint4 *>(dh + 8 * i) = ok ? src[i] : make_uint4(0, 0, 0, 0);
      }
    }
    // ---- B: one 16-byte chunk of codes per lane and N-block: k in [k0 + 32 g, +32)
    uint4 bq[2];
    float bs[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t kk = k0 + 32 * g;
      if (nvalid[b] && kk < K) {
        bq[b] = *reinterpret_cast<const uint4 *>(Be + nrow[b] * rowbytes + kk / 2);
        const int64_t sidx = FMT == 0 ? (k0 / 64) : (kk / 32);
        if (FMT == 0)
          bs[b] = reinterpret_cast<const float *>(p.B_scale)[sc_base + nrow[b] * sc_per_row + sidx];
        else
          bs[b] = e8m0_to_f32(reinterpret_cast<const uint8_t *>(p.B_scale)[sc_base + nrow[b] * sc_per_row + sidx]);
      } else {
        bq[b] = make_uint4(0, 0, 0, 0);
        bs[b] = 0.0f;
      }
    }
    __syncthreads();

    f32x16_t P[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) P[i][j][v] = 0.0f;

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t ah[2], al[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + l32;
        const int col = 32 * g + 8 * s;
        ah[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(Ahi + row * kApad + col));
        if (AF32)
          al[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(Alo + row * kApad + col));
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint32_t word = s == 0 ? bq[b].x : (s == 1 ? bq[b].y : (s == 2 ? bq[b].z : bq[b].w));
        uint2 t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = tab[((word >> (8 * q)) & 0xffu) * kMRep];
        if (FMT == 0) {
          const bf16x8_t bh = as_bf16x8(t[0].x, t[1].x, t[2].x, t[3].x);
          const bf16x8_t bl = as_bf16x8(t[0].y, t[1].y, t[2].y, t[3].y);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            P[mb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bh, P[mb][b], 0, 0, 0);
            P[mb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bl, P[mb][b], 0, 0, 0);
            if (AF32)
              P[mb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bh, P[mb][b], 0, 0, 0);
          }
        } else {
          uint32_t d[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float ve = __uint_as_float(t[q].x) * bs[b];   // exact: power-of-two scale
            const float vo = __uint_as_float(t[q].y) * bs[b];
            d[q] = (__float_as_uint(ve) >> 16) | (__float_as_uint(vo) & 0xffff0000u);
          }
          const bf16x8_t bv = as_bf16x8(d[0], d[1], d[2], d[3]);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            C[mb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[mb], bv, C[mb][b], 0, 0, 0);
            if (AF32)
              C[mb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[mb], bv, C[mb][b], 0, 0, 0);
          }
        }
      }
    }
    if (FMT == 0) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) C[mb][b][v] = fmaf(bs[b], P[mb][b][v], C[mb][b][v]);
    }
    __syncthreads();
  }

  // ---- epilogue. 32x32 accumulator: lane holds column l32, rows
  // 8 * (v / 4) + 4 * g + (v % 4) for v = 0..15.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (m >= trows) continue;
      const int64_t r = trow0 + m;
      if (EPI == EPI_SWIGLU) {
        const int64_t col = colbase + l32;
        if (col < ncol) {
          const float gt = C[mb][0][v], up = C[mb][1][v];
          reinterpret_cast<float *>(p.c)[r * ncol + col] = gt / (1.0f + expf(-gt)) * up;
        }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int64_t col = nrow[b];
          if (!nvalid[b]) continue;
          const float y = C[mb][b][v];
          if (EPI == EPI_PLAIN_F32) {
            reinterpret_cast<float *>(p.c)[r * N + col] = y;
          } else if (EPI == EPI_PLAIN_BF16) {
            reinterpret_cast<uint16_t *>(p.c)[r * N + col] = (uint16_t)f32_to_bf16_rne(y);
          } else {
            const int64_t slot = p.slot_of[r];
            reinterpret_cast<float *>(p.c)[slot * N + col] = p.slot_w[slot] * y;
          }
        }
      }
    }
  }
}

template <int FMT, int EPI, int AF32>
static hipError_t launch_mfma_t(const GemmArgs &g, hipStream_t s) {
  const int64_t ncol = (EPI == EPI_SWIGLU) ? g.N / 2 : g.N;
  const int ntn = (int)((EPI == EPI_SWIGLU) ? cdiv(ncol, 64) : cdiv(ncol, 128));
  const int64_t total = (int64_t)g.max_tiles * ntn;
  const int64_t padded = cdiv(total, 8) * 8;
  const int per = (int)(padded / 8);
  hipLaunchKernelGGL((k_mfma<FMT, EPI, AF32>), dim3((unsigned)padded), dim3(256), 0, s, g, ntn, per);
  return hipGetLastError();
}

template <int FMT>
static hipError_t mfma_pick(const GemmArgs &g, hipStream_t s) {
  switch (g.epi) {
    case EPI_SWIGLU:
      return g.a_is_f32 ? launch_mfma_t<FMT, EPI_SWIGLU, 1>(g, s) : launch_mfma_t<FMT, EPI_SWIGLU, 0>(g, s);
    case EPI_PLAIN_F32:
      return g.a_is_f32 ? launch_mfma_t<FMT, EPI_PLAIN_F32, 1>(g, s) : launch_mfma_t<FMT, EPI_PLAIN_F32, 0>(g, s);
    case EPI_PLAIN_BF16:
      return g.a_is_f32 ? launch_mfma_t<FMT, EPI_PLAIN_BF16, 1>(g, s) : launch_mfma_t<FMT, EPI_PLAIN_BF16, 0>(g, s);
    default:
      return g.a_is_f32 ? launch_mfma_t<FMT, EPI_SLOT, 1>(g, s) : launch_mfma_t<FMT, EPI_SLOT, 0>(g, s);
  }
}

hipError_t launch_mfma_grouped(const GemmArgs &g, hipStream_t s) {
  if (g.max_tiles <= 0) return hipSuccess;
  return g.fmt == 0 ? mfma_pick<0>(g, s) : mfma_pick<1>(g, s);
}

}  // namespace nf4moe
