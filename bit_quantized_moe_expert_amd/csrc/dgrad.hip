// Grouped dgrad on 4-bit packed weights with gfx950 matrix cores:
// da[r, k] = sum_n dc[r, n] * W[e(r)][n, k], W the decoded weights.
//
// The pages' dgrad_4bit_grouped (page "grouped-nf4-gemm ...", section
// "Training: the backward is a kernel too": grad_out @ dequant(B) in one
// launch, decoding exactly as the forward does, nothing materialised in
// memory). The contraction now runs along the weight rows (n), across the
// storage order, so the design differs from the forward's:
//  - tiles of up to 128 rows of one group (device tile table) by 128 output
//    columns k; n in steps of 64; 8 waves, each 64 rows x 32 columns as two
//    v_mfma_f32_32x32x16_bf16 blocks;
//  - each step's 64 x 128 weight codes are loaded byte-column-wise (one byte =
//    two neighbouring columns, eight consecutive rows per thread), decoded
//    through an LDS byte table to fp32, multiplied by their block scale (the
//    reference decode's single fp32 product, so the per-element decode is the
//    forward's), split into bf16 hi + lo and written to LDS transposed, k-major,
//    where the MFMA B operands (8 consecutive n of one column) are one 16-byte
//    read each. The scale varies along the contraction, so it is folded into
//    the values here rather than applied to an accumulator;
//  - the gradient rows (bf16, an exact operand) are double-buffered in LDS like
//    the forward's activations; next step's loads are issued before the
//    current step's MFMAs; one LDS-only barrier per step.
#include "common.h"
#include "dgrad.h"
#include "internal.h"

namespace nf4moe {

namespace {

typedef __bf16 dg_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float dg_f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kDM = 128;      // rows per tile
constexpr int kDK = 128;      // output columns per tile
constexpr int kDN = 64;       // contraction per step
constexpr int kDPad = 72;     // bf16 per LDS row (64 + 8)
constexpr int kDRep = 16;     // decode table replicas (fp32 pairs)
constexpr int kDTab = 256 * kDRep * 8;            // 32 KB
constexpr int kDTile = kDM * kDPad * 2;           // 18 KB per bf16 tile (A, Bhi or Blo)

template <int FMT, int OUT_BF16>
__global__ __launch_bounds__(512) void k_dgrad(DgradArgs p, int ktn, int per) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kDTab + 6 * kDTile];
  // XCD-aware order as in the forward: (k-tile major, tile minor) runs per XCD
  const int L = blockIdx.x;
  const int Lp = (L & 7) * per + (L >> 3);
  if (Lp >= p.max_tiles * ktn) return;
  const int kt = Lp / p.max_tiles, ti = Lp % p.max_tiles;
  if (ti >= *p.n_tiles) return;
  const int4 tile = p.tiles[ti];
  const int e = tile.x, trow0 = tile.y, trows = tile.z;

  float2 *tab = reinterpret_cast<float2 *>(smem);
  build_pair_table<FMT, kDRep>(tab, 0, 8);
  auto tileptr = [&](int which, int buf) -> uint16_t * {  // which: 0 A, 1 Bhi, 2 Blo
    return reinterpret_cast<uint16_t *>(smem + kDTab + (which * 2 + buf) * kDTile);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave & 1, wk = wave >> 1;            // 2 x 4 waves, 64 rows x 32 cols each
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t N = p.N, K = p.K;
  const int64_t k0 = (int64_t)kt * kDK;
  const int64_t rowbytes = K / 2;
  const uint8_t *Be = p.B + (int64_t)e * N * rowbytes;
  const int64_t sc_per_row = K / Fmt<FMT>::kBlock;
  const int64_t sc_base = (int64_t)e * N * sc_per_row;

  // gradient-row slice owned by this thread: row am, 16 values at n0 + 16 aq
  const int am = tid >> 2, aq = tid & 3;
  const bool arow_ok = am < trows;
  const int64_t arow = trow0 + (arow_ok ? am : 0);
  uint4 areg[2];
  auto load_a = [&](int64_t n0) {
    const uint4 *src = reinterpret_cast<const uint4 *>(p.dc + arow * N + n0 + 16 * aq);
    areg[0] = src[0];
    areg[1] = src[1];
  };
  auto store_a = [&](int buf) {
    uint16_t *d = tileptr(0, buf) + am * kDPad + 16 * aq;
    *reinterpret_cast<uint4 *>(d) = arow_ok ? areg[0] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(d + 8) = arow_ok ? areg[1] : make_uint4(0, 0, 0, 0);
  };
  // weight-code slice: byte column kp (columns k0 + 2 kp, + 1), rows
  // n0 + 8 ng .. + 7. Columns past K read column 0 and decode to zero.
  const int kp = tid & 63, ng = tid >> 6;
  const bool kok = k0 + 2 * kp < K;
  const int64_t kbyte = kok ? k0 / 2 + kp : 0;
  const int64_t sidx = (kok ? k0 + 2 * kp : 0) / Fmt<FMT>::kBlock;
  uint32_t braw[8], sraw[8];
  auto load_b = [&](int64_t n0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = n0 + 8 * ng + i;
      braw[i] = Be[n * rowbytes + kbyte];
      sraw[i] = Fmt<FMT>::raw(p.B_scale, sc_base + n * sc_per_row + sidx);
    }
  };
  const uint32_t lanerep = (uint32_t)(lane & (kDRep - 1));
  // decode: w = fp32(code value x block scale) per element, then the exact
  // bf16 split w = hi + lo (hi truncated, lo the RNE bf16 of the rest),
  // written k-major: column k holds n0 .. n0 + 63 contiguously
  auto decode_b = [&](int buf) {
    uint32_t he[4], hoo[4], le[4], lo[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 v = tab[braw[i] * kDRep + lanerep];
      const float s = kok ? Fmt<FMT>::value(sraw[i]) : 0.0f;
      const float we = v.x * s, wo = v.y * s;
      const uint32_t hbe = __float_as_uint(we) & 0xffff0000u, hbo = __float_as_uint(wo) & 0xffff0000u;
      const uint32_t lbe = f32_to_bf16_rne(we - __uint_as_float(hbe));
      const uint32_t lbo = f32_to_bf16_rne(wo - __uint_as_float(hbo));
      if ((i & 1) == 0) {
        he[i >> 1] = hbe >> 16;
        hoo[i >> 1] = hbo >> 16;
        le[i >> 1] = lbe;
        lo[i >> 1] = lbo;
      } else {
        he[i >> 1] |= hbe;
        hoo[i >> 1] |= hbo;
        le[i >> 1] |= lbe << 16;
        lo[i >> 1] |= lbo << 16;
      }
    }
    const int kl = 2 * kp, nl = 8 * ng;
    *reinterpret_cast<uint4 *>(tileptr(1, buf) + kl * kDPad + nl) = make_uint4(he[0], he[1], he[2], he[3]);
    *reinterpret_cast<uint4 *>(tileptr(1, buf) + (kl + 1) * kDPad + nl) = make_uint4(hoo[0], hoo[1], hoo[2], hoo[3]);
    *reinterpret_cast<uint4 *>(tileptr(2, buf) + kl * kDPad + nl) = make_uint4(le[0], le[1], le[2], le[3]);
    *reinterpret_cast<uint4 *>(tileptr(2, buf) + (kl + 1) * kDPad + nl) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  };

  dg_f32x16_t C[2] = {};
  load_a(0);
  load_b(0);
  lds_barrier();  // the table is complete before the first decode
  store_a(0);
  decode_b(0);
  lds_barrier();

  int cur = 0;
  for (int64_t n0 = 0; n0 < N; n0 += kDN) {
    const bool more = n0 + kDN < N;
    const int64_t nn = more ? n0 + kDN : n0;  // the last step reloads its own slice
    load_a(nn);
    load_b(nn);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t *At = tileptr(0, cur), *Bh = tileptr(1, cur), *Bl = tileptr(2, cur);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int col = 16 * s + 8 * g;
      dg_bf16x8_t a[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        a[mb] = __builtin_bit_cast(dg_bf16x8_t, *reinterpret_cast<const uint4 *>(At + (wm * 64 + mb * 32 + l32) * kDPad + col));
      const int kc = wk * 32 + l32;
      const dg_bf16x8_t bh = __builtin_bit_cast(dg_bf16x8_t, *reinterpret_cast<const uint4 *>(Bh + kc * kDPad + col));
      const dg_bf16x8_t bl = __builtin_bit_cast(dg_bf16x8_t, *reinterpret_cast<const uint4 *>(Bl + kc * kDPad + col));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) C[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], bh, C[mb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) C[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], bl, C[mb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    store_a(cur ^ 1);
    decode_b(cur ^ 1);
    lds_barrier();
    cur ^= 1;
    if (!more) break;
  }

  // 32x32 accumulator: lane holds column l32 of the wave's 32, rows
  // 8 * (v / 4) + 4 * g + (v % 4) of each 32-row block
  const int64_t k = k0 + wk * 32 + l32;
  if (k >= K) return;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = wm * 64 + mb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (m >= trows) continue;
      const int64_t o = (int64_t)(trow0 + m) * K + k;
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(p.da)[o] = (uint16_t)f32_to_bf16_rne(C[mb][v]);
      else
        reinterpret_cast<float *>(p.da)[o] = C[mb][v];
    }
  }
}

template <int FMT, int OUT_BF16>
hipError_t launch_dgrad_t(const DgradArgs &a, hipStream_t s) {
  const int ktn = (int)cdiv(a.K, kDK);
  const int64_t total = (int64_t)a.max_tiles * ktn;
  const int64_t padded = cdiv(total, 8) * 8;
  const int per = (int)(padded / 8);
  hipLaunchKernelGGL((k_dgrad<FMT, OUT_BF16>), dim3((unsigned)padded), dim3(512), 0, s, a, ktn, per);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dgrad(const DgradArgs &a, hipStream_t s) {
  if (a.max_tiles <= 0) return hipSuccess;
  if (a.fmt == 0) return a.da_bf16 ? launch_dgrad_t<0, 1>(a, s) : launch_dgrad_t<0, 0>(a, s);
  if (a.fmt == 2) return a.da_bf16 ? launch_dgrad_t<2, 1>(a, s) : launch_dgrad_t<2, 0>(a, s);
  return a.da_bf16 ? launch_dgrad_t<1, 1>(a, s) : launch_dgrad_t<1, 0>(a, s);
}

}  // namespace nf4moe
