// Large-M grouped GEMM on 4-bit packed weights with gfx950 matrix cores.
//
// Same operation as the small-M path (the pages' gemm_4bit_grouped: decode in
// registers, block scale, fp32 accumulation; "larger groups the M-tile path",
// page "How do I run a grouped GEMM directly on NF4 packed MoE expert weights
// ...", section "Supported scope"), used once per-expert row counts make it a
// dense contraction. Design for gfx950:
//  - tiles of up to 128 routed rows of one expert (from the device tile
//    table) by 256 weight rows, K in steps of 64 (one NF4 absmax block);
//    8 waves, each 128 x 32 (all rows, 32 weight rows) as 4 blocks of
//    v_mfma_f32_32x32x16_bf16, so each decoded code feeds 4 MFMAs;
//  - the activation tile is double-buffered in LDS and the next K-step's
//    activation and weight loads are issued before the current step's MFMAs,
//    so one barrier per step finds them mostly landed;
//  - A rows are gathered (token of each routed slot) into LDS as bf16; the
//    down projection's fp32 activation h arrives as (bf16 hi, bf16 lo) pairs;
//  - each lane's B operand is 8 consecutive k of one weight row; the K order
//    inside a 64-block is permuted the same way for A and B so that a lane's
//    operands for all 4 K-steps come from one 16-byte load of codes;
//  - NF4 codes become bf16 hi + lo pairs (hi + lo carries 16 significant bits
//    of the fp32 codebook value) through an LDS byte table; the per-(row,
//    block) absmax multiplies the block's accumulator in fp32. MXFP4 values
//    times their power-of-two scale are exact in bf16, so one product suffices
//    and the scale is folded into B;
//  - SwiGLU: gate column n and up column n + I are computed by paired waves
//    and meet through LDS in the epilogue.
// Workgroups are remapped so consecutive tiles sharing a weight tile land on
// the same XCD (its L2), with tiles of one expert adjacent.
#include "common.h"
#include "internal.h"

namespace nf4moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kApad = 72;     // bf16 per LDS row of A (64 + 8 padding)

__device__ inline bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, v);
}

// LDS decode table at LDS address 0: entry for byte b = 32 replicas of 8
// bytes (256 B), so entry (b, lane & 31) sits at byte offset b * 256 + 8 *
// (lane & 31), one v_perm_b32 away from the code word (tab_offset), and the
// 32 lanes of a half-wave read distinct banks whatever the codes.
// NF4 entry: (bf16 hi of even | hi of odd << 16, bf16 lo of even | lo of odd
// << 16), hi = RNE bf16 of the fp32 codebook value, lo = RNE bf16 of the rest.
// MXFP4 entry: (even value, odd value) as fp32.
constexpr int kTabBytes = 256 * 32 * 8;

template <int FMT>
__device__ inline void build_mfma_table(uint4 *tab) {
  const float cb = codebook_lane<FMT>();
  for (int f = threadIdx.x; f < kTabBytes / 16; f += blockDim.x) {  // 8 full-wave rounds
    const uint32_t b = (uint32_t)f >> 4;   // 16 words of two replicas per entry
    const float2 pv = pair_gather<FMT>(cb, b);
    uint2 v;
    if (Fmt<FMT>::kNF4) {
      const uint32_t he = f32_to_bf16_rne(pv.x), ho = f32_to_bf16_rne(pv.y);
      const uint32_t le = f32_to_bf16_rne(pv.x - bf16_to_f32(he));
      const uint32_t lo = f32_to_bf16_rne(pv.y - bf16_to_f32(ho));
      v = make_uint2(he | (ho << 16), le | (lo << 16));
    } else {
      v = make_uint2(__float_as_uint(pv.x), __float_as_uint(pv.y));
    }
    tab[f] = make_uint4(v.x, v.y, v.x, v.y);
  }
}

// One output tile: rows [trow0, trow0 + trows) of expert e against weight-row
// tile nt. AM: activation operand mode. 0: bf16 A; 2: an fp32 A given as
// 32-bit (hi, lo) bf16 pairs, its truncated bf16 hi and the RNE bf16 of the
// rest (the SwiGLU epilogue writes h so), each weight product taking three
// MFMAs. XF: the extended gate_up / down epilogue (clamped GLU, interleaved
// gate and up rows, per-expert biases); XF = 0 instantiates the plain kernel.
// MB: 32-row blocks (4: up to 128 rows; 2: up to 64 rows; 1: up to 32 rows:
// fewer MFMAs and less A traffic for the tiles of small groups and the last
// tiles of large ones).
template <int FMT, int EPI, int AM, int XF, int MB>
__device__ __forceinline__ void mfma_tile(const GemmArgs &p, uint8_t *smem, int nt, int e, int trow0,
                                          int trows) {
  static_assert(AM == 0 || AM == 2, "operand mode");
  static_assert(MB == 4 || MB == 2 || MB == 1, "row blocks");
  constexpr bool AF32 = AM != 0;                      // a lo part exists
  constexpr int kBM = 32 * MB;                        // rows per tile
  constexpr int ABUF = kBM * kApad * 2;               // bytes per A buffer

  build_mfma_table<FMT>(reinterpret_cast<uint4 *>(smem));
  auto abuf = [&](int hi_lo, int buf) -> uint16_t * {
    return reinterpret_cast<uint16_t *>(smem + kTabBytes + (hi_lo * 2 + buf) * ABUF);
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const uint32_t lanebyte = (uint32_t)l32 * 8;

  // Every wave covers all 128 rows of the tile and 32 weight rows (output
  // columns), lane column l32. SwiGLU: waves 0-3 take gate columns
  // nt * 128 + 32 w, waves 4-7 the matching up columns (+ I); the two halves
  // meet through LDS in the epilogue.
  const int64_t N = p.N, K = p.K;
  const int64_t ncol = (EPI == EPI_SWIGLU) ? N / 2 : N;
  int64_t col, nrow;
  if (EPI == EPI_SWIGLU) {
    col = (int64_t)nt * 128 + 32 * (wave & 3) + l32;
    nrow = (XF && p.glu_inter) ? 2 * col + (wave >> 2) : col + (wave >> 2) * ncol;
  } else {
    col = (int64_t)nt * 256 + 32 * wave + l32;
    nrow = col;
  }
  const bool nvalid = col < ncol;
  const int64_t nrow_c = nvalid ? nrow : 0;

  const int64_t rowbytes = K / 2;
  const uint8_t *Be = p.B + (int64_t)e * N * rowbytes;
  const int64_t sc_per_row = K / Fmt<FMT>::kBlock;
  const int64_t sc_base = (int64_t)e * N * sc_per_row;

  // A-tile slice owned by this thread for the LDS fill: row am, EPT elements
  // starting at k0 + EPT * aq. Rows past the tile read a valid row (the tile's
  // first) and are zeroed when stored (measured: storing them unmasked, which
  // the results would allow, made the 64-row kernels 2-3 % slower).
  // A 32-row bf16 tile is 256 16-byte words: there the first 256 threads fill
  // it (NFILL) and the other waves skip the store.
  constexpr int TPR = (MB == 1 && !AF32) ? 8 : 512 / kBM;  // fill threads per row
  constexpr int EPT = 64 / TPR;                       // elements per thread: 16, 8 or 4
  constexpr int NFILL = kBM * TPR;                    // threads that fill the tile
  const int am = tid / TPR, aq = tid % TPR;
  const bool arow_ok = am < trows;
  int64_t arow;
  {
    const int r = trow0 + (arow_ok ? am : 0);
    arow = p.a_row_of ? (int64_t)(p.a_row_of[r] / p.a_div) : (int64_t)r;
    arow = arow < 0 ? 0 : (arow < p.a_rows ? arow : p.a_rows - 1);  // a bad index cannot read past a
  }
  constexpr int AW = EPT * (AF32 ? 4 : 2) / 16;       // 16-byte words per thread
  // Two register sets: the slice for K-step k + 2 is loaded while the one for
  // k + 1 (loaded a step earlier) waits to be stored to LDS.
  uint4 aregs[2][AW];
  bool aoks[2] = {false, false};
  auto load_a = [&](int64_t k0, int set) {
    const int64_t kk = k0 + EPT * aq;
    aoks[set] = arow_ok && kk < K;
    const int64_t kc = kk < K ? kk : 0;
    // AM 0: EPT bf16; AM 2: EPT (hi, lo) bf16 pairs, 4 bytes each
    const uint4 *src = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(p.a) +
                                                       (arow * K + kc) * (AM == 2 ? 4 : 2));
#pragma unroll
    for (int i = 0; i < AW; ++i) aregs[set][i] = src[i];
  };
  auto store_a = [&](int buf, int set) {
    if (NFILL < 512 && tid >= NFILL) return;  // whole waves
    const uint4 *areg = aregs[set];
    const bool a_ok = aoks[set];
    uint16_t *dh = abuf(0, buf) + am * kApad + EPT * aq;
    if (AM == 2 && EPT == 4) {  // four pairs: 8 bytes into each tile
      uint16_t *dl = abuf(1, buf) + am * kApad + EPT * aq;
      const uint4 u = areg[0];
      const uint32_t h0 = a_ok ? __builtin_amdgcn_perm(u.y, u.x, 0x05040100u) : 0u;
      const uint32_t h1 = a_ok ? __builtin_amdgcn_perm(u.w, u.z, 0x05040100u) : 0u;
      const uint32_t l0 = a_ok ? __builtin_amdgcn_perm(u.y, u.x, 0x07060302u) : 0u;
      const uint32_t l1 = a_ok ? __builtin_amdgcn_perm(u.w, u.z, 0x07060302u) : 0u;
      *reinterpret_cast<uint2 *>(dh) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(dl) = make_uint2(l0, l1);
    } else if (AM == 2) {  // de-interleave the pairs into the hi and lo tiles
      uint16_t *dl = abuf(1, buf) + am * kApad + EPT * aq;
#pragma unroll
      for (int i = 0; i < EPT / 8; ++i) {
        const uint4 u = areg[2 * i], v = areg[2 * i + 1];
        const uint32_t w[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
        uint32_t h4[4], l4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h4[q] = a_ok ? __builtin_amdgcn_perm(w[2 * q + 1], w[2 * q], 0x05040100u) : 0u;
          l4[q] = a_ok ? __builtin_amdgcn_perm(w[2 * q + 1], w[2 * q], 0x07060302u) : 0u;
        }
        *reinterpret_cast<uint4 *>(dh + 8 * i) = make_uint4(h4[0], h4[1], h4[2], h4[3]);
        *reinterpret_cast<uint4 *>(dl + 8 * i) = make_uint4(l4[0], l4[1], l4[2], l4[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < AW; ++i)
        *reinterpret_cast<uint4 *>(dh + 8 * i) = a_ok ? areg[i] : make_uint4(0, 0, 0, 0);
    }
  };
  // B: one 16-byte chunk of codes per lane, k in [k0 + 32 g, +32), plus the
  // raw scale and whether it counts. The scale is masked only when it is
  // consumed, a K-step later, so nothing waits on these loads early.
  auto load_b = [&](int64_t k0, uint4 &bq, uint32_t &braw, bool &bok) {
    const int64_t kk = k0 + 32 * g;
    bok = nvalid && kk < K;
    const int64_t kc = kk < K ? kk : 0;
    bq = *reinterpret_cast<const uint4 *>(Be + nrow_c * rowbytes + kc / 2);
    const int64_t sidx = Fmt<FMT>::kNF4 ? (k0 < K ? k0 / 64 : 0) : kc / 32;
    braw = Fmt<FMT>::raw(p.B_scale, sc_base + nrow_c * sc_per_row + sidx);
  };
  auto scale_of = [&](uint32_t raw, bool ok) -> float {
    const float v = Fmt<FMT>::value(raw);
    return ok ? v : 0.0f;
  };

  const f32x16_t zero16 = {};
  f32x16_t C[MB], P[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) C[mb] = zero16;

  // One K-step on LDS buffer `cur` with codes bq and scale bs. Loads run two
  // steps ahead: the activation slice of step k + 2 into register set `aset`
  // at the start, the codes and scale of step k + 2 into bq / br / bok once
  // this step's lookups have read bq; the slice of step k + 1 (set aset ^ 1)
  // goes to the other LDS buffer at the end.
  auto step = [&](int64_t k0, int cur, int aset, uint4 &bq, float bs, uint32_t &br, bool &bok) {
    // Loads are issued (from clamped, valid addresses) and stored even past
    // the last step, so no branch splits the load/wait bookkeeping; the
    // extra data is unused.
    const bool more = k0 + kBK < K;
    load_a(k0 + 2 * kBK, aset);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    const uint16_t *Ah = abuf(0, cur);
    const uint16_t *Al = abuf(1, AF32 ? cur : 0);

    // Four units s per K-step (k = 32 g + 8 s + 0..7 of this lane). A unit's
    // B operand is 4 table lookups of code word s; its A operands are the
    // four 32-row fragments. Unit s + 1's LDS reads are issued before unit
    // s's MFMAs (fp32 A: only the lookups; its fragments would not fit).
    constexpr int NA = AF32 ? 1 : 2;
    uint2 t[2][4];
    bf16x8_t ah[NA][MB], al[NA][MB];
    auto read_a = [&](int sa, bf16x8_t *dh, bf16x8_t *dl) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = mb * 32 + l32;
        const int colk = 32 * g + 8 * sa;
        dh[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(Ah + row * kApad + colk));
        if (AF32) dl[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(Al + row * kApad + colk));
      }
    };
#pragma unroll
    for (int u = -1; u < 4; ++u) {
      if (u + 1 < 4) {
        const int sn = u + 1;
        if (!AF32) read_a(sn, ah[sn & (NA - 1)], al[sn & (NA - 1)]);
        const uint32_t word = sn == 0 ? bq.x : (sn == 1 ? bq.y : (sn == 2 ? bq.z : bq.w));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          t[sn & 1][q] = *reinterpret_cast<const uint2 *>(smem + tab_offset(word, lanebyte, q));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (u == 3) {  // every lookup of this step has read bq: reuse it for step k + 2
        load_b(k0 + 2 * kBK, bq, br, bok);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (u >= 0) {
        const int s = u;
        if (AF32) read_a(s, ah[0], al[0]);
        const uint2 *tu = t[s & 1];
        const bf16x8_t *ahs = ah[s & (NA - 1)];
        const bf16x8_t *als = al[s & (NA - 1)];
        if (Fmt<FMT>::kNF4) {
          const bf16x8_t bh = as_bf16x8(tu[0].x, tu[1].x, tu[2].x, tu[3].x);
          const bf16x8_t bl = as_bf16x8(tu[0].y, tu[1].y, tu[2].y, tu[3].y);
          // passes over the four independent accumulators, so consecutive
          // MFMAs never depend on each other
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            P[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahs[mb], bh, s == 0 ? zero16 : P[mb], 0, 0, 0);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            P[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahs[mb], bl, P[mb], 0, 0, 0);
          if (AF32) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              P[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(als[mb], bh, P[mb], 0, 0, 0);
          }
        } else {
          uint32_t d[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float ve = __uint_as_float(tu[q].x) * bs;   // exact: power-of-two scale
            const float vo = __uint_as_float(tu[q].y) * bs;
            d[q] = (__float_as_uint(ve) >> 16) | (__float_as_uint(vo) & 0xffff0000u);
          }
          const bf16x8_t bv = as_bf16x8(d[0], d[1], d[2], d[3]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            C[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahs[mb], bv, C[mb], 0, 0, 0);
          if (AF32) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              C[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(als[mb], bv, C[mb], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (Fmt<FMT>::kNF4) {  // NF4: the block's absmax scales its partial product
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) C[mb][v] = fmaf(bs, P[mb][v], C[mb][v]);
    }
    __builtin_amdgcn_sched_barrier(0);  // the A store waits for its loads: keep it last
    store_a(cur ^ 1, aset ^ 1);
    lds_barrier();
    return more;
  };

  uint4 bq0, bq1;
  uint32_t br0, br1;
  bool bok0, bok1;
  load_a(0, 0);
  load_b(0, bq0, br0, bok0);
  load_a(kBK, 1);
  load_b(kBK, bq1, br1, bok1);
  store_a(0, 0);
  lds_barrier();
  float bs0 = scale_of(br0, bok0), bs1;

  // Unrolled by two so the register sets alternate without copies: step k
  // computes on B set k % 2 and LDS buffer k % 2, loads A(k + 2) into set
  // k % 2 and stores A(k + 1) from set (k + 1) % 2.
  for (int64_t k0 = 0;; k0 += 2 * kBK) {
    if (!step(k0, 0, 0, bq0, bs0, br0, bok0)) break;
    bs1 = scale_of(br1, bok1);
    if (!step(k0 + kBK, 1, 1, bq1, bs1, br1, bok1)) break;
    bs0 = scale_of(br0, bok0);
  }

  // ---- epilogue. 32x32 accumulator: lane holds column l32, rows
  // 8 * (v / 4) + 4 * g + (v % 4) for v = 0..15 of each 32-row block mb.
  if (EPI == EPI_SWIGLU) {
    // up waves hand their values to the gate waves through LDS (the table
    // region: every lookup finished before the last step's barrier)
    float *xch = reinterpret_cast<float *>(smem);
    const int w4 = wave & 3;
    if (wave >= 4) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) xch[((w4 * MB + mb) * 16 + v) * 64 + lane] = C[mb][v];
    }
    lds_barrier();
    if (wave >= 4) return;
    float bg = 0.0f, bu = 0.0f;  // this column's gate and up biases
    if (XF && p.bias && nvalid) {
      const float *bb = p.bias + (int64_t)e * N;
      bg = bb[nrow];
      bu = bb[p.glu_inter ? nrow + 1 : nrow + ncol];
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        const float up = xch[((w4 * MB + mb) * 16 + v) * 64 + lane];
        if (m >= trows || !nvalid) continue;
        float h;
        if constexpr (XF) {
          h = glu_value(p.glu, p.glu_alpha, p.glu_limit, C[mb][v] + bg, up + bu);
        } else {
          const float gt = C[mb][v];
          h = gt / (1.0f + expf(-gt)) * up;
        }
        const int64_t o = (int64_t)(trow0 + m) * ncol + col;
        if (p.c_split) {  // (truncated bf16 hi, RNE bf16 of the rest) in one word
          const uint32_t hi = __float_as_uint(h) & 0xffff0000u;
          reinterpret_cast<uint32_t *>(p.c)[o] = (hi >> 16) | (f32_to_bf16_rne(h - __uint_as_float(hi)) << 16);
        } else {
          reinterpret_cast<float *>(p.c)[o] = h;
        }
      }
    }
    return;
  }
  if (!nvalid) return;
  const float yb = (XF && EPI == EPI_SLOT && p.bias) ? p.bias[(int64_t)e * N + col] : 0.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = mb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (m >= trows) continue;
      const int64_t r = trow0 + m;
      const float y = C[mb][v];
      if (EPI == EPI_PLAIN_F32) {
        reinterpret_cast<float *>(p.c)[r * N + col] = y;
      } else if (EPI == EPI_PLAIN_BF16) {
        reinterpret_cast<uint16_t *>(p.c)[r * N + col] = (uint16_t)f32_to_bf16_rne(y);
      } else {
        const int64_t slot = p.slot_of[r];
        reinterpret_cast<float *>(p.c)[slot * N + col] = p.slot_w[slot] * (XF ? y + yb : y);
      }
    }
  }
}

// One workgroup per (weight-row tile, row tile) of the device tile table.
// TR = 128: tiles of up to 128 rows of one expert; a tile runs the 128-, 64-
// or 32-row body by its row count (the choice is uniform over the workgroup,
// and a row's arithmetic is the same in all; the 32-row body took 6-16 % off
// batches of 16-512 tokens whose groups are mostly small). TR = 64: tiles of
// up to 64 rows, in a kernel without the 128-row body (measured 4-5 % faster
// than the kernel holding it on such tables). A kernel holding only the
// 32-row body fits two workgroups per CU, but was slower or equal: the
// LDS-bound decode gains nothing from the second workgroup, and the pairs
// leave CUs idle when the workgroups number about one per CU.
template <int FMT, int EPI, int AM, int XF, int TR>
__global__ __launch_bounds__(512) void k_mfma(GemmArgs p, int ntn, int per) {
  static_assert(TR == 64 || TR == 128, "tile rows");
  // the decode table and the A buffers of the tallest body (hi[2], and lo[2]
  // for an fp32 A)
  __shared__ __attribute__((aligned(16))) uint8_t smem[kTabBytes + (AM != 0 ? 4 : 2) * TR * kApad * 2];
  // XCD-aware order: hardware XCD = blockIdx.x % 8; give each XCD a contiguous
  // run of (n-tile major, tile minor) work, so the M-tiles of one expert and
  // one weight tile share that XCD's L2.
  const int L = blockIdx.x;
  const int Lp = (L & 7) * per + (L >> 3);
  if (Lp >= p.max_tiles * ntn) return;
  const int nt = Lp / p.max_tiles, ti = Lp % p.max_tiles;
  if (ti >= *p.n_tiles) return;
  const int4 tile = p.tiles[ti];  // expert, row0, rows, rows of the whole group
  const int rows = __builtin_amdgcn_readfirstlane(tile.z);
  if constexpr (TR == 128) {
    if (rows > 64) {
      mfma_tile<FMT, EPI, AM, XF, 4>(p, smem, nt, tile.x, tile.y, rows);
      return;
    }
  }
  if (rows > 32) {
    mfma_tile<FMT, EPI, AM, XF, 2>(p, smem, nt, tile.x, tile.y, rows);
    return;
  }
  mfma_tile<FMT, EPI, AM, XF, 1>(p, smem, nt, tile.x, tile.y, rows);
}

template <int FMT, int EPI, int AM, int XF = 0>
static hipError_t launch_mfma_t(const GemmArgs &g, hipStream_t s) {
  if (g.tile_rows != 0 && g.tile_rows != 64 && g.tile_rows != kMfmaBM) return hipErrorInvalidValue;
  const int64_t ncol = (EPI == EPI_SWIGLU) ? g.N / 2 : g.N;
  const int ntn = (int)((EPI == EPI_SWIGLU) ? cdiv(ncol, 128) : cdiv(ncol, 256));
  const int64_t total = (int64_t)g.max_tiles * ntn;
  const int64_t padded = cdiv(total, 8) * 8;
  const int per = (int)(padded / 8);
  if (g.tile_rows == 64)
    NF4MOE_LAUNCH(g, (k_mfma<FMT, EPI, AM, XF, 64>), dim3((unsigned)padded), dim3(512), s, g, ntn, per);
  else
    NF4MOE_LAUNCH(g, (k_mfma<FMT, EPI, AM, XF, 128>), dim3((unsigned)padded), dim3(512), s, g, ntn, per);
  return hipGetLastError();
}

// Instantiated operand modes: SwiGLU (gate_up) and plain outputs bf16 A; slot
// output (down projection) the pre-split planes.
template <int FMT>
static hipError_t mfma_pick(const GemmArgs &g, hipStream_t s) {
  const bool xf = g.glu != 0 || g.glu_inter != 0 || g.bias != nullptr;
  if (xf && g.epi != EPI_SWIGLU && g.epi != EPI_SLOT) return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_SWIGLU:
      if (g.a_is_f32 != 0) return hipErrorInvalidValue;
      return xf ? launch_mfma_t<FMT, EPI_SWIGLU, 0, 1>(g, s) : launch_mfma_t<FMT, EPI_SWIGLU, 0>(g, s);
    case EPI_PLAIN_F32:
      return g.a_is_f32 == 0 ? launch_mfma_t<FMT, EPI_PLAIN_F32, 0>(g, s) : hipErrorInvalidValue;
    case EPI_PLAIN_BF16:
      return g.a_is_f32 == 0 ? launch_mfma_t<FMT, EPI_PLAIN_BF16, 0>(g, s) : hipErrorInvalidValue;
    default:
      if (g.a_is_f32 != 2) return hipErrorInvalidValue;
      return xf ? launch_mfma_t<FMT, EPI_SLOT, 2, 1>(g, s) : launch_mfma_t<FMT, EPI_SLOT, 2>(g, s);
  }
}

hipError_t launch_mfma_grouped(const GemmArgs &g, hipStream_t s) {
  if (g.max_tiles <= 0) return hipSuccess;
  return g.fmt == 0 ? mfma_pick<0>(g, s) : g.fmt == 2 ? mfma_pick<2>(g, s) : mfma_pick<1>(g, s);
}

}  // namespace nf4moe
