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
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace nf4moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kCUs = 256;     // compute units: one 512-thread workgroup on each at a time
constexpr int kApad = 72;     // bf16 per LDS row of A (64 + 8 padding)
constexpr int kQrow = 144;    // bytes per LDS row of an e4m3-split A: two 64-byte planes, 2 scale bytes, pad

typedef int i32x8_t __attribute__((ext_vector_type(8)));

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
  static_assert(AM == 0 || AM == 2 || (AM == 3 && FMT == 1), "operand mode");
  static_assert(MB == 4 || MB == 2 || MB == 1, "row blocks");
  constexpr bool AF32 = AM == 2;                      // a lo part exists
  constexpr bool AQ8 = AM == 3;                       // A as e4m3 planes: block-scaled MFMAs, no decode
  constexpr int kBM = 32 * MB;                        // rows per tile
  constexpr int ABUF = AQ8 ? kBM * kQrow : kBM * kApad * 2;  // bytes per A buffer
  // Row-split SwiGLU layout of the block-scaled MXFP4 gate_up (tiles of more
  // than 32 rows): wave w takes row blocks (w & 1) * MH .. + MH against the
  // gate and the up rows of output columns 32 (w >> 1) .. + 32, so each wave
  // reads half the A tile from LDS (two e4m3 planes: 4 KB per row block and
  // step, against 1 KB of codes per weight block) and forms SwiGLU in its own
  // registers. The NF4 bodies keep all rows per wave: there a weight block's
  // LDS lookups cost twice its A fragment, so the split would move no bytes.
  constexpr bool RS = AQ8 && EPI == EPI_SWIGLU && MB >= 2;
  constexpr int MH = MB / 2 > 0 ? MB / 2 : 1;

  if constexpr (!AQ8) build_mfma_table<FMT>(reinterpret_cast<uint4 *>(smem));
  auto abuf = [&](int hi_lo, int buf) __attribute__((always_inline)) -> uint16_t * {
    return reinterpret_cast<uint16_t *>(smem + (AQ8 ? 0 : kTabBytes) + (hi_lo * 2 + buf) * ABUF);
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
  const int rs_rh = wave & 1, rs_cg = wave >> 1;      // RS: row half, output column block

  const int64_t rowbytes = K / 2;
  const uint8_t *Be = p.B + (int64_t)e * N * rowbytes;
  const int64_t sc_per_row = K / Fmt<FMT>::kBlock;
  const int64_t sc_base = (int64_t)e * N * sc_per_row;

  // A-tile slice owned by this thread for the LDS fill: row am, EPT elements
  // starting at k0 + EPT * aq. Rows past the tile read a valid row (the tile's
  // first) and are zeroed when stored (measured: storing them unmasked, which
  // the results would allow, made the 64-row kernels 2-3 % slower).
  // A 32-row bf16 tile is 256 16-byte words: there the first 256 threads fill
  // it (NFILL) and the other waves skip the store. An e4m3-split row is 128
  // bytes of planes (+ 2 scale bytes): 4 threads of 32 bytes (128-row tiles)
  // or 8 of 16.
  constexpr int TPR = AQ8 ? (MB == 4 ? 4 : 8) : (MB == 1 && !AF32) ? 8 : 512 / kBM;  // fill threads per row
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
  constexpr int AW = AQ8 ? 128 / TPR / 16 : EPT * (AF32 ? 4 : 2) / 16;  // 16-byte words per thread
  // Loads run NSET K-steps ahead, one register set per step in flight (the
  // slice of step k + NSET loads while that of k + 1 waits to be stored to
  // LDS): two, four for the 32-row body, whose short steps leave two steps
  // little time to cover the memory latency (OLMoE-shaped batches of 16 and
  // 48 tokens 2 % faster; four sets in the 64-row body too gained nothing),
  // and four for AQ8.
  constexpr int NSET = AQ8 || MB == 1 ? 4 : 2;
  static_assert(NSET == 2 || NSET == 4, "register sets");
  uint4 aregs[NSET][AW];
  bool aoks[NSET] = {};
  uint32_t ascl[NSET] = {};  // AQ8: the row's two e8m0 scale bytes of the step
  auto load_a = [&](int64_t k0, int set) __attribute__((always_inline)) {
    if constexpr (AQ8) {
      // planes a1 [a_rows][K], a2 [a_rows][K], then scales [a_rows][K / 32]
      const int plane = aq / (TPR / 2), part = aq % (TPR / 2);
      const int64_t kc = k0 < K ? k0 : 0;
      aoks[set] = arow_ok && k0 < K;
      const uint8_t *q8 = reinterpret_cast<const uint8_t *>(p.a);
      const uint4 *src = reinterpret_cast<const uint4 *>(q8 + (int64_t)plane * p.a_rows * K + arow * K + kc +
                                                         part * (AW * 16));
#pragma unroll
      for (int i = 0; i < AW; ++i) aregs[set][i] = src[i];
      if (aq == 0)
        ascl[set] = *reinterpret_cast<const uint16_t *>(q8 + 2 * (int64_t)p.a_rows * K + arow * (K / 32) + kc / 32);
      return;
    }
    const int64_t kk = k0 + EPT * aq;
    aoks[set] = arow_ok && kk < K;
    const int64_t kc = kk < K ? kk : 0;
    // AM 0: EPT bf16; AM 2: EPT (hi, lo) bf16 pairs, 4 bytes each
    const uint4 *src = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(p.a) +
                                                       (arow * K + kc) * (AM == 2 ? 4 : 2));
#pragma unroll
    for (int i = 0; i < AW; ++i) aregs[set][i] = src[i];
  };
  auto store_a = [&](int buf, int set) __attribute__((always_inline)) {
    if (NFILL < 512 && tid >= NFILL) return;  // whole waves
    const uint4 *areg = aregs[set];
    const bool a_ok = aoks[set];
    if constexpr (AQ8) {  // rows past the tile (or K) as zeros with scale 2^0
      const int plane = aq / (TPR / 2), part = aq % (TPR / 2);
      uint8_t *row = reinterpret_cast<uint8_t *>(abuf(0, buf)) + am * kQrow;
#pragma unroll
      for (int i = 0; i < AW; ++i)
        *reinterpret_cast<uint4 *>(row + plane * 64 + part * (AW * 16) + 16 * i) = a_ok ? areg[i] : make_uint4(0, 0, 0, 0);
      if (aq == 0) *reinterpret_cast<uint16_t *>(row + 128) = (uint16_t)(a_ok ? ascl[set] : 0x7f7fu);
      return;
    }
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
  auto load_b = [&](int64_t k0, uint4 &bq, uint32_t &braw, bool &bok) __attribute__((always_inline)) {
    const int64_t kk = k0 + 32 * g;
    bok = nvalid && kk < K;
    const int64_t kc = kk < K ? kk : 0;
    bq = *reinterpret_cast<const uint4 *>(Be + nrow_c * rowbytes + kc / 2);
    const int64_t sidx = Fmt<FMT>::kNF4 ? (k0 < K ? k0 / 64 : 0) : kc / 32;
    braw = Fmt<FMT>::raw(p.B_scale, sc_base + nrow_c * sc_per_row + sidx);
  };
  auto scale_of = [&](uint32_t raw, bool ok) __attribute__((always_inline)) -> float {
    const float v = Fmt<FMT>::value(raw);
    return ok ? v : 0.0f;
  };

  const f32x16_t zero16 = {};
  f32x16_t C[MB], P[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) C[mb] = zero16;

  // One K-step on LDS buffer `cur` with codes bq and scale bs. Loads run
  // NSET steps ahead: the activation slice of step k + NSET into register set
  // `aset` at the start, the codes and scale of step k + NSET into bq / br /
  // bok once this step's lookups have read bq; the slice of step k + 1 (set
  // (aset + 1) % NSET) goes to the other LDS buffer at the end.
  auto step = [&](int64_t k0, int cur, int aset, uint4 &bq, float bs, uint32_t &br, bool &bok) __attribute__((always_inline)) {
    // Loads are issued (from clamped, valid addresses) and stored even past
    // the last step, so no branch splits the load/wait bookkeeping; the
    // extra data is unused.
    const bool more = k0 + kBK < K;
    load_a(k0 + NSET * kBK, aset);
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
    auto read_a = [&](int sa, bf16x8_t *dh, bf16x8_t *dl) __attribute__((always_inline)) {
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
      if (u == 3) {  // every lookup of this step has read bq: reuse it for step k + NSET
        load_b(k0 + NSET * kBK, bq, br, bok);
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
    store_a(cur ^ 1, (aset + 1) % NSET);
    lds_barrier();
    return more;
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if constexpr (AQ8) {
    // Block-scaled MXFP4 loop. Steps are short here (no decode; half the
    // MFMA time of the NF4 products), and per-lane weight loads (each lane
    // its own weight row, 32 rows per instruction) kept the vector memory
    // unit busy 83 % of the time. So the workgroup stages its 256 weight rows
    // through LDS four K-steps at a time (a super-step: 128 bytes of codes
    // and 8 scale bytes per row), loaded 128 contiguous bytes per 8 lanes, and
    // each wave reads its MFMA operand (row l32, 32 codes of half g) from LDS.
    // A goes through LDS per step, its loads four steps ahead as before.
    constexpr int kBrow = 144;                       // LDS bytes per staged weight row
    uint8_t *Bs = smem + 2 * ABUF;                    // after the two A buffers: [2][256][kBrow]
    const int64_t n_ss = (K + 4 * kBK - 1) / (4 * kBK);  // super-steps
    // global row of staged row i (wave i / 32, column i % 32), clamped when past N
    auto staged_row = [&](int i) __attribute__((always_inline)) -> int64_t {
      const int w = i >> 5, c = i & 31;
      int64_t cl, nr;
      if (EPI == EPI_SWIGLU) {
        cl = (int64_t)nt * 128 + 32 * (w & 3) + c;
        nr = (XF && p.glu_inter) ? 2 * cl + (w >> 2) : cl + (w >> 2) * ncol;
      } else {
        cl = (int64_t)nt * 256 + 32 * w + c;
        nr = cl;
      }
      return cl < ncol ? nr : 0;
    };
    // staging registers of one super-step (named, not arrays: a loop over an
    // array here is indexed at run time when the compiler first places it)
    uint4 bst0, bst1, bst2, bst3;
    uint32_t sst0 = 0, sst1 = 0, sst2 = 0, sst3 = 0;
    auto bcode_src = [&](int64_t kb, int i) __attribute__((always_inline)) -> const uint4 * {
      const int id = i * 512 + tid, r = id >> 3, part = id & 7;
      const int64_t off = kb / 2 + 16 * part;
      return reinterpret_cast<const uint4 *>(Be + staged_row(r) * rowbytes + (off < rowbytes ? off : 0));
    };
    // the two scale bytes of step i of the super-step (byte loads: MXFP4
    // scales carry no alignment); K % 64 == 0, so both are in the row or
    // the pair is clamped to its start
    auto bscale_pair = [&](const uint8_t *sr, int64_t kb, int i) __attribute__((always_inline)) -> uint32_t {
      const int64_t k32 = kb / 32 + 2 * i;
      const uint8_t *q = sr + (k32 < sc_per_row ? k32 : 0);
      return (uint32_t)q[0] | ((uint32_t)q[1] << 8);
    };
    auto load_bss = [&](int64_t j) __attribute__((always_inline)) {  // super-step j into registers (clamped addresses)
      const int64_t kb = j * 4 * kBK;
      bst0 = *bcode_src(kb, 0);
      bst1 = *bcode_src(kb, 1);
      bst2 = *bcode_src(kb, 2);
      bst3 = *bcode_src(kb, 3);
      if (tid < 256) {
        const uint8_t *sr = reinterpret_cast<const uint8_t *>(p.B_scale) + sc_base + staged_row(tid) * sc_per_row;
        sst0 = bscale_pair(sr, kb, 0);
        sst1 = bscale_pair(sr, kb, 1);
        sst2 = bscale_pair(sr, kb, 2);
        sst3 = bscale_pair(sr, kb, 3);
      }
    };
    auto store_bss = [&](int buf) __attribute__((always_inline)) {
      uint8_t *base = Bs + buf * 256 * kBrow;
      auto dst = [&](int i) __attribute__((always_inline)) -> uint4 * {
        const int id = i * 512 + tid, r = id >> 3, part = id & 7;
        return reinterpret_cast<uint4 *>(base + r * kBrow + 16 * part);
      };
      *dst(0) = bst0;
      *dst(1) = bst1;
      *dst(2) = bst2;
      *dst(3) = bst3;
      if (tid < 256)
        *reinterpret_cast<uint2 *>(base + tid * kBrow + 128) = make_uint2(sst0 | (sst1 << 16), sst2 | (sst3 << 16));
    };
    // written out: a loop here would index the A register sets at run time
    // when the compiler first places them (in scratch)
    load_a(0, 0);
    load_a(kBK, 1);
    load_a(2 * kBK, 2);
    load_a(3 * kBK, 3);
    load_bss(0);
    store_a(0, 0);
    store_bss(0);
    if (n_ss > 1) load_bss(1);
    lds_barrier();
    // step s of super-step j: A from LDS buffer cur, B from staged buffer j % 2
    // (cur, set, s are compile-time constants: each call is its own
    // instantiation, so the register sets are never indexed at run time)
    auto qstep = [&](int64_t k0, auto cur_c, auto set_c, auto s_c, int64_t j) __attribute__((always_inline)) -> bool {
      constexpr int cur = decltype(cur_c)::value, set = decltype(set_c)::value, s = decltype(s_c)::value;
      const bool more = k0 + kBK < K;
      load_a(k0 + 4 * kBK, set);
      __builtin_amdgcn_sched_barrier(0);
      // B: this lane's 32 e2m1 codes (k0 + 32 g ...) and their e8m0 scale; A:
      // row l32 of each 32-row block, k = 16 g + 0..15 and 32 + 16 g + 0..15
      // of each plane, and the row's scale for block g. C += A1 * B + A2 * B
      // with both operands' block scales applied.
      const uint8_t *A8 = reinterpret_cast<const uint8_t *>(abuf(0, cur));
      if constexpr (RS) {
        // half the tile's rows (row blocks rh * MH ..) against the gate and
        // the up rows of the wave's 32 output columns (staged rows cg * 32
        // and (cg + 4) * 32 onwards): C[0, MH) gate, C[MH, MB) up
        const uint8_t *bb = Bs + (j & 1) * 256 * kBrow;
        const uint8_t *brg = bb + (rs_cg * 32 + l32) * kBrow;
        const uint8_t *bru = bb + ((rs_cg + 4) * 32 + l32) * kBrow;
        const uint4 qg = *reinterpret_cast<const uint4 *>(brg + 32 * s + 16 * g);
        const uint4 qu = *reinterpret_cast<const uint4 *>(bru + 32 * s + 16 * g);
        const int sbg = brg[128 + 2 * s + g], sbu = bru[128 + 2 * s + g];
        const i32x8_t bvg = {(int)qg.x, (int)qg.y, (int)qg.z, (int)qg.w, 0, 0, 0, 0};
        const i32x8_t bvu = {(int)qu.x, (int)qu.y, (int)qu.z, (int)qu.w, 0, 0, 0, 0};
#pragma unroll
        for (int mh = 0; mh < MH; ++mh) {
          const uint8_t *row = A8 + ((rs_rh * MH + mh) * 32 + l32) * kQrow;
          const uint4 p0 = *reinterpret_cast<const uint4 *>(row + 16 * g);
          const uint4 p1 = *reinterpret_cast<const uint4 *>(row + 32 + 16 * g);
          const uint4 q0 = *reinterpret_cast<const uint4 *>(row + 64 + 16 * g);
          const uint4 q1 = *reinterpret_cast<const uint4 *>(row + 96 + 16 * g);
          const int sa = row[128 + g];
          const i32x8_t a1 = {(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
          const i32x8_t a2 = {(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
          C[mh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bvg, C[mh], 0, 4, 0, sa, 0, sbg);
          C[MH + mh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bvu, C[MH + mh], 0, 4, 0, sa, 0, sbu);
          C[mh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a2, bvg, C[mh], 0, 4, 0, sa, 0, sbg);
          C[MH + mh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a2, bvu, C[MH + mh], 0, 4, 0, sa, 0, sbu);
        }
      } else {
      const uint8_t *brow = Bs + (j & 1) * 256 * kBrow + (wave * 32 + l32) * kBrow;
      const uint4 bq = *reinterpret_cast<const uint4 *>(brow + 32 * s + 16 * g);
      const int sb = brow[128 + 2 * s + g];
      const i32x8_t bv = {(int)bq.x, (int)bq.y, (int)bq.z, (int)bq.w, 0, 0, 0, 0};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint8_t *row = A8 + (mb * 32 + l32) * kQrow;
        const uint4 p0 = *reinterpret_cast<const uint4 *>(row + 16 * g);
        const uint4 p1 = *reinterpret_cast<const uint4 *>(row + 32 + 16 * g);
        const uint4 q0 = *reinterpret_cast<const uint4 *>(row + 64 + 16 * g);
        const uint4 q1 = *reinterpret_cast<const uint4 *>(row + 96 + 16 * g);
        const int sa = row[128 + g];
        const i32x8_t a1 = {(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
        const i32x8_t a2 = {(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
        C[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bv, C[mb], 0, 4, 0, sa, 0, sb);
        C[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a2, bv, C[mb], 0, 4, 0, sa, 0, sb);
      }
      }
      __builtin_amdgcn_sched_barrier(0);
      store_a(cur ^ 1, (set + 1) & 3);
      if (s == 3) {  // super-step j + 1 into the other staged buffer (read last in j - 1)
        store_bss((int)((j + 1) & 1));
        if (j + 2 < n_ss) load_bss(j + 2);
      }
      lds_barrier();
      return more;
    };
    for (int64_t j = 0;; ++j) {
      const int64_t k0 = j * 4 * kBK;
      if (!qstep(k0, I0{}, I0{}, I0{}, j)) break;
      if (!qstep(k0 + kBK, I1{}, I1{}, I1{}, j)) break;
      if (!qstep(k0 + 2 * kBK, I0{}, I2{}, I2{}, j)) break;
      if (!qstep(k0 + 3 * kBK, I1{}, I3{}, I3{}, j)) break;
    }
  } else {
    // B register sets (named, so that no array is ever indexed at run time)
    uint4 bq0, bq1, bq2, bq3;
    uint32_t br0, br1, br2 = 0, br3 = 0;
    bool bok0, bok1, bok2 = false, bok3 = false;
    load_a(0, 0);
    load_b(0, bq0, br0, bok0);
    load_a(kBK, 1);
    load_b(kBK, bq1, br1, bok1);
    if constexpr (NSET == 4) {
      load_a(2 * kBK, 2);
      load_b(2 * kBK, bq2, br2, bok2);
      load_a(3 * kBK, 3);
      load_b(3 * kBK, bq3, br3, bok3);
    }
    store_a(0, 0);
    lds_barrier();

    // Unrolled by NSET so the register sets rotate without copies: step k
    // computes on B set k % NSET and LDS buffer k % 2, loads A(k + NSET) into
    // set k % NSET and stores A(k + 1) from set (k + 1) % NSET.
    auto one = [&](int64_t k0, auto I) __attribute__((always_inline)) -> bool {
      constexpr int i = decltype(I)::value;
      uint4 &bq = i == 0 ? bq0 : (i == 1 ? bq1 : (i == 2 ? bq2 : bq3));
      uint32_t &br = i == 0 ? br0 : (i == 1 ? br1 : (i == 2 ? br2 : br3));
      bool &bok = i == 0 ? bok0 : (i == 1 ? bok1 : (i == 2 ? bok2 : bok3));
      return step(k0, i & 1, i, bq, scale_of(br, bok), br, bok);
    };
    for (int64_t k0 = 0;; k0 += NSET * kBK) {
      if (!one(k0, I0{})) break;
      if (!one(k0 + kBK, I1{})) break;
      if constexpr (NSET == 4) {
        if (!one(k0 + 2 * kBK, I2{})) break;
        if (!one(k0 + 3 * kBK, I3{})) break;
      }
    }
  }

  // ---- epilogue. 32x32 accumulator: lane holds column l32, rows
  // 8 * (v / 4) + 4 * g + (v % 4) for v = 0..15 of each 32-row block mb.
  // (truncated bf16 hi, RNE bf16 of the rest) of h values of rows m, m + 1 in
  // one word each; their lo parts share one conversion instruction
  auto store_h_pair = [&](int64_t o, int m, const float *h) __attribute__((always_inline)) {
    if (p.c_split) {
      const uint32_t b0 = __float_as_uint(h[0]), b1 = __float_as_uint(h[1]);
      const uint32_t lo = f32x2_to_bf16x2_rne(h[0] - __uint_as_float(b0 & 0xffff0000u),
                                              h[1] - __uint_as_float(b1 & 0xffff0000u));
      if (m < trows) reinterpret_cast<uint32_t *>(p.c)[o] = __builtin_amdgcn_perm(lo, b0, 0x05040302u);
      if (m + 1 < trows) reinterpret_cast<uint32_t *>(p.c)[o + ncol] = __builtin_amdgcn_perm(lo, b1, 0x07060302u);
    } else {
      if (m < trows) reinterpret_cast<float *>(p.c)[o] = h[0];
      if (m + 1 < trows) reinterpret_cast<float *>(p.c)[o + ncol] = h[1];
    }
  };
  if constexpr (RS) {  // gate in C[0, MH), up in C[MH, MB), both in this wave
    const int64_t rcol = (int64_t)nt * 128 + 32 * rs_cg + l32;
    if (rcol >= ncol) return;
    float bg = 0.0f, bu = 0.0f;
    if (XF && p.bias) {
      const float *bb = p.bias + (int64_t)e * N;
      bg = bb[p.glu_inter ? 2 * rcol : rcol];
      bu = bb[p.glu_inter ? 2 * rcol + 1 : rcol + ncol];
    }
#pragma unroll
    for (int mh = 0; mh < MH; ++mh) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int m = (rs_rh * MH + mh) * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        float h[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {  // rows past the tile compute unused values
          if constexpr (XF)
            h[q] = glu_value(p.glu, p.glu_alpha, p.glu_limit, C[mh][v + q] + bg, C[MH + mh][v + q] + bu);
          else
            h[q] = sig_gate(C[mh][v + q], 1.0f) * C[MH + mh][v + q];
        }
        store_h_pair((int64_t)(trow0 + m) * ncol + rcol, m, h);
      }
    }
    return;
  }
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
    // values v and v + 1 of a lane are rows m and m + 1 of its column: their
    // lo parts share one conversion instruction
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int m = mb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        float h[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {  // rows past the tile compute unused values
          const float up = xch[((w4 * MB + mb) * 16 + v + q) * 64 + lane];
          if constexpr (XF)
            h[q] = glu_value(p.glu, p.glu_alpha, p.glu_limit, C[mb][v + q] + bg, up + bu);
          else
            h[q] = sig_gate(C[mb][v + q], 1.0f) * up;
        }
        if (!nvalid) continue;
        store_h_pair((int64_t)(trow0 + m) * ncol + col, m, h);
      }
    }
    return;
  }
  // slot epilogue: each row's slot and routing weight, loaded once per tile
  // into LDS (free since the last K-step's closing barrier) instead of two
  // dependent global loads per row in every lane
  int *s_slot = reinterpret_cast<int *>(smem);
  float *s_w = reinterpret_cast<float *>(smem) + kBM;
  if constexpr (EPI == EPI_SLOT) {
    if (tid < trows) {
      const int sl = p.slot_of[trow0 + tid];
      s_slot[tid] = sl;
      s_w[tid] = p.slot_w[sl];
    }
    lds_barrier();
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
        const int64_t slot = s_slot[m];
        reinterpret_cast<float *>(p.c)[slot * N + col] = s_w[m] * (XF ? y + yb : y);
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
  // for an fp32 A); e4m3-split A: no table, two buffers, and room for the
  // SwiGLU epilogue's exchange of the up values
  constexpr int kXch = TR / 32 * 4 * 16 * 64 * 4;
  constexpr int kQ8 = 2 * TR * kQrow + 2 * 256 * 144;  // A buffers + staged weight rows
  constexpr int kSmem = AM == 3 ? (kQ8 > kXch ? kQ8 : kXch) : kTabBytes + (AM == 2 ? 4 : 2) * TR * kApad * 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  // XCD-aware order: hardware XCD = blockIdx.x % 8, and the XCDs take equal
  // shares of the work, in one of two orders (results do not depend on it):
  //  - tile major, n-tile minor, over the tiles the device table holds (the
  //    grid is sized for the most tiles): the workgroups an XCD runs at once
  //    cover a few row tiles across all their weight tiles, so a row tile's
  //    activations, and a weight tile read by an expert's consecutive row
  //    tiles, are fetched into that XCD's L2 once (gate_up FETCH_SIZE -64 %
  //    at the OLMoE-shaped prefill; gpt-oss-shaped T = 2048 gate_up 716 ->
  //    675 us, down 648 -> 577 us; Qwen3-shaped T = 512 gate_up 161 -> 132 us).
  //    When the launch takes more than one round of workgroups, the items come
  //    from the class-ordered table, longest tiles first (class 0: more than
  //    64 rows, then 33-64, then at most 32): each XCD takes a contiguous run
  //    of each class, the classes' remainders dealt round the XCDs so that no
  //    XCD gets more than its share of the whole, and starts its long tiles
  //    first, so the short ones fill the end of the launch (OLMoE-shaped
  //    prefill -1.8 %, gpt-oss-shaped T = 2048 -6 %, Qwen3-shaped T = 128 /
  //    512 -4 / -3 %);
  //  - n-tile major, tile minor over the whole grid, for the NF4 down
  //    projections, which ran 3-10 % slower in tile-major order (the table's
  //    class order puts long tiles first within each n-tile there too).
  constexpr bool kTileMajor = EPI == EPI_SWIGLU || FMT == 1;
  const int L = blockIdx.x;
  int ti = -1, nt = 0;
  bool by_class = false;
  if constexpr (kTileMajor) {
    const int nall = min(*p.n_tiles, p.max_tiles);
    if (nall * ntn <= kCUs) {  // one round: every tile starts at once, in group order
      const int total = nall * ntn, per_xcd = (total + 7) >> 3;
      const int Lp = (L & 7) * per_xcd + (L >> 3);
      if ((L >> 3) >= per_xcd || Lp >= total) return;
      ti = Lp / ntn;
      nt = Lp % ntn;
    } else {
      by_class = true;
      const int na = min(p.n_tiles[1], nall), nb = min(p.n_tiles[2], nall - na);
      const int x = L & 7;
      int j = L >> 3, o = 0, tbase = 0;
      for (int cls = 0; cls < 3; ++cls) {
        const int ncl = cls == 0 ? na : (cls == 1 ? nb : nall - na - nb);
        const int items = ncl * ntn, q = items >> 3, r = items & 7;
        int start = x * q, mine = q;
        for (int y = 0; y < 8; ++y) {  // this class's remainders go to XCDs o, o + 1, ... (mod 8)
          const int extra = ((y - o) & 7) < r ? 1 : 0;
          if (y < x) start += extra;
          if (y == x) mine += extra;
        }
        if (j < mine) {
          ti = tbase + (start + j) / ntn;
          nt = (start + j) % ntn;
          break;
        }
        j -= mine;
        o = (o + r) & 7;
        tbase += ncl;
      }
      if (ti < 0) return;
    }
  } else {
    const int Lp = (L & 7) * per + (L >> 3);
    if (Lp >= p.max_tiles * ntn) return;
    nt = Lp / p.max_tiles;
    ti = Lp % p.max_tiles;
    if (ti >= *p.n_tiles) return;
  }
  // expert, row0, rows, rows of the whole group (from the class-ordered table
  // when the launch runs in more than one round)
  const int4 tile = p.tiles[(by_class ? p.max_tiles : 0) + ti];
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

// ---------------------------------------------------------------------------
// bf16 activations as the MXFP4 kernels' block-scaled operand: per 32-element
// block of a row, s = floor(log2 max |x|) - 7 (so |x| / 2^s < 256, inside
// e4m3's range), the e8m0 byte s + 127, and two e4m3 parts a1 = RNE(x / 2^s),
// a2 = RNE(x / 2^s - a1). A bf16 value has 8 significant bits and e4m3 4, so
// a1 + a2 = x / 2^s exactly for every element within 2^9 of the block
// maximum (smaller ones keep an error below 2^-17 of that maximum).
// Layout: plane a1 [rows][K], plane a2 [rows][K], scales [rows][K / 32].
// ---------------------------------------------------------------------------
__device__ inline uint32_t e4m3_rne(float v) {  // finite, |v| <= 448
  const uint32_t sgn = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t c;
  if (a < 0.015625f) {  // below 2^-6: steps of 2^-9 (8 is the smallest normal, code 0x08)
    c = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {              // round the fp32 significand to 3 bits (to even), then rebias 127 -> 7
    const uint32_t b = __float_as_uint(a);
    c = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sgn | c;
}

__device__ inline float e4m3_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  const float mag = ex == 0 ? (float)m * 0.001953125f : __uint_as_float(((ex + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

__global__ __launch_bounds__(256) void k_e4m3_split(const uint16_t *__restrict__ x, int64_t rows, int K,
                                                    uint8_t *__restrict__ q) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8 elements per thread
  const int64_t n8 = rows * (K / 8);
  const bool ok = i < n8;
  const uint4 xv = ok ? reinterpret_cast<const uint4 *>(x)[i] : make_uint4(0, 0, 0, 0);
  const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  m = fmaxf(m, __shfl_xor(m, 1, 4));  // the 32-block: 4 consecutive lanes
  m = fmaxf(m, __shfl_xor(m, 2, 4));
  int sx = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xffu) - 127 - 7 : 0;
  sx = sx < -127 ? -127 : (sx > 126 ? 126 : sx);
  const float inv = __uint_as_float((uint32_t)(127 - sx) << 23);  // 2^-s
  uint32_t p1[2] = {0u, 0u}, p2[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t = f[j] * inv;
    const uint32_t c1 = e4m3_rne(t);
    const uint32_t c2 = e4m3_rne(t - e4m3_value(c1));
    p1[j / 4] |= c1 << (8 * (j % 4));
    p2[j / 4] |= c2 << (8 * (j % 4));
  }
  if (!ok) return;
  const int64_t row = i / (K / 8), c8 = i % (K / 8);
  uint8_t *a1 = q + row * K + 8 * c8;
  uint8_t *a2 = a1 + rows * K;
  *reinterpret_cast<uint2 *>(a1) = make_uint2(p1[0], p1[1]);
  *reinterpret_cast<uint2 *>(a2) = make_uint2(p2[0], p2[1]);
  if ((c8 & 3) == 0) q[2 * rows * K + row * (K / 32) + c8 / 4] = (uint8_t)(sx + 127);
}

size_t e4m3_split_bytes(int64_t rows, int K) { return (size_t)rows * K * 2 + (size_t)rows * (K / 32); }

hipError_t launch_e4m3_split(const uint16_t *x, int64_t rows, int K, uint8_t *q, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K % 32) return hipErrorInvalidValue;
  const int64_t n8 = rows * (K / 8);
  hipLaunchKernelGGL(k_e4m3_split, dim3((unsigned)cdiv(n8, 256)), dim3(256), 0, s, x, rows, K, q);
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
      if constexpr (FMT == 1) {  // MXFP4 with an e4m3-split A: block-scaled MFMAs
        if (g.a_is_f32 == 3)
          return xf ? launch_mfma_t<FMT, EPI_SWIGLU, 3, 1>(g, s) : launch_mfma_t<FMT, EPI_SWIGLU, 3>(g, s);
      }
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
