// Device-side helpers shared by the gfx950 kernels of libnf4moe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Decode tables (index = 4-bit code).
// NF4: the 16-entry NormalFloat codebook, i.e. the QLoRA construction (normal
// quantiles at offset 0.9677083, 8 positive, 7 negative, plus 0, divided by
// the largest), rounded to fp32. The pages name this codebook (grouped-nf4-gemm
// PKG-INFO intro; "How do I run a grouped GEMM directly on NF4 packed MoE
// expert weights ...", section "Why it happens") without printing it.
// MXFP4: OCP e2m1 values; bit 3 = sign ("The MXFP4 native-byte lane").
// ---------------------------------------------------------------------------
__host__ __device__ constexpr float nf4_value(int code) {
  constexpr float t[16] = {
      -0x1.000000p+0f, -0x1.647362p-1f, -0x1.0cd65cp-1f, -0x1.94653cp-2f,
      -0x1.234496p-2f, -0x1.7a6a7ap-3f, -0x1.74f0d2p-4f, 0.0f,
      0x1.45f602p-4f,  0x1.4995bep-3f,  0x1.f809b4p-3f,  0x1.5a066cp-2f,
      0x1.c3496ap-2f,  0x1.200f52p-1f,  0x1.722760p-1f,  0x1.000000p+0f};
  return t[code & 15];
}

__host__ __device__ constexpr float e2m1_value(int code) {
  constexpr float t[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                           -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};
  return t[code & 15];
}

// Value of the code stored at even k (first) and odd k (second) of a byte.
// NF4 keeps the even-k code in the high nibble, MXFP4 in the low nibble.
// Formats: 0 NF4 with fp32 absmax per 64; 1 MXFP4 (e8m0 per 32); 2 NF4 with
// the absmax stored as bf16 (the same codes and decode, 2 bytes per block).
// Fmt<FMT>: kNF4 (NF4 codebook, nibble order and absmax semantics), kBlock
// (K elements per scale), raw(scale, idx) (the stored scale as 32 bits) and
// value(raw) (the fp32 multiplier).
template <int FMT> struct Fmt;
template <> struct Fmt<0> {
  static constexpr bool kNF4 = true;
  static constexpr int kBlock = 64;
  __device__ static uint32_t raw(const void *s, int64_t i) { return reinterpret_cast<const uint32_t *>(s)[i]; }
  __device__ static float value(uint32_t r) { return __uint_as_float(r); }
};
template <> struct Fmt<1> {
  static constexpr bool kNF4 = false;
  static constexpr int kBlock = 32;
  __device__ static uint32_t raw(const void *s, int64_t i) { return reinterpret_cast<const uint8_t *>(s)[i]; }
  __device__ static float value(uint32_t r);
};
template <> struct Fmt<2> {
  static constexpr bool kNF4 = true;
  static constexpr int kBlock = 64;
  __device__ static uint32_t raw(const void *s, int64_t i) { return reinterpret_cast<const uint16_t *>(s)[i]; }
  __device__ static float value(uint32_t r) { return __uint_as_float(r << 16); }
};

template <int FMT>
__host__ __device__ constexpr float even_value(uint32_t byte) {
  return Fmt<FMT>::kNF4 ? nf4_value(byte >> 4) : e2m1_value(byte & 15);
}
template <int FMT>
__host__ __device__ constexpr float odd_value(uint32_t byte) {
  return Fmt<FMT>::kNF4 ? nf4_value(byte & 15) : e2m1_value(byte >> 4);
}

// Scale of one block as an fp32 multiplier. NF4: the stored fp32 absmax.
// MXFP4: 2^(e8m0 - 127), e8m0 = 255 -> NaN.
__device__ inline float e8m0_to_f32(uint32_t e) {
  if (e == 255u) return __builtin_nanf("");
  if (e == 0u) return 0x1p-127f;               // the one subnormal power of two
  return __uint_as_float(e << 23);
}
__device__ inline float Fmt<1>::value(uint32_t r) { return e8m0_to_f32(r); }

// ---------------------------------------------------------------------------
// bf16 helpers (bf16 tensors cross the ABI as uint16 bit patterns)
// ---------------------------------------------------------------------------
// The smallest bf16 value >= the non-negative finite fp32 value with bits b,
// as bf16 bits (b itself when it is a bf16 value).
__host__ __device__ inline uint32_t bf16_round_up_bits(uint32_t b) {
  return ((b & 0xffffu) ? b + 0x10000u : b) >> 16;
}
__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ inline float bf16lo_to_f32(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ inline float bf16hi_to_f32(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

__device__ inline uint32_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
}

// Two floats to bf16 (round to nearest even) in one instruction: a in the low
// half, b in the high half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t f32x2_to_bf16x2_rne(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Order-preserving 32-bit key of a float for the routing order (logit
// descending, expert id ascending): larger float -> larger key; -0 is folded
// onto +0 first, so floats that compare equal get equal keys. Every float has
// a key, NaN included (a positive NaN above +inf, a negative one below -inf),
// so ranking on (key, id) is a total order and always selects exactly k
// experts, whatever the logits hold.
__device__ inline uint32_t float_order_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Codebook value of a 4-bit code computed with a select tree on literals, so a
// table build touches no memory.
__device__ inline float nf4_value_sel(uint32_t c) {
  const float a0 = (c & 1) ? nf4_value(1) : nf4_value(0), a1 = (c & 1) ? nf4_value(3) : nf4_value(2);
  const float a2 = (c & 1) ? nf4_value(5) : nf4_value(4), a3 = (c & 1) ? nf4_value(7) : nf4_value(6);
  const float a4 = (c & 1) ? nf4_value(9) : nf4_value(8), a5 = (c & 1) ? nf4_value(11) : nf4_value(10);
  const float a6 = (c & 1) ? nf4_value(13) : nf4_value(12), a7 = (c & 1) ? nf4_value(15) : nf4_value(14);
  const float b0 = (c & 2) ? a1 : a0, b1 = (c & 2) ? a3 : a2, b2 = (c & 2) ? a5 : a4, b3 = (c & 2) ? a7 : a6;
  const float d0 = (c & 4) ? b1 : b0, d1 = (c & 4) ? b3 : b2;
  return (c & 8) ? d1 : d0;
}
__device__ inline float e2m1_value_sel(uint32_t c) {
  const uint32_t m = c & 7;
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6: exponent/mantissa fields of the magnitude
  const float mag = m < 2 ? 0.5f * (float)m : (float)(2 + (m & 1)) * (float)(1u << ((m >> 1) - 1)) * 0.5f;
  return (c & 8) ? -mag : mag;
}
template <int FMT>
__device__ inline float2 pair_value(uint32_t b) {
  return Fmt<FMT>::kNF4 ? make_float2(nf4_value_sel(b >> 4), nf4_value_sel(b & 15))
                  : make_float2(e2m1_value_sel(b & 15), e2m1_value_sel(b >> 4));
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes). Every lane receives the result. Within a row of
// 16 lanes: DPP (quad xor 1, quad xor 2, half-row mirror, row mirror); across
// rows: lane shuffles.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
// Sum over aligned groups of LPR lanes (LPR in {16, 32, 64}).
template <int LPR>
__device__ inline float seg_sum(float v) {
  static_assert(LPR == 16 || LPR == 32 || LPR == 64, "segment");
  v = row16_sum(v);
  if (LPR >= 32) v += __shfl_xor(v, 16, kWave);
  if (LPR >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}
__device__ inline float wave_sum(float v) { return seg_sum<64>(v); }

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Max over the 32-lane half a lane belongs to.
__device__ inline float half_max(float v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ inline uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------------------
// Codebook gather without memory: lane c (mod 16) of the wave holds the value
// of code c, and ds_bpermute fetches it for any per-lane code. All 64 lanes
// must be active when the gather runs (inactive source lanes read as 0).
// ---------------------------------------------------------------------------
template <int FMT>
__device__ inline float codebook_lane() {
  const uint32_t c = threadIdx.x & 15;
  return Fmt<FMT>::kNF4 ? nf4_value_sel(c) : e2m1_value_sel(c);
}
__device__ inline float codebook_gather(float cb_lane, uint32_t code) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute((int)(code << 2), __float_as_int(cb_lane)));
}
// (value of the even-k code, value of the odd-k code) of a packed byte.
template <int FMT>
__device__ inline float2 pair_gather(float cb_lane, uint32_t b) {
  return Fmt<FMT>::kNF4 ? make_float2(codebook_gather(cb_lane, b >> 4), codebook_gather(cb_lane, b & 15))
                  : make_float2(codebook_gather(cb_lane, b & 15), codebook_gather(cb_lane, b >> 4));
}

// g * sigmoid(a g) = g / (1 + exp(-a g)), with the hardware exp2 and
// reciprocal (about 1 ulp each; the gate epilogues spent most of their
// instructions on the full-precision exp and the IEEE division). Large
// negative a g gives 1 / inf = 0, large positive 1 / 1; NaN stays NaN.
__device__ inline float sig_gate(float g, float a) {
  const float e = __builtin_amdgcn_exp2f(g * (-1.44269504088896341f * a));
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Gate_up epilogue: glu 0 is SwiGLU, silu(g) * u; glu 1 the clamped GLU,
// (u' + 1) * g' / (1 + exp(-alpha g')) with g' = min(g, limit) and
// u' = clamp(u, -limit, limit).
__device__ inline float glu_value(int glu, float alpha, float limit, float g, float u) {
  if (glu == 1) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
    return (u + 1.0f) * sig_gate(g, alpha);
  }
  return sig_gate(g, 1.0f) * u;
}

// Barrier that orders LDS only: global loads (and stores) issued before it
// stay in flight, unlike __syncthreads(), whose workgroup fence also covers
// global memory and so waits for every outstanding vector memory operation.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);  // no work moves across it, so no early waits
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// LDS decode table: byte -> (value of even-k code, value of odd-k code) as two
// fp32, replicated kRep times so the lanes of one LDS access read distinct
// banks. Entry (byte b, replica r) lives at float2 index b * kRep + r. Built by
// whole waves (`first_wave` .. `first_wave + nwaves - 1`) with codebook
// gathers; consecutive threads write consecutive 16-byte words so the writes
// are conflict-free. The caller synchronises before reading it.
// ---------------------------------------------------------------------------
template <int FMT, int kRep>
__device__ inline void build_pair_table(float2 *tab, int first_wave, int nwaves) {
  constexpr int kWords = 256 * kRep / 2;  // float4 words, kRep / 2 per byte
  float4 *dst = reinterpret_cast<float4 *>(tab);
  const int w = (int)(threadIdx.x >> 6) - first_wave;
  if (w < 0 || w >= nwaves) return;       // uniform per wave
  const int t = w * 64 + (int)(threadIdx.x & 63), nthreads = nwaves * 64;
  const float cb = codebook_lane<FMT>();
  // Gathers in batches of 8 words, all issued before the first wait; uniform
  // trip count, so the gathers always see full waves.
  for (int f0 = 0; f0 < kWords; f0 += 8 * nthreads) {
    float2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = f0 + i * nthreads + t;
      const int fc = f < kWords ? f : kWords - 1;
      v[i] = pair_gather<FMT>(cb, (uint32_t)(fc / (kRep / 2)));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = f0 + i * nthreads + t;
      if (f < kWords) dst[f] = make_float4(v[i].x, v[i].y, v[i].x, v[i].y);
    }
  }
}

// Byte offset (b * 256 + lanebyte) of table entry (b, lane & 31) for a 32-replica
// table of 8-byte entries: one v_perm_b32 places byte j of `word` above the
// lane's replica offset.
__device__ inline uint32_t tab_offset(uint32_t word, uint32_t lanebyte, int j) {
  return __builtin_amdgcn_perm(word, lanebyte, 0x0c0c0400u + ((uint32_t)j << 8));
}

}  // namespace nf4moe
