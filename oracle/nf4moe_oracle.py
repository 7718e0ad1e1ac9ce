"""fp64 CPU oracle: quantize, dequantize, route, grouped GEMM, SwiGLU, combine.

TEST INFRASTRUCTURE ONLY -- only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may use it. It shares no code with the HIP
path and imports nothing from it.

What it computes is the plain definition that the method reaches up to fp32
reduction order: decode every 4-bit weight to its fp32 value, then run the
dense per-expert products. The page "How do I run a grouped GEMM directly on
NF4 packed MoE expert weights, without dequantizing to bf16 first?", section
"Expected result", states that the fused kernel's per-element decode is
identical to the reference decode and only the fp32 reduction order differs;
its section "Smallest correct example" asserts the kernel against the fp64
product of the reference decode, which is what this module is.

Every floating-point step here is fp64 unless a step's definition fixes fp32:
the stored absmax (fp32), the decoded weight (one fp32 product) and the e8m0
scale (a power of two).

Readings of points the pages leave open:
  * NF4 codebook values: the pages name the bitsandbytes 16-entry NormalFloat
    codebook but never print it. We build it with the published QLoRA
    construction (normal quantiles with offset 0.9677083, 8 positive, 7
    negative, plus 0, divided by the maximum), evaluated in fp64 and rounded to
    fp32. Byte compatibility with real bitsandbytes checkpoints: parity
    unpinned.
  * NF4 nibble order: high nibble = even k. MXFP4: low nibble = even k. Both
    parity unpinned against real checkpoints (none here).
  * NF4 quantize: exact nearest code, ties to the lower code; an all-zero
    block stores absmax 0 and code 7 (the 0.0 entry).
  * NF4 with bf16 absmax (the experts4bit-qlora page's --absmax-dtype bf16,
    lossless for bf16-source weights): the block absmax is rounded up to the
    nearest bf16 value (unchanged when it is one) and the codes are chosen
    against that value; the decode widens it back to fp32.
  * MXFP4 quantize: OCP MX v1.0 rule, shared exponent
    X = floor(log2(amax)) - 2 clamped to [-127, 127], e2m1 nearest with ties
    to the even code, saturating at 6; the code's sign bit is the input's
    sign bit (so -0.0, and negatives that round to 0, give code 8 = -0.0).
  * Router: logits = x . W_r^T (+ optional per-expert bias), top-k by
    (logit descending, expert id ascending), weights = softmax over the k
    selected logits (renormalize=1) or the full softmax at the selected ids
    (renormalize=0).
  * Grouping: stable counting sort of slots s = t*k + j by expert.
  * gate_up rows [0, I) are gate, [I, 2I) are up; SwiGLU = silu(gate) * up.
  * The gpt-oss expert form, which the experts4bit-qlora page names ("Scope":
    per-expert biases and a clamped-GLU epilogue) without defining: optional
    biases b13 [E, 2I] (added to the gate_up product, row order of w13) and
    b2 [E, H] (added to each expert's down output before its routing weight);
    optional interleaved gate/up rows (2c gate, 2c + 1 up); clamped GLU
    g' = min(g, limit), u' = clamp(u, -limit, limit),
    h = (u' + 1) * g' * sigmoid(alpha * g'), alpha and limit parameters.
  * Combine: out[t] = sum_j w[t, j] * y[t*k + j] in fp64, not rounded.
"""
from __future__ import annotations

import numpy as np
from scipy.special import ndtri

__all__ = [
    "FMT_NF4", "FMT_MXFP4", "FMT_NF4_BF16ABS", "NF4_BLOCK", "MXFP4_BLOCK", "bf16_round_up",
    "nf4_codebook", "e2m1_values",
    "nf4_quantize", "nf4_dequantize", "mxfp4_quantize", "mxfp4_dequantize",
    "quantize", "dequantize", "block_size",
    "bf16_bits_to_f64", "router_logits", "topk_route", "permute",
    "grouped_gemm", "grouped_dgrad", "swiglu", "clamped_glu", "GLU_SWIGLU", "GLU_CLAMPED",
    "moe_forward", "rel_err",
]

FMT_NF4 = 0
FMT_MXFP4 = 1
FMT_NF4_BF16ABS = 2      # NF4 with the block absmax stored as bf16
GLU_SWIGLU = 0
GLU_CLAMPED = 1
NF4_BLOCK = 64
MXFP4_BLOCK = 32


# --------------------------------------------------------------------------
# Codebooks
# --------------------------------------------------------------------------
def nf4_codebook() -> np.ndarray:
    """The 16 NF4 values as float32, ascending (index = 4-bit code).

    Pages: the grouped-nf4-gemm PKG-INFO intro and the page "How do I run a
    grouped GEMM directly on NF4 packed MoE expert weights ...", section "Why
    it happens", name the bitsandbytes NF4 codebook (a 16-entry codebook index
    per weight). The values are not printed; this is the QLoRA "4-bit
    NormalFloat" construction: positive part = Phi^-1 at 8 evenly spaced
    levels from delta down to 1/2 (exclusive), negative part = -Phi^-1 at 7
    levels, plus an exact zero; everything divided by the largest value.
    delta = 1 - (1/30 + 1/32) / 2.
    """
    delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    pos = ndtri(np.linspace(delta, 0.5, 9)[:-1])
    neg = -ndtri(np.linspace(delta, 0.5, 8)[:-1])
    vals = np.sort(np.concatenate([pos, neg, [0.0]]))
    vals = vals / vals.max()
    return vals.astype(np.float32)


def e2m1_values() -> np.ndarray:
    """OCP MX v1.0 FP4 (E2M1) values by 4-bit code, as float32.

    Bit 3 is the sign; bits 2..1 the exponent (bias 1); bit 0 the mantissa.
    Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (grouped-nf4-gemm PKG-INFO, "The
    MXFP4 native-byte lane": e2m1 is a 16-entry codebook served by the same
    decode with the table swapped).
    """
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    return np.array(mags + [-m for m in mags], dtype=np.float32)


def block_size(fmt: int) -> int:
    return MXFP4_BLOCK if fmt == FMT_MXFP4 else NF4_BLOCK


# --------------------------------------------------------------------------
# NF4 quantize / dequantize
# --------------------------------------------------------------------------
def bf16_round_up(a) -> np.ndarray:
    """The smallest bfloat16 value >= each non-negative finite value of a, as
    fp64 (a itself when it is one): with a = m * 2^e, m in [0.5, 1), bf16 keeps
    8 significant bits, so the grid step is 2^(e - 8)."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, e - 8)
    return np.where(a > 0, np.ceil(a / step) * step, a)


def nf4_quantize(w: np.ndarray, absmax_bf16: bool = False):
    """fp32 [N, K] -> (packed uint8 [N, K/2], absmax float32 [N, K/64]), or with
    absmax_bf16 the absmax as bf16 bits (uint16), rounded up to a bf16 value
    before the codes are chosen.

    grouped-nf4-gemm PKG-INFO, "Try it on CPU right now", block 1, and the
    page "How do I run a grouped GEMM ...", section "Supported scope": per row,
    per 64-element K block, absmax = max |w| (stored fp32); every weight is
    replaced by the index of the nearest codebook value of w / absmax; two
    codes per byte.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % NF4_BLOCK:
        raise ValueError("K must be a multiple of 64")
    cb = nf4_codebook().astype(np.float64)
    codes = np.empty((N, K), dtype=np.uint8)
    absmax = np.empty((N, K // NF4_BLOCK), dtype=np.float64)
    step = max(1, (1 << 16) // K)                             # bound the temporaries
    for r0 in range(0, N, step):
        blocks = w[r0:r0 + step].reshape(-1, K // NF4_BLOCK, NF4_BLOCK).astype(np.float64)
        a = np.abs(blocks).max(axis=2)                        # exact (a max)
        if absmax_bf16:
            a = bf16_round_up(a)
        # Nearest code to w among c_i * absmax. c_i * absmax is exact in fp64
        # (24-bit by 24-bit significands), and so is each distance near a tie;
        # argmin returns the first (lower) code on an exact tie.
        dist = np.abs(blocks[..., None] - cb * a[..., None, None])
        c = np.argmin(dist, axis=-1).astype(np.uint8)
        c[a == 0.0] = 7                                       # all-zero block -> 0.0
        codes[r0:r0 + step] = c.reshape(-1, K)
        absmax[r0:r0 + step] = a
    packed = ((codes[:, 0::2] << 4) | codes[:, 1::2]).astype(np.uint8)
    if absmax_bf16:
        bits = absmax.astype(np.float32).view(np.uint32)
        assert not np.any(bits & 0xFFFF), "absmax is not a bf16 value"
        return packed, (bits >> 16).astype(np.uint16)
    return packed, absmax.astype(np.float32)


def nf4_dequantize(packed: np.ndarray, absmax: np.ndarray, N: int, K: int) -> np.ndarray:
    """(packed [N, K/2] u8, absmax [N, K/64] f32) -> float32 [N, K].

    Each weight is codebook[code] * absmax, one fp32 product (the reference
    decode, grouped-nf4-gemm PKG-INFO "Try it on CPU right now" block 1).
    """
    packed = np.asarray(packed, dtype=np.uint8).reshape(N, K // 2)
    absmax = np.asarray(absmax, dtype=np.float32).reshape(N, K // NF4_BLOCK)
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = packed >> 4
    codes[:, 1::2] = packed & 0xF
    vals = nf4_codebook()[codes]                                   # float32
    scale = np.repeat(absmax, NF4_BLOCK, axis=1)                   # float32
    return (vals * scale).astype(np.float32)                       # fp32 multiply (RNE)


# --------------------------------------------------------------------------
# MXFP4 quantize / dequantize
# --------------------------------------------------------------------------
def mxfp4_quantize(w: np.ndarray):
    """fp32 [N, K] -> (codes uint8 [N, K/2], e8m0 scales uint8 [N, K/32]).

    grouped-nf4-gemm PKG-INFO, "Try it on CPU right now", block 2 and "The
    MXFP4 native-byte lane": OCP e2m1 codes with one e8m0 scale per 32 K
    elements. Scale rule (OCP MX v1.0): X = floor(log2(amax)) - emax(e2m1)=2,
    clamped to [-127, 127], stored X + 127; element = nearest e2m1 value of
    w / 2^X, ties to the even code, saturating at +-6.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % MXFP4_BLOCK:
        raise ValueError("K must be a multiple of 32")
    mags = e2m1_values()[:8].astype(np.float64)
    codes = np.empty((N, K), dtype=np.uint8)
    X_all = np.empty((N, K // MXFP4_BLOCK), dtype=np.int64)
    step = max(1, (1 << 16) // K)                             # bound the temporaries
    for r0 in range(0, N, step):
        blocks = w[r0:r0 + step].reshape(-1, K // MXFP4_BLOCK, MXFP4_BLOCK).astype(np.float64)
        amax = np.abs(blocks).max(axis=2)
        X = np.full(amax.shape, -127, dtype=np.int64)
        nz = amax > 0
        _, e = np.frexp(amax[nz])            # amax = m * 2^e, m in [0.5, 1)
        X[nz] = (e.astype(np.int64) - 1) - 2
        X = np.clip(X, -127, 127)
        v = np.ldexp(blocks, -X[..., None])  # exact power-of-two scaling
        av = np.abs(v)
        d = np.abs(av[..., None] - mags)
        best = d.min(axis=-1, keepdims=True)
        cand = d == best
        # among the (at most two) nearest magnitudes take the even code
        even = cand & (np.arange(8) % 2 == 0)
        mag_code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
        mag_code = np.where(av >= 6.0, 7, mag_code)             # saturate
        c = (mag_code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)
        codes[r0:r0 + step] = c.reshape(-1, K)
        X_all[r0:r0 + step] = X
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    X = X_all
    return packed, (X + 127).astype(np.uint8)


def mxfp4_dequantize(packed: np.ndarray, scales: np.ndarray, N: int, K: int) -> np.ndarray:
    """(codes [N, K/2] u8, e8m0 [N, K/32] u8) -> float32 [N, K].

    Element = e2m1(code) * 2^(e8m0 - 127), exact in fp32; e8m0 = 255 is NaN.
    """
    packed = np.asarray(packed, dtype=np.uint8).reshape(N, K // 2)
    scales = np.asarray(scales, dtype=np.uint8).reshape(N, K // MXFP4_BLOCK)
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    vals = e2m1_values()[codes].astype(np.float64).reshape(N, K // MXFP4_BLOCK, MXFP4_BLOCK)
    ex = scales.astype(np.int64)
    mult = np.ldexp(1.0, ex - 127)                 # the block's power of two, exact in fp64
    mult[ex == 255] = np.nan
    out = vals * mult[..., None]                   # exact: a 2-bit significand times 2^X
    return out.reshape(N, K).astype(np.float32)


def quantize(fmt: int, w: np.ndarray):
    if fmt == FMT_MXFP4:
        return mxfp4_quantize(w)
    return nf4_quantize(w, absmax_bf16=(fmt == FMT_NF4_BF16ABS))


def dequantize(fmt: int, packed, scale, N: int, K: int) -> np.ndarray:
    if fmt == FMT_NF4:
        return nf4_dequantize(packed, scale, N, K)
    if fmt == FMT_NF4_BF16ABS:   # widen the bf16 absmax to fp32, then the NF4 decode
        bits = np.asarray(scale, dtype=np.uint16).astype(np.uint32) << 16
        return nf4_dequantize(packed, bits.view(np.float32), N, K)
    return mxfp4_dequantize(packed, scale, N, K)


# --------------------------------------------------------------------------
# Router
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def router_logits(x_bits: np.ndarray, router_w: np.ndarray, router_b=None) -> np.ndarray:
    """L[t, e] = sum_h x[t, h] * W_r[e, h] (+ b[e]) in fp64.

    The router stays outside the kernel on the pages (page "How do I run a
    grouped GEMM ...", section "Why it happens": sorting tokens by expert and
    scattering back are outside the kernel); this library moves it in. Config
    text: softmax, then top-k, renormalised.
    """
    x = bf16_bits_to_f64(x_bits)
    L = x @ np.asarray(router_w, dtype=np.float64).T
    if router_b is not None:
        L = L + np.asarray(router_b, dtype=np.float64)[None, :]
    return L


def topk_route(logits: np.ndarray, top_k: int, renormalize: bool = True):
    """Per token: the k experts with the largest logits (ties -> lower id).

    Returns (topk_ids int32 [T, k] in selection order, topk_w float64 [T, k]).
    renormalize: w_j = exp(L_j - L_0) / sum_{j'<k} exp(L_j' - L_0), i.e. the
    softmax over all experts divided by the sum over the selected ones.
    Otherwise w_j = softmax over all E at the selected ids.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not 1 <= top_k <= E:
        raise ValueError("need 1 <= top_k <= E")
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-L[t, e], e))[:top_k]
        ids[t] = order
        sel = L[t, order]
        m = L[t].max()
        if renormalize:
            ex = np.exp(sel - sel[0])
            w[t] = ex / ex.sum()
        else:
            full = np.exp(L[t] - m)
            w[t] = full[order] / full.sum()
    return ids, w


def permute(topk_ids: np.ndarray, E: int):
    """Stable counting sort of slots s = t*k + j by expert.

    Returns (expert_offsets int32 [E+1], sorted_slots int32 [T*k]); rows of
    expert e are sorted_slots[off[e]:off[e+1]], ascending in s. This is the
    pages' "a_cat [T, K] sorted by expert, sizes + expert_ids" grouping (page
    "How do I run a grouped GEMM ...", "Why it happens" dataflow), with every
    expert listed and empty groups allowed.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    cursor = offsets[:-1].copy()
    sorted_slots = np.empty(flat.size, dtype=np.int32)
    for s, e in enumerate(flat):       # ascending s: stable by construction
        sorted_slots[cursor[e]] = s
        cursor[e] += 1
    return offsets.astype(np.int32), sorted_slots


# --------------------------------------------------------------------------
# Grouped GEMM, SwiGLU, combine
# --------------------------------------------------------------------------
def grouped_gemm(a: np.ndarray, a_row_of, fmt: int, B_packed, B_scale, N: int, K: int,
                 group_offsets, group_experts=None) -> np.ndarray:
    """c[r, :] = a[a_row_of[r]] . W[e(r)]^T in fp64, W = decoded weights.

    The pages' gemm_4bit_grouped(a_cat, B, absmax, sizes, expert_ids) (page
    "How do I run a grouped GEMM ...", sections "Smallest correct example"
    and "Supported scope"): group g covers rows [off[g], off[g+1]) and uses
    expert group_experts[g] (identity when None); output in group order.
    a: float64 [rows_a, K]; a_row_of: int [R] or None (row r reads a[r]).
    """
    off = np.asarray(group_offsets, dtype=np.int64)
    G = off.size - 1
    gexp = np.arange(G) if group_experts is None else np.asarray(group_experts, dtype=np.int64)
    R = int(off[-1])
    rows = np.arange(R) if a_row_of is None else np.asarray(a_row_of, dtype=np.int64)
    c = np.zeros((R, N), dtype=np.float64)
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        e = int(gexp[g])
        W = dequantize(fmt, B_packed[e], B_scale[e], N, K).astype(np.float64)
        c[r0:r1] = a[rows[r0:r1]] @ W.T
    return c


def grouped_dgrad(dc: np.ndarray, fmt: int, B_packed, B_scale, N: int, K: int,
                  group_offsets, group_experts=None) -> np.ndarray:
    """da[r, :] = dc[r] . W[e(r)] in fp64: the input gradient of the grouped GEMM.

    The pages' dgrad_4bit_grouped (page "grouped-nf4-gemm ...", section
    "Training: the backward is a kernel too"): grad_out @ dequant(B) per
    expert, decoding each weight exactly as the forward does. With the forward
    c = a . W^T, dL/da = dL/dc . W, W the decoded [N, K] weights of the group's
    expert. dc: float64 [R, N] in group order; output [R, K] in the same order.
    """
    off = np.asarray(group_offsets, dtype=np.int64)
    G = off.size - 1
    gexp = np.arange(G) if group_experts is None else np.asarray(group_experts, dtype=np.int64)
    R = int(off[-1])
    da = np.zeros((R, K), dtype=np.float64)
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        e = int(gexp[g])
        W = dequantize(fmt, B_packed[e], B_scale[e], N, K).astype(np.float64)
        da[r0:r1] = dc[r0:r1] @ W
    return da


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u with silu(g) = g / (1 + exp(-g)) (the configs' SwiGLU)."""
    return g / (1.0 + np.exp(-g)) * u


def clamped_glu(g: np.ndarray, u: np.ndarray, alpha: float, limit: float) -> np.ndarray:
    """The clamped GLU epilogue of the gpt-oss expert form (a reading: the
    experts4bit-qlora page, "Scope", names it without defining it):
    g' = min(g, limit), u' = clamp(u, -limit, limit),
    h = (u' + 1) * g' * sigmoid(alpha * g')."""
    g = np.minimum(g, limit)
    u = np.clip(u, -limit, limit)
    return (u + 1.0) * (g / (1.0 + np.exp(-alpha * g)))


def moe_forward(layer: dict, x_bits: np.ndarray, topk_ids_override=None, return_all=False):
    """One routed MoE layer on 4-bit weights, fp64, unrounded output [T, H].

    layer: fmt, E, H, I, top_k, renormalize, w13 [E, 2I, H/2] u8, w13_scale,
    w2 [E, H, I/2] u8, w2_scale, router_w [E, H] f32, router_b [E] or None;
    optional: glu (GLU_SWIGLU / GLU_CLAMPED), glu_alpha, glu_limit,
    glu_interleaved, b13 [E, 2I] f32, b2 [E, H] f32 (the gpt-oss expert form).
    Steps (page "How do I run a grouped GEMM ...", "Why it happens" dataflow,
    and grouped-nf4-gemm PKG-INFO "The NVMe tier": gate -> GLU -> down):
    router logits, top-k + softmax, grouping, gate_up, SwiGLU, down, weighted
    combine. topk_ids_override replaces the selection (weights are recomputed
    from the oracle's logits for the given ids, in the given order).
    """
    fmt, E, H, I, k = layer["fmt"], layer["E"], layer["H"], layer["I"], layer["top_k"]
    renorm = bool(layer.get("renormalize", 1))
    x = bf16_bits_to_f64(x_bits)
    T = x.shape[0]
    L = router_logits(x_bits, layer["router_w"], layer.get("router_b"))
    if topk_ids_override is None:
        ids, w = topk_route(L, k, renorm)
    else:
        ids = np.asarray(topk_ids_override, dtype=np.int32).reshape(T, k)
        w = np.empty((T, k))
        for t in range(T):
            sel = L[t, ids[t]]
            if renorm:
                ex = np.exp(sel - sel[0])
                w[t] = ex / ex.sum()
            else:
                full = np.exp(L[t] - L[t].max())
                w[t] = full[ids[t]] / full.sum()
    off, slots = permute(ids, E)
    tok = slots // k
    expert_of_row = np.repeat(np.arange(E), np.diff(off))    # expert of each sorted row
    gu = grouped_gemm(x, tok, fmt, layer["w13"], layer["w13_scale"], 2 * I, H, off)
    if layer.get("b13") is not None:
        gu = gu + np.asarray(layer["b13"], np.float64)[expert_of_row]
    if layer.get("glu_interleaved", 0):
        g, u = gu[:, 0::2], gu[:, 1::2]
    else:
        g, u = gu[:, :I], gu[:, I:]
    if layer.get("glu", GLU_SWIGLU) == GLU_CLAMPED:
        h = clamped_glu(g, u, float(layer["glu_alpha"]), float(layer["glu_limit"]))
    else:
        h = swiglu(g, u)
    y = grouped_gemm(h, None, fmt, layer["w2"], layer["w2_scale"], H, I, off)
    if layer.get("b2") is not None:
        y = y + np.asarray(layer["b2"], np.float64)[expert_of_row]
    y_slot = np.empty_like(y)
    y_slot[slots] = y                                  # back to slot order s = t*k + j
    out = np.zeros((T, H))
    for j in range(k):                                 # slot-order sum
        out += w[:, j:j + 1] * y_slot[j::k]
    if return_all:
        return out, dict(logits=L, topk_ids=ids, topk_w=w, expert_offsets=off,
                         sorted_slots=slots, h=h, y_slot=y_slot)
    return out


def rel_err(a, b) -> float:
    return float(np.linalg.norm(np.asarray(a, np.float64) - np.asarray(b, np.float64))
                 / np.linalg.norm(np.asarray(b, np.float64)))


