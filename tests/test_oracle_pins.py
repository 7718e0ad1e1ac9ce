"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each pin is computed by code other than the oracle's own (exact rationals,
pure-Python loops, bit-field definitions, an independent normal CDF) or is a
value the pages print (tests/golden/printed_examples.json, cited there).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import moe_synth as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_examples.json")))


# ----------------------------------------------------------------- codebooks
def test_nf4_codebook_invariants():
    c = O.nf4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert np.all(np.diff(c) > 0)
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8


def _phi(z):  # standard normal CDF from math.erfc (independent of scipy's ndtri)
    return 0.5 * math.erfc(-z / math.sqrt(2.0))


def _phi_inv(p):  # bisection on _phi
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_nf4_codebook_is_normal_quantiles():
    """Each |c| times the largest quantile sits at its NormalFloat level."""
    c = O.nf4_codebook().astype(np.float64)
    delta = 1 - 0.5 * (1 / 30 + 1 / 32)
    zmax = _phi_inv(delta)
    pos_levels = [delta - i * (delta - 0.5) / 8 for i in range(8)]      # 8 levels, descending
    neg_levels = [delta - i * (delta - 0.5) / 7 for i in range(7)]      # 7 levels, descending
    for i, p in enumerate(pos_levels):
        assert abs(_phi(c[15 - i] * zmax) - p) < 2e-7
    for i, p in enumerate(neg_levels):
        assert abs(_phi(-c[i] * zmax) - p) < 2e-7


def test_e2m1_table_from_bit_fields():
    v = O.e2m1_values()
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert v[code] == (-mag if s else mag)


# ----------------------------------------------------------------- NF4
def test_nf4_printed_roundtrip():
    g = GOLD["nf4_roundtrip"]
    for seed in range(3):
        w = np.random.default_rng(seed).standard_normal(g["w_shape"], dtype=np.float32)
        packed, absmax = O.nf4_quantize(w)
        assert list(packed.shape) == g["packed_shape"] and packed.dtype == np.uint8
        assert list(absmax.shape) == g["absmax_shape"] and absmax.dtype == np.float32
        wq = O.nf4_dequantize(packed, absmax, *g["w_shape"])
        err = O.rel_err(wq, w)
        assert round(err, 2) == g["rel_err_printed"]
        p2, a2 = O.nf4_quantize(wq)
        assert np.array_equal(p2, packed) == g["repack_idempotent"]
        assert np.array_equal(a2, absmax)


def _nearest_exact(w, a, table, tie="lower"):
    """Index of the nearest table[i]*a to w in exact rationals."""
    W, A = Fraction(float(w)), Fraction(float(a))
    d = [abs(W - Fraction(float(t)) * A) for t in table]
    best = min(d)
    cands = [i for i, x in enumerate(d) if x == best]
    if tie == "lower":
        return cands[0]
    return [i for i in cands if i % 2 == 0][0] if len(cands) > 1 else cands[0]


def test_nf4_codes_are_exact_nearest_with_ties_low():
    c = O.nf4_codebook()
    rng = np.random.default_rng(7)
    w = rng.standard_normal((3, 128)).astype(np.float32) * np.float32(0.02)
    # plant exact ties between codes 6|7 and 7|8: c[6]/2 and c[8]/2 are fp32
    w[0, 0] = 1.0
    w[0, 1] = np.float32(c[8] / 2)
    w[0, 2] = np.float32(c[6] / 2)
    w[0, 3] = -0.0
    for i in range(14):                 # other exactly representable midpoints
        m = (np.float64(c[i]) + np.float64(c[i + 1])) / 2
        if np.float64(np.float32(m)) == m:
            w[1, 64 + i] = np.float32(m)
    w[1, 64 + 15] = 1.0
    packed, absmax = O.nf4_quantize(w)
    codes = np.empty(w.shape, np.uint8)
    codes[:, 0::2], codes[:, 1::2] = packed >> 4, packed & 15
    for r in range(w.shape[0]):
        for k in range(w.shape[1]):
            a = absmax[r, k // 64]
            assert codes[r, k] == _nearest_exact(w[r, k], a, c), (r, k)
    assert codes[0, 1] == 7 and codes[0, 2] == 6


def test_nf4_absmax_error_bound_zero_block_nibble_order():
    c = O.nf4_codebook().astype(np.float64)
    rng = np.random.default_rng(3)
    w = rng.standard_normal((4, 256)).astype(np.float32)
    w[2, 64:128] = 0.0                                   # all-zero block
    w[3, 0], w[3, 1] = 5.0, -5.0                         # nibble order probe
    packed, absmax = O.nf4_quantize(w)
    wq = O.nf4_dequantize(packed, absmax, 4, 256)
    blk = np.abs(wq).reshape(4, 4, 64).max(axis=2)
    assert np.array_equal(blk.astype(np.float32), absmax)          # absmax survives exactly
    half_gap = np.max(np.diff(c)) / 2
    bound = np.repeat(absmax.astype(np.float64), 64, axis=1) * (half_gap + 2 ** -23)
    assert np.all(np.abs(wq.astype(np.float64) - w) <= bound)
    assert absmax[2, 1] == 0 and np.all(packed[2, 32:64] == 0x77) and np.all(wq[2, 64:128] == 0)
    assert packed[3, 0] == 0xF0                            # high nibble = even k


def test_nf4_absmax_share_printed():
    g = GOLD["nf4_absmax_share"]
    # one Qwen3-30B-A3B-shaped expert (gate + up + down = 3 * I * H weights,
    # I = 768, H = 2048) packed as NF4 with fp32 absmax per 64
    elems = 3 * 768 * 2048
    codes, absmax = elems // 2, (elems // 64) * 4
    assert absmax == g["absmax_bytes"] and codes + absmax == g["row_bytes"]


# ----------------------------------------------------------------- MXFP4
def test_mxfp4_printed_roundtrip():
    g = GOLD["mxfp4_roundtrip"]
    for seed in range(3):
        w = np.random.default_rng(seed).standard_normal(g["w_shape"], dtype=np.float32)
        codes, scales = O.mxfp4_quantize(w)
        assert list(codes.reshape(w.shape[0], -1, 16).shape) == g["blocks_shape"]
        assert list(scales.shape) == g["scales_shape"]
        wq = O.mxfp4_dequantize(codes, scales, *g["w_shape"])
        assert round(O.rel_err(wq, w), 2) in (0.11, g["rel_err_printed"])
        c2, s2 = O.mxfp4_quantize(wq)
        assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_mxfp4_exact_nearest_ties_even_saturation():
    mags = O.e2m1_values()[:8]
    rng = np.random.default_rng(11)
    w = rng.standard_normal((2, 64)).astype(np.float32)
    # block 0: amax 7 -> X = floor(log2 7) - 2 = 0; plant ties and saturation
    w[0, :32] = np.float32(0.1)
    w[0, 0] = 7.0                                          # 6 < v < 8: saturates to 6
    for i, t in enumerate([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -2.5, -0.25]):
        w[0, 1 + i] = t
    codes, scales = O.mxfp4_quantize(w)
    full = np.empty(w.shape, np.uint8)
    full[:, 0::2], full[:, 1::2] = codes & 15, codes >> 4
    for r in range(2):
        for b in range(2):
            blk = w[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            X = max(-127, min(127, math.floor(math.log2(amax)) - 2))
            assert scales[r, b] == X + 127
            assert 4 <= amax / 2.0 ** X < 8
            for i, v in enumerate(blk):
                q = Fraction(float(v)) / Fraction(2) ** X
                if abs(q) >= 6:
                    mag = 7
                else:
                    d = [abs(abs(q) - Fraction(float(m))) for m in mags]
                    best = min(d)
                    cands = [j for j, x in enumerate(d) if x == best]
                    mag = cands[0] if len(cands) == 1 else [j for j in cands if j % 2 == 0][0]
                expect = mag | (8 if math.copysign(1.0, v) < 0 else 0)
                assert full[r, 32 * b + i] == expect, (r, b, i, v)
    assert full[0, 0] == 7
    assert [full[0, 1 + i] & 7 for i in range(7)] == [0, 2, 2, 4, 4, 6, 6]
    assert codes[0, 0] & 15 == 7                            # low nibble = even k


def test_mxfp4_zero_block_and_nan_scale():
    w = np.zeros((1, 64), np.float32)
    w[0, 40] = 1.0
    codes, scales = O.mxfp4_quantize(w)
    assert scales[0, 0] == 0 and np.all(codes[0, :16] == 0)
    out = O.mxfp4_dequantize(codes, scales, 1, 64)
    assert np.all(out[0, :32] == 0) and out[0, 40] == 1.0
    s2 = scales.copy(); s2[0, 1] = 255
    assert np.all(np.isnan(O.mxfp4_dequantize(codes, s2, 1, 64)[0, 32:]))


# ----------------------------------------------------------------- routing
def _bf16(x):
    return S.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_router_logits_bruteforce():
    rng = np.random.default_rng(5)
    xb = _bf16(rng.standard_normal((3, 8)))
    W = rng.standard_normal((4, 8)).astype(np.float32)
    b = rng.standard_normal(4).astype(np.float32)
    L = O.router_logits(xb, W, b)
    for t in range(3):
        xs = [float(np.array([int(v) << 16], np.uint32).view(np.float32)[0]) for v in xb[t]]
        for e in range(4):
            ref = math.fsum(xs[h] * float(W[e, h]) for h in range(8)) + float(b[e])
            assert abs(L[t, e] - ref) <= 1e-12 * (1 + abs(ref))


def test_topk_bruteforce_ties_and_weights():
    rng = np.random.default_rng(9)
    L = rng.standard_normal((20, 6))
    L[0] = [1.0, 3.0, 3.0, 0.5, 3.0, -1.0]                # ties -> lower id first
    for k in (1, 2, 3, 6):
        ids, w = O.topk_route(L, k, True)
        for t in range(20):
            order = sorted(range(6), key=lambda e: (-L[t, e], e))[:k]
            assert list(ids[t]) == order
            ex = [math.exp(L[t, e]) for e in order]
            ref = [v / math.fsum(ex) for v in ex]
            assert np.allclose(w[t], ref, rtol=1e-13, atol=0)
            assert abs(w[t].sum() - 1.0) < 1e-12
        if k == 1:
            assert np.all(w == 1.0)
        if k == 6:                                           # top_k = E: the full softmax
            full = np.exp(L - L.max(1, keepdims=True)); full /= full.sum(1, keepdims=True)
            assert np.allclose(np.take_along_axis(full, ids.astype(np.int64), 1), w, rtol=1e-13)
    assert list(O.topk_route(L, 3, True)[0][0]) == [1, 2, 4]
    ids, w = O.topk_route(L, 2, False)
    full = np.exp(L) / np.exp(L).sum(1, keepdims=True)
    assert np.allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-12)


def test_permute_bruteforce_stable():
    rng = np.random.default_rng(2)
    for E, T, k in ((5, 7, 2), (8, 1, 8), (3, 10, 1), (16, 9, 4)):
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        off, slots = O.permute(ids, E)
        flat = ids.reshape(-1)
        ref = sorted(range(T * k), key=lambda s: (flat[s], s))
        assert list(slots) == ref
        for e in range(E):
            assert off[e + 1] - off[e] == int((flat == e).sum())
        assert off[0] == 0 and off[E] == T * k


# ----------------------------------------------------------------- GEMM / forward
def _deq_py(fmt, packed, scale, N, K):
    """Pure-Python decode (bit fields + tables), independent of the oracle's."""
    tab = O.nf4_codebook() if fmt == O.FMT_NF4 else O.e2m1_values()
    out = [[0.0] * K for _ in range(N)]
    for n in range(N):
        for k in range(K):
            byte = int(packed[n, k // 2])
            if fmt == O.FMT_NF4:
                code = (byte >> 4) if k % 2 == 0 else (byte & 15)
                out[n][k] = float(np.float32(tab[code]) * np.float32(scale[n, k // 64]))
            else:
                code = (byte & 15) if k % 2 == 0 else (byte >> 4)
                out[n][k] = float(tab[code]) * 2.0 ** (int(scale[n, k // 32]) - 127)
    return out


@pytest.mark.parametrize("fmt", [O.FMT_NF4, O.FMT_MXFP4])
def test_grouped_gemm_triple_loop(fmt):
    rng = np.random.default_rng(4)
    E, N, K = 3, 5, 128
    Wf = rng.standard_normal((E, N, K)).astype(np.float32) * np.float32(0.02)
    qs = [O.quantize(fmt, Wf[e]) for e in range(E)]
    Bp = np.stack([q[0] for q in qs]); Bs = np.stack([q[1] for q in qs])
    a = rng.standard_normal((6, K))
    row_of = np.array([5, 0, 2, 2, 1])
    off, gexp = [0, 2, 2, 5], [2, 0, 1]
    c = O.grouped_gemm(a, row_of, fmt, Bp, Bs, N, K, off, gexp)
    Wd = [_deq_py(fmt, Bp[e], Bs[e], N, K) for e in range(E)]
    for g in range(3):
        for r in range(off[g], off[g + 1]):
            for n in range(N):
                ref = math.fsum(a[row_of[r], kk] * Wd[gexp[g]][n][kk] for kk in range(K))
                assert abs(c[r, n] - ref) <= 1e-12 * (1 + abs(ref))


@pytest.mark.parametrize("fmt", [O.FMT_NF4, O.FMT_MXFP4])
def test_grouped_dgrad_triple_loop(fmt):
    """dgrad (page "grouped-nf4-gemm ...", "Training: the backward is a kernel
    too": grad_out @ dequant(B)) against explicit sums over n of the
    pure-Python decode, groups with an empty one in the middle."""
    rng = np.random.default_rng(14)
    E, N, K = 3, 7, 128
    Wf = rng.standard_normal((E, N, K)).astype(np.float32) * np.float32(0.02)
    qs = [O.quantize(fmt, Wf[e]) for e in range(E)]
    Bp = np.stack([q[0] for q in qs]); Bs = np.stack([q[1] for q in qs])
    off, gexp = [0, 2, 2, 5], [2, 0, 1]
    dc = rng.standard_normal((5, N))
    da = O.grouped_dgrad(dc, fmt, Bp, Bs, N, K, off, gexp)
    Wd = [_deq_py(fmt, Bp[e], Bs[e], N, K) for e in range(E)]
    for g in range(3):
        for r in range(off[g], off[g + 1]):
            for kk in range(K):
                ref = math.fsum(dc[r, n] * Wd[gexp[g]][n][kk] for n in range(N))
                assert abs(da[r, kk] - ref) <= 1e-12 * (1 + abs(ref))


def test_grouped_dgrad_is_the_adjoint_of_the_forward():
    """<dc, a W^T> = <a, dc W> per group: the backward is the forward's adjoint
    (a transposed or misindexed W in either would break the identity)."""
    rng = np.random.default_rng(15)
    E, N, K = 2, 96, 192
    Wf = rng.standard_normal((E, N, K)).astype(np.float32) * np.float32(0.05)
    qs = [O.nf4_quantize(Wf[e]) for e in range(E)]
    Bp = np.stack([q[0] for q in qs]); Bs = np.stack([q[1] for q in qs])
    off, gexp = [0, 3, 7], [1, 0]
    a = rng.standard_normal((7, K))
    dc = rng.standard_normal((7, N))
    c = O.grouped_gemm(a, None, O.FMT_NF4, Bp, Bs, N, K, off, gexp)
    da = O.grouped_dgrad(dc, O.FMT_NF4, Bp, Bs, N, K, off, gexp)
    lhs, rhs = math.fsum((dc * c).ravel()), math.fsum((a * da).ravel())
    assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs))
    # and a unit gradient row picks one decoded weight row
    e1 = np.zeros((1, N)); e1[0, 11] = 1.0
    row = O.grouped_dgrad(e1, O.FMT_NF4, Bp, Bs, N, K, [0, 1], [1])
    assert np.array_equal(row[0], O.nf4_dequantize(Bp[1], Bs[1], N, K)[11].astype(np.float64))


def test_unit_vector_picks_column():
    rng = np.random.default_rng(8)
    Wf = rng.standard_normal((1, 6, 64)).astype(np.float32)
    p, s = O.nf4_quantize(Wf[0])
    a = np.zeros((1, 64)); a[0, 17] = 1.0
    c = O.grouped_gemm(a, None, O.FMT_NF4, p[None], s[None], 6, 64, [0, 1])
    assert np.array_equal(c[0], O.nf4_dequantize(p, s, 6, 64)[:, 17].astype(np.float64))


def test_swiglu_closed_forms():
    g = np.array([0.0, 1.0, -2.0, 30.0]); u = np.array([3.0, 0.0, 1.0, 2.0])
    h = O.swiglu(g, u)
    assert h[0] == 0.0 and h[1] == 0.0
    assert abs(h[2] - (-2.0 / (1 + math.exp(2.0)))) < 1e-15
    assert abs(h[3] - 60.0) < 1e-9


def _forward_py(layer, xb, forced=None):
    """Pure-Python forward on tiny shapes: loops, math.exp, no numpy algebra.
    forced: optional [T, k] expert ids used in place of the top-k selection;
    the routing weights are then the softmax over those ids' logits
    (renormalize = 1) or the full softmax at those ids (renormalize = 0)."""
    fmt, E, H, I, k = layer["fmt"], layer["E"], layer["H"], layer["I"], layer["top_k"]
    renorm = bool(layer.get("renormalize", 1))
    W13 = [_deq_py(fmt, layer["w13"][e], layer["w13_scale"][e], 2 * I, H) for e in range(E)]
    W2 = [_deq_py(fmt, layer["w2"][e], layer["w2_scale"][e], H, I) for e in range(E)]
    out = []
    for t in range(xb.shape[0]):
        x = [float(np.array([int(v) << 16], np.uint32).view(np.float32)[0]) for v in xb[t]]
        L = [math.fsum(x[h] * float(layer["router_w"][e, h]) for h in range(H)) for e in range(E)]
        if forced is None:
            order = sorted(range(E), key=lambda e: (-L[e], e))[:k]
        else:
            order = [int(e) for e in forced[t]]
        if renorm:
            ex = [math.exp(L[e]) for e in order]
            ws = [v / math.fsum(ex) for v in ex]
        else:
            den = math.fsum(math.exp(L[e]) for e in range(E))
            ws = [math.exp(L[e]) / den for e in order]
        o = [0.0] * H
        for wj, e in zip(ws, order):
            gu = [math.fsum(x[h] * W13[e][n][h] for h in range(H)) for n in range(2 * I)]
            hh = [gu[i] / (1 + math.exp(-gu[i])) * gu[I + i] for i in range(I)]
            for n in range(H):
                o[n] += wj * math.fsum(hh[i] * W2[e][n][i] for i in range(I))
        out.append(o)
    return np.array(out)


@pytest.mark.parametrize("fmt", [O.FMT_NF4, O.FMT_MXFP4])
def test_moe_forward_bruteforce(fmt):
    wl = S.custom(E=4, top_k=2, H=64, I=64, fmt=fmt)
    W_r, _ = S.make_router(wl)
    layer = dict(fmt=fmt, E=4, H=64, I=64, top_k=2, renormalize=1, router_w=W_r, router_b=None)
    w13 = S.make_stack(wl, 0, "w13"); w2 = S.make_stack(wl, 0, "w2")
    q13 = [O.quantize(fmt, w13[e]) for e in range(4)]
    q2 = [O.quantize(fmt, w2[e]) for e in range(4)]
    layer["w13"] = np.stack([q[0] for q in q13]); layer["w13_scale"] = np.stack([q[1] for q in q13])
    layer["w2"] = np.stack([q[0] for q in q2]); layer["w2_scale"] = np.stack([q[1] for q in q2])
    xb = S.make_x(wl, 3)
    out = O.moe_forward(layer, xb)
    ref = _forward_py(layer, xb)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-14)


def _tiny_layer(fmt, E, k, renorm, wid):
    wl = S.custom(E=E, top_k=k, H=64, I=64, fmt=fmt, wid=wid, renormalize=renorm)
    W_r, _ = S.make_router(wl)
    w13 = S.make_stack(wl, 0, "w13"); w2 = S.make_stack(wl, 0, "w2")
    q13 = [O.quantize(fmt, w13[e]) for e in range(E)]
    q2 = [O.quantize(fmt, w2[e]) for e in range(E)]
    layer = dict(fmt=fmt, E=E, H=64, I=64, top_k=k, renormalize=renorm, router_w=W_r, router_b=None,
                 w13=np.stack([q[0] for q in q13]), w13_scale=np.stack([q[1] for q in q13]),
                 w2=np.stack([q[0] for q in q2]), w2_scale=np.stack([q[1] for q in q2]))
    return wl, layer


# The forward with given expert ids (topk_ids_override) is how every GPU parity
# test and the smoke check call the oracle: the GPU's fp32 selection is handed
# in, and the oracle recomputes the routing weights from its own fp64 logits.
@pytest.mark.parametrize("renorm", [1, 0])
def test_override_with_own_selection_is_the_default_path(renorm):
    """Handing the oracle its own top-k ids reproduces the default forward bit
    for bit (catches an override branch whose weights use another formula or
    normaliser than the default selection's, e.g. a renormalised softmax when
    renormalize = 0)."""
    wl, layer = _tiny_layer(O.FMT_NF4, 6, 3, renorm, wid=81)
    xb = S.make_x(wl, 5)
    out, inner = O.moe_forward(layer, xb, return_all=True)
    out2, inner2 = O.moe_forward(layer, xb, topk_ids_override=inner["topk_ids"], return_all=True)
    assert np.array_equal(out, out2)
    assert np.array_equal(inner["topk_w"], inner2["topk_w"])


@pytest.mark.parametrize("renorm", [1, 0])
def test_override_order_within_a_token_does_not_matter(renorm):
    """The layer output is a weighted sum over the selected set: listing the
    same ids in another order gives the same output (catches weights that stay
    attached to a slot position instead of to their expert, e.g. a weight
    vector not permuted with the ids)."""
    wl, layer = _tiny_layer(O.FMT_MXFP4, 6, 3, renorm, wid=82)
    xb = S.make_x(wl, 4)
    _, inner = O.moe_forward(layer, xb, return_all=True)
    ids = inner["topk_ids"]
    rev = np.ascontiguousarray(ids[:, ::-1])
    rot = np.ascontiguousarray(np.roll(ids, 1, axis=1))
    a = O.moe_forward(layer, xb, topk_ids_override=ids)
    for other in (rev, rot):
        b = O.moe_forward(layer, xb, topk_ids_override=other)
        assert np.allclose(a, b, rtol=1e-13, atol=1e-15 * np.abs(a).max())


@pytest.mark.parametrize("fmt,renorm", [(O.FMT_NF4, 1), (O.FMT_MXFP4, 0)])
def test_override_forced_selection_matches_bruteforce(fmt, renorm):
    """A forced selection that is not the top-k (the lowest logits, and a
    mixed one, in non-descending order) against the pure-Python forward given
    the same ids (catches a wrong weight order, a wrong softmax base or sum, or
    weights taken from the wrong experts)."""
    E, k = 5, 2
    wl, layer = _tiny_layer(fmt, E, k, renorm, wid=83)
    xb = S.make_x(wl, 3)
    L = O.router_logits(xb, layer["router_w"])
    forced = np.empty((3, k), np.int32)
    for t in range(3):
        asc = sorted(range(E), key=lambda e: (L[t, e], e))
        forced[t] = [asc[0], asc[2]] if t != 1 else [asc[3], asc[0]]
    out = O.moe_forward(layer, xb, topk_ids_override=forced)
    ref = _forward_py(layer, xb, forced=forced)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-14)
    assert not np.allclose(out, O.moe_forward(layer, xb))        # the forcing took effect


def test_moe_forward_single_expert_k1_closed_form():
    """k = 1 with one expert: out = y (routing weight exactly 1)."""
    wl = S.custom(E=1, top_k=1, H=64, I=64)
    W_r, _ = S.make_router(wl)
    w13, w2 = S.make_stack(wl, 0, "w13")[0], S.make_stack(wl, 0, "w2")[0]
    p13, s13 = O.nf4_quantize(w13); p2, s2 = O.nf4_quantize(w2)
    layer = dict(fmt=0, E=1, H=64, I=64, top_k=1, renormalize=1, router_w=W_r, router_b=None,
                 w13=p13[None], w13_scale=s13[None], w2=p2[None], w2_scale=s2[None])
    xb = S.make_x(wl, 2)
    x = O.bf16_bits_to_f64(xb)
    W13 = O.nf4_dequantize(p13, s13, 128, 64).astype(np.float64)
    W2 = O.nf4_dequantize(p2, s2, 64, 64).astype(np.float64)
    gu = x @ W13.T
    h = gu[:, :64] / (1 + np.exp(-gu[:, :64])) * gu[:, 64:]
    assert np.allclose(O.moe_forward(layer, xb), h @ W2.T, rtol=1e-12, atol=0)


def test_gate_up_halves_matter():
    """Swapping the gate and up halves changes the output (gate = rows [0, I))."""
    wl = S.custom(E=2, top_k=1, H=64, I=64)
    W_r, _ = S.make_router(wl)
    w13, w2 = S.make_stack(wl, 0, "w13"), S.make_stack(wl, 0, "w2")
    def build(stack13):
        q13 = [O.nf4_quantize(stack13[e]) for e in range(2)]; q2 = [O.nf4_quantize(w2[e]) for e in range(2)]
        return dict(fmt=0, E=2, H=64, I=64, top_k=1, renormalize=1, router_w=W_r, router_b=None,
                    w13=np.stack([q[0] for q in q13]), w13_scale=np.stack([q[1] for q in q13]),
                    w2=np.stack([q[0] for q in q2]), w2_scale=np.stack([q[1] for q in q2]))
    xb = S.make_x(wl, 2)
    a = O.moe_forward(build(w13), xb)
    b = O.moe_forward(build(np.concatenate([w13[:, 64:], w13[:, :64]], axis=1)), xb)
    assert not np.allclose(a, b)


# ----------------------------------------------------------------------------
# The gpt-oss expert form (experts4bit-qlora page, "Scope": per-expert biases and
# a clamped-GLU epilogue; the formula is this library's reading, a parameterised
# clamp of the gate and up values around a GLU with sigmoid(alpha * g)).
def test_clamped_glu_special_values():
    a, lim = 1.702, 7.0
    g = np.array([0.0, 0.0, 2.0, -3.0, 7.0, 50.0, 50.0, 1.0, 1.0])
    u = np.array([5.0, -9.0, -1.0, -1.0, 0.5, 0.5, 100.0, 7.0, 1e9])
    h = O.clamped_glu(g, u, a, lim)
    assert h[0] == 0.0 and h[1] == 0.0          # g = 0
    assert h[2] == 0.0 and h[3] == 0.0          # u = -1 (the +1 offset)
    assert h[5] == h[4]                          # g clamps at the limit from above
    assert h[6] == O.clamped_glu(np.array([7.0]), np.array([7.0]), a, lim)[0]   # both clamp
    assert h[8] == h[7]                          # u clamps at the limit
    # negative gates are not clamped: a large negative gate gives ~0 (sigmoid -> 0)
    assert abs(O.clamped_glu(np.array([-60.0]), np.array([0.0]), a, lim)[0]) < 1e-40
    # alpha = 1 and a limit no value reaches: (u + 1) * silu(g), the SwiGLU with up + 1
    g2 = np.linspace(-5, 5, 11); u2 = np.linspace(-3, 4, 11)
    assert np.allclose(O.clamped_glu(g2, u2, 1.0, 1e300), O.swiglu(g2, u2 + 1.0), rtol=1e-15, atol=0)


def _gptoss_layer(fmt, E, H, I, k, interleaved, alpha=1.702, limit=1.0, zero_weights=False, seed=0):
    wl = S.custom(E=E, top_k=k, H=H, I=I, fmt=fmt, wid=40 + seed)
    W_r, _ = S.make_router(wl)
    w13, w2 = S.make_stack(wl, 0, "w13"), S.make_stack(wl, 0, "w2")
    b13, b2 = S.make_biases(wl)
    if zero_weights:
        w13, w2 = np.zeros_like(w13), np.zeros_like(w2)
    if interleaved:   # the same gate and up rows, stored as 2c / 2c + 1
        perm = np.empty(2 * I, np.int64); perm[0::2] = np.arange(I); perm[1::2] = I + np.arange(I)
        w13, b13 = w13[:, perm], b13[:, perm]
    q13 = [O.quantize(fmt, w13[e]) for e in range(E)]
    q2 = [O.quantize(fmt, w2[e]) for e in range(E)]
    return wl, dict(fmt=fmt, E=E, H=H, I=I, top_k=k, renormalize=1, router_w=W_r, router_b=None,
                    w13=np.stack([q[0] for q in q13]), w13_scale=np.stack([q[1] for q in q13]),
                    w2=np.stack([q[0] for q in q2]), w2_scale=np.stack([q[1] for q in q2]),
                    glu=O.GLU_CLAMPED, glu_alpha=alpha, glu_limit=limit, glu_interleaved=int(interleaved),
                    b13=b13, b2=b2)


def _gptoss_forward_py(layer, xb):
    """Pure-Python forward of the gpt-oss form: loops, math.exp, min/max."""
    fmt, E, H, I, k = layer["fmt"], layer["E"], layer["H"], layer["I"], layer["top_k"]
    a, lim, inter = layer["glu_alpha"], layer["glu_limit"], layer["glu_interleaved"]
    W13 = [_deq_py(fmt, layer["w13"][e], layer["w13_scale"][e], 2 * I, H) for e in range(E)]
    W2 = [_deq_py(fmt, layer["w2"][e], layer["w2_scale"][e], H, I) for e in range(E)]
    out = []
    for t in range(xb.shape[0]):
        x = [float(np.array([int(v) << 16], np.uint32).view(np.float32)[0]) for v in xb[t]]
        L = [math.fsum(x[h] * float(layer["router_w"][e, h]) for h in range(H)) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-L[e], e))[:k]
        ex = [math.exp(L[e] - L[order[0]]) for e in order]
        ws = [v / math.fsum(ex) for v in ex]
        o = [0.0] * H
        for wj, e in zip(ws, order):
            gu = [math.fsum(x[h] * W13[e][n][h] for h in range(H)) + float(layer["b13"][e][n])
                  for n in range(2 * I)]
            hh = []
            for i in range(I):
                g = gu[2 * i] if inter else gu[i]
                u = gu[2 * i + 1] if inter else gu[I + i]
                g = min(g, lim)
                u = max(-lim, min(u, lim))
                hh.append((u + 1.0) * g / (1.0 + math.exp(-a * g)))
            for n in range(H):
                o[n] += wj * (math.fsum(hh[i] * W2[e][n][i] for i in range(I)) + float(layer["b2"][e][n]))
        out.append(o)
    return np.array(out)


@pytest.mark.parametrize("fmt,interleaved", [(O.FMT_NF4, False), (O.FMT_MXFP4, True)])
def test_gptoss_form_bruteforce(fmt, interleaved):
    wl, layer = _gptoss_layer(fmt, 4, 64, 64, 2, interleaved, limit=0.5)
    xb = S.make_x(wl, 3)
    out, inner = O.moe_forward(layer, xb, return_all=True)
    assert np.allclose(out, _gptoss_forward_py(layer, xb), rtol=1e-10, atol=1e-14)
    assert np.mean(np.abs(inner["h"]) > 0) > 0.5     # the epilogue saw nonzero inputs


def test_gptoss_interleaved_is_a_row_permutation():
    """Interleaved storage of the same gate / up rows gives the same layer."""
    wl, a = _gptoss_layer(O.FMT_NF4, 4, 64, 128, 2, False, limit=0.7, seed=1)
    _, b = _gptoss_layer(O.FMT_NF4, 4, 64, 128, 2, True, limit=0.7, seed=1)
    xb = S.make_x(wl, 5)
    assert np.array_equal(O.moe_forward(a, xb), O.moe_forward(b, xb))


def test_gptoss_zero_weights_leave_the_biases():
    """With every weight 0: h = clamped_glu(b13 gate, b13 up) of the row's expert,
    and out[t] = sum_j w[t, j] * b2[e_j] exactly."""
    wl, layer = _gptoss_layer(O.FMT_NF4, 4, 64, 64, 2, False, limit=0.05, zero_weights=True, seed=2)
    xb = S.make_x(wl, 4)
    out, inner = O.moe_forward(layer, xb, return_all=True)
    ids, w = inner["topk_ids"], inner["topk_w"]
    b13, b2 = layer["b13"].astype(np.float64), layer["b2"].astype(np.float64)
    for s, r in enumerate(np.argsort(inner["sorted_slots"])):     # slot s sits at sorted row r
        e = ids[s // 2, s % 2]
        assert np.array_equal(inner["h"][r], O.clamped_glu(b13[e, :64], b13[e, 64:], 1.702, 0.05))
    ref = np.zeros((4, 64))
    for j in range(2):
        ref += w[:, j:j + 1] * b2[ids[:, j]]
    assert np.allclose(out, ref, rtol=1e-15, atol=0)


# ----------------------------------------------------------------------------
# NF4 with bf16 absmax (experts4bit-qlora page, the --absmax-dtype bf16 paragraph:
# 5.6 % off every row, lossless for bf16-source weights).
def _bf16_source(rng, shape):
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    return (w.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # bf16 values


def test_bf16_round_up_grid():
    """bf16_round_up: a bf16 value, >= a, and the next bf16 value below it is < a."""
    rng = np.random.default_rng(60)
    a = np.abs(rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 8, 2000)).astype(np.float32)
    r = O.bf16_round_up(a)
    bits = r.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0) and np.all(r >= a)
    below = ((bits >> 16) - 1).astype(np.uint32) << 16
    assert np.all(below.view(np.float32).astype(np.float64) < a)
    exact = (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    assert np.array_equal(O.bf16_round_up(exact), exact.astype(np.float64))   # a bf16 value stays


def test_bf16_absmax_is_lossless_for_bf16_source():
    """For bf16-source weights the bf16-absmax form has the fp32 form's codes,
    its absmax bit for bit, and the same decoded weights."""
    rng = np.random.default_rng(61)
    w = _bf16_source(rng, (24, 512))
    p0, s0 = O.nf4_quantize(w)
    p2, s2 = O.quantize(O.FMT_NF4_BF16ABS, w)
    assert np.array_equal(p0, p2)
    assert s2.dtype == np.uint16 and np.array_equal(s2.astype(np.uint32) << 16, s0.view(np.uint32))
    assert np.array_equal(O.dequantize(O.FMT_NF4_BF16ABS, p2, s2, 24, 512), O.nf4_dequantize(p0, s0, 24, 512))


def test_bf16_absmax_rounds_up_for_fp32_source():
    """fp32-source weights: the stored absmax is the bf16 round-up of max|w|, no
    weight leaves the codebook's range, and the NF4 error bound holds for it."""
    rng = np.random.default_rng(62)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    p2, s2 = O.quantize(O.FMT_NF4_BF16ABS, w)
    a = np.abs(w.reshape(16, 4, 64).astype(np.float64)).max(axis=2)
    a2 = (s2.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(a2, O.bf16_round_up(a))
    deq = O.dequantize(O.FMT_NF4_BF16ABS, p2, s2, 16, 256).astype(np.float64).reshape(16, 4, 64)
    gap = np.max(np.diff(O.nf4_codebook().astype(np.float64))) / 2
    err = np.abs(deq - w.reshape(16, 4, 64).astype(np.float64))
    assert np.all(err <= gap * a2[..., None] * (1 + 1e-6))


def test_bf16_absmax_share_printed():
    """The page: fp32 absmax is 294,912 of 2,654,208 B of a Qwen3-30B expert row
    set, and bf16 absmax takes 5.6 % off."""
    H, I = 2048, 768
    codes = 3 * H * I // 2
    fp32_abs, bf16_abs = 3 * H * I // 64 * 4, 3 * H * I // 64 * 2
    assert fp32_abs == 294_912 and codes + fp32_abs == 2_654_208
    assert round(100 * (fp32_abs - bf16_abs) / (codes + fp32_abs), 1) == 5.6
