"""Row-count invariance of the HIP path: a token's outputs (top-k ids, routing
weights, layer output) carry the same bits whether the token is decoded alone
or inside a larger call.

The pages hold this for their GEMV and row combine (page "MoE Software Status &
Known Limits", kernel section, the row-count invariance item: one token alone
and inside 16-, 17- and 160-token calls); their grouped GEMM differs from the
GEMV only in summation order. Here: on the small-M path every step has a fixed
per-token order (router logits one workgroup per expert, a fixed softmax
denominator order, GEMV rows independent of the batch, the fused token-centric
down + combine taking the same steps as the GEMV slot output + combine), so
the property holds for every T; on the MFMA path it holds among calls that use
the same router kernel (T <= 16: the per-token kernel; T > 16: the
matrix-core one, which sums a token's logit over fixed chunks of H in chunk
order), as an MFMA row's result does not depend on the rows sharing its tile.
A property of the path at any size: the test
compares the path with itself; the oracle bound is checked once per case.
"""
import numpy as np
import pytest

import moe_synth as S
import oracle as O
from gpu_helpers import bits_to_torch_bf16, build_layers, check_bound

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_expert_amd as M  # noqa: E402

DEV = "cuda"

# Cover every lane-segment shape of the small-M kernels (down K = I: 4, 24,
# 48, 90 chunks of 32), the one-token fused routing with E <= 64 and E > 64,
# both formats and the non-renormalised softmax.
CASES = [
    S.WORKLOADS["tiny"],
    S.custom(E=128, top_k=8, H=512, I=768, zipf_s=1.2, wid=31),
    S.custom(E=16, top_k=4, H=256, I=2880, fmt=O.FMT_MXFP4, wid=32),
    S.custom(E=12, top_k=3, H=384, I=1536, renormalize=0, wid=33),
]


def _run(layer, xb):
    out, ids, w = M.moe_forward(layer, bits_to_torch_bf16(xb), return_routing=True)
    torch.cuda.synchronize()
    return (out.view(torch.int16).cpu().numpy(), ids.cpu().numpy(),
            w.view(torch.int32).cpu().numpy())


def _same(a, b, what):
    for name, u, v in zip(("out", "topk_ids", "topk_w"), a, b):
        bad = np.argwhere(u != v)
        assert bad.size == 0, f"{what}: {name} differs first at {bad[0].tolist()} ({bad.shape[0]} elements)"


def _check_invariance(wl, path, Ts, singles, n_all, on_device_rng=False, gptoss=None):
    layer, o_layer, _ = build_layers(wl, 0, DEV, on_device_rng=on_device_rng, path=path, gptoss=gptoss)
    X = S.make_x(wl, n_all)
    full = _run(layer, X)
    rows = [0, n_all - 1]
    ref = O.moe_forward(o_layer, X[rows], topk_ids_override=full[1][rows])
    check_bound(O.bf16_bits_to_f64(full[0][rows].view(np.uint16)), ref, f"{wl.name} path={path}")
    for T in Ts:
        part = _run(layer, X[:T])
        _same(part, tuple(f[:T] for f in full), f"{wl.name} path={path}: first {T} of {n_all} tokens")
    for t in singles:
        one = _run(layer, X[t:t + 1])
        _same(one, tuple(f[t:t + 1] for f in full), f"{wl.name} path={path}: token {t} alone")
    # the same tokens in another order and company
    perm = np.array([n_all - 1, 3, n_all // 2, 0, 1])
    mixed = _run(layer, np.ascontiguousarray(X[perm]))
    _same(mixed, tuple(f[perm] for f in full), f"{wl.name} path={path}: permuted subset")


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_small_m_row_count_invariance(wl):
    """Forced small-M path: 1, 2, 3, 16, 17 and 160 tokens."""
    _check_invariance(wl, M.PATH_SMALL_M, [1, 2, 3, 16, 17], [1, 16, 159], 160)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_auto_decode_sizes_row_count_invariance(wl):
    """AUTO picks the small-M path while T * top_k <= 64 (48 for MXFP4): every
    such T agrees."""
    tmax = 1
    while M.auto_path(wl.fmt, (tmax + 1) * wl.top_k, max(wl.H, wl.I)) == M.PATH_SMALL_M:
        tmax += 1                                  # the largest call AUTO keeps on the small-M path
    _check_invariance(wl, M.PATH_AUTO, list(range(1, tmax)), [1, tmax - 1], tmax)


def test_gptoss_form_row_count_invariance():
    """Clamped GLU with per-expert biases (the down bias enters the token-centric
    kernel and the GEMV slot output the same way)."""
    wl = S.custom(E=16, top_k=4, H=256, I=2880, fmt=O.FMT_MXFP4, wid=36)
    _check_invariance(wl, M.PATH_SMALL_M, [1, 2, 3, 16], [1, 15], 17,
                      gptoss=dict(alpha=1.702, limit=1.0, interleaved=True))


def test_olmoe_shape_row_count_invariance():
    """The OLMoE-1B-7B-shaped layer (E=64, top_k=8, H=2048, I=1024): one token
    alone (the fused one-token routing and token-centric down) against 2, 8
    and 17 tokens on the small-M path."""
    wl = S.custom(E=64, top_k=8, H=2048, I=1024, wid=34)
    _check_invariance(wl, M.PATH_SMALL_M, [1, 2, 8], [1, 8, 16], 17, on_device_rng=True)


@pytest.mark.parametrize("wl", CASES[:3], ids=lambda w: w.name)
def test_mfma_row_count_invariance_per_router_window(wl):
    """Forced MFMA path: calls of up to 16 tokens share the per-token router
    (with top-k and grouping in one workgroup), calls of more than 16 the
    matrix-core router (top-k in parallel; grouping in one workgroup up to
    1024 routed slots, in three kernels above); and a routed row's MFMA result
    does not depend on the rows sharing its tile or on the tile height (64- or
    128-row tables and bodies)."""
    layer, o_layer, _ = build_layers(wl, 0, DEV, path=M.PATH_MFMA)
    X = S.make_x(wl, 1100)  # the router takes 128-token waves from 1024 tokens on
    full = _run(layer, X)
    rows = [0, 599, 1099]
    ref = O.moe_forward(o_layer, X[rows], topk_ids_override=full[1][rows])
    check_bound(O.bf16_bits_to_f64(full[0][rows].view(np.uint16)), ref, f"{wl.name} MFMA")
    for T in (17, 33, 177, 256, 257, 411, 1023, 1024):
        _same(_run(layer, X[:T]), tuple(f[:T] for f in full), f"{wl.name} MFMA: first {T} of 1100")
    perm = np.array([1099, 3, 300, 0, 1] + list(range(100, 120)))  # 25 tokens, another order
    _same(_run(layer, np.ascontiguousarray(X[perm])), tuple(f[perm] for f in full), f"{wl.name} MFMA: permuted")
    upto = _run(layer, X[:16])
    for T in (1, 2, 9, 15):
        _same(_run(layer, X[:T]), tuple(f[:T] for f in upto), f"{wl.name} MFMA: first {T} of 16")
    _same(_run(layer, X[7:8]), tuple(f[7:8] for f in upto), f"{wl.name} MFMA: token 7 alone")


def test_small_m_grouped_gemm_rows_independent():
    """nf4moe_grouped_gemm on the small-M path: a row's output does not depend
    on how many rows its group (or the call) holds."""
    rng = np.random.default_rng(35)
    E, N, K = 4, 384, 1024
    Wf = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    pk, sc = M.quantize(torch.from_numpy(Wf).to(DEV), O.FMT_NF4)
    ab = S.f32_to_bf16_bits(rng.standard_normal((40, K)).astype(np.float32))
    a = bits_to_torch_bf16(ab)

    def run(sizes, experts, rows):
        off = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32, device=DEV)
        c = M.grouped_gemm(a, pk, sc, off, K, int(sum(sizes)),
                           group_experts=torch.tensor(experts, dtype=torch.int32, device=DEV),
                           a_row_of=torch.tensor(rows, dtype=torch.int32, device=DEV),
                           path=M.PATH_SMALL_M)
        torch.cuda.synchronize()
        return c.view(torch.int32).cpu().numpy()

    big = run([17, 23], [2, 1], list(range(40)))
    alone = run([1], [2], [5])
    assert np.array_equal(alone[0], big[5])
    pair = run([1, 2], [1, 2], [30, 16, 0])
    assert np.array_equal(pair[0], big[30]) and np.array_equal(pair[1], big[16])
    assert np.array_equal(pair[2], big[0])


@pytest.mark.parametrize("E,k", [(64, 8), (100, 6)])
def test_one_token_routing_ties_signed_zeros_and_nan(E, k):
    """The one-token routing folded into the gate_up kernel ranks on the same
    total order as the routing kernels (logit descending, id ascending on
    order keys): exact ties from duplicated router rows, +0 / -0 logits from
    zero rows, and a token whose activations hold a NaN. Each token alone (the
    fused routing) must pick the ids and weights the separate routing kernels
    pick for it inside a two-token call, and, for finite logits, the oracle's
    selection rule on the GPU's own fp32 logits."""
    wl = S.custom(E=E, top_k=k, H=256, I=128, wid=37 + E)
    layer, _, _ = build_layers(wl, 0, DEV, path=M.PATH_AUTO)
    W = layer.router_w.clone()
    zero = [1, 4, 9, 17, 33, 40, 41, 50, E - 1]          # 9 zero rows: a tie across the k-th place
    dup = [10, 11, 12, 20]                                # identical rows: exact ties
    W[zero] = 0.0
    W[dup[:-1]] = W[dup[-1]].clone()
    b = np.full(E, -4.0, np.float32)
    b[zero] = np.where(np.arange(len(zero)) % 2 == 0, np.float32(0.0), np.float32(-0.0))
    b[dup] = 0.0
    layer.router_w = W.contiguous()
    layer.router_b = torch.from_numpy(b).to(DEV)
    X = S.make_x(wl, 7)
    X[6, 5] = 0x7FC0                                      # a NaN activation
    Wn, bn = layer.router_w.cpu().numpy(), b
    ties_seen = 0
    for t in range(7):
        one = _run(layer, X[t:t + 1])
        two = _run(layer, np.ascontiguousarray(X[[t, (t + 1) % 6]]))
        assert np.array_equal(one[1][0], two[1][0]), f"token {t}: ids {one[1][0]} vs {two[1][0]}"
        assert len(set(one[1][0].tolist())) == k and np.all((one[1][0] >= 0) & (one[1][0] < E))
        if t == 6:
            assert np.all(np.isnan(one[2][0].view(np.float32))) and np.all(np.isnan(two[2][0].view(np.float32)))
            continue
        assert np.array_equal(one[2][0], two[2][0]), f"token {t}: weights differ"
        assert np.array_equal(one[0][0], two[0][0]), f"token {t}: outputs differ"
        L32 = M.router_logits(bits_to_torch_bf16(X[t:t + 1]), layer.router_w, layer.router_b,
                              matrix_cores=False).cpu().numpy().astype(np.float64)
        ids_o, w_o = O.topk_route(L32, k, True)
        assert np.array_equal(one[1][0], ids_o[0])
        assert np.max(np.abs(one[2][0].view(np.float32) - w_o[0])) <= 1e-6
        srt = np.sort(L32[0])[::-1]
        ties_seen += int(srt[k - 1] == srt[k])
    assert ties_seen > 0, "no token had a tie across the k-th place"
