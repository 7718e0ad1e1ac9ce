"""Shared helpers of the GPU parity tests: device layers, the oracle-side layers
built from the same fp32 inputs, the output bound, and the near-tie rule."""
from __future__ import annotations

import numpy as np

import moe_synth as S
import oracle as O

# The output contract: |gpu - oracle| <= 1e-2 * |oracle| + 1e-3 * rms(oracle),
# elementwise, against the unrounded fp64 oracle.
REL, ABS_RMS = 1e-2, 1e-3


def check_bound(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(gpu - ref)
    bound = REL * np.abs(ref) + ABS_RMS * rms
    ratio = float(np.max(err / np.maximum(bound, 1e-300))) if ref.size else 0.0
    bad = int(np.sum(err > bound))
    assert bad == 0, f"{what}: {bad} of {err.size} elements outside the bound (max err/bound {ratio:.3f})"
    return ratio


def bf16_to_np(t):
    """torch bf16 tensor -> fp64 numpy (exact)."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().astype(np.uint16)
    return O.bf16_bits_to_f64(bits)


def bits_to_torch_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class LazyStack:
    """Oracle-side packed weights, quantized by the oracle one expert at a time
    from the fp32 source (numpy array or a torch device tensor [E, N, K])."""

    def __init__(self, fmt, src):
        self.fmt, self.src, self.cache = fmt, src, {}

    def _get(self, e):
        if e not in self.cache:
            w = self.src[e]
            if not isinstance(w, np.ndarray):
                w = w.detach().cpu().numpy()
            self.cache[e] = O.quantize(self.fmt, np.ascontiguousarray(w, np.float32))
        return self.cache[e]

    def prefetch(self, experts, workers=16):
        """Quantize the listed experts ahead of use on a thread pool (numpy's
        array operations release the GIL, so the oracle's per-expert
        quantization runs in parallel); the values are those _get computes."""
        from concurrent.futures import ThreadPoolExecutor
        todo = sorted(set(int(e) for e in experts) - set(self.cache))
        if not todo:
            return
        with ThreadPoolExecutor(max(1, min(workers, len(todo)))) as ex:
            for e, q in zip(todo, ex.map(self._quantize_one, todo)):
                self.cache[e] = q

    def _quantize_one(self, e):
        w = self.src[e]
        if not isinstance(w, np.ndarray):
            w = w.detach().cpu().numpy()
        return O.quantize(self.fmt, np.ascontiguousarray(w, np.float32))

    def packed(self):
        return _Proj(self, 0)

    def scale(self):
        return _Proj(self, 1)


class _Proj:
    def __init__(self, st, i):
        self.st, self.i = st, i

    def stack(self):
        return self.st

    def __getitem__(self, e):
        return self.st._get(int(e))[self.i]


def build_layers(wl: S.Workload, layer=0, device="cuda", on_device_rng=False, path=0, gptoss=None,
                 bf16_source=False):
    """Returns (device MoELayer, oracle layer dict, fp32 sources).

    gptoss: None, or dict(alpha, limit, interleaved) for the gpt-oss expert form
    (clamped GLU, per-expert biases; interleaved gate / up rows). bf16_source:
    round the weights to bf16 values first (a bf16 checkpoint)."""
    import torch
    import bit_quantized_moe_expert_amd as M
    W_r, b_r = S.make_router(wl, layer)
    if on_device_rng:
        w13 = S.make_stack_torch(wl, layer, "w13", device)
        w2 = S.make_stack_torch(wl, layer, "w2", device)
        w13_d, w2_d = w13, w2
    else:
        w13 = S.make_stack(wl, layer, "w13")
        w2 = S.make_stack(wl, layer, "w2")
        w13_d = torch.from_numpy(w13).to(device)
        w2_d = torch.from_numpy(w2).to(device)
    if bf16_source:
        if on_device_rng:
            w13 = w13.to(torch.bfloat16).to(torch.float32)
            w2 = w2.to(torch.bfloat16).to(torch.float32)
            w13_d, w2_d = w13, w2
        else:
            w13 = O.bf16_bits_to_f64(S.f32_to_bf16_bits(w13)).astype(np.float32)
            w2 = O.bf16_bits_to_f64(S.f32_to_bf16_bits(w2)).astype(np.float32)
            w13_d = torch.from_numpy(w13).to(device)
            w2_d = torch.from_numpy(w2).to(device)
    extra, o_extra = {}, {}
    if gptoss is not None:
        b13, b2 = S.make_biases(wl, layer)
        if gptoss.get("interleaved"):
            perm = np.empty(2 * wl.I, np.int64)
            perm[0::2] = np.arange(wl.I)
            perm[1::2] = wl.I + np.arange(wl.I)
            b13 = np.ascontiguousarray(b13[:, perm])
            if on_device_rng:
                w13 = w13[:, torch.from_numpy(perm).to(device)].contiguous()
                w13_d = w13
            else:
                w13 = np.ascontiguousarray(w13[:, perm])
                w13_d = torch.from_numpy(w13).to(device)
        extra = dict(glu=M.GLU_CLAMPED, glu_alpha=float(gptoss["alpha"]), glu_limit=float(gptoss["limit"]),
                     glu_interleaved=int(bool(gptoss.get("interleaved"))),
                     b13=torch.from_numpy(b13).to(device), b2=torch.from_numpy(b2).to(device))
        o_extra = dict(glu=O.GLU_CLAMPED, glu_alpha=float(gptoss["alpha"]), glu_limit=float(gptoss["limit"]),
                       glu_interleaved=int(bool(gptoss.get("interleaved"))), b13=b13, b2=b2)
    p13, s13 = M.quantize(w13_d, wl.fmt)
    p2, s2 = M.quantize(w2_d, wl.fmt)
    dev_layer = M.MoELayer(
        fmt=wl.fmt, E=wl.E, H=wl.H, I=wl.I, top_k=wl.top_k,
        w13=p13, w13_scale=s13, w2=p2, w2_scale=s2,
        router_w=torch.from_numpy(W_r).to(device),
        router_b=None if b_r is None else torch.from_numpy(b_r).to(device),
        renormalize=wl.renormalize, path=path, **extra)
    st13, st2 = LazyStack(wl.fmt, w13), LazyStack(wl.fmt, w2)
    o_layer = dict(fmt=wl.fmt, E=wl.E, H=wl.H, I=wl.I, top_k=wl.top_k, renormalize=wl.renormalize,
                   w13=st13.packed(), w13_scale=st13.scale(), w2=st2.packed(), w2_scale=st2.scale(),
                   router_w=W_r, router_b=b_r, **o_extra)
    return dev_layer, o_layer, (w13, w2)


def check_routing_near_ties(gpu_ids, L64, k, renorm=True):
    """Tokens where the GPU (fp32 logits) picked differently from the oracle
    (fp64 logits) are allowed only where the logits that swapped are within
    tau = 1e-5 * (1 + max|L|). Returns the number of such tokens."""
    ids_o, _ = O.topk_route(L64, k, renorm)
    tau = 1e-5 * (1.0 + np.max(np.abs(L64), axis=1))
    n = 0
    for t in range(L64.shape[0]):
        if np.array_equal(gpu_ids[t], ids_o[t]):
            continue
        n += 1
        assert len(set(gpu_ids[t].tolist())) == k, f"token {t}: repeated expert"
        for j in range(k):
            a, b = int(gpu_ids[t, j]), int(ids_o[t, j])
            if a != b:
                assert abs(L64[t, a] - L64[t, b]) <= tau[t], (
                    f"token {t} slot {j}: gpu {a} ({L64[t, a]}) vs oracle {b} ({L64[t, b]})")
    return n


def prefetch_experts(o_layer, experts, workers=16):
    """Quantize (oracle side) the experts a sample will touch, in parallel."""
    for key in ("w13", "w2"):
        st = o_layer[key]
        if isinstance(st, _Proj):
            st.stack().prefetch(experts, workers)


def coverage_tokens(gids, E, tile_rows, n, seed, allowed=None):
    """Tokens to compare at full size, chosen from the GPU's routing so that
    every expert group's first row, last row and the first row of its last
    (partial) tile, and the rows on each side of its first tile boundary, are
    among the compared rows (a group's rows are its slots t*k + j in ascending
    order); then seeded random tokens up to n. allowed: optional boolean mask
    of tokens that may be chosen (e.g. those whose experts the oracle has)."""
    T, k = gids.shape
    flat = gids.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    off = np.concatenate([[0], np.cumsum(counts)])
    ok = np.ones(T, bool) if allowed is None else np.asarray(allowed, bool)
    chosen = []
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        pos = [0, c - 1, (c - 1) // tile_rows * tile_rows]
        if c > tile_rows:
            pos += [tile_rows - 1, tile_rows]
        for p in pos:
            t = int(order[off[e] + p]) // k
            if ok[t]:
                chosen.append(t)
    chosen = list(dict.fromkeys(chosen))
    rest = np.setdiff1d(np.flatnonzero(ok), chosen)
    extra = max(0, n - len(chosen))
    if extra and rest.size:
        rng = np.random.default_rng(seed)
        chosen += rng.choice(rest, min(extra, rest.size), replace=False).tolist()
    return np.array(sorted(chosen), dtype=np.int64)
