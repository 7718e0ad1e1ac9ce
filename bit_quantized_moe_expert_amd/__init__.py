"""Python binding of libnf4moe.so: the routed MoE expert layer on 4-bit packed
weights (NF4 blocksize 64, MXFP4 blocksize 32) for MI355X (gfx950).

This module only marshals arguments: every step runs in the library's HIP
kernels. torch supplies device memory and the current HIP stream. Calls with
CPU tensors raise; nothing falls back to another implementation. The library
must have been built (``python -m bit_quantized_moe_expert_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

FMT_NF4 = 0
FMT_MXFP4 = 1
FMT_NF4_BF16ABS = 2   # NF4 b64 with the absmax stored as bf16
PATH_AUTO, PATH_SMALL_M, PATH_MFMA = 0, 1, 2
DT_F32, DT_BF16 = 0, 1
GLU_SWIGLU, GLU_CLAMPED = 0, 1
BLOCK = {FMT_NF4: 64, FMT_MXFP4: 32, FMT_NF4_BF16ABS: 64}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4moe.so")
_lib = None


class Nf4MoeError(RuntimeError):
    """A non-OK status from libnf4moe (the message is nf4moe_last_error())."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Layer(ctypes.Structure):
    """Mirror of nf4moe_layer_t."""
    _fields_ = [
        ("fmt", ctypes.c_int), ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("path", ctypes.c_int32),
        ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p),
        ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
        ("glu", ctypes.c_int32), ("glu_alpha", ctypes.c_float), ("glu_limit", ctypes.c_float),
        ("glu_interleaved", ctypes.c_int32), ("b13", ctypes.c_void_p), ("b2", ctypes.c_void_p),
    ]


def lib() -> ctypes.CDLL:
    """Load libnf4moe.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m bit_quantized_moe_expert_amd.build`")
    # The library must run on the same HIP runtime as torch, which owns the
    # device memory and streams it is handed. torch ships its own
    # libamdhip64.so.7; importing torch first makes the dynamic loader bind this
    # library's libamdhip64.so.7 dependency to that copy instead of loading a
    # second runtime from the system ROCm (two runtimes in one process do not
    # share devices).
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "nf4moe_quantize": [ctypes.c_int, vp, i64, i64, vp, vp, vp],
        "nf4moe_dequantize": [ctypes.c_int, vp, vp, i64, i64, vp, vp],
        "nf4moe_absmax_to_bf16": [vp, i64, vp, vp, vp],
        "nf4moe_router_logits": [vp, i32, i32, vp, vp, i32, vp, vp, sz, vp],
        "nf4moe_router_workspace_bytes": [i32, i32, i32],
        "nf4moe_route_workspace_bytes": [i32, i32, i32],
        "nf4moe_route_permute": [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp],
        "nf4moe_gemm_workspace_bytes": [i32, i32],
        "nf4moe_grouped_gemm": [ctypes.c_int, vp, vp, i32, vp, vp, i32, i64, i64, i32, vp, vp, i32,
                                vp, ctypes.c_int, i32, vp, sz, vp],
        "nf4moe_workspace_bytes": [ctypes.POINTER(Layer), i32],
        "nf4moe_grouped_dgrad": [ctypes.c_int, vp, vp, vp, i32, i64, i64, i32, vp, vp, i32, vp,
                                 ctypes.c_int, vp, sz, vp],
        "nf4moe_moe_forward": [ctypes.POINTER(Layer), vp, i32, vp, vp, vp, vp, sz, vp],
        "nf4moe_moe_forward_noalloc": [ctypes.POINTER(Layer), vp, i32, vp, vp, vp, vp],
        "nf4moe_moe_forward_profiled": [ctypes.POINTER(Layer), vp, i32, vp, vp, sz, vp,
                                        ctypes.POINTER(ctypes.c_void_p)],
        "nf4moe_codebook": [ctypes.c_int, ctypes.POINTER(ctypes.c_float)],
        "nf4moe_auto_path": [ctypes.c_int, i64, i64],
        "nf4moe_stream_read_sink_words": [i64, i32],
        "nf4moe_stream_read": [vp, i64, i32, vp, vp],
        "nf4moe_mfma_peak_flops": [i32, i32],
        "nf4moe_mfma_peak": [i32, i32, vp, vp],
        "nf4moe_status_string": [ctypes.c_int],
        "nf4moe_last_error": [],
        "nf4moe_version": [],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    for name in ("nf4moe_route_workspace_bytes", "nf4moe_gemm_workspace_bytes", "nf4moe_workspace_bytes",
                 "nf4moe_router_workspace_bytes"):
        getattr(L, name).restype = ctypes.c_size_t
    L.nf4moe_stream_read_sink_words.restype = ctypes.c_int64
    L.nf4moe_mfma_peak_flops.restype = ctypes.c_int64
    for name in ("nf4moe_status_string", "nf4moe_last_error", "nf4moe_version"):
        getattr(L, name).restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        L = lib()
        raise Nf4MoeError(status, f"{L.nf4moe_status_string(status).decode()}: "
                                  f"{L.nf4moe_last_error().decode()}")


def version() -> str:
    return lib().nf4moe_version().decode()


def codebook(fmt: int = FMT_NF4):
    """The 16 fp32 decode values the kernels use (host copy, no device access)."""
    buf = (ctypes.c_float * 16)()
    _check(lib().nf4moe_codebook(fmt, buf))
    return [float(v) for v in buf]


# ----------------------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} is on {t.device}: libnf4moe computes on the GPU only "
                         "(the CPU reference is the test oracle, not a fallback)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t, name, shape):
    """Refuse a tensor whose shape is not `shape` (None entries match any size).
    The C ABI sees raw pointers only, so every size it is told must match the
    buffer; this runs before the device check."""
    torch = _torch()
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    got = tuple(t.shape)
    if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
        want = "(" + ", ".join("*" if w is None else str(w) for w in shape) + ")"
        raise ValueError(f"{name} has shape {got}, expected {want}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _workspace(nbytes: int, device):
    torch = _torch()
    ws = torch.empty(max(int(nbytes), 256) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws, ctypes.c_void_p(ws.data_ptr() + off), int(nbytes)


def _scale_dtype(fmt):
    torch = _torch()
    return {FMT_NF4: torch.float32, FMT_MXFP4: torch.uint8, FMT_NF4_BF16ABS: torch.int16}[fmt]


def stream_read(buf, nbytes: int, sink, loads_per_thread: int = 4):
    """Measurement aid: one launch reading the first nbytes of buf (device) once
    with 16-byte loads, loads_per_thread per thread; sink is a device int32
    tensor of at least stream_read_sink_words(nbytes, loads_per_thread) elements."""
    _dev(buf, "buf")
    _dev(sink, "sink")
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError(f"nbytes={nbytes} exceeds the buffer")
    if sink.numel() * sink.element_size() < 4 * stream_read_sink_words(nbytes, loads_per_thread):
        raise ValueError("sink too small")
    _check(lib().nf4moe_stream_read(_ptr(buf), nbytes, loads_per_thread, _ptr(sink), _stream()))


def stream_read_sink_words(nbytes: int, loads_per_thread: int = 4) -> int:
    return int(lib().nf4moe_stream_read_sink_words(nbytes, loads_per_thread))


def mfma_peak(workgroups: int, iters: int, sink) -> int:
    """Launch the bf16 matrix-core rate probe (a measurement aid) on the current
    stream; sink: float32 device tensor of at least workgroups * 512 elements.
    Returns the launch's flops."""
    torch = _torch()
    _dev(sink, "sink", torch.float32)
    if sink.numel() < workgroups * 512:
        raise ValueError(f"sink holds {sink.numel()} floats, needs {workgroups * 512}")
    _check(lib().nf4moe_mfma_peak(workgroups, iters, _ptr(sink), _stream()))
    return int(lib().nf4moe_mfma_peak_flops(workgroups, iters))


def quantize(w, fmt: int = FMT_NF4):
    """fp32 [..., K] (device) -> (packed uint8 [..., K/2], scale [..., K/block])."""
    torch = _torch()
    _dev(w, "w", torch.float32)
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    packed = torch.empty(*w.shape[:-1], K // 2, dtype=torch.uint8, device=w.device)
    scale = torch.empty(*w.shape[:-1], K // BLOCK[fmt], dtype=_scale_dtype(fmt), device=w.device)
    _check(lib().nf4moe_quantize(fmt, _ptr(w), rows, K, _ptr(packed), _ptr(scale), _stream()))
    return packed, scale


def dequantize(packed, scale, K: int, fmt: int = FMT_NF4):
    """(packed [..., K/2], scale) -> fp32 [..., K] (device)."""
    torch = _torch()
    if K <= 0 or K % BLOCK[fmt]:
        raise ValueError(f"K={K} must be a positive multiple of {BLOCK[fmt]}")
    lead = tuple(packed.shape[:-1])
    _shape(packed, "packed", lead + (K // 2,))
    _shape(scale, "scale", lead + (K // BLOCK[fmt],))
    _dev(packed, "packed", torch.uint8)
    _dev(scale, "scale", _scale_dtype(fmt))
    rows = packed.numel() // (K // 2)
    out = torch.empty(*packed.shape[:-1], K, dtype=torch.float32, device=packed.device)
    _check(lib().nf4moe_dequantize(fmt, _ptr(packed), _ptr(scale), rows, K, _ptr(out), _stream()))
    return out


def absmax_to_bf16(absmax):
    """The bf16 absmax cast of an NF4 fp32 scale tensor (device): returns
    (bf16 bits as int16, same shape; number of entries that were not bf16 values
    and were rounded up). The cast is lossless only when that number is 0."""
    torch = _torch()
    _dev(absmax, "absmax", torch.float32)
    out = torch.empty(absmax.shape, dtype=torch.int16, device=absmax.device)
    bad = torch.zeros(1, dtype=torch.int32, device=absmax.device)
    _check(lib().nf4moe_absmax_to_bf16(_ptr(absmax), absmax.numel(), _ptr(out), _ptr(bad), _stream()))
    return out, int(bad.item())


def auto_path(fmt: int, R: int, K_max: int) -> int:
    """The kernel family AUTO runs for R routed rows (PATH_SMALL_M or PATH_MFMA)."""
    return int(lib().nf4moe_auto_path(fmt, R, K_max))


def router_logits(x, router_w, router_b=None, matrix_cores: bool = True):
    """x bf16 [T, H], W_r fp32 [E, H] (+ b [E]) -> logits fp32 [T, E].
    matrix_cores: hand the library the workspace that enables its MFMA kernel
    (H % 16 == 0; the logits the forward's MFMA path routes on); False keeps
    the vector-ALU kernels (the small-M path's logits up to 256 tokens)."""
    torch = _torch()
    _shape(x, "x", (None, None))
    T, H = x.shape
    _shape(router_w, "router_w", (None, H))
    E = router_w.shape[0]
    _shape(router_b, "router_b", (E,))
    _dev(x, "x", torch.bfloat16)
    _dev(router_w, "router_w", torch.float32)
    if router_b is not None:
        _dev(router_b, "router_b", torch.float32)
    out = torch.empty(T, E, dtype=torch.float32, device=x.device)
    ws, nb = None, 0
    if matrix_cores and T > 0:
        nb = lib().nf4moe_router_workspace_bytes(T, E, H)
        if nb:
            ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    _check(lib().nf4moe_router_logits(_ptr(x), T, H, _ptr(router_w), _ptr(router_b), E, _ptr(out),
                                      _ptr(ws), nb, _stream()))
    return out


def route_permute(logits, top_k: int, renormalize: bool = True):
    """logits fp32 [T, E] -> dict(topk_ids, topk_w, expert_offsets, sorted_slots)."""
    torch = _torch()
    _shape(logits, "logits", (None, None))
    _dev(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, top_k, dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    slots = torch.empty(T * top_k, dtype=torch.int32, device=dev)
    need = lib().nf4moe_route_workspace_bytes(T, E, top_k)
    ws, wsp, nb = _workspace(need, dev)
    _check(lib().nf4moe_route_permute(_ptr(logits), T, E, top_k, int(renormalize), _ptr(ids), _ptr(w),
                                      _ptr(off), _ptr(slots), wsp, nb, _stream()))
    return dict(topk_ids=ids, topk_w=w, expert_offsets=off, sorted_slots=slots, _ws=ws)


def grouped_gemm(a, B, B_scale, group_offsets, K: int, R: int, group_experts=None, a_row_of=None,
                 fmt: int = FMT_NF4, out_dtype=None, path: int = PATH_AUTO):
    """The pages' gemm_4bit_grouped: c[r] = a[row(r)] . W[e(r)]^T, W decoded from
    4-bit codes in registers. a bf16 [rows_a, K]; B [E, N, K/2] u8; group_offsets
    int32 [G+1] (device); group_experts int32 [G] or None; a_row_of int32 [R] or None.
    Returns c [R, N] (fp32 or bf16)."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    if K <= 0 or K % BLOCK[fmt]:
        raise ValueError(f"K={K} must be a positive multiple of {BLOCK[fmt]}")
    _shape(B, "B", (None, None, K // 2))
    E, N = B.shape[0], B.shape[1]
    _shape(B_scale, "B_scale", (E, N, K // BLOCK[fmt]))
    _shape(a, "a", (None, K))
    _shape(group_offsets, "group_offsets", (None,))
    G = group_offsets.numel() - 1
    _shape(group_experts, "group_experts", (G,))
    _shape(a_row_of, "a_row_of", (R,))
    if a_row_of is None and a.shape[0] < R:
        raise ValueError(f"a has {a.shape[0]} rows, fewer than R={R} (and no a_row_of gather)")
    _dev(a, "a", torch.bfloat16)
    _dev(B, "B", torch.uint8)
    _dev(B_scale, "B_scale", _scale_dtype(fmt))
    _dev(group_offsets, "group_offsets", torch.int32)
    if group_experts is not None:
        _dev(group_experts, "group_experts", torch.int32)
    if a_row_of is not None:
        _dev(a_row_of, "a_row_of", torch.int32)
    c = torch.empty(R, N, dtype=out_dtype, device=a.device)
    need = lib().nf4moe_gemm_workspace_bytes(G, R)
    ws, wsp, nb = _workspace(need, a.device)
    dt = DT_F32 if out_dtype == torch.float32 else DT_BF16
    _check(lib().nf4moe_grouped_gemm(fmt, _ptr(a), _ptr(a_row_of), a.shape[0], _ptr(B), _ptr(B_scale),
                                     E, N, K, G, _ptr(group_offsets), _ptr(group_experts), R, _ptr(c),
                                     dt, path, wsp, nb, _stream()))
    return c


def grouped_dgrad(dc, B, B_scale, group_offsets, K: int, group_experts=None, fmt: int = FMT_NF4,
                  out_dtype=None):
    """The pages' dgrad_4bit_grouped: da[r] = dc[r] . W[e(r)], W decoded from 4-bit
    codes in registers (the input gradient of grouped_gemm). dc bf16 [R, N] in group
    order; B [E, N, K/2] u8; group_offsets int32 [G+1] (device). Returns da [R, K]."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    if K <= 0 or K % BLOCK[fmt]:
        raise ValueError(f"K={K} must be a positive multiple of {BLOCK[fmt]}")
    _shape(B, "B", (None, None, K // 2))
    E, N = B.shape[0], B.shape[1]
    _shape(B_scale, "B_scale", (E, N, K // BLOCK[fmt]))
    _shape(dc, "dc", (None, N))
    R = dc.shape[0]
    _shape(group_offsets, "group_offsets", (None,))
    G = group_offsets.numel() - 1
    _shape(group_experts, "group_experts", (G,))
    _dev(dc, "dc", torch.bfloat16)
    _dev(B, "B", torch.uint8)
    _dev(B_scale, "B_scale", _scale_dtype(fmt))
    _dev(group_offsets, "group_offsets", torch.int32)
    if group_experts is not None:
        _dev(group_experts, "group_experts", torch.int32)
    da = torch.empty(R, K, dtype=out_dtype, device=dc.device)
    need = lib().nf4moe_gemm_workspace_bytes(G, R)
    ws, wsp, nb = _workspace(need, dc.device)
    dt = DT_F32 if out_dtype == torch.float32 else DT_BF16
    _check(lib().nf4moe_grouped_dgrad(fmt, _ptr(dc), _ptr(B), _ptr(B_scale), E, N, K, G,
                                      _ptr(group_offsets), _ptr(group_experts), R, _ptr(da), dt,
                                      wsp, nb, _stream()))
    return da


@dataclass
class MoELayer:
    """One routed MoE layer held on the device in 4-bit form.

    w13 [E, 2I, H/2] u8 (rows [0, I) gate, [I, 2I) up; with glu_interleaved rows 2c
    gate, 2c + 1 up), w13_scale, w2 [E, H, I/2] u8, w2_scale, router_w fp32 [E, H],
    router_b fp32 [E] or None. glu: GLU_SWIGLU or GLU_CLAMPED (glu_alpha, glu_limit);
    b13 fp32 [E, 2I] and b2 fp32 [E, H] per-expert biases or None."""
    fmt: int
    E: int
    H: int
    I: int
    top_k: int
    w13: object
    w13_scale: object
    w2: object
    w2_scale: object
    router_w: object
    router_b: object = None
    renormalize: int = 1
    path: int = PATH_AUTO
    glu: int = 0
    glu_alpha: float = 0.0
    glu_limit: float = 0.0
    glu_interleaved: int = 0
    b13: object = None
    b2: object = None

    def check_shapes(self):
        """Refuse tensors whose shapes do not match (E, H, I) and the format."""
        if self.fmt not in BLOCK:
            raise ValueError(f"unknown format {self.fmt}")
        blk = BLOCK[self.fmt]
        E, H, I = self.E, self.H, self.I
        if E < 1 or H <= 0 or I <= 0 or H % 64 or I % blk:
            raise ValueError(f"E={E}, H={H}, I={I}: need E >= 1, H % 64 == 0, I % {blk} == 0")
        _shape(self.w13, "w13", (E, 2 * I, H // 2))
        _shape(self.w13_scale, "w13_scale", (E, 2 * I, H // blk))
        _shape(self.w2, "w2", (E, H, I // 2))
        _shape(self.w2_scale, "w2_scale", (E, H, I // blk))
        _shape(self.router_w, "router_w", (E, H))
        _shape(self.router_b, "router_b", (E,))
        _shape(self.b13, "b13", (E, 2 * I))
        _shape(self.b2, "b2", (E, H))

    def struct(self) -> Layer:
        torch = _torch()
        self.check_shapes()
        sd = _scale_dtype(self.fmt)
        _dev(self.w13, "w13", torch.uint8)
        _dev(self.w2, "w2", torch.uint8)
        _dev(self.w13_scale, "w13_scale", sd)
        _dev(self.w2_scale, "w2_scale", sd)
        _dev(self.router_w, "router_w", torch.float32)
        if self.router_b is not None:
            _dev(self.router_b, "router_b", torch.float32)
        for name in ("b13", "b2"):
            if getattr(self, name) is not None:
                _dev(getattr(self, name), name, torch.float32)
        ptr = lambda t: None if t is None else t.data_ptr()
        return Layer(self.fmt, self.E, self.H, self.I, self.top_k, self.renormalize, self.path,
                     self.w13.data_ptr(), self.w13_scale.data_ptr(), self.w2.data_ptr(),
                     self.w2_scale.data_ptr(), self.router_w.data_ptr(), ptr(self.router_b),
                     self.glu, self.glu_alpha, self.glu_limit, self.glu_interleaved,
                     ptr(self.b13), ptr(self.b2))

    def workspace_bytes(self, T: int) -> int:
        return int(lib().nf4moe_workspace_bytes(ctypes.byref(self.struct()), T))


class Forward:
    """Reusable forward call: holds the layer struct and a workspace sized for
    T_max tokens, so repeated calls allocate nothing."""

    def __init__(self, layer: MoELayer, T_max: int, device="cuda"):
        self.layer = layer
        self.st = layer.struct()
        self.T_max = T_max
        need = lib().nf4moe_workspace_bytes(ctypes.byref(self.st), T_max)
        self._ws, self.wsp, self.nb = _workspace(need, device)

    def set_layer(self, layer: MoELayer):
        """Point at another layer of the same shape (workspace is reused)."""
        self.layer = layer
        self.st = layer.struct()

    def __call__(self, x, out=None, topk_ids=None, topk_w=None):
        torch = _torch()
        check_forward_args(self.layer, x, out, topk_ids, topk_w)
        _dev(x, "x", torch.bfloat16)
        T = x.shape[0]
        if T > self.T_max:
            raise ValueError(f"T={T} > T_max={self.T_max}")
        if out is None:
            out = torch.empty(T, self.layer.H, dtype=torch.bfloat16, device=x.device)
        _dev(out, "out", torch.bfloat16)
        if topk_ids is not None:
            _dev(topk_ids, "topk_ids", torch.int32)
        if topk_w is not None:
            _dev(topk_w, "topk_w", torch.float32)
        _check(lib().nf4moe_moe_forward(ctypes.byref(self.st), _ptr(x), T, _ptr(out), _ptr(topk_ids),
                                        _ptr(topk_w), self.wsp, self.nb, _stream()))
        return out


    def profiled(self, x, out, events):
        """Same computation with 6 caller HIP event handles: [0..3] recorded between
        stages, [4], [5] the gate_up kernel's own start and end."""
        torch = _torch()
        if len(events) != 6:
            raise ValueError("profiled() takes 6 events")
        check_forward_args(self.layer, x, out, None, None)
        _dev(x, "x", torch.bfloat16)
        _dev(out, "out", torch.bfloat16)
        if x.shape[0] > self.T_max:
            raise ValueError(f"T={x.shape[0]} > T_max={self.T_max}")
        arr = (ctypes.c_void_p * 6)(*events)
        _check(lib().nf4moe_moe_forward_profiled(ctypes.byref(self.st), _ptr(x), x.shape[0], _ptr(out),
                                                 self.wsp, self.nb, _stream(), arr))
        return out


def check_forward_args(layer: MoELayer, x, out=None, topk_ids=None, topk_w=None):
    """Shapes of a forward call: x [T, H]; out [T, H]; topk_ids / topk_w [T, top_k]."""
    _shape(x, "x", (None, layer.H))
    T = x.shape[0]
    _shape(out, "out", (T, layer.H))
    _shape(topk_ids, "topk_ids", (T, layer.top_k))
    _shape(topk_w, "topk_w", (T, layer.top_k))


NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_forward_noalloc(layer: MoELayer, x, out, topk_ids=None, topk_w=None):
    """The layer through nf4moe_moe_forward_noalloc: no workspace, the library's
    per-device scratch (NOALLOC_SCRATCH_BYTES); the caller passes every output."""
    torch = _torch()
    check_forward_args(layer, x, out, topk_ids, topk_w)
    st = layer.struct()
    _dev(x, "x", torch.bfloat16)
    _dev(out, "out", torch.bfloat16)
    if topk_ids is not None:
        _dev(topk_ids, "topk_ids", torch.int32)
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32)
    _check(lib().nf4moe_moe_forward_noalloc(ctypes.byref(st), _ptr(x), x.shape[0], _ptr(out), _ptr(topk_ids),
                                            _ptr(topk_w), _stream()))
    return out


def moe_forward(layer: MoELayer, x, return_routing: bool = False):
    """out bf16 [T, H] = the routed MoE layer applied to x bf16 [T, H]."""
    torch = _torch()
    T = x.shape[0]
    fwd = Forward(layer, T, x.device)
    if not return_routing:
        return fwd(x)
    ids = torch.empty(T, layer.top_k, dtype=torch.int32, device=x.device)
    w = torch.empty(T, layer.top_k, dtype=torch.float32, device=x.device)
    out = fwd(x, topk_ids=ids, topk_w=w)
    return out, ids, w
