"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, reports the decode tables, and every invalid-argument path returns its
status before any device work (fake, never-dereferenced pointers are used)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4moe.h")

pkg = pytest.importorskip("bit_quantized_moe_expert_amd")
if not os.path.exists(pkg.LIB_PATH):
    pytest.skip("libnf4moe.so not built", allow_module_level=True)

L = pkg.lib()
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000          # aligned, never dereferenced
STREAM = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4moe_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    raw = ctypes.CDLL(pkg.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_codebooks_match_oracle():
    assert np.array_equal(np.array(pkg.codebook(pkg.FMT_NF4), np.float32), O.nf4_codebook())
    lib_e2m1 = np.array(pkg.codebook(pkg.FMT_MXFP4), np.float32)
    ref = O.e2m1_values()
    assert np.array_equal(lib_e2m1, ref) and np.array_equal(np.signbit(lib_e2m1), np.signbit(ref))


def test_status_strings_and_version():
    assert L.nf4moe_status_string(0) == b"NF4MOE_OK"
    assert L.nf4moe_status_string(3) == b"NF4MOE_ERR_WORKSPACE"
    assert b"gfx950" in L.nf4moe_version()
    buf = (ctypes.c_float * 16)()
    assert L.nf4moe_codebook(7, buf) == INVALID
    assert b"format" in L.nf4moe_last_error()


def test_quantize_validation():
    q = L.nf4moe_quantize
    assert q(0, FAKE, 4, 63, FAKE, FAKE, STREAM) == INVALID           # K not multiple of 64
    assert q(1, FAKE, 4, 48, FAKE, FAKE, STREAM) == INVALID           # K not multiple of 32
    assert q(0, FAKE, -1, 64, FAKE, FAKE, STREAM) == INVALID
    assert q(0, None, 4, 64, FAKE, FAKE, STREAM) == INVALID
    assert q(3, FAKE, 4, 64, FAKE, FAKE, STREAM) == INVALID           # unknown format
    assert q(0, FAKE + 1, 4, 64, FAKE, FAKE, STREAM) == INVALID       # misaligned
    assert q(0, FAKE, 0, 64, FAKE, FAKE, STREAM) == OK                # empty: no-op
    assert L.nf4moe_dequantize(0, FAKE, FAKE, 2, 100, FAKE, STREAM) == INVALID
    assert L.nf4moe_dequantize(2, FAKE, FAKE + 1, 2, 64, FAKE, STREAM) == INVALID   # bf16 absmax misaligned
    cast = L.nf4moe_absmax_to_bf16
    assert cast(FAKE, -1, FAKE, FAKE, STREAM) == INVALID
    assert cast(None, 4, FAKE, FAKE, STREAM) == INVALID
    assert cast(FAKE, 0, FAKE, FAKE, STREAM) == OK                    # empty: no-op


def test_router_and_route_validation():
    assert L.nf4moe_router_logits(FAKE, -1, 64, FAKE, None, 8, FAKE, None, 0, STREAM) == INVALID
    assert L.nf4moe_router_logits(FAKE, 1, 60, FAKE, None, 8, FAKE, None, 0, STREAM) == INVALID
    assert L.nf4moe_router_logits(FAKE, 1, 64, FAKE, None, 2000, FAKE, None, 0, STREAM) == INVALID
    assert L.nf4moe_router_logits(FAKE, 0, 64, FAKE, None, 8, FAKE, None, 0, STREAM) == OK
    need = L.nf4moe_router_workspace_bytes(64, 8, 64)
    assert need >= 4 * 4 * 64 * 8                       # S = 4 chunks of 16 for H = 64
    assert L.nf4moe_router_workspace_bytes(64, 8, 2048) >= 4 * 8 * 64 * 8
    assert L.nf4moe_router_workspace_bytes(64, 8, 72) == 0      # H % 16: vector path only
    assert L.nf4moe_router_workspace_bytes(0, 8, 64) == 0
    assert L.nf4moe_router_logits(FAKE, 64, 64, FAKE, None, 8, FAKE, FAKE, need - 1, STREAM) == 3  # WORKSPACE
    rp = L.nf4moe_route_permute
    need = L.nf4moe_route_workspace_bytes(16, 8, 2)
    assert need > 0
    assert rp(FAKE, 16, 8, 9, 1, FAKE, FAKE, FAKE, FAKE, FAKE, need, STREAM) == INVALID  # k > E
    assert rp(FAKE, 16, 64, 33, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, STREAM) == INVALID  # k > 32
    assert rp(FAKE, 16, 8, 2, 2, FAKE, FAKE, FAKE, FAKE, FAKE, need, STREAM) == INVALID  # renorm
    assert rp(FAKE, 16, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, STREAM) == WORKSPACE
    assert rp(FAKE, 16, 8, 2, 1, FAKE, FAKE, FAKE, FAKE, None, need, STREAM) == WORKSPACE
    assert rp(FAKE, 16, 8, 2, 1, FAKE, FAKE, None, FAKE, FAKE, need, STREAM) == INVALID
    assert L.nf4moe_route_workspace_bytes(-1, 8, 2) == 0


def test_grouped_gemm_validation():
    gg = L.nf4moe_grouped_gemm
    need = L.nf4moe_gemm_workspace_bytes(3, 8)
    args = dict(fmt=0, a=FAKE, row_of=None, a_rows=8, B=FAKE, Bs=FAKE, E=8, N=256, K=512, G=3,
                goff=FAKE, gexp=FAKE, R=8, c=FAKE, dt=0, path=0, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return gg(a["fmt"], a["a"], a["row_of"], a["a_rows"], a["B"], a["Bs"], a["E"], a["N"], a["K"],
                  a["G"], a["goff"], a["gexp"], a["R"], a["c"], a["dt"], a["path"], a["ws"], a["wsb"],
                  STREAM)
    assert call(K=500) == INVALID
    assert call(fmt=1, K=48) == INVALID
    assert call(N=0) == INVALID
    assert call(G=0) == INVALID
    assert call(R=-1) == INVALID
    assert call(a_rows=4) == INVALID          # no gather and too few rows
    assert call(row_of=FAKE, a_rows=0) == INVALID   # a gather from an empty a
    assert call(dt=5) == INVALID
    assert call(path=9) == INVALID
    assert call(goff=None) == INVALID
    assert call(a=FAKE + 2) == INVALID
    assert call(wsb=need - 1) == WORKSPACE
    assert call(path=1, K=8192, wsb=need) == UNSUPPORTED   # small-M kernels need K <= 4096


class _Layer:
    def __init__(self, **kw):
        d = dict(fmt=0, E=8, H=256, I=128, top_k=2, renormalize=1, path=0, w13=FAKE, w13_scale=FAKE,
                 w2=FAKE, w2_scale=FAKE, router_w=FAKE, router_b=None)
        d.update(kw)
        self.s = pkg.Layer(d["fmt"], d["E"], d["H"], d["I"], d["top_k"], d["renormalize"], d["path"],
                           d["w13"], d["w13_scale"], d["w2"], d["w2_scale"], d["router_w"], d["router_b"])


def _fwd(layer, T=4, ws=FAKE, wsb=1 << 40, x=FAKE, out=FAKE):
    return L.nf4moe_moe_forward(ctypes.byref(layer.s), x, T, out, None, None, ws, wsb, STREAM)


def test_forward_validation():
    assert L.nf4moe_moe_forward(None, FAKE, 4, FAKE, None, None, FAKE, 1 << 30, STREAM) == INVALID
    assert _fwd(_Layer(fmt=3)) == INVALID
    assert _fwd(_Layer(E=0)) == INVALID
    assert _fwd(_Layer(E=2000)) == INVALID
    assert _fwd(_Layer(top_k=9)) == INVALID
    assert _fwd(_Layer(E=64, top_k=33)) == INVALID
    assert _fwd(_Layer(H=100)) == INVALID
    assert _fwd(_Layer(I=96)) == INVALID                  # NF4 needs I % 64
    assert _fwd(_Layer(w13=None)) == INVALID
    assert _fwd(_Layer(w2=FAKE + 4)) == INVALID
    assert _fwd(_Layer(renormalize=3)) == INVALID
    assert _fwd(_Layer(path=7)) == INVALID
    assert _fwd(_Layer(), T=-1) == INVALID
    assert _fwd(_Layer(), T=0) == OK                      # no-op
    lay = _Layer()
    need = L.nf4moe_workspace_bytes(ctypes.byref(lay.s), 4)
    assert need > 0
    assert _fwd(lay, wsb=need - 1) == WORKSPACE
    assert _fwd(lay, ws=None) == WORKSPACE
    assert _fwd(lay, x=FAKE + 8) == INVALID               # x must be 16-byte aligned
    assert _fwd(_Layer(H=8192, path=1)) == UNSUPPORTED


def test_workspace_grows_with_tokens():
    lay = _Layer(E=64, H=2048, I=1024, top_k=8)
    a = L.nf4moe_workspace_bytes(ctypes.byref(lay.s), 1)
    b = L.nf4moe_workspace_bytes(ctypes.byref(lay.s), 4096)
    assert 0 < a < b
    # h (fp32 [R, I]) and the slot buffer (fp32 [R, H]) dominate at T = 4096
    assert b >= 4096 * 8 * (1024 + 2048) * 4


def test_cpu_tensors_are_refused():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="GPU only"):
        pkg.quantize(torch.zeros(4, 64))


def test_binding_refuses_mismatched_shapes():
    """The binding checks every tensor's shape against E, H, I, K, T before it
    passes raw pointers on (the C ABI cannot see buffer sizes); these checks run
    before the device check, so CPU tensors reach them here."""
    torch = pytest.importorskip("torch")
    f32, u8 = torch.float32, torch.uint8
    E, H, I, k = 4, 128, 64, 2

    def layer(**kw):
        d = dict(fmt=pkg.FMT_NF4, E=E, H=H, I=I, top_k=k,
                 w13=torch.zeros(E, 2 * I, H // 2, dtype=u8), w13_scale=torch.zeros(E, 2 * I, H // 64),
                 w2=torch.zeros(E, H, I // 2, dtype=u8), w2_scale=torch.zeros(E, H, I // 64),
                 router_w=torch.zeros(E, H))
        d.update(kw)
        return pkg.MoELayer(**d)

    layer().check_shapes()                                   # consistent shapes pass
    bad = [dict(w13=torch.zeros(E, 2 * I, H, dtype=u8)),     # unpacked width
           dict(w13_scale=torch.zeros(E, I, H // 64)),
           dict(w2=torch.zeros(E, I, H // 2, dtype=u8)),     # transposed down stack
           dict(w2_scale=torch.zeros(E, H, I // 32)),        # MXFP4-sized scales for NF4
           dict(router_w=torch.zeros(E + 1, H)),
           dict(router_b=torch.zeros(E - 1)),
           dict(b13=torch.zeros(E, I)), dict(b2=torch.zeros(E, I))]
    for kw in bad:
        with pytest.raises(ValueError, match="shape"):
            layer(**kw).struct()
    with pytest.raises(ValueError, match="GPU only"):        # right shapes, wrong device
        layer().struct()
    lay = layer()
    x = torch.zeros(3, H, dtype=torch.bfloat16)
    pkg.check_forward_args(lay, x, torch.zeros(3, H, dtype=torch.bfloat16),
                           torch.zeros(3, k, dtype=torch.int32), torch.zeros(3, k))
    for args in ((torch.zeros(3, H + 64, dtype=torch.bfloat16),),
                 (x, torch.zeros(2, H, dtype=torch.bfloat16)),
                 (x, None, torch.zeros(3, k + 1, dtype=torch.int32)),
                 (x, None, None, torch.zeros(k, 3))):
        with pytest.raises(ValueError, match="shape"):
            pkg.check_forward_args(lay, *args)
    B = torch.zeros(E, 256, 256, dtype=u8)
    Bs = torch.zeros(E, 256, 8)
    off = torch.zeros(3, dtype=torch.int32)
    a = torch.zeros(8, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        pkg.grouped_gemm(torch.zeros(8, 256, dtype=torch.bfloat16), B, Bs, off, 512, 8)   # a's K
    with pytest.raises(ValueError, match="shape"):
        pkg.grouped_gemm(a, B, Bs, off, 1024, 8)                                           # B's K
    with pytest.raises(ValueError, match="shape"):
        pkg.grouped_gemm(a, B, Bs, off, 512, 8, group_experts=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="shape"):
        pkg.grouped_gemm(a, B, Bs, off, 512, 8, a_row_of=torch.zeros(7, dtype=torch.int32))
    with pytest.raises(ValueError, match="fewer than R"):
        pkg.grouped_gemm(a, B, Bs, off, 512, 9)
    with pytest.raises(ValueError, match="GPU only"):
        pkg.grouped_gemm(a, B, Bs, off, 512, 8)
    with pytest.raises(ValueError, match="shape"):
        pkg.grouped_dgrad(torch.zeros(8, 128, dtype=torch.bfloat16), B, Bs, off, 512)     # dc's N
    with pytest.raises(ValueError, match="shape"):
        pkg.dequantize(B, torch.zeros(E, 256, 4), 512)
    with pytest.raises(ValueError, match="shape"):
        pkg.router_logits(x, torch.zeros(E, H + 64))


def test_mfma_peak_validation():
    assert L.nf4moe_mfma_peak_flops(2, 3) == 2 * 8 * 3 * 8 * 2 * 32 * 32 * 16
    assert L.nf4moe_mfma_peak_flops(0, 3) == 0
    assert L.nf4moe_mfma_peak_flops(2, 0) == 0
    assert L.nf4moe_mfma_peak(0, 4, FAKE, STREAM) == INVALID
    assert L.nf4moe_mfma_peak((1 << 20) + 1, 4, FAKE, STREAM) == INVALID
    assert L.nf4moe_mfma_peak(4, 0, FAKE, STREAM) == INVALID
    assert L.nf4moe_mfma_peak(4, 4, None, STREAM) == INVALID
    assert L.nf4moe_mfma_peak(4, 4, FAKE + 2, STREAM) == INVALID


def test_stream_read_validation():
    assert L.nf4moe_stream_read_sink_words(16 * 1024, 4) == 1
    assert L.nf4moe_stream_read_sink_words(16 * 1024, 1) == 4
    assert L.nf4moe_stream_read_sink_words(18, 4) == 0
    assert L.nf4moe_stream_read_sink_words(16 * 1024, 3) == 0
    assert L.nf4moe_stream_read(FAKE, 0, 4, FAKE, STREAM) == INVALID
    assert L.nf4moe_stream_read(FAKE, 24, 4, FAKE, STREAM) == INVALID
    assert L.nf4moe_stream_read(FAKE, 32, 5, FAKE, STREAM) == INVALID
    assert L.nf4moe_stream_read(FAKE + 8, 32, 4, FAKE, STREAM) == INVALID
    assert L.nf4moe_stream_read(None, 32, 4, FAKE, STREAM) == INVALID


def test_auto_path_rule():
    """AUTO's family choice, host only: the small-M kernels for at most 64 routed
    rows (NF4, both absmax storages) or 48 (MXFP4), and only while K fits their
    two 16-byte chunks per lane (K <= 4096); the MFMA kernels otherwise."""
    SMALL, MFMA = pkg.PATH_SMALL_M, pkg.PATH_MFMA
    for fmt, r_max in ((0, 64), (2, 64), (1, 48)):
        assert pkg.auto_path(fmt, 1, 2048) == SMALL
        assert pkg.auto_path(fmt, r_max, 4096) == SMALL
        assert pkg.auto_path(fmt, r_max + 1, 2048) == MFMA
        assert pkg.auto_path(fmt, 1, 4097) == MFMA
        assert pkg.auto_path(fmt, 32768, 2048) == MFMA
