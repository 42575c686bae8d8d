"""ctypes binding of libkairos.so (the C ABI of include/kairos.h)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

F32, BF16, FP8_E4M3, FP4_E2M1 = 0, 1, 2, 3
QK_BLOCKS_TOKENS, QK_BLOCKS_FRAMES = 0, 1
WINDOW_CAUSAL, WINDOW_CENTERED = 0, 1
PROLOGUE_NORMALIZE_Q, PROLOGUE_LITERAL_EQ6 = 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
# another build of this same library (the host-sanitized one the ABI tests
# load) may be named in KAIROS_LIB; there is no other fallback
lib_path = os.environ.get("KAIROS_LIB") or os.path.join(_HERE, "libkairos.so")

# every symbol include/kairos.h declares
symbols = (
    "kairos_status_string", "kairos_version", "kairos_gdn_workspace_size",
    "kairos_hlta_workspace_size", "kairos_hlta_ring_frames_required", "kairos_gdn_fwd",
    "kairos_window_fwd", "kairos_hlta_fwd", "kairos_fp8_quantize", "kairos_hlta_window_fwd",
    "kairos_gdn_prologue", "kairos_rope", "kairos_fp4_quantize", "kairos_context_create",
    "kairos_context_destroy", "kairos_gdn_fwd_noalloc", "kairos_hlta_ring_size",
    "kairos_gdn_check_gates",
)
KAIROS_ERR_RANGE = -9


class KairosError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class GdnDesc(ctypes.Structure):
    _fields_ = [("B", c_int32), ("T", c_int32), ("H", c_int32), ("dk", c_int32), ("dv", c_int32),
                ("chunk", c_int32), ("io", c_int32)]


class HltaDesc(ctypes.Structure):
    _fields_ = [("g", GdnDesc), ("L", c_int32), ("window", c_int32), ("dilation", c_int32),
                ("window_qk", c_int32), ("frame_offset", c_int64), ("ring_frames", c_int32),
                ("window_kind", c_int32), ("rope_base", c_float), ("qk_blocks", c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(f"{lib_path} is missing: build it with "
                              "`python -m video_world_model_chunkwise_amd.build`")
        L = ctypes.CDLL(lib_path)
        L.kairos_status_string.restype = c_char_p
        L.kairos_status_string.argtypes = [c_int]
        L.kairos_version.restype = c_int
        L.kairos_version.argtypes = []
        L.kairos_gdn_workspace_size.argtypes = [POINTER(GdnDesc), POINTER(c_size_t)]
        L.kairos_hlta_workspace_size.argtypes = [POINTER(HltaDesc), POINTER(c_size_t)]
        L.kairos_hlta_ring_frames_required.argtypes = [POINTER(HltaDesc), POINTER(c_int32)]
        L.kairos_hlta_ring_size.argtypes = [POINTER(HltaDesc), POINTER(c_size_t), POINTER(c_size_t)]
        L.kairos_gdn_fwd.argtypes = [POINTER(GdnDesc)] + [c_void_p] * 8 + [c_void_p, c_size_t, c_void_p]
        L.kairos_gdn_fwd_noalloc.argtypes = [POINTER(GdnDesc)] + [c_void_p] * 8 + [c_void_p]
        L.kairos_window_fwd.argtypes = [POINTER(HltaDesc), c_int32] + [c_void_p] * 9
        L.kairos_hlta_fwd.argtypes = [POINTER(HltaDesc)] + [c_void_p] * 11 + [c_void_p, c_size_t, c_void_p,
                                                                             c_void_p]
        L.kairos_context_create.argtypes = [POINTER(c_void_p)]
        L.kairos_context_destroy.argtypes = [c_void_p]
        L.kairos_hlta_window_fwd.argtypes = [POINTER(HltaDesc)] + [c_void_p] * 11 + [c_size_t, c_void_p]
        L.kairos_gdn_prologue.argtypes = [POINTER(GdnDesc), c_int32] + [c_void_p] * 11
        L.kairos_rope.argtypes = [POINTER(HltaDesc), c_int32] + [c_void_p] * 4
        L.kairos_fp8_quantize.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                          c_int32, c_void_p]
        L.kairos_fp4_quantize.argtypes = L.kairos_fp8_quantize.argtypes
        L.kairos_gdn_check_gates.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_float,
                                             c_void_p, c_void_p]
        for name in symbols:
            getattr(L, name).restype = c_int if name != "kairos_status_string" else c_char_p
        _lib = L
    return _lib


class Context:
    """A kairos_context of the current device (side stream and events of the
    layer call), destroyed with close() or when garbage-collected."""

    def __init__(self):
        h = c_void_p()
        _check(lib().kairos_context_create(byref(h)), "kairos_context_create")
        self.handle = h

    def close(self):
        if self.handle is not None and self.handle.value:
            _check(lib().kairos_context_destroy(self.handle), "kairos_context_destroy")
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def status_string(status: int) -> str:
    return lib().kairos_status_string(int(status)).decode()


def version() -> int:
    return lib().kairos_version()


def _check(status: int, where: str):
    if status != 0:
        raise KairosError(status, where)


def gdn_desc(B, T, H, d, io=BF16, chunk=64) -> GdnDesc:
    return GdnDesc(B, T, H, d, d, chunk, io)


def hlta_desc(B, T, H, d, L, window, dilation, frame_offset=0, ring_frames=0,
              window_qk=BF16, io=BF16, centered=False, rope_base=0.0,
              qk_blocks=QK_BLOCKS_TOKENS) -> HltaDesc:
    return HltaDesc(gdn_desc(B, T, H, d, io), L, window, dilation, window_qk, frame_offset,
                    ring_frames, WINDOW_CENTERED if centered else WINDOW_CAUSAL, rope_base, qk_blocks)


# ------------------------------------------------------------------ torch marshalling

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return c_void_p(stream)
    return c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _need(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def kairos_gdn_workspace_size(desc: GdnDesc) -> int:
    n = c_size_t(0)
    _check(lib().kairos_gdn_workspace_size(byref(desc), byref(n)), "kairos_gdn_workspace_size")
    return n.value


def kairos_hlta_workspace_size(desc: HltaDesc) -> int:
    n = c_size_t(0)
    _check(lib().kairos_hlta_workspace_size(byref(desc), byref(n)), "kairos_hlta_workspace_size")
    return n.value


def kairos_hlta_ring_size(desc: HltaDesc):
    """(key ring bytes, value ring bytes) of a streamed layer call."""
    kb, vb = c_size_t(0), c_size_t(0)
    _check(lib().kairos_hlta_ring_size(byref(desc), byref(kb), byref(vb)), "kairos_hlta_ring_size")
    return kb.value, vb.value


def kairos_hlta_ring_frames_required(desc: HltaDesc) -> int:
    n = c_int32(0)
    _check(lib().kairos_hlta_ring_frames_required(byref(desc), byref(n)),
           "kairos_hlta_ring_frames_required")
    return n.value


def _debug() -> bool:
    """KAIROS_DEBUG set (and not 0): the GDN and layer calls first check
    their gates with kairos_gdn_check_gates (synchronising) and raise
    KairosError(KAIROS_ERR_RANGE) if any is out of range."""
    return os.environ.get("KAIROS_DEBUG", "0") not in ("", "0")


def kairos_gdn_check_gates(alpha, beta, beta_max=1.0, count=None, stream=None) -> int:
    """Number of (b, t, h) with alpha [B, T, H] outside (0, 1] or beta outside
    [0, beta_max] (NaN counts as outside).  Synchronises the stream to read
    the count; `count` (one int32 on the device) is allocated when not given."""
    torch = _torch()
    B, T, H = alpha.shape
    dev = alpha.device
    _need(alpha, "alpha", torch.float32, (B, T, H), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=dev)
    st = lib().kairos_gdn_check_gates(_ptr(alpha), _ptr(beta), B, T, H, c_float(beta_max), _ptr(count),
                                      _stream(stream))
    _check(st, "kairos_gdn_check_gates")
    if stream is None or isinstance(stream, int):
        torch.cuda.synchronize(dev)
    else:
        stream.synchronize()
    return int(count.item()) & 0xFFFFFFFF


def _debug_gates(alpha, beta, stream, where):
    n = kairos_gdn_check_gates(alpha, beta, stream=stream)
    if n:
        raise KairosError(KAIROS_ERR_RANGE, f"{where} ({n} of {alpha.numel()} gate pairs outside alpha in (0, 1], "
                                            "beta in [0, 1]; KAIROS_DEBUG)")


def _workspace(nbytes, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kairos_gdn_fwd(q, k, v, alpha, beta, state_in=None, out=None, state_out=None,
                   keep_state=True, stream=None, workspace=None):
    """Gated delta rule forward.  q, k, v: [B, T, H, d] (bf16 or fp32, same
    dtype); alpha, beta: [B, T, H] fp32; state_in: [B, H, d, d] fp32 or None.
    Returns (out, state_out); state_out is None when keep_state is False."""
    torch = _torch()
    B, T, H, d = q.shape
    dev = q.device
    io = F32 if q.dtype == torch.float32 else BF16
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype, (B, T, H, d), dev)
    _need(alpha, "alpha", torch.float32, (B, T, H), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, d, d), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, (B, T, H, d), dev)
    if state_out is None and keep_state:
        state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (B, H, d, d), dev)
    desc = gdn_desc(B, T, H, d, io)
    nws = kairos_gdn_workspace_size(desc)
    if _debug():
        _debug_gates(alpha, beta, stream, "kairos_gdn_fwd")
    ws = workspace if workspace is not None else _workspace(nws, dev)
    st = lib().kairos_gdn_fwd(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                              _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(ws), nws,
                              _stream(stream))
    _check(st, "kairos_gdn_fwd")
    return out, state_out


def kairos_gdn_fwd_noalloc(q, k, v, alpha, beta, state_in=None, out=None, state_out=None,
                           stream=None):
    """kairos_gdn_fwd with the library's own per-device scratch array as the
    workspace (nothing is allocated for it).  out and state_out must be given
    (the point of the call is that nothing is allocated); returns them."""
    torch = _torch()
    B, T, H, d = q.shape
    dev = q.device
    io = F32 if q.dtype == torch.float32 else BF16
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _need(t, name, q.dtype, (B, T, H, d), dev)
    _need(alpha, "alpha", torch.float32, (B, T, H), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, d, d), dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (B, H, d, d), dev)
    desc = gdn_desc(B, T, H, d, io)
    st = lib().kairos_gdn_fwd_noalloc(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                      _ptr(beta), _ptr(state_in), _ptr(out), _ptr(state_out),
                                      _stream(stream))
    _check(st, "kairos_gdn_fwd_noalloc")
    return out, state_out


def kairos_fp4_quantize(x, codes=None, scales=None, stream=None):
    """Per-(b, h, 64-token block) 4-bit (E2M1) quantisation of x [B, T, H, d]
    bf16.  Returns (codes uint8 [B, T, H, d/2] (two per byte, even feature in
    the low nibble), scales fp32 [B, H, ceil(T/64)])."""
    torch = _torch()
    B, T, H, d = x.shape
    _need(x, "x", torch.bfloat16, (B, T, H, d), x.device)
    if codes is None:
        codes = torch.empty((B, T, H, d // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, (T + 63) // 64), dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8, (B, T, H, d // 2), x.device)
    _need(scales, "scales", torch.float32, (B, H, (T + 63) // 64), x.device)
    st = lib().kairos_fp4_quantize(_ptr(x), _ptr(codes), _ptr(scales), B, T, H, d, _stream(stream))
    _check(st, "kairos_fp4_quantize")
    return codes, scales


def kairos_fp8_quantize(x, codes=None, scales=None, stream=None):
    """Per-(b, h, 64-token block) E4M3 quantisation of x [B, T, H, d] bf16.
    Returns (codes uint8 [B, T, H, d], scales fp32 [B, H, ceil(T/64)])."""
    torch = _torch()
    B, T, H, d = x.shape
    _need(x, "x", torch.bfloat16, (B, T, H, d), x.device)
    if codes is None:
        codes = torch.empty((B, T, H, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, (T + 63) // 64), dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8, (B, T, H, d), x.device)
    _need(scales, "scales", torch.float32, (B, H, (T + 63) // 64), x.device)
    st = lib().kairos_fp8_quantize(_ptr(x), _ptr(codes), _ptr(scales), B, T, H, d, _stream(stream))
    _check(st, "kairos_fp8_quantize")
    return codes, scales


def _qk_format(q, d, window_qk):
    """Windowed-operand format from the tensor: bf16, E4M3 codes [.., d] or
    E2M1 codes [.., d/2] (uint8; window_qk picks between the byte formats when
    the shape does not)."""
    torch = _torch()
    if q.dtype != torch.uint8:
        return BF16
    if window_qk is not None:
        return window_qk
    return FP4_E2M1 if q.shape[-1] * 2 == d else FP8_E4M3


def _qk_shape(B, T, H, d, fmt):
    return (B, T, H, d // 2 if fmt == FP4_E2M1 else d)


def kairos_window_fwd(q, k, v, L, window, dilation, frame_offset=0, ring_frames=0,
                      k_ring=None, v_ring=None, q_scales=None, k_scales=None, out=None,
                      stream=None, centered=False, window_qk=None):
    """One windowed branch (SWA if dilation == 1, else DSWA), causal or
    centred.  q, k bf16, or uint8 codes with q_scales/k_scales (E4M3
    [B, T, H, 128], or E2M1 [B, T, H, 64]); v bf16 [B, T, H, 128]."""
    torch = _torch()
    B, T, H, d = v.shape
    dev = v.device
    fmt = _qk_format(q, d, window_qk)
    fp8 = fmt != BF16
    qk_dtype = torch.uint8 if fp8 else torch.bfloat16
    _need(q, "q", qk_dtype, _qk_shape(B, T, H, d, fmt), dev)
    _need(k, "k", qk_dtype, _qk_shape(B, T, H, d, fmt), dev)
    _need(v, "v", torch.bfloat16, (B, T, H, d), dev)
    if fp8:
        nb = (T + 63) // 64
        _need(q_scales, "q_scales", torch.float32, (B, H, nb), dev)
        _need(k_scales, "k_scales", torch.float32, (B, H, nb), dev)
    if ring_frames:
        _need(k_ring, "k_ring", torch.bfloat16, (B, ring_frames, L, H, d), dev)
        _need(v_ring, "v_ring", torch.bfloat16, (B, ring_frames, L, H, d), dev)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, H, d), dev)
    desc = hlta_desc(B, T, H, d, L, window, dilation, frame_offset, ring_frames, fmt,
                     centered=centered)
    st = lib().kairos_window_fwd(byref(desc), dilation, _ptr(q), _ptr(k), _ptr(v), _ptr(q_scales),
                                 _ptr(k_scales), _ptr(k_ring), _ptr(v_ring), _ptr(out),
                                 _stream(stream))
    _check(st, "kairos_window_fwd")
    return out


def kairos_hlta_fwd(q, k, v, alpha, beta, gate_logits, L, window, dilation, frame_offset=0,
                    state_in=None, ring_frames=0, k_ring=None, v_ring=None, window_qk=BF16,
                    out=None, state_out=None, keep_state=True, workspace=None, stream=None,
                    centered=False, rope_base=0.0, ctx=None, qk_blocks=QK_BLOCKS_TOKENS):
    """Hybrid layer forward.  q, k, v: [B, T, H, 128] bf16; alpha, beta
    [B, T, H] fp32; gate_logits [3, H] fp32; ctx an optional Context (its
    side stream runs part of the call).  Returns (out, state_out)."""
    torch = _torch()
    B, T, H, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, (B, T, H, d), dev)
    _need(alpha, "alpha", torch.float32, (B, T, H), dev)
    _need(beta, "beta", torch.float32, (B, T, H), dev)
    _need(gate_logits, "gate_logits", torch.float32, (3, H), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, d, d), dev)
    desc = hlta_desc(B, T, H, d, L, window, dilation, frame_offset, ring_frames, window_qk,
                     centered=centered, rope_base=rope_base, qk_blocks=qk_blocks)
    if ring_frames:
        kb, vb = kairos_hlta_ring_size(desc)
        for name, t, nb in (("k_ring", k_ring, kb), ("v_ring", v_ring, vb)):
            if t is None or not t.is_contiguous() or t.device != dev:
                raise ValueError(f"{name} must be a contiguous tensor on {dev}")
            if t.numel() * t.element_size() != nb:
                raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, expected {nb} "
                                 "(kairos_hlta_ring_size)")
    if out is None:
        out = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, H, d), dev)
    if state_out is None and keep_state:
        state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = kairos_hlta_workspace_size(desc)
    if _debug():
        _debug_gates(alpha, beta, stream, "kairos_hlta_fwd")
    ws = workspace if workspace is not None else _workspace(nws, dev)
    if ws is not None and ws.numel() < nws:
        raise ValueError(f"workspace too small: {ws.numel()} < {nws}")
    st = lib().kairos_hlta_fwd(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                               _ptr(gate_logits), _ptr(state_in), _ptr(k_ring), _ptr(v_ring),
                               _ptr(out), _ptr(state_out), _ptr(ws), nws,
                               None if ctx is None else ctx.handle, _stream(stream))
    _check(st, "kairos_hlta_fwd")
    return out, state_out


def ring_key_shape(B, R, L, H, d, dilation, rope_base=0.0):
    """Shape of a bf16 layer call's key ring: with RoPE and dilation > 1 it
    keeps both windowed branches' rotated keys, [2, B, R, L, H, d]."""
    return (2, B, R, L, H, d) if rope_base > 0 and dilation > 1 else (B, R, L, H, d)


def alloc_rings(B, L, H, d, window, dilation, ring_frames, window_qk=BF16, rope_base=0.0,
                qk_blocks=QK_BLOCKS_TOKENS, device="cuda:0"):
    """Zeroed key and value rings of a streamed layer call (the key ring as
    bytes, sized by kairos_hlta_ring_size)."""
    torch = _torch()
    desc = hlta_desc(B, L, H, d, L, window, dilation, 0, ring_frames, window_qk,
                     rope_base=rope_base, qk_blocks=qk_blocks)
    kb, vb = kairos_hlta_ring_size(desc)
    k_ring = torch.zeros(kb, dtype=torch.uint8, device=device)
    v_ring = torch.zeros((B, ring_frames, L, H, d), dtype=torch.bfloat16, device=device)
    assert v_ring.numel() * 2 == vb
    return k_ring, v_ring


def kairos_hlta_window_fwd(q, k, v, o_gdn, gate_logits, L, window, dilation, frame_offset=0,
                           ring_frames=0, k_ring=None, v_ring=None, q_scales=None, k_scales=None,
                           out=None, workspace=None, stream=None, centered=False, window_qk=None):
    """Windowed stage of the hybrid layer: SWA + DSWA + gated combination with
    o_gdn.  q, k bf16 or uint8 codes (E4M3 or E2M1, with scales); v, o_gdn bf16."""
    torch = _torch()
    B, T, H, d = v.shape
    dev = v.device
    fmt = _qk_format(q, d, window_qk)
    fp8 = fmt != BF16
    qk_dtype = torch.uint8 if fp8 else torch.bfloat16
    _need(q, "q", qk_dtype, _qk_shape(B, T, H, d, fmt), dev)
    _need(k, "k", qk_dtype, _qk_shape(B, T, H, d, fmt), dev)
    _need(v, "v", torch.bfloat16, (B, T, H, d), dev)
    _need(o_gdn, "o_gdn", torch.bfloat16, (B, T, H, d), dev)
    _need(gate_logits, "gate_logits", torch.float32, (3, H), dev)
    if fp8:
        nb = (T + 63) // 64
        _need(q_scales, "q_scales", torch.float32, (B, H, nb), dev)
        _need(k_scales, "k_scales", torch.float32, (B, H, nb), dev)
    if ring_frames:
        _need(k_ring, "k_ring", torch.bfloat16, (B, ring_frames, L, H, d), dev)
        _need(v_ring, "v_ring", torch.bfloat16, (B, ring_frames, L, H, d), dev)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, H, d), dev)
    desc = hlta_desc(B, T, H, d, L, window, dilation, frame_offset, ring_frames, fmt,
                     centered=centered)
    nws = 4 * B * T * H * (d + 1)
    ws = workspace if workspace is not None else _workspace(nws, dev)
    if ws.numel() < nws:
        raise ValueError(f"workspace too small: {ws.numel()} < {nws}")
    st = lib().kairos_hlta_window_fwd(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scales),
                                      _ptr(k_scales), _ptr(o_gdn), _ptr(gate_logits), _ptr(k_ring),
                                      _ptr(v_ring), _ptr(out), _ptr(ws), nws, _stream(stream))
    _check(st, "kairos_hlta_window_fwd")
    return out


def kairos_gdn_prologue(k, alpha_logits, beta_logits, q=None, v=None, literal=False,
                        k_out=None, alpha_out=None, beta_out=None, q_out=None, v_out=None,
                        stream=None):
    """Inputs of the gated delta rule from raw keys and gate logits.  k (and q
    when given) [B, T, H, d] bf16 or fp32 are L2-normalised per row;
    alpha = sigmoid(alpha_logits), beta = sigmoid(beta_logits) ([B, T, H]
    fp32).  literal=True (needs v) returns beta / alpha and alpha * v instead,
    the inputs under which the canonical recurrence is Eq. 6 as printed.
    Outputs may be passed in, also as the inputs themselves (in place).
    Returns (k_out, alpha_out, beta_out, q_out or None, v_out or None)."""
    torch = _torch()
    B, T, H, d = k.shape
    dev = k.device
    io = F32 if k.dtype == torch.float32 else BF16
    _need(k, "k", k.dtype, (B, T, H, d), dev)
    _need(alpha_logits, "alpha_logits", torch.float32, (B, T, H), dev)
    _need(beta_logits, "beta_logits", torch.float32, (B, T, H), dev)
    if q is not None:
        _need(q, "q", k.dtype, (B, T, H, d), dev)
    if literal:
        _need(v, "v", k.dtype, (B, T, H, d), dev)
    elif v is not None or v_out is not None:
        raise ValueError("v is rescaled only in the literal form")
    if q is None and q_out is not None:
        raise ValueError("q_out given without q")
    k_out = torch.empty_like(k) if k_out is None else k_out
    alpha_out = torch.empty_like(alpha_logits) if alpha_out is None else alpha_out
    beta_out = torch.empty_like(beta_logits) if beta_out is None else beta_out
    _need(k_out, "k_out", k.dtype, (B, T, H, d), dev)
    _need(alpha_out, "alpha_out", torch.float32, (B, T, H), dev)
    _need(beta_out, "beta_out", torch.float32, (B, T, H), dev)
    if q is not None:
        q_out = torch.empty_like(q) if q_out is None else q_out
        _need(q_out, "q_out", k.dtype, (B, T, H, d), dev)
    if literal:
        v_out = torch.empty_like(v) if v_out is None else v_out
        _need(v_out, "v_out", k.dtype, (B, T, H, d), dev)
    flags = (PROLOGUE_NORMALIZE_Q if q is not None else 0) | (PROLOGUE_LITERAL_EQ6 if literal else 0)
    desc = gdn_desc(B, T, H, d, io)
    st = lib().kairos_gdn_prologue(byref(desc), flags, _ptr(k), _ptr(alpha_logits),
                                   _ptr(beta_logits), _ptr(q), _ptr(v if literal else None),
                                   _ptr(k_out), _ptr(alpha_out), _ptr(beta_out), _ptr(q_out),
                                   _ptr(v_out), _stream(stream))
    _check(st, "kairos_gdn_prologue")
    return k_out, alpha_out, beta_out, q_out, v_out


def kairos_rope(x, L, dilation, rope_base, frame_offset=0, fp8=False, out=None, scales=None,
                stream=None, window_qk=None):
    """RoPE of one windowed branch's q or k (bf16 [B, T, H, 128]) at the
    positions of the branch with this dilation (1: SWA).  Returns the rotated
    bf16 tensor, or with fp8=True (window_qk=FP4_E2M1: 4-bit) (codes, scales)
    of the rotated values.  out may be x itself for bf16 (in place)."""
    torch = _torch()
    B, T, H, d = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (B, T, H, d), dev)
    fmt = window_qk if window_qk is not None else (FP8_E4M3 if fp8 else BF16)
    fp8 = fmt != BF16
    if fp8:
        shape = _qk_shape(B, T, H, d, fmt)
        out = torch.empty(shape, dtype=torch.uint8, device=dev) if out is None else out
        nb = (T + 63) // 64
        scales = torch.empty((B, H, nb), dtype=torch.float32, device=dev) if scales is None else scales
        _need(out, "out", torch.uint8, shape, dev)
        _need(scales, "scales", torch.float32, (B, H, nb), dev)
    else:
        out = torch.empty_like(x) if out is None else out
        _need(out, "out", torch.bfloat16, (B, T, H, d), dev)
    desc = hlta_desc(B, T, H, d, L, 1, 1, frame_offset, 0, fmt, rope_base=rope_base)
    st = lib().kairos_rope(byref(desc), dilation, _ptr(x), _ptr(out), _ptr(scales if fp8 else None),
                           _stream(stream))
    _check(st, "kairos_rope")
    return (out, scales) if fp8 else out
