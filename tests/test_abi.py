"""The C ABI on the host, without a GPU: the library loads, exports every
symbol include/kairos.h declares, sizes workspaces, and rejects invalid calls
with the documented status before anything is enqueued (only validation
paths are exercised here; no pointer passed below is ever dereferenced)."""
import ctypes
import os
import re

import pytest

import video_world_model_chunkwise_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, UNSUP, WS = 0, -1, -2, -3, -4, -5, -6, -7

pytestmark = pytest.mark.skipif(not os.path.exists(K.lib_path), reason="libkairos.so not built")


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0      # counts devices without initialising them


# The calls below pass fake addresses and rely on being rejected before any
# launch; they never run where a GPU is visible, so a regression in a check
# cannot turn into a launch with fake pointers.
host_only = pytest.mark.skipif(_gpu_visible(), reason="host-only validation tests")


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "kairos.h")).read()
    declared = set(re.findall(r"^\s*(?:int|const char\*)\s+(kairos_\w+)\s*\(", header, re.M))
    assert declared == set(K.symbols)
    lib = ctypes.CDLL(K.lib_path)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    assert K.version() == 202
    assert K.status_string(0) == "ok"
    assert "align" in K.status_string(ALIGN)
    assert K.status_string(12345) == "unknown status"


def _writable_symbols():
    """Demangled names of the library's own writable data symbols (.data/.bss),
    from nm; kernel launch handles (names with a parameter list) excluded."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-C", "--defined-only", K.lib_path], check=True, capture_output=True,
                         text=True).stdout
    names = []
    for line in out.splitlines():
        parts = line.split(maxsplit=2)
        if len(parts) == 3 and parts[1] in "bBdD" and "(" not in parts[2]:
            if parts[2].startswith(("kairos", "(anonymous namespace)")):
                names.append(parts[2])
    return names


# the only file-scope state: the per-device device addresses of the no-alloc
# entry point's scratch array (resolved once per device)
ALLOWED_STATE = {"kairos::scratch", "kairos::noalloc_scratch_ptr", "kairos::noalloc_scratch_mu"}


def test_no_global_state():
    """The library keeps no process-wide mutable state of its own: the layer
    call's side stream and events live in a caller-created kairos_context."""
    names = _writable_symbols()
    assert set(names) <= ALLOWED_STATE, names


@host_only
def test_gdn_noalloc_validation():
    """The no-alloc entry point checks like kairos_gdn_fwd and refuses
    problems whose workspace exceeds its 64 MiB array, before touching the
    device."""
    L = K.lib()
    cv = ctypes.c_void_p
    args = lambda: [cv(1 * G), cv(2 * G), cv(3 * G), cv(4 * G), cv(5 * G), None, cv(6 * G), None, None]
    big = K.gdn_desc(4, 57600, 24, 128)
    assert K.kairos_gdn_workspace_size(big) > 64 << 20
    assert L.kairos_gdn_fwd_noalloc(ctypes.byref(big), *args()) == WS
    d = K.gdn_desc(1, 64, 2, 128)
    a = args()
    a[6] = None                                            # out
    assert L.kairos_gdn_fwd_noalloc(ctypes.byref(d), *a) == NULL
    a = args()
    a[6] = cv(1 * G + 64)                                  # out overlaps q
    assert L.kairos_gdn_fwd_noalloc(ctypes.byref(d), *a) == ALIAS


@host_only
def test_context_arguments():
    L = K.lib()
    assert L.kairos_context_create(None) == NULL
    assert L.kairos_context_destroy(None) == OK
    h = ctypes.c_void_p(1234)
    st = L.kairos_context_create(ctypes.byref(h))     # no device here: the runtime refuses
    assert st == -8 and not h.value


def test_workspace_sizes():
    d = K.gdn_desc(4, 57600, 24, 128)
    nchunks = 900
    expect = ((4 * 24 * nchunks * 64 * 64 * 2 + 255) // 256) * 256 + 4 * 24 * nchunks * 64 * 4
    assert K.kairos_gdn_workspace_size(d) == expect
    assert K.kairos_gdn_workspace_size(K.gdn_desc(1, 64, 2, 32, io=K.F32)) == 0
    h = K.hlta_desc(4, 57600, 24, 128, 3600, 3600, 4, window_qk=K.FP8_E4M3)
    n = 4 * 57600 * 24 * 128
    assert K.kairos_hlta_workspace_size(h) >= expect + 2 * n + 4 * n + 2 * n
    assert K.kairos_hlta_ring_frames_required(K.hlta_desc(1, 1560, 24, 128, 1560, 1560, 4)) == 4
    assert K.kairos_hlta_ring_frames_required(K.hlta_desc(1, 1560, 24, 128, 1560, 1561, 4)) == 4
    assert K.kairos_hlta_ring_frames_required(K.hlta_desc(1, 1560, 24, 128, 1560, 1562, 4)) == 8
    assert K.kairos_hlta_ring_frames_required(K.hlta_desc(1, 1560, 24, 128, 1560, 1, 4)) == 0


@pytest.mark.parametrize("desc,status", [
    (K.gdn_desc(0, 64, 2, 128), SHAPE),
    (K.gdn_desc(1, -1, 2, 128), SHAPE),
    (K.gdn_desc(1, 64, 2, 96), SHAPE),
    (K.GdnDesc(1, 64, 2, 128, 64, 64, K.BF16), SHAPE),
    (K.gdn_desc(1, 64, 2, 128, chunk=32), SHAPE),
    (K.gdn_desc(1, 64, 2, 128, io=7), DTYPE),
    (K.gdn_desc(1, 64, 2, 32, io=K.BF16), UNSUP),
])
@host_only
def test_gdn_descriptor_errors(desc, status):
    n = ctypes.c_size_t(0)
    assert K.lib().kairos_gdn_workspace_size(ctypes.byref(desc), ctypes.byref(n)) == status
    rc = K.lib().kairos_gdn_fwd(ctypes.byref(desc), *([None] * 8), None, 0, None)
    assert rc == status


def _gdn_call(desc, q=0x10000, k=0x20000, v=0x30000, a=0x40000, b=0x50000, s_in=None,
              out=0x60000, s_out=None, ws=None, nws=0):
    L = K.lib()
    cv = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kairos_gdn_fwd(ctypes.byref(desc), cv(q), cv(k), cv(v), cv(a), cv(b), cv(s_in),
                            cv(out), cv(s_out), cv(ws), nws, None)


@host_only
def test_gdn_pointer_errors():
    d = K.gdn_desc(1, 64, 2, 128, io=K.F32)          # fp32: no workspace needed
    assert _gdn_call(d, q=None) == NULL
    assert _gdn_call(d, out=None) == NULL
    assert _gdn_call(d, q=0x10008) == ALIGN           # not 16-byte aligned
    assert _gdn_call(d, a=0x40002) == ALIGN           # not 4-byte aligned
    nx = 64 * 2 * 128 * 4
    assert _gdn_call(d, out=0x10000 + nx // 2) == ALIAS          # out overlaps q
    assert _gdn_call(d, s_in=0x90000, s_out=0x90000 + 16) == ALIAS  # partial state overlap
    # the chunk kernels' 32-bit row offsets: 63 * H * d * 2 + d * 2 < 2^32
    assert K.kairos_gdn_workspace_size(K.gdn_desc(1, 64, 266304, 128)) > 0
    with pytest.raises(K.KairosError) as e:
        K.kairos_gdn_workspace_size(K.gdn_desc(1, 64, 266305, 128))
    assert e.value.status == SHAPE
    db = K.gdn_desc(1, 64, 2, 128)
    assert _gdn_call(db) == WS                        # bf16 needs a workspace
    need = K.kairos_gdn_workspace_size(db)
    assert _gdn_call(db, ws=0x100040, nws=need) == ALIGN        # workspace not 256-aligned
    assert _gdn_call(db, ws=0x100000, nws=need - 1) == WS


G = 1 << 36          # fake, never dereferenced, far-apart addresses


def _hlta_call(desc, ws=None, nws=0, gates=6 * G, k_ring=None, v_ring=None, out=7 * G):
    L = K.lib()
    cv = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kairos_hlta_fwd(ctypes.byref(desc), cv(1 * G), cv(2 * G), cv(3 * G),
                             cv(4 * G), cv(5 * G), cv(gates), None, cv(k_ring), cv(v_ring),
                             cv(out), None, cv(ws), nws, None, None)


@host_only
def test_hlta_validation():
    base = dict(B=1, T=4 * 1560, H=2, d=128, L=1560, window=1560, dilation=4)
    d = K.hlta_desc(**base)
    assert _hlta_call(d) == WS
    assert _hlta_call(d, gates=None) == NULL
    assert _hlta_call(K.hlta_desc(**{**base, "d": 64})) == UNSUP
    assert _hlta_call(K.hlta_desc(**base, io=K.F32)) == DTYPE
    assert _hlta_call(K.hlta_desc(**{**base, "window": 0})) == SHAPE
    assert _hlta_call(K.hlta_desc(**{**base, "H": 65537})) == SHAPE
    assert _hlta_call(K.hlta_desc(**{**base, "dilation": 0})) == SHAPE
    assert _hlta_call(K.hlta_desc(**base, frame_offset=-1)) == SHAPE
    # a ring needs whole frames and enough of them, and no fp8
    assert _hlta_call(K.hlta_desc(**{**base, "T": 1560 + 7}, ring_frames=4)) == SHAPE
    assert _hlta_call(K.hlta_desc(**base, ring_frames=3)) == SHAPE
    assert _hlta_call(K.hlta_desc(**base, ring_frames=4)) == NULL          # ring pointers missing
    assert _hlta_call(K.hlta_desc(**base, ring_frames=4, window_qk=K.FP8_E4M3)) == UNSUP
    # quantised Q/K with a ring need quantisation blocks that restart at every frame
    assert _hlta_call(K.hlta_desc(**base, ring_frames=4, window_qk=K.FP8_E4M3,
                                  qk_blocks=K.QK_BLOCKS_FRAMES)) == NULL
    assert _hlta_call(K.hlta_desc(**base, ring_frames=4, window_qk=K.FP4_E2M1,
                                  qk_blocks=K.QK_BLOCKS_FRAMES), k_ring=8 * G, v_ring=9 * G) == WS
    d2 = K.hlta_desc(**base)
    d2.window_kind = 2
    assert _hlta_call(d2) == SHAPE
    # RoPE: base must be finite and >= 0; qk_blocks must be 0 or 1
    assert _hlta_call(K.hlta_desc(**base, rope_base=-1.0)) == SHAPE
    assert _hlta_call(K.hlta_desc(**base, rope_base=float("nan"))) == SHAPE
    assert _hlta_call(K.hlta_desc(**base, rope_base=float("inf"))) == SHAPE
    # RoPE with a ring: accepted (the ring keeps the rotated keys); here the
    # ring pointers are missing, then the workspace
    assert _hlta_call(K.hlta_desc(**base, ring_frames=4, rope_base=1e4)) == NULL
    assert _hlta_call(K.hlta_desc(**base, ring_frames=4, rope_base=1e4), k_ring=8 * G,
                      v_ring=9 * G) == WS
    assert _hlta_call(K.hlta_desc(**base, rope_base=1e4)) == WS
    d3 = K.hlta_desc(**base)
    d3.qk_blocks = 2
    assert _hlta_call(d3) == SHAPE
    # a centred window sees later frames: no ring
    assert _hlta_call(K.hlta_desc(**base, ring_frames=4, centered=True)) == UNSUP
    assert _hlta_call(K.hlta_desc(**base, centered=True)) == WS       # otherwise valid
    nws = K.kairos_hlta_workspace_size(d)
    assert _hlta_call(d, ws=8 * G, nws=nws - 256) == WS
    # workspace overlapping the output
    assert _hlta_call(d, ws=7 * G, nws=nws) == ALIAS


@host_only
def test_window_and_quantiser_validation():
    L = K.lib()
    d = K.hlta_desc(1, 1000, 2, 128, 100, 150, 2)
    cv = ctypes.c_void_p
    assert L.kairos_window_fwd(ctypes.byref(d), 0, cv(0x1000), cv(0x2000), cv(0x3000), None, None,
                               None, None, cv(0x4000), None) == SHAPE
    # bf16 windows take no scales
    assert L.kairos_window_fwd(ctypes.byref(d), 2, cv(0x1000), cv(0x2000), cv(0x3000), cv(0x5000),
                               None, None, None, cv(0x4000), None) == UNSUP
    d8 = K.hlta_desc(1, 1000, 2, 128, 100, 150, 2, window_qk=K.FP8_E4M3)
    assert L.kairos_window_fwd(ctypes.byref(d8), 2, cv(0x1000), cv(0x2000), cv(0x3000), None, None,
                               None, None, cv(0x4000), None) == NULL
    assert L.kairos_hlta_window_fwd(ctypes.byref(d), cv(0x100000), cv(0x200000), cv(0x300000), None,
                                    None, cv(0x400000), cv(0x500), None, None, cv(0x600000), None, 0,
                                    None) == WS
    assert L.kairos_fp8_quantize(cv(0x1000), cv(0x2000), cv(0x3000), 1, 64, 2, 96, None) == SHAPE
    assert L.kairos_fp8_quantize(None, cv(0x2000), cv(0x3000), 1, 64, 2, 128, None) == NULL
    assert L.kairos_fp8_quantize(cv(0x1008), cv(0x2000), cv(0x3000), 1, 64, 2, 128, None) == ALIGN
    assert L.kairos_fp8_quantize(cv(0x1000), cv(0x1000), cv(0x9000000), 1, 64, 2, 128, None) == ALIAS
    assert L.kairos_fp8_quantize(None, None, None, 1, 0, 2, 128, None) == OK   # empty: nothing to do


@host_only
def test_gate_check_validation():
    L = K.lib()
    cv, f = ctypes.c_void_p, ctypes.c_float
    a, b, c = 0x10000, 0x20000, 0x30000
    n4 = 2 * 100 * 3 * 4
    call = lambda a_=a, b_=b, B=2, T=100, H=3, bmax=1.0, c_=c: L.kairos_gdn_check_gates(
        cv(a_) if a_ else None, cv(b_) if b_ else None, B, T, H, f(bmax), cv(c_) if c_ else None, None)
    assert call(c_=0) == NULL
    assert call(a_=0) == NULL and call(b_=0) == NULL
    assert call(B=0) == SHAPE and call(H=0) == SHAPE and call(T=-1) == SHAPE
    assert call(B=1 << 20, T=1 << 20, H=2) == SHAPE                  # more than 2^40 gate pairs
    assert call(bmax=-1.0) == SHAPE and call(bmax=float("nan")) == SHAPE
    assert call(a_=a + 8) == ALIGN and call(c_=c + 2) == ALIGN
    assert call(c_=a + 16) == ALIAS and call(c_=b + n4 - 4) == ALIAS
    assert K.status_string(K.KAIROS_ERR_RANGE) == "input values out of range"


@host_only
def test_prologue_validation():
    L = K.lib()
    cv = lambda x: None if x is None else ctypes.c_void_p(x)
    d = K.gdn_desc(2, 100, 3, 128)
    nx = 2 * 100 * 3 * 128 * 2

    def call(flags=0, k=1 * G, za=2 * G, zb=3 * G, q=None, v=None, ko=4 * G, ao=5 * G, bo=6 * G,
             qo=None, vo=None, desc=d):
        return L.kairos_gdn_prologue(ctypes.byref(desc), flags, cv(k), cv(za), cv(zb), cv(q), cv(v),
                                     cv(ko), cv(ao), cv(bo), cv(qo), cv(vo), None)

    assert call(flags=4) == UNSUP                           # unknown flag bit
    assert call(q=7 * G) == UNSUP                           # q without its flag
    assert call(v=7 * G, vo=8 * G) == UNSUP                 # v without the literal flag
    assert call(flags=K.PROLOGUE_NORMALIZE_Q) == NULL       # q pointers missing
    assert call(flags=K.PROLOGUE_LITERAL_EQ6, v=7 * G) == NULL
    assert call(k=None) == NULL
    assert call(bo=None) == NULL
    assert call(k=1 * G + 8) == ALIGN
    assert call(za=2 * G + 2) == ALIGN
    assert call(ko=1 * G + nx // 2) == ALIAS                # partial overlap with its own input
    assert call(ko=2 * G) == ALIAS                          # k_out over the decay logits
    assert call(ao=6 * G) == ALIAS                          # two outputs on one buffer
    assert call(flags=K.PROLOGUE_LITERAL_EQ6, v=7 * G, vo=4 * G) == ALIAS
    assert call(desc=K.gdn_desc(1, 64, 2, 96)) == SHAPE
    assert call(desc=K.gdn_desc(1, 64, 2, 128, io=K.FP8_E4M3)) == DTYPE
    assert call(desc=K.gdn_desc(1, 0, 2, 128), k=None, za=None, zb=None, ko=None, ao=None,
                bo=None) == OK                             # empty: nothing to do


@host_only
def test_rope_validation():
    L = K.lib()
    cv = lambda x: None if x is None else ctypes.c_void_p(x)
    d = K.hlta_desc(1, 1000, 2, 128, 100, 1, 1, rope_base=1e4)
    d8 = K.hlta_desc(1, 1000, 2, 128, 100, 1, 1, window_qk=K.FP8_E4M3, rope_base=1e4)
    n = 1000 * 2 * 128
    call = lambda desc, dil=1, x=1 * G, out=2 * G, sc=None: L.kairos_rope(
        ctypes.byref(desc), dil, cv(x), cv(out), cv(sc), None)
    assert call(K.hlta_desc(1, 1000, 2, 128, 100, 1, 1)) == SHAPE          # base 0
    assert call(d, dil=0) == SHAPE
    assert call(d, sc=3 * G) == UNSUP                                      # bf16 takes no scales
    assert call(d8) == NULL                                                # fp8 needs scales
    assert call(d, x=None) == NULL
    assert call(d, x=1 * G + 8) == ALIGN
    assert call(d, out=1 * G + n) == ALIAS                                 # partial overlap
    assert call(d8, out=1 * G, sc=3 * G) == ALIAS                          # codes over the input
    # windowed stages take q, k as given: no RoPE there
    assert L.kairos_window_fwd(ctypes.byref(d), 1, cv(G), cv(2 * G), cv(3 * G), None, None, None,
                               None, cv(4 * G), None) == UNSUP


def test_workspace_grows_with_rope():
    base = dict(B=1, T=4096, H=2, d=128, L=1024, window=1024, dilation=4)
    n = 4096 * 2 * 128
    plain = K.kairos_hlta_workspace_size(K.hlta_desc(**base))
    rope = K.kairos_hlta_workspace_size(K.hlta_desc(**base, rope_base=1e4))
    assert rope - plain == 4 * n * 2                                       # two bf16 q, k pairs
    rope1 = K.kairos_hlta_workspace_size(K.hlta_desc(**{**base, "dilation": 1}, rope_base=1e4))
    assert rope1 - plain == 2 * n * 2                                      # dilation 1: one pair
    f8 = K.kairos_hlta_workspace_size(K.hlta_desc(**base, window_qk=K.FP8_E4M3))
    f8r = K.kairos_hlta_workspace_size(K.hlta_desc(**base, window_qk=K.FP8_E4M3, rope_base=1e4))
    assert f8r - f8 == 2 * n + 2 * 256 * ((2 * 64 * 4 + 255) // 256)      # codes + scales, 2nd branch


def test_binding_rejects_bad_tensors_on_cpu():
    import torch
    q = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16)
    a = torch.zeros((1, 8, 2), dtype=torch.float32)
    with pytest.raises(TypeError):
        K.kairos_gdn_fwd(q, q.float(), q, a, a)
    with pytest.raises(ValueError):
        K.kairos_gdn_fwd(q, q, q, a[:, :4], a)


def test_ring_sizes():
    """kairos_hlta_ring_size: value ring [B][R][L][H][d] bf16; key ring parts
    of rows (bf16 or codes) plus, for quantised keys, 256-aligned block scales
    [B][H][R][ceil(L/64)] fp32."""
    up = lambda x: (x + 255) // 256 * 256
    B, L, H, d, R = 2, 1560, 3, 128, 4
    toks = B * R * L * H
    kw = dict(B=B, T=L, H=H, d=d, L=L, window=1560, dilation=4, ring_frames=R)
    assert K.kairos_hlta_ring_size(K.hlta_desc(**kw)) == (toks * d * 2, toks * d * 2)
    assert K.kairos_hlta_ring_size(K.hlta_desc(**kw, rope_base=1e4)) == (2 * toks * d * 2, toks * d * 2)
    nbf = -(-L // 64)
    part8 = up(up(toks * d) + B * H * R * nbf * 4)
    fr = K.QK_BLOCKS_FRAMES
    assert K.kairos_hlta_ring_size(K.hlta_desc(**kw, window_qk=K.FP8_E4M3, qk_blocks=fr)) == \
        (part8, toks * d * 2)
    part4 = up(up(toks * d // 2) + B * H * R * nbf * 4)
    assert K.kairos_hlta_ring_size(K.hlta_desc(**kw, window_qk=K.FP4_E2M1, qk_blocks=fr,
                                               rope_base=1e4)) == (2 * part4, toks * d * 2)


@host_only
def test_window_entry_points_refuse_frame_blocks_with_codes():
    """The standalone window entry points take scales from the token-order
    quantisers: frame-aligned blocks (and quantised rings) only in the layer."""
    L = K.lib()
    cv = lambda x: None if x is None else ctypes.c_void_p(x)
    d = K.hlta_desc(1, 640, 2, 128, 320, 320, 2, window_qk=K.FP8_E4M3, qk_blocks=K.QK_BLOCKS_FRAMES)
    assert L.kairos_window_fwd(ctypes.byref(d), 2, cv(G), cv(2 * G), cv(3 * G), cv(4 * G), cv(5 * G),
                               None, None, cv(6 * G), None) == UNSUP
    assert L.kairos_hlta_window_fwd(ctypes.byref(d), cv(G), cv(2 * G), cv(3 * G), cv(4 * G), cv(5 * G),
                                    cv(6 * G), cv(7 * G), None, None, cv(8 * G), cv(9 * G), 1 << 30,
                                    None) == UNSUP
