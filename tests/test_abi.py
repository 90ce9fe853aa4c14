"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status codes
before any HIP call.  The fake device addresses below are never dereferenced:
every call here is built to fail validation, which happens on the host first."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp4.h")


@pytest.fixture(scope="module")
def lib():
    from mxfp4_routed_expert_router_amd import _lib
    return _lib


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_fp4_\w+)\s*\(", src, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_fp4_route", "moe_fp4_forward", "moe_fp4_forward_debug",
              "moe_fp4_workspace_size", "moe_fp4_prenorm_bf16", "moe_fp4_status_string",
              "moe_fp4_quant_mxfp8", "moe_fp4_router_logits", "moe_fp4_forward_routed",
              "moe_fp4_forward_saliency", "moe_fp4_shared_expert", "moe_fp4_forward_shared",
              "moe_fp4_forward_residual"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib._lib, n), n


def test_status_strings(lib):
    for s in range(6):
        assert lib.status_string(s) and lib.status_string(s) != "unknown status"
    assert lib.status_string(99) == "unknown status"


def test_header_compiles_as_c(tmp_path):
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include "moe_fp4.h"\nint main(void){moe_fp4_dims d={1,32,32,1,1};'
                   'size_t b;return moe_fp4_workspace_size(&d,0,&b);}\n')
    r = subprocess.run(["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", "-c", str(src), "-o", str(tmp_path / "use.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


# --------------------------------------------------------------------------- validation
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def _weights(lib, **over):
    w = lib.Weights()
    for i, n in enumerate(lib.TENSORS):
        setattr(w, n, over.get(n, FAKE + (i << 30)))
    for i, s in enumerate(over.get("strides", (0,) * 6)):
        w.expert_stride[i] = s
    return w


def _fwd(lib, dims=(4, 256, 128, 16, 2), x=FAKE, logits=FAKE, w=None, y=FAKE, mode=0, flags=0,
         ws=FAKE, ws_bytes=None):
    d = lib.Dims(*dims)
    if w is None:
        w = _weights(lib)
    if ws_bytes is None:
        n = ctypes.c_size_t()
        rc = lib._lib.moe_fp4_workspace_size(ctypes.byref(d), mode, ctypes.byref(n))
        ws_bytes = n.value if rc == 0 else 1 << 40
    return lib._lib.moe_fp4_forward(ctypes.byref(d), x, logits, ctypes.byref(w), y, mode, flags, ws,
                                    ws_bytes, None)


def test_workspace_size(lib):
    assert lib.moe_fp4_workspace_size(1, 5120, 2304, 384, 6) > 6 * 2304 * 2
    pre = lib.moe_fp4_workspace_size(2048, 5120, 2304, 384, 6)
    assert pre >= 12288 * 5120 * 4 + 12288 * 2304 * 2
    assert lib.moe_fp4_workspace_size(8, 256, 128, 16, 2, lib.MODE_PREFILL) > \
        lib.moe_fp4_workspace_size(8, 256, 128, 16, 2, lib.MODE_DECODE)
    with pytest.raises(lib.MoeFp4Error) as e:
        lib.moe_fp4_workspace_size(33, 256, 128, 16, 2, lib.MODE_DECODE)
    assert e.value.status == lib.EUNSUPPORTED
    # the real shape: the few-token kernels stage up to 15 activation rows
    for T in (1, 2, 6, 15):
        assert lib.moe_fp4_workspace_size(T, 5120, 2304, 384, 6, lib.MODE_DECODE) > 0
    with pytest.raises(lib.MoeFp4Error) as e:
        lib.moe_fp4_workspace_size(16, 5120, 2304, 384, 6, lib.MODE_DECODE)
    assert e.value.status == lib.EUNSUPPORTED
    n = ctypes.c_size_t()
    assert lib._lib.moe_fp4_workspace_size(None, 0, ctypes.byref(n)) == lib.EINVAL


def test_workspace_is_the_only_failure(lib):
    # every other argument valid: the call stops at the workspace check
    assert _fwd(lib, ws_bytes=0) == lib.EWORKSPACE
    assert _fwd(lib, ws=0) == lib.EINVAL


@pytest.mark.parametrize("field", ["x", "logits", "y"])
def test_null_pointers(lib, field):
    assert _fwd(lib, ws_bytes=0, **{field: 0}) == lib.EINVAL


@pytest.mark.parametrize("name", ["w1", "s1", "w3", "s3", "w2", "s2"])
def test_null_weights(lib, name):
    assert _fwd(lib, ws_bytes=0, w=_weights(lib, **{name: 0})) == lib.EINVAL


def test_null_dims(lib):
    w = _weights(lib)
    assert lib._lib.moe_fp4_forward(None, FAKE, FAKE, ctypes.byref(w), FAKE, 0, 0, FAKE, 0, None) \
        == lib.EINVAL
    assert lib._lib.moe_fp4_forward(ctypes.byref(lib.Dims(1, 32, 32, 1, 1)), FAKE, FAKE, None, FAKE,
                                    0, 0, FAKE, 0, None) == lib.EINVAL


@pytest.mark.parametrize("dims,code", [
    ((0, 256, 128, 16, 2), "EINVAL"),          # no tokens
    ((4, 256, 128, 16, 0), "EINVAL"),          # k = 0
    ((4, 256, 128, 2, 3), "EINVAL"),           # k > E
    ((4, 250, 128, 16, 2), "EUNSUPPORTED"),    # H not a multiple of 32
    ((4, 256, 100, 16, 2), "EUNSUPPORTED"),    # I not a multiple of 32
    ((4, 256, 128, 2048, 2), "EUNSUPPORTED"),  # E > 1024
    ((4, 256, 128, 64, 17), "EUNSUPPORTED"),   # k > 16
    ((70000, 256, 128, 16, 2), "EUNSUPPORTED"),
    ((4, 32768, 128, 16, 2), "EUNSUPPORTED"),
])
def test_bad_dims(lib, dims, code):
    assert _fwd(lib, dims=dims, ws_bytes=0) == getattr(lib, code)


def test_bad_mode_and_flags(lib):
    assert _fwd(lib, mode=7, ws_bytes=0) == lib.EUNSUPPORTED
    assert _fwd(lib, flags=2, ws_bytes=0) == lib.EUNSUPPORTED
    assert _fwd(lib, dims=(33, 256, 128, 16, 2), mode=lib.MODE_DECODE, ws_bytes=0) == lib.EUNSUPPORTED
    assert _fwd(lib, dims=(32, 256, 128, 16, 8), mode=lib.MODE_DECODE, ws_bytes=0) == lib.EUNSUPPORTED


def test_negative_stride(lib):
    assert _fwd(lib, w=_weights(lib, strides=(0, 0, 0, 0, -16, 0)), ws_bytes=0) == lib.EINVAL


@pytest.mark.parametrize("kw", [dict(x=FAKE + 8), dict(y=FAKE + 4), dict(ws=FAKE + 64)])
def test_misaligned(lib, kw):
    assert _fwd(lib, ws_bytes=0, **kw) == lib.EALIGN


@pytest.mark.parametrize("over", [dict(w1=FAKE + 8), dict(w3=FAKE + 1), dict(w2=FAKE + 4),
                                  dict(strides=(65544, 0, 0, 0, 0, 0)),
                                  dict(strides=(0, 0, 0, 0, 16392, 0))])
def test_misaligned_weights(lib, over):
    assert _fwd(lib, w=_weights(lib, **over), ws_bytes=0) == lib.EALIGN


def test_scale_tensors_need_no_alignment(lib):
    w = _weights(lib, s1=FAKE + 1, s3=FAKE + 3, s2=FAKE + 5, strides=(0, 7, 0, 9, 0, 11))
    assert _fwd(lib, w=w, ws_bytes=0) == lib.EWORKSPACE


def test_route_validation(lib):
    r = lib.RouteOut()
    for n in ("topk_idx", "gates", "counts", "offsets", "sorted_pairs", "pair_slot"):
        setattr(r, n, FAKE)
    f = lib._lib.moe_fp4_route
    d4 = ctypes.byref(lib.Dims(4, 0, 0, 16, 2))
    assert f(d4, None, ctypes.byref(r), None, 0, None) == lib.EINVAL
    assert f(ctypes.byref(lib.Dims(4, 0, 0, 16, 20)), FAKE, ctypes.byref(r), None, 0, None) == lib.EINVAL
    assert f(ctypes.byref(lib.Dims(4, 0, 0, 2000, 2)), FAKE, ctypes.byref(r), None, 0,
             None) == lib.EUNSUPPORTED
    assert f(d4, FAKE + 2, ctypes.byref(r), None, 0, None) == lib.EALIGN
    r.gates = 0
    assert f(d4, FAKE, ctypes.byref(r), None, 0, None) == lib.EINVAL


def test_route_workspace(lib):
    """Up to 64 tokens and 1024 pairs routing needs no workspace; the 2048-token
    chunk (12,288 pairs) needs one for the many-workgroup permutation, and a
    missing, short or misaligned one is refused before anything is enqueued."""
    r = lib.RouteOut()
    for n in ("topk_idx", "gates", "counts", "offsets", "sorted_pairs", "pair_slot"):
        setattr(r, n, FAKE)
    assert lib.moe_fp4_route_workspace_size(64, 384, 16) == 0
    assert lib.moe_fp4_route_workspace_size(6, 384, 6) == 0
    n = lib.moe_fp4_route_workspace_size(2048, 384, 6)
    assert n >= 256 * 384 * 4 + 2 * 12288 * 4 + 384 * 16
    f = lib._lib.moe_fp4_route
    d = ctypes.byref(lib.Dims(2048, 0, 0, 384, 6))
    assert f(d, FAKE, ctypes.byref(r), None, 0, None) == lib.EWORKSPACE
    assert f(d, FAKE, ctypes.byref(r), FAKE, n - 1, None) == lib.EWORKSPACE
    assert f(d, FAKE, ctypes.byref(r), FAKE + 16, n, None) == lib.EALIGN
    with pytest.raises(lib.MoeFp4Error):
        lib.moe_fp4_route_workspace_size(0, 384, 6)


def test_plan(lib):
    """The kernel path a forward call takes, by size and mode."""
    assert lib.moe_fp4_plan(1, 5120, 2304, 384, 6) == lib.PATH_DECODE_ONE
    assert lib.moe_fp4_plan(6, 5120, 2304, 384, 6) == lib.PATH_DECODE_FEW
    assert lib.moe_fp4_plan(8, 5120, 2304, 384, 6) == lib.PATH_DECODE_FEW
    # AUTO: the grouped GEMMs from 9 tokens on; DECODE still takes up to 15
    assert lib.moe_fp4_plan(9, 5120, 2304, 384, 6) == lib.PATH_PREFILL
    assert lib.moe_fp4_plan(15, 5120, 2304, 384, 6, lib.MODE_DECODE) == lib.PATH_DECODE_FEW
    assert lib.moe_fp4_plan(16, 5120, 2304, 384, 6) == lib.PATH_PREFILL
    assert lib.moe_fp4_plan(2048, 5120, 2304, 384, 6) == lib.PATH_PREFILL
    assert lib.moe_fp4_plan(1, 5120, 2304, 384, 6, lib.MODE_PREFILL) == lib.PATH_PREFILL
    assert lib.moe_fp4_plan(32, 5120, 2304, 384, 6, lib.MODE_PREFILL_MXFP8) == lib.PATH_PREFILL_MXFP8
    assert lib.moe_fp4_plan(16, 256, 128, 16, 2, lib.MODE_DECODE) == lib.PATH_DECODE_MFMA
    with pytest.raises(lib.MoeFp4Error):
        lib.moe_fp4_plan(32, 5120, 2304, 384, 6, lib.MODE_DECODE)


def test_prenorm_validation(lib):
    f = lib._lib.moe_fp4_prenorm_bf16
    assert f(None, FAKE, 1, 64, 1e-6, None) == lib.EINVAL
    assert f(FAKE, FAKE, 0, 64, 1e-6, None) == lib.EINVAL
    assert f(FAKE, FAKE, 1, 48, 1e-6, None) == lib.EUNSUPPORTED
    assert f(FAKE, FAKE, 1, 16416, 1e-6, None) == lib.EUNSUPPORTED
    assert f(FAKE + 4, FAKE, 1, 64, 1e-6, None) == lib.EALIGN
    assert f(FAKE, FAKE + 8, 1, 64, 1e-6, None) == lib.EALIGN


def test_profiled_needs_eight_events(lib):
    """Stage timing takes a start and an end event for each of the four stages."""
    d = lib.Dims(4, 256, 128, 16, 2)
    w = _weights(lib)
    n = ctypes.c_size_t()
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == lib.OK
    fake_events = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    args = (ctypes.byref(d), FAKE, FAKE, ctypes.byref(w), FAKE, 0, 0, FAKE, n.value, None)
    assert lib._lib.moe_fp4_forward_profiled(*args, None, 8) == lib.EINVAL
    assert lib._lib.moe_fp4_forward_profiled(*args, fake_events, 7) == lib.EINVAL
    fake_events[3] = None
    assert lib._lib.moe_fp4_forward_profiled(*args, fake_events, 8) == lib.EINVAL


def test_mxfp8_mode_validation(lib):
    """The MXFP8 prefill mode needs H and I to be multiples of 128."""
    assert _fwd(lib, dims=(4, 256, 128, 16, 2), mode=lib.MODE_PREFILL_MXFP8, ws_bytes=0) == lib.EWORKSPACE
    assert _fwd(lib, dims=(4, 288, 128, 16, 2), mode=lib.MODE_PREFILL_MXFP8, ws_bytes=0) == lib.EUNSUPPORTED
    assert _fwd(lib, dims=(4, 256, 96, 16, 2), mode=lib.MODE_PREFILL_MXFP8, ws_bytes=0) == lib.EUNSUPPORTED
    n_bf16, n_mx = ctypes.c_size_t(), ctypes.c_size_t()
    d = lib.Dims(4, 256, 128, 16, 2)
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), lib.MODE_PREFILL, ctypes.byref(n_bf16)) == lib.OK
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), lib.MODE_PREFILL_MXFP8, ctypes.byref(n_mx)) == lib.OK
    assert n_mx.value > n_bf16.value  # room for the FP8 activations and their scales


def test_mxfp8_scale_alignment(lib):
    """The MXFP8 GEMMs read scales a dword at a time: bases and strides 4-aligned."""
    dims = (4, 256, 128, 16, 2)
    m = lib.MODE_PREFILL_MXFP8
    assert _fwd(lib, dims=dims, mode=m, w=_weights(lib, s1=FAKE + 4), ws_bytes=0) == lib.EWORKSPACE
    assert _fwd(lib, dims=dims, mode=m, w=_weights(lib, s3=FAKE + 2), ws_bytes=0) == lib.EALIGN
    assert _fwd(lib, dims=dims, mode=m, w=_weights(lib, strides=(0, 0, 0, 0, 0, 1026)),
                ws_bytes=0) == lib.EALIGN
    assert _fwd(lib, dims=dims, mode=lib.MODE_PREFILL, w=_weights(lib, s3=FAKE + 2), ws_bytes=0) \
        == lib.EWORKSPACE


def test_quant_mxfp8_validation(lib):
    f = lib._lib.moe_fp4_quant_mxfp8
    assert f(None, 4, 64, FAKE, FAKE, None) == lib.EINVAL
    assert f(FAKE, 0, 64, FAKE, FAKE, None) == lib.EINVAL
    assert f(FAKE, 4, 48, FAKE, FAKE, None) == lib.EUNSUPPORTED
    assert f(FAKE + 8, 4, 64, FAKE, FAKE, None) == lib.EALIGN


def test_router_logits_validation(lib):
    f = lib._lib.moe_fp4_router_logits
    d = ctypes.byref(lib.Dims(4, 256, 0, 16, 0))
    assert f(None, FAKE, FAKE, FAKE, None) == lib.EINVAL
    assert f(d, None, FAKE, FAKE, None) == lib.EINVAL
    assert f(d, FAKE, None, FAKE, None) == lib.EINVAL
    assert f(d, FAKE, FAKE, None, None) == lib.EINVAL
    assert f(ctypes.byref(lib.Dims(0, 256, 0, 16, 0)), FAKE, FAKE, FAKE, None) == lib.EINVAL
    assert f(ctypes.byref(lib.Dims(4, 250, 0, 16, 0)), FAKE, FAKE, FAKE, None) == lib.EUNSUPPORTED
    assert f(ctypes.byref(lib.Dims(4, 256, 0, 2000, 0)), FAKE, FAKE, FAKE, None) == lib.EUNSUPPORTED
    assert f(d, FAKE + 8, FAKE, FAKE, None) == lib.EALIGN
    assert f(d, FAKE, FAKE + 2, FAKE, None) == lib.EALIGN
    assert f(d, FAKE, FAKE, FAKE + 2, None) == lib.EALIGN


def test_forward_routed_validation(lib):
    """Same checks as moe_fp4_forward, the router weight in place of the logits."""
    f = lib._lib.moe_fp4_forward_routed
    d = lib.Dims(4, 256, 128, 16, 2)
    w = _weights(lib)
    n = ctypes.c_size_t()
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == lib.OK
    args = lambda wr, ws_bytes: (ctypes.byref(d), FAKE, wr, ctypes.byref(w), FAKE, 0, 0, FAKE,
                                 ws_bytes, None)
    assert f(*args(None, n.value)) == lib.EINVAL
    assert f(*args(FAKE + 2, n.value)) == lib.EALIGN
    assert f(*args(FAKE, 0)) == lib.EWORKSPACE


def test_forward_saliency_validation(lib):
    """Prefill modes only; AUTO runs PREFILL, so its workspace is PREFILL's."""
    f = lib._lib.moe_fp4_forward_saliency
    d = lib.Dims(4, 256, 128, 16, 2)
    w = _weights(lib)
    n_pre, n_dec = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), lib.MODE_PREFILL, ctypes.byref(n_pre)) == 0
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), lib.MODE_DECODE, ctypes.byref(n_dec)) == 0
    call = lambda sal, mode, nb: f(ctypes.byref(d), FAKE, FAKE, ctypes.byref(w), FAKE, sal, mode, 0,
                                   FAKE, nb, None)
    assert call(None, 0, n_pre.value) == lib.EINVAL
    assert call(FAKE, lib.MODE_DECODE, n_pre.value) == lib.EUNSUPPORTED
    assert call(FAKE + 2, lib.MODE_PREFILL, n_pre.value) == lib.EALIGN
    assert call(FAKE, lib.MODE_AUTO, n_dec.value) == lib.EWORKSPACE


def _shared(lib, **over):
    sw = lib.SharedWeightsStruct()
    for i, n in enumerate(lib.TENSORS):
        setattr(sw, n, over.get(n, FAKE + (i << 30)))
    sw.I = over.get("I", 128)
    return sw


def test_shared_expert_validation(lib):
    f = lib._lib.moe_fp4_shared_expert
    d = ctypes.byref(lib.Dims(4, 256, 0, 0, 0))
    call = lambda sw, x=FAKE, y=FAKE, flags=0, h=FAKE, dims=d: f(dims, x, ctypes.byref(sw), y, flags,
                                                                 h, None)
    assert call(_shared(lib), h=None) == lib.EINVAL
    assert call(_shared(lib), x=None) == lib.EINVAL
    assert call(_shared(lib, w2=None)) == lib.EINVAL
    assert call(_shared(lib, I=100)) == lib.EUNSUPPORTED
    assert call(_shared(lib), dims=ctypes.byref(lib.Dims(4, 250, 0, 0, 0))) == lib.EUNSUPPORTED
    assert call(_shared(lib), flags=2) == lib.EUNSUPPORTED
    assert call(_shared(lib, w3=FAKE + 8)) == lib.EALIGN
    assert call(_shared(lib), h=FAKE + 2) == lib.EALIGN


def test_forward_shared_validation(lib):
    """The shared expert's h lives in the routed h section: I_s <= k * I."""
    f = lib._lib.moe_fp4_forward_shared
    d = lib.Dims(4, 256, 128, 16, 2)
    w = _weights(lib)
    n = ctypes.c_size_t()
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == lib.OK
    call = lambda sw, nb: f(ctypes.byref(d), FAKE, FAKE, ctypes.byref(w), ctypes.byref(sw), FAKE, 0,
                            0, FAKE, nb, None)
    assert call(_shared(lib, I=288), n.value) == lib.EUNSUPPORTED
    assert call(_shared(lib, s1=None), n.value) == lib.EINVAL
    assert call(_shared(lib, I=256), 0) == lib.EWORKSPACE


def test_forward_residual_validation(lib):
    f = lib._lib.moe_fp4_forward_residual
    d = lib.Dims(4, 256, 128, 16, 2)
    w = _weights(lib)
    n = ctypes.c_size_t()
    assert lib._lib.moe_fp4_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == lib.OK
    call = lambda x, nb: f(ctypes.byref(d), x, FAKE, ctypes.byref(w), 0, FAKE, nb, None)
    assert call(None, n.value) == lib.EINVAL
    assert call(FAKE + 8, n.value) == lib.EALIGN
    assert call(FAKE, 0) == lib.EWORKSPACE


def test_noalloc_rejects_before_any_hip_call(lib):
    """The no-allocation forward refuses a call whose workspace would exceed its
    static array (the 2048-token chunk), and bad arguments, before any HIP call."""
    f = lib._lib.moe_fp4_forward_noalloc
    w = _weights(lib)
    big = lib.Dims(2048, 5120, 2304, 384, 6)
    assert lib.moe_fp4_workspace_size(2048, 5120, 2304, 384, 6) > (8 << 20)
    assert f(ctypes.byref(big), FAKE, FAKE, ctypes.byref(w), FAKE, 0, 0, None) == lib.EWORKSPACE
    small = lib.Dims(4, 256, 128, 16, 2)
    assert f(ctypes.byref(small), None, FAKE, ctypes.byref(w), FAKE, 0, 0, None) == lib.EINVAL
    assert f(ctypes.byref(small), FAKE + 2, FAKE, ctypes.byref(w), FAKE, 0, 0, None) == lib.EALIGN
    assert f(ctypes.byref(small), FAKE, FAKE, ctypes.byref(w), FAKE, 7, 0, None) == lib.EUNSUPPORTED
    assert f(ctypes.byref(big), None, FAKE, ctypes.byref(w), FAKE, 0, 0, None) == lib.EINVAL
