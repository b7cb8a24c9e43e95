"""The C ABI library loads, exports every symbol include/moe.h declares, and rejects
bad arguments on the host before any launch (no GPU needed: validation returns
before the first HIP call)."""
import ctypes as C
import os
import re

import pytest

import mixture_experts_layer_33_amd as moe
from mixture_experts_layer_33_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_six_calls_and_helpers():
    names = declared_functions()
    for n in ["moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_decode",
              "moe_backward", "moe_workspace_bytes", "moe_status_string", "moe_quantize_mx"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings():
    L = _lib.lib()
    for code in range(8):
        assert L.moe_status_string(code)
    assert b"unknown" in L.moe_status_string(99)


def shape(**kw):
    base = dict(T=64, d=256, E=8, k=2, f=256, dtype="bf16")
    base.update(kw)
    return moe.make_shape(base["T"], base["d"], base["E"], base["k"], base["f"],
                          base.get("C"), base.get("fs", 0), base["dtype"])


def route(s, ws_bytes=1 << 30, x=FAKE):
    return _lib.lib().moe_route(s, x, FAKE, None, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=9), _lib.MOE_ERR_SHAPE),                     # k > E
    (dict(k=0), _lib.MOE_ERR_SHAPE),
    (dict(d=0), _lib.MOE_ERR_SHAPE),
    (dict(E=2000, k=2), _lib.MOE_ERR_SHAPE),             # more experts than one scan
    (dict(d=96, dtype="mxfp8"), _lib.MOE_ERR_SHAPE),     # MX length not a multiple of 32 * 4
    (dict(f=160, dtype="mxfp8"), _lib.MOE_ERR_SHAPE),
    (dict(d=100), _lib.MOE_ERR_SHAPE),                   # bf16 K slices of 64
    (dict(C=127), _lib.MOE_ERR_CAPACITY),                # C < T * k: would drop tokens
    (dict(dtype=7), _lib.MOE_ERR_DTYPE),
])
def test_shape_errors(kw, code):
    s = shape(**kw)
    assert route(s) == code
    L = _lib.lib()
    assert L.moe_dispatch(s, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == code
    assert L.moe_expert_ffn(s, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                            FAKE, 1 << 30, None) == code


def test_null_pointers():
    s = shape()
    L = _lib.lib()
    assert route(s, x=None) == _lib.MOE_ERR_NULL
    assert L.moe_route(None, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == _lib.MOE_ERR_NULL
    assert L.moe_combine(s, None, FAKE, FAKE, FAKE, None) == _lib.MOE_ERR_NULL
    smx = shape(dtype="mxfp8")
    # MXFP8 needs the scale buffers
    assert L.moe_dispatch(smx, FAKE, FAKE, 0, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == _lib.MOE_ERR_NULL
    assert L.moe_quantize_mx(None, 4, 32, FAKE, FAKE, None) == _lib.MOE_ERR_NULL


def test_workspace_too_small():
    s = shape()
    need = moe.workspace_bytes(s, _lib.OP_ROUTE)
    assert need >= 64 * 8 * 4
    assert route(s, ws_bytes=need - 1) == _lib.MOE_ERR_WORKSPACE
    L = _lib.lib()
    need = moe.workspace_bytes(s, _lib.OP_EXPERT_FFN)
    assert L.moe_expert_ffn(s, FAKE, None, FAKE, 0, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                            FAKE, need - 1, None) == _lib.MOE_ERR_WORKSPACE


def test_ring_head_range_and_dtype_gates():
    s = shape()
    L = _lib.lib()
    assert L.moe_dispatch(s, FAKE, FAKE, s.capacity, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                          None) == _lib.MOE_ERR_SHAPE
    assert L.moe_dispatch(s, FAKE, FAKE, -1, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                          None) == _lib.MOE_ERR_SHAPE
    # saved A|U exists for the bf16 backward only
    sf = shape(dtype="f32")
    assert L.moe_expert_ffn(sf, FAKE, None, FAKE, 0, FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE,
                            FAKE, 1 << 30, None) == _lib.MOE_ERR_DTYPE
    # decode: bf16 only, batch <= 8, widths multiples of 512
    sd = moe.make_shape(4, 1024, 16, 4, 512, fs=512, dtype="f32")
    assert L.moe_decode(sd, *([FAKE] * 12), FAKE, 1 << 30, None) == _lib.MOE_ERR_DTYPE
    sd = moe.make_shape(9, 1024, 16, 4, 512, fs=512, dtype="bf16")
    assert L.moe_decode(sd, *([FAKE] * 12), FAKE, 1 << 30, None) == _lib.MOE_ERR_SHAPE
    # the shared expert is absent or as wide as a routed one; widths in 512 steps up to the caps
    for bad in [dict(d=1024, f=512, fs=1024), dict(d=1000, f=512, fs=0), dict(d=1024, f=768, fs=0),
                dict(d=8704, f=512, fs=0), dict(d=1024, f=4608, fs=0)]:
        sd = moe.make_shape(4, bad["d"], 16, 4, bad["f"], fs=bad["fs"], dtype="bf16")
        assert L.moe_decode(sd, *([FAKE] * 12), FAKE, 1 << 30, None) == _lib.MOE_ERR_SHAPE, bad
    assert L.moe_quantize_mx(FAKE, 4, 48, FAKE, FAKE, None) == _lib.MOE_ERR_SHAPE
    # the MX backward keeps 3 f words of column maxima in one workgroup's LDS: f <= 13568
    sm = moe.make_shape(64, 256, 8, 2, 13696, dtype="mxfp8")
    assert L.moe_backward_mx(sm, *([FAKE] * 8), 0, *([FAKE] * 11), 1 << 40, None) == _lib.MOE_ERR_SHAPE


def test_workspace_sizes_of_the_workloads():
    import gen
    for cfg in [gen.TINY_F32, gen.FWD_BF16, gen.FWD_MXFP8, gen.SKEW_BWD]:
        s = moe.make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.C, cfg.fs, cfg.dtype)
        for op in range(6):
            b = moe.workspace_bytes(s, op)
            assert b % 256 == 0 and b < (8 << 30)
    s = moe.make_shape(8, 7168, 256, 8, 2048, fs=2048)
    assert moe.workspace_bytes(s, _lib.OP_DECODE) >= 8 * 8 * 2048 * 4


def test_ring_stack_capacity():
    """A shared ring must hold every layer's copies; the default is 1.25x each."""
    with pytest.raises(ValueError):
        moe.RingStack(3, T=16, d=128, E=8, k=2, f=256, C=3 * 32 - 1, device="cpu")
    st = moe.RingStack(3, T=16, d=128, E=8, k=2, f=256, device="cpu")
    assert st.shape.capacity == 3 * 40 and st.n == 32
    assert tuple(st.ring_x.shape) == (120, 128) and tuple(st.saved_au.shape) == (120, 512)


def test_rings_of_4_gib_are_rejected():
    """The grouped GEMM addresses ring_x [C, d] and H [C, f] with 32-bit byte offsets:
    a shape whose ring array reaches 4 GiB is rejected on the host, before any launch."""
    L = _lib.lib()
    d, f = 7168, 2048
    c_max = ((1 << 32) - 1) // (d * 2)            # the largest bf16 ring below 4 GiB
    ok = moe.make_shape(2048, d, 256, 8, f, C=c_max)
    bad = moe.make_shape(2048, d, 256, 8, f, C=c_max + 1)
    assert L.moe_check_shape(ok) == _lib.MOE_OK
    assert L.moe_check_shape(bad) == _lib.MOE_ERR_SHAPE
    assert route(bad) == _lib.MOE_ERR_SHAPE
    assert L.moe_expert_ffn(bad, FAKE, None, FAKE, 0, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                            FAKE, 1 << 40, None) == _lib.MOE_ERR_SHAPE
    # H decides when f > d; MX rows are one byte per element
    assert L.moe_check_shape(moe.make_shape(64, 256, 8, 2, 8192, C=(1 << 32) // (8192 * 2))) == _lib.MOE_ERR_SHAPE
    assert L.moe_check_shape(moe.make_shape(64, 7168, 8, 2, 2048, C=c_max + 1, dtype="mxfp8")) == _lib.MOE_OK
    assert L.moe_check_shape(moe.make_shape(64, 7168, 8, 2, 2048, C=-(-(1 << 32) // 7168),
                                            dtype="mxfp8")) == _lib.MOE_ERR_SHAPE
    # a ring stack of six skewed layers (d 4096, 102,400 rows each) would need 5 GB per array
    with pytest.raises(moe.MoeError):
        moe.RingStack(6, T=8192, d=4096, E=512, k=10, f=1024, device="cpu")


def test_decode_noalloc_validates_on_the_host():
    """The allocation-free decode rejects, before any HIP call, what moe_decode rejects and
    shapes whose workspace exceeds its 1 MiB static scratch."""
    L = _lib.lib()
    ok = moe.make_shape(8, 7168, 256, 8, 2048, fs=2048)
    assert moe.workspace_bytes(ok, _lib.OP_DECODE) <= (1 << 20)
    big = moe.make_shape(8, 1024, 64, 16, 4096, fs=4096)
    assert L.moe_decode_noalloc(big, *([FAKE] * 12), None) == _lib.MOE_ERR_SCRATCH
    assert L.moe_decode_noalloc(moe.make_shape(9, 1024, 16, 4, 512), *([FAKE] * 12), None) == _lib.MOE_ERR_SHAPE
    assert L.moe_decode_noalloc(ok, *([FAKE] * 9), None, FAKE, FAKE, None) == _lib.MOE_ERR_NULL
    assert b"scratch" in L.moe_status_string(_lib.MOE_ERR_SCRATCH)


def test_quantize_mx_both_validates_on_the_host():
    """The two-layout quantiser rejects, before any HIP call, NULL pointers and sizes that
    are not multiples of 128 or whose transposed columns overrun ld."""
    L = _lib.lib()
    q = L.moe_quantize_mx_both
    assert q(None, 1, 128, 128, FAKE, FAKE, FAKE, 128, 0, FAKE, None) == _lib.MOE_ERR_NULL
    assert q(FAKE, 1, 128, 128, FAKE, FAKE, FAKE, 128, 0, None, None) == _lib.MOE_ERR_NULL
    assert q(FAKE, 1, 96, 128, FAKE, FAKE, FAKE, 128, 0, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert q(FAKE, 1, 128, 160, FAKE, FAKE, FAKE, 128, 0, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert q(FAKE, 1, 128, 128, FAKE, FAKE, FAKE, 128, 64, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert q(FAKE, 1, 256, 128, FAKE, FAKE, FAKE, 128, 0, FAKE, None) == _lib.MOE_ERR_SHAPE
    assert q(FAKE, -1, 128, 128, FAKE, FAKE, FAKE, 128, 0, FAKE, None) == _lib.MOE_ERR_SHAPE

