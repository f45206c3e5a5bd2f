"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function ``include/sdpa14.h`` declares,
and reject invalid arguments with the documented codes before touching the
GPU: such calls return before any HIP call, enqueue nothing and leave the
RNG state as it was.  Device pointers here are fake, aligned addresses that
are never dereferenced.
"""

import ctypes
import math
import os
import re

import pytest

import scaled_dot_product_14_amd as sdpa
from scaled_dot_product_14_amd import _binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # inputs: 16-byte aligned, never dereferenced
FAKE_OUT = 0x7F1000000000  # outputs, LSE and workspace sit apart from the inputs
FAKE_LSE = 0x7F2000000000
FAKE_WS = 0x7F3000000000


@pytest.fixture(scope="module")
def lib():
    return bnd.load_library()


def _header_functions():
    with open(os.path.join(ROOT, "include", "sdpa14.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(sdpa_[a-z_0-9]+)\s*\(",
                          text, flags=re.M))


def test_exports_every_declared_function(lib):
    names = _header_functions()
    assert names == set(bnd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def _t(B=1, H=2, S=128, E=64, layout="BHSE", data=FAKE, dtype=0, stride=None):
    d = bnd.SdpaTensor()
    d.data = data
    d.dtype = dtype
    for i, x in enumerate((B, H, S, E)):
        d.size[i] = x
    if stride is None:
        stride = (H * S * E, S * E, E, 1) if layout == "BHSE" else (S * H * E, E, H * E, 1)
    for i, x in enumerate(stride):
        d.stride[i] = x
    return d


def _fwd(lib, q=None, k=None, v=None, out=None, p=0.0, scale=math.nan, lse=FAKE_LSE):
    q = q or _t()
    k = k or _t()
    v = v or _t()
    out = out or _t(data=FAKE_OUT)
    s, o = ctypes.c_uint64(), ctypes.c_uint64()
    return lib.sdpa_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), p, 1, scale,
                        ctypes.byref(out), lse, ctypes.byref(s), ctypes.byref(o), None)


def _err(lib):
    return lib.sdpa_last_error().decode()


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=_t(data=0)), bnd.SDPA_ERR_INVALID, "NULL"),
    (dict(v=_t(E=128), q=_t(E=128), k=_t(E=64)), bnd.SDPA_ERR_INVALID, "head dims"),
    (dict(v=_t(E=128)), bnd.SDPA_ERR_INVALID, "Ev"),
    (dict(k=_t(S=64)), bnd.SDPA_ERR_INVALID, "key lengths"),
    (dict(k=_t(H=3), v=_t(H=3)), bnd.SDPA_ERR_INVALID, "batch or heads"),
    (dict(out=_t(S=64)), bnd.SDPA_ERR_INVALID, "out"),
    (dict(p=1.0), bnd.SDPA_ERR_INVALID, "dropout"),
    (dict(p=-0.1), bnd.SDPA_ERR_INVALID, "dropout"),
    (dict(p=math.nan), bnd.SDPA_ERR_INVALID, "dropout"),
    (dict(scale=0.0), bnd.SDPA_ERR_INVALID, "scale"),
    (dict(scale=math.inf), bnd.SDPA_ERR_INVALID, "scale"),
    (dict(lse=0), bnd.SDPA_ERR_INVALID, "lse"),
    (dict(q=_t(S=0)), bnd.SDPA_ERR_INVALID, "size"),
    (dict(q=_t(dtype=2)), bnd.SDPA_ERR_UNSUPPORTED, "dtype"),
    (dict(q=_t(dtype=1)), bnd.SDPA_ERR_INVALID, "one dtype"),
    (dict(q=_t(dtype=1), k=_t(dtype=1), v=_t(dtype=1)), bnd.SDPA_ERR_INVALID, "one dtype"),
    (dict(q=_t(E=136), k=_t(E=136), v=_t(E=136), out=_t(E=136)), bnd.SDPA_ERR_UNSUPPORTED,
     "head dim"),
    (dict(q=_t(E=12, stride=(2 * 128 * 16, 128 * 16, 16, 1)),
          k=_t(E=12, stride=(2 * 128 * 16, 128 * 16, 16, 1)),
          v=_t(E=12, stride=(2 * 128 * 16, 128 * 16, 16, 1)),
          out=_t(E=12, stride=(2 * 128 * 16, 128 * 16, 16, 1))), bnd.SDPA_ERR_UNSUPPORTED,
     "multiple of 8"),
    (dict(q=_t(stride=(2 * 128 * 64, 128 * 64, 1, 128))), bnd.SDPA_ERR_UNSUPPORTED, "stride"),
    (dict(q=_t(stride=(2 * 128 * 68, 128 * 68, 68, 1))), bnd.SDPA_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(q=_t(data=FAKE + 8)), bnd.SDPA_ERR_UNSUPPORTED, "aligned"),
])
def test_forward_rejects_bad_arguments(lib, kw, code, needle):
    bnd.sdpa_set_rng_state(1234, 99)
    rc = _fwd(lib, **kw)
    assert rc == code, (rc, _err(lib))
    assert needle.lower() in _err(lib).lower()
    assert bnd.sdpa_get_rng_state() == (1234, 99)


WS_BYTES = 1 << 20  # ample for the default shapes (B*H*Sq*8 = 2 KiB)


_OUT_ADDR = {"dq": FAKE_OUT, "dk": FAKE_OUT + (1 << 32), "dv": FAKE_OUT + (2 << 32)}


def _bwd(lib, **over):
    t = {n: over.get(n) or _t(data=_OUT_ADDR.get(n, FAKE))
         for n in ("dout", "q", "k", "v", "out", "dq", "dk", "dv")}
    return lib.sdpa_bwd(*(ctypes.byref(t[n]) for n in ("dout", "q", "k", "v", "out")),
                        over.get("lse", FAKE_LSE), over.get("p", 0.0), 1, 0, 0,
                        over.get("scale", math.nan),
                        *(ctypes.byref(t[n]) for n in ("dq", "dk", "dv")),
                        over.get("ws", FAKE_WS), over.get("ws_bytes", WS_BYTES), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=_t(S=64)), bnd.SDPA_ERR_INVALID),
    (dict(dq=_t(S=64)), bnd.SDPA_ERR_INVALID),
    (dict(dout=_t(E=128)), bnd.SDPA_ERR_INVALID),
    (dict(lse=0), bnd.SDPA_ERR_INVALID),
    (dict(p=1.5), bnd.SDPA_ERR_INVALID),
    (dict(dv=_t(dtype=3)), bnd.SDPA_ERR_UNSUPPORTED),
    (dict(dq=_t(dtype=1)), bnd.SDPA_ERR_INVALID),
    (dict(scale=-1.0), bnd.SDPA_ERR_INVALID),
    (dict(out=_t(stride=(2 * 128 * 64, 128 * 64, 64, 2))), bnd.SDPA_ERR_UNSUPPORTED),
])
def test_backward_rejects_bad_arguments(lib, kw, code):
    bnd.sdpa_set_rng_state(5, 6)
    rc = _bwd(lib, **kw)
    assert rc == code, (rc, _err(lib))
    assert bnd.sdpa_get_rng_state() == (5, 6)


@pytest.mark.parametrize("kw,needle", [
    (dict(ws=0), "NULL"),
    (dict(ws=FAKE_WS + 128), "aligned"),
    (dict(ws_bytes=2047), "smaller"),
])
def test_backward_checks_workspace(lib, kw, needle):
    bnd.sdpa_set_rng_state(7, 8)
    rc = _bwd(lib, **kw)
    assert rc == bnd.SDPA_ERR_WORKSPACE, (rc, _err(lib))
    assert needle.lower() in _err(lib).lower()
    assert bnd.sdpa_get_rng_state() == (7, 8)


_BIAS_KEEP = []


def _ext(head_offset=0, heads_total=0, rng_state=None, rng_used=None, bias=None):
    e = bnd.SdpaExt()
    e.head_offset, e.heads_total, e.rng_state, e.rng_used = head_offset, heads_total, rng_state, rng_used
    if bias is not None:
        _BIAS_KEEP.append(bias)
        e.bias = ctypes.pointer(bias)
    return e


def _bias(size=(1, 2, 128, 128), stride=(0, 128 * 128, 128, 1), data=FAKE, dtype=0):
    d = bnd.SdpaTensor()
    d.data, d.dtype = data, dtype
    for i in range(4):
        d.size[i], d.stride[i] = size[i], stride[i]
    return d


@pytest.mark.parametrize("ext,code,needle", [
    (_ext(head_offset=-1), bnd.SDPA_ERR_INVALID, "head_offset"),
    (_ext(head_offset=1, heads_total=2), bnd.SDPA_ERR_INVALID, "heads_total"),
    (_ext(heads_total=1), bnd.SDPA_ERR_INVALID, "heads_total"),
    (_ext(heads_total=1 << 31), bnd.SDPA_ERR_UNSUPPORTED, "too large"),
    (_ext(rng_state=FAKE), bnd.SDPA_ERR_INVALID, "together"),
    (_ext(rng_used=FAKE), bnd.SDPA_ERR_INVALID, "together"),
    (_ext(rng_state=FAKE, rng_used=FAKE), bnd.SDPA_ERR_INVALID, "distinct"),
    (_ext(rng_state=FAKE + 4, rng_used=FAKE + 64), bnd.SDPA_ERR_UNSUPPORTED, "aligned"),
    (_ext(bias=_bias(data=0)), bnd.SDPA_ERR_INVALID, "bias data"),
    (_ext(bias=_bias(dtype=1)), bnd.SDPA_ERR_UNSUPPORTED, "bias dtype"),
    (_ext(bias=_bias(size=(1, 2, 128, 64))), bnd.SDPA_ERR_INVALID, "shape"),
    (_ext(bias=_bias(stride=(0, 0, 1, 128))), bnd.SDPA_ERR_UNSUPPORTED, "key stride"),
    (_ext(bias=_bias(stride=(0, 0, 132, 1))), bnd.SDPA_ERR_UNSUPPORTED, "multiples of 8"),
    (_ext(bias=_bias(stride=(0, -128, 128, 1))), bnd.SDPA_ERR_UNSUPPORTED, ">= 0"),
    (_ext(bias=_bias(data=FAKE + 8)), bnd.SDPA_ERR_UNSUPPORTED, "16-byte"),
    (_ext(bias=_bias(stride=(0, 0, 1 << 24, 1))), bnd.SDPA_ERR_UNSUPPORTED, "2 GiB"),
])
def test_forward_ext_rejects_bad_options(lib, ext, code, needle):
    bnd.sdpa_set_rng_state(31, 41)
    q, k, v, out = _t(), _t(), _t(), _t(data=FAKE_OUT)
    s, o = ctypes.c_uint64(), ctypes.c_uint64()
    rc = lib.sdpa_fwd_ext(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0.1, 1, math.nan,
                          ctypes.byref(out), FAKE_LSE, ctypes.byref(s), ctypes.byref(o),
                          ctypes.byref(ext), None)
    assert rc == code, (rc, _err(lib))
    assert needle.lower() in _err(lib).lower()
    assert bnd.sdpa_get_rng_state() == (31, 41)


def _ext_parts(n):
    e = _ext()
    e.bwd_parts = n
    return e


@pytest.mark.parametrize("ext,code,needle", [
    (_ext_parts(4), bnd.SDPA_ERR_INVALID, "bwd_parts"),
    (_ext_parts(-1), bnd.SDPA_ERR_INVALID, "bwd_parts"),
    (_ext(head_offset=-3), bnd.SDPA_ERR_INVALID, "head_offset"),
    (_ext(head_offset=2, heads_total=3), bnd.SDPA_ERR_INVALID, "heads_total"),
    (_ext(rng_used=FAKE + 2), bnd.SDPA_ERR_UNSUPPORTED, "aligned"),
])
def test_backward_ext_rejects_bad_options(lib, ext, code, needle):
    t = {n: _t(data=_OUT_ADDR.get(n, FAKE)) for n in ("dout", "q", "k", "v", "out", "dq", "dk", "dv")}
    rc = lib.sdpa_bwd_ext(*(ctypes.byref(t[n]) for n in ("dout", "q", "k", "v", "out")),
                          FAKE_LSE, 0.1, 1, 0, 0, math.nan,
                          *(ctypes.byref(t[n]) for n in ("dq", "dk", "dv")),
                          FAKE_WS, WS_BYTES, ctypes.byref(ext), None)
    assert rc == code, (rc, _err(lib))
    assert needle.lower() in _err(lib).lower()


FAKE_DB = 0x7F4000000000


def _ext_db(bias=True, **kw):
    e = _ext(bias=_bias() if bias else None)
    d = _bias(**{"data": FAKE_DB, "stride": (2 * 128 * 128, 128 * 128, 128, 1), **kw})
    _BIAS_KEEP.append(d)
    e.dbias = ctypes.pointer(d)
    return e


@pytest.mark.parametrize("ext,code,needle", [
    (_ext_db(bias=False), bnd.SDPA_ERR_INVALID, "needs a bias"),
    (_ext_db(data=0), bnd.SDPA_ERR_INVALID, "dbias data"),
    (_ext_db(dtype=1), bnd.SDPA_ERR_UNSUPPORTED, "dbias dtype"),
    (_ext_db(size=(1, 2, 128, 64)), bnd.SDPA_ERR_INVALID, "shape"),
    (_ext_db(stride=(2 * 128 * 128, 128 * 128, 1, 128)), bnd.SDPA_ERR_UNSUPPORTED, "key stride"),
    (_ext_db(stride=(2 * 128 * 128, 0, 128, 1)), bnd.SDPA_ERR_UNSUPPORTED, "positive"),
    (_ext_db(stride=(2 * 128 * 128, 128 * 128, 132, 1)), bnd.SDPA_ERR_UNSUPPORTED, "multiples of 8"),
    (_ext_db(data=FAKE_DB + 8), bnd.SDPA_ERR_UNSUPPORTED, "16-byte"),
    # Rows 64 elements apart with 128 keys: elements of neighbouring rows coincide.
    (_ext_db(stride=(2 * 128 * 128, 128 * 128, 64, 1)), bnd.SDPA_ERR_INVALID, "overlap"),
    # Heads 64 rows apart with 128 rows per head.
    (_ext_db(stride=(2 * 128 * 128, 64 * 128, 128, 1)), bnd.SDPA_ERR_INVALID, "overlap"),
    (_ext_db(stride=(2 * 128 * 128, 128 * 128, 1 << 24, 1)), bnd.SDPA_ERR_UNSUPPORTED, "2 GiB"),
    (_ext_db(data=FAKE), bnd.SDPA_ERR_INVALID, "dbias overlaps"),
    (_ext_db(data=FAKE_OUT), bnd.SDPA_ERR_INVALID, "dbias overlaps dq"),
    (_ext_db(data=FAKE_WS), bnd.SDPA_ERR_INVALID, "dbias overlaps workspace"),
])
def test_backward_rejects_bad_bias_gradient(lib, ext, code, needle):
    test_backward_ext_rejects_bad_options(lib, ext, code, needle)


def test_bias_gradient_layouts_pass_validation(lib, monkeypatch):
    # Accepted layouts reach the launch (the hook then returns SDPA_ERR_HIP):
    # contiguous, a batch stride that B = 1 never uses, padded rows.  The
    # forward ignores dbias.
    monkeypatch.setenv("SDPA14_FAIL_LAUNCH", "1")
    for st in ((2 * 128 * 128, 128 * 128, 128, 1), (128 * 128, 128 * 128, 128, 1),
               (2 * 128 * 136, 128 * 136, 136, 1)):
        test_backward_ext_rejects_bad_options(lib, _ext_db(stride=st), bnd.SDPA_ERR_HIP, "")
    q, k, v, out = _t(), _t(), _t(), _t(data=FAKE_OUT)
    s_, o_ = ctypes.c_uint64(), ctypes.c_uint64()
    rc = lib.sdpa_fwd_ext(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0.1, 1, math.nan,
                          ctypes.byref(out), FAKE_LSE, ctypes.byref(s_), ctypes.byref(o_),
                          ctypes.byref(_ext_db(data=FAKE)), None)
    assert rc == bnd.SDPA_ERR_HIP, _err(lib)


def test_workspace_size():
    # 8 bytes per query row (D and the base-2 LSE), rounded up to 256 bytes.
    assert sdpa.sdpa_bwd_workspace_size(1, 2, 128) == 2048
    assert sdpa.sdpa_bwd_workspace_size(1, 1, 1) == 256
    assert sdpa.sdpa_bwd_workspace_size(2, 12, 1024) == 2 * 12 * 1024 * 8
    assert sdpa.sdpa_bwd_workspace_size(3, 5, 77) == (3 * 5 * 77 * 8 + 255) // 256 * 256
    assert sdpa.sdpa_bwd_workspace_size(0, 1, 1) == 0


def test_slice_too_large_is_unsupported(lib):
    # Rows of one (batch, head) slice must sit within 2 GiB (32-bit buffer offsets).
    big = _t(B=1, H=1, S=2**20, E=64, stride=(2**20 * 2048, 2**20 * 2048, 2048, 1))
    rc = _fwd(lib, q=big, k=_t(B=1, H=1), v=_t(B=1, H=1), out=_t(B=1, H=1, S=2**20, stride=(2**20 * 2048, 2**20 * 2048, 2048, 1)))
    assert rc == bnd.SDPA_ERR_UNSUPPORTED and "2 GiB" in _err(lib)


def test_rng_state_roundtrip():
    sdpa.sdpa_set_rng_state(2**64 - 1, 2**63 + 5)
    assert sdpa.sdpa_get_rng_state() == (2**64 - 1, 2**63 + 5)
    sdpa.sdpa_set_rng_state(0, 0)
    assert sdpa.sdpa_get_rng_state() == (0, 0)


def test_status_strings(lib):
    assert lib.sdpa_status_string(0) == b"SDPA_OK"
    assert lib.sdpa_status_string(3) == b"SDPA_ERR_WORKSPACE"
    assert lib.sdpa_status_string(77) == b"SDPA_ERR_UNKNOWN"


def test_debug_mask_rejects_bad_arguments(lib):
    assert lib.sdpa_debug_dropout_mask(1, 2, 0.1, 1, 1, 4, 4, None, None) == bnd.SDPA_ERR_INVALID
    assert lib.sdpa_debug_dropout_mask(1, 2, 1.0, 1, 1, 4, 4, FAKE, None) == bnd.SDPA_ERR_INVALID
    assert lib.sdpa_debug_dropout_mask(1, 2, 0.1, 0, 1, 4, 4, FAKE, None) == bnd.SDPA_ERR_INVALID


def test_profile_kind_checked(lib):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.sdpa_profile_read(9, ctypes.byref(ms), ctypes.byref(n)) == bnd.SDPA_ERR_INVALID


def test_size_one_dims_ignore_strides(lib):
    # B = 1 with an odd batch stride is fine; it is never used.  The call then
    # fails only on the deliberately bad dropout argument, after stride checks.
    q = _t(B=1, stride=(3, 128 * 64, 64, 1))
    rc = _fwd(lib, q=q, p=2.0)
    assert rc == bnd.SDPA_ERR_INVALID and "dropout" in _err(lib)


def test_keep_bits_size():
    assert bnd.sdpa_keep_bits_size(2, 3, 5, 1000) == 2 * 3 * 5 * 32 * 4  # ceil(1000/32)=32 words
    assert bnd.sdpa_keep_bits_size(1, 1, 1, 33) == 4 * 4                # 2 words -> 4
    assert bnd.sdpa_keep_bits_size(1, 1, 1, 129) == 8 * 4               # 5 words -> 8
    assert bnd.sdpa_keep_bits_size(0, 1, 1, 1) == 0


def test_keep_bits_alignment_checked(lib):
    bnd.sdpa_set_rng_state(61, 62)
    ext = _ext()
    ext.keep_bits = FAKE + 8
    q, k, v, out = _t(), _t(), _t(), _t(data=FAKE_OUT)
    s, o = ctypes.c_uint64(), ctypes.c_uint64()
    rc = lib.sdpa_fwd_ext(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0.1, 1, math.nan,
                          ctypes.byref(out), FAKE_LSE, ctypes.byref(s), ctypes.byref(o),
                          ctypes.byref(ext), None)
    assert rc == bnd.SDPA_ERR_UNSUPPORTED and "keep_bits" in _err(lib)
    assert bnd.sdpa_get_rng_state() == (61, 62)


# ---- launch failures (SDPA_ERR_HIP) ------------------------------------------------


def test_forced_launch_failure_forward(lib, monkeypatch):
    # Valid arguments; the hook stands in for a launch the runtime refuses.  The
    # call must fail before any HIP call (there is no GPU here), leave the RNG
    # state as it was and say why.
    monkeypatch.setenv("SDPA14_FAIL_LAUNCH", "1")
    bnd.sdpa_set_rng_state(71, 72)
    rc = _fwd(lib, p=0.1)
    assert rc == bnd.SDPA_ERR_HIP, (rc, _err(lib))
    assert "SDPA14_FAIL_LAUNCH" in _err(lib) and "forward" in _err(lib)
    assert bnd.sdpa_get_rng_state() == (71, 72)
    with pytest.raises(bnd.SdpaError, match="SDPA_ERR_HIP: forward launch"):
        bnd._check(rc)


def test_forced_launch_failure_backward_and_mask(lib, monkeypatch):
    monkeypatch.setenv("SDPA14_FAIL_LAUNCH", "yes")
    bnd.sdpa_set_rng_state(73, 74)
    rc = _bwd(lib, p=0.1)
    assert rc == bnd.SDPA_ERR_HIP and "backward" in _err(lib)
    with pytest.raises(bnd.SdpaError, match="backward launch"):
        bnd._check(rc)
    rc = lib.sdpa_debug_dropout_mask(1, 2, 0.1, 1, 1, 4, 4, FAKE, None)
    assert rc == bnd.SDPA_ERR_HIP and "mask" in _err(lib)
    assert bnd.sdpa_get_rng_state() == (73, 74)


def test_forced_launch_failure_comes_after_validation(lib, monkeypatch):
    # An invalid call still reports its own error, not the launch failure.
    monkeypatch.setenv("SDPA14_FAIL_LAUNCH", "1")
    rc = _fwd(lib, p=1.0)
    assert rc == bnd.SDPA_ERR_INVALID and "dropout" in _err(lib)


def test_launch_failure_hook_off_when_zero(lib, monkeypatch):
    # "0" disables the hook; the call then fails only on its bad argument.
    monkeypatch.setenv("SDPA14_FAIL_LAUNCH", "0")
    rc = _fwd(lib, p=-1.0)
    assert rc == bnd.SDPA_ERR_INVALID


@pytest.mark.parametrize("rc,exc", [
    (bnd.SDPA_ERR_INVALID, ValueError),
    (bnd.SDPA_ERR_WORKSPACE, ValueError),
    (bnd.SDPA_ERR_UNSUPPORTED, NotImplementedError),
    (bnd.SDPA_ERR_HIP, bnd.SdpaError),
])
def test_status_maps_to_python_exception(lib, rc, exc):
    with pytest.raises(exc):
        bnd._check(rc)


# ---- the Python binding checks devices before calling the library ----------------


class _NoLibrary:
    """Stands in for the loaded library: any use of it fails the test."""

    def __getattr__(self, name):
        raise AssertionError(f"library function {name} was reached")


@pytest.fixture
def no_library(monkeypatch):
    monkeypatch.setattr(bnd, "_lib", _NoLibrary())


def _host_inputs(S=64, E=64):
    import torch

    g = torch.Generator("cpu").manual_seed(0)
    return [torch.randn((1, 2, S, E), generator=g).to(torch.bfloat16) for _ in range(4)]


def test_host_tensors_rejected_before_the_library(no_library):
    import torch

    q, k, v, do = _host_inputs()
    with pytest.raises(ValueError, match="GPU"):
        sdpa.sdpa_fwd(q, k, v, 0.0, True)
    with pytest.raises(ValueError, match="GPU"):
        sdpa.sdpa_fwd_ext(q, k, v, 0.0, True, need_lse=False)
    lse = torch.zeros((1, 2, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        sdpa.sdpa_bwd(do, q, k, v, q, lse, 0.0, True, 0, 0)
    with pytest.raises(ValueError, match="GPU"):
        sdpa.sdpa_bwd_ext(do, q, k, v, q, lse, 0.0, True)


def test_describe_rejects_host_and_meta_tensors():
    import torch

    with pytest.raises(ValueError, match="GPU"):
        bnd.describe(torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        bnd.describe(torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="meta"))


# ---- outputs must not overlap inputs -------------------------------------------


def test_forward_output_overlapping_an_input_is_rejected(lib):
    bnd.sdpa_set_rng_state(91, 92)
    assert _fwd(lib, out=_t(data=FAKE)) == bnd.SDPA_ERR_INVALID
    assert "out overlaps q" in _err(lib)
    assert _fwd(lib, lse=FAKE + 4096) == bnd.SDPA_ERR_INVALID and "lse overlaps" in _err(lib)
    # out and lse must not overlap each other either.
    assert _fwd(lib, lse=FAKE_OUT + 64) == bnd.SDPA_ERR_INVALID and "overlaps lse" in _err(lib)
    assert bnd.sdpa_get_rng_state() == (91, 92)


def test_backward_gradients_overlapping_inputs_or_workspace_are_rejected(lib):
    assert _bwd(lib, dq=_t(data=FAKE)) == bnd.SDPA_ERR_INVALID and "dq overlaps" in _err(lib)
    assert _bwd(lib, dv=_t(data=FAKE_LSE)) == bnd.SDPA_ERR_INVALID and "dv overlaps lse" in _err(lib)
    assert _bwd(lib, ws=FAKE) == bnd.SDPA_ERR_INVALID and "workspace overlaps" in _err(lib)
    assert _bwd(lib, ws=FAKE_OUT + 1024) == bnd.SDPA_ERR_INVALID and "workspace overlaps dq" in _err(lib)


def test_packed_views_pass_the_overlap_check(lib, monkeypatch):
    # q, k, v as interleaved views of one packed [B, S, 3, H, E] buffer, and
    # dq, dk, dv as views of another: shared memory within the inputs or within
    # the gradients is fine.  With the launch hook set, a call that passes
    # validation returns SDPA_ERR_HIP.
    monkeypatch.setenv("SDPA14_FAIL_LAUNCH", "1")
    B, H, S, E = 1, 2, 128, 64
    st = (S * 3 * H * E, E, 3 * H * E, 1)
    qkv = [_t(B, H, S, E, data=FAKE + i * H * E * 2, stride=st) for i in range(3)]
    dqkv = [_t(B, H, S, E, data=FAKE_OUT + i * H * E * 2, stride=st) for i in range(3)]
    out = _t(B, H, S, E, data=FAKE_OUT + (1 << 33))
    rc = _fwd(lib, q=qkv[0], k=qkv[1], v=qkv[2], out=out)
    assert rc == bnd.SDPA_ERR_HIP, _err(lib)
    rc = _bwd(lib, q=qkv[0], k=qkv[1], v=qkv[2], out=out, dq=dqkv[0], dk=dqkv[1], dv=dqkv[2])
    assert rc == bnd.SDPA_ERR_HIP, _err(lib)
