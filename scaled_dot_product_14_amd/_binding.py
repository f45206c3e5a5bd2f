"""ctypes binding of libsdpa14.so, with the same names as the C ABI.

Argument marshalling only: every step of the attention runs in the HIP library.
PyTorch supplies device memory (``torch.empty*``) and the current stream.  If
the library is not built, every call raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libsdpa14.so")

SDPA_OK = 0
SDPA_ERR_INVALID = 1
SDPA_ERR_UNSUPPORTED = 2
SDPA_ERR_WORKSPACE = 3
SDPA_ERR_HIP = 4
SDPA_BF16 = 0
SDPA_F16 = 1

KERNEL_FWD = 0
KERNEL_BWD = 1       # backward main kernel
KERNEL_BWD_ROWS = 2  # backward row pass

EXPORTED = (
    "sdpa_fwd", "sdpa_bwd", "sdpa_fwd_ext", "sdpa_bwd_ext", "sdpa_bwd_workspace_size",
    "sdpa_keep_bits_size",
    "sdpa_set_rng_state",
    "sdpa_get_rng_state", "sdpa_status_string", "sdpa_last_error",
    "sdpa_debug_dropout_mask", "sdpa_profile_enable", "sdpa_profile_read",
    "sdpa_bwd_noalloc", "sdpa_bwd_noalloc_max_rows",
)


class SdpaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("size", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class SdpaExt(ctypes.Structure):
    _fields_ = [
        ("head_offset", ctypes.c_int64),
        ("heads_total", ctypes.c_int64),
        ("rng_state", ctypes.c_void_p),
        ("rng_used", ctypes.c_void_p),
        ("bias", ctypes.POINTER(SdpaTensor)),
        ("keep_bits", ctypes.c_void_p),
        ("bwd_parts", ctypes.c_int32),
        ("dbias", ctypes.POINTER(SdpaTensor)),
    ]


class SdpaError(RuntimeError):
    """Raised for SDPA_ERR_HIP; other codes map to ValueError / NotImplementedError."""


_lib = None


def load_library(path: str = LIB_PATH):
    """Load (once) and type the shared library.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python -m scaled_dot_product_14_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(SdpaTensor)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.sdpa_fwd.argtypes = [P, P, P, ctypes.c_double, ctypes.c_int, ctypes.c_double, P,
                             ctypes.c_void_p, u64p, u64p, ctypes.c_void_p]
    lib.sdpa_fwd.restype = ctypes.c_int
    lib.sdpa_bwd.argtypes = [P, P, P, P, P, ctypes.c_void_p, ctypes.c_double, ctypes.c_int,
                             ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, P, P, P,
                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.sdpa_bwd.restype = ctypes.c_int
    E = ctypes.POINTER(SdpaExt)
    lib.sdpa_fwd_ext.argtypes = [P, P, P, ctypes.c_double, ctypes.c_int, ctypes.c_double, P,
                                 ctypes.c_void_p, u64p, u64p, E, ctypes.c_void_p]
    lib.sdpa_fwd_ext.restype = ctypes.c_int
    lib.sdpa_bwd_ext.argtypes = [P, P, P, P, P, ctypes.c_void_p, ctypes.c_double, ctypes.c_int,
                                 ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, P, P, P,
                                 ctypes.c_void_p, ctypes.c_size_t, E, ctypes.c_void_p]
    lib.sdpa_bwd_ext.restype = ctypes.c_int
    lib.sdpa_bwd_noalloc.argtypes = [P, P, P, P, P, ctypes.c_void_p, ctypes.c_double,
                                     ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_double, P, P, P, E, ctypes.c_void_p]
    lib.sdpa_bwd_noalloc.restype = ctypes.c_int
    lib.sdpa_bwd_noalloc_max_rows.argtypes = []
    lib.sdpa_bwd_noalloc_max_rows.restype = ctypes.c_size_t
    lib.sdpa_keep_bits_size.argtypes = [ctypes.c_int64] * 4
    lib.sdpa_keep_bits_size.restype = ctypes.c_size_t
    lib.sdpa_bwd_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.sdpa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_set_rng_state.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.sdpa_set_rng_state.restype = None
    lib.sdpa_get_rng_state.argtypes = [u64p, u64p]
    lib.sdpa_get_rng_state.restype = None
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_debug_dropout_mask.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.sdpa_debug_dropout_mask.restype = ctypes.c_int
    lib.sdpa_profile_enable.argtypes = [ctypes.c_int]
    lib.sdpa_profile_enable.restype = ctypes.c_int
    lib.sdpa_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
    lib.sdpa_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc == SDPA_OK:
        return
    lib = load_library()
    msg = f"{lib.sdpa_status_string(rc).decode()}: {lib.sdpa_last_error().decode()}"
    if rc in (SDPA_ERR_INVALID, SDPA_ERR_WORKSPACE):
        raise ValueError(msg)
    if rc == SDPA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise SdpaError(msg)


def _on_device(t: torch.Tensor, device: torch.device | None, name: str) -> None:
    """The C side cannot tell host from device pointers: check here, before any call."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the device of q)")


def describe(t: torch.Tensor, device: torch.device | None = None,
             name: str = "tensor") -> SdpaTensor:
    """C descriptor of a 4-D device tensor (logical [B, H, S, E], strides in elements).

    ``device``, when given, is the device every tensor of the call must be on.
    """
    _on_device(t, device, name)
    if t.dim() != 4:
        raise ValueError(f"expected a 4-D [B, H, S, E] tensor, got shape {tuple(t.shape)}")
    d = SdpaTensor()
    d.data = t.data_ptr()
    d.dtype = {torch.bfloat16: SDPA_BF16, torch.float16: SDPA_F16}.get(t.dtype, -1)
    for i in range(4):
        d.size[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _check_lse(lse, q: torch.Tensor) -> None:
    """lse: contiguous float32 [B, H, Sq] on q's device."""
    _on_device(lse, q.device, "lse")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")


def _check_workspace(ws, q: torch.Tensor) -> None:
    _on_device(ws, q.device, "workspace")
    if not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _scale_arg(scale) -> float:
    return math.nan if scale is None else float(scale)


def sdpa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dropout_p: float = 0.0,
             is_causal: bool = False, scale=None, out: torch.Tensor | None = None,
             lse: torch.Tensor | None = None):
    """Forward: returns ``(out, lse, seed, offset)``.

    ``out`` defaults to ``torch.empty_like(q)`` (q's stride order) and ``lse``
    to a contiguous fp32 ``[B, H, Sq]`` tensor.
    """
    lib = load_library()
    _on_device(q, None, "q")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check_lse(lse, q)
    dev = q.device
    dq_, dk_, dv_, do_ = (describe(t, dev, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")))
    seed, offset = ctypes.c_uint64(), ctypes.c_uint64()
    with torch.cuda.device(q.device):
        rc = lib.sdpa_fwd(ctypes.byref(dq_), ctypes.byref(dk_), ctypes.byref(dv_),
                          float(dropout_p), int(bool(is_causal)), _scale_arg(scale),
                          ctypes.byref(do_), lse.data_ptr(), ctypes.byref(seed),
                          ctypes.byref(offset), _stream(q.device))
    _check(rc)
    return out, lse, seed.value, offset.value


def sdpa_bwd_workspace_size(B: int, H: int, Sq: int) -> int:
    """Bytes of device workspace ``sdpa_bwd`` needs for ``B*H*Sq`` query rows."""
    return int(load_library().sdpa_bwd_workspace_size(int(B), int(H), int(Sq)))


def sdpa_bwd(dout, q, k, v, out, lse, dropout_p: float, is_causal: bool, seed: int,
             offset: int, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward: returns ``(dq, dk, dv)`` laid out like q, k, v.

    ``workspace`` (optional) is a device uint8 tensor of at least
    ``sdpa_bwd_workspace_size(B, H, Sq)`` bytes; one is allocated when omitted.
    """
    lib = load_library()
    _on_device(q, None, "q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    B, H, Sq = q.shape[0], q.shape[1], q.shape[2]
    _check_lse(lse, q)
    if workspace is None:
        workspace = torch.empty(max(lib.sdpa_bwd_workspace_size(B, H, Sq), 256),
                                dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    descs = [describe(t, q.device, n) for t, n in zip(
        (dout, q, k, v, out, dq, dk, dv), ("dout", "q", "k", "v", "out", "dq", "dk", "dv"))]
    with torch.cuda.device(q.device):
        rc = lib.sdpa_bwd(*(ctypes.byref(d) for d in descs[:5]), lse.data_ptr(),
                          float(dropout_p), int(bool(is_causal)), int(seed), int(offset),
                          _scale_arg(scale), *(ctypes.byref(d) for d in descs[5:]),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream(q.device))
    _check(rc)
    return dq, dk, dv


def _rng_buffer(t, name: str, device=None):
    if t is None:
        return None
    _on_device(t, device, name)
    if not (t.dtype in (torch.int64, torch.uint64) and t.numel() == 2 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device int64 tensor of 2 elements "
                         "(seed, offset)")
    return t.data_ptr()


def sdpa_keep_bits_size(B: int, H: int, Sq: int, Sk: int) -> int:
    """Bytes of the dropout keep-bit cache ``sdpa_fwd_ext``/``sdpa_bwd_ext`` can share."""
    return int(load_library().sdpa_keep_bits_size(int(B), int(H), int(Sq), int(Sk)))


def _ext(head_offset, heads_total, rng_state, rng_used, bias=None, shape=None, keep_bits=None,
         device=None, bwd_parts=0, dbias=None):
    """The options block and the objects it points into (keep both alive for the call)."""
    e = SdpaExt()
    e.bwd_parts = int(bwd_parts)
    if keep_bits is not None:
        _on_device(keep_bits, device, "keep_bits")
        if not keep_bits.is_contiguous():
            raise ValueError("keep_bits must be a contiguous device tensor")
        e.keep_bits = keep_bits.data_ptr()
    e.head_offset = int(head_offset)
    e.heads_total = int(heads_total)
    e.rng_state = _rng_buffer(rng_state, "rng_state", device)
    e.rng_used = _rng_buffer(rng_used, "rng_used", device)
    keep = None
    if bias is not None:
        if bias.dim() > 4:
            raise ValueError("bias must broadcast to [B, H, Sq, Sk]")
        full = bias.expand(*shape)  # broadcast dimensions get stride 0
        desc = describe(full, device, "bias")
        e.bias = ctypes.pointer(desc)
        keep = (full, desc)
    if dbias is not None:
        ddesc = describe(dbias, device, "dbias")
        e.dbias = ctypes.pointer(ddesc)
        keep = (keep, ddesc)
    return e, keep


def sdpa_fwd_ext(q, k, v, dropout_p: float = 0.0, is_causal: bool = False, scale=None,
                 out=None, lse=None, *, head_offset: int = 0, heads_total: int = 0,
                 rng_state=None, rng_used=None, bias=None, need_lse: bool = True,
                 keep_bits=None):
    """Forward with options: returns ``(out, lse, seed, offset)``.

    ``head_offset`` / ``heads_total`` place the call's heads in a larger problem
    for the dropout stream.  ``rng_state`` and ``rng_used`` (device int64
    tensors of two elements, {seed, offset}) keep the RNG state on the device;
    then ``seed`` and ``offset`` are returned as None and the values the call
    used land in ``rng_used``.  ``bias`` (bf16, broadcastable to
    [B, H, Sq, Sk], key dimension contiguous) is added to the scaled scores.
    ``need_lse=False`` runs the inference-only forward: no log-sum-exp is
    written and ``lse`` is returned as None.  ``keep_bits`` (a device buffer of
    ``sdpa_keep_bits_size`` bytes) receives the dropout keep bits for a backward.
    """
    lib = load_library()
    _on_device(q, None, "q")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and need_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if need_lse:
        _check_lse(lse, q)
    else:
        lse = None
    dev = q.device
    dq_, dk_, dv_, do_ = (describe(t, dev, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")))
    ext, _keep = _ext(head_offset, heads_total, rng_state, rng_used, bias,
                      (q.shape[0], q.shape[1], q.shape[2], k.shape[2]), keep_bits, dev)
    seed, offset = ctypes.c_uint64(), ctypes.c_uint64()
    with torch.cuda.device(q.device):
        rc = lib.sdpa_fwd_ext(ctypes.byref(dq_), ctypes.byref(dk_), ctypes.byref(dv_),
                              float(dropout_p), int(bool(is_causal)), _scale_arg(scale),
                              ctypes.byref(do_), None if lse is None else lse.data_ptr(),
                              ctypes.byref(seed),
                              ctypes.byref(offset), ctypes.byref(ext), _stream(q.device))
    _check(rc)
    if rng_state is not None:
        return out, lse, None, None
    return out, lse, seed.value, offset.value


def sdpa_bwd_ext(dout, q, k, v, out, lse, dropout_p: float, is_causal: bool, seed: int = 0,
                 offset: int = 0, scale=None, dq=None, dk=None, dv=None, workspace=None, *,
                 head_offset: int = 0, heads_total: int = 0, rng_used=None, bias=None,
                 keep_bits=None, bwd_parts: int = 0, dbias=None):
    """Backward with options (see ``sdpa_fwd_ext``): returns ``(dq, dk, dv)``.

    With ``rng_used`` the kernels read (seed, offset) from that device tensor
    and ``seed`` / ``offset`` are ignored.  ``bwd_parts`` picks the kernels to
    enqueue: 1 the row pass (fills ``workspace``), 2 the main kernel (reads a
    workspace a row pass filled), 0 or 3 both.  ``dbias`` (a [B, H, Sq, Sk]
    tensor of q's dtype, needs ``bias``) receives the bias gradient of every
    head; sum it over the dimensions the bias broadcasts.
    """
    lib = load_library()
    _on_device(q, None, "q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    B, H, Sq = q.shape[0], q.shape[1], q.shape[2]
    _check_lse(lse, q)
    if workspace is None:
        workspace = torch.empty(max(lib.sdpa_bwd_workspace_size(B, H, Sq), 256),
                                dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    descs = [describe(t, q.device, n) for t, n in zip(
        (dout, q, k, v, out, dq, dk, dv), ("dout", "q", "k", "v", "out", "dq", "dk", "dv"))]
    ext, _keep = _ext(head_offset, heads_total, None, rng_used, bias,
                      (q.shape[0], q.shape[1], q.shape[2], k.shape[2]), keep_bits, q.device,
                      bwd_parts, dbias)
    with torch.cuda.device(q.device):
        rc = lib.sdpa_bwd_ext(*(ctypes.byref(d) for d in descs[:5]), lse.data_ptr(),
                              float(dropout_p), int(bool(is_causal)), int(seed), int(offset),
                              _scale_arg(scale), *(ctypes.byref(d) for d in descs[5:]),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              ctypes.byref(ext), _stream(q.device))
    _check(rc)
    return dq, dk, dv


def sdpa_set_rng_state(seed: int, offset: int) -> None:
    load_library().sdpa_set_rng_state(int(seed), int(offset))


def sdpa_get_rng_state():
    s, o = ctypes.c_uint64(), ctypes.c_uint64()
    load_library().sdpa_get_rng_state(ctypes.byref(s), ctypes.byref(o))
    return s.value, o.value


def sdpa_debug_dropout_mask(seed: int, offset: int, dropout_p: float, B: int, H: int, Sq: int,
                            Sk: int, device="cuda"):
    """The keep mask the kernels use, as a uint8 [B, H, Sq, Sk] device tensor."""
    lib = load_library()
    mask = torch.empty((B, H, Sq, Sk), dtype=torch.uint8, device=device)
    with torch.cuda.device(mask.device):
        rc = lib.sdpa_debug_dropout_mask(int(seed), int(offset), float(dropout_p), B, H, Sq, Sk,
                                         mask.data_ptr(), _stream(mask.device))
    _check(rc)
    return mask


def sdpa_profile_enable(on: bool) -> None:
    _check(load_library().sdpa_profile_enable(int(bool(on))))


def sdpa_profile_read(kind: int):
    """(total_ms, launches) of one kernel kind since the last read; waits for the events."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load_library().sdpa_profile_read(int(kind), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def sdpa_bwd_noalloc_max_rows() -> int:
    """Largest B*H*Sq the allocation-free backward accepts."""
    return int(load_library().sdpa_bwd_noalloc_max_rows())


def sdpa_bwd_noalloc(dout, q, k, v, out, lse, dropout_p: float, is_causal: bool, seed: int,
                     offset: int, scale, dq, dk, dv, *, head_offset: int = 0,
                     heads_total: int = 0, rng_used=None, bias=None, keep_bits=None, dbias=None):
    """Backward that allocates nothing: the caller passes dq, dk, dv and the
    library uses its own device-resident scratch for the row pass.  Returns
    ``(dq, dk, dv)``.  Calls that overlap on one device race (shared scratch)."""
    lib = load_library()
    _on_device(q, None, "q")
    _check_lse(lse, q)
    descs = [describe(t, q.device, n) for t, n in zip(
        (dout, q, k, v, out, dq, dk, dv), ("dout", "q", "k", "v", "out", "dq", "dk", "dv"))]
    ext, _keep = _ext(head_offset, heads_total, None, rng_used, bias,
                      (q.shape[0], q.shape[1], q.shape[2], k.shape[2]), keep_bits, q.device,
                      0, dbias)
    with torch.cuda.device(q.device):
        rc = lib.sdpa_bwd_noalloc(*(ctypes.byref(d) for d in descs[:5]), lse.data_ptr(),
                                  float(dropout_p), int(bool(is_causal)), int(seed), int(offset),
                                  _scale_arg(scale), *(ctypes.byref(d) for d in descs[5:]),
                                  ctypes.byref(ext), _stream(q.device))
    _check(rc)
    return dq, dk, dv
