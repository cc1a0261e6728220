"""Mamba-2 SSD chunked-scan forward on MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/ssd.h`` (``libssd_mi355x.so``,
built in-tree by ``mamba_ssd_scan_chunked_amd.build``).  PyTorch only supplies
device memory and the current stream; every step of the computation runs in
the library's HIP kernels.  There is no CPU fallback: if the library is not
built, or no GPU is present, the calls raise.

    y, final = forward(x, dt, A_log, B, C, D=None, chunk_len=256,
                       init_state=None, seq_idx=None, nseqs=None,
                       dt_bias=None, dt_softplus=False, zoh=False)

Layouts: x (b,T,H,P) bf16|f32, dt (b,T,H) f32, A_log (H) f32, B/C (b,T,G,N) same
dtype as x, D (H) f32, init_state (nseqs,H,P,N) f32, seq_idx (b,T) int32,
dt_bias (H) f32.
Outputs: y (b,T,H,P) f32 and final_state (nseqs,H,P,N) f32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = ["forward", "forward_into", "forward_into_noalloc", "noalloc_scratch_bytes", "step", "backward", "backward_into", "backward_workspace_size", "workspace_size", "validate", "problem", "SSDError",
           "version", "library_path", "load_library", "DTYPE_F32", "DTYPE_BF16", "FLAG_DT_SCALES_X",
           "FLAG_DT_SOFTPLUS", "FLAG_ZOH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libssd_mi355x.so"

DTYPE_F32 = 0
DTYPE_BF16 = 1
FLAG_DT_SCALES_X = 1
FLAG_DT_SOFTPLUS = 2
FLAG_ZOH = 4
ABI_VERSION = 5

SSD_OK = 0
ERROR_NAMES = {1: "NULL_POINTER", 2: "BAD_SHAPE", 3: "UNSUPPORTED", 4: "ALIGNMENT", 5: "WORKSPACE",
               6: "ALIAS", 7: "HIP", 8: "NO_DEVICE", 9: "SCRATCH"}


class SSDError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("ssd error %d (%s): %s" % (code, ERROR_NAMES.get(code, "?"), msg))
        self.code = code


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk_len", ctypes.c_int64), ("nseqs", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("segments", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libssd_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError("%s is not built; run `python -m mamba_ssd_scan_chunked_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.ssd_validate.argtypes = [P]
    lib.ssd_validate.restype = ctypes.c_int
    lib.ssd_step.argtypes = [P] + [vp] * 10
    lib.ssd_step.restype = ctypes.c_int
    lib.ssd_workspace_size.argtypes = [P]
    lib.ssd_workspace_size.restype = sz
    lib.ssd_forward.argtypes = [P] + [vp] * 11 + [vp, sz, vp]
    lib.ssd_forward.restype = ctypes.c_int
    lib.ssd_forward_noalloc.argtypes = [P] + [vp] * 12
    lib.ssd_forward_noalloc.restype = ctypes.c_int
    lib.ssd_noalloc_scratch_bytes.argtypes = []
    lib.ssd_noalloc_scratch_bytes.restype = sz
    lib.ssd_backward_workspace_size.argtypes = [P]
    lib.ssd_backward_workspace_size.restype = sz
    lib.ssd_backward.argtypes = [P] + [vp] * 19 + [vp, sz, vp]
    lib.ssd_backward.restype = ctypes.c_int
    lib.ssd_strerror.argtypes = [ctypes.c_int]
    lib.ssd_strerror.restype = ctypes.c_char_p
    lib.ssd_version.restype = ctypes.c_int
    if lib.ssd_version() != ABI_VERSION:
        raise ImportError("%s has ABI %d, this binding needs %d: rebuild it" % (path, lib.ssd_version(), ABI_VERSION))
    _lib = lib
    return lib


def version() -> int:
    return int(load_library().ssd_version())


def _check(code: int):
    if code != SSD_OK:
        raise SSDError(code, load_library().ssd_strerror(code).decode())


def problem(batch, seqlen, nheads, headdim, dstate, ngroups=1, chunk_len=256, nseqs=None,
            dtype=DTYPE_BF16, flags=0, segments=0) -> Problem:
    """A problem description.  ``segments`` > 0 forces the number of segments each
    row is cut into on the split-row path (0: the library's choice); it does not
    change the result."""
    return Problem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len,
                   batch if nseqs is None else nseqs, dtype, flags, segments, 0)


def validate(p: Problem) -> int:
    return int(load_library().ssd_validate(ctypes.byref(p)))


def workspace_size(p: Problem) -> int:
    return int(load_library().ssd_workspace_size(ctypes.byref(p)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_of(device, stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _describe(x, B, dt, A_log, chunk_len, seq_idx, nseqs, dt_scales_x, dt_softplus=False, zoh=False, segments=0):
    import torch
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be (b,T,H,P) and B, C (b,T,G,N)")
    b, T, H, Pd = x.shape
    G, N = B.shape[2], B.shape[3]
    if x.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
    elif x.dtype == torch.float32:
        dtype = DTYPE_F32
    else:
        raise TypeError("x must be bfloat16 or float32")
    if seq_idx is None:
        ns = b
    else:
        if nseqs is None:
            raise ValueError("nseqs is required with seq_idx (it sizes final_state)")
        ns = int(nseqs)
    flags = (FLAG_DT_SCALES_X if dt_scales_x else 0) | (FLAG_DT_SOFTPLUS if dt_softplus else 0) | \
        (FLAG_ZOH if zoh else 0)
    return problem(b, T, H, Pd, N, G, chunk_len, ns, dtype, flags, segments)


def _check_tensors(x, dt, A_log, B, C, D, init_state, seq_idx, dt_bias=None):
    import torch
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for name, t, dt_ in (("dt", dt, torch.float32), ("A_log", A_log, torch.float32), ("D", D, torch.float32),
                         ("dt_bias", dt_bias, torch.float32),
                         ("init_state", init_state, torch.float32), ("seq_idx", seq_idx, torch.int32),
                         ("B", B, x.dtype), ("C", C, x.dtype)):
        if t is None:
            continue
        if t.device != dev:
            raise ValueError("%s is on %s, x on %s" % (name, t.device, dev))
        if t.dtype != dt_:
            raise TypeError("%s must be %s, got %s" % (name, dt_, t.dtype))
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, T, H) or tuple(A_log.shape) != (H,):
        raise ValueError("dt must be (b,T,H) and A_log (H,)")
    if tuple(B.shape) != (b, T, G, N) or tuple(C.shape) != (b, T, G, N):
        raise ValueError("B and C must be (b,T,G,N)")
    if D is not None and tuple(D.shape) != (H,):
        raise ValueError("D must be (H,)")
    if dt_bias is not None and tuple(dt_bias.shape) != (H,):
        raise ValueError("dt_bias must be (H,)")
    if seq_idx is not None and tuple(seq_idx.shape) != (b, T):
        raise ValueError("seq_idx must be (b,T)")


def _check_buffer(name, t, shape, dtype, dev):
    """A caller-supplied output must be exactly what the kernels write into: the C
    ABI takes bare pointers and cannot see a short, strided or mistyped buffer."""
    if t.device != dev:
        raise ValueError("%s is on %s, x on %s" % (name, t.device, dev))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_workspace(ws, nbytes, dev):
    if nbytes == 0:
        return
    if ws is None:
        raise ValueError("this problem needs a workspace of %d bytes" % nbytes)
    import torch
    if ws.device != dev or not ws.is_contiguous() or ws.dtype != torch.uint8:
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    if ws.numel() < nbytes:
        raise ValueError("workspace holds %d bytes, the problem needs %d" % (ws.numel(), nbytes))


def forward(x, dt, A_log, B, C, D=None, chunk_len: int = 256, init_state=None, seq_idx=None,
            nseqs: Optional[int] = None, dt_scales_x: bool = False, y=None, final_state=None,
            workspace=None, return_final: bool = True, stream=None, dt_bias=None, dt_softplus: bool = False,
            zoh: bool = False, segments: int = 0):
    """SSD forward through ``ssd_forward``.  Returns (y, final_state or None).

    The step size is dt + dt_bias (dt_bias None = 0), through softplus when
    ``dt_softplus``; x is written to the state unscaled, times the step size
    (``dt_scales_x``) or times the exact zero-order hold (exp(step A) - 1) / A
    (``zoh``).  ``segments`` > 0 forces the number of segments per row on the
    split-row path (a scheduling choice; 0: the library's)."""
    import torch
    _check_tensors(x, dt, A_log, B, C, D, init_state, seq_idx, dt_bias)
    in_place = final_state is not None and init_state is not None and final_state is init_state
    if in_place and not init_state.is_contiguous():
        raise ValueError("an init_state that is also final_state must be contiguous (it is updated in place)")
    x, dt, A_log, B, C = (t.contiguous() for t in (x, dt, A_log, B, C))
    D = D.contiguous() if D is not None else None
    dt_bias = dt_bias.contiguous() if dt_bias is not None else None
    init_state = init_state.contiguous() if init_state is not None else None
    seq_idx = seq_idx.contiguous() if seq_idx is not None else None
    p = _describe(x, B, dt, A_log, chunk_len, seq_idx, nseqs, dt_scales_x, dt_softplus, zoh, segments)
    lib = load_library()
    _check(lib.ssd_validate(ctypes.byref(p)))
    dev = x.device
    b, T, H, P = x.shape
    N = B.shape[3]
    if init_state is not None and tuple(init_state.shape) != (p.nseqs, H, P, N):
        raise ValueError("init_state must be (nseqs,H,P,N)")
    if y is None:
        y = torch.empty((b, T, H, P), dtype=torch.float32, device=dev)
    else:
        _check_buffer("y", y, (b, T, H, P), torch.float32, dev)
    if final_state is None and return_final:
        final_state = torch.empty((p.nseqs, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check_buffer("final_state", final_state, (p.nseqs, H, P, N), torch.float32, dev)
    wsb = int(lib.ssd_workspace_size(ctypes.byref(p)))
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, wsb, dev)
    forward_into(p, x, dt, A_log, B, C, D, init_state, seq_idx, y, final_state, workspace, stream, dt_bias)
    return y, final_state


def forward_into(p: Problem, x, dt, A_log, B, C, D, init_state, seq_idx, y, final_state, workspace=None,
                 stream=None, dt_bias=None):
    """``ssd_forward`` on caller-provided contiguous tensors and problem description
    (``workspace`` may be None when :func:`workspace_size` is 0).  Only the sizes of
    the outputs and the workspace are checked here, since the library cannot see
    them; everything else is the library's own validation."""
    import torch
    dev = y.device
    _check_buffer("y", y, (p.batch, p.seqlen, p.nheads, p.headdim), torch.float32, dev)
    if final_state is not None:
        _check_buffer("final_state", final_state, (p.nseqs, p.nheads, p.headdim, p.dstate), torch.float32, dev)
    _check_workspace(workspace, workspace_size(p), dev)
    wsn = workspace.numel() if workspace is not None else 0
    _check(load_library().ssd_forward(ctypes.byref(p), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(init_state), _ptr(seq_idx), _ptr(y), _ptr(final_state),
                                      _ptr(workspace), wsn, _stream_of(x.device, stream)))


def noalloc_scratch_bytes() -> int:
    return int(load_library().ssd_noalloc_scratch_bytes())


def forward_into_noalloc(p: Problem, x, dt, A_log, B, C, D, init_state, seq_idx, y, final_state, stream=None,
                         dt_bias=None):
    """``ssd_forward_noalloc`` on caller-provided contiguous tensors: :func:`forward_into`
    without a workspace (the library's static scratch array stands in for it)."""
    import torch
    dev = y.device
    _check_buffer("y", y, (p.batch, p.seqlen, p.nheads, p.headdim), torch.float32, dev)
    if final_state is not None:
        _check_buffer("final_state", final_state, (p.nseqs, p.nheads, p.headdim, p.dstate), torch.float32, dev)
    _check(load_library().ssd_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log),
                                              _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), _ptr(seq_idx), _ptr(y),
                                              _ptr(final_state), _stream_of(x.device, stream)))


def step(x, dt, A_log, B, C, D, state, y=None, dt_scales_x: bool = False, stream=None, dt_bias=None,
         dt_softplus: bool = False, zoh: bool = False):
    """``ssd_step``: one token per (row, head).  x (b,1,H,P) or (b,H,P), dt (b,1,H) or
    (b,H), B/C (b,1,G,N) or (b,G,N); ``state`` (b,H,P,N) fp32 is updated in place.
    Returns y (b,1,H,P) fp32."""
    import torch
    b = x.shape[0]
    H, P = x.shape[-2], x.shape[-1]
    G, N = B.shape[-2], B.shape[-1]
    x = x.reshape(b, 1, H, P).contiguous()
    dt = dt.reshape(b, 1, H).contiguous()
    B = B.reshape(b, 1, G, N).contiguous()
    C = C.reshape(b, 1, G, N).contiguous()
    _check_tensors(x, dt, A_log, B, C, D, state, None, dt_bias)
    if not state.is_contiguous() or tuple(state.shape) != (b, H, P, N) or state.dtype != torch.float32:
        raise ValueError("state must be a contiguous fp32 (b,H,P,N) tensor")
    p = _describe(x, B, dt, A_log, 64, None, None, dt_scales_x, dt_softplus, zoh)
    if y is None:
        y = torch.empty((b, 1, H, P), dtype=torch.float32, device=x.device)
    else:
        _check_buffer("y", y.view(b, 1, H, P) if y.is_contiguous() and y.numel() == b * H * P else y,
                      (b, 1, H, P), torch.float32, x.device)
    _check(load_library().ssd_step(ctypes.byref(p), _ptr(x), _ptr(dt),
                                   _ptr(dt_bias.contiguous() if dt_bias is not None else None), _ptr(A_log.contiguous()), _ptr(B), _ptr(C),
                                   _ptr(D.contiguous() if D is not None else None), _ptr(state), _ptr(y),
                                   _stream_of(x.device, stream)))
    return y


def backward_workspace_size(p: Problem) -> int:
    return int(load_library().ssd_backward_workspace_size(ctypes.byref(p)))


def backward(x, dt, A_log, B, C, dy, D=None, init_state=None, dfinal=None, chunk_len: int = 256,
             dt_scales_x: bool = False, dt_bias=None, dt_softplus: bool = False, zoh: bool = False,
             workspace=None, stream=None, seq_idx=None, nseqs: Optional[int] = None, segments: int = 0):
    """Gradients through ``ssd_backward`` of L = <dy, y> + <dfinal, final_state> for the
    forward map of :func:`forward` with the same arguments.  Returns a dict of fp32
    tensors: dx, ddt, dA_log, dB, dC, dD, dinit, ddt_bias (dD, dinit and ddt_bias are
    the gradients at D = 0, a zero initial state and a zero bias when those were not
    given).  With ``seq_idx`` (and ``nseqs``) the rows are packed sequences as in
    :func:`forward`; dfinal and dinit are then per sequence."""
    import torch
    _check_tensors(x, dt, A_log, B, C, D, init_state, seq_idx, dt_bias)
    x, dt, A_log, B, C = (t.contiguous() for t in (x, dt, A_log, B, C))
    D = D.contiguous() if D is not None else None
    dt_bias = dt_bias.contiguous() if dt_bias is not None else None
    init_state = init_state.contiguous() if init_state is not None else None
    seq_idx = seq_idx.contiguous() if seq_idx is not None else None
    p = _describe(x, B, dt, A_log, chunk_len, seq_idx, nseqs, dt_scales_x, dt_softplus, zoh, segments)
    lib = load_library()
    _check(lib.ssd_validate(ctypes.byref(p)))
    b, T, H, P = x.shape
    ns = p.nseqs
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    if tuple(dy.shape) != (b, T, H, P) or dy.dtype != torch.float32 or dy.device != dev:
        raise ValueError("dy must be an fp32 (b,T,H,P) tensor on the device of x")
    dy = dy.contiguous()
    if dfinal is not None:
        if tuple(dfinal.shape) != (ns, H, P, N) or dfinal.dtype != torch.float32 or dfinal.device != dev:
            raise ValueError("dfinal must be an fp32 (nseqs,H,P,N) tensor on the device of x")
        dfinal = dfinal.contiguous()
    if init_state is not None and tuple(init_state.shape) != (ns, H, P, N):
        raise ValueError("init_state must be (nseqs,H,P,N)")
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty((b, T, H, P), **f32), "ddt": torch.empty((b, T, H), **f32),
           "dA_log": torch.empty((H,), **f32), "dB": torch.empty((b, T, G, N), **f32),
           "dC": torch.empty((b, T, G, N), **f32), "dD": torch.empty((H,), **f32),
           "dinit": torch.empty((ns, H, P, N), **f32), "ddt_bias": torch.empty((H,), **f32)}
    wsb = backward_workspace_size(p)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    backward_into(p, x, dt, dt_bias, A_log, B, C, D, init_state, dy, dfinal, out, workspace, stream, seq_idx)
    return out


def backward_into(p: Problem, x, dt, dt_bias, A_log, B, C, D, init_state, dy, dfinal, out: dict, workspace=None,
                  stream=None, seq_idx=None):
    """``ssd_backward`` on caller-provided contiguous tensors; ``out`` maps dx, ddt,
    dA_log, dB, dC (required) and dD, dinit, ddt_bias (optional) to output tensors.
    The outputs' and the workspace's sizes are checked here (the library cannot
    see them)."""
    import torch
    dev = x.device
    b, T, H, P, N, G, ns = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups, p.nseqs
    shapes = {"dx": (b, T, H, P), "ddt": (b, T, H), "dA_log": (H,), "dB": (b, T, G, N), "dC": (b, T, G, N),
              "dD": (H,), "dinit": (ns, H, P, N), "ddt_bias": (H,)}
    for k, shp in shapes.items():
        if out.get(k) is not None:
            _check_buffer(k, out[k], shp, torch.float32, dev)
    _check_workspace(workspace, backward_workspace_size(p), dev)
    wsn = workspace.numel() if workspace is not None else 0
    g = out.get
    _check(load_library().ssd_backward(ctypes.byref(p), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(B),
                                       _ptr(C), _ptr(D), _ptr(init_state), _ptr(seq_idx), _ptr(dy), _ptr(dfinal),
                                       _ptr(g("dx")), _ptr(g("ddt")), _ptr(g("dA_log")), _ptr(g("dB")), _ptr(g("dC")),
                                       _ptr(g("dD")), _ptr(g("dinit")), _ptr(g("ddt_bias")), _ptr(workspace), wsn,
                                       _stream_of(x.device, stream)))
