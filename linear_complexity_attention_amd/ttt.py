"""Thin ctypes binding of the TTT-layer C ABI (include/ttt.h).

The functions ``ttt_version``, ``ttt_create``, ``ttt_workspace_bytes``,
``ttt_forward``, ``ttt_path_name``, ``ttt_destroy``, ``ttt_last_error`` and
``ttt_status_string`` marshal arguments and call the C functions of the same
name; every step of the layer runs in the HIP kernels of ``libttt.so``.  There
is no fallback: if the library is missing, importing this module raises.

``TTTLayer`` / ``forward`` are conveniences over torch tensors: PyTorch only
provides the device memory (inputs, output, workspace) and the HIP stream.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int, c_longlong, c_size_t, c_uint, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttt.so")

# torch must be imported before libttt.so is loaded: torch ships its own HIP
# runtime (soname libamdhip64.so.7), and loading it first makes libttt.so bind
# to that same runtime instead of a second copy from /opt/rocm, which would not
# share torch's device state or streams.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(python -c 'import __graft_entry__ as g; g.build()')")
_lib = ctypes.CDLL(LIB_PATH)

# ---- enums (include/ttt.h) --------------------------------------------------
TTT_OK, TTT_ERR_INVALID, TTT_ERR_UNSUPPORTED, TTT_ERR_HIP, TTT_ERR_NONFINITE, TTT_ERR_WORKSPACE = range(6)
TTT_F32, TTT_BF16 = 0, 1
TTT_LOSS_MSE, TTT_LOSS_DOT = 0, 1
TTT_INNER_LINEAR, TTT_INNER_MLP_GELU, TTT_INNER_SWIGLU = 0, 1, 2
TTT_FLAG_CHECK_FINITE, TTT_FLAG_FORCE_GENERIC, TTT_FLAG_LOG = 0x1, 0x2, 0x4

LOSSES = {"mse": TTT_LOSS_MSE, "dot": TTT_LOSS_DOT}
INNERS = {"linear": TTT_INNER_LINEAR, "mlp_gelu": TTT_INNER_MLP_GELU, "swiglu": TTT_INNER_SWIGLU}
N_MATRICES = {TTT_INNER_LINEAR: 1, TTT_INNER_MLP_GELU: 2, TTT_INNER_SWIGLU: 3}


class ttt_config(ctypes.Structure):
    _fields_ = [("B", c_int), ("H", c_int), ("N", c_int), ("d", c_int), ("hidden", c_int),
                ("dtype", c_int), ("key_norm", c_int), ("eps", c_float), ("renorm", c_int),
                ("flags", c_uint)]


class ttt_weights(ctypes.Structure):
    _fields_ = [("w", c_void_p * 3), ("batch_stride", c_longlong)]


class ttt_weights_out(ctypes.Structure):
    _fields_ = [("w", c_void_p * 3)]


class ttt_eta(ctypes.Structure):
    _fields_ = [("scale", c_float), ("per_token", c_void_p)]


_lib.ttt_version.restype = c_int
_lib.ttt_version.argtypes = []
_lib.ttt_create.restype = c_int
_lib.ttt_create.argtypes = [POINTER(ttt_config), POINTER(c_void_p)]
_lib.ttt_workspace_bytes.restype = c_int
_lib.ttt_workspace_bytes.argtypes = [c_void_p, c_int, c_int, c_int, POINTER(c_size_t)]
_lib.ttt_forward.restype = c_int
_lib.ttt_forward.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(ttt_weights), POINTER(ttt_eta),
                             c_int, c_int, c_int, c_void_p, POINTER(ttt_weights_out), c_void_p, c_size_t,
                             c_void_p]
_lib.ttt_path_name.restype = c_char_p
_lib.ttt_path_name.argtypes = [c_void_p, c_int, c_int, c_int]
_lib.ttt_set_timing_events.restype = c_int
_lib.ttt_set_timing_events.argtypes = [c_void_p, POINTER(c_void_p), c_int]
_lib.ttt_destroy.restype = c_int
_lib.ttt_destroy.argtypes = [c_void_p]
_lib.ttt_last_error.restype = c_char_p
_lib.ttt_last_error.argtypes = [c_void_p]
_lib.ttt_status_string.restype = c_char_p
_lib.ttt_status_string.argtypes = [c_int]

EXPORTED = ("ttt_version", "ttt_create", "ttt_workspace_bytes", "ttt_forward", "ttt_path_name",
            "ttt_set_timing_events", "ttt_destroy", "ttt_last_error", "ttt_status_string")


class TTTError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{ttt_status_string(status)} ({status}): {message}")


# ---- one-to-one wrappers of the C functions ---------------------------------
def ttt_version() -> int:
    return _lib.ttt_version()


def ttt_status_string(status: int) -> str:
    return _lib.ttt_status_string(status).decode()


def ttt_last_error(handle) -> str:
    return _lib.ttt_last_error(handle).decode()


def ttt_create(cfg: ttt_config):
    h = c_void_p()
    rc = _lib.ttt_create(byref(cfg), byref(h))
    if rc != TTT_OK:
        raise TTTError(rc, ttt_last_error(None))
    return h


def ttt_destroy(handle) -> None:
    _lib.ttt_destroy(handle)


def ttt_workspace_bytes(handle, loss: int, inner: int, chunk: int) -> int:
    n = c_size_t()
    rc = _lib.ttt_workspace_bytes(handle, loss, inner, chunk, byref(n))
    if rc != TTT_OK:
        raise TTTError(rc, ttt_last_error(handle))
    return n.value


def ttt_path_name(handle, loss: int, inner: int, chunk: int):
    r = _lib.ttt_path_name(handle, loss, inner, chunk)
    return r.decode() if r is not None else None


def ttt_set_timing_events(handle, events) -> None:
    """events: sequence of 8 hipEvent_t handles (ints; None entries are
    skipped), or None to switch off."""
    if events is None:
        rc = _lib.ttt_set_timing_events(handle, None, 0)
    else:
        arr = (c_void_p * len(events))(*[e if e else None for e in events])
        rc = _lib.ttt_set_timing_events(handle, arr, len(events))
    if rc != TTT_OK:
        raise TTTError(rc, ttt_last_error(handle))


def ttt_forward(handle, q, k, v, W0: ttt_weights, eta: ttt_eta, loss: int, inner: int, chunk: int, o,
                W_out, workspace, ws_bytes: int, stream) -> int:
    """Raw call: q/k/v/o/workspace/stream are integer device addresses (or
    ctypes pointers); returns the status code without raising."""
    return _lib.ttt_forward(handle, q, k, v, byref(W0), byref(eta), loss, inner, chunk, o,
                            byref(W_out) if W_out is not None else None, workspace, ws_bytes, stream)


# ---- torch convenience layer --------------------------------------------------
class TTTLayer:
    """Holds one handle (and a cached workspace) for a fixed problem shape.

    q, k, v: [B, H, N, d] cuda tensors (float32 or bfloat16, contiguous);
    W0: list of fp32 matrices [H, in, out] (shared over the batch) or
    [B, H, in, out]; eta_tok: optional fp32 [B, H, N].
    """

    def __init__(self, B, H, N, d, hidden, *, dtype="bf16", key_norm=True, eps=1e-5, renorm=False,
                 flags=0):
        self.cfg = ttt_config(B, H, N, d, hidden, TTT_BF16 if dtype == "bf16" else TTT_F32,
                              int(key_norm), float(eps), int(renorm), int(flags))
        self.handle = ttt_create(self.cfg)
        self._ws = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None:
            ttt_destroy(h)
            self.handle = None

    def workspace_bytes(self, loss="mse", inner="mlp_gelu", chunk=0) -> int:
        return ttt_workspace_bytes(self.handle, LOSSES[loss], INNERS[inner], chunk)

    def path_name(self, loss="mse", inner="mlp_gelu", chunk=0):
        return ttt_path_name(self.handle, LOSSES[loss], INNERS[inner], chunk)

    def forward(self, q, k, v, W0, *, eta=1.0, eta_tok=None, loss="mse", inner="mlp_gelu", chunk=0,
                out=None, W_out=None):
        import torch

        c = self.cfg
        tdt = torch.bfloat16 if c.dtype == TTT_BF16 else torch.float32
        for name, t in (("q", q), ("k", k), ("v", v)):
            if not t.is_cuda or t.dtype != tdt or not t.is_contiguous() or tuple(t.shape) != (c.B, c.H, c.N, c.d):
                raise ValueError(f"{name} must be a contiguous cuda {tdt} tensor of shape {(c.B, c.H, c.N, c.d)}")
        li, ii = LOSSES[loss], INNERS[inner]
        nm = N_MATRICES[ii]
        if len(W0) != nm:
            raise ValueError(f"{inner} needs {nm} weight matrices")
        stride = 0
        for w in W0:
            if not w.is_cuda or w.dtype != torch.float32 or not w.is_contiguous():
                raise ValueError("W0 matrices must be contiguous cuda float32 tensors")
            if w.dim() == 4:
                stride = w[0].numel()
        if out is None:
            out = torch.empty_like(q)
        nbytes = ttt_workspace_bytes(self.handle, li, ii, chunk)
        if self._ws is None or self._ws.numel() < nbytes or self._ws.device != q.device:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
        wts = ttt_weights()
        for i, w in enumerate(W0):
            wts.w[i] = w.data_ptr()
        wts.batch_stride = stride
        e = ttt_eta(float(eta), eta_tok.data_ptr() if eta_tok is not None else None)
        wo = None
        if W_out is not None:
            wo = ttt_weights_out()
            for i, w in enumerate(W_out):
                wo.w[i] = w.data_ptr()
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = ttt_forward(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), wts, e, li, ii, chunk,
                         out.data_ptr(), wo, self._ws.data_ptr(), self._ws.numel(), stream)
        if rc != TTT_OK:
            raise TTTError(rc, ttt_last_error(self.handle))
        return out


def forward(q, k, v, W0, *, hidden=None, eta=1.0, eta_tok=None, loss="mse", inner="mlp_gelu", chunk=0,
            key_norm=True, eps=1e-5, renorm=False, flags=0, return_weights=False):
    """One-shot TTT-layer forward; returns O (and the final weights)."""
    import torch

    B, H, N, d = q.shape
    if hidden is None:
        hidden = W0[0].shape[-1] if inner != "linear" else d
    layer = TTTLayer(B, H, N, d, hidden, dtype="bf16" if q.dtype == torch.bfloat16 else "f32",
                     key_norm=key_norm, eps=eps, renorm=renorm, flags=flags)
    W_out = None
    if return_weights:
        W_out = [torch.empty((B, H) + tuple(w.shape[-2:]), dtype=torch.float32, device=q.device) for w in W0]
    O = layer.forward(q, k, v, W0, eta=eta, eta_tok=eta_tok, loss=loss, inner=inner, chunk=chunk, W_out=W_out)
    return (O, W_out) if return_weights else O
