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
TTT_INNER_LINEAR, TTT_INNER_MLP_GELU, TTT_INNER_SWIGLU, TTT_INNER_GLU, TTT_INNER_DWCONV, TTT_INNER_VIT3 = range(6)
TTT_FLAG_CHECK_FINITE, TTT_FLAG_FORCE_GENERIC, TTT_FLAG_LOG = 0x1, 0x2, 0x4

TTT_RULE_GD, TTT_RULE_MOMENTUM, TTT_RULE_MUON = 0, 1, 2
TTT_ORDER_CAUSAL, TTT_ORDER_WRITE_THEN_QUERY = 0, 1

LOSSES = {"mse": TTT_LOSS_MSE, "dot": TTT_LOSS_DOT}
RULES = {"gd": TTT_RULE_GD, "momentum": TTT_RULE_MOMENTUM, "muon": TTT_RULE_MUON}
ORDERS = {"causal": TTT_ORDER_CAUSAL, "write_then_query": TTT_ORDER_WRITE_THEN_QUERY}
INNERS = {"linear": TTT_INNER_LINEAR, "mlp_gelu": TTT_INNER_MLP_GELU, "swiglu": TTT_INNER_SWIGLU,
          "glu": TTT_INNER_GLU, "dwconv": TTT_INNER_DWCONV, "vit3": TTT_INNER_VIT3}
N_MATRICES = {TTT_INNER_LINEAR: 1, TTT_INNER_MLP_GELU: 2, TTT_INNER_SWIGLU: 3, TTT_INNER_GLU: 2,
              TTT_INNER_DWCONV: 1, TTT_INNER_VIT3: 3}


class ttt_config(ctypes.Structure):
    _fields_ = [("B", c_int), ("H", c_int), ("N", c_int), ("d", c_int), ("hidden", c_int),
                ("dtype", c_int), ("key_norm", c_int), ("eps", c_float), ("renorm", c_int),
                ("flags", c_uint), ("grid_h", c_int), ("grid_w", c_int), ("conv_k", c_int)]


class ttt_weights(ctypes.Structure):
    _fields_ = [("w", c_void_p * 3), ("batch_stride", c_longlong)]


class ttt_weights_out(ctypes.Structure):
    _fields_ = [("w", c_void_p * 3)]


class ttt_eta(ctypes.Structure):
    _fields_ = [("scale", c_float), ("per_token", c_void_p)]


class ttt_options(ctypes.Structure):
    _fields_ = [("epochs", c_int), ("update_mask", c_uint), ("order", c_int), ("chunk_update", c_void_p),
                ("rule", c_int), ("beta", c_float), ("muon_scale", c_float), ("ns_steps", c_int)]


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
_lib.ttt_forward_ex.restype = c_int
_lib.ttt_forward_ex.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(ttt_weights), POINTER(ttt_eta),
                                c_int, c_int, c_int, POINTER(ttt_options), c_void_p, POINTER(ttt_weights_out),
                                c_void_p, c_size_t, c_void_p]
_lib.ttt_workspace_bytes_ex.restype = c_int
_lib.ttt_workspace_bytes_ex.argtypes = [c_void_p, c_int, c_int, c_int, POINTER(ttt_options), POINTER(c_size_t)]
_lib.ttt_path_name_ex.restype = c_char_p
_lib.ttt_path_name_ex.argtypes = [c_void_p, c_int, c_int, c_int, POINTER(ttt_options)]
_lib.ttt_backward_workspace_bytes.restype = c_int
_lib.ttt_backward_workspace_bytes.argtypes = [c_void_p, c_int, c_int, POINTER(c_size_t)]
_lib.ttt_backward.restype = c_int
_lib.ttt_backward.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(ttt_weights), POINTER(ttt_eta), c_int,
                              c_int, c_void_p, c_void_p, c_void_p, c_void_p, POINTER(ttt_weights_out), c_void_p,
                              c_void_p, c_size_t, c_void_p]
_lib.ttt_forward_noalloc.restype = c_int
_lib.ttt_forward_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(ttt_weights),
                                     POINTER(ttt_eta), c_int, c_int, c_int, c_void_p, POINTER(ttt_weights_out),
                                     c_void_p]
TTT_NOALLOC_SCRATCH_BYTES = 192 << 20
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

EXPORTED = ("ttt_version", "ttt_create", "ttt_workspace_bytes", "ttt_workspace_bytes_ex", "ttt_forward",
            "ttt_forward_ex", "ttt_forward_noalloc", "ttt_path_name", "ttt_path_name_ex", "ttt_set_timing_events",
            "ttt_destroy", "ttt_last_error", "ttt_status_string", "ttt_backward", "ttt_backward_workspace_bytes")


def matrix_shapes(inner: int, d: int, hidden: int, conv_k: int = 3):
    """[in, out] shape of every matrix of the inner model (include/ttt.h);
    a convolution kernel is [d, k*k]."""
    if inner == TTT_INNER_LINEAR:
        return [(d, d)]
    if inner == TTT_INNER_MLP_GELU:
        return [(d, hidden), (hidden, d)]
    if inner == TTT_INNER_SWIGLU:
        return [(d, hidden), (hidden, d), (d, hidden)]
    if inner == TTT_INNER_GLU:
        return [(d, d), (d, d)]
    if inner == TTT_INNER_DWCONV:
        return [(d, conv_k * conv_k)]
    if inner == TTT_INNER_VIT3:
        return [(d, d), (d, d), (d, conv_k * conv_k)]
    raise ValueError(f"unknown inner model {inner}")


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


def ttt_workspace_bytes_ex(handle, loss: int, inner: int, chunk: int, opt) -> int:
    n = c_size_t()
    rc = _lib.ttt_workspace_bytes_ex(handle, loss, inner, chunk, byref(opt) if opt is not None else None, byref(n))
    if rc != TTT_OK:
        raise TTTError(rc, ttt_last_error(handle))
    return n.value


def ttt_path_name_ex(handle, loss: int, inner: int, chunk: int, opt):
    r = _lib.ttt_path_name_ex(handle, loss, inner, chunk, byref(opt) if opt is not None else None)
    return r.decode() if r is not None else None


def ttt_forward_ex(handle, q, k, v, W0: ttt_weights, eta: ttt_eta, loss: int, inner: int, chunk: int, opt, o,
                   W_out, workspace, ws_bytes: int, stream) -> int:
    """Raw call with per-call options (a ttt_options or None); returns the
    status code without raising."""
    return _lib.ttt_forward_ex(handle, q, k, v, byref(W0), byref(eta), loss, inner, chunk,
                               byref(opt) if opt is not None else None, o,
                               byref(W_out) if W_out is not None else None, workspace, ws_bytes, stream)


def ttt_backward_workspace_bytes(handle, loss: int, inner: int) -> int:
    n = c_size_t()
    rc = _lib.ttt_backward_workspace_bytes(handle, loss, inner, byref(n))
    if rc != TTT_OK:
        raise TTTError(rc, ttt_last_error(handle))
    return n.value


def ttt_backward(handle, q, k, v, W0: ttt_weights, eta: ttt_eta, loss: int, inner: int, dO, dq, dk, dv, dW0, deta,
                 workspace, ws_bytes: int, stream) -> int:
    """Raw call of the outer-loop backward; returns the status code."""
    return _lib.ttt_backward(handle, q, k, v, byref(W0), byref(eta), loss, inner, dO, dq, dk, dv,
                             byref(dW0) if dW0 is not None else None, deta, workspace, ws_bytes, stream)


def make_options(*, epochs=1, update_mask=0, order="causal", chunk_update=None, rule="gd", beta=0.0,
                 muon_scale=1.0, ns_steps=5):
    """A ttt_options from keyword values; chunk_update (a sequence of 0/1 per
    chunk) is kept alive on the returned struct."""
    opt = ttt_options()
    opt.epochs = int(epochs)
    opt.update_mask = int(update_mask)
    opt.order = ORDERS[order] if isinstance(order, str) else int(order)
    opt.rule = RULES[rule] if isinstance(rule, str) else int(rule)
    opt.beta = float(beta)
    opt.muon_scale = float(muon_scale)
    opt.ns_steps = int(ns_steps)
    if chunk_update is not None:
        buf = (ctypes.c_ubyte * len(chunk_update))(*[1 if x else 0 for x in chunk_update])
        opt._chunk_update_buf = buf
        opt.chunk_update = ctypes.cast(buf, c_void_p)
    return opt


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


def ttt_forward_noalloc(handle, q, k, v, W0: ttt_weights, eta: ttt_eta, loss: int, inner: int, chunk: int, o,
                        W_out, stream) -> int:
    """Raw call of the entry point that uses the library's own per-device
    scratch array instead of a workspace; returns the status code."""
    return _lib.ttt_forward_noalloc(handle, q, k, v, byref(W0), byref(eta), loss, inner, chunk, o,
                                    byref(W_out) if W_out is not None else None, stream)


# ---- torch convenience layer --------------------------------------------------
class TTTLayer:
    """Holds one handle (and a cached workspace) for a fixed problem shape.

    q, k, v: [B, H, N, d] cuda tensors (float32 or bfloat16, contiguous);
    W0: list of fp32 matrices [H, in, out] (shared over the batch) or
    [B, H, in, out]; eta_tok: optional fp32 [B, H, N].
    """

    def __init__(self, B, H, N, d, hidden, *, dtype="bf16", key_norm=True, eps=1e-5, renorm=False,
                 flags=0, grid=(0, 0), conv_k=0):
        """grid = (grid_h, grid_w) and conv_k: the token raster and kernel size
        of the convolution inner models ("dwconv", "vit3")."""
        self.cfg = ttt_config(B, H, N, d, hidden, TTT_BF16 if dtype == "bf16" else TTT_F32,
                              int(key_norm), float(eps), int(renorm), int(flags), int(grid[0]), int(grid[1]),
                              int(conv_k))
        self.handle = ttt_create(self.cfg)
        self._ws = None

    # bound at class creation: at interpreter shutdown the module globals may
    # already be gone when __del__ runs
    _destroy = staticmethod(_lib.ttt_destroy)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None:
            self.handle = None
            try:
                self._destroy(h)
            except Exception:   # interpreter teardown: nothing left to release into
                pass

    def workspace_bytes(self, loss="mse", inner="mlp_gelu", chunk=0, options=None) -> int:
        return ttt_workspace_bytes_ex(self.handle, LOSSES[loss], INNERS[inner], chunk, options)

    def path_name(self, loss="mse", inner="mlp_gelu", chunk=0, options=None):
        return ttt_path_name_ex(self.handle, LOSSES[loss], INNERS[inner], chunk, options)

    def forward(self, q, k, v, W0, *, eta=1.0, eta_tok=None, loss="mse", inner="mlp_gelu", chunk=0,
                out=None, W_out=None, options=None):
        """options: None (the plain layer) or a ttt_options (make_options)."""
        import torch

        c = self.cfg
        tdt = torch.bfloat16 if c.dtype == TTT_BF16 else torch.float32
        for name, t in (("q", q), ("k", k), ("v", v)):
            if (not t.is_cuda or t.device != q.device or t.dtype != tdt or not t.is_contiguous()
                    or tuple(t.shape) != (c.B, c.H, c.N, c.d)):
                raise ValueError(f"{name} must be a contiguous cuda {tdt} tensor on q's device of shape "
                                 f"{(c.B, c.H, c.N, c.d)}")
        li, ii = LOSSES[loss], INNERS[inner]
        nm = N_MATRICES[ii]
        shapes = matrix_shapes(ii, c.d, c.hidden, c.conv_k)
        if len(W0) != nm:
            raise ValueError(f"{inner} needs {nm} weight matrices")
        lead = None
        for i, (w, (fi, fo)) in enumerate(zip(W0, shapes)):
            if not w.is_cuda or w.device != q.device or w.dtype != torch.float32 or not w.is_contiguous():
                raise ValueError(f"W0[{i}] must be a contiguous float32 tensor on {q.device}")
            if tuple(w.shape) not in ((c.H, fi, fo), (c.B, c.H, fi, fo)):
                raise ValueError(f"W0[{i}] must have shape {(c.H, fi, fo)} or {(c.B, c.H, fi, fo)}, "
                                 f"got {tuple(w.shape)}")
            if lead is None:
                lead = w.dim()
            elif w.dim() != lead:
                raise ValueError("all W0 matrices must share one layout ([H,in,out] or [B,H,in,out])")
        # one batch stride serves every matrix (all have in*out elements per head)
        stride = c.H * shapes[0][0] * shapes[0][1] if lead == 4 else 0
        if eta_tok is not None:
            if (not eta_tok.is_cuda or eta_tok.device != q.device or eta_tok.dtype != torch.float32
                    or not eta_tok.is_contiguous() or tuple(eta_tok.shape) != (c.B, c.H, c.N)):
                raise ValueError(f"eta_tok must be a contiguous float32 tensor on {q.device} of shape "
                                 f"{(c.B, c.H, c.N)}")
        if out is None:
            out = torch.empty_like(q)
        elif (out.device != q.device or out.dtype != tdt or not out.is_contiguous()
              or tuple(out.shape) != (c.B, c.H, c.N, c.d)):
            raise ValueError(f"out must be a contiguous {tdt} tensor on {q.device} of shape {(c.B, c.H, c.N, c.d)}")
        if W_out is not None:
            if len(W_out) != nm:
                raise ValueError(f"W_out needs {nm} matrices")
            for i, (w, (fi, fo)) in enumerate(zip(W_out, shapes)):
                if w is None:
                    continue
                if (w.device != q.device or w.dtype != torch.float32 or not w.is_contiguous()
                        or tuple(w.shape) != (c.B, c.H, fi, fo)):
                    raise ValueError(f"W_out[{i}] must be a contiguous float32 tensor on {q.device} of shape "
                                     f"{(c.B, c.H, fi, fo)}")
        nbytes = ttt_workspace_bytes_ex(self.handle, li, ii, chunk, options)
        if options is not None and options.chunk_update:
            nb = (c.N + chunk - 1) // chunk if chunk else 1
            buf = getattr(options, "_chunk_update_buf", None)
            if buf is None or len(buf) != nb:
                raise ValueError(f"chunk_update needs {nb} flags (build the options with make_options)")
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
                wo.w[i] = w.data_ptr() if w is not None else None
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = ttt_forward_ex(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), wts, e, li, ii, chunk, options,
                            out.data_ptr(), wo, self._ws.data_ptr(), self._ws.numel(), stream)
        if rc != TTT_OK:
            raise TTTError(rc, ttt_last_error(self.handle))
        return out


def _layer_backward(self, q, k, v, W0, dO, *, eta=1.0, eta_tok=None, loss="mse", inner="mlp_gelu",
                    want_deta=True):
    """Outer-loop backward: returns dict(dq, dk, dv, dW0 (list, W0's layout),
    deta or None), fp32, for the gradient dO of an outer loss with respect to
    the layer's output."""
    import torch

    c = self.cfg
    tdt = torch.bfloat16 if c.dtype == TTT_BF16 else torch.float32
    shape = (c.B, c.H, c.N, c.d)
    for name, t in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        if (not t.is_cuda or t.device != q.device or t.dtype != tdt or not t.is_contiguous()
                or tuple(t.shape) != shape):
            raise ValueError(f"{name} must be a contiguous cuda {tdt} tensor on q's device of shape {shape}")
    li, ii = LOSSES[loss], INNERS[inner]
    shapes = matrix_shapes(ii, c.d, c.hidden, c.conv_k)
    if len(W0) != len(shapes):
        raise ValueError(f"{inner} needs {len(shapes)} weight matrices")
    lead = None
    for i, (w, (fi, fo)) in enumerate(zip(W0, shapes)):
        if (not w.is_cuda or w.device != q.device or w.dtype != torch.float32 or not w.is_contiguous()
                or tuple(w.shape) not in ((c.H, fi, fo), (c.B, c.H, fi, fo))):
            raise ValueError(f"W0[{i}] must be a contiguous float32 tensor of shape {(c.H, fi, fo)} or "
                             f"{(c.B, c.H, fi, fo)}")
        if lead is None:
            lead = w.dim()
        elif w.dim() != lead:
            raise ValueError("all W0 matrices must share one layout")
    if eta_tok is not None and (eta_tok.device != q.device or eta_tok.dtype != torch.float32
                                or not eta_tok.is_contiguous() or tuple(eta_tok.shape) != (c.B, c.H, c.N)):
        raise ValueError(f"eta_tok must be a contiguous float32 tensor of shape {(c.B, c.H, c.N)}")
    nbytes = ttt_backward_workspace_bytes(self.handle, li, ii)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty(shape, dtype=torch.float32, device=q.device) for _ in range(3))
    dW = [torch.empty_like(w) for w in W0]
    deta = torch.empty((c.B, c.H, c.N), dtype=torch.float32, device=q.device) if want_deta else None
    wts = ttt_weights()
    for i, w in enumerate(W0):
        wts.w[i] = w.data_ptr()
    wts.batch_stride = c.H * shapes[0][0] * shapes[0][1] if lead == 4 else 0
    wo = ttt_weights_out()
    for i, w in enumerate(dW):
        wo.w[i] = w.data_ptr()
    e = ttt_eta(float(eta), eta_tok.data_ptr() if eta_tok is not None else None)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = ttt_backward(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), wts, e, li, ii, dO.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), wo, deta.data_ptr() if deta is not None else None,
                      ws.data_ptr(), ws.numel(), stream)
    if rc != TTT_OK:
        raise TTTError(rc, ttt_last_error(self.handle))
    return dict(dq=dq, dk=dk, dv=dv, dW0=dW, deta=deta)


TTTLayer.backward = _layer_backward


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
