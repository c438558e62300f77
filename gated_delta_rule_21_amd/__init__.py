"""Kimi Delta Attention (KDA) on MI355X: Python binding of libkda.so.

The binding only marshals arguments: torch tensors become device pointers,
the current torch stream becomes the hipStream_t, and every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: if
the library is missing or the tensors are not on a GPU, the call raises.

Entry points (same names as the C ABI in include/kda.h):
  kda_prefill(...)                  raw C call, pointers as ints
  kda_decode(...)                   raw C call
  kda_decode_window(...)            raw C call: replay + multi-token window
  kda_prefill_checkpoints(...)      raw C call: prefill + state checkpoints
  kda_qkv_shortconv(...)            raw C call: ShortConv -> Swish -> L2Norm feature path
  kda_output_gate(...)              raw C call: Sigmoid(g) * RMSNorm(o)
  kda_prefill_backward(...)         raw C call: gradients of the prefill
  kda_prefill_workspace_size(...), kda_prefill_backward_workspace_size(...)
  kda_set_prefill_segments(P), kda_prefill_segments(...)
                                    segment split of long sequences
  kda_status_string(status)
Convenience wrappers over torch tensors:
  prefill(q, k, v, z, A, beta, cu_seqlens, h0=None, ...) -> (o, hT)
  decode(q, k, v, z, A, beta, S) -> o          (S updated in place)
  decode_window(A, S, window=..., replay=..., n_accept=...) -> o
  prefill_checkpoints(..., interval) -> (o, hT, checkpoints, offsets)
  qkv_shortconv(xq, xk, xv, wq, wk, wv, cu_seqlens, ...) -> (q, k, v)
  output_gate(o, g, w, eps) -> y
  prefill_backward(q, k, v, z, A, beta, cu_seqlens, grad_o, h0=None, grad_hT=None)
      -> dict(dq, dk, dv, dz, dbeta, dA, dh0)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libkda.so")

KDA_BF16 = 0
KDA_F32 = 1

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, kda_status_string(status), status))
        self.status = status


def lib():
    """The loaded libkda.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkda.so not found at %s; build it with "
                           "`python -m gated_delta_rule_21_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.kda_prefill.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp, vp,
                              sz, vp]
    L.kda_prefill.restype = ci
    L.kda_prefill_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    L.kda_prefill_workspace_size.restype = sz
    L.kda_decode.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, vp, vp]
    L.kda_decode.restype = ci
    L.kda_qkv_shortconv.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp, vp, vp,
                                    vp, vp]
    L.kda_qkv_shortconv.restype = ci
    L.kda_output_gate.argtypes = [ci, vp, vp, vp, ctypes.c_float, ci, ci, ci, vp, vp]
    L.kda_output_gate.restype = ci
    L.kda_prefill_checkpoints.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp,
                                          vp, ci, vp, vp, vp, sz, vp]
    L.kda_prefill_checkpoints.restype = ci
    L.kda_decode_window.argtypes = [ci, vp, vp, vp, vp, vp, ci, vp, vp, vp, vp, vp, ci, vp, vp, ci, ci,
                                    ci, ci, vp, ci, vp]
    L.kda_decode_window.restype = ci
    L.kda_prefill_backward.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.kda_prefill_backward.restype = ci
    L.kda_prefill_backward_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    L.kda_prefill_backward_workspace_size.restype = sz
    L.kda_set_prefill_segments.argtypes = [ci]
    L.kda_set_prefill_segments.restype = ci
    L.kda_prefill_segments.argtypes = [ci, ci, ci, ci, ci, ci]
    L.kda_prefill_segments.restype = ci
    L.kda_status_string.argtypes = [ci]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_build_info.restype = ctypes.c_char_p
    _lib = L
    return L


# ---------------------------------------------------------------------------
# Raw C entry points
# ---------------------------------------------------------------------------
def kda_prefill(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT,
                workspace, workspace_bytes, stream) -> int:
    return lib().kda_prefill(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o,
                             hT, workspace, workspace_bytes, stream)


def kda_decode(io_dtype, q, k, v, z, A, beta, S_inout, N, H, dk, dv, o, stream) -> int:
    return lib().kda_decode(io_dtype, q, k, v, z, A, beta, S_inout, N, H, dk, dv, o, stream)


def kda_qkv_shortconv(io_dtype, xq, xk, xv, wq, wk, wv, cu_seqlens, N, T, H, dk, dv, conv_state_in,
                      conv_state_out, q, k, v, stream) -> int:
    return lib().kda_qkv_shortconv(io_dtype, xq, xk, xv, wq, wk, wv, cu_seqlens, N, T, H, dk, dv,
                                   conv_state_in, conv_state_out, q, k, v, stream)


def kda_output_gate(io_dtype, o, g, w, eps, T, H, dv, y, stream) -> int:
    return lib().kda_output_gate(io_dtype, o, g, w, eps, T, H, dv, y, stream)


def kda_prefill_checkpoints(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT,
                            interval, checkpoints, checkpoint_offsets, workspace, workspace_bytes,
                            stream) -> int:
    return lib().kda_prefill_checkpoints(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk,
                                         dv, o, hT, interval, checkpoints, checkpoint_offsets,
                                         workspace, workspace_bytes, stream)


def kda_decode_window(io_dtype, rk, rv, rz, rbeta, n_accept, Lr, q, k, v, z, beta, L, A, S_inout,
                      N, H, dk, dv, o, commit_window, stream) -> int:
    return lib().kda_decode_window(io_dtype, rk, rv, rz, rbeta, n_accept, Lr, q, k, v, z, beta, L,
                                   A, S_inout, N, H, dk, dv, o, commit_window, stream)


def kda_prefill_backward(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, grad_o,
                         grad_hT, grad_q, grad_k, grad_v, grad_z, grad_beta, grad_A, grad_h0, workspace,
                         workspace_bytes, stream) -> int:
    return lib().kda_prefill_backward(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv,
                                      grad_o, grad_hT, grad_q, grad_k, grad_v, grad_z, grad_beta, grad_A,
                                      grad_h0, workspace, workspace_bytes, stream)


def kda_prefill_backward_workspace_size(N, T, H, dk, dv, io_dtype) -> int:
    return int(lib().kda_prefill_backward_workspace_size(N, T, H, dk, dv, io_dtype))


def kda_prefill_workspace_size(N, T, H, dk, dv, io_dtype) -> int:
    return int(lib().kda_prefill_workspace_size(N, T, H, dk, dv, io_dtype))


def kda_set_prefill_segments(segments: int) -> int:
    return lib().kda_set_prefill_segments(segments)


def kda_prefill_segments(N, T, H, dk, dv, io_dtype) -> int:
    return lib().kda_prefill_segments(N, T, H, dk, dv, io_dtype)


def kda_status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def kda_build_info() -> str:
    return lib().kda_build_info().decode()


# ---------------------------------------------------------------------------
# torch wrappers (allocation and pointer marshalling only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _io_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _check_gpu(**tensors):
    torch = _torch()
    for name, t in tensors.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("%s must be a GPU tensor (the library has no CPU path)" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def prefill_workspace(N, T, H, d, io_dtype, device):
    """Allocate the prefill workspace (a byte tensor of the size the library asks)."""
    torch = _torch()
    n = kda_prefill_workspace_size(N, T, H, d, d, io_dtype)
    if n == 0:
        raise ValueError("unsupported prefill sizes N=%d T=%d H=%d d=%d" % (N, T, H, d))
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill(q, k, v, z, A, beta, cu_seqlens, h0=None, o=None, hT=None, workspace=None,
            final_state: bool = True):
    """KDA prefill over packed sequences.  Returns (o, hT); hT is None when
    final_state is False and no hT buffer is given."""
    torch = _torch()
    _check_gpu(q=q, k=k, v=v, z=z, A=A, beta=beta, cu_seqlens=cu_seqlens, h0=h0, o=o, hT=hT,
               workspace=workspace)
    io = _io_code(q)
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    if hT is None and final_state:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = prefill_workspace(N, T, H, dk, io, q.device)
    st = kda_prefill(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(h0),
                     _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(o), _ptr(hT), _ptr(workspace),
                     workspace.numel(), _stream(q.device))
    if st != 0:
        raise KdaError("kda_prefill", st)
    return o, hT


class prefill_segments:
    """Context manager: kda_prefill splits sequences into `segments`
    segments (0 = automatic, 1 = never) inside the block, then restores the
    automatic choice.  Size workspaces inside the block."""

    def __init__(self, segments: int):
        self.segments = segments

    def __enter__(self):
        st = kda_set_prefill_segments(self.segments)
        if st != 0:
            raise KdaError("kda_set_prefill_segments", st)
        return self

    def __exit__(self, *exc):
        kda_set_prefill_segments(0)
        return False


def decode(q, k, v, z, A, beta, S, o=None):
    """One decode step; S ([N, H, dv, dk] fp32) is updated in place.  Returns o."""
    torch = _torch()
    _check_gpu(q=q, k=k, v=v, z=z, A=A, beta=beta, S=S, o=o)
    io = _io_code(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    st = kda_decode(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(S), N, H,
                    dk, dv, _ptr(o), _stream(q.device))
    if st != 0:
        raise KdaError("kda_decode", st)
    return o


def decode_window(A, S, window=None, replay=None, n_accept=None, o=None, commit_window=False):
    """Multi-token decode with replay.  S ([N, H, dv, dk] fp32) is the
    committed state and is updated in place.

    replay: dict of k, v, z, beta with shapes [N, Lr, H, d] ([N, Lr, H] for
            beta), normally the window of the previous call; n_accept: [N]
            int32 accepted replay tokens.
    window: dict of q, k, v, z, beta with shapes [N, L, H, d].
    Returns o [N, L, H, dv] (None when there is no window)."""
    torch = _torch()
    N, H, dv, dk = S.shape
    _check_gpu(A=A, S=S, n_accept=n_accept, o=o)
    rk = rv = rz = rb = None
    Lr = 0
    if replay is not None:
        rk, rv, rz, rb = replay["k"], replay["v"], replay["z"], replay["beta"]
        _check_gpu(rk=rk, rv=rv, rz=rz, rbeta=rb)
        Lr = rk.shape[1]
        if n_accept is None:
            raise ValueError("n_accept is required with a replay window")
    q = k = v = z = b = None
    L = 0
    if window is not None:
        q, k, v, z, b = (window[n] for n in ("q", "k", "v", "z", "beta"))
        _check_gpu(q=q, k=k, v=v, z=z, beta=b)
        L = q.shape[1]
    ref = q if q is not None else rk
    io = _io_code(ref) if ref is not None else KDA_F32
    if L > 0 and o is None:
        o = torch.empty((N, L, H, dv), dtype=q.dtype, device=S.device)
    st = kda_decode_window(io, _ptr(rk), _ptr(rv), _ptr(rz), _ptr(rb), _ptr(n_accept), Lr,
                           _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(b), L, _ptr(A), _ptr(S),
                           N, H, dk, dv, _ptr(o), 1 if commit_window else 0, _stream(S.device))
    if st != 0:
        raise KdaError("kda_decode_window", st)
    return o if L > 0 else None


def prefill_checkpoints(q, k, v, z, A, beta, cu_seqlens, interval: int, h0=None, o=None, hT=None,
                        checkpoints=None, offsets=None, workspace=None):
    """prefill() that also saves the state every `interval` tokens of every
    sequence.  Returns (o, hT, checkpoints [T // interval, H, dv, dk],
    offsets [N + 1]): sequence n's checkpoints are
    checkpoints[offsets[n]:offsets[n + 1]], in token order."""
    torch = _torch()
    _check_gpu(q=q, k=k, v=v, z=z, A=A, beta=beta, cu_seqlens=cu_seqlens, h0=h0, o=o, hT=hT,
               checkpoints=checkpoints, offsets=offsets, workspace=workspace)
    io = _io_code(q)
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dev = q.device
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if hT is None:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    if checkpoints is None:
        checkpoints = torch.empty((T // interval, H, dv, dk), dtype=torch.float32, device=dev)
    if offsets is None:
        offsets = torch.empty(N + 1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = prefill_workspace(N, T, H, dk, io, dev)
    st = kda_prefill_checkpoints(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(h0),
                                 _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(o), _ptr(hT), interval,
                                 _ptr(checkpoints), _ptr(offsets), _ptr(workspace), workspace.numel(),
                                 _stream(dev))
    if st != 0:
        raise KdaError("kda_prefill_checkpoints", st)
    return o, hT, checkpoints, offsets


def qkv_shortconv(xq, xk, xv, wq, wk, wv, cu_seqlens, conv_state_in=None, conv_state_out=None,
                  q=None, k=None, v=None):
    """The feature path: returns (q, k, v) = (L2Norm(Swish(ShortConv(xq))), ...,
    Swish(ShortConv(xv))).  conv_state_* are [N, 3, H, 3 d] windows of the
    last pre-convolution tokens (conv_state_out may be conv_state_in)."""
    torch = _torch()
    _check_gpu(xq=xq, xk=xk, xv=xv, wq=wq, wk=wk, wv=wv, cu_seqlens=cu_seqlens,
               conv_state_in=conv_state_in, conv_state_out=conv_state_out, q=q, k=k, v=v)
    io = _io_code(xq)
    T, H, d = xq.shape
    N = cu_seqlens.numel() - 1
    q = torch.empty_like(xq) if q is None else q
    k = torch.empty_like(xk) if k is None else k
    v = torch.empty_like(xv) if v is None else v
    st = kda_qkv_shortconv(io, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv),
                           _ptr(cu_seqlens), N, T, H, d, xv.shape[-1], _ptr(conv_state_in),
                           _ptr(conv_state_out), _ptr(q), _ptr(k), _ptr(v), _stream(xq.device))
    if st != 0:
        raise KdaError("kda_qkv_shortconv", st)
    return q, k, v


def output_gate(o, g, w, eps: float, y=None):
    """y = Sigmoid(g) * RMSNorm(o) per (token, head) row; y may be o or g."""
    torch = _torch()
    _check_gpu(o=o, g=g, w=w, y=y)
    T, H, dv = o.shape
    y = torch.empty_like(o) if y is None else y
    st = kda_output_gate(_io_code(o), _ptr(o), _ptr(g), _ptr(w), float(eps), T, H, dv, _ptr(y),
                         _stream(o.device))
    if st != 0:
        raise KdaError("kda_output_gate", st)
    return y


def prefill_backward(q, k, v, z, A, beta, cu_seqlens, grad_o, h0=None, grad_hT=None, workspace=None,
                     grads=None):
    """Gradients of L = sum(grad_o * o) + sum(grad_hT * hT) for the prefill
    o, hT = prefill(q, k, v, z, A, beta, cu_seqlens, h0).  Returns a dict of
    fp32 tensors dq, dk, dv, dz [T, H, d], dbeta [T, H], dA [H] and
    dh0 [N, H, dv, dk].  `grads` may hold preallocated outputs by those names."""
    torch = _torch()
    _check_gpu(q=q, k=k, v=v, z=z, A=A, beta=beta, cu_seqlens=cu_seqlens, grad_o=grad_o, h0=h0,
               grad_hT=grad_hT, workspace=workspace)
    io = _io_code(q)
    if grad_o.dtype != q.dtype:
        raise TypeError("grad_o must have the dtype of q (%s)" % q.dtype)
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dev = q.device
    g = dict(grads or {})
    f32 = dict(dtype=torch.float32, device=dev)
    for name, shape in (("dq", (T, H, dk)), ("dk", (T, H, dk)), ("dv", (T, H, dv)), ("dz", (T, H, dk)),
                        ("dbeta", (T, H)), ("dA", (H,)), ("dh0", (N, H, dv, dk))):
        if g.get(name) is None:
            g[name] = torch.empty(shape, **f32)
    _check_gpu(**g)
    if workspace is None:
        n = kda_prefill_backward_workspace_size(N, T, H, dk, dv, io)
        if n == 0:
            raise ValueError("unsupported backward sizes N=%d T=%d H=%d d=%d" % (N, T, H, dk))
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    st = kda_prefill_backward(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(h0),
                              _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(grad_o), _ptr(grad_hT),
                              _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dz"]), _ptr(g["dbeta"]),
                              _ptr(g["dA"]), _ptr(g["dh0"]), _ptr(workspace), workspace.numel(),
                              _stream(dev))
    if st != 0:
        raise KdaError("kda_prefill_backward", st)
    return g
