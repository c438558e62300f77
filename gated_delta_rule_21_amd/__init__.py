"""Kimi Delta Attention (KDA) on MI355X: Python binding of libkda.so.

The binding only marshals arguments: torch tensors become device pointers,
the current torch stream becomes the hipStream_t, and every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: if
the library is missing or the tensors are not on a GPU, the call raises.

Entry points (same names as the C ABI in include/kda.h):
  kda_prefill(...)                  raw C call, pointers as ints
  kda_prefill_ex(..., options, ...) raw C call: prefill with per-call options
                                    (segment count, state checkpoints, block pipeline)
  kda_prefill_noalloc(...)          raw C call: prefill without a workspace (the
                                    library's fixed device scratch; no allocation)
  kda_prefill_fused(...)            raw C call: feature path -> prefill -> output gate
  kda_prefill_fused_ex(..., options, ...)  the same with per-call options (segments, blocks)
  kda_prefill_fused_workspace_size(..., options)  its workspace bytes
  kda_decode(...)                   raw C call
  kda_decode_fused(...)             raw C call: feature path -> decode step -> output gate
  kda_decode_window(...)            raw C call: replay + multi-token window
  kda_qkv_shortconv(...)            raw C call: ShortConv -> Swish -> L2Norm feature path
  kda_output_gate(...)              raw C call: Sigmoid(g) * RMSNorm(o)
  kda_prefill_backward(...)         raw C call: gradients of the prefill
  kda_prefill_workspace_size(...), kda_prefill_ex_workspace_size(..., options),
  kda_prefill_backward_workspace_size(..., options)
  kda_prefill_segments(...)         the automatic segment split of long sequences
  kda_status_string(status)
  PrefillOptions                    ctypes mirror of struct kda_prefill_options
Convenience wrappers over torch tensors (they check every tensor's device,
dtype, shape and contiguity before passing its pointer, since the C ABI
cannot see them):
  prefill(q, k, v, z, A, beta, cu_seqlens, h0=None, segments=0, ...) -> (o, hT)
  decode(q, k, v, z, A, beta, S) -> o          (S updated in place)
  decode_window(A, S, window=..., replay=..., n_accept=...) -> o
  prefill_checkpoints(..., interval, segments=0) -> (o, hT, checkpoints, offsets)
  qkv_shortconv(xq, xk, xv, wq, wk, wv, cu_seqlens, ...) -> (q, k, v)
  prefill_fused(xq, xk, xv, wq, wk, wv, z, A, beta, cu_seqlens, gate, norm_weight, eps, ...)
      -> (y, hT)                               (the three in one call, bf16)
  output_gate(o, g, w, eps) -> y
  prefill_backward(q, k, v, z, A, beta, cu_seqlens, grad_o, h0=None, grad_hT=None, segments=0)
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


class PrefillOptions(ctypes.Structure):
    """struct kda_prefill_options (include/kda.h)."""
    _fields_ = [("segments", ctypes.c_int), ("checkpoint_interval", ctypes.c_int),
                ("checkpoints", ctypes.c_void_p), ("checkpoint_offsets", ctypes.c_void_p),
                ("blocks", ctypes.c_int)]


def options(segments: int = 0, interval: int = 0, checkpoints=None, checkpoint_offsets=None, blocks: int = 0):
    """A PrefillOptions by value; pointers as ints (or None)."""
    return PrefillOptions(int(segments), int(interval), checkpoints, checkpoint_offsets, int(blocks))


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
    op = ctypes.POINTER(PrefillOptions)
    L.kda_prefill_ex.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp, op, vp,
                                 sz, vp]
    L.kda_prefill_ex.restype = ci
    L.kda_prefill_ex_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, op]
    L.kda_prefill_ex_workspace_size.restype = sz
    L.kda_prefill_noalloc.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp, vp]
    L.kda_prefill_noalloc.restype = ci
    L.kda_prefill_fused.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                    vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    L.kda_prefill_fused.restype = ci
    L.kda_prefill_fused_ex.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                       vp, vp, ctypes.c_float, vp, vp, op, vp, sz, vp]
    L.kda_prefill_fused_ex.restype = ci
    L.kda_prefill_fused_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, op]
    L.kda_prefill_fused_workspace_size.restype = sz
    L.kda_decode.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, vp, vp]
    L.kda_decode.restype = ci
    L.kda_decode_fused.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   ctypes.c_float, ci, ci, ci, ci, vp, vp]
    L.kda_decode_fused.restype = ci
    L.kda_qkv_shortconv.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp, vp, vp,
                                    vp, vp]
    L.kda_qkv_shortconv.restype = ci
    L.kda_output_gate.argtypes = [ci, vp, vp, vp, ctypes.c_float, ci, ci, ci, vp, vp]
    L.kda_output_gate.restype = ci
    L.kda_decode_window.argtypes = [ci, vp, vp, vp, vp, vp, ci, vp, vp, vp, vp, vp, ci, vp, vp, ci, ci,
                                    ci, ci, vp, ci, vp]
    L.kda_decode_window.restype = ci
    L.kda_prefill_backward.argtypes = [ci, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, vp, vp,
                                       vp, vp, vp, vp, vp, vp, vp, op, vp, sz, vp]
    L.kda_prefill_backward.restype = ci
    L.kda_prefill_backward_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, op]
    L.kda_prefill_backward_workspace_size.restype = sz
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


def _opt_ref(opts):
    return None if opts is None else ctypes.byref(opts)


def kda_prefill_ex(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT, opts,
                   workspace, workspace_bytes, stream) -> int:
    """opts: a PrefillOptions or None."""
    return lib().kda_prefill_ex(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT,
                                _opt_ref(opts), workspace, workspace_bytes, stream)


def kda_prefill_noalloc(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT,
                        stream) -> int:
    return lib().kda_prefill_noalloc(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o,
                                     hT, stream)


NOALLOC_SCRATCH_BYTES = 256 << 20   # KDA_NOALLOC_SCRATCH_BYTES


def kda_prefill_fused(io_dtype, xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A, beta, h0,
                      cu_seqlens, N, T, H, dk, dv, gate, norm_weight, eps, y, hT, workspace, workspace_bytes,
                      stream) -> int:
    return lib().kda_prefill_fused(io_dtype, xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A, beta,
                                   h0, cu_seqlens, N, T, H, dk, dv, gate, norm_weight, float(eps), y, hT,
                                   workspace, workspace_bytes, stream)


def kda_prefill_fused_workspace_size(N, T, H, dk, dv, io_dtype, opts=None) -> int:
    return int(lib().kda_prefill_fused_workspace_size(N, T, H, dk, dv, io_dtype, _opt_ref(opts)))


def kda_prefill_fused_ex(io_dtype, xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A, beta, h0,
                         cu_seqlens, N, T, H, dk, dv, gate, norm_weight, eps, y, hT, options, workspace,
                         workspace_bytes, stream) -> int:
    return lib().kda_prefill_fused_ex(io_dtype, xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A,
                                      beta, h0, cu_seqlens, N, T, H, dk, dv, gate, norm_weight, float(eps), y, hT,
                                      options, workspace, workspace_bytes, stream)


def kda_decode(io_dtype, q, k, v, z, A, beta, S_inout, N, H, dk, dv, o, stream) -> int:
    return lib().kda_decode(io_dtype, q, k, v, z, A, beta, S_inout, N, H, dk, dv, o, stream)


def kda_decode_fused(io_dtype, xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A, beta, S_inout,
                     gate, norm_weight, eps, N, H, dk, dv, y, stream) -> int:
    return lib().kda_decode_fused(io_dtype, xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, z, A, beta,
                                  S_inout, gate, norm_weight, float(eps), N, H, dk, dv, y, stream)


def kda_qkv_shortconv(io_dtype, xq, xk, xv, wq, wk, wv, cu_seqlens, N, T, H, dk, dv, conv_state_in,
                      conv_state_out, q, k, v, stream) -> int:
    return lib().kda_qkv_shortconv(io_dtype, xq, xk, xv, wq, wk, wv, cu_seqlens, N, T, H, dk, dv,
                                   conv_state_in, conv_state_out, q, k, v, stream)


def kda_output_gate(io_dtype, o, g, w, eps, T, H, dv, y, stream) -> int:
    return lib().kda_output_gate(io_dtype, o, g, w, eps, T, H, dv, y, stream)


def kda_decode_window(io_dtype, rk, rv, rz, rbeta, n_accept, Lr, q, k, v, z, beta, L, A, S_inout,
                      N, H, dk, dv, o, commit_window, stream) -> int:
    return lib().kda_decode_window(io_dtype, rk, rv, rz, rbeta, n_accept, Lr, q, k, v, z, beta, L,
                                   A, S_inout, N, H, dk, dv, o, commit_window, stream)


def kda_prefill_backward(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, grad_o,
                         grad_hT, grad_q, grad_k, grad_v, grad_z, grad_beta, grad_A, grad_h0, opts,
                         workspace, workspace_bytes, stream) -> int:
    return lib().kda_prefill_backward(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv,
                                      grad_o, grad_hT, grad_q, grad_k, grad_v, grad_z, grad_beta, grad_A,
                                      grad_h0, _opt_ref(opts), workspace, workspace_bytes, stream)


def kda_prefill_backward_workspace_size(N, T, H, dk, dv, io_dtype, opts=None) -> int:
    return int(lib().kda_prefill_backward_workspace_size(N, T, H, dk, dv, io_dtype, _opt_ref(opts)))


def kda_prefill_workspace_size(N, T, H, dk, dv, io_dtype) -> int:
    return int(lib().kda_prefill_workspace_size(N, T, H, dk, dv, io_dtype))


def kda_prefill_ex_workspace_size(N, T, H, dk, dv, io_dtype, opts=None) -> int:
    return int(lib().kda_prefill_ex_workspace_size(N, T, H, dk, dv, io_dtype, _opt_ref(opts)))


def kda_prefill_segments(N, T, H, dk, dv, io_dtype) -> int:
    return lib().kda_prefill_segments(N, T, H, dk, dv, io_dtype)


def kda_status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def kda_build_info() -> str:
    return lib().kda_build_info().decode()


# ---------------------------------------------------------------------------
# torch wrappers (allocation, argument checks and pointer marshalling only)
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


def _check(name, t, shape=None, dtype=None, device=None):
    """Raise unless t (skipped when None) is a contiguous tensor of the given
    shape (a tuple; None entries match any size) and dtype.  The C ABI sees
    only pointers, so a wrong dtype or a short tensor would be read or written
    out of bounds on the device.  Where the tensor lives is checked last, by
    _on_gpu, so that these checks run the same on any device.  (`device` is
    accepted for symmetry with the callers and checked in _on_gpu.)"""
    torch = _torch()
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and w != g for w, g in zip(shape, t.shape)):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape),
                             tuple("*" if w is None else w for w in shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _on_gpu(device, **tensors):
    """Raise unless every given tensor is on the GPU `device` (the library
    has no CPU path)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor (the library has no CPU path)" % name)
        if t.device != device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _check_prefill_inputs(q, k, v, z, A, beta, cu_seqlens, h0):
    """Check the prefill inputs against q; returns (io, N, T, H, dk, dv)."""
    torch = _torch()
    _check("q", q, (None, None, None))
    io = _io_code(q)
    T, H, dk = q.shape
    dev = q.device
    _check("k", k, (T, H, dk), q.dtype, dev)
    _check("v", v, (T, H, None), q.dtype, dev)
    dv = v.shape[-1]
    _check("z", z, (T, H, dk), torch.float32, dev)
    _check("A", A, (H,), torch.float32, dev)
    _check("beta", beta, (T, H), torch.float32, dev)
    _check("cu_seqlens", cu_seqlens, (None,), torch.int32, dev)
    if cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens needs N + 1 >= 1 entries")
    N = cu_seqlens.numel() - 1
    _check("h0", h0, (N, H, dv, dk), torch.float32, dev)
    return io, N, T, H, dk, dv


def _check_workspace(workspace, need, dev):
    if workspace.numel() < need:
        raise ValueError("workspace holds %d bytes, the call needs %d" % (workspace.numel(), need))


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def prefill_workspace(N, T, H, d, io_dtype, device, segments: int = 0, blocks: int = 0):
    """Allocate the prefill workspace (a byte tensor of the size the library asks)."""
    torch = _torch()
    n = kda_prefill_ex_workspace_size(N, T, H, d, d, io_dtype, options(segments, blocks=blocks))
    if n == 0:
        raise ValueError("unsupported prefill sizes N=%d T=%d H=%d d=%d segments=%d blocks=%d"
                         % (N, T, H, d, segments, blocks))
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill(q, k, v, z, A, beta, cu_seqlens, h0=None, o=None, hT=None, workspace=None,
            final_state: bool = True, segments: int = 0, blocks: int = 0):
    """KDA prefill over packed sequences.  Returns (o, hT); hT is None when
    final_state is False and no hT buffer is given.  segments: 0 = automatic,
    1 = never split, 2..16 = split every long sequence into that many.
    blocks: the chunk-block pipeline, 0 = automatic, 1 = off, 2..16 = that
    many blocks (bf16 path without segments or checkpoints)."""
    torch = _torch()
    io, N, T, H, dk, dv = _check_prefill_inputs(q, k, v, z, A, beta, cu_seqlens, h0)
    dev = q.device
    _check("o", o, (T, H, dv), q.dtype, dev)
    _check("hT", hT, (N, H, dv, dk), torch.float32, dev)
    _check("workspace", workspace, (None,), torch.uint8, dev)
    _on_gpu(dev, q=q, k=k, v=v, z=z, A=A, beta=beta, cu_seqlens=cu_seqlens, h0=h0, o=o, hT=hT,
            workspace=workspace)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if hT is None and final_state:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    opts = options(segments, blocks=blocks)
    if workspace is None:
        workspace = prefill_workspace(N, T, H, dk, io, dev, segments, blocks)
    _check_workspace(workspace, kda_prefill_ex_workspace_size(N, T, H, dk, dv, io, opts), dev)
    st = kda_prefill_ex(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(h0),
                        _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(o), _ptr(hT), opts, _ptr(workspace),
                        workspace.numel(), _stream(dev))
    if st != 0:
        raise KdaError("kda_prefill_ex", st)
    return o, hT


def decode(q, k, v, z, A, beta, S, o=None):
    """One decode step; S ([N, H, dv, dk] fp32) is updated in place.  Returns o."""
    torch = _torch()
    _check("q", q, (None, None, None))
    io = _io_code(q)
    N, H, dk = q.shape
    dev = q.device
    _check("k", k, (N, H, dk), q.dtype, dev)
    _check("v", v, (N, H, None), q.dtype, dev)
    dv = v.shape[-1]
    _check("z", z, (N, H, dk), torch.float32, dev)
    _check("A", A, (H,), torch.float32, dev)
    _check("beta", beta, (N, H), torch.float32, dev)
    _check("S", S, (N, H, dv, dk), torch.float32, dev)
    _check("o", o, (N, H, dv), q.dtype, dev)
    _on_gpu(dev, q=q, k=k, v=v, z=z, A=A, beta=beta, S=S, o=o)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    st = kda_decode(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(S), N, H,
                    dk, dv, _ptr(o), _stream(dev))
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
    _check("S", S, (None, None, None, None), torch.float32)
    N, H, dv, dk = S.shape
    dev = S.device
    _check("A", A, (H,), torch.float32, dev)
    io_t = None
    if window is not None:
        io_t = window["q"].dtype
    elif replay is not None:
        io_t = replay["k"].dtype
    if io_t is not None and io_t not in (torch.bfloat16, torch.float32):
        raise TypeError("window and replay tensors must be bfloat16 or float32, got %s" % io_t)
    rk = rv = rz = rb = None
    Lr = 0
    if replay is not None:
        rk, rv, rz, rb = replay["k"], replay["v"], replay["z"], replay["beta"]
        _check("replay k", rk, (N, None, H, dk), io_t, dev)
        Lr = rk.shape[1]
        _check("replay v", rv, (N, Lr, H, dv), io_t, dev)
        _check("replay z", rz, (N, Lr, H, dk), torch.float32, dev)
        _check("replay beta", rb, (N, Lr, H), torch.float32, dev)
        if n_accept is None:
            raise ValueError("n_accept is required with a replay window")
        _check("n_accept", n_accept, (N,), torch.int32, dev)
    q = k = v = z = b = None
    L = 0
    if window is not None:
        q, k, v, z, b = (window[n] for n in ("q", "k", "v", "z", "beta"))
        _check("window q", q, (N, None, H, dk), io_t, dev)
        L = q.shape[1]
        _check("window k", k, (N, L, H, dk), io_t, dev)
        _check("window v", v, (N, L, H, dv), io_t, dev)
        _check("window z", z, (N, L, H, dk), torch.float32, dev)
        _check("window beta", b, (N, L, H), torch.float32, dev)
    io = KDA_BF16 if io_t == torch.bfloat16 else KDA_F32
    if L > 0:
        _check("o", o, (N, L, H, dv), io_t, dev)
    _on_gpu(dev, S=S, A=A, n_accept=n_accept, o=o, rk=rk, rv=rv, rz=rz, rbeta=rb, q=q, k=k, v=v, z=z,
            beta=b)
    if L > 0:
        if o is None:
            o = torch.empty((N, L, H, dv), dtype=io_t, device=dev)
    st = kda_decode_window(io, _ptr(rk), _ptr(rv), _ptr(rz), _ptr(rb), _ptr(n_accept), Lr,
                           _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(b), L, _ptr(A), _ptr(S),
                           N, H, dk, dv, _ptr(o), 1 if commit_window else 0, _stream(dev))
    if st != 0:
        raise KdaError("kda_decode_window", st)
    return o if L > 0 else None


def prefill_checkpoints(q, k, v, z, A, beta, cu_seqlens, interval: int, h0=None, o=None, hT=None,
                        checkpoints=None, offsets=None, workspace=None, segments: int = 0):
    """prefill() that also saves the state every `interval` tokens of every
    sequence.  Returns (o, hT, checkpoints [T // interval, H, dv, dk],
    offsets [N + 1]): sequence n's checkpoints are
    checkpoints[offsets[n]:offsets[n + 1]], in token order."""
    torch = _torch()
    io, N, T, H, dk, dv = _check_prefill_inputs(q, k, v, z, A, beta, cu_seqlens, h0)
    if interval <= 0 or interval % 64 != 0:
        raise ValueError("interval must be a positive multiple of 64, got %d" % interval)
    dev = q.device
    _check("o", o, (T, H, dv), q.dtype, dev)
    _check("hT", hT, (N, H, dv, dk), torch.float32, dev)
    _check("checkpoints", checkpoints, (T // interval, H, dv, dk), torch.float32, dev)
    _check("offsets", offsets, (N + 1,), torch.int32, dev)
    _check("workspace", workspace, (None,), torch.uint8, dev)
    _on_gpu(dev, q=q, k=k, v=v, z=z, A=A, beta=beta, cu_seqlens=cu_seqlens, h0=h0, o=o, hT=hT,
            checkpoints=checkpoints, offsets=offsets, workspace=workspace)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if hT is None:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    if checkpoints is None:
        checkpoints = torch.empty((T // interval, H, dv, dk), dtype=torch.float32, device=dev)
    if offsets is None:
        offsets = torch.empty(N + 1, dtype=torch.int32, device=dev)
    opts = options(segments, interval, _ptr(checkpoints), _ptr(offsets))
    if workspace is None:
        workspace = prefill_workspace(N, T, H, dk, io, dev, segments)
    _check_workspace(workspace, kda_prefill_ex_workspace_size(N, T, H, dk, dv, io, opts), dev)
    st = kda_prefill_ex(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(h0),
                        _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(o), _ptr(hT), opts, _ptr(workspace),
                        workspace.numel(), _stream(dev))
    if st != 0:
        raise KdaError("kda_prefill_ex", st)
    return o, hT, checkpoints, offsets


def prefill_fused(xq, xk, xv, wq, wk, wv, z, A, beta, cu_seqlens, gate, norm_weight, eps: float, h0=None,
                  conv_state_in=None, conv_state_out=None, y=None, hT=None, workspace=None, final_state=True,
                  segments=0, blocks=0):
    """The feature path, the prefill and the output gate in one call (bf16):
    y = Sigmoid(gate) * RMSNorm(o) with o, hT = prefill(q, k, v, ...) and q, k,
    v = qkv_shortconv(xq, xk, xv, ...).  Returns (y, hT); conv_state_out (may
    be conv_state_in) receives the new conv window.  segments and blocks as for
    prefill (0: automatic)."""
    torch = _torch()
    _check("xq", xq, (None, None, None), torch.bfloat16)
    T, H, d = xq.shape
    dev = xq.device
    _check("xk", xk, (T, H, d), torch.bfloat16, dev)
    _check("xv", xv, (T, H, d), torch.bfloat16, dev)
    for name, t in (("wq", wq), ("wk", wk), ("wv", wv)):
        _check(name, t, (H, d, 4), torch.float32, dev)
    _check("z", z, (T, H, d), torch.float32, dev)
    _check("A", A, (H,), torch.float32, dev)
    _check("beta", beta, (T, H), torch.float32, dev)
    _check("cu_seqlens", cu_seqlens, (None,), torch.int32, dev)
    if cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens needs N + 1 >= 1 entries")
    N = cu_seqlens.numel() - 1
    _check("h0", h0, (N, H, d, d), torch.float32, dev)
    _check("conv_state_in", conv_state_in, (N, 3, H, 3 * d), torch.bfloat16, dev)
    _check("conv_state_out", conv_state_out, (N, 3, H, 3 * d), torch.bfloat16, dev)
    _check("gate", gate, (T, H, d), torch.bfloat16, dev)
    _check("norm_weight", norm_weight, (d,), torch.float32, dev)
    _check("y", y, (T, H, d), torch.bfloat16, dev)
    _check("hT", hT, (N, H, d, d), torch.float32, dev)
    _check("workspace", workspace, (None,), torch.uint8, dev)
    _on_gpu(dev, xq=xq, xk=xk, xv=xv, wq=wq, wk=wk, wv=wv, z=z, A=A, beta=beta, cu_seqlens=cu_seqlens, h0=h0,
            conv_state_in=conv_state_in, conv_state_out=conv_state_out, gate=gate, norm_weight=norm_weight, y=y,
            hT=hT, workspace=workspace)
    if y is None:
        y = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    if hT is None and final_state:
        hT = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    opts = options(segments, blocks=blocks)
    need = kda_prefill_fused_workspace_size(N, T, H, d, d, KDA_BF16, opts)
    if need == 0:
        raise ValueError("unsupported fused prefill sizes N=%d T=%d H=%d d=%d segments=%d blocks=%d"
                         % (N, T, H, d, segments, blocks))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, need, dev)
    st = kda_prefill_fused_ex(KDA_BF16, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv),
                              _ptr(conv_state_in), _ptr(conv_state_out), _ptr(z), _ptr(A), _ptr(beta), _ptr(h0),
                              _ptr(cu_seqlens), N, T, H, d, d, _ptr(gate), _ptr(norm_weight), eps, _ptr(y),
                              _ptr(hT), opts, _ptr(workspace), workspace.numel(), _stream(dev))
    if st != 0:
        raise KdaError("kda_prefill_fused_ex", st)
    return y, hT


def decode_fused(xq, xk, xv, wq, wk, wv, z, A, beta, S, gate, norm_weight, eps: float, conv_state_in=None,
                 conv_state_out=None, y=None):
    """One fused decode step (bf16): y = Sigmoid(gate) * RMSNorm(o) with
    o = decode(q, k, v, z, A, beta, S) and q, k, v the feature path of the new
    token over the carried window.  S is updated in place; conv_state_out
    (may be conv_state_in) receives the window after the token.  Returns y."""
    torch = _torch()
    _check("xq", xq, (None, None, None), torch.bfloat16)
    N, H, d = xq.shape
    dev = xq.device
    _check("xk", xk, (N, H, d), torch.bfloat16, dev)
    _check("xv", xv, (N, H, d), torch.bfloat16, dev)
    for name, t in (("wq", wq), ("wk", wk), ("wv", wv)):
        _check(name, t, (H, d, 4), torch.float32, dev)
    _check("z", z, (N, H, d), torch.float32, dev)
    _check("A", A, (H,), torch.float32, dev)
    _check("beta", beta, (N, H), torch.float32, dev)
    _check("S", S, (N, H, d, d), torch.float32, dev)
    _check("conv_state_in", conv_state_in, (N, 3, H, 3 * d), torch.bfloat16, dev)
    _check("conv_state_out", conv_state_out, (N, 3, H, 3 * d), torch.bfloat16, dev)
    _check("gate", gate, (N, H, d), torch.bfloat16, dev)
    _check("norm_weight", norm_weight, (d,), torch.float32, dev)
    _check("y", y, (N, H, d), torch.bfloat16, dev)
    _on_gpu(dev, xq=xq, xk=xk, xv=xv, wq=wq, wk=wk, wv=wv, z=z, A=A, beta=beta, S=S, conv_state_in=conv_state_in,
            conv_state_out=conv_state_out, gate=gate, norm_weight=norm_weight, y=y)
    if y is None:
        y = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    st = kda_decode_fused(KDA_BF16, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv),
                          _ptr(conv_state_in), _ptr(conv_state_out), _ptr(z), _ptr(A), _ptr(beta), _ptr(S),
                          _ptr(gate), _ptr(norm_weight), eps, N, H, d, d, _ptr(y), _stream(dev))
    if st != 0:
        raise KdaError("kda_decode_fused", st)
    return y


def qkv_shortconv(xq, xk, xv, wq, wk, wv, cu_seqlens, conv_state_in=None, conv_state_out=None,
                  q=None, k=None, v=None):
    """The feature path: returns (q, k, v) = (L2Norm(Swish(ShortConv(xq))), ...,
    Swish(ShortConv(xv))).  conv_state_* are [N, 3, H, 3 d] windows of the
    last pre-convolution tokens (conv_state_out may be conv_state_in)."""
    torch = _torch()
    _check("xq", xq, (None, None, None))
    io = _io_code(xq)
    T, H, d = xq.shape
    dev = xq.device
    for name, t in (("xk", xk), ("xv", xv), ("q", q), ("k", k), ("v", v)):
        _check(name, t, (T, H, d), xq.dtype, dev)
    for name, t in (("wq", wq), ("wk", wk), ("wv", wv)):
        _check(name, t, (H, d, 4), torch.float32, dev)
    _check("cu_seqlens", cu_seqlens, (None,), torch.int32, dev)
    if cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens needs N + 1 >= 1 entries")
    N = cu_seqlens.numel() - 1
    _check("conv_state_in", conv_state_in, (N, 3, H, 3 * d), xq.dtype, dev)
    _check("conv_state_out", conv_state_out, (N, 3, H, 3 * d), xq.dtype, dev)
    _on_gpu(dev, xq=xq, xk=xk, xv=xv, wq=wq, wk=wk, wv=wv, cu_seqlens=cu_seqlens, conv_state_in=conv_state_in,
            conv_state_out=conv_state_out, q=q, k=k, v=v)
    q = torch.empty_like(xq) if q is None else q
    k = torch.empty_like(xk) if k is None else k
    v = torch.empty_like(xv) if v is None else v
    st = kda_qkv_shortconv(io, _ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv),
                           _ptr(cu_seqlens), N, T, H, d, d, _ptr(conv_state_in),
                           _ptr(conv_state_out), _ptr(q), _ptr(k), _ptr(v), _stream(dev))
    if st != 0:
        raise KdaError("kda_qkv_shortconv", st)
    return q, k, v


def output_gate(o, g, w, eps: float, y=None):
    """y = Sigmoid(g) * RMSNorm(o) per (token, head) row; y may be o or g."""
    torch = _torch()
    _check("o", o, (None, None, None))
    io = _io_code(o)
    T, H, dv = o.shape
    dev = o.device
    _check("g", g, (T, H, dv), o.dtype, dev)
    _check("w", w, (dv,), torch.float32, dev)
    _check("y", y, (T, H, dv), o.dtype, dev)
    _on_gpu(dev, o=o, g=g, w=w, y=y)
    y = torch.empty_like(o) if y is None else y
    st = kda_output_gate(io, _ptr(o), _ptr(g), _ptr(w), float(eps), T, H, dv, _ptr(y), _stream(dev))
    if st != 0:
        raise KdaError("kda_output_gate", st)
    return y


def prefill_backward(q, k, v, z, A, beta, cu_seqlens, grad_o, h0=None, grad_hT=None, workspace=None,
                     grads=None, segments: int = 0):
    """Gradients of L = sum(grad_o * o) + sum(grad_hT * hT) for the prefill
    o, hT = prefill(q, k, v, z, A, beta, cu_seqlens, h0).  Returns a dict of
    fp32 tensors dq, dk, dv, dz [T, H, d], dbeta [T, H], dA [H] and
    dh0 [N, H, dv, dk].  `grads` may hold preallocated outputs by those names.
    segments: the forward recompute's segment split (0 = automatic)."""
    torch = _torch()
    io, N, T, H, dk, dv = _check_prefill_inputs(q, k, v, z, A, beta, cu_seqlens, h0)
    dev = q.device
    _check("grad_o", grad_o, (T, H, dv), q.dtype, dev)
    _check("grad_hT", grad_hT, (N, H, dv, dk), torch.float32, dev)
    shapes = dict(dq=(T, H, dk), dk=(T, H, dk), dv=(T, H, dv), dz=(T, H, dk), dbeta=(T, H), dA=(H,),
                  dh0=(N, H, dv, dk))
    g = dict(grads or {})
    for name, shape in shapes.items():
        _check(name, g.get(name), shape, torch.float32, dev)
    _check("workspace", workspace, (None,), torch.uint8, dev)
    _on_gpu(dev, q=q, k=k, v=v, z=z, A=A, beta=beta, cu_seqlens=cu_seqlens, grad_o=grad_o, h0=h0,
            grad_hT=grad_hT, workspace=workspace, **{n: t for n, t in g.items() if n in shapes})
    for name, shape in shapes.items():
        if g.get(name) is None:
            g[name] = torch.empty(shape, dtype=torch.float32, device=dev)
    opts = options(segments)
    n = kda_prefill_backward_workspace_size(N, T, H, dk, dv, io, opts)
    if n == 0:
        raise ValueError("unsupported backward sizes N=%d T=%d H=%d d=%d segments=%d" % (N, T, H, dk, segments))
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, n, dev)
    st = kda_prefill_backward(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(h0),
                              _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(grad_o), _ptr(grad_hT),
                              _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dz"]), _ptr(g["dbeta"]),
                              _ptr(g["dA"]), _ptr(g["dh0"]), opts, _ptr(workspace), workspace.numel(),
                              _stream(dev))
    if st != 0:
        raise KdaError("kda_prefill_backward", st)
    return g
