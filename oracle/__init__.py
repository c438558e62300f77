"""fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg are the only callers.  Nothing here is imported by
the HIP path, and the HIP path has no CPU fallback to this module.

Contents
  build()            compile kda_oracle.c (plain C, fp64, OpenMP)
  prefill(...)       token-loop recurrence over packed sequences (C)
  decode(...)        one decode step (C)
  backward(...)      reverse-mode gradients of the prefill (C)
  gate(A, z)         the bounded log-decay, numpy fp64
  chunkwise.prefill  the chunkwise-parallel form, numpy fp64 (a cross-check)
  features           the q/k/v feature path (ShortConv -> Swish -> L2Norm) and
                     the output gate (Sigmoid(g) * RMSNorm(o)), numpy fp64

Every input array is numpy: q, k, v either float32 or the raw uint16 bits of
bfloat16 (``workloads.as_numpy`` makes them); z, A, beta float32; the
initial state float32 or float64 (widened exactly); cu_seqlens int32.
Outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libkda_oracle.so")

G_MIN = -5.0
CFLAGS = ["-O3", "-march=x86-64-v2", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared", "-std=c11", "-Wall", "-Wextra"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc.  Returns the path of the shared library."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_lib_cache = {}


def load(path: str = _LIB):
    """Load (building first if needed) the oracle library at `path`."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != _LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    vp, fp, dp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    ci = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [ci, vp, vp, vp, fp, fp, fp, fp, vp, ci, ci, ci,
                                       ci, dp, dp, ci]
    lib.kda_oracle_prefill.restype = ci
    lib.kda_oracle_decode.argtypes = [ci, vp, vp, vp, fp, fp, fp, fp, ci, ci, ci, ci,
                                      dp, dp, ci]
    lib.kda_oracle_decode.restype = ci
    lib.kda_oracle_backward.argtypes = [ci, vp, vp, vp, fp, fp, fp, fp, vp, ci, ci, ci, ci, dp, dp,
                                        dp, dp, dp, dp, dp, dp, dp, ci]
    lib.kda_oracle_backward.restype = ci
    lib.kda_oracle_gate.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.kda_oracle_gate.restype = ctypes.c_double
    lib.kda_oracle_max_threads.restype = ci
    _lib_cache[path] = lib
    return lib


def _io_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return 1
    if x.dtype == np.uint16:
        return 0
    raise TypeError("q/k/v must be float32 or bfloat16 bits (uint16), got %s" % x.dtype)


def _ptr(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _c(x, dtype=None):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if dtype is not None and x.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, x.dtype))
    return x


def prefill(q, k, v, z, A, beta, h0, cu_seqlens, nthreads: int = 0, lib_path: str = _LIB):
    """Token-loop KDA over packed sequences.  Returns (o, hT) as float64.

    q, k: [T, H, dk]; v: [T, H, dv]; z: [T, H, dk]; A: [H]; beta: [T, H];
    h0: [N, H, dv, dk] (float32 or float64; widened to float64) or None;
    cu_seqlens: [N + 1].
    """
    q, k, v = _c(q), _c(k), _c(v)
    io = _io_code(q)
    assert _io_code(k) == io and _io_code(v) == io
    z, A, beta = _c(z, np.float32), _c(A, np.float32), _c(beta, np.float32)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    cu = _c(np.asarray(cu_seqlens, dtype=np.int32), np.int32)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and z.shape == (T, H, dk) and v.shape[:2] == (T, H)
    assert beta.shape == (T, H) and A.shape == (H,) and int(cu[-1]) == T
    if h0 is not None:
        assert h0.shape == (N, H, dv, dk)
    o = np.zeros((T, H, dv), dtype=np.float64)
    hT = np.zeros((N, H, dv, dk), dtype=np.float64)
    rc = load(lib_path).kda_oracle_prefill(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A),
                                           _ptr(beta), _ptr(h0), _ptr(cu), N, H, dk, dv,
                                           _ptr(o), _ptr(hT), int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_prefill failed (%d)" % rc)
    return o, hT


def decode(q, k, v, z, A, beta, S, nthreads: int = 0, lib_path: str = _LIB):
    """One decode step.  q, k, z: [N, H, dk]; v: [N, H, dv]; beta: [N, H];
    S: [N, H, dv, dk] float32 or float64.  Returns (o [N, H, dv], S_new) as float64."""
    q, k, v = _c(q), _c(k), _c(v)
    io = _io_code(q)
    z, A, beta = _c(z, np.float32), _c(A, np.float32), _c(beta, np.float32)
    S = np.ascontiguousarray(S, dtype=np.float64)
    N, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((N, H, dv), dtype=np.float64)
    S_out = np.zeros((N, H, dv, dk), dtype=np.float64)
    rc = load(lib_path).kda_oracle_decode(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A),
                                          _ptr(beta), _ptr(S), N, H, dk, dv, _ptr(o),
                                          _ptr(S_out), int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode failed (%d)" % rc)
    return o, S_out


def backward(q, k, v, z, A, beta, h0, cu_seqlens, dO, dhT=None, nthreads: int = 0,
             lib_path: str = _LIB) -> dict:
    """Gradients of L = sum(dO * o) + sum(dhT * hT) through the prefill
    (token recurrence, reverse mode; see kda_oracle.c).  Inputs as for
    prefill(); dO [T, H, dv] and dhT [N, H, dv, dk] (or None) are widened to
    float64.  Returns float64 arrays dq, dk, dv, dz, dbeta, dA, dh0 (dh0 is
    the gradient of h0, whether h0 was given or zero)."""
    q, k, v = _c(q), _c(k), _c(v)
    io = _io_code(q)
    assert _io_code(k) == io and _io_code(v) == io
    z, A, beta = _c(z, np.float32), _c(A, np.float32), _c(beta, np.float32)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    cu = _c(np.asarray(cu_seqlens, dtype=np.int32), np.int32)
    dO = np.ascontiguousarray(dO, dtype=np.float64)
    dhT = None if dhT is None else np.ascontiguousarray(dhT, dtype=np.float64)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    assert dO.shape == (T, H, dv) and int(cu[-1]) == T
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dz=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)), dA=np.zeros(H),
               dh0=np.zeros((N, H, dv, dk)))
    rc = load(lib_path).kda_oracle_backward(io, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A),
                                            _ptr(beta), _ptr(h0), _ptr(cu), N, H, dk, dv,
                                            _ptr(dO), _ptr(dhT), _ptr(out["dq"]), _ptr(out["dk"]),
                                            _ptr(out["dv"]), _ptr(out["dz"]), _ptr(out["dbeta"]),
                                            _ptr(out["dA"]), _ptr(out["dh0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_backward failed (%d)" % rc)
    return out


def gate(A, z):
    """g = g_min * sigmoid(exp(A_h) * z) in fp64 ("Kimi K3：架构、训练与推理系统研究"
    §3.2; the devpress K3 walk-through §3.2, Eq 5).

    A broadcasts over the head axis: z [..., H, dk], A [H]."""
    A = np.asarray(A, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    x = np.exp(A)[:, None] * z
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-x))
    return G_MIN * s


def max_threads(lib_path: str = _LIB) -> int:
    return int(load(lib_path).kda_oracle_max_threads())


def widen(x: np.ndarray) -> np.ndarray:
    """float32 or bfloat16 bits (uint16) -> float64, exactly."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)
