"""Helpers for the GPU parity tests: move seeded inputs to the GPU, run the
oracle on the same (already rounded) values, compare by relative L2."""
import numpy as np
import torch

import oracle
from gated_delta_rule_21_amd import workloads as W

BF16_TOL = 2e-3     # rel-L2, bf16 inputs with an fp32 state
F32_TOL = 1e-5      # rel-L2, fp32 path


def rel_l2(x, y) -> float:
    x = np.asarray(x, np.float64).ravel()
    y = np.asarray(y, np.float64).ravel()
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def to_gpu(d: dict) -> dict:
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def host(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def oracle_prefill(d: dict, heads=None, nthreads: int = 0):
    """Oracle on the inputs of `d` (CPU or GPU tensors), optionally on a
    subset of heads (sliced before the call, so the oracle runs H' heads)."""
    sel = lambda t: t if heads is None else t[:, heads]
    q, k, v, z, beta = (W.as_numpy(sel(d[n])) for n in ("q", "k", "v", "z", "beta"))
    A = W.as_numpy(d["A"] if heads is None else d["A"][heads])
    h0 = None
    if d.get("h0") is not None:
        h0 = W.as_numpy(d["h0"] if heads is None else d["h0"][:, heads])
    cu = W.as_numpy(d["cu_seqlens"]).astype(np.int32)
    return oracle.prefill(q, k, v, z, A, beta, h0, cu, nthreads=nthreads)


def tol(io: str) -> float:
    return F32_TOL if io == "f32" else BF16_TOL
