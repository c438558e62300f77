"""Chunkwise-parallel KDA in numpy fp64 -- a second, independent algorithm.

TEST INFRASTRUCTURE ONLY.  It cross-checks the token-loop oracle on tiny
inputs; it is never run on large shapes and never called by the HIP path.

It follows the chunk formulas of the s1mplewind "kimi-k3" notes, section
"Chunkwise 形式" (derivation steps 1-6 in the same section), written in the
d_k x d_v state orientation of "Kimi K3：架构、训练与推理系统研究" §3.1.  For
a chunk of C rows with stacked K, Q (C x d_k), V (C x d_v), beta (C) and the
inclusive cumulative decay Gamma_r = prod_{j<=r} alpha_j (C x d_k),
gamma_C = Gamma_C:

  M  = (I + StrictTril(Diag(beta) (Gamma*K) (K/Gamma)^T))^{-1} Diag(beta)
  W  = M (Gamma*K)            U = M V
  V' = U - W S                ("pseudo"-value term)
  O  = (Gamma*Q) S + Tril((Gamma*Q)(K/Gamma)^T) V'
  S <- Diag(gamma_C) S + ((gamma_C/Gamma)*K)^T V'

Gamma and K/Gamma are formed naively, as printed.  That is safe in fp64 for
C <= 141 only: the bounded gate keeps each alpha above e^-5 (devpress K3
walk-through §3.2, Eq 5), so 1/Gamma stays below e^(5*141) < DBL_MAX.
Chunks start at every sequence start; the last chunk of a sequence may be
partial.  The triangular solve is a library call (scipy's solve_triangular).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

from . import gate as _gate, widen as _widen

MAX_SAFE_CHUNK = 141


def prefill(q, k, v, z, A, beta, h0, cu_seqlens, chunk: int = 64):
    """Returns (o [T, H, dv], hT [N, H, dv, dk]) in float64."""
    if not 1 <= chunk <= MAX_SAFE_CHUNK:
        raise ValueError("chunk must be in [1, %d] for the naive fp64 form" % MAX_SAFE_CHUNK)
    Q, K, V = _widen(q), _widen(k), _widen(v)
    T, H, dk = Q.shape
    dv = V.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    alpha = np.exp(_gate(A, z))            # [T, H, dk]
    B = np.asarray(beta, dtype=np.float64)  # [T, H]
    o = np.zeros((T, H, dv))
    hT = np.zeros((N, H, dv, dk))
    for n in range(N):
        for h in range(H):
            # state in the mathematical orientation, d_k x d_v
            S = np.zeros((dk, dv)) if h0 is None else np.asarray(h0[n, h], np.float64).T.copy()
            for c0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[n + 1]))
                Kc, Qc, Vc = K[c0:c1, h], Q[c0:c1, h], V[c0:c1, h]
                bc = B[c0:c1, h]
                Gam = np.cumprod(alpha[c0:c1, h], axis=0)   # inclusive, C x dk
                gC = Gam[-1]
                Kg, Kinv, Qg = Gam * Kc, Kc / Gam, Gam * Qc
                L = np.tril(bc[:, None] * (Kg @ Kinv.T), -1)
                C = c1 - c0
                Minv_rhs = np.diag(bc)
                M = solve_triangular(np.eye(C) + L, Minv_rhs, lower=True, unit_diagonal=True)
                W = M @ Kg
                U = M @ Vc
                Vp = U - W @ S
                o[c0:c1, h] = Qg @ S + np.tril(Qg @ Kinv.T) @ Vp
                S = gC[:, None] * S + ((gC / Gam) * Kc).T @ Vp
            hT[n, h] = S.T
    return o, hT
