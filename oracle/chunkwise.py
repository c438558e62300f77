"""Chunkwise-parallel KDA in numpy fp64 -- a second, independent algorithm.

TEST INFRASTRUCTURE ONLY.  It cross-checks the token-loop oracle on tiny
inputs (forward and backward); it is never run on large shapes and never
called by the HIP path.

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


def backward(q, k, v, z, A, beta, h0, cu_seqlens, dO, dhT=None, chunk: int = 64) -> dict:
    """Gradients of L = sum(dO * o) + sum(dhT * hT), chunk by chunk (fp64).

    The same chunk form as prefill(), differentiated as matrices.  Per chunk,
    with S the state at its start, dS' the gradient at its end, P = Tril(Qg
    Kinv^T), Kt = (gamma_C / Gamma) * K and T = (I + A_kk)^{-1}:
      dV' = P^T dO + Kt dS'
      dS  = Qg^T dO + Diag(gamma_C) dS' - W^T dV'        (to the previous chunk)
      dP = Tril(dO V'^T),  dW = -dV' S^T,  dM = dW Kg^T + dV' V^T
      dT = dM Diag(beta),  dA_kk = -T^T dT T^T (strictly lower)
    and the products back to K, Q, V, beta and the log-decay G = log Gamma,
    whose gradient turns into dg by a reverse cumulative sum over the chunk.
    A second algorithm for the token-sweep backward of the C oracle."""
    if not 1 <= chunk <= MAX_SAFE_CHUNK:
        raise ValueError("chunk must be in [1, %d] for the naive fp64 form" % MAX_SAFE_CHUNK)
    Q, K, V = _widen(q), _widen(k), _widen(v)
    T, H, dk = Q.shape
    dv = V.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    Af = np.asarray(A, np.float64)
    Z = np.asarray(z, np.float64)
    alpha = np.exp(_gate(A, z))
    B = np.asarray(beta, dtype=np.float64)
    dO = np.asarray(dO, np.float64)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dz=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)), dA=np.zeros(H), dh0=np.zeros((N, H, dv, dk)))
    for n in range(N):
        for h in range(H):
            S0 = np.zeros((dk, dv)) if h0 is None else np.asarray(h0[n, h], np.float64).T.copy()
            bounds = [(c0, min(c0 + chunk, int(cu[n + 1]))) for c0 in range(int(cu[n]), int(cu[n + 1]), chunk)]
            # forward: the state at every chunk start
            starts, S = [], S0
            for c0, c1 in bounds:
                starts.append(S)
                Kc, Vc, bc = K[c0:c1, h], V[c0:c1, h], B[c0:c1, h]
                Gam = np.cumprod(alpha[c0:c1, h], axis=0)
                gC = Gam[-1]
                Kg, Kinv = Gam * Kc, Kc / Gam
                C = c1 - c0
                M = solve_triangular(np.eye(C) + np.tril(bc[:, None] * (Kg @ Kinv.T), -1), np.diag(bc), lower=True,
                                     unit_diagonal=True)
                S = gC[:, None] * S + ((gC / Gam) * Kc).T @ (M @ Vc - M @ Kg @ S)
            dS = np.zeros((dk, dv)) if dhT is None else np.asarray(dhT[n, h], np.float64).T.copy()
            for (c0, c1), S in reversed(list(zip(bounds, starts))):
                Kc, Qc, Vc, bc = K[c0:c1, h], Q[c0:c1, h], V[c0:c1, h], B[c0:c1, h]
                C = c1 - c0
                Gam = np.cumprod(alpha[c0:c1, h], axis=0)
                gC = Gam[-1]
                Kg, Kinv, Qg, Kt = Gam * Kc, Kc / Gam, Gam * Qc, (gC / Gam) * Kc
                R = Kg @ Kinv.T
                Akk = np.tril(bc[:, None] * R, -1)
                Tm = solve_triangular(np.eye(C) + Akk, np.eye(C), lower=True, unit_diagonal=True)
                M = Tm * bc[None, :]
                W, U = M @ Kg, M @ Vc
                Vp = U - W @ S
                P = np.tril(Qg @ Kinv.T)
                dOc = dO[c0:c1, h]
                dVp = P.T @ dOc + Kt @ dS
                dS_prev = Qg.T @ dOc + gC[:, None] * dS - W.T @ dVp
                dP = np.tril(dOc @ Vp.T)
                dQg = dOc @ S.T + dP @ Kinv
                dKinv = dP.T @ Qg
                dKt = Vp @ dS.T
                dgC = np.sum(dS * S, axis=1)
                dW = -dVp @ S.T
                dM = dW @ Kg.T + dVp @ Vc.T
                dKg = M.T @ dW
                dVc = M.T @ dVp
                dT = dM * bc[None, :]
                db = np.sum(dM * Tm, axis=0)
                dAkk = np.tril(-Tm.T @ dT @ Tm.T, -1)
                db += np.sum(dAkk * R, axis=1)
                dR = dAkk * bc[:, None]
                dKg += dR @ Kinv
                dKinv += dR.T @ Kg
                dK = dKg * Gam + dKinv / Gam + dKt * (gC / Gam)
                dQ = dQg * Gam
                dG = dKg * Kg - dKinv * Kinv + dQg * Qg - dKt * Kt
                dG[-1] += np.sum(dKt * Kt, axis=0) + dgC * gC
                dg = np.cumsum(dG[::-1], axis=0)[::-1]        # dg_tau = sum_{r >= tau} dG_r
                x = np.exp(Af[h]) * Z[c0:c1, h]
                s = 1.0 / (1.0 + np.exp(-x))
                dx = dg * (-5.0) * s * (1.0 - s)                 # dg/dx, g = g_min sigmoid(x)
                out["dq"][c0:c1, h] = dQ
                out["dk"][c0:c1, h] = dK
                out["dv"][c0:c1, h] = dVc
                out["dbeta"][c0:c1, h] = db
                out["dz"][c0:c1, h] = dx * np.exp(Af[h])
                out["dA"][h] += np.sum(dx * x)
                dS = dS_prev
            out["dh0"][n, h] = dS.T
    return out
