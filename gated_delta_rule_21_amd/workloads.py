"""Seeded synthetic inputs for the KDA prefill and decode paths.

This module only draws random tensors and packs them in the layouts the
library takes.  It holds none of the method's arithmetic: no gate, no decay,
no recurrence.  Both the HIP path (tests, bench) and the fp64 oracle read the
tensors it makes, so it is the one piece of code the two sides share.

Shapes follow the model configuration printed on the pages (96 heads, key and
value head dim 128, "Kimi K3：架构、训练与推理系统研究" §1 table and §3.4; the
devpress K3 walk-through, Table 1).  There is no public dataset for this
kernel: every workload is synthetic.

Distributions (identical for every workload unless noted):
  q, k ~ N(0, 1) per element, then L2-normalised over the key dim per
         (token, head) in fp32, then rounded to the I/O dtype (RNE).  The
         pages make unit-norm q and k a property of the caller's feature path
         (ShortConv -> Swish -> L2Norm, "Kimi K3：架构、训练与推理系统研究" §3.2), not of
         the recurrence.
  v    ~ N(0, 1), rounded to the I/O dtype.
  beta = sigmoid(N(0, 1)) in fp32, used by the library as given.
  z    ~ N(0, 1) in fp32, per token, head and key channel.
  A_h  ~ U(-1, 1) in fp32, one per head.
  h0   ~ N(0, sigma^2) in fp32 with the per-workload sigma, or absent.

Layouts: q, k, z [T_tot, H, dk]; v, o [T_tot, H, dv]; beta [T_tot, H];
A [H]; h0 / hT / decode state [N, H, dv, dk] (row j = value channel,
contiguous over key channels); cu_seqlens [N + 1] int32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    kind: str                 # "prefill" or "decode"
    N: int                    # sequences
    H: int                    # heads
    d: int                    # dk = dv
    io: str                   # "bf16" or "f32" for q, k, v, o
    lens: Optional[tuple] = None          # prefill: per-sequence lengths
    lognormal_total: Optional[int] = None  # varlen: total tokens
    h0_std: Optional[float] = None        # None: no initial state (zeros)
    state_std: Optional[float] = None     # decode: state distribution
    chunk: int = 64
    description: str = ""


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", 0, "prefill", N=1, H=2, d=32, io="f32", lens=(256,),
        description="tiny fp32 KDA forward, B=1 H=2 T=256 d=32, h0=0"),
    "small_head": Workload(
        "small_head", 1, "prefill", N=2, H=8, d=128, io="bf16",
        lens=(8192, 8192), h0_std=0.01,
        description="small-head prefill, B=2 H=8 T=8192 d=128, bf16 q/k/v"),
    "k3_prefill": Workload(
        "k3_prefill", 2, "prefill", N=1, H=96, d=128, io="bf16",
        lens=(65536,),
        description="K3-shaped single-layer prefill, B=1 H=96 T=65536 d=128"),
    "k3_decode": Workload(
        "k3_decode", 3, "decode", N=256, H=96, d=128, io="bf16",
        state_std=0.05,
        description="batched decode step, 256 sequences x H=96 x 128x128 fp32 state"),
    "k3_varlen": Workload(
        "k3_varlen", 4, "prefill", N=32, H=96, d=128, io="bf16",
        lognormal_total=262144, h0_std=0.01,
        description="varlen packed prefill, 32 lognormal lengths summing to 262144, H=96"),
}

BASE_SEED = 1000


def torch_dtype(io: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[io]


def lognormal_lengths(n: int, total: int, seed: int, mu: float = math.log(8192.0),
                      sigma: float = 1.0) -> list:
    """n lognormal(mu, sigma) draws scaled to sum exactly to `total`.

    Scale, floor, then hand the remaining tokens one each to the largest
    fractional remainders (ties broken by index).  Every length is >= 1.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.lognormal(mean=mu, sigma=sigma, size=n)
    x = x / x.sum() * total
    base = np.maximum(np.floor(x).astype(np.int64), 1)
    rem = total - int(base.sum())
    frac = x - np.floor(x)
    order = sorted(range(n), key=lambda i: (-frac[i], i))
    i = 0
    while rem > 0:
        base[order[i % n]] += 1
        rem -= 1
        i += 1
    while rem < 0:  # only if the >=1 clamp overshot
        j = int(np.argmax(base))
        base[j] -= 1
        rem += 1
    assert int(base.sum()) == total
    return [int(v) for v in base]


def seq_lengths(w: Workload, seed: Optional[int] = None) -> list:
    if w.lens is not None:
        return list(w.lens)
    s = BASE_SEED + w.index if seed is None else seed
    return lognormal_lengths(w.N, w.lognormal_total, s + 7919)


def cu_from_lengths(lens) -> torch.Tensor:
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    # L2-normalise over the last dim in fp32 (input preparation, not the method)
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def random_prefill(lens, H: int, d: int, io: str = "bf16", h0_std: Optional[float] = None,
                   seed: int = BASE_SEED, device="cpu", z_shift: float = 0.0,
                   dk: Optional[int] = None, dv: Optional[int] = None) -> dict:
    """Draw one prefill batch.  Returns a dict of tensors on `device`.

    `z_shift` moves the decay logits (-4: weak decay, +6: saturated decay).
    """
    dk = d if dk is None else dk
    dv = d if dv is None else dv
    device = torch.device(device)
    T = int(sum(lens))
    N = len(lens)
    g = _gen(device, seed)
    f32 = torch.float32
    A = torch.rand(H, generator=g, device=device, dtype=f32) * 2.0 - 1.0
    q = _unit_rows(torch.randn(T, H, dk, generator=g, device=device, dtype=f32))
    q = q.to(torch_dtype(io))
    k = _unit_rows(torch.randn(T, H, dk, generator=g, device=device, dtype=f32))
    k = k.to(torch_dtype(io))
    v = torch.randn(T, H, dv, generator=g, device=device, dtype=f32).to(torch_dtype(io))
    beta = torch.sigmoid(torch.randn(T, H, generator=g, device=device, dtype=f32))
    z = torch.randn(T, H, dk, generator=g, device=device, dtype=f32)
    if z_shift:
        z += z_shift
    h0 = None
    if h0_std is not None:
        h0 = torch.randn(N, H, dv, dk, generator=g, device=device, dtype=f32) * h0_std
    cu = cu_from_lengths(lens).to(device)
    return dict(q=q, k=k, v=v, z=z, A=A, beta=beta, h0=h0, cu_seqlens=cu,
                N=N, H=H, dk=dk, dv=dv, T=T, io=io)


def random_cotangents(T: int, N: int, H: int, d: int, io: str = "bf16", final_state: bool = True,
                      seed: int = BASE_SEED + 7, device="cpu") -> dict:
    """Upstream gradients for the prefill backward: dO ~ N(0, 1) [T, H, d] in
    the io dtype and, optionally, dhT ~ N(0, 1) [N, H, d, d] fp32."""
    device = torch.device(device)
    g = _gen(device, seed)
    f32 = torch.float32
    dO = torch.randn(T, H, d, generator=g, device=device, dtype=f32).to(torch_dtype(io))
    dhT = torch.randn(N, H, d, d, generator=g, device=device, dtype=f32) if final_state else None
    return dict(dO=dO, dhT=dhT)


def random_decode(N: int, H: int, d: int, io: str = "bf16", state_std: float = 0.05,
                  seed: int = BASE_SEED + 3, device="cpu", z_shift: float = 0.0) -> dict:
    """Draw one decode batch: one token per sequence plus the fp32 state."""
    device = torch.device(device)
    g = _gen(device, seed)
    f32 = torch.float32
    A = torch.rand(H, generator=g, device=device, dtype=f32) * 2.0 - 1.0
    q = _unit_rows(torch.randn(N, H, d, generator=g, device=device, dtype=f32)).to(torch_dtype(io))
    k = _unit_rows(torch.randn(N, H, d, generator=g, device=device, dtype=f32)).to(torch_dtype(io))
    v = torch.randn(N, H, d, generator=g, device=device, dtype=f32).to(torch_dtype(io))
    beta = torch.sigmoid(torch.randn(N, H, generator=g, device=device, dtype=f32))
    z = torch.randn(N, H, d, generator=g, device=device, dtype=f32)
    if z_shift:
        z += z_shift
    S = torch.randn(N, H, d, d, generator=g, device=device, dtype=f32) * state_std
    return dict(q=q, k=k, v=v, z=z, A=A, beta=beta, S=S, N=N, H=H, dk=d, dv=d, io=io)


def random_decode_window(N: int, H: int, d: int, Lr: int, L: int, io: str = "bf16",
                         state_std: float = 0.05, seed: int = BASE_SEED + 5, device="cpu") -> dict:
    """Draw a decode-window batch: the committed state, a replay window of Lr
    tokens with n_accept ~ U{0..Lr} per sequence, and a new window of L
    tokens.  Per-token inputs are drawn as in random_decode (unit-norm q and
    k); layouts [N][len][H][d]."""
    device = torch.device(device)
    g = _gen(device, seed)
    f32 = torch.float32
    A = torch.rand(H, generator=g, device=device, dtype=f32) * 2.0 - 1.0
    S = torch.randn(N, H, d, d, generator=g, device=device, dtype=f32) * state_std

    def tokens(n_tok, with_q):
        out = {}
        if with_q:
            out["q"] = _unit_rows(torch.randn(N, n_tok, H, d, generator=g, device=device,
                                              dtype=f32)).to(torch_dtype(io))
        out["k"] = _unit_rows(torch.randn(N, n_tok, H, d, generator=g, device=device,
                                          dtype=f32)).to(torch_dtype(io))
        out["v"] = torch.randn(N, n_tok, H, d, generator=g, device=device, dtype=f32).to(torch_dtype(io))
        out["z"] = torch.randn(N, n_tok, H, d, generator=g, device=device, dtype=f32)
        out["beta"] = torch.sigmoid(torch.randn(N, n_tok, H, generator=g, device=device, dtype=f32))
        return out

    replay = tokens(Lr, False)
    window = tokens(L, True)
    n_accept = torch.randint(0, Lr + 1, (N,), generator=g, device=device, dtype=torch.int32)
    return dict(A=A, S=S, replay=replay, window=window, n_accept=n_accept, N=N, H=H, dk=d, dv=d,
                Lr=Lr, L=L, io=io)


def random_features(lens, H: int, d: int, io: str = "bf16", window: bool = True,
                    seed: int = BASE_SEED + 6, device="cpu") -> dict:
    """Draw inputs of the feature path and output gate: pre-convolution
    projections x ~ N(0, 1) in the io dtype, taps ~ N(0, 1/4) fp32, an
    optional carried window [N, 3, H, 3 d] ~ N(0, 1), the recurrence output o
    ~ N(0, 1) and gate g ~ N(0, 4) in the io dtype, RMSNorm weight ~ 1 + N(0, 0.1)."""
    device = torch.device(device)
    g = _gen(device, seed)
    f32 = torch.float32
    T, N = int(sum(lens)), len(lens)
    io_t = torch_dtype(io)
    x = lambda: torch.randn(T, H, d, generator=g, device=device, dtype=f32).to(io_t)
    taps = lambda: torch.randn(H, d, 4, generator=g, device=device, dtype=f32) * 0.5
    out = dict(xq=x(), xk=x(), xv=x(), wq=taps(), wk=taps(), wv=taps(), cu_seqlens=cu_from_lengths(lens).to(device),
               N=N, T=T, H=H, d=d, io=io)
    out["window"] = (torch.randn(N, 3, H, 3 * d, generator=g, device=device, dtype=f32).to(io_t)
                     if window else None)
    out["o"] = x()
    out["g"] = (torch.randn(T, H, d, generator=g, device=device, dtype=f32) * 2.0).to(io_t)
    out["w"] = 1.0 + 0.1 * torch.randn(d, generator=g, device=device, dtype=f32)
    return out


def make(name: str, device="cpu", seed: Optional[int] = None, **over) -> dict:
    """Inputs for a named workload (see WORKLOADS)."""
    w = WORKLOADS[name]
    s = BASE_SEED + w.index if seed is None else seed
    if w.kind == "decode":
        return random_decode(w.N, w.H, w.d, w.io, w.state_std, seed=s, device=device, **over)
    return random_prefill(seq_lengths(w, s), w.H, w.d, w.io, w.h0_std, seed=s,
                          device=device, **over)


def as_numpy(x: Optional[torch.Tensor]):
    """Host numpy view of a tensor; bf16 comes back as its raw uint16 bits."""
    if x is None:
        return None
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()
