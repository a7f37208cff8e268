"""Gradients of the gated delta-rule forward pass, for checking a backward pass.

TEST INFRASTRUCTURE ONLY (as the rest of ``oracle/``): nothing in the product
path may import or call it.

The pages derive no backward pass; the chunked mode is the training mode
(blog summary on the DeltaNet family, "Kernel Triton recurrente fusionado" and
"Pipeline Triton por chunks").  The gradient of a loss through the forward
pass is fixed by the forward pass itself, so this oracle is the token
recurrence of ``gdr_oracle.c`` (the same seven steps, the same order: forget,
write strength, predict from the decayed state, residual, rank-1 write, read
after the write) written again in plain PyTorch CPU ops in float64, and
differentiated by torch's reverse mode.  The loss is
    L = sum(o * do) + sum(S_final * ds_final),
so the returned gradients are the vector-Jacobian products of (o, S_final)
with (do, ds_final).  Pinned against central finite differences of the C
oracle (an independent forward implementation) in tests/test_oracle_backward.py.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(a, requires_grad=True):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64, requires_grad=requires_grad)


def forward_torch(q, k, v, g, beta, s0=None, *, per_channel=False, kaczmarz=False, eps=0.0, scale=1.0,
                  delta_off=False):
    """The token recurrence in float64 torch ops (differentiable).  Shapes as
    for oracle_fwd: q, k [B,T,H,Dk]; v [B,T,H,Dv]; g [B,T,H] or [B,T,H,Dk];
    beta [B,T,H] (eta when kaczmarz; unused with delta_off, the additive write
    S = S~ + k v^T of the textbook page's update table); s0 [B,H,Dk,Dv] or None."""
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    S = s0 if s0 is not None else torch.zeros((B, H, Dk, Dv), dtype=torch.float64)
    outs = []
    for t in range(T):
        kt, qt, vt = k[:, t], q[:, t], v[:, t]            # [B,H,Dk], [B,H,Dk], [B,H,Dv]
        a = torch.exp(g[:, t])                             # [B,H] or [B,H,Dk]
        S = S * (a[..., :, None] if per_channel else a[..., None, None])   # forget: rows of S
        if delta_off:
            S = S + kt[..., :, None] * vt[..., None, :]
            outs.append(scale * torch.einsum("bhij,bhi->bhj", S, qt))
            continue
        if kaczmarz:
            bt = beta[:, t] / ((kt * kt).sum(-1) + eps)
        else:
            bt = beta[:, t]
        p = torch.einsum("bhij,bhi->bhj", S, kt)           # prediction from the decayed state
        e = vt - p
        S = S + bt[..., None, None] * kt[..., :, None] * e[..., None, :]
        outs.append(scale * torch.einsum("bhij,bhi->bhj", S, qt))   # read after the write
    o = torch.stack(outs, dim=1) if T > 0 else torch.zeros((B, 0, H, Dv), dtype=torch.float64)
    return o, S


def oracle_bwd(q, k, v, g, beta, do, *, ds_final=None, s0=None, per_channel=False, kaczmarz=False,
               eps=0.0, scale=1.0, delta_off=False):
    """Returns dict(dq, dk, dv, dg, dbeta, ds0) as float64 numpy arrays
    (dbeta is d eta when kaczmarz, None with delta_off; ds0 is None when s0
    is None)."""
    tq, tk, tv, tg = _t(q), _t(k), _t(v), _t(g)
    tb = None if delta_off else _t(beta)
    ts0 = _t(s0)
    o, S = forward_torch(tq, tk, tv, tg, tb, ts0, per_channel=per_channel, kaczmarz=kaczmarz, eps=eps,
                         scale=scale, delta_off=delta_off)
    loss = (o * _t(do, False)).sum()
    if ds_final is not None:
        loss = loss + (S * _t(ds_final, False)).sum()
    loss.backward()

    def grad(x):
        return None if x is None else (x.grad.numpy() if x.grad is not None else np.zeros(tuple(x.shape)))

    return {"dq": grad(tq), "dk": grad(tk), "dv": grad(tv), "dg": grad(tg), "dbeta": grad(tb),
            "ds0": grad(ts0)}
