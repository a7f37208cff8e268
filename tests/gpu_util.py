"""Helpers shared by the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

DEV = torch.device("cuda:0")
TOL = {"f32": 1e-5, "bf16": 2e-3}   # relative L2 bars: fp32 inputs / bf16 inputs


def to_dev(x: dict, dtype: str) -> dict:
    """numpy float32 arrays -> device tensors; q, k, v in the workload dtype."""
    out = {}
    for key, val in x.items():
        if val is None:
            out[key] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(val)).to(DEV)
        if key in ("q", "k", "v") and dtype == "bf16":
            t = t.to(torch.bfloat16)
        out[key] = t
    return out


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def head_parity(gpu_o, ref_o, gpu_s, ref_s, *, tol, o_round=0.0):
    """Compare outputs [B,T,H,Dv] and final states [B,H,Dk,Dv] head by head.

    Returns the aggregate relative L2 of o and of S over every head, the
    largest per-(b,h) relative L2 of each, and the largest element-wise ratio
    |gpu - ref| / (8 tol rms(ref of that head) + o_round |ref|) of each (the
    element bound holds when that ratio is <= 1).  ``o_round`` is the relative
    half-ulp of the output format (2^-8 for bf16 outputs, 0 for fp32), so that
    rounding a correct value to the output dtype stays inside the bound.
    Heads are copied one at a time so that host memory stays small.
    """
    B, T, H = ref_o.shape[:3]
    acc = {"o": [0.0, 0.0], "s": [0.0, 0.0]}
    worst = {"o": 0.0, "s": 0.0}
    elem = {"o": 0.0, "s": 0.0}
    worst_at = {"o": None, "s": None}
    for b in range(B):
        for h in range(H):
            for key, g, r, rnd in (("o", gpu_o[b, :, h], ref_o[b, :, h], o_round),
                                   ("s", gpu_s[b, h], ref_s[b, h], 0.0)):
                g = np.asarray(g, dtype=np.float64)
                r = np.asarray(r, dtype=np.float64)
                if r.size == 0:
                    continue
                d = np.abs(g - r)
                d2, r2 = float(np.sum(d * d)), float(np.sum(r * r))
                acc[key][0] += d2
                acc[key][1] += r2
                rel_h = (d2 / r2) ** 0.5 if r2 > 0 else d2 ** 0.5
                if not np.isfinite(rel_h) or rel_h > worst[key]:
                    worst[key] = rel_h if np.isfinite(rel_h) else float("inf")
                    worst_at[key] = (b, h)
                rms = (r2 / r.size) ** 0.5
                ratio = float(np.max(d / (8.0 * tol * rms + rnd * np.abs(r) + 1e-300)))
                elem[key] = max(elem[key], ratio if np.isfinite(ratio) else float("inf"))
    agg = {key: ((v[0] / v[1]) ** 0.5 if v[1] > 0 else v[0] ** 0.5) for key, v in acc.items()}
    return {"agg_o": agg["o"], "agg_s": agg["s"], "head_o": worst["o"], "head_s": worst["s"],
            "head_o_at": worst_at["o"], "head_s_at": worst_at["s"], "elem_o": elem["o"], "elem_s": elem["s"]}
