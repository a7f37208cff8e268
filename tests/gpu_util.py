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
