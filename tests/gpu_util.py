"""Shared helpers for the GPU parity tests: error metrics against the fp64
oracle at the tolerances the method is held to (bf16 outputs: max-abs
2e-2 and relative L2 4e-3 on O; 1e-3 absolute on the fp32 LSE)."""

from __future__ import annotations

import numpy as np
import torch

O_MAX_ABS = 2e-2
O_REL_L2 = 4e-3
LSE_MAX_ABS = 1e-3

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def to_np(t):
    return t.detach().float().cpu().double().numpy()


def errors(o, lse, o_ref, lse_ref, mask=None):
    """Error metrics over the entries where mask (broadcast over D) is true."""
    o = to_np(o) if isinstance(o, torch.Tensor) else o
    lse = to_np(lse) if isinstance(lse, torch.Tensor) else lse
    if mask is not None:
        o, o_ref = o[mask], o_ref[mask]
    fin = np.isfinite(lse_ref)
    # rows with no visible key: O must be exactly 0 and LSE exactly -inf
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), "empty-row pattern differs"
    assert np.all(np.isfinite(o)), "non-finite output"
    d = np.abs(o - o_ref)
    nrm = np.linalg.norm(o_ref)
    rel = float(np.linalg.norm(o - o_ref) / nrm) if nrm > 0 else float(np.linalg.norm(o))
    lerr = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    return float(d.max()) if d.size else 0.0, rel, lerr


def assert_parity(o, lse, o_ref, lse_ref, what="", mask=None):
    err, rel, lerr = errors(o, lse, o_ref, lse_ref, mask)
    msg = f"{what}: max-abs {err:.3e} rel-L2 {rel:.3e} lse {lerr:.3e}"
    print(msg, flush=True)
    assert err <= O_MAX_ABS and rel <= O_REL_L2 and lerr <= LSE_MAX_ABS, msg
