"""Helpers shared by the GPU tests: host<->device transfer of the generator's
arrays and the comparison rules.  No method arithmetic lives here."""
import numpy as np
import torch

import kvsynth


def to_dev(a, device="cuda"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def row_rel_err(out_dev_or_host, ref):
    """Per (b, h) row: ||o - ref||_inf / ||ref||_inf (ref fp64)."""
    o = out_dev_or_host
    if isinstance(o, torch.Tensor):
        o = to_host(o)
    of = kvsynth.as_float(o).astype(np.float64)
    num = np.abs(of - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def tol_for(dtype):
    return 1e-5 if dtype in ("f32", np.float32, torch.float32) else 2e-2
