"""Move a seeded workload onto the GPU in the library's layout (torch as plumbing).

The cache becomes one packed [rows, d_c + d_r] tensor of rows [c^KV ; k^R], the
layout the bf16 decode kernel streams; c_kv and k_r are its two column views.
"""

from __future__ import annotations

import numpy as np

from . import workloads as W


def _tensor(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def packed_rows(w: W.Workload) -> np.ndarray:
    """Host array [rows, d_c + d_r] in the storage type: each row is [c_kv ; k_r]."""
    return np.concatenate([w.c_kv, w.k_r], axis=1)


def to_device(w: W.Workload, device="cuda") -> dict:
    import torch
    cache = _tensor(packed_rows(w), w.dtype, device)
    return dict(
        cache=cache,
        c_kv=cache[:, :w.d_c],
        k_r=cache[:, w.d_c:],
        offsets=torch.from_numpy(w.offsets.astype(np.int64)).to(device),
        q_c=_tensor(w.q_c, w.dtype, device),
        q_r=_tensor(w.q_r, w.dtype, device),
        w_uk=_tensor(w.w_uk, w.dtype, device),
        w_uv=_tensor(w.w_uv, w.dtype, device),
    )


def to_numpy_f64(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> fp64 numpy array, exactly."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)
