"""Seeded synthetic inputs for the workloads in `configs`.

Serves both the GPU path and the CPU oracle (tests copy the generated
tensors to the host).  It holds no optimizer arithmetic: it draws normals,
scales them, takes absolute values, scales a seeded subset of entries, and
narrows to bf16 with torch's own conversion.

Every tensor is drawn from its own generator, seeded from (workload, tensor
index, field), so any one tensor can be regenerated alone.  The same seed
gives the same values on the same device type; CPU and CUDA generators give
different (equally distributed) values.
"""
from typing import Dict, List, Optional

import torch

from .configs import Workload

FIELD_MASTER, FIELD_GRAD, FIELD_M, FIELD_V, FIELD_OUTLIER = range(5)
_SALT = 0x4D5053


def seed_for(cfg: int, tensor_idx: int, field: int) -> int:
    """A 63-bit seed from (workload, tensor, field)."""
    x = (_SALT * 1_000_003 + cfg) * 1_000_003 + tensor_idx
    x = x * 16 + field
    return x % (1 << 63)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(n: int, std: float, seed: int, device) -> torch.Tensor:
    """n float32 samples of N(0, std^2)."""
    x = torch.randn(n, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x.mul_(std)


def tensor_inputs(w: Workload, i: int, device, cfg_key: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """master, exp_avg, exp_avg_sq, grad (and param_bf16 buffer) of tensor i."""
    cfg = w.cfg if cfg_key is None else cfg_key
    n = w.tensors[i][1]
    master = normal(n, w.master_std, seed_for(cfg, i, FIELD_MASTER), device)
    if w.m_std is None:
        m = torch.zeros(n, dtype=torch.float32, device=device)
    else:
        m = normal(n, w.m_std, seed_for(cfg, i, FIELD_M), device)
    if w.v_std is None:
        v = torch.zeros(n, dtype=torch.float32, device=device)
    else:
        v = normal(n, w.v_std, seed_for(cfg, i, FIELD_V), device).abs_()
    g = normal(n, w.grad_std, seed_for(cfg, i, FIELD_GRAD), device)
    if w.outlier_frac > 0.0:
        k = int(round(w.outlier_frac * n))
        idx = torch.randperm(n, generator=_gen(seed_for(cfg, i, FIELD_OUTLIER), device),
                             device=device)[:k]
        g[idx] *= w.outlier_scale
    if w.grad_bf16:
        g = g.to(torch.bfloat16)
    out = {"master": master, "exp_avg": m, "exp_avg_sq": v, "grad": g}
    if w.copy_bf16:
        out["param_bf16"] = torch.zeros(n, dtype=torch.bfloat16, device=device)
    return out


def workload_inputs(w: Workload, device, cfg_key: Optional[int] = None) -> Dict[str, List[torch.Tensor]]:
    """Lists (one entry per tensor) of every input of the workload."""
    cols: Dict[str, List[torch.Tensor]] = {"master": [], "exp_avg": [], "exp_avg_sq": [],
                                           "grad": [], "param_bf16": []}
    for i in range(w.n_tensors):
        t = tensor_inputs(w, i, device, cfg_key)
        for k in cols:
            cols[k].append(t.get(k))
    return cols


def to_numpy(t: torch.Tensor):
    """Host numpy view of a tensor; bf16 becomes its uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view("uint16")
    return t.cpu().numpy()
