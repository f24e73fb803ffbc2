"""Helpers that move a synthetic workload to the GPU and run the library on it."""
from __future__ import annotations

import numpy as np
import torch

from tenant_composite_lora_amd import tclora
from tenant_composite_lora_amd import workloads as W

DEV = "cuda:0"


def to_dev(a: np.ndarray, device=DEV) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def composites_to_dev(c: W.Composites, device=DEV):
    return (to_dev(c.group_tok_ptr.astype(np.int32), device),
            to_dev(c.group_pair_ptr.astype(np.int32), device),
            to_dev(c.pair_adapter.astype(np.int32), device),
            to_dev(c.pair_alpha.astype(np.float32), device))


def make_plan(c: W.Composites, device=DEV, max_tuples=None, buf=None) -> tclora.Plan:
    gtp, gpp, pa, pw = composites_to_dev(c, device)
    cap = c.n_tuples() if max_tuples is None else max_tuples
    return tclora.Plan(gtp, gpp, pa, pw, c.n_adapters, n_tokens=c.n_tokens, max_tuples=cap,
                       buf=buf)


def make_module(m: W.Module, device=DEV, k="module") -> tclora.Module:
    kk = m.k if isinstance(k, str) else k
    return tclora.Module(to_dev(m.A_t, device), to_dev(m.B_t, device), kk)


def run_fused(wl: W.Workload, y_dtype=torch.float32, k="module", plan=None, mods=None):
    """fused_apply over all modules; returns (ys as float64 numpy, plan, mods)."""
    plan = plan or make_plan(wl.composites)
    mods = mods or [make_module(m, k=k) for m in wl.modules]
    xs = [to_dev(x) for x in wl.x]
    ys = [to_dev(y).to(y_dtype) for y in wl.y_base]
    tclora.fused_apply(plan, mods, xs, ys)
    torch.cuda.synchronize()
    return [y.to(torch.float64).cpu().numpy() for y in ys], plan, mods


def run_split(wl: W.Workload, mi: int = 0, y_dtype=torch.float32, k="module"):
    """tcl_shrink then tcl_expand for module mi; returns (y, z) as float64."""
    plan = make_plan(wl.composites)
    mod = make_module(wl.modules[mi], k=k)
    x = to_dev(wl.x[mi])
    y = to_dev(wl.y_base[mi]).to(y_dtype)
    z = tclora.shrink(plan, mod, x)
    tclora.expand(plan, mod, z, y)
    torch.cuda.synchronize()
    return y.to(torch.float64).cpu().numpy(), z.cpu().numpy().astype(np.float64), plan


def rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |got - want| / max |want| (normwise, so near-zero entries do not
    dominate); 0 when both are empty or identically zero."""
    if want.size == 0:
        return 0.0
    den = float(np.max(np.abs(want)))
    num = float(np.max(np.abs(got - want)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
