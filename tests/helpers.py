"""Test helpers: config from a workload shape, device tensors, error metrics."""
from __future__ import annotations

import numpy as np

import synth


def config_for(s: "synth.CfmShape", **cap):
    import flow_matching_tts_amd as F
    return F.config_from_shape(s, **cap)


def dev(a, dtype=None):
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def rel_l2(got: np.ndarray, want: np.ndarray, valid=None) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if valid is not None:
        got = got[valid]
        want = want[valid]
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


# relative L2 bounds after all steps: fp32 path and bf16 path
TOL = {"f32": 1e-4, "bf16": 2e-2}


def run_sampler(s, W, I, *, guidance=None, n_steps=None, mask="auto", sampler=None, out_alias=False):
    """Runs the HIP sampler on workload shape ``s``; returns (out numpy, sampler)."""
    import torch
    import flow_matching_tts_amd as F
    if sampler is None:
        sampler = F.Sampler(config_for(s), W)
    m = I["mask"] if isinstance(mask, str) else mask
    x0 = dev(I["x0"])
    out = x0 if out_alias else None
    res = sampler.sample(x0, dev(I["cond"]), mask=dev(m), spk=dev(I["spk"]),
                         n_steps=s.n_steps if n_steps is None else n_steps,
                         guidance=s.guidance if guidance is None else guidance, out=out)
    torch.cuda.synchronize()
    return res.cpu().numpy(), sampler
