"""Writes the variant oracle's outputs for sampled requests of the full-size
block-variant workloads (cross-attention DiT, LocDiT tail with SwiGLU + RMSNorm +
RoPE).

Calls only ``oracle`` and the seeded generators in ``synth``. Requests never
interact, so each chosen request runs through the whole variant sampler on its
own (one process per request). Stored as float32 with the sha256 of the oracle
sources they came from (oracle/variants.py, then oracle/sampler.py, whose
functions it reuses): every frame of the LocDiT tail's four patch frames, every
4th frame of the cross-attention DiT. The chosen requests reach the
row-dependent paths of the packed three-branch layout: the shortest and the
longest request and the last request of the batch (its rows come last in every
branch). Run from the repository root:

    python tests/golden/make_variant_refs.py [workload ...]
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import variants as V  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
STRIDE = 4
ALL_FRAMES = 64
REQUESTS = {"cross_dit": [0, 6, 7], "locdit_swiglu": [0, 21, 63]}


def oracle_hash() -> str:
    h = hashlib.sha256()
    for f in ("variants.py", "sampler.py"):
        with open(os.path.join(ROOT, "oracle", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _one(name: str, r: int) -> np.ndarray:
    s = synth.workload(name)
    W, I = synth.make_weights(s), synth.make_inputs(s)
    return V.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance, requests=[r])[0]


def make(name: str) -> str:
    s = synth.workload(name)
    reqs = REQUESTS[name]
    t0 = time.time()
    with cf.ProcessPoolExecutor(max_workers=len(reqs)) as ex:
        outs = list(ex.map(_one, [name] * len(reqs), reqs))
    out = np.stack(outs)
    frames = np.arange(s.n_frames) if s.n_frames <= ALL_FRAMES else np.arange(0, s.n_frames, STRIDE)
    path = os.path.join(HERE, f"variant_{name}.npz")
    np.savez_compressed(path, out=out[:, frames, :].astype(np.float32), requests=np.array(reqs),
                        frames=frames, oracle_sha256=np.array(oracle_hash()))
    print(f"{name}: requests {reqs}, {time.time() - t0:.1f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    for n in sys.argv[1:] or list(REQUESTS):
        make(n)
