"""Writes the CPU oracle's outputs for sampled requests of the full-size workloads.

Calls only ``oracle`` and the seeded generators in ``synth``. The GPU parity
tests at full size compare the HIP sampler against these stored values (the
oracle needs minutes to hours per full workload, too long for a test).

For each workload a few requests are run through the whole oracle sampler
(requests never interact, so a subset is exact). Their outputs are stored as
float32 together with the sha256 of the oracle source they came from: every
frame when a request has at most ``ALL_FRAMES`` frames (the LocDiT decode tail's
four patch frames), else every ``STRIDE``-th frame. The requests are chosen to
reach the row-dependent paths of the batched layout: the last request of a
batch, a packed row that starts past 16k tokens, speaker-branch rows of
requests other than the first. Run from the repository root:

    python tests/golden/make_oracle_refs.py [workload ...]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import sampler as O  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
STRIDE = 4
ALL_FRAMES = 64


def oracle_hash() -> str:
    with open(os.path.join(ROOT, "oracle", "sampler.py"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def chosen_requests(s, inputs) -> list:
    if s.name == "locdit_tail":
        return [0, 21, 37, 63]
    if s.name == "varlen_masked":
        # shortest, longest, and request 26, whose packed unconditional row
        # starts past token 16384 (its conditional row past 40k)
        L = inputs["lengths"]
        return sorted({int(np.argmin(L)), int(np.argmax(L)), 7, 26})
    if s.name == "mel_dit":
        return [0, 5, 7]
    if s.name == "multicond_rf":
        return [0, 6, 11]
    return list(range(s.n_requests))


def make(name: str) -> str:
    s = synth.workload(name)
    W = synth.make_weights(s)
    I = synth.make_inputs(s)
    reqs = chosen_requests(s, I)
    t0 = time.time()
    out = O.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance,
                   requests=reqs, workers=min(len(reqs), O.host_cores()))
    frames = np.arange(s.n_frames) if s.n_frames <= ALL_FRAMES else np.arange(0, s.n_frames, STRIDE)
    path = os.path.join(HERE, f"oracle_{name}.npz")
    np.savez_compressed(path, out=out[:, frames, :].astype(np.float32), requests=np.array(reqs),
                        frames=frames, oracle_sha256=np.array(oracle_hash()))
    print(f"{name}: requests {reqs}, {time.time() - t0:.1f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    names = sys.argv[1:] or ["tiny_f32", "locdit_tail", "varlen_masked", "mel_dit", "multicond_rf"]
    for n in names:
        make(n)
