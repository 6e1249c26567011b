"""Seeded synthetic workloads for batched conditional-flow-matching sampling.

This module is the only code shared by the CPU oracle and the HIP path's tests
and benchmark. It holds shapes and random draws only: none of the sampler's
arithmetic (no embedding, projection, attention, guidance or Euler step).

Sources of the shapes (VoiceHub "Diffusion and flow TTS optimization" page and
the vLLM-Omni TTS blog, section "CFM/LocDiT decode-tail batching"):
  * the velocity estimator is a DiT evaluated over a CFG-expanded batch of many
    requests at once (the blog's decode-tail batching; VoiceHub's packed CFG
    lanes in its "Semantic-preserving and approximate changes" table);
  * variable-length TTS batches are padded to a bucket and keep a frame mask
    (VoiceHub, "Static shapes and CUDA graphs").
The five workloads below carry the sizes of the five benchmark cases this
library is measured on.

Draw recipe (documented so that any reader can regenerate the exact inputs):
  * generator: numpy.random.Generator(PCG64(seed)); weights use seed
    1000 + workload index, inputs use seed 2000 + workload index;
  * weights: every tensor of ``weight_specs`` in list order, drawn as
    float32 standard normals times 0.02; for bf16 workloads each value is then
    rounded to the nearest bfloat16 (ties to even) and kept as float32;
  * inputs, in this order: x0 [R, Tx, C] ~ N(0,1) float32; cond [R, Tc, Cc]
    ~ N(0,1) float32; spk [R, spk_dim] ~ N(0,1) float32 (only when spk_dim>0);
    frame lengths ``rng.integers(lo, hi + 1, R)`` (only for variable-length
    workloads). Padded frames of x0 and cond are filled with N(0,1) draws too,
    so that a leak through the mask is visible.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "CfmShape", "WORKLOADS", "WORKLOAD_ORDER", "workload", "weight_specs",
    "make_weights", "make_inputs", "round_bf16",
    "lengths_to_mask",
]


@dataclass(frozen=True)
class CfmShape:
    """Sizes of one sampling workload.

    ``cond_mode`` is "channel" (a per-frame condition of ``cond_dim`` channels
    concatenated after the latent channels of every generated frame), "prefix"
    (``n_prefix`` condition frames of the latent width placed before the
    generated frames in the sequence) or "cross" (``n_prefix`` context tokens of
    ``cond_dim`` channels that every block reads through cross-attention).

    Block variants: ``norm`` "layer" or "rms"; ``mlp`` "gelu" (FC1 of ffn_dim
    rows) or "swiglu" (one fused gate-up FC1 of 2 ffn_dim rows, gate rows first);
    ``rope`` rotates the self-attention queries and keys by token position.
    """
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    ffn_dim: int
    latent_dim: int
    cond_dim: int
    cond_mode: str
    n_prefix: int
    spk_dim: int
    n_branches: int
    dtype: str                      # "f32" or "bf16"
    n_requests: int
    n_frames: int                   # generated (patch) frames per request, padded length
    n_steps: int
    guidance: Tuple[float, ...]     # n_branches - 1 scales
    varlen: Optional[Tuple[int, int]] = None   # inclusive [lo, hi] frame lengths
    t_freq_dim: int = 256
    weight_std: float = 0.02
    index: int = -1                 # seed offset (position in WORKLOAD_ORDER for the five main cases)
    norm: str = "layer"             # "layer" | "rms"
    mlp: str = "gelu"               # "gelu" | "swiglu"
    rope: bool = False
    rope_base: float = 10000.0

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    @property
    def seq_len(self) -> int:
        """Tokens per row seen by attention (prefix frames + generated frames)."""
        return self.n_frames + (self.n_prefix if self.cond_mode == "prefix" else 0)

    @property
    def cond_frames(self) -> int:
        return self.n_prefix if self.cond_mode in ("prefix", "cross") else self.n_frames

    @property
    def in_dim(self) -> int:
        """Input width of the input projection."""
        return self.latent_dim + (self.cond_dim if self.cond_mode == "channel" else 0)

    @property
    def n_rows(self) -> int:
        return self.n_requests * self.n_branches

    def replace(self, **kw) -> "CfmShape":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, CfmShape] = {
    # Tiny fp32 sampler: 2 layers, d=64, 4 heads, FFN 256, latent 16, 32 frames,
    # 1 request with CFG, per-frame condition 32x16, 4 uniform Euler steps, s=2.
    "tiny_f32": CfmShape(
        name="tiny_f32", n_layers=2, d_model=64, n_heads=4, ffn_dim=256,
        latent_dim=16, cond_dim=16, cond_mode="channel", n_prefix=0, spk_dim=0,
        n_branches=2, dtype="f32", n_requests=1, n_frames=32, n_steps=4,
        guidance=(2.0,), index=0),
    # LocDiT-style patch decode tail: 64 requests x CFG, 4 prefix-condition
    # frames + 4 patch frames of latent 64, d=1024, 4 layers, FFN 4096, 10 steps.
    "locdit_tail": CfmShape(
        name="locdit_tail", n_layers=4, d_model=1024, n_heads=16, ffn_dim=4096,
        latent_dim=64, cond_dim=64, cond_mode="prefix", n_prefix=4, spk_dim=0,
        n_branches=2, dtype="bf16", n_requests=64, n_frames=4, n_steps=10,
        guidance=(2.0,), index=1),
    # Mel DiT generator: 22 layers, d=1024, FFN 2048, 100-channel mel latent,
    # 1000 frames, 8 requests x CFG, text condition 1000x512, 32 steps.
    "mel_dit": CfmShape(
        name="mel_dit", n_layers=22, d_model=1024, n_heads=16, ffn_dim=2048,
        latent_dim=100, cond_dim=512, cond_mode="channel", n_prefix=0, spk_dim=0,
        n_branches=2, dtype="bf16", n_requests=8, n_frames=1000, n_steps=32,
        guidance=(2.0,), index=2),
    # Variable-length masked batch: 32 requests, lengths U[200,1500] padded to
    # 1500, d=512, 8 layers, 8 heads, FFN 2048, latent 80, s=2.5, 16 steps.
    "varlen_masked": CfmShape(
        name="varlen_masked", n_layers=8, d_model=512, n_heads=8, ffn_dim=2048,
        latent_dim=80, cond_dim=80, cond_mode="channel", n_prefix=0, spk_dim=0,
        n_branches=2, dtype="bf16", n_requests=32, n_frames=1500, n_steps=16,
        guidance=(2.5,), varlen=(200, 1500), index=3),
    # Multi-condition rectified flow: 3 branches (uncond, text, text+speaker),
    # 16 requests, 750 frames of latent 32, d=1024, 12 layers, FFN 4096,
    # speaker vector 256-d, s_t=3.0, s_s=1.5, 40 steps.
    "multicond_rf": CfmShape(
        name="multicond_rf", n_layers=12, d_model=1024, n_heads=16, ffn_dim=4096,
        latent_dim=32, cond_dim=512, cond_mode="channel", n_prefix=0, spk_dim=256,
        n_branches=3, dtype="bf16", n_requests=16, n_frames=750, n_steps=40,
        guidance=(3.0, 1.5), index=4),
    # Block variants (parity and measurement cases beside the five main ones).
    # LocDiT decode tail with RMSNorm, a fused gate-up SwiGLU MLP and rotary
    # positions over the prefix + patch tokens: 64 requests x CFG, 4 + 4 tokens.
    "locdit_swiglu": CfmShape(
        name="locdit_swiglu", n_layers=4, d_model=1024, n_heads=16, ffn_dim=2048,
        latent_dim=64, cond_dim=64, cond_mode="prefix", n_prefix=4, spk_dim=0,
        n_branches=2, dtype="bf16", n_requests=64, n_frames=4, n_steps=10,
        guidance=(2.0,), index=5, norm="rms", mlp="swiglu", rope=True),
    # Cross-attention DiT: 200 context tokens of 512 channels read by every block
    # through cross-attention (keys/values computed once per call), rotary
    # self-attention over 600 frames of latent 64, 8 requests x 3 branches
    # (uncond, text, text+speaker), 12 layers, d=1024, FFN 4096, 16 steps.
    "cross_dit": CfmShape(
        name="cross_dit", n_layers=12, d_model=1024, n_heads=16, ffn_dim=4096,
        latent_dim=64, cond_dim=512, cond_mode="cross", n_prefix=200, spk_dim=128,
        n_branches=3, dtype="bf16", n_requests=8, n_frames=600, n_steps=16,
        guidance=(2.0, 1.5), varlen=(300, 600), index=6, rope=True),
    # Tiny fp32 case with every variant on: cross-attention to 12 context tokens,
    # RMSNorm, SwiGLU, rotary positions; 2 requests with CFG, 24 frames.
    "tiny_f32_variants": CfmShape(
        name="tiny_f32_variants", n_layers=2, d_model=64, n_heads=4, ffn_dim=96,
        latent_dim=16, cond_dim=20, cond_mode="cross", n_prefix=12, spk_dim=0,
        n_branches=2, dtype="f32", n_requests=2, n_frames=24, n_steps=4,
        guidance=(2.0,), index=7, norm="rms", mlp="swiglu", rope=True),
}
WORKLOAD_ORDER: List[str] = ["tiny_f32", "locdit_tail", "mel_dit", "varlen_masked", "multicond_rf"]


def workload(name: str) -> CfmShape:
    return WORKLOADS[name]


def weight_specs(s: CfmShape) -> List[Tuple[str, Tuple[int, ...]]]:
    """Named parameter tensors, PyTorch Linear convention ([out, in], bias [out]).

    The list order is the draw order.
    """
    d, f = s.d_model, s.ffn_dim
    specs: List[Tuple[str, Tuple[int, ...]]] = [
        ("t_embed.fc1.weight", (d, s.t_freq_dim)), ("t_embed.fc1.bias", (d,)),
        ("t_embed.fc2.weight", (d, d)), ("t_embed.fc2.bias", (d,)),
    ]
    if s.spk_dim > 0:
        specs += [("spk_proj.weight", (d, s.spk_dim)), ("spk_proj.bias", (d,))]
    specs += [("in_proj.weight", (d, s.in_dim)), ("in_proj.bias", (d,))]
    f1 = 2 * f if s.mlp == "swiglu" else f      # fused gate-up: gate rows, then up rows
    for l in range(s.n_layers):
        p = f"blocks.{l}."
        specs += [
            (p + "ada.weight", (6 * d, d)), (p + "ada.bias", (6 * d,)),
            (p + "qkv.weight", (3 * d, d)), (p + "qkv.bias", (3 * d,)),
            (p + "proj.weight", (d, d)), (p + "proj.bias", (d,)),
            (p + "fc1.weight", (f1, d)), (p + "fc1.bias", (f1,)),
            (p + "fc2.weight", (d, f)), (p + "fc2.bias", (d,)),
        ]
        if s.cond_mode == "cross":
            specs += [
                (p + "xattn.q.weight", (d, d)), (p + "xattn.q.bias", (d,)),
                (p + "xattn.kv.weight", (2 * d, s.cond_dim)), (p + "xattn.kv.bias", (2 * d,)),
                (p + "xattn.out.weight", (d, d)), (p + "xattn.out.bias", (d,)),
            ]
    specs += [
        ("final.ada.weight", (2 * d, d)), ("final.ada.bias", (2 * d,)),
        ("final.out.weight", (s.latent_dim, d)), ("final.out.bias", (s.latent_dim,)),
    ]
    return specs


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(a)
    out[nan] = a[nan]
    return out


def make_weights(s: CfmShape, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every parameter of ``s`` (see the module docstring for the recipe)."""
    if seed is None:
        seed = 1000 + max(s.index, 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    std = np.float32(s.weight_std)
    out: Dict[str, np.ndarray] = {}
    for name, shape in weight_specs(s):
        w = rng.standard_normal(shape, dtype=np.float32) * std
        if s.dtype == "bf16":
            w = round_bf16(w)
        out[name] = w
    return out


def lengths_to_mask(lengths: np.ndarray, n_frames: int) -> np.ndarray:
    """Prefix frame mask [R, n_frames] uint8 (1 = valid) from per-request lengths."""
    lengths = np.asarray(lengths)
    return (np.arange(n_frames)[None, :] < lengths[:, None]).astype(np.uint8)


def make_inputs(s: CfmShape, seed: Optional[int] = None) -> Dict[str, Optional[np.ndarray]]:
    """Draw x0, cond, spk and the frame mask of ``s`` (recipe in the module docstring)."""
    if seed is None:
        seed = 2000 + max(s.index, 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    R, Tx, C = s.n_requests, s.n_frames, s.latent_dim
    x0 = rng.standard_normal((R, Tx, C), dtype=np.float32)
    cond = rng.standard_normal((R, s.cond_frames, s.cond_dim), dtype=np.float32)
    spk = rng.standard_normal((R, s.spk_dim), dtype=np.float32) if s.spk_dim > 0 else None
    if s.varlen is not None:
        lo, hi = s.varlen
        lengths = rng.integers(lo, hi + 1, R)
        mask = lengths_to_mask(lengths, Tx)
    else:
        lengths = np.full(R, Tx, dtype=np.int64)
        mask = None
    return {"x0": x0, "cond": cond, "spk": spk, "mask": mask, "lengths": lengths}
