"""Block variants of cfm_sample on the GPU against the CPU oracle (oracle/variants.py):
RMSNorm, the fused gate-up SwiGLU MLP, rotary self-attention positions and
cross-attention to context keys/values computed once per call.

Each case runs the HIP library through the C ABI and compares with the oracle at
the sampler's tolerance (relative L2 over valid frames 1e-4 fp32, 2e-2 bf16, on
the output and on the displacement out - x0); padded frames must come back as x0
bit for bit. The cases cover the fp32 path with every variant on, the prefix
(LocDiT) layout with the short attention kernel, the packed variable-length
three-branch speaker batch with cross-attention on the long attention kernel,
cross-attention with one key tile, few queries against many context keys, a
channel-condition batch with SwiGLU + RoPE through the large GEMM tiles, and
unguided evaluations (the conditional rows alone read their branch's context).
The SwiGLU GEMM epilogue is also checked element by element on every tile. At full
size (the cross-attention DiT and the LocDiT tail with every variant) the sampler is
compared on sampled requests with stored outputs of the variant oracle
(tests/golden/make_variant_refs.py).
"""
import hashlib
import os

import numpy as np
import pytest

import synth
from oracle import variants as V
from tests.helpers import TOL, dev, rel_l2, run_sampler

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flow_matching_tts_amd as F
    F.load()


def _valid(I, s):
    return np.ones((s.n_requests, s.n_frames), bool) if I["mask"] is None else I["mask"].astype(bool)


def _check(s, I, got, want):
    valid = _valid(I, s)
    err = rel_l2(got, want, valid)
    disp = rel_l2(got - I["x0"], want - I["x0"], valid)
    print(f"{s.name}: rel-L2 {err:.3e}, displacement {disp:.3e} (bound {TOL[s.dtype]:g})")
    assert err <= TOL[s.dtype] and disp <= TOL[s.dtype], (err, disp)
    np.testing.assert_array_equal(got[~valid], I["x0"][~valid])


def _tiny(**kw):
    return synth.workload("tiny_f32_variants").replace(**kw)


CASES = {
    "f32_all_variants": lambda: _tiny(),
    "f32_prefix_rms_swiglu_rope": lambda: _tiny(cond_mode="prefix", n_prefix=5, cond_dim=16),
    "f32_channel_rope": lambda: _tiny(cond_mode="channel", n_prefix=0, norm="layer", mlp="gelu", n_requests=3,
                                      varlen=(9, 24)),
    "locdit_swiglu": lambda: synth.workload("locdit_swiglu").replace(n_requests=9, n_steps=3, n_layers=2),
    "cross_dit_packed_long": lambda: synth.workload("cross_dit").replace(n_layers=2, n_requests=3, n_frames=150,
                                                                         n_prefix=70, n_steps=3, varlen=(40, 150)),
    "cross_dit_one_tile": lambda: synth.workload("cross_dit").replace(n_layers=2, n_requests=2, n_frames=48,
                                                                      n_prefix=40, n_steps=3, varlen=None),
    "cross_dit_few_queries": lambda: synth.workload("cross_dit").replace(n_layers=1, n_requests=2, n_frames=40,
                                                                         n_prefix=100, n_steps=2, varlen=None),
    "mel_swiglu_rope": lambda: synth.workload("mel_dit").replace(n_layers=2, n_frames=300, n_requests=2, n_steps=3,
                                                                 mlp="swiglu", rope=True, index=8),
}


@pytest.mark.parametrize("case", list(CASES))
def test_variant_sampler_matches_oracle(case):
    s = CASES[case]()
    W, I = synth.make_weights(s), synth.make_inputs(s)
    got, _ = run_sampler(s, W, I)
    want = V.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance)
    _check(s, I, got, want)


def test_cross_attention_unguided_evaluations_read_the_conditioned_context():
    """An empty guidance interval makes every evaluation unguided: the conditional
    rows run alone, so the result is the one-branch sampler of the fully
    conditioned branch (whose context rows sit after the other branches')."""
    s = synth.workload("cross_dit").replace(n_layers=2, n_requests=3, n_frames=96, n_prefix=70, n_steps=3,
                                            varlen=(40, 96))
    W, I = synth.make_weights(s), synth.make_inputs(s)
    import flow_matching_tts_amd as F
    from tests.helpers import config_for
    smp = F.Sampler(config_for(s), W)
    out = smp.sample(dev(I["x0"]), dev(I["cond"]), mask=dev(I["mask"]), spk=dev(I["spk"]), n_steps=s.n_steps,
                     guidance=s.guidance, guidance_mode="interval", interval=(0.9, 0.95))
    got = out.cpu().numpy()
    s1 = s.replace(n_branches=1, guidance=())
    want = V.sample(W, s1, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, ())
    _check(s, I, got, want)


@pytest.mark.parametrize("tile", [0, 1, 6, 10, 14, 15])
@pytest.mark.parametrize("M,N,K", [(333, 512, 256), (64, 192, 96), (1000, 1024, 512)])
def test_gemm_swiglu_epilogue(M, N, K, tile):
    import flow_matching_tts_amd as F
    rng = np.random.default_rng(M + N + K)
    bf = lambda a: synth.round_bf16(np.asarray(a, np.float32))
    A = bf(rng.standard_normal((M, K)))
    W = bf(rng.standard_normal((N, K)) * 0.05)
    bias = rng.standard_normal(N).astype(np.float32) * 0.1
    out = torch.zeros((M, N // 2), dtype=torch.bfloat16, device="cuda")
    F.gemm_bf16(dev(A, torch.bfloat16), dev(W, torch.bfloat16), dev(bias), epilogue=4, out=out, tile=tile)
    z = A.astype(np.float64) @ W.astype(np.float64).T + bias            # interleaved columns
    blocks = z.reshape(M, N // 32, 2, 16)
    g, u = blocks[:, :, 0, :].reshape(M, N // 2), blocks[:, :, 1, :].reshape(M, N // 2)
    want = g / (1.0 + np.exp(-g)) * u
    np.testing.assert_allclose(out.float().cpu().numpy(), want, rtol=2 ** -8, atol=1e-5)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _variant_golden(name):
    path = os.path.join(GOLDEN, f"variant_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    z = np.load(path)
    h = hashlib.sha256()
    for f in ("variants.py", "sampler.py"):
        with open(os.path.join(os.path.dirname(GOLDEN), "..", "oracle", f), "rb") as fh:
            h.update(fh.read())
    assert str(z["oracle_sha256"]) == h.hexdigest(), "stale oracle reference"
    return z


@pytest.mark.parametrize("name", ["locdit_swiglu", "cross_dit"])
def test_full_variant_workload_matches_stored_oracle(name):
    """Full-size bench configuration: stored requests (shortest, longest, last of the
    packed three-branch batch for the cross-attention DiT) at the tolerance, each on its
    own too; a second call gives the same bits; padded frames come back as x0."""
    s = synth.workload(name)
    z = _variant_golden(name)
    W, I = synth.make_weights(s), synth.make_inputs(s)
    got, smp = run_sampler(s, W, I)
    again, _ = run_sampler(s, W, I, sampler=smp)
    np.testing.assert_array_equal(again, got)
    reqs, frames = z["requests"], z["frames"]
    g = got[reqs][:, frames, :]
    valid = _valid(I, s)[reqs][:, frames]
    x0 = I["x0"][reqs][:, frames, :]
    err = rel_l2(g, z["out"], valid)
    disp = rel_l2(g - x0, z["out"] - x0, valid)
    print(f"{name}: full size, requests {list(reqs)}, {len(frames)} frames each: rel-L2 {err:.3e} "
          f"(displacement {disp:.3e})")
    assert err <= TOL[s.dtype] and disp <= TOL[s.dtype], (err, disp)
    for i, r in enumerate(reqs):
        assert rel_l2(g[i:i + 1], z["out"][i:i + 1], valid[i:i + 1]) <= TOL[s.dtype], int(r)
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got[~_valid(I, s)], I["x0"][~_valid(I, s)])
