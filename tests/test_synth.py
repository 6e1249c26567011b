"""The seeded input generators: determinism, bf16 rounding and shapes."""
import numpy as np
import torch

import synth


def test_weights_and_inputs_are_deterministic():
    s = synth.workload("tiny_f32")
    a, b = synth.make_weights(s), synth.make_weights(s)
    assert list(a) == [n for n, _ in synth.weight_specs(s)]
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    ia, ib = synth.make_inputs(s), synth.make_inputs(s)
    np.testing.assert_array_equal(ia["x0"], ib["x0"])
    np.testing.assert_array_equal(ia["cond"], ib["cond"])
    assert not np.array_equal(synth.make_inputs(s, 7)["x0"], ia["x0"])


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -2.5, 1.00390625, 1.01171875], np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.round_bf16(a), want)


def test_bf16_workload_weights_are_bf16_exact():
    s = synth.workload("locdit_tail").replace(n_layers=1, d_model=64, n_heads=1, ffn_dim=64)
    w = synth.make_weights(s)
    for v in w.values():
        assert np.all((v.view(np.uint32) & 0xFFFF) == 0)


def test_workload_shapes():
    s = synth.workload("varlen_masked")
    inp = synth.make_inputs(s)
    assert inp["x0"].shape == (32, 1500, 80) and inp["cond"].shape == (32, 1500, 80)
    L = inp["lengths"]
    assert L.min() >= 200 and L.max() <= 1500
    np.testing.assert_array_equal(inp["mask"].sum(1), L)
    p = synth.workload("locdit_tail")
    assert p.seq_len == 8 and p.in_dim == 64 and synth.make_inputs(p)["cond"].shape == (64, 4, 64)
    m = synth.workload("multicond_rf")
    assert m.n_rows == 48 and synth.make_inputs(m)["spk"].shape == (16, 256)
    sizes = {n: shp for n, shp in synth.weight_specs(m)}
    assert sizes["spk_proj.weight"] == (1024, 256) and sizes["in_proj.weight"] == (1024, 544)
