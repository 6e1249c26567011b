"""The C ABI on the host (no GPU): exports, size queries, manifest, and argument
validation that must fail before anything is enqueued."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import synth
from tests.helpers import config_for

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import flow_matching_tts_amd as F
    try:
        return F.load()
    except ImportError as e:
        pytest.fail(f"library not built: {e}")


def header_functions():
    text = open(os.path.join(ROOT, "include", "cfm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cfm_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    import flow_matching_tts_amd as F
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(F.EXPORTS) == names


def test_status_strings(lib):
    for s in range(8):
        assert lib.cfm_status_string(s)
    assert lib.cfm_status_string(99) == b"unknown status"


VARIANT_WORKLOADS = ["locdit_swiglu", "cross_dit", "tiny_f32_variants"]


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER + VARIANT_WORKLOADS)
def test_sizes_and_manifest_cover_every_parameter(lib, name):
    import flow_matching_tts_amd as F
    s = synth.workload(name)
    cfg = config_for(s)
    wb, ws = F.weights_bytes(cfg), F.workspace_bytes(cfg)
    assert wb > 0 and ws > 0 and wb % 256 == 0
    man = F.weight_manifest(cfg)
    specs = dict(synth.weight_specs(s))
    covered = {}
    es = {0: 4, 1: 2}
    spans = []
    for e in man:
        shp = specs[e["name"]]
        rows, cols = (1, shp[0]) if len(shp) == 1 else shp
        assert e["row0"] + e["rows"] <= rows and e["col0"] + e["cols"] <= cols
        assert e["ld"] >= e["cols"] and e["offset"] % (2 if e["dtype"] == 1 else 4) == 0
        if e["dtype"] == 1 and len(shp) == 2:
            assert e["ld"] % 8 == 0
        covered[e["name"]] = covered.get(e["name"], 0) + e["rows"] * e["cols"]
        spans.append((e["offset"], e["offset"] + e["rows"] * e["ld"] * es[e["dtype"]]))
    for n, shp in specs.items():
        assert covered.get(n) == int(np.prod(shp)), n
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= wb


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_variants"])
def test_pack_weights_places_every_value(lib, name):
    import flow_matching_tts_amd as F
    s = synth.workload(name)
    cfg = config_for(s)
    W = synth.make_weights(s)
    buf = F.pack_weights(cfg, W)
    n_il = 0
    for e in F.weight_manifest(cfg):
        src = W[e["name"]].reshape(-1, W[e["name"]].shape[-1]) if W[e["name"]].ndim == 2 else W[e["name"]][None]
        blk = buf[e["offset"]:e["offset"] + e["rows"] * e["ld"] * 4].view(np.float32).reshape(e["rows"], e["ld"])
        want = src[e["row0"]:e["row0"] + e["rows"], e["col0"]:e["col0"] + e["cols"]]
        if e["interleave"]:
            # the fused gate-up FC1: groups of 16 gate rows alternate with the 16 up rows
            # of the same features (elements for the bias)
            n_il += 1
            assert e["interleave"] == 16 and e["name"].startswith("blocks.") and ".fc1." in e["name"]
            k, f = 16, (want.shape[0] if want.shape[0] > 1 else want.shape[1]) // 2
            flat = want if want.shape[0] > 1 else want.T
            perm = [(g // 2) * k + (g % 2) * f + i for g in range(2 * f // k) for i in range(k)]
            want = flat[perm] if want.shape[0] > 1 else flat[perm].T
        else:
            assert not (e["name"].startswith("blocks.") and ".fc1." in e["name"] and s.mlp == "swiglu")
        np.testing.assert_array_equal(blk[:, :e["cols"]], want)
    assert n_il == (2 * s.n_layers if s.mlp == "swiglu" else 0)


def test_variant_configs_are_validated(lib):
    ctx = C.c_void_p()
    fake = 1 << 20
    base = synth.workload("tiny_f32_variants")
    good = config_for(base)
    ws = lib.cfm_workspace_bytes(C.byref(good))
    assert ws > 0 and lib.cfm_create(C.byref(good), fake, fake, ws, C.byref(ctx)) == 0
    lib.cfm_destroy(ctx)
    for kw, code, text in ((dict(ffn_dim=104), 5, b"SwiGLU"), (dict(rope_base=0.0), 4, b"rope_base"),
                           (dict(rope_base=float("inf")), 4, b"rope_base"), (dict(n_prefix=0), 5, b"cross")):
        bad = config_for(base.replace(**kw))
        assert lib.cfm_create(C.byref(bad), fake, fake, 1 << 40, C.byref(ctx)) == code, kw
        assert text in lib.cfm_last_error_detail(), kw
    for field, value in (("norm", 2), ("mlp", 2), ("cond_mode", 3)):
        bad = config_for(base)
        setattr(bad, field, value)
        assert lib.cfm_create(C.byref(bad), fake, fake, 1 << 40, C.byref(ctx)) == 5, field
    assert lib.cfm_weights_bytes(C.byref(config_for(base.replace(rope=False, rope_base=-1.0)))) > 0   # base unused


def _cfg(**kw):
    s = synth.workload("mel_dit").replace(**kw) if kw else synth.workload("mel_dit")
    return config_for(s)


def test_create_validation(lib):
    ctx = C.c_void_p()
    cfg = _cfg()
    fake = 1 << 20   # never dereferenced: cfm_create only records pointers
    ws = lib.cfm_workspace_bytes(C.byref(cfg))
    assert lib.cfm_create(C.byref(cfg), None, fake, ws, C.byref(ctx)) == 1
    assert lib.cfm_create(C.byref(cfg), fake, fake, ws - 1, C.byref(ctx)) == 6
    assert lib.cfm_create(C.byref(cfg), fake + 16, fake, ws, C.byref(ctx)) == 2
    assert lib.cfm_create(None, fake, fake, ws, C.byref(ctx)) == 1
    bad = _cfg(n_heads=8)            # head_dim 128 on the bf16 path
    assert lib.cfm_create(C.byref(bad), fake, fake, ws, C.byref(ctx)) == 5
    assert b"head_dim" in lib.cfm_last_error_detail()
    bad = _cfg(n_branches=4)
    assert lib.cfm_create(C.byref(bad), fake, fake, ws, C.byref(ctx)) == 5
    bad = _cfg(latent_dim=98)
    assert lib.cfm_weights_bytes(C.byref(bad)) == 0
    assert lib.cfm_create(C.byref(cfg), fake, fake, ws, C.byref(ctx)) == 0 and ctx.value
    lib.cfm_destroy(ctx)
    lib.cfm_destroy(None)


def test_sample_validation_fails_before_any_device_work(lib):
    cfg = _cfg()
    fake = 1 << 20
    ws = lib.cfm_workspace_bytes(C.byref(cfg))
    ctx = C.c_void_p()
    assert lib.cfm_create(C.byref(cfg), fake, fake, ws, C.byref(ctx)) == 0
    g = (C.c_float * 1)(2.0)
    x, cond, out = 1 << 24, 1 << 26, 1 << 28
    R, T, S = 8, 1000, 32
    call = lambda **k: lib.cfm_sample(ctx, k.get("x0", x), k.get("cond", cond), None, None,
                                      k.get("R", R), k.get("T", T), k.get("S", S), k.get("g", g),
                                      k.get("out", out), None)
    assert call(R=-1) == 4
    assert call(S=-2) == 4
    assert call(R=9) == 3
    assert call(T=1001) == 3
    assert call(S=33) == 3
    assert call(g=None) == 1
    assert call(g=(C.c_float * 1)(math.inf)) == 4
    assert call(g=(C.c_float * 1)(math.nan)) == 4
    assert call(x0=None) == 1
    assert call(cond=None) == 1
    assert call(out=None) == 1
    assert call(x0=x + 4) == 2                          # misaligned
    assert call(out=x + 16) == 2                        # partial overlap with x0
    assert call(R=0) == 0 and call(R=0, x0=None) == 0   # empty batch: no-op
    assert call(T=0) == 0
    lib.cfm_destroy(ctx)


def test_single_kernel_entry_validation(lib):
    g = (C.c_float * 2)(0.5, 0.5)
    assert lib.cfm_cfg_euler(None, g, 2, C.c_float(0.1), None, 2, 3, 4, None, None) == 1
    assert lib.cfm_cfg_euler(1 << 20, g, 2, C.c_float(0.1), None, 2, 3, 6, 1 << 21, None) == 2
    assert lib.cfm_cfg_euler(1 << 20, g, 4, C.c_float(0.1), None, 2, 3, 4, 1 << 21, None) == 4
    assert lib.cfm_cfg_euler(None, g, 2, C.c_float(0.1), None, 0, 3, 4, None, None) == 0
    assert lib.cfm_gemm_bf16(1 << 20, 0, 12, 1 << 21, 16, None, 4, 4, 12, 0, None, 1 << 22, 4, 0, None) == 2
    assert lib.cfm_gemm_bf16(1 << 20, 0, 16, 1 << 21, 16, None, 4, 4, 16, 3, None, 1 << 22, 4, 0, None) == 1
    assert lib.cfm_gemm_bf16(1 << 20, 0, 16, 1 << 21, 16, None, 4, 4, 16, 9, None, 1 << 22, 4, 0, None) == 4
    assert lib.cfm_gemm_bf16(1 << 20, 1, 16, 1 << 21, 16, None, 4, 4, 16, 0, None, 1 << 22, 4, 2, None) == 4
    assert lib.cfm_attention_bf16(None, None, None, None, 2, 8, 1, None, 0, None, None) == 1
    assert lib.cfm_attention_bf16(None, None, None, None, 0, 8, 1, None, 0, None, None) == 0
    f = 1 << 20
    assert lib.cfm_attention_bf16(f, f, f, None, 2, 8, 1, f, 10, f, None) == 6
    assert lib.cfm_adaln(1 << 20, 1 << 21, 1 << 22, 4, 30, 0, 1 << 23, None) == 2


def test_config_launch_limits_rejected_at_create(lib):
    """Configs whose kernels could not be launched are refused when the context is
    created (and by the size queries), never half-way through a sampling call."""
    fake = 1 << 20
    ctx = C.c_void_p()
    small = dict(d_model=64, n_heads=1, ffn_dim=64)
    cases = [
        (dict(small, n_requests=40000, n_frames=1), b"attention grid"),   # 80000 branch rows
        (dict(n_steps=70000), b"max_steps"),                              # timestep-embedding grid
        (dict(n_frames=100000, n_requests=1), b"LDS"),                    # attention key tables
    ]
    for kw, why in cases:
        cfg = _cfg(**kw)
        assert lib.cfm_workspace_bytes(C.byref(cfg)) == 0, kw
        assert lib.cfm_create(C.byref(cfg), fake, fake, 1 << 40, C.byref(ctx)) == 5, kw
        assert why in lib.cfm_last_error_detail(), (kw, lib.cfm_last_error_detail())
    prefix = config_for(synth.workload("locdit_tail").replace(n_requests=17000, d_model=512, n_heads=8,
                                                               ffn_dim=1024))
    assert lib.cfm_create(C.byref(prefix), fake, fake, 1 << 40, C.byref(ctx)) == 5
    assert b"n_prefix" in lib.cfm_last_error_detail()
    ok = _cfg(n_frames=90000, n_requests=1)        # still inside the LDS budget
    assert lib.cfm_workspace_bytes(C.byref(ok)) > 0


def test_gemm_entry_rejects_misaligned_outputs(lib):
    a, w, c = 1 << 20, 1 << 21, 1 << 22
    ok = lambda **k: lib.cfm_gemm_bf16(k.get("A", a), 0, 16, w, 16, k.get("bias", None), 4, 4, 16,
                                       k.get("epi", 0), k.get("gate", None), k.get("C", c),
                                       k.get("ldc", 4), k.get("tile", 0), None)
    assert ok(ldc=6) == 2                 # ldc % 4 != 0: the vector epilogues need 16-byte rows
    assert ok(C=c + 8) == 2
    assert ok(bias=c + 4) == 2
    assert ok(epi=3, gate=c + 4) == 2
    assert ok(tile=2) == 4 and ok(tile=13) == 4 and ok(tile=16) == 4   # tiles the library does not have


def test_binding_rejects_bad_shapes_before_any_launch():
    import torch
    import flow_matching_tts_amd as F
    s = synth.workload("multicond_rf").replace(n_requests=2, n_frames=10, n_steps=3)
    cfg = config_for(s)
    R, Tx = 2, 10
    x0 = torch.zeros(R, Tx, s.latent_dim)
    cond = torch.zeros(R, Tx, s.cond_dim)
    spk = torch.zeros(R, s.spk_dim)
    good = dict(x0=x0, cond=cond, spk=spk, n_steps=3, guidance=(3.0, 1.5))

    def bad(**kw):
        args = dict(good, **kw)
        with pytest.raises(ValueError) as e:
            F.check_sample_args(cfg, args["x0"], args["cond"], args.get("mask"), args.get("spk"),
                                args.get("out"), args["n_steps"], args["guidance"])
        return str(e.value)

    assert "x0" in bad(x0=torch.zeros(R, Tx, s.latent_dim + 4))
    assert "cond" in bad(cond=torch.zeros(R, Tx - 1, s.cond_dim))
    assert "cond" in bad(cond=torch.zeros(R, Tx, s.cond_dim, dtype=torch.float64))
    assert "mask" in bad(mask=torch.ones(R, Tx + 1, dtype=torch.uint8))
    assert "mask" in bad(mask=torch.ones(R, Tx, dtype=torch.int32))
    assert "spk" in bad(spk=None)
    assert "spk" in bad(spk=torch.zeros(R, s.spk_dim - 4))
    assert "out" in bad(out=torch.zeros(R, Tx - 1, s.latent_dim))
    assert "guidance" in bad(guidance=(2.0,))
    assert "capacity" in bad(n_steps=4)
    assert "contiguous" in bad(x0=torch.zeros(R, s.latent_dim, Tx).transpose(1, 2))
    # every shape right: only the device is wrong (host tensors here)
    assert "CUDA" in bad()
    prefix = synth.workload("locdit_tail").replace(n_requests=2)
    pcfg = config_for(prefix)
    with pytest.raises(ValueError, match="cond"):
        F.check_sample_args(pcfg, torch.zeros(2, 4, 64), torch.zeros(2, 4, 64 + 4), n_steps=1,
                            guidance=(2.0,))
    with pytest.raises(ValueError, match="no speaker"):
        F.check_sample_args(config_for(synth.workload("mel_dit")), torch.zeros(1, 5, 100),
                            torch.zeros(1, 5, 512), spk=torch.zeros(1, 4), n_steps=1, guidance=(2.0,))


def test_single_kernel_wrappers_reject_bad_shapes_before_any_launch():
    import torch
    import flow_matching_tts_amd as F
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="x"):
        F.cfg_euler(torch.zeros(2, 3, 5, 8), [0.5, 0.5], 0.1, torch.zeros(3, 5, 4))
    with pytest.raises(ValueError, match="weights"):
        F.cfg_euler(torch.zeros(2, 3, 5, 8), [1.0], 0.1, torch.zeros(3, 5, 8))
    with pytest.raises(ValueError, match="mask"):
        F.cfg_euler(torch.zeros(2, 3, 5, 8), [0.5, 0.5], 0.1, torch.zeros(3, 5, 8),
                    mask=torch.ones(3, 4, dtype=torch.uint8))
    A, W = torch.zeros(10, 16, dtype=bf), torch.zeros(12, 16, dtype=bf)
    with pytest.raises(ValueError, match="columns"):
        F.gemm_bf16(A, W, epilogue=0, out=torch.zeros(10, 8))
    with pytest.raises(ValueError, match="out"):
        F.gemm_bf16(A, W, epilogue=0, out=torch.zeros(9, 12))
    with pytest.raises(ValueError, match="out"):
        F.gemm_bf16(A, W, epilogue=1, out=torch.zeros(10, 12))           # bf16 epilogue, fp32 out
    with pytest.raises(ValueError, match="bias"):
        F.gemm_bf16(A, W, torch.zeros(11), epilogue=0, out=torch.zeros(10, 12))
    with pytest.raises(ValueError, match="gate"):
        F.gemm_bf16(A, W, epilogue=3, out=torch.zeros(10, 12))
    with pytest.raises(ValueError, match="K"):
        F.gemm_bf16(A, W, epilogue=0, out=torch.zeros(10, 12), K=24)
    qk = torch.zeros(2, 70, 2 * 64, dtype=bf)
    vt = torch.zeros(2, 1, 64, 128, dtype=bf)
    kv = torch.zeros(2, dtype=torch.int32)
    o = torch.zeros(2, 70, 64, dtype=bf)
    with pytest.raises(ValueError, match="vt"):
        F.attention_bf16(qk, torch.zeros(2, 1, 64, 70, dtype=bf), kv, o, n_heads=1)
    with pytest.raises(ValueError, match="kv_len"):
        F.attention_bf16(qk, vt, torch.zeros(3, dtype=torch.int32), o, n_heads=1)
    with pytest.raises(ValueError, match="o"):
        F.attention_bf16(qk, vt, kv, torch.zeros(2, 69, 64, dtype=bf), n_heads=1)
    with pytest.raises(ValueError, match="qk"):
        F.attention_bf16(qk, vt, kv, o, n_heads=2)
    with pytest.raises(ValueError, match="CUDA"):
        F.attention_bf16(qk, vt, kv, o, n_heads=1)
    with pytest.raises(ValueError, match="shift"):
        F.adaln(torch.zeros(5, 64), torch.zeros(60), torch.zeros(64), torch.zeros(5, 64))
    with pytest.raises(ValueError, match="y"):
        F.adaln(torch.zeros(5, 64), torch.zeros(64), torch.zeros(64), torch.zeros(5, 32))
