"""The allocation-free attention entry point against the one that takes a
scratch buffer (GPU only). Both launch the same kernels; the no-alloc variant
keeps its key-validity tables in the library's built-in per-GPU buffer, which
keeps the previous call's contents, so two calls in a row (the second on a
smaller problem, with a different mask) must each match the scratch-buffer
entry point bit for bit."""
import numpy as np
import pytest

import synth
from tests.helpers import dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flow_matching_tts_amd as F
    F.load()


def _case(rows, T, H, seed):
    rng = np.random.default_rng(seed)
    d = H * 64
    qkv = synth.round_bf16(rng.standard_normal((rows, T, 3 * d)).astype(np.float32) * 1.5)
    Tp = (T + 63) // 64 * 64
    vt = np.zeros((rows, H, 64, Tp), np.float32)
    vt[..., :T] = qkv[..., 2 * d:].reshape(rows, T, H, 64).transpose(0, 2, 3, 1)
    kv_len = rng.integers(1, T + 1, rows).astype(np.int32)
    kv_len[0] = T
    mask = (rng.random((rows, T)) > 0.25).astype(np.uint8)
    return (dev(qkv[..., :2 * d], torch.bfloat16), dev(vt, torch.bfloat16), dev(kv_len), dev(mask))


def test_noalloc_attention_matches_scratch_entry_point_twice():
    import flow_matching_tts_amd as F
    for rows, T, H, seed in [(6, 700, 3, 1), (2, 130, 2, 2)]:   # second call smaller
        qk, vt, kv_len, mask = _case(rows, T, H, seed)
        ref = torch.full((rows, T, H * 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = torch.full_like(ref, float("nan"))
        F.attention_bf16(qk, vt, kv_len, ref, n_heads=H, key_mask=mask)
        F.attention_bf16_noalloc(qk, vt, kv_len, got, n_heads=H, key_mask=mask)
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (rows, T, H)


def test_noalloc_attention_rejects_problems_beyond_its_buffer():
    import flow_matching_tts_amd as F
    rows, T, H = 130, 64000, 1                # 130 * 64 000 key bytes > 8 MiB
    qk = torch.zeros((rows, T, 128), dtype=torch.bfloat16, device="cuda")
    vt = torch.zeros((rows, H, 64, T), dtype=torch.bfloat16, device="cuda")
    kv = torch.full((rows,), T, dtype=torch.int32, device="cuda")
    o = torch.zeros((rows, T, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.CfmError, match="CAPACITY"):
        F.attention_bf16_noalloc(qk, vt, kv, o, n_heads=H)
