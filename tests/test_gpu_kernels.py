"""Kernel-level parity of the HIP kernels against the CPU oracle's pieces (GPU only).

Each kernel is called through its C-ABI entry point on seeded inputs with
ragged sizes (not multiples of the tile sizes), and compared element by
element with the oracle function it implements, evaluated in float64 on the
same (bf16-rounded where the kernel reads bf16) operands.
"""
import numpy as np
import pytest

import synth
from oracle import sampler as O
from tests.helpers import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flow_matching_tts_amd as F
    F.load()


def _bf(a):
    return synth.round_bf16(np.asarray(a, np.float32))


# ---------------------------------------------------------------- CFG + Euler

@pytest.mark.parametrize("nb,scales", [(1, ()), (2, (2.0,)), (3, (3.0, 1.5))])
def test_cfg_euler_matches_combine_and_update(nb, scales):
    import flow_matching_tts_amd as F
    rng = np.random.default_rng(nb)
    R, Tx, C = 5, 37, 100
    v = rng.standard_normal((nb, R, Tx, C)).astype(np.float32)
    x = rng.standard_normal((R, Tx, C)).astype(np.float32)
    mask = (rng.random((R, Tx)) > 0.3).astype(np.uint8)
    mask[2] = 0
    w = {1: [1.0], 2: [1 - scales[0], scales[0]] if nb == 2 else None,
         3: [1 - scales[0], scales[0] - scales[1], scales[1]] if nb == 3 else None}[nb]
    dt = 1.0 / 7
    xt = dev(x)
    F.cfg_euler(dev(v), w, dt, xt, mask=dev(mask))
    got = xt.cpu().numpy()
    want = x.astype(np.float64) + np.float32(dt) * O.guidance_combine(v.astype(np.float64), scales)
    valid = mask.astype(bool)
    np.testing.assert_allclose(got[valid], want[valid], rtol=2e-6, atol=2e-6)
    np.testing.assert_array_equal(got[~valid], x[~valid])


@pytest.mark.parametrize("S", [1, 4, 32])
def test_cfg_euler_analytic_field_reaches_x1(S):
    import flow_matching_tts_amd as F
    rng = np.random.default_rng(S)
    R, Tx, C = 3, 50, 32
    x0 = rng.standard_normal((R, Tx, C)).astype(np.float32)
    x1 = rng.standard_normal((R, Tx, C)).astype(np.float32)
    v = np.broadcast_to((x1 - x0)[None], (3, R, Tx, C)).copy()
    vt = dev(v)
    xt = dev(x0)
    s_t, s_s = 3.0, 1.5
    for k in range(S):
        dt = (k + 1) / S - k / S
        F.cfg_euler(vt, [1 - s_t, s_t - s_s, s_s], dt, xt)
    got = xt.cpu().numpy()
    # fp32: each step rounds; the error stays within a few ulp per step of |x| + |v| scale
    err = np.abs(got - x1).max()
    assert err < 8 * S * np.finfo(np.float32).eps * (np.abs(x0).max() + 4 * np.abs(x1 - x0).max()), err


# ---------------------------------------------------------------- GEMM

def _gemm_ref(A, W, bias, epi, gate=None, c0=None):
    acc = A.astype(np.float64) @ W.astype(np.float64).T + bias
    if epi in (0, 1):
        return acc
    if epi == 2:
        return O.gelu(acc)
    return c0.astype(np.float64) + gate.astype(np.float64) * acc


@pytest.mark.parametrize("M,N,K", [(300, 200, 136), (128, 128, 64), (1, 3, 8), (1000, 100, 1024), (257, 3072, 1024),
                                   (520, 600, 2048)])
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
@pytest.mark.parametrize("tile", [0, 1, 6, 10, 14, 15])
def test_gemm_bf16_epilogues(M, N, K, epi, tile):
    import flow_matching_tts_amd as F
    rng = np.random.default_rng(M * 7 + N + K + epi)
    A = _bf(rng.standard_normal((M, K)))
    W = _bf(rng.standard_normal((N, K)) * 0.05)
    bias = rng.standard_normal(N).astype(np.float32) * 0.1
    gate = rng.standard_normal(N).astype(np.float32)
    c0 = rng.standard_normal((M, N)).astype(np.float32)
    if epi in (1, 2):
        out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    else:
        out = dev(c0 if epi == 3 else np.zeros((M, N), np.float32))
    F.gemm_bf16(dev(A, torch.bfloat16), dev(W, torch.bfloat16), dev(bias), epilogue=epi, out=out,
                gate=dev(gate), tile=tile)
    got = out.float().cpu().numpy()
    want = _gemm_ref(A, W, bias, epi, gate, c0)
    if epi in (1, 2):      # bf16 output: within one bf16 rounding (2^-8 relative) of the fp64 value
        np.testing.assert_allclose(got, want, rtol=2 ** -8, atol=1e-5)
    else:
        np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-5 * np.sqrt(K))


@pytest.mark.parametrize("M,K,lda", [(300, 100, 100), (77, 80, 80), (64, 32, 36), (513, 512, 512)])
def test_gemm_fp32_a_operand_with_k_tail(M, K, lda):
    import flow_matching_tts_amd as F
    rng = np.random.default_rng(K + lda)
    N = 192
    A = rng.standard_normal((M, lda)).astype(np.float32)
    ldw = (K + 7) // 8 * 8
    W = np.zeros((N, ldw), np.float32)
    W[:, :K] = _bf(rng.standard_normal((N, K)) * 0.05)
    bias = rng.standard_normal(N).astype(np.float32)
    out = dev(np.zeros((M, N), np.float32))
    F.gemm_bf16(dev(A), dev(W, torch.bfloat16), dev(bias), epilogue=0, out=out, K=K)
    want = _bf(A[:, :K]).astype(np.float64) @ W[:, :K].astype(np.float64).T + bias
    np.testing.assert_allclose(out.cpu().numpy(), want, rtol=1e-5, atol=1e-5 * np.sqrt(K))


# ---------------------------------------------------------------- attention

def _attn_case(rows, T, H, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    qkv = _bf(rng.standard_normal((rows, T, 3 * H * 64)) * scale)
    return qkv


def _attn_call(qkv, H, kv_len, o, mask=None):
    """Split a [rows, T, 3d] q|k|v tensor into the kernel's q|k rows and per-head V^T."""
    import flow_matching_tts_amd as F
    rows, T, _ = qkv.shape
    d = H * 64
    Tp = (T + 63) // 64 * 64
    vt = np.full((rows, H, 64, Tp), np.nan, np.float32)        # padding must never be read as valid
    vt[..., :T] = qkv[..., 2 * d:].reshape(rows, T, H, 64).transpose(0, 2, 3, 1)
    F.attention_bf16(dev(qkv[..., :2 * d], torch.bfloat16), dev(vt, torch.bfloat16), dev(kv_len), o,
                     n_heads=H, key_mask=None if mask is None else dev(mask))
    return o


def _attn_ref(qkv, H, valid):
    rows, T, _ = qkv.shape
    d = H * 64
    q, k, v = (qkv[..., i * d:(i + 1) * d].reshape(rows, T, H, 64).transpose(0, 2, 1, 3).astype(np.float64)
               for i in range(3))
    o = O.masked_attention(q, k, v, valid)
    return o.transpose(0, 2, 1, 3).reshape(rows, T, d)


@pytest.mark.parametrize("rows,T,H", [(3, 200, 2), (2, 1, 1), (1, 128, 4), (2, 1000, 1), (4, 65, 3), (2, 513, 2), (3, 40, 2),
                                      (2, 64, 1), (5, 8, 16), (3, 17, 5), (2, 32, 3), (2, 33, 2)])
def test_attention_bf16_matches_oracle(rows, T, H):
    import flow_matching_tts_amd as F
    qkv = _attn_case(rows, T, H, rows * T + H, scale=1.5)
    rng = np.random.default_rng(T)
    kv_len = rng.integers(1, T + 1, rows).astype(np.int32)
    kv_len[0] = T
    mask = (rng.random((rows, T)) > 0.2).astype(np.uint8)
    mask[:, 0] = 1
    valid = (np.arange(T)[None] < kv_len[:, None]) & mask.astype(bool)
    o = torch.zeros((rows, T, H * 64), dtype=torch.bfloat16, device="cuda")
    _attn_call(qkv, H, kv_len, o, mask)
    got = o.float().cpu().numpy()
    want = _attn_ref(qkv, H, valid)
    # Per element: o = sum_k p_k v_k / sum_k p_k with each p_k rounded to bf16 before
    # the P.V product (relative error <= 2^-8) and o rounded to bf16 on store (<= 2^-8
    # of |o|), so |o - o_ref| <= 2^-8 (max_k |v_k| + |o_ref|), max over the valid keys
    # of that row, head and head dimension; 1.5x margin for the fp32 score and sum.
    d = H * 64
    v = np.abs(qkv[..., 2 * d:]).reshape(rows, T, d)
    vmax = np.where(valid[:, :, None], v, 0.0).max(axis=1, keepdims=True)     # [rows, 1, d]
    bound = 1.5 * 2.0 ** -8 * (vmax + np.abs(want)) + 1e-6
    err = np.abs(got - want)
    assert np.all(err <= bound), (err.max(), float((err / bound).max()))
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 6e-3, rel


@pytest.mark.parametrize("T", [150, 24])
def test_attention_bf16_empty_and_single_key_rows(T):
    import flow_matching_tts_amd as F
    rows, H = 3, 2
    qkv = _attn_case(rows, T, H, 5)
    kv_len = np.array([0, 1, T], np.int32)
    mask = np.ones((rows, T), np.uint8)
    key = min(77, T - 3)
    mask[2] = 0
    mask[2, key] = 1
    o = torch.full((rows, T, H * 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    _attn_call(qkv, H, kv_len, o, mask)
    got = o.float().cpu().numpy()
    assert np.all(got[0] == 0.0)                      # no valid key -> 0
    d = H * 64
    v = qkv[..., 2 * d:]
    np.testing.assert_array_equal(got[1], np.broadcast_to(v[1, 0], (T, d)))    # only key 0
    np.testing.assert_array_equal(got[2], np.broadcast_to(v[2, key], (T, d)))  # only that key


@pytest.mark.parametrize("T,n", [(130, 100), (30, 19)])
def test_attention_bf16_masked_keys_never_leak_non_finite_values(T, n):
    import flow_matching_tts_amd as F
    rows, H = 2, 1
    qkv = _attn_case(rows, T, H, 9)
    qkv[:, n:, 64:] = np.inf          # k and v of padded keys
    kv_len = np.array([n, n], np.int32)
    o = torch.zeros((rows, T, 64), dtype=torch.bfloat16, device="cuda")
    _attn_call(qkv, H, kv_len, o)
    got = o.float().cpu().numpy()
    assert np.all(np.isfinite(got[:, :n]))
    valid = np.arange(T)[None].repeat(rows, 0) < n
    want = _attn_ref(np.where(np.isfinite(qkv), qkv, 0), H, valid)
    assert np.abs(got[:, :n] - want[:, :n]).max() < 0.03 * 4


# ---------------------------------------------------------------- adaLN LayerNorm

@pytest.mark.parametrize("M,d", [(37, 1024), (5, 64), (300, 512), (3, 4096)])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_adaln_matches_oracle(M, d, out_bf16):
    import flow_matching_tts_amd as F
    rng = np.random.default_rng(M + d)
    h = (rng.standard_normal((M, d)) * 3 + 1.25).astype(np.float32)
    h[0] = 2.5                            # constant row -> output = shift
    shift = rng.standard_normal(d).astype(np.float32)
    scale = rng.standard_normal(d).astype(np.float32)
    y = torch.zeros((M, d), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    F.adaln(dev(h), dev(shift), dev(scale), y)
    got = y.float().cpu().numpy()
    want = O.modulate(O.layer_norm(h.astype(np.float64)), shift, scale)
    if out_bf16:
        np.testing.assert_allclose(got, want, rtol=2 ** -8, atol=1e-4)
    else:
        np.testing.assert_allclose(got, want, rtol=2e-5, atol=2e-5)
