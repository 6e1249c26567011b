"""ctypes binding of libcfm_mi355x.so (the C ABI in include/cfm.h).

Argument marshalling only: every step of the sampler runs in the library's
HIP kernels. torch supplies device memory and the current stream. There is no
fallback: if the library is missing or was not built, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Mapping, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcfm_mi355x.so")

CFM_F32, CFM_BF16 = 0, 1
CFM_COND_CHANNEL, CFM_COND_PREFIX, CFM_COND_CROSS = 0, 1, 2
NORMS = {"layer": 0, "rms": 1}
MLPS = {"gelu": 0, "swiglu": 1}
STATUS = {0: "CFM_OK", 1: "CFM_E_NULL", 2: "CFM_E_SHAPE", 3: "CFM_E_CAPACITY", 4: "CFM_E_VALUE",
          5: "CFM_E_UNSUPPORTED", 6: "CFM_E_WORKSPACE", 7: "CFM_E_HIP"}
KERNEL_CLASSES = {"gemm_qkv": 0, "gemm_proj": 1, "gemm_fc1": 2, "gemm_fc2": 3, "attention": 4,
                  "adaln": 5, "cfg_euler": 6, "gemm_in": 7, "gemm_out": 8, "hoisted": 9,
                  "xattn": 10, "gemm_xattn": 11}

EXPORTS = ["cfm_weights_bytes", "cfm_workspace_bytes", "cfm_weight_manifest", "cfm_create",
           "cfm_sample", "cfm_sample_ex", "cfm_destroy", "cfm_status_string", "cfm_last_error_detail",
           "cfm_profile_enable", "cfm_profile_read", "cfm_profile_disable", "cfm_cfg_euler",
           "cfm_gemm_bf16", "cfm_attention_bf16", "cfm_attention_bf16_noalloc", "cfm_adaln"]


class cfm_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "d_model", "n_heads", "ffn_dim", "latent_dim", "cond_dim", "cond_mode",
        "n_prefix", "spk_dim", "t_freq_dim", "n_branches", "dtype", "max_requests",
        "max_frames", "max_steps", "norm", "mlp", "rope")] + [("rope_base", C.c_float)]


class cfm_tensor_desc(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("row0", C.c_int64), ("col0", C.c_int64),
                ("rows", C.c_int64), ("cols", C.c_int64), ("ld", C.c_int64),
                ("offset", C.c_int64), ("dtype", C.c_int32), ("interleave", C.c_int32)]


SCHEDULES = {"uniform": 0, "quadratic": 1, "trailing": 2, "native": 3}
SOLVERS = {"euler": 0, "midpoint": 1}
GUIDANCE_MODES = {"full": 0, "interval": 1, "adaptive": 2}


class cfm_sample_options(C.Structure):
    _fields_ = [("schedule", C.c_int32), ("native_steps", C.c_int32), ("solver", C.c_int32),
                ("guidance_mode", C.c_int32), ("interval_start", C.c_float), ("interval_end", C.c_float),
                ("adaptive_threshold", C.c_float), ("adaptive_warmup", C.c_int32),
                ("adaptive_patience", C.c_int32), ("reserved", C.c_int32), ("guided_evals", C.c_void_p),
                ("cache", C.c_int32), ("cache_front", C.c_int32), ("cache_back", C.c_int32),
                ("cache_warmup", C.c_int32), ("cache_max_consecutive", C.c_int32),
                ("cache_max_cached", C.c_int32), ("cache_threshold", C.c_float), ("cache_budget", C.c_float),
                ("cache_force", C.c_void_p), ("cache_hits", C.c_void_p)]


CACHE_DEFAULTS = dict(front=1, back=1, warmup=3, max_consecutive=2, max_cached=-1, threshold=0.05, budget=0.12,
                      force=())


class CfmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def load() -> C.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m flow_matching_tts_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp, i32, f32p = C.c_void_p, C.c_int, C.POINTER(C.c_float)
    cfgp = C.POINTER(cfm_config)
    lib.cfm_weights_bytes.argtypes = [cfgp]
    lib.cfm_weights_bytes.restype = C.c_size_t
    lib.cfm_workspace_bytes.argtypes = [cfgp]
    lib.cfm_workspace_bytes.restype = C.c_size_t
    lib.cfm_weight_manifest.argtypes = [cfgp, C.POINTER(cfm_tensor_desc), i32]
    lib.cfm_weight_manifest.restype = i32
    lib.cfm_create.argtypes = [cfgp, vp, vp, C.c_size_t, C.POINTER(vp)]
    lib.cfm_create.restype = i32
    lib.cfm_sample.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32p, vp, vp]
    lib.cfm_sample.restype = i32
    lib.cfm_sample_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32p, C.POINTER(cfm_sample_options), vp, vp]
    lib.cfm_sample_ex.restype = i32
    lib.cfm_destroy.argtypes = [vp]
    lib.cfm_destroy.restype = None
    lib.cfm_status_string.argtypes = [i32]
    lib.cfm_status_string.restype = C.c_char_p
    lib.cfm_last_error_detail.argtypes = []
    lib.cfm_last_error_detail.restype = C.c_char_p
    lib.cfm_profile_enable.argtypes = [vp, i32, i32]
    lib.cfm_profile_enable.restype = i32
    lib.cfm_profile_read.argtypes = [vp, C.POINTER(C.c_double), C.POINTER(i32), C.POINTER(i32)]
    lib.cfm_profile_read.restype = i32
    lib.cfm_profile_disable.argtypes = [vp]
    lib.cfm_profile_disable.restype = i32
    lib.cfm_cfg_euler.argtypes = [vp, f32p, i32, C.c_float, vp, i32, i32, i32, vp, vp]
    lib.cfm_cfg_euler.restype = i32
    lib.cfm_gemm_bf16.argtypes = [vp, i32, i32, vp, i32, vp, i32, i32, i32, i32, vp, vp, i32, i32, vp]
    lib.cfm_gemm_bf16.restype = i32
    lib.cfm_attention_bf16.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, C.c_size_t, vp, vp]
    lib.cfm_attention_bf16.restype = i32
    lib.cfm_attention_bf16_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp]
    lib.cfm_attention_bf16_noalloc.restype = i32
    lib.cfm_adaln.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
    lib.cfm_adaln.restype = i32
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        detail = load().cfm_last_error_detail().decode()
        raise CfmError(status, detail)


def make_config(*, n_layers, d_model, n_heads, ffn_dim, latent_dim, cond_dim, cond_mode,
                n_prefix, spk_dim, n_branches, dtype, max_requests, max_frames, max_steps,
                t_freq_dim=256, norm="layer", mlp="gelu", rope=False, rope_base=10000.0) -> cfm_config:
    cm = {"channel": CFM_COND_CHANNEL, "prefix": CFM_COND_PREFIX, "cross": CFM_COND_CROSS}.get(cond_mode, cond_mode)
    dt = {"f32": CFM_F32, "bf16": CFM_BF16}.get(dtype, dtype)
    return cfm_config(n_layers, d_model, n_heads, ffn_dim, latent_dim, cond_dim, cm, n_prefix,
                      spk_dim, t_freq_dim, n_branches, dt, max_requests, max_frames, max_steps,
                      NORMS.get(norm, norm), MLPS.get(mlp, mlp), int(bool(rope)), float(rope_base))


def config_from_shape(s, *, max_requests: Optional[int] = None, max_frames: Optional[int] = None,
                      max_steps: Optional[int] = None) -> cfm_config:
    """cfm_config of a workload description: any object with the model attributes
    (n_layers, d_model, n_heads, ffn_dim, latent_dim, cond_dim, cond_mode, n_prefix,
    spk_dim, n_branches, dtype, t_freq_dim; optionally norm, mlp, rope, rope_base) and
    its n_requests / n_frames / n_steps, which give the capacity unless overridden."""
    return make_config(
        n_layers=s.n_layers, d_model=s.d_model, n_heads=s.n_heads, ffn_dim=s.ffn_dim,
        latent_dim=s.latent_dim, cond_dim=s.cond_dim, cond_mode=s.cond_mode, n_prefix=s.n_prefix,
        spk_dim=s.spk_dim, n_branches=s.n_branches, dtype=s.dtype, t_freq_dim=s.t_freq_dim,
        norm=getattr(s, "norm", "layer"), mlp=getattr(s, "mlp", "gelu"), rope=getattr(s, "rope", False),
        rope_base=getattr(s, "rope_base", 10000.0),
        max_requests=s.n_requests if max_requests is None else max_requests,
        max_frames=s.n_frames if max_frames is None else max_frames,
        max_steps=s.n_steps if max_steps is None else max_steps)


def weights_bytes(cfg: cfm_config) -> int:
    return int(load().cfm_weights_bytes(C.byref(cfg)))


def workspace_bytes(cfg: cfm_config) -> int:
    return int(load().cfm_workspace_bytes(C.byref(cfg)))


def weight_manifest(cfg: cfm_config):
    lib = load()
    n = lib.cfm_weight_manifest(C.byref(cfg), None, 0)
    if n < 0:
        check(-n)
    arr = (cfm_tensor_desc * n)()
    check(0 if lib.cfm_weight_manifest(C.byref(cfg), arr, n) == n else 4)
    return [dict(name=a.name.decode(), row0=a.row0, col0=a.col0, rows=a.rows, cols=a.cols,
                 ld=a.ld, offset=a.offset, dtype=a.dtype, interleave=a.interleave) for a in arr]


def interleave_rows(blk: np.ndarray, k: int) -> np.ndarray:
    """Row order of a slot with interleave k: groups of k rows of the first half
    alternate with the matching groups of the second half."""
    if k <= 0:
        return blk
    half = blk.shape[0] // 2
    a, b = blk[:half].reshape(-1, k, blk.shape[1]), blk[half:].reshape(-1, k, blk.shape[1])
    return np.stack([a, b], axis=1).reshape(blk.shape)


def pack_weights(cfg: cfm_config, weights: Mapping[str, np.ndarray]) -> np.ndarray:
    """Host byte image of the flat weight buffer, laid out as the manifest says."""
    import torch
    buf = np.zeros(weights_bytes(cfg), dtype=np.uint8)
    for e in weight_manifest(cfg):
        src = np.asarray(weights[e["name"]], dtype=np.float32)
        if src.ndim == 1:
            src = src[None, :]
        blk = src[e["row0"]:e["row0"] + e["rows"], e["col0"]:e["col0"] + e["cols"]]
        if blk.shape != (e["rows"], e["cols"]):
            raise ValueError(f"{e['name']}: shape {src.shape} does not cover slot {e}")
        if e["interleave"]:     # a bias slot is one row: interleave its elements
            blk = interleave_rows(blk.T, e["interleave"]).T if blk.shape[0] == 1 else interleave_rows(blk, e["interleave"])
        pad = np.zeros((e["rows"], e["ld"]), dtype=np.float32)
        pad[:, :e["cols"]] = blk
        if e["dtype"] == CFM_BF16:
            raw = torch.from_numpy(pad).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
        else:
            raw = pad.view(np.uint8)
        raw = raw.reshape(-1)
        buf[e["offset"]:e["offset"] + raw.size] = raw
    return buf


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _shape(t):
    return tuple(int(v) for v in t.shape)


def _need(name, t, shape, dtype, optional=False):
    """Shape, dtype and layout of one tensor argument (ValueError before any launch).

    ``shape`` entries that are None are not checked. Device placement is checked
    separately, after every shape, so that a wrong shape is reported as such."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if len(t.shape) != len(shape) or any(w is not None and g != w for g, w in zip(_shape(t), shape)):
        raise ValueError(f"{name} has shape {_shape(t)}, expected {tuple('*' if w is None else w for w in shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    devs = {n: t.device for n, t in tensors.items() if t is not None}
    for n, d in devs.items():
        if d.type != "cuda":
            raise ValueError(f"{n} must be a CUDA tensor (got {d})")
    if len(set(devs.values())) > 1:
        raise ValueError(f"tensors on different devices: {devs}")


def check_sample_args(cfg: cfm_config, x0, cond, mask=None, spk=None, out=None, n_steps: int = 0,
                      guidance: Sequence[float] = ()):
    """Validates every argument of Sampler.sample against the context's config.

    cfm_sample receives bare pointers and only R, Tx and S: a tensor smaller than
    those imply would be read or written past its end on the device, so every
    shape is checked here first."""
    import torch
    if len(x0.shape) != 3:
        raise ValueError(f"x0 must be [R, Tx, latent_dim], got shape {_shape(x0)}")
    R, Tx = int(x0.shape[0]), int(x0.shape[1])
    _need("x0", x0, (R, Tx, cfg.latent_dim), torch.float32)
    if cfg.cond_mode == CFM_COND_PREFIX:
        _need("cond", cond, (R, cfg.n_prefix, cfg.latent_dim), torch.float32)
    elif cfg.cond_mode == CFM_COND_CROSS:
        _need("cond", cond, (R, cfg.n_prefix, cfg.cond_dim), torch.float32)
    else:
        _need("cond", cond, (R, Tx, cfg.cond_dim), torch.float32)
    _need("mask", mask, (R, Tx), torch.uint8, optional=True)
    if cfg.spk_dim > 0:
        _need("spk", spk, (R, cfg.spk_dim), torch.float32)
    elif spk is not None:
        raise ValueError("spk given, but the config has no speaker path (spk_dim == 0)")
    _need("out", out, (R, Tx, cfg.latent_dim), torch.float32, optional=True)
    if len(guidance) != cfg.n_branches - 1:
        raise ValueError(f"{cfg.n_branches} branches take {cfg.n_branches - 1} guidance scales, "
                         f"got {len(guidance)}")
    if int(n_steps) < 0:
        raise ValueError("n_steps must be >= 0")
    if R > cfg.max_requests or Tx > cfg.max_frames or int(n_steps) > cfg.max_steps:
        raise ValueError(f"R={R} Tx={Tx} S={n_steps} above the capacity "
                         f"{cfg.max_requests}/{cfg.max_frames}/{cfg.max_steps}")
    _on_device(x0=x0, cond=cond, mask=mask, spk=spk, out=out)


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Sampler:
    """Owns the device weight buffer and workspace of one context (torch tensors)."""

    def __init__(self, cfg: cfm_config, weights: Mapping[str, np.ndarray], device: str = "cuda"):
        import torch
        lib = load()
        self.cfg = cfg
        host = pack_weights(cfg, weights)
        self.weights = torch.from_numpy(host).to(device)
        self.workspace = torch.empty(max(workspace_bytes(cfg), 256), dtype=torch.uint8, device=device)
        ctx = C.c_void_p()
        check(lib.cfm_create(C.byref(cfg), self.weights.data_ptr(), self.workspace.data_ptr(),
                             self.workspace.numel(), C.byref(ctx)))
        self._ctx = ctx

    @property
    def ctx(self):
        return self._ctx

    def close(self):
        if getattr(self, "_ctx", None) is not None and self._ctx.value:
            load().cfm_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sample(self, x0, cond, *, mask=None, spk=None, n_steps: int, guidance: Sequence[float] = (),
               out=None, stream=None, schedule: str = "uniform", native_steps: Optional[int] = None,
               solver: str = "euler", guidance_mode: str = "full", interval=(0.0, 1.0),
               adaptive=(0.015, 4, 2), guided_evals=None, cache=None, cache_hits=None):
        """out[R, Tx, C] (fp32, device) after n_steps solver steps; out may be x0 itself.

        schedule / native_steps / solver / guidance_mode / interval / adaptive
        (threshold, warmup, patience) select the sampler-level options of
        cfm_sample_ex; guided_evals, an int32 [R] device tensor, receives per request
        the number of evaluations that ran its unconditional rows. cache (a dict over
        CACHE_DEFAULTS' keys; None = off) turns on the block-residual cache, and
        cache_hits, an int32 [1] device tensor, receives its number of hits."""
        import torch
        guidance = tuple(guidance)
        evals = int(n_steps) * (2 if solver == "midpoint" else 1)
        check_sample_args(self.cfg, x0, cond, mask, spk, out, evals, guidance)
        if x0.device != self.weights.device:
            raise ValueError(f"inputs on {x0.device}, sampler on {self.weights.device}")
        R, Tx = int(x0.shape[0]), int(x0.shape[1])
        if guided_evals is not None:
            _need("guided_evals", guided_evals, (R,), torch.int32)
            _on_device(x0=x0, guided_evals=guided_evals)
        for name, val, table in (("schedule", schedule, SCHEDULES), ("solver", solver, SOLVERS),
                                 ("guidance_mode", guidance_mode, GUIDANCE_MODES)):
            if val not in table:
                raise ValueError(f"{name} {val!r} not one of {sorted(table)}")
        if cache_hits is not None:
            _need("cache_hits", cache_hits, (1,), torch.int32)
            _on_device(x0=x0, cache_hits=cache_hits)
        if out is None:
            out = torch.empty_like(x0)
        g = (C.c_float * max(1, len(guidance)))(*[float(v) for v in guidance])
        opt = cfm_sample_options(SCHEDULES[schedule], int(native_steps or 0), SOLVERS[solver],
                                 GUIDANCE_MODES[guidance_mode], float(interval[0]), float(interval[1]),
                                 float(adaptive[0]), int(adaptive[1]), int(adaptive[2]), 0, _ptr(guided_evals))
        force = None
        if cache is not None:
            unknown = set(cache) - set(CACHE_DEFAULTS)
            if unknown:
                raise ValueError(f"unknown cache options {sorted(unknown)}")
            cc = dict(CACHE_DEFAULTS, **cache)
            force = (C.c_uint8 * max(1, evals))(*[1 if v else 0 for v in list(cc["force"])[:evals]])
            opt.cache, opt.cache_front, opt.cache_back = 1, int(cc["front"]), int(cc["back"])
            opt.cache_warmup, opt.cache_max_consecutive = int(cc["warmup"]), int(cc["max_consecutive"])
            opt.cache_max_cached = int(cc["max_cached"])
            opt.cache_threshold, opt.cache_budget = float(cc["threshold"]), float(cc["budget"])
            opt.cache_force = C.cast(force, C.c_void_p)
        opt.cache_hits = _ptr(cache_hits)
        check(load().cfm_sample_ex(self._ctx, _ptr(x0), _ptr(cond), _ptr(spk), _ptr(mask), R, Tx,
                                   int(n_steps), g, C.byref(opt), _ptr(out), _stream(stream)))
        return out

    def profile_enable(self, kernel_class: str, capacity: int):
        check(load().cfm_profile_enable(self._ctx, KERNEL_CLASSES[kernel_class], int(capacity)))

    def profile_read(self):
        ms, n, dropped = C.c_double(), C.c_int(), C.c_int()
        check(load().cfm_profile_read(self._ctx, C.byref(ms), C.byref(n), C.byref(dropped)))
        return ms.value, n.value, dropped.value

    def profile_disable(self):
        check(load().cfm_profile_disable(self._ctx))


# ---------------------------------------------------------------- single kernels

def cfg_euler(v, w: Sequence[float], dt: float, x, mask=None, stream=None):
    """x[r, t] += dt * sum_b w[b] v[b, r, t] on valid frames; v [nb, R, Tx, C], x [R, Tx, C] fp32."""
    import torch
    if len(v.shape) != 4:
        raise ValueError(f"v must be [nb, R, Tx, C], got shape {_shape(v)}")
    nb, R, Tx, Cc = _shape(v)
    _need("v", v, (nb, R, Tx, Cc), torch.float32)
    _need("x", x, (R, Tx, Cc), torch.float32)
    _need("mask", mask, (R, Tx), torch.uint8, optional=True)
    if len(w) != nb:
        raise ValueError(f"{nb} branches take {nb} weights, got {len(w)}")
    _on_device(v=v, x=x, mask=mask)
    ww = (C.c_float * nb)(*[float(a) for a in w])
    check(load().cfm_cfg_euler(_ptr(v), ww, nb, float(dt), _ptr(mask), R, Tx, Cc, _ptr(x), _stream(stream)))
    return x


def gemm_bf16(A, W, bias=None, *, epilogue: int, out, gate=None, K: Optional[int] = None, tile: int = 0,
              stream=None):
    """out = epilogue(A[:, :K] W[:, :K]^T + bias); A bf16 or fp32 [M, lda], W bf16 [N, ldw]."""
    import torch
    if len(A.shape) != 2 or len(W.shape) != 2 or len(out.shape) != 2:
        raise ValueError("A, W and out must be 2-D")
    M, lda = _shape(A)
    N, ldw = _shape(W)
    K = lda if K is None else int(K)
    if not 0 <= K <= lda:
        raise ValueError(f"K={K} outside [0, lda={lda}]")
    if A.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"A must be bf16 or fp32, got {A.dtype}")
    _need("A", A, (M, lda), A.dtype)
    _need("W", W, (N, ldw), torch.bfloat16)
    _need("bias", bias, (N,), torch.float32, optional=True)
    out_dtype = torch.bfloat16 if epilogue in (1, 2, 4) else torch.float32
    _need("out", out, (M, None), out_dtype)
    ncols = N // 2 if epilogue == 4 else N
    if epilogue == 4 and N % 32:
        raise ValueError(f"the SwiGLU epilogue needs N % 32 == 0, got N={N}")
    if int(out.shape[1]) < ncols:
        raise ValueError(f"out has {int(out.shape[1])} columns, needs at least {ncols}")
    if epilogue == 3:
        _need("gate", gate, (N,), torch.float32)
    a_f32 = 1 if A.dtype == torch.float32 else 0
    _on_device(A=A, W=W, bias=bias, out=out, gate=gate)
    check(load().cfm_gemm_bf16(_ptr(A), a_f32, lda, _ptr(W), ldw, _ptr(bias), M, N, K, int(epilogue),
                               _ptr(gate), _ptr(out), int(out.shape[1]), int(tile), _stream(stream)))
    return out


def _check_attention(qk, vt, kv_len, o, H, key_mask):
    import torch
    if len(qk.shape) != 3:
        raise ValueError(f"qk must be [rows, T, 2*H*64], got shape {_shape(qk)}")
    rows, T = int(qk.shape[0]), int(qk.shape[1])
    Tp = (T + 63) // 64 * 64
    _need("qk", qk, (rows, T, 2 * H * 64), torch.bfloat16)
    _need("vt", vt, (rows, H, 64, Tp), torch.bfloat16)
    _need("kv_len", kv_len, (rows,), torch.int32)
    _need("key_mask", key_mask, (rows, T), torch.uint8, optional=True)
    _need("o", o, (rows, T, H * 64), torch.bfloat16)
    _on_device(qk=qk, vt=vt, kv_len=kv_len, key_mask=key_mask, o=o)
    return rows, T, Tp


def attention_bf16(qk, vt, kv_len, o, *, n_heads: int, key_mask=None, stream=None):
    """qk bf16 [rows, T, 2*H*64], vt bf16 [rows, H, 64, Tp] (Tp = T rounded up to 64),
    kv_len int32 [rows], key_mask uint8 [rows, T] or None, o bf16 [rows, T, H*64]."""
    import torch
    H = int(n_heads)
    rows, T, Tp = _check_attention(qk, vt, kv_len, o, H, key_mask)
    scratch = torch.empty(rows * 4 + rows * Tp + rows * (Tp // 64) + 64, dtype=torch.uint8, device=qk.device)
    check(load().cfm_attention_bf16(_ptr(qk), _ptr(vt), _ptr(kv_len), _ptr(key_mask), rows, T,
                                    H, _ptr(scratch), scratch.numel(), _ptr(o), _stream(stream)))
    return o


def attention_bf16_noalloc(qk, vt, kv_len, o, *, n_heads: int, key_mask=None, stream=None):
    """attention_bf16 through the entry point that allocates nothing (its key tables
    live in the library's own per-GPU buffer)."""
    H = int(n_heads)
    rows, T, _ = _check_attention(qk, vt, kv_len, o, H, key_mask)
    check(load().cfm_attention_bf16_noalloc(_ptr(qk), _ptr(vt), _ptr(kv_len), _ptr(key_mask), rows, T,
                                            H, _ptr(o), _stream(stream)))
    return o


def adaln(h, shift, scale, y, stream=None):
    """y = LN(h) * (1 + scale) + shift; h fp32 [M, d], shift / scale fp32 [d], y fp32 or bf16 [M, d]."""
    import torch
    if len(h.shape) != 2:
        raise ValueError(f"h must be [M, d], got shape {_shape(h)}")
    M, d = _shape(h)
    _need("h", h, (M, d), torch.float32)
    _need("shift", shift, (d,), torch.float32)
    _need("scale", scale, (d,), torch.float32)
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"y must be fp32 or bf16, got {y.dtype}")
    _need("y", y, (M, d), y.dtype)
    _on_device(h=h, shift=shift, scale=scale, y=y)
    check(load().cfm_adaln(_ptr(h), _ptr(shift), _ptr(scale), M, d, 1 if y.dtype == torch.bfloat16 else 0,
                           _ptr(y), _stream(stream)))
    return y
