"""Python binding of the gfx950 GPT training-step library (``libgpt_mi355x.so``).

The functions here only marshal arguments to the C ABI declared in
``include/gpt.h``; every step of the computation runs in the library's HIP
kernels.  PyTorch is used by ``Session`` for device memory and the stream.
Importing this package without the built library raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgpt_mi355x.so")

GPT_OK, GPT_EINVAL, GPT_ENULL, GPT_ETOKEN, GPT_EHIP, GPT_ENONFINITE, GPT_ESPACE, GPT_EALIGN = 0, -1, -2, -3, -4, -5, -6, -7
GPT_FP32, GPT_BF16, GPT_FP8 = 0, 1, 2

EXPORTED = ["gpt_param_layout", "gpt_workspace_bytes", "gpt_create", "gpt_step", "gpt_step_accum", "gpt_step_micro",
            "gpt_optim_state_bytes", "gpt_optim_init", "gpt_optim_step", "gpt_optim_master",
            "gpt_kv_cache_bytes", "gpt_prefill", "gpt_decode", "gpt_rope_table", "gpt_overlap_enable",
            "gpt_rope_epilogue_enable", "gpt_destroy",
            "gpt_debug_tensor", "gpt_gemm", "gpt_gemm_noalloc", "gpt_fp8_quantize", "gpt_gemm_fp8", "gpt_profile_enable",
            "gpt_profile_sites", "gpt_profile_get", "gpt_strerror", "gpt_last_error"]


class gpt_config(ctypes.Structure):
    _fields_ = [
        ("depth", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_head", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("mlp_hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("seq_len", ctypes.c_int32), ("batch", ctypes.c_int32), ("window", ctypes.c_int32),
        ("window_pattern", ctypes.c_char * 8), ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("precision", ctypes.c_int32), ("weights", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p), ("n_kv_head", ctypes.c_int32),
    ]


class gpt_optim_params(ctypes.Structure):
    _fields_ = [
        ("matrix_lr", ctypes.c_float), ("momentum", ctypes.c_float), ("nesterov", ctypes.c_int32),
        ("ns_steps", ctypes.c_int32), ("embedding_lr", ctypes.c_float), ("unembedding_lr", ctypes.c_float),
        ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float), ("grad_clip", ctypes.c_float), ("step", ctypes.c_int32),
    ]


def optim_params(**kw) -> gpt_optim_params:
    """Optimizer parameters; every field must be given (no defaults are
    implied by the library)."""
    names = [f[0] for f in gpt_optim_params._fields_]
    missing = [n for n in names if n not in kw]
    extra = [n for n in kw if n not in names]
    if missing or extra:
        raise ValueError(f"optim_params: missing {missing}, unknown {extra}")
    return gpt_optim_params(**{n: kw[n] for n in names})


class gpt_tensor_desc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("offset", ctypes.c_int64),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


def _load():
    # One HIP runtime per process: torch ships its own libamdhip64 with the
    # same soname as ROCm's.  Loading torch first makes this library bind to
    # that already-loaded runtime instead of pulling in a second copy.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run decoder_only_transformer_fwd_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.gpt_param_layout.argtypes = [ctypes.POINTER(gpt_config), ctypes.POINTER(gpt_tensor_desc), I,
                                     ctypes.POINTER(I), ctypes.POINTER(I64)]
    lib.gpt_workspace_bytes.argtypes = [ctypes.POINTER(gpt_config), ctypes.POINTER(ctypes.c_size_t)]
    lib.gpt_create.argtypes = [ctypes.POINTER(gpt_config), ctypes.POINTER(P)]
    lib.gpt_step.argtypes = [P, P, P, P, ctypes.POINTER(F)]
    lib.gpt_step_accum.argtypes = [P, P, P, P, F, I, ctypes.POINTER(F)]
    lib.gpt_step_micro.argtypes = [P, P, P, I, P, F, I, ctypes.POINTER(F)]
    lib.gpt_optim_state_bytes.argtypes = [ctypes.POINTER(gpt_config), ctypes.POINTER(ctypes.c_size_t)]
    lib.gpt_optim_init.argtypes = [P, P, ctypes.c_size_t]
    lib.gpt_optim_step.argtypes = [P, P, P, ctypes.POINTER(gpt_optim_params), ctypes.POINTER(F)]
    lib.gpt_optim_master.argtypes = [P, ctypes.POINTER(P)]
    lib.gpt_kv_cache_bytes.argtypes = [ctypes.POINTER(gpt_config), ctypes.POINTER(ctypes.c_size_t)]
    lib.gpt_prefill.argtypes = [P, P, I, P, P]
    lib.gpt_decode.argtypes = [P, P, I, P, P]
    lib.gpt_rope_table.argtypes = [ctypes.POINTER(gpt_config), P, P]
    lib.gpt_overlap_enable.argtypes = [P, I]
    lib.gpt_rope_epilogue_enable.argtypes = [P, I]
    lib.gpt_destroy.argtypes = [P]
    lib.gpt_destroy.restype = None
    lib.gpt_debug_tensor.argtypes = [P, I, I, ctypes.POINTER(P), ctypes.POINTER(I64), ctypes.POINTER(I64),
                                     ctypes.POINTER(I)]
    lib.gpt_gemm.argtypes = [I, I, I, I, I, P, P, P, P, I, I, P]
    lib.gpt_gemm_noalloc.argtypes = [I, I, I, I, I, P, P, P, I, I, P]
    lib.gpt_fp8_quantize.argtypes = [I, P, I, I, P, P, P, P, P]
    lib.gpt_gemm_fp8.argtypes = [I, I, I, I, P, P, P, P, P, P, I, P]
    D = ctypes.c_double
    lib.gpt_profile_enable.argtypes = [P, I]
    lib.gpt_profile_sites.argtypes = [P, ctypes.POINTER(I)]
    lib.gpt_profile_get.argtypes = [P, I, ctypes.c_char_p, I, ctypes.c_char_p, I, ctypes.POINTER(I64),
                                    ctypes.POINTER(D), ctypes.POINTER(D), ctypes.POINTER(I)]
    lib.gpt_strerror.argtypes = [I]
    lib.gpt_strerror.restype = ctypes.c_char_p
    lib.gpt_last_error.argtypes = []
    lib.gpt_last_error.restype = ctypes.c_char_p
    for name in ("gpt_param_layout", "gpt_workspace_bytes", "gpt_create", "gpt_step", "gpt_step_accum", "gpt_step_micro",
                 "gpt_optim_state_bytes", "gpt_optim_init", "gpt_optim_step", "gpt_optim_master",
                 "gpt_kv_cache_bytes", "gpt_prefill", "gpt_decode", "gpt_rope_table", "gpt_overlap_enable",
                 "gpt_rope_epilogue_enable", "gpt_debug_tensor", "gpt_gemm", "gpt_gemm_noalloc", "gpt_fp8_quantize", "gpt_gemm_fp8", "gpt_profile_enable",
                 "gpt_profile_sites", "gpt_profile_get"):
        getattr(lib, name).restype = I
    return lib


_lib = _load()


class GPTError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.gpt_strerror(code).decode()
        detail = _lib.gpt_last_error().decode()
        super().__init__(f"{where}: {msg} ({code}): {detail}")


def _check(code: int, where: str) -> None:
    if code != GPT_OK:
        raise GPTError(code, where)


_PREC = {"fp32": GPT_FP32, "bf16": GPT_BF16, "fp8": GPT_FP8}


def make_config(shape, weights: int = 0, workspace: int = 0, workspace_bytes: int = 0,
                stream: int = 0) -> gpt_config:
    """gpt_config from a workload description (any object with the fields of
    ``gpt_inputs.GPTShape``) plus raw device pointers."""
    c = gpt_config()
    c.depth, c.d_model, c.n_head, c.head_dim = shape.depth, shape.d_model, shape.n_head, shape.head_dim
    c.mlp_hidden, c.vocab, c.seq_len, c.batch = shape.mlp_hidden, shape.vocab, shape.seq_len, shape.batch
    c.window = shape.window
    c.window_pattern = shape.window_pattern.encode()
    c.rope_base, c.norm_eps = shape.rope_base, shape.norm_eps
    c.precision = _PREC[shape.precision]
    c.n_kv_head = getattr(shape, "n_kv_head", 0)
    c.weights, c.workspace, c.workspace_bytes, c.stream = weights or None, workspace or None, workspace_bytes, stream or None
    return c


def gpt_param_layout(cfg: gpt_config) -> Tuple[List[Tuple[str, int, int, int]], int]:
    """[(name, element offset, rows, cols)], total elements."""
    n = ctypes.c_int()
    tot = ctypes.c_int64()
    _check(_lib.gpt_param_layout(ctypes.byref(cfg), None, 0, ctypes.byref(n), ctypes.byref(tot)), "gpt_param_layout")
    arr = (gpt_tensor_desc * n.value)()
    _check(_lib.gpt_param_layout(ctypes.byref(cfg), arr, n.value, ctypes.byref(n), ctypes.byref(tot)),
           "gpt_param_layout")
    return [(a.name.decode(), a.offset, a.rows, a.cols) for a in arr], tot.value


def gpt_workspace_bytes(cfg: gpt_config) -> int:
    b = ctypes.c_size_t()
    _check(_lib.gpt_workspace_bytes(ctypes.byref(cfg), ctypes.byref(b)), "gpt_workspace_bytes")
    return b.value


def gpt_create(cfg: gpt_config) -> int:
    h = ctypes.c_void_p()
    _check(_lib.gpt_create(ctypes.byref(cfg), ctypes.byref(h)), "gpt_create")
    return h.value


def gpt_step(model: int, tokens: int, targets: int, grads: int) -> float:
    loss = ctypes.c_float()
    _check(_lib.gpt_step(model, tokens, targets, grads, ctypes.byref(loss)), "gpt_step")
    return loss.value


def gpt_step_rc(model: int, tokens: int, targets: int, grads: int) -> Tuple[int, float]:
    """Like gpt_step but returns (code, loss) instead of raising."""
    loss = ctypes.c_float()
    rc = _lib.gpt_step(model, tokens, targets, grads, ctypes.byref(loss))
    return rc, loss.value


def gpt_step_accum(model: int, tokens: int, targets: int, grads: int, grad_scale: float, accumulate: bool) -> float:
    """grads <- (grads if accumulate else 0) + grad_scale * d(mean loss)/d(weights)."""
    loss = ctypes.c_float()
    _check(_lib.gpt_step_accum(model, tokens, targets, grads, float(grad_scale), int(bool(accumulate)),
                               ctypes.byref(loss)), "gpt_step_accum")
    return loss.value


def gpt_optim_state_bytes(cfg: gpt_config) -> int:
    b = ctypes.c_size_t()
    _check(_lib.gpt_optim_state_bytes(ctypes.byref(cfg), ctypes.byref(b)), "gpt_optim_state_bytes")
    return b.value


def gpt_optim_init(model: int, state: int, nbytes: int) -> None:
    _check(_lib.gpt_optim_init(model, state, nbytes), "gpt_optim_init")


def gpt_optim_step(model: int, state: int, grads: int, hp: gpt_optim_params, want_norm: bool = False):
    """Enqueue one optimizer step; returns the gradient norm when asked
    (which waits for the stream), else None."""
    if want_norm:
        n = ctypes.c_float()
        _check(_lib.gpt_optim_step(model, state, grads, ctypes.byref(hp), ctypes.byref(n)), "gpt_optim_step")
        return n.value
    _check(_lib.gpt_optim_step(model, state, grads, ctypes.byref(hp), None), "gpt_optim_step")
    return None


def gpt_optim_master(model: int) -> int:
    p = ctypes.c_void_p()
    _check(_lib.gpt_optim_master(model, ctypes.byref(p)), "gpt_optim_master")
    return p.value


def gpt_kv_cache_bytes(cfg: gpt_config) -> int:
    b = ctypes.c_size_t()
    _check(_lib.gpt_kv_cache_bytes(ctypes.byref(cfg), ctypes.byref(b)), "gpt_kv_cache_bytes")
    return b.value


def gpt_prefill(model: int, tokens: int, n_tokens: int, kv_cache: int, logits: int) -> None:
    _check(_lib.gpt_prefill(model, tokens, n_tokens, kv_cache, logits), "gpt_prefill")


def gpt_decode(model: int, tokens: int, pos: int, kv_cache: int, logits: int) -> None:
    _check(_lib.gpt_decode(model, tokens, pos, kv_cache, logits), "gpt_decode")


def gpt_step_micro(model: int, tokens: int, targets: int, n_micro: int, grads: int, grad_scale: float,
                   accumulate: bool) -> List[float]:
    """n_micro micro-batches ([n_micro, B, T] device token buffers) in one
    graph replay; returns the micro-batch losses."""
    losses = (ctypes.c_float * n_micro)()
    _check(_lib.gpt_step_micro(model, tokens, targets, n_micro, grads, float(grad_scale), int(bool(accumulate)),
                               losses), "gpt_step_micro")
    return list(losses)


def gpt_rope_table(cfg: gpt_config) -> Tuple[np.ndarray, np.ndarray]:
    """The library's RoPE table (host computation): cos, sin as fp32 [T, Dh/2]."""
    half = cfg.head_dim // 2
    c = np.zeros((cfg.seq_len, half), dtype=np.float32)
    s = np.zeros((cfg.seq_len, half), dtype=np.float32)
    _check(_lib.gpt_rope_table(ctypes.byref(cfg), c.ctypes.data, s.ctypes.data), "gpt_rope_table")
    return c, s


def gpt_overlap_enable(model: int, on: bool) -> None:
    _check(_lib.gpt_overlap_enable(model, 1 if on else 0), "gpt_overlap_enable")


def gpt_rope_epilogue_enable(model: int, on: bool) -> None:
    _check(_lib.gpt_rope_epilogue_enable(model, 1 if on else 0), "gpt_rope_epilogue_enable")


def gpt_destroy(model: int) -> None:
    _lib.gpt_destroy(model)


def gpt_debug_tensor(model: int, which: int, layer: int = 0) -> Tuple[int, int, int, int]:
    p = ctypes.c_void_p()
    r, c, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    _check(_lib.gpt_debug_tensor(model, which, layer, ctypes.byref(p), ctypes.byref(r), ctypes.byref(c),
                                 ctypes.byref(e)), "gpt_debug_tensor")
    return p.value, r.value, c.value, e.value


def gpt_gemm(dtype: int, layout: int, M: int, N: int, K: int, A: int, B: int, C: int,
             workspace: int = 0, splits: int = 1, tile: int = -1, stream: int = 0) -> None:
    _check(_lib.gpt_gemm(dtype, layout, M, N, K, A, B, C, workspace or None, splits, tile, stream or None),
           "gpt_gemm")


NOALLOC_SCRATCH_BYTES = 64 << 20


def gpt_gemm_noalloc(dtype: int, layout: int, M: int, N: int, K: int, A: int, B: int, C: int,
                     splits: int = 1, tile: int = -1, stream: int = 0) -> None:
    """gpt_gemm with the split-K partials in the library's own scratch array."""
    _check(_lib.gpt_gemm_noalloc(dtype, layout, M, N, K, A, B, C, splits, tile, stream or None), "gpt_gemm_noalloc")


def gpt_fp8_quantize(fmt: int, x: int, rows: int, cols: int, amax: int, scale: int, q: int, qT: int = 0,
                     stream: int = 0) -> None:
    _check(_lib.gpt_fp8_quantize(fmt, x, rows, cols, amax, scale, q, qT or None, stream or None), "gpt_fp8_quantize")


def gpt_gemm_fp8(fmt_a: int, M: int, N: int, K: int, A: int, B: int, scale_a: int, scale_b: int, C: int,
                 workspace: int = 0, splits: int = 1, stream: int = 0) -> None:
    _check(_lib.gpt_gemm_fp8(fmt_a, M, N, K, A, B, scale_a, scale_b, C, workspace or None, splits, stream or None),
           "gpt_gemm_fp8")


def gpt_profile_enable(model: int, on: bool) -> None:
    _check(_lib.gpt_profile_enable(model, 1 if on else 0), "gpt_profile_enable")


def gpt_profile_sites(model: int) -> int:
    n = ctypes.c_int()
    _check(_lib.gpt_profile_sites(model, ctypes.byref(n)), "gpt_profile_sites")
    return n.value


def gpt_profile_get(model: int, index: int) -> dict:
    name = ctypes.create_string_buffer(64)
    kern = ctypes.create_string_buffer(160)
    la, ms, wk, kind = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    _check(_lib.gpt_profile_get(model, index, name, 64, kern, 160, ctypes.byref(la), ctypes.byref(ms),
                                ctypes.byref(wk), ctypes.byref(kind)), "gpt_profile_get")
    return dict(name=name.value.decode(), kernel=kern.value.decode(), launches=la.value, total_ms=ms.value,
                work=wk.value, work_kind="flops" if kind.value == 0 else "bytes")


def gpt_strerror(code: int) -> str:
    return _lib.gpt_strerror(code).decode()


def gpt_create_rc(cfg: gpt_config) -> int:
    """Return code of gpt_create (the handle, if any, is destroyed)."""
    h = ctypes.c_void_p()
    rc = _lib.gpt_create(ctypes.byref(cfg), ctypes.byref(h))
    if rc == GPT_OK:
        _lib.gpt_destroy(h)
    return rc


# ---------------------------------------------------------------------------
# Session: device buffers owned by torch, one handle, one stream.
# ---------------------------------------------------------------------------

class Session:
    """Holds the weights, workspace, gradients and token buffers of one
    workload on a torch device and a library handle bound to them."""

    def __init__(self, shape, weights: Dict[str, np.ndarray], device: str = "cuda:0", stream=None):
        import torch
        self.torch = torch
        self.shape = shape
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        cfg = make_config(shape)
        self.layout, self.total = gpt_param_layout(cfg)
        pdt = torch.float32 if shape.precision == "fp32" else torch.bfloat16
        host = np.zeros(self.total, dtype=np.float32 if pdt == torch.float32 else np.uint16)
        for name, off, r, c in self.layout:
            w = weights[name]
            assert w.shape == (r, c), (name, w.shape, (r, c))
            host[off:off + r * c] = w.reshape(-1).view(host.dtype)
        ht = torch.from_numpy(host)
        if pdt == torch.bfloat16:
            ht = ht.view(torch.bfloat16)
        # allocations are 256-byte aligned by torch's caching allocator
        self.weights = ht.to(self.device)
        self.grads = torch.empty(self.total, dtype=torch.float32, device=self.device)
        cfg = make_config(shape, weights=self.weights.data_ptr())
        self.ws_bytes = gpt_workspace_bytes(cfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        cfg = make_config(shape, self.weights.data_ptr(), self.workspace.data_ptr(), self.ws_bytes,
                          self.stream.cuda_stream)
        self.cfg = cfg
        self.handle = gpt_create(cfg)
        self.tokens = None
        self.targets = None

    def set_tokens(self, X: np.ndarray, Y: np.ndarray) -> None:
        t = self.torch
        self.tokens = t.from_numpy(np.ascontiguousarray(X, dtype=np.int32)).to(self.device)
        self.targets = t.from_numpy(np.ascontiguousarray(Y, dtype=np.int32)).to(self.device)

    def step(self) -> float:
        return gpt_step(self.handle, self.tokens.data_ptr(), self.targets.data_ptr(), self.grads.data_ptr())

    def step_accum(self, grad_scale: float, accumulate: bool) -> float:
        return gpt_step_accum(self.handle, self.tokens.data_ptr(), self.targets.data_ptr(), self.grads.data_ptr(),
                              grad_scale, accumulate)

    def step_micro(self, X: np.ndarray, Y: np.ndarray, grad_scale: float, accumulate: bool) -> List[float]:
        """X, Y: int32 [n, B, T] (host arrays or device tensors)."""
        t = self.torch
        xs = X if isinstance(X, t.Tensor) else t.from_numpy(np.ascontiguousarray(X, np.int32))
        ys = Y if isinstance(Y, t.Tensor) else t.from_numpy(np.ascontiguousarray(Y, np.int32))
        xs = xs.to(self.device).contiguous()
        ys = ys.to(self.device).contiguous()
        self._micro = (xs, ys)   # keep the buffers the captured graph reads alive
        return gpt_step_micro(self.handle, xs.data_ptr(), ys.data_ptr(), xs.shape[0], self.grads.data_ptr(),
                              grad_scale, accumulate)

    def optim_init(self) -> None:
        """Allocate (torch) and prepare the optimizer state of this model."""
        t = self.torch
        self.optim_bytes = gpt_optim_state_bytes(self.cfg)
        self.optim_state = t.empty(self.optim_bytes, dtype=t.uint8, device=self.device)
        gpt_optim_init(self.handle, self.optim_state.data_ptr(), self.optim_bytes)

    def optim_step(self, hp: gpt_optim_params, want_norm: bool = False):
        return gpt_optim_step(self.handle, self.optim_state.data_ptr(), self.grads.data_ptr(), hp, want_norm)

    def master_numpy(self) -> Dict[str, np.ndarray]:
        """fp32 master weights (copied to the host), per tensor."""
        t = self.torch
        ptr = gpt_optim_master(self.handle)
        n = self.total
        buf = t.empty(n, dtype=t.float32, device=self.device)
        self.stream.synchronize()
        rc = _hip().hipMemcpy(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(ptr), ctypes.c_size_t(n * 4), 3)
        if rc != 0:
            raise RuntimeError(f"hipMemcpy failed: {rc}")
        g = buf.cpu().numpy()
        return {name: g[off:off + r * c].reshape(r, c).copy() for name, off, r, c in self.layout}

    def infer_init(self) -> None:
        """Allocate (torch) the KV cache and a logits buffer."""
        t = self.torch
        self.kv_bytes = gpt_kv_cache_bytes(self.cfg)
        self.kv = t.empty(self.kv_bytes, dtype=t.uint8, device=self.device)
        self.logits = t.empty((self.shape.batch, self.shape.vocab), dtype=t.float32, device=self.device)

    def prefill(self, prompt) -> "np.ndarray":
        """prompt: int32 [B, n] (host array or device tensor); returns the
        next-token logits [B, V] as a device tensor."""
        t = self.torch
        x = prompt if isinstance(prompt, t.Tensor) else t.from_numpy(np.ascontiguousarray(prompt, np.int32))
        x = x.to(self.device).contiguous()
        gpt_prefill(self.handle, x.data_ptr(), x.shape[1], self.kv.data_ptr(), self.logits.data_ptr())
        return self.logits

    def decode(self, tokens, pos: int):
        """tokens: int32 [B] at position pos; returns logits [B, V] (device)."""
        t = self.torch
        x = tokens if isinstance(tokens, t.Tensor) else t.from_numpy(np.ascontiguousarray(tokens, np.int32))
        x = x.to(self.device).contiguous()
        gpt_decode(self.handle, x.data_ptr(), pos, self.kv.data_ptr(), self.logits.data_ptr())
        return self.logits

    def step_rc(self) -> Tuple[int, float]:
        return gpt_step_rc(self.handle, self.tokens.data_ptr(), self.targets.data_ptr(), self.grads.data_ptr())

    def grads_numpy(self) -> Dict[str, np.ndarray]:
        g = self.grads.cpu().numpy()
        return {name: g[off:off + r * c].reshape(r, c).copy() for name, off, r, c in self.layout}

    def grad_samples(self, indices: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
        """Gradient values at flat per-tensor indices, gathered on the device."""
        t = self.torch
        out = {}
        offs = {name: off for name, off, _, _ in self.layout}
        for name, idx in indices.items():
            gi = t.from_numpy(idx + offs[name]).to(self.device)
            out[name] = self.grads[gi].cpu().numpy().astype(np.float64)
        return out

    def grad_norms(self) -> Dict[str, float]:
        return {name: float(self.grads[off:off + r * c].double().norm().item()) for name, off, r, c in self.layout}

    def debug_tensor(self, which: int, layer: int = 0) -> np.ndarray:
        t = self.torch
        ptr, rows, cols, eb = gpt_debug_tensor(self.handle, which, layer)
        n = rows * cols
        dt = t.float32 if eb == 4 else t.bfloat16
        # copy through a torch buffer on the same stream
        buf = t.empty(n, dtype=dt, device=self.device)
        import ctypes as _c
        hip = _hip()
        self.stream.synchronize()
        rc = hip.hipMemcpy(_c.c_void_p(buf.data_ptr()), _c.c_void_p(ptr), _c.c_size_t(n * eb), 3)
        if rc != 0:
            raise RuntimeError(f"hipMemcpy failed: {rc}")
        return buf.float().cpu().numpy().reshape(rows, cols)

    def profile(self, on: bool = True) -> None:
        gpt_profile_enable(self.handle, on)

    def overlap(self, on: bool = True) -> None:
        gpt_overlap_enable(self.handle, on)

    def rope_epilogue(self, on: bool = True) -> None:
        gpt_rope_epilogue_enable(self.handle, on)

    def profile_sites(self) -> List[dict]:
        return [gpt_profile_get(self.handle, i) for i in range(gpt_profile_sites(self.handle))]

    def close(self) -> None:
        if self.handle:
            gpt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_hip_lib = None


def _hip():
    global _hip_lib
    if _hip_lib is None:
        _hip_lib = ctypes.CDLL("libamdhip64.so")
        _hip_lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip_lib.hipMemcpy.restype = ctypes.c_int
    return _hip_lib
