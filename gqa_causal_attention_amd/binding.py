"""ctypes binding of the decoder-block C ABI (include/gqa_block.h).

Argument marshalling only: every step of the block runs in the HIP library.
torch supplies device memory (weights, state buffers, workspace, inputs and
outputs) and the current HIP stream.  If the built library is missing, loading
fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libgqa_block.so")

GQA_F32, GQA_BF16 = 0, 1
STATUS = {0: "OK", -1: "ARG", -2: "SHAPE", -3: "DTYPE", -4: "NONFINITE", -5: "CAPACITY",
          -6: "POSITION", -7: "STATE", -8: "WORKSPACE", -9: "BUSY", -10: "HIP", -11: "UNSUPPORTED"}

# Exported entry points declared in include/gqa_block.h.
EXPORTS = ("gqa_block_create", "gqa_block_destroy", "gqa_state_bytes", "gqa_block_allocate_state",
           "gqa_state_set_lengths", "gqa_state_get_lengths", "gqa_state_free", "gqa_workspace_bytes",
           "gqa_block_forward", "gqa_block_forward_ragged", "gqa_backward_workspace_bytes", "gqa_block_backward",
           "gqa_block_step", "gqa_block_step_noalloc", "gqa_block_status",
           "gqa_block_describe_plan", "gqa_block_set_timing",
           "gqa_block_kernel_times", "gqa_last_error", "gqa_version")


class GqaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.name = STATUS.get(code, str(code))


class Config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("window", ctypes.c_int32),
                ("max_positions", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("attn_softcap", ctypes.c_float), ("norm", ctypes.c_int32), ("mlp", ctypes.c_int32),
                ("qkv_bias", ctypes.c_int32), ("qk_norm", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("rope_scaling", ctypes.c_int32), ("rope_factor", ctypes.c_float),
                ("rope_low_freq_factor", ctypes.c_float), ("rope_high_freq_factor", ctypes.c_float),
                ("rope_original_max_positions", ctypes.c_int32), ("o_bias", ctypes.c_int32),
                ("mlp_bias", ctypes.c_int32), ("norm_bias", ctypes.c_int32), ("sandwich_norms", ctypes.c_int32)]

NORM_KINDS = {"rmsnorm": 0, "rmsnorm_offset": 1, "layernorm": 2}
MLP_KINDS = {"swiglu": 0, "geglu_tanh": 1, "geglu": 2, "gelu": 3, "gelu_tanh": 4}

ROPE_SCALING = {None: 0, "linear": 1, "llama3": 2}


class Tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data_dev", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 2)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"HIP library not built: {path} (run python -m gqa_causal_attention_amd.build)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "gqa_block_create": ([ctypes.POINTER(Config), ctypes.POINTER(Tensor), I32, ctypes.POINTER(P)], I32),
        "gqa_block_destroy": ([P], None),
        "gqa_state_bytes": ([P, I32, I32, ctypes.POINTER(SZ)], I32),
        "gqa_block_allocate_state": ([P, I32, I32, P, P, P, ctypes.POINTER(P)], I32),
        "gqa_state_set_lengths": ([P, ctypes.POINTER(I32), P], I32),
        "gqa_state_get_lengths": ([P, ctypes.POINTER(I32)], I32),
        "gqa_state_free": ([P], None),
        "gqa_workspace_bytes": ([P, I32, I32, ctypes.POINTER(SZ)], I32),
        "gqa_block_forward": ([P, P, P, P, I32, I32, P, SZ, P], I32),
        "gqa_block_forward_ragged": ([P, P, P, I32, I32, ctypes.POINTER(I32), P, SZ, P], I32),
        "gqa_backward_workspace_bytes": ([P, I32, I32, ctypes.POINTER(SZ)], I32),
        "gqa_block_backward": ([P, P, P, P, ctypes.POINTER(P), I32, I32, P, SZ, P], I32),
        "gqa_block_step": ([P, P, P, P, I32, P, SZ, P], I32),
        "gqa_block_step_noalloc": ([P, P, P, P, I32, P], I32),
        "gqa_block_status": ([P, P], I32),
        "gqa_block_describe_plan": ([P, I32, I32, I32, ctypes.c_char_p, SZ, ctypes.POINTER(SZ)], I32),
        "gqa_block_set_timing": ([P, I32], I32),
        "gqa_block_kernel_times": ([P, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64), I32], I32),
        "gqa_last_error": ([], ctypes.c_char_p),
        "gqa_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise GqaError(rc, load_library().gqa_last_error().decode())
    return rc


def make_config(cfg: dict) -> Config:
    return Config(
        d_model=cfg["d_model"], n_heads=cfg["n_heads"], n_kv_heads=cfg["n_kv_heads"],
        head_dim=cfg["head_dim"], intermediate=cfg["intermediate"], window=cfg.get("window", 0),
        max_positions=cfg.get("max_positions", 8192), rope_theta=cfg.get("rope_theta", 10000.0),
        norm_eps=cfg.get("norm_eps", 1e-6), attn_softcap=cfg.get("attn_softcap", 0.0) or 0.0,
        norm=_kind(NORM_KINDS, cfg.get("norm", "rmsnorm"), "norm"),
        mlp=_kind(MLP_KINDS, cfg.get("mlp", "swiglu"), "mlp"),
        qkv_bias=int(bool(cfg.get("qkv_bias"))), qk_norm=int(bool(cfg.get("qk_norm"))),
        o_bias=int(bool(cfg.get("o_bias"))), mlp_bias=int(bool(cfg.get("mlp_bias"))),
        norm_bias=int(bool(cfg.get("norm_bias"))), sandwich_norms=int(bool(cfg.get("sandwich_norms"))),
        weight_dtype=GQA_BF16 if cfg.get("dtype", "f32") == "bf16" else GQA_F32,
        rope_dim=cfg.get("rope_dim") or 0, **_rope_scaling_fields(cfg.get("rope_scaling")))


def _kind(table: dict, name: str, what: str) -> int:
    if name not in table:
        raise ValueError(f"unknown {what} {name!r} (one of {', '.join(table)})")
    return table[name]


def _rope_scaling_fields(sc) -> dict:
    """mojolearn ``rope_scaling`` (None, {"type": "linear", "factor": f} or
    {"type": "llama3", "factor", "low_freq_factor", "high_freq_factor",
    "original_max_position_embeddings"}) as the C config's fields."""
    if not sc:
        return {}
    kind = sc.get("type", sc.get("rope_type"))
    if kind not in ("linear", "llama3"):
        raise ValueError(f"unknown rope_scaling type {kind!r}")
    out = dict(rope_scaling=ROPE_SCALING[kind], rope_factor=float(sc["factor"]))
    if kind == "llama3":
        out.update(rope_low_freq_factor=float(sc["low_freq_factor"]),
                   rope_high_freq_factor=float(sc["high_freq_factor"]),
                   rope_original_max_positions=int(sc["original_max_position_embeddings"]))
    return out


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _require(t, name: str, shape: tuple, device) -> None:
    """Raise ValueError unless t is a contiguous float32 tensor of `shape` on
    `device` (checked before any pointer reaches the library, so a mis-shaped
    or host tensor never becomes an out-of-bounds device access)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the block is on {device}")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


_MATRICES = ("q_proj.weight", "k_proj.weight", "v_proj.weight", "o_proj.weight", "gate_proj.weight",
             "up_proj.weight", "down_proj.weight")


class Block:
    """One decoder block on the GPU (mojolearn TransformerBlock semantics).

    ``weights``: HF name -> numpy array or torch tensor, [out, in] layout.
    Matrices are placed on the device in the block's dtype, norm weights and
    biases in float32; the block keeps them alive.
    """

    def __init__(self, cfg: dict, weights: dict, device: str = "cuda"):
        import torch
        self.lib = load_library()
        self.cfg = dict(cfg)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.ccfg = make_config(cfg)
        self.bf16 = self.ccfg.weight_dtype == GQA_BF16
        self.tensors = {}
        recs = []
        for name, w in weights.items():
            t = torch.as_tensor(np.asarray(w)) if not isinstance(w, torch.Tensor) else w
            if name in _MATRICES and self.bf16:
                t = t.to(device=self.device, dtype=torch.bfloat16).contiguous()
                dt = GQA_BF16
            else:
                t = t.to(device=self.device, dtype=torch.float32).contiguous()
                dt = GQA_F32
            self.tensors[name] = t
            shape = (ctypes.c_int64 * 2)(*(list(t.shape) + [0, 0])[:2])
            recs.append(Tensor(name.encode(), ctypes.c_void_p(t.data_ptr()), dt, t.dim(), shape))
        arr = (Tensor * len(recs))(*recs)
        h = ctypes.c_void_p()
        _check(self.lib.gqa_block_create(ctypes.byref(self.ccfg), arr, len(recs), ctypes.byref(h)))
        self.handle = h
        self._ws = None
        self._ws_captured = False
        self._retired = []   # workspaces a captured graph may still use

    def close(self):
        if getattr(self, "handle", None):
            self.lib.gqa_block_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def act_dtype(self):
        import torch
        return torch.bfloat16 if self.bf16 else torch.float32

    def workspace(self, B: int, L: int):
        """The block's device workspace, grown on demand.  A buffer used while
        a HIP graph is being captured stays alive with the block (a replay
        keeps using it), so growing it later never frees memory a graph holds."""
        import torch
        n = ctypes.c_size_t()
        _check(self.lib.gqa_workspace_bytes(self.handle, B, L, ctypes.byref(n)))
        if self._ws is None or self._ws.numel() < n.value:
            if self._ws is not None and self._ws_captured:
                self._retired.append(self._ws)
            self._ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=self.device)
            self._ws_captured = False
        if torch.cuda.is_current_stream_capturing():
            self._ws_captured = True
        return self._ws, n.value

    def allocate_state(self, batch: int, max_tokens: int) -> "State":
        return State(self, batch, max_tokens)

    def forward(self, x, state: "State | None" = None, out=None, stream=None, lengths=None):
        """mojolearn TransformerBlock.forward; `lengths` (B ints in [1, L], no
        state) makes the batch ragged: padding positions output +0.0."""
        import torch
        if not isinstance(x, torch.Tensor) or x.dim() != 3:
            raise ValueError("x must be a [B, L, d_model] tensor")
        B, L, _ = x.shape
        _require(x, "x", (B, L, self.cfg["d_model"]), self.device)
        y = torch.empty_like(x) if out is None else out
        _require(y, "out", tuple(x.shape), self.device)
        if state is not None:
            self._check_state(state)
        if lengths is not None:
            if state is not None:
                raise ValueError("lengths is not allowed together with state")
            if len(lengths) != B:
                raise ValueError(f"lengths holds {len(lengths)} values, x has {B} rows")
        ws, nb = self.workspace(B, L)
        if lengths is not None:
            lens = (ctypes.c_int32 * B)(*[int(v) for v in lengths])
            _check(self.lib.gqa_block_forward_ragged(self.handle, ctypes.c_void_p(x.data_ptr()),
                                                     ctypes.c_void_p(y.data_ptr()), B, L, lens,
                                                     ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                                     _stream_ptr(stream)))
            return y
        _check(self.lib.gqa_block_forward(self.handle, state.handle if state else None,
                                          ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                          B, L, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                          _stream_ptr(stream)))
        return y

    BACKWARD_WEIGHTS = ("input_layernorm.weight", "post_attention_layernorm.weight", "q_proj.weight",
                        "k_proj.weight", "v_proj.weight", "o_proj.weight", "gate_proj.weight", "up_proj.weight",
                        "down_proj.weight")

    def backward(self, x, grad_output, stream=None, grads=None):
        """mojolearn TransformerBlock.backward: gradients of a zero-state
        prefill -> {"x": [B, L, d], weight name: gradient in its shape}, all
        float32 torch tensors on the device (``grads`` may supply them)."""
        import torch
        if not isinstance(x, torch.Tensor) or x.dim() != 3:
            raise ValueError("x must be a [B, L, d_model] tensor")
        B, L, _ = x.shape
        _require(x, "x", (B, L, self.cfg["d_model"]), self.device)
        _require(grad_output, "grad_output", tuple(x.shape), self.device)
        if grads is not None:
            _require(grads.get("x"), "grads['x']", tuple(x.shape), self.device)
            for name in self.BACKWARD_WEIGHTS:
                _require(grads.get(name), f"grads[{name!r}]", tuple(self.tensors[name].shape), self.device)
        nb = ctypes.c_size_t()
        _check(self.lib.gqa_backward_workspace_bytes(self.handle, B, L, ctypes.byref(nb)))
        ws = torch.empty(max(nb.value, 1), dtype=torch.uint8, device=self.device)
        if grads is None:
            grads = {"x": torch.empty_like(x)}
            for name in self.BACKWARD_WEIGHTS:
                grads[name] = torch.empty(tuple(self.tensors[name].shape), dtype=torch.float32, device=self.device)
        table = (ctypes.c_void_p * 9)(*[grads[n].data_ptr() for n in self.BACKWARD_WEIGHTS])
        _check(self.lib.gqa_block_backward(self.handle, ctypes.c_void_p(x.data_ptr()),
                                           ctypes.c_void_p(grad_output.data_ptr()),
                                           ctypes.c_void_p(grads["x"].data_ptr()), table, B, L,
                                           ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_ptr(stream)))
        return grads

    def step(self, x, state: "State", out=None, stream=None):
        import torch
        d = self.cfg["d_model"]
        if not isinstance(x, torch.Tensor) or x.dim() not in (2, 3) or (x.dim() == 3 and x.shape[1] != 1):
            raise ValueError("x must be a [B, d_model] or [B, 1, d_model] tensor")
        B = x.shape[0]
        _require(x, "x", (B, d) if x.dim() == 2 else (B, 1, d), self.device)
        if state is not None:
            self._check_state(state)
        y = torch.empty((B, 1, d), dtype=torch.float32, device=x.device) if out is None else out
        if not isinstance(y, torch.Tensor) or y.numel() != B * d:
            raise ValueError(f"out must hold B * d_model = {B * d} values")
        _require(y, "out", tuple(y.shape), self.device)
        ws, nb = self.workspace(B, 1)
        _check(self.lib.gqa_block_step(self.handle, state.handle if state else None,
                                       ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), B,
                                       ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_ptr(stream)))
        return y

    def step_noalloc(self, x, state: "State", out=None, stream=None):
        """step() through the entry point that allocates nothing: the library's
        fixed per-GPU scratch replaces the workspace (``out`` must be given by a
        caller that cannot allocate)."""
        import torch
        d = self.cfg["d_model"]
        if not isinstance(x, torch.Tensor) or x.dim() not in (2, 3) or (x.dim() == 3 and x.shape[1] != 1):
            raise ValueError("x must be a [B, d_model] or [B, 1, d_model] tensor")
        B = x.shape[0]
        _require(x, "x", (B, d) if x.dim() == 2 else (B, 1, d), self.device)
        self._check_state(state)
        y = torch.empty((B, 1, d), dtype=torch.float32, device=x.device) if out is None else out
        if not isinstance(y, torch.Tensor) or y.numel() != B * d:
            raise ValueError(f"out must hold B * d_model = {B * d} values")
        _require(y, "out", tuple(y.shape), self.device)
        _check(self.lib.gqa_block_step_noalloc(self.handle, state.handle, ctypes.c_void_p(x.data_ptr()),
                                               ctypes.c_void_p(y.data_ptr()), B, _stream_ptr(stream)))
        return y

    def _check_state(self, state):
        if not isinstance(state, State) or state.block is not self:
            raise ValueError("state was not allocated by this block")

    def status(self, stream=None):
        _check(self.lib.gqa_block_status(self.handle, _stream_ptr(stream)))

    def describe_plan(self, B: int, L: int, backward: bool = False) -> str:
        """The library's launch plan for a forward (or backward) of B x L tokens."""
        n = ctypes.c_size_t()
        _check(self.lib.gqa_block_describe_plan(self.handle, int(backward), B, L, None, 0, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(n.value)
        _check(self.lib.gqa_block_describe_plan(self.handle, int(backward), B, L, buf, n.value, None))
        return buf.value.decode()

    def set_timing(self, enable: bool):
        _check(self.lib.gqa_block_set_timing(self.handle, int(enable)))

    def kernel_times(self) -> dict:
        cap = 64
        names = (ctypes.c_char_p * cap)()
        ms = (ctypes.c_double * cap)()
        cnt = (ctypes.c_int64 * cap)()
        n = self.lib.gqa_block_kernel_times(self.handle, names, ms, cnt, cap)
        if n < 0:
            _check(n)
        return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n, cap))}


class State:
    """Caller-owned KV cache (mojolearn TransformerState): k/v buffers
    [batch, n_kv_heads, capacity, head_dim] in the block's dtype and int32
    per-row lengths, all torch device tensors."""

    def __init__(self, block: Block, batch: int, max_tokens: int):
        import torch
        self.block = block
        n = ctypes.c_size_t()
        _check(block.lib.gqa_state_bytes(block.handle, batch, max_tokens, ctypes.byref(n)))
        cfg = block.cfg
        w = cfg.get("window", 0)
        cap = w if w > 0 else max_tokens
        shape = (batch, cfg["n_kv_heads"], cap, cfg["head_dim"])
        self.k = torch.zeros(shape, dtype=block.act_dtype, device=block.device)
        self.v = torch.zeros(shape, dtype=block.act_dtype, device=block.device)
        assert self.k.numel() * self.k.element_size() == n.value
        self.lengths = torch.zeros(batch, dtype=torch.int32, device=block.device)
        h = ctypes.c_void_p()
        _check(block.lib.gqa_block_allocate_state(block.handle, batch, max_tokens,
                                                  ctypes.c_void_p(self.k.data_ptr()),
                                                  ctypes.c_void_p(self.v.data_ptr()),
                                                  ctypes.c_void_p(self.lengths.data_ptr()), ctypes.byref(h)))
        self.handle = h
        self.batch, self.max_tokens, self.capacity = batch, max_tokens, cap

    def set_lengths(self, lengths, stream=None):
        arr = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
        assert arr.shape == (self.batch,)
        _check(self.block.lib.gqa_state_set_lengths(self.handle,
                                                    arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                    _stream_ptr(stream)))

    def host_lengths(self) -> np.ndarray:
        arr = np.zeros(self.batch, dtype=np.int32)
        _check(self.block.lib.gqa_state_get_lengths(self.handle, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return arr

    def close(self):
        if getattr(self, "handle", None):
            self.block.lib.gqa_state_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
