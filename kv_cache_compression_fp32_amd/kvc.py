"""Python binding of libkvc.so (include/kvc.h).

Argument marshalling only: the functions below take torch tensors, check their
device, dtype and contiguity, and pass raw device pointers, sizes and the
current HIP stream to the C entry points of the same names. Every step of the
compressor runs in the library's HIP kernels; nothing here computes.

The library is loaded on first use. torch is imported first so that libkvc.so
binds to the HIP runtime torch has already loaded (both carry the soname
libamdhip64.so.7) and device pointers and streams are shared.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK, KVC_EINVAL, KVC_EUNSUPPORTED, KVC_ESPACE, KVC_EHIP = 0, -1, -2, -3, -4
KVC_FP4_E4M3_B16, KVC_FP4_E8M0_B32 = 0, 1
KVC_X_F32, KVC_X_BF16 = 0, 1
KVC_PROJ_AUTO, KVC_PROJ_F32_MFMA, KVC_PROJ_F16_SPLIT, KVC_PROJ_BF16_SPLIT = 0, 1, 2, 3

_lib = None


class KvcError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


class _Config(ctypes.Structure):
    _fields_ = [("ratio", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dim", ctypes.c_int64), ("eps", ctypes.c_float), ("fp4_format", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("x_format", ctypes.c_int32), ("projection", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("wkv", ctypes.c_void_p), ("wgate", ctypes.c_void_p),
                ("ape", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("rope_cs", ctypes.c_void_p), ("rope_rows", ctypes.c_int64)]


class _Outputs(ctypes.Structure):
    _fields_ = [("latent", ctypes.c_void_p), ("pooled", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("dequant", ctypes.c_void_p), ("rotated", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGNATURES = {
    "kvc_proj_width": (_I64, [ctypes.POINTER(_Config)]),
    "kvc_state_rows": (_I64, [ctypes.POINTER(_Config)]),
    "kvc_prefill_workspace_floats": (_I64, [ctypes.POINTER(_Config), _I64, _I64]),
    "kvc_decode_workspace_floats": (_I64, [ctypes.POINTER(_Config), _I64]),
    "compressor_prefill": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), _P, _I64, _I64,
                                          _P, _I64, _P, _P, _I64, ctypes.POINTER(_Outputs),
                                          ctypes.POINTER(_I64), _P]),
    "kvc_time_next_projection": (ctypes.c_int, [_P, _P]),
    "compressor_decode_step": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), _P, _I64, _I64,
                                              _P, _I64, _P, _P, _I64, ctypes.POINTER(_Outputs),
                                              ctypes.POINTER(ctypes.c_int32), _P]),
    "compressor_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), _P, _I64,
                                                      _I64, _P, _P, _I64, ctypes.POINTER(_Outputs),
                                                      ctypes.POINTER(ctypes.c_int32), _P]),
    "kvc_ratio1_workspace_floats": (_I64, [ctypes.POINTER(_Config), _I64]),
    "compressor_ratio1_forward": (ctypes.c_int, [ctypes.POINTER(_Config), _P, _P, _P, _I64, _P, _I64,
                                                 ctypes.POINTER(_Outputs), _P]),
    "latent_fp4_quant": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
    "latent_rope": (ctypes.c_int, [_P, _I64, _I64, ctypes.c_int32, _P, _I64, _I64, _P, _P]),
    "indexer_fp4_quant": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
    "kvc_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "kvc_version": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """The loaded libkvc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_compression_fp32_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().kvc_strerror(code).decode()


def version() -> str:
    return lib().kvc_version().decode()


# ----------------------------------------------------------------- config
@dataclass(frozen=True)
class Config:
    ratio: int
    head_dim: int
    dim: int = 0
    eps: float = 1e-6
    fp4_format: int = KVC_FP4_E4M3_B16
    rope_dim: int = 0
    x_format: int = KVC_X_F32  # KVC_X_BF16: x is the bf16 hidden state
    projection: int = KVC_PROJ_AUTO  # f32 matrix cores for f32 x, exact bf16 split for bf16 x

    @property
    def proj(self) -> int:
        return 2 * self.head_dim if self.ratio == 4 else self.head_dim

    @property
    def state_rows(self) -> int:
        return 2 * self.ratio if self.ratio == 4 else self.ratio

    @property
    def fp4_block(self) -> int:
        return 32 if self.fp4_format == KVC_FP4_E8M0_B32 else 16

    def c(self) -> _Config:
        return _Config(self.ratio, self.head_dim, self.dim, self.eps, self.fp4_format, self.rope_dim,
                       self.x_format, self.projection)


def kvc_proj_width(cfg: Config) -> int:
    return _check(lib().kvc_proj_width(ctypes.byref(cfg.c())), "kvc_proj_width")


def kvc_state_rows(cfg: Config) -> int:
    return _check(lib().kvc_state_rows(ctypes.byref(cfg.c())), "kvc_state_rows")


def kvc_prefill_workspace_floats(cfg: Config, batch: int, seqlen: int) -> int:
    return _check(lib().kvc_prefill_workspace_floats(ctypes.byref(cfg.c()), batch, seqlen),
                  "kvc_prefill_workspace_floats")


def kvc_decode_workspace_floats(cfg: Config, batch: int) -> int:
    return _check(lib().kvc_decode_workspace_floats(ctypes.byref(cfg.c()), batch),
                  "kvc_decode_workspace_floats")


def kvc_ratio1_workspace_floats(cfg: Config, tokens: int) -> int:
    return _check(lib().kvc_ratio1_workspace_floats(ctypes.byref(cfg.c()), tokens),
                  "kvc_ratio1_workspace_floats")


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise KvcError(rc, what)
    return rc


# ----------------------------------------------------------------- marshalling
def _ptr(t, dtype=None, name="tensor") -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _need(t, n: int, name: str) -> None:
    """The C ABI takes bare pointers: a tensor of the wrong size would be read
    or written out of bounds on the GPU, so every size is checked here."""
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} holds {t.numel()} elements, expected {n}")


def _check_state(cfg: "Config", kv_state, score_state, batch: int) -> int:
    """Both state planes [state_batch, state_rows, proj], state_batch >= batch;
    returns state_batch (0 without a state)."""
    if (kv_state is None) != (score_state is None):
        raise ValueError("kv_state and score_state go together")
    if kv_state is None:
        return 0
    for t, name in ((kv_state, "kv_state"), (score_state, "score_state")):
        if t.dim() != 3 or tuple(t.shape[1:]) != (cfg.state_rows, cfg.proj):
            raise ValueError(f"{name} must be [state_batch, {cfg.state_rows}, {cfg.proj}], got {tuple(t.shape)}")
    if kv_state.shape[0] != score_state.shape[0] or kv_state.shape[0] < batch:
        raise ValueError("state planes must share a batch capacity of at least batch rows")
    return kv_state.shape[0]


def _check_weights(cfg: "Config", w: "Weights", projection: bool) -> None:
    if projection:
        if w.wkv is None or w.wgate is None:
            raise ValueError("wkv and wgate are required with x")
        _need(w.wkv, cfg.proj * cfg.dim, "wkv")
        _need(w.wgate, cfg.proj * cfg.dim, "wgate")
    _need(w.ape, cfg.ratio * cfg.proj, "ape")
    _need(w.norm_w, cfg.head_dim, "norm_w")
    if w.rope_cs is not None:
        if w.rope_cs.dim() != 3 or tuple(w.rope_cs.shape[1:]) != (cfg.rope_dim // 2, 2):
            raise ValueError(f"rope_cs must be [rows, {cfg.rope_dim // 2}, 2]")


def _check_outputs(cfg: "Config", out: "Outputs | None", batch: int, groups: int) -> None:
    if out is None:
        return
    hd, n = cfg.head_dim, batch * groups
    for t, name in ((out.latent, "latent"), (out.pooled, "pooled"), (out.dequant, "dequant"),
                    (out.rotated, "rotated")):
        _need(t, n * hd, name)
    _need(out.codes, n * hd // 2, "codes")
    _need(out.scales, n * hd // cfg.fp4_block, "scales")


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream or None


@dataclass
class Weights:
    wkv: torch.Tensor | None = None
    wgate: torch.Tensor | None = None
    ape: torch.Tensor | None = None
    norm_w: torch.Tensor | None = None
    rope_cs: torch.Tensor | None = None  # [rows, rope_dim // 2, 2] float32 (cos, sin)

    def c(self) -> _Weights:
        rows = self.rope_cs.shape[0] if self.rope_cs is not None else 0
        return _Weights(_ptr(self.wkv, torch.float32, "wkv"), _ptr(self.wgate, torch.float32, "wgate"),
                        _ptr(self.ape, torch.float32, "ape"), _ptr(self.norm_w, torch.float32, "norm_w"),
                        _ptr(self.rope_cs, torch.float32, "rope_cs"), rows)


@dataclass
class Outputs:
    latent: torch.Tensor | None = None   # bf16 (or int16 bit patterns)
    pooled: torch.Tensor | None = None   # float32
    codes: torch.Tensor | None = None    # uint8
    scales: torch.Tensor | None = None   # uint8
    dequant: torch.Tensor | None = None  # bf16
    rotated: torch.Tensor | None = None  # bf16

    def c(self) -> _Outputs:
        def bf(t, n):
            if t is None:
                return None
            if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
                raise TypeError(f"{n} must be bf16")
            return _ptr(t, None, n)
        return _Outputs(bf(self.latent, "latent"), _ptr(self.pooled, torch.float32, "pooled"),
                        _ptr(self.codes, torch.uint8, "codes"), _ptr(self.scales, torch.uint8, "scales"),
                        bf(self.dequant, "dequant"), bf(self.rotated, "rotated"))


def _x_ptr(cfg: Config, x):
    return _bf16_ptr(x, "x") if cfg.x_format == KVC_X_BF16 else _ptr(x, torch.float32, "x")


def compressor_prefill(cfg: Config, w: Weights, x: torch.Tensor | None, batch: int, seqlen: int,
                       workspace: torch.Tensor, kv_state: torch.Tensor | None = None,
                       score_state: torch.Tensor | None = None, out: Outputs | None = None,
                       stream=None) -> int:
    """Enqueue a prefill; returns the number of groups (seqlen // ratio)."""
    n = ctypes.c_int64(0)
    if batch < 1 or seqlen < 0:
        raise ValueError("batch must be >= 1 and seqlen >= 0")
    _need(x, batch * seqlen * cfg.dim, "x")
    _check_weights(cfg, w, x is not None)
    state_batch = _check_state(cfg, kv_state, score_state, batch)
    _check_outputs(cfg, out, batch, seqlen // cfg.ratio)
    rc = lib().compressor_prefill(
        ctypes.byref(cfg.c()), ctypes.byref(w.c()), _x_ptr(cfg, x), batch, seqlen,
        _ptr(workspace, torch.float32, "workspace"), workspace.numel(),
        _ptr(kv_state, torch.float32, "kv_state"), _ptr(score_state, torch.float32, "score_state"),
        state_batch, ctypes.byref(out.c()) if out is not None else None, ctypes.byref(n), _stream(stream))
    _check(rc, "compressor_prefill")
    return n.value


def compressor_decode_step(cfg: Config, w: Weights, x: torch.Tensor | None, batch: int, start_pos: int,
                           workspace: torch.Tensor, kv_state: torch.Tensor, score_state: torch.Tensor,
                           out: Outputs | None = None, stream=None) -> bool:
    """Enqueue one decode step; returns True if entries were written. The
    workspace must be zero-filled before its first use (new_decode_workspace);
    steps leave its arrival counters zero."""
    e = ctypes.c_int32(0)
    if batch < 1 or start_pos < 0:
        raise ValueError("batch must be >= 1 and start_pos >= 0")
    _need(x, batch * cfg.dim, "x")
    _check_weights(cfg, w, x is not None)
    if kv_state is None or score_state is None:
        raise ValueError("decode needs both state planes")
    state_batch = _check_state(cfg, kv_state, score_state, batch)
    _check_outputs(cfg, out, batch, 1)
    rc = lib().compressor_decode_step(
        ctypes.byref(cfg.c()), ctypes.byref(w.c()), _x_ptr(cfg, x), batch, start_pos,
        _ptr(workspace, torch.float32, "workspace"), workspace.numel(),
        _ptr(kv_state, torch.float32, "kv_state"), _ptr(score_state, torch.float32, "score_state"),
        state_batch, ctypes.byref(out.c()) if out is not None else None, ctypes.byref(e),
        _stream(stream))
    _check(rc, "compressor_decode_step")
    return bool(e.value)


def compressor_decode_step_noalloc(cfg: Config, w: Weights, x: torch.Tensor, batch: int, start_pos: int,
                                   kv_state: torch.Tensor, score_state: torch.Tensor, out: Outputs | None = None,
                                   stream=None) -> bool:
    """compressor_decode_step without a workspace: the library's own scratch
    array on the current GPU holds the partial sums (calls that overlap on
    one GPU race). Returns True if entries were written."""
    e = ctypes.c_int32(0)
    if batch < 1 or start_pos < 0:
        raise ValueError("batch must be >= 1 and start_pos >= 0")
    if x is None:
        raise ValueError("the step without a workspace needs x")
    _need(x, batch * cfg.dim, "x")
    _check_weights(cfg, w, True)
    if kv_state is None or score_state is None:
        raise ValueError("decode needs both state planes")
    state_batch = _check_state(cfg, kv_state, score_state, batch)
    _check_outputs(cfg, out, batch, 1)
    rc = lib().compressor_decode_step_noalloc(
        ctypes.byref(cfg.c()), ctypes.byref(w.c()), _x_ptr(cfg, x), batch, start_pos,
        _ptr(kv_state, torch.float32, "kv_state"), _ptr(score_state, torch.float32, "score_state"),
        state_batch, ctypes.byref(out.c()) if out is not None else None, ctypes.byref(e), _stream(stream))
    _check(rc, "compressor_decode_step_noalloc")
    return bool(e.value)


def _bf16_ptr(t, name):
    if t is not None and t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bf16")
    return _ptr(t, None, name)


def compressor_ratio1_forward(cfg: Config, wkv: torch.Tensor, x: torch.Tensor, tokens: int,
                              workspace: torch.Tensor, out: Outputs | None = None,
                              norm_w: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue the ratio-1 compressor over `tokens` rows of bf16 x [tokens,
    dim] with bf16 wkv [head_dim, dim]; every token is one entry."""
    if tokens < 0:
        raise ValueError("tokens must be >= 0")
    _need(x, tokens * cfg.dim, "x")
    _need(wkv, cfg.head_dim * cfg.dim, "wkv")
    _need(norm_w, cfg.head_dim, "norm_w")
    _check_outputs(cfg, out, 1, tokens)
    rc = lib().compressor_ratio1_forward(
        ctypes.byref(cfg.c()), _bf16_ptr(wkv, "wkv"), _ptr(norm_w, torch.float32, "norm_w"), _bf16_ptr(x, "x"),
        tokens, _ptr(workspace, torch.float32, "workspace"), workspace.numel(),
        ctypes.byref(out.c()) if out is not None else None, _stream(stream))
    _check(rc, "compressor_ratio1_forward")


def latent_rope(inp: torch.Tensor, rope_dim: int, rope_cs: torch.Tensor, first_row: int = 0,
                out: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue RoPE of [rows, width] bf16 rows (in place when out is None or
    inp): row r turns its last rope_dim features by rope_cs[first_row + r]."""
    if inp.dim() != 2:
        raise ValueError("inp must be [rows, width]")
    rows, width = inp.shape
    dst = inp if out is None else out
    _need(dst, rows * width, "out")
    if rope_cs.dim() != 3 or tuple(rope_cs.shape[1:]) != (rope_dim // 2, 2):
        raise ValueError(f"rope_cs must be [rows, {rope_dim // 2}, 2]")
    rc = lib().latent_rope(_bf16_ptr(inp, "inp"), rows, width, rope_dim, _ptr(rope_cs, torch.float32, "rope_cs"),
                           rope_cs.shape[0], first_row, _bf16_ptr(dst, "out"), _stream(stream))
    _check(rc, "latent_rope")


def _fp4_quant(fn, name, block, inp, codes, scales, out, stream):
    if inp.dim() != 2:
        raise ValueError("inp must be [rows, width]")
    if inp.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("inp must be bf16")
    if out is not None and out.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("out must be bf16")
    rows, width = inp.shape
    if width % block:
        raise ValueError(f"width must be a multiple of {block}")
    _need(codes, rows * width // 2, "codes")
    _need(scales, rows * width // block, "scales")
    _need(out, rows * width, "out")
    rc = fn(_ptr(inp, None, "inp"), rows, width, _ptr(codes, torch.uint8, "codes"),
            _ptr(scales, torch.uint8, "scales"), _ptr(out, None, "out"), _stream(stream))
    _check(rc, name)


def latent_fp4_quant(inp: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue the latent's fp4 round trip (e4m3 scales, blocks of 16) of
    [rows, width] bf16 values."""
    _fp4_quant(lib().latent_fp4_quant, "latent_fp4_quant", 16, inp, codes, scales, out, stream)


def indexer_fp4_quant(inp: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue the indexer's fp4 round trip (power-of-two scales, blocks of
    32) of [rows, width] bf16 values."""
    _fp4_quant(lib().indexer_fp4_quant, "indexer_fp4_quant", 32, inp, codes, scales, out, stream)


def time_next_projection(start: "torch.cuda.Event | None", stop: "torch.cuda.Event | None") -> None:
    """Measurement hook: the next compressor call of this thread records
    `start` / `stop` (torch.cuda.Event with enable_timing, already recorded
    once so that they exist) right before and after its projection kernel on
    its stream. None, None clears a pending request."""
    a = start.cuda_event if start is not None else None
    b = stop.cuda_event if stop is not None else None
    _check(lib().kvc_time_next_projection(a or None, b or None), "kvc_time_next_projection")


# ----------------------------------------------------------------- convenience
def new_decode_workspace(cfg: Config, batch: int, device="cuda") -> torch.Tensor:
    """A zero-filled decode workspace (its arrival counters must start at 0)."""
    return torch.zeros(kvc_decode_workspace_floats(cfg, batch), dtype=torch.float32, device=device)


def new_state(cfg: Config, batch: int, device="cuda") -> tuple[torch.Tensor, torch.Tensor]:
    """kv_state / score_state planes initialised as the model does (kv 0,
    score -inf)."""
    rows, proj = kvc_state_rows(cfg), kvc_proj_width(cfg)
    kv = torch.zeros((batch, rows, proj), dtype=torch.float32, device=device)
    sc = torch.full((batch, rows, proj), float("-inf"), dtype=torch.float32, device=device)
    return kv, sc


def new_outputs(cfg: Config, batch: int, groups: int, latent=True, pooled=False, fp4=False,
                dequant=False, rotated=False, device="cuda") -> Outputs:
    hd = cfg.head_dim
    o = Outputs()
    if latent:
        o.latent = torch.empty((batch, groups, hd), dtype=torch.bfloat16, device=device)
    if pooled:
        o.pooled = torch.empty((batch, groups, hd), dtype=torch.float32, device=device)
    if fp4:
        o.codes = torch.empty((batch, groups, hd // 2), dtype=torch.uint8, device=device)
        o.scales = torch.empty((batch, groups, hd // cfg.fp4_block), dtype=torch.uint8, device=device)
    if dequant:
        o.dequant = torch.empty((batch, groups, hd), dtype=torch.bfloat16, device=device)
    if rotated:
        o.rotated = torch.empty((batch, groups, hd), dtype=torch.bfloat16, device=device)
    return o
