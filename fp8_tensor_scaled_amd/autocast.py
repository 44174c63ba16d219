"""Scaling policy and autograd layer over the C-ABI.

The layer the pages put above their fp8 primitives (compare view
3e57cc8...main, astrai/extension/fp8.py: FP8Format, FP8Recipe, _ScaleRing,
FP8TensorMeta, FP8State, fp8_autocast, fp8_linear_forward, _LinearFp8):

* ``FP8Format``: E4M3, E5M2, or HYBRID (E4M3 forward, E5M2 gradients).
* ``FP8Recipe``: delayed scaling over an amax history of ``history_len``
  steps (the default), or dynamic (current-amax) scaling; ``margin`` divides
  the step by 2^margin.
* ``fp8_autocast``: a context (a ContextVar, so threads and nested regions
  each see their own) that turns the fp8 path on for ``fp8_linear`` /
  ``FP8Linear`` with a recipe and a format.
* Per-weight delayed-scaling state: one ring each for x, w and g, created on
  a weight's first fp8 use and kept as long as the weight lives.
* ``_LinearFp8``: forward and backward of ``y = x w^T + b`` for inputs of any
  leading shape [..., K], flattened to 2-D for the kernels.

Every number is computed in libfp8lin (``fp8_linear_fwd`` /
``fp8_linear_bwd`` under dynamic scaling; under delayed scaling the
forward's quantize and GEMM entry points, which read x and w once per step
and keep the backward's codes, and ``fp8_linear_bwd`` given those codes;
``fp8_quantize`` / ``fp8_mm`` for pre-quantized weights); this module only
keeps the rings, picks formats, allocates outputs and reshapes.  Inputs,
weights and biases are bf16.

Pre-quantized weights: a ``torch.float8_e4m3fn`` / ``torch.float8_e5m2``
weight is used as its codes with a step given by the caller (``w_scale``,
fp32 [1] on the device); it is not re-quantized, has no ring and gets no
gradient.  Its format must be the one the pass uses: the forward format,
and for an input gradient the backward format too (E4M3 weights train
under FP8Format.E4M3; under HYBRID only the forward is defined).  Such a
weight may come with an fp8 bias of the same format and its step
(``b_scale``), dequantized in the GEMM's epilogue, also without gradient.

The backward reads everything it needs from the forward's context, so it
runs in fp8 wherever ``backward()`` is called, inside the region or not.
"""

from __future__ import annotations

import contextvars
import dataclasses
import enum
import functools
import weakref

import torch

from . import (E4M3, E5M2, OUT_BF16, Ring, _linear_bwd_call, _linear_fwd_call, _stream,
               fp8_colsum, fp8_colsum_workspace,
               fp8_linear_bwd, fp8_linear_bwd_workspace, fp8_linear_bwd_workspace_codes,
               fp8_linear_fwd, fp8_linear_fwd_workspace, fp8_mm,
               fp8_mm_ex, fp8_quantize, fp8_quantize_colsum)

__all__ = ["FP8Format", "FP8Recipe", "FP8TensorMeta", "FP8State", "fp8_state", "fp8_autocast",
           "current_config", "fp8_linear", "FP8Linear", "fp8_linear_enable",
           "fp8_linear_enabled"]

_FP8_DTYPES = {torch.float8_e4m3fn: E4M3, torch.float8_e5m2: E5M2}


class FP8Format(str, enum.Enum):
    E4M3 = "e4m3"
    E5M2 = "e5m2"
    HYBRID = "hybrid"

    def fwd(self) -> int:
        """Format of the forward operands (x, w)."""
        return E5M2 if self is FP8Format.E5M2 else E4M3

    def bwd(self) -> int:
        """Format of the backward operands (g, and x, w re-quantized)."""
        return E4M3 if self is FP8Format.E4M3 else E5M2


@dataclasses.dataclass(frozen=True)
class FP8Recipe:
    """step = max(peak / FP8_MAX / 2^margin, 1e-12) with peak the max of the
    amax history (delayed) or the current amax (dynamic)."""
    history_len: int = 16
    margin: int = 0
    dynamic: bool = False

    def __post_init__(self):
        if not 1 <= self.history_len <= 4096:
            raise ValueError(f"history_len {self.history_len} outside [1, 4096]")
        if not 0 <= self.margin <= 64:
            raise ValueError(f"margin {self.margin} outside [0, 64]")


@dataclasses.dataclass(frozen=True)
class _Config:
    enabled: bool
    recipe: FP8Recipe
    fp8_format: FP8Format


class FP8TensorMeta:
    """Delayed-scaling rings of one weight's x, w and g operands."""
    __slots__ = ("recipe", "x", "w", "g")

    def __init__(self, device: torch.device, recipe: FP8Recipe):
        self.recipe = recipe
        self.x = Ring(recipe.history_len, device)
        self.w = Ring(recipe.history_len, device)
        self.g = Ring(recipe.history_len, device)


class FP8State:
    """Defaults that apply outside any fp8_autocast region, and the
    per-weight metas (held weakly: a meta lives as long as its weight)."""

    def __init__(self):
        self.default_enabled = False
        self.default_recipe = FP8Recipe()
        self.default_format = FP8Format.HYBRID
        # id(weight) -> (weak reference to the weight, meta); an entry leaves
        # when its weight is collected (tensors compare elementwise, so they
        # cannot be weak dictionary keys themselves)
        self._metas: dict = {}

    def get_weight_meta(self, w: torch.Tensor, recipe: FP8Recipe) -> FP8TensorMeta:
        key = id(w)
        entry = self._metas.get(key)
        meta = entry[1] if entry is not None and entry[0]() is w else None
        if meta is None or meta.recipe.history_len != recipe.history_len:
            meta = FP8TensorMeta(w.device, recipe)
            if entry is None or entry[0]() is not w:
                weakref.finalize(w, self._drop, key)
            self._metas[key] = (weakref.ref(w), meta)
        return meta

    def _drop(self, key: int) -> None:
        entry = self._metas.get(key)
        if entry is not None and entry[0]() is None:
            del self._metas[key]

    def reset(self) -> None:
        """Defaults back to their initial values; every meta dropped."""
        self.default_enabled = False
        self.default_recipe = FP8Recipe()
        self.default_format = FP8Format.HYBRID
        self._metas.clear()


_STATE = FP8State()
_ACTIVE: contextvars.ContextVar = contextvars.ContextVar("fp8_active_config", default=None)


def fp8_state() -> FP8State:
    return _STATE


def current_config() -> _Config:
    cfg = _ACTIVE.get()
    if cfg is not None:
        return cfg
    return _Config(_STATE.default_enabled, _STATE.default_recipe, _STATE.default_format)


class fp8_autocast:
    """``with fp8_autocast(enabled=True, recipe=FP8Recipe(), fp8_format=
    FP8Format.HYBRID):`` -- fp8_linear / FP8Linear inside use the fp8 path
    with that recipe and format; regions nest and restore on exit."""

    def __init__(self, enabled: bool = True, recipe: FP8Recipe | None = None,
                 fp8_format: FP8Format | str = FP8Format.HYBRID):
        self._cfg = _Config(bool(enabled), recipe if recipe is not None else FP8Recipe(),
                            FP8Format(fp8_format))
        self._tokens: list = []

    def __enter__(self):
        self._tokens.append(_ACTIVE.set(self._cfg))
        return self

    def __exit__(self, *exc):
        _ACTIVE.reset(self._tokens.pop())
        return False


# Linear workspaces.  Their control block starts at zero and every call
# leaves it so; the rest is scratch that a call uses only while its kernels
# run.  So one zero-filled buffer per (device, stream) serves every linear
# call on that stream, forward and backward, of any shape: it grows (a new
# zero-filled buffer replaces it) when a call needs more, and never holds
# more than the largest call on that stream asked for.  Calls on one stream
# are ordered, so they never use it at the same time.
_WS: dict = {}


@functools.lru_cache(maxsize=256)
def _ws_sizes(M: int, N: int, K: int) -> tuple:
    """(forward, backward, backward given the forward's codes) workspace
    bytes of a linear call shape."""
    return (fp8_linear_fwd_workspace(M, N, K), fp8_linear_bwd_workspace(M, N, K),
            fp8_linear_bwd_workspace_codes(M, N, K))


def _workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    key = (dev.index, _stream().value)  # the stream the library call will use
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)
        _WS[key] = ws
    return ws


def _bf16(t: torch.Tensor | None, what: str) -> torch.Tensor | None:
    if t is None:
        return None
    if t.dtype != torch.bfloat16:
        raise ValueError(f"fp8_linear: {what} must be bfloat16 (got {t.dtype})")
    return t.contiguous()


class _LinearFp8(torch.autograd.Function):
    """y[..., N] = x[..., K] w[N][K]^T + b and its gradients in fp8 ([CMP]
    fp8.py _LinearFp8).

    Dynamic scaling: fp8_linear_fwd / fp8_linear_bwd (the backward measures
    its own steps in the backward format, so it re-reads x and w).

    Delayed scaling: the same operations as those two entry points, bit for
    bit, in fewer passes.  The backward's x and w codes use the forward's
    steps, so the forward writes them from its own read of x and w
    (fp8_linear_fwd with x8_bwd / w8_bwd when the formats differ: x and w in
    one launch; under one format they are the forward codes) and keeps them
    -- one byte per element instead of bf16 x and w -- only when a gradient
    that needs them can follow.  The backward is fp8_linear_bwd given those
    codes: g quantized
    with its ring and the bias gradient's column sums from the same pass,
    then dX (NN) and dW (TN) in one paired launch that also finishes the
    bias gradient."""

    @staticmethod
    def forward(ctx, x, w, bias, cfg, grad_enabled):
        N, K = w.shape
        x2 = x.reshape(-1, K)
        M = x2.shape[0]
        dev = x.device
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        scales = torch.empty(2, dtype=torch.float32, device=dev)
        recipe, fmt = cfg.recipe, cfg.fp8_format.fwd()
        ctx.recipe, ctx.fmt_bwd = recipe, cfg.fp8_format.bwd()
        ctx.has_bias, ctx.x_shape, ctx.mnk = bias is not None, x.shape, (M, N, K)
        bias16 = None if bias is None else bias.view(torch.int16)
        if recipe.dynamic:
            ctx.meta = None
            # buffers sized from the operands here, so the unchecked call
            _linear_fwd_call(x2.view(torch.int16), w.view(torch.int16), bias16, M, N, K, fmt,
                             True, recipe.margin, None, None,
                             _workspace(dev, _ws_sizes(M, N, K)[0]), scales,
                             out.view(torch.int16), None, E5M2, None, None)
            ctx.save_for_backward(x2, w, scales)
            return out.reshape(*x.shape[:-1], N)
        meta = ctx.meta = _STATE.get_weight_meta(w, recipe)
        m = recipe.margin
        xi, wi = x2.view(torch.int16), w.view(torch.int16)
        # backward codes only when a backward can follow (grad mode on at the
        # call, and that input's gradient wanted)
        need_x = grad_enabled and ctx.needs_input_grad[0]
        need_w = grad_enabled and ctx.needs_input_grad[1]
        if ctx.fmt_bwd != fmt:
            # fp8_linear_fwd: x and w quantized in one launch, each writing
            # its backward codes (other format, same step) when they are
            # wanted; it seeds, folds and advances the rings
            x8b = torch.empty(M * K, dtype=torch.uint8, device=dev) if need_w else None
            w8b = torch.empty(N * K, dtype=torch.uint8, device=dev) if need_x else None
            _linear_fwd_call(xi, wi, bias16, M, N, K, fmt, False, m, meta.x, meta.w,
                             _workspace(dev, _ws_sizes(M, N, K)[0]), scales,
                             out.view(torch.int16), None, ctx.fmt_bwd, x8b, w8b)
            ctx.save_for_backward(x8b, w8b, scales)
            return out.reshape(*x.shape[:-1], N)
        # one format both ways: the forward's codes are the backward's
        for ring, t in ((meta.x, xi), (meta.w, wi)):
            if not ring.initialized:  # first use: the ring starts from this tensor's amax
                fp8_quantize(t, fmt, ring=ring, margin=m)
                ring.initialized = True
        x8 = torch.empty(M * K, dtype=torch.uint8, device=dev)
        w8 = torch.empty(N * K, dtype=torch.uint8, device=dev)
        fp8_quantize(xi, fmt, scale=meta.x.scale, out=x8, ring=meta.x, margin=m,
                     scale_used=scales[0:1])
        fp8_quantize(wi, fmt, scale=meta.w.scale, out=w8, ring=meta.w, margin=m,
                     scale_used=scales[1:2])
        fp8_mm(x8, w8, fmt, 0, 1, M, N, K, K, K, 1, 0, 0, scales[0:1], scales[1:2], bias16,
               out.view(torch.int16))
        for ring in (meta.x, meta.w):
            ring.idx = (ring.idx + 1) % ring.len
        ctx.save_for_backward(x8 if need_w else None, w8 if need_x else None, scales)
        return out.reshape(*x.shape[:-1], N)

    @staticmethod
    def backward(ctx, g):
        M, N, K = ctx.mnk
        g2 = _bf16(g.reshape(-1, N), "the output gradient")
        need_x, need_w, need_b = ctx.needs_input_grad[:3]
        dev = g.device
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if need_x else None
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev) if need_w else None
        db = torch.empty(N, dtype=torch.bfloat16, device=dev) if need_b and ctx.has_bias else None
        if dx is None and dw is None and db is None:
            return None, None, None, None, None
        i16 = (lambda t: None if t is None else t.view(torch.int16))
        fmt, m = ctx.fmt_bwd, ctx.recipe.margin
        if ctx.meta is None:
            x2, w, scales = ctx.saved_tensors
            _linear_bwd_call(i16(g2), i16(x2), i16(w), M, N, K, fmt, True, m, scales, None,
                             _workspace(dev, _ws_sizes(M, N, K)[1]), None, i16(dx), i16(dw),
                             i16(db), None, None, None)
        else:
            # the forward kept x8b when dW is wanted and w8b when dX is; the
            # call seeds, uses and advances the g ring
            x8b, w8b, scales = ctx.saved_tensors
            _linear_bwd_call(i16(g2), None, None, M, N, K, fmt, False, m, scales, ctx.meta.g,
                             _workspace(dev, _ws_sizes(M, N, K)[2]), None,
                             i16(dx), i16(dw), i16(db), None,
                             x8b if dw is not None else None,
                             w8b if dx is not None else None)
        return (None if dx is None else dx.reshape(ctx.x_shape), dw, db, None, None)


class _LinearFp8Weight(torch.autograd.Function):
    """y = x w8^T * (sx * sw) + b with a pre-quantized weight (codes and a
    caller-given step): x is quantized (ring or dynamic), the weight is
    used as is ([CMP] fp8.py fp8_linear_forward, the fp8-weight branch)."""

    @staticmethod
    def forward(ctx, x, w8, w_scale, bias, b_scale, cfg):
        N, K = w8.shape
        fmt = _FP8_DTYPES[w8.dtype]
        if fmt != cfg.fp8_format.fwd():
            raise ValueError("fp8_linear: the weight's fp8 format is not the forward format")
        bias8 = bias is not None and bias.dtype in _FP8_DTYPES
        if bias8 and _FP8_DTYPES[bias.dtype] != fmt:
            raise ValueError("fp8_linear: an fp8 bias must be in the weight's format")
        x2 = x.reshape(-1, K)
        M = x2.shape[0]
        dev = x.device
        x8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sx = torch.empty(1, dtype=torch.float32, device=dev)
        recipe = cfg.recipe
        if recipe.dynamic:
            scratch = Ring(1, dev)
            fp8_quantize(x2.view(torch.int16), fmt, ring=scratch, margin=recipe.margin)
            fp8_quantize(x2.view(torch.int16), fmt, scale=scratch.scale, out=x8,
                         scale_used=sx)
        else:
            ring = _STATE.get_weight_meta(w8, recipe).x
            if not ring.initialized:
                fp8_quantize(x2.view(torch.int16), fmt, ring=ring, margin=recipe.margin)
                ring.initialized = True
            fp8_quantize(x2.view(torch.int16), fmt, scale=ring.scale, out=x8, ring=ring,
                         margin=recipe.margin, scale_used=sx)
            ring.idx = (ring.idx + 1) % ring.len
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if bias8:  # fp8 bias codes and their step, dequantized in the epilogue
            fp8_mm_ex(x8, w8.view(torch.uint8), fmt, 0, 1, M, N, K, K, K, 1, 0, 0, sx, w_scale,
                      bias.view(torch.uint8), b_scale, OUT_BF16, None, out.view(torch.int16))
        else:
            fp8_mm(x8, w8.view(torch.uint8), fmt, 0, 1, M, N, K, K, K, 1, 0, 0, sx, w_scale,
                   None if bias is None else bias.view(torch.int16), out.view(torch.int16))
        ctx.save_for_backward(w8, w_scale)
        # a pre-quantized bias, like the weight, takes no gradient
        ctx.recipe, ctx.fmt_bwd = recipe, cfg.fp8_format.bwd()
        ctx.has_bias = bias is not None and not bias8
        ctx.x_shape = x.shape
        return out.reshape(*x.shape[:-1], N)

    @staticmethod
    def backward(ctx, g):
        w8, w_scale = ctx.saved_tensors
        N, K = w8.shape
        g2 = _bf16(g.reshape(-1, N), "the output gradient")
        M = g2.shape[0]
        dev = g.device
        dx = db = None
        gi = g2.view(torch.int16)
        if ctx.needs_input_grad[3] and ctx.has_bias:
            db = torch.empty(N, dtype=torch.bfloat16, device=dev)
            cs_ws = torch.empty(fp8_colsum_workspace(M, N), dtype=torch.uint8, device=dev)
        if ctx.needs_input_grad[0]:
            fmt = ctx.fmt_bwd
            if fmt != _FP8_DTYPES[w8.dtype]:
                raise NotImplementedError(
                    "fp8_linear: an input gradient through a pre-quantized weight needs the "
                    "weight in the backward format (use FP8Format.E4M3 for E4M3 weights)")
            scratch = Ring(1, dev)
            g8 = torch.empty((M, N), dtype=torch.uint8, device=dev)
            sg = torch.empty(1, dtype=torch.float32, device=dev)
            fp8_quantize(gi, fmt, ring=scratch, margin=ctx.recipe.margin)
            if db is not None:  # the codes and the bias gradient from one read of g
                fp8_quantize_colsum(gi, M, N, fmt, scratch.scale, g8, db.view(torch.int16),
                                    cs_ws, scale_used=sg)
            else:
                fp8_quantize(gi, fmt, scale=scratch.scale, out=g8, scale_used=sg)
            dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            # dX[M][K] = g8[M][N] . w8[N][K]  (NN)
            fp8_mm(g8, w8.view(torch.uint8), fmt, 0, 0, M, K, N, N, K, 1, 0, 0, sg, w_scale,
                   None, dx.view(torch.int16))
            dx = dx.reshape(ctx.x_shape)
        elif db is not None:
            fp8_colsum(gi, M, N, db.view(torch.int16), cs_ws)
        return dx, None, None, db, None, None


def fp8_linear(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
               w_scale: torch.Tensor | None = None,
               b_scale: torch.Tensor | None = None) -> torch.Tensor:
    """``F.linear`` with the fp8 path when an fp8_autocast region (or the
    default switch) enables it.  w: bf16 [N][K], or fp8 codes [N][K] with
    their step ``w_scale`` (fp32 [1], device).  With fp8 weight codes the
    bias may be fp8 codes [N] of the same format with their step
    ``b_scale`` ([LOG1] bias_scale), dequantized in the GEMM's epilogue."""
    cfg = current_config()
    if w.dim() != 2 or x.dim() < 1 or x.shape[-1] != w.shape[1]:
        raise ValueError(f"fp8_linear: input of shape {tuple(x.shape)} and weight of shape "
                         f"{tuple(w.shape)} do not match")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != w.shape[0]):
        raise ValueError(f"fp8_linear: bias of shape {tuple(bias.shape)} for {w.shape[0]} "
                         "outputs")
    bias8 = bias is not None and bias.dtype in _FP8_DTYPES
    if bias8 and (w.dtype not in _FP8_DTYPES or b_scale is None):
        raise ValueError("fp8_linear: an fp8 bias needs fp8 weight codes and b_scale")
    if w.dtype in _FP8_DTYPES:
        if w_scale is None:
            raise ValueError("fp8_linear: a pre-quantized weight needs w_scale")
        if not cfg.enabled:
            raise ValueError("fp8_linear: a pre-quantized weight needs the fp8 path enabled")
        return _LinearFp8Weight.apply(_bf16(x, "x"), w, w_scale,
                                      bias if bias8 else _bf16(bias, "bias"), b_scale, cfg)
    if not cfg.enabled:
        return torch.nn.functional.linear(x, w, bias)
    return _LinearFp8.apply(_bf16(x, "x"), _bf16(w, "w"), _bf16(bias, "bias"), cfg,
                            torch.is_grad_enabled())


class FP8Linear(torch.nn.Linear):
    """nn.Linear whose forward takes the fp8 path inside fp8_autocast."""

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return fp8_linear(x, self.weight, self.bias)


# --------------------------------------------------------------------------
# Routing of torch's own linear (nn.Linear, F.linear) -- opt in
# --------------------------------------------------------------------------
#
# The pages register their fp8 linear as the aten::linear kernel of CUDA
# tensors, on the autograd key (training and no_grad) and on the CUDA key
# (inference_mode, where the autograd keys are skipped), so that existing
# models need no module swap (compare view 3e57cc8...main, commit log of
# astrai/extension: the _LinearFp8 registration).  fp8_linear_enable() does
# the same with torch.library, as an explicit switch: while it is on, every
# aten::linear call on CUDA tensors comes here; the fp8 path runs when an
# fp8_autocast region (or the default switch) enables it and the operands are
# bf16, and every other call runs torch's own decomposition of linear.

_ROUTE_LIB = None


def _plain_linear(x, w, b):
    """torch's decomposition of aten::linear (addmm for 2-D inputs, and for
    contiguous 3-D inputs with a bias; else matmul, then the bias)."""
    if b is not None and x.dim() == 2:
        return torch.addmm(b, x, w.t())
    if b is not None and x.dim() == 3 and x.is_contiguous():
        out = torch.addmm(b, x.reshape(-1, x.shape[-1]), w.t())
        return out.view(*x.shape[:-1], w.shape[0])
    out = torch.matmul(x, w.t())
    return out if b is None else out + b


def _routed_linear(x, w, b=None):
    if (current_config().enabled and x.dtype == torch.bfloat16 and w.dtype == torch.bfloat16
            and (b is None or b.dtype == torch.bfloat16) and x.dim() >= 1 and w.dim() == 2):
        return fp8_linear(x, w, b)
    return _plain_linear(x, w, b)


def fp8_linear_enable(enabled: bool = True) -> None:
    """Route torch's linear on CUDA tensors (nn.Linear, F.linear) through
    fp8_linear (True), or give it back to torch (False).  With the routing on,
    a stock nn.Linear takes the fp8 path inside fp8_autocast exactly as
    FP8Linear does, and torch's own computation outside it."""
    global _ROUTE_LIB
    if enabled and _ROUTE_LIB is None:
        lib = torch.library.Library("aten", "IMPL")
        lib.impl("linear", _routed_linear, "AutogradCUDA")
        lib.impl("linear", _routed_linear, "CUDA")
        _ROUTE_LIB = lib
    elif not enabled and _ROUTE_LIB is not None:
        _ROUTE_LIB._destroy()
        _ROUTE_LIB = None


def fp8_linear_enabled() -> bool:
    """Whether torch's linear is routed here (fp8_linear_enable)."""
    return _ROUTE_LIB is not None
