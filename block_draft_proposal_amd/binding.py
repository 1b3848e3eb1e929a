"""Thin Python binding of libdflash.so (argument marshalling only).

Every function has the name of the C entry point it calls, takes torch
tensors that already live on the GPU, passes their device pointers and the
current HIP stream, and returns the output tensors it allocated with torch.
No step of the computation runs here: if the library is missing, importing
this module's functions raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np
import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libdflash.so")

DFLASH_OK = 0
DFLASH_ERR_INVALID_ARG = -1
DFLASH_ERR_UNSUPPORTED = -2
DFLASH_ERR_WORKSPACE = -3
DFLASH_ERR_LAUNCH = -4
DFLASH_F32 = 0
DFLASH_BF16 = 1
MAX_TOP_K = 32

_c_i32, _c_i64, _c_f32, _c_size, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class DraftConfig(ctypes.Structure):
    """Mirror of dflash_draft_config."""
    _fields_ = [
        ("conv_kernel_size", _c_i32),
        ("conv_group_size", _c_i32),
        ("selector_rank", _c_i32),
        ("selector_top_k", _c_i32),
        ("output_multiplier", _c_f32),
        ("final_logit_softcapping", _c_f32),
        ("block_size", _c_i32),
        ("hidden_size", _c_i32),
    ]


class BlockArgs(ctypes.Structure):
    """Mirror of dflash_block_args."""
    _fields_ = [
        ("x", _c_vp), ("conv_base", _c_vp), ("conv_delta", _c_vp), ("delta_row_stride", _c_i64),
        ("logits", _c_vp), ("logits_row_stride", _c_i64), ("vocab", _c_i64), ("valid_vocab", _c_i64),
        ("anchor_ids", _c_vp), ("sel_a", _c_vp), ("sel_b", _c_vp), ("proj", _c_vp),
        ("uniforms", _c_vp), ("temperatures", _c_vp), ("greedy_mask", _c_vp),
        ("conv_out", _c_vp), ("ids_out", _c_vp), ("unary_out", _c_vp), ("tokens_out", _c_vp),
        ("q_out", _c_vp), ("scores_out", _c_vp),
        ("workspace", _c_vp), ("workspace_bytes", _c_size),
        ("stage_events", _c_vp),
        ("n_req", _c_i32), ("dtype", _c_i32),
    ]


_SIGNATURES = {
    "dflash_abi_version": (_c_i32, []),
    "dflash_validate_config": (_c_i32, [ctypes.POINTER(DraftConfig)]),
    "dflash_last_error": (ctypes.c_char_p, []),
    "dflash_conv": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i64, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp]),
    "dflash_conv_prepare_workspace_size": (_c_size, [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32]),
    "dflash_conv_prepare": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                     _c_i32, _c_vp, _c_size, _c_vp]),
    "dflash_philox_uniforms": (_c_i32, [_c_vp, _c_i64, _c_vp, _c_vp]),
    "dflash_hbm_ceiling": (_c_i32, [_c_i32, _c_vp, _c_vp, _c_i64, _c_vp]),
    "dflash_verify_workspace_size": (_c_size, [_c_i32, _c_i32, _c_i64]),
    "dflash_verify": (_c_i32, [_c_vp, _c_i64, _c_i32, _c_i32, _c_i64, _c_i64, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp,
                               _c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "dflash_topk_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i32]),
    "dflash_topk": (_c_i32, [_c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i32, _c_f32, _c_f32, _c_i32, _c_vp, _c_vp,
                             _c_vp, _c_size, _c_vp]),
    "dflash_lattice_workspace_size": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "dflash_lattice": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32,
                                _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_vp, _c_vp, _c_size, _c_vp]),
    "dflash_walk": (_c_i32, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp]),
    "dflash_lm_head": (_c_i32, [_c_vp, _c_i64, _c_vp, _c_i64, _c_i32, _c_i64, _c_vp, _c_i64, _c_i32, _c_vp]),
    "dflash_lm_head_topk_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i32]),
    "dflash_lm_head_topk": (_c_i32, [_c_vp, _c_i64, _c_vp, _c_i64, _c_i32, _c_i64, _c_i64, _c_i32, _c_f32, _c_f32,
                                     _c_i32, _c_vp, _c_vp, _c_vp, _c_size, _c_vp]),
    "dflash_propose_block_workspace_size": (_c_size, [ctypes.POINTER(DraftConfig), _c_i32, _c_i64]),
    "dflash_propose_block": (_c_i32, [ctypes.POINTER(DraftConfig), ctypes.POINTER(BlockArgs), _c_vp]),
    "dflash_propose_block_noalloc": (_c_i32, [ctypes.POINTER(DraftConfig), ctypes.POINTER(BlockArgs), _c_vp]),
    "dflash_propose_block_schedule": (_c_i32, [ctypes.POINTER(DraftConfig), _c_i32, _c_i32]),
}
EXPORTED = tuple(_SIGNATURES)

_lib = None


class DFlashError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libdflash.so (built in-tree by ``block_draft_proposal_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_draft_proposal_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().dflash_last_error().decode()


def _check(status: int) -> None:
    if status != DFLASH_OK:
        raise DFlashError(status, last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DFLASH_BF16
    if t.dtype == torch.float32:
        return DFLASH_F32
    raise TypeError(f"unsupported float dtype {t.dtype}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need_inner_contiguous(t: torch.Tensor, name: str):
    if t.dim() > 1 and t.shape[0] > 0 and not t[0].is_contiguous():
        raise ValueError(f"{name}: every row must be contiguous")


def make_config(*, taps: int, group_size: int, rank: int, top_k: int, multiplier: float = 1.0,
                softcap: float = 0.0, block_size: int, hidden: int) -> DraftConfig:
    return DraftConfig(taps, group_size, rank, top_k, multiplier, softcap, block_size, hidden)


def dflash_validate_config(cfg: DraftConfig) -> None:
    _check(lib().dflash_validate_config(ctypes.byref(cfg)))


def dflash_conv(x: torch.Tensor, base: torch.Tensor, delta: torch.Tensor, *, block_size: int,
                group_size: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """x [N, H]; base [T, H]; delta [N, T, G] (rows may be strided, e.g. one
    side of a packed [N, 2, T, G] projection).  Returns out [N, H]."""
    if not (x.is_contiguous() and base.is_contiguous()):
        raise ValueError("x and base must be contiguous")
    _need_inner_contiguous(delta, "delta")
    N, H = x.shape
    T = base.shape[0]
    if out is None:
        out = torch.empty_like(x)
    _check(lib().dflash_conv(_p(x), _p(base), _p(delta), delta.stride(0) if N else T * (H // group_size), _p(out),
                             N, H, group_size, T, block_size, _dtype_code(x), _stream(stream)))
    return out


def dflash_conv_prepare(x: torch.Tensor, proj_weight: torch.Tensor, base2: torch.Tensor, *, block_size: int,
                        group_size: int, out: Optional[torch.Tensor] = None, coeff_out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """x [N, H]; proj_weight [2*T*G, H]; base2 [2, T, H].  Returns (out [N, H]:
    x convolved with side 0, coeff [N, 2, T, G]: both sides' coefficients).
    finish is dflash_conv(y, base2[1], coeff[:, 1], ...)."""
    if not (x.is_contiguous() and proj_weight.is_contiguous() and base2.is_contiguous()):
        raise ValueError("x, proj_weight and base2 must be contiguous")
    N, H = x.shape
    T = base2.shape[1]
    G = H // group_size
    if out is None:
        out = torch.empty_like(x)
    if coeff_out is None:
        coeff_out = torch.empty((N, 2, T, G), dtype=x.dtype, device=x.device)
    if workspace is None:
        nbytes = lib().dflash_conv_prepare_workspace_size(N, H, group_size, T, _dtype_code(x))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib().dflash_conv_prepare(_p(x), _p(proj_weight), _p(base2), _p(out), _p(coeff_out), N, H, group_size, T,
                                     block_size, _dtype_code(x), _p(workspace), workspace.numel(), _stream(stream)))
    return out, coeff_out


def dflash_verify(target_logits: torch.Tensor, cand_ids: torch.Tensor, q: torch.Tensor, tokens: torch.Tensor,
                  u_accept: torch.Tensor, u_residual: torch.Tensor, temperatures: torch.Tensor,
                  greedy_mask: torch.Tensor, *, valid_vocab: Optional[int] = None, accepted_out=None,
                  committed_out=None, workspace=None, stream=None):
    """target_logits [R, S+1, V] (rows contiguous); cand_ids / q [R, S, K];
    tokens / u_accept [R, S]; u_residual, temperatures, greedy_mask [R].
    Returns (accepted int32 [R], committed int64 [R, S+1])."""
    R, S1, V = target_logits.shape
    S = S1 - 1
    K = cand_ids.shape[-1] if cand_ids.numel() else 1
    if target_logits.dim() != 3 or target_logits.stride(2) != 1 or \
            (R and S1 > 1 and target_logits.stride(0) != S1 * target_logits.stride(1)):
        raise ValueError("target_logits must be [R, S+1, V] rows of one row stride")
    valid_vocab = V if valid_vocab is None else valid_vocab
    dev = target_logits.device
    accepted_out = torch.empty(R, dtype=torch.int32, device=dev) if accepted_out is None else accepted_out
    committed_out = torch.empty((R, S1), dtype=torch.int64, device=dev) if committed_out is None else committed_out
    if workspace is None:
        workspace = torch.empty(max(1, lib().dflash_verify_workspace_size(R, S, valid_vocab)), dtype=torch.uint8, device=dev)
    for t, name in ((cand_ids, "cand_ids"), (q, "q"), (tokens, "tokens"), (u_accept, "u_accept"),
                    (u_residual, "u_residual"), (temperatures, "temperatures"), (greedy_mask, "greedy_mask")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _check(lib().dflash_verify(_p(target_logits), target_logits.stride(1) if R else V, R, S, V, valid_vocab, K,
                               _p(cand_ids), _p(q), _p(tokens), _p(u_accept), _p(u_residual), _p(temperatures),
                               _p(greedy_mask), _dtype_code(target_logits), _p(accepted_out), _p(committed_out),
                               _p(workspace), workspace.numel(), _stream(stream)))
    return accepted_out, committed_out


def dflash_topk(logits: torch.Tensor, *, top_k: int, valid_vocab: Optional[int] = None,
                multiplier: float = 1.0, softcap: float = 0.0, vocab: Optional[int] = None,
                ids_out=None, unary_out=None, workspace=None, stream=None):
    """logits [rows, >= vocab] (row stride = logits.stride(0)).  Returns
    (ids int64 [rows, K], unary fp32 [rows, K])."""
    rows = logits.shape[0]
    vocab = logits.shape[1] if vocab is None else vocab
    valid_vocab = vocab if valid_vocab is None else valid_vocab
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [rows, V] with contiguous rows")
    dev = logits.device
    ids_out = torch.empty((rows, top_k), dtype=torch.int64, device=dev) if ids_out is None else ids_out
    unary_out = torch.empty((rows, top_k), dtype=torch.float32, device=dev) if unary_out is None else unary_out
    ws_bytes = lib().dflash_topk_workspace_size(rows, valid_vocab, top_k)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().dflash_topk(_p(logits), logits.stride(0), rows, vocab, valid_vocab, top_k, multiplier, softcap,
                             _dtype_code(logits), _p(ids_out), _p(unary_out), _p(workspace),
                             workspace.numel(), _stream(stream)))
    return ids_out, unary_out


def dflash_lattice(ids: torch.Tensor, unary: torch.Tensor, hidden: torch.Tensor, anchor: torch.Tensor,
                   sel_a: torch.Tensor, sel_b: torch.Tensor, proj: torch.Tensor, *, scores_out=None,
                   workspace=None, stream=None) -> torch.Tensor:
    """ids, unary [R, S, K]; hidden [R, S, H] (strided views allowed, rows
    contiguous); anchor [R]; sel_a, sel_b [V, r]; proj [r, H].
    Returns scores fp32 [R, S, K, K]."""
    R, S, K = ids.shape
    H = hidden.shape[-1]
    r = proj.shape[0]
    if hidden.stride(-1) != 1:
        raise ValueError("hidden rows must be contiguous")
    for t, n in ((ids, "ids"), (unary, "unary"), (anchor, "anchor"), (sel_a, "sel_a"), (sel_b, "sel_b"),
                 (proj, "proj")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    dev = ids.device
    scores_out = torch.empty((R, S, K, K), dtype=torch.float32, device=dev) if scores_out is None else scores_out
    ws_bytes = lib().dflash_lattice_workspace_size(R, S, r, H)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().dflash_lattice(_p(ids), _p(unary), _p(hidden), hidden.stride(0), hidden.stride(1), _p(anchor),
                                _p(sel_a), _p(sel_b), _p(proj), R, S, K, H, r, sel_a.shape[0],
                                _dtype_code(hidden), _p(scores_out), _p(workspace), workspace.numel(),
                                _stream(stream)))
    return scores_out


def dflash_walk(scores: torch.Tensor, ids: torch.Tensor, uniforms: torch.Tensor, temperatures: torch.Tensor,
                greedy_mask: torch.Tensor, *, tokens_out=None, q_out=None, stream=None):
    """scores [R, S, K, K] fp32; ids [R, S, K]; uniforms [R, S]; temperatures
    [R]; greedy_mask [R] bool/uint8.  Returns (tokens int64 [R, S], q fp32 [R, S, K])."""
    R, S, K = ids.shape
    for t, n in ((scores, "scores"), (ids, "ids"), (uniforms, "uniforms"), (temperatures, "temperatures"),
                 (greedy_mask, "greedy_mask")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if greedy_mask.element_size() != 1:
        raise TypeError("greedy_mask must be bool or uint8")
    dev = ids.device
    tokens_out = torch.empty((R, S), dtype=torch.int64, device=dev) if tokens_out is None else tokens_out
    q_out = torch.empty((R, S, K), dtype=torch.float32, device=dev) if q_out is None else q_out
    _check(lib().dflash_walk(_p(scores), _p(ids), _p(uniforms), _p(temperatures), _p(greedy_mask), R, S, K,
                             _p(tokens_out), _p(q_out), _stream(stream)))
    return tokens_out, q_out


def dflash_lm_head(hidden: torch.Tensor, weight: torch.Tensor, *, vocab: Optional[int] = None,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """hidden [rows, H] bf16 (rows may be strided); weight [V, H] bf16.
    Returns logits [rows, V] bf16 = hidden @ weight.T rounded once."""
    if hidden.dim() != 2 or hidden.stride(1) != 1 or not weight.is_contiguous():
        raise ValueError("hidden rows and weight must be contiguous")
    rows, H = hidden.shape
    V = weight.shape[0] if vocab is None else vocab
    if out is None:
        out = torch.empty((rows, V), dtype=hidden.dtype, device=hidden.device)
    _check(lib().dflash_lm_head(_p(hidden), hidden.stride(0) if rows else H, _p(weight), rows, H, V, _p(out),
                                out.stride(0) if rows else V, _dtype_code(hidden), _stream(stream)))
    return out


def dflash_lm_head_topk(hidden: torch.Tensor, weight: torch.Tensor, *, top_k: int,
                        valid_vocab: Optional[int] = None, multiplier: float = 1.0, softcap: float = 0.0,
                        ids_out=None, unary_out=None, workspace=None, stream=None):
    """hidden [rows, H] bf16 (rows may be strided); weight [V, H] bf16.
    Returns (ids int64 [rows, K], unary fp32 [rows, K]) of the head's
    logits, without materialising them."""
    if hidden.dim() != 2 or hidden.stride(1) != 1 or not weight.is_contiguous():
        raise ValueError("hidden rows and weight must be contiguous")
    rows, H = hidden.shape
    V = weight.shape[0]
    valid_vocab = V if valid_vocab is None else valid_vocab
    dev = hidden.device
    ids_out = torch.empty((rows, top_k), dtype=torch.int64, device=dev) if ids_out is None else ids_out
    unary_out = torch.empty((rows, top_k), dtype=torch.float32, device=dev) if unary_out is None else unary_out
    if workspace is None:
        nbytes = lib().dflash_lm_head_topk_workspace_size(rows, V, top_k)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().dflash_lm_head_topk(_p(hidden), hidden.stride(0) if rows else H, _p(weight), rows, H, V,
                                     valid_vocab, top_k, multiplier, softcap, _dtype_code(hidden), _p(ids_out),
                                     _p(unary_out), _p(workspace), workspace.numel(), _stream(stream)))
    return ids_out, unary_out


def propose_block_workspace_size(cfg: DraftConfig, n_req: int, valid_vocab: int) -> int:
    return lib().dflash_propose_block_workspace_size(ctypes.byref(cfg), n_req, valid_vocab)


SCHEDULE_ONE_LAUNCH = 1    # conv + projection inside the top-K's launch
SCHEDULE_AUX_STREAM = 2    # conv then projection on the auxiliary stream beside the top-K


def propose_block_schedule(cfg: DraftConfig, n_req: int, dtype: str) -> int:
    """The schedule dflash_propose_block takes for this config, batch and
    dtype ("bf16" or "f32"): SCHEDULE_ONE_LAUNCH or SCHEDULE_AUX_STREAM."""
    code = {"f32": 0, "bf16": 1}[dtype]
    got = lib().dflash_propose_block_schedule(ctypes.byref(cfg), n_req, code)
    if got == 0:
        raise DFlashError(DFLASH_ERR_INVALID_ARG, last_error() or "dflash_propose_block_schedule: rejected shape")
    return got


class ProposeBlock:
    """Marshalled arguments of dflash_propose_block on one fixed set of
    buffers: built once, then each call only hands the prepared struct to the
    library (what a serving loop whose buffers stay put does every step).
    Inputs as for dflash_propose_block; the outputs dict and the workspace are
    allocated here unless given, and are rewritten by every call.  noalloc:
    call dflash_propose_block_noalloc instead (no workspace: the library's
    own scratch; the call itself allocates nothing)."""

    def __init__(self, cfg: DraftConfig, *, x, conv_base, conv_delta, logits, anchor, sel_a, sel_b, proj,
                 uniforms, temperatures, greedy_mask, valid_vocab: Optional[int] = None,
                 vocab: Optional[int] = None, keep_scores: bool = False,
                 outputs: Optional[Dict[str, torch.Tensor]] = None, workspace=None, noalloc: bool = False):
        B, K = cfg.block_size, cfg.selector_top_k
        S = B - 1
        N = x.shape[0]
        R = N // B
        vocab = logits.shape[1] if vocab is None else vocab
        valid_vocab = vocab if valid_vocab is None else valid_vocab
        dev = x.device
        _need_inner_contiguous(conv_delta, "conv_delta")
        if logits.stride(-1) != 1:
            raise ValueError("logits rows must be contiguous")
        o = dict(outputs or {})
        shapes = {"conv_out": (tuple(x.shape), x.dtype), "ids": ((R, S, K), torch.int64),
                  "unary": ((R, S, K), torch.float32), "tokens": ((R, S), torch.int64),
                  "q": ((R, S, K), torch.float32)}
        if keep_scores:
            shapes["scores"] = ((R, S, K, K), torch.float32)
        for k, (shape, dt) in shapes.items():
            if k not in o:
                o[k] = torch.empty(shape, dtype=dt, device=dev)
        if noalloc:
            workspace = None                 # the library's own scratch (dflash_propose_block_noalloc)
        elif workspace is None:
            nbytes = propose_block_workspace_size(cfg, max(R, 1), valid_vocab)
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        self.outputs = o
        # the struct holds raw pointers: keep every tensor it names alive
        self._keep = (x, conv_base, conv_delta, logits, anchor, sel_a, sel_b, proj, uniforms, temperatures,
                      greedy_mask, workspace)
        self._ev = None
        self._cfg = cfg
        self._args = BlockArgs(
            _p(x), _p(conv_base), _p(conv_delta), conv_delta.stride(0),
            _p(logits), logits.stride(0), vocab, valid_vocab,
            _p(anchor), _p(sel_a), _p(sel_b), _p(proj),
            _p(uniforms), _p(temperatures), _p(greedy_mask),
            _p(o["conv_out"]), _p(o["ids"]), _p(o["unary"]), _p(o["tokens"]), _p(o["q"]), _p(o.get("scores")),
            _p(workspace), 0 if workspace is None else workspace.numel(), None, R, _dtype_code(x))
        self._cfg_ref = ctypes.byref(cfg)
        self._args_ref = ctypes.byref(self._args)
        self._fn = lib().dflash_propose_block_noalloc if noalloc else lib().dflash_propose_block

    @staticmethod
    def event_array(stage_events: Sequence):
        """8 entries (torch.cuda.Event or None: that record is skipped) as the
        host array dflash_block_args.stage_events points to."""
        return (ctypes.c_void_p * 8)(*[None if e is None else e.cuda_event for e in stage_events])

    def __call__(self, stream_handle=None, stage_events=None) -> Dict[str, torch.Tensor]:
        """stream_handle: a raw HIP stream (``torch.cuda.Stream.cuda_stream``)
        or None for torch's current stream; stage_events: None or an array
        from ``event_array``."""
        if stream_handle is None:
            stream_handle = torch.cuda.current_stream().cuda_stream
        if stage_events is not self._ev:
            self._ev = stage_events
            self._args.stage_events = None if stage_events is None else ctypes.cast(stage_events, ctypes.c_void_p)
        st = self._fn(self._cfg_ref, self._args_ref, stream_handle)
        if st != DFLASH_OK:
            raise DFlashError(st, last_error())
        return self.outputs


def dflash_philox_uniforms(seed_offset: torch.Tensor, n: int, *, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """seed_offset: device int64 [2] = {seed, offset} (read as unsigned by the
    kernel).  Returns out fp32 [n]: Philox-4x32-10 uniforms in [0, 1)."""
    if seed_offset.numel() != 2 or seed_offset.dtype != torch.int64 or not seed_offset.is_contiguous():
        raise ValueError("seed_offset must be a contiguous int64 tensor of 2 elements")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=seed_offset.device)
    _check(lib().dflash_philox_uniforms(_p(seed_offset), n, _p(out), _stream(stream)))
    return out


CEILING_READ, CEILING_COPY = 0, 1


def dflash_hbm_ceiling(kind: int, src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Measurement support: streams src's bytes (kind CEILING_READ, dst a
    4-byte sink) or copies them into dst (CEILING_COPY) with the path's
    streaming load and store forms."""
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    nbytes = src.numel() * src.element_size()
    if kind == CEILING_COPY and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    if kind == CEILING_READ and dst.numel() * dst.element_size() < 4:
        raise ValueError("the read sink needs 4 bytes")
    _check(lib().dflash_hbm_ceiling(kind, _p(src), _p(dst), nbytes, _stream(stream)))


_hip_rt = None


def _hip():
    """The HIP runtime (for the staging copy and its event in ProposeGraph)."""
    global _hip_rt
    if _hip_rt is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipMemcpyAsync.argtypes = [_c_vp, _c_vp, _c_size, ctypes.c_int, _c_vp]
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_c_vp), ctypes.c_uint]
        h.hipEventRecord.argtypes = [_c_vp, _c_vp]
        h.hipEventSynchronize.argtypes = [_c_vp]
        _hip_rt = h
    return _hip_rt


def _as_i64(v: int) -> int:
    """An unsigned 64-bit value as the int64 with the same bits."""
    v &= (1 << 64) - 1
    return v - (1 << 64) if v >= 1 << 63 else v


class ProposeGraph:
    """One draft step captured as a HIP graph: the walk's uniforms drawn in the
    graph by dflash_philox_uniforms from a staged {seed, offset}, then
    dflash_propose_block (its auxiliary-stream branch captured through the
    library's fork/join events).  Temperatures, the greedy mask and {seed,
    offset} live in device buffers the graph reads; replay() stages new host
    values into them on the stream (outside the graph) and replays, so one
    graph serves greedy and sampled requests alike.  The other inputs are
    fixed buffers (as for ProposeBlock); the outputs are rewritten by every
    replay."""

    def __init__(self, cfg: DraftConfig, *, x, conv_base, conv_delta, logits, anchor, sel_a, sel_b, proj,
                 valid_vocab: Optional[int] = None, vocab: Optional[int] = None):
        B = cfg.block_size
        R, S = x.shape[0] // B, B - 1
        dev = x.device
        self.n = R * S
        self.uniforms = torch.empty((R, S), dtype=torch.float32, device=dev)
        # everything staged per replay in one buffer (one copy): {seed, offset}
        # (16 bytes), temperatures (4 R), greedy mask (R)
        nbytes = 16 + 4 * R + R
        self._stage_dev = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self._stage_host = torch.zeros(nbytes, dtype=torch.uint8).pin_memory()
        self.seed_offset = self._stage_dev[:16].view(torch.int64)
        self.temperatures = self._stage_dev[16:16 + 4 * R].view(torch.float32)
        self.greedy_mask = self._stage_dev[16 + 4 * R:]
        host = self._stage_host.numpy()             # shares the pinned memory
        self._h_so = host[:16].view(np.uint64)
        self._h_temp = host[16:16 + 4 * R].view(np.float32)
        self._h_mask = host[16 + 4 * R:]
        self.temperatures.fill_(1.0)
        self.greedy_mask.fill_(1)
        # the staging copy is ordered by a plain HIP event (no timing, no
        # system-scope fence): the next replay's host writes wait for it
        hip = _hip()
        ev = _c_vp()
        if hip.hipEventCreateWithFlags(ctypes.byref(ev), 0x2 | 0x20000000) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self._staged = ev
        self._stage_args = (_c_vp(self._stage_dev.data_ptr()), _c_vp(self._stage_host.data_ptr()), nbytes)
        self.call = ProposeBlock(cfg, x=x, conv_base=conv_base, conv_delta=conv_delta, logits=logits, anchor=anchor,
                                 sel_a=sel_a, sel_b=sel_b, proj=proj, uniforms=self.uniforms,
                                 temperatures=self.temperatures, greedy_mask=self.greedy_mask,
                                 valid_vocab=valid_vocab, vocab=vocab)
        self._philox = lib().dflash_philox_uniforms
        # one eager step first: the library creates its auxiliary stream and
        # events on first use, which must not happen inside the capture
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self._step(side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._step(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()

    def _step(self, stream_handle) -> None:
        st = self._philox(_p(self.seed_offset), self.n, _p(self.uniforms), stream_handle)
        if st != DFLASH_OK:
            raise DFlashError(st, last_error())
        self.call(stream_handle)

    def _stage(self, temperatures, greedy_mask, seed: int, offset: int, stream) -> None:
        hip = _hip()
        if hip.hipEventSynchronize(self._staged) != 0:     # the previous staging copy has read the pinned buffer
            raise RuntimeError("hipEventSynchronize failed")
        self._h_temp[:] = np.asarray(temperatures, dtype=np.float32)
        self._h_mask[:] = np.asarray(greedy_mask, dtype=np.uint8)
        self._h_so[0] = seed & ((1 << 64) - 1)
        self._h_so[1] = offset & ((1 << 64) - 1)
        dst, src, nbytes = self._stage_args
        if hip.hipMemcpyAsync(dst, src, nbytes, 1, stream) != 0 or hip.hipEventRecord(self._staged, stream) != 0:
            raise RuntimeError("staging copy failed")

    def replay(self, temperatures, greedy_mask, seed: int, offset: int) -> Dict[str, torch.Tensor]:
        """Stage the sampling parameters and {seed, offset} (host values), then
        replay on torch's current stream.  Returns the outputs dict."""
        self._stage(temperatures, greedy_mask, seed, offset, torch.cuda.current_stream().cuda_stream)
        self.graph.replay()
        return self.call.outputs

    def step_eager(self, temperatures, greedy_mask, seed: int, offset: int) -> Dict[str, torch.Tensor]:
        """The same step without the graph: the same staging copy, then the
        uniforms and the propose call launched one by one on torch's current
        stream (the like-for-like comparison for replay)."""
        stream = torch.cuda.current_stream().cuda_stream
        self._stage(temperatures, greedy_mask, seed, offset, stream)
        self._step(stream)
        return self.call.outputs


def dflash_propose_block_noalloc(cfg: DraftConfig, *, stage_events: Optional[Sequence] = None, stream=None,
                                 **kw) -> Dict[str, torch.Tensor]:
    """dflash_propose_block through the entry point that allocates nothing
    (its scratch is the library's own); same inputs and outputs."""
    return dflash_propose_block(cfg, stage_events=stage_events, stream=stream, noalloc=True, **kw)


def dflash_propose_block(cfg: DraftConfig, *, stage_events: Optional[Sequence] = None, stream=None,
                         **kw) -> Dict[str, torch.Tensor]:
    """One draft block.  x [n_req*B, H]; conv_base [T, H]; conv_delta
    [N, T, G] (rows may be strided: one side of the packed projection);
    logits [n_req*(B-1), >= vocab]; anchor [n_req]; sel_a, sel_b [V, r];
    proj [r, H]; uniforms [n_req, B-1]; temperatures, greedy_mask [n_req].
    Keywords of ProposeBlock besides.  Returns a dict with conv_out, ids,
    unary, tokens, q (and scores when keep_scores)."""
    call = ProposeBlock(cfg, **kw)
    ev = None if stage_events is None else ProposeBlock.event_array(stage_events)
    return call(None if stream is None else stream.cuda_stream, ev)
