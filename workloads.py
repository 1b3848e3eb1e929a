"""Seeded synthetic workloads for the DFlash2 draft-block path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no convolution, no transform, no selection, no lattice, no
walk).  Both the CPU oracle (through the tests and the benchmark) and the HIP
library are fed from the tensors it returns, so the two sides always see the
same input bits.

Workloads follow the shapes the DFlash2 pages give ("[Spec] DFlash2: local
convolution + candidate selector", sglang PR 35371): a batch of requests, each
one draft block of ``block_size`` tokens whose position 0 is the verified
anchor; a hidden width split into conv groups; a vocabulary of logits per
proposal slot (151936, or 201024 physical with 200058 logical as on the DSpark
padded-vocab page, vllm PR 55133); and a rank-r selector.

Recipe (every tensor has its own named sub-stream, so drawing one never shifts
another):
  * sub-stream seed = first 8 bytes of SHA-256("<master seed>:<tensor name>"),
    fed to a ``torch.Generator`` on the device the tensor is made on;
  * normals come from ``torch.randn`` in fp32, scaled by sigma, then rounded
    once (round-to-nearest-even) to the storage dtype;
  * uniforms come from ``torch.rand`` in fp32 (multiples of 2^-24 in [0, 1));
  * integer ids come from ``torch.randint``.
Big tensors are drawn in fixed row chunks, each chunk with its own sub-stream,
so that the result does not depend on how much memory the device has.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Tuple

import torch

# Rows drawn per chunk for large 2-D tensors (fixed so results never depend on
# the device's memory).
_CHUNK_ELEMS = 1 << 26


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic draft-block workload (sizes and value distributions)."""

    name: str
    n_req: int            # R: requests in the batch
    block_size: int       # B: tokens per draft block (position 0 = anchor)
    hidden: int           # H
    group_size: int       # gs: channels per conv group, G = H / gs
    taps: int             # T: conv kernel size
    vocab: int            # V: physical vocabulary (row length of the logits)
    valid_vocab: int      # logical vocabulary; ids >= this are padding
    top_k: int            # K: candidates per slot
    rank: int             # r: selector rank
    dtype: str            # "bf16" or "f32": storage dtype of every float input
    multiplier: float     # output_multiplier m
    softcap: float        # final_logit_softcapping (0 = off)
    logit_sigma: float = 3.0
    x_sigma: float = 1.0
    base_sigma: float = 0.1
    delta_sigma: float = 0.05
    sel_sigma: float = 0.2
    plant_peak: bool = False     # one planted top-1 per slot row (max + 8)
    pad_neg_inf: bool = False    # logits at ids >= valid_vocab set to -inf
    # per-request sampling mode: "greedy", or a temperature as a float
    modes: str = "greedy"        # "greedy" | "sampled:<T>" | "alt:<T>" | "half:<T>" | "first:<T>"

    @property
    def slots(self) -> int:
        return self.block_size - 1

    @property
    def n_tokens(self) -> int:
        return self.n_req * self.block_size

    @property
    def n_slot_rows(self) -> int:
        return self.n_req * self.slots

    @property
    def groups(self) -> int:
        return self.hidden // self.group_size

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def greedy_and_temps(self) -> Tuple[list, list]:
        """Per-request (greedy flag, temperature) lists for this workload."""
        R = self.n_req
        kind, _, arg = self.modes.partition(":")
        t = float(arg) if arg else 1.0
        if kind == "greedy":
            return [True] * R, [1.0] * R
        if kind == "sampled":
            return [False] * R, [t] * R
        if kind == "alt":        # even requests greedy, odd requests sampled
            return [r % 2 == 0 for r in range(R)], [1.0 if r % 2 == 0 else t for r in range(R)]
        if kind == "half":       # first half greedy, second half sampled
            return [r < R // 2 for r in range(R)], [1.0 if r < R // 2 else t for r in range(R)]
        if kind == "first":      # request 0 greedy, the rest sampled
            return [r == 0 for r in range(R)], [1.0 if r == 0 else t for r in range(R)]
        raise ValueError(f"unknown sampling mode {self.modes!r}")

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, in the order the path's measurement plan lists them.
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        name="tiny_fp32", n_req=2, block_size=4, hidden=64, group_size=8, taps=3,
        vocab=512, valid_vocab=512, top_k=4, rank=8, dtype="f32",
        multiplier=1.0, softcap=30.0, modes="first:1.0"),
    "bf16_b16_v151936": Workload(
        name="bf16_b16_v151936", n_req=32, block_size=16, hidden=4096, group_size=64,
        taps=4, vocab=151936, valid_vocab=151936, top_k=8, rank=64, dtype="bf16",
        multiplier=1.0, softcap=30.0, plant_peak=True, modes="greedy"),
    "nonpow2_b10_v151936": Workload(
        name="nonpow2_b10_v151936", n_req=64, block_size=10, hidden=5120, group_size=64,
        taps=5, vocab=151936, valid_vocab=151936, top_k=8, rank=64, dtype="bf16",
        multiplier=1.0, softcap=0.0, modes="alt:0.8"),
    "padded_v201024_k16": Workload(
        name="padded_v201024_k16", n_req=256, block_size=16, hidden=4096, group_size=64,
        taps=4, vocab=201024, valid_vocab=200058, top_k=16, rank=128, dtype="bf16",
        multiplier=0.5, softcap=30.0, pad_neg_inf=True, modes="half:1.0"),
    "stress_r1024_k32": Workload(
        name="stress_r1024_k32", n_req=1024, block_size=16, hidden=7168, group_size=64,
        taps=8, vocab=201024, valid_vocab=201024, top_k=32, rank=128, dtype="bf16",
        multiplier=1.0, softcap=30.0, modes="sampled:0.7"),
}
WORKLOAD_ORDER = list(WORKLOADS)
# Master seed of workload i (1-based position in WORKLOAD_ORDER).
MASTER_SEED_BASE = 0xDF1A5B00


def master_seed(w: Workload) -> int:
    if w.name in WORKLOADS:
        return MASTER_SEED_BASE + WORKLOAD_ORDER.index(w.name) + 1
    return MASTER_SEED_BASE


def _substream(master: int, name: str) -> int:
    digest = hashlib.sha256(f"{master}:{name}".encode()).digest()
    return int.from_bytes(digest[:8], "little") & ((1 << 63) - 1)


def _gen(master: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_substream(master, name))
    return g


def torch_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def normal(shape, sigma: float, dtype: str, master: int, name: str, device) -> torch.Tensor:
    """N(0, sigma^2) draws in fp32, rounded once to ``dtype``; row-chunked."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=torch_dtype(dtype), device=device)
    if out.numel() == 0:
        return out
    rows = shape[0]
    per_row = max(1, out.numel() // rows)
    chunk = max(1, _CHUNK_ELEMS // per_row)
    for c0 in range(0, rows, chunk):
        c1 = min(rows, c0 + chunk)
        g = _gen(master, f"{name}#{c0 // chunk}", device)
        v = torch.randn((c1 - c0,) + shape[1:], generator=g, device=device, dtype=torch.float32)
        out[c0:c1] = (v * sigma).to(out.dtype)
    return out


def uniform(shape, master: int, name: str, device) -> torch.Tensor:
    g = _gen(master, name, device)
    return torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)


def randint(high: int, shape, master: int, name: str, device) -> torch.Tensor:
    g = _gen(master, name, device)
    return torch.randint(0, int(high), tuple(shape), generator=g, device=device, dtype=torch.int64)


def make_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                parts=("conv", "logits", "selector", "sampling")) -> Dict[str, torch.Tensor]:
    """Draw every input of workload ``w`` on ``device``.

    Returned tensors (row-major, contiguous):
      x        [N, H]        conv input (storage dtype)
      base     [2, T, H]     static conv kernel, both sides (input / output)
      delta    [N, 2, T, G]  per-token dynamic coefficients, both sides, packed
                             the way one kernel projection emits them
      logits   [N_s, V]      unary logits of the proposal slots
      anchor   [R] int64     verified anchor token per request
      sel_a    [V, r]        selector predecessor table A
      sel_b    [V, r]        selector candidate table B
      proj     [r, H]        rank-r projection P
      uniforms [R, S] fp32   supplied uniforms for sampled rows
      temperatures [R] fp32, greedy_mask [R] bool
    """
    m = master_seed(w) if seed is None else int(seed)
    dev = torch.device(device)
    N, H, T, G = w.n_tokens, w.hidden, w.taps, w.groups
    out: Dict[str, torch.Tensor] = {}
    if "conv" in parts:
        out["x"] = normal((N, H), w.x_sigma, w.dtype, m, "x", dev)
        out["base"] = normal((2, T, H), w.base_sigma, w.dtype, m, "base", dev)
        out["delta"] = normal((N, 2, T, G), w.delta_sigma, w.dtype, m, "delta", dev)
    if "logits" in parts:
        logits = normal((w.n_slot_rows, w.vocab), w.logit_sigma, w.dtype, m, "logits", dev)
        if w.pad_neg_inf and w.valid_vocab < w.vocab:
            logits[:, w.valid_vocab:] = float("-inf")
        if w.plant_peak and w.n_slot_rows > 0:
            ids = randint(w.valid_vocab, (w.n_slot_rows,), m, "plant", dev)
            rows = torch.arange(w.n_slot_rows, device=dev)
            peak = logits[:, : w.valid_vocab].float().amax(dim=1) + 8.0
            logits[rows, ids] = peak.to(logits.dtype)
            out["planted"] = ids
        out["logits"] = logits
    if "selector" in parts:
        out["anchor"] = randint(w.valid_vocab, (w.n_req,), m, "anchor", dev)
        out["sel_a"] = normal((w.vocab, w.rank), w.sel_sigma, w.dtype, m, "sel_a", dev)
        out["sel_b"] = normal((w.vocab, w.rank), w.sel_sigma, w.dtype, m, "sel_b", dev)
        out["proj"] = normal((w.rank, H), w.sel_sigma, w.dtype, m, "proj", dev)
    if "sampling" in parts:
        greedy, temps = w.greedy_and_temps()
        out["uniforms"] = uniform((w.n_req, w.slots), m, "uniforms", dev)
        out["temperatures"] = torch.tensor(temps, dtype=torch.float32, device=dev)
        out["greedy_mask"] = torch.tensor(greedy, dtype=torch.bool, device=dev)
    return out


def sha256_of(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's bytes (host copy), for logging input identity."""
    b = t.detach().contiguous().cpu().view(torch.uint8).numpy().tobytes()
    return hashlib.sha256(b).hexdigest()


def make_head_inputs(w: Workload, device="cpu", seed: Optional[int] = None, n_rows: Optional[int] = None
                     ) -> Dict[str, torch.Tensor]:
    """Inputs of the candidates-from-hidden step for workload ``w``:
      hidden [N_s, H]  slot hidden rows, N(0, 1), storage dtype
      weight [V, H]    dense head, N(0, (logit_sigma / sqrt(H))^2), so the
                       logits spread like the workload's logits
    The padded tail of a physical vocabulary gets the same draws (its ids are
    excluded by valid_vocab, as on the pages)."""
    m = master_seed(w) if seed is None else int(seed)
    dev = torch.device(device)
    rows = w.n_slot_rows if n_rows is None else int(n_rows)
    return {"hidden": normal((rows, w.hidden), 1.0, w.dtype, m, "head_hidden", dev),
            "weight": normal((w.vocab, w.hidden), w.logit_sigma / math.sqrt(w.hidden), w.dtype, m, "head_weight", dev)}


def make_conv_module_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                            n_tokens: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Inputs of the conv module's prepare / finish for workload ``w``:
      x           [N, H]          module input, N(0, 1), storage dtype
      y           [N, H]          a sublayer output for finish, N(0, 1)
      proj_weight [2*T*G, H]      kernel projection, N(0, (delta_sigma / sqrt(H))^2),
                                  so the coefficients spread like the workload's delta
      base2       [2, T, H]       base kernel, both sides, N(0, base_sigma^2)
    N defaults to the workload's token count (whole blocks)."""
    m = master_seed(w) if seed is None else int(seed)
    dev = torch.device(device)
    N = w.n_tokens if n_tokens is None else int(n_tokens)
    H, T, G = w.hidden, w.taps, w.hidden // w.group_size
    return {"x": normal((N, H), 1.0, w.dtype, m, "module_x", dev),
            "y": normal((N, H), 1.0, w.dtype, m, "module_y", dev),
            "proj_weight": normal((2 * T * G, H), w.delta_sigma / math.sqrt(H), w.dtype, m, "module_proj", dev),
            "base2": normal((2, T, H), w.base_sigma, w.dtype, m, "module_base", dev)}


def make_verify_inputs(w: Workload, device="cpu", seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Target side of a verify for workload ``w`` (the drafted tokens, their
    candidates and q come from the draft path):
      target_logits [R, S+1, V]  N(0, logit_sigma^2), storage dtype; ids past
                                 the logical vocabulary are -inf, as in the draft logits
      u_accept      [R, S]       uniforms in [0, 1) (multiples of 2^-24)
      u_residual    [R]          uniforms in [0, 1)"""
    m = master_seed(w) if seed is None else int(seed)
    dev = torch.device(device)
    R, S, V = w.n_req, w.slots, w.vocab
    z = normal((R * (S + 1), V), w.logit_sigma, w.dtype, m, "target_logits", dev).view(R, S + 1, V)
    if w.valid_vocab < V:
        z[:, :, w.valid_vocab:] = float("-inf")
    return {"target_logits": z,
            "u_accept": uniform((R, S), m, "verify_accept", dev),
            "u_residual": uniform((R,), m, "verify_residual", dev)}
