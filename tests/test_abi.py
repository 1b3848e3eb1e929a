"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, its structs have the layout the binding mirrors, and the
host-side validation rejects contract violations (the DFlash2 pages' config
pairing and hidden % group_size errors) before anything is launched.  No
call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

import block_draft_proposal_amd as D
from block_draft_proposal_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    names = _declared_functions()
    assert "dflash_propose_block" in names and len(names) == 22
    lib = D.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(Bd.EXPORTED) == names
    out = subprocess.run(["nm", "-D", "--defined-only", D.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_abi_version():
    assert D.lib().dflash_abi_version() == 1


def test_struct_layout_matches_c(tmp_path):
    fields_cfg = [f for f, _ in Bd.DraftConfig._fields_]
    fields_args = [f for f, _ in Bd.BlockArgs._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "dflash.h"', "int main(void){"]
    src.append('printf("cfg %zu\\n", sizeof(dflash_draft_config));')
    src.append('printf("args %zu\\n", sizeof(dflash_block_args));')
    for f in fields_cfg:
        src.append(f'printf("cfg.{f} %zu\\n", offsetof(dflash_draft_config, {f}));')
    for f in fields_args:
        src.append(f'printf("args.{f} %zu\\n", offsetof(dflash_block_args, {f}));')
    src.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    assert int(got["cfg"]) == ctypes.sizeof(Bd.DraftConfig)
    assert int(got["args"]) == ctypes.sizeof(Bd.BlockArgs)
    for f in fields_cfg:
        assert int(got[f"cfg.{f}"]) == getattr(Bd.DraftConfig, f).offset, f
    for f in fields_args:
        assert int(got[f"args.{f}"]) == getattr(Bd.BlockArgs, f).offset, f


def _cfg(**kw):
    base = dict(taps=4, group_size=64, rank=64, top_k=8, multiplier=1.0, softcap=30.0, block_size=16, hidden=4096)
    base.update(kw)
    return D.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(taps=0, group_size=0), 0),
    (dict(rank=0, top_k=0), 0),
    (dict(taps=4, group_size=0), -1),
    (dict(taps=0, group_size=64), -1),
    (dict(rank=0, top_k=8), -1),
    (dict(rank=64, top_k=0), -1),
    (dict(group_size=48), -1),                  # 48 does not divide 4096
    (dict(multiplier=0.0), -1),
    (dict(multiplier=float("nan")), -1),
    (dict(softcap=-1.0), -1),
    (dict(block_size=0), -1),
    (dict(top_k=33), -2),
])
def test_validate_config(kw, code):
    cfg = _cfg(**kw)
    assert D.lib().dflash_validate_config(ctypes.byref(cfg)) == code
    if code:
        assert D.last_error()


FAKE = 1 << 20          # never dereferenced: validation fails first


def test_conv_validation():
    L = D.lib()
    # hidden % group_size
    assert L.dflash_conv(FAKE, FAKE, FAKE, 4 * 85, FAKE + (1 << 24), 16, 4096, 48, 4, 16, 1, None) == -1
    assert "must divide" in D.last_error()
    # ragged token count
    assert L.dflash_conv(FAKE, FAKE, FAKE, 4 * 64, FAKE + (1 << 24), 17, 4096, 64, 4, 16, 1, None) == -1
    # delta stride too small
    assert L.dflash_conv(FAKE, FAKE, FAKE, 3 * 64, FAKE + (1 << 24), 16, 4096, 64, 4, 16, 1, None) == -1
    # misaligned x
    assert L.dflash_conv(FAKE + 2, FAKE, FAKE, 4 * 64, FAKE + (1 << 24), 16, 4096, 64, 4, 16, 1, None) == -1
    # out overlapping x
    assert L.dflash_conv(FAKE, FAKE, FAKE, 4 * 64, FAKE + 64, 16, 4096, 64, 4, 16, 1, None) == -1
    # null pointer
    assert L.dflash_conv(None, FAKE, FAKE, 4 * 64, FAKE + (1 << 24), 16, 4096, 64, 4, 16, 1, None) == -1
    # bad dtype
    assert L.dflash_conv(FAKE, FAKE, FAKE, 4 * 64, FAKE + (1 << 24), 16, 4096, 64, 4, 16, 7, None) == -1
    # hidden not a multiple of the 16-byte vector
    assert L.dflash_conv(FAKE, FAKE, FAKE, 4 * 1, FAKE + (1 << 24), 16, 4, 4, 4, 16, 1, None) == -2
    # empty input is a no-op
    assert L.dflash_conv(None, None, None, 4 * 64, None, 0, 4096, 64, 4, 16, 1, None) == 0


def test_topk_validation():
    L = D.lib()
    assert L.dflash_topk_workspace_size(480, 151936, 8) == 0      # one workgroup per row: no partials
    ws = L.dflash_topk_workspace_size(100, 151936, 8)              # rows split over workgroups
    assert ws > 0
    args = lambda **k: dict(dict(logits=FAKE, stride=151936, rows=100, vocab=151936, valid=151936, k=8, m=1.0,
                                 cap=30.0, dtype=1, ids=FAKE, unary=FAKE, ws=FAKE, wsb=ws), **k)

    def call(a):
        return L.dflash_topk(a["logits"], a["stride"], a["rows"], a["vocab"], a["valid"], a["k"], a["m"],
                             a["cap"], a["dtype"], a["ids"], a["unary"], a["ws"], a["wsb"], None)

    assert call(args(k=0)) == -1
    assert call(args(k=33)) == -2
    assert call(args(valid=4)) == -1                 # K > valid_vocab
    assert call(args(valid=151937)) == -1            # valid_vocab > vocab
    assert call(args(stride=151935)) == -1           # row stride < vocab
    assert call(args(m=0.0)) == -1
    assert call(args(m=-1.0)) == -1
    assert call(args(cap=-2.0)) == -1
    assert call(args(wsb=ws - 1)) == -3
    assert call(args(logits=FAKE + 8)) == -1         # misaligned rows
    assert call(args(stride=151937, vocab=151936)) == -1
    assert call(args(vocab=1 << 24, valid=1 << 24, stride=1 << 24)) == -2
    assert call(args(rows=0, logits=None, ids=None, unary=None, ws=None, wsb=0)) == 0


def test_lattice_and_walk_validation():
    L = D.lib()
    # rank beyond what the bf16 projection supports
    assert L.dflash_lattice(FAKE, FAKE, FAKE, 16 * 4096, 4096, FAKE, FAKE, FAKE, FAKE, 32, 15, 8, 4096, 256, 151936,
                            1, FAKE, FAKE, 1 << 30, None) == -2
    # hidden row stride misaligned
    assert L.dflash_lattice(FAKE, FAKE, FAKE, 16 * 4096 + 1, 4096, FAKE, FAKE, FAKE, FAKE, 32, 15, 8, 4096, 64,
                            151936, 1, FAKE, FAKE, 1 << 30, None) == -1
    # workspace too small
    need = L.dflash_lattice_workspace_size(32, 15, 64, 4096)
    assert L.dflash_lattice(FAKE, FAKE, FAKE, 16 * 4096, 4096, FAKE, FAKE, FAKE, FAKE, 32, 15, 8, 4096, 64, 151936,
                            1, FAKE, FAKE, need - 1, None) == -3
    assert L.dflash_walk(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 3, 0, FAKE, FAKE, None) == -1
    assert L.dflash_walk(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 3, 40, FAKE, FAKE, None) == -2
    assert L.dflash_walk(None, FAKE, FAKE, FAKE, FAKE, 4, 3, 4, FAKE, FAKE, None) == -1
    assert L.dflash_walk(None, None, None, None, None, 0, 3, 4, None, None, None) == 0


def test_propose_block_validation():
    L = D.lib()
    cfg = _cfg()
    args = Bd.BlockArgs()
    args.n_req = 32
    args.dtype = 1
    assert L.dflash_propose_block(ctypes.byref(cfg), ctypes.byref(args), None) == -1   # null pointers
    bad = _cfg(taps=0, group_size=0)
    assert L.dflash_propose_block(ctypes.byref(bad), ctypes.byref(args), None) == -1
    assert "conv and the selector" in D.last_error()
    bad = _cfg(block_size=1)
    assert L.dflash_propose_block(ctypes.byref(bad), ctypes.byref(args), None) == -1
    assert L.dflash_propose_block_workspace_size(ctypes.byref(cfg), 32, 151936) > 0


@pytest.mark.parametrize("kw,n_req,dtype,want", [
    (dict(), 32, "bf16", D.SCHEDULE_ONE_LAUNCH),                   # 480 slot rows, blocks of 16, 4 taps
    (dict(), 136, "bf16", D.SCHEDULE_ONE_LAUNCH),                  # 2040 slot rows: still one launch
    (dict(), 137, "bf16", D.SCHEDULE_AUX_STREAM),               # 2055 rows: the tiled projection
    (dict(), 32, "f32", D.SCHEDULE_AUX_STREAM),                    # fp32 never shares the top-K's launch
    (dict(block_size=10, hidden=5120, taps=5), 64, "bf16", D.SCHEDULE_ONE_LAUNCH),   # blocks of 10, 576 rows
    (dict(block_size=2, hidden=512, taps=1), 64, "bf16", D.SCHEDULE_ONE_LAUNCH),     # blocks of 2: one slot
    (dict(block_size=20, hidden=512), 64, "bf16", D.SCHEDULE_AUX_STREAM),            # blocks above 16 tokens
    (dict(block_size=10, hidden=5120, taps=5), 240, "bf16", D.SCHEDULE_AUX_STREAM),   # 2160 rows
    (dict(taps=9), 32, "bf16", D.SCHEDULE_AUX_STREAM),             # more than 8 taps
    (dict(taps=8, rank=128, top_k=32, hidden=7168), 1024, "bf16", D.SCHEDULE_AUX_STREAM),
    (dict(rank=256), 32, "bf16", D.SCHEDULE_AUX_STREAM),           # rank above 128
])
def test_propose_block_schedule(kw, n_req, dtype, want):
    # host-only decision: which branch dflash_propose_block takes
    assert D.propose_block_schedule(_cfg(**kw), n_req, dtype) == want


def test_propose_block_schedule_rejects_what_propose_rejects():
    L = D.lib()
    for cfg, n_req, dt in [(_cfg(taps=0, group_size=0), 32, 1), (_cfg(block_size=1), 32, 1), (_cfg(), 0, 1),
                           (_cfg(), 32, 7), (_cfg(top_k=33), 32, 1)]:
        assert L.dflash_propose_block_schedule(ctypes.byref(cfg), n_req, dt) == 0
    with pytest.raises(D.DFlashError):
        D.propose_block_schedule(_cfg(block_size=1), 32, "bf16")


def test_lm_head_validation():
    L = Bd.lib()
    V8 = ctypes.c_void_p(16)
    call = lambda **kw: L.dflash_lm_head(*[kw.get(k, d) for k, d in (
        ("h", V8), ("hs", 64), ("w", V8), ("n", 4), ("H", 64), ("V", 128), ("o", ctypes.c_void_p(1 << 40)),
        ("os", 128), ("dt", 1), ("st", None))])
    assert call(dt=0) == Bd.DFLASH_ERR_UNSUPPORTED            # fp32
    assert call(dt=7) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(H=60, hs=64) == Bd.DFLASH_ERR_UNSUPPORTED      # hidden_size not a multiple of 8
    assert call(hs=32) == Bd.DFLASH_ERR_INVALID_ARG            # stride shorter than a row
    assert call(os=130) == Bd.DFLASH_ERR_INVALID_ARG           # stride not a multiple of 8
    assert call(n=-1) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(V=1 << 31, os=1 << 31) == Bd.DFLASH_ERR_UNSUPPORTED
    assert call(hs=1 << 22) == Bd.DFLASH_ERR_UNSUPPORTED       # tile offsets are 32-bit
    assert call(h=ctypes.c_void_p(18)) == Bd.DFLASH_ERR_INVALID_ARG   # misaligned
    assert call(o=ctypes.c_void_p(16)) == Bd.DFLASH_ERR_INVALID_ARG   # overlaps the inputs
    assert call(n=0) == Bd.DFLASH_OK and call(V=0, os=0) == Bd.DFLASH_OK   # nothing to do


def test_lm_head_topk_validation():
    L = Bd.lib()
    V8 = ctypes.c_void_p(16)
    ws_need = L.dflash_lm_head_topk_workspace_size(4, 1000, 8)
    assert ws_need > 0 and L.dflash_lm_head_topk_workspace_size(0, 1000, 8) == 0
    call = lambda **kw: L.dflash_lm_head_topk(*[kw.get(k, d) for k, d in (
        ("h", V8), ("hs", 64), ("w", V8), ("n", 4), ("H", 64), ("V", 1000), ("vv", 1000), ("K", 8), ("m", 1.0),
        ("cap", 0.0), ("dt", 1), ("ids", V8), ("un", V8), ("ws", ctypes.c_void_p(256)), ("wsb", ws_need),
        ("st", None))])
    assert call(dt=0) == Bd.DFLASH_ERR_UNSUPPORTED
    assert call(vv=1001) == Bd.DFLASH_ERR_INVALID_ARG          # valid_vocab > vocab
    assert call(K=0) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(K=33, vv=1000) == Bd.DFLASH_ERR_UNSUPPORTED
    assert call(m=0.0) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(cap=-1.0) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(wsb=ws_need - 1) == Bd.DFLASH_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(128)) == Bd.DFLASH_ERR_INVALID_ARG   # not 256-byte aligned
    assert call(hs=1 << 22) == Bd.DFLASH_ERR_UNSUPPORTED       # tile offsets are 32-bit
    assert call(n=0) == Bd.DFLASH_OK


def test_conv_prepare_validation():
    L = Bd.lib()
    A = ctypes.c_void_p
    N, H, gs, T, B = 32, 64, 8, 3, 4
    ws_need = L.dflash_conv_prepare_workspace_size(N, H, gs, T, 1)
    assert L.dflash_conv_prepare_workspace_size(N, H, gs, T, 0) == 0          # fp32 needs none
    assert L.dflash_conv_prepare_workspace_size(0, H, gs, T, 1) == 0
    # disjoint fake device addresses: x, weight, base2, out, coeff, workspace
    x, w, b2, o, c, ws = A(1 << 20), A(2 << 20), A(3 << 20), A(4 << 20), A(5 << 20), A(6 << 20)
    call = lambda **kw: L.dflash_conv_prepare(*[kw.get(k, d) for k, d in (
        ("x", x), ("w", w), ("b2", b2), ("o", o), ("c", c), ("n", N), ("H", H), ("gs", gs), ("T", T), ("B", B),
        ("dt", 1), ("ws", ws), ("wsb", ws_need), ("st", None))])
    assert call(dt=7) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(gs=12) == Bd.DFLASH_ERR_INVALID_ARG              # does not divide hidden
    assert call(n=30) == Bd.DFLASH_ERR_INVALID_ARG               # not whole blocks
    assert call(H=60, gs=4) == Bd.DFLASH_ERR_UNSUPPORTED         # bf16 hidden not a multiple of 8
    assert call(w=None) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(w=A((2 << 20) + 8)) == Bd.DFLASH_ERR_INVALID_ARG  # misaligned weight
    assert call(c=A((1 << 20) + 64)) == Bd.DFLASH_ERR_INVALID_ARG   # coefficients overlap x
    if ws_need:
        assert call(wsb=ws_need - 1) == Bd.DFLASH_ERR_WORKSPACE
        assert call(ws=A((6 << 20) + 128)) == Bd.DFLASH_ERR_INVALID_ARG   # not 256-byte aligned
    assert call(n=0) == Bd.DFLASH_OK


def test_verify_validation():
    L = Bd.lib()
    A = ctypes.c_void_p
    R, S, V, K = 4, 3, 100, 8
    need = L.dflash_verify_workspace_size(R, S, V)
    assert need >= R * (S + 1) * 24 and L.dflash_verify_workspace_size(0, S, V) == 0
    assert L.dflash_verify_workspace_size(R, S, 0) == 0
    # the chunk sums cover every vector of a row: at least 8 bytes per 1024 ids
    big = 151936
    assert L.dflash_verify_workspace_size(R, S, big) >= R * (S + 1) * (4 * 24 + 8 * (big // 1024))
    call = lambda **kw: L.dflash_verify(*[kw.get(k, d) for k, d in (
        ("z", A(1 << 20)), ("rs", V), ("R", R), ("S", S), ("V", V), ("vv", V), ("K", K), ("ids", A(2 << 20)),
        ("q", A(3 << 20)), ("tok", A(4 << 20)), ("ua", A(5 << 20)), ("ur", A(6 << 20)), ("t", A(7 << 20)),
        ("g", A(8 << 20)), ("dt", 1), ("acc", A(9 << 20)), ("com", A(10 << 20)), ("ws", A(11 << 20)),
        ("wsb", need), ("st", None))])
    assert call(dt=5) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(K=0) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(K=33) == Bd.DFLASH_ERR_UNSUPPORTED
    assert call(vv=101) == Bd.DFLASH_ERR_INVALID_ARG           # valid_vocab > vocab
    assert call(rs=99) == Bd.DFLASH_ERR_INVALID_ARG            # row stride < vocab
    assert call(S=-1) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(q=None) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(z=A((1 << 20) + 1)) == Bd.DFLASH_ERR_INVALID_ARG   # not element aligned
    assert call(wsb=need - 1) == Bd.DFLASH_ERR_WORKSPACE
    assert call(ws=A((11 << 20) + 4)) == Bd.DFLASH_ERR_INVALID_ARG   # not 8-byte aligned
    assert call(R=0) == Bd.DFLASH_OK


def test_hbm_ceiling_validation():
    L = Bd.lib()
    A = ctypes.c_void_p
    call = lambda kind=1, src=A(1 << 20), dst=A(2 << 20), n=1 << 16: L.dflash_hbm_ceiling(kind, src, dst, n, None)
    assert call(kind=2) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(n=24) == Bd.DFLASH_ERR_INVALID_ARG               # not a multiple of 16
    assert call(n=-16) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(src=None) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(src=A((1 << 20) + 8)) == Bd.DFLASH_ERR_INVALID_ARG
    assert call(dst=A((2 << 20) + 4)) == Bd.DFLASH_ERR_INVALID_ARG   # a copy needs 16-byte alignment
    assert call(dst=A((1 << 20) + 4096)) == Bd.DFLASH_ERR_INVALID_ARG   # overlaps src
    assert call(kind=0, dst=A((1 << 20) + 4)) == Bd.DFLASH_ERR_INVALID_ARG   # sink inside src
    assert call(n=0) == Bd.DFLASH_OK


def test_error_message_is_per_call():
    L = D.lib()
    cfg = _cfg(group_size=48)
    assert L.dflash_validate_config(ctypes.byref(cfg)) == -1
    assert "divide" in D.last_error()
    cfg = _cfg()
    assert L.dflash_validate_config(ctypes.byref(cfg)) == 0
    assert D.last_error() == ""


def test_propose_block_noalloc_rejects_batches_beyond_its_scratch():
    # Host-side checks only (nothing reaches the GPU): a batch whose
    # workspace exceeds the 64 MiB static scratch is refused up front.
    L = D.lib()
    cfg = D.make_config(taps=4, group_size=64, rank=128, top_k=32, multiplier=1.0, softcap=30.0, block_size=16,
                        hidden=4096)
    n_req = 16384                                       # 245760 slot rows: 126 MB of partials at least
    assert L.dflash_propose_block_workspace_size(ctypes.byref(cfg), n_req, 201024) > 64 << 20
    args = Bd.BlockArgs()
    args.n_req, args.valid_vocab, args.vocab, args.dtype = n_req, 201024, 201024, 1
    st = L.dflash_propose_block_noalloc(ctypes.byref(cfg), ctypes.byref(args), None)
    assert st == Bd.DFLASH_ERR_WORKSPACE
    assert b"static scratch" in L.dflash_last_error()
    assert L.dflash_propose_block_noalloc(ctypes.byref(cfg), None, None) == Bd.DFLASH_ERR_INVALID_ARG
