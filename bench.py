"""Benchmark of the DFlash2 draft-block hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one dflash_propose_block call (conv -> transform + top-K ->
projection -> lattice -> walk; the library runs conv and projection beside
the top-K on a second stream) over one batch of synthetic draft blocks,
issued through a prepared call whose arguments were marshalled once per input
set, as a serving loop with fixed buffers does.  The
default workload is the largest one, 1024 requests x block 16 (hidden 7168 =
112 x 64, 8 taps, vocab 201024, K = 32, rank 128, all sampled at T = 0.7).  Activations (x,
delta, logits, uniforms) rotate over several independent input sets whose
logits total more than twice the 256 MB Infinity Cache, so every step streams
its logits from HBM; selector tables and projection weights stay fixed like
model weights.  Inputs are resident in HBM before the timed region starts.

Prints one JSON line: draft tokens/s over the timed steps, the top-K kernel's
achieved HBM bandwidth against the 8 TB/s peak (timed with HIP events recorded
by the library around that kernel on its stream; the events are created for
timing only, without a system-scope fence), and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft tokens/s through conv+topK+lattice walk; conv/topK HBM GB/s % of peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFS = 2500.0      # MI355X dense bf16 matrix peak, TFLOP/s
DEFAULT_WORKLOAD = "stress_r1024_k32"
MALL_BYTES = 256 * 1024 * 1024
TIMED_EVERY = 4          # top-K events on every 4th timed step
SPIN_CYCLES = 400_000    # GPU spin before each swept call (~0.2 ms): longer than any call's host enqueue


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w):
    """Bytes each step must move, per kernel (inputs read once, outputs written once)."""
    e = w.elem_bytes
    N, H, T, G = w.n_tokens, w.hidden, w.taps, w.groups
    Ns, K, r, V = w.n_slot_rows, w.top_k, w.rank, w.valid_vocab
    return {
        "conv": 2 * N * H * e + N * T * G * e + T * H * e,
        "topk": Ns * V * e + 12 * Ns * K,
        "proj": Ns * H * e + r * H * e + 4 * Ns * r,
        "lattice_walk": 2 * Ns * K * r * e + 4 * Ns * r + 12 * Ns * K + 4 * Ns * K * K * 2 + 16 * Ns + 12 * Ns * K,
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "topk_traffic.json")
# the first-stage kernel's sources: the top-K file and the device code it
# inlines (the conv + slot projection workgroups share its launch)
TOPK_SOURCES = tuple(os.path.join(ROOT, "block_draft_proposal_amd", "csrc", f)
                     for f in ("topk.hip", "device_common.h", "conv_slot_proj.h", "conv_core.h", "gemm_tile.h"))


def sources_sha256(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per top-K launch from the committed counter runs (FETCH_SIZE
    + WRITE_SIZE, scaled by a copy kernel of known size), or None when they
    were taken on another workload or on top-K sources other than the ones
    built now."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        sha = sources_sha256(TOPK_SOURCES)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sha or t.get("workload") != workload:
        return None
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]


class TimingEvent:
    """A HIP event for timing only: created through the HIP runtime with
    hipEventDisableSystemFence, so recording it adds no system-scope cache
    write-back to the stream it times (torch's timing events carry one).
    Exposes ``cuda_event`` like torch.cuda.Event for the library's stage-event
    array."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        import ctypes
        if cls._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ctypes = ctypes
        h = ctypes.c_void_p()
        st = self._lib().hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {st}")
        self.cuda_event = h.value

    def record(self, stream_handle):
        st = self._lib().hipEventRecord(self.cuda_event, stream_handle)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = self._ctypes.c_float()
        st = self._lib().hipEventElapsedTime(self._ctypes.byref(ms), self.cuda_event, end.cuda_event)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return ms.value

    def __del__(self):
        if self._hip is not None and getattr(self, "cuda_event", None):
            self._hip.hipEventDestroy(self.cuda_event)


def copy_calibration(n_bytes: int, reps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = n_bytes // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_dispatch": n * 4, "bytes_written_per_dispatch": n * 4,
                                           "dispatches": reps}}), flush=True)


def call_bytes(w):
    """Algorithmic bytes of each C-ABI call on workload w (inputs read once,
    outputs written once; the lattice includes its projection)."""
    e = w.elem_bytes
    N, H, T, G = w.n_tokens, w.hidden, w.taps, w.groups
    Ns, K, r, V, R = w.n_slot_rows, w.top_k, w.rank, w.valid_vocab, w.n_req
    conv = 2 * N * H * e + N * T * G * e + T * H * e
    topk = Ns * V * e + 12 * Ns * K
    proj = Ns * H * e + r * H * e
    gathers = 2 * Ns * K * r * e
    lattice = proj + gathers + 12 * Ns * K + 8 * R + 4 * Ns * K * K
    walk = 4 * Ns * K * K + 8 * Ns * K + 4 * Ns + 5 * R + 8 * Ns + 4 * Ns * K
    propose = conv + topk + proj + gathers + 8 * R + 4 * Ns + 5 * R + 8 * Ns + 4 * Ns * K
    # x and the projection weight in, side-0 base in, out and both sides' coefficients written
    prepare = 2 * N * H * e + 2 * T * G * H * e + T * H * e + 2 * N * T * G * e
    # target rows (every logical id) in; candidates, q, tokens, uniforms in; counts and tokens out
    verify = R * (w.slots + 1) * V * e + 12 * Ns * K + 12 * Ns + 4 * R + 9 * R + 4 * R + 8 * R * (w.slots + 1)
    return {"dflash_conv": conv, "dflash_conv_prepare": prepare, "dflash_topk": topk, "dflash_lattice": lattice,
            "dflash_walk": walk, "dflash_verify": verify, "dflash_propose_block": propose,
            "ProposeGraph.step_eager": propose + 4 * Ns + 5 * R + 16,
            "ProposeGraph.replay": propose + 4 * Ns + 5 * R + 16,
            "hbm_ceiling.read": Ns * w.vocab * e, "hbm_ceiling.copy": 2 * N * H * e}


def sweep(iters: int = 50, warm: int = 5, only=None):
    """Per-call GPU time of every C-ABI entry point on every workload: HIP
    events around each call on one stream; before each call a 1 GiB scratch
    write (flushes the 256 MB Infinity Cache) and then a GPU spin without
    memory traffic (the write drains, and the GPU stays busy while the host
    enqueues the call); median and p10/p90 over the timed calls."""
    import torch
    import block_draft_proposal_amd as D
    import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def timed(fn):
        out = []
        for it in range(warm + iters):
            scratch.fill_(it & 0xff)
            # a spin with no memory traffic: the scratch write drains, and
            # the GPU stays busy while the host enqueues the timed call
            torch.cuda._sleep(SPIN_CYCLES)
            a, b = TimingEvent(), TimingEvent()
            a.record(stream)
            fn()
            b.record(stream)
            out.append((a, b))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in out[warm:])
        pick = lambda q: t[min(len(t) - 1, int(q * (len(t) - 1) + 0.5))]
        return pick(0.5), pick(0.1), pick(0.9)

    # copy ceiling: 1 GiB device-to-device (reads 1 GiB, writes 1 GiB), by
    # torch's copy and by the library's streaming copy; and a 1 GiB read
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    med, _, _ = timed(lambda: dst.copy_(src))
    copy_gbs = 2 * (1 << 30) / (med * 1e-6) / 1e9
    med_s, _, _ = timed(lambda: D.dflash_hbm_ceiling(D.CEILING_COPY, src, dst))
    med_r, _, _ = timed(lambda: D.dflash_hbm_ceiling(D.CEILING_READ, src, sink))
    del src, dst
    print(f"copy ceiling: 1 GiB torch device copy {med:.1f} us -> {copy_gbs:.0f} GB/s (read + write); "
          f"streaming copy (dflash_hbm_ceiling) {med_s:.1f} us -> {2 * (1 << 30) / (med_s * 1e-6) / 1e9:.0f} GB/s; "
          f"streaming read of 1 GiB {med_r:.1f} us -> {(1 << 30) / (med_r * 1e-6) / 1e9:.0f} GB/s\n")
    print("Rows hbm_ceiling.read / hbm_ceiling.copy: dflash_hbm_ceiling streams of the workload's logits (the "
          "top-K's bytes) and of its x copied into the conv output (the conv's rows), for reading the kernels "
          "against a plain stream of the same size.\n")
    print("| workload | call | median us | p10 us | p90 us | algorithmic MB | GB/s | % of 8 TB/s | % of copy |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, w in W.WORKLOADS.items():
        if only and name not in only:
            continue
        cfg = D.make_config(taps=w.taps, group_size=w.group_size, rank=w.rank, top_k=w.top_k,
                            multiplier=w.multiplier, softcap=w.softcap, block_size=w.block_size, hidden=w.hidden)
        inp = W.make_inputs(w, device=dev)
        R, B, S, K, H = w.n_req, w.block_size, w.slots, w.top_k, w.hidden
        conv_out = torch.empty_like(inp["x"])
        ids = torch.empty((R * S, K), dtype=torch.int64, device=dev)
        unary = torch.empty((R * S, K), dtype=torch.float32, device=dev)
        tk_ws = torch.empty(max(1, D.lib().dflash_topk_workspace_size(R * S, w.valid_vocab, K)), dtype=torch.uint8,
                            device=dev)
        D.dflash_conv(inp["x"], inp["base"][0], inp["delta"][:, 0], block_size=B, group_size=w.group_size, out=conv_out)
        D.dflash_topk(inp["logits"], top_k=K, valid_vocab=w.valid_vocab, multiplier=w.multiplier, softcap=w.softcap,
                      ids_out=ids, unary_out=unary, workspace=tk_ws)
        hid = conv_out.view(R, B, H)[:, 1:, :]
        lat_ws = torch.empty(max(1, D.lib().dflash_lattice_workspace_size(R, S, w.rank, H)), dtype=torch.uint8,
                             device=dev)
        scores = torch.empty((R, S, K, K), dtype=torch.float32, device=dev)
        idv, unv = ids.view(R, S, K), unary.view(R, S, K)
        tokens = torch.empty((R, S), dtype=torch.int64, device=dev)
        q = torch.empty((R, S, K), dtype=torch.float32, device=dev)
        call = D.ProposeBlock(cfg, x=inp["x"], conv_base=inp["base"][0], conv_delta=inp["delta"][:, 0],
                              logits=inp["logits"], anchor=inp["anchor"], sel_a=inp["sel_a"], sel_b=inp["sel_b"],
                              proj=inp["proj"], uniforms=inp["uniforms"], temperatures=inp["temperatures"],
                              greedy_mask=inp["greedy_mask"], valid_vocab=w.valid_vocab)
        mod = W.make_conv_module_inputs(w, device=dev)
        ver = W.make_verify_inputs(w, device=dev)
        graph = D.ProposeGraph(cfg, x=inp["x"], conv_base=inp["base"][0], conv_delta=inp["delta"][:, 0],
                               logits=inp["logits"], anchor=inp["anchor"], sel_a=inp["sel_a"], sel_b=inp["sel_b"],
                               proj=inp["proj"], valid_vocab=w.valid_vocab)
        g_temps, g_mask = inp["temperatures"].cpu(), inp["greedy_mask"].cpu()
        v_acc = torch.empty(R, dtype=torch.int32, device=dev)
        v_com = torch.empty((R, S + 1), dtype=torch.int64, device=dev)
        v_ws = torch.empty(max(1, D.lib().dflash_verify_workspace_size(R, S, w.valid_vocab)), dtype=torch.uint8, device=dev)
        coeff = torch.empty((w.n_tokens, 2, w.taps, w.groups), dtype=inp["x"].dtype, device=dev)
        prep_ws = torch.empty(max(1, D.lib().dflash_conv_prepare_workspace_size(
            w.n_tokens, H, w.group_size, w.taps, 1 if w.dtype == "bf16" else 0)), dtype=torch.uint8, device=dev)
        fns = {
            "dflash_conv": lambda: D.dflash_conv(inp["x"], inp["base"][0], inp["delta"][:, 0], block_size=B,
                                                 group_size=w.group_size, out=conv_out),
            "dflash_conv_prepare": lambda: D.dflash_conv_prepare(mod["x"], mod["proj_weight"], mod["base2"],
                                                                 block_size=B, group_size=w.group_size,
                                                                 out=conv_out, coeff_out=coeff, workspace=prep_ws),
            "dflash_topk": lambda: D.dflash_topk(inp["logits"], top_k=K, valid_vocab=w.valid_vocab,
                                                 multiplier=w.multiplier, softcap=w.softcap, ids_out=ids,
                                                 unary_out=unary, workspace=tk_ws),
            "dflash_lattice": lambda: D.dflash_lattice(idv, unv, hid, inp["anchor"], inp["sel_a"], inp["sel_b"],
                                                       inp["proj"], scores_out=scores, workspace=lat_ws),
            "dflash_walk": lambda: D.dflash_walk(scores, idv, inp["uniforms"], inp["temperatures"],
                                                 inp["greedy_mask"], tokens_out=tokens, q_out=q),
            "dflash_verify": lambda: D.dflash_verify(ver["target_logits"], idv, q, tokens, ver["u_accept"],
                                                     ver["u_residual"], inp["temperatures"], inp["greedy_mask"],
                                                     valid_vocab=w.valid_vocab, accepted_out=v_acc,
                                                     committed_out=v_com, workspace=v_ws),
            "dflash_propose_block": lambda: call(stream),
            "ProposeGraph.step_eager": lambda: graph.step_eager(g_temps, g_mask, 1234, 0),
            "ProposeGraph.replay": lambda: graph.replay(g_temps, g_mask, 1234, 0),
            "hbm_ceiling.read": lambda: D.dflash_hbm_ceiling(D.CEILING_READ, inp["logits"], sink),
            "hbm_ceiling.copy": lambda: D.dflash_hbm_ceiling(D.CEILING_COPY, inp["x"], conv_out),
        }
        nbytes = call_bytes(w)
        for cname, fn in fns.items():
            med, p10, p90 = timed(fn)
            gbs = nbytes[cname] / (med * 1e-6) / 1e9
            print(f"| {name} | {cname} | {med:.2f} | {p10:.2f} | {p90:.2f} | {nbytes[cname] / 1e6:.2f} | {gbs:.0f} | "
                  f"{100 * gbs / HBM_PEAK_GBS:.1f} | {100 * gbs / copy_gbs:.1f} |", flush=True)
        del inp, call, fns, mod, coeff, prep_ws, ver, v_acc, v_com, v_ws, graph
        torch.cuda.empty_cache()

    # the dense head in front of the top-K (bf16 workloads): plain, and fused with the top-K
    print("\n| workload | call | rows x hidden x vocab | median us | p10 us | p90 us | GFLOP | TFLOP/s | "
          "% of 2.5 PFLOP/s |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, w in W.WORKLOADS.items():
        if (only and name not in only) or w.dtype != "bf16":
            continue
        d = W.make_head_inputs(w, device=dev)
        hid, wt = d["hidden"], d["weight"]
        M, H, V, K = hid.shape[0], hid.shape[1], wt.shape[0], w.top_k
        logits = torch.empty((M, V), dtype=hid.dtype, device=dev)
        ids = torch.empty((M, K), dtype=torch.int64, device=dev)
        unary = torch.empty((M, K), dtype=torch.float32, device=dev)
        ws = torch.empty(D.lib().dflash_lm_head_topk_workspace_size(M, V, K), dtype=torch.uint8, device=dev)
        fns = {
            "dflash_lm_head": lambda: D.dflash_lm_head(hid, wt, out=logits),
            "dflash_lm_head_topk": lambda: D.dflash_lm_head_topk(hid, wt, top_k=K, valid_vocab=w.valid_vocab,
                                                                 multiplier=w.multiplier, softcap=w.softcap,
                                                                 ids_out=ids, unary_out=unary, workspace=ws),
        }
        flop = 2.0 * M * H * V
        for cname, fn in fns.items():
            med, p10, p90 = timed(fn)
            tfs = flop / (med * 1e-6) / 1e12
            print(f"| {name} | {cname} | {M} x {H} x {V} | {med:.1f} | {p10:.1f} | {p90:.1f} | {flop / 1e9:.1f} | "
                  f"{tfs:.0f} | {100 * tfs / MFMA_PEAK_TFS:.1f} |", flush=True)
        del d, hid, wt, logits, ids, unary, ws, fns
        torch.cuda.empty_cache()


def _oracle_host_inputs(name: str, n_req_sample: int, seed: int):
    import torch
    import workloads as W
    ws = W.WORKLOADS[name].replace(n_req=n_req_sample)
    inp = W.make_inputs(ws, device="cpu", seed=seed)
    return ws, {k: (v.to(torch.float64).numpy() if v.is_floating_point() else v.numpy()) for k, v in inp.items()}


def _run_oracle(ws, host):
    from oracle import dflash_oracle as O
    O.propose_block(host, block_size=ws.block_size, group_size=ws.group_size, valid_vocab=ws.valid_vocab,
                    top_k=ws.top_k, multiplier=ws.multiplier, softcap=ws.softcap, dtype=ws.dtype)


def _single_thread():
    import torch
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:   # pragma: no cover - threadpoolctl is optional
        pass
    torch.set_num_threads(1)


_START = None


def _worker_init(barrier):
    global _START
    _START = barrier
    _single_thread()
    import oracle.dflash_oracle  # noqa: F401
    import workloads  # noqa: F401


def _worker_batch(name: str, n_req_sample: int, seed: int):
    """One batch in a worker: inputs first, then every worker starts the
    oracle together (barrier); returns the oracle's wall-clock interval."""
    ws, host = _oracle_host_inputs(name, n_req_sample, seed)
    _START.wait()
    t0 = time.time()
    _run_oracle(ws, host)
    return t0, time.time()


def _host_cores() -> int:
    """Cores this process may run on, capped at the 16 a one-GPU share gets."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(w, n_req_sample: int, min_seconds: float = 8.0):
    """The oracle (as it stands, never tuned) on bounded samples of the
    workload, on the host's cores: one single-threaded process, then one
    single-threaded process per core, each on its own batch (fresh seeds),
    all started together once their inputs exist and timed by wall clock
    from the first start to the last end.  Input generation is not timed.
    Called before the GPU is touched; the worker processes are spawned fresh."""
    import concurrent.futures
    import multiprocessing
    import workloads as W
    base_seed = W.master_seed(w)
    per_batch = n_req_sample * w.slots
    _single_thread()
    dt1, b1 = 0.0, 0
    while dt1 < min_seconds:
        ws, host = _oracle_host_inputs(w.name, n_req_sample, base_seed + 7919 * b1)
        t0 = time.perf_counter()
        _run_oracle(ws, host)
        dt1 += time.perf_counter() - t0
        b1 += 1
    one = {"value": b1 * per_batch / dt1, "cores": 1,
           "sample": f"{b1} batches of {n_req_sample} of the {w.n_req} requests ({b1 * per_batch} draft tokens), "
                     f"{dt1:.1f} s in one single-threaded process"}
    cores = _host_cores()
    ctx = multiprocessing.get_context("spawn")
    barrier = ctx.Barrier(cores)
    with concurrent.futures.ProcessPoolExecutor(max_workers=cores, mp_context=ctx, initializer=_worker_init,
                                                initargs=(barrier,)) as ex:
        futs = [ex.submit(_worker_batch, w.name, n_req_sample, base_seed + 7919 * (1000 + c)) for c in range(cores)]
        spans = [f.result() for f in futs]
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    tokens = cores * per_batch
    return {"value": tokens / wall, "unit": "draft tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{cores} batches of {n_req_sample} of the {w.n_req} requests ({tokens} draft tokens), one "
                      f"per single-threaded process on {cores} cores started together, {wall:.1f} s wall clock; "
                      f"full vocab/hidden; numpy float64 (walk in fp32)",
            "single_core": one}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-requests", type=int, default=8)
    ap.add_argument("--sweep", action="store_true",
                    help="only time every C-ABI call on every workload (markdown table) and exit")
    ap.add_argument("--sweep-only", nargs="*", default=None, metavar="WORKLOAD",
                    help="with --sweep: only these workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling rocprofv3 byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards requests with no "
              f"exchange, so per-GPU throughput is the single-GPU figure", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_draft_proposal_amd as D
    import workloads as W

    if args.copy_calibration:
        copy_calibration(1 << 30, 10)
        return
    if args.sweep:
        sweep(only=args.sweep_only)
        return

    w = W.WORKLOADS[args.workload]
    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is initialised: the oracle's worker processes start
        # from a process with no GPU state
        log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(w, min(args.cpu_sample_requests, w.n_req))
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = D.make_config(taps=w.taps, group_size=w.group_size, rank=w.rank, top_k=w.top_k,
                        multiplier=w.multiplier, softcap=w.softcap, block_size=w.block_size, hidden=w.hidden)
    logits_bytes = w.n_slot_rows * w.vocab * w.elem_bytes
    n_sets = max(2, min(16, -(-2 * MALL_BYTES // max(logits_bytes, 1)) + 1))
    log(f"[bench] workload {w.name}: {n_sets} rotating input sets, logits {logits_bytes / 1e6:.1f} MB each")
    weights = W.make_inputs(w, device=dev, parts=("selector",))
    sets = []
    for i in range(n_sets):
        seed = W.master_seed(w) + 1000 * i
        s = W.make_inputs(w, device=dev, seed=seed, parts=("conv", "logits", "sampling"))
        s.update({k: weights[k] for k in ("sel_a", "sel_b", "proj")})
        s["anchor"] = W.make_inputs(w, device=dev, seed=seed, parts=("selector",))["anchor"]
        sets.append(s)
    del weights
    ws_bytes = D.propose_block_workspace_size(cfg, w.n_req, w.valid_vocab)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    # One prepared call per input set; all of them write the same outputs.
    calls = []
    outs = None
    for s in sets:
        c = D.ProposeBlock(cfg, x=s["x"], conv_base=s["base"][0], conv_delta=s["delta"][:, 0],
                           logits=s["logits"], anchor=s["anchor"], sel_a=s["sel_a"], sel_b=s["sel_b"],
                           proj=s["proj"], uniforms=s["uniforms"], temperatures=s["temperatures"],
                           greedy_mask=s["greedy_mask"], valid_vocab=w.valid_vocab, outputs=outs,
                           workspace=workspace)
        outs = c.outputs
        calls.append(c)
    stream = torch.cuda.current_stream().cuda_stream

    for i in range(args.warmup):
        calls[i % n_sets](stream)
    torch.cuda.synchronize()

    def event_sets(n, stages):
        """n arrays of 8 stage events, recorded once up front so they exist;
        only the listed stages get events (the library skips NULL entries)."""
        evs = []
        for _ in range(n):
            row = [TimingEvent() if k // 2 in stages else None for k in range(8)]
            for e in row:
                if e is not None:
                    e.record(stream)
            evs.append((row, D.ProposeBlock.event_array(row)))
        torch.cuda.synchronize()
        return evs

    # Timed region: every TIMED_EVERY-th step carries the two events around
    # the top-K (the dominant kernel), on the stream it runs on.  Each event
    # record adds a few microseconds to the stream, so sampling keeps the
    # instrumentation from inflating the step time it sits in.
    sampled = [i for i in range(args.steps) if i % TIMED_EVERY == 0]
    timed = dict(zip(sampled, event_sets(len(sampled), stages=(1,))))
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev = timed.get(i)
        calls[(args.warmup + i) % n_sets](stream, ev[1] if ev else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    topk_ms = sum(r[2].elapsed_time(r[3]) for r, _ in timed.values()) / len(timed)

    # Per-stage breakdown from a shorter pass with all eight events.
    n_stage = min(args.steps, 50)
    staged = event_sets(n_stage, stages=(0, 1, 2, 3))
    for i in range(n_stage):
        calls[i % n_sets](stream, staged[i][1])
    torch.cuda.synchronize()
    stage_ms = [[r[2 * k].elapsed_time(r[2 * k + 1]) for k in range(4)] for r, _ in staged]
    avg_ms = [sum(x[k] for x in stage_ms) / n_stage for k in range(4)]
    avg_ms[1] = topk_ms
    nbytes = algorithmic_bytes(w)
    # the schedule the library takes for this batch (host-only query)
    fused = D.propose_block_schedule(cfg, w.n_req, w.dtype) == D.SCHEDULE_ONE_LAUNCH
    # the dominant kernel: the first stage (top-K, plus conv and slot
    # projection when they share its launch: x, base, delta and P read,
    # conv_out and u written)
    if fused:
        stage1_bytes = (nbytes["topk"] + nbytes["conv"] + w.rank * w.hidden * w.elem_bytes
                        + 4 * w.n_slot_rows * w.rank)
        stage1_name = "topk_conv_proj_bf16 (top-K + conv + slot projection)"
    else:
        stage1_bytes, stage1_name = nbytes["topk"], "topk_rows"
    topk_gbs = stage1_bytes / (avg_ms[1] * 1e-3) / 1e9
    # The conv's own rate: dflash_conv alone on the same rotating inputs (beside
    # the top-K its events are stretched by the shared HBM), median of 20.
    conv_out = torch.empty_like(sets[0]["x"])
    conv_ev = []
    for i in range(25):
        st = sets[i % n_sets]
        a, b = TimingEvent(), TimingEvent()
        # a spin without memory traffic keeps the GPU busy while the host
        # enqueues the call, so the events bracket GPU work only
        torch.cuda._sleep(SPIN_CYCLES)
        a.record(stream)
        D.dflash_conv(st["x"], st["base"][0], st["delta"][:, 0], block_size=w.block_size, group_size=w.group_size,
                      out=conv_out)
        b.record(stream)
        conv_ev.append((a, b))
    torch.cuda.synchronize()
    conv_us = sorted(a.elapsed_time(b) for a, b in conv_ev[5:])[10] * 1e3
    conv_gbs = nbytes["conv"] / (conv_us * 1e-6) / 1e9
    # What this chip sustains for plain streams of the same sizes, in the
    # kernels' load and store forms: a read of one input set's logits (the
    # top-K's bytes) and a copy of its x into conv_out (the conv's rows).
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def ceiling(kind, src_of, dst_of):
        evs = []
        for i in range(25):
            a, b = TimingEvent(), TimingEvent()
            torch.cuda._sleep(SPIN_CYCLES)
            a.record(stream)
            D.dflash_hbm_ceiling(kind, src_of(sets[i % n_sets]), dst_of(sets[i % n_sets]))
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs[5:])[10] * 1e3

    read_bytes = sets[0]["logits"].numel() * sets[0]["logits"].element_size()
    copy_bytes = 2 * sets[0]["x"].numel() * sets[0]["x"].element_size()
    read_us = ceiling(D.CEILING_READ, lambda st: st["logits"], lambda st: sink)
    copy_us = ceiling(D.CEILING_COPY, lambda st: st["x"], lambda st: conv_out)
    read_gbs = read_bytes / (read_us * 1e-6) / 1e9
    copy_gbs = copy_bytes / (copy_us * 1e-6) / 1e9
    tokens = w.n_slot_rows * args.steps
    line = {
        "metric": METRIC,
        "value": tokens / elapsed,
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "requests": w.n_req, "block_size": w.block_size, "hidden": w.hidden,
                   "groups": w.groups, "taps": w.taps, "vocab": w.vocab, "valid_vocab": w.valid_vocab,
                   "top_k": w.top_k, "rank": w.rank, "draft_tokens_per_step": w.n_slot_rows,
                   "input_sets": n_sets},
        "roofline": {"bound": "hbm", "kernel": stage1_name, "achieved": topk_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": topk_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(w.name),
                     "algorithmic_bytes_per_launch": stage1_bytes, "avg_launch_us": avg_ms[1] * 1e3},
        "hbm_kernels": {
            "topk": {"achieved": topk_gbs, "frac": topk_gbs / HBM_PEAK_GBS, "unit": "GB/s",
                     "how": "the roofline kernel above (events around it inside the timed steps)",
                     "read_ceiling": {"GBps": read_gbs, "us": read_us, "bytes": read_bytes,
                                      "how": "dflash_hbm_ceiling read of one input set's logits, median of 20"},
                     "of_read_ceiling": topk_gbs / read_gbs},
            "conv": {"achieved": conv_gbs, "frac": conv_gbs / HBM_PEAK_GBS, "unit": "GB/s", "us": conv_us,
                     "algorithmic_bytes": nbytes["conv"],
                     "how": "dflash_conv alone on the same rotating inputs, median of 20 calls by HIP events, "
                            "each after a GPU spin",
                     "copy_ceiling": {"GBps": copy_gbs, "us": copy_us, "bytes": copy_bytes,
                                      "how": "dflash_hbm_ceiling copy of one input set's x into the conv output, "
                                             "median of 20"},
                     "of_copy_ceiling": conv_gbs / copy_gbs}},
        "stage_us": {"conv": avg_ms[0] * 1e3, "topk": avg_ms[1] * 1e3, "proj": avg_ms[2] * 1e3,
                     "lattice_walk": avg_ms[3] * 1e3, "note": f"top-K from every {TIMED_EVERY}th timed step, the other stages "
                     f"from {n_stage} further steps with all stage events; "
                     + ("conv and projection are workgroups of the top-K's launch (their events bracket it; "
                        "the projection stage is empty)" if fused else
                        "conv and projection run beside the top-K on a second stream")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
