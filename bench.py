#!/usr/bin/env python3
"""Benchmark of the activation-sparse ReLU FFN decode step on one MI355X.

One step = one decode token through all L distinct layers of the workload
(every layer's weights resident in HBM; walking all L layers per token keeps
the 256 MB Infinity Cache from serving repeats).  Each token's L-layer chain is
captured once as a HIP graph and replayed; HIP events bracket exactly --steps
replays.  Reported value: layers/s.  Also reported: effective HBM GB/s on the
step's algorithmic bytes, the FFN-only tokens/s equivalent, a per-kernel
breakdown measured with HIP events around each kernel, the roofline of the
dominant kernel, the rate of a plain 1 GiB device copy on the same GPU (as
context), and the CPU oracle timed on a bounded sample on the host.

    python bench.py [--config llama70b] [--mode predicted] [--batch 1] [--steps K] [--warmup W]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse-FFN decode layers/s + effective HBM GB/s on active-neuron bytes"
def esize(dt: str) -> float:
    return {"f32": 4.0, "f16": 2.0}[dt]


def row_bytes(dt: str, k: int) -> float:
    if dt == "q4g32":
        return k / 2 + (k / 32) * 2          # nibbles + fp16 group scales
    return k * esize(dt)


def step_bytes(cfg, mode: str, B: int, count: int, n_hot: int = 0) -> float:
    """Algorithmic bytes of one layer-step: what the method must move.

    Predictor weights and bias (predicted mode; with a hot head of n_hot neurons, only the
    tail's P2 rows and b_p), the dense pre-activation matrix and bias (exact mode), the selected
    neurons' rows of every matrix the mode touches (q4 scales included) and their fp32 bias, x,
    y and the index list.  Split partials and other scratch traffic are excluded.
    """
    d, n, r = cfg.d_model, cfg.d_ffn, cfg.rank
    ea, rb = esize(cfg.act_dtype), row_bytes(cfg.w_dtype, d)
    io = 2 * B * d * ea + 4 * count
    if mode == "predicted":
        pred = (r * d + (n - n_hot) * r) * esize(cfg.p_dtype) + 4 * (n - n_hot)
        rows = (3 if cfg.gated else 2) * rb
        return pred + count * (rows + 4) + io
    if mode == "exact":
        pre = n * rb + 4 * n
        rows = (2 if cfg.gated else 1) * rb     # up (gated) + down; the pre-activation matrix was read densely
        return pre + count * rows + io
    rows = (3 if cfg.gated else 2) * rb
    return count * (rows + 4) + io


def phase_bytes(cfg, mode: str, phase: str, B: int, count: int, phases, n_hot: int = 0) -> float:
    """Algorithmic bytes one launch of a phase's kernel moves.

    pred_hidden: P1, x, h.  group: the mask source (P2 + b_p, or the dense
    pre-activation rows + b), the selected rows of every matrix the mode reads
    with their bias, x and the mask bits; its partial-sum writes are scratch
    and not counted.  Where a down kernel runs, the group kernel reads only the
    gate/up rows and the down kernel the selected down rows (the activations
    handed between them are scratch).  The finish kernel writes y and the index
    list; on the one-token split path (a down kernel and no finish kernel) the
    down kernel writes them, reading the mask bits to find the list.
    `phases` is the library's launch plan for the call.  With a hot head of n_hot neurons
    (predicted mode) the group kernel reads only the tail's P2 rows and b_p.
    """
    d, n, r = cfg.d_model, cfg.d_ffn, cfg.rank
    ea, rb = esize(cfg.act_dtype), row_bytes(cfg.w_dtype, d)
    split = "down" in phases and "finish" not in phases
    down = 0 if "down" in phases else 1      # down rows read by the group kernel
    hidden = r * d * esize(cfg.p_dtype) + B * d * ea + B * r * 4
    out = B * d * ea + 4 * count             # y and the index list
    if phase == "pred_hidden":
        return hidden
    if phase == "group":
        xb = B * d * ea + n / 8
        if mode == "predicted":
            tail = n - n_hot
            return (tail * r * esize(cfg.p_dtype) + 4 * tail + B * r * 4 + count * ((1 + down + cfg.gated) * rb + 4)
                    + xb)
        if mode == "exact":
            return n * rb + 4 * n + count * ((down + cfg.gated) * rb) + xb
        if split:
            return count * ((1 + cfg.gated) * rb + 4) + B * d * ea
        return count * ((1 + down + cfg.gated) * rb + 4) + xb
    if phase == "down":
        mask = 0 if mode == "dense" else n / 8
        return count * rb + mask + (out if split else 0)
    if phase == "finish":
        return out
    raise KeyError(phase)


def mode_run(mode: str, B: int) -> str:
    """The mask mode the library runs for a call: past 16 tokens a PREDICTED call runs as EXACT_RELU
    (the predictor is not run; the union of the per-token masks covers most of the layer there)."""
    return "exact" if (mode == "predicted" and B > 16) else mode


def expected_active(p, B: int) -> float:
    """Expected size of the batch-union mask: sum over neurons of 1 - (1 - p_i)^B."""
    import numpy as np
    return float(np.sum(1.0 - (1.0 - np.asarray(p, dtype=np.float64)) ** B))


def budget_rank(cfg, p, B: int, frac: float, step: int = 64) -> int:
    """Per-layer predictor rank under a byte budget: the largest multiple of `step`, at most the
    workload's rank and at least `step`, whose predictor bytes (P1, P2 and b_p) stay within `frac`
    of the layer's expected active-row bytes (its firing probabilities standing in for the offline
    profile).  The pages quote the predictor at under 3 % of the total computation."""
    d, n = cfg.d_model, cfg.d_ffn
    active = expected_active(p, B) * ((3 if cfg.gated else 2) * row_bytes(cfg.w_dtype, d) + 4)
    best = step
    for r in range(step, cfg.rank + 1, step):
        if (r * d + n * r) * esize(cfg.p_dtype) + 4 * n <= frac * active:
            best = r
    return best


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "activation_sparse_decode_relu_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counters_apply(rank: int, rank_policy: str, hot: float) -> bool:
    """Whether stored counter bytes describe this run: they were taken on each workload as
    configured, and a changed predictor rank, a per-layer rank policy or a hot set changes how many
    predictor bytes the kernels read."""
    return rank == 0 and rank_policy == "fixed" and hot == 0


def stored_traffic(kernel_phase: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current kernels."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    rec = data.get(f"{workload}/{kernel_phase}")
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


class HipEvent:
    """A raw timing hipEvent_t.

    Created with hipEventDisableSystemFence: a timing-only event then skips the system-scope
    cache writeback and invalidate that a default event performs on record, which would
    otherwise add microseconds to every bracketed kernel.
    """

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
            HipEvent._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            HipEvent._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                          ctypes.c_void_p]
            HipEvent._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._ev = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._ev), HipEvent.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = self._ev.value

    def elapsed_ms(self, stop: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self._ev, stop._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self._ev:
            HipEvent._hip.hipEventDestroy(self._ev)


def copy_calibration(mb: int) -> None:
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 3 copies of {mb} MiB", file=sys.stderr, flush=True)


def copy_ceiling(mib: int = 1024, reps: int = 10) -> float:
    """Practical HBM rate on this GPU: a plain device-to-device copy of `mib` MiB, (read + write bytes) / time.

    Context for the roofline fractions, which are always taken against the published 8 TB/s peak.
    """
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbps = 2.0 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


def read_ceiling(mib: int = 2048, reps: int = 10) -> float:
    """Practical HBM read rate on this GPU: the library's read probe (every 16-byte unit of a
    `mib` MiB buffer read once with streaming loads), bytes / time.  Context for the roofline
    fractions, which are always taken against the published 8 TB/s peak."""
    import torch
    import activation_sparse_decode_relu_amd as pi
    n = mib << 20
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sums = torch.zeros(512, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pi.probe_read(buf, sums)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pi.probe_read(buf, sums)
    e1.record()
    e1.synchronize()
    gbps = float(n) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sums
    return gbps


def summarize_pmc(fetch_csv: str, write_csv: str, copy_mib: int, workload: str, steps: int) -> dict:
    """Per-launch HBM bytes of each kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter files.

    Each counter is scaled by what it reads for the plain copy of copy_mib MiB
    (expected: copy_mib MiB fetched and written).
    """
    import csv
    from collections import defaultdict

    def load(path, counter):
        per = defaultdict(list)
        for row in csv.DictReader(open(path)):
            if row.get("Counter_Name") != counter:
                continue
            per[row["Kernel_Name"]].append(float(row["Counter_Value"]))
        return per

    fetch = load(fetch_csv, "FETCH_SIZE")
    write = load(write_csv, "WRITE_SIZE")
    copy_names = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
    expect_kib = copy_mib * 1024.0
    # only the calibration copy: FETCH_SIZE reads about half its size, WRITE_SIZE all of it; other
    # copies in the process (weight uploads, larger device copies) fall outside this window
    big_f = [v for k in copy_names for v in fetch[k] if 0.4 * expect_kib <= v <= 1.1 * expect_kib]
    big_w = [v for k in copy_names for v in write.get(k, []) if 0.4 * expect_kib <= v <= 1.1 * expect_kib]
    f_scale = expect_kib / (sum(big_f) / len(big_f)) if big_f else None
    w_scale = expect_kib / (sum(big_w) / len(big_w)) if big_w else None
    out = {"copy_mib": copy_mib, "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    phase_of = {"k_pred_hidden": "pred_hidden", "k_ffn_group": "group", "k_ffn_bgroup": "group",
                "k_act": "group", "k_ffn_bdown": "down", "k_down": "down", "k_finish": "finish"}
    for name, vals in fetch.items():
        phase = next((p for k, p in phase_of.items() if k in name), None)
        if phase is None or f_scale is None:
            continue
        wv = write.get(name, [])
        f_b = 1024.0 * f_scale * sum(vals) / len(vals)
        w_b = 1024.0 * w_scale * sum(wv) / len(wv) if wv and w_scale else None
        out["kernels"][f"{workload}/{phase}"] = {
            "kernel": name, "dispatches": len(vals), "fetch_bytes_per_launch": round(f_b),
            "write_bytes_per_launch": None if w_b is None else round(w_b),
            "bytes_per_launch": round(f_b + (w_b or 0.0)), "source_hash": source_hash()}
    return out


def cpu_baseline(cfg, mode: str, B: int, host_layers: dict, budget_s: float):
    """The CPU oracle, as it stands, on a bounded sample of the same workload.

    Timed twice: with the BLAS library's own thread pool (every core this process may run on),
    then limited to one thread, each on about half of `budget_s`.
    """
    import numpy as np
    import oracle
    from synth import make_tokens
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    blas_threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1) if threadpool_info else None
    ntok = min(cfg.tokens // B, 256)
    decoded = {}
    for l, layer in host_layers.items():
        # decode the stored weights once per layer, outside the timed region
        decoded[l] = (oracle.dense_weights(layer.w_gate, layer.s_gate) if layer.gated else None,
                      oracle.dense_weights(layer.w_up, layer.s_up),
                      oracle.dense_weights(layer.w_down_t, layer.s_down))

    def run(budget):
        done, elapsed = 0, 0.0
        per_layer = budget / max(1, len(host_layers))
        for l, layer in host_layers.items():
            x = make_tokens(cfg, l, ntok * B)
            spent = 0.0
            for t in range(ntok):
                t0 = time.perf_counter()
                oracle.forward(layer, x[t * B:(t + 1) * B], mode, weights=decoded[l])
                spent += time.perf_counter() - t0
                done += 1
                if spent > per_layer:
                    break
            elapsed += spent
        return done, elapsed

    done, elapsed = run(0.5 * budget_s)
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            d1, e1 = run(0.5 * budget_s)
        single = d1 / e1 if e1 > 0 else None
    return {"value": done / elapsed if elapsed > 0 else None, "unit": "layers/s", "cores": cores,
            "blas_threads": blas_threads, "single_core_value": single, "kind": "oracle",
            "sample": f"{done} layer-steps (batch {B}, {mode}) on layers {sorted(host_layers)} in {elapsed:.1f} s; "
                      f"float64 numpy, weights decoded outside the timed region; single_core_value: the same "
                      f"with BLAS limited to one thread"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed steps (one step = one token through all layers)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="llama70b",
                    help="workload (default: the largest single-GPU one, Llama2-70B-ReLU-shaped, 80 layers)")
    ap.add_argument("--mode", default="predicted", choices=("predicted", "exact", "dense"))
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=64, help="distinct token inputs per layer, replayed round-robin")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's own)")
    ap.add_argument("--rank", type=int, default=0,
                    help="override the predictor rank r (0 = the workload's own); for rank sweeps")
    ap.add_argument("--hot", type=float, default=0.0, metavar="F",
                    help="hot set: profile each layer on 64 calibration tokens (exact-ReLU firing counts) and "
                         "compute the neurons that fired on at least F of them without the predictor "
                         "(predicted mode, batch 1); 0 = off")
    ap.add_argument("--rank-policy", default="fixed", metavar="fixed|budget:F",
                    help="per-layer predictor rank: the workload's own (fixed), or per layer the largest rank "
                         "whose predictor bytes stay within F of the layer's expected active-row bytes")
    ap.add_argument("--profile-tokens", type=int, default=4, help="tokens of the per-kernel event pass")
    ap.add_argument("--repeats", type=int, default=5, help="further timed regions of --steps steps, for the spread")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter files and exit")
    args = ap.parse_args()

    if args.summarize_pmc:
        from synth import config_by_name
        cfg = config_by_name(args.config)
        res = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.copy_calib or 256,
                            f"{cfg.name}-{args.mode}-b{args.batch}", args.steps)
        path = os.path.join(ROOT, "profiles", "traffic.json")
        try:
            data = json.load(open(path))
        except (OSError, ValueError):
            data = {}
        data.update(res["kernels"])
        data.setdefault("_calibration", {})[f"{cfg.name}-{args.mode}-b{args.batch}"] = {
            k: res[k] for k in ("copy_mib", "fetch_scale", "write_scale")}
        json.dump(data, open(path, "w"), indent=1, sort_keys=True)
        print(json.dumps(res, indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the sparse FFN path here runs "
              "on one MI355X; see the sharding design notes).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import activation_sparse_decode_relu_amd as pi
    from synth import config_by_name, make_layer, make_tokens

    import dataclasses
    cfg = config_by_name(args.config)
    if args.rank:
        cfg = dataclasses.replace(cfg, rank=args.rank,
                                  workload=cfg.workload.replace(f"r={cfg.rank}", f"r={args.rank}"))
    B, mode = args.batch, args.mode
    run_mode = mode_run(mode, B)   # bytes and the CPU baseline follow what runs
    if args.hot > 0 and (mode != "predicted" or B != 1):
        ap.error("--hot applies to the predicted mode at batch 1 (a hot set runs on the one-token route)")
    if B not in cfg.batches and not (cfg.name == "toy" and B <= 16):
        print(f"note: batch {B} is not one of {cfg.name}'s configured batches {cfg.batches}", file=sys.stderr)
    L = args.layers or cfg.n_layers
    T = max(1, min(args.tokens, cfg.tokens // B))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calib:
        copy_calibration(args.copy_calib)

    # ---- setup: every layer resident in HBM --------------------------------------------------
    t_setup = time.time()
    handles, xs, ys, idxs = [], [], [], []
    host_sample = {}
    sample_layers = sorted({0, L // 2})
    ws = None
    ranks, lcfgs, hots = [], [], []
    for l in range(L):
        lcfg = cfg
        if args.rank_policy.startswith("budget:") and mode == "predicted":
            from synth import firing_probs
            lcfg = dataclasses.replace(cfg, rank=budget_rank(cfg, firing_probs(cfg, l), B,
                                                               float(args.rank_policy.split(":", 1)[1])))
        ranks.append(lcfg.rank)
        lcfgs.append(lcfg)
        layer = make_layer(lcfg, l, with_predictor=(mode == "predicted"))
        h = pi.upload_layer(layer, dev, max_batch=B, workspace=ws)
        n_hot = 0
        if args.hot > 0 and mode == "predicted":
            from activation_sparse_decode_relu_amd.hotset import firing_counts, hot_set, hot_words
            cal = torch.from_numpy(make_tokens(cfg, l, 64, start=cfg.tokens - 64)).to(dev)   # not timed
            hot = hot_set(firing_counts(h, cal), 64, args.hot)
            n_hot = int(hot.sum())
            h.set_hot(torch.from_numpy(hot_words(hot).view(np.int32)).to(dev))
        hots.append(n_hot)
        ws = h.workspace
        handles.append(h)
        if l in sample_layers and not args.no_cpu:
            host_sample[l] = layer
        xs.append(torch.from_numpy(make_tokens(cfg, l, T * B)).to(dev))
        ys.append(torch.empty((B, cfg.d_model), dtype=xs[-1].dtype, device=dev))
        idxs.append(torch.empty(cfg.d_ffn, dtype=torch.int32, device=dev))
        del layer
        if l % 8 == 7 or l == L - 1:
            print(f"[bench] {cfg.name}: {l + 1}/{L} layers resident ({time.time() - t_setup:.0f} s)", file=sys.stderr,
                  flush=True)
    counts = torch.zeros((T, L), dtype=torch.int32, device=dev)

    def token_step(t: int) -> None:
        for l in range(L):
            handles[l].forward(xs[l][t * B:(t + 1) * B], ys[l], mode, idxs[l], counts[t, l:l + 1])

    # ---- capture one graph per distinct token -------------------------------------------------
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(cap):
        token_step(0)
        cap.synchronize()
        for t in range(T):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                token_step(t)
            graphs.append(g)
    torch.cuda.synchronize()
    print(f"[bench] captured {T} token graphs x {L} layers", file=sys.stderr, flush=True)

    # ---- timed region --------------------------------------------------------------------------
    for k in range(args.warmup):
        graphs[k % T].replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for k in range(args.steps):
        graphs[k % T].replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    print(f"[bench] timed {args.steps} steps: {ms:.2f} ms", file=sys.stderr, flush=True)
    # the same timed region repeated, for the spread between runs (the headline is the first)
    repeats = []
    for _ in range(args.repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(args.steps):
            graphs[k % T].replay()
        e1.record()
        torch.cuda.synchronize()
        repeats.append(e0.elapsed_time(e1) / args.steps)

    cnt = counts.cpu().numpy().astype(np.int64)          # [T][L], deterministic per (token, layer)
    bytes_per_token = np.array([sum(step_bytes(lcfgs[l], run_mode, B, int(cnt[t, l]), hots[l]) for l in range(L))
                                for t in range(T)])
    total_bytes = sum(bytes_per_token[k % T] for k in range(args.steps))
    sec = ms / 1e3
    layers_per_s = L * args.steps / sec
    gbps = total_bytes / sec / 1e9

    # ---- per-kernel durations: HIP events around each kernel --------------------------------
    # HIP records events under stream capture as dependencies, not timed nodes, so the
    # instrumented pass is eager: a backlog of queued graph replays keeps the GPU busy while the
    # host enqueues one token's L layers, each with an event pair around the phase's kernel.
    phase_stats = {}
    n_prof = min(args.profile_tokens, T)
    plan = handles[0].launch_plan(B, mode)
    for phase in plan:
        durs, nbytes = [], []
        for t in range(n_prof):
            starts = [HipEvent() for _ in range(L)]
            stops = [HipEvent() for _ in range(L)]
            for k in range(16):
                graphs[(t + k + 1) % T].replay()
            for l in range(L):
                handles[l].profile_next(phase, starts[l], stops[l])
                handles[l].forward(xs[l][t * B:(t + 1) * B], ys[l], mode, idxs[l], counts[t, l:l + 1])
            torch.cuda.synchronize()
            for l in range(L):
                durs.append(starts[l].elapsed_ms(stops[l]) * 1e-3)
                nbytes.append(phase_bytes(lcfgs[l], run_mode, phase, B, int(cnt[t, l]), plan, hots[l]))
        tot_s = sum(durs)
        phase_stats[phase] = {"avg_us": 1e6 * tot_s / len(durs), "min_us": 1e6 * min(durs),
                              "launches": len(durs),
                              "alg_bytes_per_launch": sum(nbytes) / len(nbytes),
                              "achieved_gbps": sum(nbytes) / tot_s / 1e9,
                              "frac_of_peak": sum(nbytes) / tot_s / 1e9 / HBM_PEAK_GBPS}
    dom = max(phase_stats, key=lambda p: phase_stats[p]["avg_us"])
    ds = phase_stats[dom]
    sum_kernels_us = sum(v["avg_us"] for v in phase_stats.values())

    workload = f"{cfg.name}-{mode}-b{B}"
    traffic = stored_traffic(dom, workload) if counters_apply(args.rank, args.rank_policy, args.hot) else None
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ds["achieved_gbps"], 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(ds["achieved_gbps"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "avg_launch_us": round(ds["avg_us"], 3),
                "alg_bytes_per_launch": round(ds["alg_bytes_per_launch"])}

    cpu = None
    if not args.no_cpu:
        print(f"[bench] timing the CPU oracle (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, run_mode, B, host_sample, args.cpu_seconds)

    copy_gbps = None if args.copy_calib else copy_ceiling()   # counter runs keep only their calibration copy
    read_gbps = None if args.copy_calib else read_ceiling()

    replayed = sorted({k % T for k in range(args.steps)})   # tokens the timed region ran
    mean_count = float(cnt[replayed].mean())
    out = {
        "metric": METRIC,
        "value": round(layers_per_s, 1),
        "unit": "layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.w_dtype if cfg.w_dtype != "q4g32" else "q4g32+f16",
        "data": "synthetic",
        "config": {"workload": cfg.workload, "name": cfg.name, "mode": mode, "mode_run": run_mode, "batch": B,
                   "layers": L,
                   "d_model": cfg.d_model, "d_ffn": cfg.d_ffn, "rank": cfg.rank, "gated": cfg.gated,
                   "rank_policy": args.rank_policy, "hot_fraction": args.hot,
                   "mean_hot_neurons": round(float(np.mean(hots)), 1),
                   "layer_ranks": {str(r): ranks.count(r) for r in sorted(set(ranks))},
                   "act_dtype": cfg.act_dtype, "accumulate": "f32", "distinct_tokens": T,
                   "mean_active_neurons": round(mean_count, 1), "timing": "hipGraph per token, hipEvents"},
        "effective_hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "hbm_copy_gbps": round(copy_gbps, 1) if copy_gbps else None,   # context: a plain 1 GiB device copy
        "hbm_read_gbps": round(read_gbps, 1) if read_gbps else None,   # context: the read probe over 2 GiB
        "ffn_tokens_per_s": round(layers_per_s * B / L, 1),
        "alg_bytes_per_layer_step": round(total_bytes / (args.steps * L)),
        "us_per_layer_step": round(1e6 * sec / (L * args.steps), 3),
        "repeat_ms_per_step": [round(v, 4) for v in repeats],
        "median_layers_per_s": round(L / (1e-3 * float(np.median(repeats))), 1) if repeats else None,
        "kernel_sum_us_per_layer_step": round(sum_kernels_us, 3),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in phase_stats.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "source_hash": source_hash(),
    }
    print(json.dumps(out), flush=True)
    for h in handles:
        h.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
