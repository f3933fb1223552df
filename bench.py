"""Benchmark of the VAR-Q packed-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one full block-by-block decode pass of the workload: for every
scale k of the 10-scale VAR schedule and every layer, quantize + bit-pack the
freshly decoded block's K and V into that layer's packed cache, then run
block-causal attention of the block's queries over the packed cache, both in
one launch (kvq_quantize_attend; head_dim 64, blocks of up to 256 tokens).
Other blocks, and every block with --unfused, call kvq_quantize_block then
kvq_attend_packed_split (up to 8 key ranges per query tile in a workspace
allocated up front; --no-split calls kvq_attend_packed instead).
Inputs (K, V, Q of every block of every layer, bf16, synthetic VAR-shaped
data drawn on the device) and caches are
resident in HBM before the timed region; every layer has its own buffers, so
the 256 MB last-level cache cannot serve repeats.

Printed: one JSON line.  `value` is packed-KV attention tokens/s over the whole
step (query tokens x layers per second, quantize+pack included).  Per-kernel
figures (`kernels`) come from HIP events on the launch stream over the timed
steps: when every launch is of one kind (the fused VAR step) one event pair per
step, otherwise events at every launch boundary; `per_block_us` are per-launch
times of each block (in the one-kind case from a separate pass after the timed
steps, with events only where the block changes: a block's span over its
layers' back-to-back launches, divided by their number).
`roofline` is for the kernel kind with the largest share of the step, over the
launches of that kind (`blocks`); `cpu_baseline` is the CPU oracle timed on a
bounded sample of the same workload on the host's cores.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "var_d20_b128_int4"
FUSED_MAX_TOKENS = 256  # blocks kvq_quantize_attend runs as one launch (head_dim 64, bf16)
MAX_SPLITS = 8  # key ranges per query tile for kvq_attend_packed_split
KERNEL_SOURCES = {
    "quant_pack": "visual_autoregressive_kv_amd/csrc/quant_pack.hip",
    "attend": "visual_autoregressive_kv_amd/csrc/attend.hip",
    "fused": "visual_autoregressive_kv_amd/csrc/attend.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="quantize and attend with separate calls for every block")
    ap.add_argument("--no-split", action="store_true",
                    help="attend with kvq_attend_packed instead of kvq_attend_packed_split")
    ap.add_argument("--roctx", action="store_true",
                    help="mark every timed step and every (block, layer) call with roctx ranges "
                         "(for rocprofv3 --marker-trace; adds host work to the timed loop)")
    ap.add_argument("--pack-mode", type=int, default=0, choices=(0, 2),
                    help="cache layout: 0 dense rows, 2 block-aligned 32-bit words")
    ap.add_argument("--layers", type=int, default=0,
                    help="run this many of the workload's layers (0: all); for shapes whose "
                         "inputs for every layer do not fit in HBM at once")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic bytes / flops (per launch)
# ---------------------------------------------------------------------------

PACK_MODE = 0  # cache layout of the run (--pack-mode)


def block_code_bytes(wl, k: int) -> int:
    """Packed codes of block k in one (sequence, head) cache: dense rows of
    ceil(b D / 8) bytes, or (block-aligned words) ceil(n_k D / floor(32 / b))
    32-bit words."""
    n, D = wl.blocks[k], wl.head_dim
    if PACK_MODE == 2:
        cpw = 32 // wl.bits
        return 4 * ((n * D + cpw - 1) // cpw)
    return n * ((wl.bits * D + 7) // 8)


def quant_bytes(wl, k: int) -> int:
    """Read the block's K and V once, write their packed codes and statistics."""
    B, H, D, n = wl.batch, wl.heads, wl.head_dim, wl.blocks[k]
    src = 2 if wl.src == "bf16" else 4
    return 2 * (B * n * H * D * src + B * H * block_code_bytes(wl, k) + B * H * D * 4)


def attend_bytes(wl, k: int) -> int:
    """Packed K/V prefix + their stats once per (sequence, head), Q in, O out (fp32)."""
    B, H, D, n = wl.batch, wl.heads, wl.head_dim, wl.blocks[k]
    prefix = sum(block_code_bytes(wl, j) for j in range(k + 1))
    return B * H * (2 * prefix + 2 * (k + 1) * D * 4 + n * D * 2 + n * D * 4)


def attend_flops(wl, k: int) -> int:
    B, H, D, n = wl.batch, wl.heads, wl.head_dim, wl.blocks[k]
    T = wl.offset(k) + n
    return 4 * B * H * n * T * D


def source_sha(rel: str) -> str:
    return hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].strip().split(": ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(wl, target_s: float):
    """The oracle as it stands, on the host's cores: quantize + pack every block
    and attend every block's queries, for a sample of (layer, sequence) pairs
    taken in order (all sequences of layer 0, then layer 1, ...), sized to about
    target_s seconds.  Threads each take whole pairs (the oracle itself is
    single-threaded); inputs are generated before the clock starts."""
    import varq_inputs as vi
    from oracle import binding as ob

    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    # every core this process may run on, unless the host caps its CPU share
    # through OMP_NUM_THREADS (the oracle is single-threaded per pair; the
    # threads below each take whole pairs)
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = max(1, min(affinity, share) if share > 0 else affinity)
    Lo = ob.layout_of(wl.with_(batch=1))

    def run_pairs(pairs):
        chunks = [c for c in (pairs[i::threads] for i in range(threads)) if c]
        ready = threading.Barrier(len(chunks) + 1)
        errors = []

        def work(items):
            try:
                data = [[(vi.kv_block(wl, l, "k", j, [b]), vi.kv_block(wl, l, "v", j, [b]),
                          vi.q_block(wl, l, j, [b])) for j in range(len(wl.blocks))]
                        for l, b in items]
            except BaseException as e:  # release the others instead of leaving them waiting
                errors.append(e)
                ready.abort()
                return
            try:
                ready.wait()
            except threading.BrokenBarrierError:
                return
            for kv in data:
                kc, vc = ob.alloc_cache(Lo), ob.alloc_cache(Lo)
                for j, (kb, vb, qb) in enumerate(kv):
                    ob.quantize_block(Lo, j, kb, vb, kc, vc)
                    ob.attend(Lo, j, qb, kc, vc)

        ths = [threading.Thread(target=work, args=(c,)) for c in chunks]
        for t in ths:
            t.start()
        try:
            ready.wait()
        except threading.BrokenBarrierError:
            pass
        t0 = time.perf_counter()
        for t in ths:
            t.join()
        if errors:
            raise errors[0]
        return time.perf_counter() - t0, len(ths)

    # calibrate on one pair, then size the sample to about target_s
    t1, _ = run_pairs([(0, 0)])
    total = wl.layers * wl.batch
    n = int(max(1, round(target_s * threads / max(t1, 1e-3))))
    if n >= threads:
        n = (n // threads) * threads
    n = min(n, total)
    pairs = [(l, b) for l in range(wl.layers) for b in range(wl.batch)][:n]
    secs, used = run_pairs(pairs)
    layers = (n + wl.batch - 1) // wl.batch
    tokens = n * wl.total_tokens  # query tokens, summed over the sampled layers
    return {"value": tokens / secs, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "host_cores": {"affinity": affinity, "cpu_count": os.cpu_count(),
                           "omp_num_threads": share or None},
            "sample": f"{n} (layer, sequence) pairs of {total}: sequences in order over "
                      f"{layers} of {wl.layers} layers, all {len(wl.blocks)} scales "
                      f"(quantize+pack then attend each block), {secs:.1f} s on {used} "
                      f"threads (host: {affinity} cores in this process's affinity mask, "
                      f"cpu_count {os.cpu_count()}); tokens/s = query tokens x layers per "
                      f"second, same unit as value"}


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------

def main():
    global PACK_MODE
    args = parse()
    PACK_MODE = args.pack_mode
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the packed-KV path runs on a single MI355X "
              "(it would shard across GPUs by batch or heads with no exchange; that "
              "sharding is not implemented); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import varq_inputs as vi
    import visual_autoregressive_kv_amd as K
    from visual_autoregressive_kv_amd import kvq as kb

    wl = vi.WORKLOADS[args.workload]
    if args.layers:
        wl = wl.with_(layers=min(args.layers, wl.layers))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = K.lib()
    L = K.make_layout(wl.batch, wl.heads, wl.head_dim, wl.bits, wl.blocks, PACK_MODE)
    NB = len(wl.blocks)
    print(f"[bench] {wl.name}: {wl.layers} layers, batch {wl.batch}, {wl.heads}x{wl.head_dim}, "
          f"INT{wl.bits}, {NB} blocks ({wl.total_tokens} tokens); drawing inputs", flush=True)

    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    Kin = [[vi.torch_block(wl, l, "k", j, dev, gen) for j in range(NB)] for l in range(wl.layers)]
    Vin = [[vi.torch_block(wl, l, "v", j, dev, gen) for j in range(NB)] for l in range(wl.layers)]
    Qin = [[vi.torch_block(wl, l, "q", j, dev, gen) for j in range(NB)] for l in range(wl.layers)]
    Out = [[torch.empty(Qin[l][j].shape, dtype=torch.float32, device=dev) for j in range(NB)]
           for l in range(wl.layers)]
    kcs = [K.alloc_cache(L, dev) for _ in range(wl.layers)]
    vcs = [K.alloc_cache(L, dev) for _ in range(wl.layers)]
    torch.cuda.synchronize()

    # HBM copy peak on this machine (context for the roofline)
    a = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    c = torch.empty_like(a)
    for _ in range(3):
        K.kvq_stream_copy(a, c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        K.kvq_stream_copy(a, c)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        K.kvq_stream_read(a, sink)
    e0.record()
    for _ in range(10):
        K.kvq_stream_read(a, sink)
    e1.record()
    torch.cuda.synchronize()
    read_gbps = 10 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, c, sink

    # pre-marshalled calls: the timed loop only crosses into the library
    stream = torch.cuda.current_stream()
    sh = C.c_void_p(stream.cuda_stream)
    Lref = C.byref(L)

    def cache(cd):
        return kb.Cache(cd["codes"].data_ptr(), cd["zero"].data_ptr(), cd["scale"].data_ptr())

    kC = [cache(x) for x in kcs]
    vC = [cache(x) for x in vcs]
    # Decode order: for every block, for every layer, that layer's decode step.
    # Blocks the library fuses (head_dim 64, at most FUSED_MAX_TOKENS tokens) go
    # through kvq_quantize_attend (one launch); larger blocks, and every block of
    # the separate-pass measurement, through kvq_quantize_block then
    # kvq_attend_packed_split (or kvq_attend_packed with --no-split).
    def can_fuse(j):
        return (wl.head_dim == 64 and wl.blocks[j] <= FUSED_MAX_TOKENS
                and (wl.src == "bf16" or wl.blocks[j] <= 32))

    # workspace of kvq_attend_packed_split, sized for the largest block
    split = not args.no_split
    ws_bytes = max(K.kvq_attend_split_workspace(L, j, MAX_SPLITS) for j in range(NB)) if split else 0
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ws_ptr, ws_n = ws.data_ptr(), C.c_uint64(ws.numel())

    call_labels = {}  # id(calls) -> one roctx label per call

    def build_calls(fuse: bool):
        calls = []  # (kind, block, function, arguments), in launch order
        labs = []
        for j in range(NB):
            for l in range(wl.layers):
                labs.extend([f"block {j + 1} layer {l}".encode()] *
                            (1 if fuse and can_fuse(j) else 2))
                # shapes are fixed by construction; checked once here
                assert tuple(Kin[l][j].shape) == (wl.batch, wl.blocks[j], wl.heads, wl.head_dim)
                if fuse and can_fuse(j):
                    calls.append(("fused", j, lib.kvq_quantize_attend,
                                  (Lref, j, kb.BF16, Kin[l][j].data_ptr(), Vin[l][j].data_ptr(),
                                   Qin[l][j].data_ptr(), kC[l], vC[l], C.c_float(0.0),
                                   Out[l][j].data_ptr(), None, sh)))
                    continue
                calls.append(("quant_pack", j, lib.kvq_quantize_block,
                              (Lref, j, kb.BF16, Kin[l][j].data_ptr(), Vin[l][j].data_ptr(),
                               kC[l], vC[l], None, sh)))
                if split:
                    calls.append(("attend", j, lib.kvq_attend_packed_split,
                                  (Lref, j, Qin[l][j].data_ptr(), kC[l], vC[l], C.c_float(0.0),
                                   Out[l][j].data_ptr(), MAX_SPLITS, ws_ptr, ws_n, sh)))
                else:
                    calls.append(("attend", j, lib.kvq_attend_packed,
                                  (Lref, j, Qin[l][j].data_ptr(), kC[l], vC[l], C.c_float(0.0),
                                   Out[l][j].data_ptr(), sh)))
        call_labels[id(calls)] = labs
        return calls

    calls = build_calls(fuse=not args.unfused)
    # one checked call of each kind through the binding before the raw loop
    K.kvq_quantize_block(L, 0, Kin[0][0], Vin[0][0], kcs[0], vcs[0])
    K.kvq_attend_packed(L, 0, Qin[0][0], kcs[0], vcs[0], Out[0][0])
    K.kvq_quantize_attend(L, 0, Kin[0][0], Vin[0][0], Qin[0][0], kcs[0], vcs[0], Out[0][0])

    # roctx ranges (--roctx): one per timed step, one per (block, layer) call
    roctx = None
    if args.roctx:
        roctx = C.CDLL("libroctx64.so")
        roctx.roctxRangePushA.argtypes = [C.c_char_p]
        roctx.roctxRangePushA.restype = C.c_int
        roctx.roctxRangePop.restype = C.c_int

    def step(cs, events=None, mark=None):
        """One decode step; events[c] before call c and events[c + 1] after it
        (a list with every boundary, or a dict with some of them)."""
        def record(k):
            ev = events.get(k) if isinstance(events, dict) else events[k]
            if ev is not None:
                ev.record(stream)

        if mark is not None:
            roctx.roctxRangePushA(mark)
        if events is not None:
            record(0)
        names = call_labels[id(cs)] if mark is not None else None
        for c, (_, _, fn, cargs) in enumerate(cs):
            if names is not None:
                roctx.roctxRangePushA(names[c])
            rc = fn(*cargs)
            if names is not None:
                roctx.roctxRangePop()
            if events is not None:
                record(c + 1)
            if rc:
                raise RuntimeError(f"kvq launch failed (rc={rc}) at call {c}")
        if mark is not None:
            roctx.roctxRangePop()

    for w in range(args.warmup):
        step(calls)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", flush=True)

    def new_events(k, steps):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(k)] for _ in range(steps)]

    # Timed region.  When every launch of a step is of one kind (the fused VAR
    # decode step), one event pair per step gives that kind's average launch
    # duration (the spans of its launches tile the step), so nothing but the
    # library calls runs between the events.  With several kinds, events mark
    # every launch boundary.  Per-block spans then come from a separate pass
    # after the timed region.
    single_kind = len({c[0] for c in calls}) == 1
    evs = new_events(2 if single_kind else len(calls) + 1, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        mark = f"kvq step {s_}".encode() if roctx is not None else None
        if single_kind:
            evs[s_][0].record(stream)
            step(calls, mark=mark)
            evs[s_][1].record(stream)
        else:
            step(calls, evs[s_], mark=mark)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch spans: the timed events (several kinds), or a separate pass
    # with events where the block changes (a block's launches, one per layer,
    # run back to back; an event between every two would add its own cost to
    # each span)
    if single_kind:
        bounds = [c for c in range(len(calls)) if c == 0 or calls[c][1] != calls[c - 1][1]]
        bounds.append(len(calls))
        blk_evs = [{c: torch.cuda.Event(enable_timing=True) for c in bounds}
                   for _ in range(args.steps)]
        for s_ in range(args.steps):
            step(calls, blk_evs[s_])
        torch.cuda.synchronize()
        span_evs = None
    else:
        span_evs = evs

    # per kind: summed event time, launches, algorithmic bytes and flops
    byte_model = {"quant_pack": quant_bytes, "attend": attend_bytes,
                  "fused": lambda w, k: quant_bytes(w, k) + attend_bytes(w, k)}

    def kind_totals(cs, span, steps):
        """Per kind: event time (0 without span events), launches, bytes, flops;
        per kind and block: the per-launch times."""
        kinds, per_block = {}, {}
        for c, (kind, j, _, _) in enumerate(cs):
            ms = (sum(span[s_][c].elapsed_time(span[s_][c + 1]) for s_ in range(steps))
                  if span is not None else 0.0)
            k = kinds.setdefault(kind, {"ms": 0.0, "launches": 0, "bytes": 0, "flops": 0,
                                        "tokens": 0})
            k["ms"] += ms
            k["launches"] += steps
            k["bytes"] += byte_model[kind](wl, j) * steps
            if kind in ("attend", "fused"):
                k["flops"] += attend_flops(wl, j) * steps
                k["tokens"] += wl.batch * wl.blocks[j] * steps
            per_block.setdefault(kind, {}).setdefault(j, []).append(ms / steps)
        return kinds, per_block

    kinds, per_block = kind_totals(calls, span_evs, args.steps)
    if single_kind:  # the kind's time is the timed steps' span
        only = kinds[calls[0][0]]
        only["ms"] = sum(e[0].elapsed_time(e[1]) for e in evs)
        per_block = {calls[0][0]: {}}
        for a, z in zip(bounds[:-1], bounds[1:]):
            ms = sum(blk_evs[s_][a].elapsed_time(blk_evs[s_][z]) for s_ in range(args.steps))
            per_block[calls[0][0]][calls[a][1]] = [ms / args.steps / (z - a)]
    per_block_us = {kind: [round(1e3 * sum(v) / len(v), 2) for _, v in sorted(d.items())]
                    for kind, d in per_block.items()}
    per_block_blocks = {kind: sorted(d) for kind, d in per_block.items()}

    def gbps(k):
        return k["bytes"] / (k["ms"] * 1e-3) / 1e9 if k["ms"] > 0 else 0.0

    ms_per_step = wall * 1e3 / args.steps
    tokens = wl.batch * wl.total_tokens * wl.layers  # query tokens x layers per step
    value = tokens * args.steps / wall

    dominant = max(kinds, key=lambda k: kinds[k]["ms"])
    dk = kinds[dominant]
    avg_bytes, avg_ms = dk["bytes"] / dk["launches"], dk["ms"] / dk["launches"]
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(dominant, wl.name if PACK_MODE == 0 else f"{wl.name}_pm{PACK_MODE}")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "kernel": dominant,
                "blocks": per_block_blocks[dominant],
                "avg_launch_us": round(avg_ms * 1e3, 3),
                "algorithmic_bytes_per_launch": round(avg_bytes),
                "frac_of_copy_peak": round(achieved / copy_gbps, 4),
                "frac_of_read_peak": round(achieved / read_gbps, 4)}

    def stats_of(k, steps):
        g = gbps(k)
        e = {"ms_per_step": round(k["ms"] / steps, 4), "GBps": round(g, 1),
             "pct_hbm_peak": round(100 * g / HBM_PEAK_GBPS, 2)}
        if k["flops"]:
            tf = k["flops"] / (k["ms"] * 1e-3) / 1e12
            e["tokens_per_s"] = round(k["tokens"] / (k["ms"] * 1e-3), 1)  # query tokens x layers
            e["TFLOPs"] = round(tf, 2)
            e["pct_bf16_mfma_peak"] = round(100 * tf / BF16_PEAK_TFLOPS, 2)
        return e

    kind_stats = {}
    for kind, k in sorted(kinds.items()):
        kind_stats[kind] = stats_of(k, args.steps)
        kind_stats[kind]["blocks"] = per_block_blocks[kind]

    # The two passes the metric names, timed separately in the same run after
    # the headline steps: every block as kvq_quantize_block (quantize + pack)
    # then the attention call, events at every launch boundary.
    passes = None
    if "fused" in kinds:
        sep = build_calls(fuse=False)
        step(sep)
        torch.cuda.synchronize()
        sep_steps = max(1, min(args.steps, 5))
        sep_evs = new_events(len(sep) + 1, sep_steps)
        for s_ in range(sep_steps):
            step(sep, sep_evs[s_])
        torch.cuda.synchronize()
        sk, sb = kind_totals(sep, sep_evs, sep_steps)
        passes = {"steps": sep_steps,
                  "timing": "events at every launch boundary (each span: the kernel plus the "
                            "gap since the previous launch)",
                  "quantize_pack": stats_of(sk["quant_pack"], sep_steps),
                  "attention": stats_of(sk["attend"], sep_steps),
                  "per_block_us": {kind: [round(1e3 * sum(v) / len(v), 2)
                                          for _, v in sorted(d.items())]
                                   for kind, d in sb.items()}}
        passes["attention"]["call"] = ("kvq_attend_packed" if not split else
                                       f"kvq_attend_packed_split (max {MAX_SPLITS} key ranges)")
    elif "quant_pack" in kinds and "attend" in kinds:
        passes = {"steps": args.steps, "timing": "the timed steps' events",
                  "quantize_pack": stats_of(kinds["quant_pack"], args.steps),
                  "attention": stats_of(kinds["attend"], args.steps)}

    out = {
        "metric": "packed-KV attention tokens/s + quantize/pack GB/s, % of HBM peak (1 GPU)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "batch": wl.batch,
                   "heads": wl.heads, "head_dim": wl.head_dim, "bits": wl.bits,
                   "schedule": list(wl.blocks), "tokens_per_seq": wl.total_tokens,
                   "pack_mode": PACK_MODE,
                   "parallelism": "none (1 GPU)"},
        "kernels": kind_stats,
        "passes": passes,
        "copy_peak_GBps": round(copy_gbps, 1),
        "read_peak_GBps": round(read_gbps, 1),
        "timing": ("one event pair per timed step; per-block spans from a separate pass with "
                   "events where the block changes (a block's span over its layers' launches "
                   "divided by their number)"
                   if single_kind else "events at every launch boundary of the timed steps"),
        "per_block_us": per_block_us,
        "roofline": roofline,
    }
    if "attend" in kinds:
        out["config"]["attention_call"] = ("kvq_attend_packed" if not split else
                                           f"kvq_attend_packed_split (max {MAX_SPLITS} key ranges)")
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
