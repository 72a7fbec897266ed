#!/usr/bin/env python3
"""Selection-latency benchmark of the pyramid Top-K block selection on one GPU.

A step is one pass of the whole selection stage over one synthetic batch:
pisa_build_pyramid (mean pyramid over all keys) followed by
pisa_select_prefill (the coarse-to-fine walk for every query position and KV
head). Inputs are seeded N(0,1) bf16 Q/K shaped like the selection-latency
benchmark of the pages (B=1, Hq=32, Hkv=2, d=64, C=64, g=2, K=8), resident in
HBM before timing starts; attention over the selected blocks is not part of a
step. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long256k]
                  [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBS = 8000.0


def _hash_sources(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_selection_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def walk_counts(N: int, topk: int, GQ: int, Hkv: int, C: int = 64):
    """Algorithmic work of one prefill selection, from the level geometry alone.

    For each position t the number of candidates at level l is the eligible
    children of min(K, eligible-at-level-above) survivors, capped by the
    eligible node count; a level is scored only when it has more than K.
    A scored upper candidate costs (eligible children) logits per head, a scored
    leaf its eligible raw keys per head; every scored candidate costs one LSE
    (one log) per head. The count assumes the causal frontier node survives
    (exact for full-depth walks). Returns a dict of totals over all walks:
    leaf_logits, leaf_lse, upper_logits, upper_lse, leaf_pairs, and leaf_entries (the
    leaf stage's incidences: one per scored walk and level-2 survivor, whose children form
    one sibling pair).
    """
    t = np.arange(N, dtype=np.int64)
    sizes, span = [], C
    m = -(-N // C)
    while True:
        sizes.append((m, span))
        if m == 1:
            break
        m, span = -(-m // 2), span * 2
    L = len(sizes)
    out = dict(leaf_logits=0.0, leaf_lse=0.0, upper_logits=0.0, upper_lse=0.0, leaf_pairs=0.0, leaf_entries=0.0)
    surv = np.ones(N, np.int64)
    for l in range(L, 0, -1):
        M, sp = sizes[l - 1]
        elig = np.minimum(M, t // sp + 1)
        cand = np.ones(N, np.int64) if l == L else np.minimum(2 * surv, elig)
        scored = cand > topk
        if l >= 2:
            child_elig = np.minimum(sizes[l - 2][0], t // sizes[l - 2][1] + 1)
            n_children = np.minimum(2 * cand, child_elig)
            out["upper_logits"] += float(np.where(scored, n_children, 0).sum()) * GQ * Hkv
            out["upper_lse"] += float(np.where(scored, cand, 0).sum()) * GQ * Hkv
        else:
            keys = np.minimum(cand * C, t + 1)
            out["leaf_logits"] += float(np.where(scored, keys, 0).sum()) * GQ * Hkv
            out["leaf_lse"] += float(np.where(scored, cand, 0).sum()) * GQ * Hkv
            out["leaf_pairs"] += float(np.where(scored, cand, 0).sum()) * Hkv
            out["leaf_entries"] += float(np.where(scored, surv, 0).sum()) * Hkv
        surv = np.where(scored, topk, cand)
    return out


# MI355X transcendental peak: 256 CUs x 32 lanes/clock (v_exp_f32 / v_log_f32 issue at a quarter
# of the 128 lanes/clock of fp32 FMA that the published 157.3 TFLOP/s fp32 vector peak implies)
# x 2.4 GHz. device_ceilings() measures it (exp2 98% of this on an MI355X, profiles/).
TRANSCENDENTAL_PEAK = 256 * 32 * 2.4e9
# fp32 FMA lane operations: 256 CUs x 128 lanes/clock x 2.4 GHz (157.3 TFLOP/s / 2)
VALU_SLOT_PEAK = 256 * 128 * 2.4e9
# dense bf16 MFMA peak of MI355X (published, no sparsity)
MFMA_BF16_PEAK = 2.5e15


# sources of the two walk kernels (a traffic figure is only valid for the code it was taken on)
LEAF_SOURCES = ["cluster.hip", "walk_math.h", "lanes.h", "pisa_device.h"]
UPPER_SOURCES = ["upper.hip", "walk_math.h", "lanes.h", "pisa_device.h"]
ATTN_SOURCES = ["attention.hip", "walk_math.h", "lanes.h", "pisa_device.h"]
FLAT_SOURCES = ["flat.hip", "walk_math.h", "lanes.h", "pisa_device.h"]
COPY_BYTES = 256 << 20          # the calibration copy: 256 MiB read + 256 MiB written


def write_traffic(fetch_dir: str, write_dir: str, workload: str = "long256k") -> None:
    """Summarise two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
    `bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-extras --copy-calibration` into
    profiles/hbm_traffic.json: HBM bytes per launch of the two walk kernels, each counter
    scaled by what it reads for the calibration copy of known size."""
    import csv
    import glob

    def per_kernel(d, counter):
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not path:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = {}
        with open(path[0]) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def find(tab, key, first_only=False):
        hits = [v for k, v in tab.items() if key in k]
        if not hits:
            raise SystemExit(f"kernel {key} not in the counter runs")
        if first_only:   # the calibration copy is the program's first copy; later ones differ in size
            return min(hits[0])[1]
        return float(np.mean([x for _, x in hits[0]]))

    copy_f, copy_w = find(fetch, "copyBuffer", True), find(write, "copyBuffer", True)
    fs, wsc = COPY_BYTES / (copy_f * 1024), COPY_BYTES / (copy_w * 1024)
    out = {"_calibration": {
        "copy_bytes_each_way": COPY_BYTES, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
        "fetch_scale": fs, "write_scale": wsc,
        "command": ("rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o run -- "
                    "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-extras --copy-calibration; "
                    "python3 bench.py --write-traffic <fetch dir> <write dir>")}}
    # the LSE builds (score template argument 0) that the headline step runs
    for key, srcs in (("leaf_cluster_kernel<0, false>", LEAF_SOURCES), ("walk_upper_delta_kernel<16, 0>", UPPER_SOURCES)):
        f_kib, w_kib = find(fetch, key), find(write, key)
        out[f"{key.split('<')[0]}:{workload}"] = {
            "fetch_kib": f_kib, "write_kib": w_kib,
            "bytes_per_launch": f_kib * 1024 * fs + w_kib * 1024 * wsc,
            "source_hash": _hash_sources(srcs)}
    if any("flat_select_kernel" in k for k in fetch):
        f_kib, w_kib = find(fetch, "flat_select_kernel"), find(write, "flat_select_kernel")
        out[f"flat_select_kernel:{workload}"] = {
            "fetch_kib": f_kib, "write_kib": w_kib,
            "bytes_per_launch": f_kib * 1024 * fs + w_kib * 1024 * wsc,
            "source_hash": _hash_sources(FLAT_SOURCES)}
    if any("sparse_attention_kernel" in k for k in fetch):
        f_kib, w_kib = find(fetch, "sparse_attention_kernel"), find(write, "sparse_attention_kernel")
        out[f"sparse_attention_kernel:{workload}"] = {
            "fetch_kib": f_kib, "write_kib": w_kib,
            "bytes_per_launch": f_kib * 1024 * fs + w_kib * 1024 * wsc,
            "source_hash": _hash_sources(ATTN_SOURCES)}
    with open(os.path.join(PROFILES, "hbm_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def measured_traffic(kernel_key: str, src_hash: str):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters (already scaled by
    the copy-kernel calibration), or None when the kernel sources changed since."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(kernel_key)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("bytes_per_launch")


def copy_bandwidth(torch, dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Device-to-device copy rate (GB/s, bytes read + written) of a 1 GiB buffer: the
    achievable HBM bandwidth the measured kernel traffic is compared with."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms / 1e3) / 1e9


def device_ceilings(torch, dev, log, iters: int = 512, grid: int = 2048, reps: int = 5) -> dict:
    """Issue rates measured on this GPU by the probes of libpisa_ceilings.so: v_exp_f32 and
    v_log_f32 (lane results/s), v_fma_f32 (lane ops/s) and v_mfma_f32_16x16x32_bf16 (flop/s).
    Each probe runs 2048 workgroups of 256 threads issuing one instruction kind over
    independent chains; the best of five launches, timed with events on the launch stream."""
    lib = ctypes.CDLL(os.path.join(ROOT, "block_selection_amd", "libpisa_ceilings.so"))
    lib.pisa_ceiling_ops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.pisa_ceiling_ops.restype = ctypes.c_double
    lib.pisa_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.pisa_ceiling_launch.restype = ctypes.c_int
    out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    res = {"probe": f"{grid} workgroups x 256 threads, {iters} loop trips, best of {reps} launches"}
    for kind, name in ((0, "exp2_per_s"), (1, "log2_per_s"), (2, "fma_lane_ops_per_s"), (3, "mfma_bf16_flop_per_s")):
        if lib.pisa_ceiling_launch(kind, iters, grid, ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("ceiling probe launch failed")
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lib.pisa_ceiling_launch(kind, iters, grid, ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        res[name] = lib.pisa_ceiling_ops(kind, iters, grid) / (best / 1e3)
    res["exp2_frac_of_derived_peak"] = res["exp2_per_s"] / TRANSCENDENTAL_PEAK
    res["log2_frac_of_derived_peak"] = res["log2_per_s"] / TRANSCENDENTAL_PEAK
    res["fma_frac_of_derived_peak"] = res["fma_lane_ops_per_s"] / VALU_SLOT_PEAK
    res["mfma_bf16_frac_of_published_peak"] = res["mfma_bf16_flop_per_s"] / MFMA_BF16_PEAK
    log(f"ceilings: exp2 {res['exp2_per_s'] / 1e12:.2f} T/s ({100 * res['exp2_frac_of_derived_peak']:.0f}% of "
        f"{TRANSCENDENTAL_PEAK / 1e12:.2f}), log2 {res['log2_per_s'] / 1e12:.2f} T/s, fma "
        f"{res['fma_lane_ops_per_s'] / 1e12:.1f} T lane-ops/s ({100 * res['fma_frac_of_derived_peak']:.0f}% of "
        f"{VALU_SLOT_PEAK / 1e12:.1f}), bf16 MFMA {res['mfma_bf16_flop_per_s'] / 1e15:.2f} PFLOP/s")
    del out
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, topk: int, n_positions: int, seed: int = 1, gpu_idx=None, gpu_pyr=None):
    """The fp64 oracle on the host cores: the pyramid build over all N keys, then the walks of
    every query position (n_positions <= 0) or of a seeded sample of them. When the GPU's
    selection of the same inputs is given, every walked (position, KV head) is also compared
    with the oracle's under the parity rule (bit-exact, or a near-tie whose mismatch
    validates), and the result is returned as a second dict."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    env_t = os.environ.get("OMP_NUM_THREADS")
    if env_t and env_t.isdigit():
        threads = min(threads, int(env_t))
    N = inp.q.shape[1]
    k0 = inp.k[0]
    if n_positions <= 0 or n_positions >= N:
        ts = np.arange(N, dtype=np.int64)
        q_rows = inp.q[0]
        what = f"every one of the {N} query positions"
    else:
        rng = np.random.default_rng(seed)
        ts = np.sort(rng.choice(N, size=n_positions, replace=False)).astype(np.int64)
        q_rows = np.ascontiguousarray(inp.q[0, ts])
        what = f"{len(ts)} seeded random query positions"
    t0 = time.perf_counter()
    pyr = oracle.build_pyramid(k0, nthreads=threads)
    t1 = time.perf_counter()
    o_idx, o_gap, o_lvl = oracle.walk(q_rows, ts, k0, pyr, topk, nthreads=threads)
    t2 = time.perf_counter()
    build_s, walk_s = t1 - t0, t2 - t1
    per_query = walk_s / len(ts) + build_s / N
    base = {"value": 1.0 / per_query, "unit": "queries/s", "cores": threads, "kind": "oracle", "cpu": _cpu_model(),
            "sample": (f"full fp64 pyramid build over N={N} keys ({build_s:.2f} s) plus walks for {what} x "
                       f"{inp.k.shape[2]} KV heads ({walk_s:.2f} s); queries/s = 1/(walk_s/positions + build_s/N)")}
    if gpu_idx is None:
        return base, None
    return base, parity_against_oracle(gpu_idx[0, ts], ts, inp.q[0], k0, pyr, topk, (o_idx, o_gap, o_lvl), gpu_pyr)


NEAR_TIE = 1e-3


def parity_against_oracle(gpu_idx, ts, q, k, pyr, topk, ora, gpu_pyr=None) -> dict:
    """The parity rule on the benchmark's own output: per (position, KV head) the GPU's index
    set equals the oracle's, or the oracle's walk had a near-tie (K-th and (K+1)-th scores
    closer than 1e-3 at some scored level) and the GPU's set is reachable by resolving those
    ties (oracle.validate; an undecided search counts against parity)."""
    import oracle
    o_idx, o_gap, o_lvl = ora
    eq = np.all(gpu_idx == o_idx, axis=-1)
    near = o_gap < NEAR_TIE
    rec = {"walks": int(eq.size), "all_positions": bool(len(ts) == q.shape[0]), "exact": int(eq.sum()),
           "near_tie_walks": int(near.sum()), "near_tie_rule": "gap < 1e-3 at any scored level",
           "mismatch_valid": 0, "mismatch_invalid": 0, "mismatch_undecided": 0, "mismatch_outside_near_tie": 0}
    lv, cnt = np.unique(o_lvl[near], return_counts=True)
    rec["near_tie_by_level"] = {str(int(a)): int(b) for a, b in zip(lv, cnt)}
    fin = np.isfinite(o_gap)
    rec["min_gap"] = float(o_gap[fin].min()) if fin.any() else None
    for i, j in zip(*np.nonzero(~eq)):
        t = int(ts[i])
        if not near[i, j]:
            rec["mismatch_outside_near_tie"] += 1
            continue
        v = oracle.validate(q[t], t, int(j), k, pyr, topk, gpu_idx[i, j], NEAR_TIE, 200000)
        if v < 0:
            v = oracle.validate(q[t], t, int(j), k, pyr, topk, gpu_idx[i, j], NEAR_TIE, 5000000)
        rec["mismatch_valid" if v == 1 else "mismatch_invalid" if v == 0 else "mismatch_undecided"] += 1
    rec["green"] = (rec["mismatch_invalid"] + rec["mismatch_undecided"] + rec["mismatch_outside_near_tie"]) == 0
    if gpu_pyr is not None:
        # pyramid: per node ||gpu - ref||_2 <= 1e-5 ||ref||_2 and max|gpu - ref| <= 1e-5 max|ref|
        worst = 0.0
        for j in range(pyr.shape[0]):
            ref = pyr[j]
            got = gpu_pyr[0, j, :ref.shape[0]].astype(np.float64)
            diff = got - ref
            n2 = np.linalg.norm(diff, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
            ninf = np.abs(diff).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)
            worst = max(worst, float(n2.max()), float(ninf.max()))
        rec["pyramid_worst_rel"] = worst
        rec["green"] = rec["green"] and worst <= 1e-5
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long256k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-positions", type=int, default=0,
                    help="query positions the CPU oracle walks (0: all of them)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the device-ceiling probes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device-to-device copy first (reference kernel for HBM counters)")
    ap.add_argument("--decode-only", action="store_true", help="time only the decode workload")
    ap.add_argument("--packed-only", action="store_true", help="time only the packed-document workloads")
    ap.add_argument("--batched-only", action="store_true", help="time only the batched (B > 1) workloads")
    ap.add_argument("--flat-exact-only", action="store_true",
                    help="time only the exact flat selection (pisa_select_flat_exact) on the planted 32K workload")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs into profiles/hbm_traffic.json (no GPU)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the selection shards by KV head or query range with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_selection_amd import ops, synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]

    def setup(wl, N=None):
        t0 = time.perf_counter()
        inp = synth.make_prefill(wl, N=N)
        N = inp.q.shape[1]
        dims = ops.make_dims(wl.B, wl.Hq, wl.Hkv, wl.topk, wl.dtype)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

        def dev_t(x):
            if wl.dtype == "bf16":
                return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(x).to(dev)
        q, k = dev_t(inp.q), dev_t(inp.k)
        assert q.dtype == tdt
        pyr = ops.alloc_pyramid(dims, N, dev)
        out = torch.empty((wl.B, N, wl.Hkv, wl.topk), dtype=torch.int32, device=dev)
        ws = ops.alloc_workspace(dims, N, N, device=dev)
        log(f"inputs {wl.name} N={N} ready in {time.perf_counter() - t0:.1f} s")
        return inp, N, dims, q, k, pyr, out, ws

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def hip_events(n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def hip_ms(e0, e1):
        f = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(e0), ctypes.c_void_p(e1)) != 0:
            return float("nan")
        return f.value

    def time_steps(N, dims, q, k, pyr, out, ws, steps, warmup):
        """K timed steps bracketed by synchronisations, with nothing recorded between them (an
        event record inside the step costs the stream about 6 us); then K more steps with HIP
        events on the library's stream around every step's build and select and, inside
        select, the upper-walk and leaf-scoring stages: the per-stage breakdown."""
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            ops.build_pyramid(k, N, N, dims, pyr)
            ops.select_prefill(q, k, pyr, N, N, dims, out, ws)
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(steps):
            ops.build_pyramid(k, N, N, dims, pyr)
            ops.select_prefill(q, k, pyr, N, N, dims, out, ws)
        t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        stage = [hip_events(4) for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            ops.build_pyramid(k, N, N, dims, pyr)
            ev[i][1].record(stream)
            ops.select_prefill_profiled(q, k, pyr, N, N, dims, out, ws, stage[i])
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        build = np.array([e[0].elapsed_time(e[1]) for e in ev])
        walk = np.array([e[1].elapsed_time(e[2]) for e in ev])
        upper = np.array([hip_ms(sg[0], sg[1]) for sg in stage])
        leaf = np.array([hip_ms(sg[2], sg[3]) for sg in stage])
        for sg in stage:
            for e in sg:
                hip.hipEventDestroy(ctypes.c_void_p(e))
        return total_ms, build, walk, upper, leaf

    def time_flat(N, dims, q, k, pyr, steps, warmup):
        """K steps of the flat stage-one selection (pyramid build, whose leaf means it scores, then
        pisa_select_flat), timed like time_steps; returns (ms per step, selection ms per step, out)."""
        stream = torch.cuda.current_stream()
        out_f = torch.empty((dims.B, N, dims.Hkv, dims.topk), dtype=torch.int32, device=dev)
        ws_f = ops.alloc_flat_workspace(dims, N, device=dev)
        for _ in range(warmup):
            ops.build_pyramid(k, N, N, dims, pyr)
            ops.select_flat(q, pyr, N, N, dims, out_f, ws_f)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            ops.build_pyramid(k, N, N, dims, pyr)
            ev[i][1].record(stream)
            ops.select_flat(q, pyr, N, N, dims, out_f, ws_f)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        tot = float(np.mean([e[0].elapsed_time(e[2]) for e in ev]))
        sel = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        del ws_f
        return tot, sel, out_f

    if args.decode_only:
        print(json.dumps({"decode": decode_bench(torch, ops, synth, dev, log)}), flush=True)
        return
    if args.packed_only:
        print(json.dumps({"packed": packed_bench(torch, ops, synth, dev, log)}), flush=True)
        return
    if args.batched_only:
        print(json.dumps({"batched": batched_bench(torch, ops, dev, log)}), flush=True)
        return
    if args.flat_exact_only:
        wl = synth.WORKLOADS["mid_planted"]
        inp, N, dims, q, k, pyr, out, ws = setup(wl)
        ws_x = ops.alloc_flat_exact_workspace(dims, N, device=dev)
        for _ in range(2):
            ops.select_flat_exact(q, k, N, N, dims, out, ws_x)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            ops.select_flat_exact(q, k, N, N, dims, out, ws_x)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        exps = float(N) * (N + 1) / 2 * wl.Hq * wl.B
        res = {"N": N, "ms": ms, "exp_per_s": exps / (ms / 1e3),
               "transcendental_frac": exps / (ms / 1e3) / TRANSCENDENTAL_PEAK}
        log(f"exact flat selection N={N}: {ms:.3f} ms ({res['transcendental_frac']:.3f} of the exp peak)")
        print(json.dumps({"flat_exact": res}), flush=True)
        return

    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 268435456 bytes read + 268435456 bytes written")
        del src, dst
    inp, N, dims, q, k, pyr, out, ws = setup(wl)
    total_ms, build_ms, walk_ms, upper_ms, leaf_ms_steps = time_steps(N, dims, q, k, pyr, out, ws, args.steps,
                                                                      args.warmup)
    ms_per_step = total_ms / args.steps
    value = wl.B * N / (ms_per_step / 1e3)
    # the last timed step's output, for the parity check beside the CPU baseline
    idx_host = out.cpu().numpy()
    pyr_host = pyr.cpu().numpy()
    log(f"N={N}: {ms_per_step:.3f} ms/step (build {build_ms.mean():.3f} ms, select {walk_ms.mean():.3f} ms: "
        f"upper walk {np.mean(upper_ms):.3f} ms, leaf scoring {np.mean(leaf_ms_steps):.3f} ms)")

    GQ = wl.Hq // wl.Hkv
    wc = walk_counts(N, wl.topk, GQ, wl.Hkv)
    clustered = wl.dtype == "bf16"
    kname = "leaf_cluster_kernel" if clustered else "leaf_walk_kernel"
    traffic = measured_traffic(f"{kname}:{wl.name}", _hash_sources(LEAF_SOURCES))
    upper_traffic = measured_traffic(f"walk_upper_delta_kernel:{wl.name}", _hash_sources(UPPER_SOURCES))
    # dominant kernel: the clustered leaf scoring; its duration is measured with HIP events
    # on the stream the library launches on, around a separate timed pass of the same call
    leaf_ms = float(np.mean(leaf_ms_steps))
    transc = wc["leaf_logits"] + wc["leaf_lse"]
    achieved = transc / (leaf_ms / 1e3)
    roofline = {
        "kernel": f"{kname} (exact raw-key LSE of every scored (walk, leaf) pair)",
        "bound": "alu",
        "achieved": achieved / 1e9,
        "peak": TRANSCENDENTAL_PEAK / 1e9,
        "unit": "G transcendental/s (one exp per leaf logit + one log per leaf LSE)",
        "frac": achieved / TRANSCENDENTAL_PEAK,
        "traffic": traffic,
        "algorithmic_per_launch": transc,
        "leaf_pairs_per_launch": wc["leaf_pairs"],
        "launch_ms": leaf_ms,
        # the launch's floor at the transcendental peak (every other instruction overlapped)
        "transcendental_floor_ms": transc / TRANSCENDENTAL_PEAK * 1e3,
    }
    if clustered:
        # the design's query stream: each entry (a walk and one sibling pair of leaves) reads the
        # walk's GQ query rows once; the pair's keys stay in registers for a whole work item
        qbytes = wc["leaf_entries"] * GQ * wl.d * 2
        roofline["query_stream_bytes_per_launch"] = qbytes
        roofline["query_stream_GBs"] = qbytes / (leaf_ms / 1e3) / 1e9
    walk_s = walk_ms.mean() / 1e3
    upper_transc = wc["upper_logits"] + wc["upper_lse"]
    upper_ms = float(np.mean(upper_ms))
    # the second kernel: the coarse-to-fine walk above the leaves (one exp per child logit and
    # one log per candidate LSE, the pairwise form log2(1 + 2^d) of two children)
    roofline_upper = {
        "kernel": "walk_upper_delta_kernel (scored levels above the leaves)",
        "bound": "alu",
        "achieved": upper_transc / (upper_ms / 1e3) / 1e9,
        "peak": TRANSCENDENTAL_PEAK / 1e9,
        "unit": "G transcendental/s",
        "frac": upper_transc / (upper_ms / 1e3) / TRANSCENDENTAL_PEAK,
        "traffic": upper_traffic,
        "algorithmic_per_launch": upper_transc,
        "launch_ms": upper_ms,
    }
    # the peaks above are derived from unit counts and clock; the probes measure what this
    # GPU issues (v_exp_f32 at half the VALU rate, the bf16 MFMA) for the same comparison
    ceil = None if args.no_ceilings else device_ceilings(torch, dev, log)
    if ceil:
        for rf in (roofline, roofline_upper):
            rf["measured_exp2_peak"] = ceil["exp2_per_s"] / 1e9
            rf["frac_of_measured_exp2_peak"] = rf["achieved"] * 1e9 / ceil["exp2_per_s"]
    elt = 2 if wl.dtype == "bf16" else 4
    # the pyramid build is HBM-bound: compulsory bytes = keys read once + every node written once
    build_bytes = wl.B * N * wl.Hkv * wl.d * elt + wl.B * wl.Hkv * ops.pyramid_nodes(dims, N) * wl.d * 4
    # compulsory HBM bytes of the selection: Q read once, K read once, indices written once
    walk_bytes = wl.B * N * (wl.Hq * wl.d * elt + wl.Hkv * wl.d * elt + wl.Hkv * wl.topk * 4)
    hbm = {
        "build_ms": build_ms.mean(),
        "build_compulsory_GBs": build_bytes / (build_ms.mean() / 1e3) / 1e9,
        "build_frac_of_8TBs": build_bytes / (build_ms.mean() / 1e3) / 1e9 / HBM_PEAK_GBS,
        "select_compulsory_GBs": walk_bytes / walk_s / 1e9,
        "select_compulsory_frac_of_8TBs": walk_bytes / walk_s / 1e9 / HBM_PEAK_GBS,
    }
    # the pages' IO ledger (reading note section 5.1: per walk, gK candidate blocks whose queries
    # (GQ heads) and keys (C rows, shared by a tile of Qtile = 4 queries) cross HBM, 2-byte elements)
    ledger = wl.B * N * wl.Hkv * wl.g * wl.topk * wl.d * (GQ + wl.C / 4) * 2
    # the pages' modelled bytes, not bytes that cross HBM: a rate, never a fraction of HBM peak
    hbm["ledger_model_bytes"] = ledger
    hbm["ledger_model_GBs"] = ledger / (ms_per_step / 1e3) / 1e9
    copy_gbs = copy_bandwidth(torch, q.device)
    hbm["device_copy_GBs"] = copy_gbs
    if "query_stream_GBs" in roofline:
        roofline["query_stream_frac_of_copy"] = roofline["query_stream_GBs"] / copy_gbs
    # rocprofv3 FETCH_SIZE / WRITE_SIZE (calibrated) count bytes that miss L2; the Infinity
    # Cache may serve part of them, so they bound the HBM bytes from above
    if traffic:
        hbm["leaf_kernel_l2_miss_GBs_upper_bound"] = traffic / (leaf_ms / 1e3) / 1e9
        hbm["leaf_kernel_l2_miss_frac_of_copy"] = traffic / (leaf_ms / 1e3) / 1e9 / copy_gbs
    if upper_traffic:
        hbm["upper_kernel_l2_miss_GBs_upper_bound"] = upper_traffic / (upper_ms / 1e3) / 1e9
        hbm["upper_kernel_l2_miss_frac_of_copy"] = upper_traffic / (upper_ms / 1e3) / 1e9 / copy_gbs
    work = {
        "select_ms": walk_ms.mean(),
        "upper_walk_ms": upper_ms,
        "leaf_scoring_ms": leaf_ms,
        "all_transcendentals_per_step": transc + upper_transc,
        "select_transcendental_frac": (transc + upper_transc) / walk_s / TRANSCENDENTAL_PEAK,
        "upper_logits": wc["upper_logits"], "leaf_logits": wc["leaf_logits"],
    }

    result = {
        "metric": "Top-K selection latency (ms) + queries/s at N=64K-256K, Hq=32 Hkv=2 d=64",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,1) Q/K rounded to bf16 (numpy default_rng(0))",
        "config": {"workload": f"prefill selection {wl.name}", "B": wl.B, "N": N, "Hq": wl.Hq,
                   "Hkv": wl.Hkv, "d": wl.d, "C": wl.C, "g": wl.g, "K": wl.topk,
                   "step": "pisa_build_pyramid + pisa_select_prefill"},
        "walks_per_s": wl.B * N * wl.Hkv / (ms_per_step / 1e3),
        "latency_ms": {"mean": ms_per_step, "median_build_plus_walk": float(np.median(build_ms + walk_ms)),
                       "min_build_plus_walk": float(np.min(build_ms + walk_ms))},
        "roofline": roofline,
        "roofline_upper": roofline_upper,
        "ceilings": ceil,
        "hbm": hbm,
        "work": work,
    }
    result["attention"] = attention_bench(torch, ops, synth, wl, N, dims, q, k, out, args.steps, args.warmup,
                                          ms_per_step, log)
    if not args.no_extras:
        # the pages' two ablation scores on the same workload and launch configuration
        variants = {}
        for sc in ("mean", "mean_half_var"):
            dims_s = ops.make_dims(wl.B, wl.Hq, wl.Hkv, wl.topk, wl.dtype, score=sc)
            tot_s, b_s, wk_s, up_s, lf_s = time_steps(N, dims_s, q, k, pyr, out, ws, 10, 3)
            variants[sc] = {"ms_per_step": tot_s / 10, "queries_per_s": wl.B * N / (tot_s / 10 / 1e3),
                            "upper_walk_ms": float(up_s.mean()), "leaf_scoring_ms": float(lf_s.mean())}
            log(f"score {sc}: {tot_s / 10:.3f} ms/step (upper walk {up_s.mean():.3f} ms, "
                f"leaf scoring {lf_s.mean():.3f} ms)")
        result["score_variants"] = variants
        # larger budgets on the same inputs (the pages' continued-pretraining setting uses K = 32)
        ksweep = {}
        for kk in (16, 32):
            dims_k = ops.make_dims(wl.B, wl.Hq, wl.Hkv, kk, wl.dtype)
            out_k = torch.empty((wl.B, N, wl.Hkv, kk), dtype=torch.int32, device=dev)
            ws_k = ops.alloc_workspace(dims_k, N, N, device=dev)
            tot_k, b_k, wk_k, up_k, lf_k = time_steps(N, dims_k, q, k, pyr, out_k, ws_k, 10, 3)
            ksweep[f"K{kk}"] = {"ms_per_step": tot_k / 10, "queries_per_s": wl.B * N / (tot_k / 10 / 1e3),
                                "upper_walk_ms": float(up_k.mean()), "leaf_scoring_ms": float(lf_k.mean())}
            log(f"K={kk}: {tot_k / 10:.3f} ms/step (upper walk {up_k.mean():.3f} ms, leaf scoring {lf_k.mean():.3f} ms)")
            del out_k, ws_k
        result["topk_sweep"] = ksweep
    # the flat stage-one selection (every leaf summary scored) at the headline length, beside
    # the pyramid walk: a dense contraction (one dot product of the group-summed query with each
    # eligible leaf mean) feeding a streaming top K
    ftot, fsel, out_flat = time_flat(N, dims, q, k, pyr, 10, 3)
    del out_flat
    n_scores = float(np.minimum(np.arange(N) // wl.C + 1, -(-N // wl.C)).sum()) * wl.B * wl.Hkv
    flat_flops = n_scores * wl.d * 2
    traffic_flat = measured_traffic(f"flat_select_kernel:{wl.name}", _hash_sources(FLAT_SOURCES))
    flat = {args.workload: {"N": N, "pyramid_step_ms": ms_per_step, "flat_step_ms": ftot,
                            "flat_select_ms": fsel, "pyramid_over_flat": ms_per_step / ftot,
                            "roofline": {"kernel": "flat_select_kernel (+ flat_planes_kernel)", "bound": "mfma",
                                         "achieved": flat_flops / (fsel / 1e3) / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
                                         "unit": "TFLOP/s", "frac": flat_flops / (fsel / 1e3) / MFMA_BF16_PEAK,
                                         "traffic": traffic_flat, "algorithmic_per_launch": flat_flops,
                                         "scores_per_launch": n_scores,
                                         "algorithmic_model": "one 64-dim dot product per (position, KV head, "
                                                              "eligible leaf); the kernel issues three bf16 products "
                                                              "per dot product (hi/lo split)"}}}
    log(f"flat stage-one selection at N={N}: {ftot:.3f} ms per step ({fsel:.3f} ms selection), pyramid walk "
        f"{ms_per_step:.3f} ms")
    result["flat"] = flat
    del q, k, pyr, out, ws

    if not args.no_extras:
        # the headline shape at other lengths (the pages' benchmark spans short sequences, where
        # selection is launch-bound, to 256K), the flat selection beside it
        sweep = {}
        for name, n2 in (("N4096", 4096), ("N16384", 16384), ("N32768", 32768), ("long64k", None),
                         ("long128k", None)):
            if name == args.workload:
                continue
            w2 = synth.WORKLOADS[name] if n2 is None else wl
            _, N2, d2, q2, k2, p2, o2, ws2 = setup(w2, N=n2)
            tot2, b2, wk2, _, _ = time_steps(N2, d2, q2, k2, p2, o2, ws2, 10, 3)
            sweep[name] = {"N": N2, "ms": tot2 / 10, "queries_per_s": N2 / (tot2 / 10 / 1e3),
                           "build_ms": float(b2.mean()), "walk_ms": float(wk2.mean())}
            ftot, fsel, _ = time_flat(N2, d2, q2, k2, p2, 10, 3)
            flat[name] = {"N": N2, "pyramid_step_ms": tot2 / 10, "flat_step_ms": ftot,
                          "flat_select_ms": fsel, "pyramid_over_flat": (tot2 / 10) / ftot}
            del q2, k2, p2, o2, ws2
        result["sweep"] = sweep
        log("flat stage-one selection beside the pyramid walk (ms per step, build included): " +
            ", ".join(f"N={v['N']}: {v['flat_step_ms']:.3f} vs {v['pyramid_step_ms']:.3f}" for v in flat.values()))
        result["planted"] = planted_bench(torch, ops, synth, setup, time_steps, log)
        result["decode"] = decode_bench(torch, ops, synth, dev, log)
        result["packed"] = packed_bench(torch, ops, synth, dev, log)
        result["batched"] = batched_bench(torch, ops, dev, log)

    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline, then comparing the timed steps' selection with it")
        result["cpu_baseline"], par = cpu_baseline(inp, wl.topk, args.cpu_positions, gpu_idx=idx_host,
                                                   gpu_pyr=pyr_host)
        if par is not None:
            result["parity"] = par
            log(f"parity: {par['walks']} walks, {par['exact']} bit-exact, {par['near_tie_walks']} near-tie, "
                f"mismatches valid {par['mismatch_valid']} / invalid {par['mismatch_invalid']} / undecided "
                f"{par['mismatch_undecided']} / outside a near-tie {par['mismatch_outside_near_tie']}; "
                f"pyramid worst {par.get('pyramid_worst_rel', float('nan')):.2e}")
    print(json.dumps(result), flush=True)


def planted_bench(torch, ops, synth, setup, time_steps, log, n_flat: int = 96, seed: int = 5):
    """The 32K workload with 64 planted leaf blocks: time, and recall of the planted blocks
    (mean over walks at t >= K*C with an eligible planted block of |selected & planted| /
    min(K, eligible planted)); beside it the chance level and, on a seeded sample of positions,
    flat exact top-K by raw-key LogSumExp over all eligible leaves (numpy, fp64): its planted
    recall, its overlap with the walk's selection, and the block-selection diagnostic against the
    K blocks of most attention mass (full softmax over keys <= t, mean over the group's heads):
    Recall@K and the ratio of the selection's mass to theirs."""
    wl = synth.WORKLOADS["mid_planted"]
    inp, N, dims, q, k, pyr, out, ws = setup(wl)
    tot, b, wk, _, _ = time_steps(N, dims, q, k, pyr, out, ws, 10, 3)
    idx = out.cpu().numpy()[0]
    planted = np.sort(inp.planted)
    K, C = wl.topk, wl.C
    ts = np.arange(K * C, N)
    n_elig = ts // C + 1
    p_elig = np.searchsorted(planted, n_elig)           # planted blocks with index < n_elig
    keep = p_elig > 0
    ts, n_elig, p_elig = ts[keep], n_elig[keep], p_elig[keep]
    hit = np.isin(idx[ts], planted).sum(axis=2)          # [positions, Hkv]
    denom = np.minimum(K, p_elig)[:, None]
    recall = float((hit / denom).mean())
    chance = float((K * p_elig / n_elig / np.minimum(K, p_elig)).mean())
    # the flat stage-one selection (pisa_select_flat: every leaf mean scored) on the same inputs
    out_f = torch.empty_like(out)
    ops.build_pyramid(k, N, N, dims, pyr)
    ops.select_flat(q, pyr, N, N, dims, out_f, ops.alloc_flat_workspace(dims, N, device=q.device))
    fidx = out_f.cpu().numpy()[0]
    recall_flat_mean = float((np.isin(fidx[ts], planted).sum(axis=2) / denom).mean())
    # flat exact top-K at every position on the GPU (pisa_select_flat_exact: every eligible leaf
    # scored by its raw-key LogSumExp, the walk's leaf arithmetic), timed on the library's stream
    stream = torch.cuda.current_stream()
    out_x = torch.empty_like(out)
    ws_x = ops.alloc_flat_exact_workspace(dims, N, device=q.device)
    ops.select_flat_exact(q, k, N, N, dims, out_x, ws_x)
    torch.cuda.synchronize()
    ex0, ex1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ex0.record(stream)
    for _ in range(3):
        ops.select_flat_exact(q, k, N, N, dims, out_x, ws_x)
    ex1.record(stream)
    torch.cuda.synchronize()
    exact_ms = ex0.elapsed_time(ex1) / 3
    # its algorithmic exponentials: one per (query head, key <= t) at every position
    exact_exps = float(N) * (N + 1) / 2 * wl.Hq * wl.B
    xidx = out_x.cpu().numpy()[0]
    recall_exact = float((np.isin(xidx[ts], planted).sum(axis=2) / denom).mean())
    # overlap Recall@K against flat exact top-K at every position with more than K eligible leaves
    # (both sets then hold K blocks)
    tk = np.arange(K * C, N)

    def overlap_all(sel):
        a, b = sel[tk], xidx[tk]
        return float(((a[..., :, None] == b[..., None, :]).any(axis=-1).sum(axis=-1) / K).mean())

    overlap_walk_all, overlap_flat_mean_all = overlap_all(idx), overlap_all(fidx)
    del out_x, ws_x
    # flat exact top-K on a sample
    rng = np.random.default_rng(seed)
    sample = np.sort(rng.choice(ts, size=min(n_flat, len(ts)), replace=False))
    GQ = wl.Hq // wl.Hkv
    qf, kf = inp.q[0].astype(np.float64), inp.k[0].astype(np.float64)
    flat, walk, overlap, mref, mratio, mratio_flat, mratio_rand = [], [], [], [], [], [], []
    mratio_fm, overlap_fm = [], []
    for t in sample:
        nl = t // C + 1
        pe = planted[planted < nl]
        for j in range(wl.Hkv):
            z = qf[t, j * GQ:(j + 1) * GQ] @ kf[:t + 1, j].T / np.sqrt(wl.d)       # [GQ, t+1]
            zp = np.full((GQ, nl * C), -np.inf)
            zp[:, :t + 1] = z
            zp = zp.reshape(GQ, nl, C)
            m = zp.max(axis=2, keepdims=True)
            lse_h = np.log(np.exp(zp - m).sum(axis=2)) + m[:, :, 0]                 # [GQ, nl]
            lse = lse_h.sum(axis=0)                                                   # [nl]
            top = np.argsort(-lse, kind="stable")[:K]
            d = min(K, len(pe))
            flat.append(len(set(top.tolist()) & set(pe.tolist())) / d)
            walk.append(len(set(idx[t, j].tolist()) & set(pe.tolist())) / d)
            sel = [x for x in idx[t, j].tolist() if x >= 0]
            overlap.append(len(set(sel) & set(top.tolist())) / min(K, nl))
            # attention mass of each block (full softmax over keys <= t, mean over the group's
            # heads); the reference set is the K blocks of largest mass
            top_h = lse_h.max(axis=1, keepdims=True)
            mass = (np.exp(lse_h - top_h) / np.exp(lse_h - top_h).sum(axis=1, keepdims=True)).mean(axis=0)
            ref = np.argsort(-mass, kind="stable")[:K]
            mref.append(len(set(sel) & set(ref.tolist())) / min(K, nl))
            mratio.append(float(mass[sel].sum() / mass[ref].sum()))
            mratio_flat.append(float(mass[top].sum() / mass[ref].sum()))
            mratio_rand.append(float(mass[rng.choice(nl, K, replace=False)].sum() / mass[ref].sum()))
            fsel = [x for x in fidx[t, j].tolist() if x >= 0]
            mratio_fm.append(float(mass[fsel].sum() / mass[ref].sum()))
            overlap_fm.append(len(set(fsel) & set(top.tolist())) / min(K, nl))
    res = {"N": N, "ms": tot / 10, "queries_per_s": N / (tot / 10 / 1e3), "planted_recall": recall,
           "chance_recall": chance, "flat_exact_recall_sample": float(np.mean(flat)),
           "walk_recall_same_sample": float(np.mean(walk)), "sample_positions": int(len(sample)),
           "overlap_recall_at_K_vs_flat_exact": float(np.mean(overlap)),
           "recall_at_K_vs_attention_mass_top_K": float(np.mean(mref)),
           "attention_mass_ratio": float(np.mean(mratio)),
           "attention_mass_ratio_flat_exact": float(np.mean(mratio_flat)),
           "attention_mass_ratio_random_K": float(np.mean(mratio_rand)),
           "flat_mean_summary_planted_recall": recall_flat_mean,
           "flat_mean_summary_attention_mass_ratio": float(np.mean(mratio_fm)),
           "flat_mean_summary_overlap_vs_flat_exact": float(np.mean(overlap_fm)),
           "flat_exact_gpu": {"ms": exact_ms, "planted_recall": recall_exact,
                              "exp_per_s": exact_exps / (exact_ms / 1e3),
                              "transcendental_frac": exact_exps / (exact_ms / 1e3) / TRANSCENDENTAL_PEAK,
                              "walk_overlap_recall_at_K": overlap_walk_all,
                              "flat_mean_summary_overlap_recall_at_K": overlap_flat_mean_all,
                              "positions": int(len(tk))}}
    log(f"planted 32K: {res['ms']:.3f} ms, planted recall {recall:.3f} (chance {chance:.3f}; on "
        f"{len(sample)} sampled positions flat exact top-K {res['flat_exact_recall_sample']:.3f}, the walk "
        f"{res['walk_recall_same_sample']:.3f}; overlap with flat exact top-K "
        f"{res['overlap_recall_at_K_vs_flat_exact']:.3f}; against the K blocks of most attention mass: "
        f"recall {res['recall_at_K_vs_attention_mass_top_K']:.3f}, mass ratio {res['attention_mass_ratio']:.4f} "
        f"(flat exact top-K {res['attention_mass_ratio_flat_exact']:.4f}, K random eligible blocks "
        f"{res['attention_mass_ratio_random_K']:.4f})); flat stage-one selection by leaf means: planted recall "
        f"{recall_flat_mean:.3f}, mass ratio {res['flat_mean_summary_attention_mass_ratio']:.4f}")
    log(f"flat exact top-K on the GPU at all {len(tk)} positions with more than K eligible blocks: "
        f"{exact_ms:.3f} ms, planted recall {recall_exact:.3f}; overlap Recall@K against it: the walk "
        f"{overlap_walk_all:.4f}, the flat leaf-mean selection {overlap_flat_mean_all:.4f}")
    del q, k, pyr, out, ws, out_f
    return res


def attention_bench(torch, ops, synth, wl, N, dims, q, k, idx, steps, warmup, select_ms, log):
    """Stage two on the step's own selection: attention of every query head over the keys of
    its KV head's selected blocks (pisa_sparse_attention), timed on its own with CUDA events
    on the stream the library launches on."""
    dev = q.device
    v = torch.from_numpy(synth.bf16_bits(synth.make_values(wl.B, N, wl.Hkv, seed=wl.seed)).view(np.int16)).view(
        torch.bfloat16).to(dev)
    out = torch.empty((wl.B, N, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    ws = ops.alloc_attention_workspace(dims, N, N, device=dev)
    for _ in range(warmup):
        ops.sparse_attention(q, k, v, idx, N, N, dims, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ops.sparse_attention(q, k, v, idx, N, N, dims, out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the pages' stage-two cost model: each query reads the keys and values of its (at most K)
    # selected blocks; plus its queries and its output rows
    GQ = wl.Hq // wl.Hkv
    nsel = int(np.minimum(wl.topk, np.arange(N) // wl.C + 1).sum()) * wl.B * wl.Hkv
    blk_bytes = wl.C * wl.d * 2 * 2
    walks = wl.B * N * wl.Hkv
    alg = nsel * blk_bytes + walks * GQ * wl.d * (2 + 4)
    traffic = measured_traffic(f"sparse_attention_kernel:{wl.name}", _hash_sources(ATTN_SOURCES))
    flops = nsel * GQ * wl.C * wl.d * 2 * 2
    # compulsory bytes of the call: Q, K and V once, the indices once, the fp32 output once
    compulsory = walks * GQ * wl.d * 2 + 2 * walks * wl.d * 2 + walks * wl.topk * 4 + walks * GQ * wl.d * 4
    res = {"ms": ms, "queries_per_s": wl.B * N / (ms / 1e3),
           "step_plus_attention_ms": select_ms + ms, "selection_share": select_ms / (select_ms + ms),
           "roofline": {"kernel": "sparse_attention_kernel (+ vt_tiles_kernel, the per-call V re-layout)",
                        "bound": "hbm", "achieved": compulsory / (ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": compulsory / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                        "traffic": None,
                        "algorithmic_per_launch": compulsory,
                        "algorithmic_model": "compulsory bytes: Q (bf16), K and V (bf16) and the indices read "
                                             "once, the fp32 output written once",
                        "mfma_tflops": flops / (ms / 1e3) / 1e12,
                        "mfma_frac_of_bf16_peak": flops / (ms / 1e3) / MFMA_BF16_PEAK,
                        # what the kernel actually moves: every query gathers its K blocks' keys and
                        # values; L2 and the Infinity Cache serve part of it, so neither figure is HBM
                        "per_query_block_reads_per_launch": alg,
                        "per_query_block_reads_GBs": alg / (ms / 1e3) / 1e9,
                        "l2_miss_bytes_per_launch": traffic,
                        "l2_miss_GBs": None if not traffic else traffic / (ms / 1e3) / 1e9}}
    log(f"attention over the selected blocks: {ms:.3f} ms ({res['roofline']['per_query_block_reads_GBs']:.0f} GB/s "
        f"of per-query block reads, {res['roofline']['mfma_tflops']:.0f} TFLOP/s on the MFMA); selection is "
        f"{100 * res['selection_share']:.0f}% of selection + attention")
    del v, out, ws
    return res


def decode_bench(torch, ops, synth, dev, log):
    """Decode workload: 131072 prebuilt keys, then 256 sequential refresh+select steps (K=32)."""
    wl = synth.WORKLOADS["decode128k"]
    inp = synth.make_decode(wl)
    N0, steps = wl.N, wl.decode_steps
    cap = N0 + steps
    dims = ops.make_dims(1, wl.Hq, wl.Hkv, wl.topk, "bf16")

    def dev_t(x):
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    kc = np.zeros((1, cap, wl.Hkv, wl.d), np.float32)
    kc[0, :N0] = inp.k_ctx[0]
    k_cache = dev_t(kc)
    k_new, q_new = dev_t(inp.k_new), dev_t(inp.q_new)
    pyr = ops.alloc_pyramid(dims, cap, dev)
    out = torch.empty((1, wl.Hkv, wl.topk), dtype=torch.int32, device=dev)
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True, device=dev)
    kn = [k_new[s].contiguous() for s in range(steps)]
    qn = [q_new[s].contiguous() for s in range(steps)]
    stream = torch.cuda.current_stream()
    times = []
    for rep in range(3):   # first repetition is warm-up
        ops.build_pyramid(k_cache, N0, cap, dims, pyr)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for s in range(steps):
            ops.decode_update_select(qn[s], kn[s], k_cache, pyr, N0 + s, cap, dims, out, ws)
            ev[s + 1].record(stream)
        torch.cuda.synchronize()
        if rep:
            times.append([ev[s].elapsed_time(ev[s + 1]) * 1e3 for s in range(steps)])
    # launch floor: an empty kernel (torch's zero-cycle sleep) enqueued and timed the same way
    fl = []
    for rep in range(2):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for s in range(steps):
            torch.cuda._sleep(0)
            ev[s + 1].record(stream)
        torch.cuda.synchronize()
        if rep:
            fl = [ev[s].elapsed_time(ev[s + 1]) * 1e3 for s in range(steps)]
    # the same steps, each followed by attention over its selection (pisa_decode_attention,
    # which also appends the step's value row)
    vals = synth.make_values(1, cap, wl.Hkv, seed=wl.seed)
    v_cache = dev_t(vals)
    vn = [v_cache[0, N0 + s].unsqueeze(0).contiguous() for s in range(steps)]
    att = torch.empty((1, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    wsd = ops.alloc_decode_attention_workspace(dims, device=dev)
    att_times = []
    for rep in range(2):
        ops.build_pyramid(k_cache, N0, cap, dims, pyr)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for s in range(steps):
            ops.decode_update_select(qn[s], kn[s], k_cache, pyr, N0 + s, cap, dims, out, ws)
            ops.decode_attention(qn[s], vn[s], k_cache, v_cache, out, N0 + s, cap, dims, att, wsd)
            ev[s + 1].record(stream)
        torch.cuda.synchronize()
        if rep:
            att_times = [ev[s].elapsed_time(ev[s + 1]) * 1e3 for s in range(steps)]
    # the same steps with K = 8 (the budget of the pages' selection-latency setting)
    dims8 = ops.make_dims(1, wl.Hq, wl.Hkv, 8, "bf16")
    out8 = torch.empty((1, wl.Hkv, 8), dtype=torch.int32, device=dev)
    ws8 = ops.alloc_workspace(dims8, 1, cap, is_decode=True, device=dev)
    k8_times = []
    for rep in range(2):
        ops.build_pyramid(k_cache, N0, cap, dims8, pyr)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for s in range(steps):
            ops.decode_update_select(qn[s], kn[s], k_cache, pyr, N0 + s, cap, dims8, out8, ws8)
            ev[s + 1].record(stream)
        torch.cuda.synchronize()
        if rep:
            k8_times = [ev[s].elapsed_time(ev[s + 1]) * 1e3 for s in range(steps)]
    per = np.array(times)
    res = {"context": N0, "steps": steps, "K": wl.topk, "us_per_step_mean": float(per.mean()),
           "us_per_step_K8": float(np.mean(k8_times)),
           "us_per_step_with_attention": float(np.mean(att_times)),
           "empty_kernel_launch_us": float(np.mean(fl)),
           "us_per_step_median": float(np.median(per)), "us_per_step_p90": float(np.percentile(per, 90)),
           "steps_per_s": 1e6 / float(per.mean())}
    log(f"decode: {res['us_per_step_mean']:.1f} us/step, {res['us_per_step_with_attention']:.1f} us/step with "
        f"attention over the selected blocks; K=8: {res['us_per_step_K8']:.1f} us/step")
    return res


def batched_bench(torch, ops, dev, log, seed: int = 11):
    """Batches of independent sequences (B > 1): prefill of 4 x 65536 positions (the
    headline's token count, K = 8) and decoding steps for 64 sequences of 32768 keys at
    once (K = 32). Inputs: standard normal draws on the device from a seeded generator,
    rounded to bf16 (timing only; batches are checked element by element against the
    oracle by the tests)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn(*shape):
        return torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    res = {}
    B, N = 4, 65536
    dims = ops.make_dims(B, 32, 2, 8, "bf16")
    q, k = randn(B, N, 32, 64), randn(B, N, 2, 64)
    pyr = ops.alloc_pyramid(dims, N, dev)
    out = torch.empty((B, N, 2, 8), dtype=torch.int32, device=dev)
    ws = ops.alloc_workspace(dims, N, N, device=dev)
    for _ in range(3):
        ops.build_pyramid(k, N, N, dims, pyr)
        ops.select_prefill(q, k, pyr, N, N, dims, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        ops.build_pyramid(k, N, N, dims, pyr)
        ops.select_prefill(q, k, pyr, N, N, dims, out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    res["prefill_4x65536"] = {"B": B, "N": N, "K": 8, "ms_per_step": ms, "queries_per_s": B * N / (ms / 1e3)}
    del q, k, pyr, out, ws

    B, N0, steps, K = 64, 32768, 64, 32
    cap = N0 + steps
    dims = ops.make_dims(B, 32, 2, K, "bf16")
    k_cache = torch.zeros((B, cap, 2, 64), dtype=torch.bfloat16, device=dev)
    k_cache[:, :N0] = randn(B, N0, 2, 64)
    k_new, q_new = randn(steps, B, 2, 64), randn(steps, B, 32, 64)
    pyr = ops.alloc_pyramid(dims, cap, dev)
    out = torch.empty((B, 2, K), dtype=torch.int32, device=dev)
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True, device=dev)
    per = []
    for rep in range(3):   # first repetition is warm-up; each starts from the same prebuilt pyramid
        ops.build_pyramid(k_cache, N0, cap, dims, pyr)
        torch.cuda.synchronize()
        e0.record()
        for s_ in range(steps):
            ops.decode_update_select(q_new[s_], k_new[s_], k_cache, pyr, N0 + s_, cap, dims, out, ws)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            per.append(e0.elapsed_time(e1) * 1e3 / steps)
    us = float(np.mean(per))
    # the same steps, each followed by attention over its selection (which appends the value row)
    v_cache = torch.zeros_like(k_cache)
    v_cache[:, :N0] = randn(B, N0, 2, 64)
    v_new = randn(steps, B, 2, 64)
    att = torch.empty((B, 32, 64), dtype=torch.float32, device=dev)
    wsd = ops.alloc_decode_attention_workspace(dims, device=dev)
    per_att = []
    for rep in range(2):
        ops.build_pyramid(k_cache, N0, cap, dims, pyr)
        torch.cuda.synchronize()
        e0.record()
        for s_ in range(steps):
            ops.decode_update_select(q_new[s_], k_new[s_], k_cache, pyr, N0 + s_, cap, dims, out, ws)
            ops.decode_attention(q_new[s_], v_new[s_], k_cache, v_cache, out, N0 + s_, cap, dims, att, wsd)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            per_att.append(e0.elapsed_time(e1) * 1e3 / steps)
    us_att = float(np.mean(per_att))
    res["decode_64x32768"] = {"B": B, "context": N0, "K": K, "steps": steps, "us_per_step": us,
                              "sequence_steps_per_s": B / (us / 1e6), "us_per_step_with_attention": us_att,
                              "sequence_steps_per_s_with_attention": B / (us_att / 1e6)}
    del k_cache, v_cache, k_new, v_new, q_new, pyr, out, ws, att, wsd
    log(f"batched: prefill 4 x 65536 {ms:.3f} ms ({res['prefill_4x65536']['queries_per_s'] / 1e6:.1f} M queries/s); "
        f"decode 64 sequences x 32768 keys {us:.1f} us/step ({res['decode_64x32768']['sequence_steps_per_s'] / 1e6:.2f} M "
        f"sequence-steps/s), {us_att:.1f} us/step with attention over the selected blocks")
    return res


def packed_bench(torch, ops, synth, dev, log):
    """Packed documents (varlen): one pisa_build_pyramid_packed + pisa_select_prefill_packed per
    step over a pack of random-length documents, next to the same documents selected one call
    per document through the single-sequence entry points."""
    res = {}
    for name, T, mean_len, K in (("packed256k_mean8k", 262144, 8192.0, 8), ("packed16k_k32", 16384, 2048.0, 32)):
        v = synth.make_varlen(T, 32, 2, "bf16", mean_len=mean_len, seed=1)
        D = len(v.cu) - 1
        dims = ops.make_dims(1, 32, 2, K, "bf16")

        def dev_t(x):
            return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
        q, k = dev_t(v.q), dev_t(v.k)
        cu = torch.from_numpy(v.cu.astype(np.int32)).to(dev)
        pyr = ops.alloc_pack_pyramid(dims, T, D, dev)
        out = torch.empty((T, 2, K), dtype=torch.int32, device=dev)
        ws = ops.alloc_pack_workspace(dims, T, D, dev)

        def packed_step():
            ops.build_pyramid_packed(k, cu, dims, pyr)
            ops.select_prefill_packed(q, k, pyr, cu, dims, out, ws)
        # the same documents, one build + select per document
        lens = np.diff(v.cu).astype(np.int64)
        nmax = int(lens.max())
        pyr1 = ops.alloc_pyramid(dims, nmax, dev)
        ws1 = ops.alloc_workspace(dims, nmax, nmax, device=dev)
        out1 = torch.empty((T, 2, K), dtype=torch.int32, device=dev)
        docs = [(int(v.cu[j]), int(v.cu[j + 1])) for j in range(D) if v.cu[j + 1] > v.cu[j]]

        def per_doc_step():
            for lo, hi in docs:
                n = hi - lo
                p1 = pyr1.view(-1)[: 2 * ops.pyramid_nodes(dims, n) * 64].view(1, 2, -1, 64)
                ops.build_pyramid(k[lo:hi], n, n, dims, p1)
                ops.select_prefill(q[lo:hi], k[lo:hi], p1, n, n, dims, out1[lo:hi], ws1)
        row = {"T": T, "documents": D, "mean_len": mean_len, "K": K}
        for label, fn in (("packed", packed_step), ("per_document_calls", per_doc_step)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            steps = 10
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            row[label + "_ms"] = ms
            row[label + "_queries_per_s"] = T / (ms / 1e3)
        row["same_selection"] = bool(torch.equal(out, out1))
        log(f"{name}: D={D} packed {row['packed_ms']:.3f} ms, per-document calls "
            f"{row['per_document_calls_ms']:.3f} ms, identical={row['same_selection']}")
        res[name] = row
        del q, k, cu, pyr, out, ws, pyr1, ws1, out1
    return res


if __name__ == "__main__":
    main()
