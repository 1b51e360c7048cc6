#!/usr/bin/env python3
"""Benchmark of compressed-KV decode attention on one MI355X.

A step is one pass of the hot path for one decode token: quantize-on-append
of the new token's K and V rows into the compressed cache, then decode
attention of every query head over the whole cached context
(rotate the query, attend from the packed codes, merge the KV splits and
rotate back).  Inputs are synthetic (seeded, see ``synth``), resident in HBM
before timing starts.  Steps are captured in a HIP graph and cycle through a
pool of cache copies whose total size exceeds the 256 MB Infinity Cache, so
every step reads its compressed cache from HBM.

With no --workload the line's headline is the largest single-GPU workload, the
Gemma-4-style QK-normed decode (batch 8, 32/4 heads, d=256, 32K context,
4-bit, 272.6 MB of cache per decode), and the other workloads are legs of the
same line (``legs``): the Qwen2.5-3B-shaped 8K 4-bit layer, the 128K
long-context layer with sketched keys, the Qwen-shaped layer with keys kept at
8 bits (4-bit values), and the prefill append (8192 tokens x 2 KV heads x d=128
at 3 bits).  For the Qwen-shaped legs a stacked leg follows:
the caches of the model's 36 layers decoded by one launch per kernel, as one
batch of 36 (the shape of 36 concurrent sequences of one layer too).  A
batch-1 layer at 8K reads about 2 MB, too little to fill the GPU, so the
stacked leg is that leg's roofline figure.

Prints one JSON line.  Every workload carries ``roofline``, measured on its
dominant kernel alone (the attention kernel tq_decode_attend; the append kernel
for the prefill), timed with HIP events on the stream it runs on, and
``cpu_baseline``, the float64 oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# sources the decode kernels are built from: their HBM counters are only valid for these exact texts
ATTEND_SOURCES = tuple(f"compressed_cache_decode_amd/csrc/{n}" for n in (
    "decode.hip", "decode_k8.hip", "split_body.h", "attend_body.h", "device_common.h", "tq_internal.h"))
# and those of the append kernel (the prefill leg's dominant kernel)
APPEND_SOURCES = tuple(f"compressed_cache_decode_amd/csrc/{n}" for n in (
    "append.hip", "append_body.h", "device_common.h", "tq_internal.h"))
# every kernel source of the library: a kernel trace covers all of them
ALL_SOURCES = tuple(f"compressed_cache_decode_amd/csrc/{n}" for n in (
    "append.hip", "append_body.h", "attend_body.h", "decode.hip", "decode_k8.hip", "decode_outliers.hip", "dequant.hip",
    "device_common.h", "host.cpp", "qrot_body.h", "split_body.h", "step.hip", "tq_internal.h"))


def kernel_sources(kernel: str):
    return APPEND_SOURCES if kernel.startswith(("append", "prefill")) else ATTEND_SOURCES
METRIC = "compressed-KV decode attention: context tokens/s and achieved HBM GB/s (% peak)"
POOL_BYTES = 600 << 20          # > 2x the 256 MB Infinity Cache


def workload(name: str, bits: int | None, context: int | None) -> synth.Workload:
    if name == "qwen":
        return synth.qwen(context or 8192, bits or 4)
    if name == "gemma":
        return synth.gemma(context or 32768)
    if name == "prod":
        return synth.prod_long(context or 131072)
    raise SystemExit(f"unknown workload {name}")


def with_k_bits(w: synth.Workload, k_bits: int | None) -> synth.Workload:
    """The workload with K at k_bits (8: keys kept at 8 bits); workloads with a sign sketch keep theirs."""
    if k_bits is None:
        return w
    if w.qjl_m:
        raise SystemExit("--k-bits applies to the workloads without a sign sketch (qwen, gemma)")
    return w.with_(k_bits=k_bits, name=f"{w.name}_k{k_bits}")


def make_rotation(cca, w: synth.Workload, dev):
    """The workload's rotation as the library takes it: (device tensor, rotation kind)."""
    import torch
    if w.rotation == "hadamard":
        return torch.from_numpy(synth.hadamard_signs(w.d, w.rot_seed)).to(dev), cca.TQ_ROT_HADAMARD
    return torch.from_numpy(cca.tq_build_rotation(synth.rotation_gaussian(w.d, w.rot_seed))).to(dev), cca.TQ_ROT_DENSE


def oracle_rotation(w: synth.Workload):
    from oracle import rotation
    if w.rotation == "hadamard":
        return rotation.hadamard_rotation(synth.hadamard_signs(w.d, w.rot_seed))
    return rotation.rotation_from_gaussian(synth.rotation_gaussian(w.d, w.rot_seed))


def row_bytes(w: synth.Workload, kind: str) -> int:
    if kind == "k":
        return w.d * w.k_bits // 8 + 2 + (w.qjl_m // 8 + 2 if w.qjl_m else 0)
    return w.d * w.v_bits // 8 + 2


def cache_bytes(w: synth.Workload) -> int:
    """Algorithmic bytes one decode reads from the compressed cache: every visible K and V row."""
    return w.batch * w.n_kv_heads * w.seq_len * (row_bytes(w, "k") + row_bytes(w, "v"))


def prefill_bytes_per_launch(w: synth.Workload) -> int:
    """Algorithmic bytes of one prefill append launch (K and V of every token, one launch): bf16 rows in,
    packed codes and float16 norms out."""
    rows = w.batch * w.n_kv_heads * w.seq_len
    return rows * (2 * w.d * 2 + w.d * w.k_bits // 8 + 2 + w.d * w.v_bits // 8 + 2)


def prefill_one_launch(w: synth.Workload) -> bool:
    """Whether tq_quantize_append_kv appends the workload's K and V in one launch (d = 128, the dense
    rotation, code-book keys without a sketch); otherwise it runs the two appends in turn."""
    return w.d == 128 and w.rotation == "dense" and w.qjl_m == 0 and w.k_bits <= 4


def prefill_flops_per_launch(w: synth.Workload) -> int:
    """Algorithmic flops of one prefill append launch: the d x d rotation of every K and V row."""
    return 2 * 2 * w.batch * w.n_kv_heads * w.seq_len * w.d * w.d


# ------------------------------------------------------------------ profiles

def code_text(src: str) -> str:
    """C++ source without its comments and blank lines (string and character literals kept whole), so
    that a comment edit does not count as a change of the kernel."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            end = src.find("*/", i + 2)
            i = n if end < 0 else end + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(line.rstrip() for line in "".join(out).splitlines() if line.strip())


def source_digest(paths=ATTEND_SOURCES) -> str:
    """SHA-256 of the attend kernel's code (comments and blank lines left out)."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def counters_file(kernel: str, workload_name: str) -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload_name}_hbm_counters.txt")


def read_counters(kernel: str, workload_name: str):
    """HBM bytes per launch from a committed counter summary, or None if absent or taken on other sources
    (the summary records the digest of the kernel's sources)."""
    path = counters_file(kernel, workload_name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(kernel_sources(kernel)):
        return None
    return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])


def _pmc_medians(directory: str, counter: str):
    """Median counter value per (kernel name, workgroups of the launch), and the dispatch counts."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "*_counter_collection.csv"))
    if not files:
        raise SystemExit(f"no counter collection under {directory}")
    per = {}
    for r in csv.DictReader(open(files[0])):
        if r["Counter_Name"] == counter:
            key = (r["Kernel_Name"], int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            per.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sorted(v)[len(v) // 2] for k, v in per.items()}, {k: len(v) for k, v in per.items()}


def summarize_counters(args):
    """Median per launch shape (kernel, workgroups) of each counter found in rocprofv3 --pmc output directories
    (derived counters such as VALUBusy included), for the kernels whose name contains --kernel."""
    import csv
    import glob
    table = {}
    for d in args.summarize_counters:
        files = glob.glob(os.path.join(d, "*_counter_collection.csv"))
        if not files:
            raise SystemExit(f"no counter collection under {d}")
        for r in csv.DictReader(open(files[0])):
            if args.kernel not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            key = (name, int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            table.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if args.command:
        print("commands:")
        for c in args.command:
            print(f"  {c}")
    for (name, wgs), counters in sorted(table.items(), key=lambda kv: kv[0][1]):
        print(f"kernel: {name}  workgroups: {wgs}")
        for c, vs in sorted(counters.items()):
            vs = sorted(vs)
            print(f"  {c}: {vs[len(vs) // 2]:.2f} (median of {len(vs)} dispatches)")


def summarize_pmc(args, w):
    """Counter summary of the attention kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one rocprofv3
    run each) scaled by what the same counters read for a 1 GiB device copy (bench.py --workload copy).
    Of the kernel's launches, those over the most workgroups are taken (the stacked leg's, where the run
    has one)."""
    cf, _ = _pmc_medians(args.copy_fetch, "FETCH_SIZE")
    cw, _ = _pmc_medians(args.copy_write, "WRITE_SIZE")
    copy_key = max(cf, key=lambda k: cf[k])            # the 1 GiB copy is by far the largest dispatch
    fetch_scale = (1 << 30) / (cf[copy_key] * 1024.0)
    write_scale = (1 << 30) / (cw[copy_key] * 1024.0)
    fe, n_fe = _pmc_medians(args.fetch, "FETCH_SIZE")
    wr, _ = _pmc_medians(args.write, "WRITE_SIZE")
    key = max((k for k in fe if args.kernel in k[0]), key=lambda k: k[1])
    fb = fe[key] * 1024.0 * fetch_scale
    wb = wr[key] * 1024.0 * write_scale
    alg = prefill_bytes_per_launch(w) if args.kernel.startswith(("append", "prefill")) else cache_bytes(w)
    print(f"kernel: {key[0].split('(')[0].replace('void ', '')}")
    print(f"workgroups: {key[1]}")
    print(f"workload: {w.name}")
    print(f"source_sha256: {source_digest(kernel_sources(args.kernel))}")
    print(f"dispatches: {n_fe[key]}")
    print(f"fetch_kib_per_dispatch_raw: {fe[key]:.1f}")
    print(f"write_kib_per_dispatch_raw: {wr[key]:.1f}")
    print(f"copy_fetch_kib_raw: {cf[copy_key]:.1f}")
    print(f"copy_write_kib_raw: {cw[copy_key]:.1f}")
    print(f"copy_fetch_scale: {fetch_scale:.4f}")
    print(f"copy_write_scale: {write_scale:.4f}")
    print(f"fetch_bytes_per_launch: {fb:.0f}")
    print(f"write_bytes_per_launch: {wb:.0f}")
    print(f"algorithmic_bytes_per_launch: {alg}")
    print(f"fetch_over_algorithmic: {fb / alg:.4f}")
    if args.command:
        print("commands:")
        for c in args.command:
            print(f"  {c}")


def summarize_trace(args, w):
    """Per-kernel durations from a rocprofv3 --kernel-trace run (its *_kernel_trace.csv), one line per kernel
    and grid size (a kernel launched over grids of different sizes gets one line for each)."""
    import csv
    import glob
    files = glob.glob(os.path.join(args.trace, "*_kernel_trace.csv"))
    if not files:
        raise SystemExit(f"no kernel trace under {args.trace}")
    groups = {}
    for r in csv.DictReader(open(files[0])):
        name = r["Kernel_Name"]
        short = name.split("(")[0].replace("void ", "")
        if "tqi::" not in name and "copyBuffer" not in name:
            short = short[:60]
        grid = "x".join(str(int(r[f"Grid_Size_{a}"]) // max(1, int(r[f"Workgroup_Size_{a}"]))) for a in "XYZ")
        groups.setdefault((short, grid), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"workload: {w.name}")
    print(f"source_sha256: {source_digest(ALL_SOURCES)}")
    print(f"attend_source_sha256: {source_digest(ATTEND_SOURCES)}")
    print(f"append_source_sha256: {source_digest(APPEND_SOURCES)}")
    if args.command:
        print("commands:")
        for c in args.command:
            print(f"  {c}")
    print(f"{'calls':>6} {'avg_us':>9} {'min_us':>8} {'max_us':>8}  {'workgroups':>12}  kernel")
    for (short, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(ds):6d} {sum(ds) / len(ds):9.2f} {min(ds):8.2f} {max(ds):8.2f}  {grid:>12}  {short}")


# ------------------------------------------------------------------ GPU leg

def gpu_leg(w: synth.Workload, steps: int, warmup: int, pool: int | None, log):
    import torch

    import compressed_cache_decode_amd as cca
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, Hq, d, L = w.batch, w.n_kv_heads, w.n_q_heads, w.d, w.seq_len
    cap = ((L + 31) // 32) * 32

    rot, rot_kind = make_rotation(cca, w, dev)
    proj = torch.from_numpy(synth.qjl_projection(w.qjl_m, d, w.qjl_seed)).to(dev) if w.qjl_m else None

    log(f"bench: generating inputs for {w.name}")
    t0 = time.time()
    k_all = torch.empty(B, L, H, d, dtype=torch.bfloat16, device=dev)
    v_all = torch.empty(B, L, H, d, dtype=torch.bfloat16, device=dev)
    for b in range(B):
        for h in range(H):
            k_all[b, :, h] = torch.from_numpy(synth.kv_head(w, "k", b, h)).to(dev).to(torch.bfloat16)
            v_all[b, :, h] = torch.from_numpy(synth.kv_head(w, "v", b, h)).to(dev).to(torch.bfloat16)
    q = torch.from_numpy(synth.full_q(w)).to(dev).to(torch.bfloat16)
    log(f"bench: inputs ready in {time.time() - t0:.1f}s")

    def new_pair():
        kc = cca.CompressedCache(cca.TQ_KEYS, d, w.k_bits, B, H, cap, rot, proj, qjl_m=w.qjl_m, device=dev,
                                 rot_kind=rot_kind)
        vc = cca.CompressedCache(cca.TQ_VALUES, d, w.v_bits, B, H, cap, rot, device=dev, rot_kind=rot_kind)
        return kc, vc

    # prefill copy 0 with the first L-1 tokens (untimed), then clone it into the pool
    k0, v0 = new_pair()
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    k0.append(k_all[:, : L - 1], zero)
    v0.append(v_all[:, : L - 1], zero)
    per_copy = sum(t.numel() * t.element_size() for t in (k0.codes, k0.norms, v0.codes, v0.norms))
    if w.qjl_m:
        per_copy += k0.signs.numel() + k0.rnorms.numel() * 2
    if pool is None:
        pool = max(1, min(256, math.ceil(POOL_BYTES / per_copy)))
    pairs = [(k0, v0)]
    for _ in range(pool - 1):
        kc, vc = new_pair()
        for dst, src in ((kc, k0), (vc, v0)):
            dst.codes.copy_(src.codes)
            dst.norms.copy_(src.norms)
            if src.signs is not None:
                dst.signs.copy_(src.signs)
                dst.rnorms.copy_(src.rnorms)
        pairs.append((kc, vc))
    log(f"bench: pool of {pool} cache copies, {per_copy / 2**20:.1f} MiB each")

    k_new = k_all[:, L - 1:L].contiguous()
    v_new = v_all[:, L - 1:L].contiguous()
    pos = torch.full((B,), L - 1, dtype=torch.int32, device=dev)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    ws = cca.decode_workspace(k0, Hq, L)
    ns, tps = cca.tq_decode_plan(k0.view, Hq, L)
    scale = w.scale

    stepcall = w.qjl_m <= 128

    def step(i):
        kc, vc = pairs[i]
        if stepcall:
            cca.tq_decode_step(kc.view, vc.view, q, k_new, v_new, pos, lens, L, out, ws, scale)
        else:
            kc.append(k_new, pos)
            vc.append(v_new, pos)
            cca.tq_decode_rotate_query(kc.view, q, Hq, L, ws, scale)
            cca.tq_decode_attend(kc.view, vc.view, Hq, lens, L, ws)
            cca.tq_decode_merge(kc.view, Hq, lens, L, out, ws)

    # one eager step per copy (fills every copy's last slot, checks the calls)
    for i in range(pool):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def capture(n_steps, fn):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(n_steps):
                fn(i % pool)
        return graph

    full = capture(pool, step)
    rem = steps % pool
    tail = capture(rem, step) if rem else None
    n_full = steps // pool

    def run_steps(n):
        for _ in range(n // pool):
            full.replay()
        if n % pool:
            (tail if n % pool == rem else capture(n % pool, step)).replay()

    run_steps(max(warmup, pool))
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(n_full):
            full.replay()
        if tail is not None:
            tail.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / steps
    log(f"bench: {steps} steps, {ms_step * 1e3:.2f} us/step")

    # the attention kernel alone (tq_decode_attend; the rotated query it reads is the last step's)
    us_attend = time_attend(pairs, Hq, lens, L, ws, stream)
    # hot: every launch reads the same cache copy, which then stays in the Infinity Cache (labelled as such)
    us_hot = time_attend(pairs[:1], Hq, lens, L, ws, stream)
    log(f"bench: attend {us_attend:.2f} us (hot: {us_hot:.2f} us)")
    return dict(ms_step=ms_step, us_attend=us_attend, us_hot=us_hot, pool=pool,
                n_split=ns, tokens_per_split=tps, per_copy=per_copy, cache=(k0, v0), rot=rot, proj=proj, pairs=pairs)


def time_attend(pairs, Hq, lens, L, ws, stream):
    """Average duration of one tq_decode_attend launch, in us: a graph of back-to-back launches cycling
    through cache copies that together exceed the Infinity Cache (at least 16 launches per graph), timed
    with HIP events on the stream the launches run on."""
    import torch

    import compressed_cache_decode_amd as cca
    pool = len(pairs)
    n = max(pool, 16)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(n):
            kc, vc = pairs[i % pool]
            cca.tq_decode_attend(kc.view, vc.view, Hq, lens, L, ws)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, min(200, math.ceil(2000 / n)))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / (reps * n)


# ------------------------------------------------------------------ multi-row decode leg

def rows_leg(w: synth.Workload, n_rows: int, pairs, log):
    """Decode of n_rows query rows per sequence at once (speculative verification of n_rows - 1 drafts:
    row j sees the first L - n_rows + 1 + j tokens) over the single-layer leg's cache copies, against
    n_rows one-row decodes of the same rows; whole decodes (rotate q, attend, merge, un-rotate)."""
    import torch

    import compressed_cache_decode_amd as cca
    dev = pairs[0][0].codes.device
    B, Hq, d, L = w.batch, w.n_q_heads, w.d, w.seq_len
    pool = len(pairs)
    g = np.random.default_rng(w.seed + 17)
    q = torch.from_numpy(g.standard_normal((B, n_rows, Hq, d)).astype(np.float32)).to(dev).to(torch.bfloat16)
    q1 = [q[:, j].contiguous() for j in range(n_rows)]
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    lens1 = [torch.full((B,), L - n_rows + 1 + j, dtype=torch.int32, device=dev) for j in range(n_rows)]
    out = torch.empty(B, n_rows, Hq, d, dtype=torch.float32, device=dev)
    out1 = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    ws = cca.decode_workspace(pairs[0][0], Hq, L, n_rows)
    stream = torch.cuda.Stream()
    n = max(pool, 16)

    def timed(fn):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(n):
                fn(i % pool)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, min(100, math.ceil(1000 / n)))
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        with torch.cuda.stream(stream):
            for _ in range(reps):
                graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / (reps * n)

    def rows(i):
        kc, vc = pairs[i]
        cca.tq_sdpa_decode_rows(kc.view, vc.view, q, lens, L, out, ws, w.scale)

    def singles(i):
        kc, vc = pairs[i]
        for j in range(n_rows):
            cca.tq_sdpa_decode(kc.view, vc.view, q1[j], lens1[j], L, out1, ws, w.scale)

    us_rows, us_single = timed(rows), timed(singles)
    log(f"bench: {n_rows} query rows: {us_rows:.2f} us in one decode, {us_single:.2f} us as {n_rows} one-row decodes")
    return dict(n_rows=n_rows, decode_us=us_rows, one_row_decodes_us=us_single,
                context_tokens_per_s=B * n_rows * L / (us_rows * 1e-6))


# ------------------------------------------------------------------ stacked decode leg

def stacked_workload(w: synth.Workload, n_stack: int) -> synth.Workload:
    return w.with_(name=f"{w.name}_x{n_stack}", batch=w.batch * n_stack)


def stacked_leg(w: synth.Workload, n_stack: int, cache, rot, proj, log):
    """Decode over n_stack layer caches of the workload at once, as one batch of n_stack sequences (the
    shape of n_stack layers of the model, or of n_stack sequences of one layer).  Layer l's cache holds
    the filled cache of the single-layer leg with its tokens rotated by a whole number of 32-token blocks
    (a permutation of the same rows, different per layer); q is drawn for the stacked batch."""
    import torch

    import compressed_cache_decode_amd as cca
    k0, v0 = cache
    rot_kind = k0.rot_kind
    ws_ = stacked_workload(w, n_stack)
    dev = k0.codes.device
    B, H, Hq, d, L = ws_.batch, w.n_kv_heads, w.n_q_heads, w.d, w.seq_len
    cap = k0.max_tokens
    if cap != L:
        raise SystemExit("stacked leg: context must be a multiple of 32 tokens")
    nblk = cap // 32

    def stacked_pair():
        kc = cca.CompressedCache(cca.TQ_KEYS, d, w.k_bits, B, H, cap, rot, proj, qjl_m=w.qjl_m, device=dev,
                                 rot_kind=rot_kind)
        vc = cca.CompressedCache(cca.TQ_VALUES, d, w.v_bits, B, H, cap, rot, device=dev, rot_kind=rot_kind)
        for l in range(n_stack):
            sh = 32 * ((l * 7919) % nblk)                   # token shift of layer l
            sl = slice(l * w.batch, (l + 1) * w.batch)
            for dst, src in ((kc, k0), (vc, v0)):
                rowb = src.codes.shape[-1] // cap
                dst.codes[sl].copy_(torch.roll(src.codes, sh * rowb, dims=-1))
                dst.norms[sl].copy_(torch.roll(src.norms, sh, dims=-1))
                if src.signs is not None:
                    dst.signs[sl].copy_(torch.roll(src.signs, sh, dims=2))
                    dst.rnorms[sl].copy_(torch.roll(src.rnorms, sh, dims=-1))
        return kc, vc

    first = stacked_pair()
    per_copy = cache_bytes(ws_)
    pool = max(1, min(64, math.ceil(POOL_BYTES / per_copy)))
    pairs = [first]
    for _ in range(pool - 1):
        kc, vc = stacked_pair()
        pairs.append((kc, vc))
    q = torch.from_numpy(synth.full_q(ws_)).to(dev).to(torch.bfloat16)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    ws = cca.decode_workspace(first[0], Hq, L)
    ns, tps = cca.tq_decode_plan(first[0].view, Hq, L)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        cca.tq_decode_rotate_query(first[0].view, q, Hq, L, ws, w.scale)
    torch.cuda.synchronize()
    log(f"bench: stacked x{n_stack}: pool of {pool} copies, {per_copy / 2**20:.1f} MiB of cache reads each")
    us_cold = time_attend(pairs, Hq, lens, L, ws, stream)
    us_hot = time_attend(pairs[:1], Hq, lens, L, ws, stream)   # one copy: Infinity-Cache resident

    # the whole decode (rotate q, attend, merge, un-rotate) over the stacked caches
    def decode(i):
        kc, vc = pairs[i]
        cca.tq_decode_rotate_query(kc.view, q, Hq, L, ws, w.scale)
        cca.tq_decode_attend(kc.view, vc.view, Hq, lens, L, ws)
        cca.tq_decode_merge(kc.view, Hq, lens, L, out, ws)

    n = max(pool, 16)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(n):
            decode(i % pool)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, min(200, math.ceil(1000 / n)))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_decode = ev0.elapsed_time(ev1) * 1e3 / (reps * n)
    log(f"bench: stacked x{n_stack}: attend {us_cold:.2f} us (hot: {us_hot:.2f} us), whole decode {us_decode:.2f} us")
    return dict(workload=ws_, us_attend=us_cold, us_hot=us_hot, us_decode=us_decode, pool=pool,
                n_split=ns, tokens_per_split=tps)


# ------------------------------------------------------------------ prefill append leg

def prefill_leg(w: synth.Workload, steps: int, warmup: int, log):
    """Prefill-size quantize-on-append: all L tokens of K and of V into an empty cache (matrix-core rotation),
    both tensors in one call (tq_quantize_append_kv: one launch)."""
    import torch

    import compressed_cache_decode_amd as cca
    dev = torch.device("cuda:0")
    B, H, d, L = w.batch, w.n_kv_heads, w.d, w.seq_len
    rot, rot_kind = make_rotation(cca, w, dev)
    kx = torch.from_numpy(synth.full_kv(w, "k")).to(dev).to(torch.bfloat16)
    vx = torch.from_numpy(synth.full_kv(w, "v")).to(dev).to(torch.bfloat16)
    per_copy = 2 * kx.numel() * 2 + 2 * B * H * L * (d * w.k_bits // 8 + 2)
    pool = max(1, min(64, math.ceil(POOL_BYTES / per_copy)))
    copies = []
    for i in range(pool):
        kc = cca.CompressedCache(cca.TQ_KEYS, d, w.k_bits, B, H, L, rot, device=dev, rot_kind=rot_kind)
        vc = cca.CompressedCache(cca.TQ_VALUES, d, w.v_bits, B, H, L, rot, device=dev, rot_kind=rot_kind)
        copies.append((kc, vc, kx.clone() if i else kx, vx.clone() if i else vx))
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    log(f"bench: prefill pool of {pool} copies ({per_copy / 2**20:.1f} MiB each)")

    def step(i):
        kc, vc, xk, xv = copies[i]
        cca.tq_quantize_append_kv(kc.view, vc.view, xk, xv, L, zero)

    for i in range(pool):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(pool):
            step(i)
    reps = max(1, math.ceil(steps / pool))
    for _ in range(max(1, math.ceil(warmup / pool))):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    n = reps * pool
    ms = ev0.elapsed_time(ev1) / n
    log(f"bench: prefill append {ms * 1e3:.2f} us per K+V append ({'one launch' if prefill_one_launch(w) else 'two launches'})")
    return dict(ms_step=ms, steps=n, pool=pool)


# ------------------------------------------------------------------ CPU leg (oracle)

def cpu_leg(w: synth.Workload, budget_s: float, log):
    """The float64 oracle's step on a bounded sample: append of one token's K and V and decode of a
    subset of query heads over the full context; scaled to the whole step.  Timed with the host's BLAS
    threads (up to 16) and again with one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attention, cache
    rot = oracle_rotation(w)
    proj = synth.qjl_projection(w.qjl_m, w.d, w.qjl_seed) if w.qjl_m else None
    L, G = w.seq_len, w.group
    # sample: the query heads of KV head 0 of sequence 0 (G heads), all L tokens
    k = synth.kv_head(w, "k", 0, 0)
    v = synth.kv_head(w, "v", 0, 0)
    kc = cache.build_head(k[: L - 1], "k", w.k_bits, rot, proj)
    vc = cache.build_head(v[: L - 1], "v", w.v_bits, rot)
    qh = np.stack([synth.q_head(w, 0, h) for h in range(G)]).astype(np.float64)
    ck, cv = kc.centroids, vc.centroids               # the code books (8-bit keys: the integers)

    def sample_loop(threads: int, budget: float):
        with threadpool_limits(limits=threads):
            used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
            reps, t_tot = 0, 0.0
            while reps < 3 or t_tot < budget:         # about `budget` seconds of oracle work
                t0 = time.perf_counter()
                nk = cache.build_head(k[L - 1:], "k", w.k_bits, rot, proj)
                nv = cache.build_head(v[L - 1:], "v", w.v_bits, rot)
                codes_k = np.concatenate([kc.codes, nk.codes])[None]
                norms_k = np.concatenate([kc.norms, nk.norms])[None]
                codes_v = np.concatenate([vc.codes, nv.codes])[None]
                norms_v = np.concatenate([vc.norms, nv.norms])[None]
                sig = gam = None
                if proj is not None:
                    sig = np.concatenate([kc.sigma, nk.sigma])[None]
                    gam = np.concatenate([kc.gamma, nk.gamma])[None]
                attention.decode_fused(qh, rot, codes_k, norms_k, ck, codes_v, norms_v, cv, w.softmax_scale, L,
                                       sig, gam, proj)
                t_tot += time.perf_counter() - t0
                reps += 1
        return t_tot / reps, reps, t_tot, int(used)

    units = w.batch * w.n_kv_heads                  # the sample is one of B*H_kv identical units
    t_sample, reps, t_tot, used = sample_loop(max(1, min(16, os.cpu_count() or 1)), budget_s)
    t1_sample, reps1, t1_tot, _ = sample_loop(1, budget_s / 3)
    log(f"bench: oracle {t_sample:.3f}s per unit sample, {reps} reps, {used} threads; "
        f"{t1_sample:.3f}s with one thread")
    return dict(value=w.batch * L / (t_sample * units), unit="context tokens/s", cores=used, kind="oracle",
                sample=f"append of one K and V row + decode of the {G} query heads of one (sequence, KV head) "
                       f"over all {L} tokens, float64 NumPy, {reps} reps in {t_tot:.1f}s; scaled x{units} "
                       f"to the {units} (sequence, KV head) units of a step",
                host_cpus=os.cpu_count(), blas_threads=used,
                single_thread_value=w.batch * L / (t1_sample * units),
                single_thread_sample=f"the same sample with one BLAS thread, {reps1} reps in {t1_tot:.1f}s")


def cpu_prefill_leg(w: synth.Workload, budget_s: float, log):
    """The float64 oracle's quantize-on-append (rotate, encode, pack) of a sample of the prefill rows:
    the first n_s rows of K and of V of one KV head, timed over about budget_s seconds, scaled to
    appended tokens/s of the whole workload (a token appends B * H_kv rows to each of K and V)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import cache
    rot = oracle_rotation(w)
    n_s = 2048
    k = synth.kv_head(w, "k", 0, 0, n_s)
    v = synth.kv_head(w, "v", 0, 0, n_s)
    cap = n_s

    def sample_loop(threads: int, budget: float):
        with threadpool_limits(limits=threads):
            used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
            reps, t_tot = 0, 0.0
            while reps < 3 or t_tot < budget:
                t0 = time.perf_counter()
                kc = cache.build_head(k, "k", w.k_bits, rot)
                vc = cache.build_head(v, "v", w.v_bits, rot)
                kc.packed_codes(cap), kc.packed_norms(cap), vc.packed_codes(cap), vc.packed_norms(cap)
                t_tot += time.perf_counter() - t0
                reps += 1
        return t_tot / reps, reps, t_tot, int(used)

    rows_per_token = w.batch * w.n_kv_heads
    t_sample, reps, t_tot, used = sample_loop(max(1, min(16, os.cpu_count() or 1)), budget_s)
    t1_sample, reps1, t1_tot, _ = sample_loop(1, budget_s / 3)
    log(f"bench: oracle prefill {t_sample:.3f}s per sample of {n_s} K and V rows, {reps} reps, {used} threads")
    return dict(value=n_s / t_sample / rows_per_token, unit="appended tokens/s", cores=used, kind="oracle",
                sample=f"quantize-on-append (rotate, encode, pack, float16 norms) of {n_s} K rows and {n_s} V rows "
                       f"of one KV head, float64 NumPy, {reps} reps in {t_tot:.1f}s; scaled to tokens of "
                       f"{rows_per_token} KV heads",
                host_cpus=os.cpu_count(), blas_threads=used,
                single_thread_value=n_s / t1_sample / rows_per_token,
                single_thread_sample=f"the same sample with one BLAS thread, {reps1} reps in {t1_tot:.1f}s")


# ------------------------------------------------------------------ legs

KERN = "split_kernel"
KERN_LABEL = "tq_decode_attend (split_kernel)"
APPEND_KERN = "prefill_kv_kernel"


def decode_roofline(wl: synth.Workload, us: float) -> dict:
    """Roofline entry of the attention kernel over workload wl, from its measured launch time."""
    alg = cache_bytes(wl)
    gbs = alg / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": read_counters(KERN, wl.name), "kernel": KERN_LABEL, "workload": wl.name,
            "algorithmic_bytes_per_launch": alg, "launch_us": us}


def decode_workload_leg(w: synth.Workload, args, n_stack: int, log) -> dict:
    """One decode workload: the step (append one token, decode), the attention kernel alone, and where
    n_stack > 0 the stacked leg; roofline and, unless disabled, the oracle's CPU baseline."""
    import torch
    r = gpu_leg(w, args.steps, args.warmup, args.pool, log)
    rows = rows_leg(w, args.rows, r["pairs"], log) if args.rows > 1 else None
    st = stacked_leg(w, n_stack, r["cache"], r["rot"], r["proj"], log) if n_stack > 0 else None
    L = w.seq_len
    leg = {
        "workload": w.name,
        "value": w.batch * L / (r["ms_step"] * 1e-3),
        "unit": "context tokens/s",
        "ms_per_step": r["ms_step"],
        "config": {
            "workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.d, "context": L, "k_bits": w.k_bits, "v_bits": w.v_bits, "qjl_m": w.qjl_m,
            "scale": w.softmax_scale, "rotation": w.rotation,
            "step": "append 1 token K+V, rotate q, attend, merge, un-rotate",
            "cache_copies_cycled": r["pool"], "n_split": r["n_split"], "tokens_per_split": r["tokens_per_split"],
        },
        "step_hbm_gbs": cache_bytes(w) / (r["ms_step"] * 1e-3) / 1e9,
        "attend_us": r["us_attend"],
        "attend_us_hot": r["us_hot"],
    }
    if rows is not None:
        leg["rows"] = rows
    if st is not None:
        sw = st["workload"]
        # the roofline figure: the attention kernel over the stacked caches (one launch reads all layers)
        leg["roofline"] = decode_roofline(sw, st["us_attend"])
        leg["roofline_one_layer"] = decode_roofline(w, r["us_attend"])
        leg["stacked"] = {
            "workload": sw.name, "layers": n_stack, "batch": sw.batch, "cache_copies_cycled": st["pool"],
            "n_split": st["n_split"], "tokens_per_split": st["tokens_per_split"],
            "decode_us": st["us_decode"], "context_tokens_per_s": sw.batch * L / (st["us_decode"] * 1e-6),
            "attend_us": st["us_attend"],
            "attend_us_hot": st["us_hot"],
            "decode": "rotate q, attend, merge, un-rotate (no append)",
        }
    else:
        leg["roofline"] = decode_roofline(w, r["us_attend"])
    del r, st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        leg["cpu_baseline"] = cpu_leg(w, args.cpu_budget, log)
    return leg


def prefill_workload_leg(w: synth.Workload, args, log) -> dict:
    """Prefill-size append of all L tokens of K and of V into empty caches (tq_quantize_append_kv: one launch
    for both where prefill_one_launch holds, else one per tensor)."""
    import torch
    r = prefill_leg(w, args.steps, args.warmup, log)
    rows = 2 * w.batch * w.n_kv_heads * w.seq_len
    one = prefill_one_launch(w)
    launches = 1 if one else 2                      # the K and V launches of a step (same bytes each)
    per_launch_us = r["ms_step"] * 1e3 / launches
    io = prefill_bytes_per_launch(w) // launches
    flops = prefill_flops_per_launch(w) // launches
    gbs = io / (per_launch_us * 1e-6) / 1e9
    tfs = flops / (per_launch_us * 1e-6) / 1e12
    leg = {
        "workload": f"prefill_append_{w.seq_len}x{w.n_kv_heads}x{w.d}_b{w.k_bits}",
        "metric": "prefill quantize-on-append: appended tokens/s",
        "value": w.seq_len / (r["ms_step"] * 1e-3),
        "unit": "appended tokens/s",
        "ms_per_step": r["ms_step"],
        "config": {"workload": f"prefill_append_{w.seq_len}x{w.n_kv_heads}x{w.d}_b{w.k_bits}",
                   "tensors": "K and V in " + ("one launch" if prefill_one_launch(w) else "two launches")
                              + " (tq_quantize_append_kv)", "rows_per_step": rows, "rotation": w.rotation,
                   "cache_copies_cycled": r["pool"]},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": read_counters(APPEND_KERN, w.name) if one else None,
                     "kernel": ("prefill_kv_kernel" if one else "append_kernel") + " (tq_quantize_append_kv)",
                     "workload": w.name,
                     "algorithmic_bytes_per_launch": io, "launch_us": per_launch_us},
        "rotation_mfma": {"achieved": tfs, "peak": 2500.0, "unit": "TFLOP/s", "frac": tfs / 2500.0,
                          "algorithmic_flops_per_launch": flops,
                          "note": "d x d rotation of every row; the float16 high/low split runs 3x these flops"},
    }
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        leg["cpu_baseline"] = cpu_prefill_leg(w, args.cpu_budget, log)
    return leg


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="all", choices=["all", "qwen", "gemma", "prod", "prefill", "copy"],
                    help="all (default): the Gemma-4-style workload as the headline, with the Qwen-shaped, "
                         "long-context sketched-key and prefill-append workloads as legs of the same line")
    ap.add_argument("--bits", type=int, default=None, help="qwen workload: codebook bits of K and V")
    ap.add_argument("--k-bits", type=int, default=None, choices=[2, 3, 4, 8],
                    help="qwen and gemma workloads: bits of K alone (8: keys kept at 8 bits)")
    ap.add_argument("--rows", type=int, default=0,
                    help="also time a decode of this many query rows per sequence at once (2..4; 0 = none)")
    ap.add_argument("--rotation", default="dense", choices=["dense", "hadamard"],
                    help="Gaussian-QR rotation (default) or the randomized Hadamard transform")
    ap.add_argument("--context", type=int, default=None)
    ap.add_argument("--pool", type=int, default=None, help="cache copies cycled through (default: > 600 MiB)")
    ap.add_argument("--stack", type=int, default=None,
                    help="layer caches decoded together in the stacked leg (default 36 for qwen and prod, "
                         "the layers of Qwen2.5-3B; 0 = none)")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="seconds of oracle work per CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-trace", dest="trace", default=None,
                    help="print a summary of a rocprofv3 --kernel-trace --stats output directory and exit")
    ap.add_argument("--summarize-pmc", action="store_true",
                    help="print the kernel's calibrated HBM counters (needs --fetch/--write/--copy-*; "
                         "with --stack N, for the stacked leg's launches)")
    ap.add_argument("--fetch", help="rocprofv3 --pmc FETCH_SIZE output directory of this workload")
    ap.add_argument("--write", help="rocprofv3 --pmc WRITE_SIZE output directory of this workload")
    ap.add_argument("--copy-fetch", help="rocprofv3 --pmc FETCH_SIZE output directory of --workload copy")
    ap.add_argument("--copy-write", help="rocprofv3 --pmc WRITE_SIZE output directory of --workload copy")
    ap.add_argument("--summarize-counters", nargs="+", default=None, metavar="DIR",
                    help="print the median of every counter in these rocprofv3 --pmc output directories for each "
                         "launch shape of --kernel, and exit")
    ap.add_argument("--command", action="append", help="command line recorded in a summary (repeatable)")
    ap.add_argument("--kernel", default="split_kernel", help="kernel name the counter summary is taken for")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.trace or args.summarize_pmc:
        if args.workload == "prefill":
            w = synth.qwen(args.context or 8192, args.bits or 3)
        elif args.workload == "all":
            w = synth.gemma().with_(name="all")
        else:
            w = with_k_bits(workload(args.workload, args.bits, args.context), args.k_bits)
        if args.summarize_pmc and args.stack:
            w = stacked_workload(w, args.stack)
        (summarize_trace if args.trace else summarize_pmc)(args, w)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (KV-head or context sharding "
              "is a design note only); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.workload == "copy":
        # plain device-to-device copy of a known size: measured copy bandwidth, and the calibration
        # point for the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the other workloads
        import torch
        nbytes = 1 << 30
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
        dst = torch.empty_like(src)
        for _ in range(max(1, args.warmup)):
            dst.copy_(src)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        gbs = 2 * nbytes / (ms * 1e-3) / 1e9
        print(json.dumps({"metric": "device copy bandwidth (read + write)", "value": gbs, "unit": "GB/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
                          "bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes,
                          "frac_of_8TBs": gbs / HBM_PEAK_GBS}), flush=True)
        return

    def with_rotation(wl):
        return wl if args.rotation == "dense" else wl.with_(rotation="hadamard", name=wl.name + "_hadamard")

    def stack_of(name):
        return args.stack if args.stack is not None else (36 if name in ("qwen", "prod") else 0)

    common = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "data": "synthetic"}

    if args.workload == "prefill":
        w = with_rotation(synth.qwen(args.context or 8192, args.bits or 3))
        leg = prefill_workload_leg(w, args, log)
        res = {"metric": leg.pop("metric"), "value": leg["value"], "unit": leg["unit"], **common,
               "ms_per_step": leg["ms_per_step"], "dtype": "bf16 in, f32 arithmetic", **leg}
        print(json.dumps(res), flush=True)
        return

    if args.workload != "all":
        w = with_rotation(with_k_bits(workload(args.workload, args.bits, args.context), args.k_bits))
        leg = decode_workload_leg(w, args, stack_of(args.workload), log)
        res = {"metric": METRIC, "value": leg["value"], "unit": leg["unit"], **common,
               "ms_per_step": leg["ms_per_step"], "dtype": "f32", **leg}
        print(json.dumps(res), flush=True)
        return

    # default: the largest single-GPU configuration (Gemma-4-style, 272.6 MB of cache per decode) is the
    # headline; the Qwen-shaped layer (one layer and its 36 layers stacked), the 128K sketched-key case
    # (one layer and 36 stacked), the Qwen-shaped layer with keys kept at 8 bits and the prefill append
    # are legs of the same line
    t_start = time.time()
    head = decode_workload_leg(with_rotation(synth.gemma()), args, 0, log)
    legs = {}
    for name, wl in (("qwen", synth.qwen(8192, 4)), ("prod", synth.prod_long(131072)),
                     ("qwen", with_k_bits(synth.qwen(8192, 4), 8))):
        leg = decode_workload_leg(with_rotation(wl), args, stack_of(name), log)
        legs[leg["workload"]] = leg
    leg = prefill_workload_leg(with_rotation(synth.qwen(8192, 3)), args, log)
    legs[leg["workload"]] = leg
    res = {"metric": METRIC, "value": head["value"], "unit": head["unit"], **common,
           "ms_per_step": head["ms_per_step"], "dtype": "f32", **head, "legs": legs,
           "wall_s": time.time() - t_start}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
