"""Benchmark: one MLA decode step over a paged latent cache on one MI355X.

A step is the whole path for one batch: cache append (one new row per sequence), query absorption
through W_UK, latent decode attention (with its split merge) and the W_UV out-projection.  Inputs are
seeded synthetic data resident in HBM before timing starts.  Default workload: 32 sequences x 4,096
cached tokens, each appending its new token's row (so 4,097 are attended), 128 heads, 64-token pages
with a shuffled block table.  The 151 MB cache fits in the 256 MB Infinity Cache, so the steps
rotate through independent input sets.

Prints one JSON line.  `value` is latent-cache GB/s over the whole step (tokens x 1,152 B / step
time), from K steps timed between two synchronisations with nothing else on the stream.
`roofline` reports the dominant call, mla_decode, timed with HIP events on the launch stream in a
second pass of the same K steps (mean and median), against the datasheet peaks and against what
this GPU measures on plain library work (a device copy, a bf16 matrix product); for a
cache that fits in the Infinity Cache also warm, labelled.
`sparse_topk` times attention over each sequence's 2,048 best tokens of a cheap int8 index (scores and
top-k, then the decode over the kept rows read in place; beside it the form that first gathers them
into compact pages) against the dense decode call.
`out_proj_hidden` times the projection of the step's per-head output to the hidden width through W^O.
`producer` (workloads that append) times mla_cache_append_hidden, the producer side of the cache,
graph-replayed over 48 weight copies.  `fp6` times mla_decode_fp6 over the ~6-bit form of the same
cache (FP6 codes and a power-of-two scale per row, 436 bytes per token).
`cpu_baseline` times the CPU oracle (decompressed form, float64) on a bounded sample: whole
sequences (gather + every head), in order, until about --cpu-seconds of work is done.

    python bench.py [--steps K] [--warmup W] [--config 1..5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode: latent-cache GB/s, TFLOP/s, tokens/s; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MALL_BYTES = 256 << 20       # MI355X Infinity Cache
MFMA_BF16_PEAK_TF = 2500.0   # MI355X dense bf16 MFMA
ROW_BYTES = 1152
ROW_ELEMS = 576
FP6_ROW_BYTES = 436          # ~6-bit cache: 432 bytes of codes + a 4-byte scale per row
D_MODEL = 5120
D_C, D_R, D_NOPE, D_V = 512, 64, 128, 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--sets", type=int, default=0, help="independent input sets (0 = auto)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-run", action="store_true",
                    help="for counter runs: a few untimed steps, then mla_decode alone, then one "
                         "1 GiB device copy that calibrates the byte counters; prints no JSON")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of "
                         "--profile-run into profiles/traffic_<workload>.json; needs no GPU")
    return ap.parse_args()


# Sources of the decode call's kernels and of its work split; the traffic record is valid only for
# the sources it was taken on.
DECODE_SOURCES = ("decode.hip", "decode_mfma.hip", "mla_api.cpp", "mla_device.h", "mla_internal.h")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "head_latent_attention_17_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_record(workload: str):
    """HBM bytes per mla_decode call from committed rocprofv3 counter runs, if they were taken on
    the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec


def producer_timing(lib, synth, wl, dev, cache, bt, lens, steps: int):
    """The producer side of the cache on the same batch: mla_cache_append_hidden writing each
    sequence's next row ([h W_DKV | RoPE(h W_KR)], the slots the step's append fills), with the
    weights rotated through more copies than the Infinity Cache holds.  One call per weight copy is
    captured in a HIP graph and the graph is replayed, timed with HIP events around the replays: the
    Python marshalling of a call (longer than the call's GPU time at this batch) is not what is
    timed.  The rows the replays leave are checked bit for bit against an eager call with the last
    weights.  bytes = weights + hidden rows + written rows."""
    import torch
    h = synth.hidden_states(wl, 0, device=dev).view(torch.bfloat16)
    copies = 48                                   # 48 x 5.9 MB > 256 MB
    wts = [tuple(w.view(torch.bfloat16) for w in synth.producer_weights(wl, 1000 + i, device=dev))
           for i in range(copies)]
    ws = torch.empty(lib.mla_cache_append_hidden_workspace_size(wl.batch), dtype=torch.uint8, device=dev)
    b_idx = torch.arange(wl.batch, device=dev)
    page_of = bt[b_idx, lens.long() // 64].long()
    slots = (page_of * 64 + lens.long() % 64)

    def written():
        return cache.view(-1, ROW_ELEMS)[slots].clone()

    lib.mla_cache_append_hidden(cache, bt, lens, h, *wts[copies - 1], 10000.0, ws)
    torch.cuda.synchronize()
    expect = written()
    for i in range(copies):
        lib.mla_cache_append_hidden(cache, bt, lens, h, *wts[i], 10000.0, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(copies):
            lib.mla_cache_append_hidden(cache, bt, lens, h, *wts[i], 10000.0, ws)
    torch.cuda.synchronize()
    replays = max(2, -(-steps // copies))
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(written(), expect):
            raise RuntimeError("graph replay of mla_cache_append_hidden wrote other rows than an eager call")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    if not torch.equal(written(), expect):
        raise RuntimeError("graph replay of mla_cache_append_hidden wrote other rows than an eager call")
    ms = a.elapsed_time(b) / (replays * copies)
    del g
    nbytes = D_MODEL * ROW_ELEMS * 2 + wl.batch * D_MODEL * 2 + wl.batch * ROW_BYTES
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"call": "mla_cache_append_hidden", "batch": wl.batch, "ms_per_call": round(ms, 5),
            "bytes": nbytes, "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "weights": "48 rotated copies, cold", "timing": "graph replay"}


def fp6_timing(lib, synth, wl, dev, q_abs, bt, att, o_lat, lse, ws, steps: int, splits: int,
               bf16_ms: float):
    """The decode over the ~6-bit cache (mla_decode_fp6) on the same workload and query: the
    synthetic cache quantized on the GPU (mla_cache_quantize_fp6) into enough independent copies that
    together they exceed the Infinity Cache, then `steps` calls rotating through them, each between
    HIP events on the launch stream.  Algorithmic bytes = attended tokens x 436 (codes and scale of
    each row); at 2,176 x heads flop per token that is past the bf16 ridge, so the matrix cores
    (bf16 after the exact conversion) are the roofline reported."""
    import torch
    if wl.heads not in (64, 128) or wl.layers > 1:
        return None
    N = wl.tokens
    copies = max(2, min(8, -(-400_000_000 // (N * FP6_ROW_BYTES))))
    caches = []
    for i in range(copies):
        src = synth.cache_pages(wl, 100 + i, device=dev, chunk_pages=2048).view(torch.bfloat16)
        c6 = torch.empty((wl.num_pages, lib.FP6_PAGE_BYTES), dtype=torch.uint8, device=dev)
        lib.mla_cache_quantize_fp6(src, c6)
        del src
        caches.append(c6)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for i in range(3):
        lib.mla_decode_fp6(q_abs, caches[i % copies], bt, att, wl.scale, o_lat, lse, ws, splits)
    ev = []
    for i in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        lib.mla_decode_fp6(q_abs, caches[i % copies], bt, att, wl.scale, o_lat, lse, ws, splits)
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    del caches
    torch.cuda.empty_cache()
    flops = N * 2 * wl.heads * (D_C + D_R + D_C)
    tf = flops / (ms * 1e-3) / 1e12
    gbs = N * FP6_ROW_BYTES / (ms * 1e-3) / 1e9
    return {"call": "mla_decode_fp6 (decode + merge kernels)",
            "cache": "FP6 E2M3 codes + power-of-two row scale, 436 B per token",
            "cache_copies": copies, "ms_per_call": round(ms, 5), "tokens_per_s": round(N / (ms * 1e-3), 1),
            "bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TF, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TF, 4), "hbm_gbs": round(gbs, 2),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bf16_cache_ms_per_call": round(bf16_ms, 5),
            "speedup_vs_bf16_cache": round(bf16_ms / ms, 3)}


def out_hidden_timing(lib, synth, wl, dev, out, steps: int):
    """The output projection to the hidden width (mla_out_proj_hidden) on the step's per-head output:
    W^O [heads * 128][5120] rotated through enough copies to exceed the Infinity Cache, calls
    between HIP events.  bytes = weights + per-head rows read + hidden rows written."""
    import torch
    if wl.layers > 1:
        return None
    B, H = wl.batch, wl.heads
    wbytes = H * D_V * D_MODEL * 2
    copies = max(2, -(-400_000_000 // wbytes))
    ws_ = [synth.output_weights(wl, i, device=dev).view(torch.bfloat16) for i in range(copies)]
    hidden = torch.empty(B, D_MODEL, dtype=torch.bfloat16, device=dev)
    work = torch.empty(lib.mla_out_proj_hidden_workspace_size(B, H), dtype=torch.uint8, device=dev)
    for i in range(3):
        lib.mla_out_proj_hidden(out, ws_[i % copies], hidden, work)
    torch.cuda.synchronize()
    n = max(steps, 2 * copies)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        lib.mla_out_proj_hidden(out, ws_[i % copies], hidden, work)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    del ws_
    torch.cuda.empty_cache()
    nbytes = wbytes + B * H * D_V * 2 + B * D_MODEL * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"call": "mla_out_proj_hidden", "weights_bytes": wbytes, "weight_copies": copies,
            "ms_per_call": round(ms, 5), "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}


def sparse_timing(lib, synth, wl, dev, q_abs, bt, att, cache, steps: int, dense_ms: float, k: int = 2048):
    """Attention over the top-k tokens of a cheap int8 index on the same workload: index scores and
    top-k (mla_index_topk), then the decode over the kept tokens read in place (mla_decode_topk);
    beside it the two-step form, the gather of the kept rows into compact pages (mla_gather_rows)
    and mla_decode over them.  Each stage between HIP events, `steps` times; the two forms' outputs
    are checked to agree bit for bit.  Algorithmic bytes = every token's 128-byte index vector +
    each kept row once (1,152 bytes)."""
    import torch
    if wl.layers > 1:
        return None
    B, H = wl.batch, wl.heads
    idx = synth.index_cache(wl, 0, device=dev)
    qi = synth.index_queries(wl, 0, device=dev)
    pos = torch.empty((B, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    ws_t = torch.empty(lib.mla_index_topk_workspace_size(B, wl.max_blocks), dtype=torch.uint8, device=dev)
    pk = -(-k // 64)
    comp = torch.empty((B * pk, 64, ROW_ELEMS), dtype=torch.bfloat16, device=dev)
    comp_bt = torch.empty((B, pk), dtype=torch.int32, device=dev)
    ws_d = torch.empty(lib.mla_decode_workspace_size(B, H, pk, 0), dtype=torch.uint8, device=dev)
    inplace = H >= 32                  # the in-place decode runs on the matrix-core kernel only
    ws_i = torch.empty(lib.mla_decode_topk_workspace_size(B, H, k) if inplace else 0, dtype=torch.uint8, device=dev)
    o_g = torch.empty(B, H, D_C, dtype=torch.bfloat16, device=dev)
    o_i = torch.empty(B, H, D_C, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def run(ev=None):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if ev is not None else None
        if marks: marks[0].record(stream)
        lib.mla_index_topk(idx, bt, att, qi, k, pos, cnt, ws_t)
        if marks: marks[1].record(stream)
        lib.mla_gather_rows(cache, bt, pos, cnt, comp, comp_bt)
        if marks: marks[2].record(stream)
        lib.mla_decode(q_abs, comp, comp_bt, cnt, wl.scale, o_g, lse, ws_d)
        if marks: marks[3].record(stream)
        if inplace:
            lib.mla_decode_topk(q_abs, cache, bt, pos, cnt, wl.scale, o_i, lse, ws_i)
        if marks:
            marks[4].record(stream)
            ev.append(marks)

    for _ in range(3):
        run()
    ev = []
    for _ in range(steps):
        run(ev)
    torch.cuda.synchronize()
    if inplace and not torch.equal(o_g.view(torch.int16), o_i.view(torch.int16)):
        raise SystemExit("mla_decode_topk differs from mla_gather_rows + mla_decode")
    st = [sum(m[i].elapsed_time(m[i + 1]) for m in ev) / len(ev) for i in range(4)]
    ms_gather_path = st[0] + st[1] + st[2]
    ms = st[0] + st[3] if inplace else ms_gather_path
    kept = int(cnt.sum().item())
    nbytes = wl.tokens * 128 + kept * ROW_BYTES
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"calls": "mla_index_topk + mla_decode_topk" if inplace else
            f"mla_index_topk + mla_gather_rows + mla_decode (no in-place decode at {H} heads)",
            "k": k, "kept_tokens": kept, "scored_tokens": wl.tokens, "ms_per_call": round(ms, 5),
            "ms_topk": round(st[0], 5), "ms_decode_topk": round(st[3], 5) if inplace else None,
            "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "dense_decode_ms": round(dense_ms, 5),
            "speedup_vs_dense": round(dense_ms / ms, 3),
            "gather_form": {"calls": "mla_index_topk + mla_gather_rows + mla_decode",
                            "ms_per_call": round(ms_gather_path, 5), "ms_gather": round(st[1], 5),
                            "ms_decode": round(st[2], 5),
                            "speedup_vs_dense": round(dense_ms / ms_gather_path, 3)}}


def measured_peaks(dev):
    """What this GPU reaches on plain library work, as the second reference the roofline fractions are
    quoted against: a 2 GiB device copy (bytes read + written; torch's float32 sum over the same
    array reads at only about 4 TB/s, so it is no measure of the peak) and an 8,192-cube bf16 matrix
    product (torch / hipBLASLt).  Each timed with HIP events, best of five after two untimed runs."""
    import torch

    def best(fn, reps=5):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    n = 1 << 29                                   # 2 GiB of float32
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    copy_gbs = 2 * 4 * n / best(lambda: y.copy_(x)) / 1e9
    del x, y
    m = 8192
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(m, m, device=dev, generator=g).to(torch.bfloat16).contiguous()
    b = torch.randn(m, m, device=dev, generator=g).to(torch.bfloat16).contiguous()
    tf = 2 * m ** 3 / best(lambda: torch.matmul(a, b)) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": round(copy_gbs, 1), "mfma_bf16_tflops": round(tf, 1),
            "how": "2 GiB device copy (read + write bytes); 8192^3 bf16 matmul; best of 5"}


def cpu_baseline(wl, seconds: float):
    """The oracle (decompressed form, float64) on whole sequences of the same workload, in order,
    until `seconds` of work are done.  Rate = latent-cache bytes of the finished sequences per
    second of oracle time (gathering the rows included)."""
    from threadpoolctl import threadpool_info

    import synth
    from oracle import mla_oracle as O

    q = synth.to_numpy_u16(synth.queries(wl))
    w_uk, w_uv = (synth.to_numpy_u16(w) for w in synth.weights(wl))
    qf, wk, wv = O.bf16_to_f64(q), O.bf16_to_f64(w_uk), O.bf16_to_f64(w_uv)
    new = synth.to_numpy_u16(synth.new_rows(wl)) if wl.append else None
    done_tokens, seqs, busy = 0, 0, 0.0
    for b in range(wl.batch):
        pages = wl.block_table[b][wl.block_table[b] >= 0]
        cache = np.zeros((wl.num_pages, 64, 576), np.uint16)
        cache[pages] = synth.to_numpy_u16(synth.cache_pages(wl, 0, pages=pages))
        n = int(wl.attended_lens[b])
        t0 = time.perf_counter()
        if wl.append:
            cache = O.append_rows(cache, wl.block_table[b:b + 1], wl.lens[b:b + 1], new[b:b + 1])
        rows = O.bf16_to_f64(O.gather_rows(cache, wl.block_table, b, n))
        for h in range(wl.heads):
            O.decode_head(qf[b, h], rows, wk[h], wv[h], wl.scale)
        busy += time.perf_counter() - t0
        done_tokens += n
        seqs += 1
        if busy >= seconds:
            break
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] or [1])
    blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in pools
                             if i.get("user_api") == "blas"})) or "none found"
    gbs = done_tokens * ROW_BYTES / busy / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle", "blas": blas,
            "sample": f"decode_reference (decompressed, float64): {seqs} of {wl.batch} sequences "
                      f"({done_tokens} attended tokens, all {wl.heads} heads, append + gather included) "
                      f"in {busy:.1f} s of oracle time; host has {len(os.sched_getaffinity(0))} usable cores"}


CALIB_BYTES = 1 << 30   # the calibration copy: 1 GiB read and 1 GiB written


def _pmc_rows(folder: str):
    import csv
    import glob

    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def traffic_summary(fetch_dir: str, write_dir: str, workload: str):
    """Per-call HBM bytes of mla_decode (decode kernel + merge kernel) from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the reading of the same counter on a copy of known size."""
    out = {"workload": workload, "kernel_source_sha": kernel_source_sha(), "per_kernel": {}}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _pmc_rows(folder) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) * 1024 for r in rows if "copyBuffer" in r["Kernel_Name"]
                  or "copy" in r["Kernel_Name"].lower()]
        calib = max(copies) if copies else 0.0
        if calib < 0.5 * CALIB_BYTES:
            raise SystemExit(f"{counter}: no calibration copy found in {folder}")
        scale = CALIB_BYTES / calib
        total = 0.0
        for tag in ("decode_mfma_kernel", "merge"):
            vals = [float(r["Counter_Value"]) * 1024 for r in rows if tag in r["Kernel_Name"]]
            if not vals:
                raise SystemExit(f"{counter}: no {tag} dispatch in {folder}")
            avg = sum(vals) / len(vals) * scale
            out["per_kernel"].setdefault(tag, {})[counter] = {"dispatches": len(vals), "bytes": round(avg)}
            total += avg
        out[counter.lower() + "_scale"] = round(scale, 5)
        out[counter.lower().replace("_size", "") + "_bytes_per_call"] = round(total)
    out["bytes_per_call"] = out["fetch_bytes_per_call"] + out["write_bytes_per_call"]
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def bench_workload(config: int):
    """The timed workload: the numbered configuration, with one appended row per sequence when the
    configuration itself has none (a decode step appends the new token before attending)."""
    import synth

    wl = synth.make_config(config)
    if wl.append or wl.layers > 1:
        return wl
    return synth.make_custom(wl.lens, wl.heads, wl.seed, shuffle=config != 1, append=True,
                             name=wl.name + "+append")


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, bench_workload(args.config).name)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import head_latent_attention_17_amd as lib
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = bench_workload(args.config)
    B, H = wl.batch, wl.heads
    layers = wl.layers
    N = wl.tokens                           # attended tokens per layer
    cache_bytes = N * ROW_BYTES
    sets = args.sets or (4 if cache_bytes < 256e6 else 1)
    n_inst = max(layers, sets)              # independent input sets actually allocated

    bt = torch.as_tensor(wl.block_table, device=dev)
    lens = torch.as_tensor(wl.lens, device=dev)
    att = torch.as_tensor(wl.attended_lens.astype(np.int32), device=dev)
    inst = []
    for i in range(n_inst):
        # config seeds give each layer its own draws; extra rotation sets reuse the layer streams
        # with a distinct layer index so their bytes differ
        layer = i
        cache = synth.cache_pages(wl, layer, device=dev, chunk_pages=2048).view(torch.bfloat16)
        q = synth.queries(wl, layer, device=dev).view(torch.bfloat16)
        w_uk, w_uv = (w.view(torch.bfloat16) for w in synth.weights(wl, layer, device=dev))
        rows = synth.new_rows(wl, layer, device=dev).view(torch.bfloat16)
        inst.append(dict(cache=cache, q=q, w_uk=w_uk, w_uv=w_uv, c_new=rows[:, :D_C].contiguous(),
                         kpe_new=rows[:, D_C:].contiguous()))
    q_abs = torch.empty(B, H, D_C + D_R, dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty(B, H, D_C, dtype=torch.bfloat16, device=dev)
    out = torch.empty(B, H, D_V, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    ws = torch.empty(lib.mla_decode_workspace_size(B, H, wl.max_blocks, args.splits), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    ev = []

    def one_layer(d, timed):
        if wl.append:
            lib.mla_cache_append(d["cache"], bt, lens, d["c_new"], d["kpe_new"])
        lib.mla_absorb_q(d["q"], d["w_uk"], q_abs)
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
        lib.mla_decode(q_abs, d["cache"], bt, att, wl.scale, o_lat, lse, ws, args.splits)
        if timed:
            b.record(stream)
            ev.append((a, b))
        lib.mla_out_proj(o_lat, d["w_uv"], out)

    def step(i, timed=False):
        if layers > 1:
            for l in range(layers):
                one_layer(inst[l], timed)
        else:
            one_layer(inst[i % sets], timed)

    print(f"bench: {wl.name}, {N} tokens per layer, {layers} layer(s), {sets} input set(s)",
          file=sys.stderr, flush=True)
    if args.profile_run:
        for i in range(args.warmup):
            step(i)
        d = inst[0]
        for _ in range(args.steps):
            lib.mla_decode(q_abs, d["cache"], bt, att, wl.scale, o_lat, lse, ws, args.splits)
        torch.cuda.synchronize()
        del inst
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile run done: {args.steps} mla_decode calls, one {CALIB_BYTES} B copy", file=sys.stderr,
              flush=True)
        return
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    # The decode call's own time comes from a second pass of the same steps with HIP events around
    # each mla_decode (event records between kernels lengthen a step, so they stay out of the pass
    # above).
    for i in range(args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    dec_times = sorted(a.elapsed_time(b) for a, b in ev)
    dec_ms = sum(dec_times) / len(dec_times)
    dec_median = dec_times[len(dec_times) // 2]
    # Warm numbers, labelled: when the cache fits in the 256 MB Infinity Cache, the same input set
    # every call (the steps above rotate sets so that each call reads HBM).
    warm = None
    if cache_bytes < MALL_BYTES and layers == 1:
        d = inst[0]
        for _ in range(3):
            lib.mla_decode(q_abs, d["cache"], bt, att, wl.scale, o_lat, lse, ws, args.splits)
        wev = []
        for _ in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            lib.mla_decode(q_abs, d["cache"], bt, att, wl.scale, o_lat, lse, ws, args.splits)
            b.record(stream)
            wev.append((a, b))
        torch.cuda.synchronize()
        wms = sum(a.elapsed_time(b) for a, b in wev) / len(wev)
        warm = {"label": "warm: one input set, cache resident in the Infinity Cache",
                "ms_per_launch": round(wms, 5), "achieved": round(cache_bytes / (wms * 1e-3) / 1e9, 2)}
    peaks = measured_peaks(dev)

    decode_flops = N * 2 * H * (D_C + D_R + D_C)
    proj_flops = 2 * 2 * B * H * D_NOPE * D_C
    step_flops = layers * (decode_flops + proj_flops)
    step_cache = layers * cache_bytes
    value = step_cache / (ms_step * 1e-3) / 1e9
    dec_gbs = cache_bytes / (dec_ms * 1e-3) / 1e9
    dec_tf = decode_flops / (dec_ms * 1e-3) / 1e12
    traffic = traffic_record(wl.name)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based draws, bf16)",
        "config": {"workload": wl.name, "batch": B, "heads": H, "layers": layers,
                   "attended_tokens_per_layer": N, "page_size": 64, "input_sets": sets,
                   "step": ("append+" if wl.append else "") + "absorb+decode+merge+out_proj",
                   "num_splits": args.splits or "auto"},
        "tflops": round(step_flops / (ms_step * 1e-3) / 1e12, 3),
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "mla_decode (decode + merge kernels)", "bound": "hbm",
                     "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_call"],
                     "ms_per_launch": round(dec_ms, 5),
                     "ms_per_launch_median": round(dec_median, 5),
                     "mfma_tflops": round(dec_tf, 2),
                     "mfma_frac": round(dec_tf / MFMA_BF16_PEAK_TF, 4),
                     "measured_peaks": peaks,
                     "frac_of_measured_copy": round(dec_gbs / peaks["hbm_copy_gbs"], 4),
                     "mfma_frac_of_measured": round(dec_tf / peaks["mfma_bf16_tflops"], 4)},
    }
    if warm is not None:
        line["roofline"]["warm"] = warm
    if wl.append:  # the table has a slot at each sequence's next position only when the workload appends
        line["producer"] = producer_timing(lib, synth, wl, dev, inst[0]["cache"], bt, lens, args.steps)
    sp = sparse_timing(lib, synth, wl, dev, q_abs, bt, att, inst[0]["cache"], args.steps, dec_ms)
    if sp is not None:
        line["sparse_topk"] = sp
    oh = out_hidden_timing(lib, synth, wl, dev, out, args.steps)
    if oh is not None:
        line["out_proj_hidden"] = oh
    fp6 = fp6_timing(lib, synth, wl, dev, q_abs, bt, att, o_lat, lse, ws, args.steps, args.splits, dec_ms)
    if fp6 is not None:
        line["fp6"] = fp6
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
