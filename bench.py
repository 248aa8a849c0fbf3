"""Benchmark: MLA decode steps over a paged latent cache on one MI355X.

A step is the whole path for one batch and every layer: query absorption through W_UK (mla_absorb_q),
then latent decode attention with its split merge and the W_UV out-projection in one call
(mla_decode_out_proj: the decode kernel, then one kernel for the merge and the projection), plus the
cache append of one new row per sequence in the one-layer workloads.  The same steps with the decode
and the out-projection as two calls (mla_decode, mla_out_proj) are timed beside them.  Inputs are seeded synthetic data resident in HBM
before timing starts.

Default workload (the headline line): the full 60-layer decode step, 64 sequences with cached
lengths uniform in [4,096, 8,192], 128 heads, 64-token pages with a shuffled block table, each layer
with its own cache, W_UK, W_UV and query (27 GB of cache per step).

Prints one JSON line.  `value` is latent-cache GB/s over the whole step (layers x tokens x 1,152 B /
step time), from K steps timed between two synchronisations with nothing else on the stream.
`roofline` reports the dominant call, mla_decode, timed with HIP events on the launch stream in a
second pass of the same K steps (mean and median per layer call), against the datasheet peaks and
against what this GPU measures on plain library work (a device copy, a bf16 matrix product).
`calls_per_layer` gives the calls of a layer the same way (the fused call against its algorithmic
bytes: cache, W_UV and the output rows).

Blocks `c3`, `c2`, `c4`, `c1` time the other workloads the same way (a whole step, then each call):
4 x 131,072 tokens (the long-context decode), 32 x 4,096 (the batched decode whose matrix-core
fraction is the one to read), 128 ragged sequences and the 16-head single sequence.  A cache that
fits the 256 MB Infinity Cache is rotated through four independent input sets and also timed warm,
labelled.  The further calls are measured on the long-context and batched workloads:
`sparse_topk` (attention over each sequence's 2,048 best tokens of a cheap int8 index, read in
place, beside the form that first gathers them), `fp6` (mla_decode_fp6 over the ~6-bit form of the
same cache), and on the batched one `out_proj_hidden` (the projection to the hidden width through
W^O) and `producer` (mla_cache_append_hidden, graph-replayed over 48 weight copies).
`cpu_baseline` times the CPU oracle (decompressed form, float64) on a bounded sample of the headline
workload: whole sequences of its first layer (gather + every head), in order, until about
--cpu-seconds of work is done.

    python bench.py [--steps K] [--warmup W] [--config 1..5] [--main-only] [--no-cpu-baseline]
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
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--main-only", action="store_true", help="time only the --config workload")
    ap.add_argument("--sets", type=int, default=0, help="independent input sets (0 = auto)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-side-records", action="store_true",
                    help="skip the further calls on the main workload (top-k, ~6-bit, hidden-width "
                         "projection, producer): for kernel traces whose per-kernel averages must "
                         "hold only the step's own dispatches")
    ap.add_argument("--profile-run", action="store_true",
                    help="for counter runs: a few untimed steps, then mla_decode alone, then "
                         "mla_decode_out_proj, then mla_decode_fp6 over the cache's ~6-bit form, "
                         "then one 1 GiB device copy that calibrates the byte counters; prints no JSON")
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
    ws_i = torch.empty(lib.mla_decode_topk_workspace_size(B, H, k), dtype=torch.uint8, device=dev)
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
    if not torch.equal(o_g.view(torch.int16), o_i.view(torch.int16)):
        raise SystemExit("mla_decode_topk differs from mla_gather_rows + mla_decode")
    st = [sum(m[i].elapsed_time(m[i + 1]) for m in ev) / len(ev) for i in range(4)]
    ms_gather_path = st[0] + st[1] + st[2]
    ms = st[0] + st[3]
    kept = int(cnt.sum().item())
    nbytes = wl.tokens * 128 + kept * ROW_BYTES
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"calls": "mla_index_topk + mla_decode_topk",
            "k": k, "kept_tokens": kept, "scored_tokens": wl.tokens, "ms_per_call": round(ms, 5),
            "ms_topk": round(st[0], 5), "ms_decode_topk": round(st[3], 5),
            "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "dense_decode_ms": round(dense_ms, 5),
            "speedup_vs_dense": round(dense_ms / ms, 3),
            "gather_form": {"calls": "mla_index_topk + mla_gather_rows + mla_decode",
                            "ms_per_call": round(ms_gather_path, 5), "ms_gather": round(st[1], 5),
                            "ms_decode": round(st[2], 5),
                            "speedup_vs_dense": round(dense_ms / ms_gather_path, 3)}}


def measured_peaks(dev, lib=None):
    """What this GPU reaches on plain work, as the second reference the roofline fractions are quoted
    against: a 2 GiB device copy (bytes read + written; torch's float32 sum over the same array reads
    at only about 4 TB/s, so it is no measure of the peak), plain reads moved the way the decode moves
    its tiles (mla_calibrate_read), an 8,192-cube bf16 matrix product (torch / hipBLASLt), and the
    matrix-core rate itself (mla_calibrate_mfma: every SIMD issuing independent
    v_mfma_f32_32x32x16_bf16 back to back, the decode's instruction).  Each timed with HIP events,
    best of five after two untimed runs."""
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
    out = {"hbm_copy_gbs": round(copy_gbs, 1), "mfma_bf16_tflops": round(tf, 1),
           "how": "2 GiB device copy (read + write bytes); 8192^3 bf16 matmul; best of 5"}
    if lib is not None:
        blocks, iters = 1024, 4096
        buf = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
        t = best(lambda: lib.mla_calibrate_mfma(buf, blocks, iters))
        out["mfma_issue_bf16_tflops"] = round(blocks * 4 * iters * 4 * 32 * 32 * 16 * 2 / t / 1e12, 1)
        out["how"] += ("; mla_calibrate_mfma: 1,024 workgroups x 4 waves x 16,384 independent "
                       "v_mfma_f32_32x32x16_bf16 each")
        # plain reads moved like the decode's tiles: 2.25 GiB, HBM -> LDS in 36 KB chunks
        src = torch.empty(65536 * 36 * 1024, dtype=torch.uint8, device=dev)
        res = torch.empty(512, dtype=torch.int32, device=dev)
        t = best(lambda: lib.mla_calibrate_read(src, res, 512))
        out["hbm_read_gbs"] = round(src.numel() / t / 1e9, 1)
        out["how"] += ("; mla_calibrate_read: 2.25 GiB read HBM -> LDS in 36,864-byte chunks by 512 "
                       "workgroups, three chunks in flight each")
        del src
        torch.cuda.empty_cache()
    return out


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
                      f"({done_tokens} attended tokens, all {wl.heads} heads, "
                      f"{'append + ' if wl.append else ''}gather included{', first layer' if wl.layers > 1 else ''}) "
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
        # the decode kernel (the 16-head one at 16 heads; never the ~6-bit one), then the merge
        tags = ("decode_h16_kernel",) if any("decode_h16_kernel" in r["Kernel_Name"] for r in rows) \
            else ("decode_mfma_kernel",)
        for tag in tags + ("merge",):
            vals = [float(r["Counter_Value"]) * 1024 for r in rows
                    if tag in r["Kernel_Name"] and "out_proj" not in r["Kernel_Name"]]
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
    configuration itself has none and is one layer (a decode step appends the new token before
    attending).  The 60-layer workload is timed as it is stated: absorb, decode and out-projection
    per layer, no append."""
    import synth

    wl = synth.make_config(config)
    if wl.append or wl.layers > 1:
        return wl
    return synth.make_custom(wl.lens, wl.heads, wl.seed, shuffle=config != 1, append=True,
                             name=wl.name + "+append")


class Resident:
    """One workload's inputs resident in HBM: per-layer (or per rotation set) cache, query and weights,
    the shared block table and lengths, and the step's outputs."""

    def __init__(self, lib, synth, wl, dev, sets: int, splits: int):
        import torch
        self.wl, self.splits = wl, splits
        B, H = wl.batch, wl.heads
        self.layers = wl.layers
        self.cache_bytes = wl.tokens * ROW_BYTES
        self.sets = sets or (4 if self.cache_bytes < 256e6 else 1)
        n_inst = max(self.layers, self.sets)
        self.bt = torch.as_tensor(wl.block_table, device=dev)
        self.lens = torch.as_tensor(wl.lens, device=dev)
        self.att = torch.as_tensor(wl.attended_lens.astype(np.int32), device=dev)
        self.inst = []
        for i in range(n_inst):
            # config seeds give each layer its own draws; extra rotation sets reuse the layer streams
            # with a distinct layer index so their bytes differ
            cache = synth.cache_pages(wl, i, device=dev, chunk_pages=2048).view(torch.bfloat16)
            q = synth.queries(wl, i, device=dev).view(torch.bfloat16)
            w_uk, w_uv = (w.view(torch.bfloat16) for w in synth.weights(wl, i, device=dev))
            rows = synth.new_rows(wl, i, device=dev).view(torch.bfloat16)
            self.inst.append(dict(cache=cache, q=q, w_uk=w_uk, w_uv=w_uv, c_new=rows[:, :D_C].contiguous(),
                                  kpe_new=rows[:, D_C:].contiguous()))
        self.q_abs = torch.empty(B, H, D_C + D_R, dtype=torch.bfloat16, device=dev)
        self.o_lat = torch.empty(B, H, D_C, dtype=torch.bfloat16, device=dev)
        self.out = torch.empty(B, H, D_V, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(B, H, dtype=torch.float32, device=dev)
        self.ws = torch.empty(lib.mla_decode_out_proj_workspace_size(B, H, wl.max_blocks, splits),
                              dtype=torch.uint8, device=dev)

    def decode(self, lib, d):
        wl = self.wl
        lib.mla_decode(self.q_abs, d["cache"], self.bt, self.att, wl.scale, self.o_lat, self.lse, self.ws,
                       self.splits)

    def layer(self, lib, d, marks=None, separate=False):
        """One layer of the step: append (one-layer workloads), absorb, then the decode with its merge
        and the W_UV projection in one call (mla_decode_out_proj), or with `separate` as the two calls
        mla_decode and mla_out_proj.  With `marks` (four events) each call is bracketed on the
        stream."""
        wl = self.wl
        if marks: marks[0].record()
        if wl.append:
            lib.mla_cache_append(d["cache"], self.bt, self.lens, d["c_new"], d["kpe_new"])
        if marks: marks[1].record()
        lib.mla_absorb_q(d["q"], d["w_uk"], self.q_abs)
        if marks: marks[2].record()
        if separate:
            self.decode(lib, d)
            lib.mla_out_proj(self.o_lat, d["w_uv"], self.out)
        else:
            lib.mla_decode_out_proj(self.q_abs, d["cache"], self.bt, self.att, wl.scale, d["w_uv"], self.out,
                                    None, None, self.ws, self.splits)
        if marks: marks[3].record()

    def step(self, lib, i, marks_out=None, separate=False):
        import torch
        ds = self.inst[:self.layers] if self.layers > 1 else [self.inst[i % self.sets]]
        for d in ds:
            marks = None
            if marks_out is not None:
                marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                marks_out.append(marks)
            self.layer(lib, d, marks, separate)


def graph_timing(lib, res: Resident, steps: int) -> dict:
    """The step, and mla_decode alone, captured in HIP graphs and replayed: the kernels run back to
    back, without the host's per-call work (argument checks, marshalling, launches) between them,
    which is what a serving loop that replays a captured decode step sees.  One capture covers one
    step per input set (all layers of a multi-layer step); the replays are timed between two
    synchronisations.  Each graph's first replay is checked against the eager calls' outputs."""
    import torch
    wl = res.wl
    n_cap = 1 if res.layers > 1 else res.sets
    reps = max(2, steps // n_cap)
    out = {"how": "torch.cuda.CUDAGraph capture of the library calls, replays between synchronisations"}

    def timed(g, per):
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / (reps * per)

    # eager reference of the last captured step's output, then the captured form
    for i in range(n_cap):
        res.step(lib, i)
    torch.cuda.synchronize()
    ref = res.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_cap):
            res.step(lib, i)
    res.out.zero_()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(ref.view(torch.int16), res.out.view(torch.int16)):
        raise RuntimeError("graph replay of the step differs from the eager step")
    out["ms_per_step"] = round(timed(g, n_cap), 5)
    del g
    ds = res.inst[:res.layers] if res.layers > 1 else res.inst[:res.sets]
    gd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gd):
        for d in ds:
            res.decode(lib, d)
    ms = timed(gd, len(ds))
    del gd
    gbs = res.cache_bytes / (ms * 1e-3) / 1e9
    out["decode_call"] = {"ms_per_launch": round(ms, 5), "achieved": round(gbs, 2), "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def time_workload(lib, res: Resident, steps: int, warmup: int) -> dict:
    """Whole steps between two synchronisations (nothing but the path's kernels on the stream); a
    second pass of the same steps with HIP events around every call of every layer, on the stream
    the calls are launched on (torch's current stream, which the binding passes to the library);
    then mla_decode alone (decode + merge kernels, the call the roofline reports) between events on
    the same inputs; then the same steps with the decode and the out-projection as two calls."""
    import torch
    wl = res.wl
    for i in range(warmup):
        res.step(lib, i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        res.step(lib, i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    marks = []
    for i in range(steps):
        res.step(lib, i, marks)
    torch.cuda.synchronize()
    per_call = {}
    for k, name in enumerate(("append", "absorb", "decode_out_proj")):
        ts = sorted(m[k].elapsed_time(m[k + 1]) for m in marks)
        per_call[name] = (sum(ts) / len(ts), ts[len(ts) // 2])
    # mla_decode alone, every layer / rotation set in turn
    ds = res.inst[:res.layers] if res.layers > 1 else res.inst[:res.sets]
    ev = []
    for i in range(max(steps, 1) * (res.layers if res.layers > 1 else 1)):
        d = ds[i % len(ds)]
        lib.mla_absorb_q(d["q"], d["w_uk"], res.q_abs)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        res.decode(lib, d)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    dec_ms, dec_med = sum(ts) / len(ts), ts[len(ts) // 2]
    # the same steps with mla_decode and mla_out_proj as separate calls, against the one-call form in
    # alternating blocks (so that clock drift falls on both alike); medians of three blocks each
    blocks = {False: [], True: []}
    for rnd in range(3):
        for sep in (True, False):
            res.step(lib, 0, separate=sep)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                res.step(lib, i, separate=sep)
            torch.cuda.synchronize()
            blocks[sep].append((time.perf_counter() - t0) * 1e3 / steps)
    ms_sep = sorted(blocks[True])[1]
    ms_one = sorted(blocks[False])[1]
    graph = graph_timing(lib, res, steps)

    N = wl.tokens
    decode_flops = N * 2 * wl.heads * (D_C + D_R + D_C)
    proj_flops = 2 * wl.batch * wl.heads * D_NOPE * D_C
    dec_gbs = res.cache_bytes / (dec_ms * 1e-3) / 1e9
    dec_tf = decode_flops / (dec_ms * 1e-3) / 1e12
    traffic = traffic_record(wl.name)
    wbytes = wl.heads * D_NOPE * D_C * 2
    f_ms, f_med = per_call["decode_out_proj"]
    f_bytes = res.cache_bytes + wbytes + wl.batch * wl.heads * D_V * 2
    f_gbs = f_bytes / (f_ms * 1e-3) / 1e9
    calls = {"decode_out_proj": {"ms_per_launch": round(f_ms, 5), "ms_per_launch_median": round(f_med, 5),
                                 "bytes": f_bytes, "achieved": round(f_gbs, 2), "unit": "GB/s",
                                 "frac": round(f_gbs / HBM_PEAK_GBS, 4),
                                 "mfma_tflops": round((decode_flops + proj_flops) / (f_ms * 1e-3) / 1e12, 2)}}
    ms = per_call["absorb"][0]
    abytes = wbytes + wl.batch * wl.heads * (D_NOPE + D_R + D_C + D_R) * 2
    calls["absorb"] = {"ms_per_launch": round(ms, 5), "bytes": abytes,
                       "achieved": round(abytes / (ms * 1e-3) / 1e9, 1),
                       "frac": round(abytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if wl.append:
        calls["append"] = {"ms_per_launch": round(per_call["append"][0], 5)}
    out = {
        "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "layers": res.layers,
        "attended_tokens_per_layer": N, "input_sets": res.sets, "ms_per_step": round(ms_step, 5),
        "step": ("append+" if wl.append else "") + "absorb+decode_out_proj",
        "ms_per_step_separate_calls": round(ms_sep, 5),
        "ms_per_step_one_call_alternating": round(ms_one, 5),
        "decode_call": {"kernels": "mla_decode (decode + merge kernels)", "bound": "hbm",
                        "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                        "traffic": None if traffic is None else traffic["bytes_per_call"],
                        "ms_per_launch": round(dec_ms, 5), "ms_per_launch_median": round(dec_med, 5),
                        "mfma_tflops": round(dec_tf, 2), "mfma_frac": round(dec_tf / MFMA_BF16_PEAK_TF, 4)},
        "calls_per_layer": calls,
        "graph": graph,
    }
    # Warm numbers, labelled: when the cache fits in the 256 MB Infinity Cache, the same input set
    # every call (the steps above rotate sets so that each call reads HBM).
    if res.cache_bytes < MALL_BYTES and res.layers == 1:
        d = res.inst[0]
        for _ in range(3):
            res.decode(lib, d)
        wev = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            res.decode(lib, d)
            b.record()
            wev.append((a, b))
        torch.cuda.synchronize()
        wms = sum(a.elapsed_time(b) for a, b in wev) / len(wev)
        out["decode_call"]["warm"] = {"label": "warm: one input set, cache resident in the Infinity Cache",
                                      "ms_per_launch": round(wms, 5),
                                      "achieved": round(res.cache_bytes / (wms * 1e-3) / 1e9, 2)}
    return out


def side_records(lib, synth, res: Resident, dev, steps: int, which) -> dict:
    """The further calls on one workload's inputs (layer 0): top-k attention, the ~6-bit decode, the
    output to the hidden width and the producer side of the cache."""
    wl = res.wl
    d = res.inst[0]
    dec_ms = None
    rec = {}
    # a fresh decode time on this workload's first input set, the baseline of the two ratios
    import torch
    for _ in range(3):
        res.decode(lib, d)
    ev = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        res.decode(lib, d)
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    lib.mla_absorb_q(d["q"], d["w_uk"], res.q_abs)
    if "sparse_topk" in which:
        sp = sparse_timing(lib, synth, wl, dev, res.q_abs, res.bt, res.att, d["cache"], steps, dec_ms)
        if sp is not None:
            rec["sparse_topk"] = sp
    if "fp6" in which:
        fp6 = fp6_timing(lib, synth, wl, dev, res.q_abs, res.bt, res.att, res.o_lat, res.lse, res.ws, steps,
                         res.splits, dec_ms)
        if fp6 is not None:
            rec["fp6"] = fp6
    if "out_proj_hidden" in which:
        res.decode(lib, d)
        lib.mla_out_proj(res.o_lat, d["w_uv"], res.out)
        oh = out_hidden_timing(lib, synth, wl, dev, res.out, steps)
        if oh is not None:
            rec["out_proj_hidden"] = oh
    if "producer" in which and wl.append:
        rec["producer"] = producer_timing(lib, synth, wl, dev, d["cache"], res.bt, res.lens, steps)
    return rec


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
    say = lambda *a: print("bench:", *a, file=sys.stderr, flush=True)  # noqa: E731
    say(f"{wl.name}, {wl.tokens} tokens per layer, {wl.layers} layer(s)")
    res = Resident(lib, synth, wl, dev, args.sets, args.splits)

    if args.profile_run:
        for i in range(args.warmup):
            res.step(lib, i)
        d = res.inst[0]
        for _ in range(args.steps):
            res.decode(lib, d)
        for _ in range(args.steps):
            lib.mla_decode_out_proj(res.q_abs, d["cache"], res.bt, res.att, wl.scale, d["w_uv"], res.out, None,
                                    None, res.ws, res.splits)
        fp6 = wl.heads in (64, 128)     # the ~6-bit cache path takes 64 or 128 heads only
        if fp6:
            c6 = torch.empty((d["cache"].shape[0], lib.FP6_PAGE_BYTES), dtype=torch.uint8, device=dev)
            lib.mla_cache_quantize_fp6(d["cache"], c6)
            for _ in range(args.steps):
                lib.mla_decode_fp6(res.q_abs, c6, res.bt, res.att, wl.scale, res.o_lat, res.lse, res.ws,
                                   res.splits)
            del c6
        torch.cuda.synchronize()
        del res
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        say(f"profile run done: {args.steps} mla_decode and mla_decode_out_proj calls"
            f"{', ' + str(args.steps) + ' mla_decode_fp6 calls' if fp6 else ''}, one {CALIB_BYTES} B copy")
        return

    main_rec = time_workload(lib, res, args.steps, args.warmup)
    say(f"main workload timed: {main_rec['ms_per_step']} ms per step")
    B, H, layers, N = wl.batch, wl.heads, wl.layers, wl.tokens
    ms_step = main_rec["ms_per_step"]
    decode_flops = N * 2 * H * (D_C + D_R + D_C)
    proj_flops = 2 * 2 * B * H * D_NOPE * D_C
    step_flops = layers * (decode_flops + proj_flops)
    value = layers * res.cache_bytes / (ms_step * 1e-3) / 1e9
    side = {}
    if layers == 1 and not args.no_side_records:
        side = side_records(lib, synth, res, dev, args.steps,
                            ("sparse_topk", "fp6", "out_proj_hidden", "producer"))
    del res
    torch.cuda.empty_cache()
    peaks = measured_peaks(dev, lib)
    dc = main_rec["decode_call"]
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded counter-based draws, bf16)",
        "config": {"workload": wl.name, "batch": B, "heads": H, "layers": layers,
                   "attended_tokens_per_layer": N, "page_size": 64, "input_sets": main_rec["input_sets"],
                   "step": main_rec["step"], "num_splits": args.splits or "auto"},
        "tflops": round(step_flops / (ms_step * 1e-3) / 1e12, 3),
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": dict(dc, kernel="mla_decode (decode + merge kernels, one call per layer)",
                         measured_peaks=peaks,
                         frac_of_measured_copy=round(dc["achieved"] / peaks["hbm_copy_gbs"], 4),
                         frac_of_measured_read=round(dc["achieved"] / peaks["hbm_read_gbs"], 4),
                         mfma_frac_of_measured=round(dc["mfma_tflops"] / peaks["mfma_bf16_tflops"], 4),
                         mfma_frac_of_issue_rate=round(dc["mfma_tflops"] / peaks["mfma_issue_bf16_tflops"], 4)),
        "calls_per_layer": main_rec["calls_per_layer"],
        "ms_per_step_separate_calls": main_rec["ms_per_step_separate_calls"],
        "ms_per_step_one_call_alternating": main_rec["ms_per_step_one_call_alternating"],
        "graph": main_rec["graph"],
    }
    line["roofline"].pop("kernels", None)
    line.update(side)
    # The other workloads, each its own block: the long-context decode (4 x 131,072 tokens) with the
    # further calls measured on it, the batched one (32 x 4,096) whose matrix-core fraction is the
    # one to read, the 16-head one and the ragged one.
    if not args.main_only:
        for cfg in (3, 2, 4, 1):
            if cfg == args.config:
                continue
            wl_c = bench_workload(cfg)
            say(f"{wl_c.name}, {wl_c.tokens} tokens")
            r = Resident(lib, synth, wl_c, dev, 0, args.splits)
            rec = time_workload(lib, r, args.steps, args.warmup)
            if cfg in (2, 3):
                rec.update(side_records(lib, synth, r, dev, args.steps,
                                        ("sparse_topk", "fp6") if cfg == 3 else
                                        ("sparse_topk", "fp6", "out_proj_hidden", "producer")))
            del r
            torch.cuda.empty_cache()
            line[f"c{cfg}"] = rec
    if not args.no_cpu_baseline:
        say("cpu baseline")
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
