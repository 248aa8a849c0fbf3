"""Benchmark: one MLA decode step over a paged latent cache on one MI355X.

A step is the whole path for one batch: cache append (one new row per sequence), query absorption
through W_UK, latent decode attention (with its split merge) and the W_UV out-projection.  Inputs are
seeded synthetic data resident in HBM before timing starts.  Default workload: 32 sequences x 4,096
cached tokens (+1 appended), 128 heads, 64-token pages with a shuffled block table.  The 151 MB
cache fits in the 256 MB Infinity Cache, so the steps rotate through independent input sets.

Prints one JSON line.  `value` is latent-cache GB/s over the whole step (tokens x 1,152 B / step
time).  `roofline` reports the dominant call, mla_decode, timed with HIP events on the launch stream.
`cpu_baseline` times the CPU oracle (decompressed form, float64) on a bounded sample.

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
MFMA_BF16_PEAK_TF = 2500.0   # MI355X dense bf16 MFMA
ROW_BYTES = 1152
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
    return ap.parse_args()


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "head_latent_attention_17_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
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


def cpu_baseline(wl, seconds: float):
    """The oracle (decompressed form, float64) on sequence 0: heads in order until `seconds` pass.
    Rate = latent-cache bytes that the processed heads cover, per second."""
    from threadpoolctl import threadpool_info

    import synth
    from oracle import mla_oracle as O

    b = 0
    n = int(wl.attended_lens[b])
    pages = wl.block_table[b][wl.block_table[b] >= 0]
    cache = np.zeros((wl.num_pages, 64, 576), np.uint16)
    cache[pages] = synth.to_numpy_u16(synth.cache_pages(wl, 0, pages=pages))
    if wl.append:
        cache = O.append_rows(cache, wl.block_table, wl.lens, synth.to_numpy_u16(synth.new_rows(wl)))
    q = synth.to_numpy_u16(synth.queries(wl))
    w_uk, w_uv = (synth.to_numpy_u16(w) for w in synth.weights(wl))
    rows = O.bf16_to_f64(O.gather_rows(cache, wl.block_table, b, n))
    qf, wk, wv = O.bf16_to_f64(q), O.bf16_to_f64(w_uk), O.bf16_to_f64(w_uv)
    t0 = time.perf_counter()
    heads = 0
    while heads < wl.heads:
        O.decode_head(qf[b, heads], rows, wk[heads], wv[heads], wl.scale)
        heads += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    gbs = n * ROW_BYTES * heads / wl.heads / dt / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"decode_reference (decompressed, float64) of sequence 0 ({n} tokens), "
                      f"{heads} of {wl.heads} heads in {dt:.1f} s; host has "
                      f"{len(os.sched_getaffinity(0))} usable cores"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import head_latent_attention_17_amd as lib
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.make_config(args.config)
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
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    dec_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)

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
                   "step": "append+absorb+decode+merge+out_proj" if wl.append or True else "",
                   "num_splits": args.splits or "auto"},
        "tflops": round(step_flops / (ms_step * 1e-3) / 1e12, 3),
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "mla_decode (decode + merge kernels)", "bound": "hbm",
                     "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_call"],
                     "ms_per_launch": round(dec_ms, 5),
                     "mfma_tflops": round(dec_tf, 2),
                     "mfma_frac": round(dec_tf / MFMA_BF16_PEAK_TF, 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
