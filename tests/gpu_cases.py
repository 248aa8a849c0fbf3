"""Helpers for the GPU parity tests: upload synthetic workloads, run the HIP path through the C ABI,
and compare with the CPU oracle.  Not collected by pytest (no test_ prefix)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import synth
from oracle import mla_oracle as O

BF16_TOL = 1e-2   # normwise max relative error, bf16 inputs with fp32 accumulation
F32_TOL = 1e-4    # same metric, fp32 debug mode


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref) -> float:
    """Largest over rows of max|g - r| / max|r| (each row = one (sequence, head) output vector)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    num = np.abs(g - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def lse_err(gpu, ref) -> float:
    """Largest absolute error of the log-sum-exp.  lse is a logarithm, so its absolute error is the
    relative error of the softmax denominator; it is compared absolutely against the same 1e-2 /
    1e-4 bounds.  Entries where the reference is -inf (empty sequences) must be -inf too."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    empty = np.isneginf(r)
    if not np.array_equal(np.isneginf(g), empty):
        return math.inf
    if empty.all():
        return 0.0
    return float(np.abs(g[~empty] - r[~empty]).max())


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return O.bf16_to_f64(t.view(torch.int16).cpu().numpy())
    return t.detach().cpu().double().numpy()


def act(bits16: torch.Tensor, f32: bool) -> torch.Tensor:
    """bf16 bit patterns (int16) -> the activation tensor type of the chosen mode."""
    bf = bits16.view(torch.bfloat16)
    return bf.float() if f32 else bf


class Gpu:
    """A workload resident on the GPU."""

    def __init__(self, wl: synth.Workload, layer: int = 0, f32: bool = False, device="cuda"):
        self.wl, self.layer, self.f32 = wl, layer, f32
        self.cache = synth.cache_pages(wl, layer, device=device).view(torch.bfloat16)
        self.bt = torch.as_tensor(wl.block_table, device=device)
        self.lens = torch.as_tensor(wl.lens, device=device)
        self.attended = torch.as_tensor(wl.attended_lens.astype(np.int32), device=device)
        B, H = wl.batch, wl.heads
        self.q = act(synth.queries(wl, layer, device=device), f32)
        self.q_lat_in = act(synth.latent_queries(wl, layer, device=device), f32)
        w_uk, w_uv = synth.weights(wl, layer, device=device)
        self.w_uk, self.w_uv = act(w_uk, f32), act(w_uv, f32)
        rows = synth.new_rows(wl, layer, device=device)
        self.c_new = act(rows[:, :synth.D_C].contiguous(), f32)
        self.kpe_new = act(rows[:, synth.D_C:].contiguous(), f32)
        dt = torch.float32 if f32 else torch.bfloat16
        self.q_abs = torch.empty(B, H, synth.ROW, dtype=dt, device=device)
        self.o_lat = torch.empty(B, H, synth.D_C, dtype=dt, device=device)
        self.out = torch.empty(B, H, synth.D_V, dtype=dt, device=device)
        self.lse = torch.empty(B, H, dtype=torch.float32, device=device)
        self.ws = None

    def workspace(self, lib, splits=0):
        n = lib.mla_decode_workspace_size(self.wl.batch, self.wl.heads, self.wl.max_blocks, splits,
                                          lib.MLA_F32 if self.f32 else lib.MLA_BF16)
        if self.ws is None or self.ws.numel() < n:
            self.ws = torch.empty(n, dtype=torch.uint8, device=self.cache.device)
        return self.ws

    def step(self, lib, splits=0, q_abs_from_absorb=True):
        """The whole path: append (if the workload appends), absorb, decode, out-projection."""
        wl = self.wl
        if wl.append:
            lib.mla_cache_append(self.cache, self.bt, self.lens, self.c_new, self.kpe_new)
        if q_abs_from_absorb:
            lib.mla_absorb_q(self.q, self.w_uk, self.q_abs)
            qa = self.q_abs
        else:
            qa = self.q_lat_in
        lib.mla_decode(qa, self.cache, self.bt, self.attended, wl.scale, self.o_lat, self.lse,
                       self.workspace(lib, splits), splits)
        lib.mla_out_proj(self.o_lat, self.w_uv, self.out)


def host_inputs(wl: synth.Workload, layer: int, batch_sel):
    """The oracle's view of the inputs for the selected sequences: only their pages are generated
    (on the CPU), plus the appended row when the workload appends."""
    pages = np.unique(np.concatenate([wl.block_table[b][wl.block_table[b] >= 0] for b in batch_sel]))
    cache = np.zeros((wl.num_pages, synth.PAGE, synth.ROW), np.uint16)
    cache[pages] = synth.to_numpy_u16(synth.cache_pages(wl, layer, pages=pages))
    if wl.append:
        rows = synth.to_numpy_u16(synth.new_rows(wl, layer))
        cache = O.append_rows(cache, wl.block_table, wl.lens, rows)
    q = synth.to_numpy_u16(synth.queries(wl, layer))
    q_lat = synth.to_numpy_u16(synth.latent_queries(wl, layer))
    w_uk, w_uv = synth.weights(wl, layer)
    return dict(cache=cache, q=q, q_lat=q_lat, w_uk=synth.to_numpy_u16(w_uk),
                w_uv=synth.to_numpy_u16(w_uv))


def scale_of(wl):
    return wl.scale


def pick(n, k, seed):
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(n, size=min(k, n), replace=False).tolist())
