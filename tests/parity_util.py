"""Helpers shared by the GPU parity tests: run a workload through the HIP path (via the
C-ABI binding) and through the oracle on the same seeded inputs, and compare."""

from __future__ import annotations

import concurrent.futures as cf
import os
import sys
import time

import numpy as np

from mixed_head_kv_amd import inputs as I
from oracle import attention as OA
from oracle import int4 as OQ

TOL = {"bf16": 2e-2, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_synth(w: I.Workload, layer: int, kind: str, pos0: int, T: int):
    """Q/K/V rows [T, H, D] for positions [pos0, pos0+T) generated on the device by the
    library's fill kernel (same definition as inputs.synth)."""
    import torch
    from mixed_head_kv_amd import binding as B
    H = w.n_q_heads if kind == "q" else w.n_kv_heads
    dt = torch.float32 if w.io_dtype == "f32" else torch.bfloat16
    t = torch.empty((T, H, w.head_dim), dtype=dt, device="cuda")
    B.duo_synth_fill(t, B.DUO_DTYPE_F32 if w.io_dtype == "f32" else B.DUO_DTYPE_BF16, w.seed,
                     layer * 4 + I.KIND_STREAM[kind], pos0 * H * w.head_dim, T * H * w.head_dim)
    return t


def host_rows(w: I.Workload, layer: int, kind: str, pos0: int, T: int) -> np.ndarray:
    H = w.n_q_heads if kind == "q" else w.n_kv_heads
    return OA.upcast(I.synth(w.seed, layer, kind, pos0, T, H, w.head_dim, w.io_dtype), w.io_dtype)


def host_history(w: I.Workload, layer: int, kind: str, L: int) -> np.ndarray:
    """Full K or V history [L, Hkv, D] as the caches hold it: exact for bf16/f32, the
    oracle codec's dequantised values for int4."""
    raw = I.synth(w.seed, layer, kind, 0, L, w.n_kv_heads, w.head_dim, w.io_dtype)
    if w.kv_format == "int4":
        codes, s, z = OQ.quantize(raw)
        return OQ.dequantize(codes, s, z).astype(np.float64)
    return OA.upcast(raw, w.io_dtype)


THREADS = max(1, min(16, os.cpu_count() or 1))


def head_history(w: I.Workload, layer: int, kind: str, g: int, positions) -> np.ndarray:
    """K or V rows [n, D] (float64) of KV head g at the given positions, as the cache
    holds them (int4: the oracle codec's dequantised values).  Processed in slices, in
    parallel threads (each vector is quantised on its own), so a 3.3M-token head is
    prepared in seconds and fits in host memory."""
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((len(positions), w.head_dim), dtype=np.float64)
    step = 1 << 16

    def fill(a):
        raw = I.synth_head(w.seed, layer, kind, positions[a:a + step], g, w.n_kv_heads, w.head_dim, w.io_dtype)
        if w.kv_format == "int4":
            codes, s, z = OQ.quantize(raw)
            out[a:a + step] = OQ.dequantize(codes, s, z)
        else:
            out[a:a + step] = OA.upcast(raw, w.io_dtype)

    starts = list(range(0, len(positions), step))
    if len(starts) <= 1:
        for a in starts:
            fill(a)
    else:
        with cf.ThreadPoolExecutor(THREADS) as ex:
            list(ex.map(fill, starts))
    return out


def oracle_decode_steps(w: I.Workload, layer: int, t0: int, n_steps: int, kv_heads, q) -> dict:
    """Oracle decode outputs at positions t0 .. t0 + n_steps - 1 (one token per step, the
    history through each step's own position) for the query heads of the given KV heads.
    q: [n_steps, Hq, D] stored query values.  Returns {query head: [n_steps, D]}.  Each
    KV head's history is prepared once; KV heads run in parallel threads."""
    qf = OA.upcast(q, w.io_dtype)
    mask = w.mask(layer)
    t_last = t0 + n_steps - 1
    pos_q = np.arange(t0, t0 + n_steps)

    def one(g):
        if mask[g]:
            pos = np.arange(t_last + 1)
            K = head_history(w, layer, "k", g, pos)
            V = head_history(w, layer, "v", g, pos)
        else:  # the sinks and every step's window (other rows are never visible)
            pos = np.unique(np.concatenate([np.arange(min(w.sink, t_last + 1)),
                                            np.arange(max(0, t0 - w.recent + 1), t_last + 1)]))
            K = np.zeros((t_last + 1, w.head_dim))
            V = np.zeros((t_last + 1, w.head_dim))
            K[pos] = head_history(w, layer, "k", g, pos)
            V[pos] = head_history(w, layer, "v", g, pos)
        return {g * w.group + i: OA.head_attention(qf[:, g * w.group + i], pos_q, K, V, bool(mask[g]), w.sink,
                                                   w.recent)
                for i in range(w.group)}

    out = {}
    with cf.ThreadPoolExecutor(min(len(kv_heads), 4)) as ex:  # (each history is gigabytes)
        for d in ex.map(one, kv_heads):
            out.update(d)
    return out


def oracle_rows_threaded(w: I.Workload, layer: int, rows, total: int, heads=None) -> np.ndarray:
    """Oracle outputs [len(rows), Hq, D] at absolute positions `rows`, like oracle_rows,
    with the query heads computed in parallel threads (NumPy releases the interpreter
    lock inside its array operations)."""
    rows = np.asarray(rows, dtype=np.int64)
    Kh = host_history(w, layer, "k", total)
    Vh = host_history(w, layer, "v", total)
    Qh = OA.upcast(q_rows(w, layer, rows), w.io_dtype)
    mask = w.mask(layer)
    out = np.full((len(rows), w.n_q_heads, w.head_dim), np.nan)

    def one(h):
        g = h // w.group
        out[:, h] = OA.head_attention(Qh[:, h], rows, Kh[:, g], Vh[:, g], bool(mask[g]), w.sink, w.recent)

    with cf.ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(one, range(w.n_q_heads) if heads is None else heads))
    return out


def q_rows(w: I.Workload, layer: int, rows) -> np.ndarray:
    """Q [len(rows), Hq, D] at arbitrary absolute positions (stored dtype)."""
    rows = np.asarray(rows, dtype=np.uint64)
    HD = w.n_q_heads * w.head_dim
    counters = rows[:, None] * np.uint64(HD) + np.arange(HD, dtype=np.uint64)[None, :]
    x = I.values_f32(w.seed, layer * 4 + I.KIND_STREAM["q"], counters)
    x = I.f32_to_bf16_bits(x) if w.io_dtype == "bf16" else x
    return x.reshape(len(rows), w.n_q_heads, w.head_dim)


def fill_stack(w: I.Workload, kv, chunk: int = 65536):
    """Fill every layer's caches with positions [0, context) via duo_kv_append."""
    import torch
    from mixed_head_kv_amd import binding as B
    kbuf = torch.empty((chunk, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    for layer in range(w.n_layers):
        for c0 in range(0, w.context, chunk):
            T = min(chunk, w.context - c0)
            n = T * w.n_kv_heads * w.head_dim
            B.duo_synth_fill(kbuf, B.DUO_DTYPE_BF16, w.seed, layer * 4 + 1, c0 * w.n_kv_heads * w.head_dim, n)
            B.duo_synth_fill(vbuf, B.DUO_DTYPE_BF16, w.seed, layer * 4 + 2, c0 * w.n_kv_heads * w.head_dim, n)
            kv.append(layer, kbuf[:T], vbuf[:T])
    torch.cuda.synchronize()


def guard_violations(kv) -> list:
    """Byte offsets of the guard bands of a DuoKV's workspace that no longer hold the
    pattern duo_kv_init wrote there (a kernel wrote outside its region)."""
    import struct
    import torch
    from mixed_head_kv_amd import binding as B
    offs = B.duo_kv_guard_bands(kv.h)
    if not offs:
        return []
    ws = kv.workspace
    idx = (torch.tensor(offs, dtype=torch.int64, device=ws.device)[:, None] +
           torch.arange(B.DUO_GUARD_BYTES, dtype=torch.int64, device=ws.device)[None, :])
    pat = torch.tensor(list(struct.pack("<I", B.DUO_GUARD_WORD)) * (B.DUO_GUARD_BYTES // 4), dtype=torch.uint8,
                       device=ws.device)
    bad = (ws[idx] != pat[None, :]).any(dim=1).cpu().numpy()
    return [o for o, b in zip(offs, bad) if b]


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_layer(w: I.Workload, chunks, decode_steps: int, layer: int = 0, kv=None, append_only_chunks=False):
    """Prefill the chunks (or append them, for int4 / bulk fill) and run decode steps on
    one layer.  Returns (kv, prefill outputs [sum(chunks), Hq, D] or None, decode outputs
    [steps, Hq, D], total tokens)."""
    import torch
    from mixed_head_kv_amd.binding import DuoKV
    if kv is None:
        kv = DuoKV.for_workload(w)
    total = sum(chunks) + decode_steps
    Q = device_synth(w, layer, "q", 0, total)
    K = device_synth(w, layer, "k", 0, total)
    V = device_synth(w, layer, "v", 0, total)
    pre = []
    t = 0
    for T in chunks:
        if append_only_chunks:
            kv.append(layer, K[t:t + T], V[t:t + T])
        else:
            pre.append(kv.prefill(layer, Q[t:t + T], K[t:t + T], V[t:t + T]))
        t += T
    dec = []
    for _ in range(decode_steps):
        dec.append(kv.decode(layer, Q[t], K[t], V[t]))
        t += 1
    torch.cuda.synchronize()
    pre_out = torch.cat(pre, 0) if pre else None
    dec_out = torch.stack(dec, 0) if dec else None
    return kv, pre_out, dec_out, total


def oracle_rows(w: I.Workload, layer: int, rows, total: int, heads=None) -> np.ndarray:
    """Oracle outputs [len(rows), Hq, D] at absolute positions `rows`."""
    rows = np.asarray(rows, dtype=np.int64)
    Kh = host_history(w, layer, "k", total)
    Vh = host_history(w, layer, "v", total)
    Qh = OA.upcast(q_rows(w, layer, rows), w.io_dtype)
    return OA.layer_attention(Qh, rows, Kh, Vh, w.mask(layer), w.sink, w.recent, heads=heads)


def compare(name: str, got: np.ndarray, ref: np.ndarray, tol: float):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    say(f"  {name}: max-abs err {err:.3e} (tol {tol:g}) over {got.size} values")
    assert err <= tol, f"{name}: max-abs error {err} > {tol}"
    return err


class Timer:
    def __enter__(self):
        self.t = time.perf_counter()
        return self

    def __exit__(self, *a):
        self.dt = time.perf_counter() - self.t
