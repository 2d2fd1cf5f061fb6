"""Benchmark of the mixed-head attention hot path on one MI355X.

One step = one pass of the whole path over one synthetic sequence of the workload:
head regrouping (handle init), every prefill chunk (append/evict, retrieval causal
attention, streaming sink + window attention) and every decode step (append/evict,
split-K retrieval decode + streaming decode + merge).  Inputs (Q, K, V for every
position) are generated on the device before timing and stay resident in HBM.

Default workload: Llama-3-8B-shaped GQA layer (32 query / 8 KV heads, head_dim 128, bf16,
4 of 8 KV heads retrieval, sink 64 + recent 256), 131072-token prefill in 8192-token
chunks, then 256 decode steps: the largest single-layer configuration, which carries
both halves of the metric (decode us/step and prefill tok/s).  Prints one JSON line;
`value` is the step's whole-job throughput, (prefill + decode tokens) / step time, and
`components` carries the metric's two numbers.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
# Kernel arguments in device memory (HIP runtime setting, read when HIP initialises):
# the command processor then does not fetch them from host memory at every dispatch,
# which shortens the gap between dependent launches (32K decode: 32.1 -> 29.3 us/step).
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

METRIC = "DuoAttn layer decode µs/step & prefill tok/s at context L; % HBM/MFMA roofline"
DEFAULT_WORKLOAD = "llama3_8b_gqa_128k"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, vendor figure


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {
    "decode_attention": "mixed_head_kv_amd/csrc/decode_mfma.hip",
    "prefill_attention": "mixed_head_kv_amd/csrc/prefill_mfma.hip",
    "prefill_streaming_attention": "mixed_head_kv_amd/csrc/prefill_mfma.hip",
    "prefill_chunk_tiles": "mixed_head_kv_amd/csrc/prefill_mfma.hip",
    "qkv_rope_decode": "mixed_head_kv_amd/csrc/linear_w8.hip",
    "out_proj_decode": "mixed_head_kv_amd/csrc/linear_w8.hip",
    "qkv_rope_prefill": "mixed_head_kv_amd/csrc/linear_w8.hip",
    "out_proj_prefill": "mixed_head_kv_amd/csrc/linear_w8.hip",
    "prefill_dual_attention": "mixed_head_kv_amd/csrc/prefill_mfma.hip",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(kernel):
    """The kernel's source file and the hipcc flags it builds with."""
    import hashlib
    from mixed_head_kv_amd import build
    path = os.path.join(ROOT, KERNEL_SOURCES[kernel])
    flags = " ".join(build.flags_for(os.path.basename(path))).encode()
    return hashlib.sha256(open(path, "rb").read() + b"\0" + flags).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/traffic.json), or None when none was taken for this kernel and workload or
    the kernel's source has changed since."""
    try:
        entries = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    for e in entries:
        if e.get("kernel") == kernel and e.get("workload") == workload and e.get("source") == source_digest(kernel):
            return e.get("bytes_per_launch")
    return None


def copy_probe():
    """A plain device copy of a known size (1 GiB read + 1 GiB written), so counter runs
    can calibrate FETCH_SIZE / WRITE_SIZE against known bytes."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def esize(w):
    return 4 if w.io_dtype == "f32" else 2


def decode_bytes(w, t, layer=0):
    """Algorithmic HBM bytes of one decode-attention launch at query position t, one
    layer: K+V of every visible key counted once per KV head (GQA sharing), plus Q and O.
    int4 vectors cost 64 code bytes + 4 bytes of scale/zero."""
    mask = w.mask(layer)
    nr = int(mask.sum())
    ns = w.n_kv_heads - nr
    vec = 68 if w.kv_format == "int4" else w.head_dim * esize(w)
    kv = 2 * vec * (nr * (t + 1) + ns * min(t + 1, w.sink + w.recent))
    qo = 2 * w.n_q_heads * w.head_dim * esize(w)
    return kv + qo


def prefill_flops(w, t0, T, retrieval=True):
    """Algorithmic flops of one prefill chunk [t0, t0+T): 4*D per visible (query, key)
    pair (QK^T and PV), retrieval heads over causal pairs, streaming heads over
    min(i+1, sink+recent) pairs."""
    mask = w.mask(0)
    G = w.group
    if retrieval:
        pairs = T * t0 + T * (T + 1) // 2
        return 4 * w.head_dim * pairs * int(mask.sum()) * G
    cap = w.sink + w.recent
    pairs = sum(min(i + 1, cap) for i in range(t0, t0 + T))
    return 4 * w.head_dim * pairs * int((~mask).sum()) * G


STAGE_TOKENS = 4096  # queries per streaming-head prefill launch (the library's staging capacity)


def chunk_tile_bytes(w, t0, T):
    """Algorithmic HBM bytes of the chunk-tile launches of one prefill chunk [t0, t0+T):
    the chunk's K+V rows read and written once per retrieval KV head (the append), and
    per streaming KV head and launch of at most STAGE_TOKENS queries the staged rows
    written (sink rows, window rows from R-1 positions before the first query, the
    queries' own rows, each rounded up to 64) plus the K+V rows read (sinks and window
    positions that hold a key)."""
    al = lambda x: (x + 63) // 64 * 64
    nr = int(w.mask(0).sum())
    ns = w.n_kv_heads - nr
    vec = 2 * w.head_dim * esize(w)  # K + V of one row
    sp, win = al(w.sink), al(w.recent - 1)
    total = nr * vec * 2 * T
    tc = min(STAGE_TOKENS, al(w.max_context))
    for q0 in range(0, T, tc):
        nq = min(tc, T - q0)
        u0 = t0 + q0
        written = sp + win + al(nq)
        read = min(w.sink, u0 + nq) + (u0 + nq - max(w.sink, u0 - win, t0 - w.recent, 0))
        total += ns * vec * (written + read)
    return total


def measure_projections(w, chunk, reps_decode=40, reps_prefill=5):
    """The 8-bit-weight layers around the attention at the workload's model shape (hidden =
    n_q_heads * head_dim): the fused QKV projection with the rotary encoding and the output
    projection, for one decoding token (HBM-bound on the codes) and, when chunk > 0, a
    pre-filling chunk of that many tokens (MFMA-bound).  Synthetic int8 weights; every
    launch is stamped at its dispatch (duo_profile_thread_*).  Returns roofline entries
    (algorithmic work: codes + scales + activations in + outputs for the decoding token,
    2 M N K flops for the chunk)."""
    import numpy as np
    import torch

    from mixed_head_kv_amd import binding as B
    from mixed_head_kv_amd import inputs as I

    D, Hq, Hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    hidden = Hq * D
    Nqkv = (Hq + 2 * Hkv) * D
    base = 10000.0 if Hq == Hkv else 500000.0  # Llama-2 (MHA) / Llama-3 (GQA)
    dev = torch.device("cuda", 0)

    def weights(which, N, K):
        wt = torch.empty((N, K), dtype=torch.int8, device=dev)
        B.duo_synth_fill(wt, B.DUO_SYNTH_INT8, w.seed, I.weight_stream(0, which), 0, N * K)
        return wt, torch.from_numpy(I.weight_scales(w.seed, 0, which, N, K)).to(dev)

    wq, sq = weights("qkv", Nqkv, hidden)
    wo, so = weights("o", hidden, hidden)
    out = []
    for M, reps in ((1, reps_decode), (chunk, reps_prefill)):
        if M <= 0:
            continue
        x = torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)
        B.duo_synth_fill(x, B.DUO_DTYPE_BF16, w.seed, I.KIND_STREAM["x"], 0, M * hidden)
        pos = torch.arange(w.context - M, w.context, dtype=torch.int64, device=dev).clamp_(min=0)
        q = torch.empty((M, Hq, D), dtype=torch.bfloat16, device=dev)
        k = torch.empty((M, Hkv, D), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        y = torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)
        st = B._stream(torch.cuda.current_stream())
        for _ in range(2):  # warm-up
            B.duo_qkv_rope_w8(x, M, hidden, pos, wq, sq, Hq, Hkv, D, base, q, k, v, st)
            B.duo_linear_w8(q, M, hidden, wo, so, hidden, y, st)
        torch.cuda.synchronize()
        B.duo_profile_thread_enable(True)
        for _ in range(reps):
            B.duo_qkv_rope_w8(x, M, hidden, pos, wq, sq, Hq, Hkv, D, base, q, k, v, st)
        for _ in range(reps):
            B.duo_linear_w8(q, M, hidden, wo, so, hidden, y, st)
        B.duo_profile_thread_enable(False)
        tot = B.duo_profile_thread_collect()
        for cls, name, N in (("qkv_rope", "qkv_rope", Nqkv), ("linear", "out_proj", hidden)):
            ms, n = tot[cls]
            us = ms * 1e3 / n
            if M == 1:
                work = N * hidden + 4 * N + 2 * hidden + 2 * N + (8 if cls == "qkv_rope" else 0)
                a = work / (us * 1e-6) / 1e9
                out.append({"kernel": f"{name}_decode", "bound": "hbm", "achieved": round(a, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
                            "avg_launch_us": round(us, 3), "tokens": 1, "n_out": N, "k": hidden,
                            "traffic": None})
            else:
                a = 2.0 * M * N * hidden / (us * 1e-6) / 1e12
                out.append({"kernel": f"{name}_prefill", "bound": "mfma", "achieved": round(a, 2),
                            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4), "avg_launch_us": round(us, 2),
                            "tokens": M, "n_out": N, "k": hidden, "traffic": None})
        del x, q, k, v, y
    for r in out:
        r["traffic"] = measured_traffic(r["kernel"], w.name)
    return out


def measure_identification(w, chunks):
    """Head-identification pre-filling (duo_prefill_dual) over the workload's chunks with
    every KV head holding a full cache: every head's full causal output and its
    sinks + window output.  Algorithmic flops: the causal pairs of every head plus its
    sink + window pairs (4 D flops each).  One pass after a warm-up pass."""
    import numpy as np
    import torch

    from mixed_head_kv_amd import binding as B
    from mixed_head_kv_amd import inputs as I

    wa = w.scaled(n_retrieval=w.n_kv_heads, fixed_retrieval=None)
    dev = torch.device("cuda", 0)
    L = sum(chunks)
    cfg = B.make_config(1, 1, wa.n_q_heads, wa.n_kv_heads, wa.head_dim, wa.sink, wa.recent, L,
                        B.DUO_DTYPE_BF16, B.DUO_KV_SAME_AS_IO, np.ones(wa.n_kv_heads, dtype=np.uint8))
    ws = torch.empty(B.duo_kv_bytes(cfg), dtype=torch.uint8, device=dev)

    def synth(kind, H):
        t = torch.empty((L, H, wa.head_dim), dtype=torch.bfloat16, device=dev)
        B.duo_synth_fill(t, B.DUO_DTYPE_BF16, wa.seed, I.KIND_STREAM[kind], 0, t.numel())
        return t

    Q, K, V = synth("q", wa.n_q_heads), synth("k", wa.n_kv_heads), synth("v", wa.n_kv_heads)
    of = torch.empty((max(chunks), wa.n_q_heads, wa.head_dim), dtype=torch.bfloat16, device=dev)
    os_ = torch.empty_like(of)
    st = B._stream(torch.cuda.current_stream())
    ms = 0.0
    for rep in range(2):
        h = B.duo_kv_init(cfg, ws, st)
        if rep:
            B.duo_profile_enable(h, True)
        t = 0
        for T in chunks:
            B.duo_prefill_dual(h, 0, Q[t:t + T], K[t:t + T], V[t:t + T], T, of, os_, st)
            t += T
        if rep:
            ms = B.duo_profile_collect(h)["prefill_retrieval"][0]
        B.duo_kv_free(h)
    torch.cuda.synchronize()
    full = stream = 0
    t = 0
    for T in chunks:
        full += prefill_flops(wa, t, T, True)
        ws_ = wa.scaled(n_retrieval=0, fixed_retrieval=None)
        stream += prefill_flops(ws_, t, T, False)
        t += T
    a = (full + stream) / (ms * 1e-3) / 1e12
    return {"kernel": "prefill_dual_attention", "bound": "mfma", "achieved": round(a, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4),
            "avg_launch_us": round(ms * 1e3 / len(chunks), 2), "ms_per_pass": round(ms, 4),
            "tokens": L, "traffic": measured_traffic("prefill_dual_attention", w.name)}


def run_extras(args):
    """The projections and the identification pre-filling of the workload, alone."""
    import torch
    w = workload_for(args)
    torch.cuda.set_device(0)
    chunks = []
    if w.prefill_chunk:
        chunks = [w.prefill_chunk] * (w.context // w.prefill_chunk)
        if sum(chunks) < w.context:
            chunks.append(w.context - sum(chunks))
    roof = measure_projections(w, w.prefill_chunk)
    if chunks and w.kv_format == "same":
        roof.append(measure_identification(w, chunks))
    return {"metric": METRIC, "config": {"workload": w.name}, "roofline_all": roof}


def workload_for(args):
    """The named workload, or with --full-attention the same shapes and inputs with every
    KV head a retrieval head (the full-attention baseline of the same kernels)."""
    from mixed_head_kv_amd import inputs as I
    w = I.WORKLOADS[args.workload]
    if args.full_attention:
        w = w.scaled(name=w.name + "_full_attention", n_retrieval=w.n_kv_heads, fixed_retrieval=None)
    return w


def capacity(budget_gb):
    """Largest context (tokens) whose caches fit in `budget_gb` of device memory, per
    layout, from the library's own workspace arithmetic (duo_kv_bytes; no GPU): the int4
    32-layer GQA shape with 4 of 8 KV heads retrieval, the same shape in bf16, and both
    with every head retrieval (full attention)."""
    import numpy as np

    from mixed_head_kv_amd import binding as B
    from mixed_head_kv_amd import inputs as I
    w = I.WORKLOADS["llama3_8b_gqa_32layer_int4_3p3m"]
    budget = int(budget_gb * 1e9)
    res = {}
    for label, fmt, full in (("int4_duo", B.DUO_KV_INT4_G128, False), ("bf16_duo", B.DUO_KV_SAME_AS_IO, False),
                             ("int4_full", B.DUO_KV_INT4_G128, True), ("bf16_full", B.DUO_KV_SAME_AS_IO, True)):
        mask = np.ones((w.n_layers, w.n_kv_heads), np.uint8) if full else w.masks().astype(np.uint8)

        def nbytes(ctx):
            return B.duo_kv_bytes(B.make_config(w.n_layers, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.sink,
                                                w.recent, ctx, B.DUO_DTYPE_BF16, fmt, mask))
        lo, hi = 1, 1 << 40
        while lo < hi:  # largest ctx with nbytes(ctx) <= budget
            mid = (lo + hi + 1) // 2
            if nbytes(mid) <= budget:
                lo = mid
            else:
                hi = mid - 1
        res[label] = {"max_context": lo, "bytes": nbytes(lo)}
    res["int4_duo_vs_bf16_full"] = round(res["int4_duo"]["max_context"] / res["bf16_full"]["max_context"], 2)
    res["bf16_duo_vs_bf16_full"] = round(res["bf16_duo"]["max_context"] / res["bf16_full"]["max_context"], 2)
    return {"capacity_budget_gb": budget_gb, "layers": w.n_layers, "n_kv_heads": w.n_kv_heads,
            "retrieval_kv_heads": int(w.mask(0).sum()), "sink": w.sink, "recent": w.recent, **res}


def capacity_run(args):
    """Measured capacity: the Llama-3-8B-shaped 32-layer stack with an int4 cache (4 of 8
    KV heads retrieval, sink 64 + recent 256) at the largest context, in whole 65536-token
    blocks, whose workspace fits the GPU's free memory less a 4 GB margin.  Every layer's
    history repeats one synthetic 65536-token block (appended block by block; the cost of
    the path does not depend on the values, and the parity tests check a periodic history
    of 2^25 tokens exactly), then `--steps` decode tokens run through all 32 layers.
    Reports the context, the workspace, the fill rate and the decode time per token with
    its HBM rate (algorithmic bytes: every cached vector read once per KV head)."""
    import numpy as np
    import torch

    from mixed_head_kv_amd import binding as B
    from mixed_head_kv_amd import inputs as I

    w = I.WORKLOADS["llama3_8b_gqa_32layer_int4_3p3m"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    P = 1 << 16
    free, _ = torch.cuda.mem_get_info()
    budget = free - (4 << 30)
    masks = w.masks().astype(np.uint8)

    def cfg_for(ctx):
        return B.make_config(w.n_layers, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.sink, w.recent,
                             ctx + args.steps + args.warmup, B.DUO_DTYPE_BF16, B.DUO_KV_INT4_G128, masks)
    blocks = 1
    while B.duo_kv_bytes(cfg_for((blocks + 1) * P)) <= budget:
        blocks += 1
    ctx = blocks * P
    cfg = cfg_for(ctx)
    ws = torch.empty(B.duo_kv_bytes(cfg), dtype=torch.uint8, device=dev)
    st = B._stream(torch.cuda.current_stream())
    h = B.duo_kv_init(cfg, ws, st)
    kb = torch.empty((P, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    vb = torch.empty_like(kb)
    q = torch.empty((w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    n = P * w.n_kv_heads * w.head_dim
    torch.cuda.synchronize()
    t_fill = time.perf_counter()
    for layer in range(w.n_layers):
        B.duo_synth_fill(kb, B.DUO_DTYPE_BF16, w.seed, layer * 4 + 1, 0, n)
        B.duo_synth_fill(vb, B.DUO_DTYPE_BF16, w.seed, layer * 4 + 2, 0, n)
        for _ in range(blocks):
            B.duo_kv_append(h, layer, kb, vb, P, st)
        log(f"capacity: layer {layer} filled ({ctx} tokens)")
    torch.cuda.synchronize()
    fill_s = time.perf_counter() - t_fill
    # decode tokens continue the period: position t holds block row t mod P
    row = kb[0].numel() * kb.element_size()

    def token(t):
        for layer in range(w.n_layers):
            B.duo_synth_fill(q, B.DUO_DTYPE_BF16, w.seed, layer * 4, t * q.numel(), q.numel())
            r = t % P
            B.duo_decode(h, layer, q, kb.data_ptr() + r * row, vb.data_ptr() + r * row, out, st)

    t = ctx
    for _ in range(args.warmup):
        token(t)
        t += 1
    torch.cuda.synchronize()
    B.duo_profile_enable(h, True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        token(t)
        t += 1
    ev1.record()
    torch.cuda.synchronize()
    ms_token = ev0.elapsed_time(ev1) / args.steps
    prof = B.duo_profile_collect(h)
    dec_ms = prof["decode"][0] / args.steps
    bytes_token = sum(decode_bytes(w, tt, layer) for tt in range(ctx + args.warmup, ctx + args.warmup + args.steps)
                      for layer in range(w.n_layers)) / args.steps
    B.duo_kv_free(h)
    a = bytes_token / (dec_ms * 1e-3) / 1e9
    return {"metric": "measured capacity: longest int4 context decoded on one GPU", "context_tokens": ctx,
            "workspace_gb": round(ws.numel() / 1e9, 2), "free_gb_before": round(free / 1e9, 2),
            "layers": w.n_layers, "fill_s": round(fill_s, 2),
            "fill_tok_s_per_layer": round(ctx * w.n_layers / fill_s, 1),
            "decode_ms_per_token": round(ms_token, 3), "decode_kernel_ms_per_token": round(dec_ms, 3),
            "roofline": {"kernel": "decode_attention", "bound": "hbm", "achieved": round(a, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4)},
            "vs_pages_context": round(ctx / 3.3e6, 2), "steps": args.steps, "data": "synthetic, periodic (65536)"}


def run(args):
    import numpy as np
    import torch

    from mixed_head_kv_amd import binding as B
    from mixed_head_kv_amd import inputs as I

    w = workload_for(args)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    io = B.DUO_DTYPE_F32 if w.io_dtype == "f32" else B.DUO_DTYPE_BF16
    tdt = torch.float32 if w.io_dtype == "f32" else torch.bfloat16
    if w.prefill_chunk == 0:
        return run_stack(args, w)
    total = w.context + w.decode_steps
    chunks = [w.prefill_chunk] * (w.context // w.prefill_chunk)
    if sum(chunks) < w.context:
        chunks.append(w.context - sum(chunks))

    def synth(kind, H):
        t = torch.empty((total, H, w.head_dim), dtype=tdt, device=dev)
        B.duo_synth_fill(t, io, w.seed, I.KIND_STREAM[kind], 0, t.numel())
        return t

    Q, K, V = synth("q", w.n_q_heads), synth("k", w.n_kv_heads), synth("v", w.n_kv_heads)
    out_pre = torch.empty((max(chunks), w.n_q_heads, w.head_dim), dtype=tdt, device=dev)
    out_dec = torch.empty((w.n_q_heads, w.head_dim), dtype=tdt, device=dev)
    cfg = B.make_config(w.n_layers, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.sink, w.recent, w.max_context,
                        io, B.DUO_KV_INT4_G128 if w.kv_format == "int4" else B.DUO_KV_SAME_AS_IO,
                        w.masks().astype(np.uint8))
    ws = torch.empty(B.duo_kv_bytes(cfg), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    handles = []
    # Per-call marshalling is kept off the GPU's critical path: the stream handle and the
    # row addresses are computed once (the calls and kernels are the same).
    st_handle = B._stream(torch.cuda.current_stream())
    qrow, kvrow = Q[0].numel() * Q.element_size(), K[0].numel() * K.element_size()
    q0, k0, v0, o_pre, o_dec = Q.data_ptr(), K.data_ptr(), V.data_ptr(), out_pre.data_ptr(), out_dec.data_ptr()

    def step(profile=False):
        h = B.duo_kv_init(cfg, ws, st_handle)
        handles.append(h)
        if profile:
            B.duo_profile_enable(h, True)
        t = 0
        for T in chunks:
            B.duo_prefill(h, 0, q0 + t * qrow, k0 + t * kvrow, v0 + t * kvrow, T, o_pre, st_handle)
            t += T
        for _ in range(w.decode_steps):
            B.duo_decode(h, 0, q0 + t * qrow, k0 + t * kvrow, v0 + t * kvrow, o_dec, st_handle)
            t += 1
        return h

    for _ in range(args.warmup):
        B.duo_kv_free(step())
        handles.pop()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    totals = {c: [0.0, 0] for c in B.KERNEL_CLASSES[:5]}
    # Timed steps: the whole path with nothing added.
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    for h in handles:
        B.duo_kv_free(h)
    handles.clear()
    ms_per_step = ms_total / args.steps
    # The same steps again with every launch's start/stop events stamped at its dispatch
    # (duo_profile.h): each kernel's own duration, for the rooflines.  The events add a
    # few microseconds between launches, so these steps are not the ones timed above.
    ev0.record(stream)
    for _ in range(args.steps):
        step(profile=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_profiled = ev0.elapsed_time(ev1) / args.steps
    for h in handles:
        for c, (ms, n) in B.duo_profile_collect(h).items():
            if c in totals:
                totals[c][0] += ms
                totals[c][1] += n
        B.duo_kv_free(h)
    handles.clear()

    tokens = w.context + w.decode_steps
    # component figures (per step)
    dec_ms = totals["decode"][0] / args.steps
    app_ms = totals["append"][0] / args.steps
    pre_r_ms = totals["prefill_retrieval"][0] / args.steps
    pre_s_ms = totals["prefill_streaming"][0] / args.steps
    stage_ms = totals["prefill_stage"][0] / args.steps

    # algorithmic work per step
    dec_bytes = sum(decode_bytes(w, t) for t in range(w.context, total))
    fl_r = fl_s = fl_s_rest = st_bytes = 0
    tc = min(STAGE_TOKENS, (w.max_context + 63) // 64 * 64)
    t = 0
    for T in chunks:
        fl_r += prefill_flops(w, t, T, True)
        fl_s += prefill_flops(w, t, T, False)
        # streaming-head queries after the first tc of a chunk run in launches of their own
        fl_s_rest += prefill_flops(w, t + tc, T - tc, False) if T > tc else 0
        st_bytes += chunk_tile_bytes(w, t, T)
        t += T

    rooflines = []
    if totals["decode"][1]:
        a = dec_bytes / (dec_ms * 1e-3) / 1e9
        rooflines.append({"kernel": "decode_attention", "bound": "hbm", "achieved": round(a, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
                          "avg_launch_us": round(dec_ms * 1e3 / w.decode_steps, 3), "ms_per_step": round(dec_ms, 4),
                          "traffic": None})
    if totals["prefill_retrieval"][1]:
        # one launch per chunk: retrieval heads and (MFMA path: the first tc; fp32 path: all)
        # streaming-head queries
        fl = fl_r + fl_s - (fl_s_rest if totals["prefill_streaming"][1] else 0)
        a = fl / (pre_r_ms * 1e-3) / 1e12
        peak = MFMA_BF16_PEAK_TFLOPS if w.io_dtype == "bf16" else FP32_VALU_PEAK_TFLOPS
        rooflines.append({"kernel": "prefill_attention", "bound": "mfma", "achieved": round(a, 2),
                          "peak": peak, "unit": "TFLOP/s", "frac": round(a / peak, 4),
                          "avg_launch_us": round(pre_r_ms * 1e3 / len(chunks), 2), "ms_per_step": round(pre_r_ms, 4),
                          "traffic": None})
    if totals["prefill_streaming"][1]:
        a = fl_s_rest / (pre_s_ms * 1e-3) / 1e12
        rooflines.append({"kernel": "prefill_streaming_attention", "bound": "mfma", "achieved": round(a, 2),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4),
                          "avg_launch_us": round(pre_s_ms * 1e3 / totals["prefill_streaming"][1] * args.steps, 2),
                          "ms_per_step": round(pre_s_ms, 4), "traffic": None})
    if totals["prefill_stage"][1]:
        a = st_bytes / (stage_ms * 1e-3) / 1e9
        rooflines.append({"kernel": "prefill_chunk_tiles", "bound": "hbm", "achieved": round(a, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
                          "avg_launch_us": round(stage_ms * 1e3 / totals["prefill_stage"][1] * args.steps, 2),
                          "ms_per_step": round(stage_ms, 4), "traffic": None})
    for r in rooflines:
        r["traffic"] = measured_traffic(r["kernel"], w.name)
    dominant = max(rooflines, key=lambda r: r["ms_per_step"]) if rooflines else None

    # append launches: one per prefill chunk (the streaming caches, last; on the MFMA path
    # the retrieval rows go in with the chunk-tile launch); a decode step appends inside
    # its attention launch on the MFMA path, or in one extra launch otherwise
    n_app = totals["append"][1] / args.steps
    per_app = app_ms / n_app if n_app else 0.0
    pre_app = min(n_app, len(chunks))
    dec_app_launches = max(0.0, n_app - pre_app) / w.decode_steps
    prefill_ms = pre_r_ms + pre_s_ms + stage_ms + per_app * pre_app
    res = {
        "metric": METRIC,
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "global_batch": 1, "seq_len": w.context, "decode_steps": w.decode_steps,
                   "prefill_chunk": w.prefill_chunk, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "retrieval_kv_heads": int(w.mask(0).sum()), "sink": w.sink,
                   "recent": w.recent, "kv_format": w.kv_format, "parallelism": "single_gpu"},
        "components": {
            "value_is": (f"(prefill {w.context} + decode {w.decode_steps} tokens) / step time; the metric's two "
                         "numbers are decode_us_per_step and prefill_tok_s"),
            "decode_us_per_step": round(dec_ms * 1e3 / w.decode_steps, 3),
            "decode_append_plus_attention_us_per_step": None,
            "prefill_tok_s": round(w.context / (prefill_ms * 1e-3), 1) if prefill_ms > 0 else None,
            "kernel_ms_per_step": {c: round(totals[c][0] / args.steps, 4) for c in totals},
            "kernel_launches_per_step": {c: totals[c][1] // args.steps for c in totals},
            "ms_per_step_with_kernel_events": round(ms_profiled, 4),
            "wall_s": round(wall, 3),
        },
        "roofline": dominant,
        "roofline_all": rooflines,
        "cpu_baseline": None,
    }
    # decode step including its append (fused into the decode launch on the MFMA path)
    res["components"]["decode_append_plus_attention_us_per_step"] = round(
        (dec_ms / w.decode_steps + per_app * dec_app_launches) * 1e3, 3)
    if not args.no_projections and w.io_dtype == "bf16" and w.head_dim == 128:
        # the linear layers around the attention, measured beside the step (not in it)
        res["roofline_all"] += measure_projections(w, w.prefill_chunk)
    if not args.no_identification and w.io_dtype == "bf16" and w.head_dim == 128 and w.kv_format == "same":
        res["roofline_all"].append(measure_identification(w, chunks))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, total, args.cpu_seconds)
    return res


def run_stack(args, w):
    """Decode-only stack (32 layers): every layer's caches are filled to `context` tokens
    with duo_kv_append (untimed; int4 caches quantise on the way in), then one step =
    one decode token through all layers (append/evict + attention per layer)."""
    import numpy as np
    import torch

    from mixed_head_kv_amd import binding as B
    from mixed_head_kv_amd import inputs as I

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    steps_total = args.warmup + 2 * args.steps  # warmup, timed, then event-timed steps
    w = w.scaled(decode_steps=steps_total)
    io = B.DUO_DTYPE_BF16
    kvf = B.DUO_KV_INT4_G128 if w.kv_format == "int4" else B.DUO_KV_SAME_AS_IO
    cfg = B.make_config(w.n_layers, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.sink, w.recent, w.max_context,
                        io, kvf, w.masks().astype(np.uint8))
    ws = torch.empty(B.duo_kv_bytes(cfg), dtype=torch.uint8, device=dev)
    h = B.duo_kv_init(cfg, ws)
    fill_chunk = 65536
    kbuf = torch.empty((fill_chunk, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    vbuf = torch.empty_like(kbuf)
    t_fill = time.perf_counter()
    for layer in range(w.n_layers):
        for c0 in range(0, w.context, fill_chunk):
            T = min(fill_chunk, w.context - c0)
            n = T * w.n_kv_heads * w.head_dim
            B.duo_synth_fill(kbuf, io, w.seed, layer * 4 + 1, c0 * w.n_kv_heads * w.head_dim, n)
            B.duo_synth_fill(vbuf, io, w.seed, layer * 4 + 2, c0 * w.n_kv_heads * w.head_dim, n)
            B.duo_kv_append(h, layer, kbuf[:T], vbuf[:T], T)
    torch.cuda.synchronize()
    log(f"stack fill: {w.n_layers} layers x {w.context} tokens in {time.perf_counter() - t_fill:.1f}s")
    del kbuf, vbuf

    def gen(layer, kind, H):
        t = torch.empty((steps_total, H, w.head_dim), dtype=torch.bfloat16, device=dev)
        B.duo_synth_fill(t, io, w.seed, layer * 4 + I.KIND_STREAM[kind], w.context * H * w.head_dim, t.numel())
        return t

    Qs = [gen(l, "q", w.n_q_heads) for l in range(w.n_layers)]
    Ks = [gen(l, "k", w.n_kv_heads) for l in range(w.n_layers)]
    Vs = [gen(l, "v", w.n_kv_heads) for l in range(w.n_layers)]
    out = torch.empty((w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    st_handle = B._stream(torch.cuda.current_stream())
    qrow, kvrow = Qs[0][0].numel() * 2, Ks[0][0].numel() * 2
    addr = [(Qs[l].data_ptr(), Ks[l].data_ptr(), Vs[l].data_ptr()) for l in range(w.n_layers)]
    o_addr = out.data_ptr()

    def step(s):
        for layer in range(w.n_layers):
            qa, ka, va = addr[layer]
            B.duo_decode(h, layer, qa + s * qrow, ka + s * kvrow, va + s * kvrow, o_addr, st_handle)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    evs[0].record(stream)
    for i, s in enumerate(range(args.warmup, args.warmup + args.steps)):  # timed: nothing added
        step(s)
        evs[i + 1].record(stream)  # (a marker between steps: per-step times for the median and p90)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    # the next tokens with each launch's dispatch-stamped events: kernel durations
    B.duo_profile_collect(h)
    B.duo_profile_enable(h, True)
    prof_steps = range(args.warmup + args.steps, steps_total)
    for s in prof_steps:
        step(s)
    torch.cuda.synchronize()
    prof = B.duo_profile_collect(h)
    B.duo_profile_enable(h, False)
    dec_ms = prof["decode"][0] / args.steps
    app_ms = prof["append"][0] / args.steps
    dec_bytes = 0
    for s in prof_steps:
        t = w.context + s
        for layer in range(w.n_layers):
            dec_bytes += decode_bytes(w, t, layer)
    dec_bytes /= args.steps
    a = dec_bytes / (dec_ms * 1e-3) / 1e9
    roof = {"kernel": "decode_attention", "bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(prof["decode"][0] * 1e3 / max(1, prof["decode"][1]), 3),
            "ms_per_step": round(dec_ms, 4), "traffic": measured_traffic("decode_attention", w.name)}
    res = {
        "metric": METRIC,
        "value": round(1.0 / (ms_per_step * 1e-3), 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "global_batch": 1, "seq_len": w.context, "n_layers": w.n_layers,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "retrieval_kv_heads_per_layer": int(w.mask(0).sum()), "sink": w.sink, "recent": w.recent,
                   "kv_format": w.kv_format, "parallelism": "single_gpu"},
        "components": {"value_is": "decoded tokens per second through all 32 layers (1 / step time)",
                       "decode_us_per_step": round(ms_per_step * 1e3, 2),
                       "decode_us_per_step_median": round(float(np.median(step_ms)) * 1e3, 2),
                       "decode_us_per_step_p90": round(float(np.percentile(step_ms, 90)) * 1e3, 2),
                       "decode_attention_us_per_step": round(dec_ms * 1e3, 2),
                       "append_us_per_step": round(app_ms * 1e3, 2),
                       "workspace_gb": round(ws.numel() / 1e9, 2),
                       "wall_s": round(wall, 3)},
        "roofline": roof,
        "roofline_all": [roof],
        "cpu_baseline": None,
    }
    B.duo_kv_free(h)
    del ws
    torch.cuda.empty_cache()
    if not args.no_projections:
        # per layer, beside the step: the decoding token's QKV / output projections
        res["roofline_all"] += measure_projections(w, 0)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_stack(w, w.context + args.warmup)
    return res


STACK_SAMPLE_LAYERS = (0, 15, 31)


def stored_history(w, layer, kind, g, pos):
    """K or V rows of KV head g at positions `pos` as the caches store them: bf16 bit
    patterns, or for int4 caches the codec's dequantised fp32 values.  Input
    preparation for the oracle (not timed): slices in parallel threads."""
    import concurrent.futures as cf
    import numpy as np

    from mixed_head_kv_amd import inputs as I
    from oracle import int4 as OQ

    def part(a):
        raw = I.synth_head(w.seed, layer, kind, pos[a:a + (1 << 16)], g, w.n_kv_heads, w.head_dim, "bf16")
        if w.kv_format == "int4":
            codes, sc, z = OQ.quantize(raw)
            return OQ.dequantize(codes, sc, z)
        return raw

    with cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        return np.concatenate(list(ex.map(part, range(0, len(pos), 1 << 16))))


def cpu_baseline_stack(w, t):
    """The oracle's decode of one token at position t on layers 0, 15 and 31 (every KV
    head's history as the caches hold it, upcast to fp64: every earlier token for
    retrieval heads, the sinks and the recent window for streaming heads; one query head
    per KV head timed and counted for the group), timed on the host cores and scaled to
    32 layers.  History generation (and int4 quantisation) is excluded from the timing;
    the fp64 upcast is included."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from mixed_head_kv_amd import inputs as I
    from oracle import attention as OA

    elapsed = 0.0
    for layer in STACK_SAMPLE_LAYERS:
        mask = w.mask(layer)
        q = I.synth(w.seed, layer, "q", t, 1, w.n_q_heads, w.head_dim, "bf16")[0]
        for g in range(w.n_kv_heads):
            pos = (np.arange(t + 1) if mask[g] else
                   np.unique(np.concatenate([np.arange(min(w.sink, t + 1)), np.arange(max(0, t - w.recent + 1), t + 1)])))
            hist = {kind: stored_history(w, layer, kind, g, pos) for kind in ("k", "v")}
            t0 = time.perf_counter()
            K = np.zeros((t + 1, w.head_dim))
            V = np.zeros((t + 1, w.head_dim))
            up = (lambda a: a.astype(np.float64)) if w.kv_format == "int4" else (lambda a: OA.upcast(a, "bf16"))
            K[pos] = up(hist["k"])
            V[pos] = up(hist["v"])
            t_up = time.perf_counter() - t0
            # the G query heads of a KV head attend over the same keys at the same cost:
            # one is timed and counted G times
            t1 = time.perf_counter()
            h = g * w.group
            OA.head_attention(OA.upcast(q[h], "bf16")[None], [t], K, V, bool(mask[g]), w.sink, w.recent)
            elapsed += t_up + w.group * (time.perf_counter() - t1)
            del K, V, hist
    per_step = elapsed * w.n_layers / len(STACK_SAMPLE_LAYERS)
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    return {"value": round(1.0 / per_step, 6), "unit": "tok/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": (f"one decode token at position {t}: layers {list(STACK_SAMPLE_LAYERS)}, each KV head's history "
                       f"upcast and one of its {w.group} query heads timed (x{w.group}), {elapsed:.1f}s of oracle time, "
                       f"extrapolated x{w.n_layers / len(STACK_SAMPLE_LAYERS):.2f} to {w.n_layers} layers"),
            "extrapolated": True, "host_cpus": os.cpu_count()}


def cpu_baseline(w, total, budget_s):
    """The oracle on the host cores over a bounded, uniformly random sample of the step's
    rows (prefill positions and decode positions alike, all heads), scaled to the whole
    step by the row count.  Input generation is excluded from the timing."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from mixed_head_kv_amd import inputs as I
    from oracle import attention as OA

    t_gen = time.perf_counter()
    K = OA.upcast(I.synth(w.seed, 0, "k", 0, total, w.n_kv_heads, w.head_dim, w.io_dtype), w.io_dtype)
    V = OA.upcast(I.synth(w.seed, 0, "v", 0, total, w.n_kv_heads, w.head_dim, w.io_dtype), w.io_dtype)
    log(f"cpu_baseline: host inputs generated in {time.perf_counter() - t_gen:.1f}s")
    rng = np.random.default_rng(1234)
    order = rng.permutation(total)
    HD = w.n_q_heads * w.head_dim
    done = 0
    elapsed = 0.0
    batch = 32
    while done < total and elapsed < budget_s:
        rows = np.sort(order[done:done + batch])
        counters = rows.astype(np.uint64)[:, None] * np.uint64(HD) + np.arange(HD, dtype=np.uint64)[None, :]
        qb = I.values_f32(w.seed, I.KIND_STREAM["q"], counters)
        if w.io_dtype == "bf16":
            qb = I.f32_to_bf16_bits(qb)
        qb = qb.reshape(len(rows), w.n_q_heads, w.head_dim)
        t0 = time.perf_counter()
        OA.layer_attention(OA.upcast(qb, w.io_dtype), rows, K, V, w.mask(0), w.sink, w.recent)
        elapsed += time.perf_counter() - t0
        done += len(rows)
    est = elapsed * total / done
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    return {"value": round(total / est, 2), "unit": "tok/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"{done} of {total} step rows drawn uniformly (all {w.n_q_heads} heads), "
                      f"{elapsed:.1f}s, scaled by row count",
            "host_cpus": os.cpu_count()}


# --- rocprofv3 output summaries (host only; no GPU) ---------------------------------

PROFILED_KERNELS = {"decode_attention": ["k_decode_mfma(", "k_decode_mfma_int4(", "k_decode_mfma<", "k_decode_valu"],
                    "prefill_attention": ["k_prefill_mfma<", "k_prefill_valu"],
                    "prefill_chunk_tiles": ["k_chunk_tiles<false>"]}


def streaming_only_grid(workload):
    """Grid (threads) of the prefill launches that hold only streaming-head queries (the
    queries of a chunk after its first 4096), or None when the workload has none; the
    k_prefill_mfma launches of any other grid are the chunk's main launch (retrieval
    heads plus the first 4096 streaming-head queries)."""
    import math
    from mixed_head_kv_amd import inputs as I
    w = I.WORKLOADS[workload]
    if not w.prefill_chunk or w.prefill_chunk <= STAGE_TOKENS:
        return None
    n_str = int((~w.mask(0)).sum()) * w.group
    pack = 4 if w.group % 4 == 0 else (2 if w.group % 2 == 0 else 1)  # query heads per workgroup
    rows = 128 // pack                       # queries per 4-wavefront workgroup (these launches' shape)
    return n_str // pack * math.ceil(min(STAGE_TOKENS, w.prefill_chunk - STAGE_TOKENS) / rows) * 256


def launch_kind(name, grid, workload):
    """The roofline entry a profiled dispatch belongs to (None: not a path kernel)."""
    for k, pats in PROFILED_KERNELS.items():
        if any(p in name for p in pats):
            if k == "prefill_attention" and grid == streaming_only_grid(workload):
                return "prefill_streaming_attention"
            return k
    return None


def extra_kernels(workload):
    """Kernels of `bench.py --extras-only` (the projections and the identification
    pre-filling): label -> (name pattern, grid size in threads or None).  The projections'
    two layers run the same kernel and are told apart by their grids."""
    import math
    from mixed_head_kv_amd import inputs as I
    w = I.WORKLOADS[workload]
    hidden, nqkv = w.n_q_heads * w.head_dim, (w.n_q_heads + 2 * w.n_kv_heads) * w.head_dim
    out = {"qkv_rope_decode": ("k_w8_gemv<1>", nqkv // 16 * 512), "out_proj_decode": ("k_w8_gemv<1>", hidden // 16 * 512)}
    if w.prefill_chunk:
        tm = math.ceil(w.prefill_chunk / 256)
        out["qkv_rope_prefill"] = ("k_w8_gemm<", tm * nqkv // 256 * 512)
        out["out_proj_prefill"] = ("k_w8_gemm<", tm * hidden // 256 * 512)
        out["prefill_dual_attention"] = ("k_prefill_mfma<", None)
    return out


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def summarize_stats(d, extras_workload=None, path_workload=None):
    """Text table of a `rocprofv3 --kernel-trace --stats` run: calls, mean and total time
    per kernel, as the profiler reports them.  With path_workload, also the path's
    launches by roofline entry (the prefill kernel's two launch kinds apart); with
    extras_workload, the extras' launches split by grid (both from the kernel trace)."""
    import csv
    rows = []
    for f in _csvs(d, "kernel_stats.csv"):
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"{'kernel':<58} {'calls':>7} {'avg_us':>10} {'total_ms':>10} {'pct':>6}"]
    for r in rows:
        lines.append(f"{_short(r['Name'])[:58]:<58} {int(r['Calls']):>7} {float(r['AverageNs']) / 1e3:>10.3f} "
                     f"{float(r['TotalDurationNs']) / 1e6:>10.3f} {float(r['Percentage']):>6.2f}")
    trace = []
    for f in _csvs(d, "kernel_trace.csv"):
        trace += list(csv.DictReader(open(f)))
    if path_workload and trace:
        by = {}
        for r in trace:
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            k = launch_kind(r["Kernel_Name"], grid, path_workload)
            if k:
                by.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines.append("")
        lines.append(f"{'launches by roofline entry':<40} {'calls':>7} {'avg_us':>10}")
        for k, ds in sorted(by.items()):
            lines.append(f"{k:<40} {len(ds):>7} {sum(ds) / len(ds):>10.3f}")
    if extras_workload:
        lines.append("")
        lines.append(f"{'launches by grid':<40} {'grid':>9} {'calls':>7} {'avg_us':>10}")
        for label, (pat, grid) in extra_kernels(extras_workload).items():
            ds = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                  if pat in r["Kernel_Name"] and (grid is None or int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"])
                                                   * int(r["Grid_Size_Z"]) == grid)]
            if ds:
                lines.append(f"{label:<40} {str(grid or 'any'):>9} {len(ds):>7} {sum(ds) / len(ds):>10.3f}")
    return "\n".join(lines)


def summarize_traffic(fetch_dir, write_dir, workload, extras=False):
    """Per-launch HBM bytes of the path's kernels from two `rocprofv3 --pmc` runs of
    `bench.py --copy-probe` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled
    by what the same counter reads for the probe's 1 GiB device copy.  Updates the
    entries of profiles/traffic.json for this workload and returns a text summary."""
    import collections
    import csv

    def load(d, counter):
        per = collections.defaultdict(float)
        for f in _csvs(d, "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    per[(r["Dispatch_Id"], r["Kernel_Name"], int(r["Grid_Size"]))] += float(r["Counter_Value"])
        return per

    kmap = ({k: (pat, grid) for k, (pat, grid) in extra_kernels(workload).items()} if extras else
            {k: (None, None) for k in list(PROFILED_KERNELS) + ["prefill_streaming_attention"]})

    def match(name, grid, pat, want):
        if pat is None:  # the path's kernels, by launch kind
            return launch_kind(name, grid, workload) == k_now[0]
        pats = pat if isinstance(pat, list) else [pat]
        return any(p in name for p in pats) and (want is None or grid == want)

    k_now = [None]

    out, lines = {}, []
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = load(d, counter)
        copies = [v for (_, n, _g), v in vals.items() if "copy" in n.lower() or "elementwise" in n.lower()]
        ref = max(copies)
        factor = (1 << 30) / 1024.0 / ref
        lines.append(f"{counter}: the 1 GiB copy reads {ref:.0f} KiB -> scale factor {factor:.4f}")
        out[counter] = {"factor": factor}
        for k, (pat, grid) in kmap.items():
            k_now[0] = k
            xs = [v for (_, n, g), v in vals.items() if match(n, g, pat, grid)]
            if xs:
                out[counter][k] = (len(xs), sum(xs) / len(xs))
    try:
        entries = [e for e in json.load(open(TRAFFIC_FILE)) if e["kernel"] in KERNEL_SOURCES]
    except (OSError, ValueError):
        entries = []
    for k in kmap:
        if k not in out["FETCH_SIZE"] or k not in out["WRITE_SIZE"]:
            continue
        n, fk = out["FETCH_SIZE"][k]
        fb = fk * 1024 * out["FETCH_SIZE"]["factor"]
        wb = out["WRITE_SIZE"][k][1] * 1024 * out["WRITE_SIZE"]["factor"]
        entries = [e for e in entries if not (e["kernel"] == k and e["workload"] == workload)]
        entries.append({"kernel": k, "workload": workload, "source": source_digest(k),
                        "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                        "bytes_per_launch": round(fb + wb), "launches": n,
                        "fetch_factor": round(out["FETCH_SIZE"]["factor"], 4),
                        "write_factor": round(out["WRITE_SIZE"]["factor"], 4)})
        lines.append(f"{k}: {n} launches, mean per launch: fetch {fb / 1e6:.3f} MB + write {wb / 1e6:.3f} MB "
                     f"= {(fb + wb) / 1e6:.3f} MB (scaled)")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(sorted(entries, key=lambda e: (e["workload"], e["kernel"])), f, indent=1)
    return "\n".join(lines)


# Counters of the summary below, one rocprofv3 --pmc pass each (within the per-pass
# hardware limits of 8 SQ counters).
COUNTER_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES",
    "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SALU SQ_INSTS_VMEM SQ_WAIT_INST_LDS",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_MISC",
]


def summarize_counters(dirs, workload, n_cu=256):
    """MFMA utilisation and instruction mix of the prefill and decode launches from
    `rocprofv3 --pmc` passes (COUNTER_PASSES, one directory each), per launch kind.
    Normalisation: SQ_BUSY_CU_CYCLES sums busy cycles over the CUs, so per-CU cycles =
    it / n_cu and the shader clock = per-CU cycles / kernel duration;
    SQ_VALU_MFMA_BUSY_CYCLES sums matrix-core busy cycles over the SIMDs (32 per
    32x32x16 bf16 MFMA), so the MFMA busy fraction = it / (4 * SQ_BUSY_CU_CYCLES);
    SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_* count in the same (quad-cycle) unit, so
    their ratios are fractions of wave time."""
    import collections
    import csv
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    n = collections.defaultdict(lambda: collections.defaultdict(int))
    dur = collections.defaultdict(list)
    for d in dirs:
        for f in _csvs(d, "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                k = launch_kind(r["Kernel_Name"], int(r["Grid_Size"]), workload)
                if k is None:
                    continue
                c = r["Counter_Name"]
                agg[k][c] += float(r["Counter_Value"])
                n[k][c] += 1
                if c in ("SQ_BUSY_CU_CYCLES", "SQ_INSTS_MFMA"):
                    dur[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = []
    for k in sorted(agg):
        v = {c: agg[k][c] / n[k][c] for c in agg[k]}  # per dispatch
        t_ns = sum(dur[k]) / len(dur[k]) if dur[k] else float("nan")
        lines.append(f"{k}: {max(n[k].values())} dispatches counted, mean duration {t_ns / 1e3:.2f} us (under counters)")
        cu = v.get("SQ_BUSY_CU_CYCLES")
        if cu:
            lines.append(f"  shader clock        {cu / n_cu / t_ns:.3f} GHz (SQ_BUSY_CU_CYCLES / {n_cu} CUs / duration)")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in v:
                lines.append(f"  MFMA busy           {v['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * cu):.3f} of SIMD cycles "
                             f"(SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES))")
        mf = v.get("SQ_INSTS_MFMA")
        if mf:
            valu = v.get("SQ_INSTS_VALU", 0) - mf
            lines.append(f"  per MFMA            {valu / mf:.2f} other VALU (of which "
                         f"{v.get('SQ_INSTS_VALU_TRANS_F32', 0) / mf:.2f} transcendental), "
                         f"{v.get('SQ_INSTS_LDS', 0) / mf:.2f} LDS, {v.get('SQ_INSTS_SALU', 0) / mf:.2f} SALU, "
                         f"{v.get('SQ_INSTS_VMEM', 0) / mf:.3f} VMEM instructions")
        wc = v.get("SQ_WAVE_CYCLES")
        if wc:
            parts = [f"{name} {v[c] / wc:.2f}" for name, c in (("issuing any", "SQ_ACTIVE_INST_ANY"),
                                                               ("issuing VALU+MFMA", "SQ_ACTIVE_INST_VALU"),
                                                               ("waiting on dependencies", "SQ_WAIT_INST_ANY"),
                                                               ("waiting at s_waitcnt", "SQ_WAIT_ANY"),
                                                               ("waiting on LDS", "SQ_WAIT_INST_LDS")) if c in v]
            lines.append("  of wave time        " + ", ".join(parts))
    return "\n".join(lines)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        sp = argparse.ArgumentParser()
        sp.add_argument("dirs", nargs="+")
        sp.add_argument("--workload", default=DEFAULT_WORKLOAD)
        a = sp.parse_args(sys.argv[2:])
        print(summarize_counters(a.dirs, a.workload))
        return
    if len(sys.argv) > 1 and sys.argv[1] in ("--summarize-stats", "--summarize-traffic"):
        sp = argparse.ArgumentParser()
        sp.add_argument("dirs", nargs="+")
        sp.add_argument("--workload", default=DEFAULT_WORKLOAD)
        sp.add_argument("--extras", action="store_true", help="the run was `bench.py --extras-only`")
        a = sp.parse_args(sys.argv[2:])
        if sys.argv[1] == "--summarize-stats":
            print(summarize_stats(a.dirs[0], a.workload if a.extras else None, None if a.extras else a.workload))
        else:
            print(summarize_traffic(a.dirs[0], a.dirs[1], a.workload, a.extras))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-identification", action="store_true",
                    help="skip the timing of the head-identification pre-filling beside the step")
    ap.add_argument("--no-projections", action="store_true",
                    help="skip the timing of the 8-bit-weight QKV / output projections beside the step")
    ap.add_argument("--capacity-run", action="store_true",
                    help="decode the int4 32-layer stack at the largest context the GPU's memory holds")
    ap.add_argument("--extras-only", action="store_true",
                    help="run only the projections and the identification pre-filling (for profiling them alone)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--full-attention", action="store_true",
                    help="every KV head a retrieval head: the full-attention baseline on the same kernels")
    ap.add_argument("--capacity", type=float, metavar="GB", default=None,
                    help="print the largest contexts whose caches fit in GB of device memory (no GPU) and exit")
    args = ap.parse_args()
    if args.capacity is not None:
        print(json.dumps(capacity(args.capacity)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.capacity_run:
        res = capacity_run(args)
    elif args.extras_only:
        res = run_extras(args)
    else:
        res = run(args)
    if args.copy_probe:
        copy_probe()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
