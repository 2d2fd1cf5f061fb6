"""ctypes binding of libduo_attn.so (include/duo_attn.h, include/duo_synth.h).

Argument marshalling only: the functions below carry the C names and pass device
pointers, sizes and the current HIP stream through; every step of the attention path
runs in the library's HIP kernels.  PyTorch supplies device memory and streams.  If the
built library is missing this module raises on first use; there is no fallback.

``DuoKV`` is a small convenience owner of one handle and its workspace tensor.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libduo_attn.so")

DUO_OK = 0
DUO_E_INVALID = -1
DUO_E_UNSUPPORTED = -2
DUO_E_CAPACITY = -3
DUO_E_STATE = -4
DUO_E_HIP = -5
DUO_DTYPE_F32 = 0
DUO_DTYPE_BF16 = 1
DUO_KV_SAME_AS_IO = 0
DUO_KV_INT4_G128 = 1
DUO_SYNTH_INT8 = 2
DUO_STATIC_SCRATCH_BYTES = 16 << 20
DUO_GUARD_BYTES = 256
DUO_GUARD_WORD = 0xD0A5C3E1

EXPORTS = ["duo_kv_bytes", "duo_kv_init", "duo_prefill", "duo_kv_append", "duo_decode", "duo_decode_static",
           "duo_kv_length",
           "duo_prefill_seq", "duo_kv_append_seq", "duo_kv_length_seq", "duo_prefill_dual", "duo_kv_free", "duo_last_error", "duo_kv_read", "duo_kv_read_int4", "duo_synth_fill",
           "duo_profile_enable", "duo_profile_collect", "duo_linear_w8", "duo_qkv_rope_w8",
           "duo_profile_thread_enable", "duo_profile_thread_collect", "duo_kv_guard_bands", "duo_kv_attach"]
KERNEL_CLASSES = ["append", "prefill_retrieval", "prefill_streaming", "decode", "prefill_stage", "qkv_rope",
                  "linear"]


class DuoError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class duo_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("sink", ctypes.c_int32),
        ("recent", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("kv_format", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("max_context", ctypes.c_int64), ("scale", ctypes.c_float),
        ("retrieval_mask", ctypes.POINTER(ctypes.c_uint8)),
    ]


_lib = None


def lib():
    """Load libduo_attn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixed_head_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    cfgp = ctypes.POINTER(duo_config)
    sig = {
        "duo_kv_bytes": (ctypes.c_int, [cfgp, ctypes.POINTER(u64)]),
        "duo_kv_init": (ctypes.c_int, [cfgp, vp, u64, vp, ctypes.POINTER(vp)]),
        "duo_kv_attach": (ctypes.c_int, [cfgp, vp, u64, ctypes.POINTER(i64), ctypes.POINTER(vp)]),
        "duo_prefill": (ctypes.c_int, [vp, i32, vp, vp, vp, i32, vp, vp]),
        "duo_kv_append": (ctypes.c_int, [vp, i32, vp, vp, i32, vp]),
        "duo_decode": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp]),
        "duo_decode_static": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp]),
        "duo_kv_length": (ctypes.c_int, [vp, i32, ctypes.POINTER(i64)]),
        "duo_prefill_seq": (ctypes.c_int, [vp, i32, i32, vp, vp, vp, i32, vp, vp]),
        "duo_prefill_dual": (ctypes.c_int, [vp, i32, vp, vp, vp, i32, vp, vp, vp]),
        "duo_kv_append_seq": (ctypes.c_int, [vp, i32, i32, vp, vp, i32, vp]),
        "duo_kv_length_seq": (ctypes.c_int, [vp, i32, i32, ctypes.POINTER(i64)]),
        "duo_kv_free": (None, [vp]),
        "duo_kv_guard_bands": (ctypes.c_int, [vp, ctypes.POINTER(u64), i32, ctypes.POINTER(i32)]),
        "duo_last_error": (ctypes.c_char_p, []),
        "duo_kv_read": (ctypes.c_int, [vp, i32, i32, i32, i32, i64, i32, vp, vp]),
        "duo_kv_read_int4": (ctypes.c_int, [vp, i32, i32, i32, i32, i64, i32, vp, vp, vp]),
        "duo_synth_fill": (ctypes.c_int, [vp, i32, u64, ctypes.c_uint32, u64, u64, vp]),
        "duo_profile_enable": (ctypes.c_int, [vp, i32]),
        "duo_profile_collect": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]),
        "duo_linear_w8": (ctypes.c_int, [vp, i64, i32, vp, vp, i32, vp, vp]),
        "duo_profile_thread_enable": (ctypes.c_int, [i32]),
        "duo_profile_thread_collect": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]),
        "duo_qkv_rope_w8": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc: int):
    if rc != DUO_OK:
        raise DuoError(rc, lib().duo_last_error().decode())


def make_config(n_layers, batch, n_q_heads, n_kv_heads, head_dim, sink, recent, max_context, io_dtype,
                kv_format, retrieval_mask, scale=0.0):
    """Build a duo_config; `retrieval_mask` is any [n_layers, n_kv_heads] 0/1 array.
    The returned object keeps the mask buffer alive."""
    import numpy as np
    m = np.ascontiguousarray(np.asarray(retrieval_mask, dtype=np.uint8).reshape(-1))
    cfg = duo_config(n_layers, batch, n_q_heads, n_kv_heads, head_dim, sink, recent,
                     io_dtype, kv_format, 0, max_context, scale,
                     m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    cfg._mask_keepalive = m
    return cfg


def _stream(stream=None):
    """A torch stream, a raw hipStream_t (int or c_void_p), or None for torch's current."""
    if isinstance(stream, ctypes.c_void_p):
        return stream
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    """A tensor's device address, or a raw address given as an int; None stays NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


# ---- the C entry points, same names ------------------------------------------------

def duo_kv_bytes(cfg) -> int:
    out = ctypes.c_uint64()
    _check(lib().duo_kv_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def duo_kv_init(cfg, workspace, stream=None):
    h = ctypes.c_void_p()
    _check(lib().duo_kv_init(ctypes.byref(cfg), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream), ctypes.byref(h)))
    return h


def duo_kv_attach(cfg, workspace, lengths):
    """A handle over a workspace holding an earlier handle's state; lengths: the tokens
    held per (layer, sequence), layer-major."""
    h = ctypes.c_void_p()
    arr = (ctypes.c_int64 * max(len(lengths), 1))(*[int(x) for x in lengths])
    _check(lib().duo_kv_attach(ctypes.byref(cfg), _ptr(workspace), workspace.numel() * workspace.element_size(), arr,
                               ctypes.byref(h)))
    return h


def duo_prefill(h, layer, q, k, v, n_tokens, out, stream=None):
    _check(lib().duo_prefill(h, layer, _ptr(q), _ptr(k), _ptr(v), n_tokens, _ptr(out), _stream(stream)))


def duo_kv_append(h, layer, k, v, n_tokens, stream=None):
    _check(lib().duo_kv_append(h, layer, _ptr(k), _ptr(v), n_tokens, _stream(stream)))


def duo_decode(h, layer, q, k_new, v_new, out, stream=None):
    _check(lib().duo_decode(h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _stream(stream)))


def duo_decode_static(h, layer, q, k_new, v_new, out, stream=None):
    _check(lib().duo_decode_static(h, layer, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _stream(stream)))


def duo_kv_length(h, layer) -> int:
    out = ctypes.c_int64()
    _check(lib().duo_kv_length(h, layer, ctypes.byref(out)))
    return out.value


def duo_prefill_seq(h, layer, seq, q, k, v, n_tokens, out, stream=None):
    _check(lib().duo_prefill_seq(h, layer, seq, _ptr(q), _ptr(k), _ptr(v), n_tokens, _ptr(out), _stream(stream)))


def duo_prefill_dual(h, layer, q, k, v, n_tokens, out_full, out_streaming, stream=None):
    _check(lib().duo_prefill_dual(h, layer, _ptr(q), _ptr(k), _ptr(v), n_tokens, _ptr(out_full), _ptr(out_streaming),
                                  _stream(stream)))


def duo_kv_append_seq(h, layer, seq, k, v, n_tokens, stream=None):
    _check(lib().duo_kv_append_seq(h, layer, seq, _ptr(k), _ptr(v), n_tokens, _stream(stream)))


def duo_kv_length_seq(h, layer, seq) -> int:
    out = ctypes.c_int64()
    _check(lib().duo_kv_length_seq(h, layer, seq, ctypes.byref(out)))
    return out.value


def duo_linear_w8(x, M, K, w, scale, N, y, stream=None):
    _check(lib().duo_linear_w8(_ptr(x), M, K, _ptr(w), _ptr(scale), N, _ptr(y), _stream(stream)))


def duo_qkv_rope_w8(x, M, hidden, positions, w, scale, n_q_heads, n_kv_heads, head_dim, rope_base, q, k, v,
                    stream=None):
    _check(lib().duo_qkv_rope_w8(_ptr(x), M, hidden, _ptr(positions), _ptr(w), _ptr(scale), n_q_heads, n_kv_heads,
                                 head_dim, float(rope_base), _ptr(q), _ptr(k), _ptr(v), _stream(stream)))


def linear_w8(x, w, scale, out=None):
    """y [M, N] = x [M, K] (bf16) times the int8 weight w [N, K] scaled per row by scale [N]."""
    import torch
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    duo_linear_w8(x, M, K, w, scale, N, out)
    return out


def qkv_rope_w8(x, positions, w, scale, n_q_heads, n_kv_heads, head_dim, rope_base):
    """(q [M, Hq, D], k [M, Hkv, D], v [M, Hkv, D]) of tokens x [M, hidden] at positions [M]."""
    import torch
    M, hidden = x.shape
    q = torch.empty((M, n_q_heads, head_dim), dtype=torch.bfloat16, device=x.device)
    k = torch.empty((M, n_kv_heads, head_dim), dtype=torch.bfloat16, device=x.device)
    v = torch.empty_like(k)
    duo_qkv_rope_w8(x, M, hidden, positions, w, scale, n_q_heads, n_kv_heads, head_dim, rope_base, q, k, v)
    return q, k, v


def duo_kv_free(h):
    lib().duo_kv_free(h)


def duo_kv_guard_bands(h) -> list:
    """Byte offsets of the workspace's guard bands (DUO_GUARD_BYTES each)."""
    n = ctypes.c_int32()
    _check(lib().duo_kv_guard_bands(h, None, 0, ctypes.byref(n)))
    offs = (ctypes.c_uint64 * max(n.value, 1))()
    _check(lib().duo_kv_guard_bands(h, offs, n.value, ctypes.byref(n)))
    return list(offs[:n.value])


def duo_last_error() -> str:
    return lib().duo_last_error().decode()


def duo_kv_read(h, layer, b, kv_head, which, pos0, n, out, stream=None):
    _check(lib().duo_kv_read(h, layer, b, kv_head, which, pos0, n, _ptr(out), _stream(stream)))


def duo_kv_read_int4(h, layer, b, kv_head, which, pos0, n, codes, meta, stream=None):
    _check(lib().duo_kv_read_int4(h, layer, b, kv_head, which, pos0, n, _ptr(codes), _ptr(meta), _stream(stream)))


def duo_synth_fill(out, dtype, seed, stream_id, counter0, n, stream=None):
    _check(lib().duo_synth_fill(_ptr(out), dtype, seed, stream_id, counter0, n, _stream(stream)))


def duo_profile_enable(h, on: bool):
    _check(lib().duo_profile_enable(h, 1 if on else 0))


def duo_profile_collect(h) -> dict:
    """{class name: (total_ms, launches)} since the last collect."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().duo_profile_collect(h, ms, cnt))
    return {KERNEL_CLASSES[i]: (ms[i], cnt[i]) for i in range(n)}


def duo_profile_thread_enable(on: bool):
    _check(lib().duo_profile_thread_enable(1 if on else 0))


def duo_profile_thread_collect() -> dict:
    """{class name: (total_ms, launches)} of this thread's handle-free calls."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().duo_profile_thread_collect(ms, cnt))
    return {KERNEL_CLASSES[i]: (ms[i], cnt[i]) for i in range(n)}


# ---- convenience owner -------------------------------------------------------------

class DuoKV:
    """One handle plus its workspace (a torch uint8 tensor on the current device)."""

    def __init__(self, n_layers, n_q_heads, n_kv_heads, head_dim, sink, recent, max_context, retrieval_mask,
                 io_dtype="bf16", kv_format="same", batch=1, scale=0.0, device="cuda"):
        import torch
        self.io = DUO_DTYPE_F32 if io_dtype == "f32" else DUO_DTYPE_BF16
        self.torch_dtype = torch.float32 if io_dtype == "f32" else torch.bfloat16
        self.cfg = make_config(n_layers, batch, n_q_heads, n_kv_heads, head_dim, sink, recent, max_context,
                               self.io, DUO_KV_INT4_G128 if kv_format == "int4" else DUO_KV_SAME_AS_IO,
                               retrieval_mask, scale)
        self.nbytes = duo_kv_bytes(self.cfg)
        self.workspace = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.h = duo_kv_init(self.cfg, self.workspace)
        self.B, self.Hq, self.Hkv, self.D = batch, n_q_heads, n_kv_heads, head_dim

    @classmethod
    def for_workload(cls, w, **kw):
        return cls(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, w.sink, w.recent, w.max_context,
                   w.masks().astype("uint8"), io_dtype=w.io_dtype, kv_format=w.kv_format, **kw)

    def close(self):
        if self.h:
            duo_kv_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def length(self, layer):
        return duo_kv_length(self.h, layer)

    def prefill(self, layer, q, k, v, out=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        duo_prefill(self.h, layer, q, k, v, q.shape[-3], out)
        return out

    def append(self, layer, k, v):
        duo_kv_append(self.h, layer, k, v, k.shape[-3])

    def length_seq(self, layer, seq):
        return duo_kv_length_seq(self.h, layer, seq)

    def lengths(self):
        """Tokens held per (layer, sequence), layer-major (what duo_kv_attach takes)."""
        return [duo_kv_length_seq(self.h, layer, b) for layer in range(self.cfg.n_layers) for b in range(self.B)]

    @classmethod
    def attach(cls, like, workspace, lengths):
        """A handle with `like`'s config over `workspace`, a saved copy of a workspace of
        that config taken between calls, holding `lengths` tokens (duo_kv_attach)."""
        self = cls.__new__(cls)
        self.io, self.torch_dtype, self.cfg, self.nbytes = like.io, like.torch_dtype, like.cfg, like.nbytes
        self.B, self.Hq, self.Hkv, self.D = like.B, like.Hq, like.Hkv, like.D
        self.workspace = workspace
        self.h = None
        self.h = duo_kv_attach(self.cfg, workspace, lengths)
        return self

    def prefill_seq(self, layer, seq, q, k, v, out=None):
        """One sequence's chunk: q, k, v of shape [1, T, heads, D] (or [T, heads, D])."""
        import torch
        if out is None:
            out = torch.empty_like(q)
        duo_prefill_seq(self.h, layer, seq, q, k, v, q.shape[-3], out)
        return out

    def prefill_dual(self, layer, q, k, v):
        """(full output, streaming output) of every head for a chunk (head identification)."""
        import torch
        full, stream = torch.empty_like(q), torch.empty_like(q)
        duo_prefill_dual(self.h, layer, q, k, v, q.shape[-3], full, stream)
        return full, stream

    def append_seq(self, layer, seq, k, v):
        duo_kv_append_seq(self.h, layer, seq, k, v, k.shape[-3])

    def decode(self, layer, q, k_new=None, v_new=None, out=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        duo_decode(self.h, layer, q, k_new, v_new, out)
        return out

    def read(self, layer, kv_head, which, pos0, n, b=0):
        import torch
        out = torch.empty((n, self.D), dtype=torch.float32, device=self.workspace.device)
        duo_kv_read(self.h, layer, b, kv_head, which, pos0, n, out)
        return out

    def read_int4(self, layer, kv_head, which, pos0, n, b=0):
        import torch
        codes = torch.empty((n, 64), dtype=torch.uint8, device=self.workspace.device)
        meta = torch.empty((n, 2), dtype=torch.int16, device=self.workspace.device)
        duo_kv_read_int4(self.h, layer, b, kv_head, which, pos0, n, codes, meta)
        return codes, meta
