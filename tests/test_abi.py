"""The C-ABI library on the CPU: it loads, exports every function the public headers
declare, and rejects bad arguments before touching the GPU (no compute calls here)."""

import ctypes
import glob
import os
import re

import numpy as np
import pytest

from mixed_head_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libduo_attn.so not built (python -m mixed_head_kv_amd.build)")
    return B.lib()


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s+\**(duo_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_headers_declare_the_boundary():
    names = declared_functions()
    for n in ["duo_kv_bytes", "duo_kv_init", "duo_prefill", "duo_kv_append", "duo_decode", "duo_kv_length",
              "duo_prefill_seq", "duo_kv_append_seq", "duo_kv_length_seq", "duo_prefill_dual", "duo_kv_free",
              "duo_last_error",
              "duo_synth_fill", "duo_linear_w8", "duo_qkv_rope_w8"]:
        assert n in names
    assert set(names) == set(B.EXPORTS)


def test_every_declared_symbol_is_exported():
    L = _lib_or_skip()
    for n in declared_functions():
        assert hasattr(L, n), n


def _cfg(**kw):
    base = dict(n_layers=2, batch=1, n_q_heads=8, n_kv_heads=4, head_dim=128, sink=4, recent=16,
                max_context=1000, io_dtype=B.DUO_DTYPE_BF16, kv_format=B.DUO_KV_SAME_AS_IO,
                retrieval_mask=np.array([[1, 0, 1, 0], [0, 0, 1, 1]]))
    base.update(kw)
    return B.make_config(**base)


def _bytes(cfg):
    out = ctypes.c_uint64()
    rc = B.lib().duo_kv_bytes(ctypes.byref(cfg), ctypes.byref(out))
    return rc, out.value


def expected_bytes(n_layers, batch, hq, hkv, D, S, R, max_ctx, esize, int4, mask):
    al = lambda x, a: (x + a - 1) // a * a
    reg = lambda off, size: al(off + size, 256) + B.DUO_GUARD_BYTES  # a region, then its guard band
    cap, nslot = al(max_ctx, 64), al(S + R, 64)
    vec = D // 2 if int4 else D * esize
    off = 0
    for l in range(n_layers):
        nr = int(mask[l].sum())
        ns = hkv - nr
        for rows in (batch * nr * cap, batch * nr * cap, batch * ns * nslot, batch * ns * nslot):
            off = reg(off, rows * vec)
        if int4:
            for rows in (batch * nr * cap, batch * nr * cap, batch * ns * nslot, batch * ns * nslot):
                off = reg(off, rows * 4)
    off = reg(off, batch * hq * 2048 * (D + 2) * 4)
    off = reg(off, batch * hkv * 4)
    off = reg(off, 65536 * 4)
    if esize == 2 and D == 128 and not int4:  # streaming-head prefill staging, K then V
        stage_rows = al(S, 64) + al(R - 1, 64) + min(cap, 4096)
        n_str = max(hkv - int(mask[l].sum()) for l in range(n_layers))
        for _ in range(2):
            off = reg(off, batch * n_str * stage_rows * D * 2)
    return off


@pytest.mark.parametrize("kw", [
    dict(),
    dict(io_dtype=B.DUO_DTYPE_F32, head_dim=64, max_context=513),
    dict(kv_format=B.DUO_KV_INT4_G128, max_context=3_300_000),
    dict(batch=3, sink=0, recent=1),
    dict(sink=1 << 28, recent=1 << 28, max_context=64),   # the largest window
])
def test_kv_bytes_matches_layout_arithmetic(kw):
    _lib_or_skip()
    cfg = _cfg(**kw)
    rc, nbytes = _bytes(cfg)
    assert rc == B.DUO_OK
    mask = np.array([[1, 0, 1, 0], [0, 0, 1, 1]])
    assert nbytes == expected_bytes(cfg.n_layers, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.sink,
                                    cfg.recent, cfg.max_context, 4 if cfg.io_dtype == 0 else 2,
                                    cfg.kv_format == 1, mask)


@pytest.mark.parametrize("kw,code", [
    (dict(n_layers=0), B.DUO_E_INVALID),
    (dict(batch=0), B.DUO_E_INVALID),
    (dict(n_q_heads=6), B.DUO_E_INVALID),
    (dict(n_q_heads=4 * 17), B.DUO_E_UNSUPPORTED),
    (dict(head_dim=96), B.DUO_E_UNSUPPORTED),
    (dict(sink=-1), B.DUO_E_INVALID),
    (dict(recent=0), B.DUO_E_INVALID),
    (dict(sink=(1 << 28) + 1), B.DUO_E_UNSUPPORTED),   # windows are bounded so slot sums fit int32
    (dict(recent=(1 << 28) + 1), B.DUO_E_UNSUPPORTED),
    (dict(max_context=0), B.DUO_E_INVALID),
    (dict(io_dtype=7), B.DUO_E_INVALID),
    (dict(kv_format=3), B.DUO_E_INVALID),
    (dict(kv_format=B.DUO_KV_INT4_G128, io_dtype=B.DUO_DTYPE_F32), B.DUO_E_UNSUPPORTED),
    (dict(kv_format=B.DUO_KV_INT4_G128, head_dim=64), B.DUO_E_UNSUPPORTED),
    (dict(retrieval_mask=np.array([[2, 0, 0, 0], [0, 0, 0, 0]])), B.DUO_E_INVALID),
    (dict(n_kv_heads=65, n_q_heads=65, retrieval_mask=np.zeros((2, 65))), B.DUO_E_INVALID),
])
def test_bad_configs_are_rejected(kw, code):
    _lib_or_skip()
    rc, _ = _bytes(_cfg(**kw))
    assert rc == code
    assert B.duo_last_error()
    h = ctypes.c_void_p()
    rc2 = B.lib().duo_kv_init(ctypes.byref(_cfg(**kw)), ctypes.c_void_p(256), 1 << 40, None, ctypes.byref(h))
    assert rc2 == code and not h.value


def test_init_rejects_small_or_misaligned_workspace():
    L = _lib_or_skip()
    cfg = _cfg()
    _, need = _bytes(cfg)
    h = ctypes.c_void_p()
    assert L.duo_kv_init(ctypes.byref(cfg), ctypes.c_void_p(4096), need - 1, None, ctypes.byref(h)) == B.DUO_E_CAPACITY
    assert L.duo_kv_init(ctypes.byref(cfg), ctypes.c_void_p(4096 + 16), need, None, ctypes.byref(h)) == B.DUO_E_INVALID
    assert L.duo_kv_init(ctypes.byref(cfg), None, need, None, ctypes.byref(h)) == B.DUO_E_INVALID
    assert L.duo_kv_init(ctypes.byref(cfg), ctypes.c_void_p(4096), need, None, None) == B.DUO_E_INVALID
    assert not h.value


def test_null_handle_calls_fail_cleanly():
    L = _lib_or_skip()
    p = ctypes.c_void_p(4096)
    assert L.duo_prefill(None, 0, p, p, p, 4, p, None) == B.DUO_E_INVALID
    assert L.duo_kv_append(None, 0, p, p, 4, None) == B.DUO_E_INVALID
    assert L.duo_decode(None, 0, p, p, p, p, None) == B.DUO_E_INVALID
    assert L.duo_decode_static(None, 0, p, p, p, p, None) == B.DUO_E_INVALID
    n = ctypes.c_int64()
    assert L.duo_kv_length(None, 0, ctypes.byref(n)) == B.DUO_E_INVALID
    assert L.duo_prefill_seq(None, 0, 0, p, p, p, 4, p, None) == B.DUO_E_INVALID
    assert L.duo_kv_append_seq(None, 0, 0, p, p, 4, None) == B.DUO_E_INVALID
    assert L.duo_kv_length_seq(None, 0, 0, ctypes.byref(n)) == B.DUO_E_INVALID
    assert L.duo_prefill_dual(None, 0, p, p, p, 4, p, p, None) == B.DUO_E_INVALID
    assert L.duo_kv_read(None, 0, 0, 0, 0, 0, 1, p, None) == B.DUO_E_INVALID
    L.duo_kv_free(None)
    assert L.duo_synth_fill(None, 1, 1, 0, 0, 10, None) == B.DUO_E_INVALID
    assert L.duo_synth_fill(ctypes.c_void_p(4098), 1, 1, 0, 0, 10, None) == B.DUO_E_INVALID
    assert L.duo_synth_fill(p, 5, 1, 0, 0, 10, None) == B.DUO_E_INVALID
    assert L.duo_synth_fill(p, 1, 1 << 40, 0, 0, 10, None) == B.DUO_E_INVALID


def test_linear_calls_validate_before_launching():
    """Shape and pointer checks of the 8-bit-weight layers (no launch happens)."""
    L = _lib_or_skip()
    p = ctypes.c_void_p(4096)
    assert L.duo_linear_w8(p, 4, 100, p, p, 256, p, None) == B.DUO_E_UNSUPPORTED    # K % 128
    assert L.duo_linear_w8(p, 4, 128, p, p, 300, p, None) == B.DUO_E_UNSUPPORTED    # N % 256
    assert L.duo_linear_w8(p, 0, 128, p, p, 256, p, None) == B.DUO_E_INVALID        # M
    assert L.duo_linear_w8(None, 4, 128, p, p, 256, p, None) == B.DUO_E_INVALID
    assert L.duo_linear_w8(p, 4, 128, p, p, 256, ctypes.c_void_p(4100), None) == B.DUO_E_INVALID
    f = ctypes.c_float
    assert L.duo_qkv_rope_w8(p, 4, 256, p, p, p, 4, 2, 64, f(1e4), p, p, p, None) == B.DUO_E_UNSUPPORTED
    assert L.duo_qkv_rope_w8(p, 4, 256, p, p, p, 4, 2, 128, f(0.5), p, p, p, None) == B.DUO_E_INVALID
    assert L.duo_qkv_rope_w8(p, 4, 256, None, p, p, 4, 2, 128, f(1e4), p, p, p, None) == B.DUO_E_INVALID
    assert L.duo_qkv_rope_w8(p, 4, 256, p, p, p, 3, 2, 128, f(1e4), p, p, p, None) == B.DUO_E_UNSUPPORTED  # N % 256
    assert L.duo_synth_fill(p, B.DUO_SYNTH_INT8, 1 << 40, 0, 0, 10, None) == B.DUO_E_INVALID


def test_product_package_has_no_oracle_or_cpu_fallback():
    """The HIP path never reaches the oracle: no module of the package names it."""
    pkg = os.path.join(ROOT, "mixed_head_kv_amd")
    for fn in glob.glob(os.path.join(pkg, "**", "*.*"), recursive=True):
        if fn.endswith((".py", ".hip", ".cpp", ".h")):
            text = open(fn).read()
            assert "import oracle" not in text and "from oracle" not in text, fn


def test_capacity_arithmetic_orders_the_layouts():
    """bench.py --capacity (workspace arithmetic only, no GPU): int4 Duo holds the longest
    context, then int4 full attention (int4 saves 3.76x, the head split 2x), bf16 Duo,
    bf16 full attention; the int4 Duo context fits its budget and one more token does
    not."""
    _lib_or_skip()
    import bench
    from mixed_head_kv_amd import inputs as I
    import numpy as np
    r = bench.capacity(288)
    c = {k: r[k]["max_context"] for k in ("int4_duo", "bf16_duo", "int4_full", "bf16_full")}
    assert c["int4_duo"] > c["int4_full"] > c["bf16_duo"] > c["bf16_full"] > 1_000_000
    assert abs(r["int4_duo_vs_bf16_full"] - c["int4_duo"] / c["bf16_full"]) < 0.01
    w = I.WORKLOADS["llama3_8b_gqa_32layer_int4_3p3m"]
    cfg = B.make_config(w.n_layers, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.sink, w.recent,
                        c["int4_duo"] + 1, B.DUO_DTYPE_BF16, B.DUO_KV_INT4_G128, w.masks().astype(np.uint8))
    assert r["int4_duo"]["bytes"] <= 288e9 < B.duo_kv_bytes(cfg)


class _FakeWorkspace:
    """Stands in for a workspace tensor in calls that must fail before using it."""

    def __init__(self, nbytes):
        self.nbytes = nbytes

    def data_ptr(self):
        return 1 << 20  # 256-byte aligned, never dereferenced

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def test_fault_injection_fails_init_after_validation(monkeypatch):
    """DUO_FAULT_INJECT naming duo_kv_init makes it return DUO_E_HIP after its argument
    checks and before any HIP call (no handle is returned); the binding raises it as a
    DuoError with that code.  Validation errors still take precedence."""
    _lib_or_skip()
    cfg = _cfg()
    rc, nbytes = _bytes(cfg)
    assert rc == B.DUO_OK
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 20)
    for value in ("duo_decode,duo_kv_init", "all", "duo_kv_init"):
        monkeypatch.setenv("DUO_FAULT_INJECT", value)
        rc = B.lib().duo_kv_init(ctypes.byref(cfg), fake, nbytes, None, ctypes.byref(h))
        assert rc == B.DUO_E_HIP and not h.value
        assert "fault injected" in B.duo_last_error() and "duo_kv_init" in B.duo_last_error()
        rc = B.lib().duo_kv_init(ctypes.byref(cfg), fake, nbytes - 1, None, ctypes.byref(h))
        assert rc == B.DUO_E_CAPACITY and not h.value
        with pytest.raises(B.DuoError) as ei:
            B.duo_kv_init(cfg, _FakeWorkspace(nbytes), stream=0)
        assert ei.value.code == B.DUO_E_HIP


def test_guard_band_call_rejects_bad_arguments():
    _lib_or_skip()
    n = ctypes.c_int32()
    assert B.lib().duo_kv_guard_bands(None, None, 0, ctypes.byref(n)) == B.DUO_E_INVALID


def test_attach_rejects_bad_arguments_before_any_hip_call(monkeypatch):
    """duo_kv_attach (resume over a saved workspace) validates the config, the workspace and
    every length before touching the device; an injected fault comes after that."""
    _lib_or_skip()
    cfg = _cfg()
    rc, nbytes = _bytes(cfg)
    assert rc == B.DUO_OK
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 20)
    n = cfg.n_layers * cfg.batch
    ok = (ctypes.c_int64 * n)(*([5] * n))
    cases = [
        (None, nbytes, B.DUO_E_INVALID),                                          # null lengths
        ((ctypes.c_int64 * n)(*([-1] + [0] * (n - 1))), nbytes, B.DUO_E_INVALID),  # negative
        ((ctypes.c_int64 * n)(*([cfg.max_context + 1] * n)), nbytes, B.DUO_E_INVALID),
        (ok, nbytes - 1, B.DUO_E_CAPACITY),
    ]
    for lengths, size, want in cases:
        rc = B.lib().duo_kv_attach(ctypes.byref(cfg), fake, size, lengths, ctypes.byref(h))
        assert rc == want and not h.value, (rc, want)
    monkeypatch.setenv("DUO_FAULT_INJECT", "duo_kv_attach")
    rc = B.lib().duo_kv_attach(ctypes.byref(cfg), fake, nbytes, ok, ctypes.byref(h))
    assert rc == B.DUO_E_HIP and not h.value and "fault injected" in B.duo_last_error()
