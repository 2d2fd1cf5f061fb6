"""Mixed-head (retrieval / streaming) KV attention for MI355X (gfx950).

The compute lives in ``libduo_attn.so`` (HIP kernels behind a C ABI, declared in
``include/duo_attn.h``).  ``mixed_head_kv_amd.binding`` is the thin ctypes layer over
it; ``mixed_head_kv_amd.inputs`` holds the seeded synthetic inputs.  Importing this
package loads nothing: the library is loaded on first use of the binding, and the
binding raises if the built library is missing (there is no CPU fallback).
"""
