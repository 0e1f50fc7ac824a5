"""Chunked ring attention and Ulysses layout kernels for AMD MI355X (gfx950).

The compute runs in the HIP library ``libsqkv.so`` (C ABI declared in
``include/sqkv.h``); ``sequence_kv_chunk_amd.api`` is a thin ctypes binding that
passes torch tensors' device pointers, strides and the current HIP stream.
Importing the binding loads the library and fails loudly if it is not built.

``sequence_kv_chunk_amd.synth`` (seeded input generators) can be imported
without the library.
"""
_API = ("ra_chunk_attention", "ra_ring_attention", "ra_lse_merge",
        "ulysses_seq_to_head", "ulysses_head_to_seq", "SqkvError")


def __getattr__(name):
    if name in _API:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
