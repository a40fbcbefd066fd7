"""KVSlimmer asymmetric KV merging, native on AMD MI355X (gfx950).

The hot path lives in the C-ABI library ``libkvslim.so`` (HIP kernels for
gfx950); ``long_context_kv_kvslimmer_amd.kvslim`` is the thin ctypes binding
with the same entry-point names.  ``synth`` draws seeded synthetic inputs and
``configs`` names the five workloads.
"""
