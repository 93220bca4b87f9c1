"""Paged-attention decode for MI355X (gfx950): HIP kernels behind a C ABI.

``paged_kv_cache_467_amd.binding`` loads the compiled library and exposes its
entry points; ``paged_kv_cache_467_amd.workloads`` builds seeded synthetic
batches.  Importing the package itself loads nothing.
"""
