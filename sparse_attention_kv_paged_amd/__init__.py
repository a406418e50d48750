"""MI355X (gfx950) CSA indexer: paged fp8 key scoring + per-query top-k.

The compute path lives in the HIP library `csrc/` builds (libidx.so); the
Python module `lib` is a thin ctypes binding over its C ABI.  `workloads`
draws the seeded synthetic inputs.
"""
