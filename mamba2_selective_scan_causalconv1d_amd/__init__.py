"""Mamba2 mixer hot path on MI355X (gfx950): causal conv1d + SiLU, chunked/decode selective
scan and gated RMSNorm as hand-written HIP kernels behind a C ABI (``include/mamba2.h``).

The GPU entry points live in :mod:`.ops` (imported on demand: it loads the HIP library and
fails loudly when it is missing).  :mod:`.workloads` holds the seeded synthetic inputs.
"""

__all__ = ["ops", "workloads", "build"]
